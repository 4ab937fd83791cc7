// Router: affinity logits of every token for every expert, then top-k and
// combine weights.
//
// The router weight is replicated on every expert-parallel rank and scores
// all E experts; the rank then keeps its local ones ("Expert Parallelism
// (EP)", AWS Neuron vLLM design doc, sections "Router Weights" and
// "Collective Patterns / Prefill", step 1: [T, H] @ [H, E] -> [T, E]).
//
// Logits are float32-accurate while running on the bf16 matrix cores: the
// float32 weight w is cut into three bfloat16 parts hi + mid + lo that add up
// to w exactly (each part takes the next 8 significant bits), every
// bf16 x bf16 product is exact in float32, and the three products are
// accumulated in float32. This costs three bf16 MFMAs per product instead of
// one float32 FMA, which the matrix cores run several times faster.
#include "gemm_dma.h"
#include "gemm_tile.h"
#include "moe_kernels.h"

namespace moe {

// w (float32) -> hi, mid, lo (bf16 planes of n elements each), hi+mid+lo == w.
// Four elements per thread (n is a multiple of 8): one 16-byte load, three
// 8-byte stores.
__global__ void route_split_kernel(const float* __restrict__ w, uint16_t* __restrict__ planes, int64_t n) {
  const int64_t n4 = n / 4;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 x4 = reinterpret_cast<const float4*>(w)[i];
    const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
    uint32_t hi[4], mid[4], lo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float x = xs[q];
      hi[q] = __float_as_uint(x) >> 16;
      const float r1 = x - __uint_as_float(hi[q] << 16);
      mid[q] = __float_as_uint(r1) >> 16;
      const float r2 = r1 - __uint_as_float(mid[q] << 16);
      lo[q] = __float_as_uint(r2) >> 16;
    }
    reinterpret_cast<uint2*>(planes)[i] = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
    reinterpret_cast<uint2*>(planes + n)[i] = make_uint2(mid[0] | (mid[1] << 16), mid[2] | (mid[3] << 16));
    reinterpret_cast<uint2*>(planes + 2 * n)[i] = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
  }
}

// logits[t, e] = sum_h x[t, h] * (hi + mid + lo)[e, h] + bias[e]
// Tile: 128 tokens x 128 experts per workgroup, waves 2 x 2 of 64 x 64.
__global__ void __launch_bounds__(kThreads)
route_logits_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ planes,
                    const float* __restrict__ bias, float* __restrict__ logits, int T, int H, int E) {
  constexpr int BM = 128, BN = 128, FM = 2, FN = 2, NP = 3;
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * kLdk];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[NP * BN * kLdk];

  const int t0 = blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;
  const int64_t plane = int64_t(E) * H;
  const int w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  const int lane = lane_id();

  auto rows_a = [&](int r) { return x + int64_t(min(t0 + r, T - 1)) * H; };
  auto rows_b0 = [&](int r) { return planes + int64_t(min(n0 + r, E - 1)) * H; };
  auto rows_b1 = [&](int r) { return planes + plane + int64_t(min(n0 + r, E - 1)) * H; };
  auto rows_b2 = [&](int r) { return planes + 2 * plane + int64_t(min(n0 + r, E - 1)) * H; };

  f32x16 acc[FM][FN];
  zero_acc(acc);
  KRowsLoader<BM> la;
  KRowsLoader<BN> lb0, lb1, lb2;
  const int nk = (H + kBK - 1) / kBK;
  la.load(rows_a, 0, H);
  lb0.load(rows_b0, 0, H);
  lb1.load(rows_b1, 0, H);
  lb2.load(rows_b2, 0, H);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    la.store(As);
    lb0.store(Bs);
    lb1.store(Bs + BN * kLdk);
    lb2.store(Bs + 2 * BN * kLdk);
    __syncthreads();
    if (kt + 1 < nk) {
      const int k0 = (kt + 1) * kBK;
      la.load(rows_a, k0, H);
      lb0.load(rows_b0, k0, H);
      lb1.load(rows_b1, k0, H);
      lb2.load(rows_b2, k0, H);
    }
    mma_stage<FM, FN, NP, BN>(As, Bs, wm * 64, wn * 64, acc);
  }

#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int e = n0 + wn * 64 + fn * 32 + (lane & 31);
      const float b = (bias != nullptr && e < E) ? bias[e] : 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = t0 + wm * 64 + fm * 32 + mfma_c_row(v, lane);
        if (t < T && e < E) logits[int64_t(t) * E + e] = acc[fm][fn][v] + b;
      }
    }
}

// Same logits through the direct-to-LDS pipeline (H a multiple of 64), with
// the k range split into S parts that run as separate workgroups
// (blockIdx.z): tiles of 256 tokens x 128 experts per part, 8 waves of
// 64 x 64 (each token fragment read from LDS serves 2 x 3 products, each
// weight fragment 2), so LDS reads per product are about a quarter lower than
// with 128 x 128 tiles. S is 2 when the tiles alone fill the chip (T = 16384,
// E = 256: 256 workgroups) and grows as T shrinks, down to 4 stages per part
// (a decode step of 256 tokens: 28 parts). The token rows and the three
// weight planes come in 64-deep stages (every request a whole 128-byte line)
// through two LDS buffers; stage s + 2 is issued right after the barrier at
// which every wave has finished reading stage s. Part z writes its raw
// partial sums to out0 (z = 0) or out1 + (z - 1) T E; the top-k kernel adds
// the parts in order, then the bias.
namespace routedma {

constexpr int kBM = 256, kBN = 128, kFM = 2, kFN = 2, kPlanes = 3;
constexpr int kSK = 64;                                            // k per stage
constexpr int kAStage = kBM * kSK * 2;                             // 32 KiB of token rows
constexpr int kPStage = kBN * kSK * 2;                             // 16 KiB per weight plane
constexpr int kStage = kAStage + kPlanes * kPStage;                // 80 KiB
constexpr int kBufs = 2;

__global__ void __launch_bounds__(dma::kThreads)
route_logits_dma_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ planes, float* __restrict__ out0,
                        float* __restrict__ out1, int T, int H, int E, int per) {
  using namespace dma;
  __shared__ __attribute__((aligned(1024))) char smem[kBufs * kStage];
  MOE_LDS char* lds = (MOE_LDS char*)smem;
  const int t0 = blockIdx.x * kBM;
  const int n0 = blockIdx.y * kBN;
  const int w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  const int lane = lane_id();
  const int nk_all = H / kSK;
  const int s0 = blockIdx.z * per;
  const int nk = max(0, min(nk_all, s0 + per) - s0);  // stages of this part
  const int64_t plane = int64_t(E) * H;
  float* __restrict__ out = blockIdx.z == 0 ? out0 : out1 + int64_t(blockIdx.z - 1) * T * E;

  RowLoader64<kBM> la;
  RowLoader64<kBN> lb[kPlanes];
  la.init(x + int64_t(t0) * H, H, min(kBM, T - t0));
#pragma unroll
  for (int p = 0; p < kPlanes; ++p) lb[p].init(planes + p * plane + int64_t(n0) * H, H, min(kBN, E - n0));
  auto issue = [&](int st) {
    if (st < nk) {
      MOE_LDS char* dst = lds + (st % kBufs) * kStage;
      la.issue(dst, (s0 + st) * kSK);
#pragma unroll
      for (int p = 0; p < kPlanes; ++p) lb[p].issue(dst + kAStage + p * kPStage, (s0 + st) * kSK);
    }
  };
  // fragment offsets of 16-deep step ks (0..3): A rows wm*64 + fm*32 + lane%32,
  // B rows wn*64 + fn*32 + lane%32, chunk 2 ks + lane/32, swizzled as RowLoader64
  const int khalf = lane >> 5;
  const int ma = wm * 64 + (lane & 31);
  const int mb = wn * 64 + (lane & 31);
  uint32_t aoff[kSK / 16], boff[kSK / 16];
#pragma unroll
  for (int ks = 0; ks < kSK / 16; ++ks) {
    aoff[ks] = uint32_t(ma * 128 + 16 * ((2 * ks + khalf) ^ ((ma >> 1) & 7)));
    boff[ks] = uint32_t(mb * 128 + 16 * ((2 * ks + khalf) ^ ((mb >> 1) & 7)));
  }
  struct F {
    u32x4 a[kFM];
    u32x4 b[kPlanes][kFN];
  };
  auto load = [&](const MOE_LDS char* st, int ks, F& f) {
#pragma unroll
    for (int fm = 0; fm < kFM; ++fm)
      f.a[fm] = *reinterpret_cast<const MOE_LDS u32x4*>(st + aoff[ks] + fm * 32 * 128);
#pragma unroll
    for (int p = 0; p < kPlanes; ++p)
#pragma unroll
      for (int fn = 0; fn < kFN; ++fn)
        f.b[p][fn] = *reinterpret_cast<const MOE_LDS u32x4*>(st + kAStage + p * kPStage + boff[ks] + fn * 32 * 128);
  };
  f32x16 acc[kFM][kFN];
#pragma unroll
  for (int fm = 0; fm < kFM; ++fm)
#pragma unroll
    for (int fn = 0; fn < kFN; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
  auto mma = [&](const F& f) {
#pragma unroll
    for (int p = 0; p < kPlanes; ++p)
#pragma unroll
      for (int fm = 0; fm < kFM; ++fm)
#pragma unroll
        for (int fn = 0; fn < kFN; ++fn) acc[fm][fn] = mfma32x32x16(f.a[fm], f.b[p][fn], acc[fm][fn]);
  };
  auto interleave = [&]() {
    constexpr int kM = kFM * kFN * kPlanes, kR = kFM + kPlanes * kFN;
#pragma unroll
    for (int i = 0; i < kM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < kR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  constexpr int kLoads = RowLoader64<kBM>::kPer + kPlanes * RowLoader64<kBN>::kPer;  // DMA instructions per wave per stage

  if (nk > 0) {
    issue(0);
    issue(1);
    if (nk > 1)
      wait_vm_barrier<kLoads>();
    else
      wait_vm_barrier<0>();
    F f0, f1;
    load(lds, 0, f0);
    for (int kt = 0; kt < nk; ++kt) {
      const MOE_LDS char* cur = lds + (kt % kBufs) * kStage;
      // steps 0..2: each step's MFMAs cover the next step's LDS reads
      load(cur, 1, f1);
      mma(f0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      load(cur, 2, f0);
      mma(f1);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      load(cur, 3, f1);
      mma(f0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      // step 3: every wave is done reading stage kt and stage kt+1 (the only
      // one in flight) landed; refill this buffer with stage kt+2
      wait_lgkm0();
      wait_vm_barrier<0>();
      issue(kt + 2);
      load(lds + ((kt + 1) % kBufs) * kStage, 0, f0);  // stage nk: a finished buffer, values unused
      mma(f1);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_lgkm0();
  }

#pragma unroll
  for (int fn = 0; fn < kFN; ++fn) {
    const int e = n0 + mb + fn * 32;
#pragma unroll
    for (int fm = 0; fm < kFM; ++fm)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = t0 + wm * 64 + fm * 32 + mfma_c_row(v, lane);
        if (t < T && e < E) out[int64_t(t) * E + e] = acc[fm][fn][v];
      }
  }
}

// The same product with the float32 weight rows staged as they are (4
// bytes per value, instead of 6 for the three bf16 planes) and cut into
// hi + mid + lo in registers, by the same exact steps as route_split_kernel,
// just before the matrix-core products: the bf16 operands, the products and
// their order are those of route_logits_dma_kernel, so are the logits, bit
// for bit. A stage is 32 KiB of token rows and 32 KiB of weight rows (256
// bytes of one expert's row per stage; 16-byte chunk c of row r sits at
// chunk position c ^ (r & 15), so the 16 rows a 16-lane read takes hit 16
// different 16-byte slots). Every token tile repeats the cut (about 88 vector
// instructions per 16-deep step per wave), so launch_route takes this kernel
// only for a few token tiles, where dropping the plane pass pays.
constexpr int kWStage = kBN * kSK * 4;                             // 32 KiB of float32 weight rows
constexpr int kStageW = kAStage + kWStage;                         // 64 KiB

// ROWS float32 rows x 64 k of a k-contiguous matrix: load i of wave w fills
// rows 4 (i * 8 + w) .. +3, 16 lanes (16 bytes each) per row.
template <int ROWS>
struct RowLoaderF32 {
  static constexpr int kPer = ROWS / 4 / dma::kWaves;
  dma::i32x4 rsrc;
  uint32_t voff[kPer];
  __device__ __forceinline__ void init(const float* tile_base, int ld, int rows) {
    rsrc = dma::buffer_rsrc(tile_base, int64_t(rows) * ld * 4);
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = 4 * (i * dma::kWaves + w) + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      voff[i] = uint32_t(min(r, rows - 1)) * uint32_t(ld) * 4u + 16u * uint32_t(c);
    }
  }
  __device__ __forceinline__ void issue(MOE_LDS char* dst, int k0) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < kPer; ++i) dma::dma16(rsrc, voff[i], 4u * uint32_t(k0), dst + 1024 * (i * dma::kWaves + w));
  }
};

// 8 float32 values (two chunks) -> their hi, mid and lo bf16 parts, packed
// as MFMA operands (value 2 d in the low half of dword d).
__device__ __forceinline__ void split3(const u32x4& c0, const u32x4& c1, u32x4& hi, u32x4& mid, u32x4& lo) {
  uint32_t x[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  uint32_t h[8], m[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = x[e] & 0xFFFF0000u;
    const float r1 = __uint_as_float(x[e]) - __uint_as_float(h[e]);
    m[e] = __float_as_uint(r1) & 0xFFFF0000u;
    const float r2 = r1 - __uint_as_float(m[e]);
    l[e] = __float_as_uint(r2);
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    // high halves of values 2 d (low half of the dword) and 2 d + 1
    hi[d] = __builtin_amdgcn_perm(h[2 * d + 1], h[2 * d], 0x07060302u);
    mid[d] = __builtin_amdgcn_perm(m[2 * d + 1], m[2 * d], 0x07060302u);
    lo[d] = __builtin_amdgcn_perm(l[2 * d + 1], l[2 * d], 0x07060302u);
  }
}

// BM tokens x kBN experts per workgroup: 256 tokens as 4 x 2 waves of 64 x 64
// (2 x 2 fragments of 32 x 32), or 64 tokens as 2 x 4 waves of 32 x 32 (one
// fragment), for few tokens, where four times the workgroups keep four times
// the CUs busy.
template <int BM>
__global__ void __launch_bounds__(dma::kThreads)
route_logits_w32_kernel(const uint16_t* __restrict__ x, const float* __restrict__ w_router, float* __restrict__ out0,
                        float* __restrict__ out1, int T, int H, int E, int per) {
  using namespace dma;
  static_assert(BM == 256 || BM == 64, "tile heights");
  constexpr int kWM = BM == 256 ? 4 : 2;  // wave rows
  constexpr int kWN = kWaves / kWM;       // wave columns
  constexpr int kRM = BM / kWM;           // tokens per wave
  constexpr int kCN = kBN / kWN;          // experts per wave
  constexpr int FM = kRM / 32, FN = kCN / 32;
  constexpr int kAStg = BM * kSK * 2;
  constexpr int kStg = kAStg + kWStage;
  __shared__ __attribute__((aligned(1024))) char smem[kBufs * kStg];
  MOE_LDS char* lds = (MOE_LDS char*)smem;
  const int t0 = blockIdx.x * BM;
  const int n0 = blockIdx.y * kBN;
  const int w = threadIdx.x >> 6, wm = w / kWN, wn = w % kWN;
  const int lane = lane_id();
  const int nk_all = H / kSK;
  const int s0 = blockIdx.z * per;
  const int nk = max(0, min(nk_all, s0 + per) - s0);  // stages of this part
  float* __restrict__ out = blockIdx.z == 0 ? out0 : out1 + int64_t(blockIdx.z - 1) * T * E;

  RowLoader64<BM> la;
  RowLoaderF32<kBN> lb;
  la.init(x + int64_t(t0) * H, H, min(BM, T - t0));
  lb.init(w_router + int64_t(n0) * H, H, min(kBN, E - n0));
  auto issue = [&](int st) {
    if (st < nk) {
      MOE_LDS char* dst = lds + (st % kBufs) * kStg;
      la.issue(dst, (s0 + st) * kSK);
      lb.issue(dst + kAStg, (s0 + st) * kSK);
    }
  };
  // fragment offsets of 16-deep step ks (0..3): A rows wm*kRM + fm*32 +
  // lane%32, chunk 2 ks + lane/32 (swizzled as RowLoader64); weight rows
  // wn*kCN + fn*32 + lane%32, float32 chunks 4 ks + 2 (lane/32) and +1
  // (swizzled as RowLoaderF32; the row bits the swizzle uses are those of
  // lane%32)
  const int khalf = lane >> 5;
  const int ma = wm * kRM + (lane & 31);
  const int mb = wn * kCN + (lane & 31);
  uint32_t aoff[kSK / 16], woff[kSK / 16][2];
#pragma unroll
  for (int ks = 0; ks < kSK / 16; ++ks) {
    aoff[ks] = uint32_t(ma * 128 + 16 * ((2 * ks + khalf) ^ ((ma >> 1) & 7)));
#pragma unroll
    for (int e = 0; e < 2; ++e) woff[ks][e] = uint32_t(mb * 256 + 16 * ((4 * ks + 2 * khalf + e) ^ (mb & 15)));
  }
  struct F {
    u32x4 a[FM];
    u32x4 wv[FN][2];
  };
  auto load = [&](const MOE_LDS char* st, int ks, F& f) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      f.a[fm] = *reinterpret_cast<const MOE_LDS u32x4*>(st + aoff[ks] + fm * 32 * 128);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        f.wv[fn][e] = *reinterpret_cast<const MOE_LDS u32x4*>(st + kAStg + woff[ks][e] + fn * 32 * 256);
  };
  f32x16 acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
  auto mma = [&](const F& f) {
    u32x4 b[kPlanes][FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) split3(f.wv[fn][0], f.wv[fn][1], b[0][fn], b[1][fn], b[2][fn]);
#pragma unroll
    for (int p = 0; p < kPlanes; ++p)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma32x32x16(f.a[fm], b[p][fn], acc[fm][fn]);
  };
  constexpr int kLoads = RowLoader64<BM>::kPer + RowLoaderF32<kBN>::kPer;  // DMA instructions per wave per stage

  if (nk > 0) {
    issue(0);
    issue(1);
    if (nk > 1)
      wait_vm_barrier<kLoads>();
    else
      wait_vm_barrier<0>();
    F f0, f1;
    load(lds, 0, f0);
    for (int kt = 0; kt < nk; ++kt) {
      const MOE_LDS char* cur = lds + (kt % kBufs) * kStg;
      // steps 0..2: each step's MFMAs cover the next step's LDS reads
      load(cur, 1, f1);
      mma(f0);
      __builtin_amdgcn_sched_barrier(0);
      load(cur, 2, f0);
      mma(f1);
      __builtin_amdgcn_sched_barrier(0);
      load(cur, 3, f1);
      mma(f0);
      __builtin_amdgcn_sched_barrier(0);
      // step 3: every wave is done reading stage kt and stage kt+1 (the only
      // one in flight) landed; refill this buffer with stage kt+2
      wait_lgkm0();
      wait_vm_barrier<0>();
      issue(kt + 2);
      load(lds + ((kt + 1) % kBufs) * kStg, 0, f0);  // stage nk: a finished buffer, values unused
      mma(f1);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_lgkm0();
  }

#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int e = n0 + mb + fn * 32;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = t0 + wm * kRM + fm * 32 + mfma_c_row(v, lane);
        if (t < T && e < E) out[int64_t(t) * E + e] = acc[fm][fn][v];
      }
  }
}

}  // namespace routedma

// One wave per token: top-k by (logit descending, expert id ascending), then
// softmax weights. Lane l holds experts l, l+64, ... (EPL per lane). Each of
// the k rounds takes the wave maximum of the experts not yet taken (DPP, no
// LDS) and then the lowest expert id holding it (one ballot per EPL slot).
template <int EPL>
__global__ void __launch_bounds__(kThreads)
route_topk_kernel(float* __restrict__ logits, const float* __restrict__ part, int nparts, const float* __restrict__ bias,
                  int T, int E, int k, int renormalize, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float* row = logits + int64_t(t) * E;
  float v[EPL];
  uint32_t live = 0;  // bit i: expert lane + 64 i exists and is not taken yet
  float lm = -INFINITY;
  if (part != nullptr) {  // logits hold the first k part: add the others in order, then the bias; store the sum
    const float* prow = part + int64_t(t) * E;
    const int64_t pstride = int64_t(T) * E;
    float l[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      l[i] = e < E ? row[e] : 0.f;
    }
    // eight parts' loads in flight at a time, added in part order
    for (int z0 = 0; z0 < nparts; z0 += 8) {
      float pv[8][EPL];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          const int e = lane + 64 * i;
          pv[u][i] = (z0 + u < nparts && e < E) ? prow[(z0 + u) * pstride + e] : 0.f;
        }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (z0 + u < nparts)
#pragma unroll
          for (int i = 0; i < EPL; ++i) l[i] += pv[u][i];
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        const float b = l[i] + (bias != nullptr ? bias[e] : 0.f);
        row[e] = b;
        v[i] = b;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (part == nullptr) v[i] = e < E ? row[e] : -INFINITY;
    if (e >= E) v[i] = -INFINITY;
    if (e < E) {
      live |= 1u << i;
      lm = fmaxf(lm, v[i]);
    }
  }
  const float m = wave_max_dpp(lm);

  float den_all = 0.f;
  if (!renormalize) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if ((live >> i) & 1u) s += expf(v[i] - m);
    den_all = wave_sum(s);
  }

  int my_e = 0;
  float my_v = 0.f;
  for (int j = 0; j < k; ++j) {
    float cm = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if ((live >> i) & 1u) cm = fmaxf(cm, v[i]);
    const float bv = wave_max_dpp(cm);
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = EPL - 1; i >= 0; --i) {
      const uint64_t hit = ballot(((live >> i) & 1u) && v[i] == bv);
      if (hit) be = 64 * i + (__ffsll((unsigned long long)hit) - 1);
    }
    if (lane == (be & 63)) live &= ~(1u << (be >> 6));
    if (lane == j) {
      my_e = be;
      my_v = bv;
    }
  }
  const float p = lane < k ? expf(my_v - m) : 0.f;
  float den = den_all;
  if (renormalize) {
    den = 0.f;
    for (int j = 0; j < k; ++j) den += shfl(p, j);
  }
  if (lane < k) {
    topk_idx[int64_t(t) * k + lane] = my_e;
    topk_w[int64_t(t) * k + lane] = p / den;
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
// Top-k for E = 64 Q experts (Q = 1, 2, 4, 8, 16; logits 16-byte aligned):
// lane l holds the Q consecutive experts Q l .. Q l + Q - 1, so every row
// moves with one or a few vector loads per lane and no per-lane bounds
// checks. Same arithmetic and the same choices
// as route_topk_kernel: the k-range parts are added in part order, then the
// bias; each round takes the largest live logit, the lowest expert id among
// equal ones (the lowest lane holding it, then its lowest slot); weights are
// the softmax over all E (or over the k taken, renormalised). Four tokens per
// workgroup, one per wave.
template <int Q>
__device__ __forceinline__ void load_q(const float* __restrict__ p, float (&v)[Q]) {
  if constexpr (Q % 4 == 0) {
#pragma unroll
    for (int i = 0; i < Q / 4; ++i) {
      const float4 f = reinterpret_cast<const float4*>(p)[i];
      v[4 * i] = f.x;
      v[4 * i + 1] = f.y;
      v[4 * i + 2] = f.z;
      v[4 * i + 3] = f.w;
    }
  } else if constexpr (Q == 2) {
    const float2 f = *reinterpret_cast<const float2*>(p);
    v[0] = f.x;
    v[1] = f.y;
  } else {
    v[0] = p[0];
  }
}
template <int Q>
__device__ __forceinline__ void store_q(float* __restrict__ p, const float (&v)[Q]) {
  if constexpr (Q % 4 == 0) {
#pragma unroll
    for (int i = 0; i < Q / 4; ++i)
      reinterpret_cast<float4*>(p)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  } else if constexpr (Q == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  } else {
    p[0] = v[0];
  }
}

template <int Q>
__global__ void __launch_bounds__(kThreads)
route_topk_vec_kernel(float* __restrict__ logits, const float* __restrict__ part, int nparts,
                      const float* __restrict__ bias, int T, int k, int renormalize, int32_t* __restrict__ topk_idx,
                      float* __restrict__ topk_w) {
  constexpr int E = 64 * Q;
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float* row = logits + int64_t(t) * E + Q * lane;
  float v[Q];
  load_q<Q>(row, v);
  if (part != nullptr) {  // logits hold the first k part: add the others in order, then the bias; store the sum
    const float* prow = part + int64_t(t) * E + Q * lane;
    const int64_t pstride = int64_t(T) * E;
    // U parts' loads in flight at a time (64 values a lane), added in part
    // order (a decode step with 28 parts: 19.7 -> 18.8 us for the route
    // stage against four at a time)
    constexpr int U = 64 / Q < 4 ? 4 : (64 / Q > 16 ? 16 : 64 / Q);
    for (int z0 = 0; z0 < nparts; z0 += U) {
      float pv[U][Q];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (z0 + u < nparts) load_q<Q>(prow + (z0 + u) * pstride, pv[u]);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (z0 + u < nparts)
#pragma unroll
          for (int i = 0; i < Q; ++i) v[i] += pv[u][i];
    }
    if (bias != nullptr)  // the bias may sit at any float address: scalar loads
#pragma unroll
      for (int i = 0; i < Q; ++i) v[i] += bias[Q * lane + i];
    store_q<Q>(row, v);
  }
  float lm = v[0];
#pragma unroll
  for (int i = 1; i < Q; ++i) lm = fmaxf(lm, v[i]);
  const float m = wave_max_dpp(lm);

  float den_all = 0.f;
  if (!renormalize) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < Q; ++i) s += expf(v[i] - m);
    den_all = wave_sum(s);
  }

  uint32_t live = (Q == 32 ? ~0u : ((1u << Q) - 1u));  // bit i: expert Q lane + i not taken yet
  int my_e = 0;
  float my_v = 0.f;
  for (int j = 0; j < k; ++j) {
    float cm = -INFINITY;
#pragma unroll
    for (int i = 0; i < Q; ++i)
      if ((live >> i) & 1u) cm = fmaxf(cm, v[i]);
    const float bv = wave_max_dpp(cm);
    int fi = Q;  // this lane's lowest live slot holding the maximum
#pragma unroll
    for (int i = Q - 1; i >= 0; --i)
      if (((live >> i) & 1u) && v[i] == bv) fi = i;
    const uint64_t hit = ballot(fi < Q);
    const int bl = __ffsll((unsigned long long)hit) - 1;
    const int bi = __builtin_amdgcn_readlane(fi, bl);
    if (lane == bl) live &= ~(1u << bi);
    if (lane == j) {
      my_e = Q * bl + bi;
      my_v = bv;
    }
  }
  const float p = lane < k ? expf(my_v - m) : 0.f;
  float den = den_all;
  if (renormalize) {
    den = 0.f;
    for (int j = 0; j < k; ++j) den += shfl(p, j);
  }
  if (lane < k) {
    topk_idx[int64_t(t) * k + lane] = my_e;
    topk_w[int64_t(t) * k + lane] = p / den;
  }
}

// Reductions over one row of 16 lanes, the result in all 16: swap
// neighbours, swap pairs, mirror the halves of 8, mirror the 16. Each step
// combines a lane with its partner, and a partner's result with its own in
// the other order, so (the operations being commutative) every lane of the
// row ends with the same bits.
template <int CTRL>
__device__ __forceinline__ int row_peer(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, __int_as_float(row_peer<0xB1>(__float_as_int(v))));   // quad_perm [1,0,3,2]
  v = fmaxf(v, __int_as_float(row_peer<0x4E>(__float_as_int(v))));   // quad_perm [2,3,0,1]
  v = fmaxf(v, __int_as_float(row_peer<0x141>(__float_as_int(v))));  // row_half_mirror
  v = fmaxf(v, __int_as_float(row_peer<0x140>(__float_as_int(v))));  // row_mirror
  return v;
}
__device__ __forceinline__ float row_sum16(float v) {
  v += __int_as_float(row_peer<0xB1>(__float_as_int(v)));
  v += __int_as_float(row_peer<0x4E>(__float_as_int(v)));
  v += __int_as_float(row_peer<0x141>(__float_as_int(v)));
  v += __int_as_float(row_peer<0x140>(__float_as_int(v)));
  return v;
}
__device__ __forceinline__ uint32_t row_min16(uint32_t v) {
  v = min(v, uint32_t(row_peer<0xB1>(int(v))));
  v = min(v, uint32_t(row_peer<0x4E>(int(v))));
  v = min(v, uint32_t(row_peer<0x141>(int(v))));
  v = min(v, uint32_t(row_peer<0x140>(int(v))));
  return v;
}

// Top-k for E = 16 Q experts (Q = 2, 4, 8, 16) and k <= 16, one row of 16
// lanes per token, four tokens per wave: lane r of a row holds experts
// Q r .. Q r + Q - 1. Same choices as route_topk_vec_kernel (part sums in
// part order, then the bias; each round the largest live logit and, among
// equal ones, the lowest expert id), with the wave-wide reductions replaced
// by row-wide ones: a round is a row maximum of the lanes' live maxima, then
// a row minimum of the ids that hold it. One token per wave leaves the vector
// units doing a 64-lane reduction per selected expert; four per wave cut the
// instructions per token about fourfold, and the kernel becomes bound by
// its loads and stores. The softmax denominator over all E is a row sum
// (summation order differs from the one-wave kernels, within float32
// rounding); the renormalised one adds the k taken in order.
template <int Q>
__global__ void __launch_bounds__(kThreads)
route_topk_row_kernel(float* __restrict__ logits, const float* __restrict__ part, int nparts,
                      const float* __restrict__ bias, int T, int k, int renormalize, int32_t* __restrict__ topk_idx,
                      float* __restrict__ topk_w) {
  constexpr int E = 16 * Q;
  const int lane = lane_id();
  const int l16 = lane & 15;
  const int t = int((int64_t(blockIdx.x) * kThreads + threadIdx.x) >> 4);
  if (t >= T) return;  // whole rows: the row reductions below read only lanes of the same row
  float* row = logits + int64_t(t) * E + Q * l16;
  float v[Q];
  load_q<Q>(row, v);
  if (part != nullptr) {  // logits hold the first k part: add the others in order, then the bias; store the sum
    const float* prow = part + int64_t(t) * E + Q * l16;
    const int64_t pstride = int64_t(T) * E;
    for (int z0 = 0; z0 < nparts; z0 += 4) {
      float pv[4][Q];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (z0 + u < nparts) load_q<Q>(prow + (z0 + u) * pstride, pv[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (z0 + u < nparts)
#pragma unroll
          for (int i = 0; i < Q; ++i) v[i] += pv[u][i];
    }
    if (bias != nullptr) {
      float b[Q];
      if ((reinterpret_cast<uintptr_t>(bias) & 15u) == 0) {  // the same for every lane
        load_q<Q>(bias + Q * l16, b);
      } else {  // the bias may sit at any float address: one value per load
#pragma unroll
        for (int i = 0; i < Q; ++i) b[i] = bias[Q * l16 + i];
      }
#pragma unroll
      for (int i = 0; i < Q; ++i) v[i] += b[i];
    }
    store_q<Q>(row, v);
  }
  float lm = v[0];
#pragma unroll
  for (int i = 1; i < Q; ++i) lm = fmaxf(lm, v[i]);
  const float m = row_max16(lm);

  float den_all = 0.f;
  if (!renormalize) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < Q; ++i) s += expf(v[i] - m);
    den_all = row_sum16(s);
  }

  // A taken expert's value becomes NaN: the maximum ignores NaN and no NaN
  // equals the row maximum, so it is never chosen again (a logit of -inf
  // stays selectable).
  const uint32_t base = uint32_t(Q * l16);
  int my_e = 0;
  float my_v = 0.f;
  for (int j = 0; j < k; ++j) {
    float cm = -INFINITY;
#pragma unroll
    for (int i = 0; i < Q; ++i) cm = fmaxf(cm, v[i]);
    const float bv = row_max16(cm);
    uint32_t cand = uint32_t(E);  // this lane's lowest expert holding the maximum
#pragma unroll
    for (int i = Q - 1; i >= 0; --i)
      if (v[i] == bv) cand = base + uint32_t(i);
    const uint32_t best = row_min16(cand);
#pragma unroll
    for (int i = 0; i < Q; ++i)
      if (best == base + uint32_t(i)) v[i] = __int_as_float(0x7FC00000);
    if (l16 == j) {
      my_e = int(best);
      my_v = bv;
    }
  }
  const float p = l16 < k ? expf(my_v - m) : 0.f;
  float den = den_all;
  if (renormalize) {
    den = 0.f;
    for (int j = 0; j < k; ++j) den += shfl(p, (lane & ~15) + j);
  }
  if (l16 < k) {
    topk_idx[int64_t(t) * k + l16] = my_e;
    topk_w[int64_t(t) * k + l16] = p / den;
  }
}

int route_k_parts(int T, int H, int E) {
  if (H % routedma::kSK != 0) return 1;
  const int nk_all = H / routedma::kSK;
  const int64_t tiles = int64_t((T + routedma::kBM - 1) / routedma::kBM) * ((E + routedma::kBN - 1) / routedma::kBN);
  // enough parts for about 256 workgroups, at least 2, each part at least 4
  // stages deep (1 when the T x E partial sums the top-k kernel adds are
  // small: measured on decode steps, a GPT-OSS-20B-shaped one, T E = 8K,
  // routes in 19 instead of 22 us at one stage per part, a DeepSeek-R1-shaped
  // one, T E = 64K, in 37 instead of 29); then as few parts as that depth
  // needs
  int64_t want = std::max<int64_t>(2, (256 + tiles - 1) / std::max<int64_t>(tiles, 1));
  const int min_depth = int64_t(T) * E <= 16384 ? 1 : 4;
  want = std::min<int64_t>(want, std::max(2, nk_all / min_depth));
  want = std::min<int64_t>(want, nk_all);
  if (want < 2) return 1;
  const int per = int((nk_all + want - 1) / want);
  return (nk_all + per - 1) / per;
}

hipError_t launch_route(const uint16_t* x, const float* w_router, const float* bias, int T, int H, int E, int k,
                        int renormalize, float* logits, int32_t* topk_idx, float* topk_w, uint16_t* planes, float* part,
                        hipStream_t stream) {
  const int64_t n = int64_t(E) * H;
  const int parts = route_k_parts(T, H, E);
  const bool split = parts > 1;
  // Cutting the float32 weights in registers is repeated by every token tile:
  // it pays (no plane pass, a third less weight traffic) for a few tiles and
  // loses beyond (measured: ahead at 1 and 8 tiles of 256 tokens, behind at
  // 32 and 64)
  const bool w32 = split && (T + routedma::kBM - 1) / routedma::kBM <= 8;
  if (!w32) {
    const int threads = 256;
    const int64_t blocks = std::min<int64_t>((n / 4 + threads - 1) / threads, 4096);
    hipLaunchKernelGGL(route_split_kernel, dim3(unsigned(blocks)), dim3(threads), 0, stream, w_router, planes, n);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  {
    if (split) {
      const int nk_all = H / routedma::kSK;
      const int per = (nk_all + parts - 1) / parts;
      dim3 grid(unsigned((T + routedma::kBM - 1) / routedma::kBM), unsigned((E + routedma::kBN - 1) / routedma::kBN),
                unsigned(parts));
      if (w32 && T <= 512)  // decode-sized batches: 64-token tiles, four times the workgroups
        hipLaunchKernelGGL(routedma::route_logits_w32_kernel<64>, dim3(unsigned((T + 63) / 64), grid.y, grid.z),
                           dim3(dma::kThreads), 0, stream, x, w_router, logits, part, T, H, E, per);
      else if (w32)
        hipLaunchKernelGGL(routedma::route_logits_w32_kernel<256>, grid, dim3(dma::kThreads), 0, stream, x, w_router,
                           logits, part, T, H, E, per);
      else
        hipLaunchKernelGGL(routedma::route_logits_dma_kernel, grid, dim3(dma::kThreads), 0, stream, x, planes, logits,
                           part, T, H, E, per);
    } else {
      dim3 grid(unsigned((T + 127) / 128), unsigned((E + 127) / 128));
      hipLaunchKernelGGL(route_logits_kernel, grid, dim3(kThreads), 0, stream, x, planes, bias, logits, T, H, E);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  {
    const float* pt = split ? part : nullptr;
    // the vector loads and stores need 16-byte aligned rows (8-byte for two
    // experts per lane; the partial sums live in the workspace, which is)
    const uintptr_t la = reinterpret_cast<uintptr_t>(logits);
    // (with few tokens the one-wave kernels spread the partial sums over
    // more waves: a DeepSeek-R1-shaped decode step, T = 256 with 28 parts,
    // routes in 24 us that way against 28 with rows)
    if ((E == 32 || E == 64 || E == 128 || E == 256) && k <= 16 && T >= 2048 && (la & (E == 32 ? 7u : 15u)) == 0) {
      dim3 rgrid(unsigned((int64_t(T) * 16 + kThreads - 1) / kThreads));
#define MOE_TOPK_ROW(Q)                                                                                           \
  hipLaunchKernelGGL(route_topk_row_kernel<Q>, rgrid, dim3(kThreads), 0, stream, logits, pt, parts - 1, bias, T, k, \
                     renormalize, topk_idx, topk_w)
      if (E == 32)
        MOE_TOPK_ROW(2);
      else if (E == 64)
        MOE_TOPK_ROW(4);
      else if (E == 128)
        MOE_TOPK_ROW(8);
      else
        MOE_TOPK_ROW(16);
#undef MOE_TOPK_ROW
      return hipGetLastError();
    }
    dim3 grid(unsigned((T + 3) / 4));
    const int epl = (E + 63) / 64;
#define MOE_TOPK_VEC(Q)                                                                                          \
  hipLaunchKernelGGL(route_topk_vec_kernel<Q>, grid, dim3(kThreads), 0, stream, logits, pt, parts - 1, bias, T, k, \
                     renormalize, topk_idx, topk_w)
    // the vector loads and stores need 16-byte aligned rows (the partial
    // sums live in the workspace, which is)
    if (E % 64 == 0 && (epl == 1 || epl == 2 || epl == 4 || epl == 8 || epl == 16) &&
        (reinterpret_cast<uintptr_t>(logits) & 15u) == 0) {
      if (epl == 1)
        MOE_TOPK_VEC(1);
      else if (epl == 2)
        MOE_TOPK_VEC(2);
      else if (epl == 4)
        MOE_TOPK_VEC(4);
      else if (epl == 8)
        MOE_TOPK_VEC(8);
      else
        MOE_TOPK_VEC(16);
      return hipGetLastError();
    }
#undef MOE_TOPK_VEC
#define MOE_TOPK_LAUNCH(EPL)                                                                                       \
  hipLaunchKernelGGL(route_topk_kernel<EPL>, grid, dim3(kThreads), 0, stream, logits, pt, parts - 1, bias, T, E, k, \
                     renormalize, topk_idx, topk_w)
    if (epl <= 1)
      MOE_TOPK_LAUNCH(1);
    else if (epl <= 2)
      MOE_TOPK_LAUNCH(2);
    else if (epl <= 4)
      MOE_TOPK_LAUNCH(4);
    else if (epl <= 8)
      MOE_TOPK_LAUNCH(8);
    else
      MOE_TOPK_LAUNCH(16);
#undef MOE_TOPK_LAUNCH
    return hipGetLastError();
  }
}

}  // namespace moe
