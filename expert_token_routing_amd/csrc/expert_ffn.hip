// Expert MLPs as grouped GEMMs over ragged expert segments.
//
// Each local expert i owns gate_up [H, 2I] (gate = columns [0, I), up =
// columns [I, 2I)) and down [I, H] ("Expert Parallelism (EP)", AWS Neuron
// vLLM design doc, weight-shape table under "Expert Weight Distribution").
// Its rows are the dispatched segment [offsets[i], offsets[i+1]), stacked into
// one matmul because every token is transformed on its own ("EP: Partition
// Experts and Route Tokens", "Send tokens to experts and return their
// results"). Segment lengths are data dependent and read on the device, so no
// host synchronisation sits between dispatch and the GEMMs.
//
//   GEMM1:  h   = silu(X Wg) * (X Wu)   fused: one tile computes matching
//                                      gate and up columns and writes h
//   GEMM2:  out = h Wd
//
// Both are persistent kernels: every workgroup rebuilds the tile list from
// `offsets` and strides over it. Two implementations:
//  * panel_gemm_kernel (k a multiple of 32): direct global->LDS loads in
//    64-deep stages, tiles of up to 288 rows of one expert x 256 weight
//    columns, 16x16x32 MFMAs; the weight operand is read from LDS with
//    transposing reads.
//  * grouped_gemm_kernel (any k that is a multiple of 8): register-staged
//    loads, weights transposed 8 x 8 in registers on their way to LDS.
#include "gemm_dma.h"
#include "gemm_tile.h"
#include "moe_kernels.h"

namespace moe {

constexpr int kMaxLocal = 1024;
// Row caps the panel GEMM chooses from per launch (largest first; all are
// multiples of 32 and at most the 288 rows a tile holds). (Caps of 96 and 64
// rows, which give a down GEMM with few experts and few column panels tiles
// for every CU, measured no faster: such tiles are bound by the operand bytes
// one CU fetches per cycle, not by the idle CUs.)
constexpr int kRowCaps = 6;
__device__ constexpr int kRowCap[kRowCaps] = {288, 256, 224, 192, 160, 128};
constexpr int kRowCapMin = 128;

template <int BM, bool SWIGLU>
__global__ void __launch_bounds__(kThreads)
grouped_gemm_kernel(const uint16_t* __restrict__ A, int lda, const int32_t* __restrict__ offsets, int E_local,
                    int64_t capacity, const uint16_t* __restrict__ W, int64_t w_expert_stride, int ldw,
                    uint16_t* __restrict__ C, int ldc, int K, int N, int up_off) {
  constexpr int BN = 256;
  constexpr int FM = BM / 64;
  constexpr int FN = 4;
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * kLdk];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * kLdk];
  __shared__ int s_off[kMaxLocal + 1];
  __shared__ int s_tpre[kMaxLocal + 1];
  __shared__ int s_tmp[4];

  // Segment bounds (clamped into [0, capacity]) and the m-tile prefix.
  int mt[4];
  int sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = threadIdx.x * 4 + q;
    mt[q] = 0;
    if (i < E_local) {
      const int64_t a = min<int64_t>(max<int64_t>(offsets[i], 0), capacity);
      const int64_t b = max<int64_t>(a, min<int64_t>(offsets[i + 1], capacity));
      s_off[i] = int(a);
      mt[q] = int((b - a + BM - 1) / BM);
      if (i == E_local - 1) s_off[E_local] = int(b);
    }
    sum += mt[q];
  }
  int total_mt;
  int pre = block_exclusive_scan(sum, s_tmp, total_mt);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = threadIdx.x * 4 + q;
    if (i < E_local) s_tpre[i] = pre;
    pre += mt[q];
  }
  __syncthreads();

  const int ntn = SWIGLU ? (N + 127) / 128 : (N + 255) / 256;
  const int total = total_mt * ntn;
  const int w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  const int lane = lane_id();
  const int nk = (K + kBK - 1) / kBK;

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int gm = tile / ntn;
    const int nj = tile - gm * ntn;
    int lo = 0, hi = E_local - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tpre[mid] <= gm)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int e = lo;
    const int r0 = s_off[e] + (gm - s_tpre[e]) * BM;
    const int rows = min(BM, s_off[e + 1] - r0);
    const uint16_t* We = W + int64_t(e) * w_expert_stride;

    auto row_ptr = [&](int r) { return A + int64_t(r0 + min(r, rows - 1)) * lda; };
    auto col_of = [&](int s0) -> int {
      if (SWIGLU) {
        const int q = s0 & 127;
        const int oc = nj * 128 + (s0 >> 7) * 64 + (q & 63);
        if (oc >= N) return -1;
        return q < 64 ? oc : up_off + oc;
      } else {
        const int oc = nj * 256 + s0;
        return oc < N ? oc : -1;
      }
    };

    f32x16 acc[FM][FN];
    zero_acc(acc);
    KRowsLoader<BM> la;
    NColsTransposeLoader lb;
    la.load(row_ptr, 0, K);
    lb.load(We, ldw, col_of, 0, K);
    for (int kt = 0; kt < nk; ++kt) {
      __syncthreads();
      la.store(As);
      lb.store(Bs);
      __syncthreads();
      if (kt + 1 < nk) {
        la.load(row_ptr, (kt + 1) * kBK, K);
        lb.load(We, ldw, col_of, (kt + 1) * kBK, K);
      }
      mma_stage<FM, FN, 1, BN>(As, Bs, wm * (BM / 2), wn * 128, acc);
    }

    if (SWIGLU) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn) {
          const int col = nj * 128 + wn * 64 + fn * 32 + (lane & 31);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = wm * (BM / 2) + fm * 32 + mfma_c_row(v, lane);
            if (row < rows && col < N) {
              const float g = acc[fm][fn][v];
              const float u = acc[fm][fn + 2][v];
              const float hv = g / (1.f + __expf(-g)) * u;
              C[int64_t(r0 + row) * ldc + col] = uint16_t(f32_to_bf16_bits(hv));
            }
          }
        }
    } else {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int col = nj * 256 + wn * 128 + fn * 32 + (lane & 31);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = wm * (BM / 2) + fm * 32 + mfma_c_row(v, lane);
            if (row < rows && col < N)
              C[int64_t(r0 + row) * ldc + col] = uint16_t(f32_to_bf16_bits(acc[fm][fn][v]));
          }
        }
    }
  }
}

// Expert-panel grouped GEMM (k a multiple of 32). A tile is a block of up to
// 288 rows of one expert (an expert's rows are split evenly into
// ceil(M / 288) blocks, so padding stays below 16 rows per block) x 256
// weight columns; 8 waves as 2 wave rows x 4 wave columns of 64.
//
// Memory requests, not bytes, bound this kernel: every operand request is a
// whole 128-byte line (64-deep stages: a token row's 64 k are one line), and
// the tile shape keeps requests per output low. Stages come in through a
// ring of two LDS buffers; stage s is read into registers during iteration
// s - 1 and multiplied in iteration s, and its buffer is refilled with stage
// s + 2 right after the barrier of iteration s that follows the last read.
namespace panelffn {

using namespace dma::panel;

// Ask the scheduler to alternate the region's MFMAs with its LDS reads, one
// read after each MFMA while reads remain, so that the reads spread over the
// MFMA time instead of bunching up (a read that must wait for an earlier MFMA
// simply takes a later slot).
template <int NM, int NR>
__device__ __forceinline__ void alternate_mfma_reads() {
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // one MFMA
    if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);       // one LDS read
  }
#pragma unroll
  for (int i = NM; i < NR; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
}

// One tile: FMT fragments per wave row (16 * kWR * FMT >= rows), `rows` rows
// from the row source, weight columns given by col_of.
// FUSE (down GEMM only): s_ri holds, for each tile row, the destination
// token and combine weight of a row whose token has exactly one local
// selection (token -1 otherwise); such rows go to y as the combine would
// write them, the others to C.
// HALF: K % 64 == 32, so the last stage holds half a stage of k values; its
// loads then stay inside the operands (issue_half).
template <int FMT, bool SWIGLU, bool FUSE, bool HALF, typename SrcRow, typename ColOf>
__device__ __forceinline__ void run_tile(MOE_LDS char* lds, const uint16_t* __restrict__ Abase, int64_t a_bytes,
                                         int lda, int rows, SrcRow src_row, const uint16_t* __restrict__ We, int ldw,
                                         int K, ColOf col_of, int out_c0, int N, uint16_t* __restrict__ C, int ldc,
                                         int r0, const MOE_LDS int* s_ri, uint16_t* __restrict__ y) {
  const int w = threadIdx.x >> 6, wm = w % kWR, wn = w / kWR;
  const int lane = lane_id();
  // GEMM1 multiplies weight x row fragments, i.e. produces the transposed
  // tile, so that each lane ends up with 4 consecutive h columns of one row
  // (8-byte stores); GEMM2 keeps the direct form (a column per lane).
  auto mma = [](const u32x4& ra, const u32x4& wb, const f32x4v& c) {
    if constexpr (SWIGLU)
      return mfma16x16x32(wb, ra, c);
    else
      return mfma16x16x32(ra, wb, c);
  };
  // stages of kSK; K is a multiple of 32, so the last stage may hold only
  // its first k step (the second is multiplied as zeros)
  const int nk = (K + kSK - 1) / kSK;
  const bool half_tail = (K % kSK) != 0;
  const int r16 = (rows + 15) & ~15;
  constexpr int kAStage = a_stage_bytes(FMT);
  constexpr int kStages = stages_for(FMT);
  MOE_LDS char* const ldsA = lds;
  MOE_LDS char* const ldsB = lds + kStages * kAStage;

  f32x4v acc[FMT][kFN];
#pragma unroll
  for (int i = 0; i < FMT; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};

  ALoaderP la;
  la.init(Abase, a_bytes, lda, rows, r16, src_row);
  BLoaderP lb;
  lb.init(We, ldw, K, col_of);
  const int nl = la.count + BLoaderP::kPer;  // DMA instructions of this wave per stage
  auto issue = [&](int st) {
    if (st < nk) {
      const int buf = st % kStages;
      if (HALF && st == nk - 1) {
        la.issue_half(ldsA + buf * kAStage, st * kSK);
        lb.issue_half(ldsB + buf * kBStage, st);
      } else {
        la.issue(ldsA + buf * kAStage, st * kSK);
        lb.issue(ldsB + buf * kBStage, st);
      }
    }
  };
  // Wait until stage s landed, then barrier. Stages complete in issue order;
  // the ones issued after s (s+1 .. min(last, nk-1)) may stay in flight.
  auto wait_stage = [&](int s, int last) {
    const int ahead = max(0, min(last, nk - 1) - s);
    dma::wait_vm_barrier_dyn<(kStages - 1) * (ALoaderP::kPerMax + BLoaderP::kPer)>(ahead * nl);
  };
  FragAddrP fa;
  fa.init(wm, wn);
  u32x4 a[FMT], b[kFN];

  for (int st = 0; st < kStages; ++st) issue(st);
  wait_stage(0, kStages - 1);
#pragma unroll
  for (int j = 0; j < kFN; ++j) b[j] = read_b<0>(ldsB, fa, j);
#pragma unroll
  for (int i = 0; i < FMT; ++i) a[i] = read_a<0>(ldsA, fa, i);

  constexpr int kH1 = (FMT + 1) / 2;  // fragment rows multiplied before the barrier
  for (int kt = 0; kt < nk; ++kt) {
    if constexpr (kSub == 2) {
      // k step 0 of stage kt; step 1's fragments (same buffer, landed) stream
      // in behind it, each A row right after its last use
      const int cb = kt % kStages;
      const MOE_LDS char* cA = ldsA + cb * kAStage;
      const MOE_LDS char* cB = ldsB + cb * kBStage;
      u32x4 bs[kFN];
#pragma unroll
      for (int j = 0; j < kFN; ++j) bs[j] = read_b<1>(cB, fa, j);
#pragma unroll
      for (int i = 0; i < FMT; ++i) {
#pragma unroll
        for (int j = 0; j < kFN; ++j) acc[i][j] = mma(a[i], b[j], acc[i][j]);
        a[i] = read_a<1>(cA, fa, i);
      }
      alternate_mfma_reads<FMT * kFN, 2 * kFN + FMT>();
#pragma unroll
      for (int j = 0; j < kFN; ++j) b[j] = bs[j];
      if (half_tail && kt == nk - 1) {  // k beyond K: LDS holds other data
#pragma unroll
        for (int j = 0; j < kFN; ++j) b[j] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < FMT; ++i) a[i] = u32x4{0u, 0u, 0u, 0u};
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // last k step of stage kt. First half: rows 0 .. kH1-1 (registers only)
#pragma unroll
    for (int i = 0; i < kH1; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j) acc[i][j] = mma(a[i], b[j], acc[i][j]);
    __builtin_amdgcn_sched_barrier(0);
    // every wave has read stage kt (its reads were waited for), and stage
    // kt+1 landed: refill stage kt's buffer with stage kt+kStages, read stage kt+1
    dma::wait_lgkm0();
    // stages issued so far: up to kt + kStages - 1
    if (kt + 1 < nk) wait_stage(kt + 1, kt + kStages - 1); else dma::wait_vm_barrier<0>();
    issue(kt + kStages);
    const int nb = (kt + 1) % kStages;
    const MOE_LDS char* nA = ldsA + nb * kAStage;
    const MOE_LDS char* nB = ldsB + nb * kBStage;
    u32x4 bn[kFN];
#pragma unroll
    for (int j = 0; j < kFN; ++j) bn[j] = read_b<0>(nB, fa, j);
#pragma unroll
    for (int i = 0; i < kH1; ++i) a[i] = read_a<0>(nA, fa, i);
    // second half, then this stage's last A registers take the next stage's
#pragma unroll
    for (int i = kH1; i < FMT; ++i) {
#pragma unroll
      for (int j = 0; j < kFN; ++j) acc[i][j] = mma(a[i], b[j], acc[i][j]);
      a[i] = read_a<0>(nA, fa, i);
    }
    alternate_mfma_reads<(FMT - kH1) * kFN, 2 * kFN + FMT>();
#pragma unroll
    for (int j = 0; j < kFN; ++j) b[j] = bn[j];
    __builtin_amdgcn_sched_barrier(0);
  }
  dma::wait_lds_barrier();

  const int l16 = lane & 15;        // lane within a 16-lane group
  const int g4 = 4 * (lane >> 4);   // 4 x the lane's group
  if constexpr (SWIGLU) {
    // transposed tile: fragment (i, j), lane l, element v is tile row
    // 16 (kWR i + wm) + (l & 15), tile column 64 wn + 16 j + 4 (l >> 4) + v;
    // wave columns: 32 gate then the matching 32 up outputs
#pragma unroll
    for (int i = 0; i < FMT; ++i) {
      const int row = 16 * (kWR * i + wm) + l16;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = out_c0 + 32 * wn + 16 * j + g4;
        if (row < rows && col < N) {  // N is a multiple of 8: all 4 columns are in range
          float hv[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float g = acc[i][j][v];
            hv[v] = g / (1.f + __expf(-g)) * acc[i][j + 2][v];
          }
          *reinterpret_cast<uint2*>(C + int64_t(r0 + row) * ldc + col) =
              make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
        }
      }
    }
  } else if constexpr (FUSE) {
    // as below; a row of a single-selection token becomes w * out in its
    // token's y row, rounded like the combine's one-term sum (fmaf onto -0,
    // then bf16). The row info is read at constant offsets from one base
    // (immediate LDS offsets, no per-row address registers).
    typedef int i32x2v __attribute__((ext_vector_type(2)));
    const MOE_LDS i32x2v* const rib = reinterpret_cast<const MOE_LDS i32x2v*>(s_ri) + 16 * wm + g4;
#pragma unroll
    for (int i = 0; i < FMT; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 16 * (kWR * i + wm) + g4 + v;
        if (row < rows) {
          const i32x2v ri = rib[16 * kWR * i + v];
          const int dst = ri.x;
          const float wt = __int_as_float(ri.y);
          uint16_t* const base = dst >= 0 ? y + int64_t(dst) * ldc : C + int64_t(r0 + row) * ldc;
#pragma unroll
          for (int j = 0; j < kFN; ++j) {
            const int col = out_c0 + 64 * wn + 16 * j + l16;
            if (col < N) {
              const uint32_t ob = f32_to_bf16_bits(acc[i][j][v]);
              base[col] = uint16_t(dst >= 0 ? f32_to_bf16_bits(fmaf(wt, bf16_to_f32(uint16_t(ob)), -0.f)) : ob);
            }
          }
        }
      }
  } else {
    // fragment (i, j), lane l, element v is tile row 16 (kWR i + wm) + 4 (l >> 4) + v,
    // tile column 64 wn + 16 j + (l & 15)
#pragma unroll
    for (int i = 0; i < FMT; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j) {
        const int col = out_c0 + 64 * wn + 16 * j + l16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = 16 * (kWR * i + wm) + g4 + v;
          if (row < rows && col < N) C[int64_t(r0 + row) * ldc + col] = uint16_t(f32_to_bf16_bits(acc[i][j][v]));
        }
      }
  }
}

}  // namespace panelffn

// Tiles: expert i has nrt_i = ceil(M_i / 288) row blocks of equal height (a
// multiple of 16) times ntn column tiles, ordered expert-major, column-major
// inside the expert (the row blocks sharing a weight panel are adjacent and
// run together); each XCD takes a contiguous range, dealt round robin to its
// workgroups (workgroup b runs on XCD b % 8).
// FUSE (down GEMM): row_info[n] = {token, combine weight bits} for row n of a
// token with exactly one local selection, {-1, 0} otherwise; those rows are
// written to y [T, ldc] instead of C.
template <bool SWIGLU, bool FUSE, bool HALF>
__global__ void __launch_bounds__(dma::kThreads)
panel_gemm_kernel(const uint16_t* __restrict__ A, int lda, const int32_t* __restrict__ offsets, int E_local,
                  int64_t capacity, const uint16_t* __restrict__ W, int64_t w_expert_stride, int ldw,
                  uint16_t* __restrict__ C, int ldc, int K, int N, int up_off, const int32_t* __restrict__ gather_src,
                  int gather_k, int gather_rows, const int2* __restrict__ row_info, uint16_t* __restrict__ y) {
  using namespace dma::panel;
  static_assert(!(FUSE && SWIGLU), "the combine is fused into the down GEMM only");
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  // row info of the tile: 3 waves x 64 lanes x 16 bytes cover the 288 rows.
  // Two buffers by tile parity: a wave copies the next tile's info while
  // slower waves may still read this tile's in their epilogue (the next
  // tile's first barrier orders everything after that).
  __shared__ __attribute__((aligned(1024))) int s_ri[FUSE ? 2 * 768 : 4];
  __shared__ int s_off[kMaxLocal + 1];
  __shared__ int s_tpre[kMaxLocal + 1];
  __shared__ int s_tmp[dma::kWaves];
  __shared__ unsigned long long s_ntile[kRowCaps];
  __shared__ int s_cand[kRowCaps];
  MOE_LDS char* lds = (MOE_LDS char*)smem;

  const int ntn = SWIGLU ? (N + kBN / 2 - 1) / (kBN / 2) : (N + kBN - 1) / kBN;
  constexpr int kPerT = (kMaxLocal + dma::kThreads - 1) / dma::kThreads;
  int me[kPerT];
  if (threadIdx.x < kRowCaps) {
    s_ntile[threadIdx.x] = 0;
    s_cand[threadIdx.x] = 0;
  }
#pragma unroll
  for (int q = 0; q < kPerT; ++q) {
    const int i = threadIdx.x * kPerT + q;
    me[q] = 0;
    if (i < E_local) {
      const int64_t a = min<int64_t>(max<int64_t>(offsets[i], 0), capacity);
      const int64_t b = max<int64_t>(a, min<int64_t>(offsets[i + 1], capacity));
      s_off[i] = int(a);
      me[q] = int(b - a);
      if (i == E_local - 1) s_off[E_local] = int(b);
    }
  }
  __syncthreads();
  // Row cap of the launch: for each candidate cap, the tile count and the
  // tallest row block; the cap whose estimate ceil(tiles / grid) x (tallest
  // block + 256) is lowest wins (a tile's time grows with its rows plus its
  // 256 weight columns), the larger cap on ties. A cap whose tile count does
  // not fit the 31-bit tile indices is skipped (the host rejects launches
  // where even the largest cap's does not). Every workgroup gets the same
  // sums and picks the same cap.
#pragma unroll
  for (int c = 0; c < kRowCaps; ++c) {
    unsigned long long tl = 0;
    int hm = 0;
#pragma unroll
    for (int q = 0; q < kPerT; ++q) {
      if (me[q] > 0) {
        const int nrt = (me[q] + kRowCap[c] - 1) / kRowCap[c];
        tl += (unsigned long long)nrt * (unsigned long long)ntn;
        hm = max(hm, (((me[q] + nrt - 1) / nrt) + 15) & ~15);
      }
    }
    if (tl > 0) atomicAdd(&s_ntile[c], tl);
    if (hm > 0) atomicMax(&s_cand[c], hm);
  }
  __syncthreads();
  int row_cap = kRowCap[0];
  {
    unsigned long long best = ~0ull;
#pragma unroll
    for (int c = 0; c < kRowCaps; ++c) {
      const unsigned long long tl = s_ntile[c];
      if (tl >= (1ull << 31)) continue;
      const unsigned long long est = (tl + gridDim.x - 1) / gridDim.x * (unsigned long long)(s_cand[c] + kBN);
      if (est < best) {
        best = est;
        row_cap = kRowCap[c];
      }
    }
  }
  int mt[kPerT];
  int sum = 0;
#pragma unroll
  for (int q = 0; q < kPerT; ++q) {
    mt[q] = (me[q] + row_cap - 1) / row_cap * ntn;
    sum += mt[q];
  }
  int total;
  int pre = block_exclusive_scan<dma::kThreads>(sum, s_tmp, total);
#pragma unroll
  for (int q = 0; q < kPerT; ++q) {
    const int i = threadIdx.x * kPerT + q;
    if (i < E_local) s_tpre[i] = pre;
    pre += mt[q];
  }
  if (threadIdx.x == 0) s_tpre[E_local] = total;
  __syncthreads();

  const int nxcd = 8;
  const int xcd = blockIdx.x % nxcd;
  const int per_xcd = gridDim.x / nxcd;
  const int lo_t = int((int64_t(total) * xcd) / nxcd);
  const int hi_t = int((int64_t(total) * (xcd + 1)) / nxcd);
  int parity = 0;
  for (int tile = lo_t + int(blockIdx.x / nxcd); tile < hi_t; tile += per_xcd) {
    int lo = 0, hi = E_local - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tpre[mid] <= tile)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int e = __builtin_amdgcn_readfirstlane(lo);
    const int t0 = __builtin_amdgcn_readfirstlane(s_tpre[e]);
    const int seg0 = __builtin_amdgcn_readfirstlane(s_off[e]);
    const int m_e = __builtin_amdgcn_readfirstlane(s_off[e + 1]) - seg0;
    const int nrt = (m_e + row_cap - 1) / row_cap;
    const int local = tile - t0;
    const int nj = local / nrt;
    const int mi = local - nj * nrt;
    const int height = ((m_e + nrt - 1) / nrt + 15) & ~15;
    const int r0 = seg0 + mi * height;
    const int rows = min(height, seg0 + m_e - r0);
    if (rows <= 0) continue;
    const uint16_t* We = W + int64_t(e) * w_expert_stride;
    MOE_LDS int* const ri_buf = (MOE_LDS int*)s_ri + (FUSE ? 768 * parity : 0);
    parity ^= 1;
    auto col_of = [&](int s0) -> int {
      if (SWIGLU) {  // tile column s: wave column s/64, gate (s%64 < 32) or up of output o0 + 32*(s/64) + s%32
        const int q = s0 & 63;
        const int oc = nj * (kBN / 2) + (s0 >> 6) * 32 + (q & 31);
        if (oc >= N) return 0;
        return q < 32 ? oc : up_off + oc;
      } else {
        const int oc = nj * kBN + s0;
        return oc < N ? oc : 0;
      }
    };
    const int out_c0 = SWIGLU ? nj * (kBN / 2) : nj * kBN;
    const int fmt = (rows + 16 * kWR - 1) / (16 * kWR);
    if constexpr (FUSE) {
      // direct-to-LDS copy of the tile rows' info (bytes beyond the tile's
      // rows read as zero); issued before the tile's first stage, so the
      // tile's first stage wait covers it
      const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      if (w < 3) {
        const dma::i32x4 rs = dma::buffer_rsrc(row_info + r0, int64_t(rows) * 8);
        // the wave's offset goes in the per-lane offset, which the buffer's
        // range check covers (the scalar offset is not checked)
        dma::dma16(rs, 1024u * uint32_t(w) + 16u * uint32_t(lane_id()), 0u, (MOE_LDS char*)ri_buf + 1024 * w);
      }
    }
    auto go = [&](auto fm_t) {
      constexpr int FMT = decltype(fm_t)::value;
      if (gather_src != nullptr) {
        panelffn::run_tile<FMT, SWIGLU, FUSE, HALF>(lds, A, int64_t(gather_rows) * lda * 2, lda, rows,
                                              [&](int r) { return gather_src[r0 + r] / gather_k; }, We, ldw, K,
                                              col_of, out_c0, N, C, ldc, r0, (const MOE_LDS int*)ri_buf, y);
      } else {
        panelffn::run_tile<FMT, SWIGLU, FUSE, HALF>(lds, A + int64_t(r0) * lda, int64_t(rows) * lda * 2, lda, rows,
                                              [](int r) { return r; }, We, ldw, K, col_of, out_c0, N, C, ldc, r0,
                                              (const MOE_LDS int*)ri_buf, y);
      }
    };
    switch (fmt) {
      case 1: go(std::integral_constant<int, 1>{}); break;
      case 2: go(std::integral_constant<int, 2>{}); break;
      case 3: go(std::integral_constant<int, 3>{}); break;
      case 4: go(std::integral_constant<int, 4>{}); break;
      case 5: go(std::integral_constant<int, 5>{}); break;
      case 6: go(std::integral_constant<int, 6>{}); break;
      case 7: go(std::integral_constant<int, 7>{}); break;
      case 8: go(std::integral_constant<int, 8>{}); break;
      default: go(std::integral_constant<int, 9>{}); break;
    }
  }
}

namespace {
constexpr int kFfnBM = 128;
unsigned persistent_grid(int64_t tiles) {
  return unsigned(std::max<int64_t>(1, std::min<int64_t>(tiles, int64_t(device_cu_count()))));
}
}  // namespace

unsigned dma_grid(int64_t tiles) {
  // a multiple of the 8 XCDs, at most one workgroup per CU
  const int64_t cus = device_cu_count() / 8 * 8;
  const int64_t want = std::max<int64_t>(8, std::min<int64_t>(cus, (tiles + 7) / 8 * 8));
  return unsigned(want);
}

// The panel kernel for k extent K (HALF when K ends in half a 64-deep stage).
template <bool SWIGLU, bool FUSE>
hipError_t launch_panel(int64_t tiles, hipStream_t stream, const uint16_t* A, int lda, const int32_t* offsets,
                        int E_local, int64_t capacity, const uint16_t* W, int64_t w_expert_stride, int ldw,
                        uint16_t* C, int ldc, int K, int N, int up_off, const int32_t* gather_src, int gather_k,
                        int gather_rows, const int2* row_info, uint16_t* y, int64_t rows_hint) {
  // With few rows per expert expected, the grouped GEMV takes every expert.
  if (grouped_gemv_usable(rows_hint, K, N, E_local, SWIGLU))
    return SWIGLU ? launch_grouped_gemv1(A, lda, gather_src, gather_k, gather_rows, offsets, E_local, capacity, W, K,
                                         N, C, stream)
                  : launch_grouped_gemv2(A, offsets, E_local, capacity, W, N, K, row_info, C, y, stream);
  // the kernel indexes tiles with 31 bits; at the largest row cap the count
  // must fit (smaller caps are taken only where theirs fits too)
  const int64_t ntn = SWIGLU ? ceil_div(N, dma::panel::kBN / 2) : ceil_div(N, dma::panel::kBN);
  if ((ceil_div(capacity, 288) + E_local) * ntn >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const bool half = K % dma::panel::kSK != 0;
  auto* kern = half ? panel_gemm_kernel<SWIGLU, FUSE, true> : panel_gemm_kernel<SWIGLU, FUSE, false>;
  hipLaunchKernelGGL(kern, dim3(dma_grid(tiles)), dim3(dma::kThreads), 0, stream, A, lda, offsets, E_local, capacity,
                     W, w_expert_stride, ldw, C, ldc, K, N, up_off, gather_src, gather_k, gather_rows, row_info, y);
  return hipGetLastError();
}

hipError_t launch_expert_gemm1(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_gate_up, int H,
                               int I, int E_local, int64_t capacity, uint16_t* h, hipStream_t stream,
                               int64_t rows_hint) {
  if (H % dma::kBK == 0) {
    const int64_t tiles = (ceil_div(capacity, kRowCapMin) + E_local) * ceil_div(I, dma::panel::kBN / 2);
    return launch_panel<true, false>(tiles, stream, x_perm, H, offsets, E_local, capacity, w_gate_up,
                                     int64_t(H) * 2 * I, 2 * I, h, I, H, I, I, nullptr, 1, 0, nullptr, nullptr,
                                     rows_hint);
  }
  const int64_t mt_bound = ceil_div(capacity, kFfnBM) + E_local;
  const unsigned grid = persistent_grid(mt_bound * ceil_div(I, 128));
  hipLaunchKernelGGL((grouped_gemm_kernel<kFfnBM, true>), dim3(grid), dim3(kThreads), 0, stream, x_perm, H, offsets,
                     E_local, capacity, w_gate_up, int64_t(H) * 2 * I, 2 * I, h, I, H, I, I);
  return hipGetLastError();
}

hipError_t launch_expert_gemm2(const uint16_t* h, const int32_t* offsets, const uint16_t* w_down, int H, int I,
                               int E_local, int64_t capacity, uint16_t* out, hipStream_t stream, int64_t rows_hint) {
  if (I % dma::kBK == 0) {
    const int64_t tiles = (ceil_div(capacity, kRowCapMin) + E_local) * ceil_div(H, dma::panel::kBN);
    return launch_panel<false, false>(tiles, stream, h, I, offsets, E_local, capacity, w_down, int64_t(I) * H, H,
                                      out, H, I, H, 0, nullptr, 1, 0, nullptr, nullptr, rows_hint);
  }
  const int64_t mt_bound = ceil_div(capacity, kFfnBM) + E_local;
  const unsigned grid = persistent_grid(mt_bound * ceil_div(H, 256));
  hipLaunchKernelGGL((grouped_gemm_kernel<kFfnBM, false>), dim3(grid), dim3(kThreads), 0, stream, h, I, offsets,
                     E_local, capacity, w_down, int64_t(I) * H, H, out, H, I, H, 0);
  return hipGetLastError();
}

bool expert_gemm2_can_fuse(int I) { return I % dma::kBK == 0; }

hipError_t launch_expert_gemm2_fused(const uint16_t* h, const int32_t* offsets, const uint16_t* w_down, int H, int I,
                                     int E_local, int64_t capacity, const int2* row_info, uint16_t* out, uint16_t* y,
                                     hipStream_t stream, int64_t rows_hint) {
  const int64_t tiles = (ceil_div(capacity, kRowCapMin) + E_local) * ceil_div(H, dma::panel::kBN);
  return launch_panel<false, true>(tiles, stream, h, I, offsets, E_local, capacity, w_down, int64_t(I) * H, H, out,
                                   H, I, H, 0, nullptr, 1, 0, row_info, y, rows_hint);
}

bool expert_gemm1_can_gather(int T, int H) { return H % dma::kBK == 0 && int64_t(T) * H * 2 < (int64_t(1) << 31); }

hipError_t launch_expert_gemm1_gather(const uint16_t* x, const int32_t* perm_src, int T, int k, const int32_t* offsets,
                                      const uint16_t* w_gate_up, int H, int I, int E_local, int64_t capacity,
                                      uint16_t* h, hipStream_t stream, int64_t rows_hint) {
  const int64_t tiles = (ceil_div(capacity, kRowCapMin) + E_local) * ceil_div(I, dma::panel::kBN / 2);
  return launch_panel<true, false>(tiles, stream, x, H, offsets, E_local, capacity, w_gate_up, int64_t(H) * 2 * I,
                                   2 * I, h, I, H, I, I, perm_src, k, T, nullptr, nullptr, rows_hint);
}

hipError_t launch_expert_ffn(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_gate_up,
                             const uint16_t* w_down, int H, int I, int E_local, int64_t capacity, uint16_t* h,
                             uint16_t* out, hipStream_t stream) {
  // without the routing, the capacity spread over the local experts is the
  // expected row count
  const int64_t rows_hint = ceil_div(capacity, E_local);
  hipError_t err = launch_expert_gemm1(x_perm, offsets, w_gate_up, H, I, E_local, capacity, h, stream, rows_hint);
  if (err != hipSuccess) return err;
  return launch_expert_gemm2(h, offsets, w_down, H, I, E_local, capacity, out, stream, rows_hint);
}

}  // namespace moe
