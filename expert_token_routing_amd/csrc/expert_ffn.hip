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
// `offsets` (m-tiles of BM rows per segment x n-tiles) and strides over it.
// Weights are n-contiguous in memory and are transposed 8 x 8 in registers on
// their way to LDS, so both MFMA operands are read k-contiguous from LDS.
#include "gemm_dma.h"
#include "gemm_tile.h"
#include "moe_kernels.h"

namespace moe {

constexpr int kMaxLocal = 1024;

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

// Same computation with a deeper memory pipeline, for k a multiple of 32:
// direct global->LDS loads into a ring of stages (three in flight while one is
// multiplied), B read from LDS with transposing reads instead of a register
// transpose, and the LDS reads of the next 16-deep step interleaved with the
// MFMAs of the current one. Tiles go to XCDs in contiguous expert-major
// ranges (workgroup b runs on XCD b % 8), so the workgroups sharing an
// expert's weight and row panels share one L2.
namespace dmaffn {

// One output tile: rows [r0, r0 + rows) of A (rows <= FM*64), 256 columns of
// the expert's weight (n-tile nj). LOAD_BM rows are brought into LDS (rows past
// the end repeat the last one); the 8 waves, 2 x 4, multiply FM*32 x 64 each.
template <int LOAD_BM, int FM, bool SWIGLU>
__device__ __forceinline__ void run_tile(MOE_LDS char* lds, const uint16_t* __restrict__ A, int lda, int r0,
                                         int rows, const uint16_t* __restrict__ We, int ldw, int K, int N,
                                         int up_off, int nj, uint16_t* __restrict__ C, int ldc,
                                         const int32_t* __restrict__ gather_src, int gather_k, int gather_rows) {
  using namespace dma;
  constexpr int FN = 2;
  constexpr int kAStage = LOAD_BM * kARowBytes;
  constexpr int kStage = kAStage + kBStageBytes;
  constexpr int kLoads = ALoader<LOAD_BM>::kPer + BLoader::kPer;  // DMA instructions per thread per stage
  static_assert(dma::kBK == 32, "two 16-deep steps per stage");
  const int w = threadIdx.x >> 6, wm = w >> 2, wn = w & 3;
  const int lane = lane_id();
  const int nk = K / dma::kBK;

  auto col_of = [&](int s0) -> int {
    if (SWIGLU) {  // wave wn's 64 columns: 32 gate then the matching 32 up
      const int q = s0 & 63;
      const int oc = nj * 128 + (s0 >> 6) * 32 + (q & 31);
      if (oc >= N) return 0;
      return q < 32 ? oc : up_off + oc;
    } else {
      const int oc = nj * 256 + s0;
      return oc < N ? oc : 0;
    }
  };

  f32x16 acc[FM][FN];
  zero_acc(acc);
  ALoader<LOAD_BM> la;
  BLoader lb;
  if (gather_src != nullptr)  // A rows are token vectors: row r0+r is token src[r0+r] / k
    la.init_gather(A, lda, gather_rows, rows, [&](int r) { return gather_src[r0 + r] / gather_k; });
  else
    la.init(A + int64_t(r0) * lda, lda, rows);
  lb.init(We, ldw, K, col_of);
  // ring of kStages buffers: stages kt+1 .. kt+kStages-1 in flight while
  // stage kt is multiplied
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p)
    if (p < nk) {
      la.issue(lds + p * kStage, p * dma::kBK);
      lb.issue(lds + p * kStage + kAStage, p * dma::kBK);
    }
  FragAddr fa;
  fa.init(wm * FM * 32, wn * 64);
  Frags<FM, FN> f0, f1;
  {  // stage 0 landed (stages 1 and 2 may be in flight)
    const int ahead0 = min(kStages - 2, nk - 1);
    if (ahead0 >= 2)
      wait_vm_barrier<2 * kLoads>();
    else if (ahead0 == 1)
      wait_vm_barrier<kLoads>();
    else
      wait_vm_barrier<0>();
  }
  load_frags<FM, FN>(lds, lds + kAStage, fa, 0, f0);
  for (int kt = 0; kt < nk; ++kt) {
    MOE_LDS char* cur = lds + (kt % kStages) * kStage;
    // refill the buffer of stage kt-1 (every wave is past it) with stage kt+3
    if (kt + kStages - 1 < nk) {
      MOE_LDS char* nxt = lds + ((kt + kStages - 1) % kStages) * kStage;
      la.issue(nxt, (kt + kStages - 1) * dma::kBK);
      lb.issue(nxt + kAStage, (kt + kStages - 1) * dma::kBK);
    }
    // second step's fragments stream in under the first step's MFMAs
    load_frags<FM, FN>(cur, cur + kAStage, fa, 1, f1);
    mma_frags<FM, FN>(f0, acc);
    interleave_mfma_with_reads<FM, FN>();
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) {
      // stage kt+1 landed (its successors may be in flight); all LDS reads of
      // this wave returned before the barrier, so no buffer is refilled early
      wait_lgkm0();
      const int ahead = min(kStages - 2, nk - 2 - kt);
      if (ahead >= 2)
        wait_vm_barrier<2 * kLoads>();
      else if (ahead == 1)
        wait_vm_barrier<kLoads>();
      else
        wait_vm_barrier<0>();
    }
    // next stage's first step streams in under this stage's second step (after
    // the last stage this reads a finished buffer; the values are not used)
    MOE_LDS char* nx = lds + ((kt + 1) % kStages) * kStage;
    load_frags<FM, FN>(nx, nx + kAStage, fa, 0, f0);
    mma_frags<FM, FN>(f1, acc);
    interleave_mfma_with_reads<FM, FN>();
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_lds_barrier();

  if (SWIGLU) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      __builtin_amdgcn_sched_barrier(0);
      const int col = nj * 128 + wn * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * FM * 32 + fm * 32 + mfma_c_row(v, lane);
        if (row < rows && col < N) {
          const float g = acc[fm][0][v];
          const float u = acc[fm][1][v];
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
        __builtin_amdgcn_sched_barrier(0);
        const int col = nj * 256 + wn * 64 + fn * 32 + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * FM * 32 + fm * 32 + mfma_c_row(v, lane);
          if (row < rows && col < N) C[int64_t(r0 + row) * ldc + col] = uint16_t(f32_to_bf16_bits(acc[fm][fn][v]));
        }
      }
  }
}

}  // namespace dmaffn

template <bool SWIGLU>
__global__ void __launch_bounds__(dma::kThreads)
grouped_gemm_dma_kernel(const uint16_t* __restrict__ A, int lda, const int32_t* __restrict__ offsets, int E_local,
                        int64_t capacity, const uint16_t* __restrict__ W, int64_t w_expert_stride, int ldw,
                        uint16_t* __restrict__ C, int ldc, int K, int N, int up_off,
                        const int32_t* __restrict__ gather_src, int gather_k, int gather_rows) {
  using namespace dma;
  __shared__ __attribute__((aligned(1024))) char smem[kStages * (256 * kARowBytes + kBStageBytes)];
  __shared__ int s_off[kMaxLocal + 1];
  __shared__ int s_tpre[kMaxLocal + 1];
  __shared__ int s_tmp[kWaves];
  MOE_LDS char* lds = (MOE_LDS char*)smem;

  const int ntn = SWIGLU ? (N + 127) / 128 : (N + 255) / 256;
  // Tiles of expert i: ceil(M_i / 256) row tiles x ntn n-tiles, ordered
  // n-major so that the row tiles sharing one weight panel are adjacent (and
  // run together).
  constexpr int kPerT = (kMaxLocal + dma::kThreads - 1) / dma::kThreads;
  int mt[kPerT];
  int sum = 0;
#pragma unroll
  for (int q = 0; q < kPerT; ++q) {
    const int i = threadIdx.x * kPerT + q;
    mt[q] = 0;
    if (i < E_local) {
      const int64_t a = min<int64_t>(max<int64_t>(offsets[i], 0), capacity);
      const int64_t b = max<int64_t>(a, min<int64_t>(offsets[i + 1], capacity));
      s_off[i] = int(a);
      mt[q] = int((b - a + 255) / 256) * ntn;
      if (i == E_local - 1) s_off[E_local] = int(b);
    }
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

  // This XCD's contiguous range of the tile list, dealt round robin to its
  // workgroups: tiles of equal cost keep the workgroups in step, so the tiles
  // sharing a panel stream it through the XCD's L2 together.
  const int nxcd = 8;
  const int xcd = blockIdx.x % nxcd;
  const int per_xcd = gridDim.x / nxcd;
  const int lo_t = int((int64_t(total) * xcd) / nxcd);
  const int hi_t = int((int64_t(total) * (xcd + 1)) / nxcd);
  for (int tile = lo_t + int(blockIdx.x / nxcd); tile < hi_t; tile += per_xcd) {
    int lo = 0, hi = E_local - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tpre[mid] <= tile)
        lo = mid;
      else
        hi = mid - 1;
    }
    // per-tile values are uniform across the workgroup
    const int e = __builtin_amdgcn_readfirstlane(lo);
    const int t0 = __builtin_amdgcn_readfirstlane(s_tpre[e]);
    const int local = tile - t0;
    const int mte = (__builtin_amdgcn_readfirstlane(s_tpre[e + 1]) - t0) / ntn;
    const int nj = local / mte;
    const int mi = local - nj * mte;
    const int seg0 = __builtin_amdgcn_readfirstlane(s_off[e]);
    const int r0 = seg0 + mi * 256;
    const int rows = min(256, __builtin_amdgcn_readfirstlane(s_off[e + 1]) - r0);
    dmaffn::run_tile<256, 4, SWIGLU>(lds, A, lda, r0, rows, W + int64_t(e) * w_expert_stride, ldw, K, N, up_off, nj,
                                      C, ldc, gather_src, gather_k, gather_rows);
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

hipError_t launch_expert_gemm1(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_gate_up, int H,
                               int I, int E_local, int64_t capacity, uint16_t* h, hipStream_t stream) {
  if (H % dma::kBK == 0) {
    const int64_t tiles = (ceil_div(capacity, 256) + 2 * E_local) * ceil_div(I, 128);
    hipLaunchKernelGGL((grouped_gemm_dma_kernel<true>), dim3(dma_grid(tiles)), dim3(dma::kThreads), 0, stream,
                       x_perm, H, offsets, E_local, capacity, w_gate_up, int64_t(H) * 2 * I, 2 * I, h, I, H, I, I,
                       nullptr, 1, 0);
    return hipGetLastError();
  }
  const int64_t mt_bound = ceil_div(capacity, kFfnBM) + E_local;
  const unsigned grid = persistent_grid(mt_bound * ceil_div(I, 128));
  hipLaunchKernelGGL((grouped_gemm_kernel<kFfnBM, true>), dim3(grid), dim3(kThreads), 0, stream, x_perm, H, offsets,
                     E_local, capacity, w_gate_up, int64_t(H) * 2 * I, 2 * I, h, I, H, I, I);
  return hipGetLastError();
}

hipError_t launch_expert_gemm2(const uint16_t* h, const int32_t* offsets, const uint16_t* w_down, int H, int I,
                               int E_local, int64_t capacity, uint16_t* out, hipStream_t stream) {
  if (I % dma::kBK == 0) {
    const int64_t tiles = (ceil_div(capacity, 256) + 2 * E_local) * ceil_div(H, 256);
    hipLaunchKernelGGL((grouped_gemm_dma_kernel<false>), dim3(dma_grid(tiles)), dim3(dma::kThreads), 0,
                       stream, h, I, offsets, E_local, capacity, w_down, int64_t(I) * H, H, out, H, I, H, 0, nullptr, 1,
                       0);
    return hipGetLastError();
  }
  const int64_t mt_bound = ceil_div(capacity, kFfnBM) + E_local;
  const unsigned grid = persistent_grid(mt_bound * ceil_div(H, 256));
  hipLaunchKernelGGL((grouped_gemm_kernel<kFfnBM, false>), dim3(grid), dim3(kThreads), 0, stream, h, I, offsets,
                     E_local, capacity, w_down, int64_t(I) * H, H, out, H, I, H, 0);
  return hipGetLastError();
}

bool expert_gemm1_can_gather(int T, int H) { return H % dma::kBK == 0 && int64_t(T) * H * 2 < (int64_t(1) << 31); }

hipError_t launch_expert_gemm1_gather(const uint16_t* x, const int32_t* perm_src, int T, int k, const int32_t* offsets,
                                      const uint16_t* w_gate_up, int H, int I, int E_local, int64_t capacity,
                                      uint16_t* h, hipStream_t stream) {
  const int64_t tiles = (ceil_div(capacity, 256) + 2 * E_local) * ceil_div(I, 128);
  hipLaunchKernelGGL((grouped_gemm_dma_kernel<true>), dim3(dma_grid(tiles)), dim3(dma::kThreads), 0, stream, x, H,
                     offsets, E_local, capacity, w_gate_up, int64_t(H) * 2 * I, 2 * I, h, I, H, I, I, perm_src, k, T);
  return hipGetLastError();
}

hipError_t launch_expert_ffn(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_gate_up,
                             const uint16_t* w_down, int H, int I, int E_local, int64_t capacity, uint16_t* h,
                             uint16_t* out, hipStream_t stream) {
  hipError_t err = launch_expert_gemm1(x_perm, offsets, w_gate_up, H, I, E_local, capacity, h, stream);
  if (err != hipSuccess) return err;
  return launch_expert_gemm2(h, offsets, w_down, H, I, E_local, capacity, out, stream);
}

}  // namespace moe
