// Combine: weighted sum of a token's expert outputs, written at the token's
// original position.
//
// At the source the results of the selected experts are summed with the
// combine weights, e.g. y(A2) = 0.7 u0 + 0.3 u2 ("EP: Partition Experts and
// Route Tokens", "Return multiple expert results to the same token"), and the
// outputs return in input order. A token whose experts all live on other
// ranks gets zeros, so the ranks' outputs add up to the full layer ("Expert
// Parallelism (EP)", "Why a Single All-Reduce/Reduce-Scatter Works").
//
// One wave per token (per column block of the token's row when there are few
// tokens); the sum runs in float32 over the slots in order and is
// rounded to bf16 once, or stored as float32 as it stands (the partial-output
// form: the shares of all ranks are summed afterwards, and a float32 share is
// not rounded before that sum). The expert rows are read with non-temporal
// loads: each is read exactly once, so it should not evict other data from the
// caches.
#include "gemm_tile.h"
#include "moe_kernels.h"

namespace moe {

template <int KMAX, bool F32, bool SKIP1>
__global__ void __launch_bounds__(kThreads)
combine_kernel(const uint16_t* __restrict__ expert_out, const int32_t* __restrict__ inv,
               const float* __restrict__ topk_w, int T, int H, int k, int vpb, void* __restrict__ y) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const int d = lane < k ? inv[int64_t(t) * k + lane] : -1;
  const float wl = lane < k ? topk_w[int64_t(t) * k + lane] : 0.f;
  const uint64_t dests = ballot(d >= 0);
  // Local slots in slot order, broadcast to every lane.
  int rows[KMAX];
  float wts[KMAX];
  int nl = 0;
  {
    uint64_t mm = dests;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      rows[j] = 0;
      wts[j] = 0.f;
      if (mm) {
        const int s = __ffsll((unsigned long long)mm) - 1;
        mm &= mm - 1;
        rows[j] = shfl(d, s);
        wts[j] = shfl(wl, s);
        ++nl;
      }
    }
  }
  // With SKIP1 the down GEMM's epilogue already wrote tokens with exactly
  // one local slot.
  if (SKIP1 && nl == 1) return;
  // Start from -0 so that a single term passes through bit for bit (-0 + -0 = -0);
  // a token with no local slot is written as +0.
  const float init = nl > 0 ? -0.f : 0.f;
  if constexpr (F32) {
    // 4 values per lane and vector, so each store instruction covers one
    // contiguous 1 KiB span of y; the stores are non-temporal (y is twice the
    // bytes of the bf16 form and is not read again here). With bf16 output,
    // non-temporal stores measured slower, so that path keeps plain ones.
    const int nv = min(H / 4, 2 * vpb * int(blockIdx.y + 1));
    f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(y) + int64_t(t) * H);
    constexpr int U = 4;
    for (int v0 = 2 * vpb * blockIdx.y + lane; v0 < nv; v0 += 64 * U) {
      u32x2 q[KMAX][U];
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (j < nl && v0 + 64 * u < nv)
            q[j][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(expert_out + int64_t(rows[j]) * H) + v0 + 64 * u);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (v0 + 64 * u >= nv) break;
        float acc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = init;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (j < nl) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              acc[2 * i] = fmaf(wts[j], bf16_lo(q[j][u][i]), acc[2 * i]);
              acc[2 * i + 1] = fmaf(wts[j], bf16_hi(q[j][u][i]), acc[2 * i + 1]);
            }
          }
        }
        __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, dst + v0 + 64 * u);
      }
    }
    return;
  }
  const int nv = min(H / 8, vpb * int(blockIdx.y + 1));
  u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + int64_t(t) * H);
  // U vectors per lane per pass; all of a pass's loads are issued before the
  // first one is used, so each lane keeps up to U * nl loads in flight.
  constexpr int U = 2;
  for (int v0 = vpb * blockIdx.y + lane; v0 < nv; v0 += 64 * U) {
    u32x4 q[KMAX][U];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (j < nl && v0 + 64 * u < nv)
          q[j][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(expert_out + int64_t(rows[j]) * H) + v0 + 64 * u);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (v0 + 64 * u >= nv) break;
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = init;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < nl) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(wts[j], bf16_lo(q[j][u][i]), acc[2 * i]);
            acc[2 * i + 1] = fmaf(wts[j], bf16_hi(q[j][u][i]), acc[2 * i + 1]);
          }
        }
      }
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
      dst[v0 + 64 * u] = o;
    }
  }
}

template <bool F32, bool SKIP1>
static void launch_combine_t(const uint16_t* expert_out, const int32_t* inv, const float* topk_w, int T, int H,
                             int k, void* y, hipStream_t stream) {
  // Few tokens: each token's row is cut into column blocks (blockIdx.y) of
  // vpb 8-column vectors (a multiple of 64), so that about 4096 waves run;
  // with many tokens one wave takes a whole row.
  const int nv = H / 8;
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>(ceil_div(4096, T), ceil_div(nv, 128)));
  const int vpb = int(ceil_div(ceil_div(nv, want), 64) * 64);
  const dim3 grid(unsigned(ceil_div(T, 4)), unsigned(ceil_div(nv, vpb)));
#define MOE_COMBINE_LAUNCH(KM)                                                                                     \
  hipLaunchKernelGGL((combine_kernel<KM, F32, SKIP1>), grid, dim3(kThreads), 0, stream, expert_out, inv, topk_w, T, H, k, \
                     vpb, y)
  if (k <= 1)
    MOE_COMBINE_LAUNCH(1);
  else if (k <= 2)
    MOE_COMBINE_LAUNCH(2);
  else if (k <= 4)
    MOE_COMBINE_LAUNCH(4);
  else if (k <= 8)
    MOE_COMBINE_LAUNCH(8);
  else if (k <= 16)
    MOE_COMBINE_LAUNCH(16);
  else
    MOE_COMBINE_LAUNCH(32);
#undef MOE_COMBINE_LAUNCH
}

hipError_t launch_combine(const uint16_t* expert_out, const int32_t* inv, const float* topk_w, int T, int H, int k,
                          void* y, bool y_f32, hipStream_t stream, bool skip_single) {
  if (y_f32)
    launch_combine_t<true, false>(expert_out, inv, topk_w, T, H, k, y, stream);
  else if (skip_single)
    launch_combine_t<false, true>(expert_out, inv, topk_w, T, H, k, y, stream);
  else
    launch_combine_t<false, false>(expert_out, inv, topk_w, T, H, k, y, stream);
  return hipGetLastError();
}

// For the combine fused into the down GEMM: one thread per token counts its
// local slots; the row of a token with exactly one gets {token, weight bits},
// every other local row {-1, 0}. Every local row is written once.
__global__ void __launch_bounds__(kThreads)
single_rows_kernel(const int32_t* __restrict__ inv, const float* __restrict__ topk_w, int T, int k,
                   int2* __restrict__ row_info) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= T) return;
  const int32_t* d = inv + int64_t(t) * k;
  int nl = 0, js = 0;
  for (int j = 0; j < k; ++j)
    if (d[j] >= 0) {
      ++nl;
      js = j;
    }
  if (nl == 1) {
    row_info[d[js]] = make_int2(t, __float_as_int(topk_w[int64_t(t) * k + js]));
  } else {
    for (int j = 0; j < k; ++j)
      if (d[j] >= 0) row_info[d[j]] = make_int2(-1, 0);
  }
}

hipError_t launch_single_rows(const int32_t* inv, const float* topk_w, int T, int k, int2* row_info,
                              hipStream_t stream) {
  hipLaunchKernelGGL(single_rows_kernel, dim3(unsigned(ceil_div(T, kThreads))), dim3(kThreads), 0, stream, inv,
                     topk_w, T, k, row_info);
  return hipGetLastError();
}

}  // namespace moe
