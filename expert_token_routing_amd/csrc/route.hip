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
#include "gemm_tile.h"
#include "moe_kernels.h"

namespace moe {

// w (float32) -> hi, mid, lo (bf16 planes of n elements each), hi+mid+lo == w.
__global__ void route_split_kernel(const float* __restrict__ w, uint16_t* __restrict__ planes, int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float x = w[i];
    const uint32_t hi = __float_as_uint(x) >> 16;
    const float r1 = x - __uint_as_float(hi << 16);
    const uint32_t mid = __float_as_uint(r1) >> 16;
    const float r2 = r1 - __uint_as_float(mid << 16);
    const uint32_t lo = __float_as_uint(r2) >> 16;
    planes[i] = uint16_t(hi);
    planes[n + i] = uint16_t(mid);
    planes[2 * n + i] = uint16_t(lo);
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

// One wave per token: top-k by (logit descending, expert id ascending), then
// softmax weights. Lane l holds experts l, l+64, ... (EPL per lane).
template <int EPL>
__global__ void __launch_bounds__(kThreads)
route_topk_kernel(const float* __restrict__ logits, int T, int E, int k, int renormalize,
                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + int64_t(t) * E;
  float v[EPL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -INFINITY;
    m = fmaxf(m, v[i]);
  }
  m = wave_max(m);

  float den_all = 0.f;
  if (!renormalize) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + 64 * i < E) s += expf(v[i] - m);
    den_all = wave_sum(s);
  }

  uint32_t taken = 0;
  int my_e = 0;
  float my_v = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      const bool ok = e < E && !((taken >> i) & 1u);
      if (ok && (v[i] > bv || (v[i] == bv && e < be))) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
      const float ov = shfl_xor(bv, s);
      const int oe = shfl_xor(be, s);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if (lane == (be & 63)) taken |= 1u << (be >> 6);
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
hipError_t launch_route(const uint16_t* x, const float* w_router, const float* bias, int T, int H, int E, int k,
                        int renormalize, float* logits, int32_t* topk_idx, float* topk_w, uint16_t* planes,
                        hipStream_t stream) {
  const int64_t n = int64_t(E) * H;
  {
    const int threads = 256;
    const int64_t blocks = std::min<int64_t>((n + threads - 1) / threads, 4096);
    hipLaunchKernelGGL(route_split_kernel, dim3(unsigned(blocks)), dim3(threads), 0, stream, w_router, planes, n);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  {
    dim3 grid(unsigned((T + 127) / 128), unsigned((E + 127) / 128));
    hipLaunchKernelGGL(route_logits_kernel, grid, dim3(kThreads), 0, stream, x, planes, bias, logits, T, H, E);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  {
    dim3 grid(unsigned((T + 3) / 4));
    const int epl = (E + 63) / 64;
    if (epl <= 1)
      hipLaunchKernelGGL(route_topk_kernel<1>, grid, dim3(kThreads), 0, stream, logits, T, E, k, renormalize, topk_idx, topk_w);
    else if (epl <= 2)
      hipLaunchKernelGGL(route_topk_kernel<2>, grid, dim3(kThreads), 0, stream, logits, T, E, k, renormalize, topk_idx, topk_w);
    else if (epl <= 4)
      hipLaunchKernelGGL(route_topk_kernel<4>, grid, dim3(kThreads), 0, stream, logits, T, E, k, renormalize, topk_idx, topk_w);
    else if (epl <= 8)
      hipLaunchKernelGGL(route_topk_kernel<8>, grid, dim3(kThreads), 0, stream, logits, T, E, k, renormalize, topk_idx, topk_w);
    else
      hipLaunchKernelGGL(route_topk_kernel<16>, grid, dim3(kThreads), 0, stream, logits, T, E, k, renormalize, topk_idx, topk_w);
    return hipGetLastError();
  }
}

}  // namespace moe
