// Dispatch: group the rank's (token, slot) selections by expert.
//
// Token vectors, not weights and not router scores, move to the selected
// experts, and each expert's rows are stacked so one matmul serves them
// ("EP: Partition Experts and Route Tokens", section "Send tokens to experts
// and return their results"); counting every expert's selections gives the
// per-expert load that "Equal expert counts can receive different token
// counts" is about. The rank keeps only its contiguous expert block
// [e0, e0 + E_local) ("Expert Parallelism (EP)", "Limitations").
//
// Row order is deterministic: segment of expert e0+i first by i, inside a
// segment by token. Up to 2048 tokens (1024 when the rows are copied too),
// one workgroup builds every table in one launch (dispatch_small_kernel);
// above that, four kernels (three when the rows are copied: placement then
// happens in the copy kernel), no host synchronisation:
//   1. histogram: one wave per chunk of 64 tokens counts its selections of
//      every expert with LDS atomics -> chunk_table[e][chunk];
//   2. scan: one workgroup per expert turns its row of chunk_table into
//      exclusive prefixes and writes counts[e];
//   3. index: one wave per chunk gives every local selection its row
//      (segment start + chunk prefix + rank among earlier lanes that picked
//      the same expert, a popcount of the 64-bit set of lanes that picked
//      it) and fills perm_src and inv;
//   4. copy: one wave per token reads the token vector once and writes it to
//      each of its rows, with non-temporal stores (the rows are not read
//      again soon, so they should not evict other data from the caches).
#include "gemm_tile.h"
#include "moe_kernels.h"

namespace moe {

// With mask_table, also stores for chunk c and local expert i the 64-bit set
// of the chunk's lanes (tokens) that picked it, at mask_table[c E_local + i].
__global__ void __launch_bounds__(kThreads)
dispatch_hist_kernel(const int32_t* __restrict__ topk_idx, int T, int E, int k, int nchunks,
                     int32_t* __restrict__ chunk_table, int e0, int E_local,
                     unsigned long long* __restrict__ mask_table) {
  extern __shared__ int s_hist[];  // 4 waves x E
  __shared__ unsigned long long s_mask[4][1024];
  const int w = threadIdx.x >> 6;
  const int lane = lane_id();
  int* hist = s_hist + w * E;
  for (int e = lane; e < E; e += 64) hist[e] = 0;
  if (mask_table != nullptr)
    for (int i = lane; i < E_local; i += 64) s_mask[w][i] = 0ull;
  __syncthreads();
  const int c = blockIdx.x * 4 + w;
  const int t = c * kChunk + lane;
  if (c < nchunks && t < T) {
    const int32_t* sel = topk_idx + int64_t(t) * k;
    for (int j = 0; j < k; ++j) {
      const int e = sel[j];
      atomicAdd(&hist[e], 1);
      if (mask_table != nullptr && e >= e0 && e < e0 + E_local) atomicOr(&s_mask[w][e - e0], 1ull << lane);
    }
  }
  __syncthreads();
  if (c < nchunks) {
    for (int e = lane; e < E; e += 64) chunk_table[int64_t(e) * nchunks + c] = hist[e];
    if (mask_table != nullptr)
      for (int i = lane; i < E_local; i += 64) mask_table[int64_t(c) * E_local + i] = s_mask[w][i];
  }
}

__global__ void __launch_bounds__(kThreads)
dispatch_scan_kernel(int32_t* __restrict__ chunk_table, int nchunks, int32_t* __restrict__ counts) {
  __shared__ int s_tmp[4];
  const int e = blockIdx.x;
  int32_t* row = chunk_table + int64_t(e) * nchunks;
  int carry = 0;
  for (int base = 0; base < nchunks; base += kThreads) {
    const int i = base + threadIdx.x;
    const int v = i < nchunks ? row[i] : 0;
    int tot;
    const int pre = block_exclusive_scan(v, s_tmp, tot);
    if (i < nchunks) row[i] = carry + pre;
    carry += tot;
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

// Gives every local selection of this wave's 64 tokens its row: segment
// start seg[i] of local expert i, plus chunk_base(i) (the expert's selections
// in earlier chunks), plus the number of earlier lanes of this wave that
// picked the same expert. That count comes from mask[i], a 64-bit set of the
// lanes that picked local expert i (every lane ORs in its bit first), so all
// lanes place their selections at once. Non-local slots get inv = -1.
// mask must be zero for this wave's local experts on entry.
template <int KMAX, typename ChunkBase>
__device__ __forceinline__ void place_wave(const int (&ev)[KMAX], int k, bool valid, int t, int e0, int E_local,
                                           const int* seg, ChunkBase chunk_base, unsigned long long* mask,
                                           int32_t* __restrict__ perm_src, int32_t* __restrict__ inv) {
  const int lane = lane_id();
  const unsigned long long bit = 1ull << lane;
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j < k && valid && ev[j] >= e0 && ev[j] < e0 + E_local) atomicOr(&mask[ev[j] - e0], bit);
  __builtin_amdgcn_wave_barrier();
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k && valid) {
      const int e = ev[j];
      const int64_t slot = int64_t(t) * k + j;
      if (e >= e0 && e < e0 + E_local) {
        const int i = e - e0;
        const int row = seg[i] + chunk_base(i) + __popcll(mask[i] & lt);
        perm_src[row] = int32_t(slot);
        inv[slot] = row;
      } else {
        inv[slot] = -1;
      }
    }
  }
}

template <int KMAX>
__global__ void __launch_bounds__(kThreads)
dispatch_index_kernel(const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ chunk_base,
                      const int32_t* __restrict__ counts, int T, int k, int e0, int E_local, int nchunks,
                      int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src, int32_t* __restrict__ inv) {
  __shared__ int s_seg[1024 + 1];
  __shared__ int s_base[4][1024];
  __shared__ unsigned long long s_mask[4][1024];
  __shared__ int s_tmp[4];
  const int wv = threadIdx.x >> 6;
  const int c = blockIdx.x * 4 + wv;
  const int lane = lane_id();
  const int t = c * kChunk + lane;
  const bool valid = c < nchunks && t < T;
  // All independent global loads first, so that their latencies overlap:
  // this lane's selections, the local experts' counts (4 per thread), and this
  // chunk's offset inside every local segment (16 per lane at most).
  int ev[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) ev[j] = (j < k && valid) ? topk_idx[int64_t(t) * k + j] : -1;
  int cnt[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = threadIdx.x * 4 + q;
    cnt[q] = i < E_local ? counts[e0 + i] : 0;
  }
  int cb[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = lane + 64 * q;
    cb[q] = (c < nchunks && i < E_local) ? chunk_base[int64_t(e0 + i) * nchunks + c] : 0;
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = lane + 64 * q;
    if (i < E_local) {
      s_base[wv][i] = cb[q];
      s_mask[wv][i] = 0ull;
    }
  }
  // Segment starts: exclusive scan of the local experts' counts.
  int sum = cnt[0] + cnt[1] + cnt[2] + cnt[3];
  int tot;
  int pre = block_exclusive_scan(sum, s_tmp, tot);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = threadIdx.x * 4 + q;
    if (i < E_local) s_seg[i] = pre;
    pre += cnt[q];
  }
  if (threadIdx.x == 0) s_seg[E_local] = tot;
  __syncthreads();
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= E_local; i += kThreads) offsets[i] = s_seg[i];

  if (c >= nchunks) return;
  place_wave<KMAX>(ev, k, valid, t, e0, E_local, s_seg, [&](int i) { return s_base[wv][i]; }, s_mask[wv], perm_src,
                   inv);
}

// Whole dispatch table build in one workgroup, for T up to kSmallMaxTokens:
// one launch instead of three (for few tokens the three launches cost more
// than their work). First every selection is counted with LDS atomics
// (counts, and the local segment starts by a scan). Then the tokens go by in
// rounds of 16 chunks of 64, one chunk per wave: every lane ORs its bit into
// s_mask[w][i] for each local expert i it picked, and a selection's row is
// its segment start, plus the expert's selections in earlier rounds (s_run)
// and in earlier chunks of this round, plus the earlier lanes of its chunk
// that picked it (popcounts of those sets): the rows of the multi-kernel
// path, bit for bit. Two rounds at most: the tables of `small_top2` (T =
// 2048, top-2 of 8) take 10.5 us this way against 12.3 with three launches,
// while the GPT-OSS-20B share (T = 8192, top-4 of 32; eight rounds) took 46
// against 13.
constexpr int kSmallWaves = 16;
constexpr int kSmallTokens = kSmallWaves * kChunk;  // tokens per round
constexpr int kSmallMaxTokens = 2 * kSmallTokens;

template <int KMAX>
__global__ void __launch_bounds__(kSmallWaves * 64)
dispatch_small_kernel(const int32_t* __restrict__ topk_idx, int T, int E, int k, int e0, int E_local,
                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
                      int32_t* __restrict__ inv) {
  __shared__ unsigned long long s_mask[kSmallWaves][1024];  // lanes of chunk w that picked local expert i
  __shared__ int s_cnt[1024];
  __shared__ int s_seg[1024 + 1];
  __shared__ int s_run[1024];  // local expert i: its selections in earlier rounds
  __shared__ int s_tmp[kSmallWaves];
  constexpr int kBlock = kSmallWaves * 64;
  const int wv = threadIdx.x >> 6;
  const int lane = lane_id();
  for (int e = threadIdx.x; e < E; e += kBlock) s_cnt[e] = 0;
  for (int i = threadIdx.x; i < E_local; i += kBlock) s_run[i] = 0;
  __syncthreads();
  const int64_t nsel = int64_t(T) * k;
  for (int64_t s = threadIdx.x; s < nsel; s += kBlock) {
    const int e = topk_idx[s];
    if (unsigned(e) < unsigned(E)) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kBlock) counts[e] = s_cnt[e];
  const int c = int(threadIdx.x) < E_local ? s_cnt[e0 + threadIdx.x] : 0;
  int tot;
  const int pre = block_exclusive_scan<kBlock>(c, s_tmp, tot);
  if (int(threadIdx.x) < E_local) {
    s_seg[threadIdx.x] = pre;
    offsets[threadIdx.x] = pre;
  }
  if (threadIdx.x == 0) {
    s_seg[E_local] = tot;
    offsets[E_local] = tot;
  }
  const uint64_t lt = lanemask_lt();
  const unsigned long long bit = 1ull << lane;
  for (int r0 = 0; r0 < T; r0 += kSmallTokens) {
    const int t = r0 + wv * kChunk + lane;
    const bool valid = t < T;
    // (this wave's row only: its own LDS operations stay in order)
    for (int i = lane; i < E_local; i += 64) s_mask[wv][i] = 0ull;
    int ev[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) ev[j] = (j < k && valid) ? topk_idx[int64_t(t) * k + j] - e0 : -1;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k && valid && unsigned(ev[j]) < unsigned(E_local)) atomicOr(&s_mask[wv][ev[j]], bit);
    __syncthreads();  // every chunk's sets complete; s_seg and s_run written
    if (valid) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
          const int i = ev[j];
          const int64_t slot = int64_t(t) * k + j;
          if (unsigned(i) < unsigned(E_local)) {
            int row = s_seg[i] + s_run[i] + __popcll(s_mask[wv][i] & lt);
            for (int w = 0; w < wv; ++w) row += __popcll(s_mask[w][i]);
            perm_src[row] = int32_t(slot);
            inv[slot] = row;
          } else {
            inv[slot] = -1;
          }
        }
      }
    }
    __syncthreads();  // every placement read s_run and the sets
    for (int i = threadIdx.x; i < E_local; i += kBlock) {
      int add = 0;
      for (int w = 0; w < kSmallWaves; ++w) add += __popcll(s_mask[w][i]);
      s_run[i] += add;
    }
    __syncthreads();  // s_run updated before the next round's placements; sets free
  }
}

// One wave per token; U 16-byte chunks in flight per lane.
__global__ void __launch_bounds__(kThreads)
dispatch_copy_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ inv, int T, int H, int k,
                     uint16_t* __restrict__ x_perm) {
  constexpr int U = 4;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const int d = lane < k ? inv[int64_t(t) * k + lane] : -1;
  const uint64_t dests = ballot(d >= 0);
  if (dests == 0) return;
  const int nv = H / 8;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + int64_t(t) * H);
  for (int v0 = 0; v0 < nv; v0 += 64 * U) {
    u32x4 q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * 64 + lane;
      if (v < nv) q[u] = src[v];
    }
    uint64_t mm = dests;
    while (mm) {
      const int j = __ffsll((unsigned long long)mm) - 1;
      mm &= mm - 1;
      const int row = shfl(d, j);
      u32x4* dst = reinterpret_cast<u32x4*>(x_perm + int64_t(row) * H);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * 64 + lane;
        if (v < nv) __builtin_nontemporal_store(q[u], dst + v);
      }
    }
  }
}

// Row placement fused into the row copy (moe_dispatch with T above the
// one-workgroup size): one wave per token; the workgroup first scans the local
// experts' counts into segment starts, then lane j of a token's wave places
// slot j: row = segment start + the expert's selections in earlier chunks
// (the scanned chunk table) + the chunk's earlier lanes that picked it (a
// popcount of the stored lane set). Same rows as dispatch_index_kernel, one
// launch fewer; then the token vector is copied to each of its rows.
__global__ void __launch_bounds__(kThreads)
dispatch_place_copy_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ topk_idx,
                           const int32_t* __restrict__ chunk_base, const unsigned long long* __restrict__ mask_table,
                           const int32_t* __restrict__ counts, int T, int H, int k, int e0, int E_local, int nchunks,
                           int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src, int32_t* __restrict__ inv,
                           uint16_t* __restrict__ x_perm) {
  __shared__ int s_seg[1024 + 1];
  __shared__ int s_tmp[4];
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  // this lane's slot and its placement inputs, loaded before the scan
  int e = -1, base = 0;
  unsigned long long m = 0ull;
  if (t < T && lane < k) {
    e = topk_idx[int64_t(t) * k + lane];
    if (e >= e0 && e < e0 + E_local) {
      const int c = t / kChunk;
      base = chunk_base[int64_t(e) * nchunks + c];
      m = mask_table[int64_t(c) * E_local + (e - e0)];
    }
  }
  int cnt[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = threadIdx.x * 4 + q;
    cnt[q] = i < E_local ? counts[e0 + i] : 0;
  }
  int tot;
  int pre = block_exclusive_scan(cnt[0] + cnt[1] + cnt[2] + cnt[3], s_tmp, tot);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = threadIdx.x * 4 + q;
    if (i < E_local) s_seg[i] = pre;
    pre += cnt[q];
  }
  if (threadIdx.x == 0) s_seg[E_local] = tot;
  __syncthreads();
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= E_local; i += kThreads) offsets[i] = s_seg[i];
  if (t >= T) return;
  int d = -1;
  if (lane < k) {
    if (e >= e0 && e < e0 + E_local) {
      d = s_seg[e - e0] + base + __popcll(m & ((1ull << (t % kChunk)) - 1ull));
      perm_src[d] = int32_t(int64_t(t) * k + lane);
    }
    inv[int64_t(t) * k + lane] = d;
  }
  const uint64_t dests = ballot(d >= 0);
  if (dests == 0) return;
  // 16 vectors per lane in flight (measured: 4 -> 16 took moe_dispatch from
  // about 70.0 to 69.4 us at the DeepSeek-R1 share)
  constexpr int U = 16;
  const int nv = H / 8;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + int64_t(t) * H);
  for (int v0 = 0; v0 < nv; v0 += 64 * U) {
    u32x4 q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * 64 + lane;
      if (v < nv) q[u] = src[v];
    }
    uint64_t mm = dests;
    while (mm) {
      const int j = __ffsll((unsigned long long)mm) - 1;
      mm &= mm - 1;
      const int row = shfl(d, j);
      u32x4* dst = reinterpret_cast<u32x4*>(x_perm + int64_t(row) * H);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * 64 + lane;
        if (v < nv) __builtin_nontemporal_store(q[u], dst + v);
      }
    }
  }
}

size_t dispatch_table_bytes(int T, int E) {
  const size_t cells = size_t(E) * size_t(ceil_div(T, kChunk));
  return ((cells + 1) / 2 * 2) * sizeof(int32_t) + cells * sizeof(unsigned long long);
}

hipError_t launch_dispatch_index(const int32_t* topk_idx, int T, int E, int k, int e0, int E_local, int32_t* counts,
                                 int32_t* offsets, int32_t* perm_src, int32_t* inv, int32_t* chunk_table,
                                 hipStream_t stream) {
  if (T <= kSmallMaxTokens) {
#define MOE_SMALL_LAUNCH(KM)                                                                                  \
  hipLaunchKernelGGL(dispatch_small_kernel<KM>, dim3(1), dim3(kSmallWaves * 64), 0, stream, topk_idx, T, E, k, \
                     e0, E_local, counts, offsets, perm_src, inv)
    if (k <= 1)
      MOE_SMALL_LAUNCH(1);
    else if (k <= 2)
      MOE_SMALL_LAUNCH(2);
    else if (k <= 4)
      MOE_SMALL_LAUNCH(4);
    else if (k <= 8)
      MOE_SMALL_LAUNCH(8);
    else if (k <= 16)
      MOE_SMALL_LAUNCH(16);
    else
      MOE_SMALL_LAUNCH(32);
#undef MOE_SMALL_LAUNCH
    return hipGetLastError();
  }
  const int nchunks = int(ceil_div(T, kChunk));
  const unsigned wgs = unsigned(ceil_div(nchunks, 4));
  hipLaunchKernelGGL(dispatch_hist_kernel, dim3(wgs), dim3(kThreads), size_t(4) * E * sizeof(int), stream,
                     topk_idx, T, E, k, nchunks, chunk_table, e0, E_local, nullptr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(unsigned(E)), dim3(kThreads), 0, stream, chunk_table, nchunks,
                     counts);
  if ((err = hipGetLastError()) != hipSuccess) return err;
#define MOE_INDEX_LAUNCH(KM)                                                                                  \
  hipLaunchKernelGGL(dispatch_index_kernel<KM>, dim3(wgs), dim3(kThreads), 0, stream, topk_idx, chunk_table, \
                     counts, T, k, e0, E_local, nchunks, offsets, perm_src, inv)
  if (k <= 1)
    MOE_INDEX_LAUNCH(1);
  else if (k <= 2)
    MOE_INDEX_LAUNCH(2);
  else if (k <= 4)
    MOE_INDEX_LAUNCH(4);
  else if (k <= 8)
    MOE_INDEX_LAUNCH(8);
  else if (k <= 16)
    MOE_INDEX_LAUNCH(16);
  else
    MOE_INDEX_LAUNCH(32);
#undef MOE_INDEX_LAUNCH
  return hipGetLastError();
}

hipError_t launch_dispatch(const uint16_t* x, const int32_t* topk_idx, int T, int H, int E, int k, int e0,
                           int E_local, int32_t* counts, int32_t* offsets, int32_t* perm_src, int32_t* inv,
                           uint16_t* x_perm, int32_t* chunk_table, hipStream_t stream) {
  if (T <= kSmallTokens) {
    hipError_t err =
        launch_dispatch_index(topk_idx, T, E, k, e0, E_local, counts, offsets, perm_src, inv, chunk_table, stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(dispatch_copy_kernel, dim3(unsigned(ceil_div(T, 4))), dim3(kThreads), 0, stream, x, inv, T,
                       H, k, x_perm);
    return hipGetLastError();
  }
  const int nchunks = int(ceil_div(T, kChunk));
  const size_t cells = size_t(E) * size_t(nchunks);
  auto* masks = reinterpret_cast<unsigned long long*>(chunk_table + (cells + 1) / 2 * 2);
  const unsigned wgs = unsigned(ceil_div(nchunks, 4));
  hipLaunchKernelGGL(dispatch_hist_kernel, dim3(wgs), dim3(kThreads), size_t(4) * E * sizeof(int), stream,
                     topk_idx, T, E, k, nchunks, chunk_table, e0, E_local, masks);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(unsigned(E)), dim3(kThreads), 0, stream, chunk_table, nchunks,
                     counts);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_place_copy_kernel, dim3(unsigned(ceil_div(T, 4))), dim3(kThreads), 0, stream, x,
                     topk_idx, chunk_table, masks, counts, T, H, k, e0, E_local, nchunks, offsets, perm_src, inv,
                     x_perm);
  return hipGetLastError();
}

}  // namespace moe
