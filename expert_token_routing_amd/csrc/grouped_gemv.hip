// Grouped GEMV: the expert MLPs when each expert holds only a few token rows.
//
// In a decode step every rank runs all tokens through its local experts
// ("Expert Parallelism (EP)", "Collective Patterns / Decode (TKG kernel)"),
// and a batch of a few hundred tokens leaves each expert a handful of rows.
// The two GEMMs then do a few flops per weight byte and are bound by
// streaming the local experts' weights from HBM.
//
// No LDS is used for the operands: every wave streams its own weight panel
// straight into registers, 4 k-steps ahead of the matrix cores, for up to 32
// token rows of one expert (one or two groups of 16, both multiplied with
// every weight load); an expert with more rows gets one wave per 32 rows and
// panel.
//
// Wave geometry. A wave owns one panel of 16 CPL weight columns of one expert
// (CPL = 4 or 8 columns per lane) and walks k in steps of 32. Lane l = 16 g + m
// loads, per step, CPL columns (2 CPL bytes) from each of the 8 weight rows
// k0 + 8 g .. k0 + 8 g + 7, and the 16 bytes of token row m of each 16-row
// group at the same 8 k.
// Transposing its 8 x CPL block in registers gives the lane, for each of its
// columns c, the 8 k-values that lane (g, m) of a v_mfma_f32_16x16x32_bf16 A
// operand holds for A row m. So MFMA c multiplies the 16 columns
// colbase(m) + c (A rows m = 0..15) by a group's token rows (B columns m),
// and CPL MFMAs per step and group cover the panel. Afterwards lane (g, m)
// holds, in accumulator c of a group, element v, column colbase(4 g + v) + c
// of the group's token row m.
//
// Panel columns. Down GEMM: the panel is 16 CPL consecutive output columns,
// colbase(m) = CPL m, so a lane ends with the 4 CPL consecutive columns
// from 4 CPL g. Gate/up GEMM: the panel is 8 CPL outputs o0 .. with their gate
// and up columns side by side: colbase(4 g' + v') is gate column
// o0 + 2 CPL g' + CPL v' (v' < 2) or the up column of o0 + 2 CPL g' +
// CPL (v' - 2) (v' >= 2), so a lane ends with the gate (v = 0, 1) and up
// (v = 2, 3) values of its 2 CPL consecutive outputs from o0 + 2 CPL g. With
// CPL = 8 the 16 lanes of a group read whole 128-byte lines of gate and of
// up per weight row.
//
// Every output element is one MFMA chain over k in steps of 32 from k = 0,
// with the weights as the A operand, as in the tile kernel's gate/up GEMM.
#include <type_traits>
#include <utility>

#include "gemm_dma.h"
#include "gemm_tile.h"
#include "moe_kernels.h"

namespace moe {
namespace gemv {

using dma::panel::f32x4v;
using dma::panel::mfma16x16x32;

constexpr int kStepK = 32;            // k per step
constexpr int kGroupRows = 32;        // token rows of one wave (two groups of 16)
constexpr int kMaxLocal = 1024;       // local experts (the limit on E)

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  // bytes < 2^31 on every path (checked by the callers)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}

// Loads of one step: 8 weight rows x CPL columns, and the 8 k of the G token
// rows the lane feeds (one per group of 16 rows).
template <int D, int CPL, int G>
struct Ring {
  typedef typename std::conditional<CPL == 8, u32x4, u32x2>::type WRow;
  WRow w[D][8];
  u32x4 x[D][G];
};

struct GemvArgs {
  const uint16_t* A;
  int lda;
  const int32_t* gather_src;
  int gather_k, gather_rows;
  const uint16_t* W;  // this expert's weight matrix [K, ldw]
  int ldw, K, N, up_off;
  uint16_t* C;
  int ldc;
  const int2* row_info;
  uint16_t* y;
};

// One wave's panel p of an expert with `rows` (<= 16 G) token rows starting
// at row r0: G groups of 16 rows share every weight load.
// WAUX: cache policy of the weight loads (2: non-temporal; each weight byte
// is read once).
template <bool SWIGLU, bool FUSE, int CPL, int WAUX, int G, int D>
__device__ __forceinline__ void gemv_panel(const GemvArgs& a, int p, int rows, int r0) {
  static_assert(D >= 1 && (8 + G) * (D - 1) <= 63, "loads in flight must fit the vmcnt counter");
  constexpr int kOut = SWIGLU ? 8 * CPL : 16 * CPL;  // outputs per panel
  const int N = a.N;
  const int lane = lane_id();
  const int g = lane >> 4, m = lane & 15;

  // this lane's CPL weight columns (N is a multiple of 8: a block of CPL
  // columns is wholly inside or wholly past the end)
  int col;
  if (SWIGLU) {
    const int o = kOut * p + 2 * CPL * (m >> 2) + CPL * (m & 1);
    col = o < N ? ((m & 2) ? a.up_off + o : o) : 0;
  } else {
    const int c = kOut * p + CPL * m;
    col = c < N ? c : 0;
  }
  const rsrc_t wr = make_rsrc(a.W, int64_t(a.K) * a.ldw * 2);
  const uint32_t wvo = uint32_t(8 * g * a.ldw + col) * 2u;
  const int wrow = a.ldw * 2;  // bytes per weight row

  // token row 16 gi + m of group gi (the last row again past the expert's rows)
  rsrc_t xr;
  uint32_t xvo[G];
  if (a.gather_src != nullptr) {
    xr = make_rsrc(a.A, int64_t(a.gather_rows) * a.lda * 2);
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int rm = min(16 * gi + m, rows - 1);
      xvo[gi] = uint32_t(a.gather_src[r0 + rm] / a.gather_k) * uint32_t(a.lda) * 2u + 16u * uint32_t(g);
    }
  } else {
    xr = make_rsrc(a.A + int64_t(r0) * a.lda, int64_t(rows) * a.lda * 2);
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int rm = min(16 * gi + m, rows - 1);
      xvo[gi] = uint32_t(rm) * uint32_t(a.lda) * 2u + 16u * uint32_t(g);
    }
  }

  const int nsteps = a.K / kStepK;
  Ring<D, CPL, G> q;
  // step s (clamped to the last one, so every lane issues the same loads)
  auto load = [&](auto d_t, int s) {
    constexpr int d = decltype(d_t)::value;
    s = min(s, nsteps - 1);
    const int so = s * kStepK * wrow;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if constexpr (CPL == 8)
        q.w[d][r] = __builtin_amdgcn_raw_buffer_load_b128(wr, wvo, so + r * wrow, WAUX);
      else
        q.w[d][r] = __builtin_amdgcn_raw_buffer_load_b64(wr, wvo, so + r * wrow, WAUX);
    }
#pragma unroll
    for (int gi = 0; gi < G; ++gi) q.x[d][gi] = __builtin_amdgcn_raw_buffer_load_b128(xr, xvo[gi], s * kStepK * 2, 0);
    // keep the slots' loads in slot order: the wait before a slot is used
    // counts the loads of the slots issued after it
    __builtin_amdgcn_sched_barrier(0);
  };
  f32x4v acc[G][CPL];
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[gi][c] = f32x4v{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](auto d_t) {
    constexpr int d = decltype(d_t)::value;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      // column c of the 8 x CPL block: dword j = rows 2j (low half), 2j+1
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = __builtin_amdgcn_perm(q.w[d][2 * j + 1][c >> 1], q.w[d][2 * j][c >> 1], sel);
#pragma unroll
      for (int gi = 0; gi < G; ++gi) acc[gi][c] = mfma16x16x32(w, q.x[d][gi], acc[gi][c]);
    }
  };

  static_for<D>([&](auto d_t) { load(d_t, decltype(d_t)::value); });
  for (int s0 = 0; s0 < nsteps; s0 += D) {
    // slot d holds step s0 + d; once it is used, it takes step s0 + d + D
    static_for<D>([&](auto d_t) {
      constexpr int d = decltype(d_t)::value;
      if (s0 + d < nsteps) consume(d_t);
      load(d_t, s0 + d + D);
    });
  }

#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int row = 16 * gi + m;  // token row of this lane in group gi
    if (row >= rows) continue;
    if constexpr (SWIGLU) {
      // outputs o0 + 2 CPL g + CPL v + c (v = 0, 1): gate in element v, up in
      // element v + 2; 8-output chunks
      const int o = kOut * p + 2 * CPL * g;
#pragma unroll
      for (int u = 0; u < CPL / 4; ++u) {
        if (o + 8 * u < N) {
          float hv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int v = (8 * u + i) / CPL, c = (8 * u + i) % CPL;
            const float gt = acc[gi][c][v];
            hv[i] = gt / (1.f + __expf(-gt)) * acc[gi][c][v + 2];
          }
          *reinterpret_cast<u32x4*>(a.C + int64_t(r0 + row) * a.ldc + o + 8 * u) =
              u32x4{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]), pack_bf16x2(hv[4], hv[5]),
                    pack_bf16x2(hv[6], hv[7])};
        }
      }
    } else {
      // columns c0 + 4 CPL g + CPL v + c; 8-column chunks
      int dst = -1;
      float wt = 0.f;
      if constexpr (FUSE) {
        const int2 ri = a.row_info[r0 + row];
        dst = ri.x;
        wt = __int_as_float(ri.y);
      }
      uint16_t* const base = dst >= 0 ? a.y + int64_t(dst) * a.ldc : a.C + int64_t(r0 + row) * a.ldc;
      const int c0 = kOut * p + 4 * CPL * g;
#pragma unroll
      for (int u = 0; u < CPL / 2; ++u) {
        if (c0 + 8 * u < N) {
          uint32_t o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = 8 * u + 2 * i;  // column pair (j, j + 1) of the lane's 4 CPL
            uint32_t lo = f32_to_bf16_bits(acc[gi][j % CPL][j / CPL]);
            uint32_t hi = f32_to_bf16_bits(acc[gi][(j + 1) % CPL][(j + 1) / CPL]);
            if (FUSE && dst >= 0) {
              lo = f32_to_bf16_bits(fmaf(wt, bf16_to_f32(uint16_t(lo)), -0.f));
              hi = f32_to_bf16_bits(fmaf(wt, bf16_to_f32(uint16_t(hi)), -0.f));
            }
            o[i] = lo | (hi << 16);
          }
          *reinterpret_cast<u32x4*>(base + c0 + 8 * u) = u32x4{o[0], o[1], o[2], o[3]};
        }
      }
    }
  }
}

// Waves: expert e with m_e rows gets ceil(m_e / 32) row groups of up to 32
// rows for each of its panels, row group fastest, so the waves reading one
// weight panel for different row groups run side by side and share its
// lines through L2 (those use plain loads). Every workgroup builds the prefix of waves per expert
// from the offsets; the grid covers the most waves any routing can need,
// (ceil(capacity / 32) + E_local) x panels, and waves past the total exit.
// NW waves per workgroup (independent but for the table). At most 256
// registers per lane (accumulators included), so that two waves share a SIMD.
template <bool SWIGLU, bool FUSE, int CPL, int WAUX, int NW>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
grouped_gemv_kernel(const uint16_t* __restrict__ A, int lda, const int32_t* __restrict__ gather_src, int gather_k,
                    int gather_rows, const int32_t* __restrict__ offsets, int E_local, int64_t capacity,
                    const uint16_t* __restrict__ W, int64_t w_expert_stride, int ldw, int K, int N, int up_off,
                    uint16_t* __restrict__ C, int ldc, const int2* __restrict__ row_info, uint16_t* __restrict__ y) {
  static_assert(!(FUSE && SWIGLU), "the combine is fused into the down GEMM only");
  static_assert(CPL == 4 || CPL == 8, "4 or 8 columns per lane");
  constexpr int kOut = SWIGLU ? 8 * CPL : 16 * CPL;  // outputs per panel
  constexpr int kThreads = 64 * NW;
  constexpr int kPerT = kMaxLocal / kThreads;
  __shared__ int s_off[kMaxLocal + 1];   // segment bounds, clamped into [0, capacity]
  __shared__ int s_wpre[kMaxLocal + 1];  // first wave of each expert
  __shared__ int s_tmp[NW];
  const int npanel = (N + kOut - 1) / kOut;
  int nw[kPerT];
  int sum = 0;
#pragma unroll
  for (int q = 0; q < kPerT; ++q) {
    const int i = int(threadIdx.x) * kPerT + q;
    nw[q] = 0;
    if (i < E_local) {
      const int64_t a = min<int64_t>(max<int64_t>(offsets[i], 0), capacity);
      const int64_t b = max<int64_t>(a, min<int64_t>(offsets[i + 1], capacity));
      s_off[i] = int(a);
      if (i == E_local - 1) s_off[E_local] = int(b);
      nw[q] = int((b - a + kGroupRows - 1) / kGroupRows) * npanel;
      sum += nw[q];
    }
  }
  int total;
  int pre = block_exclusive_scan<kThreads>(sum, s_tmp, total);
#pragma unroll
  for (int q = 0; q < kPerT; ++q) {
    const int i = int(threadIdx.x) * kPerT + q;
    if (i < E_local) s_wpre[i] = pre;
    pre += nw[q];
  }
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * NW + int(threadIdx.x >> 6));
  if (wave >= total) return;
  // the expert: the last one whose first wave is at or before this one
  // (experts without rows own no waves)
  int lo = 0, hi = E_local - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_wpre[mid] <= wave)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int e = __builtin_amdgcn_readfirstlane(lo);
  const int seg0 = __builtin_amdgcn_readfirstlane(s_off[e]);
  const int m_e = __builtin_amdgcn_readfirstlane(s_off[e + 1]) - seg0;
  const int ngroups = (m_e + kGroupRows - 1) / kGroupRows;
  const int local = wave - __builtin_amdgcn_readfirstlane(s_wpre[e]);
  const int p = local / ngroups;
  const int j = local - p * ngroups;
  const int r0 = seg0 + kGroupRows * j;
  const int rows = min(kGroupRows, m_e - kGroupRows * j);
  const GemvArgs args{A, lda, gather_src, gather_k, gather_rows, W + int64_t(e) * w_expert_stride, ldw, K, N, up_off,
                      C, ldc, row_info, y};
  // one or two groups of 16 rows; when other waves read the same panel for
  // the expert's other rows, plain loads, so that its lines stay in L2 for
  // them
  if (ngroups == 1) {
    if (rows <= 16)
      gemv_panel<SWIGLU, FUSE, CPL, WAUX, 1, 4>(args, p, rows, r0);
    else
      gemv_panel<SWIGLU, FUSE, CPL, WAUX, 2, 4>(args, p, rows, r0);
  } else {
    if (rows <= 16)
      gemv_panel<SWIGLU, FUSE, CPL, 0, 1, 4>(args, p, rows, r0);
    else
      gemv_panel<SWIGLU, FUSE, CPL, 0, 2, 4>(args, p, rows, r0);
  }
}

template <bool SWIGLU, bool FUSE>
hipError_t launch(const uint16_t* A, int lda, const int32_t* gather_src, int gather_k, int gather_rows,
                  const int32_t* offsets, int E_local, int64_t capacity, const uint16_t* W, int64_t w_expert_stride,
                  int ldw, int K, int N, int up_off, uint16_t* C, int ldc, const int2* row_info, uint16_t* y,
                  hipStream_t stream) {
  constexpr int CPL = 8;
  constexpr int WAUX = 2;
  const int64_t npanel = ceil_div(N, SWIGLU ? 8 * CPL : 16 * CPL);
  const int64_t waves = (ceil_div(capacity, kGroupRows) + E_local) * npanel;
  // Four waves per workgroup (neighbouring panels on one CU) when there are
  // panels enough to fill the chip; with few (few local experts, narrow
  // outputs) one, so that the waves spread over as many CUs as possible.
  // Measured: the DeepSeek-R1 decode step's 1024 / 1792 waves run 279 / 148 us
  // in fours and 339 / 162 us alone; a GPT-OSS-20B decode step's down GEMM
  // (4 experts x 23 panels) 86 us in fours and 34 us alone.
  if (E_local * npanel >= 512) {
    hipLaunchKernelGGL((grouped_gemv_kernel<SWIGLU, FUSE, CPL, WAUX, 4>), dim3(unsigned(ceil_div(waves, 4))),
                       dim3(256), 0, stream, A, lda, gather_src, gather_k, gather_rows, offsets, E_local, capacity, W,
                       w_expert_stride, ldw, K, N, up_off, C, ldc, row_info, y);
  } else {
    hipLaunchKernelGGL((grouped_gemv_kernel<SWIGLU, FUSE, CPL, WAUX, 1>), dim3(unsigned(waves)), dim3(64), 0,
                       stream, A, lda, gather_src, gather_k, gather_rows, offsets, E_local, capacity, W,
                       w_expert_stride, ldw, K, N, up_off, C, ldc, row_info, y);
  }
  return hipGetLastError();
}

}  // namespace gemv

bool grouped_gemv_usable(int64_t rows_hint, int K, int N, int E_local, bool gate_up) {
  // Measured against the tile kernel: the down GEMM wins up to 32 expected
  // rows per local expert; the gate/up GEMM up to 16 when the local experts
  // have 512 panels or more (DeepSeek-R1 shapes: at 24 and 32 rows it lost)
  // and up to 32 when they have fewer (GPT-OSS-20B decode step, 4 experts x
  // 48 panels at 32 rows: 40 against 50 us). K in whole steps.
  const int64_t panels = int64_t(E_local) * ceil_div(N, gate_up ? 64 : 128);
  const int64_t limit = gate_up && panels >= 512 ? gemv::kGroupRows / 2 : gemv::kGroupRows;
  return K % gemv::kStepK == 0 && rows_hint <= limit;
}

hipError_t launch_grouped_gemv1(const uint16_t* A, int lda, const int32_t* gather_src, int gather_k, int gather_rows,
                                const int32_t* offsets, int E_local, int64_t capacity, const uint16_t* w_gate_up,
                                int H, int I, uint16_t* h, hipStream_t stream) {
  return gemv::launch<true, false>(A, lda, gather_src, gather_k, gather_rows, offsets, E_local, capacity, w_gate_up,
                                   int64_t(H) * 2 * I, 2 * I, H, I, I, h, I, nullptr, nullptr, stream);
}

hipError_t launch_grouped_gemv2(const uint16_t* h, const int32_t* offsets, int E_local, int64_t capacity,
                                const uint16_t* w_down, int H, int I, const int2* row_info, uint16_t* out,
                                uint16_t* y, hipStream_t stream) {
  if (row_info != nullptr)
    return gemv::launch<false, true>(h, I, nullptr, 1, 0, offsets, E_local, capacity, w_down, int64_t(I) * H, H, I, H,
                                     0, out, H, row_info, y, stream);
  return gemv::launch<false, false>(h, I, nullptr, 1, 0, offsets, E_local, capacity, w_down, int64_t(I) * H, H, I, H,
                                    0, out, H, nullptr, nullptr, stream);
}

}  // namespace moe
