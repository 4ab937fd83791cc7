// Host-side launchers of the MoE kernels (internal; the public C-ABI is moe.h).
// Every launcher only enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

constexpr int kChunk = 64;  // tokens per dispatch chunk (one wave)

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Router: planes must hold 3*E*H bf16.
// planes: 3 x E x H bf16 scratch; part: T x E float32 scratch (second k half)
// Parts the router's k range is split into (1: no split); the workspace holds
// parts - 1 float32 [T, E] partials besides the logits.
int route_k_parts(int T, int H, int E);

hipError_t launch_route(const uint16_t* x, const float* w_router, const float* bias, int T, int H, int E, int k,
                        int renormalize, float* logits, int32_t* topk_idx, float* topk_w, uint16_t* planes, float* part,
                        hipStream_t stream);

// Dispatch: chunk_table must hold E * ceil(T/64) int32.
hipError_t launch_dispatch(const uint16_t* x, const int32_t* topk_idx, int T, int H, int E, int k, int e0,
                           int E_local, int32_t* counts, int32_t* offsets, int32_t* perm_src, int32_t* inv,
                           uint16_t* x_perm, int32_t* chunk_table, hipStream_t stream);

// Grouped SwiGLU expert MLPs over the segments given by device `offsets`.
hipError_t launch_expert_ffn(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_gate_up,
                             const uint16_t* w_down, int H, int I, int E_local, int64_t capacity, uint16_t* h,
                             uint16_t* out, hipStream_t stream);

// The two grouped GEMMs on their own (what launch_expert_ffn runs in order).
// rows_hint: the rows a local expert is expected to hold; few select the
// grouped GEMV (any routing gives correct results either way).
hipError_t launch_expert_gemm1(const uint16_t* x_perm, const int32_t* offsets, const uint16_t* w_gate_up, int H,
                               int I, int E_local, int64_t capacity, uint16_t* h, hipStream_t stream,
                               int64_t rows_hint);
hipError_t launch_expert_gemm2(const uint16_t* h, const int32_t* offsets, const uint16_t* w_down, int H, int I,
                               int E_local, int64_t capacity, uint16_t* out, hipStream_t stream, int64_t rows_hint);

// GEMM1 reading the token vectors of x in place (row n of a segment is token
// perm_src[n] / k) instead of a dispatched copy; usable when
// expert_gemm1_can_gather(T, H).
bool expert_gemm1_can_gather(int T, int H);
hipError_t launch_expert_gemm1_gather(const uint16_t* x, const int32_t* perm_src, int T, int k, const int32_t* offsets,
                                      const uint16_t* w_gate_up, int H, int I, int E_local, int64_t capacity,
                                      uint16_t* h, hipStream_t stream, int64_t rows_hint);

// Down GEMM with the combine of single-selection tokens in its epilogue:
// row_info[n] = {token, bits of its combine weight} when row n's token has
// exactly one local selection, else {-1, 0}; such rows are written to y [T, H]
// as w * out (rounded as the combine rounds a one-term sum), the others to
// out. Usable when expert_gemm2_can_fuse(I).
bool expert_gemm2_can_fuse(int I);
hipError_t launch_expert_gemm2_fused(const uint16_t* h, const int32_t* offsets, const uint16_t* w_down, int H, int I,
                                     int E_local, int64_t capacity, const int2* row_info, uint16_t* out, uint16_t* y,
                                     hipStream_t stream, int64_t rows_hint);

// Grouped GEMV for few rows per expert: each wave streams one weight panel
// of one expert for up to 32 of its rows (an expert with more gets more
// waves). Usable when K (H for the gate/up GEMM, I for the down GEMM) is a
// multiple of 32; chosen when the expected rows per local expert
// (rows_hint) are at most 32 (gate/up GEMM with 512 panels or more: 16).
// N: outputs (I for the gate/up GEMM, H for the down GEMM).
bool grouped_gemv_usable(int64_t rows_hint, int K, int N, int E_local, bool gate_up);
// gate/up + SwiGLU: rows from A [.., H] (row n of a segment is row
// gather_src[n] / gather_k of A when gather_src is given) into h [capacity, I]
hipError_t launch_grouped_gemv1(const uint16_t* A, int lda, const int32_t* gather_src, int gather_k, int gather_rows,
                                const int32_t* offsets, int E_local, int64_t capacity, const uint16_t* w_gate_up,
                                int H, int I, uint16_t* h, hipStream_t stream);
// down: h [capacity, I] into out [capacity, H]; with row_info, rows of
// single-selection tokens go to y as launch_expert_gemm2_fused writes them
hipError_t launch_grouped_gemv2(const uint16_t* h, const int32_t* offsets, int E_local, int64_t capacity,
                                const uint16_t* w_down, int H, int I, const int2* row_info, uint16_t* out,
                                uint16_t* y, hipStream_t stream);

// row_info of launch_expert_gemm2_fused from inv and topk_w (one thread per
// token); rows of tokens with two or more local selections get {-1, 0}.
hipError_t launch_single_rows(const int32_t* inv, const float* topk_w, int T, int k, int2* row_info,
                              hipStream_t stream);

// Bytes of the dispatch tables in the workspace: the per-chunk histogram
// table [E][ceil(T/64)] i32, then the per-chunk lane sets (at most E per
// chunk) u64.
size_t dispatch_table_bytes(int T, int E);

// Dispatch without the row copy (counts, offsets, perm_src, inv only).
hipError_t launch_dispatch_index(const int32_t* topk_idx, int T, int E, int k, int e0, int E_local, int32_t* counts,
                                 int32_t* offsets, int32_t* perm_src, int32_t* inv, int32_t* chunk_table,
                                 hipStream_t stream);

// Weighted top-k sum in token order; y is bf16, or float32 when y_f32. With
// skip_single, tokens with exactly one local selection are left untouched
// (the fused down GEMM wrote them; bf16 y only).
hipError_t launch_combine(const uint16_t* expert_out, const int32_t* inv, const float* topk_w, int T, int H, int k,
                          void* y, bool y_f32, hipStream_t stream, bool skip_single = false);

// Cached device facts of the current device.
int device_cu_count();

}  // namespace moe
