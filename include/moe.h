/*
 * moe.h -- one expert-parallel rank's share of a Mixture-of-Experts layer on
 * one AMD Instinct MI355X (gfx950): router top-k, dispatch, grouped SwiGLU
 * expert MLPs, combine.
 *
 * The problem follows the expert-parallelism pages' statement of it:
 *   - T tokens of hidden size H; E experts in total, of which this rank owns
 *     the contiguous block [e0, e0 + E_local) ("Expert Parallelism (EP)",
 *     AWS Neuron vLLM design doc, section "Limitations": rank r owns experts
 *     [r*E_L, (r+1)*E_L));
 *   - the router weight [E, H] is replicated and scores every expert; the
 *     rank then keeps its local experts (same page, "Router Weights" and
 *     "Collective Patterns / Prefill", steps 1 and 3);
 *   - expert weights: gate_up [E_local, H, 2I] and down [E_local, I, H], the
 *     expert index first (same page, "Expert Weight Distribution" table);
 *   - tokens are grouped by selected expert, each expert's rows are stacked
 *     for one matmul, and the results return to their tokens in the original
 *     order, weighted by combine weights kept apart from the selection
 *     ("EP: Partition Experts and Route Tokens", sections "Send tokens to
 *     experts and return their results" and "Return multiple expert results
 *     to the same token");
 *   - a token none of whose selected experts is local gets a zero output row,
 *     so adding every rank's output gives the full layer ("Expert Parallelism
 *     (EP)", "Why a Single All-Reduce/Reduce-Scatter Works").
 *
 * Conventions for every entry point:
 *   - every pointer is DEVICE memory unless stated otherwise; the caller owns
 *     all buffers (inputs, outputs, workspaces). The library never allocates,
 *     frees or synchronises; each call only enqueues kernels on `stream`.
 *   - bfloat16 values are passed as raw 16-bit patterns (moe_bf16).
 *   - row-major layouts, densely packed, no padding.
 *   - argument checks run on the host before any launch; a call that fails a
 *     check returns a negative moe_status and launches nothing. A failed
 *     kernel launch returns MOE_ERR_HIP. Outputs are valid once the stream
 *     has reached the call's point.
 *   - T = 0 is valid: the call returns MOE_OK and launches nothing.
 *   - supported sizes: 1 <= k <= min(E, 32); E <= 1024; H and I multiples
 *     of 8 (16-byte vectors); T * k < 2^31; H * I < 2^29 (one expert's
 *     gate_up matrix below 2 GiB), else MOE_ERR_UNSUPPORTED.
 *   - matrix pointers (x, w_router, w_gate_up, w_down, x_perm, h, out,
 *     expert_out, y) are 16-byte aligned; a misaligned one is
 *     MOE_ERR_INVALID_ARG.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* a size, index range or required pointer is wrong */
  MOE_ERR_UNSUPPORTED = -2, /* valid problem outside the supported envelope (E > 1024, k > 32, ...) */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the *_workspace_size result */
  MOE_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef uint16_t moe_bf16; /* raw bfloat16 bits */

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(int status);

/* ------------------------------------------------------------------------ */
/* Router: logits, top-k selection and combine weights.                      */
/* ------------------------------------------------------------------------ */

/* Bytes of device workspace moe_route needs: a bfloat16 three-way split of
 * the float32 router weight, and float32 [T, E] partial logits for all but one
 * of the parts the hidden dimension is split into (2 parts when the token
 * count alone fills the GPU, more for few tokens). */
size_t moe_route_workspace_size(int T, int H, int E, int k);

/*
 * Scores every token against every expert and picks its top-k experts.
 * ("Expert Parallelism (EP)", "Collective Patterns / Prefill" step 1: the
 * affinities are [T, H] @ [H, E]; "Router Weights": all experts are scored.)
 *
 *   x         [T, H]  bf16   token vectors
 *   w_router  [E, H]  f32    router weight (one row per expert)
 *   bias      [E]     f32    added to every token's logits, or NULL
 *   renormalize       nonzero: the k softmax probabilities are rescaled to
 *                     sum to one; zero: plain softmax over all E experts
 *   logits    [T, E]  f32    OUT: x . w_router^T + bias, the values the
 *                     selection and the softmax use. Computed with float32
 *                     accuracy (exact bf16 products, float32 accumulation).
 *   topk_idx  [T, k]  i32    OUT: expert ids by descending logit; equal
 *                     logits put the lower expert id first
 *   topk_w    [T, k]  f32    OUT: combine weight of each selected expert
 *   workspace, workspace_bytes: at least moe_route_workspace_size bytes,
 *                     256-byte aligned
 */
int moe_route(const moe_bf16* x, const float* w_router, const float* bias, int T, int H, int E,
              int k, int renormalize, float* logits, int32_t* topk_idx, float* topk_w,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Dispatch: group the local (token, slot) selections by expert.             */
/* ------------------------------------------------------------------------ */

/* Bytes of device workspace moe_dispatch needs (per-64-token-chunk histograms
 * of all E experts and per-chunk 64-bit sets of the tokens that picked each
 * local expert). */
size_t moe_dispatch_workspace_size(int T, int E, int k);

/*
 * Counts the selections of every expert and lays the token vectors of this
 * rank's selections out grouped by expert ("EP: Partition Experts and Route
 * Tokens", "Send tokens to experts ...": dispatch groups token vectors by the
 * selected expert; the association of each row with its token is kept).
 *
 *   x         [T, H] bf16   token vectors
 *   topk_idx  [T, k] i32    selected experts, each in [0, E), distinct per token
 *   e0, E_local             this rank's experts are [e0, e0 + E_local)
 *   capacity                rows of perm_src / x_perm; must be >= T*min(k, E_local)
 *   counts    [E]   i32     OUT: selections of every expert, local or not
 *                           (sum = T*k)
 *   offsets   [E_local+1] i32 OUT: offsets[0] = 0,
 *                           offsets[i+1] = offsets[i] + counts[e0+i]
 *   perm_src  [capacity] i32 OUT: for row n < offsets[E_local], the flat slot
 *                           t*k + j it came from. Rows of expert e0+i are
 *                           [offsets[i], offsets[i+1]) in ascending t.
 *   inv       [T*k] i32     OUT: row of slot t*k + j, or -1 if its expert is
 *                           not local
 *   x_perm    [capacity, H] bf16 OUT: x_perm[n] = x[perm_src[n] / k], bit exact
 *   Rows at and beyond offsets[E_local] of perm_src and x_perm are left
 *   unspecified. Behaviour is undefined if topk_idx holds ids outside [0, E)
 *   or repeats an id within one token.
 */
int moe_dispatch(const moe_bf16* x, const int32_t* topk_idx, int T, int H, int E, int k, int e0,
                 int E_local, int64_t capacity, int32_t* counts, int32_t* offsets,
                 int32_t* perm_src, int32_t* inv, moe_bf16* x_perm, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Expert MLPs: grouped SwiGLU GEMMs over the ragged expert segments.        */
/* ------------------------------------------------------------------------ */

/*
 * For every local expert i and every row n in [offsets[i], offsets[i+1]):
 *   g = x_perm[n] . Wg_i, u = x_perm[n] . Wu_i   (Wg_i = w_gate_up[i][:, :I],
 *                                                 Wu_i = w_gate_up[i][:, I:])
 *   h[n]   = silu(g) * u,  silu(z) = z / (1 + exp(-z))   (stored as bf16)
 *   out[n] = h[n] . w_down[i]                            (stored as bf16)
 * with float32 accumulation. ("Expert Parallelism (EP)", weight-shape table:
 * gate_up [H, 2I] and down [I, H] per expert; "EP: Partition Experts and
 * Route Tokens": an expert's rows are stacked and transformed independently.)
 *
 *   x_perm    [capacity, H] bf16   rows grouped by expert (see moe_dispatch)
 *   offsets   [E_local+1]   i32    DEVICE memory, read by the kernels (no
 *                                  host synchronisation); non-decreasing,
 *                                  offsets[0] = 0, offsets[E_local] <= capacity
 *   w_gate_up [E_local, H, 2I] bf16
 *   w_down    [E_local, I, H]  bf16
 *   h         [capacity, I] bf16   OUT (intermediate activations)
 *   out       [capacity, H] bf16   OUT; rows >= offsets[E_local] untouched
 */
int moe_expert_ffn(const moe_bf16* x_perm, const int32_t* offsets, const moe_bf16* w_gate_up,
                   const moe_bf16* w_down, int H, int I, int E_local, int64_t capacity,
                   moe_bf16* h, moe_bf16* out, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Combine: weighted top-k sum back in the original token order.             */
/* ------------------------------------------------------------------------ */

/*
 * y[t] = sum over j = 0..k-1 with inv[t*k+j] >= 0 of
 *        topk_w[t, j] * expert_out[inv[t*k+j]],
 * summed in float32 in slot order, rounded once to bf16; rows with no local
 * slot are zeros. ("EP: Partition Experts and Route Tokens", "Return multiple
 * expert results to the same token": y(A2) = 0.7 u0 + 0.3 u2 at the source;
 * "Expert Parallelism (EP)": tokens without a local expert contribute zeros.)
 *
 *   expert_out [rows, H] bf16, inv [T*k] i32, topk_w [T, k] f32,
 *   y [T, H] bf16 OUT (every row written)
 */
int moe_combine(const moe_bf16* expert_out, const int32_t* inv, const float* topk_w, int T, int H,
                int k, moe_bf16* y, hipStream_t stream);

/*
 * moe_combine with a float32 output: the same float32 sum, stored without the
 * final rounding. This is the partial-output form of an expert-parallel
 * share: every rank's output is one partial sum of the layer, and the layer is
 * their sum over ranks ("Expert Parallelism (EP)", "Why a Single
 * All-Reduce/Reduce-Scatter Works"). Keeping the shares in float32 rounds the
 * layer once, after that sum, instead of once per share. Rounding y to bf16
 * (round to nearest even) gives moe_combine's y bit for bit.
 *
 *   y [T, H] f32 OUT (every row written), 16-byte aligned.
 * Checks and status codes are moe_combine's.
 */
int moe_combine_f32(const moe_bf16* expert_out, const int32_t* inv, const float* topk_w, int T, int H,
                    int k, float* y, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Whole share: route -> dispatch -> expert MLPs -> combine, one stream.     */
/* ------------------------------------------------------------------------ */

/* Bytes of device workspace moe_forward needs for T, H, I, E, k, E_local. */
size_t moe_forward_workspace_size(int T, int H, int I, int E, int k, int E_local);

/*
 * The rank's share of the MoE layer for T tokens: y [T, H] bf16. All
 * intermediates (logits, selections, dispatch tables, grouped rows, expert
 * activations and outputs) live in `workspace`, which must hold at least
 * moe_forward_workspace_size(...) bytes and be 256-byte aligned. Arguments
 * and their checks are those of the four steps above; the dispatch capacity
 * is T*min(k, E_local). No host synchronisation between the steps.
 */
int moe_forward(const moe_bf16* x, const float* w_router, const float* bias,
                const moe_bf16* w_gate_up, const moe_bf16* w_down, int T, int H, int I, int E,
                int k, int e0, int E_local, int renormalize, moe_bf16* y, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/*
 * moe_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The caller passes inputs and y as for moe_forward; the intermediates live
 * in a static device array of MOE_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends, so no workspace is
 * passed and the call allocates nothing.
 *   - MOE_ERR_WORKSPACE (nothing launched) when the problem needs more than
 *     the array holds, i.e. moe_forward_workspace_size(T, H, I, E, k,
 *     E_local) > MOE_NOALLOC_SCRATCH_BYTES (a DeepSeek-R1-shaped EP=8 rank
 *     share needs about 54 MB at T = 256 tokens, 183 MB at T = 1024; the
 *     limit admits up to T = 698).
 *   - the array is shared by every call on one GPU and keeps the last call's
 *     contents; no part of it needs to start at zero. Calls that overlap on
 *     one GPU (two streams, two threads) race on it and must be ordered by
 *     the caller.
 *   - the first call on a device looks up that device's copy
 *     (hipGetSymbolAddress); a caller that captures a graph may make one
 *     call before capturing.
 * Other arguments, checks and results are moe_forward's; y equals
 * moe_forward's y bit for bit.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int moe_forward_noalloc(const moe_bf16* x, const float* w_router, const float* bias,
                        const moe_bf16* w_gate_up, const moe_bf16* w_down, int T, int H, int I,
                        int E, int k, int e0, int E_local, int renormalize, moe_bf16* y,
                        hipStream_t stream);

/*
 * moe_forward whose share y [T, H] is float32 (the partial-output form of
 * moe_combine_f32, same citation): every step is moe_forward's, only the
 * combine stores its float32 sums unrounded. Rounding y to bf16 gives
 * moe_forward's y bit for bit; the float32 shares of ranks that split
 * [0, E) add up to the whole layer with one rounding. Workspace and checks
 * are moe_forward's.
 */
int moe_forward_f32(const moe_bf16* x, const float* w_router, const float* bias,
                    const moe_bf16* w_gate_up, const moe_bf16* w_down, int T, int H, int I, int E,
                    int k, int e0, int E_local, int renormalize, float* y, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * moe_forward with timing marks: records events[0..5] on `stream` before the
 * router, after the router, after dispatch, after the gate/up GEMM (with its
 * SwiGLU epilogue), after the down GEMM and after combine. `events` is a host
 * array of 6 events the caller created (with timing enabled); the work done
 * is exactly moe_forward's. MOE_ERR_INVALID_ARG if events or one of them is
 * NULL.
 */
int moe_forward_profiled(const moe_bf16* x, const float* w_router, const float* bias,
                         const moe_bf16* w_gate_up, const moe_bf16* w_down, int T, int H, int I,
                         int E, int k, int e0, int E_local, int renormalize, moe_bf16* y,
                         void* workspace, size_t workspace_bytes, hipEvent_t* events,
                         hipStream_t stream);

/*
 * moe_forward with the combine fused into the down-projection GEMM where it
 * needs no reduction across expert tiles. A token's local selections sit in
 * different expert segments, so summing them inside the GEMM would need
 * float atomics across the chip's L2 domains (and lose the fixed slot
 * order); a token with exactly one local selection needs no sum: its y row
 * is w * out, and the down GEMM's epilogue writes it straight to y in token
 * order ("EP: Partition Experts and Route Tokens", "Return multiple expert
 * results to the same token": the weighted return of an expert's result to
 * its token). The combine kernel then sums only tokens with two or more local
 * selections and zero-fills those with none. The epilogue rounds exactly as
 * the separate combine rounds a one-term sum, so y equals moe_forward's y
 * bit for bit. Arguments, workspace size and checks are moe_forward's; where
 * the down GEMM's k extent I is not a multiple of 32 the separate path runs.
 */
int moe_forward_fused(const moe_bf16* x, const float* w_router, const float* bias,
                      const moe_bf16* w_gate_up, const moe_bf16* w_down, int T, int H, int I, int E,
                      int k, int e0, int E_local, int renormalize, moe_bf16* y, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * moe_forward_fused with the timing marks of moe_forward_profiled (the
 * single-selection table is built between the second and third marks).
 */
int moe_forward_fused_profiled(const moe_bf16* x, const float* w_router, const float* bias,
                               const moe_bf16* w_gate_up, const moe_bf16* w_down, int T, int H, int I,
                               int E, int k, int e0, int E_local, int renormalize, moe_bf16* y,
                               void* workspace, size_t workspace_bytes, hipEvent_t* events,
                               hipStream_t stream);

/*
 * Byte offsets of the intermediates inside the moe_forward workspace, so a
 * caller can read them after the call (for checks and measurements). Writes
 * 9 values into `offsets_out` (host memory): logits, topk_idx, topk_w, counts,
 * offsets, perm_src, inv, x_perm, expert_out. The x_perm region is empty
 * (the forward's gate/up GEMM reads the token vectors of x in place) unless
 * H is not a multiple of 32 or T * H * 2 >= 2^31. Returns MOE_OK or
 * MOE_ERR_INVALID_ARG.
 */
int moe_forward_workspace_layout(int T, int H, int I, int E, int k, int E_local,
                                 size_t* offsets_out);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
