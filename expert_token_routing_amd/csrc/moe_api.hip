// C-ABI of the MoE rank-share library: argument checks, workspace layout and
// the one-stream forward pass. Every check runs on the host before any launch.
#include <mutex>

#include "moe.h"
#include "moe_kernels.h"

namespace moe {

namespace {
constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

std::mutex g_dev_mu;
int g_cu_count[64] = {0};
void* g_scratch_ptr[64] = {nullptr};
}  // namespace

// The forward workspace of moe_forward_noalloc, for callers that cannot
// allocate. Each GPU the library runs on holds its own copy, from the load
// of the library's code on that GPU until the process ends.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

// This device's address of `scratch`, looked up once per device with the
// device current (the array's name is not a device address in host code).
static int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_HIP;
  if (dev >= 64) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_cu_count[dev] == 0) {
      int cus = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
      g_cu_count[dev] = cus;
    }
    return g_cu_count[dev];
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  return cus;
}

// Common checks of the problem statement (T, H, E, k, local block).
static int check_route_dims(int T, int H, int E, int k) {
  if (T < 0 || H <= 0 || (H % 8) != 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE || k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (int64_t(T) * k >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}
static int check_local(int E, int e0, int E_local) {
  if (E_local < 1 || e0 < 0 || int64_t(e0) + E_local > E) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}
static int64_t min_capacity(int T, int k, int E_local) { return int64_t(T) * std::min(k, E_local); }
// The GEMMs address one expert's weight matrix through a buffer resource
// whose range and offsets are 32-bit: gate_up (H x 2I bf16, the larger of the
// two) must stay below 2 GiB, i.e. H * I < 2^29.
static bool expert_weights_fit(int H, int I) { return int64_t(H) * I * 4 < (int64_t(1) << 31); }
static int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Workspace layout of moe_forward.
struct ForwardLayout {
  size_t planes, part, logits, topk_idx, topk_w, counts, offsets, perm_src, inv, chunks, x_perm, h, out, row_info,
      total;
};
static ForwardLayout forward_layout(int T, int H, int I, int E, int k, int E_local) {
  ForwardLayout L{};
  const int64_t cap = min_capacity(T, k, E_local);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.planes = take(size_t(3) * E * H * sizeof(uint16_t));
  L.part = take(size_t(route_k_parts(T, H, E) - 1) * T * E * sizeof(float));
  L.logits = take(size_t(T) * E * sizeof(float));
  L.topk_idx = take(size_t(T) * k * sizeof(int32_t));
  L.topk_w = take(size_t(T) * k * sizeof(float));
  L.counts = take(size_t(E) * sizeof(int32_t));
  L.offsets = take(size_t(E_local + 1) * sizeof(int32_t));
  L.perm_src = take(size_t(cap) * sizeof(int32_t));
  L.inv = take(size_t(T) * k * sizeof(int32_t));
  L.chunks = take(dispatch_table_bytes(T, E));
  // the dispatched rows: only when GEMM1 cannot read the token vectors in place
  L.x_perm = take(expert_gemm1_can_gather(T, H) ? 0 : size_t(cap) * H * sizeof(uint16_t));
  L.h = take(size_t(cap) * I * sizeof(uint16_t));
  L.out = take(size_t(cap) * H * sizeof(uint16_t));
  L.row_info = take(size_t(cap) * sizeof(int2));
  L.total = o;
  return L;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid size, index range or null pointer";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: outside the supported sizes (E <= 1024, k <= 32, T*k < 2^31, H*I < 2^29)";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
    default: return "unknown moe_status";
  }
}

size_t moe_route_workspace_size(int T, int H, int E, int k) {
  (void)k;
  if (H <= 0 || E <= 0 || T < 0) return 0;
  return align_up(size_t(3) * E * H * sizeof(uint16_t)) +
         align_up(size_t(route_k_parts(T, H, E) - 1) * T * E * sizeof(float));
}

int moe_route(const moe_bf16* x, const float* w_router, const float* bias, int T, int H, int E, int k,
              int renormalize, float* logits, int32_t* topk_idx, float* topk_w, void* workspace,
              size_t workspace_bytes, hipStream_t stream) {
  int st = check_route_dims(T, H, E, k);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !logits || !topk_idx || !topk_w || !aligned16(x) || !aligned16(w_router))
    return MOE_ERR_INVALID_ARG;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0 ||
      workspace_bytes < moe_route_workspace_size(T, H, E, k))
    return MOE_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  return hip_status(launch_route(x, w_router, bias, T, H, E, k, renormalize, logits, topk_idx, topk_w,
                                 reinterpret_cast<uint16_t*>(ws),
                                 reinterpret_cast<float*>(ws + align_up(size_t(3) * E * H * sizeof(uint16_t))),
                                 stream));
}

size_t moe_dispatch_workspace_size(int T, int E, int k) {
  (void)k;
  if (T < 0 || E <= 0) return 0;
  return align_up(dispatch_table_bytes(T, E));
}

int moe_dispatch(const moe_bf16* x, const int32_t* topk_idx, int T, int H, int E, int k, int e0, int E_local,
                 int64_t capacity, int32_t* counts, int32_t* offsets, int32_t* perm_src, int32_t* inv,
                 moe_bf16* x_perm, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_route_dims(T, H, E, k);
  if (st != MOE_OK) return st;
  if ((st = check_local(E, e0, E_local)) != MOE_OK) return st;
  if (capacity < min_capacity(T, k, E_local)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !topk_idx || !counts || !offsets || !perm_src || !inv || !x_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_INVALID_ARG;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0 ||
      workspace_bytes < moe_dispatch_workspace_size(T, E, k))
    return MOE_ERR_WORKSPACE;
  return hip_status(launch_dispatch(x, topk_idx, T, H, E, k, e0, E_local, counts, offsets, perm_src, inv, x_perm,
                                    static_cast<int32_t*>(workspace), stream));
}

int moe_expert_ffn(const moe_bf16* x_perm, const int32_t* offsets, const moe_bf16* w_gate_up,
                   const moe_bf16* w_down, int H, int I, int E_local, int64_t capacity, moe_bf16* h,
                   moe_bf16* out, hipStream_t stream) {
  if (H <= 0 || I <= 0 || (H % 8) != 0 || (I % 8) != 0 || E_local < 1 || capacity < 0) return MOE_ERR_INVALID_ARG;
  if (E_local > kMaxE || !expert_weights_fit(H, I)) return MOE_ERR_UNSUPPORTED;
  if (capacity >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (capacity == 0) return MOE_OK;
  if (!x_perm || !offsets || !w_gate_up || !w_down || !h || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(h) || !aligned16(out))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_expert_ffn(x_perm, offsets, w_gate_up, w_down, H, I, E_local, capacity, h, out, stream));
}

static int combine_impl(const moe_bf16* expert_out, const int32_t* inv, const float* topk_w, int T, int H, int k,
                        void* y, bool y_f32, hipStream_t stream) {
  if (T < 0 || H <= 0 || (H % 8) != 0 || k < 1) return MOE_ERR_INVALID_ARG;
  if (k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (int64_t(T) * k >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!expert_out || !inv || !topk_w || !y || !aligned16(expert_out) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(expert_out, inv, topk_w, T, H, k, y, y_f32, stream));
}

int moe_combine(const moe_bf16* expert_out, const int32_t* inv, const float* topk_w, int T, int H, int k,
                moe_bf16* y, hipStream_t stream) {
  return combine_impl(expert_out, inv, topk_w, T, H, k, y, false, stream);
}

int moe_combine_f32(const moe_bf16* expert_out, const int32_t* inv, const float* topk_w, int T, int H, int k,
                    float* y, hipStream_t stream) {
  return combine_impl(expert_out, inv, topk_w, T, H, k, y, true, stream);
}

size_t moe_forward_workspace_size(int T, int H, int I, int E, int k, int E_local) {
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || E_local <= 0) return 0;
  return forward_layout(T, H, I, E, k, E_local).total;
}

int moe_forward_workspace_layout(int T, int H, int I, int E, int k, int E_local, size_t* offsets_out) {
  if (!offsets_out || T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || E_local <= 0) return MOE_ERR_INVALID_ARG;
  const ForwardLayout L = forward_layout(T, H, I, E, k, E_local);
  const size_t v[9] = {L.logits, L.topk_idx, L.topk_w, L.counts, L.offsets, L.perm_src, L.inv, L.x_perm, L.out};
  for (int i = 0; i < 9; ++i) offsets_out[i] = v[i];
  return MOE_OK;
}

static int forward_impl(const moe_bf16* x, const float* w_router, const float* bias, const moe_bf16* w_gate_up,
                        const moe_bf16* w_down, int T, int H, int I, int E, int k, int e0, int E_local,
                        int renormalize, void* y, bool y_f32, void* workspace, size_t workspace_bytes,
                        hipEvent_t* events, hipStream_t stream, bool fuse_combine = false) {
  int st = check_route_dims(T, H, E, k);
  if (st != MOE_OK) return st;
  if ((st = check_local(E, e0, E_local)) != MOE_OK) return st;
  if (I <= 0 || (I % 8) != 0) return MOE_ERR_INVALID_ARG;
  if (!expert_weights_fit(H, I)) return MOE_ERR_UNSUPPORTED;
  if (min_capacity(T, k, E_local) >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !w_gate_up || !w_down || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(y))
    return MOE_ERR_INVALID_ARG;
  const ForwardLayout L = forward_layout(T, H, I, E, k, E_local);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0 || workspace_bytes < L.total)
    return MOE_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  auto at = [&](size_t off) { return static_cast<void*>(ws + off); };
  const int64_t cap = min_capacity(T, k, E_local);
  float* logits = static_cast<float*>(at(L.logits));
  int32_t* topk_idx = static_cast<int32_t*>(at(L.topk_idx));
  float* topk_w = static_cast<float*>(at(L.topk_w));
  int32_t* counts = static_cast<int32_t*>(at(L.counts));
  int32_t* offsets = static_cast<int32_t*>(at(L.offsets));
  int32_t* perm_src = static_cast<int32_t*>(at(L.perm_src));
  int32_t* inv = static_cast<int32_t*>(at(L.inv));
  int32_t* chunks = static_cast<int32_t*>(at(L.chunks));
  uint16_t* x_perm = static_cast<uint16_t*>(at(L.x_perm));
  uint16_t* h = static_cast<uint16_t*>(at(L.h));
  uint16_t* out = static_cast<uint16_t*>(at(L.out));
  int2* row_info = static_cast<int2*>(at(L.row_info));
  // the combine of single-selection tokens runs in the down GEMM's epilogue
  const bool fuse = fuse_combine && !y_f32 && expert_gemm2_can_fuse(I);
  auto mark = [&](int i) { return events ? hipEventRecord(events[i], stream) : hipSuccess; };

  hipError_t err = mark(0);
  if (err == hipSuccess)
    err = launch_route(x, w_router, bias, T, H, E, k, renormalize, logits, topk_idx, topk_w,
                       static_cast<uint16_t*>(at(L.planes)), static_cast<float*>(at(L.part)), stream);
  if (err == hipSuccess) err = mark(1);
  // GEMM1 reads the token vectors in place when it can, so dispatch only
  // builds the tables; otherwise the rows are copied out first.
  const bool gather = expert_gemm1_can_gather(T, H);
  // rows a local expert holds when the T k selections spread evenly over
  // the E experts (the GEMMs take the grouped GEMV when that is small)
  const int64_t rows_hint = ceil_div(int64_t(T) * k, E);
  if (err == hipSuccess)
    err = gather ? launch_dispatch_index(topk_idx, T, E, k, e0, E_local, counts, offsets, perm_src, inv, chunks, stream)
                 : launch_dispatch(x, topk_idx, T, H, E, k, e0, E_local, counts, offsets, perm_src, inv, x_perm,
                                   chunks, stream);
  if (err == hipSuccess && fuse) err = launch_single_rows(inv, topk_w, T, k, row_info, stream);
  if (err == hipSuccess) err = mark(2);
  if (err == hipSuccess)
    err = gather ? launch_expert_gemm1_gather(x, perm_src, T, k, offsets, w_gate_up, H, I, E_local, cap, h, stream,
                                              rows_hint)
                 : launch_expert_gemm1(x_perm, offsets, w_gate_up, H, I, E_local, cap, h, stream, rows_hint);
  if (err == hipSuccess) err = mark(3);
  if (err == hipSuccess)
    err = fuse ? launch_expert_gemm2_fused(h, offsets, w_down, H, I, E_local, cap, row_info, out,
                                           static_cast<uint16_t*>(y), stream, rows_hint)
               : launch_expert_gemm2(h, offsets, w_down, H, I, E_local, cap, out, stream, rows_hint);
  if (err == hipSuccess) err = mark(4);
  if (err == hipSuccess) err = launch_combine(out, inv, topk_w, T, H, k, y, y_f32, stream, fuse);
  if (err == hipSuccess) err = mark(5);
  return hip_status(err);
}

int moe_forward(const moe_bf16* x, const float* w_router, const float* bias, const moe_bf16* w_gate_up,
                const moe_bf16* w_down, int T, int H, int I, int E, int k, int e0, int E_local, int renormalize,
                moe_bf16* y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return forward_impl(x, w_router, bias, w_gate_up, w_down, T, H, I, E, k, e0, E_local, renormalize, y, false,
                      workspace, workspace_bytes, nullptr, stream);
}

int moe_forward_noalloc(const moe_bf16* x, const float* w_router, const float* bias, const moe_bf16* w_gate_up,
                        const moe_bf16* w_down, int T, int H, int I, int E, int k, int e0, int E_local, int renormalize,
                        moe_bf16* y, hipStream_t stream) {
  // the argument checks first, so that a rejected call has no side effect
  int st = check_route_dims(T, H, E, k);
  if (st != MOE_OK) return st;
  if ((st = check_local(E, e0, E_local)) != MOE_OK) return st;
  if (I <= 0 || (I % 8) != 0) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (forward_layout(T, H, I, E, k, E_local).total > size_t(MOE_NOALLOC_SCRATCH_BYTES)) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != MOE_OK) return st;
  return forward_impl(x, w_router, bias, w_gate_up, w_down, T, H, I, E, k, e0, E_local, renormalize, y, false, ws,
                      size_t(MOE_NOALLOC_SCRATCH_BYTES), nullptr, stream);
}

int moe_forward_f32(const moe_bf16* x, const float* w_router, const float* bias, const moe_bf16* w_gate_up,
                    const moe_bf16* w_down, int T, int H, int I, int E, int k, int e0, int E_local, int renormalize,
                    float* y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return forward_impl(x, w_router, bias, w_gate_up, w_down, T, H, I, E, k, e0, E_local, renormalize, y, true,
                      workspace, workspace_bytes, nullptr, stream);
}

int moe_forward_profiled(const moe_bf16* x, const float* w_router, const float* bias, const moe_bf16* w_gate_up,
                         const moe_bf16* w_down, int T, int H, int I, int E, int k, int e0, int E_local,
                         int renormalize, moe_bf16* y, void* workspace, size_t workspace_bytes,
                         hipEvent_t* events, hipStream_t stream) {
  if (!events) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < 6; ++i)
    if (!events[i]) return MOE_ERR_INVALID_ARG;
  return forward_impl(x, w_router, bias, w_gate_up, w_down, T, H, I, E, k, e0, E_local, renormalize, y, false,
                      workspace, workspace_bytes, events, stream);
}

int moe_forward_fused(const moe_bf16* x, const float* w_router, const float* bias, const moe_bf16* w_gate_up,
                      const moe_bf16* w_down, int T, int H, int I, int E, int k, int e0, int E_local,
                      int renormalize, moe_bf16* y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return forward_impl(x, w_router, bias, w_gate_up, w_down, T, H, I, E, k, e0, E_local, renormalize, y, false,
                      workspace, workspace_bytes, nullptr, stream, true);
}

int moe_forward_fused_profiled(const moe_bf16* x, const float* w_router, const float* bias,
                               const moe_bf16* w_gate_up, const moe_bf16* w_down, int T, int H, int I, int E, int k,
                               int e0, int E_local, int renormalize, moe_bf16* y, void* workspace,
                               size_t workspace_bytes, hipEvent_t* events, hipStream_t stream) {
  if (!events) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < 6; ++i)
    if (!events[i]) return MOE_ERR_INVALID_ARG;
  return forward_impl(x, w_router, bias, w_gate_up, w_down, T, H, I, E, k, e0, E_local, renormalize, y, false,
                      workspace, workspace_bytes, events, stream, true);
}

}  // extern "C"
