"""ctypes binding of ``libmoe.so`` (the C-ABI declared in include/moe.h).

Argument marshalling only: every step of the MoE share runs in the library's
HIP kernels. PyTorch provides device memory and the current stream. There is
no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import pathlib
from ctypes import c_int, c_int64, c_size_t, c_void_p

LIB_PATH = pathlib.Path(__file__).resolve().parent / "libmoe.so"

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4

# symbol -> (restype, argtypes)
_P = c_void_p
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [c_int]),
    "moe_route_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int]),
    "moe_route": (c_int, [_P, _P, _P, c_int, c_int, c_int, c_int, c_int, _P, _P, _P, _P, c_size_t, _P]),
    "moe_dispatch_workspace_size": (c_size_t, [c_int, c_int, c_int]),
    "moe_dispatch": (c_int, [_P, _P, c_int, c_int, c_int, c_int, c_int, c_int, c_int64,
                             _P, _P, _P, _P, _P, _P, c_size_t, _P]),
    "moe_expert_ffn": (c_int, [_P, _P, _P, _P, c_int, c_int, c_int, c_int64, _P, _P, _P]),
    "moe_combine": (c_int, [_P, _P, _P, c_int, c_int, c_int, _P, _P]),
    "moe_combine_f32": (c_int, [_P, _P, _P, c_int, c_int, c_int, _P, _P]),
    "moe_forward_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int]),
    "moe_forward_workspace_layout": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, ctypes.POINTER(c_size_t)]),
    "moe_forward": (c_int, [_P, _P, _P, _P, _P, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                            _P, _P, c_size_t, _P]),
    "moe_forward_f32": (c_int, [_P, _P, _P, _P, _P, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                _P, _P, c_size_t, _P]),
    "moe_forward_profiled": (c_int, [_P, _P, _P, _P, _P, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                     _P, _P, c_size_t, _P, _P]),
    "moe_forward_fused": (c_int, [_P, _P, _P, _P, _P, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                  _P, _P, c_size_t, _P]),
    "moe_forward_fused_profiled": (c_int, [_P, _P, _P, _P, _P, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                           c_int, _P, _P, c_size_t, _P, _P]),
    "moe_forward_noalloc": (c_int, [_P, _P, _P, _P, _P, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                    _P, _P]),
}

# bytes of the static scratch moe_forward_noalloc works in (MOE_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 128 << 20

_lib = None


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m expert_token_routing_amd.build_lib`; there is no fallback path")
        h = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoEError(status, where)


# --------------------------------------------------------------------------- #
# torch-facing wrappers                                                        #
# --------------------------------------------------------------------------- #
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _stream(stream, device):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return c_void_p(s.cuda_stream)


def _need(t, dtype, name, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on a GPU (this library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _workspace(nbytes, device, workspace):
    torch = _torch()
    if workspace is None:
        return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, needs {nbytes}")
    return workspace


def moe_route(x, w_router, bias, k, renormalize=True, *, logits=None, topk_idx=None, topk_w=None,
              workspace=None, stream=None):
    """Router logits [T,E] f32, top-k ids [T,k] i32 and combine weights [T,k] f32."""
    torch = _torch()
    _need(x, torch.bfloat16, "x", 2)
    _need(w_router, torch.float32, "w_router", 2)
    if bias is not None:
        _need(bias, torch.float32, "bias", 1)
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if logits is None else logits
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_idx is None else topk_idx
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_w is None else topk_w
    L = lib()
    ws = _workspace(L.moe_route_workspace_size(T, H, E, k), dev, workspace)
    st = L.moe_route(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, k, int(bool(renormalize)), _ptr(logits),
                     _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws.numel(), _stream(stream, dev))
    check(st, "moe_route")
    return logits, topk_idx, topk_w


def moe_dispatch(x, topk_idx, E, e0, E_local, *, capacity=None, counts=None, offsets=None, perm_src=None,
                 inv=None, x_perm=None, workspace=None, stream=None):
    """counts [E], offsets [E_local+1], perm_src [cap], inv [T*k], x_perm [cap,H]."""
    torch = _torch()
    _need(x, torch.bfloat16, "x", 2)
    _need(topk_idx, torch.int32, "topk_idx", 2)
    T, H = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    cap = T * min(k, E_local) if capacity is None else int(capacity)
    counts = torch.empty(E, dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(E_local + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    perm_src = torch.empty(max(cap, 1), dtype=torch.int32, device=dev) if perm_src is None else perm_src
    inv = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev) if inv is None else inv
    x_perm = torch.empty((max(cap, 1), H), dtype=torch.bfloat16, device=dev) if x_perm is None else x_perm
    L = lib()
    ws = _workspace(L.moe_dispatch_workspace_size(T, E, k), dev, workspace)
    st = L.moe_dispatch(_ptr(x), _ptr(topk_idx), T, H, E, k, e0, E_local, cap, _ptr(counts), _ptr(offsets),
                        _ptr(perm_src), _ptr(inv), _ptr(x_perm), _ptr(ws), ws.numel(), _stream(stream, dev))
    check(st, "moe_dispatch")
    return counts, offsets, perm_src, inv, x_perm


def moe_expert_ffn(x_perm, offsets, w_gate_up, w_down, *, h=None, out=None, stream=None):
    """h [cap, I] and expert outputs [cap, H] for the segments in ``offsets``."""
    torch = _torch()
    _need(x_perm, torch.bfloat16, "x_perm", 2)
    _need(offsets, torch.int32, "offsets", 1)
    _need(w_gate_up, torch.bfloat16, "w_gate_up", 3)
    _need(w_down, torch.bfloat16, "w_down", 3)
    cap, H = x_perm.shape
    E_local, H2, I2 = w_gate_up.shape
    if H2 != H or tuple(w_down.shape) != (E_local, I2 // 2, H) or offsets.numel() != E_local + 1:
        raise ValueError("shape mismatch between x_perm, offsets, w_gate_up and w_down")
    I = I2 // 2
    dev = x_perm.device
    h = torch.empty((cap, I), dtype=torch.bfloat16, device=dev) if h is None else h
    out = torch.empty((cap, H), dtype=torch.bfloat16, device=dev) if out is None else out
    st = lib().moe_expert_ffn(_ptr(x_perm), _ptr(offsets), _ptr(w_gate_up), _ptr(w_down), H, I, E_local, cap,
                              _ptr(h), _ptr(out), _stream(stream, dev))
    check(st, "moe_expert_ffn")
    return h, out


def _combine(name, out_dtype, expert_out, inv, topk_w, y, stream):
    torch = _torch()
    _need(expert_out, torch.bfloat16, "expert_out", 2)
    _need(inv, torch.int32, "inv")
    _need(topk_w, torch.float32, "topk_w", 2)
    T, k = topk_w.shape
    H = expert_out.shape[1]
    dev = expert_out.device
    y = torch.empty((T, H), dtype=out_dtype, device=dev) if y is None else y
    _need(y, out_dtype, "y", 2)
    if tuple(y.shape) != (T, H):
        raise ValueError(f"y must have shape {(T, H)}, got {tuple(y.shape)}")
    st = getattr(lib(), name)(_ptr(expert_out), _ptr(inv), _ptr(topk_w), T, H, k, _ptr(y), _stream(stream, dev))
    check(st, name)
    return y


def moe_combine(expert_out, inv, topk_w, *, y=None, stream=None):
    """y [T, H] bf16: weighted sum of each token's local expert outputs."""
    return _combine("moe_combine", _torch().bfloat16, expert_out, inv, topk_w, y, stream)


def moe_combine_f32(expert_out, inv, topk_w, *, y=None, stream=None):
    """y [T, H] float32: moe_combine's sums before their rounding to bf16."""
    return _combine("moe_combine_f32", _torch().float32, expert_out, inv, topk_w, y, stream)


def forward_workspace_size(T, H, I, E, k, E_local) -> int:
    return int(lib().moe_forward_workspace_size(T, H, I, E, k, E_local))


def forward_workspace_layout(T, H, I, E, k, E_local) -> dict:
    arr = (c_size_t * 9)()
    check(lib().moe_forward_workspace_layout(T, H, I, E, k, E_local, arr), "moe_forward_workspace_layout")
    names = ["logits", "topk_idx", "topk_w", "counts", "offsets", "perm_src", "inv", "x_perm", "expert_out"]
    return dict(zip(names, [int(v) for v in arr]))


def _forward(name, out_dtype, x, w_router, bias, w_gate_up, w_down, k, e0, renormalize, y, workspace, stream):
    torch = _torch()
    _need(x, torch.bfloat16, "x", 2)
    _need(w_router, torch.float32, "w_router", 2)
    if bias is not None:
        _need(bias, torch.float32, "bias", 1)
    _need(w_gate_up, torch.bfloat16, "w_gate_up", 3)
    _need(w_down, torch.bfloat16, "w_down", 3)
    T, H = x.shape
    E = w_router.shape[0]
    E_local, _, I2 = w_gate_up.shape
    I = I2 // 2
    dev = x.device
    y = torch.empty((T, H), dtype=out_dtype, device=dev) if y is None else y
    _need(y, out_dtype, "y", 2)
    if tuple(y.shape) != (T, H):
        raise ValueError(f"y must have shape {(T, H)}, got {tuple(y.shape)}")
    ws = _workspace(forward_workspace_size(T, H, I, E, k, E_local), dev, workspace)
    st = getattr(lib(), name)(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate_up), _ptr(w_down), T, H, I, E, k,
                              e0, E_local, int(bool(renormalize)), _ptr(y), _ptr(ws), ws.numel(),
                              _stream(stream, dev))
    check(st, name)
    return y, ws


def moe_forward(x, w_router, bias, w_gate_up, w_down, k, e0, renormalize=True, *, y=None, workspace=None,
                stream=None):
    """The rank's share of the MoE layer: y [T, H] bf16. ``E_local`` is
    ``w_gate_up.shape[0]``; the rank owns experts [e0, e0 + E_local)."""
    return _forward("moe_forward", _torch().bfloat16, x, w_router, bias, w_gate_up, w_down, k, e0, renormalize, y,
                    workspace, stream)


def moe_forward_f32(x, w_router, bias, w_gate_up, w_down, k, e0, renormalize=True, *, y=None, workspace=None,
                    stream=None):
    """moe_forward with the share kept in float32 (y [T, H] float32), for
    summing the shares of several ranks before one rounding."""
    return _forward("moe_forward_f32", _torch().float32, x, w_router, bias, w_gate_up, w_down, k, e0, renormalize,
                    y, workspace, stream)


def moe_forward_fused(x, w_router, bias, w_gate_up, w_down, k, e0, renormalize=True, *, y=None, workspace=None,
                      stream=None):
    """moe_forward with the combine of tokens that have exactly one local
    selection done in the down GEMM's epilogue; y equals moe_forward's."""
    return _forward("moe_forward_fused", _torch().bfloat16, x, w_router, bias, w_gate_up, w_down, k, e0,
                    renormalize, y, workspace, stream)


def moe_forward_profiled(x, w_router, bias, w_gate_up, w_down, k, e0, renormalize, y, workspace, events,
                         stream=None, fused=False):
    """moe_forward (moe_forward_fused with ``fused``) into preallocated ``y`` /
    ``workspace``, recording the six torch.cuda.Event objects in ``events``
    (already recorded once, so they exist) around the router, dispatch,
    gate/up GEMM, down GEMM and combine."""
    T, H = x.shape
    E = w_router.shape[0]
    E_local, _, I2 = w_gate_up.shape
    arr = (c_void_p * 6)(*[c_void_p(ev.cuda_event) for ev in events])
    name = "moe_forward_fused_profiled" if fused else "moe_forward_profiled"
    st = getattr(lib(), name)(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate_up), _ptr(w_down), T, H, I2 // 2, E,
                              k, e0, E_local, int(bool(renormalize)), _ptr(y), _ptr(workspace), workspace.numel(),
                              arr, _stream(stream, x.device))
    check(st, name)


def moe_forward_noalloc(x, w_router, bias, w_gate_up, w_down, k, e0, renormalize=True, *, y, stream=None):
    """moe_forward with the intermediates in the library's static scratch
    (no workspace; the call allocates nothing on the device). ``y`` [T, H]
    bf16 is the caller's. Raises MoEError(MOE_ERR_WORKSPACE) when the problem
    needs more than NOALLOC_SCRATCH_BYTES."""
    torch = _torch()
    _need(x, torch.bfloat16, "x", 2)
    _need(w_router, torch.float32, "w_router", 2)
    if bias is not None:
        _need(bias, torch.float32, "bias", 1)
    _need(w_gate_up, torch.bfloat16, "w_gate_up", 3)
    _need(w_down, torch.bfloat16, "w_down", 3)
    _need(y, torch.bfloat16, "y", 2)
    T, H = x.shape
    E = w_router.shape[0]
    E_local, _, I2 = w_gate_up.shape
    if tuple(y.shape) != (T, H):
        raise ValueError(f"y must have shape {(T, H)}, got {tuple(y.shape)}")
    st = lib().moe_forward_noalloc(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate_up), _ptr(w_down), T, H, I2 // 2,
                                   E, k, e0, E_local, int(bool(renormalize)), _ptr(y), _stream(stream, x.device))
    check(st, "moe_forward_noalloc")
    return y
