"""ctypes binding of ``libmoe.so`` (the C-ABI declared in include/moe.h).

Argument marshalling only: every step of the MoE share runs in the library's
HIP kernels. PyTorch provides device memory and the current stream. There is
no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import numbers
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


def _need(t, dtype, name, shape=None, dev=None, min_rows=False):
    """``t`` must be a ``dtype`` tensor of ``shape`` (None entries: any size;
    with ``min_rows`` the first dimension may also be larger). The library
    sees only pointers, so a wrong size would otherwise become an
    out-of-bounds access on the GPU. Contiguity and device are checked
    afterwards by _placed, once every shape has been checked, so that a
    mismatch is reported as one whatever the tensors' device."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None:
        got = tuple(t.shape)
        ok = len(got) == len(shape) and all(
            want is None or g == want or (min_rows and i == 0 and g >= want) for i, (g, want) in enumerate(zip(got, shape)))
        if not ok:
            want_s = "(" + ", ".join("*" if v is None else (f">={v}" if min_rows and i == 0 else str(v))
                                     for i, v in enumerate(shape)) + ")"
            raise ValueError(f"{name} has shape {got}, expected shape {want_s}")


def _placed(dev, **tensors):
    """Every given tensor (None: skipped) is contiguous and on the GPU dev."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if not t.is_cuda:
            raise ValueError(f"{name} must live on a GPU (this library has no CPU path)")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the call's other tensors on {dev}")


def _nbytes(t):
    return t.numel() * t.element_size()


def _workspace(nbytes, device, workspace, name="workspace"):
    torch = _torch()
    if workspace is None:
        return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if _nbytes(workspace) < nbytes:
        raise ValueError(f"{name} holds {_nbytes(workspace)} bytes, needs {nbytes}")
    if not workspace.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not workspace.is_cuda or workspace.device != device:
        raise ValueError(f"{name} must live on {device}")
    return workspace


def _out(t, shape, dtype, dev, name):
    """The caller's output tensor, checked, or a new one."""
    torch = _torch()
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    _need(t, dtype, name, shape, dev)
    _placed(dev, **{name: t})
    return t


def _check_k(k, E):
    if not isinstance(k, numbers.Integral) or k < 1 or k > E:
        raise ValueError(f"k must be an int in [1, E = {E}], got {k!r}")


def moe_route(x, w_router, bias, k, renormalize=True, *, logits=None, topk_idx=None, topk_w=None,
              workspace=None, stream=None):
    """Router logits [T,E] f32, top-k ids [T,k] i32 and combine weights [T,k] f32."""
    torch = _torch()
    _need(x, torch.bfloat16, "x", (None, None))
    T, H = x.shape
    dev = x.device
    _need(w_router, torch.float32, "w_router", (None, H), dev)
    E = w_router.shape[0]
    if bias is not None:
        _need(bias, torch.float32, "bias", (E,), dev)
    _check_k(k, E)
    for name, t, shp, dt in (("logits", logits, (T, E), torch.float32), ("topk_idx", topk_idx, (T, k), torch.int32),
                             ("topk_w", topk_w, (T, k), torch.float32)):
        if t is not None:
            _need(t, dt, name, shp)
    _placed(dev, x=x, w_router=w_router, bias=bias)
    logits = _out(logits, (T, E), torch.float32, dev, "logits")
    topk_idx = _out(topk_idx, (T, k), torch.int32, dev, "topk_idx")
    topk_w = _out(topk_w, (T, k), torch.float32, dev, "topk_w")
    L = lib()
    ws = _workspace(L.moe_route_workspace_size(T, H, E, k), dev, workspace)
    st = L.moe_route(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, k, int(bool(renormalize)), _ptr(logits),
                     _ptr(topk_idx), _ptr(topk_w), _ptr(ws), _nbytes(ws), _stream(stream, dev))
    check(st, "moe_route")
    return logits, topk_idx, topk_w


def moe_dispatch(x, topk_idx, E, e0, E_local, *, capacity=None, counts=None, offsets=None, perm_src=None,
                 inv=None, x_perm=None, workspace=None, stream=None):
    """counts [E], offsets [E_local+1], perm_src [cap], inv [T*k], x_perm [cap,H]."""
    torch = _torch()
    _need(x, torch.bfloat16, "x", (None, None))
    T, H = x.shape
    dev = x.device
    _need(topk_idx, torch.int32, "topk_idx", (T, None), dev)
    k = topk_idx.shape[1]
    if not (0 <= e0 and E_local >= 1 and e0 + E_local <= E):
        raise ValueError(f"local experts [e0, e0 + E_local) = [{e0}, {e0 + E_local}) must lie in [0, E = {E})")
    _check_k(k, E)
    cap = T * min(k, E_local) if capacity is None else int(capacity)
    if cap < T * min(k, E_local):
        raise ValueError(f"capacity {cap} < T * min(k, E_local) = {T * min(k, E_local)}")
    for name, t, shp, dt, mr in (("counts", counts, (E,), torch.int32, False),
                                 ("offsets", offsets, (E_local + 1,), torch.int32, False),
                                 ("perm_src", perm_src, (max(cap, 1),), torch.int32, True),
                                 ("inv", inv, (max(T * k, 1),), torch.int32, True),
                                 ("x_perm", x_perm, (max(cap, 1), H), torch.bfloat16, True)):
        if t is not None:
            _need(t, dt, name, shp, min_rows=mr)
    _placed(dev, x=x, topk_idx=topk_idx)
    counts = _out(counts, (E,), torch.int32, dev, "counts")
    offsets = _out(offsets, (E_local + 1,), torch.int32, dev, "offsets")
    if perm_src is None:
        perm_src = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    else:
        _placed(dev, perm_src=perm_src)
    if inv is None:
        inv = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    else:
        _placed(dev, inv=inv)
    if x_perm is None:
        x_perm = torch.empty((max(cap, 1), H), dtype=torch.bfloat16, device=dev)
    else:
        _placed(dev, x_perm=x_perm)
    L = lib()
    ws = _workspace(L.moe_dispatch_workspace_size(T, E, k), dev, workspace)
    st = L.moe_dispatch(_ptr(x), _ptr(topk_idx), T, H, E, k, e0, E_local, cap, _ptr(counts), _ptr(offsets),
                        _ptr(perm_src), _ptr(inv), _ptr(x_perm), _ptr(ws), _nbytes(ws), _stream(stream, dev))
    check(st, "moe_dispatch")
    return counts, offsets, perm_src, inv, x_perm


def moe_expert_ffn(x_perm, offsets, w_gate_up, w_down, *, h=None, out=None, stream=None):
    """h [cap, I] and expert outputs [cap, H] for the segments in ``offsets``."""
    torch = _torch()
    _need(x_perm, torch.bfloat16, "x_perm", (None, None))
    cap, H = x_perm.shape
    dev = x_perm.device
    _need(w_gate_up, torch.bfloat16, "w_gate_up", (None, H, None), dev)
    E_local, _, I2 = w_gate_up.shape
    if I2 % 2:
        raise ValueError(f"w_gate_up's last dimension 2I must be even, got {I2}")
    I = I2 // 2
    _need(w_down, torch.bfloat16, "w_down", (E_local, I, H), dev)
    _need(offsets, torch.int32, "offsets", (E_local + 1,), dev)
    if h is not None:
        _need(h, torch.bfloat16, "h", (cap, I))
    if out is not None:
        _need(out, torch.bfloat16, "out", (cap, H))
    _placed(dev, x_perm=x_perm, offsets=offsets, w_gate_up=w_gate_up, w_down=w_down)
    h = _out(h, (cap, I), torch.bfloat16, dev, "h")
    out = _out(out, (cap, H), torch.bfloat16, dev, "out")
    st = lib().moe_expert_ffn(_ptr(x_perm), _ptr(offsets), _ptr(w_gate_up), _ptr(w_down), H, I, E_local, cap,
                              _ptr(h), _ptr(out), _stream(stream, dev))
    check(st, "moe_expert_ffn")
    return h, out


def _combine(name, out_dtype, expert_out, inv, topk_w, y, stream):
    torch = _torch()
    _need(topk_w, torch.float32, "topk_w", (None, None))
    T, k = topk_w.shape
    dev = topk_w.device
    _need(expert_out, torch.bfloat16, "expert_out", (None, None), dev)
    H = expert_out.shape[1]
    if inv.dim() != 1:
        raise ValueError(f"inv has shape {tuple(inv.shape)}, expected shape ({T * k},)")
    _need(inv, torch.int32, "inv", (T * k,), dev)
    if y is not None:
        _need(y, out_dtype, "y", (T, H))
    _placed(dev, expert_out=expert_out, inv=inv, topk_w=topk_w)
    y = _out(y, (T, H), out_dtype, dev, "y")
    st = getattr(lib(), name)(_ptr(expert_out), _ptr(inv), _ptr(topk_w), T, H, k, _ptr(y), _stream(stream, dev))
    check(st, name)
    return y


def moe_combine(expert_out, inv, topk_w, *, y=None, stream=None):
    """y [T, H] bf16: weighted sum of each token's local expert outputs.
    Every inv entry that is not -1 must be a row of expert_out (the library
    cannot check device values)."""
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


def _forward_args(x, w_router, bias, w_gate_up, w_down, k, e0):
    """Checks the forward's inputs; returns (T, H, I, E, E_local, device)."""
    torch = _torch()
    _need(x, torch.bfloat16, "x", (None, None))
    T, H = x.shape
    dev = x.device
    _need(w_router, torch.float32, "w_router", (None, H), dev)
    E = w_router.shape[0]
    if bias is not None:
        _need(bias, torch.float32, "bias", (E,), dev)
    _need(w_gate_up, torch.bfloat16, "w_gate_up", (None, H, None), dev)
    E_local, _, I2 = w_gate_up.shape
    if I2 % 2:
        raise ValueError(f"w_gate_up's last dimension 2I must be even, got {I2}")
    I = I2 // 2
    _need(w_down, torch.bfloat16, "w_down", (E_local, I, H), dev)
    _check_k(k, E)
    if not (0 <= e0 and e0 + E_local <= E):
        raise ValueError(f"local experts [e0, e0 + E_local) = [{e0}, {e0 + E_local}) must lie in [0, E = {E})")
    return T, H, I, E, E_local, dev


def _forward_placed(dev, x, w_router, bias, w_gate_up, w_down):
    _placed(dev, x=x, w_router=w_router, bias=bias, w_gate_up=w_gate_up, w_down=w_down)


def _forward(name, out_dtype, x, w_router, bias, w_gate_up, w_down, k, e0, renormalize, y, workspace, stream):
    T, H, I, E, E_local, dev = _forward_args(x, w_router, bias, w_gate_up, w_down, k, e0)
    if y is not None:
        _need(y, out_dtype, "y", (T, H))
    _forward_placed(dev, x, w_router, bias, w_gate_up, w_down)
    y = _out(y, (T, H), out_dtype, dev, "y")
    ws = _workspace(forward_workspace_size(T, H, I, E, k, E_local), dev, workspace)
    st = getattr(lib(), name)(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate_up), _ptr(w_down), T, H, I, E, k,
                              e0, E_local, int(bool(renormalize)), _ptr(y), _ptr(ws), _nbytes(ws),
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
    torch = _torch()
    T, H, I, E, E_local, dev = _forward_args(x, w_router, bias, w_gate_up, w_down, k, e0)
    _need(y, torch.bfloat16, "y", (T, H))
    if workspace is None:
        raise ValueError("workspace is required")
    if len(events) != 6:
        raise ValueError(f"events must hold 6 events, got {len(events)}")
    _forward_placed(dev, x, w_router, bias, w_gate_up, w_down)
    _placed(dev, y=y)
    ws = _workspace(forward_workspace_size(T, H, I, E, k, E_local), dev, workspace)
    arr = (c_void_p * 6)(*[c_void_p(ev.cuda_event) for ev in events])
    name = "moe_forward_fused_profiled" if fused else "moe_forward_profiled"
    st = getattr(lib(), name)(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate_up), _ptr(w_down), T, H, I, E, k, e0,
                              E_local, int(bool(renormalize)), _ptr(y), _ptr(ws), _nbytes(ws), arr,
                              _stream(stream, dev))
    check(st, name)


def moe_forward_noalloc(x, w_router, bias, w_gate_up, w_down, k, e0, renormalize=True, *, y, stream=None):
    """moe_forward with the intermediates in the library's static scratch
    (no workspace; the call allocates nothing on the device). ``y`` [T, H]
    bf16 is the caller's. Raises MoEError(MOE_ERR_WORKSPACE) when the problem
    needs more than NOALLOC_SCRATCH_BYTES."""
    torch = _torch()
    T, H, I, E, E_local, dev = _forward_args(x, w_router, bias, w_gate_up, w_down, k, e0)
    _need(y, torch.bfloat16, "y", (T, H))
    _forward_placed(dev, x, w_router, bias, w_gate_up, w_down)
    _placed(dev, y=y)
    st = lib().moe_forward_noalloc(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate_up), _ptr(w_down), T, H, I, E, k,
                                   e0, E_local, int(bool(renormalize)), _ptr(y), _stream(stream, dev))
    check(st, "moe_forward_noalloc")
    return y
