"""The C-ABI library on the CPU: it loads, exports every entry point that
include/moe.h declares, sizes workspaces, and rejects invalid arguments on the
host before any launch (no GPU needed: every call here fails its checks, or
is a T = 0 no-op, before touching HIP)."""
import ctypes
import pathlib
import re

import pytest

import expert_token_routing_amd as M
from expert_token_routing_amd import _binding as B

HEADER = pathlib.Path(__file__).resolve().parent.parent / "include" / "moe.h"
CALIB_HEADER = HEADER.with_name("moe_calib.h")
CALIB_LIB = pathlib.Path(M.__file__).resolve().parent / "libmoe_calib.so"
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below is rejected first
FAKE_ODD = ctypes.c_void_p(0x10002)  # not 16-byte aligned


def header_functions(header=HEADER):
    text = header.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(moe_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_library_exports_every_header_symbol():
    L = M.lib()
    names = header_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(L, n), f"libmoe.so lacks {n}"
    assert set(names) == set(B.SIGNATURES), (set(names) ^ set(B.SIGNATURES))


def test_calibration_library_exports_and_host_checks():
    """libmoe_calib.so (the counter-calibration read) exports exactly what
    include/moe_calib.h declares and rejects bad sizes and pointers on the
    host; bytes = 0 launches nothing."""
    names = header_functions(CALIB_HEADER)
    assert names == ["moe_calib_dma_read", "moe_calib_mfma_loop"]
    L = ctypes.CDLL(str(CALIB_LIB))
    for n in names:
        assert hasattr(L, n), n
    f = L.moe_calib_dma_read
    f.restype, f.argtypes = ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert f(FAKE, 0, None) == M.MOE_OK
    for ptr, nbytes in ((FAKE, 1000), (FAKE, 1024 + 16), (FAKE_ODD, 1024), (None, 1024), (FAKE, (1 << 30) + 1024)):
        assert f(ptr, nbytes, None) == M.MOE_ERR_INVALID_ARG, (ptr, nbytes)
    g = L.moe_calib_mfma_loop
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    flop = ctypes.c_double(0)
    for iters, wps, sink in ((0, 2, FAKE), (10, 0, FAKE), (10, 9, FAKE), (10, 2, None)):
        assert g(iters, wps, sink, ctypes.byref(flop), None) == M.MOE_ERR_INVALID_ARG


def test_status_strings():
    for st in (M.MOE_OK, M.MOE_ERR_INVALID_ARG, M.MOE_ERR_UNSUPPORTED, M.MOE_ERR_WORKSPACE, M.MOE_ERR_HIP):
        assert M.status_string(st).startswith("MOE_")
    assert "unknown" in M.status_string(12345)


def test_workspace_sizes():
    L = M.lib()
    assert L.moe_route_workspace_size(16384, 7168, 256, 8) >= 3 * 256 * 7168 * 2
    assert L.moe_dispatch_workspace_size(16384, 256, 8) >= 256 * 256 * 4
    assert L.moe_dispatch_workspace_size(1, 4, 1) >= 16
    T, H, I, E, k, El = 16384, 7168, 2048, 256, 8, 32
    # the gate/up GEMM reads the token vectors in place (H a multiple of 32,
    # T*H*2 < 2^31): no dispatched copy x_perm in the workspace
    ws = M.forward_workspace_size(T, H, I, E, k, El)
    cap = T * min(k, El)
    assert cap * H * 2 + cap * I * 2 + T * E * 4 <= ws < 2 * cap * H * 2
    lay = M.forward_workspace_layout(T, H, I, E, k, El)
    offs = sorted(lay.values())
    assert all(o % 256 == 0 for o in offs)
    assert len(set(offs)) == len(offs) and offs[-1] < ws
    assert lay["expert_out"] + cap * H * 2 <= ws
    assert lay["expert_out"] - lay["x_perm"] == cap * I * 2  # x_perm empty, h between
    # H not a multiple of 32: the rows are copied out first, x_perm takes cap x H
    H2 = 7176
    ws2 = M.forward_workspace_size(T, H2, I, E, k, El)
    lay2 = M.forward_workspace_layout(T, H2, I, E, k, El)
    assert ws2 >= 2 * cap * H2 * 2 + cap * I * 2 + T * E * 4
    assert lay2["expert_out"] - lay2["x_perm"] >= cap * H2 * 2 + cap * I * 2
    # T*H*2 >= 2^31 also copies the rows out
    T3 = 150000
    lay3 = M.forward_workspace_layout(T3, H, I, E, k, El)
    assert lay3["expert_out"] - lay3["x_perm"] >= T3 * min(k, El) * H * 2
    assert L.moe_forward_workspace_size(-1, H, I, E, k, El) == 0


def _route(**kw):
    a = dict(x=FAKE, w=FAKE, b=None, T=4, H=8, E=4, k=1, renorm=1, logits=FAKE, idx=FAKE, wts=FAKE,
             ws=ctypes.c_void_p(0x100000), wsb=1 << 20, stream=None)
    a.update(kw)
    return M.lib().moe_route(a["x"], a["w"], a["b"], a["T"], a["H"], a["E"], a["k"], a["renorm"], a["logits"],
                             a["idx"], a["wts"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(k=0), M.MOE_ERR_INVALID_ARG),
    (dict(k=5), M.MOE_ERR_INVALID_ARG),          # k > E
    (dict(E=0), M.MOE_ERR_INVALID_ARG),
    (dict(H=12), M.MOE_ERR_INVALID_ARG),         # H % 8
    (dict(H=0), M.MOE_ERR_INVALID_ARG),
    (dict(T=-1), M.MOE_ERR_INVALID_ARG),
    (dict(E=2048, k=2), M.MOE_ERR_UNSUPPORTED),
    (dict(E=64, k=33), M.MOE_ERR_UNSUPPORTED),
    (dict(T=1 << 28, E=64, k=8), M.MOE_ERR_UNSUPPORTED),  # T*k >= 2^31
    (dict(x=None), M.MOE_ERR_INVALID_ARG),
    (dict(logits=None), M.MOE_ERR_INVALID_ARG),
    (dict(x=FAKE_ODD), M.MOE_ERR_INVALID_ARG),
    (dict(w=FAKE_ODD), M.MOE_ERR_INVALID_ARG),   # router weight read as 16-byte vectors
    (dict(ws=None), M.MOE_ERR_WORKSPACE),
    (dict(wsb=16), M.MOE_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x100010)), M.MOE_ERR_WORKSPACE),  # not 256-byte aligned
    (dict(T=0, x=None, logits=None), M.MOE_OK),  # empty batch: no-op
])
def test_route_rejects(kw, want):
    assert _route(**kw) == want


def _dispatch(**kw):
    a = dict(x=FAKE, idx=FAKE, T=8, H=8, E=4, k=2, e0=0, El=2, cap=16, counts=FAKE, offsets=FAKE, perm=FAKE,
             inv=FAKE, xp=FAKE, ws=ctypes.c_void_p(0x100000), wsb=1 << 20)
    a.update(kw)
    return M.lib().moe_dispatch(a["x"], a["idx"], a["T"], a["H"], a["E"], a["k"], a["e0"], a["El"], a["cap"],
                                a["counts"], a["offsets"], a["perm"], a["inv"], a["xp"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(El=0), M.MOE_ERR_INVALID_ARG),
    (dict(e0=-1), M.MOE_ERR_INVALID_ARG),
    (dict(e0=3, El=2), M.MOE_ERR_INVALID_ARG),     # e0 + E_local > E
    (dict(cap=15), M.MOE_ERR_INVALID_ARG),         # capacity < T*min(k, E_local)
    (dict(El=1, cap=7), M.MOE_ERR_INVALID_ARG),
    (dict(k=5), M.MOE_ERR_INVALID_ARG),
    (dict(inv=None), M.MOE_ERR_INVALID_ARG),
    (dict(xp=FAKE_ODD), M.MOE_ERR_INVALID_ARG),
    (dict(wsb=0), M.MOE_ERR_WORKSPACE),
    (dict(T=0, cap=0, x=None), M.MOE_OK),
])
def test_dispatch_rejects(kw, want):
    assert _dispatch(**kw) == want


@pytest.mark.parametrize("args,want", [
    ((FAKE, FAKE, FAKE, FAKE, 8, 8, 0, 16, FAKE, FAKE, None), M.MOE_ERR_INVALID_ARG),      # E_local = 0
    ((FAKE, FAKE, FAKE, FAKE, 12, 8, 2, 16, FAKE, FAKE, None), M.MOE_ERR_INVALID_ARG),     # H % 8
    ((FAKE, FAKE, FAKE, FAKE, 8, 4, 2, 16, FAKE, FAKE, None), M.MOE_ERR_INVALID_ARG),      # I % 8
    ((FAKE, FAKE, FAKE, FAKE, 8, 8, 2000, 16, FAKE, FAKE, None), M.MOE_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, 16384, 32768, 2, 16, FAKE, FAKE, None), M.MOE_ERR_UNSUPPORTED),  # gate_up >= 2 GiB
    ((FAKE, FAKE, FAKE, FAKE, 16384, 32760, 2, 16, FAKE, None, None), M.MOE_ERR_INVALID_ARG),  # just below: h checked
    ((FAKE, None, FAKE, FAKE, 8, 8, 2, 16, FAKE, FAKE, None), M.MOE_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE_ODD, 8, 8, 2, 16, FAKE, FAKE, None), M.MOE_ERR_INVALID_ARG),
    ((None, None, None, None, 8, 8, 2, 0, None, None, None), M.MOE_OK),                    # no rows
])
def test_expert_ffn_rejects(args, want):
    assert M.lib().moe_expert_ffn(*args) == want


@pytest.mark.parametrize("args,want", [
    ((FAKE, FAKE, FAKE, 4, 8, 0, FAKE, None), M.MOE_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, 4, 8, 33, FAKE, None), M.MOE_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, 4, 6, 1, FAKE, None), M.MOE_ERR_INVALID_ARG),
    ((FAKE, FAKE, None, 4, 8, 1, FAKE, None), M.MOE_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, 4, 8, 1, FAKE_ODD, None), M.MOE_ERR_INVALID_ARG),
    ((None, None, None, 0, 8, 1, None, None), M.MOE_OK),
])
@pytest.mark.parametrize("name", ["moe_combine", "moe_combine_f32"])
def test_combine_rejects(name, args, want):
    assert getattr(M.lib(), name)(*args) == want


def _forward(name="moe_forward", **kw):
    a = dict(x=FAKE, w=FAKE, b=None, gu=FAKE, d=FAKE, T=8, H=8, I=8, E=4, k=2, e0=0, El=4, renorm=1, y=FAKE,
             ws=ctypes.c_void_p(0x100000), wsb=1 << 30)
    a.update(kw)
    return getattr(M.lib(), name)(a["x"], a["w"], a["b"], a["gu"], a["d"], a["T"], a["H"], a["I"], a["E"],
                                  a["k"], a["e0"], a["El"], a["renorm"], a["y"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(I=0), M.MOE_ERR_INVALID_ARG),
    (dict(I=12), M.MOE_ERR_INVALID_ARG),
    (dict(El=5), M.MOE_ERR_INVALID_ARG),
    (dict(e0=1), M.MOE_ERR_INVALID_ARG),
    (dict(y=None), M.MOE_ERR_INVALID_ARG),
    (dict(gu=FAKE_ODD), M.MOE_ERR_INVALID_ARG),
    (dict(w=FAKE_ODD), M.MOE_ERR_INVALID_ARG),
    (dict(wsb=1024), M.MOE_ERR_WORKSPACE),
    (dict(ws=None), M.MOE_ERR_WORKSPACE),
    (dict(k=0), M.MOE_ERR_INVALID_ARG),
    (dict(H=16384, I=32768), M.MOE_ERR_UNSUPPORTED),  # one expert's gate_up matrix >= 2 GiB
    (dict(T=0, x=None, y=None), M.MOE_OK),
])
@pytest.mark.parametrize("name", ["moe_forward", "moe_forward_f32", "moe_forward_fused"])
def test_forward_rejects(name, kw, want):
    assert _forward(name, **kw) == want


def test_noalloc_host_checks():
    """moe_forward_noalloc rejects bad arguments and problems larger than its
    static scratch on the host, before it looks up the device array."""
    L = M.lib()
    assert B.NOALLOC_SCRATCH_BYTES == 128 << 20
    args = [FAKE, FAKE, None, FAKE, FAKE]
    # T, H, I, E, k, e0, E_local, renormalize, y, stream
    assert L.moe_forward_noalloc(*args, 16, 64, 32, 8, 0, 0, 4, 1, FAKE, None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_forward_noalloc(*args, 16, 64, 32, 8, 2, 6, 4, 1, FAKE, None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_forward_noalloc(*args, 16, 64, 30, 8, 2, 0, 4, 1, FAKE, None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_forward_noalloc(*args, 0, 64, 32, 8, 2, 0, 4, 1, FAKE, None) == M.MOE_OK
    T, H, I, E, k, El = 16384, 7168, 2048, 256, 8, 32
    assert L.moe_forward_workspace_size(T, H, I, E, k, El) > B.NOALLOC_SCRATCH_BYTES
    assert L.moe_forward_noalloc(*args, T, H, I, E, k, 0, El, 1, FAKE, None) == M.MOE_ERR_WORKSPACE


# --------------------------------------------------------------------------- #
# The Python binding checks every tensor's dtype and shape before any launch:  #
# the library sees only pointers, so a wrong size would otherwise become an    #
# out-of-bounds access on the GPU. Shapes are checked before the device, so    #
# these CPU tensors are rejected for their shapes.                             #
# --------------------------------------------------------------------------- #
def _fwd_tensors(T=16, H=64, I=32, E=8, El=4):
    import torch
    bf = torch.bfloat16
    return dict(x=torch.zeros(T, H, dtype=bf), w_router=torch.zeros(E, H), bias=torch.zeros(E),
                w_gate_up=torch.zeros(El, H, 2 * I, dtype=bf), w_down=torch.zeros(El, I, H, dtype=bf))


@pytest.mark.parametrize("fn", ["moe_forward", "moe_forward_f32", "moe_forward_fused"])
@pytest.mark.parametrize("bad,match", [
    ("w_router", "w_router has shape"), ("bias", "bias has shape"), ("w_gate_up", "w_gate_up has shape"),
    ("w_down", "w_down has shape"), ("y", "y has shape"), ("k", "k must be"), ("e0", "local experts")])
def test_forward_rejects_mismatched_shapes(fn, bad, match):
    import torch
    t = _fwd_tensors()
    kw = dict(k=2, e0=0)
    if bad == "w_router":
        t["w_router"] = torch.zeros(8, 72)
    elif bad == "bias":
        t["bias"] = torch.zeros(9)
    elif bad == "w_gate_up":
        t["w_gate_up"] = torch.zeros(4, 56, 64, dtype=torch.bfloat16)
    elif bad == "w_down":
        t["w_down"] = torch.zeros(4, 32, 72, dtype=torch.bfloat16)
    elif bad == "y":
        kw["y"] = torch.zeros(16, 72, dtype=torch.float32 if fn == "moe_forward_f32" else torch.bfloat16)
    elif bad == "k":
        kw["k"] = 9
    elif bad == "e0":
        kw["e0"] = 5
    with pytest.raises(ValueError, match=match):
        getattr(M, fn)(t["x"], t["w_router"], t["bias"], t["w_gate_up"], t["w_down"], **kw)


def test_forward_rejects_wrong_dtype_and_device():
    import torch
    t = _fwd_tensors()
    with pytest.raises(TypeError, match="w_router must be"):
        M.moe_forward(t["x"], t["w_router"].double(), None, t["w_gate_up"], t["w_down"], 2, 0)
    with pytest.raises(ValueError, match="must live on a GPU"):
        M.moe_forward(t["x"], t["w_router"], None, t["w_gate_up"], t["w_down"], 2, 0)


def test_noalloc_and_profiled_reject_mismatched_shapes():
    import torch
    t = _fwd_tensors()
    with pytest.raises(ValueError, match="y has shape"):
        M.moe_forward_noalloc(t["x"], t["w_router"], None, t["w_gate_up"], t["w_down"], 2, 0,
                              y=torch.zeros(15, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="w_down has shape"):
        M.moe_forward_profiled(t["x"], t["w_router"], None, t["w_gate_up"], torch.zeros(4, 31, 64, dtype=torch.bfloat16),
                               2, 0, True, torch.zeros(16, 64, dtype=torch.bfloat16), torch.zeros(16, dtype=torch.uint8),
                               [None] * 6)


def test_route_rejects_mismatched_shapes():
    import torch
    x = torch.zeros(16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="w_router has shape"):
        M.moe_route(x, torch.zeros(8, 32), None, 2)
    with pytest.raises(ValueError, match="bias has shape"):
        M.moe_route(x, torch.zeros(8, 64), torch.zeros(7), 2)
    with pytest.raises(ValueError, match="k must be"):
        M.moe_route(x, torch.zeros(8, 64), None, 0)
    for name, bad in (("logits", torch.zeros(16, 7)), ("topk_idx", torch.zeros(16, 3, dtype=torch.int32)),
                      ("topk_w", torch.zeros(15, 2))):
        with pytest.raises(ValueError, match=f"{name} has shape"):
            M.moe_route(x, torch.zeros(8, 64), None, 2, **{name: bad})


def test_dispatch_rejects_mismatched_shapes():
    import torch
    x = torch.zeros(16, 64, dtype=torch.bfloat16)
    idx = torch.zeros(16, 2, dtype=torch.int32)
    with pytest.raises(ValueError, match="topk_idx has shape"):
        M.moe_dispatch(x, torch.zeros(15, 2, dtype=torch.int32), 8, 0, 4)
    with pytest.raises(ValueError, match="local experts"):
        M.moe_dispatch(x, idx, 8, 6, 4)
    with pytest.raises(ValueError, match="capacity"):
        M.moe_dispatch(x, idx, 8, 0, 4, capacity=31)
    for name, bad in (("counts", torch.zeros(7, dtype=torch.int32)), ("offsets", torch.zeros(4, dtype=torch.int32)),
                      ("perm_src", torch.zeros(31, dtype=torch.int32)), ("inv", torch.zeros(31, dtype=torch.int32)),
                      ("x_perm", torch.zeros(32, 56, dtype=torch.bfloat16))):
        with pytest.raises(ValueError, match=f"{name} has shape"):
            M.moe_dispatch(x, idx, 8, 0, 4, **{name: bad})


def test_expert_ffn_and_combine_reject_mismatched_shapes():
    import torch
    bf = torch.bfloat16
    xp = torch.zeros(32, 64, dtype=bf)
    gu = torch.zeros(4, 64, 64, dtype=bf)
    dn = torch.zeros(4, 32, 64, dtype=bf)
    off = torch.zeros(5, dtype=torch.int32)
    with pytest.raises(ValueError, match="w_gate_up has shape"):
        M.moe_expert_ffn(xp, off, torch.zeros(4, 72, 64, dtype=bf), dn)
    with pytest.raises(ValueError, match="w_down has shape"):
        M.moe_expert_ffn(xp, off, gu, torch.zeros(4, 32, 72, dtype=bf))
    with pytest.raises(ValueError, match="offsets has shape"):
        M.moe_expert_ffn(xp, torch.zeros(4, dtype=torch.int32), gu, dn)
    with pytest.raises(ValueError, match="h has shape"):
        M.moe_expert_ffn(xp, off, gu, dn, h=torch.zeros(32, 31, dtype=bf))
    with pytest.raises(ValueError, match="out has shape"):
        M.moe_expert_ffn(xp, off, gu, dn, out=torch.zeros(31, 64, dtype=bf))
    w = torch.zeros(16, 2)
    with pytest.raises(ValueError, match="inv has shape"):
        M.moe_combine(xp, torch.zeros(31, dtype=torch.int32), w)
    with pytest.raises(ValueError, match="y has shape"):
        M.moe_combine(xp, torch.zeros(32, dtype=torch.int32), w, y=torch.zeros(16, 56, dtype=bf))
    with pytest.raises(ValueError, match="y has shape"):
        M.moe_combine_f32(xp, torch.zeros(32, dtype=torch.int32), w, y=torch.zeros(15, 64))
