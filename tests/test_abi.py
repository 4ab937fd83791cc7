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
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below is rejected first
FAKE_ODD = ctypes.c_void_p(0x10002)  # not 16-byte aligned


def header_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(moe_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_library_exports_every_header_symbol():
    L = M.lib()
    names = header_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(L, n), f"libmoe.so lacks {n}"
    assert set(names) == set(B.SIGNATURES), (set(names) ^ set(B.SIGNATURES))


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
    ws = M.forward_workspace_size(T, H, I, E, k, El)
    cap = T * min(k, El)
    assert ws >= cap * H * 2 * 2 + cap * I * 2 + T * E * 4
    lay = M.forward_workspace_layout(T, H, I, E, k, El)
    offs = sorted(lay.values())
    assert all(o % 256 == 0 for o in offs)
    assert len(set(offs)) == len(offs) and offs[-1] < ws
    assert lay["expert_out"] + cap * H * 2 <= ws
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
