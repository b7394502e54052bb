"""The C ABI on the host: the library loads, exports every declared symbol,
and rejects invalid arguments with the documented status before touching
the device (these calls return before any HIP call, so no GPU is needed)."""

import ctypes
import os
import re

import pytest

import routed_expert_ffn_gemv_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20      # an aligned non-null address; never dereferenced here


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(moe.EXPORTS)
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    assert moe.status_string(0) == "ok"
    assert "workspace" in moe.status_string(3)
    assert moe.moe_version() >= 100


def _desc(**kw):
    d = moe.moe_layer_desc()
    d.E, d.k, d.H, d.I, d.num_slots = 512, 10, 2048, 768, 512
    d.router_fmt = moe.MOE_W_BF16
    d.router_w = FAKE
    for name in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
        m = getattr(d, name)
        m.fmt, m.data, m.scale, m.min = moe.MOE_W_Q2B32, FAKE, FAKE, FAKE
    for k_, v in kw.items():
        setattr(d, k_, v)
    return d


def _ws(d, T):
    n = ctypes.c_size_t(0)
    st = moe.lib.moe_workspace_size(ctypes.byref(d), T, ctypes.byref(n))
    return st, n.value


def test_workspace_size_valid():
    st, n = _ws(_desc(), 16)
    assert st == moe.MOE_OK and n > 0
    st0, n0 = _ws(_desc(), 0)
    assert st0 == moe.MOE_OK


@pytest.mark.parametrize("field,value,status", [
    ("k", 0, moe.MOE_ERR_INVALID),
    ("k", 513, moe.MOE_ERR_INVALID),
    ("k", 33, moe.MOE_ERR_UNSUPPORTED),
    ("E", 0, moe.MOE_ERR_INVALID),
    ("E", 2048, moe.MOE_ERR_UNSUPPORTED),
    ("H", 2000, moe.MOE_ERR_INVALID),
    ("H", 2080, moe.MOE_ERR_INVALID),        # q2 needs multiples of 64
    ("I", 16, moe.MOE_ERR_INVALID),
    ("num_slots", 0, moe.MOE_ERR_INVALID),
    ("num_slots", 100, moe.MOE_ERR_INVALID),  # identity table needs S == E
    ("router_fmt", 2, moe.MOE_ERR_UNSUPPORTED),
    ("router_w", None, moe.MOE_ERR_INVALID),
    ("router_w", FAKE + 2, moe.MOE_ERR_INVALID),
])
def test_invalid_desc(field, value, status):
    assert _ws(_desc(**{field: value}), 4)[0] == status


def test_invalid_pools():
    d = _desc()
    d.down.fmt = moe.MOE_W_Q4B32
    assert _ws(d, 4)[0] == moe.MOE_ERR_INVALID
    d = _desc()
    d.gate.scale = None
    assert _ws(d, 4)[0] == moe.MOE_ERR_INVALID
    d = _desc()
    d.up.data = FAKE + 8            # codes must be 16-byte aligned
    assert _ws(d, 4)[0] == moe.MOE_ERR_INVALID
    d = _desc()
    d.gate.fmt = d.up.fmt = d.down.fmt = moe.MOE_W_BF16
    assert _ws(d, 4)[0] == moe.MOE_ERR_UNSUPPORTED


def test_calls_validate_before_launch():
    d = _desc()
    st, n = _ws(d, 4)
    L = moe.lib
    ref = ctypes.byref(d)
    # T < 0, T too large for moe_layer, T = 0 no-op
    assert L.moe_route(ref, FAKE, -1, FAKE, FAKE, FAKE, n, None) == moe.MOE_ERR_INVALID
    assert L.moe_layer(ref, FAKE, 17, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n,
                       None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_route(ref, FAKE, 0, None, None, None, 0, None) == moe.MOE_OK
    assert L.moe_layer(ref, None, 0, None, None, None, None, None, None, None, 0,
                       None) == moe.MOE_OK
    # null outputs, short or misaligned workspace
    assert L.moe_route(ref, FAKE, 4, None, FAKE, FAKE, n, None) == moe.MOE_ERR_INVALID
    assert L.moe_route(ref, FAKE, 4, FAKE, FAKE, FAKE, n - 1, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_route(ref, FAKE, 4, FAKE, FAKE, FAKE + 64, n, None) == moe.MOE_ERR_INVALID
    assert L.moe_route(ref, FAKE, 4, FAKE, FAKE, None, n, None) == moe.MOE_ERR_INVALID
    assert L.moe_route(ref, FAKE + 2, 4, FAKE, FAKE, FAKE, n, None) == moe.MOE_ERR_INVALID
    assert L.moe_resolve_slots(ref, FAKE, FAKE, 4, FAKE, FAKE, FAKE, None, FAKE, FAKE, n,
                               None) == moe.MOE_ERR_INVALID
    assert L.moe_expert_ffn(ref, FAKE, 4, FAKE, FAKE, FAKE, None, FAKE, n,
                            None) == moe.MOE_ERR_INVALID      # shared expert needs shared_out
    assert L.moe_combine(ref, 4, FAKE, FAKE, FAKE, None, FAKE + 4, None) == moe.MOE_ERR_INVALID
    assert L.moe_layer(ref, FAKE, 4, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, n,
                       None) == moe.MOE_ERR_INVALID           # miss list is required
    assert L.moe_route(None, FAKE, 4, FAKE, FAKE, FAKE, n, None) == moe.MOE_ERR_INVALID


def _pool(**kw):
    p = moe.moe_slot_pool()
    p.L, p.E, p.H, p.I, p.num_slots = 48, 512, 2048, 768, 4176
    for name in ("gate", "up", "down", "store_gate", "store_up", "store_down"):
        m = getattr(p, name)
        m.fmt, m.data, m.scale, m.min = moe.MOE_W_Q2B32, FAKE, FAKE, FAKE
    p.usage, p.slot_of, p.expert_of = FAKE, FAKE, FAKE
    for k_, v in kw.items():
        setattr(p, k_, v)
    return p


def test_slot_refresh_validates_before_launch():
    L = moe.lib
    n = ctypes.c_size_t(7)
    assert L.moe_slot_refresh_workspace_size(ctypes.byref(_pool()), ctypes.byref(n)) == moe.MOE_OK
    assert n.value == 0
    ok = ctypes.byref(_pool())
    assert L.moe_slot_refresh(ok, 1025, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_slot_refresh(ok, -1, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_INVALID
    assert L.moe_slot_refresh(ok, 96, None, FAKE, None, 0, None) == moe.MOE_ERR_INVALID
    assert L.moe_slot_refresh(ok, 96, FAKE, None, None, 0, None) == moe.MOE_ERR_INVALID
    assert L.moe_slot_refresh(None, 96, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_INVALID
    for kw, status in [({"L": 200}, moe.MOE_ERR_UNSUPPORTED),       # L*E > 65536
                       ({"num_slots": 0}, moe.MOE_ERR_INVALID),
                       ({"num_slots": 20000}, moe.MOE_ERR_UNSUPPORTED),
                       ({"usage": None}, moe.MOE_ERR_INVALID),
                       ({"expert_of": None}, moe.MOE_ERR_INVALID),
                       ({"H": 2080}, moe.MOE_ERR_INVALID)]:
        assert L.moe_slot_refresh(ctypes.byref(_pool(**kw)), 96, FAKE, FAKE, None, 0,
                                  None) == status, kw
    p = _pool()
    p.store_down.fmt = moe.MOE_W_Q4B32                      # store and pool differ
    assert L.moe_slot_refresh(ctypes.byref(p), 96, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_INVALID


def test_verify_accept_validation():
    """Shapes and pointers are checked on the host before any launch."""
    import ctypes
    import routed_expert_ffn_gemv_amd as moe
    n = ctypes.c_size_t(0)
    assert moe.lib.moe_verify_workspace_size(0, 10, ctypes.byref(n)) == moe.MOE_ERR_INVALID
    assert moe.lib.moe_verify_workspace_size(4, 0, ctypes.byref(n)) == moe.MOE_ERR_INVALID
    assert moe.lib.moe_verify_workspace_size(65, 10, ctypes.byref(n)) == moe.MOE_ERR_UNSUPPORTED
    assert moe.lib.moe_verify_workspace_size(4, 151936, None) == moe.MOE_ERR_INVALID
    assert moe.lib.moe_verify_workspace_size(4, 151936, ctypes.byref(n)) == moe.MOE_OK
    assert n.value > 0 and n.value % 256 == 0
    fake = 1 << 20   # never dereferenced: every call below fails validation
    assert moe.lib.moe_verify_accept(None, 4, 100, fake, fake, fake, fake, 1 << 20,
                                     None) == moe.MOE_ERR_INVALID
    assert moe.lib.moe_verify_accept(fake, 4, 100, None, fake, fake, fake, 1 << 20,
                                     None) == moe.MOE_ERR_INVALID
    assert moe.lib.moe_verify_accept(fake, 4, 100, fake, fake, fake, fake + 8, 1 << 20,
                                     None) == moe.MOE_ERR_INVALID
    assert moe.lib.moe_verify_accept(fake, 4, 100, fake, fake, fake, fake, 8,
                                     None) == moe.MOE_ERR_WORKSPACE
