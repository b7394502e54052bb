"""moe_layer_noalloc -- the fused launch on the library's static hand-off
region, for callers that cannot allocate -- against moe_layer with a caller
workspace, through the C ABI."""

import numpy as np
import pytest

import oracle
import synth
from helpers import (ORACLE_THREADS, TOL, DeviceLayer, check_routing, host, rowwise_rel_err,
                     say, small_cfg)

pytestmark = pytest.mark.gpu


def _noalloc(L):
    import routed_expert_ffn_gemv_amd as moe
    o = L.outputs()
    moe.moe_layer_noalloc(L.desc, L.inp["x"], L.T, o["y"], o["idx"], o["gate"], o["slot_idx"],
                          o["miss"], o["miss_off"])
    return o


def test_noalloc_matches_moe_layer():
    """Two calls in a row, the second with a smaller input: a 4-token verify
    layer of the stack's shape, then a one-token decode layer.  Each against
    moe_layer with a workspace: indices, gates, slots and miss lists equal
    bit for bit, y within tolerance of it (the fused launch sums experts in
    no fixed order) and of the oracle."""
    import torch
    import routed_expert_ffn_gemv_amd as moe
    for cfg, layer in ((synth.CONFIGS["c3"], 5), (synth.CONFIGS["c2"], 2)):
        say(f"[gpu] noalloc: {cfg.name} layer {layer}, T={cfg.T}")
        x, _ = oracle.margin_x(cfg, layer)
        L = DeviceLayer(cfg, layer, x=x)
        o = _noalloc(L)
        moe.moe_layer_check(None)
        w = L.run_layer()
        torch.cuda.synchronize()
        for key in ("idx", "gate", "slot_idx", "miss_off"):
            np.testing.assert_array_equal(host(o[key]), host(w[key]))
        n = int(host(w["miss_off"])[-1])
        np.testing.assert_array_equal(host(o["miss"])[: 3 * n], host(w["miss"])[: 3 * n])
        err_w = rowwise_rel_err(host(o["y"]), host(w["y"]).astype(np.float64))
        ref = oracle.layer_from_synth(cfg, layer, x, threads=ORACLE_THREADS)
        check_routing(o, ref, cfg.k)
        err = rowwise_rel_err(host(o["y"]), ref["y"])
        say(f"  against moe_layer {err_w:.2e}, against the oracle {err:.2e}")
        assert err_w <= TOL and err <= TOL


def test_noalloc_fixed_order_matches_moe_layer_bit_for_bit():
    """With fixed-order sums (moe_set_deterministic) y no longer depends on
    the order of the float additions: noalloc and moe_layer give the same y
    bit for bit, again on two calls in a row, the second smaller."""
    import torch
    import routed_expert_ffn_gemv_amd as moe
    moe.moe_set_deterministic(True)
    try:
        for cfg, layer in ((synth.CONFIGS["c3"], 7), (synth.CONFIGS["c2"], 3)):
            say(f"[gpu] noalloc, fixed-order sums: {cfg.name} layer {layer}, T={cfg.T}")
            x, _ = oracle.margin_x(cfg, layer)
            L = DeviceLayer(cfg, layer, x=x)
            o = _noalloc(L)
            moe.moe_layer_check(None)
            w = L.run_layer()
            torch.cuda.synchronize()
            yo, yw = host(o["y"]), host(w["y"])
            assert np.isfinite(yo).all()
            assert np.array_equal(yo.view(np.uint32), yw.view(np.uint32))
            for key in ("idx", "gate", "slot_idx", "miss_off"):
                np.testing.assert_array_equal(host(o[key]), host(w[key]))
    finally:
        moe.moe_set_deterministic(False)


def test_noalloc_rejects_unfused_shapes():
    """A shape moe_layer runs as separate steps (T * k > 256) needs a
    workspace: MOE_ERR_UNSUPPORTED, nothing launched."""
    import torch
    import routed_expert_ffn_gemv_amd as moe
    cfg = small_cfg(E=64, k=20, H=256, I=128, T=16, seed=91)
    L = DeviceLayer(cfg, 0)
    with pytest.raises(moe.MoEError) as err:
        _noalloc(L)
    assert err.value.status == moe.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()


def test_noalloc_gives_up_and_recovers():
    """A noalloc call that runs out of its wait budget (test hold) marks the
    static region failed; moe_layer_check(None) reports it and clears the
    region, after which calls match the oracle again."""
    import torch
    import routed_expert_ffn_gemv_amd as moe
    cfg = small_cfg(E=64, k=8, H=1024, I=256, T=3, bias="zipf", seed=82)
    x, _ = oracle.margin_x(cfg, 0)
    L = DeviceLayer(cfg, 0, x=x)
    ref = L.oracle()
    try:
        moe.moe_set_wait_budget(1_000_000, hold=True)
        _noalloc(L)
        torch.cuda.synchronize()
    finally:
        moe.moe_set_wait_budget(0, hold=False)
    with pytest.raises(moe.MoEError) as err:
        moe.moe_layer_check(None)
    assert err.value.status == moe.MOE_ERR_DEVICE
    moe.moe_layer_check(None)   # cleared by the check above
    o = _noalloc(L)
    moe.moe_layer_check(None)
    check_routing(o, ref, cfg.k)
    assert rowwise_rel_err(host(o["y"]), ref["y"]) <= TOL
