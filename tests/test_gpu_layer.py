"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Routing indices, slots, miss lists and buckets must be bit-exact; floating
outputs within 2e-3 relative error (normwise per token row).  Inputs carry a
routing margin (every gap among a token's top-(k+1) logits >= 1e-3)."""

import numpy as np
import pytest

import oracle
import synth
from helpers import (ORACLE_THREADS, TOL, DeviceLayer, check_routing, host,
                     rowwise_rel_err, say, small_cfg)

pytestmark = pytest.mark.gpu

SMALL = {
    # ragged shapes: partial row chunks, several units per expert, odd T
    "q2_ragged": small_cfg(E=40, k=3, H=192, I=128, T=7, bias="zipf", seed=11),
    "q4_ragged": small_cfg(E=24, k=5, H=96, I=160, T=13, wfmt="q4", shared=False, seed=12),
    "f32_ragged": small_cfg(E=9, k=4, H=96, I=32, T=3, wfmt="f32", router_fmt="f32",
                            shared=False, seed=13),
    "q2_k_eq_E": small_cfg(E=8, k=8, H=128, I=64, T=5, seed=14),
    "q4_T16": small_cfg(E=64, k=10, H=256, I=128, T=16, wfmt="q4", bias="zipf", seed=15),
    "c1": synth.CONFIGS["c1"],
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("path", ["layer", "steps"])
def test_small_layer(name, path):
    cfg = SMALL[name]
    say(f"[gpu] small layer {name} via {path}: E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I} T={cfg.T}")
    x, _ = oracle.margin_x(cfg, 0)
    L = DeviceLayer(cfg, 0, x=x)
    o = L.run_layer() if path == "layer" else L.run_steps()
    ref = L.oracle()
    check_routing(o, ref, cfg.k)
    assert rowwise_rel_err(host(o["y"]), ref["y"]) <= TOL
    if path == "steps":
        np.testing.assert_array_equal(host(o["bucket_off"]), ref["bucket_off"])
        np.testing.assert_array_equal(host(o["bucket_pair"])[: len(ref["bucket_pair"])],
                                      ref["bucket_pair"])
        hit = ref["slot_idx"].ravel() >= 0
        assert rowwise_rel_err(host(o["pair_out"])[hit], ref["pair_out"][hit]) <= TOL
        if cfg.shared:
            assert rowwise_rel_err(host(o["shared_out"]), ref["shared_out"]) <= TOL


# Shapes that take the fused launch (gate/up rows of whole 16-lane chunk
# sets, down rows of whole 4- or 8-lane sets), for every token-count bucket
# of the kernel, with and without the shared expert.
FUSED = {
    "q2_T1": small_cfg(E=64, k=8, H=1024, I=256, T=1, bias="zipf", seed=81),
    "q2_T1_E1024": small_cfg(E=1024, k=16, H=1024, I=256, T=1, bias="zipf", seed=88),
    "q4_T1_E300_k20": small_cfg(E=300, k=20, H=1024, I=256, T=1, wfmt="q4", seed=89),
    "q2_T3": small_cfg(E=64, k=8, H=1024, I=256, T=3, bias="zipf", seed=82),
    # up to four tokens outside the fast routing path (E > 512; k > 16, so
    # that the pairs outnumber a wave's lanes)
    "q2_T2_E600_k12": small_cfg(E=600, k=12, H=1024, I=256, T=2, bias="zipf", seed=90),
    "q4_T4_E300_k20": small_cfg(E=300, k=20, H=1024, I=256, T=4, wfmt="q4", seed=91),
    "q2_T9": small_cfg(E=96, k=6, H=1024, I=256, T=9, bias="zipf", seed=83),
    "q4_T16": small_cfg(E=64, k=10, H=1024, I=256, T=16, wfmt="q4", bias="zipf", seed=84),
    "q2_T16_no_shared": small_cfg(E=48, k=10, H=1024, I=256, T=16, shared=False, seed=85),
}


@pytest.mark.parametrize("name", list(FUSED))
def test_fused_small(name):
    cfg = FUSED[name]
    say(f"[gpu] fused small {name}: E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I} T={cfg.T}")
    x, _ = oracle.margin_x(cfg, 0)
    L = DeviceLayer(cfg, 0, x=x)
    o = L.run_layer()
    ref = L.oracle()
    check_routing(o, ref, cfg.k)
    assert rowwise_rel_err(host(o["y"]), ref["y"]) <= TOL


def test_fused_large_activations():
    """Activations 2^8 times larger (h near 10^5, beyond the fp16 range):
    the down projection's per-block scaling keeps the outputs within
    tolerance.  Routing comes from the bias alone (zero router weights), so
    the large activations do not reach the logits."""
    import torch
    cfg = small_cfg(E=64, k=8, H=1024, I=256, T=3, bias="zipf", seed=86)
    say("[gpu] fused layer, large activations")
    x, _ = oracle.margin_x(cfg, 0)
    f = (x.astype(np.uint32) << 16).view(np.float32) * np.float32(256.0)
    x = (f.view(np.uint32) >> 16).astype(np.uint16)          # exact: a power of two
    L = DeviceLayer(cfg, 0, x=x)
    bias = (np.random.default_rng(4).permutation(cfg.E) * 0.01).astype(np.float32)
    L.inp["router_w"].zero_()
    L.inp["bias"].copy_(torch.from_numpy(bias))
    o = L.run_layer()
    logits = oracle.router(x, np.zeros((cfg.E, cfg.H), np.uint16), cfg.router_fmt, bias)
    idx, gate = oracle.topk(logits, cfg.k)
    slot_idx, me, mt, mg, moff = oracle.resolve(idx, gate, cfg.E)
    route = {"logits": logits, "idx": idx, "gate": gate, "slot_idx": slot_idx,
             "miss_expert": me, "miss_token": mt, "miss_gate": mg, "miss_off": moff}
    ref = oracle.layer_from_synth(cfg, 0, x, route=route)
    check_routing(o, ref, cfg.k)
    y = host(o["y"])
    assert np.isfinite(y).all() and np.abs(ref["y"]).max() > 65504
    assert rowwise_rel_err(y, ref["y"]) <= TOL


def test_fused_tiered_small_with_misses():
    """The fused launch on a partial slot table: misses listed bit-exactly,
    y holds the hits."""
    cfg = small_cfg(E=64, k=6, H=1024, I=256, T=5, bias="zipf", seed=87)
    say("[gpu] fused tiered small layer with misses")
    x, _ = oracle.margin_x(cfg, 0)
    rng = np.random.default_rng(3)
    resident = np.sort(rng.choice(cfg.E, 24, replace=False))
    slot_of = np.full(cfg.E, -1, np.int32)
    slot_of[resident] = np.arange(len(resident))[::-1]
    from synth import device as sdev
    pool = sdev.expert_pool(cfg, [0] * len(resident),
                            [int(resident[len(resident) - 1 - s]) for s in range(len(resident))])
    L = DeviceLayer(cfg, 0, x=x, pool=pool, slot_of=slot_of, num_slots=len(resident))
    o = L.run_layer()
    ref = L.oracle()
    assert len(ref["miss_expert"]) > 0
    check_routing(o, ref, cfg.k)
    assert rowwise_rel_err(host(o["y"]), ref["y"]) <= TOL


def _tie_bias(pattern, E, seed):
    e = np.arange(E)
    if pattern == "levels":      # four values, ~E/4 experts each
        return (np.random.default_rng(seed).integers(0, 4, E) * 0.25).astype(np.float32)
    if pattern == "equal":
        return np.zeros(E, np.float32)
    if pattern == "crowd128":    # 224 equal leaders above one runner-up
        return np.where(e % 128 < 28, 2.0, np.where(e % 128 < 32, 1.5, 0.0)).astype(np.float32)
    if pattern == "crowd32":     # every 32nd expert ahead
        return np.where(e % 32 == 0, 1.0, 0.0).astype(np.float32)
    raise ValueError(pattern)


TIES = {
    "T1_levels": dict(E=512, k=10, T=1, pattern="levels"),
    "T3_equal": dict(E=256, k=8, T=3, pattern="equal"),
    # more keys at or above a token's threshold than the selection keeps
    "T3_crowd": dict(E=1024, k=8, T=3, pattern="crowd128"),
    "T9_crowd": dict(E=1024, k=10, T=9, pattern="crowd32"),
    "T4_k20": dict(E=64, k=20, T=4, pattern="levels"),
    # one token in the fused launch (H = 1024, I = 256): ties at the
    # threshold within 64 candidates, more than 64 candidates, k above the
    # threshold selection's limit, two logits per thread (E > 512)
    "T1_fused_crowd32": dict(E=1024, k=10, T=1, pattern="crowd32", H=1024, I=256),
    "T1_fused_crowd128": dict(E=1024, k=8, T=1, pattern="crowd128", H=1024, I=256),
    "T1_fused_levels": dict(E=512, k=10, T=1, pattern="levels", H=1024, I=256),
    "T1_fused_equal": dict(E=256, k=8, T=1, pattern="equal", H=1024, I=256),
    "T1_fused_k20": dict(E=64, k=20, T=1, pattern="levels", H=1024, I=256),
}


@pytest.mark.parametrize("name", list(TIES))
@pytest.mark.parametrize("path", ["layer", "steps"])
def test_tied_logits(name, path):
    """Exactly equal logits (zero router weights, bias on a few levels): the
    lower expert id wins every tie, bit for bit."""
    import torch
    c = TIES[name]
    cfg = small_cfg(E=c["E"], k=c["k"], H=c.get("H", 128), I=c.get("I", 64), T=c["T"],
                    bias="zipf", seed=41)
    say(f"[gpu] tied logits {name} via {path}: E={cfg.E} k={cfg.k} T={cfg.T}")
    L = DeviceLayer(cfg, 0)
    bias = _tie_bias(c["pattern"], cfg.E, 5)
    L.inp["router_w"].zero_()
    L.inp["bias"].copy_(torch.from_numpy(bias))
    o = L.run_layer() if path == "layer" else L.run_steps()
    logits = oracle.router(L.inp["x_host"], np.zeros((cfg.E, cfg.H), np.uint16),
                           cfg.router_fmt, bias)
    idx, gate = oracle.topk(logits, cfg.k)
    slot_idx, me, mt, mg, moff = oracle.resolve(idx, gate, cfg.E)
    route = {"logits": logits, "idx": idx, "gate": gate, "slot_idx": slot_idx,
             "miss_expert": me, "miss_token": mt, "miss_gate": mg, "miss_off": moff}
    ref = oracle.layer_from_synth(cfg, 0, L.inp["x_host"], route=route)
    check_routing(o, ref, cfg.k)
    assert rowwise_rel_err(host(o["y"]), ref["y"]) <= TOL


@pytest.mark.parametrize("shared", [True, False])
def test_fused_every_choice_its_own_expert(shared):
    """16 tokens, k = 16, every token on 16 experts of its own: 256 buckets of
    one token.  With the shared expert's four token groups that is more down
    buckets than a 256-workgroup grid holds (the contiguous split), without
    it exactly one workgroup per bucket."""
    import torch
    E, k, T, H = 512, 16, 16, 1024
    cfg = small_cfg(E=E, k=k, H=H, I=256, T=T, shared=shared, seed=47)
    say(f"[gpu] every choice its own expert: E={E} k={k} T={T} shared={shared}")
    # token t: a one-hot row at coordinate t; expert e: weight 1 + (e % 16) / 16
    # (exact in bf16) at coordinate e // 16, so token t's logits are those 16
    # distinct values on experts 16 t .. 16 t + 15 and zero elsewhere
    one = synth.bf16_bits(np.array([1.0]))[0]
    x = np.zeros((T, H), np.uint16)
    x[np.arange(T), np.arange(T)] = one
    W = np.zeros((E, H), np.uint16)
    e = np.arange(E)
    W[e, e // 16] = synth.bf16_bits(1.0 + (e % 16) / 16.0)
    L = DeviceLayer(cfg, 0, x=x)
    L.inp["router_w"].copy_(torch.from_numpy(W.view(np.int16)))
    o = L.run_layer()
    logits = oracle.router(x, W, cfg.router_fmt, None)
    idx, gate = oracle.topk(logits, k)
    assert len(np.unique(idx)) == T * k
    slot_idx, me, mt, mg, moff = oracle.resolve(idx, gate, E)
    route = {"logits": logits, "idx": idx, "gate": gate, "slot_idx": slot_idx,
             "miss_expert": me, "miss_token": mt, "miss_gate": mg, "miss_off": moff}
    ref = oracle.layer_from_synth(cfg, 0, x, route=route)
    check_routing(o, ref, k)
    assert rowwise_rel_err(host(o["y"]), ref["y"]) <= TOL


def test_tiered_small_with_misses():
    """A partial slot table: misses listed bit-exactly; y holds hits only and
    y + sum over misses of gate * FFN equals the all-resident layer."""
    cfg = small_cfg(E=32, k=4, H=128, I=64, T=9, bias="zipf", seed=21)
    say("[gpu] tiered small layer with misses")
    x, _ = oracle.margin_x(cfg, 0)
    resident = [1, 3, 4, 8, 9, 15, 16, 20, 27, 31]
    slot_of = np.full(cfg.E, -1, np.int32)
    slot_of[resident] = np.arange(len(resident))[::-1]      # slots not in id order
    from synth import device as sdev
    pool = sdev.expert_pool(cfg, [0] * len(resident), [resident[len(resident) - 1 - s]
                                                          for s in range(len(resident))])
    L = DeviceLayer(cfg, 0, x=x, pool=pool, slot_of=slot_of, num_slots=len(resident))
    for path in ("layer", "steps"):
        o = L.run_layer() if path == "layer" else L.run_steps()
        ref = L.oracle(with_misses=True)
        assert len(ref["miss_expert"]) > 0
        check_routing(o, ref, cfg.k)
        assert rowwise_rel_err(host(o["y"]), ref["y"]) <= TOL
    # completion invariant on the GPU's partial output
    y = host(o["y"]).astype(np.float64)
    for e, t, g in zip(ref["miss_expert"], ref["miss_token"], ref["miss_gate"]):
        y[t] += g * oracle.ffn(cfg.wfmt, cfg.H, cfg.I, synth.gen_expert(cfg, 0, int(e)),
                               L.inp["x_host"][t:t + 1])[0]
    assert rowwise_rel_err(y, ref["y_full"]) <= TOL


def test_all_miss_table():
    cfg = small_cfg(E=16, k=3, H=64, I=64, T=5, seed=22)
    say("[gpu] all-miss slot table")
    x, _ = oracle.margin_x(cfg, 0)
    slot_of = np.full(cfg.E, -1, np.int32)
    from synth import device as sdev
    pool = sdev.expert_pool(cfg, [0], [0])
    L = DeviceLayer(cfg, 0, x=x, pool=pool, slot_of=slot_of, num_slots=1)
    o = L.run_layer()
    ref = L.oracle()
    check_routing(o, ref, cfg.k)
    assert len(ref["miss_expert"]) == cfg.T * cfg.k
    assert rowwise_rel_err(host(o["y"]), ref["y"]) <= TOL   # shared expert only


def _tiered_small():
    """A partial slot table (24 of 64 experts resident): (cfg, layer kwargs)."""
    cfg = small_cfg(E=64, k=6, H=1024, I=256, T=5, bias="zipf", seed=87)
    rng = np.random.default_rng(3)
    resident = np.sort(rng.choice(cfg.E, 24, replace=False))
    slot_of = np.full(cfg.E, -1, np.int32)
    slot_of[resident] = np.arange(len(resident))[::-1]
    from synth import device as sdev
    pool = sdev.expert_pool(cfg, [0] * len(resident),
                            [int(resident[len(resident) - 1 - s]) for s in range(len(resident))])
    return cfg, dict(pool=pool, slot_of=slot_of, num_slots=len(resident))


DET_CASES = ["q2_T1", "q2_T9", "q4_T16", "q2_T16_no_shared", "tiered_misses", "c2", "c3"]


@pytest.mark.parametrize("name", DET_CASES)
def test_fused_deterministic_sums(name):
    """moe_set_deterministic: every element of y is summed by one thread in
    choice order (hits only), then the shared expert.  Two calls on one
    workspace give bit-identical y, every element written (y starts as
    NaN), within tolerance of the oracle; the atomic-sum mode agrees within
    tolerance."""
    import torch
    import routed_expert_ffn_gemv_amd as moe
    kw = {}
    if name == "tiered_misses":
        cfg, kw = _tiered_small()
    elif name in ("c2", "c3"):
        cfg = synth.CONFIGS[name]
    else:
        cfg = FUSED[name]
    say(f"[gpu] fixed-order sums {name}: E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I} T={cfg.T}")
    x, _ = oracle.margin_x(cfg, 0)
    L = DeviceLayer(cfg, 0, x=x, **kw)
    ws = moe.workspace(L.desc, L.T)
    moe.moe_set_deterministic(True)
    try:
        o1 = L.run_layer(ws)
        o2 = L.run_layer(ws)
    finally:
        moe.moe_set_deterministic(False)
    o3 = L.run_layer(ws)
    moe.moe_layer_check(ws)
    ref = L.oracle()
    for o in (o1, o2, o3):
        check_routing(o, ref, cfg.k)
    y1, y2 = host(o1["y"]), host(o2["y"])
    assert np.isfinite(y1).all()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    err = rowwise_rel_err(y1, ref["y"])
    say(f"  rel err {err:.2e} (atomic sums: {rowwise_rel_err(host(o3['y']), ref['y']):.2e})")
    assert err <= TOL
    assert rowwise_rel_err(host(o3["y"]), ref["y"]) <= TOL


def test_c2_decode_layer():
    """The decode layer at full size, the launch bench.py times (moe_layer, T=1)."""
    cfg = synth.CONFIGS["c2"]
    say("[gpu] c2 decode layer E=512 k=10 H=2048 I=768 q2 + shared, T=1")
    for layer in (0, 1):
        x, _ = oracle.margin_x(cfg, layer)
        L = DeviceLayer(cfg, layer, x=x)
        o = L.run_layer()
        ref = L.oracle()
        check_routing(o, ref, cfg.k)
        err = rowwise_rel_err(host(o["y"]), ref["y"])
        say(f"  layer {layer}: rel err {err:.2e}")
        assert err <= TOL


WAIT_CASES = {"c2_T1": synth.CONFIGS["c2"],
              "q2_T9": small_cfg(E=96, k=6, H=1024, I=256, T=9, bias="zipf", seed=83)}


@pytest.mark.parametrize("name", list(WAIT_CASES))
def test_fused_wait_gives_up_and_poisons_workspace(name):
    """The fused launch's waits are bounded.  With the test hold set,
    workgroup 0 first waits on a word nothing writes: the launch gives up
    after its budget (1 ms here) instead of hanging, every workgroup exits,
    and moe_layer_check reports MOE_ERR_DEVICE.  Later calls on the
    poisoned workspace write nothing; once the workspace is zeroed again,
    calls match the oracle."""
    import torch
    import routed_expert_ffn_gemv_amd as moe
    cfg = WAIT_CASES[name]
    say(f"[gpu] bounded waits ({name}): forced give-up, poisoned workspace, recovery")
    x, _ = oracle.margin_x(cfg, 0)
    L = DeviceLayer(cfg, 0, x=x)
    ref = L.oracle()
    ws = moe.workspace(L.desc, cfg.T)
    o = L.run_layer(ws)
    moe.moe_layer_check(ws)
    check_routing(o, ref, cfg.k)
    try:
        moe.moe_set_wait_budget(1_000_000, hold=True)
        L.run_layer(ws)
        torch.cuda.synchronize()
    finally:
        moe.moe_set_wait_budget(0, hold=False)
    with pytest.raises(moe.MoEError) as err:
        moe.moe_layer_check(ws)
    assert err.value.status == moe.MOE_ERR_DEVICE
    o = L.run_layer(ws)
    torch.cuda.synchronize()
    assert torch.isnan(o["y"]).all() and bool((o["idx"] == -7).all())
    with pytest.raises(moe.MoEError):
        moe.moe_layer_check(ws)
    ws.zero_()
    o = L.run_layer(ws)
    moe.moe_layer_check(ws)
    check_routing(o, ref, cfg.k)
    assert rowwise_rel_err(host(o["y"]), ref["y"]) <= TOL


def test_repeated_calls_share_one_workspace():
    """Back-to-back fused calls on one workspace (counters and flag are
    reused across calls), alternating layers and token counts."""
    import routed_expert_ffn_gemv_amd as moe
    cfg = small_cfg(E=64, k=6, H=256, I=128, T=16, bias="zipf", seed=31)
    say("[gpu] repeated moe_layer calls on one workspace")
    layers = []
    for l in range(3):
        x, _ = oracle.margin_x(cfg, l)
        layers.append(DeviceLayer(cfg, l, x=x))
    ws = moe.workspace(layers[0].desc, cfg.T)
    refs = [L.oracle() for L in layers]
    for rep in range(3):
        for l, L in enumerate(layers):
            o = L.run_layer(ws)
            check_routing(o, refs[l], cfg.k)
            assert rowwise_rel_err(host(o["y"]), refs[l]["y"]) <= TOL


def _float_layers(cfg, must, n=8, seed=7):
    """n layers for the float checks: the ones named in `must` plus seeded
    picks from the rest."""
    rest = [l for l in range(cfg.layers) if l not in must]
    pick = np.random.default_rng(seed).choice(rest, n - len(must), replace=False)
    return sorted(set(must) | set(int(v) for v in pick))


def test_c3_verify_stack_all_layers():
    """4-token verify batch through all 48 full-size layers of the stack
    (Zipf-biased routing, all experts resident), moe_layer as bench.py times
    it: every layer's indices, slots and miss lists bit-exact and gates within
    tolerance; y of 8 layers (the first and the last among them) within
    tolerance."""
    cfg = synth.CONFIGS["c3"]
    floats = _float_layers(cfg, [0, cfg.layers - 1])
    say(f"[gpu] c3 stack: routing of all {cfg.layers} layers, floats on layers {floats}")
    for layer in range(cfg.layers):
        x, _ = oracle.margin_x(cfg, layer)
        L = DeviceLayer(cfg, layer, x=x)
        o = L.run_layer()
        r = oracle.route_from_synth(cfg, layer, x)
        check_routing(o, r, cfg.k)
        msg = f"  c3 layer {layer}: routing exact, distinct experts {len(np.unique(r['idx']))}"
        if layer in floats:
            ref = oracle.layer_from_synth(cfg, layer, x, route=r, threads=ORACLE_THREADS)
            err = rowwise_rel_err(host(o["y"]), ref["y"])
            msg += f", rel err {err:.2e}"
            assert err <= TOL, msg
        say(msg)
        del L, o


def test_c4_slot_tiering_all_layers():
    """16 tokens per layer against the 4,176-expert global slot table, all 48
    layers: every layer's indices, slots and miss lists (expert, token,
    offsets) bit-exact; on 8 layers -- among them the smallest (57) and the
    largest (109) resident sets -- y (hits only) within tolerance and the
    completion invariant y + sum of the listed misses' gate * FFN = the
    all-resident layer."""
    from synth import device as sdev
    cfg = synth.CONFIGS["c4"]
    slot_of, sl, se, S = synth.slot_layout(cfg)
    n_l = (slot_of >= 0).sum(axis=1)
    lo, hi = int(np.argmin(n_l)), int(np.argmax(n_l))
    assert n_l[lo] == 57 and n_l[hi] == 109
    floats = _float_layers(cfg, [lo, hi, 0, cfg.layers - 1])
    say(f"[gpu] c4: filling the global pool of {S} slots; floats on layers {floats}")
    pool = sdev.expert_pool(cfg, sl, se)
    for layer in range(cfg.layers):
        x, _ = oracle.margin_x(cfg, layer)
        L = DeviceLayer(cfg, layer, x=x, pool=pool, slot_of=slot_of[layer], num_slots=S)
        o = L.run_layer()
        r = oracle.route_from_synth(cfg, layer, x, slot_of=slot_of[layer], num_slots=S)
        check_routing(o, r, cfg.k)
        hit = (r["slot_idx"] >= 0).mean()
        msg = (f"  c4 layer {layer}: resident {int(n_l[layer])}, routing and miss list exact, "
               f"hit rate {hit:.2f}, misses {len(r['miss_expert'])}")
        if layer in floats:
            ref = oracle.layer_from_synth(cfg, layer, x, slot_of=slot_of[layer], num_slots=S,
                                          with_misses=True, route=r, threads=ORACLE_THREADS)
            y = host(o["y"]).astype(np.float64)
            err = rowwise_rel_err(y, ref["y"])
            for e, t, g in zip(ref["miss_expert"], ref["miss_token"], ref["miss_gate"]):
                y[t] += g * ref["pair_out"][t * cfg.k + list(ref["idx"][t]).index(e)]
            err_full = rowwise_rel_err(y, ref["y_full"])
            msg += f", rel err {err:.2e}, completed {err_full:.2e}"
            assert err <= TOL and err_full <= TOL, msg
        say(msg)
        del L, o


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_separate_calls_full_size(name):
    """The four separate calls (moe_route, moe_resolve_slots, moe_expert_ffn,
    moe_combine) at the decode (T = 1) and verify (T = 4) shapes, H = 2048,
    I = 768: the router GEMV, the one-block resolution and the dequant-fused
    gate/up and down GEMVs at full width.  Indices, slots, miss lists and
    buckets bit-exact; pair outputs, shared-expert outputs and y within
    tolerance."""
    cfg = synth.CONFIGS[name]
    layer = 3
    say(f"[gpu] separate calls at full size: {cfg.name} layer {layer}")
    x, _ = oracle.margin_x(cfg, layer)
    L = DeviceLayer(cfg, layer, x=x)
    o = L.run_steps()
    ref = oracle.layer_from_synth(cfg, layer, x, threads=ORACLE_THREADS)
    check_routing(o, ref, cfg.k)
    np.testing.assert_array_equal(host(o["bucket_off"]), ref["bucket_off"])
    np.testing.assert_array_equal(host(o["bucket_pair"])[: len(ref["bucket_pair"])],
                                  ref["bucket_pair"])
    hit = ref["slot_idx"].ravel() >= 0
    e_pair = rowwise_rel_err(host(o["pair_out"])[hit], ref["pair_out"][hit])
    e_sh = rowwise_rel_err(host(o["shared_out"]), ref["shared_out"])
    e_y = rowwise_rel_err(host(o["y"]), ref["y"])
    say(f"  rel err: pairs {e_pair:.2e}, shared {e_sh:.2e}, y {e_y:.2e}")
    assert max(e_pair, e_sh, e_y) <= TOL
