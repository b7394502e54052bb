"""Pins of the fp64 oracle to facts outside itself: hand-packed blocks,
closed forms, brute force, special cases and invariants (CPU only).

Each test names the kind of mistake it would catch."""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _bf16(vals):
    return synth.bf16_bits(np.asarray(vals, np.float64))


# ------------------------------------------------------------ number formats
@pytest.mark.parametrize("bits,val", [
    (0x3F80, 1.0), (0xC000, -2.0), (0x4049, 3.140625), (0x0000, 0.0),
    (0x0001, 2.0 ** -133), (0x7F7F, 3.3895313892515355e38), (0x3C00, 2.0 ** -7)])
def test_bf16_decoding(bits, val):
    assert oracle.bf16(bits) == val


@pytest.mark.parametrize("bits,val", [
    (0x3C00, 1.0), (0xC000, -2.0), (0x7BFF, 65504.0), (0x0001, 2.0 ** -24),
    (0x0400, 2.0 ** -14), (0x3555, 0.333251953125), (0x03FF, 1023 * 2.0 ** -24),
    (0x1400, 2.0 ** -10)])
def test_f16_decoding(bits, val):
    # catches a wrong exponent bias or a missing subnormal branch
    assert oracle.f16(bits) == val


def test_f16_negative_zero_sign():
    assert math.copysign(1.0, oracle.f16(0x8000)) == -1.0


# ------------------------------------------------------------ dequantisation
def _pack_rows(row_bytes):
    rows = []
    for spec in row_bytes:
        r = []
        for i in range(0, len(spec), 2):
            r += [int(spec[i], 16)] * spec[i + 1]
        rows.append(r)
    return np.array(rows, np.uint8).ravel()


@pytest.mark.parametrize("fmt", ["q2", "q4"])
def test_dequant_hand_packed(fmt):
    """Bit order inside a byte, block indexing of scale/min and the affine
    form d*q + m against hand-derived values."""
    g = _gold("dequant_blocks.json")[fmt]
    rows, cols = g["rows"], g["cols"]
    codes = _pack_rows(g["row_bytes"])
    scale = np.array([int(s, 16) for s in g["scale"]], np.uint16)
    mn = np.array([int(s, 16) for s in g["min"]], np.uint16)
    w = oracle.dequant(fmt, rows, cols, codes, scale, mn)
    for r in range(rows):
        for b in range(cols // 32):
            pat = g["expected"][r][b]
            want = np.array(pat * (32 // len(pat)))
            np.testing.assert_array_equal(w[r, 32 * b: 32 * b + 32], want)


def test_dequant_roundtrip_random_codes():
    """Pack random codes by the layout rule, unpack with the oracle: codes
    come back exactly (d = 1, m = 0), for both widths."""
    rng = np.random.default_rng(7)
    for bits, fmt in ((2, "q2"), (4, "q4")):
        rows, cols = 3, 96
        q = rng.integers(0, 1 << bits, (rows, cols))
        per = 8 // bits
        packed = np.zeros((rows, cols // per), np.uint8)
        for c in range(cols):
            packed[:, c // per] |= (q[:, c] << (bits * (c % per))).astype(np.uint8)
        one = np.full(rows * cols // 32, 0x3C00, np.uint16)
        zero = np.zeros(rows * cols // 32, np.uint16)
        w = oracle.dequant(fmt, rows, cols, packed.ravel(), one, zero)
        np.testing.assert_array_equal(w, q.astype(np.float64))


def test_dequant_f32_identity():
    a = np.arange(12, dtype=np.float32).reshape(3, 4) - 5.5
    np.testing.assert_array_equal(oracle.dequant("f32", 3, 4, a), a.astype(np.float64))


# ------------------------------------------------------------ router
def test_router_onehot_and_bias():
    """W one-hot picks single activations exactly; the bias is added (catches
    a dropped bias or transposed W)."""
    H, E = 8, 5
    x = _bf16(np.array([[0.5, -1.0, 2.0, 3.0, -0.25, 1.5, 7.0, -4.0]]))
    W = np.zeros((E, H), np.float32)
    for e, h in enumerate([2, 0, 7, 3, 6]):
        W[e, h] = 1.0
    bias = np.array([0.0, 1.0, -2.0, 0.5, 0.0], np.float32)
    l = oracle.router(x, W, "f32", bias)
    np.testing.assert_array_equal(l[0], [2.0, 1.5, -6.0, 3.5, 7.0])
    Wb = synth.bf16_bits(W.astype(np.float64))
    np.testing.assert_array_equal(oracle.router(x, Wb, "bf16", None)[0], [2.0, 0.5, -4.0, 3.0, 7.0])


def test_router_small_dot_products():
    x = _bf16([[1.0, 2.0, 3.0]])
    W = np.array([[1.0, 1.0, 1.0], [0.5, -0.25, 2.0]], np.float32)
    np.testing.assert_array_equal(oracle.router(x, W, "f32")[0], [6.0, 6.0])


# ------------------------------------------------------------ top-k
def _rank_topk(l, k):
    """Independent definition: an expert's rank is the number of experts with
    a larger logit, or an equal logit and a smaller id."""
    E = len(l)
    rank = [sum(1 for f in range(E) if l[f] > l[e] or (l[f] == l[e] and f < e))
            for e in range(E)]
    return [rank.index(r) for r in range(k)]


def test_topk_exhaustive_ties():
    """Every logit vector over {0,1,2}^6 and every k: order and tie rule
    (lower id first) against the rank definition."""
    E = 6
    vecs = np.array(list(itertools.product([0.0, 1.0, 2.0], repeat=E)))
    for k in range(1, E + 1):
        idx, _ = oracle.topk(vecs, k)
        for v, got in zip(vecs, idx):
            assert list(got) == _rank_topk(list(v), k)


def test_topk_negative_zero_ties_positive_zero():
    l = np.array([[0.0, -0.0, -1.0, -0.0, 0.0]])
    idx, _ = oracle.topk(l, 3)
    assert list(idx[0]) == [0, 1, 3]


def test_topk_random_against_rank_definition():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((50, 16))
    idx, _ = oracle.topk(l, 4)
    for v, got in zip(l, idx):
        assert list(got) == _rank_topk(list(v), 4)


# ------------------------------------------------------------ gates
def test_gates_sum_to_one_and_ratio():
    """Softmax over the selected logits only: sum is 1 and the ratio of two
    gates is exp of their logit difference (catches a softmax over all E)."""
    rng = np.random.default_rng(4)
    l = rng.standard_normal((20, 32))
    idx, g = oracle.topk(l, 5)
    np.testing.assert_allclose(g.sum(1), 1.0, rtol=0, atol=1e-14)
    for t in range(20):
        sel = l[t, idx[t]]
        np.testing.assert_allclose(np.log(g[t, 0] / g[t, 1:]), sel[0] - sel[1:], atol=1e-12)
        assert np.all(np.diff(g[t]) <= 0)


def test_gates_closed_form_two_experts():
    l = np.array([[math.log(2.0), 0.0, -5.0]])
    idx, g = oracle.topk(l, 2)
    assert list(idx[0]) == [0, 1]
    np.testing.assert_allclose(g[0], [2.0 / 3.0, 1.0 / 3.0], rtol=1e-15)


def test_gates_k1_is_one():
    _, g = oracle.topk(np.random.default_rng(5).standard_normal((7, 9)), 1)
    assert np.all(g == 1.0)


def test_zero_router_gives_first_ids_and_uniform_gates():
    H, E, k = 64, 16, 4
    x = _bf16(np.random.default_rng(6).standard_normal((3, H)))
    l = oracle.router(x, np.zeros((E, H), np.float32), "f32")
    idx, g = oracle.topk(l, k)
    assert np.all(idx == np.arange(k))
    assert np.all(g == 1.0 / k)


# ------------------------------------------------------------ resolve / buckets
def _idx_gate(T, k, E, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    gate = rng.random((T, k))
    return idx, gate


def test_resolve_identity_has_no_misses():
    idx, gate = _idx_gate(5, 3, 10, 1)
    slot_idx, me, mt, mg, moff = oracle.resolve(idx, gate, 10, None)
    np.testing.assert_array_equal(slot_idx, idx)
    assert len(me) == 0 and np.all(moff == 0)


def test_resolve_empty_table_misses_everything_in_order():
    T, k, E = 4, 3, 10
    idx, gate = _idx_gate(T, k, E, 2)
    slot_of = np.full(E, -1, np.int32)
    slot_idx, me, mt, mg, moff = oracle.resolve(idx, gate, E, slot_of)
    assert np.all(slot_idx == -1)
    np.testing.assert_array_equal(me, idx.ravel())
    np.testing.assert_array_equal(mt, np.repeat(np.arange(T), k))
    np.testing.assert_array_equal(mg, gate.ravel())
    np.testing.assert_array_equal(moff, np.arange(T + 1) * k)


def test_resolve_partial_table_counts_and_offsets():
    T, k, E = 6, 4, 12
    idx, gate = _idx_gate(T, k, E, 3)
    slot_of = np.full(E, -1, np.int32)
    resident = [1, 4, 5, 9, 11]
    slot_of[resident] = np.arange(len(resident)) + 100
    slot_idx, me, mt, mg, moff = oracle.resolve(idx, gate, E, slot_of)
    hits = (slot_idx >= 0).sum()
    assert hits + len(me) == T * k
    for t in range(T):
        want = [(int(e), t) for e in idx[t] if e not in resident]
        got = list(zip(me[moff[t]:moff[t + 1]].tolist(), mt[moff[t]:moff[t + 1]].tolist()))
        assert got == want
    np.testing.assert_array_equal(slot_idx, slot_of[idx])


def test_bucket_is_stable_permutation():
    rng = np.random.default_rng(8)
    T, k, S = 9, 5, 7
    slot_idx = rng.integers(-1, S, (T, k)).astype(np.int32)
    off, pairs = oracle.bucket(slot_idx, S)
    flat = slot_idx.ravel()
    want = sorted((int(flat[p]), p) for p in range(T * k) if flat[p] >= 0)
    assert pairs.tolist() == [p for _, p in want]
    counts = np.bincount(flat[flat >= 0], minlength=S)
    np.testing.assert_array_equal(np.diff(off), counts)


# ------------------------------------------------------------ FFN
def test_ffn_hand_worked():
    """silu on the gate projection (not the up), D not transposed."""
    g = _gold("ffn_hand.json")
    ex = {m: {"w": np.array(g[k], np.float32)} for m, k in (("gate", "G"), ("up", "U"), ("down", "D"))}
    x = np.array([[int(v, 16) for v in g["x_bf16"]]], np.uint16)
    o = oracle.ffn("f32", 2, 2, ex, x)
    np.testing.assert_allclose(o[0], g["expected_o"], rtol=1e-15)


def test_ffn_zero_gate_gives_zero():
    """silu(0) = 0: an expert whose gate rows dequantise to 0 outputs 0."""
    cfg = synth.CONFIGS["c2"]
    ex = synth.gen_expert(synth.MoEConfig(**{**cfg.__dict__, "H": 64, "I": 32}), 0, 5)
    ex["gate"]["scale"][:] = 0
    ex["gate"]["min"][:] = 0
    x = _bf16(np.random.default_rng(9).standard_normal((2, 64)))
    assert np.all(oracle.ffn("q2", 64, 32, ex, x) == 0.0)


def test_ffn_q_matches_dense_f32_of_dequantised():
    """The quantised FFN equals the fp32 FFN on exactly-representable
    dequantised weights (2-bit values d*q+m are exact in fp32 here)."""
    small = synth.MoEConfig(**{**synth.CONFIGS["c2"].__dict__, "H": 64, "I": 32})
    ex = synth.gen_expert(small, 0, 11)
    dense = {}
    for m in ("gate", "up", "down"):
        rows, cols = (32, 64) if m != "down" else (64, 32)
        w = oracle.dequant("q2", rows, cols, ex[m]["codes"], ex[m]["scale"], ex[m]["min"])
        assert np.all(w.astype(np.float32) == w)
        dense[m] = {"w": w.astype(np.float32)}
    x = _bf16(np.random.default_rng(10).standard_normal((3, 64)))
    np.testing.assert_array_equal(oracle.ffn("q2", 64, 32, ex, x), oracle.ffn("f32", 64, 32, dense, x))


def test_ffn_linear_in_down_and_swiglu_structure():
    rng = np.random.default_rng(12)
    H, I = 6, 4
    ex = {m: {"w": (rng.standard_normal(s) * 0.3).astype(np.float32)}
          for m, s in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I)))}
    x = _bf16(rng.standard_normal((2, H)))
    o1 = oracle.ffn("f32", H, I, ex, x)
    ex2 = dict(ex, down={"w": ex["down"]["w"] * 2})
    np.testing.assert_allclose(oracle.ffn("f32", H, I, ex2, x), 2 * o1, rtol=1e-15)
    # up enters linearly, gate does not
    ex3 = dict(ex, up={"w": ex["up"]["w"] * 2})
    np.testing.assert_allclose(oracle.ffn("f32", H, I, ex3, x), 2 * o1, rtol=1e-14)
    ex4 = dict(ex, gate={"w": ex["gate"]["w"] * 2})
    assert not np.allclose(oracle.ffn("f32", H, I, ex4, x), 2 * o1)


# ------------------------------------------------------------ whole layer
def _tiny_layer_inputs(E=6, H=32, I=32, T=3, seed=13, fmt="q2"):
    cfg = synth.MoEConfig(name="pin", E=E, k=2, H=H, I=I, T=T, layers=1, wfmt=fmt,
                          router_fmt="f32", shared=True, bias="none", slots="identity",
                          seed=seed)
    x = synth.gen_x(cfg, 0)
    W = synth.gen_router(cfg, 0) * 20.0          # spread the logits
    pairs = [(0, e) for e in range(E)]
    pools = {m: synth.gen_pool(cfg, pairs, m) for m in ("gate", "up", "down")}
    shared = {m: synth.gen_pool(cfg, [(0, synth.SHARED_ID)], m) for m in ("gate", "up", "down")}
    return cfg, x, W, pools, shared


def test_layer_k_equals_E_is_dense_softmax_mixture():
    """With k = E the layer equals sum_e softmax(logits)_e * FFN_e(x) + shared,
    computed here with a separately written dense softmax."""
    cfg, x, W, pools, shared = _tiny_layer_inputs()
    E, H, I = cfg.E, cfg.H, cfg.I
    out = oracle.layer(x, W, "f32", None, E, "q2", pools, I, shared=shared)
    logits = oracle.router(x, W, "f32")
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    want = np.zeros((cfg.T, H))
    for e in range(E):
        ex = {m: {"codes": pools[m][0][e], "scale": pools[m][1][e], "min": pools[m][2][e]}
              for m in ("gate", "up", "down")}
        want += p[:, e:e + 1] * oracle.ffn("q2", H, I, ex, x)
    sh = {m: {"codes": shared[m][0][0], "scale": shared[m][1][0], "min": shared[m][2][0]}
          for m in ("gate", "up", "down")}
    want += oracle.ffn("q2", H, I, sh, x)
    np.testing.assert_allclose(out["y"], want, rtol=1e-12, atol=1e-12)


def test_layer_shared_expert_adds_exactly_its_output():
    cfg, x, W, pools, shared = _tiny_layer_inputs()
    a = oracle.layer(x, W, "f32", None, 2, "q2", pools, cfg.I, shared=shared)
    b = oracle.layer(x, W, "f32", None, 2, "q2", pools, cfg.I, shared=None)
    sh = {m: {"codes": shared[m][0][0], "scale": shared[m][1][0], "min": shared[m][2][0]}
          for m in ("gate", "up", "down")}
    np.testing.assert_allclose(a["y"] - b["y"], oracle.ffn("q2", cfg.H, cfg.I, sh, x),
                               rtol=1e-12, atol=1e-12)


def test_layer_zero_expert_contributes_nothing():
    """An expert whose down matrix is zero adds nothing: the layer equals the
    layer in which that expert is not resident (a miss)."""
    cfg, x, W, pools, shared = _tiny_layer_inputs()
    base = oracle.layer(x, W, "f32", None, 2, "q2", pools, cfg.I, shared=shared)
    e0 = int(base["idx"][0, 0])
    pools0 = {m: tuple(a.copy() for a in pools[m]) for m in pools}
    pools0["down"][1][e0][:] = 0
    pools0["down"][2][e0][:] = 0
    zeroed = oracle.layer(x, W, "f32", None, 2, "q2", pools0, cfg.I, shared=shared)
    slot_of = np.arange(cfg.E, dtype=np.int32)
    slot_of[e0] = -1
    missing = oracle.layer(x, W, "f32", None, 2, "q2", pools, cfg.I, slot_of=slot_of,
                           shared=shared)
    np.testing.assert_allclose(zeroed["y"], missing["y"], rtol=0, atol=0)
    assert len(missing["miss_expert"]) >= 1


def test_layer_completion_invariant():
    """y_partial + sum over misses of gate * FFN_expert(x_token) = y_full."""
    cfg, x, W, pools, shared = _tiny_layer_inputs(T=4)
    full = oracle.layer(x, W, "f32", None, 2, "q2", pools, cfg.I, shared=shared)
    slot_of = np.array([0, -1, 1, -1, 2, -1], np.int32)
    S = 3
    sub = {m: tuple(a[[0, 2, 4]] for a in pools[m]) for m in pools}
    part = oracle.layer(x, W, "f32", None, 2, "q2", sub, cfg.I, slot_of=slot_of, shared=shared,
                        num_slots=S)
    y = part["y"].copy()
    for e, t, g in zip(part["miss_expert"], part["miss_token"], part["miss_gate"]):
        ex = {m: {"codes": pools[m][0][e], "scale": pools[m][1][e], "min": pools[m][2][e]}
              for m in ("gate", "up", "down")}
        y[t] += g * oracle.ffn("q2", cfg.H, cfg.I, ex, x[t:t + 1])[0]
    np.testing.assert_allclose(y, full["y"], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(part["idx"], full["idx"])
    assert len(part["miss_expert"]) + (part["slot_idx"] >= 0).sum() == 4 * 2


def test_layer_from_synth_matches_whole_layer():
    """The composed per-expert path used for big configurations equals the
    all-in-memory layer."""
    cfg = synth.MoEConfig(name="pin2", E=8, k=3, H=64, I=32, T=5, layers=2, wfmt="q4",
                          router_fmt="bf16", shared=True, bias="zipf", slots="identity",
                          seed=99)
    layer = 1
    x = synth.gen_x(cfg, layer)
    r = oracle.layer_from_synth(cfg, layer, x)
    pools = {m: synth.gen_pool(cfg, [(layer, e) for e in range(cfg.E)], m)
             for m in ("gate", "up", "down")}
    shared = {m: synth.gen_pool(cfg, [(layer, synth.SHARED_ID)], m) for m in ("gate", "up", "down")}
    full = oracle.layer(x, synth.gen_router(cfg, layer), "bf16", synth.gen_bias(cfg, layer),
                        cfg.k, "q4", pools, cfg.I, shared=shared)
    np.testing.assert_array_equal(r["idx"], full["idx"])
    np.testing.assert_allclose(r["y"], full["y"], rtol=1e-13, atol=1e-13)


# ---- usage counts and the slot-table refresh
def test_count_usage_is_a_histogram():
    rng = np.random.default_rng(3)
    idx = rng.integers(0, 37, size=(9, 5)).astype(np.int32)
    base = rng.integers(0, 4, size=37).astype(np.uint32)
    got = oracle.count_usage(idx, 37, base)
    np.testing.assert_array_equal(got, base + np.bincount(idx.ravel(), minlength=37))


def test_refresh_hand_worked():
    """6 experts, 3 slots (one free).  Candidates by count: 4 (7), 2 (3),
    5 (2); victims: free slot 2, then slot 1 (expert 3, count 1), slot 0
    (expert 0, count 5).  4 -> slot 2, 2 -> slot 1 (3 > 1), 5 stays out
    (2 > 5 fails)."""
    usage = [5, 0, 3, 1, 7, 2]
    slot_of = [0, -1, -1, 1, -1, -1]
    expert_of = [0, 3, -1]
    swaps, u, so, eo = oracle.slot_refresh(usage, slot_of, expert_of, 4)
    np.testing.assert_array_equal(swaps, [[2, 4, -1], [1, 2, 3]])
    np.testing.assert_array_equal(so, [0, -1, 1, -1, 2, -1])
    np.testing.assert_array_equal(eo, [0, 2, 4])
    np.testing.assert_array_equal(u, [2, 0, 1, 0, 3, 1])


def test_refresh_ties_do_not_swap_and_limits_hold():
    # equal counts: no swap; max_swaps = 0: tables unchanged, counts halved
    swaps, u, so, eo = oracle.slot_refresh([4, 4, 4, 4], [0, 1, -1, -1], [0, 1], 8)
    assert len(swaps) == 0 and list(so) == [0, 1, -1, -1] and list(u) == [2, 2, 2, 2]
    swaps, u, so, eo = oracle.slot_refresh([1, 9, 9], [0, -1, -1], [0], 0)
    assert len(swaps) == 0 and list(so) == [0, -1, -1] and list(u) == [0, 4, 4]
    # counts above 65535 rank as 65535: the lower id wins
    swaps, *_ = oracle.slot_refresh([0, 70000, 65535], [0, -1, -1], [0], 1)
    np.testing.assert_array_equal(swaps, [[0, 1, 0]])


def _resident_sets(so, eo):
    res = {int(j) for j in np.flatnonzero(np.asarray(so) >= 0)}
    assert res == {int(j) for j in eo if j >= 0}
    for s, j in enumerate(eo):
        if j >= 0:
            assert so[j] == s
    return res


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_refresh_unbounded_leaves_no_better_outsider(seed):
    """With enough swaps, afterwards no expert outside the pool has a count
    (before halving) above any resident's, tables stay inverse, and free
    slots fill before any resident is evicted."""
    rng = np.random.default_rng(seed)
    N, S = 300, 60
    usage = rng.zipf(1.3, N).clip(0, 100000).astype(np.uint32) * (rng.random(N) < 0.8)
    slot_of = np.full(N, -1, np.int32)
    expert_of = np.full(S, -1, np.int32)
    init = rng.choice(N, 45, replace=False)           # 15 free slots
    slots = rng.choice(S, 45, replace=False)
    slot_of[init] = slots
    expert_of[slots] = init
    swaps, u, so, eo = oracle.slot_refresh(usage, slot_of, expert_of, 1024)
    res = _resident_sets(so, eo)
    cap = np.minimum(usage.astype(np.int64), 65535)
    outside = [j for j in range(N) if j not in res]
    if all(e >= 0 for e in eo):      # pool full: nothing outside beats anything inside
        assert max(cap[outside]) <= min(cap[list(res)])
    else:                            # free slots left: every outsider had count 0
        assert all(cap[j] == 0 for j in outside)
    n_free_before = int((expert_of < 0).sum())
    n_cand = int(((slot_of < 0) & (cap > 0)).sum())
    assert sum(1 for sw in swaps if sw[2] < 0) == min(n_free_before, n_cand)
    assert all(sw[2] < 0 for sw in swaps[:min(n_free_before, n_cand)])
    np.testing.assert_array_equal(u, usage >> 1)


def test_refresh_bounded_takes_the_best_first():
    """max_swaps = 3 of many possible: the three swapped-in experts are the
    three highest-count outsiders (ties by lower id), the victims the three
    lowest-count residents."""
    rng = np.random.default_rng(9)
    N, S = 50, 10
    usage = rng.integers(1, 30, N).astype(np.uint32)
    slot_of = np.full(N, -1, np.int32)
    expert_of = np.arange(S, dtype=np.int32)          # experts 0..9 resident
    slot_of[:S] = np.arange(S)
    usage[:S] = rng.integers(0, 5, S)                  # weak residents
    swaps, *_ = oracle.slot_refresh(usage, slot_of, expert_of, 3)
    outs = sorted(range(S, N), key=lambda j: (-int(usage[j]), j))[:3]
    vics = sorted(range(S), key=lambda s: (int(usage[s]), s))[:3]
    np.testing.assert_array_equal(swaps[:, 1], outs)
    np.testing.assert_array_equal(swaps[:, 0], vics)
    np.testing.assert_array_equal(swaps[:, 2], vics)


# ---- verify acceptance ([MD] "予測してから検証する")

def test_verify_accept_hand_cases():
    V = 5
    rows = np.full((4, V), -1.0)
    for i, g in enumerate([2, 0, 4, 1]):
        rows[i, g] = 3.0
    assert oracle.verify_accept(rows, [2, 0, 3]).tolist() == [2, 0, 4]     # third draft rejected
    assert oracle.verify_accept(rows, [2, 0, 4]).tolist() == [2, 0, 4, 1]  # all kept + own token
    assert oracle.verify_accept(rows, [1, 0, 4]).tolist() == [2]           # first draft rejected
    assert oracle.verify_accept(rows, [2, 1, 4]).tolist() == [2, 0]        # a later match is not kept
    assert oracle.verify_accept(rows[:1], []).tolist() == [2]              # no drafts: one token


def test_verify_accept_ties_take_the_lowest_index():
    rows = np.array([[0.0, 7.0, 1.0, 7.0, 7.0],
                     [-0.0, 0.0, -1.0, -2.0, -3.0],
                     [0.0, -0.0, 0.0, -5.0, -5.0]])
    out = oracle.verify_accept(rows, [1, 0])
    assert out.tolist() == [1, 0, 0]


def test_verify_accept_equals_greedy_decoding():
    """A bigram 'model' (next-token logits depend on the last token) decoded
    greedily, and the same model run as drafts + verify passes with a drafter
    that is right about two times in three: the two token streams are equal."""
    rng = np.random.default_rng(7)
    V, steps = 11, 60
    table = rng.standard_normal((V, V))
    table[:, 3] = table[:, 5] = table.max(axis=1)   # exact ties everywhere
    greedy = [4]
    while len(greedy) < steps + 1:
        greedy.append(int(np.argmax(table[greedy[-1]])))
    spec = [4]
    while len(spec) < steps + 1:
        D = int(rng.integers(0, 4))
        drafts, last = [], spec[-1]
        for _ in range(D):   # the drafter: the model's token, or a wrong one
            nxt = int(np.argmax(table[last])) if rng.random() < 0.67 else int(rng.integers(0, V))
            drafts.append(nxt)
            last = nxt
        inputs = [spec[-1]] + drafts
        spec += oracle.verify_accept(table[inputs], drafts).tolist()
    assert spec[: steps + 1] == greedy
