"""GPU parity of the prefill path (MFMA router GEMM, multi-block slot
resolution, grouped expert GEMMs, combine) against the fp64 oracle."""

import numpy as np
import pytest

import oracle
import synth
from helpers import TOL, DeviceLayer, check_routing, host, rowwise_rel_err, say, small_cfg

pytestmark = pytest.mark.gpu

MID = {
    "q4_T600": small_cfg(E=64, k=6, H=256, I=128, T=600, wfmt="q4", bias="zipf", seed=41),
    "q2_T517": small_cfg(E=48, k=5, H=256, I=192, T=517, wfmt="q2", bias="zipf", seed=42),
    "q4_T700_noshared": small_cfg(E=32, k=4, H=384, I=64, T=700, wfmt="q4", shared=False,
                                  seed=43),
}


@pytest.mark.parametrize("name", list(MID))
def test_prefill_mid(name):
    cfg = MID[name]
    say(f"[gpu] prefill {name}: E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I} T={cfg.T}")
    x, _ = oracle.margin_x(cfg, 0)
    L = DeviceLayer(cfg, 0, x=x)
    o = L.run_steps()
    ref = L.oracle()
    check_routing(o, ref, cfg.k)
    np.testing.assert_array_equal(host(o["bucket_off"]), ref["bucket_off"])
    np.testing.assert_array_equal(host(o["bucket_pair"]), ref["bucket_pair"])
    hit = ref["slot_idx"].ravel() >= 0
    assert rowwise_rel_err(host(o["pair_out"])[hit], ref["pair_out"][hit]) <= TOL
    if cfg.shared:
        assert rowwise_rel_err(host(o["shared_out"]), ref["shared_out"]) <= TOL
    assert rowwise_rel_err(host(o["y"]), ref["y"]) <= TOL


def test_prefill_mid_partial_slots():
    """Large-T resolution with misses: bit-exact miss list and offsets."""
    cfg = small_cfg(E=64, k=6, H=256, I=128, T=450, wfmt="q4", bias="zipf", seed=44)
    say("[gpu] prefill with a partial slot table")
    x, _ = oracle.margin_x(cfg, 0)
    rank = synth.popularity_rank(cfg, 0)
    resident = np.sort(np.argsort(rank)[:40])
    slot_of = np.full(cfg.E, -1, np.int32)
    slot_of[resident] = np.arange(len(resident))
    from synth import device as sdev
    pool = sdev.expert_pool(cfg, [0] * len(resident), resident.tolist())
    L = DeviceLayer(cfg, 0, x=x, pool=pool, slot_of=slot_of, num_slots=len(resident))
    o = L.run_steps()
    ref = L.oracle()
    assert len(ref["miss_expert"]) > 100
    check_routing(o, ref, cfg.k)
    np.testing.assert_array_equal(host(o["bucket_off"]), ref["bucket_off"])
    np.testing.assert_array_equal(host(o["bucket_pair"])[: len(ref["bucket_pair"])],
                                  ref["bucket_pair"])
    assert rowwise_rel_err(host(o["y"]), ref["y"]) <= TOL


def test_c5_prefill_full_size():
    """32,768 tokens through one layer, 4-bit experts, Zipf routing, in the
    calls bench.py times: every token's routing and every bucket bit-exact,
    floats on a sample that includes the largest and the smallest bucket."""
    cfg = synth.CONFIGS["c5"]
    say("[gpu] c5: drawing 32768 tokens with a routing margin (threaded oracle router)")
    x, att = oracle.margin_x(cfg, 0, threads=16)
    say(f"  re-drawn tokens: {int((att > 0).sum())}")
    L = DeviceLayer(cfg, 0, x=x)
    o = L.run_steps()
    say("  GPU done; oracle routing")
    r = oracle.route_from_synth(cfg, 0, x, threads=16)
    check_routing(o, r, cfg.k)
    np.testing.assert_array_equal(host(o["bucket_off"]), r["bucket_off"])
    np.testing.assert_array_equal(host(o["bucket_pair"]), r["bucket_pair"])
    sizes = np.diff(r["bucket_off"])
    say(f"  bucket sizes: max {sizes.max()}, min non-empty {sizes[sizes > 0].min()}, "
        f"empty {(sizes == 0).sum()}")
    big = int(np.argmax(sizes))
    small = int(np.nonzero(sizes == sizes[sizes > 0].min())[0][0])
    pick = [r["bucket_pair"][r["bucket_off"][big]] // cfg.k,
            r["bucket_pair"][r["bucket_off"][big + 1] - 1] // cfg.k,
            r["bucket_pair"][r["bucket_off"][small]] // cfg.k]
    rng = np.random.default_rng(5)
    tokens = np.unique(np.concatenate([pick, rng.choice(cfg.T, 29, replace=False)]))
    ref = oracle.layer_from_synth(cfg, 0, x, tokens=tokens, route=r)
    err = rowwise_rel_err(host(o["y"])[tokens], ref["y"][tokens])
    say(f"  sampled {len(tokens)} tokens: rel err {err:.2e}")
    assert err <= TOL
