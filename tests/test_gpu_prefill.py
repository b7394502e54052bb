"""GPU parity of the prefill path (MFMA router GEMM, multi-block slot
resolution, grouped expert GEMMs, combine) against the fp64 oracle."""

import numpy as np
import pytest

import oracle
import synth
from helpers import (ORACLE_THREADS, TOL, DeviceLayer, check_routing, host, rowwise_rel_err,
                     say, small_cfg)

pytestmark = pytest.mark.gpu

MID = {
    "q4_T600": small_cfg(E=64, k=6, H=256, I=128, T=600, wfmt="q4", bias="zipf", seed=41),
    "q2_T517": small_cfg(E=48, k=5, H=256, I=192, T=517, wfmt="q2", bias="zipf", seed=42),
    "q4_T700_noshared": small_cfg(E=32, k=4, H=384, I=64, T=700, wfmt="q4", shared=False,
                                  seed=43),
    # MFMA router over several ragged expert tiles (E = 600) and a ragged
    # token tile, with the 16-keys-per-lane top-k
    "q2_T300_E600_k12": small_cfg(E=600, k=12, H=256, I=64, T=300, wfmt="q2", bias="zipf", seed=48),
    # grouped-GEMM shapes (H and I multiples of 256, at least 2048 pairs):
    # buckets of several row tiles with last tiles of 1-4 MFMA row tiles,
    # K loops of one scale group (K = 256) and of two (K = 512)
    "gemm_q2_T1100": small_cfg(E=32, k=4, H=512, I=256, T=1100, wfmt="q2", bias="zipf", seed=45),
    "gemm_q4_T900_noshared": small_cfg(E=24, k=3, H=256, I=512, T=900, wfmt="q4", shared=False,
                                       bias="zipf", seed=46),
}


def _uses_gemm(cfg):
    return cfg.T * cfg.k >= 2048 and cfg.H % 256 == 0 and cfg.I % 256 == 0


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
    if name.startswith("gemm"):
        assert _uses_gemm(cfg)
        sizes = np.diff(ref["bucket_off"])
        tails = {int((n - 1) % 128) // 32 + 1 for n in sizes if n > 0}
        say(f"  bucket sizes {sizes.min()}..{sizes.max()}, last-tile row tiles {sorted(tails)}")
        assert sizes.max() > 128 and len(tails) >= 3
    hit = ref["slot_idx"].ravel() >= 0
    assert rowwise_rel_err(host(o["pair_out"])[hit], ref["pair_out"][hit]) <= TOL
    if cfg.shared:
        assert rowwise_rel_err(host(o["shared_out"]), ref["shared_out"]) <= TOL
    assert rowwise_rel_err(host(o["y"]), ref["y"]) <= TOL


ACCUM = ["q4_T600", "q2_T517", "gemm_q2_T1100", "gemm_q4_T900_noshared"]


@pytest.mark.parametrize("name", ACCUM)
def test_expert_ffn_accum(name):
    """moe_expert_ffn_accum (the combine fused into the down projection, by
    the GEMVs or the grouped GEMMs): y = base + shared + sum of gate * o
    within tolerance of the oracle, on a nonzero base."""
    import torch
    cfg = MID[name]
    say(f"[gpu] expert FFN, accumulate mode ({name}, {'GEMM' if _uses_gemm(cfg) else 'GEMV'})")
    x, _ = oracle.margin_x(cfg, 0)
    L = DeviceLayer(cfg, 0, x=x)
    o = L.run_steps()
    ref = L.oracle()
    base = torch.from_numpy(np.random.default_rng(9).standard_normal((cfg.T, cfg.H))
                            .astype(np.float32)).cuda()
    y = L.run_accum(o, base)
    err = rowwise_rel_err(host(y), host(base).astype(np.float64) + ref["y"])
    say(f"  rel err {err:.2e}")
    assert err <= TOL


def test_expert_ffn_accum_partial_slots():
    """Accumulate mode with a partial slot table: misses add nothing."""
    cfg = PARTIAL_CFG
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
    assert len(ref["miss_expert"]) > 100 and _uses_gemm(cfg)
    assert rowwise_rel_err(host(L.run_accum(o)), ref["y"]) <= TOL


PARTIAL = {
    "gemv": small_cfg(E=64, k=6, H=256, I=128, T=450, wfmt="q4", bias="zipf", seed=44),
    "gemm": small_cfg(E=64, k=6, H=256, I=256, T=800, wfmt="q4", bias="zipf", seed=47),
}
PARTIAL_CFG = PARTIAL["gemm"]


@pytest.mark.parametrize("name", list(PARTIAL))
def test_prefill_mid_partial_slots(name):
    """Large-T resolution with misses: bit-exact miss list and offsets; the
    expert FFN of the hits by GEMV or by grouped GEMM."""
    cfg = PARTIAL[name]
    assert _uses_gemm(cfg) == (name == "gemm")
    say(f"[gpu] prefill with a partial slot table ({name})")
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
    y on 1,024 sampled tokens that include the first and last tokens of the
    largest bucket and the first of the smallest non-empty one."""
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
    others = np.setdiff1d(np.arange(cfg.T), pick)
    tokens = np.unique(np.concatenate([pick, rng.choice(others, 1024 - len(set(pick)),
                                                        replace=False)]))
    assert len(tokens) == 1024
    ref = oracle.layer_from_synth(cfg, 0, x, tokens=tokens, route=r, threads=ORACLE_THREADS)
    err = rowwise_rel_err(host(o["y"])[tokens], ref["y"][tokens])
    y_acc = host(L.run_accum(o))
    err_acc = rowwise_rel_err(y_acc[tokens], ref["y"][tokens])
    say(f"  sampled {len(tokens)} tokens: rel err {err:.2e} (pairs + combine), "
        f"{err_acc:.2e} (accumulate mode)")
    assert err <= TOL and err_acc <= TOL


RANGE = {
    "q4": small_cfg(E=32, k=4, H=512, I=512, T=1100, wfmt="q4", bias="zipf", seed=51),
    "q2": small_cfg(E=24, k=3, H=256, I=768, T=900, wfmt="q2", bias="zipf", seed=52),
}


@pytest.mark.parametrize("name", list(RANGE))
def test_prefill_gemm_activation_range(name):
    """The grouped-GEMM path with token rows scaled by 2^-24 .. 2^16 (exact
    in bf16): tokens beyond the fp16 range (|x| > 65504), h beyond it (up to
    ~10^14), and rows so small that fp16 would flush them.  Each token row
    and h row slab outside the fp16 working range is carried with a power-
    of-two scale, so y stays within tolerance on every row.  Routing comes
    from the bias alone (zero router weights), so the scaled tokens do not
    reach the logits."""
    import torch
    cfg = RANGE[name]
    assert _uses_gemm(cfg)
    say(f"[gpu] prefill GEMM activation range ({name}): T={cfg.T} H={cfg.H} I={cfg.I}")
    x = synth.gen_x(cfg, 0, cfg.T)
    f = (x.astype(np.uint32) << 16).view(np.float32)
    scale = np.float32(2.0) ** np.array([-24, -10, 0, 8, 16], np.float32)[np.arange(cfg.T) % 5]
    x = ((f * scale[:, None]).view(np.uint32) >> 16).astype(np.uint16)   # exact: powers of two
    L = DeviceLayer(cfg, 0, x=x)
    bias = (np.random.default_rng(6).permutation(cfg.E) * 0.01).astype(np.float32)
    L.inp["router_w"].zero_()
    L.inp["bias"].copy_(torch.from_numpy(bias))
    o = L.run_steps()
    logits = oracle.router(x, np.zeros((cfg.E, cfg.H), np.uint16), cfg.router_fmt, bias)
    idx, gate = oracle.topk(logits, cfg.k)
    slot_idx, me, mt, mg, moff = oracle.resolve(idx, gate, cfg.E)
    route = {"logits": logits, "idx": idx, "gate": gate, "slot_idx": slot_idx,
             "miss_expert": me, "miss_token": mt, "miss_gate": mg, "miss_off": moff}
    ref = oracle.layer_from_synth(cfg, 0, x, route=route, threads=ORACLE_THREADS)
    check_routing(o, ref, cfg.k)
    y = host(o["y"])
    assert np.isfinite(y).all()
    ay = np.abs(ref["y"]).max(axis=1)
    say(f"  |y| row maxima {ay.min():.2e} .. {ay.max():.2e}")
    assert ay.max() > 1e10 and ay.min() < 1e-12
    for sc in np.unique(scale):
        rows = scale == sc
        err = rowwise_rel_err(y[rows], ref["y"][rows])
        say(f"  rows scaled by 2^{int(np.log2(sc))}: rel err {err:.2e}")
        assert err <= TOL


CHUNKED = {
    # name: (config, chunk, aux stream)
    "q4_T600_chunk256_aux": (MID["q4_T600"], 256, True),
    "q2_T517_chunk100_aux": (MID["q2_T517"], 100, True),
    "q4_T700_noshared_chunk700": (MID["q4_T700_noshared"], 700, False),
    "q4_T600_chunk7_main": (MID["q4_T600"], 7, False),
    # first chunk through the grouped GEMMs (2,400 pairs), last through the
    # GEMVs (2,000 pairs)
    "gemm_q2_T1100_chunk600_aux": (MID["gemm_q2_T1100"], 600, True),
}


@pytest.mark.parametrize("name", list(CHUNKED))
def test_prefill_layer_chunked(name):
    """moe_prefill_layer (routing of chunk c + 1 on a second stream while
    chunk c's experts run) against the oracle: routing bit-exact for every
    token, y within tolerance, and the same as the one-chunk call."""
    import torch
    import routed_expert_ffn_gemv_amd as moe
    cfg, chunk, use_aux = CHUNKED[name]
    say(f"[gpu] prefill layer {name}: T={cfg.T} chunk={chunk} aux={use_aux}")
    x, _ = oracle.margin_x(cfg, 0)
    L = DeviceLayer(cfg, 0, x=x)
    T, k, H = cfg.T, cfg.k, cfg.H
    dev = "cuda"

    def run(c, aux):
        ws = torch.zeros(moe.moe_prefill_workspace_size(L.desc, T, c), dtype=torch.uint8,
                         device=dev)
        y = torch.full((T, H), float("nan"), dtype=torch.float32, device=dev)
        idx = torch.full((T, k), -3, dtype=torch.int32, device=dev)
        gate = torch.full((T, k), -3.0, dtype=torch.float32, device=dev)
        sl = torch.full((T, k), -3, dtype=torch.int32, device=dev)
        moe.moe_prefill_layer(L.desc, L.inp["x"], T, c, y, idx, gate, sl, ws,
                              aux_stream=torch.cuda.Stream() if aux else None)
        torch.cuda.synchronize()
        return {"y": y, "idx": idx, "gate": gate, "slot_idx": sl}

    o = run(chunk, use_aux)
    ref = L.oracle()
    np.testing.assert_array_equal(host(o["idx"]), ref["idx"])
    np.testing.assert_array_equal(host(o["slot_idx"]), ref["slot_idx"])
    g = host(o["gate"]).astype(np.float64)
    assert np.all(np.abs(g - ref["gate"]) <= TOL * np.abs(ref["gate"]))
    assert rowwise_rel_err(host(o["y"]), ref["y"]) <= TOL
    whole = run(T, False)
    np.testing.assert_array_equal(host(whole["idx"]), host(o["idx"]))
    assert rowwise_rel_err(host(o["y"]), host(whole["y"]).astype(np.float64)) <= TOL
