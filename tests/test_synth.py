"""The synthetic generator: determinism, formats and the statistics the
pages give for the workloads (CPU only)."""

import hashlib

import numpy as np

import oracle
import synth


def test_deterministic_bytes():
    cfg = synth.CONFIGS["c2"]
    a = synth.gen_matrix(cfg, 0, 17, "down")
    b = synth.gen_matrix(cfg, 0, 17, "down")
    for p in ("codes", "scale", "min"):
        assert np.array_equal(a[p], b[p])
    c = synth.gen_matrix(cfg, 0, 18, "down")
    assert not np.array_equal(a["codes"], c["codes"])
    # random access: one expert does not depend on which others are drawn
    x1 = synth.gen_x_rows(cfg, 3, [5])
    x2 = synth.gen_x(cfg, 3, 8)[5:6]
    assert np.array_equal(x1, x2)


def test_splitmix64_reference_values():
    # SplitMix64 with state 0 (Steele, Lea, Flood 2014; the generator of the
    # xoshiro reference code): first outputs are fixed published numbers.
    w = synth.words(0, 3)
    assert [int(v) for v in w] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_block_scales_and_mins_are_exact_fp16():
    for name, dlo, dhi in (("c2", 256 * 2.0 ** -13, 511 * 2.0 ** -13),
                           ("c5", 64 * 2.0 ** -13, 127 * 2.0 ** -13)):
        cfg = synth.CONFIGS[name]
        m = synth.gen_matrix(cfg, 0, 1, "gate")
        d = synth.f16_to_f64(m["scale"])
        mn = synth.f16_to_f64(m["min"])
        assert d.min() >= dlo and d.max() <= dhi
        # d is an integer multiple of 2^-13, m of 2^-14: exact fp16 values
        assert np.all(d * 2 ** 13 == np.round(d * 2 ** 13))
        assert np.all(mn * 2 ** 14 == np.round(mn * 2 ** 14))
        qmid = 1.5 if cfg.wfmt == "q2" else 7.5
        # mean weight d*qmid + m stays within 16 * 2^-14 of zero
        assert np.abs(d * qmid + mn).max() <= 16 * 2.0 ** -14 + 1e-12


def test_weight_statistics():
    for name in ("c2", "c5"):
        cfg = synth.CONFIGS[name]
        m = synth.gen_matrix(cfg, 0, 2, "up")
        w = oracle.dequant(cfg.wfmt, cfg.I, cfg.H, m["codes"], m["scale"], m["min"])
        assert abs(w.mean()) < 2e-3
        assert 0.04 < w.std() < 0.065


def test_activation_and_router_statistics():
    cfg = synth.CONFIGS["c2"]
    x = synth.bf16_to_f64(synth.gen_x(cfg, 0, 64))
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    W = synth.bf16_to_f64(synth.gen_router(cfg, 0))
    assert abs(W.std() - 0.02) < 2e-4


def test_resident_counts():
    cfg = synth.CONFIGS["c4"]
    n = synth.resident_counts(cfg)
    assert len(n) == 48 and n.sum() == 4176 and n.min() == 57 and n.max() == 109
    slot_of, sl, se, S = synth.slot_layout(cfg)
    assert S == 4176
    assert np.array_equal((slot_of >= 0).sum(1), n)
    # resident experts are the most popular ones of each layer, in rank order
    for l in (0, 17, 47):
        rank = synth.popularity_rank(cfg, l)
        res = np.nonzero(slot_of[l] >= 0)[0]
        assert rank[res].max() == n[l] - 1
        order = res[np.argsort(slot_of[l, res])]
        assert np.array_equal(rank[order], np.arange(n[l]))
        assert np.all(sl[slot_of[l, res]] == l) and np.array_equal(se[slot_of[l, res]], res)


def test_zipf_routing_share_and_hit_rate():
    """Top 16 % of experts take ~75 % of selections (pages: 15-18 % serve
    70-78 %); the tiered slot table hits in the pages' range."""
    cfg = synth.CONFIGS["c4"]
    W = synth.gen_router(cfg, 0)
    bias = synth.gen_bias(cfg, 0)
    x = synth.gen_x(cfg, 0, 1024)
    idx, _ = oracle.topk(oracle.router_threads(x, W, "bf16", bias), cfg.k)
    cnt = np.bincount(idx.ravel(), minlength=cfg.E)
    share = np.sort(cnt)[::-1][:82].sum() / cnt.sum()
    assert 0.70 <= share <= 0.80
    slot_of, _, _, _ = synth.slot_layout(cfg)
    hit = (slot_of[0][idx] >= 0).mean()
    assert 0.55 <= hit <= 0.88


def test_margin_x_gaps():
    cfg = synth.CONFIGS["c2"]
    x, att = oracle.margin_x(cfg, 0, T=16)
    l = oracle.router(x, synth.gen_router(cfg, 0), "bf16", None)
    assert oracle.min_top_gap(l, cfg.k).min() >= 1e-3
    assert np.array_equal(x[att == 0], synth.gen_x(cfg, 0, 16)[att == 0])


def test_fingerprints():
    """Self-generated fingerprints of a few planes, so an accidental change to
    the generator shows up (values recorded from this generator)."""
    cfg = synth.CONFIGS["c3"]
    m = synth.gen_matrix(cfg, 7, 300, "gate")
    h = hashlib.sha256(m["codes"][:4096].tobytes() + m["scale"][:64].tobytes()
                       + m["min"][:64].tobytes()).hexdigest()[:16]
    x = synth.gen_x(cfg, 7, 2)
    hx = hashlib.sha256(x.tobytes()).hexdigest()[:16]
    assert (h, hx) == FINGERPRINT


FINGERPRINT = ("1bcdc6251b47f9c6", "003a31d3b47c230c")
