"""The host tier (moe_host_miss_ffn): the listed misses computed on the CPU.

Runs without a GPU.  With the oracle's routing over a partial slot table,
the oracle's partial output plus the host tier's misses must equal the
oracle's all-resident output (the completion invariant y_partial + misses =
y_full); results must not depend on the thread count; bad lists are refused
without touching y."""

import numpy as np
import pytest

import oracle
import synth
from helpers import TOL, rowwise_rel_err, small_cfg

CASES = {
    "q2": small_cfg(E=24, k=4, H=128, I=64, T=6, bias="zipf", seed=91),
    "q4": small_cfg(E=16, k=3, H=96, I=160, T=5, wfmt="q4", seed=92),
    "f32": small_cfg(E=9, k=4, H=96, I=32, T=3, wfmt="f32", router_fmt="f32", seed=93),
    # one expert missed by several tokens (its weights read once for them)
    "q2_crowded": small_cfg(E=8, k=6, H=64, I=64, T=9, bias="zipf", seed=94),
}


def _store(cfg, layer=0):
    pairs = [(layer, e) for e in range(cfg.E)]
    return {m: synth.gen_pool(cfg, pairs, m) for m in ("gate", "up", "down")}


def _route(cfg, resident):
    """x, the oracle's layer (with y_full) for the slot table holding the
    experts `resident` at slot = id, and the miss list as moe_miss words."""
    x, _ = oracle.margin_x(cfg, 0)
    slot_of = np.full(cfg.E, -1, np.int32)
    slot_of[resident] = resident
    r = oracle.layer_from_synth(cfg, 0, x, slot_of=slot_of, num_slots=cfg.E, with_misses=True)
    n = len(r["miss_expert"])
    miss = np.zeros((n, 3), np.int32)
    miss[:, 0] = r["miss_expert"]
    miss[:, 1] = r["miss_token"]
    miss[:, 2] = np.asarray(r["miss_gate"], np.float32).view(np.int32)
    return x, r, miss.ravel().copy(), np.asarray(r["miss_off"], np.int32)


def _run(cfg, st, x, miss, moff, y, threads=0):
    import routed_expert_ffn_gemv_amd as moe
    moe.moe_host_miss_ffn(cfg.E, cfg.H, cfg.I, cfg.wfmt, st["gate"], st["up"], st["down"], x,
                          x.shape[0], miss, moff, y, threads)


@pytest.mark.parametrize("name", list(CASES))
def test_completion_invariant(name):
    cfg = CASES[name]
    resident = np.arange(0, cfg.E, 2)   # every other expert on the card
    x, r, miss, moff = _route(cfg, resident)
    assert moff[-1] > 0
    st = _store(cfg)
    y = np.asarray(r["y"], np.float32).copy()
    _run(cfg, st, x, miss, moff, y)
    assert rowwise_rel_err(y, r["y_full"]) <= TOL
    # the additions alone equal the misses' share
    y0 = np.zeros((x.shape[0], cfg.H), np.float32)
    _run(cfg, st, x, miss, moff, y0)
    share = r["y_full"] - r["y"]
    rows = moff[1:] > moff[:-1]
    assert rowwise_rel_err(y0[rows], share[rows]) <= TOL
    assert not y0[~rows].any()


def test_thread_count_does_not_change_the_result():
    cfg = CASES["q2_crowded"]
    x, r, miss, moff = _route(cfg, np.array([0, 3]))
    st = _store(cfg)
    ys = []
    for threads in (1, 2, 5, 0):
        y = np.zeros((x.shape[0], cfg.H), np.float32)
        _run(cfg, st, x, miss, moff, y, threads)
        ys.append(y)
    for y in ys[1:]:
        np.testing.assert_array_equal(y, ys[0])


def test_no_misses_and_no_tokens():
    cfg = CASES["q2"]
    x, r, miss, moff = _route(cfg, np.arange(cfg.E))   # everything resident
    assert moff[-1] == 0
    st = _store(cfg)
    y = np.full((x.shape[0], cfg.H), 7.0, np.float32)
    _run(cfg, st, x, miss, moff, y)
    assert (y == 7.0).all()
    _run(cfg, st, x[:0], miss, np.zeros(1, np.int32), y[:0])


@pytest.mark.parametrize("bad", ["expert_high", "expert_negative", "token", "duplicate",
                                 "offsets"])
def test_bad_lists_are_refused(bad):
    import routed_expert_ffn_gemv_amd as moe
    cfg = CASES["q2"]
    x, r, miss, moff = _route(cfg, np.arange(0, cfg.E, 2))
    st = _store(cfg)
    m = miss.reshape(-1, 3).copy()
    o = moff.copy()
    t = int(np.argmax(o[1:] - o[:-1] >= 2))   # a token with two misses
    assert o[t + 1] - o[t] >= 2
    i = o[t]
    if bad == "expert_high":
        m[i, 0] = cfg.E
    elif bad == "expert_negative":
        m[i, 0] = -1
    elif bad == "token":
        m[i, 1] = (t + 1) % x.shape[0]
    elif bad == "duplicate":
        m[i + 1, 0] = m[i, 0]
    else:
        o[1] = o[2] + 1
    y = np.full((x.shape[0], cfg.H), 3.0, np.float32)
    with pytest.raises(moe.MoEError):
        _run(cfg, st, x, m.ravel().copy(), o, y)
    assert (y == 3.0).all()


def test_generic_code_matches():
    """The plain C++ path (MOE_HOST_ISA=generic, a fresh process) gives the
    same invariant; both paths agree to rounding."""
    import os
    import subprocess
    import sys
    code = (
        "import numpy as np, sys; sys.path[:0] = ['tests', '.'];"
        "import test_host_tier as h, routed_expert_ffn_gemv_amd as moe;"
        "cfg = h.CASES['q4']; x, r, miss, moff = h._route(cfg, np.arange(0, cfg.E, 2));"
        "y = np.zeros((x.shape[0], cfg.H), np.float32);"
        "h._run(cfg, h._store(cfg), x, miss, moff, y);"
        "np.save(sys.argv[1], y); print(moe.moe_host_isa())")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = {}
    for isa in ("generic", "auto"):
        env = dict(os.environ, MOE_HOST_ISA=isa)
        path = os.path.join(os.environ.get("TMPDIR", "/tmp"), f"host_tier_{isa}_{os.getpid()}.npy")
        res = subprocess.run([sys.executable, "-c", code, path], cwd=root, env=env,
                             capture_output=True, text=True, timeout=300)
        assert res.returncode == 0, res.stderr[-2000:]
        outs[isa] = (int(res.stdout.split()[-1]), np.load(path))
        os.remove(path)
    assert outs["generic"][0] == 0
    cfg = CASES["q4"]
    x, r, miss, moff = _route(cfg, np.arange(0, cfg.E, 2))
    share = r["y_full"] - r["y"]
    rows = moff[1:] > moff[:-1]
    for isa, (_, y) in outs.items():
        assert rowwise_rel_err(y[rows], share[rows]) <= TOL, isa
