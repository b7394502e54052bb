"""GPU hits plus host-tier misses equal the all-resident layer.

moe_layer (fused launch, and the step-wise path) runs with a partial slot
table; its miss list, copied to the host, goes to moe_host_miss_ffn with the
layer's experts in host memory; y_partial + misses must match the oracle's
all-resident output."""

import numpy as np
import pytest

import oracle
import synth
from helpers import TOL, DeviceLayer, check_routing, host, rowwise_rel_err, say, small_cfg

pytestmark = pytest.mark.gpu

CASES = {
    # name: (config, resident experts)
    "fused_T9": (small_cfg(E=64, k=8, H=1024, I=256, T=9, bias="zipf", seed=101), 24),
    "fused_T1": (small_cfg(E=64, k=8, H=1024, I=256, T=1, bias="zipf", seed=102), 20),
    "steps_q4": (small_cfg(E=24, k=4, H=96, I=160, T=7, wfmt="q4", bias="zipf", seed=103), 10),
}


@pytest.mark.parametrize("name", list(CASES))
def test_gpu_hits_plus_host_misses(name):
    import routed_expert_ffn_gemv_amd as moe
    from synth import device as sdev
    cfg, n_res = CASES[name]
    say(f"[gpu] host tier {name}: E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I} T={cfg.T}")
    x, _ = oracle.margin_x(cfg, 0)
    rng = np.random.default_rng(cfg.seed)
    resident = np.sort(rng.choice(cfg.E, n_res, replace=False))
    slot_of = np.full(cfg.E, -1, np.int32)
    slot_of[resident] = np.arange(n_res)
    pool = sdev.expert_pool(cfg, [0] * n_res, resident.tolist())
    L = DeviceLayer(cfg, 0, x=x, pool=pool, slot_of=slot_of, num_slots=n_res)
    o = L.run_steps() if name.startswith("steps") else L.run_layer()
    ref = L.oracle(with_misses=True)
    check_routing(o, ref, cfg.k)
    moff = host(o["miss_off"]).astype(np.int32)
    assert moff[-1] > 0
    miss = host(o["miss"])[: 3 * moff[-1]].astype(np.int32).copy()
    pairs = [(0, e) for e in range(cfg.E)]
    store = {m: synth.gen_pool(cfg, pairs, m) for m in ("gate", "up", "down")}
    y = host(o["y"]).astype(np.float32).copy()
    moe.moe_host_miss_ffn(cfg.E, cfg.H, cfg.I, cfg.wfmt, store["gate"], store["up"],
                          store["down"], L.inp["x_host"], cfg.T, miss, moff, y)
    assert rowwise_rel_err(y, ref["y_full"]) <= TOL
