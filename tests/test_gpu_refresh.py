"""GPU parity of the usage counts and of the slot-table refresh
(moe_slot_refresh) against the oracle, through the C ABI.

Swap lists, tables and halved counts must match bit for bit; after a
refresh every occupied slot must hold, byte for byte, the store's copy of
the expert its table names; and layers run on the refreshed pool must match
the oracle."""

import numpy as np
import pytest

import oracle
import synth
from helpers import TOL, DeviceLayer, check_routing, host, rowwise_rel_err, say, small_cfg

pytestmark = pytest.mark.gpu


def _setup(cfg, L, S, n_res, seed, zipf=1.4):
    """A store of all L*E experts, a pool of S slots with n_res of them
    holding random experts, random counts.  Returns device tensors and the
    host copies of the tables."""
    import torch
    import routed_expert_ffn_gemv_amd as moe
    from synth import device as sdev
    E = cfg.E
    N = L * E
    rng = np.random.default_rng(seed)
    store = sdev.expert_pool(cfg, np.repeat(np.arange(L), E), np.tile(np.arange(E), L))
    held = rng.choice(N, n_res, replace=False)
    slots = rng.choice(S, n_res, replace=False)
    slot_of = np.full(N, -1, np.int32)
    expert_of = np.full(S, -1, np.int32)
    slot_of[held] = slots
    expert_of[slots] = held
    fill = np.where(expert_of >= 0, expert_of, 0)     # free slots hold expert 0
    pool = sdev.expert_pool(cfg, fill // E, fill % E)
    usage = (rng.zipf(zipf, N) * (rng.random(N) < 0.7)).clip(0, 70000).astype(np.uint32)
    dev = {
        "usage": torch.as_tensor(usage.view(np.int32), device="cuda"),
        "slot_of": torch.as_tensor(slot_of, device="cuda"),
        "expert_of": torch.as_tensor(expert_of, device="cuda"),
    }
    sp = moe.SlotPool(L, E, cfg.H, cfg.I, cfg.wfmt, pool, store, dev["usage"], dev["slot_of"],
                      dev["expert_of"], S)
    return sp, pool, store, dev, usage, slot_of, expert_of


def _planes_equal(pool, store, s, j):
    for m in ("gate", "up", "down"):
        for a, b in zip(pool[m], store[m]):
            if not bool((a[s] == b[j]).all()):
                return False
    return True


CASES = {
    # name: (E, H, I, L, S, resident, max_swaps)
    "small_free_slots": (40, 128, 64, 3, 30, 24, 64),
    "small_bounded": (40, 128, 64, 3, 30, 30, 5),
    "no_swaps_allowed": (16, 64, 64, 2, 8, 6, 0),
    "stack_shape": (512, 128, 64, 48, 4176, 4176, 96),
}


@pytest.mark.parametrize("name", list(CASES))
def test_refresh_matches_oracle(name):
    import torch
    import routed_expert_ffn_gemv_amd as moe
    E, H, I, L, S, n_res, M = CASES[name]
    cfg = small_cfg(E=E, k=4, H=H, I=I, T=1, seed=51)
    say(f"[gpu] slot refresh {name}: L={L} E={E} S={S} resident={n_res} max_swaps={M}")
    sp, pool, store, dev, usage, slot_of, expert_of = _setup(cfg, L, S, n_res, seed=len(name))
    swaps = torch.full((max(M, 1) * 3,), -9, dtype=torch.int32, device="cuda")
    n_swaps = torch.full((1,), -9, dtype=torch.int32, device="cuda")
    moe.moe_slot_refresh(sp, M, swaps, n_swaps)
    torch.cuda.synchronize()
    ref_swaps, ref_u, ref_so, ref_eo = oracle.slot_refresh(usage, slot_of, expert_of, M)
    n = int(host(n_swaps)[0])
    assert n == len(ref_swaps)
    np.testing.assert_array_equal(host(swaps)[: 3 * n].reshape(n, 3), ref_swaps)
    np.testing.assert_array_equal(host(dev["usage"]).view(np.uint32), ref_u)
    np.testing.assert_array_equal(host(dev["slot_of"]), ref_so)
    np.testing.assert_array_equal(host(dev["expert_of"]), ref_eo)
    if name == "small_free_slots":
        assert n > 0 and any(sw[2] < 0 for sw in ref_swaps)
    # every occupied slot holds its expert's planes
    for s, j in enumerate(ref_eo):
        if j >= 0 and (n > 0 and s in set(ref_swaps[:, 0]) or s % 97 == 0):
            assert _planes_equal(pool, store, s, int(j)), (s, j)


def test_usage_counts_fused_and_steps():
    """usage_counts after moe_layer (fused launch) and after the separate
    steps equal the oracle's count of its own routing choices."""
    import torch
    cfg = small_cfg(E=48, k=6, H=128, I=64, T=7, bias="zipf", seed=61)
    say("[gpu] usage counts, fused and steps")
    x, _ = oracle.margin_x(cfg, 0)
    for path in ("layer", "steps"):
        L = DeviceLayer(cfg, 0, x=x)
        usage = torch.zeros(cfg.E, dtype=torch.int32, device="cuda") + 3
        L.desc.desc.usage_counts = usage.data_ptr()
        L.desc._keep.append(usage)
        for _ in range(2):
            o = L.run_layer() if path == "layer" else L.run_steps()
        torch.cuda.synchronize()
        ref = L.oracle()
        check_routing(o, ref, cfg.k)
        want = oracle.count_usage(np.concatenate([ref["idx"], ref["idx"]]), cfg.E,
                                  np.full(cfg.E, 3, np.uint32))
        np.testing.assert_array_equal(host(usage).view(np.uint32), want)


def test_layers_run_on_the_refreshed_pool():
    """Routing, miss lists and outputs of every layer after a refresh match
    the oracle on the refreshed tables (the copied weights are the ones the
    layers read)."""
    import torch
    import routed_expert_ffn_gemv_amd as moe
    cfg = small_cfg(E=32, k=4, H=128, I=64, T=5, bias="zipf", seed=71)
    L, S = 3, 40
    say("[gpu] layers after a refresh")
    sp, pool, store, dev, usage, slot_of, expert_of = _setup(cfg, L, S, 30, seed=5)
    swaps = torch.zeros(64 * 3, dtype=torch.int32, device="cuda")
    n_swaps = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_slot_refresh(sp, 64, swaps, n_swaps)
    torch.cuda.synchronize()
    assert int(host(n_swaps)[0]) > 0
    so = host(dev["slot_of"]).reshape(L, cfg.E)
    for layer in range(L):
        x, _ = oracle.margin_x(cfg, layer)
        D = DeviceLayer(cfg, layer, x=x, pool=pool, slot_of=so[layer], num_slots=S)
        o = D.run_layer()
        ref = D.oracle()
        check_routing(o, ref, cfg.k)
        assert rowwise_rel_err(host(o["y"]), ref["y"]) <= TOL
