"""Shared helpers of the GPU parity tests: build a layer on the device from
the synthetic generator, call the library through its C ABI, compare with
the oracle."""

import os
import sys

import numpy as np

import oracle
import synth

TOL = 2e-3   # max relative error of floating outputs (normwise per token row)
# threads for the oracle's per-expert calls (each call single-threaded)
ORACLE_THREADS = min(16, os.cpu_count() or 1)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rowwise_rel_err(got, ref):
    """max over rows of max_i |got - ref| / max_i |ref| (rows of ref that are
    all zero are compared absolutely)."""
    got = np.asarray(got, np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    den = np.abs(ref).max(axis=1)
    den[den == 0] = 1.0
    return float((np.abs(got - ref).max(axis=1) / den).max()) if ref.size else 0.0


def small_cfg(**kw):
    base = dict(name="small", E=16, k=2, H=64, I=64, T=4, layers=1, wfmt="q2",
                router_fmt="bf16", shared=True, bias="none", slots="identity", seed=1234)
    base.update(kw)
    return synth.MoEConfig(**base)


class DeviceLayer:
    """One layer of a synthetic config on the device, with its LayerDesc."""

    def __init__(self, cfg, layer, x=None, pool=None, slot_of=None, num_slots=None,
                 device="cuda"):
        import torch
        import routed_expert_ffn_gemv_amd as moe
        from synth import device as sdev
        self.cfg, self.layer = cfg, layer
        self.inp = sdev.layer_inputs(cfg, layer, device, x=x)
        if pool is None:
            pool = sdev.expert_pool(cfg, [layer] * cfg.E, list(range(cfg.E)), device)
        self.pool = pool
        self.slot_of_host = slot_of
        self.slot_of = (torch.as_tensor(np.asarray(slot_of, np.int32), device=device)
                        if slot_of is not None else None)
        self.S = num_slots if num_slots is not None else cfg.E
        self.desc = moe.LayerDesc(cfg.E, cfg.k, cfg.H, cfg.I, self.inp["router_w"],
                                  cfg.router_fmt, cfg.wfmt, pool, shared=self.inp["shared"],
                                  router_bias=self.inp["bias"], slot_of_expert=self.slot_of,
                                  num_slots=self.S)
        self.T = self.inp["x"].shape[0]

    def outputs(self):
        import torch
        T, k, H = self.T, self.cfg.k, self.cfg.H
        dev = self.inp["x"].device
        return {
            "y": torch.full((T, H), float("nan"), dtype=torch.float32, device=dev),
            "idx": torch.full((T, k), -7, dtype=torch.int32, device=dev),
            "gate": torch.full((T, k), float("nan"), dtype=torch.float32, device=dev),
            "slot_idx": torch.full((T, k), -7, dtype=torch.int32, device=dev),
            "miss": torch.full((max(T * k, 1) * 3,), -7, dtype=torch.int32, device=dev),
            "miss_off": torch.full((T + 1,), -7, dtype=torch.int32, device=dev),
        }

    def run_layer(self, ws=None):
        import routed_expert_ffn_gemv_amd as moe
        o = self.outputs()
        ws = ws if ws is not None else moe.workspace(self.desc, self.T)
        moe.moe_layer(self.desc, self.inp["x"], self.T, o["y"], o["idx"], o["gate"],
                      o["slot_idx"], o["miss"], o["miss_off"], ws)
        return o

    def run_steps(self):
        """The same layer through the four separate calls."""
        import torch
        import routed_expert_ffn_gemv_amd as moe
        T, k, H, S = self.T, self.cfg.k, self.cfg.H, self.S
        dev = self.inp["x"].device
        o = self.outputs()
        ws = moe.workspace(self.desc, T)
        moe.moe_route(self.desc, self.inp["x"], T, o["idx"], o["gate"], ws)
        o["bucket_off"] = torch.full((S + 1,), -7, dtype=torch.int32, device=dev)
        o["bucket_pair"] = torch.full((max(T * k, 1),), -7, dtype=torch.int32, device=dev)
        moe.moe_resolve_slots(self.desc, o["idx"], o["gate"], T, o["slot_idx"], o["bucket_off"],
                              o["bucket_pair"], o["miss"], o["miss_off"], ws)
        o["pair_out"] = torch.zeros((T * k, H), dtype=torch.float32, device=dev)
        o["shared_out"] = (torch.zeros((T, H), dtype=torch.float32, device=dev)
                           if self.cfg.shared else None)
        moe.moe_expert_ffn(self.desc, self.inp["x"], T, o["bucket_off"], o["bucket_pair"],
                           o["pair_out"], o["shared_out"], ws)
        moe.moe_combine(self.desc, T, o["slot_idx"], o["gate"], o["pair_out"], o["shared_out"],
                        o["y"])
        return o

    def run_accum(self, o, base=None):
        """moe_expert_ffn_accum on the buckets of a run_steps result: y =
        base (zeros by default) + the gate-weighted expert outputs + the
        shared expert's."""
        import torch
        import routed_expert_ffn_gemv_amd as moe
        T, H = self.T, self.cfg.H
        y = (torch.zeros((T, H), dtype=torch.float32, device=self.inp["x"].device)
             if base is None else base.clone())
        ws = moe.workspace(self.desc, T)
        moe.moe_expert_ffn_accum(self.desc, self.inp["x"], T, o["bucket_off"], o["bucket_pair"],
                                 o["gate"], y, ws)
        return y

    def oracle(self, tokens=None, with_misses=False):
        return oracle.layer_from_synth(self.cfg, self.layer, self.inp["x_host"],
                                       slot_of=self.slot_of_host, num_slots=self.S,
                                       tokens=tokens, with_misses=with_misses)


def host(t):
    return t.detach().cpu().numpy()


def check_routing(o, ref, k):
    """Bit-exact indices, slots, miss list; gates within TOL."""
    import routed_expert_ffn_gemv_amd as moe
    np.testing.assert_array_equal(host(o["idx"]), ref["idx"])
    g = host(o["gate"]).astype(np.float64)
    assert np.abs(g - ref["gate"]).max() <= TOL * np.abs(ref["gate"]).max()
    assert np.all(np.abs(g - ref["gate"]) <= TOL * np.abs(ref["gate"]))
    np.testing.assert_array_equal(host(o["slot_idx"]), ref["slot_idx"])
    moff = host(o["miss_off"])
    np.testing.assert_array_equal(moff, ref["miss_off"])
    n = int(moff[-1])
    me, mt, mg = moe.unpack_miss(o["miss"], n)
    np.testing.assert_array_equal(me, ref["miss_expert"])
    np.testing.assert_array_equal(mt, ref["miss_token"])
    # the miss gate is the GPU's own gate, bit for bit
    gflat = host(o["gate"]).ravel()
    sl = ref["slot_idx"].ravel()
    np.testing.assert_array_equal(mg, gflat[sl < 0])
