"""Benchmark of the routed-MoE layer on one MI355X.

Default workload: the decode layer (E = 512 experts, top-10, hidden 2048,
intermediate 768, 2-bit experts + a shared expert, 1 token per step).  One
step = one moe_layer call: router, top-k and gates, slot resolution, the
expert FFN of the chosen experts, the shared expert and the combine.  To
keep the weights out of the 256 MB Infinity Cache, steps cycle through
`--layers` independent copies of the layer (48 by default, like the model's
stack: 43.5 GB of expert weights) and through distinct tokens, so every
step streams its experts from HBM as a real decode step does.

Prints one JSON line (see the keys below).  By default the line is the
decode layer's, and it carries two more legs under "legs": the 48-layer
4-token verify stack (c3, step = 48 moe_layer calls) and the prefill of
32,768 tokens through one layer (c5), each with its own roofline and CPU
baseline.  --config c2/c3/c4/c4a/c5 measures one workload alone (c4: the
16-token slot-table stack; c4a: the same with the adaptive slot table).

No timed step repeats a (layer, tokens) pair of the warm-up: steps draw
their tokens from a step counter that runs on from the warm-up.  The
distinct experts of every timed call (for the algorithmic bytes) come from
the slot tables those calls write, one buffer per call.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode/4-tok verify); prefill MFMA util"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


_SLEEP_NS_PER_CYCLE = []


def hold_queue(n_launches, per_launch_us=40.0):
    """Queue a spin kernel on the current stream ahead of a timed region, long
    enough for the host to enqueue the region's n_launches launches behind
    it (per_launch_us is a generous bound on the host's cost per launch).
    The region then runs back to back, and its first event is not stamped
    while the GPU still waits for the first launch: without this, a short
    region also times the host's marshalling of its first calls."""
    import torch
    if not _SLEEP_NS_PER_CYCLE:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        a.record()
        torch.cuda._sleep(1 << 20)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_NS_PER_CYCLE.append(a.elapsed_time(b) * 1e6 / (1 << 20))
    ns = (n_launches * per_launch_us + 2000.0) * 1e3
    torch.cuda._sleep(int(ns / max(_SLEEP_NS_PER_CYCLE[0], 1e-3)))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


class pinned_core:
    """Runs the block with this process pinned to one host core (the last
    one it may use), then restores the affinity.  Reports the host."""

    def __enter__(self):
        self.before = os.sched_getaffinity(0)
        self.core = max(self.before)
        os.sched_setaffinity(0, {self.core})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.before)

    def info(self):
        return {"cores": 1, "pinned_core": self.core, "cpu_model": cpu_model(),
                "host_cpus": os.cpu_count(), "cpus_allowed": len(self.before)}


# HBM bytes per launch of the roofline kernel(s), from two rocprofv3 --pmc
# passes (FETCH_SIZE, then WRITE_SIZE) over the same bench command, each
# scaled by what the counter reads for a 256 MiB device copy run in the same
# process (--copy-probe 256).  The summaries are under profiles/.  A figure
# is reported only while the kernel sources it was measured on are unchanged
# (their SHA-256 below); otherwise traffic is null.
KERNEL_SOURCES = {
    "decode": ["routed_expert_ffn_gemv_amd/csrc/layer.hip", "routed_expert_ffn_gemv_amd/csrc/layer.h",
               "routed_expert_ffn_gemv_amd/csrc/gemv_core.h", "routed_expert_ffn_gemv_amd/csrc/common.h",
               "routed_expert_ffn_gemv_amd/build.py"],
    "prefill": ["routed_expert_ffn_gemv_amd/csrc/ffn_gemm.hip", "routed_expert_ffn_gemv_amd/csrc/resolve.hip",
                "routed_expert_ffn_gemv_amd/csrc/gemv_core.h", "routed_expert_ffn_gemv_amd/csrc/common.h",
                "routed_expert_ffn_gemv_amd/build.py"],
}
TRAFFIC = {
    # workload: {"sha256": ..., "bytes": fetched + written per launch}
    # c2: the moe_layer kernel (profiles/c2_decode_layer_hbm_traffic.md)
    "c2_decode_layer_q2": {"sha256": "414b3dd770c9eb0f8add72ac88e3a3adf9ba262d609e90a6f800f95b8d7e2690",
                           "bytes": 23067323},
    # c3: the moe_layer kernel (profiles/c3_verify_stack_hbm_traffic.md)
    "c3_verify_stack_q2": {"sha256": "414b3dd770c9eb0f8add72ac88e3a3adf9ba262d609e90a6f800f95b8d7e2690",
                           "bytes": 69957373},
    # c4: the moe_layer kernel (profiles/c4_slot_tiering_hbm_traffic.md)
    "c4_slot_tiering_q2": {"sha256": "414b3dd770c9eb0f8add72ac88e3a3adf9ba262d609e90a6f800f95b8d7e2690",
                           "bytes": 122847317},
    # c5: the kernels of one moe_expert_ffn call (active list, schedule, x16,
    # gate/up and down GEMMs; profiles/c5_prefill_hbm_traffic.md)
    "c5_prefill_q4": {"sha256": "60e44c72388bf65f02e182f4083d57b020dc015a61f0d171f19085e8a1ed5810",
                      "bytes": 8853574533},
}


def sources_sha256(kind):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kind):
    t = TRAFFIC.get(workload)
    if t is None or t["sha256"] != sources_sha256(kind):
        return None
    return t["bytes"]


def algorithmic_bytes_decode(cfg, n_experts_read, T):
    """HBM bytes one layer must move: router weights + bias, each distinct
    expert read once (gate, up, down planes), the shared expert, the
    activations in and the fp32 outputs out."""
    import synth
    router = cfg.E * cfg.H * (2 if cfg.router_fmt == "bf16" else 4)
    bias = cfg.E * 4 if cfg.bias != "none" else 0
    experts = (n_experts_read + (1 if cfg.shared else 0)) * synth.expert_bytes(cfg)
    io = T * cfg.H * 2 + T * cfg.H * 4
    return router + bias + experts + io


def cpu_baseline_decode(cfg, n_calls, layers):
    """The oracle (single-threaded fp64, pinned to one core) on a bounded
    sample: n_calls layer calls of cfg's T tokens, each on its own layer;
    input generation untimed.  Returns (seconds per layer call, elapsed, host
    info)."""
    import oracle
    import synth
    elapsed = 0.0
    with pinned_core() as pc:
        for i in range(n_calls):
            layer = i % layers
            x = synth.gen_x_rows(cfg, layer, 1000 + np.arange(cfg.T) + i * cfg.T)
            W = synth.gen_router(cfg, layer)
            bias = synth.gen_bias(cfg, layer)
            t0 = time.perf_counter()
            logits = oracle.router(x, W, cfg.router_fmt, bias)
            idx, gate = oracle.topk(logits, cfg.k)
            slot_idx, *_ = oracle.resolve(idx, gate, cfg.E, None)
            elapsed += time.perf_counter() - t0
            experts = {int(e): synth.gen_expert(cfg, layer, int(e)) for e in np.unique(idx)}
            shared = synth.gen_expert(cfg, layer, synth.SHARED_ID) if cfg.shared else None
            t0 = time.perf_counter()
            pair_out = np.zeros((cfg.T * cfg.k, cfg.H))
            for e in sorted(experts):
                ps = np.nonzero(idx.ravel() == e)[0]
                pair_out[ps] = oracle.ffn(cfg.wfmt, cfg.H, cfg.I, experts[e], x[ps // cfg.k])
            sh = oracle.ffn(cfg.wfmt, cfg.H, cfg.I, shared, x) if shared else None
            oracle.combine(slot_idx, gate, pair_out, sh)
            elapsed += time.perf_counter() - t0
        info = pc.info()
    return elapsed / n_calls, elapsed, info


def bench_decode(args, cfg_name, steps=None, warmup=None, cpu_calls=None):
    """One decode workload: c2 (a step = one moe_layer call, cycling through
    --layers layer copies) or a 48-layer stack c3 / c4 (a step = 48 calls)."""
    import torch
    import routed_expert_ffn_gemv_amd as moe
    import synth
    from synth import device as sdev

    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    cfg = synth.CONFIGS[cfg_name]
    T = cfg.T
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    L = args.layers if cfg.layers == 1 else cfg.layers
    n_steps = warmup + steps + args.phase_trace
    # token groups: c2 uses group s // L on layer s % L; a stack uses group
    # s mod 64 (every layer) -- so no (layer, tokens) pair occurs twice within
    # 64 steps of a stack (a stack step streams ~3 GB, far beyond the 256 MB
    # Infinity Cache, so later repeats find nothing cached either)
    ngroups = n_steps // L + 1 if cfg.layers == 1 else min(n_steps, 64)
    log(f"[bench] {cfg.name}: building {L} layers on the device ({ngroups} token groups)")
    t0 = time.time()
    slot_of, sl, se, S = synth.slot_layout(cfg) if cfg.slots == "tiered" else (None, None, None, cfg.E)
    global_pool = sdev.expert_pool(cfg, sl, se, dev) if cfg.slots == "tiered" else None
    layers = []
    for l in range(L):
        inp = sdev.layer_inputs(cfg, l, dev, x=synth.gen_x(cfg, l, T * ngroups))
        pool = global_pool if global_pool is not None else sdev.expert_pool(
            cfg, [l] * cfg.E, list(range(cfg.E)), dev)
        so = (torch.as_tensor(slot_of[l], device=dev) if slot_of is not None else None)
        desc = moe.LayerDesc(cfg.E, cfg.k, cfg.H, cfg.I, inp["router_w"], cfg.router_fmt,
                             cfg.wfmt, pool, shared=inp["shared"], router_bias=inp["bias"],
                             slot_of_expert=so, num_slots=S)
        layers.append((desc, inp, pool, so))
    torch.cuda.synchronize()
    log(f"[bench] setup {time.time() - t0:.1f}s")
    k, H = cfg.k, cfg.H
    ws = moe.workspace(layers[0][0], T, dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    calls_per_step = 1 if cfg.layers == 1 else L
    moe.moe_set_deterministic(bool(args.fixed_order))
    # one slot table per timed call: the distinct experts those calls read
    slot_rec = torch.empty((max(steps, 1), calls_per_step, T, k), dtype=torch.int32, device=dev)
    slot_tmp = torch.empty((T, k), dtype=torch.int32, device=dev)
    miss = torch.empty((T * k * 3,), dtype=torch.int32, device=dev)
    miss_off = torch.empty((T + 1,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step(s, rec):
        """Step s: one layer (c2) or the whole stack (c3/c4); rec: the step's
        slot-table buffer [calls][T][k] or None."""
        if cfg.layers == 1:
            desc, inp, _, _ = layers[s % L]
            g = s // L
            moe.moe_layer(desc, inp["x"][g * T:(g + 1) * T], T, y, idx, gate,
                          rec[0] if rec is not None else slot_tmp, miss, miss_off, ws, stream)
        else:
            g = s % ngroups
            for l, (desc, inp, _, _) in enumerate(layers):
                moe.moe_layer(desc, inp["x"][g * T:(g + 1) * T], T, y, idx, gate,
                              rec[l] if rec is not None else slot_tmp, miss, miss_off, ws, stream)

    for s in range(warmup):
        step(s, None)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_queue(steps * calls_per_step)
    e0.record(stream)
    for i in range(steps):
        step(warmup + i, slot_rec[i])
    e1.record(stream)
    torch.cuda.synchronize()
    moe.moe_layer_check(ws)
    ms = e0.elapsed_time(e1) / steps
    ms_call = ms / calls_per_step
    rec = slot_rec.cpu().numpy().reshape(steps * calls_per_step, T * k)
    uniq = [len(np.unique(r[r >= 0])) for r in rec]
    u = float(np.mean(uniq))
    bytes_call = algorithmic_bytes_decode(cfg, u, T)
    gbs = bytes_call / (ms_call * 1e-3) / 1e9
    tokens_per_s = T / (ms * 1e-3)
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q2 weights, bf16 activations, f32 accumulation" if cfg.wfmt == "q2" else cfg.wfmt,
        "data": "synthetic",
        "config": {"workload": cfg.name, "E": cfg.E, "k": cfg.k, "H": cfg.H, "I": cfg.I,
                   "T": T, "layers": L, "weights": cfg.wfmt, "shared_expert": cfg.shared,
                   "slots": cfg.slots, "step": "one moe_layer call" if cfg.layers == 1
                   else f"{L} moe_layer calls (one per layer)",
                   "sums": "fixed order" if args.fixed_order else "float atomics"},
        "hbm_gbs": round(gbs, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(cfg.name, "decode"),
                     "kernel": "moe_layer (whole call)", "bytes_per_launch": int(bytes_call),
                     "launch_ms": round(ms_call, 5), "distinct_experts_per_layer": round(u, 2)},
    }
    if args.host_tier and cfg.slots == "tiered":
        out["host_tier"] = host_tier_leg(cfg, layers, ws, ms)
    if args.phase_trace:
        out["phase_trace"] = phase_trace(args.phase_trace, lambda s: step(s, None),
                                         warmup + steps, n_steps)
    del layers, global_pool
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        n = cpu_calls if cpu_calls is not None else (args.cpu_tokens if cfg.layers == 1 else 3)
        log(f"[bench] cpu baseline: oracle on {n} layer calls of {T} tokens")
        sec, el, info = cpu_baseline_decode(cfg, n, L)
        step_s = sec * calls_per_step
        out["cpu_baseline"] = dict({"value": round(T / step_s, 4), "unit": "tokens/s",
                                    "kind": "oracle",
                                    "sample": f"{n} layer calls of {T} token(s) of {cfg.name} "
                                              f"(router..combine, fp64, one pinned thread, "
                                              f"{el:.1f}s), scaled to a step of "
                                              f"{calls_per_step} call(s)"}, **info)
    return out


PHASES = [(0, "start"), (2, "tokens staged"), (3, "router/shared tasks (wave 0)"),
          (21, "router/shared tasks (last wave)"), (4, "every logit seen (wave 0)"),
          (11, "every logit seen (all waves)"),
          (22, "  top-k: segment maxima"), (23, "  top-k: thresholds"),
          (28, "  top-k: candidates listed"),
          (16, "  routing: candidates listed"), (17, "  routing: second barrier"),
          (18, "  routing: ranks"), (19, "  routing: gates"), (20, "  routing: resolved"),
          (5, "routing done"), (6, "gate/up done (wave 0)"), (7, "gate/up done (last wave)"),
          (12, "down phase entered"), (24, "  down: LDS free (barrier)"),
          (25, "  down: h sources set (barrier)"), (13, "first unit's h present"),
          (26, "  down: h converted (thread 0)"), (27, "  down: staging barrier"),
          (8, "first h staged"), (9, "down done"), (10, "end")]


def phase_trace(n_calls, run_step, first_step, n_distinct):
    """Phase stamps of n_calls further fused launches (steps after the timed
    ones, so cold), one call per step: per phase, the median and the maximum
    over workgroups of the time since the first workgroup started, then the
    median over calls; and each XCD's median start offset (us)."""
    import torch
    import routed_expert_ffn_gemv_amd as moe
    tr = torch.zeros((1024, 32), dtype=torch.int64, device="cuda")
    per_phase = {name: [] for _, name in PHASES}
    polls = {"lg": [], "h": []}
    xcd_start = {}
    moe.moe_set_trace(tr)
    try:
        for i in range(n_calls):
            s = first_step + i
            if s >= n_distinct:
                break
            tr.zero_()
            run_step(s)
            torch.cuda.synchronize()
            t = tr.cpu().numpy()
            t = t[t[:, 0] > 0]
            t0 = t[:, 0].min()
            for slot, name in PHASES:
                v = t[:, slot]
                v = v[v > 0]
                if len(v):
                    per_phase[name].append((np.median(v - t0) / 100.0, (v.max() - t0) / 100.0))
            polls["lg"] += [int(v) for v in t[:, 15] if v > 0]
            polls["h"] += [int(v) for v in t[:, 14] if v > 0]
            for x in np.unique(t[:, 1]):
                xcd_start.setdefault(int(x), []).append(np.median(t[t[:, 1] == x, 0] - t0) / 100.0)
    finally:
        moe.moe_set_trace(None)
    res = {"calls": len(per_phase["start"]), "unit": "us since the first workgroup started",
           "poll_rounds_median": {"logits (thread 0)": float(np.median(polls["lg"])) if polls["lg"] else None,
                                  "first h (thread 0)": float(np.median(polls["h"])) if polls["h"] else None},
           "phases": {name: {"median_over_wgs": round(float(np.median([a for a, _ in v])), 2),
                             "max_over_wgs": round(float(np.median([b for _, b in v])), 2)}
                      for name, v in per_phase.items() if v},
           "xcd_start_median": {str(x): round(float(np.median(v)), 2)
                                for x, v in sorted(xcd_start.items())}}
    log("[bench] phase trace (us since the first workgroup started; medians over calls)")
    log("| phase | median over workgroups | last workgroup |")
    log("|---|---:|---:|")
    for name, v in res["phases"].items():
        log(f"| {name} | {v['median_over_wgs']:.2f} | {v['max_over_wgs']:.2f} |")
    log("XCD start offsets: " + ", ".join(f"{x}: {v:.2f}" for x, v in res["xcd_start_median"].items()))
    log(f"poll rounds (median over workgroups and calls): {res['poll_rounds_median']}")
    return res


def host_tier_leg(cfg, layers, ws, gpu_ms):
    """The misses of one step of a tiered stack, computed by the host tier
    (moe_host_miss_ffn) from host copies of the missed experts' weights.
    One extra GPU step keeps every layer's miss list; the host then runs the
    48 layers' lists in turn (each call multi-threaded), timed as a whole."""
    import torch
    import routed_expert_ffn_gemv_amd as moe
    from synth import device as sdev
    dev = torch.device("cuda", 0)
    T, k, H = cfg.T, cfg.k, cfg.H
    lists = []
    for l, (desc, inp, _, _) in enumerate(layers):
        y = torch.empty((T, H), dtype=torch.float32, device=dev)
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        gate = torch.empty((T, k), dtype=torch.float32, device=dev)
        slot_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        miss = torch.empty((T * k * 3,), dtype=torch.int32, device=dev)
        miss_off = torch.empty((T + 1,), dtype=torch.int32, device=dev)
        moe.moe_layer(desc, inp["x"], T, y, idx, gate, slot_idx, miss, miss_off, ws)
        lists.append((miss, miss_off))
    torch.cuda.synchronize()
    work = []   # per layer: host store of the missed experts, remapped list, x
    n_miss = n_uniq = 0
    for l, ((miss, miss_off), (desc, inp, _, _)) in enumerate(zip(lists, layers)):
        moff = miss_off.cpu().numpy().astype(np.int32)
        m = miss.cpu().numpy()[: 3 * moff[-1]].reshape(-1, 3).copy()
        experts = np.unique(m[:, 0])
        n_miss += len(m)
        n_uniq += len(experts)
        if len(m) == 0:
            continue
        m[:, 0] = np.searchsorted(experts, m[:, 0])
        pool = sdev.expert_pool(cfg, [l] * len(experts), experts.tolist(), dev)
        store = {name: tuple(t.cpu().numpy() for t in pool[name]) for name in ("gate", "up", "down")}
        del pool
        work.append((len(experts), store, m.ravel().copy(), moff, inp["x"].cpu().numpy()))
    torch.cuda.empty_cache()
    threads = min(16, os.cpu_count() or 1)
    ys = np.zeros((T, H), np.float32)

    def one_step():
        for n_e, store, m, moff, x in work:
            moe.moe_host_miss_ffn(n_e, H, cfg.I, cfg.wfmt, store["gate"], store["up"],
                                  store["down"], x, T, m, moff, ys, threads)
    one_step()   # first touch of the host copies
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        one_step()
        times.append(time.perf_counter() - t0)
    ms = float(np.median(times)) * 1e3
    import synth
    gb = n_uniq * synth.expert_bytes(cfg) / 1e9
    return {"ms_per_step": round(ms, 3), "misses_per_step": int(n_miss),
            "distinct_missed_experts": int(n_uniq), "weight_gb_per_step": round(gb, 3),
            "gbs": round(gb / (ms * 1e-3), 1), "threads": threads,
            "isa": "avx512" if moe.moe_host_isa() else "generic",
            "gpu_ms_per_step": round(gpu_ms, 4),
            "note": "host tier (CPU) computing the step's misses from host-memory weights; "
                    "the GPU figure is the same step's hits and shared expert"}


def bench_adaptive(args):
    """c4's 48-layer, 16-token stack on a pool filled from a profile that does
    not match the traffic (each layer's residents drawn at random), with the
    adaptive tier on: usage counted by every layer call, moe_slot_refresh
    with at most 96 swaps every 4 rounds.  A round is one step (48 layer
    calls) on fresh tokens.  Reports the hit rate as the pool adapts, then
    times steady-state rounds, refreshes included."""
    import torch
    import routed_expert_ffn_gemv_amd as moe
    import synth
    from synth import device as sdev

    cfg = synth.CONFIGS["c4"]
    T, k, E, H, L = cfg.T, cfg.k, cfg.E, cfg.H, cfg.layers
    N = L * E
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log("[bench] c4a: store of every expert, cold pool, layer inputs")
    t0 = time.time()
    n_l = synth.resident_counts(cfg)
    rng = np.random.default_rng(0xC4A)
    slot_layer, slot_expert = [], []
    for l in range(L):
        for e in rng.permutation(E)[: n_l[l]]:
            slot_layer.append(l)
            slot_expert.append(int(e))
    S = len(slot_expert)
    slot_of_h = np.full(N, -1, np.int32)
    slot_of_h[np.array(slot_layer) * E + np.array(slot_expert)] = np.arange(S, dtype=np.int32)
    expert_of_h = (np.array(slot_layer) * E + np.array(slot_expert)).astype(np.int32)
    store = sdev.expert_pool(cfg, np.repeat(np.arange(L), E), np.tile(np.arange(E), L), dev)
    pool = sdev.expert_pool(cfg, slot_layer, slot_expert, dev)
    usage = torch.zeros(N, dtype=torch.int32, device=dev)
    slot_of = torch.as_tensor(slot_of_h, device=dev)
    expert_of = torch.as_tensor(expert_of_h, device=dev)
    sp = moe.SlotPool(L, E, H, cfg.I, cfg.wfmt, pool, store, usage, slot_of, expert_of, S)
    n_x = 32                      # distinct rounds of tokens, cycled
    layers = []
    for l in range(L):
        inp = sdev.layer_inputs(cfg, l, dev, x=synth.gen_x(cfg, l, T * n_x))
        desc = moe.LayerDesc(E, k, H, cfg.I, inp["router_w"], cfg.router_fmt, cfg.wfmt, pool,
                             shared=inp["shared"], router_bias=inp["bias"],
                             slot_of_expert=slot_of[l * E:(l + 1) * E], num_slots=S,
                             usage_counts=usage[l * E:(l + 1) * E])
        layers.append((desc, inp))
    torch.cuda.synchronize()
    log(f"[bench] setup {time.time() - t0:.1f}s")
    ws = moe.workspace(layers[0][0], T, dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    slot_idx = torch.empty((L, T, k), dtype=torch.int32, device=dev)
    miss = torch.empty((T * k * 3,), dtype=torch.int32, device=dev)
    miss_off = torch.empty((L, T + 1), dtype=torch.int32, device=dev)
    swaps = torch.empty((96 * 3,), dtype=torch.int32, device=dev)
    n_swaps = torch.zeros((1,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def round_(r):
        j = r % n_x
        for l, (desc, inp) in enumerate(layers):
            moe.moe_layer(desc, inp["x"][j * T:(j + 1) * T], T, y, idx, gate, slot_idx[l], miss,
                          miss_off[l], ws, stream)
        if r % 4 == 3:
            moe.moe_slot_refresh(sp, 96, swaps, n_swaps, stream)

    # adaptation: hit rate per round (untimed; reads the miss counts)
    R = 256
    hits, swapped = [], 0
    uniq = []
    for r in range(R):
        round_(r)
        mo = miss_off[:, T].cpu().numpy()
        hits.append(1.0 - mo.sum() / (L * T * k))
        if r % 4 == 3:
            swapped += int(n_swaps.item())
        if r >= R - 8:
            for sl_h in slot_idx.cpu().numpy():
                uniq.append(len(np.unique(sl_h[sl_h >= 0])))
    # refresh cost alone
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(10):
        moe.moe_slot_refresh(sp, 96, swaps, n_swaps, stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    refresh_ms = ev[0].elapsed_time(ev[1]) / 10
    # timed steady state
    for r in range(args.warmup):
        round_(R + r)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_queue(args.steps * L * 2)
    e0.record(stream)
    for r in range(args.steps):
        round_(R + args.warmup + r)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    u = float(np.mean(uniq))
    bytes_step = L * algorithmic_bytes_decode(cfg, u, T)
    gbs = bytes_step / (ms * 1e-3) / 1e9
    hr = np.array(hits)
    return {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "q2 weights, bf16 activations, f32 accumulation",
        "data": "synthetic",
        "config": {"workload": "c4a_adaptive_slots_q2", "E": E, "k": k, "H": H, "I": cfg.I,
                   "T": T, "layers": L, "weights": cfg.wfmt, "shared_expert": cfg.shared,
                   "slots": S, "step": "48 moe_layer calls (one per layer); every 4th step "
                                       "also one moe_slot_refresh (<= 96 swaps)",
                   "initial_placement": "per layer, n_l experts drawn at random"},
        "hit_rate": {"round_0": round(float(hr[0]), 4),
                     "rounds_60_63": round(float(hr[60:64].mean()), 4),
                     "rounds_124_127": round(float(hr[124:128].mean()), 4),
                     "rounds_252_255": round(float(hr[252:256].mean()), 4)},
        "swaps_in_256_rounds": swapped,
        "refresh_ms": round(refresh_ms, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "48 moe_layer calls + refreshes", "bytes_per_step": int(bytes_step),
                     "distinct_hit_experts_per_layer": round(u, 2)},
    }


def gemm_flops(cfg, n_hit, T):
    """Algorithmic MFMA flops of the expert FFN: 2*H*I for each of gate, up
    and down, per hit pair and per token of the shared expert (no padding)."""
    per = 6 * cfg.H * cfg.I
    return per * (n_hit + (T if cfg.shared else 0))


def cpu_baseline_prefill(cfg, n_route, n_ffn):
    """Oracle (one pinned thread) on a bounded sample of the prefill layer:
    routing of n_route tokens and the FFN + combine of n_ffn of them;
    tokens/s extrapolated from the per-token times (input generation
    untimed).  Returns (tokens/s, elapsed, host info)."""
    import oracle
    import synth
    x = synth.gen_x_rows(cfg, 0, np.arange(n_route))
    W = synth.gen_router(cfg, 0)
    bias = synth.gen_bias(cfg, 0)
    with pinned_core() as pc:
        t0 = time.perf_counter()
        logits = oracle.router(x, W, cfg.router_fmt, bias)
        idx, gate = oracle.topk(logits, cfg.k)
        slot_idx, *_ = oracle.resolve(idx, gate, cfg.E, None)
        oracle.bucket(slot_idx, cfg.E)
        t_route = (time.perf_counter() - t0) / n_route
        experts = {int(e): synth.gen_expert(cfg, 0, int(e)) for e in np.unique(idx[:n_ffn])}
        shared = synth.gen_expert(cfg, 0, synth.SHARED_ID) if cfg.shared else None
        t0 = time.perf_counter()
        for t in range(n_ffn):
            po = np.stack([oracle.ffn(cfg.wfmt, cfg.H, cfg.I, experts[int(e)], x[t:t + 1])[0]
                           for e in idx[t]])
            sh = oracle.ffn(cfg.wfmt, cfg.H, cfg.I, shared, x[t:t + 1]) if shared else None
            oracle.combine(slot_idx[t:t + 1], gate[t:t + 1], po, sh)
        t_ffn = (time.perf_counter() - t0) / n_ffn
        info = pc.info()
    return 1.0 / (t_route + t_ffn), t_route * n_route + t_ffn * n_ffn, info


def bench_prefill(args, cfg_name, steps=None, warmup=None):
    """Prefill: one step = moe_route + moe_resolve_slots + moe_expert_ffn +
    moe_combine over the whole prompt (the same synthetic prompt every step:
    a step streams ~4.5 GB, so nothing of one step is cached for the next)."""
    import torch
    import routed_expert_ffn_gemv_amd as moe
    import synth
    from synth import device as sdev
    cfg = synth.CONFIGS[cfg_name]
    T, k, H, E = cfg.T, cfg.k, cfg.H, cfg.E
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"[bench] {cfg.name}: building the layer ({T} tokens)")
    t0 = time.time()
    inp = sdev.layer_inputs(cfg, 0, dev)
    pool = sdev.expert_pool(cfg, [0] * E, list(range(E)), dev)
    desc = moe.LayerDesc(E, k, H, cfg.I, inp["router_w"], cfg.router_fmt, cfg.wfmt, pool,
                         shared=inp["shared"], router_bias=inp["bias"])
    ws = moe.workspace(desc, T, dev)
    i32 = dict(dtype=torch.int32, device=dev)
    idx = torch.empty((T, k), **i32)
    gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    slot_idx = torch.empty((T, k), **i32)
    boff = torch.empty((E + 1,), **i32)
    bpair = torch.empty((T * k,), **i32)
    miss = torch.empty((T * k * 3,), **i32)
    moff = torch.empty((T + 1,), **i32)
    pair_out = torch.empty((T * k, H), dtype=torch.float32, device=dev)
    shared_out = torch.empty((T, H), dtype=torch.float32, device=dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] setup {time.time() - t0:.1f}s")
    stream = torch.cuda.current_stream()
    x = inp["x"]
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup

    def step(mode, ev=None):
        """One prefill step.  pairs: moe_expert_ffn writes every pair's output
        and moe_combine sums them; accum: y is zeroed and
        moe_expert_ffn_accum adds the gate-weighted outputs into it.  ev: five
        events recorded on the stream around the four calls (no host wait)."""
        if ev is not None:
            ev[0].record(stream)
        moe.moe_route(desc, x, T, idx, gate, ws, stream)
        if ev is not None:
            ev[1].record(stream)
        moe.moe_resolve_slots(desc, idx, gate, T, slot_idx, boff, bpair, miss, moff, ws, stream)
        if ev is not None:
            ev[2].record(stream)
        if mode == "pairs":
            moe.moe_expert_ffn(desc, x, T, boff, bpair, pair_out, shared_out, ws, stream)
        else:
            y.zero_()
            moe.moe_expert_ffn_accum(desc, x, T, boff, bpair, gate, y, ws, stream)
        if ev is not None:
            ev[3].record(stream)
        if mode == "pairs":
            moe.moe_combine(desc, T, slot_idx, gate, pair_out, shared_out, y, stream)
        if ev is not None:
            ev[4].record(stream)

    modes = ["pairs", "accum"] if args.prefill_mode == "both" else [args.prefill_mode]
    res = {}
    for mode in modes:
        for _ in range(warmup):
            step(mode)
        torch.cuda.synchronize()
        # the parts of every timed step, from events recorded on the stream
        # inside the timed region (averages over its steps)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        hold_queue(steps * 8)
        e0.record(stream)
        for i in range(steps):
            step(mode, evs[i])
        e1.record(stream)
        torch.cuda.synchronize()
        parts = np.array([[ev[j].elapsed_time(ev[j + 1]) for j in range(4)] for ev in evs])
        res[mode] = (e0.elapsed_time(e1) / steps, parts.mean(axis=0))
        log(f"[bench] prefill ({mode}): {res[mode][0]:.4f} ms per step, parts {res[mode][1]}")
    best = min(res, key=lambda m: res[m][0])
    ms, parts = res[best]
    n_hit = int(boff[-1].item())
    flops = gemm_flops(cfg, n_hit, T)
    ffn_ms = float(parts[2])
    tflops = flops / (ffn_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "q4 weights dequantised to fp16 tiles, fp16 MFMA, fp32 accumulation",
        "data": "synthetic",
        "config": {"workload": cfg.name, "E": E, "k": k, "H": H, "I": cfg.I, "T": T,
                   "weights": cfg.wfmt, "shared_expert": cfg.shared,
                   "step": ("moe_route + moe_resolve_slots + moe_expert_ffn + moe_combine"
                            if best == "pairs" else
                            "moe_route + moe_resolve_slots + zero y + moe_expert_ffn_accum")},
        "ms_route": round(float(parts[0]), 4), "ms_resolve": round(float(parts[1]), 4),
        "ms_expert_ffn": round(ffn_ms, 4), "ms_combine": round(float(parts[3]), 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(cfg.name, "prefill") if best == "pairs" else None,
                     "kernel": ("moe_expert_ffn (grouped gate/up + down GEMMs)" if best == "pairs"
                                else "zero y + moe_expert_ffn_accum (grouped gate/up + down "
                                     "GEMMs, combine fused into the down epilogue)"),
                     "flops_per_launch": int(flops)},
    }
    if len(res) > 1:
        other = [m for m in res if m != best][0]
        out["other_path"] = {"mode": other, "ms_per_step": round(res[other][0], 4),
                             "ms_expert_ffn": round(float(res[other][1][2]), 4),
                             "ms_combine": round(float(res[other][1][3]), 4)}
    if args.prefill_chunks:
        out["prefill_layer"] = []
        aux = torch.cuda.Stream()
        for c in [int(v) for v in args.prefill_chunks.split(",")]:
            for use_aux in (False, True):
                wsp = torch.zeros(moe.moe_prefill_workspace_size(desc, T, c), dtype=torch.uint8,
                                  device=dev)

                def run():
                    moe.moe_prefill_layer(desc, x, T, c, y, idx, gate, slot_idx, wsp, stream,
                                          aux if use_aux else None)
                for _ in range(2):
                    run()
                torch.cuda.synchronize()
                e0.record(stream)
                n = max(3, args.steps // 2)
                for _ in range(n):
                    run()
                e1.record(stream)
                torch.cuda.synchronize()
                out["prefill_layer"].append({"chunk": c, "aux_stream": use_aux,
                                             "ms": round(e0.elapsed_time(e1) / n, 4)})
                del wsp
                torch.cuda.empty_cache()
        log(f"[bench] prefill layer: {out['prefill_layer']}")
    del pair_out, shared_out, ws, pool
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline: oracle on a sample")
        tps, el, info = cpu_baseline_prefill(cfg, 512, 4)
        out["cpu_baseline"] = dict({"value": round(tps, 3), "unit": "tokens/s", "kind": "oracle",
                                    "sample": f"routing of 512 tokens + FFN/combine of 4 tokens "
                                              f"of {cfg.name}, extrapolated per token (fp64, one "
                                              f"pinned thread, {el:.1f}s)"}, **info)
    return out


def copy_probe(mib):
    """A plain copy of mib MiB: reads and writes exactly mib MiB of HBM."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default=None, choices=["c2", "c3", "c4", "c4a", "c5"],
                    help="one workload alone (default: c2 with the c3 and c5 legs)")
    ap.add_argument("--legs", default="c3,c5",
                    help="legs added to the default c2 line (comma-separated; '' for none)")
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--cpu-tokens", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-mode", default="both", choices=["pairs", "accum", "both"],
                    help="c5: pair outputs + moe_combine, the fused accumulate path, or both "
                         "(the faster one is the line; the other is reported beside it)")
    ap.add_argument("--prefill-chunks", default="", metavar="C1,C2,...",
                    help="c5: also time moe_prefill_layer at these chunk sizes, with and "
                         "without a second stream")
    ap.add_argument("--host-tier", action="store_true",
                    help="c4: also time the host tier on one step's misses")
    ap.add_argument("--fixed-order", action="store_true",
                    help="decode workloads: fixed-order sums into y (moe_set_deterministic)")
    ap.add_argument("--phase-trace", type=int, default=0, metavar="N",
                    help="decode workloads: after the timed steps, N more cold calls with the "
                         "fused launch's phase stamps on (medians reported)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="first run a plain device-to-device copy of MIB MiB (3 times): the "
                         "known-size kernel that scales the HBM byte counters of a profile")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
    if args.config == "c5":
        out = bench_prefill(args, "c5")
    elif args.config == "c4a":
        out = bench_adaptive(args)
    elif args.config is not None:
        out = bench_decode(args, args.config)
    else:
        out = bench_decode(args, "c2")
        legs = [l for l in args.legs.split(",") if l]
        if legs:
            out["legs"] = []
        for leg in legs:
            log(f"[bench] leg {leg}")
            out["legs"].append(bench_prefill(args, leg) if leg == "c5" else bench_decode(args, leg))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
