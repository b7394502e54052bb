"""ctypes binding of the fp64 reference oracle (liboracle.so, oracle.cpp).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product path
(``routed_expert_ffn_gemv_amd``) never does and shares no code with it.

Besides thin wrappers of the C functions, ``layer_from_synth`` composes the
oracle's own steps for one layer of a big configuration, regenerating on the
host (through ``synth``) only the experts the routing chose.  All of the
layer's arithmetic happens inside liboracle.so.
"""

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

FMT = {"f32": 0, "bf16": 1, "q2": 2, "q4": 3}

_P = ctypes.c_void_p


def build():
    """Compile liboracle.so with g++ (plain -O2, no fast-math)."""
    src = os.path.join(_HERE, "oracle.cpp")
    out = os.path.join(_HERE, "liboracle.so")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared",
                           "-fno-fast-math", "-ffp-contract=off", src, "-o", out])
    return out


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            build()
        L = ctypes.CDLL(path)
        L.oracle_bf16.restype = ctypes.c_double
        L.oracle_bf16.argtypes = [ctypes.c_uint16]
        L.oracle_f16.restype = ctypes.c_double
        L.oracle_f16.argtypes = [ctypes.c_uint16]
        for name in ("oracle_dequant", "oracle_router", "oracle_topk", "oracle_resolve",
                     "oracle_bucket", "oracle_ffn", "oracle_combine", "oracle_layer",
                     "oracle_count_usage", "oracle_slot_refresh", "oracle_verify_accept"):
            getattr(L, name).restype = ctypes.c_int
        _LIB = L
    return _LIB


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_P)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what}: oracle rejected the arguments (status {rc})")


def bf16(b):
    return lib().oracle_bf16(int(b))


def f16(b):
    return lib().oracle_f16(int(b))


def dequant(fmt, rows, cols, data, scale=None, mn=None):
    out = np.empty((rows, cols), np.float64)
    data = np.ascontiguousarray(data)
    scale, mn = _c(scale, np.uint16), _c(mn, np.uint16)
    _check(lib().oracle_dequant(FMT[fmt], rows, cols, _ptr(data), _ptr(scale), _ptr(mn),
                                _ptr(out)), "dequant")
    return out


def router(x, W, router_fmt, bias=None):
    x = _c(x, np.uint16)
    T, H = x.shape
    W = np.ascontiguousarray(W)
    E = W.shape[0]
    bias = _c(bias, np.float32)
    out = np.empty((T, E), np.float64)
    _check(lib().oracle_router(T, E, H, _ptr(x), FMT[router_fmt], _ptr(W), _ptr(bias),
                               _ptr(out)), "router")
    return out


def topk(logits, k):
    logits = _c(logits, np.float64)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    gate = np.empty((T, k), np.float64)
    _check(lib().oracle_topk(T, E, k, _ptr(logits), _ptr(idx), _ptr(gate)), "topk")
    return idx, gate


def verify_accept(logits, draft):
    """Tokens kept by a verify pass: the model's greedy tokens g_0 .. g_a,
    where the first a drafts equal g_0 .. g_{a-1} (oracle_verify_accept)."""
    logits = _c(logits, np.float64)
    T, V = logits.shape
    draft = np.zeros(max(T - 1, 1), np.int32) if T == 1 else _c(draft, np.int32)
    out = np.empty(T, np.int32)
    n = np.zeros(1, np.int32)
    _check(lib().oracle_verify_accept(T, V, _ptr(logits), _ptr(draft), _ptr(out), _ptr(n)),
           "verify_accept")
    return out[: int(n[0])].copy()


def resolve(idx, gate, E, slot_of=None):
    idx, gate = _c(idx, np.int32), _c(gate, np.float64)
    T, k = idx.shape
    slot_of = _c(slot_of, np.int32)
    slot_idx = np.empty((T, k), np.int32)
    me = np.empty(T * k, np.int32)
    mt = np.empty(T * k, np.int32)
    mg = np.empty(T * k, np.float64)
    moff = np.empty(T + 1, np.int32)
    _check(lib().oracle_resolve(T, k, E, _ptr(idx), _ptr(gate), _ptr(slot_of), _ptr(slot_idx),
                                _ptr(me), _ptr(mt), _ptr(mg), _ptr(moff)), "resolve")
    n = int(moff[T])
    return slot_idx, me[:n].copy(), mt[:n].copy(), mg[:n].copy(), moff


def bucket(slot_idx, S):
    slot_idx = _c(slot_idx, np.int32)
    T, k = slot_idx.shape
    off = np.empty(S + 1, np.int32)
    pairs = np.empty(max(T * k, 1), np.int32)
    _check(lib().oracle_bucket(T, k, S, _ptr(slot_idx), _ptr(off), _ptr(pairs)), "bucket")
    return off, pairs[: int(off[S])].copy()


def count_usage(idx, E, usage=None):
    """usage[e] += number of choices of e in idx [T][k] (uint32 [E])."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    usage = np.zeros(E, np.uint32) if usage is None else np.ascontiguousarray(usage, np.uint32).copy()
    _check(lib().oracle_count_usage(T, k, E, _ptr(idx), _ptr(usage)), "count_usage")
    return usage


def slot_refresh(usage, slot_of, expert_of, max_swaps):
    """One refresh of a global slot table.  Returns (swaps [n][3], usage,
    slot_of, expert_of) after it, the inputs left unchanged."""
    usage = np.array(usage, np.uint32)
    slot_of = np.array(slot_of, np.int32)
    expert_of = np.array(expert_of, np.int32)
    swaps = np.zeros((max(max_swaps, 1), 3), np.int32)
    n = np.zeros(1, np.int32)
    _check(lib().oracle_slot_refresh(len(usage), len(expert_of), _ptr(usage), _ptr(slot_of),
                                     _ptr(expert_of), int(max_swaps), _ptr(swaps), _ptr(n)),
           "slot_refresh")
    return swaps[: int(n[0])].copy(), usage, slot_of, expert_of


def _mat_args(fmt, m):
    if fmt == "f32":
        return [_ptr(_c(m["w"], np.float32)), None, None], [m["w"]]
    keep = [np.ascontiguousarray(m["codes"]), _c(m["scale"], np.uint16), _c(m["min"], np.uint16)]
    return [_ptr(a) for a in keep], keep


def ffn(fmt, H, I, expert, x):
    """o [n][H] fp64 of one expert (dict gate/up/down of synth.gen_matrix
    layout) for bf16 tokens x [n][H]."""
    x = _c(x, np.uint16).reshape(-1, H)
    n = x.shape[0]
    o = np.empty((n, H), np.float64)
    args, keep = [], []
    for m in ("gate", "up", "down"):
        a, kp = _mat_args(fmt, expert[m])
        args += a
        keep += kp
    _check(lib().oracle_ffn(FMT[fmt], H, I, *args, n, _ptr(x), _ptr(o)), "ffn")
    return o


def combine(slot_idx, gate, pair_out, shared=None):
    slot_idx, gate = _c(slot_idx, np.int32), _c(gate, np.float64)
    T, k = slot_idx.shape
    pair_out = _c(pair_out, np.float64)
    H = pair_out.shape[-1]
    shared = _c(shared, np.float64)
    y = np.empty((T, H), np.float64)
    _check(lib().oracle_combine(T, k, H, _ptr(slot_idx), _ptr(gate), _ptr(pair_out),
                                _ptr(shared), _ptr(y)), "combine")
    return y


def layer(x, router_w, router_fmt, bias, k, fmt, pools, I, slot_of=None, shared=None,
          num_slots=None):
    """Whole layer with host pools.  pools: {'gate','up','down'} each f32
    [S][rows][cols] or (codes, scale, min) stacked by slot; shared: the same
    for one expert (leading dim 1) or None."""
    x = _c(x, np.uint16)
    T, H = x.shape
    E = router_w.shape[0]
    S = num_slots if num_slots is not None else E
    keep = [x]

    def planes(p):
        if p is None:
            return [None, None, None]
        if fmt == "f32":
            a = _c(p, np.float32)
            keep.append(a)
            return [_ptr(a), None, None]
        arrs = [np.ascontiguousarray(p[0]), _c(p[1], np.uint16), _c(p[2], np.uint16)]
        keep.extend(arrs)
        return [_ptr(a) for a in arrs]

    W = np.ascontiguousarray(router_w)
    bias = _c(bias, np.float32)
    slot_of = _c(slot_of, np.int32)
    y = np.empty((T, H), np.float64)
    idx = np.empty((T, k), np.int32)
    gate = np.empty((T, k), np.float64)
    slot_idx = np.empty((T, k), np.int32)
    me = np.empty(T * k, np.int32)
    mt = np.empty(T * k, np.int32)
    mg = np.empty(T * k, np.float64)
    moff = np.empty(T + 1, np.int32)
    boff = np.empty(S + 1, np.int32)
    bpair = np.empty(max(T * k, 1), np.int32)
    sh = shared or {}
    args = (planes(pools["gate"]) + planes(pools["up"]) + planes(pools["down"])
            + planes(sh.get("gate")) + planes(sh.get("up")) + planes(sh.get("down")))
    _check(lib().oracle_layer(T, E, k, H, I, S, _ptr(x), FMT[router_fmt], _ptr(W), _ptr(bias),
                              _ptr(slot_of), FMT[fmt], *args, _ptr(y), _ptr(idx), _ptr(gate),
                              _ptr(slot_idx), _ptr(me), _ptr(mt), _ptr(mg), _ptr(moff),
                              _ptr(boff), _ptr(bpair)), "layer")
    n = int(moff[T])
    return {"y": y, "idx": idx, "gate": gate, "slot_idx": slot_idx,
            "miss_expert": me[:n].copy(), "miss_token": mt[:n].copy(),
            "miss_gate": mg[:n].copy(), "miss_off": moff,
            "bucket_off": boff, "bucket_pair": bpair[: int(boff[S])].copy()}


def route_from_synth(cfg, layer_id, x, slot_of=None, num_slots=None, threads=1):
    """Oracle routing of one layer of a synthetic config: logits, top-k,
    gates, slot resolution, miss list and buckets (all in liboracle.so;
    threads > 1 splits the router rows over threads)."""
    import synth
    W = synth.gen_router(cfg, layer_id)
    bias = synth.gen_bias(cfg, layer_id)
    logits = (router_threads(x, W, cfg.router_fmt, bias, threads) if threads > 1
              else router(x, W, cfg.router_fmt, bias))
    idx, gate = topk(logits, cfg.k)
    S = num_slots if num_slots is not None else cfg.E
    slot_idx, me, mt, mg, moff = resolve(idx, gate, cfg.E, slot_of)
    boff, bpair = bucket(slot_idx, S)
    return {"logits": logits, "idx": idx, "gate": gate, "slot_idx": slot_idx,
            "miss_expert": me, "miss_token": mt, "miss_gate": mg, "miss_off": moff,
            "bucket_off": boff, "bucket_pair": bpair}


def layer_from_synth(cfg, layer_id, x, slot_of=None, num_slots=None, tokens=None,
                     with_misses=False, route=None, threads=1):
    """Oracle outputs of one layer of a synthetic config.

    Routing covers every token of x; the FFN and combine cover `tokens`
    (default: all).  Each expert's weights are regenerated by synth on the
    host.  with_misses also returns y_full, where missed experts are added
    as if they were resident.  route: a result of route_from_synth to reuse.
    threads > 1 runs the router rows and the experts' FFN calls in threads;
    every call is still the single-threaded oracle and each expert's rows
    land at fixed places, so the result does not depend on the thread
    count."""
    import synth
    r = dict(route) if route is not None else route_from_synth(cfg, layer_id, x, slot_of,
                                                                num_slots, threads)
    T = x.shape[0]
    k, H, I = cfg.k, cfg.H, cfg.I
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    pair_out = np.zeros((T * k, H), np.float64)
    by_expert = {}
    for t in tokens.tolist():
        for j in range(k):
            p = t * k + j
            if r["slot_idx"].ravel()[p] >= 0 or with_misses:
                by_expert.setdefault(int(r["idx"].ravel()[p]), []).append(p)
    jobs = [(e, np.array(ps)) for e, ps in sorted(by_expert.items())]
    if cfg.shared:
        jobs.append((synth.SHARED_ID, None))

    def one(job):
        e, ps = job
        ex = synth.gen_expert(cfg, layer_id, e)
        toks = tokens if ps is None else ps // k
        return ffn(cfg.wfmt, H, I, ex, x[toks])

    if threads > 1 and len(jobs) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(min(threads, len(jobs))) as pool:
            outs = list(pool.map(one, jobs))
    else:
        outs = [one(j) for j in jobs]
    shared = None
    for (e, ps), o in zip(jobs, outs):
        if ps is None:
            shared = np.zeros((T, H), np.float64)
            shared[tokens] = o
        else:
            pair_out[ps] = o
    y = combine(r["slot_idx"], r["gate"], pair_out, shared)
    r["y"] = y
    r["pair_out"] = pair_out
    r["shared_out"] = shared
    r["tokens"] = tokens
    if with_misses:
        all_hit = np.zeros_like(r["slot_idx"])
        r["y_full"] = combine(all_hit, r["gate"], pair_out, shared)
    return r


def router_threads(x, W, router_fmt, bias=None, threads=None):
    """oracle.router over row chunks in parallel threads (each call is the
    single-threaded oracle; ctypes releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    x = _c(x, np.uint16)
    T = x.shape[0]
    threads = threads or min(16, os.cpu_count() or 1)
    if T < 64 or threads <= 1:
        return router(x, W, router_fmt, bias)
    chunks = np.array_split(np.arange(T), threads)
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda c: router(x[c], W, router_fmt, bias), chunks))
    return np.concatenate(parts)


def min_top_gap(logits, k):
    """Smallest difference between consecutive values among the k+1 largest
    logits of each row (descending)."""
    top = -np.sort(-logits, axis=1)[:, : k + 1]
    return (top[:, :-1] - top[:, 1:]).min(axis=1)


def margin_x(cfg, layer_id, T=None, min_gap=1e-3, max_attempts=64, threads=None):
    """Synthetic activations with a routing margin: token rows are re-drawn
    (synth attempt counter) until every gap between consecutive logits of the
    top-(k+1), by the oracle's fp64 router, is at least min_gap.  Returns
    (x bf16 bits [T][H], attempts [T])."""
    import synth
    T = cfg.T if T is None else T
    W = synth.gen_router(cfg, layer_id)
    bias = synth.gen_bias(cfg, layer_id)
    attempts = np.zeros(T, np.int64)
    x = synth.gen_x(cfg, layer_id, T)
    todo = np.arange(T)
    for _ in range(max_attempts):
        l = router_threads(x[todo], W, cfg.router_fmt, bias, threads)
        bad = todo[min_top_gap(l, cfg.k) < min_gap]
        if len(bad) == 0:
            return x, attempts
        attempts[bad] += 1
        x[bad] = synth.gen_x_rows(cfg, layer_id, bad, attempts[bad])
        todo = bad
    raise RuntimeError("could not draw activations with the requested routing margin")
