"""Python binding of libmoe.so, the MI355X (gfx950) routed-MoE layer.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch provides device memory (tensors) and the stream; functions take
torch tensors, pass their device pointers and the current HIP stream, and
raise MoEError on a non-zero status.  The names follow include/moe.h.

The library must be built (``__graft_entry__.build()`` or
``python -m routed_expert_ffn_gemv_amd.build``); importing fails loudly when
it is missing -- there is no fallback implementation.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
MOE_W_F32, MOE_W_BF16, MOE_W_Q2B32, MOE_W_Q4B32 = range(4)
MOE_LAYER_MAX_T = 16
FORMATS = {"f32": MOE_W_F32, "bf16": MOE_W_BF16, "q2": MOE_W_Q2B32, "q4": MOE_W_Q4B32}

# Every symbol include/moe.h declares.
EXPORTS = ("moe_status_string", "moe_version", "moe_workspace_size", "moe_route",
           "moe_resolve_slots", "moe_expert_ffn", "moe_combine", "moe_layer",
           "moe_slot_refresh_workspace_size", "moe_slot_refresh", "moe_host_miss_ffn",
           "moe_host_isa", "moe_verify_workspace_size", "moe_verify_accept",
           "moe_prefill_workspace_size", "moe_prefill_layer", "moe_layer_check",
           "moe_set_wait_budget", "moe_set_trace", "moe_layer_noalloc",
           "moe_expert_ffn_accum", "moe_set_deterministic")
MOE_REFRESH_MAX_SWAPS = 1024


class MoEError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class moe_mat(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("data", ctypes.c_void_p),
                ("scale", ctypes.c_void_p), ("min", ctypes.c_void_p)]


class moe_layer_desc(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("k", ctypes.c_int32), ("H", ctypes.c_int32),
                ("I", ctypes.c_int32), ("num_slots", ctypes.c_int32),
                ("router_fmt", ctypes.c_int32), ("router_w", ctypes.c_void_p),
                ("router_bias", ctypes.c_void_p), ("slot_of_expert", ctypes.c_void_p),
                ("gate", moe_mat), ("up", moe_mat), ("down", moe_mat),
                ("sh_gate", moe_mat), ("sh_up", moe_mat), ("sh_down", moe_mat),
                ("usage_counts", ctypes.c_void_p)]


class moe_slot_pool(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("E", ctypes.c_int32), ("H", ctypes.c_int32),
                ("I", ctypes.c_int32), ("num_slots", ctypes.c_int32),
                ("gate", moe_mat), ("up", moe_mat), ("down", moe_mat),
                ("store_gate", moe_mat), ("store_up", moe_mat), ("store_down", moe_mat),
                ("usage", ctypes.c_void_p), ("slot_of", ctypes.c_void_p),
                ("expert_of", ctypes.c_void_p)]


class moe_miss(ctypes.Structure):
    _fields_ = [("expert", ctypes.c_int32), ("token", ctypes.c_int32), ("gate", ctypes.c_float)]


def _load():
    # libmoe.so must bind to the HIP runtime PyTorch loads (one runtime per
    # process), so PyTorch is imported before the library is opened.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                          "(there is no CPU fallback for the MoE layer)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D = ctypes.POINTER(moe_layer_desc)
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [I32]
    lib.moe_version.restype = I32
    lib.moe_version.argtypes = []
    lib.moe_workspace_size.restype = I32
    lib.moe_workspace_size.argtypes = [D, I32, ctypes.POINTER(SZ)]
    lib.moe_route.restype = I32
    lib.moe_route.argtypes = [D, P, I32, P, P, P, SZ, P]
    lib.moe_resolve_slots.restype = I32
    lib.moe_resolve_slots.argtypes = [D, P, P, I32, P, P, P, P, P, P, SZ, P]
    lib.moe_expert_ffn.restype = I32
    lib.moe_expert_ffn.argtypes = [D, P, I32, P, P, P, P, P, SZ, P]
    lib.moe_expert_ffn_accum.restype = I32
    lib.moe_expert_ffn_accum.argtypes = [D, P, I32, P, P, P, P, P, SZ, P]
    lib.moe_combine.restype = I32
    lib.moe_combine.argtypes = [D, I32, P, P, P, P, P, P]
    lib.moe_layer.restype = I32
    lib.moe_layer.argtypes = [D, P, I32, P, P, P, P, P, P, P, SZ, P]
    lib.moe_layer_noalloc.restype = I32
    lib.moe_layer_noalloc.argtypes = [D, P, I32, P, P, P, P, P, P, P]
    lib.moe_layer_check.restype = I32
    lib.moe_layer_check.argtypes = [P, SZ, P]
    lib.moe_set_wait_budget.restype = None
    lib.moe_set_wait_budget.argtypes = [ctypes.c_uint64, I32]
    lib.moe_set_trace.restype = None
    lib.moe_set_trace.argtypes = [P]
    lib.moe_set_deterministic.restype = None
    lib.moe_set_deterministic.argtypes = [I32]
    SP = ctypes.POINTER(moe_slot_pool)
    lib.moe_slot_refresh_workspace_size.restype = I32
    lib.moe_slot_refresh_workspace_size.argtypes = [SP, ctypes.POINTER(SZ)]
    lib.moe_slot_refresh.restype = I32
    lib.moe_slot_refresh.argtypes = [SP, I32, P, P, P, SZ, P]
    lib.moe_prefill_workspace_size.restype = I32
    lib.moe_prefill_workspace_size.argtypes = [D, I32, I32, ctypes.POINTER(SZ)]
    lib.moe_prefill_layer.restype = I32
    lib.moe_prefill_layer.argtypes = [D, P, I32, I32, P, P, P, P, P, SZ, P, P]
    lib.moe_verify_workspace_size.restype = I32
    lib.moe_verify_workspace_size.argtypes = [I32, I32, ctypes.POINTER(SZ)]
    lib.moe_verify_accept.restype = I32
    lib.moe_verify_accept.argtypes = [P, I32, I32, P, P, P, P, SZ, P]
    lib.moe_host_isa.restype = I32
    lib.moe_host_isa.argtypes = []
    lib.moe_host_miss_ffn.restype = I32
    lib.moe_host_miss_ffn.argtypes = [I32, I32, I32, moe_mat, moe_mat, moe_mat, P, I32, P, P, P,
                                      I32]
    return lib


lib = _load()


def status_string(status):
    return lib.moe_status_string(int(status)).decode()


def moe_version():
    return lib.moe_version()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status, what):
    if status != MOE_OK:
        raise MoEError(status, what)


class LayerDesc:
    """A moe_layer_desc built from torch tensors (kept alive here).

    router_w: [E][H] fp32 or bf16-bits (int16/uint16/bfloat16) tensor;
    pools: dict gate/up/down -> tensor (f32) or (codes, scale, min) tensors
    stacked by slot; shared: the same dict for the shared expert or None."""

    def __init__(self, E, k, H, I, router_w, router_fmt, wfmt, pools, shared=None,
                 router_bias=None, slot_of_expert=None, num_slots=None, usage_counts=None):
        self._keep = [router_w, router_bias, slot_of_expert, pools, shared, usage_counts]
        d = moe_layer_desc()
        d.E, d.k, d.H, d.I = E, k, H, I
        d.num_slots = E if num_slots is None else num_slots
        d.router_fmt = FORMATS[router_fmt] if isinstance(router_fmt, str) else router_fmt
        d.router_w = _ptr(router_w)
        d.router_bias = _ptr(router_bias)
        d.slot_of_expert = _ptr(slot_of_expert)
        d.usage_counts = _ptr(usage_counts)
        fmt = FORMATS[wfmt] if isinstance(wfmt, str) else wfmt
        for name in ("gate", "up", "down"):
            setattr(d, name, self._mat(fmt, pools[name]))
            if shared is not None:
                setattr(d, "sh_" + name, self._mat(fmt, shared[name]))
        self.desc = d
        self.E, self.k, self.H, self.I, self.fmt = E, k, H, I, fmt
        self.num_slots = d.num_slots
        self.has_shared = shared is not None

    @staticmethod
    def _mat(fmt, p):
        m = moe_mat()
        m.fmt = fmt
        if fmt == MOE_W_F32 or fmt == MOE_W_BF16:
            m.data = _ptr(p)
        else:
            m.data, m.scale, m.min = _ptr(p[0]), _ptr(p[1]), _ptr(p[2])
        return m

    @property
    def ref(self):
        return ctypes.byref(self.desc)


def moe_workspace_size(desc, T):
    n = ctypes.c_size_t(0)
    _check(lib.moe_workspace_size(desc.ref, int(T), ctypes.byref(n)), "moe_workspace_size")
    return n.value


def workspace(desc, T, device="cuda"):
    """A zeroed uint8 device tensor large enough for every call at this T
    (moe_layer needs the workspace zeroed before its first use)."""
    import torch
    n = moe_workspace_size(desc, T)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def moe_route(desc, x, T, topk_idx, topk_gate, ws, stream=None):
    _check(lib.moe_route(desc.ref, _ptr(x), int(T), _ptr(topk_idx), _ptr(topk_gate), _ptr(ws),
                         ws.numel() if ws is not None else 0, _stream(stream)), "moe_route")


def moe_resolve_slots(desc, topk_idx, topk_gate, T, slot_idx, bucket_off, bucket_pair, miss,
                      miss_off, ws, stream=None):
    """miss: a device tensor of T*k*3 int32 words (moe_miss records)."""
    _check(lib.moe_resolve_slots(desc.ref, _ptr(topk_idx), _ptr(topk_gate), int(T),
                                 _ptr(slot_idx), _ptr(bucket_off), _ptr(bucket_pair), _ptr(miss),
                                 _ptr(miss_off), _ptr(ws), ws.numel() if ws is not None else 0,
                                 _stream(stream)), "moe_resolve_slots")


def moe_expert_ffn(desc, x, T, bucket_off, bucket_pair, pair_out, shared_out, ws, stream=None):
    _check(lib.moe_expert_ffn(desc.ref, _ptr(x), int(T), _ptr(bucket_off), _ptr(bucket_pair),
                              _ptr(pair_out), _ptr(shared_out), _ptr(ws),
                              ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_expert_ffn")


def moe_expert_ffn_accum(desc, x, T, bucket_off, bucket_pair, topk_gate, y, ws, stream=None):
    """y [T][H] += the gate-weighted expert outputs and the shared expert's."""
    _check(lib.moe_expert_ffn_accum(desc.ref, _ptr(x), int(T), _ptr(bucket_off),
                                    _ptr(bucket_pair), _ptr(topk_gate), _ptr(y), _ptr(ws),
                                    ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_expert_ffn_accum")


def moe_combine(desc, T, slot_idx, topk_gate, pair_out, shared_out, y, stream=None):
    _check(lib.moe_combine(desc.ref, int(T), _ptr(slot_idx), _ptr(topk_gate), _ptr(pair_out),
                           _ptr(shared_out), _ptr(y), _stream(stream)), "moe_combine")


def moe_layer(desc, x, T, y, topk_idx, topk_gate, slot_idx, miss, miss_off, ws, stream=None):
    _check(lib.moe_layer(desc.ref, _ptr(x), int(T), _ptr(y), _ptr(topk_idx), _ptr(topk_gate),
                         _ptr(slot_idx), _ptr(miss), _ptr(miss_off), _ptr(ws),
                         ws.numel() if ws is not None else 0, _stream(stream)), "moe_layer")


def moe_layer_noalloc(desc, x, T, y, topk_idx, topk_gate, slot_idx, miss, miss_off, stream=None):
    """moe_layer without a workspace: the hand-off region is the library's
    static device array (fused shapes only)."""
    _check(lib.moe_layer_noalloc(desc.ref, _ptr(x), int(T), _ptr(y), _ptr(topk_idx),
                                 _ptr(topk_gate), _ptr(slot_idx), _ptr(miss), _ptr(miss_off),
                                 _stream(stream)), "moe_layer_noalloc")


def moe_layer_check(ws, stream=None):
    """Raises MoEError(MOE_ERR_DEVICE) if a fused moe_layer call on ws (None:
    moe_layer_noalloc's static region of this GPU) gave up a bounded wait
    (waits for the stream)."""
    _check(lib.moe_layer_check(_ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_layer_check")


def moe_set_wait_budget(ns=0, hold=False):
    """Budget of the fused launch's waits in ns (0: the default, 100 ms);
    hold=True makes later fused launches run out of it (test hook)."""
    lib.moe_set_wait_budget(int(ns), 1 if hold else 0)


def moe_set_trace(trace):
    """Phase stamps of later fused moe_layer launches into trace (a uint64-
    sized int64 device tensor of [1024][32] words), or None to stop."""
    lib.moe_set_trace(_ptr(trace))


def moe_set_deterministic(on=True):
    """Fixed-order sums into y for later fused moe_layer launches (True), or
    the float-atomic sums (False, the default)."""
    lib.moe_set_deterministic(1 if on else 0)


class SlotPool:
    """A moe_slot_pool built from torch tensors (kept alive here): pools and
    store as dicts gate/up/down -> tensor (f32) or (codes, scale, min);
    usage uint32-as-int32 [L*E], slot_of int32 [L*E], expert_of int32 [S]."""

    def __init__(self, L, E, H, I, wfmt, pool, store, usage, slot_of, expert_of, num_slots):
        self._keep = [pool, store, usage, slot_of, expert_of]
        p = moe_slot_pool()
        p.L, p.E, p.H, p.I, p.num_slots = L, E, H, I, num_slots
        fmt = FORMATS[wfmt] if isinstance(wfmt, str) else wfmt
        for name in ("gate", "up", "down"):
            setattr(p, name, LayerDesc._mat(fmt, pool[name]))
            setattr(p, "store_" + name, LayerDesc._mat(fmt, store[name]))
        p.usage, p.slot_of, p.expert_of = _ptr(usage), _ptr(slot_of), _ptr(expert_of)
        self.pool = p

    @property
    def ref(self):
        return ctypes.byref(self.pool)


def moe_slot_refresh(pool, max_swaps, swaps, n_swaps, stream=None):
    """swaps: int32 device tensor [>= max_swaps * 3]; n_swaps: int32 [1]."""
    _check(lib.moe_slot_refresh(pool.ref, int(max_swaps), _ptr(swaps), _ptr(n_swaps), None, 0,
                                _stream(stream)), "moe_slot_refresh")


def moe_prefill_workspace_size(desc, T, chunk):
    n = ctypes.c_size_t(0)
    _check(lib.moe_prefill_workspace_size(desc.ref, int(T), int(chunk), ctypes.byref(n)),
           "moe_prefill_workspace_size")
    return n.value


def moe_prefill_layer(desc, x, T, chunk, y, topk_idx, topk_gate, slot_idx, ws, stream=None,
                      aux_stream=None):
    """aux_stream: a second torch.cuda.Stream (or None: everything on stream)."""
    aux = None if aux_stream is None else (aux_stream if isinstance(aux_stream, int)
                                           else aux_stream.cuda_stream)
    _check(lib.moe_prefill_layer(desc.ref, _ptr(x), int(T), int(chunk), _ptr(y), _ptr(topk_idx),
                                 _ptr(topk_gate), _ptr(slot_idx), _ptr(ws),
                                 ws.numel() if ws is not None else 0, _stream(stream), aux),
           "moe_prefill_layer")


def moe_verify_workspace_size(T, V):
    n = ctypes.c_size_t(0)
    _check(lib.moe_verify_workspace_size(int(T), int(V), ctypes.byref(n)),
           "moe_verify_workspace_size")
    return n.value


def moe_verify_accept(logits, T, V, draft, out_tokens, n_out, ws, stream=None):
    """logits: fp32 device [T][V]; draft: int32 [T-1] (None when T = 1);
    out_tokens: int32 [T]; n_out: int32 [1]; ws: uint8 device tensor of at
    least moe_verify_workspace_size(T, V) bytes."""
    _check(lib.moe_verify_accept(_ptr(logits), int(T), int(V), _ptr(draft), _ptr(out_tokens),
                                 _ptr(n_out), _ptr(ws), ws.numel() if ws is not None else 0,
                                 _stream(stream)), "moe_verify_accept")


def _hptr(a, dtype):
    """Address of a C-contiguous host array (numpy, or a CPU torch tensor)."""
    import numpy as np
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        want = np.dtype(dtype)
        same_bits = (a.dtype.kind in "iu" and want.kind in "iu" and a.dtype.itemsize == want.itemsize)
        if not a.flags["C_CONTIGUOUS"] or not (a.dtype == want or same_bits):
            raise ValueError(f"host array must be C-contiguous {want}")
        return a.ctypes.data
    if getattr(a, "is_cuda", False) or not a.is_contiguous():
        raise ValueError("host tensor must be a contiguous CPU tensor")
    return a.data_ptr()


def moe_host_miss_ffn(E, H, I, wfmt, gate, up, down, x, T, miss, miss_off, y, n_threads=0):
    """Host tier: y [T][H] float32 += each listed miss's expert output, on
    the CPU.  gate/up/down: the layer's experts by id in host memory, f32
    arrays [n][rows][cols] or (codes uint8, scale uint16, min uint16) tuples;
    x: uint16 bf16 bits [T][H]; miss: int32 words of moe_miss records;
    miss_off: int32 [T+1].  Host arrays only; synchronous."""
    import numpy as np
    fmt = FORMATS[wfmt] if isinstance(wfmt, str) else wfmt

    def mat(p):
        m = moe_mat()
        m.fmt = fmt
        if fmt == MOE_W_F32:
            m.data = _hptr(p, np.float32)
        else:
            m.data, m.scale, m.min = _hptr(p[0], np.uint8), _hptr(p[1], np.uint16), _hptr(p[2], np.uint16)
        return m
    mats = [mat(gate), mat(up), mat(down)]
    _check(lib.moe_host_miss_ffn(int(E), int(H), int(I), *mats, _hptr(x, np.uint16), int(T),
                                 _hptr(miss, np.int32), _hptr(miss_off, np.int32),
                                 _hptr(y, np.float32), int(n_threads)), "moe_host_miss_ffn")


def moe_host_isa():
    """1: the host tier runs AVX-512 code; 0: plain C++."""
    return lib.moe_host_isa()


def unpack_miss(miss_tensor, n):
    """(expert, token, gate) numpy arrays of the first n moe_miss records of
    a device or host int32 tensor [>= 3n]."""
    import numpy as np
    raw = miss_tensor[: 3 * n].cpu().numpy().astype(np.int32).reshape(n, 3)
    return raw[:, 0].copy(), raw[:, 1].copy(), raw[:, 2].copy().view(np.float32)
