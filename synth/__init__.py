"""Seeded synthetic inputs for the routed-MoE layer, shared by the oracle and
the HIP path.

This module only draws numbers; it holds none of the layer's arithmetic
(no routing, no dequantisation, no FFN).  Every value is a pure function of
(seed, tag, layer, index) through a counter-based SplitMix64 hash, so any
expert of any layer can be regenerated on its own (random access), and the
GPU fill kernel in ``fill.hip`` reproduces the integer-only planes (packed
codes, fp16 scales and mins) byte for byte.

Definitions (all arithmetic mod 2**64):
  mix64(z)        = SplitMix64 finaliser (Steele, Lea, Flood 2014).
  key(s,t,l,i)    = mix64(mix64(mix64(mix64(s) ^ t) ^ l) ^ i)
  word(key, n)    = mix64(key + (n + 1) * 0x9E3779B97F4A7C15)
Normals use Box-Muller in fp64 on two words; bf16 values are the
round-to-nearest-even of the fp32 rounding of that normal.

Quantised blocks (32 weights along a row, one fp16 scale d and one fp16
min m per block, weight = d*q + m):
  2-bit: d = (256+u) * 2^-13, u in [0,256);   m = -(768 + 3u + v) * 2^-14
  4-bit: d = (64+u)  * 2^-13, u in [0,64);    m = -(960 + 15u + v) * 2^-14
with v in [-16, 16]; both are exact fp16 numbers built from integers, so the
weights have mean ~0 and standard deviation ~0.05.
"""

import ctypes
import math
import os

import numpy as np

from .configs import (CONFIGS, MoEConfig, ZIPF_ALPHA, ZIPF_R0, ZIPF_S,
                      bits_of, expert_bytes, matrix_bytes)

__all__ = ["CONFIGS", "MoEConfig", "bits_of", "expert_bytes", "matrix_bytes",
           "mix64", "key", "words", "normals", "bf16_bits", "bf16_to_f64",
           "f16_to_f64", "gen_x", "gen_x_rows", "gen_router", "gen_bias",
           "popularity_rank", "resident_counts", "slot_layout",
           "gen_matrix", "gen_expert", "gen_pool", "SHARED_ID",
           "TAG_X", "TAG_ROUTER", "TAG_BIAS", "mat_tag"]

GOLDEN = 0x9E3779B97F4A7C15
M64 = (1 << 64) - 1

TAG_X = 1
TAG_ROUTER = 2
TAG_BIAS = 3
TAG_RESIDENT = 4
SHARED_ID = 0xFFFFF          # expert index used for the shared expert
MATRICES = ("gate", "up", "down")
PLANE_CODES, PLANE_BLOCKS, PLANE_F32 = 0, 1, 2


def mat_tag(matrix, plane):
    """Tag of one plane of one expert matrix (matrix in gate/up/down)."""
    return 16 + 4 * MATRICES.index(matrix) + plane


def _mix64_int(z):
    z &= M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def mix64(z):
    """SplitMix64 finaliser on a uint64 numpy array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def key(seed, tag, layer, index):
    k = _mix64_int(seed)
    k = _mix64_int(k ^ tag)
    k = _mix64_int(k ^ layer)
    return _mix64_int(k ^ index)


def words(k, n, start=0):
    ctr = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(k) + ctr * np.uint64(GOLDEN))


def normals(k, n):
    """n standard normals: Box-Muller (cosine branch) on word pairs."""
    w = words(k, 2 * n).reshape(n, 2)
    u1 = ((w[:, 0] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = (w[:, 1] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def bf16_bits(a):
    """bf16 bit patterns (uint16) of fp64 values: fp64 -> fp32 -> bf16, RNE."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f64(b):
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f16_to_f64(b):
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- activations
def gen_x_rows(cfg, layer, tokens, attempts=None):
    """bf16 bits [len(tokens)][H] of N(0,1) activations.  Row t of attempt a
    is drawn from key(seed, TAG_X, layer, t*256 + a); attempt > 0 re-draws a
    token (used when a caller needs a margin between routing logits)."""
    tokens = np.asarray(tokens, dtype=np.int64).ravel()
    if attempts is None:
        attempts = np.zeros_like(tokens)
    out = np.empty((len(tokens), cfg.H), dtype=np.uint16)
    for r, (t, a) in enumerate(zip(tokens.tolist(), np.asarray(attempts).ravel().tolist())):
        out[r] = bf16_bits(normals(key(cfg.seed, TAG_X, layer, t * 256 + a), cfg.H))
    return out


def gen_x(cfg, layer, T=None, attempts=None):
    T = cfg.T if T is None else T
    return gen_x_rows(cfg, layer, np.arange(T), attempts)


# ---------------------------------------------------------------- router
def gen_router(cfg, layer):
    """Router weights [E][H], N(0, 0.02): fp32 array (router_fmt f32) or
    bf16 bits uint16 (router_fmt bf16)."""
    W = np.empty((cfg.E, cfg.H), dtype=np.float64)
    for e in range(cfg.E):
        W[e] = 0.02 * normals(key(cfg.seed, TAG_ROUTER, layer, e), cfg.H)
    if cfg.router_fmt == "f32":
        return W.astype(np.float32)
    return bf16_bits(W)


def popularity_rank(cfg, layer):
    """Seeded per-layer popularity rank of each expert (0 = most popular), so
    popular experts are not the low ids."""
    w = words(key(cfg.seed, TAG_BIAS, layer, 0), cfg.E)
    order = np.argsort(w, kind="stable")
    rank = np.empty(cfg.E, dtype=np.int64)
    rank[order] = np.arange(cfg.E)
    return rank


def gen_bias(cfg, layer):
    """Per-expert popularity bias [E] fp32, or None when the config has none."""
    if cfg.bias == "none":
        return None
    r = popularity_rank(cfg, layer).astype(np.float64)
    return (-ZIPF_ALPHA * ZIPF_S * np.log(r + ZIPF_R0)).astype(np.float32)


# ---------------------------------------------------------------- slot table
def resident_counts(cfg):
    """Experts resident per layer for a tiered config: integers in
    resident_range, both ends present, summing to resident_total.  Starts
    from an even split and applies seeded transfers between layers."""
    lo, hi = cfg.resident_range
    L, total = cfg.layers, cfg.resident_total
    w = [int(v) for v in words(key(cfg.seed, TAG_RESIDENT, 0, 0), 3 * 2000)]
    n = [total // L] * L
    for i in range(total - sum(n)):
        n[i] += 1
    for i in range(0, len(w), 3):
        a, b, amt = w[i] % L, w[i + 1] % L, w[i + 2] % 9
        if a != b and n[a] - amt > lo and n[b] + amt < hi:
            n[a] -= amt
            n[b] += amt
    a = min(range(L), key=lambda l: (n[l], l))
    b = max(range(L), key=lambda l: (n[l], -l))
    n[a], n[b] = lo, hi
    l = 0
    while sum(n) != total:          # restore the total on the other layers
        if l not in (a, b):
            if sum(n) > total and n[l] > lo + 1:
                n[l] -= 1
            elif sum(n) < total and n[l] < hi - 1:
                n[l] += 1
        l = (l + 1) % L
    return np.array(n, dtype=np.int64)


def slot_layout(cfg):
    """Slot tables of a config.

    Returns (slot_of, slot_layer, slot_expert, num_slots):
      slot_of[layer][E] int32   slot id of each expert, -1 if not resident;
      slot_layer/slot_expert    the (layer, expert) each slot holds.
    identity: every layer has its own pool of E slots, slot = expert id
    (slot_layer is then the layer of the pool).  tiered: one pool of
    resident_total slots shared by all layers, layer l's n_l most popular
    experts (by popularity_rank) placed in rank order after layer l-1's.
    """
    if cfg.slots == "identity":
        slot_of = np.tile(np.arange(cfg.E, dtype=np.int32), (cfg.layers, 1))
        return slot_of, None, None, cfg.E
    n = resident_counts(cfg)
    slot_of = np.full((cfg.layers, cfg.E), -1, dtype=np.int32)
    slot_layer, slot_expert = [], []
    s = 0
    for l in range(cfg.layers):
        rank = popularity_rank(cfg, l)
        for e in np.argsort(rank, kind="stable")[: n[l]]:
            slot_of[l, e] = s
            slot_layer.append(l)
            slot_expert.append(int(e))
            s += 1
    return (slot_of, np.array(slot_layer, np.int32),
            np.array(slot_expert, np.int32), s)


# ---------------------------------------------------------------- experts
def _f16_from_int(N, e=-14):
    """fp16 bits of N * 2^e for integer arrays N in [512, 2048)."""
    N = np.asarray(N, dtype=np.int64)
    p = np.where(N >= 1024, 10, 9)
    expo = p + e + 15
    mant = (N - (1 << p)) << (10 - p)
    return ((expo << 10) | mant).astype(np.uint16)


def _blocks(kk, nblocks, bits):
    w = words(kk, nblocks)
    u_mask = np.uint64(0xFF if bits == 2 else 0x3F)
    u = (w & u_mask).astype(np.int64)
    v = ((w >> np.uint64(32)) % np.uint64(33)).astype(np.int64) - 16
    if bits == 2:
        d = ((10 << 10) | (u << 2)).astype(np.uint16)      # (256+u) 2^-13
        m = _f16_from_int(768 + 3 * u + v) | np.uint16(0x8000)
    else:
        d = ((8 << 10) | (u << 4)).astype(np.uint16)       # (64+u) 2^-13
        m = _f16_from_int(960 + 15 * u + v) | np.uint16(0x8000)
    return d, m


def gen_matrix(cfg, layer, expert, matrix):
    """One expert matrix.  gate/up are [I][H], down is [H][I] (row-major,
    K contiguous).  f32: {'w': float32 [rows][cols]}, N(0, 0.05).
    q2/q4: {'codes': uint8 [rows*cols*bits/8], 'scale': uint16 [rows][cols/32],
            'min': uint16 [rows][cols/32]} (fp16 bits)."""
    rows, cols = (cfg.I, cfg.H) if matrix != "down" else (cfg.H, cfg.I)
    if cfg.wfmt == "f32":
        kk = key(cfg.seed, mat_tag(matrix, PLANE_F32), layer, expert)
        w = (0.05 * normals(kk, rows * cols)).astype(np.float32)
        return {"w": w.reshape(rows, cols)}
    bits = bits_of(cfg.wfmt)
    nbytes = rows * cols * bits // 8
    codes = words(key(cfg.seed, mat_tag(matrix, PLANE_CODES), layer, expert),
                  nbytes // 8).view(np.uint8)
    d, m = _blocks(key(cfg.seed, mat_tag(matrix, PLANE_BLOCKS), layer, expert),
                   rows * cols // 32, bits)
    return {"codes": codes, "scale": d.reshape(rows, cols // 32),
            "min": m.reshape(rows, cols // 32)}


def gen_expert(cfg, layer, expert):
    return {m: gen_matrix(cfg, layer, expert, m) for m in MATRICES}


def gen_pool(cfg, layer_expert_pairs, matrix):
    """Host pool of one matrix for a list of (layer, expert) slots, planes
    stacked by slot: f32 -> float32 [S][rows][cols]; q -> (codes [S][bytes],
    scale [S][rows][cols/32], min [S][rows][cols/32])."""
    mats = [gen_matrix(cfg, l, e, matrix) for (l, e) in layer_expert_pairs]
    if cfg.wfmt == "f32":
        return np.stack([m["w"] for m in mats])
    return (np.stack([m["codes"] for m in mats]),
            np.stack([m["scale"] for m in mats]),
            np.stack([m["min"] for m in mats]))


# ---------------------------------------------------------------- GPU fill
_LIB = None
_HERE = os.path.dirname(os.path.abspath(__file__))


def fill_lib():
    """The GPU fill library (libsynth.so, built from fill.hip)."""
    global _LIB
    if _LIB is None:
        import torch  # noqa: F401  (bind to PyTorch's HIP runtime first)
        path = os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(path):
            raise RuntimeError("synth/libsynth.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.synth_fill_q.restype = ctypes.c_int
        lib.synth_fill_q.argtypes = [
            ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p]
        _LIB = lib
    return _LIB


def fill_pool_device(cfg, matrix, slot_layers, slot_experts, codes, scale, mn,
                     stream=0):
    """Fill a device pool of one quantised matrix on the GPU.

    slot_layers / slot_experts: device int32 tensors [S] naming the (layer,
    expert) held by each slot (SHARED_ID for the shared expert).  codes /
    scale / mn: device tensors sized for S slots.  Byte-identical to
    gen_matrix() for every slot."""
    rows, cols = (cfg.I, cfg.H) if matrix != "down" else (cfg.H, cfg.I)
    S = int(slot_experts.numel())
    rc = fill_lib().synth_fill_q(
        ctypes.c_uint64(cfg.seed), MATRICES.index(matrix), bits_of(cfg.wfmt),
        rows, cols, 0, ctypes.c_void_p(slot_layers.data_ptr()),
        ctypes.c_void_p(slot_experts.data_ptr()), S,
        ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scale.data_ptr()),
        ctypes.c_void_p(mn.data_ptr()), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill_q failed with status {rc}")


def build():
    """Compile libsynth.so (the GPU fill kernel) for gfx950."""
    import subprocess
    src = os.path.join(_HERE, "fill.hip")
    out = os.path.join(_HERE, "libsynth.so")
    subprocess.check_call(["/opt/rocm/bin/hipcc", "-O3", "-std=c++17", "-fPIC", "-shared",
                           "--offload-arch=gfx950", "-mcode-object-version=5", "-Xclang", "-target-feature", "-Xclang",
                           "-packed-fp32-ops", "-x", "hip", src, "-o", out],
                          stderr=subprocess.DEVNULL)
    return out
