"""Synthetic workloads as torch device tensors (inputs only).

Activations, router weights, biases and fp32 expert weights are drawn on the
host by this package and copied to the device; packed expert planes are
filled directly in HBM by the GPU fill kernel (byte-identical to the host
generator).  Nothing here computes any part of the MoE layer.
"""

import numpy as np

from . import (SHARED_ID, bits_of, fill_pool_device, gen_bias, gen_pool, gen_router,
               gen_x, slot_layout)


def _i16(a):
    return np.ascontiguousarray(a).view(np.int16)


def to_device_bf16(a, device):
    import torch
    return torch.from_numpy(_i16(np.asarray(a, np.uint16))).to(device)


def _alloc_pool(cfg, S, matrix, device):
    import torch
    rows, cols = (cfg.I, cfg.H) if matrix != "down" else (cfg.H, cfg.I)
    if cfg.wfmt == "f32":
        return torch.empty((S, rows, cols), dtype=torch.float32, device=device)
    nbytes = rows * cols * bits_of(cfg.wfmt) // 8
    return (torch.empty((S, nbytes), dtype=torch.uint8, device=device),
            torch.empty((S, rows, cols // 32), dtype=torch.int16, device=device),
            torch.empty((S, rows, cols // 32), dtype=torch.int16, device=device))


def expert_pool(cfg, slot_layers, slot_experts, device="cuda"):
    """Device pools {gate, up, down} holding expert slot_experts[s] of layer
    slot_layers[s] in slot s."""
    import torch
    S = len(slot_experts)
    pools = {}
    for m in ("gate", "up", "down"):
        if cfg.wfmt == "f32":
            pools[m] = torch.from_numpy(
                gen_pool(cfg, list(zip(np.asarray(slot_layers).tolist(),
                                       np.asarray(slot_experts).tolist())), m)).to(device)
            continue
        p = _alloc_pool(cfg, S, m, device)
        sl = torch.as_tensor(np.asarray(slot_layers, np.int32), device=device)
        se = torch.as_tensor(np.asarray(slot_experts, np.int32), device=device)
        for s0 in range(0, S, 65535):
            s1 = min(S, s0 + 65535)
            fill_pool_device(cfg, m, sl[s0:s1], se[s0:s1], p[0][s0:s1], p[1][s0:s1],
                             p[2][s0:s1], torch.cuda.current_stream().cuda_stream)
        pools[m] = p
    return pools


def layer_inputs(cfg, layer, device="cuda", x=None, T=None):
    """Device tensors of one layer except the routed pool: x (bf16 bits as
    int16 [T][H]), router weights, bias, shared-expert pool."""
    import torch
    if x is None:
        x = gen_x(cfg, layer, T)
    W = gen_router(cfg, layer)
    out = {
        "x_host": np.asarray(x, np.uint16),
        "x": to_device_bf16(x, device),
        "router_w": (torch.from_numpy(W).to(device) if cfg.router_fmt == "f32"
                     else to_device_bf16(W, device)),
        "bias": None,
        "shared": None,
    }
    b = gen_bias(cfg, layer)
    if b is not None:
        out["bias"] = torch.from_numpy(b).to(device)
    if cfg.shared:
        out["shared"] = expert_pool(cfg, [layer], [SHARED_ID], device)
    return out


def routed_pools(cfg, layers, device="cuda"):
    """Routed pools for the given layers.  identity: {layer: pool of E
    slots}; tiered: one global pool under key None plus the slot tables.
    Returns (pools, slot_of [L][E] int32 numpy, num_slots)."""
    slot_of, sl, se, S = slot_layout(cfg)
    if cfg.slots == "identity":
        pools = {l: expert_pool(cfg, [l] * cfg.E, list(range(cfg.E)), device) for l in layers}
        return pools, None, S
    return {None: expert_pool(cfg, sl, se, device)}, slot_of, S
