"""The five synthetic workloads of the routed-MoE layer, as plain data.

Shapes follow the model the Strata pages describe: 48 layers of 512 experts
with 10 chosen per token ("Why Strata is fast on low-VRAM GPUs", section on
the problem), a 4-token verify batch of 1 token + 3 drafts (same page,
"predict, then verify"), a resident-expert slot table of 4,176 experts with
57-109 per layer (same page, placement figure) and prefill of long prompts
(same page, "reading long prompts").  Hidden 2048 / intermediate 768 are the
assumed expert dimensions (the pages only give totals).

Nothing here computes any part of the MoE layer.
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class MoEConfig:
    name: str
    E: int              # experts per layer
    k: int              # experts chosen per token
    H: int              # hidden size
    I: int              # expert intermediate size
    T: int              # tokens per step
    layers: int         # layers in the stack
    wfmt: str           # expert weight format: "f32" | "q2" | "q4"
    router_fmt: str     # "f32" | "bf16"
    shared: bool        # one shared expert of the same shape
    bias: str           # "none" | "zipf" (per-expert popularity bias)
    slots: str          # "identity" (all resident) | "tiered" (resident pool)
    seed: int
    resident_total: int = 0          # tiered: experts resident over all layers
    resident_range: tuple = (0, 0)   # tiered: min/max resident per layer
    note: str = ""


# Popularity bias b_e = -ZIPF_ALPHA * ZIPF_S * ln(rank_e + ZIPF_R0); alpha was
# calibrated once by Monte Carlo so the top 16 % of experts take ~75 % of the
# top-10 selections (the pages: 15-18 % of experts serve 70-78 % of lookups).
ZIPF_S = 1.1
ZIPF_R0 = 80.0
ZIPF_ALPHA = 1.07

CONFIGS = {
    "c1": MoEConfig(
        name="c1_tiny_f32", E=16, k=2, H=64, I=32, T=4, layers=1,
        wfmt="f32", router_fmt="f32", shared=False, bias="none",
        slots="identity", seed=0x5EED0000,
        note="tiny single layer, fp32 weights, no shared expert"),
    "c2": MoEConfig(
        name="c2_decode_layer_q2", E=512, k=10, H=2048, I=768, T=1, layers=1,
        wfmt="q2", router_fmt="bf16", shared=True, bias="none",
        slots="identity", seed=0x5EED0001,
        note="one decode layer, 2-bit experts + shared expert, 1 token"),
    "c3": MoEConfig(
        name="c3_verify_stack_q2", E=512, k=10, H=2048, I=768, T=4, layers=48,
        wfmt="q2", router_fmt="bf16", shared=True, bias="zipf",
        slots="identity", seed=0x5EED0002,
        note="48-layer stack, 4-token verify batch, all 24,576 experts resident"),
    "c4": MoEConfig(
        name="c4_slot_tiering_q2", E=512, k=10, H=2048, I=768, T=16, layers=48,
        wfmt="q2", router_fmt="bf16", shared=True, bias="zipf",
        slots="tiered", seed=0x5EED0003, resident_total=4176,
        resident_range=(57, 109),
        note="48-layer stack, 16 tokens, 4,176 resident experts, miss list"),
    "c5": MoEConfig(
        name="c5_prefill_q4", E=512, k=10, H=2048, I=768, T=32768, layers=1,
        wfmt="q4", router_fmt="bf16", shared=True, bias="zipf",
        slots="identity", seed=0x5EED0004,
        note="prefill of 32,768 tokens, 4-bit experts, grouped GEMM"),
}


def bits_of(wfmt):
    return {"q2": 2, "q4": 4}.get(wfmt, 0)


def matrix_bytes(wfmt, rows, cols):
    """Bytes one [rows][cols] expert matrix occupies in HBM (all planes)."""
    if wfmt == "f32":
        return rows * cols * 4
    if wfmt == "bf16":
        return rows * cols * 2
    b = bits_of(wfmt)
    return rows * cols * b // 8 + 2 * (rows * cols // 32) * 2


def expert_bytes(cfg):
    return (2 * matrix_bytes(cfg.wfmt, cfg.I, cfg.H)
            + matrix_bytes(cfg.wfmt, cfg.H, cfg.I))
