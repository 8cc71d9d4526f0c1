"""Synthetic workloads for the routed-experts decode step.

Each workload is named by what it is. Shapes follow the pages' decode step of
a 2/3-bit mixed-K routed-expert pack (lna-lab README, "What is in the pack":
43 routed layers, EXL3 2/3 bit mixed; LNA-CANON, "制式": TP8, 4 streams with
3 speculative tokens, i.e. 16 rows per step) and the NVFP4 MLP format of
"V100 換引擎", section 4.0.

This module holds sizes and recipe switches only; it computes nothing.
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    config_id: int          # seed namespace, see moe_synth.gen
    num_experts: int
    top_k: int
    hidden: int
    inter: int
    fmt: str                # "codebook" or "nvfp4"
    bits_mix: str           # "all2" | "alternate" | "mix62" | "pack" | "nvfp4"
    router: str             # "normal" | "zipf"
    token_counts: Tuple[int, ...]
    layers: int = 1
    zipf_s: float = 1.1
    shared_bits: int = 0    # > 0: an always-on shared expert with these codebook bits
    nv_scales: str = "exp6to8"  # NVFP4 block scales: "exp6to8" (0.5..3.75) or "all_finite"
    ts_scale: float = 0.004     # NVFP4 tensor scale = ts_scale * U(0.8, 1.2)

    @property
    def max_tokens(self) -> int:
        return max(self.token_counts)


# Layers of the "pack" mix whose routed experts are all 2-bit: the three
# replaced routed layers and the three MTP draft layers after the 43 routed ones.
PACK_ALL2_LAYERS = (3, 21, 41, 43, 44, 45)


WORKLOADS = {
    # 8 experts, top-2, hidden 256, expert intermediate 128, 2-bit codes.
    "tiny": Workload("tiny", 1, 8, 2, 256, 128, "codebook", "all2", "normal", (1,)),
    # One rank's share of an 8-way tensor-parallel layer: I = 2048 / 8.
    "rank_share": Workload("rank_share", 2, 256, 8, 4096, 256, "codebook", "alternate",
                           "normal", (1, 4)),
    # The unsharded layer with Zipf-skewed routing.
    "full_layer": Workload("full_layer", 3, 256, 8, 4096, 2048, "codebook", "mix62", "zipf",
                           (1, 2, 4, 8, 16, 24)),
    # 43 such layers back to back at the 16-row decode batch.
    "stack43": Workload("stack43", 4, 256, 8, 4096, 2048, "codebook", "mix62", "zipf",
                        (16,), layers=43),
    # The pack as shipped (lna-lab README, "What is in the pack"): the 43 routed
    # layers with layers 3, 21 and 41 all 2-bit, followed by the 3 MTP draft
    # MoE layers, all 2-bit (layers 43..45), same shapes, 16 rows per step.
    "pack46": Workload("pack46", 6, 256, 8, 4096, 2048, "codebook", "pack", "zipf",
                       (16,), layers=46),
    # The full layer plus its always-on shared expert, stored 6-bit like the
    # pack's dense linears (lna-lab README, "What is in the pack": attention
    # and shared experts in EXL3 6 bit); the shared expert has the routed
    # experts' shape.
    "shared_layer": Workload("shared_layer", 7, 256, 8, 4096, 2048, "codebook", "mix62", "zipf",
                             (1, 16, 24), shared_bits=6),
    # The 43-layer stack with the shared expert in every layer.
    "stack43_shared": Workload("stack43_shared", 8, 256, 8, 4096, 2048, "codebook", "mix62",
                               "zipf", (16,), layers=43, shared_bits=6),
    # Prefill / batched verify: the full layer at 64..512 tokens (one batch of
    # BT = 512 at most), four layers in one graph.
    "prefill": Workload("prefill", 9, 256, 8, 4096, 2048, "codebook", "mix62", "zipf",
                        (64, 128, 256, 512), layers=4),
    # NVFP4 experts (e2m1 values, e4m3 per-16 scales, fp32 tensor scale).
    "nvfp4": Workload("nvfp4", 5, 256, 8, 4096, 2048, "nvfp4", "nvfp4", "normal", (2, 8)),
}


def small_workload(name, num_experts, top_k, hidden, inter, fmt="codebook",
                   bits_mix="alternate", router="normal", config_id=100, shared_bits=0,
                   nv_scales="exp6to8", ts_scale=0.004):
    """A reduced shape for fast tests (same recipe, smaller sizes)."""
    return Workload(name, config_id, num_experts, top_k, hidden, inter, fmt, bits_mix,
                    router, (1,), shared_bits=shared_bits, nv_scales=nv_scales,
                    ts_scale=ts_scale)
