"""Byte arithmetic of paged experts.  TEST INFRASTRUCTURE (oracle).

Per-expert bytes of one SwiGLU expert (W13 [2I, H] and W2 [H, I]) in each
format, per-slot bytes over all MoE layers ("Choosing K" on the docs page:
one resident expert per layer costs per-expert bytes times the number of MoE
layers), and the blog's bandwidth arithmetic ("¿Por qué es rápido si los
expertos cruzan el PCIe en cada paso?"): a batch-1 token activates
layers x top_k experts, an all-miss token moves that many experts over the
link, and a measured token rate bounds the miss rate.
"""


def expert_bytes(wtype: str, hidden: int, inter: int) -> int:
    """Algorithmic bytes of one expert: weights plus scales, no padding."""
    n = 3 * hidden * inter                               # W13 has 2*I*H, W2 has H*I elements
    if wtype == "bf16":
        return 2 * n
    if wtype == "fp8":                                   # 1 B codes + fp32 per 128x128 block
        blocks = (2 * inter // 128) * (hidden // 128) + (hidden // 128) * (inter // 128)
        return n + 4 * blocks
    if wtype == "int4":                                  # 4-bit codes + fp16 per 128 inputs per row
        groups = 2 * inter * (hidden // 128) + hidden * (inter // 128)
        return n // 2 + 2 * groups
    if wtype == "int8":                                  # 8-bit codes + fp16 per 128 inputs per row
        groups = 2 * inter * (hidden // 128) + hidden * (inter // 128)
        return n + 2 * groups
    if wtype == "mxfp4":                                 # 4-bit codes + one E8M0 byte per 32 inputs per row
        blocks = 2 * inter * (hidden // 32) + hidden * (inter // 32)
        return n // 2 + blocks
    raise ValueError(wtype)


def slot_bytes(wtype: str, hidden: int, inter: int, moe_layers: int) -> int:
    """GPU memory of one resident slot in every MoE layer."""
    return expert_bytes(wtype, hidden, inter) * moe_layers


def suggest_k(budget_bytes: float, per_slot_bytes: float, num_experts: int) -> int:
    """The docs' sizing rule read as K = floor(budget / per-slot bytes), capped at E."""
    return int(min(num_experts, budget_bytes // per_slot_bytes))


def all_miss_bytes_per_token(per_expert: float, moe_layers: int, top_k: int) -> float:
    return per_expert * moe_layers * top_k


def link_rate_needed(all_miss_bytes: float, tokens_per_s: float) -> float:
    """Bytes/s to page every activation of a token in 1/tokens_per_s."""
    return all_miss_bytes * tokens_per_s


def max_miss_rate(tokens_per_s: float, link_bytes_per_s: float, all_miss_bytes: float) -> float:
    """Largest miss fraction a measured rate allows: time per token x link rate / all-miss bytes."""
    return link_bytes_per_s / tokens_per_s / all_miss_bytes


def uniform_miss_rate(num_resident: int, num_experts: int) -> float:
    """Miss rate of i.i.d. uniform routing with K of E resident: 1 - K/E."""
    return 1.0 - num_resident / num_experts
