"""The synthetic workloads of the paged-expert MoE layer.

Shapes follow the pages' model (48 MoE layers, 128 routed experts, top-8;
hidden 2048 and expert intermediate 768, which give the 4.72 MB block-FP8
and 2.43 MB int4 expert sizes the blog quotes).  Routing is synthetic
(Zipf popularity plus token-to-token persistence) and stands in for the
ShareGPT-driven router decisions the pages measured with.  The MXFP4 workload
takes the gpt-oss-20b expert shape instead (hidden = inter = 2880).
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    experts: int          # E
    top_k: int            # k
    resident: int         # K slots per layer
    hidden: int           # H
    inter: int            # I (expert SwiGLU intermediate)
    wtype: str            # "bf16" | "fp8" | "int4" | "int8" | "mxfp4"
    batch: int            # decode tokens per step (independent chains)
    steps: int            # decode steps
    routing: str          # "persist_uniform" | "persist_zipf" | "prefill_zipf"
    keep_p: float         # probability a routed id is kept from the previous token
    zipf_s: float         # Zipf exponent of the per-layer expert popularity
    prefill_tokens: int = 0

    @property
    def captured(self) -> bool:
        """Decode steps fit one device-planned wave: tokens x top_k <= K."""
        return self.batch * self.top_k <= self.resident


WORKLOADS = {
    # 1 layer, E=8, top-2, K=4, H=64, I=128; 32 decode steps at batch 1.
    "tiny_bf16": Workload("tiny_bf16", 1, 8, 2, 4, 64, 128, "bf16", 1, 32,
                          "persist_uniform", 0.5, 0.0),
    # 48 layers, E=128, top-8, K=40, bf16 experts, batch 1, 512 steps.
    "decode_bf16_k40_b1": Workload("decode_bf16_k40_b1", 48, 128, 8, 40, 2048, 768, "bf16", 1, 512,
                                   "persist_zipf", 0.7, 1.0),
    # Same shapes, 128x128 block-FP8 experts, K=40, batch 4 (32 entries, one captured wave).
    "decode_fp8_k40_b4": Workload("decode_fp8_k40_b4", 48, 128, 8, 40, 2048, 768, "fp8", 4, 512,
                                  "persist_zipf", 0.7, 1.0),
    # Same shapes, group-128 int4 experts, K=26, batch 4 (32 entries > K: host-planned).
    "decode_int4_k26_b4": Workload("decode_int4_k26_b4", 48, 128, 8, 26, 2048, 768, "int4", 4, 512,
                                   "persist_zipf", 0.7, 1.0),
    # Same shapes, GPTQ-style int8 experts (group-128 fp16 scales), K=40, batch 4 (one captured wave).
    "decode_int8_k40_b4": Workload("decode_int8_k40_b4", 48, 128, 8, 40, 2048, 768, "int8", 4, 512,
                                   "persist_zipf", 0.7, 1.0),
    # MXFP4 experts in the shape of the blog's gpt-oss-20b runs: 24 MoE layers, 32
    # experts, top-4, hidden and expert intermediate 2880; K=16, batch 1 (every
    # expert has one entry a step and takes the GEMV kernels).
    "decode_mxfp4_k16_b1": Workload("decode_mxfp4_k16_b1", 24, 32, 4, 16, 2880, 2880, "mxfp4", 1, 512,
                                    "persist_zipf", 0.7, 1.0),
    # bf16, K=92: a cold 2048-token prefill chunk (Zipf 0.8, 8 distinct ids per token),
    # then 256 decode steps at batch 1 continuing from the last prefill token.
    "prefill_bf16_k92": Workload("prefill_bf16_k92", 48, 128, 8, 92, 2048, 768, "bf16", 1, 256,
                                 "prefill_zipf", 0.7, 0.8, prefill_tokens=2048),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (e.g. fewer layers or steps)."""
    from dataclasses import replace
    return replace(WORKLOADS[name], **overrides)
