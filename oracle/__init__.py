"""CPU oracle for the paged-expert MoE layer.  TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy code that states what the paged layer
must compute.  It shares no code with the GPU library (`host_paged_expert_amd`)
and neither imports the other; both take their inputs from `synth`.  Only
`tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of `bench.py`
may import it.

Contents (citations are to the SGLang "Paged Experts" documentation page,
docs.sglang.io/docs/advanced_features/paged_experts, and the DonWeb blog post
"SGLang Paged Experts: corré MoE más grandes que tu VRAM"):

- formats: decoding of bf16, OCP e4m3fn block-FP8, group-128 int4 and int8,
  and OCP MXFP4 expert weights into fp32.
- moe: the unpaged MoE layer — the docs page ("Why Paged Experts?", and step 4
  of "A step: waves, page-in, merge") says the paged layer returns exactly
  this.
- lru: the per-layer LRU / wave simulator of steps 1-2 of "A step: waves,
  page-in, merge", with the tie-breaks the page leaves open.
- paged: a CPU paged layer (waves, merge buffer, fixed-order top-k sum, steps
  3-4) built on the simulator, used to check that the result does not depend
  on the wave split.
- sizes: per-expert / per-slot / per-token byte arithmetic ("Choosing K" on
  the docs page; the blog's "¿Por qué es rápido...?" section).

Every function here is pinned by `tests/` against something other than
itself (brute force, closed forms, special cases, the pages' printed values).
"""
