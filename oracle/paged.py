"""A CPU paged MoE layer built on the LRU simulator.  TEST INFRASTRUCTURE (oracle).

Steps 3-4 of "A step: waves, page-in, merge" (SGLang Paged Experts docs):
a wave computes, for each routed entry whose expert it holds, the expert's
output scaled by the entry's router weight and stores it in its row of one
merged buffer; once every wave has run, one top-k sum over the merged rows
gives the layer output.  Every entry is stored exactly once, by the wave of
its expert, so the wave split has no way to change the result.  Slot
contents are modelled explicitly (a slot holds whatever expert was last
copied into it), so a wrong plan shows up as wrong output.
"""
import numpy as np

from .lru import LayerLRU
from .moe import moe_entries, topk_sum


class PagedLayerCPU:
    def __init__(self, num_experts: int, num_resident: int, expert_weights):
        self.lru = LayerLRU(num_experts, num_resident)
        self.host = expert_weights                 # host store: expert -> weights
        self.slots = [None] * num_resident         # GPU slot table contents

    def forward(self, x, ids, w, dtype=np.float32):
        ids = np.asarray(ids)
        T, k = ids.shape
        merged = np.zeros((T, k, x.shape[1]), dtype)
        waves = self.lru.step(ids.ravel())
        for wv in waves:
            for e, j in zip(wv.plan_experts, wv.plan_slots):      # page-in
                self.slots[j] = (e, self.host(e))
            held = set(wv.experts)

            def from_slot(e, wv=wv):
                se, wts = self.slots[wv.slot_of[e]]
                assert se == e, "slot %d holds expert %d, wave wants %d" % (wv.slot_of[e], se, e)
                return wts
            part, written = moe_entries(x, ids, w, from_slot, dtype, select=lambda e: e in held,
                                        num_experts=self.lru.E)
            merged[written] = part[written]
        return topk_sum(merged), waves
