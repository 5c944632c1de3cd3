"""Pins for oracle/paged.py: the CPU paged layer equals the unpaged layer bitwise
for every K >= top_k, and a wrong plan or slot content is caught."""
import numpy as np
import pytest

import synth
from oracle import formats, moe
from oracle.paged import PagedLayerCPU


def _tiny_weights(wl, layer=0):
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = formats.dequant_expert(wl.wtype, *synth.expert_tensors(wl, layer, e))
        return cache[e]
    return get


def test_tiny_workload_paged_equals_unpaged_for_every_k():
    wl = synth.WORKLOADS["tiny_bf16"]
    r = synth.routing_for(wl)
    get = _tiny_weights(wl)
    xs = [formats.bf16_to_f32(synth.hidden_states(wl, s, 1)) for s in range(wl.steps)]
    ref = [moe.moe_layer(xs[s], r["decode_ids"][s, 0], r["decode_w"][s, 0], get) for s in range(wl.steps)]
    for K in range(wl.top_k, wl.experts + 1):
        layer = PagedLayerCPU(wl.experts, K, get)
        for s in range(wl.steps):
            out, waves = layer.forward(xs[s], r["decode_ids"][s, 0], r["decode_w"][s, 0])
            assert np.array_equal(out, ref[s]), (K, s)


@pytest.mark.parametrize("wtype", ["bf16", "fp8", "int4", "int8", "mxfp4"])
def test_multi_wave_prefill_like_paged_equals_unpaged(wtype):
    wl = synth.workload("prefill_bf16_k92", layers=1, experts=12, top_k=3, hidden=128, inter=128,
                        wtype=wtype, prefill_tokens=24, steps=4)
    r = synth.routing_for(wl)
    get = _tiny_weights(wl)
    x = formats.bf16_to_f32(synth.hidden_states(wl, 0, 24))
    ids, w = r["prefill_ids"][0], r["prefill_w"][0]
    ref = moe.moe_layer(x, ids, w, get)
    for K in (3, 4, 5, 7, 12):
        layer = PagedLayerCPU(wl.experts, K, get)
        out, waves = layer.forward(x, ids, w)
        assert len(waves) == -(-len(np.unique(ids)) // K)
        assert np.array_equal(out, ref)
        # decode continuation on the same table
        for s in range(wl.steps):
            xd = formats.bf16_to_f32(synth.hidden_states(wl, 100 + s, 1))
            od, _ = layer.forward(xd, r["decode_ids"][s, 0], r["decode_w"][s, 0])
            assert np.array_equal(od, moe.moe_layer(xd, r["decode_ids"][s, 0], r["decode_w"][s, 0], get))


def test_swapped_slot_contents_are_detected():
    """Plant a mistake in the CPU paged layer: two slots' contents swapped after a
    step.  The next step that uses them must not silently match the reference."""
    wl = synth.WORKLOADS["tiny_bf16"]
    get = _tiny_weights(wl)
    layer = PagedLayerCPU(wl.experts, 4, get)
    x = formats.bf16_to_f32(synth.hidden_states(wl, 0, 1))
    ids = np.array([[1, 2]], np.int32)
    w = np.array([[0.5, 0.5]], np.float32)
    layer.forward(x, ids, w)
    a, b = layer.lru.expert_slot[1], layer.lru.expert_slot[2]
    layer.slots[a], layer.slots[b] = layer.slots[b], layer.slots[a]
    with pytest.raises(AssertionError):
        layer.forward(x, ids, w)


def test_stale_slot_without_page_in_gives_wrong_output():
    """Plant a mistake: drop one page-in (the slot keeps its previous expert's
    weights, as with a tensor left unpaged).  The output must differ."""
    wl = synth.WORKLOADS["tiny_bf16"]
    get = _tiny_weights(wl)
    layer = PagedLayerCPU(wl.experts, 2, get)
    x = formats.bf16_to_f32(synth.hidden_states(wl, 0, 1))
    w = np.array([[0.5, 0.5]], np.float32)
    layer.forward(x, np.array([[0, 1]], np.int32), w)
    # next step routes to 2 and 3: both slots are overwritten; skip the copy of expert 3
    ids = np.array([[2, 3]], np.int32)
    waves = layer.lru.step(ids.ravel())
    for e, j in zip(waves[0].plan_experts, waves[0].plan_slots):
        if e != 3:
            layer.slots[j] = (e, get(e))
    stale = {e: layer.slots[waves[0].slot_of[e]][1] for e in (2, 3)}
    out = moe.moe_layer(x, ids, w, lambda e: stale[e])
    assert not np.array_equal(out, moe.moe_layer(x, ids, w, get))
