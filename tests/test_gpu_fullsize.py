"""GPU parity at the workloads' full sizes (48 layers, E=128, top-8, H=2048,
I=768; MXFP4 at the gpt-oss-20b expert shape, 24 layers, E=32, top-4,
H=I=2880; every decode step of the window), launched as bench.py times them:
device-planned workloads as one replayed hipGraph per step, host-planned ones
eagerly (harness.DecodeRunner).

Per workload:
- the paged run's outputs equal, bit for bit, an unpaged run of the same
  kernels (K = E, every expert resident) over every step and layer;
- its plans (every layer at three sampled steps), final LRU state of every
  layer and page-in / distinct counts over the window equal the oracle's LRU
  simulator;
- sampled (step, layer) outputs are within the stated tolerance of the CPU
  oracle's fp32 unpaged layer (for the prefill chunk: 32 sampled tokens of
  the first and last layer, which the oracle computes token by token).
"""
import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
import harness
import host_paged_expert_amd as pe
from oracle import formats, moe
from oracle.lru import LayerLRU

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"bf16": 1e-2, "fp8": 1e-2, "int4": 2e-2, "int8": 1e-2, "mxfp4": 2e-2}


def _sample_layers(L):
    return (0, L // 2, L - 1)


def _say(msg):
    print("[fullsize] " + msg, flush=True)


def _expert_fn(wl, layer):
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = formats.dequant_expert(wl.wtype, *synth.expert_tensors(wl, layer, e))
        return cache[e]
    return get


def _close(got_bits, ref, wtype, what):
    got = harness.bf16_to_f32(got_bits)
    err, scale = float(np.abs(got - ref).max()), float(np.abs(ref).max())
    assert err <= TOL[wtype] * scale, "%s: max|d|=%g max|ref|=%g" % (what, err, scale)


def _contexts(wl, max_tokens=None):
    t0 = time.time()
    paged = harness.make_moe(wl, max_tokens=max_tokens)
    unpaged = harness.make_moe(wl, flags=pe.PE_FLAG_UNPAGED, max_tokens=max_tokens)
    harness.load_store([paged, unpaged], wl)
    _say("%s: paged (K=%d) and unpaged contexts loaded in %.1fs" % (wl.name, wl.resident, time.time() - t0))
    return paged, unpaged


def _check_plans(m, layer, waves):
    for wi, wv in enumerate(waves):
        p = m.plan(layer, wi)
        got = (p["count"], p["experts"].tolist(), p["slots"].tolist(), p["evicted"].tolist())
        assert got == (wv.count, wv.plan_experts, wv.plan_slots, wv.evicted), (layer, wi)
        assert p["n_waves"] == len(waves)


def _check_state(m, layer, sim):
    se, lu, tick = m.lru_state(layer)
    assert (se.tolist(), lu.tolist(), tick) == (sim.slot_expert, sim.last_use, sim.tick), layer


def _decode_window(m, wl, r, sims, x, ids, w, check_steps):
    """Every decode step of the window through harness.DecodeRunner (bench's
    launch configuration); returns all outputs [S, L, B, H] and the counter
    deltas.  With `sims`, plans are checked at `check_steps`."""
    S, L, B, H = wl.steps, wl.layers, wl.batch, wl.hidden
    out = torch.empty((L, B, H), dtype=torch.bfloat16, device=DEV)
    outs = torch.empty((S, L, B, H), dtype=torch.bfloat16, device=DEV)
    stream = torch.cuda.current_stream()
    runner = harness.DecodeRunner(m, wl, x, ids, w, out, stream)
    before = m.stats()
    for s in range(S):
        runner.run(1)
        outs[s].copy_(out)
        if sims is not None:
            for l in range(L):
                waves = sims[l].step(r["decode_ids"][s, l].ravel())
                if s in check_steps:
                    _check_plans(m, l, waves)
    torch.cuda.synchronize()
    after = m.stats()
    return outs, {k: after[k] - before[k] for k in after}, runner.captured


def _first_diff(a, b):
    ne = (a.view(torch.int16) != b.view(torch.int16)).nonzero()
    return ne[0].tolist() if len(ne) else None


@pytest.mark.parametrize("name", ["decode_bf16_k40_b1", "decode_fp8_k40_b4", "decode_int4_k26_b4",
                                  "decode_mxfp4_k16_b1"])
def test_fullsize_decode(name):
    wl = synth.WORKLOADS[name]
    _say("case %s: %d steps x %d layers, batch %d" % (name, wl.steps, wl.layers, wl.batch))
    r = synth.routing_for(wl)
    paged, unpaged = _contexts(wl)
    x, ids, w = harness.decode_inputs(wl, r, DEV)
    sims = [LayerLRU(wl.experts, wl.resident) for _ in range(wl.layers)]
    check_steps = {0, wl.steps // 2, wl.steps - 1}
    out_p, st, captured = _decode_window(paged, wl, r, sims, x, ids, w, check_steps)
    assert captured == wl.captured
    for l in range(wl.layers):
        _check_state(paged, l, sims[l])
    _say("%s: paged window done (%d page-ins); plans and LRU state match the simulator" % (name, st["page_ins"]))
    out_u, _, _ = _decode_window(unpaged, wl, r, None, x, ids, w, ())
    assert torch.equal(out_p.view(torch.int16), out_u.view(torch.int16)), _first_diff(out_p, out_u)
    _say("%s: paged == unpaged bitwise over %d outputs" % (name, out_p.numel()))
    # counters over the window against a fresh simulator pass
    check = [LayerLRU(wl.experts, wl.resident) for _ in range(wl.layers)]
    want_m = want_d = 0
    for s in range(wl.steps):
        for l in range(wl.layers):
            e = r["decode_ids"][s, l].ravel()
            want_m += sum(wv.count for wv in check[l].step(e))
            want_d += len(set(e.tolist()))
    assert (st["page_ins"], st["distinct"]) == (want_m, want_d)
    # oracle on sampled (step, layer) pairs
    got = harness.bf16_bits(out_p[sorted(check_steps)])
    for i, s in enumerate(sorted(check_steps)):
        xr = formats.bf16_to_f32(harness.bf16_bits(x[s]))
        for l in _sample_layers(wl.layers):
            ref = moe.moe_layer(xr, r["decode_ids"][s, l], r["decode_w"][s, l], _expert_fn(wl, l))
            _close(got[i, l], ref, wl.wtype, "%s step %d layer %d" % (name, s, l))
    _say("%s: %d sampled (step, layer) outputs within %g of the oracle" %
         (name, len(check_steps) * 3, TOL[wl.wtype]))
    paged.close()
    unpaged.close()


def test_fullsize_prefill_then_decode():
    wl = synth.WORKLOADS["prefill_bf16_k92"]
    T, L, H = wl.prefill_tokens, wl.layers, wl.hidden
    _say("case %s: %d-token chunk, then %d decode steps" % (wl.name, T, wl.steps))
    r = synth.routing_for(wl)
    paged, unpaged = _contexts(wl, max_tokens=T)
    xp_np = synth.hidden_states(wl, -1, T)
    xp = torch.from_numpy(xp_np.view(np.int16)).view(torch.bfloat16).to(DEV)
    idsp = torch.from_numpy(np.ascontiguousarray(r["prefill_ids"])).to(DEV)
    wp = torch.from_numpy(np.ascontiguousarray(r["prefill_w"])).to(DEV)
    x, ids, w = harness.decode_inputs(wl, r, DEV)
    sims = [LayerLRU(wl.experts, wl.resident) for _ in range(L)]
    outs = {}
    for tag, m in (("paged", paged), ("unpaged", unpaged)):
        outp = torch.empty((L, T, H), dtype=torch.bfloat16, device=DEV)
        for l in range(L):
            m.forward(l, xp, idsp[l], wp[l], outp[l])
            if m is paged:
                waves = sims[l].step(r["prefill_ids"][l].ravel())
                _check_plans(m, l, waves)
                _check_state(m, l, sims[l])
        torch.cuda.synchronize()
        dec, st, captured = _decode_window(m, wl, r, sims if m is paged else None, x, ids, w,
                                           {0, wl.steps // 2, wl.steps - 1})
        assert captured
        outs[tag] = (outp, dec)
        _say("%s run done" % tag)
    for l in range(L):
        _check_state(paged, l, sims[l])
    pp, pd = outs["paged"]
    up, ud = outs["unpaged"]
    assert torch.equal(pp.view(torch.int16), up.view(torch.int16)), _first_diff(pp, up)
    assert torch.equal(pd.view(torch.int16), ud.view(torch.int16)), _first_diff(pd, ud)
    _say("paged == unpaged bitwise: prefill and continuation")
    rows = np.random.default_rng(7).choice(T, 32, replace=False)
    rows.sort()
    xr = formats.bf16_to_f32(xp_np[rows])
    for l in (0, L - 1):
        ref = moe.moe_layer(xr, r["prefill_ids"][l][rows], r["prefill_w"][l][rows], _expert_fn(wl, l))
        _close(harness.bf16_bits(pp[l])[rows], ref, wl.wtype, "prefill layer %d" % l)
    for s in (0, wl.steps - 1):
        xd = formats.bf16_to_f32(harness.bf16_bits(x[s]))
        for l in _sample_layers(L):
            ref = moe.moe_layer(xd, r["decode_ids"][s, l], r["decode_w"][s, l], _expert_fn(wl, l))
            _close(harness.bf16_bits(pd[s, l]), ref, wl.wtype, "continuation step %d layer %d" % (s, l))
    _say("sampled prefill tokens and continuation outputs within %g of the oracle" % TOL[wl.wtype])
    paged.close()
    unpaged.close()
