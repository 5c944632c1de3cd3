"""GPU parity at the workloads' full sizes (48 layers, E=128, top-8, H=2048,
I=768; MXFP4 at the gpt-oss-20b expert shape, 24 layers, E=32, top-4,
H=I=2880; every decode step of the window), launched as bench.py times them:
device-planned workloads as one replayed hipGraph per step, host-planned ones
eagerly (harness.DecodeRunner).

Per workload:
- the paged run's outputs equal, bit for bit, an unpaged run of the same
  kernels (K = E, every expert resident) over every step and layer;
- every step of every layer, read back from the plan log after the window:
  its waves' page-in plans (count, experts, slots, evicted), its slot map
  and the LRU state it left equal the oracle's LRU simulator, and the
  page-in / distinct counters over the window agree;
- sampled (step, layer) outputs are within the stated tolerance of the CPU
  oracle's fp32 unpaged layer (for the prefill chunk: 32 sampled tokens of
  the first and last layer, which the oracle computes token by token).
The concurrency sweep's host-planned multi-wave points (batch 8 at K = 24 in
FP8 and K = 26 in int4) are checked the same way over 128 steps.
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
TOL = {"bf16": 1e-2, "fp8": 1e-2, "int4": 2e-2, "int8": 1e-2, "mxfp4": 1e-2}


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


def _contexts(wl, max_tokens=None, log_steps=None):
    t0 = time.time()
    paged = harness.make_moe(wl, max_tokens=max_tokens, plan_log_steps=log_steps or wl.steps)
    unpaged = harness.make_moe(wl, flags=pe.PE_FLAG_UNPAGED, max_tokens=max_tokens)
    harness.load_store([paged, unpaged], wl)
    _say("%s: paged (K=%d) and unpaged contexts loaded in %.1fs" % (wl.name, wl.resident, time.time() - t0))
    return paged, unpaged


def _check_log(m, wl, steps_ids):
    """Every logged step of every layer against a fresh simulator run over the
    same id sequence (steps_ids(l) -> list of flat id arrays, in step order):
    plans of every wave, slot map, LRU state after the step.  Returns the
    simulator's page-in and distinct totals."""
    misses = distinct = 0
    for l in range(wl.layers):
        sim = LayerLRU(wl.experts, wl.resident)
        seq = steps_ids(l)
        recs = m.plan_log(l)
        assert len(recs) == len(seq), (l, len(recs), len(seq))
        for s, (ids, rec) in enumerate(zip(seq, recs)):
            waves = sim.step(ids)
            misses += sum(wv.count for wv in waves)
            distinct += len(set(int(e) for e in ids if 0 <= e < wl.experts))
            where = (l, s)
            assert rec["seq"] == s and rec["n_waves"] == len(waves), where
            for g, wv in zip(rec["waves"], waves):
                assert (g["count"], g["experts"].tolist(), g["slots"].tolist(), g["evicted"].tolist()) == \
                    (wv.count, wv.plan_experts, wv.plan_slots, wv.evicted), where
            want = [next((wv.slot_of[e] for wv in waves if e in wv.slot_of), -1) for e in (int(v) for v in ids)]
            assert rec["slot_of"][:len(ids)].tolist() == want, where
            assert (rec["slot_expert"].tolist(), rec["last_use"].tolist(), rec["tick"]) == \
                (sim.slot_expert, sim.last_use, sim.tick), where
    return misses, distinct


def _decode_window(m, wl, x, ids, w):
    """Every decode step of the window through harness.DecodeRunner (bench's
    launch configuration); returns all outputs [S, L, B, H] and the counter
    deltas."""
    S, L, B, H = wl.steps, wl.layers, wl.batch, wl.hidden
    out = torch.empty((L, B, H), dtype=torch.bfloat16, device=DEV)
    outs = torch.empty((S, L, B, H), dtype=torch.bfloat16, device=DEV)
    stream = torch.cuda.current_stream()
    runner = harness.DecodeRunner(m, wl, x, ids, w, out, stream)
    before = m.stats()
    for s in range(S):
        runner.run(1)
        outs[s].copy_(out)
    torch.cuda.synchronize()
    after = m.stats()
    return outs, {k: after[k] - before[k] for k in after}, runner.captured


def _first_diff(a, b):
    ne = (a.view(torch.int16) != b.view(torch.int16)).nonzero()
    return ne[0].tolist() if len(ne) else None


def _decode_case(wl, oracle_steps):
    name = wl.name
    r = synth.routing_for(wl)
    paged, unpaged = _contexts(wl)
    x, ids, w = harness.decode_inputs(wl, r, DEV)
    out_p, st, captured = _decode_window(paged, wl, x, ids, w)
    assert captured == wl.captured
    want_m, want_d = _check_log(paged, wl, lambda l: [r["decode_ids"][s, l].ravel() for s in range(wl.steps)])
    assert (st["page_ins"], st["distinct"]) == (want_m, want_d)
    assert st["host_planned" if not wl.captured else "device_planned"] == wl.steps * wl.layers
    _say("%s: paged window done (%d page-ins, %d waves); plans, slot maps and LRU state of all %d steps x %d "
         "layers match the simulator" % (name, st["page_ins"], st["waves"], wl.steps, wl.layers))
    out_u, _, _ = _decode_window(unpaged, wl, x, ids, w)
    assert torch.equal(out_p.view(torch.int16), out_u.view(torch.int16)), _first_diff(out_p, out_u)
    _say("%s: paged == unpaged bitwise over %d outputs" % (name, out_p.numel()))
    got = harness.bf16_bits(out_p[list(oracle_steps)])
    for i, s in enumerate(oracle_steps):
        xr = formats.bf16_to_f32(harness.bf16_bits(x[s]))
        for l in _sample_layers(wl.layers):
            ref = moe.moe_layer(xr, r["decode_ids"][s, l], r["decode_w"][s, l], _expert_fn(wl, l))
            _close(got[i, l], ref, wl.wtype, "%s step %d layer %d" % (name, s, l))
    _say("%s: %d sampled (step, layer) outputs within %g of the oracle" %
         (name, len(oracle_steps) * 3, TOL[wl.wtype]))
    paged.close()
    unpaged.close()
    return st


@pytest.mark.parametrize("name", ["decode_bf16_k40_b1", "decode_fp8_k40_b4", "decode_int4_k26_b4",
                                  "decode_int8_k40_b4", "decode_mxfp4_k16_b1"])
def test_fullsize_decode(name):
    wl = synth.WORKLOADS[name]
    _say("case %s: %d steps x %d layers, batch %d" % (name, wl.steps, wl.layers, wl.batch))
    _decode_case(wl, (0, wl.steps // 2, wl.steps - 1))


@pytest.mark.parametrize("name,K", [("decode_fp8_k40_b4", 24), ("decode_int4_k26_b4", 26)])
def test_fullsize_sweep_host_planned_multi_wave(name, K):
    """Batch 8 (64 entries > K): host-planned, often two waves, each paging in
    its own misses -- the sweep's points past K // top_k."""
    wl = synth.workload(name, resident=K, batch=8, steps=128)
    _say("case sweep %s K=%d batch 8: %d steps x %d layers" % (wl.wtype, K, wl.steps, wl.layers))
    st = _decode_case(wl, (0, wl.steps - 1))
    assert st["waves"] > wl.steps * wl.layers        # some steps took more than one wave


def test_fullsize_prefill_then_decode():
    wl = synth.WORKLOADS["prefill_bf16_k92"]
    T, L, H = wl.prefill_tokens, wl.layers, wl.hidden
    _say("case %s: %d-token chunk, then %d decode steps" % (wl.name, T, wl.steps))
    r = synth.routing_for(wl)
    paged, unpaged = _contexts(wl, max_tokens=T, log_steps=wl.steps + 1)
    xp_np = synth.hidden_states(wl, -1, T)
    xp = torch.from_numpy(xp_np.view(np.int16)).view(torch.bfloat16).to(DEV)
    idsp = torch.from_numpy(np.ascontiguousarray(r["prefill_ids"])).to(DEV)
    wp = torch.from_numpy(np.ascontiguousarray(r["prefill_w"])).to(DEV)
    x, ids, w = harness.decode_inputs(wl, r, DEV)
    outs = {}
    for tag, m in (("paged", paged), ("unpaged", unpaged)):
        outp = torch.empty((L, T, H), dtype=torch.bfloat16, device=DEV)
        for l in range(L):
            m.forward(l, xp, idsp[l], wp[l], outp[l])
        torch.cuda.synchronize()
        dec, st, captured = _decode_window(m, wl, x, ids, w)
        assert captured
        outs[tag] = (outp, dec)
        _say("%s run done" % tag)
    _check_log(paged, wl, lambda l: [r["prefill_ids"][l].ravel()] +
               [r["decode_ids"][s, l].ravel() for s in range(wl.steps)])
    _say("plans, slot maps and LRU state of the prefill chunk and all %d continuation steps match" % wl.steps)
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
