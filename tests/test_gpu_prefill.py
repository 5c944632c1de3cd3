"""GPU parity of prefill-sized steps: host-planned multi-wave steps whose
experts with >= 16 entries run on the MFMA grouped-GEMM kernels (the others on
the GEMV kernels), against the CPU oracle, the LRU simulator and an unpaged
run; then a decode continuation on the same slot tables."""
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


def _expert_fn(wl, layer):
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = formats.dequant_expert(wl.wtype, *synth.expert_tensors(wl, layer, e))
        return cache[e]
    return get


def _close(got_bits, ref, wtype, what):
    got = harness.bf16_to_f32(got_bits)
    err, scale = np.abs(got - ref).max(), np.abs(ref).max()
    assert err <= TOL[wtype] * scale, "%s: max|d|=%g max|ref|=%g" % (what, err, scale)


def _prefill_run(wl, flags=0, check=True):
    r = synth.routing_for(wl)
    T = wl.prefill_tokens
    m = harness.make_moe(wl, flags=flags, max_tokens=T)
    harness.load_store(m, wl)
    x_np = synth.hidden_states(wl, 0, T)
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(DEV)
    ids = torch.from_numpy(np.ascontiguousarray(r["prefill_ids"])).to(DEV)
    w = torch.from_numpy(np.ascontiguousarray(r["prefill_w"])).to(DEV)
    out = torch.empty((wl.layers, T, wl.hidden), dtype=torch.bfloat16, device=DEV)
    sims = [LayerLRU(wl.experts, m.K) for _ in range(wl.layers)]
    for l in range(wl.layers):
        m.forward(l, x, ids[l], w[l], out[l])
        if check and not flags & pe.PE_FLAG_UNPAGED:
            waves = sims[l].step(r["prefill_ids"][l].ravel())
            for wi, wv in enumerate(waves):
                p = m.plan(l, wi)
                assert (p["count"], p["experts"].tolist(), p["slots"].tolist(), p["evicted"].tolist()) == \
                    (wv.count, wv.plan_experts, wv.plan_slots, wv.evicted), (l, wi)
                assert p["n_waves"] == len(waves)
            se, lu, tick = m.lru_state(l)
            assert se.tolist() == sims[l].slot_expert and lu.tolist() == sims[l].last_use and tick == sims[l].tick
        if check:
            xr = formats.bf16_to_f32(x_np)
            ref = moe.moe_layer(xr, r["prefill_ids"][l], r["prefill_w"][l], _expert_fn(wl, l))
            _close(harness.bf16_bits(out[l]), ref, wl.wtype, "prefill layer %d" % l)
    # decode continuation from the prefill's slot tables
    steps = wl.steps
    xd, idsd, wd = harness.decode_inputs(wl, r, DEV, steps)
    outd = torch.empty((steps, wl.layers, wl.batch, wl.hidden), dtype=torch.bfloat16, device=DEV)
    for s in range(steps):
        for l in range(wl.layers):
            m.forward(l, xd[s], idsd[s, l], wd[s, l], outd[s, l])
            if check and not flags & pe.PE_FLAG_UNPAGED:
                waves = sims[l].step(r["decode_ids"][s, l].ravel())
                p = m.plan(l, 0)
                assert (p["experts"].tolist(), p["slots"].tolist()) == (waves[0].plan_experts, waves[0].plan_slots)
            if check:
                ref = moe.moe_layer(formats.bf16_to_f32(harness.bf16_bits(xd[s])), r["decode_ids"][s, l],
                                    r["decode_w"][s, l], _expert_fn(wl, l))
                _close(harness.bf16_bits(outd[s, l]), ref, wl.wtype, "decode %d layer %d" % (s, l))
    torch.cuda.synchronize()
    res = harness.bf16_bits(out), harness.bf16_bits(outd)
    st = m.stats()
    m.close()
    return res, st


@pytest.mark.parametrize("wtype", ["bf16", "fp8", "int4", "int8", "mxfp4"])
def test_prefill_multi_wave_mfma_vs_oracle_and_unpaged(wtype):
    wl = synth.workload("prefill_bf16_k92", layers=2, experts=16, top_k=4, resident=6, hidden=256, inter=384,
                        wtype=wtype, prefill_tokens=100, steps=4)
    print("case prefill %s" % wtype, flush=True)
    r = synth.routing_for(wl)
    counts = np.bincount(r["prefill_ids"][0].ravel(), minlength=16)
    assert counts.max() >= 16 and counts.min() < 16          # both expert kernels are exercised
    (p_out, d_out), st = _prefill_run(wl)
    assert st["host_planned"] == wl.layers and st["waves"] >= 3 * wl.layers
    (u_out, ud_out), _ = _prefill_run(wl, flags=pe.PE_FLAG_UNPAGED, check=False)
    assert np.array_equal(p_out, u_out)
    assert np.array_equal(d_out, ud_out)


def test_prefill_dma_page_in_matches_kernel_bitwise():
    wl = synth.workload("prefill_bf16_k92", layers=1, experts=16, top_k=4, resident=7, hidden=256, inter=256,
                        wtype="fp8", prefill_tokens=80, steps=2)
    a, sa = _prefill_run(wl, check=False)
    b, sb = _prefill_run(wl, flags=pe.PE_FLAG_PAGEIN_DMA, check=False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert sa["page_ins"] == sb["page_ins"]


@pytest.mark.parametrize("wtype", ["bf16", "int4"])
def test_device_planned_step_with_a_many_token_expert(wtype):
    """T*k <= K with one expert holding 20 entries: the device planner must build
    MFMA tiles and the captured path must run them."""
    E, k, K, H, I, T = 32, 1, 32, 256, 256, 24
    wl = synth.workload("decode_bf16_k40_b1", layers=1, experts=E, top_k=k, resident=K, hidden=H, inter=I,
                        wtype=wtype, batch=T, steps=1)
    m = harness.make_moe(wl, max_tokens=T)
    harness.load_store(m, wl)
    ids_np = np.array([[3]] * 20 + [[5], [7], [3], [30]], np.int32)
    w_np = np.linspace(0.2, 1.0, T, dtype=np.float32).reshape(T, 1)
    x_np = synth.hidden_states(wl, 0, T)
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    m.forward(0, x, torch.from_numpy(ids_np).to(DEV), torch.from_numpy(w_np).to(DEV), out)
    torch.cuda.synchronize()
    assert m.stats()["device_planned"] == 1
    ref = moe.moe_layer(formats.bf16_to_f32(x_np), ids_np, w_np, _expert_fn(wl, 0))
    _close(harness.bf16_bits(out), ref, wtype, "device-planned MFMA")
    got_dev = harness.bf16_bits(out)
    m.close()
    # the host-planned path computes the same tiles: identical bits
    m = harness.make_moe(wl, flags=pe.PE_FLAG_FORCE_HOST_PLAN, max_tokens=T)
    harness.load_store(m, wl)
    m.forward(0, x, torch.from_numpy(ids_np).to(DEV), torch.from_numpy(w_np).to(DEV), out)
    torch.cuda.synchronize()
    assert np.array_equal(harness.bf16_bits(out), got_dev)
    m.close()


@pytest.mark.parametrize("wtype,H,I", [("bf16", 320, 192), ("mxfp4", 320, 448)])
def test_prefill_mfma_at_multiples_of_64(wtype, H, I):
    """bf16 and MXFP4 take the 32x32 MFMA kernels whenever H and I are multiples
    of 64: K is staged 64 wide, and the last block of weight rows lies partly
    outside the matrix (gate/up blocks of 128 rows: I = 192 is 128 + 64; down
    blocks of 256 rows: H = 320 is 256 + 64)."""
    wl = synth.workload("prefill_bf16_k92", layers=2, experts=16, top_k=4, resident=6, hidden=H, inter=I,
                        wtype=wtype, prefill_tokens=100, steps=3)
    print("case prefill %s H=%d I=%d" % (wtype, H, I), flush=True)
    r = synth.routing_for(wl)
    counts = np.bincount(r["prefill_ids"][0].ravel(), minlength=16)
    assert counts.max() >= 16
    (p_out, d_out), st = _prefill_run(wl)
    (u_out, ud_out), _ = _prefill_run(wl, flags=pe.PE_FLAG_UNPAGED, check=False)
    assert np.array_equal(p_out, u_out) and np.array_equal(d_out, ud_out)


def test_prefill_mxfp4_gpt_oss_expert_shape():
    """MXFP4 at gpt-oss-20b's expert shape (H = I = 2880, 32 experts, top-4): a
    256-token chunk, host-planned in waves of K = 16, whose experts (about 32
    entries each) take the MFMA kernels (2880 = 45 K blocks of 64; weight-row
    blocks end partly outside the matrix), then decode steps; against the
    oracle, the simulator and an unpaged run."""
    wl = synth.workload("prefill_bf16_k92", layers=1, experts=32, top_k=4, resident=16, hidden=2880, inter=2880,
                        wtype="mxfp4", prefill_tokens=256, steps=2)
    print("case prefill mxfp4 2880", flush=True)
    r = synth.routing_for(wl)
    assert np.bincount(r["prefill_ids"][0].ravel(), minlength=32).max() >= 16
    (p_out, d_out), st = _prefill_run(wl)
    assert st["waves"] >= 2 + wl.steps
    (u_out, ud_out), _ = _prefill_run(wl, flags=pe.PE_FLAG_UNPAGED, check=False)
    assert np.array_equal(p_out, u_out) and np.array_equal(d_out, ud_out)


@pytest.mark.parametrize("wtype", ["bf16", "int4"])
def test_mfma_tile_boundaries(wtype):
    """Experts whose entry counts sit on the MFMA thresholds and tile edges
    (15 and 16 entries, 127..129, 255..257, a full 300) in one host-planned step
    of 300 tokens, over two waves (K below the distinct count): against the
    oracle row by row, and bit-identical to an unpaged run."""
    E, k, T, K = 24, 8, 300, 10
    wl = synth.workload("decode_bf16_k40_b1", wtype=wtype, layers=1, experts=E, top_k=k, resident=K,
                        hidden=256, inter=256, batch=1, steps=1)
    counts = {0: 300, 1: 257, 2: 256, 3: 255, 4: 129, 5: 128, 6: 127, 7: 16, 8: 15}
    rng = np.random.default_rng(7)
    ids = np.full((T, k), -1, np.int32)
    fill = np.zeros(T, np.int32)
    for e, c in counts.items():             # expert e in tokens 0..c-1 (rotated so the tails differ)
        rows = (np.arange(c) + 53 * e) % T
        for t in rows:
            ids[t, fill[t]] = e
            fill[t] += 1
    assert fill.max() <= k
    for t in range(T):                      # the remaining positions from the other experts, no repeats
        rest = [e for e in rng.permutation(np.arange(9, E)) if e not in ids[t]]
        for j in range(fill[t], k):
            ids[t, j] = rest[j - fill[t]]
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(1, keepdims=True)
    cnt = np.bincount(ids.ravel(), minlength=E)
    for e, c in counts.items():
        assert cnt[e] == c, (e, cnt[e], c)
    x_np = synth.hidden_states(wl, 0, T)
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(DEV)
    outs = {}
    for flags in (0, pe.PE_FLAG_UNPAGED):
        print("case tile boundaries %s flags %d" % (wtype, flags), flush=True)
        m = harness.make_moe(wl, flags=flags, max_tokens=T)
        harness.load_store(m, wl)
        out = torch.empty((T, wl.hidden), dtype=torch.bfloat16, device=DEV)
        m.forward(0, x, torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), out)
        torch.cuda.synchronize()
        outs[flags] = harness.bf16_bits(out)
        if not flags:
            waves = LayerLRU(E, K).step(ids.ravel())
            assert len(waves) > 1 and m.plan(0, 0)["n_waves"] == len(waves)
        m.close()
    assert np.array_equal(outs[0], outs[pe.PE_FLAG_UNPAGED])
    ref = moe.moe_layer(formats.bf16_to_f32(x_np), ids, w, _expert_fn(wl, 0))
    _close(outs[0], ref, wtype, "tile boundaries")
