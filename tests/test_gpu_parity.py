"""GPU parity of libpe against the CPU oracle (MI355X only).

- Plans, LRU state and slot maps are bit-exact against the oracle's simulator.
- Outputs are within max|gpu - ref| <= 1e-2 * max|ref| (bf16, FP8, int8, MXFP4) or
  2e-2 (int4) of the oracle's fp32 unpaged layer.
- Paged output is bit-identical to an unpaged run of the same kernels
  (PE_FLAG_UNPAGED: K = E, every expert resident), for every K.
"""
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


def _check_close(got_bits, ref, wtype, what=""):
    got = harness.bf16_to_f32(got_bits)
    err = np.abs(got - ref).max()
    scale = np.abs(ref).max()
    assert err <= TOL[wtype] * scale, "%s: max|d|=%g, max|ref|=%g" % (what, err, scale)


def _check_plan(moe_obj, layer, waves, T, k, ids_flat):
    st = torch.cuda.current_stream()
    nw = None
    for w, wv in enumerate(waves):
        p = moe_obj.plan(layer, w, st)
        nw = p["n_waves"]
        assert p["count"] == wv.count, (w, p, wv)
        assert p["experts"].tolist() == wv.plan_experts
        assert p["slots"].tolist() == wv.plan_slots
        assert p["evicted"].tolist() == wv.evicted
    if waves:
        assert nw == len(waves)
    sm = moe_obj.slot_map(layer, T, st)
    want = []
    for e in ids_flat:
        e = int(e)
        s = -1
        for wv in waves:
            if e in wv.slot_of:
                s = wv.slot_of[e]
        want.append(s)
    assert sm.tolist() == want


def _check_state(moe_obj, layer, sim):
    se, lu, tick = moe_obj.lru_state(layer, torch.cuda.current_stream())
    assert se.tolist() == sim.slot_expert
    assert lu.tolist() == sim.last_use
    assert tick == sim.tick


def _run_decode(wl, flags=0, steps=None, check_oracle=True, sims=None, collect=True):
    """Run the workload's decode steps eagerly; check plans/state every step."""
    steps = wl.steps if steps is None else steps
    r = synth.routing_for(wl)
    m = harness.make_moe(wl, flags=flags)
    harness.load_store(m, wl)
    x, ids, w = harness.decode_inputs(wl, r, DEV, steps)
    B, H, k = wl.batch, wl.hidden, wl.top_k
    out = torch.empty((steps, wl.layers, B, H), dtype=torch.bfloat16, device=DEV)
    unpaged = bool(flags & pe.PE_FLAG_UNPAGED)
    sims = sims if sims is not None else [LayerLRU(wl.experts, m.K) for _ in range(wl.layers)]
    fns = [_expert_fn(wl, l) for l in range(wl.layers)]
    for s in range(steps):
        for l in range(wl.layers):
            m.forward(l, x[s], ids[s, l], w[s, l], out[s, l])
            if not unpaged:
                waves = sims[l].step(r["decode_ids"][s, l].ravel())
                _check_plan(m, l, waves, B, k, r["decode_ids"][s, l].ravel())
                _check_state(m, l, sims[l])
            if check_oracle:
                xr = formats.bf16_to_f32(harness.bf16_bits(x[s]))
                ref = moe.moe_layer(xr, r["decode_ids"][s, l], r["decode_w"][s, l], fns[l])
                _check_close(harness.bf16_bits(out[s, l]), ref, wl.wtype, "step %d layer %d" % (s, l))
    torch.cuda.synchronize()
    res = harness.bf16_bits(out) if collect else None
    stats = m.stats()
    m.close()
    return res, stats


def test_tiny_workload_vs_oracle_and_simulator():
    wl = synth.WORKLOADS["tiny_bf16"]
    print("case tiny_bf16 K=%d" % wl.resident, flush=True)
    out, st = _run_decode(wl)
    assert st["steps"] == wl.steps and st["device_planned"] == wl.steps and st["bad_ids"] == 0


def test_tiny_paged_bit_identical_to_unpaged_for_every_k():
    base = synth.WORKLOADS["tiny_bf16"]
    ref, _ = _run_decode(base, flags=pe.PE_FLAG_UNPAGED, check_oracle=False)
    for K in range(base.top_k, base.experts + 1):
        print("case tiny_bf16 K=%d vs unpaged" % K, flush=True)
        wl = synth.workload("tiny_bf16", resident=K)
        got, _ = _run_decode(wl, check_oracle=False)
        assert np.array_equal(got, ref), K


SMALL = dict(layers=2, experts=16, top_k=4, hidden=256, inter=256, steps=10)


@pytest.mark.parametrize("wtype", ["bf16", "fp8", "int4", "int8", "mxfp4"])
@pytest.mark.parametrize("batch,K", [(1, 6), (3, 6), (2, 8)])
def test_small_formats_paged_vs_oracle_and_unpaged(wtype, batch, K):
    """Device-planned (batch*k <= K) and host-planned multi-wave (batch*k > K)
    steps, three formats, against the oracle and an unpaged run."""
    wl = synth.workload("decode_bf16_k40_b1", wtype=wtype, batch=batch, resident=K, **SMALL)
    print("case small %s B=%d K=%d" % (wtype, batch, K), flush=True)
    got, st = _run_decode(wl)
    if batch * wl.top_k > K:
        assert st["host_planned"] == wl.steps * wl.layers
    else:
        assert st["device_planned"] == wl.steps * wl.layers
    ref, _ = _run_decode(wl, flags=pe.PE_FLAG_UNPAGED, check_oracle=False)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("batch", [2, 9])
def test_many_experts_take_the_general_planner(batch):
    """E above 256 (the copiers' one-wavefront planner covers E <= 256): the
    device-planned step (batch*k <= K) runs the general planner + page-in +
    expert kernels, the host-planned one (batch*k > K) its usual waves."""
    wl = synth.workload("decode_bf16_k40_b1", layers=2, experts=320, top_k=4, resident=24, hidden=256, inter=256,
                        batch=batch, steps=6)
    print("case E=320 batch %d" % batch, flush=True)
    got, st = _run_decode(wl)
    if batch * wl.top_k <= wl.resident:
        assert st["device_planned"] == wl.steps * wl.layers
    else:
        assert st["host_planned"] == wl.steps * wl.layers
    ref, _ = _run_decode(wl, flags=pe.PE_FLAG_UNPAGED, check_oracle=False)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("wtype", ["bf16", "int4", "mxfp4"])
@pytest.mark.parametrize("batch", [1, 3])
def test_largest_hidden_and_inter(wtype, batch):
    """H = I = 4096, the largest the library takes (a bf16 expert is 100 MB):
    device-planned steps (batch 1) and host-planned ones (batch 3: 6 entries >
    K = 3, mostly two waves), against the oracle and an unpaged run."""
    wl = synth.workload("decode_bf16_k40_b1", layers=1, experts=8, top_k=2, resident=3, hidden=4096, inter=4096,
                        wtype=wtype, batch=batch, steps=4)
    print("case H=I=4096 %s batch %d" % (wtype, batch), flush=True)
    got, st = _run_decode(wl)
    assert st["host_planned" if batch * wl.top_k > wl.resident else "device_planned"] == wl.steps
    ref, _ = _run_decode(wl, flags=pe.PE_FLAG_UNPAGED, check_oracle=False)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("wtype", ["fp8", "int4", "mxfp4"])
def test_widest_token_batch_at_largest_hidden(wtype):
    """Batch 8, the widest GEMV token batch, at H = 4096: a gate/up workgroup
    stages 64 KB of token vectors and its rows' scales (more LDS than one
    workgroup may take on parts before gfx950).  16 entries fill K = 16: a
    device-planned step, then the same steps host-planned (one wave each),
    bitwise equal, and both against the oracle."""
    wl = synth.workload("decode_bf16_k40_b1", layers=1, experts=16, top_k=2, resident=16, hidden=4096, inter=256,
                        wtype=wtype, batch=8, steps=3)
    print("case batch 8 H=4096 %s" % wtype, flush=True)
    got, st = _run_decode(wl)
    assert st["device_planned"] == wl.steps
    hp, st = _run_decode(wl, flags=pe.PE_FLAG_FORCE_HOST_PLAN)
    assert st["host_planned"] == wl.steps
    assert np.array_equal(got, hp)


@pytest.mark.parametrize("batch", [4, 9])
def test_most_experts(batch):
    """E = 1024, the largest expert count: 32 entries fill K = 32 exactly (one
    device-planned wave); 72 entries over ~55 distinct experts take two
    host-planned waves."""
    wl = synth.workload("decode_bf16_k40_b1", layers=1, experts=1024, top_k=8, resident=32, hidden=128, inter=128,
                        batch=batch, steps=6)
    print("case E=1024 batch %d" % batch, flush=True)
    got, st = _run_decode(wl)
    assert st["device_planned" if batch * wl.top_k <= wl.resident else "host_planned"] == wl.steps
    ref, _ = _run_decode(wl, flags=pe.PE_FLAG_UNPAGED, check_oracle=False)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("wtype", ["bf16", "int4", "mxfp4"])
def test_ragged_shapes(wtype):
    """Row lengths that leave lanes idle and token batches past the GEMV batch
    (MXFP4: multiples of 64 but not of 128, GEMV only)."""
    H, I = {"int4": (384, 640), "mxfp4": (320, 448), "bf16": (200, 72)}[wtype]
    wl = synth.workload("decode_bf16_k40_b1", layers=1, experts=12, top_k=3, resident=12, hidden=H, inter=I,
                        wtype=wtype, batch=5, steps=3)
    print("case ragged %s H=%d I=%d" % (wtype, H, I), flush=True)
    _run_decode(wl)


@pytest.mark.parametrize("wtype", ["bf16", "fp8", "int4", "int8", "mxfp4"])
def test_force_host_plan_and_dma_match_device_plan_bitwise(wtype):
    wl = synth.workload("decode_bf16_k40_b1", wtype=wtype, batch=1, resident=6, **SMALL)
    print("case host-plan/dma equivalence %s" % wtype, flush=True)
    a, sa = _run_decode(wl, check_oracle=False)
    b, sb = _run_decode(wl, flags=pe.PE_FLAG_FORCE_HOST_PLAN, check_oracle=False)
    c, sc = _run_decode(wl, flags=pe.PE_FLAG_FORCE_HOST_PLAN | pe.PE_FLAG_PAGEIN_DMA, check_oracle=False)
    assert np.array_equal(a, b) and np.array_equal(a, c)
    assert sb["host_planned"] == wl.steps * wl.layers and sa["device_planned"] == wl.steps * wl.layers
    for key in ("page_ins", "distinct", "entries", "waves"):
        assert sa[key] == sb[key] == sc[key], key


def test_stats_count_simulator_misses():
    wl = synth.workload("decode_bf16_k40_b1", batch=2, resident=5, **SMALL)
    sims = [LayerLRU(wl.experts, wl.resident) for _ in range(wl.layers)]
    _, st = _run_decode(wl, check_oracle=False, sims=sims)
    r = synth.routing_for(wl)
    misses = distinct = 0
    check = [LayerLRU(wl.experts, wl.resident) for _ in range(wl.layers)]
    for s in range(wl.steps):
        for l in range(wl.layers):
            ids = r["decode_ids"][s, l].ravel()
            misses += sum(w.count for w in check[l].step(ids))
            distinct += len(set(ids.tolist()))
    assert st["page_ins"] == misses and st["distinct"] == distinct
    _, copied = pe.pe_expert_bytes("bf16", wl.hidden, wl.inter)
    assert st["page_in_bytes"] == misses * copied


def test_invalid_ids_are_counted_and_contribute_nothing():
    wl = synth.workload("decode_bf16_k40_b1", layers=1, experts=8, top_k=2, resident=4, hidden=64, inter=128,
                        batch=2, steps=1)
    print("case invalid ids", flush=True)
    m = harness.make_moe(wl)
    harness.load_store(m, wl)
    x = torch.from_numpy(synth.hidden_states(wl, 0, 2).view(np.int16)).view(torch.bfloat16).to(DEV)
    ids_np = np.array([[3, 9], [-2, 5]], np.int32)
    w_np = np.array([[0.5, 0.5], [0.25, 0.75]], np.float32)
    out = torch.empty((2, 64), dtype=torch.bfloat16, device=DEV)
    m.forward(0, x, torch.from_numpy(ids_np).to(DEV), torch.from_numpy(w_np).to(DEV), out)
    torch.cuda.synchronize()
    assert m.stats()["bad_ids"] == 2
    ref = moe.moe_layer(formats.bf16_to_f32(harness.bf16_bits(x)), ids_np, w_np, _expert_fn(wl, 0), num_experts=8)
    _check_close(harness.bf16_bits(out), ref, "bf16")
    assert m.slot_map(0, 2).tolist()[1] == -1 and m.slot_map(0, 2).tolist()[2] == -1
    m.close()


@pytest.mark.parametrize("wtype", ["bf16", "int4"])
def test_repeated_ids_within_a_token(wtype):
    """A token may name one expert at several of its k positions: each position
    is its own entry (own router weight), summed in position order.  One
    device-planned step (6 entries <= K = 6) and one host-planned step (9
    entries > K, one of them invalid), against the oracle and an unpaged run."""
    wl = synth.workload("decode_bf16_k40_b1", layers=1, experts=12, top_k=3, resident=6, hidden=256, inter=256,
                        wtype=wtype, batch=3, steps=1)
    print("case repeated ids %s" % wtype, flush=True)
    x = torch.from_numpy(synth.hidden_states(wl, 0, 3).view(np.int16)).view(torch.bfloat16).to(DEV)
    cases = [(np.array([[4, 4, 7], [7, 1, 7]], np.int32), 2),
             (np.array([[2, 2, 2], [0, 5, 0], [9, 11, -1]], np.int32), 3)]
    rng = np.random.default_rng(3)
    outs = {}
    for flags in (0, pe.PE_FLAG_UNPAGED):
        m = harness.make_moe(wl, flags=flags)
        harness.load_store(m, wl)
        for ci, (ids_np, T) in enumerate(cases):
            w_np = rng.random(ids_np.shape).astype(np.float32) if flags == 0 else outs[("w", ci)]
            outs[("w", ci)] = w_np
            out = torch.empty((T, wl.hidden), dtype=torch.bfloat16, device=DEV)
            m.forward(0, x[:T], torch.from_numpy(ids_np).to(DEV), torch.from_numpy(w_np).to(DEV), out, T=T)
            torch.cuda.synchronize()
            outs[(flags, ci)] = harness.bf16_bits(out)
            if flags == 0:
                ref = moe.moe_layer(formats.bf16_to_f32(harness.bf16_bits(x[:T])), ids_np, w_np, _expert_fn(wl, 0),
                                    num_experts=wl.experts)
                _check_close(outs[(flags, ci)], ref, wtype, "case %d" % ci)
        st = m.stats()
        if flags == 0:
            assert st["device_planned"] == 1 and st["host_planned"] == 1 and st["bad_ids"] == 1
        m.close()
    for ci in range(len(cases)):
        assert np.array_equal(outs[(0, ci)], outs[(pe.PE_FLAG_UNPAGED, ci)]), ci


@pytest.mark.parametrize("wtype", ["bf16", "fp8", "int4"])
def test_expert_with_more_entries_than_a_token_batch(wtype):
    """An expert routed by 10 or 11 of a step's tokens runs its GEMV rows in two
    token batches (8, then the rest), re-staging the token vectors but keeping
    the scales staged with the first.  Three steps: device-planned with the
    expert paged in (streamed), device-planned with it resident, host-planned
    (13 entries > K = 12, one wave); against the oracle and an unpaged run."""
    wl = synth.workload("decode_bf16_k40_b1", layers=1, experts=16, top_k=1, resident=12, hidden=512, inter=256,
                        wtype=wtype, batch=13, steps=1)
    print("case long expert %s" % wtype, flush=True)
    x = torch.from_numpy(synth.hidden_states(wl, 0, 13).view(np.int16)).view(torch.bfloat16).to(DEV)
    a_ids = np.array([3] * 10 + [5, 7], np.int32).reshape(12, 1)
    b_ids = np.array([3] * 6 + [9] + [3] * 5 + [5], np.int32).reshape(13, 1)
    cases = [a_ids, a_ids, b_ids]
    rng = np.random.default_rng(5)
    ws = [rng.random(c.shape).astype(np.float32) for c in cases]
    outs = {}
    for flags in (0, pe.PE_FLAG_UNPAGED):
        m = harness.make_moe(wl, flags=flags)
        harness.load_store(m, wl)
        for ci, ids_np in enumerate(cases):
            T = ids_np.shape[0]
            out = torch.empty((T, wl.hidden), dtype=torch.bfloat16, device=DEV)
            m.forward(0, x[:T], torch.from_numpy(ids_np).to(DEV), torch.from_numpy(ws[ci]).to(DEV), out, T=T)
            torch.cuda.synchronize()
            outs[(flags, ci)] = harness.bf16_bits(out)
            if flags == 0:
                ref = moe.moe_layer(formats.bf16_to_f32(harness.bf16_bits(x[:T])), ids_np, ws[ci],
                                    _expert_fn(wl, 0), num_experts=wl.experts)
                _check_close(outs[(flags, ci)], ref, wtype, "case %d" % ci)
        st = m.stats()
        if flags == 0:
            assert st["device_planned"] == 2 and st["host_planned"] == 1 and st["page_ins"] == 4
        m.close()
    for ci in range(len(cases)):
        assert np.array_equal(outs[(0, ci)], outs[(pe.PE_FLAG_UNPAGED, ci)]), ci


@pytest.mark.parametrize("wtype", ["int4", "mxfp4", "fp8", "int8"])
def test_one_wave_host_step_with_h_outside_lds(wtype):
    """One-wave host-planned steps (60 entries > K = 12 over at most 10 distinct
    experts) whose h does not fit in LDS (60 x 1024 bf16 = 120 KiB), so launch B
    reads h from global memory, and whose busiest expert has 6 tokens (8-token
    batches): the launch B variants whose lane-group reduction is a rolled loop
    (int4, MXFP4) or unrolled (FP8, int8).  Two steps, the first all page-ins,
    the second 6 hits and 4 page-ins; plans and state against the simulator,
    outputs against the oracle and bitwise against an unpaged run."""
    T, k = 15, 4
    wl = synth.workload("decode_bf16_k40_b1", layers=1, experts=16, top_k=k, resident=12, hidden=256, inter=1024,
                        wtype=wtype, batch=T, steps=1)
    print("case one-wave host step, h outside LDS, %s" % wtype, flush=True)
    rng = np.random.default_rng(11)

    def step_ids(pool, busy):
        # `busy` in the first 6 tokens, the other k (or k - 1) ids distinct, from `pool`
        rest = [e for e in pool if e != busy]
        rows = []
        for t in range(T):
            if t < 6:
                rows.append([busy] + [int(v) for v in rng.choice(rest, size=k - 1, replace=False)])
            else:
                rows.append([int(v) for v in rng.choice(rest, size=k, replace=False)])
        return np.array(rows, np.int32)

    cases = [step_ids(list(range(10)), 3), step_ids(list(range(4, 14)), 7)]
    for c in cases:
        assert all(len(set(r.tolist())) == k for r in c) and len(set(c.ravel().tolist())) <= 10
        assert max(np.bincount(c.ravel())) >= 5
    ws = [rng.random(c.shape).astype(np.float32) for c in cases]
    x = torch.from_numpy(synth.hidden_states(wl, 0, T).view(np.int16)).view(torch.bfloat16).to(DEV)
    xr = formats.bf16_to_f32(harness.bf16_bits(x))
    outs = {}
    for flags in (0, pe.PE_FLAG_UNPAGED):
        m = harness.make_moe(wl, flags=flags)
        harness.load_store(m, wl)
        sim = LayerLRU(wl.experts, m.K)
        want_page_ins = 0
        for ci, ids_np in enumerate(cases):
            out = torch.empty((T, wl.hidden), dtype=torch.bfloat16, device=DEV)
            m.forward(0, x, torch.from_numpy(ids_np).to(DEV), torch.from_numpy(ws[ci]).to(DEV), out)
            torch.cuda.synchronize()
            outs[(flags, ci)] = harness.bf16_bits(out)
            if flags == 0:
                waves = sim.step(ids_np.ravel())
                assert len(waves) == 1
                want_page_ins += waves[0].count
                _check_plan(m, 0, waves, T, k, ids_np.ravel())
                _check_state(m, 0, sim)
                ref = moe.moe_layer(xr, ids_np, ws[ci], _expert_fn(wl, 0), num_experts=wl.experts)
                _check_close(outs[(flags, ci)], ref, wtype, "case %d" % ci)
        st = m.stats()
        if flags == 0:
            assert st["host_planned"] == 2 and st["page_ins"] == want_page_ins
        m.close()
    for ci in range(len(cases)):
        assert np.array_equal(outs[(0, ci)], outs[(pe.PE_FLAG_UNPAGED, ci)]), ci


def test_zero_tokens_is_a_noop():
    wl = synth.workload("tiny_bf16")
    m = harness.make_moe(wl)
    out = torch.zeros((1, wl.hidden), dtype=torch.bfloat16, device=DEV)
    m.forward(0, out, torch.zeros((1, 2), dtype=torch.int32, device=DEV),
              torch.zeros((1, 2), dtype=torch.float32, device=DEV), out, T=0)
    assert m.stats()["steps"] == 0
    m.close()


def _graph_case(wl):
    r = synth.routing_for(wl)
    m = harness.make_moe(wl)
    harness.load_store(m, wl)
    x, ids, w = harness.decode_inputs(wl, r, DEV)
    return r, m, x, ids, w


def test_captured_graph_matches_eager():
    """Capture one decode step of every layer into a hipGraph; replay it over
    the steps (inputs copied in between replays) and compare bit-for-bit with
    an eager run from the same cold state, plans included."""
    wl = synth.workload("decode_bf16_k40_b1", wtype="int4", batch=2, resident=8, **SMALL)
    print("case graph capture", flush=True)
    r, m, x, ids, w = _graph_case(wl)
    L, B, H = wl.layers, wl.batch, wl.hidden
    # eager reference
    eager = torch.empty((wl.steps, L, B, H), dtype=torch.bfloat16, device=DEV)
    for s in range(wl.steps):
        for l in range(L):
            m.forward(l, x[s], ids[s, l], w[s, l], eager[s, l])
    torch.cuda.synchronize()
    st_eager = [m.lru_state(l) for l in range(L)]
    m.reset_lru()
    m.reset_stats()
    xin = torch.empty_like(x[0])
    iin = torch.empty_like(ids[0])
    win = torch.empty_like(w[0])
    oout = torch.empty((L, B, H), dtype=torch.bfloat16, device=DEV)
    xin.copy_(x[0]); iin.copy_(ids[0]); win.copy_(w[0])
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for l in range(L):
                m.forward(l, xin, iin[l], win[l], oout[l], stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    m.reset_lru()          # capture does not run the kernels; start cold like the eager run
    m.reset_stats()
    torch.cuda.synchronize()
    for s in range(wl.steps):
        xin.copy_(x[s]); iin.copy_(ids[s]); win.copy_(w[s])
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(harness.bf16_bits(oout), harness.bf16_bits(eager[s])), s
    for l in range(L):
        se, lu, tick = m.lru_state(l)
        assert np.array_equal(se, st_eager[l][0]) and np.array_equal(lu, st_eager[l][1]) and tick == st_eager[l][2]
    assert m.stats()["device_planned"] == wl.steps * L
    m.close()


def test_host_planned_step_refuses_capture():
    wl = synth.workload("decode_bf16_k40_b1", batch=3, resident=6, **SMALL)
    r, m, x, ids, w = _graph_case(wl)
    out = torch.empty((wl.batch, wl.hidden), dtype=torch.bfloat16, device=DEV)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    rc = None
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            rc = pe.pe_forward_rc(m.ctx, 0, x[0], ids[0, 0], w[0, 0], wl.batch, out, side)
    torch.cuda.synchronize()
    assert rc == pe.PE_ERR_NOT_CAPTURABLE
    assert m.stats()["steps"] == 0
    m.close()


def test_reset_lru_midway_matches_resetting_simulator():
    wl = synth.workload("decode_bf16_k40_b1", batch=1, resident=5, **SMALL)
    r = synth.routing_for(wl)
    m = harness.make_moe(wl)
    harness.load_store(m, wl)
    x, ids, w = harness.decode_inputs(wl, r, DEV)
    sims = [LayerLRU(wl.experts, wl.resident) for _ in range(wl.layers)]
    out = torch.empty((wl.batch, wl.hidden), dtype=torch.bfloat16, device=DEV)
    for s in range(wl.steps):
        if s == 4:
            m.reset_lru(1)
            sims[1].reset()
        for l in range(wl.layers):
            m.forward(l, x[s], ids[s, l], w[s, l], out)
            waves = sims[l].step(r["decode_ids"][s, l].ravel())
            _check_plan(m, l, waves, wl.batch, wl.top_k, r["decode_ids"][s, l].ravel())
            _check_state(m, l, sims[l])
    m.close()


def _plans_match(rec, waves, ids_flat, E):
    """A parsed plan-log record against the simulator's waves of the same step."""
    assert rec["n_waves"] == len(waves)
    for g, wv in zip(rec["waves"], waves):
        assert (g["count"], g["experts"].tolist(), g["slots"].tolist(), g["evicted"].tolist()) == \
            (wv.count, wv.plan_experts, wv.plan_slots, wv.evicted)
    want = [next((wv.slot_of[e] for wv in waves if e in wv.slot_of), -1) if 0 <= e < E else -1
            for e in (int(v) for v in ids_flat)]
    assert rec["slot_of"][:len(want)].tolist() == want


def _state_matches(rec, sim):
    assert rec["slot_expert"].tolist() == sim.slot_expert
    assert rec["last_use"].tolist() == sim.last_use
    assert rec["tick"] == sim.tick


def test_plan_log_records_every_step_and_wraps():
    """The plan log holds the plan, slot map and LRU state of every step of every
    layer; with fewer records than steps it keeps the most recent ones."""
    wl = synth.workload("decode_bf16_k40_b1", batch=1, resident=5, **SMALL)
    r = synth.routing_for(wl)
    cap = 7
    m = harness.make_moe(wl, plan_log_steps=cap)
    harness.load_store(m, wl)
    x, ids, w = harness.decode_inputs(wl, r, DEV)
    out = torch.empty((wl.batch, wl.hidden), dtype=torch.bfloat16, device=DEV)
    sims = [LayerLRU(wl.experts, wl.resident) for _ in range(wl.layers)]
    want = {l: [] for l in range(wl.layers)}
    for s in range(wl.steps):
        for l in range(wl.layers):
            m.forward(l, x[s], ids[s, l], w[s, l], out)
            e = r["decode_ids"][s, l].ravel()
            want[l].append((sims[l].step(e), e, sims[l].state()))
    for l in range(wl.layers):
        recs = m.plan_log(l)
        assert len(recs) == cap
        for i, rec in enumerate(recs):
            s = wl.steps - cap + i
            assert rec["seq"] == s and rec["T"] == wl.batch
            waves, e, (se, lu, tick) = want[l][s]
            _plans_match(rec, waves, e, wl.experts)
            assert (rec["slot_expert"].tolist(), rec["last_use"].tolist(), rec["tick"]) == (se, lu, tick)
    assert len(m.plan_log(0, max_records=3)) == 3
    m.close()


def test_replayed_graph_then_host_planned_steps_share_the_lru_state():
    """Device-planned steps replayed from a hipGraph and host-planned steps
    interleaved on one context: every host-planned step must plan from the state
    the replays left (the host never trusts an older copy of it).  Plans, slot
    maps and states (read from the plan log) match the simulator at every step,
    outputs equal an unpaged run bitwise and the oracle within tolerance."""
    wl = synth.workload("decode_bf16_k40_b1", layers=2, experts=16, top_k=4, resident=8, hidden=256, inter=256,
                        wtype="int4", batch=3, steps=12)
    print("case replay + host-planned", flush=True)
    r = synth.routing_for(wl)
    L, H, k = wl.layers, wl.hidden, wl.top_k
    x_np = np.stack([synth.hidden_states(wl, s, 3) for s in range(wl.steps)])
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(DEV)
    ids = torch.from_numpy(np.ascontiguousarray(r["decode_ids"])).to(DEV)      # [S, L, 3, k]
    w = torch.from_numpy(np.ascontiguousarray(r["decode_w"])).to(DEV)
    # steps 0, 5, 9 and 11 take all 3 tokens (12 entries > K: host-planned); the
    # others take the first 2 (8 entries <= K) through the captured graph
    host_steps = {0, 5, 9, 11}
    outs = {}
    for flags in (0, pe.PE_FLAG_UNPAGED):
        m = harness.make_moe(wl, flags=flags, plan_log_steps=wl.steps)
        harness.load_store(m, wl)
        xin = torch.empty((2, H), dtype=torch.bfloat16, device=DEV)
        iin = torch.empty((L, 2, k), dtype=torch.int32, device=DEV)
        win = torch.empty((L, 2, k), dtype=torch.float32, device=DEV)
        gout = torch.empty((L, 2, H), dtype=torch.bfloat16, device=DEV)
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for l in range(L):
                    m.forward(l, xin, iin[l], win[l], gout[l], stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        res = []
        for s in range(wl.steps):
            if s in host_steps:
                o = torch.empty((L, 3, H), dtype=torch.bfloat16, device=DEV)
                for l in range(L):
                    m.forward(l, x[s], ids[s, l], w[s, l], o[l])
                torch.cuda.synchronize()
                res.append(harness.bf16_bits(o))
            else:
                xin.copy_(x[s, :2]); iin.copy_(ids[s, :, :2]); win.copy_(w[s, :, :2])
                g.replay()
                torch.cuda.synchronize()
                res.append(harness.bf16_bits(gout))
        st = m.stats()
        if flags == 0:
            assert st["host_planned"] == len(host_steps) * L
            assert st["device_planned"] == (wl.steps - len(host_steps)) * L
            sims = [LayerLRU(wl.experts, wl.resident) for _ in range(L)]
            recs = [m.plan_log(l) for l in range(L)]
            fns = [_expert_fn(wl, l) for l in range(L)]
            for s in range(wl.steps):
                T = 3 if s in host_steps else 2
                for l in range(L):
                    e = r["decode_ids"][s, l, :T]
                    waves = sims[l].step(e.ravel())
                    rec = recs[l][s]
                    assert rec["seq"] == s and rec["T"] == T
                    _plans_match(rec, waves, e.ravel(), wl.experts)
                    _state_matches(rec, sims[l])
                    ref = moe.moe_layer(formats.bf16_to_f32(x_np[s, :T]), e, r["decode_w"][s, l, :T], fns[l])
                    _check_close(res[s][l], ref, wl.wtype, "step %d layer %d" % (s, l))
        outs[flags] = res
        m.close()
    for s in range(wl.steps):
        assert np.array_equal(outs[0][s], outs[pe.PE_FLAG_UNPAGED][s]), s
