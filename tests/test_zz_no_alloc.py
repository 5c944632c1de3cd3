"""pe_forward_static -- pe_forward for callers that cannot allocate, with the
step's activations in the library's fixed device scratch area -- against
pe_forward itself, through the C ABI: two contexts with the same weights take
the same steps, one through each entry point, and must give the same bits.
Every case makes two calls in a row, the second with a smaller input."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
import harness
import host_paged_expert_amd as pe

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(wl, T, seed, always=None):
    """Seeded step inputs: T tokens of k distinct ids (each including expert
    `always` if given), router weights in [0, 1)."""
    rng = np.random.default_rng(seed)
    x = synth.hidden_states(wl, seed, T)
    rows = []
    for _ in range(T):
        if always is None:
            rows.append(rng.choice(wl.experts, wl.top_k, replace=False))
        else:
            rest = rng.choice([e for e in range(wl.experts) if e != always], wl.top_k - 1, replace=False)
            rows.append(np.concatenate([[always], rest]))
    ids = np.stack(rows).astype(np.int32)
    w = rng.random((T, wl.top_k)).astype(np.float32)
    return (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV), torch.from_numpy(ids).to(DEV),
            torch.from_numpy(w).to(DEV))


@pytest.mark.parametrize("wtype", ["bf16", "int4"])
def test_static_scratch_matches_forward(wtype):
    wl = synth.workload("decode_bf16_k40_b1", layers=2, experts=16, top_k=4, resident=8, hidden=256, inter=256,
                        wtype=wtype, batch=1, steps=1)
    a = harness.make_moe(wl, max_tokens=32)
    b = harness.make_moe(wl, max_tokens=32)
    harness.load_store([a, b], wl)
    # (T, expert every token routes to): device-planned 2 then 1 token; host-planned
    # 5 then 3 tokens (20 and 12 entries > K = 8); MFMA steps of 24 then 17 tokens
    # (one expert with >= 16 entries)
    cases = [(2, None), (1, None), (5, None), (3, None), (24, 3), (17, 3)]
    for seed, (T, always) in enumerate(cases):
        print("case %s T=%d" % (wtype, T), flush=True)
        x, ids, w = _inputs(wl, T, seed, always)
        for l in range(wl.layers):
            oa = torch.empty((T, wl.hidden), dtype=torch.bfloat16, device=DEV)
            ob = torch.full((T, wl.hidden), 7.0, dtype=torch.bfloat16, device=DEV)
            pe.pe_forward(a.ctx, l, x, ids, w, T, oa, None)
            pe.pe_forward_static(b.ctx, l, x, ids, w, T, ob, None)
            torch.cuda.synchronize()
            assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), (T, l)
    sa, sb = a.stats(), b.stats()
    assert sa == sb and sa["host_planned"] == 4 * wl.layers and sa["device_planned"] == 2 * wl.layers
    a.close()
    b.close()


def test_static_scratch_under_graph_capture():
    """A device-planned step through pe_forward_static captured into a hipGraph and
    replayed with new inputs equals the same steps through pe_forward, eagerly;
    the second replay's step has fewer valid entries (one token's ids invalid)."""
    wl = synth.workload("decode_bf16_k40_b1", layers=2, experts=16, top_k=4, resident=8, hidden=256, inter=256,
                        wtype="fp8", batch=2, steps=1)
    a = harness.make_moe(wl, max_tokens=2)
    b = harness.make_moe(wl, max_tokens=2)
    harness.load_store([a, b], wl)
    L, H = wl.layers, wl.hidden
    xin = torch.empty((2, H), dtype=torch.bfloat16, device=DEV)
    iin = torch.empty((L, 2, wl.top_k), dtype=torch.int32, device=DEV)
    win = torch.empty((L, 2, wl.top_k), dtype=torch.float32, device=DEV)
    gout = torch.empty((L, 2, H), dtype=torch.bfloat16, device=DEV)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for l in range(L):
                pe.pe_forward_static(b.ctx, l, xin, iin[l], win[l], 2, gout[l], side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        x, ids, w = _inputs(wl, 2, 100 + rep)
        ids_l = torch.stack([ids.clone() for _ in range(L)])
        if rep == 1:
            ids_l[:, 1] = -1          # the second token routes nowhere: fewer entries
        w_l = torch.stack([w for _ in range(L)])
        xin.copy_(x); iin.copy_(ids_l); win.copy_(w_l)
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            oa = torch.empty((2, H), dtype=torch.bfloat16, device=DEV)
            pe.pe_forward(a.ctx, l, x, ids_l[l], w_l[l], 2, oa, None)
            torch.cuda.synchronize()
            assert torch.equal(oa.view(torch.int16), gout[l].view(torch.int16)), (rep, l)
    a.close()
    b.close()


def test_static_scratch_rejects_steps_beyond_its_size():
    """H = I = 4096: an entry needs 24 KiB, so 800 entries exceed the 16 MiB area."""
    m = pe.PagedMoE(1, 8, 4, 4, 4096, 4096, 200)
    x = torch.zeros((200, 4096), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((200, 4), dtype=torch.int32, device=DEV)
    w = torch.zeros((200, 4), dtype=torch.float32, device=DEV)
    out = torch.zeros((200, 4096), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(pe.PEError) as ei:
        pe.pe_forward_static(m.ctx, 0, x, ids, w, 200, out, None)
    assert ei.value.code == pe.PE_ERR_INVALID_ARG and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert m.stats()["steps"] == 0
    m.close()
