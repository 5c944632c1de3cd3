"""Harness around libpe for tests, the benchmark and smoke(): builds a context
for a synthetic workload, fills its host store from `synth` (in parallel
threads: the generator and pe_load_expert both release the GIL), and turns
the workload's routing into device tensors.  No method arithmetic here.
"""
import os
import sys
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import synth
import host_paged_expert_amd as pe


def host_threads() -> int:
    """Worker threads for loading: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 4
    return max(1, min(16, n))


def make_moe(wl, flags=0, max_tokens=None, device=0, plan_log_steps=0):
    """A PagedMoE context for the workload; plan_log_steps > 0 turns on the plan log."""
    if max_tokens is None:
        max_tokens = max(wl.batch, wl.prefill_tokens, 1)
    if plan_log_steps:
        flags |= pe.PE_FLAG_PLAN_LOG
    return pe.PagedMoE(wl.layers, wl.experts, wl.top_k, wl.resident, wl.hidden, wl.inter, max_tokens,
                       wl.wtype, device, flags, plan_log_steps)


def load_store(moe, wl, threads=None, layers=None, experts=None, progress=None):
    """Generate every expert of the workload and write it with pe_load_expert
    into `moe`, or into each context of a list (one generation per expert)."""
    moes = list(moe) if isinstance(moe, (list, tuple)) else [moe]
    layers = range(wl.layers) if layers is None else layers
    experts = range(wl.experts) if experts is None else experts
    jobs = [(l, e) for l in layers for e in experts]
    done = [0]
    lock = threading.Lock()

    def one(job):
        l, e = job
        t13, t2, s13, s2 = synth.expert_tensors(wl, l, e)
        for m in moes:
            m.load_expert(l, e, t13, t2, s13, s2)
        if progress is not None:
            with lock:
                done[0] += 1
                if done[0] % progress == 0:
                    print("  loaded %d/%d experts" % (done[0], len(jobs)), file=sys.stderr, flush=True)

    with ThreadPoolExecutor(threads or host_threads()) as ex:
        list(ex.map(one, jobs))


def decode_inputs(wl, routing, device, steps=None):
    """Device tensors for decode: x [S, B, H] bf16 (as int16 bits viewed bf16),
    ids [S, L, B, k] int32, w [S, L, B, k] fp32."""
    import torch
    steps = wl.steps if steps is None else steps
    B = wl.batch
    x = np.stack([synth.hidden_states(wl, s, B) for s in range(steps)])
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(device)
    ids = torch.from_numpy(np.ascontiguousarray(routing["decode_ids"][:steps])).to(device)
    w = torch.from_numpy(np.ascontiguousarray(routing["decode_w"][:steps])).to(device)
    return xt, ids, w


class DecodeRunner:
    """Decode steps of a workload, launched the way bench.py times them.

    When every step fits one device-planned wave (batch x top_k <= K) and
    `capture` is set, one step through every layer is captured once as a
    hipGraph and replayed; the graph picks its step's inputs from x_all /
    ids_all / w_all on the device with a step counter that it advances itself.
    Otherwise pe_forward runs eagerly per layer, called straight through the
    C ABI with addresses worked out once (the tensors are checked once, here).
    The latest step's output is in `out` [L, B, H].  `rewind()` makes the next
    step step 0 again.
    """

    def __init__(self, moe, wl, x_all, ids_all, w_all, out, stream, capture=True):
        import torch
        self.moe, self.wl, self.out, self.stream = moe, wl, out, stream
        self.x_all, self.ids_all, self.w_all = x_all, ids_all, w_all
        self.captured = bool(capture) and wl.batch * wl.top_k <= moe.K
        self.s = 0
        self.sidx = torch.zeros(1, dtype=torch.long, device=out.device)
        self.graph = None
        S, L, B = ids_all.shape[0], wl.layers, wl.batch
        assert tuple(x_all.shape) == (S, B, wl.hidden) and tuple(ids_all.shape) == (S, L, B, wl.top_k)
        assert tuple(w_all.shape) == (S, L, B, wl.top_k) and tuple(out.shape) == (L, B, wl.hidden)
        moe._check_step(x_all.view(S * B, wl.hidden), ids_all.view(S * L * B, wl.top_k),
                        w_all.view(S * L * B, wl.top_k), out.view(L * B, wl.hidden), B)
        self._xs, self._ids, self._ws = x_all.data_ptr(), ids_all.data_ptr(), w_all.data_ptr()
        self._out = out.data_ptr()
        self._sx, self._sid = B * wl.hidden * 2, B * wl.top_k * 4       # bytes per step / layer
        self._handle = stream.cuda_stream
        self.S = S
        if self.captured:
            side = torch.cuda.Stream(device=out.device)
            side.wait_stream(stream)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    xs = torch.index_select(x_all, 0, self.sidx)[0]
                    ids_s = torch.index_select(ids_all, 0, self.sidx)[0]
                    w_s = torch.index_select(w_all, 0, self.sidx)[0]
                    cs = torch.cuda.current_stream()
                    for l in range(wl.layers):
                        moe.forward(l, xs, ids_s[l], w_s[l], out[l], stream=cs)
                    self.sidx.add_(1)
            stream.wait_stream(side)
            torch.cuda.synchronize()
            self.graph = g

    def run(self, n):
        if n < 0 or self.s + n > self.S:
            raise IndexError("steps %d..%d outside the %d-step input window" % (self.s, self.s + n - 1, self.S))
        if self.captured:
            for _ in range(n):
                self.graph.replay()
        else:
            fwd, ctx, L, B, h = pe.lib().pe_forward, self.moe.ctx, self.wl.layers, self.wl.batch, self._handle
            for i in range(n):
                s = self.s + i
                x = self._xs + s * self._sx
                for l in range(L):
                    at = (s * L + l) * self._sid
                    rc = fwd(ctx, l, x, self._ids + at, self._ws + at, B, self._out + l * self._sx, h)
                    if rc != pe.PE_OK:
                        raise pe.PEError(rc, pe.pe_last_error())
        self.s += n

    def rewind(self):
        self.sidx.zero_()
        self.s = 0


def bf16_bits(t) -> np.ndarray:
    """A bf16 torch tensor's raw bits as numpy uint16."""
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)
