#!/usr/bin/env python3
"""Paged-MoE decode benchmark on one MI355X.

A step is one decode token batch through every MoE layer of the workload
(48 layers, E=128, top-8 by default): per layer the device LRU planner, the
page-in of missing experts from pinned host memory, the SwiGLU expert GEMVs
and the fixed-order top-k sum.  Device-planned workloads (tokens x top_k <= K)
are captured as one hipGraph per step (48 layers) and replayed; host-planned
workloads run eagerly.  Inputs (hidden states, routed ids and weights of every
step) are resident in HBM before the timed region; the timed region starts
from an empty slot table (pe_reset_lru) so the roofline covers the same
window.

Output: one JSON line with tok/s, the HBM + host-link roofline of the window
(D*S / 8 TB/s + M*S / measured link rate, D and M counted by the library),
the page-in kernel's achieved link rate, the gate/up GEMV's HBM rate, and the
CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
DTYPES = {"bf16": "bf16", "fp8": "fp8e4m3-w/bf16-x", "int4": "int4-w/bf16-x", "int8": "int8-w/bf16-x",
          "mxfp4": "mxfp4-w/bf16-x"}


def part_bytes(wtype, hidden, inter):
    """Bytes of an expert's four parts (w13, w2, s13, s2) in the library's
    formats: bf16; e4m3 + fp32 per 128x128 block; int4 / int8 codes + fp16 per
    row and 128 inputs; MXFP4 codes + one E8M0 byte per row and 32 inputs."""
    H, I = hidden, inter
    if wtype == "bf16":
        return 4 * I * H, 2 * I * H, 0, 0
    if wtype == "fp8":
        return 2 * I * H, I * H, (2 * I // 128) * (H // 128) * 4, (H // 128) * (I // 128) * 4
    if wtype == "int4":
        return I * H, I * H // 2, 2 * I * (H // 128) * 2, H * (I // 128) * 2
    if wtype == "int8":
        return 2 * I * H, I * H, 2 * I * (H // 128) * 2, H * (I // 128) * 2
    if wtype == "mxfp4":
        return I * H, I * H // 2, 2 * I * (H // 32), H * (I // 32)
    raise ValueError(wtype)


PCIE5_X16_GBS = 32.0 * 16 * 128 / 130 / 8   # 63.0 GB/s per direction


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed decode steps (default: the workload's)")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="decode_bf16_k40_b1")
    ap.add_argument("--cpu-samples", type=int, default=None, help="decode steps the CPU oracle runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of CPU oracle time to sample")
    ap.add_argument("--no-timing-pass", action="store_true")
    ap.add_argument("--dma", action="store_true", help="host-planned page-in with hipMemcpyAsync")
    ap.add_argument("--repeats", type=int, default=2, help="timed repetitions (best and median reported)")
    ap.add_argument("--eager", action="store_true",
                    help="profiling: run device-planned steps without the hipGraph (per-dispatch counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="concurrency sweep: decode tok/s for every batch in --sweep-batches at every K in "
                         "--sweep-resident (the workload's format and routing), one JSON line per point")
    ap.add_argument("--sweep-batches", default="1,2,3,4,5,6,7,8")
    ap.add_argument("--sweep-resident", default="24,40")
    ap.add_argument("--warm-prefill", action="store_true",
                    help="prefill workloads: also time the chunk with every expert resident (K = E, no page-in), "
                         "which exposes the MFMA expert kernels")
    ap.add_argument("--others", default=None,
                    help="comma-separated workloads measured after the main one, each on a window of "
                         "min(steps, 128) steps with its own oracle check (default: the other configs when "
                         "--workload is not given, none otherwise)")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MIB",
                    help="profiling: first run one plain device-to-device copy of this many MiB, "
                         "a known-size kernel to scale memory counters by")
    return ap.parse_args()


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--pmc-summary":
        pmc_summary(*sys.argv[2:6])
        return
    args = parse()
    if args.sweep and args.gpus == 1:
        sweep(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this method keeps its slot tables and LRU state on one GPU, "
              "and multi-GPU runs are out of scope; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import harness
    import synth
    import host_paged_expert_amd as pe

    base = synth.WORKLOADS[args.workload]
    steps = args.steps or base.steps
    warmup = max(0, args.warmup)
    over = {"steps": max(steps, warmup, base.steps)}
    wl = synth.workload(args.workload, **over)
    dev = "cuda:0"
    torch.cuda.init()
    if args.copy_reference:
        n = args.copy_reference << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("reference copy: %d MiB device-to-device" % args.copy_reference)
        del src, dst
    flags = pe.PE_FLAG_PAGEIN_DMA if args.dma else 0
    device_planned = wl.batch * wl.top_k <= wl.resident
    captured = device_planned and not args.eager

    t0 = time.time()
    m = harness.make_moe(wl, flags=flags)
    log("context: %d layers x %d experts, K=%d, %s; pinned store ready in %.1fs" %
        (wl.layers, wl.experts, wl.resident, wl.wtype, time.time() - t0))
    t0 = time.time()
    harness.load_store(m, wl, progress=wl.layers * wl.experts // 8)
    log("host store filled in %.1fs" % (time.time() - t0))

    link_dma = pe.pe_link_probe(m.ctx, 1 << 30, 0, 5)
    link_kernel = pe.pe_link_probe(m.ctx, 1 << 30, 1, 5)
    link = max(link_dma, link_kernel)
    log("host->device link: DMA %.2f GB/s, mapped-read kernel %.2f GB/s" % (link_dma, link_kernel))

    routing = synth.routing_for(wl)
    x_all, ids_all, w_all = harness.decode_inputs(wl, routing, dev)
    L, B, H = wl.layers, wl.batch, wl.hidden
    out = torch.empty((L, B, H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    # Prefill workloads: a cold chunk of prefill_tokens tokens through every layer
    # (host-planned waves, MFMA expert kernels), then the decode continuation.
    has_prefill = wl.routing == "prefill_zipf"
    if has_prefill:
        Tp = wl.prefill_tokens
        xp_np = synth.hidden_states(wl, -1, Tp)
        xp = torch.from_numpy(xp_np.view(np.int16)).view(torch.bfloat16).to(dev)
        idsp = torch.from_numpy(np.ascontiguousarray(routing["prefill_ids"])).to(dev)
        wp = torch.from_numpy(np.ascontiguousarray(routing["prefill_w"])).to(dev)
        outp = torch.empty((L, Tp, H), dtype=torch.bfloat16, device=dev)

    def run_prefill():
        for l in range(L):
            m.forward(l, xp, idsp[l], wp[l], outp[l], stream=stream)

    runner = harness.DecodeRunner(m, wl, x_all, ids_all, w_all, out, stream, capture=captured)
    if captured:
        log("captured one %d-layer decode step as a hipGraph" % L)

    def run(n):
        runner.run(n)

    def cold():
        torch.cuda.synchronize()
        m.reset_lru(-1, stream)
        runner.rewind()
        torch.cuda.synchronize()
        m.reset_stats()

    def diff(a, b):
        return {k: a[k] - b[k] for k in a}

    # warm-up (untimed), then timed repetitions from a cold slot table
    cold()
    if has_prefill:
        run_prefill()
    run(warmup)
    torch.cuda.synchronize()
    times = []
    stats = None
    prefill_ms, prefill_stats = [], None
    for rep in range(max(1, args.repeats)):
        cold()
        before = m.stats()
        if has_prefill:
            p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            p0.record(stream)
            run_prefill()
            p1.record(stream)
            torch.cuda.synchronize()
            prefill_ms.append(p0.elapsed_time(p1))
            after_p = m.stats()
            prefill_stats = diff(after_p, before)
            before = after_p
            log("rep %d: prefill of %d tokens in %.1f ms, %d page-ins" % (rep, Tp, prefill_ms[-1],
                                                                         prefill_stats["page_ins"]))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        run(steps)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        times.append(ms)
        st = diff(m.stats(), before)
        if stats is None:
            stats = st
        elif st["page_ins"] != stats["page_ins"] or st["distinct"] != stats["distinct"]:
            raise RuntimeError("repetitions planned differently: %r vs %r" % (st, stats))
        log("rep %d: %d steps in %.1f ms (%.2f tok/s), %d page-ins, %d distinct" %
            (rep, steps, ms, steps * B / (ms / 1e3), st["page_ins"], st["distinct"]))
    best_ms = min(times)
    med_ms = sorted(times)[len(times) // 2]
    value = steps * B / (best_ms / 1e3)

    S_alg, S_copy = pe.pe_expert_bytes(wl.wtype, wl.hidden, wl.inter)
    D, M = stats["distinct"], stats["page_ins"]
    t_roof = D * S_alg / (HBM_PEAK_GBS * 1e9) + M * S_alg / (link * 1e9)
    roof_tok_s = steps * B / t_roof

    # Per-kernel timing pass: the same window, eager, each stage bracketed by hipEvents.
    kernel = {}
    sample_steps = []
    samples = {}
    if not args.no_cpu_baseline:
        n_samp = args.cpu_samples or 16
        sample_steps = sorted(set(int(round(v)) for v in np.linspace(0, steps - 1, n_samp)))
    prefill_kernel = None
    if not args.no_timing_pass:
        cold()
        if has_prefill:
            m.set_timing(1)
            run_prefill()
            prefill_kernel = m.timing()
            if not args.no_cpu_baseline:
                samples["prefill"] = harness.bf16_bits(outp)
        before = m.stats()
        m.set_timing(1)
        for s in range(steps):
            for l in range(L):
                m.forward(l, x_all[s], ids_all[s, l], w_all[s, l], out[l], stream=stream)
            if s in sample_steps:
                samples[s] = harness.bf16_bits(out)
        tm = m.timing()
        m.set_timing(0)
        st2 = diff(m.stats(), before)
        if st2["page_ins"] != M or st2["distinct"] != D:
            raise RuntimeError("timing pass planned differently from the timed run")
        _, w2b, _, s2b = part_bytes(wl.wtype, wl.hidden, wl.inter)
        n_pi, ms_pi = tm["page_in"]
        n_dn, ms_dn = tm["down"]
        # the launches each stage brackets on this path
        if device_planned:
            pi_name, dn_name = "step_a_kernel", "down_sum_kernel"
        elif args.dma:
            pi_name, dn_name = "hipMemcpyAsync page-in", "gemv_down_kernel"
        else:
            pi_name, dn_name = "wave_a_kernel", HOST_DOWN
        kernel = {
            "page_in": {"name": pi_name, "launches": n_pi, "avg_us": 1e3 * ms_pi / max(n_pi, 1),
                        "bytes_per_launch": M * S_alg / max(n_pi, 1),
                        "gbs": (M * S_alg / 1e9) / (ms_pi / 1e3) if ms_pi > 0 else None},
            "down": {"name": dn_name, "launches": n_dn, "avg_us": 1e3 * ms_dn / max(n_dn, 1),
                     "bytes_per_launch": D * (w2b + s2b) / max(n_dn, 1),
                     "gbs": (D * (w2b + s2b) / 1e9) / (ms_dn / 1e3) if ms_dn > 0 else None},
            "stages_ms": {k: v[1] for k, v in tm.items()},
        }
        log("stage totals (ms): %s" % ", ".join("%s %.1f" % (k, v[1]) for k, v in tm.items()))

    result = {
        "metric": "paged-MoE decode tok/s, 48-layer 128-expert top-8; HBM & page-in GB/s % peak",
        "value": round(value, 3),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(best_ms / steps, 4),
        "ms_per_step_median": round(med_ms / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPES[wl.wtype],
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "experts": wl.experts, "top_k": wl.top_k,
                   "resident": wl.resident, "hidden": H, "inter": wl.inter, "wtype": wl.wtype,
                   "batch": B, "path": "captured" if captured else ("device-planned eager" if device_planned
                                                                     else "host-planned"),
                   "pagein": "dma" if (args.dma and not captured) else "kernel"},
        "window": {"distinct": D, "page_ins": M, "expert_bytes": S_alg,
                   "miss_rate": M / max(stats["entries"], 1)},
        "roofline_path": {"model": "D*S/HBM + M*S/link", "hbm_gbs": HBM_PEAK_GBS, "link_gbs": round(link, 2),
                          "link_dma_gbs": round(link_dma, 2), "link_kernel_gbs": round(link_kernel, 2),
                          "roof_tok_s": round(roof_tok_s, 2), "frac": round(value / roof_tok_s, 4)},
    }
    if kernel:
        pi = kernel["page_in"]
        result["roofline"] = {"kernel": pi["name"], "bound": "link",
                              "achieved": round(pi["gbs"], 2) if pi["gbs"] else None,
                              "peak": round(PCIE5_X16_GBS, 2), "unit": "GB/s",
                              "frac": round(pi["gbs"] / PCIE5_X16_GBS, 4) if pi["gbs"] else None,
                              "traffic": traffic_for(pi["name"], wl.name, alg_bytes(
                                  pi["name"], wl.wtype, H, wl.inter, D, M, pi["launches"])),
                              "avg_launch_us": round(pi["avg_us"], 2),
                              "launches": pi["launches"], "bytes_per_launch": round(pi["bytes_per_launch"])}
        dn = kernel["down"]
        result["roofline_hbm"] = {"kernel": dn["name"], "bound": "hbm",
                                  "achieved": round(dn["gbs"], 2) if dn["gbs"] else None,
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(dn["gbs"] / HBM_PEAK_GBS, 4) if dn["gbs"] else None,
                                  "traffic": traffic_for(dn["name"], wl.name, alg_bytes(
                                      dn["name"], wl.wtype, H, wl.inter, D, M, dn["launches"])),
                                  "avg_launch_us": round(dn["avg_us"], 2),
                                  "launches": dn["launches"], "bytes_per_launch": round(dn["bytes_per_launch"])}
        result["stages_ms"] = {k: round(v, 2) for k, v in kernel["stages_ms"].items()}

    if has_prefill:
        Dp, Mp = prefill_stats["distinct"], prefill_stats["page_ins"]
        flops = prefill_stats["entries"] * 2.0 * 3 * wl.hidden * wl.inter
        roof_p = Dp * S_alg / (HBM_PEAK_GBS * 1e9) + Mp * S_alg / (link * 1e9)
        best_p = min(prefill_ms)
        pre = {"tokens": Tp, "ms": round(best_p, 2), "ms_median": round(sorted(prefill_ms)[len(prefill_ms) // 2], 2),
               "tok_s": round(Tp / (best_p / 1e3), 1), "distinct": Dp, "page_ins": Mp,
               "waves": prefill_stats["waves"], "roof_ms": round(roof_p * 1e3, 2),
               "frac": round(roof_p * 1e3 / best_p, 4), "gflop": round(flops / 1e9, 1)}
        if prefill_kernel:
            ex_ms = prefill_kernel["gate_up"][1] + prefill_kernel["down"][1]
            pre["expert_kernels_ms"] = round(ex_ms, 2)
            pre["expert_tflops"] = round(flops / (ex_ms / 1e3) / 1e12, 2) if ex_ms > 0 else None
            pre["mfma_frac_bf16_peak"] = round(flops / (ex_ms / 1e3) / 2.5e15, 4) if ex_ms > 0 else None
            pre["page_in_ms"] = round(prefill_kernel["page_in"][1], 2)
            pre["page_in_gbs"] = round(Mp * S_alg / 1e9 / (prefill_kernel["page_in"][1] / 1e3), 2)
        result["prefill"] = pre
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["sample_parity"] = cpu_baseline(wl, routing, steps, sample_steps, samples,
                                                                       M, D, has_prefill, args.cpu_budget)
    m.close()
    if has_prefill and args.warm_prefill:
        del m, runner
        torch.cuda.empty_cache()
        result["prefill_warm"] = warm_prefill(wl, xp, idsp, wp, outp, stream)
    others = others_for(args, sys.argv[1:])
    if others:
        m = runner = xp = idsp = wp = outp = x_all = ids_all = w_all = out = None
        torch.cuda.empty_cache()
        result["other_workloads"] = [other_workload(n, min(steps, 128), warmup, link) for n in others]
    print(json.dumps(result), flush=True)


# Workloads the default run measures after the main one (the other configs of
# the paged-MoE layer), each on a short window with its own oracle check.
OTHER_WORKLOADS = ("decode_fp8_k40_b4", "decode_int4_k26_b4", "decode_int8_k40_b4", "decode_mxfp4_k16_b1",
                   "prefill_bf16_k92")


def others_for(args, argv):
    """The workloads to measure after the main one: `--others` if given, else
    OTHER_WORKLOADS when `--workload` was not given (none otherwise, so a run
    aimed at one workload, a profile for instance, covers that one only); the
    DMA variant measures the main workload only."""
    if args.dma:
        return []
    names = args.others
    if names is None:
        explicit = any(a == "--workload" or a.startswith("--workload=") for a in argv)
        names = "" if explicit else ",".join(OTHER_WORKLOADS)
    return [n for n in names.split(",") if n and n != args.workload]


def other_workload(name, steps, warmup, link):
    """One more workload on a window of `steps` decode steps from an empty slot
    table (after `warmup` untimed steps; prefill workloads time their cold
    chunk first and then the continuation), one repetition, the path roofline
    of the same window, and the same run's checks: page-in, distinct and wave
    counts against the LRU simulator, and outputs of the first and last layer
    at the first and last step (for prefill also three rows of the chunk)
    against the fp32 unpaged oracle."""
    import numpy as np
    import torch

    import harness
    import synth
    import host_paged_expert_amd as pe
    from oracle import formats, moe
    from oracle.lru import LayerLRU

    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    warmup = max(0, min(warmup, steps))
    wl = synth.workload(name, steps=steps)
    t0 = time.time()
    m = harness.make_moe(wl)
    harness.load_store(m, wl)
    log("%s: context loaded in %.1fs" % (name, time.time() - t0))
    routing = synth.routing_for(wl)
    x, ids, w = harness.decode_inputs(wl, routing, dev)
    L, B, H = wl.layers, wl.batch, wl.hidden
    out = torch.empty((L, B, H), dtype=torch.bfloat16, device=dev)
    runner = harness.DecodeRunner(m, wl, x, ids, w, out, stream)
    prefill = wl.routing == "prefill_zipf"
    if prefill:
        Tp = wl.prefill_tokens
        xp = torch.from_numpy(synth.hidden_states(wl, -1, Tp).view(np.int16)).view(torch.bfloat16).to(dev)
        idsp = torch.from_numpy(np.ascontiguousarray(routing["prefill_ids"])).to(dev)
        wp = torch.from_numpy(np.ascontiguousarray(routing["prefill_w"])).to(dev)
        outp = torch.empty((L, Tp, H), dtype=torch.bfloat16, device=dev)

    def cold():
        torch.cuda.synchronize()
        m.reset_lru(-1, stream)
        runner.rewind()
        torch.cuda.synchronize()
        m.reset_stats()

    def chunk():
        for l in range(L):
            m.forward(l, xp, idsp[l], wp[l], outp[l], stream=stream)

    cold()
    if prefill:
        chunk()
    runner.run(warmup)
    cold()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    if prefill:
        chunk()
    ev[1].record(stream)
    got = {}
    for s in range(steps):
        runner.run(1)
        if s in (0, steps - 1):
            got[s] = out.clone()
    ev[2].record(stream)
    torch.cuda.synchronize()
    st = m.stats()
    chunk_ms, ms = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])
    got = {s: harness.bf16_bits(v) for s, v in got.items()}
    got_p = harness.bf16_bits(outp) if prefill else None
    captured = runner.captured
    del runner
    m.close()

    S_alg, _ = pe.pe_expert_bytes(wl.wtype, H, wl.inter)
    misses = distinct = waves = 0
    for l in range(L):
        sim = LayerLRU(wl.experts, wl.resident)
        step_ids = ([routing["prefill_ids"][l].ravel()] if prefill else []) + \
                   [routing["decode_ids"][s, l].ravel() for s in range(steps)]
        for v in step_ids:
            wv = sim.step(v)
            misses += sum(u.count for u in wv)
            waves += len(wv)
            distinct += len(set(v.tolist()))
    counts_ok = (misses, distinct, waves) == (st["page_ins"], st["distinct"], st["waves"])
    # the outputs' sample (copied out after the step that made them, outside the window's timing)
    worst = 0.0
    for l in sorted({0, L - 1}):
        canon = {}

        def expert(e):
            if e not in canon:
                canon[e] = formats.dequant_expert(wl.wtype, *synth.expert_tensors(wl, l, e))
            return canon[e]
        for s in sorted(got):
            xs = formats.bf16_to_f32(synth.hidden_states(wl, s, B))
            ref = moe.moe_layer(xs, routing["decode_ids"][s, l], routing["decode_w"][s, l], expert)
            g = harness.bf16_to_f32(got[s][l])
            worst = max(worst, float(np.abs(g - ref).max() / np.abs(ref).max()))
        if prefill:
            rows = [0, Tp // 2, Tp - 1]
            xr = formats.bf16_to_f32(synth.hidden_states(wl, -1, Tp))[rows]
            ref = moe.moe_layer(xr, routing["prefill_ids"][l][rows], routing["prefill_w"][l][rows], expert)
            g = harness.bf16_to_f32(got_p[l])[rows]
            worst = max(worst, float(np.abs(g - ref).max() / np.abs(ref).max()))
    tol = {"bf16": 1e-2, "fp8": 1e-2, "int4": 2e-2, "int8": 1e-2, "mxfp4": 1e-2}[wl.wtype]
    # the decode window's roofline: its share of distinct experts and page-ins
    # (the prefill chunk's are counted apart)
    Dd, Md = distinct, misses
    res = {"workload": name, "path": "captured" if captured else "host-planned", "steps": steps,
           "warmup": warmup, "dtype": DTYPES[wl.wtype], "batch": B, "resident": wl.resident}
    if prefill:
        sim_p = [LayerLRU(wl.experts, wl.resident) for _ in range(L)]
        Dp = sum(len(set(routing["prefill_ids"][l].ravel().tolist())) for l in range(L))
        Mp = sum(sum(u.count for u in sim_p[l].step(routing["prefill_ids"][l].ravel())) for l in range(L))
        roof_p = Dp * S_alg / (HBM_PEAK_GBS * 1e9) + Mp * S_alg / (link * 1e9)
        res["prefill"] = {"tokens": Tp, "ms": round(chunk_ms, 2), "tok_s": round(Tp / (chunk_ms / 1e3), 1),
                          "roof_ms": round(roof_p * 1e3, 2), "frac": round(roof_p * 1e3 / chunk_ms, 4)}
        Dd, Md = distinct - Dp, misses - Mp
    t_roof = Dd * S_alg / (HBM_PEAK_GBS * 1e9) + Md * S_alg / (link * 1e9)
    value = steps * B / (ms / 1e3)
    res.update({"value": round(value, 3), "unit": "tok/s", "ms_per_step": round(ms / steps, 4),
                "roof_tok_s": round(steps * B / t_roof, 2), "frac": round(value / (steps * B / t_roof), 4),
                "sample_parity": {"max_rel_err": worst, "tol": tol, "counts_match_simulator": counts_ok,
                                  "ok": bool(counts_ok and worst <= tol)}})
    log("%s (%s): %.1f tok/s, %.3f of its path roofline%s, parity %s" % (
        name, res["path"], value, res["frac"],
        (", prefill chunk %.1f ms (%.3f)" % (chunk_ms, res["prefill"]["frac"])) if prefill else "",
        "ok" if res["sample_parity"]["ok"] else "FAILED"))
    return res


MFMA_BF16_PEAK = 2.5e15        # MI355X dense bf16 MFMA, FLOP/s


def warm_prefill(wl, xp, idsp, wp, outp, stream):
    """The prefill chunk with every expert resident: an unpaged context (K = E,
    slot e holds expert e, no page-in), so the step is planning, the MFMA (and
    GEMV) expert kernels and the top-k sum.  Each expert kernel is set against
    its own roofline, the larger of its MFMA time at the bf16 peak and its HBM
    time for the bytes it must move once: gate/up reads D experts' gate/up
    weights and the chunk's x and writes h (bf16, one row per entry); down reads
    D experts' down weights and h and writes the merged fp32 row of every entry
    that the top-k sum then reads."""
    import torch

    import harness
    import host_paged_expert_amd as pe

    L = wl.layers
    m = harness.make_moe(wl, flags=pe.PE_FLAG_UNPAGED, max_tokens=wl.prefill_tokens)
    harness.load_store(m, wl, progress=L * wl.experts // 4)
    log("warm prefill: unpaged context loaded")

    def chunk():
        for l in range(L):
            m.forward(l, xp, idsp[l], wp[l], outp[l], stream=stream)
    chunk()
    torch.cuda.synchronize()
    times = []
    for _ in range(2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        chunk()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    m.reset_stats()
    m.set_timing(1)
    chunk()
    tm = m.timing()
    m.set_timing(0)
    st = m.stats()
    m.close()
    H, I = wl.hidden, wl.inter
    w13, w2, s13, s2 = part_bytes(wl.wtype, H, I)
    ent, D = st["entries"], st["distinct"]
    x_bytes = L * wl.prefill_tokens * H * 2          # the chunk's x, read once per layer
    h_bytes = ent * I * 2                            # h: written by gate/up, read by down
    merged_bytes = ent * H * 4                       # merged fp32 rows written by down
    out = {"ms": round(min(times), 2), "tok_s": round(wl.prefill_tokens / (min(times) / 1e3), 1), "distinct": D}
    for name, flops, wbytes in (("gate_up", ent * 2.0 * 2 * H * I, D * (w13 + s13) + x_bytes + h_bytes),
                                ("down", ent * 2.0 * H * I, D * (w2 + s2) + h_bytes + merged_bytes)):
        n, ms = tm[name]
        roof_ms = max(flops / MFMA_BF16_PEAK, wbytes / (HBM_PEAK_GBS * 1e9)) * 1e3
        out[name] = {"launches": n, "ms": round(ms, 3), "tflops": round(flops / (ms / 1e3) / 1e12, 1) if ms else None,
                     "roof_ms": round(roof_ms, 3), "frac": round(roof_ms / ms, 4) if ms else None,
                     "bound": "mfma" if flops / MFMA_BF16_PEAK > wbytes / (HBM_PEAK_GBS * 1e9) else "hbm"}
    log("warm prefill: %.1f ms for %d tokens; gate/up %.1f ms (%.3f of its roofline), down %.1f ms (%.3f)" % (
        out["ms"], wl.prefill_tokens, out["gate_up"]["ms"], out["gate_up"]["frac"] or 0, out["down"]["ms"],
        out["down"]["frac"] or 0))
    return out


def sweep(args):
    """Decode throughput against batch size at several K (the docs page's
    "Captured decode": batch x top_k <= K runs one device-planned captured
    wave, larger batches are host-planned; the blog measures the drop past
    K // top_k concurrent requests).  One context per K, loaded once; every
    point is timed from an empty slot table over the same number of steps."""
    import torch

    import harness
    import synth
    import host_paged_expert_amd as pe

    dev = "cuda:0"
    torch.cuda.init()
    Bs = [int(v) for v in args.sweep_batches.split(",")]
    Ks = [int(v) for v in args.sweep_resident.split(",")]
    steps = args.steps or 128
    warmup = max(0, min(args.warmup, steps))
    link = None
    for K in Ks:
        wl0 = synth.workload(args.workload, resident=K, batch=max(Bs), steps=steps)
        m = harness.make_moe(wl0, max_tokens=max(Bs))
        t0 = time.time()
        harness.load_store(m, wl0)
        log("sweep: K=%d context loaded in %.1fs" % (K, time.time() - t0))
        if link is None:
            link = max(pe.pe_link_probe(m.ctx, 1 << 30, 0, 5), pe.pe_link_probe(m.ctx, 1 << 30, 1, 5))
        S_alg, _ = pe.pe_expert_bytes(wl0.wtype, wl0.hidden, wl0.inter)
        stream = torch.cuda.current_stream()
        for B in Bs:
            wl = synth.workload(args.workload, resident=K, batch=B, steps=steps)
            routing = synth.routing_for(wl)
            x, ids, w = harness.decode_inputs(wl, routing, dev)
            out = torch.empty((wl.layers, B, wl.hidden), dtype=torch.bfloat16, device=dev)
            runner = harness.DecodeRunner(m, wl, x, ids, w, out, stream)

            def cold():
                torch.cuda.synchronize()
                m.reset_lru(-1, stream)
                runner.rewind()
                torch.cuda.synchronize()
                m.reset_stats()
            cold()
            runner.run(warmup)
            cold()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            runner.run(steps)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            st = m.stats()
            D, M = st["distinct"], st["page_ins"]
            t_roof = D * S_alg / (HBM_PEAK_GBS * 1e9) + M * S_alg / (link * 1e9)
            value = steps * B / (ms / 1e3)
            res = {"metric": "paged-MoE decode tok/s, 48-layer 128-expert top-8; HBM & page-in GB/s % peak",
                   "value": round(value, 3), "unit": "tok/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
                   "ms_per_step": round(ms / steps, 4), "higher_is_better": True, "scaling": "weak",
                   "vs_baseline": None, "dtype": DTYPES[wl.wtype],
                   "data": "synthetic",
                   "config": {"workload": "sweep:" + args.workload, "layers": wl.layers, "experts": wl.experts,
                              "top_k": wl.top_k, "resident": K, "hidden": wl.hidden, "inter": wl.inter,
                              "wtype": wl.wtype, "batch": B, "max_captured_batch": m.max_captured_batch,
                              "path": "captured" if runner.captured else "host-planned"},
                   "window": {"distinct": D, "page_ins": M, "waves": st["waves"],
                              "miss_rate": round(M / max(st["entries"], 1), 4)},
                   "roofline_path": {"model": "D*S/HBM + M*S/link", "link_gbs": round(link, 2),
                                     "roof_tok_s": round(steps * B / t_roof, 2),
                                     "frac": round(value / (steps * B / t_roof), 4)}}
            res["sample_parity"] = sweep_parity(m, wl, routing, runner, cold, st)
            log("sweep: K=%d batch %d (%s): %.1f tok/s, %.3f of roofline, %d waves, parity %s" % (
                K, B, res["config"]["path"], value, res["roofline_path"]["frac"], st["waves"],
                "ok" if res["sample_parity"]["ok"] else "FAILED"))
            print(json.dumps(res), flush=True)
            del runner
        m.close()


def sweep_parity(m, wl, routing, runner, cold, st):
    """One sweep point checked against the oracle: the window's page-in,
    distinct and wave counts against the LRU simulator, and the outputs of the
    first and last layer at the first and last step (from one more pass over
    the window, from an empty table) against the fp32 unpaged layer."""
    import numpy as np
    import torch

    import harness
    import synth
    from oracle import formats, moe
    from oracle.lru import LayerLRU

    L, S = wl.layers, wl.steps
    misses = distinct = waves = 0
    for l in range(L):
        sim = LayerLRU(wl.experts, wl.resident)
        for s in range(S):
            ids = routing["decode_ids"][s, l].ravel()
            w = sim.step(ids)
            misses += sum(v.count for v in w)
            waves += len(w)
            distinct += len(set(ids.tolist()))
    counts_ok = (misses, distinct, waves) == (st["page_ins"], st["distinct"], st["waves"])
    pick = sorted({0, S - 1})
    cold()
    got = {}
    for s in range(S):
        runner.run(1)
        if s in pick:
            got[s] = harness.bf16_bits(runner.out)
    torch.cuda.synchronize()
    worst = 0.0
    for s in pick:
        x = formats.bf16_to_f32(synth.hidden_states(wl, s, wl.batch))
        for l in sorted({0, L - 1}):
            ids, w = routing["decode_ids"][s, l], routing["decode_w"][s, l]
            canon = {int(e): synth.expert_tensors(wl, l, int(e)) for e in np.unique(ids)}
            ref = moe.moe_layer(x, ids, w, lambda e: formats.dequant_expert(wl.wtype, *canon[e]))
            g = harness.bf16_to_f32(got[s][l])
            worst = max(worst, float(np.abs(g - ref).max() / np.abs(ref).max()))
    tol = {"bf16": 1e-2, "fp8": 1e-2, "int4": 2e-2, "int8": 1e-2, "mxfp4": 1e-2}[wl.wtype]
    return {"pairs": len(pick) * len({0, L - 1}), "steps": pick, "max_rel_err": worst, "tol": tol,
            "counts_match_simulator": counts_ok, "ok": bool(counts_ok and worst <= tol)}


def cpu_baseline(wl, routing, steps, sample_steps, samples, M, D, has_prefill=False, budget_s=20.0):
    """The CPU oracle as it stands, on a bounded sample: the LRU simulator over the
    whole window, and the fp32 unpaged layer on (step, layer) pairs of a few evenly
    spaced steps until about `budget_s` seconds of oracle time are spent.  Expert
    tensors are generated untimed (they are inputs)."""
    import numpy as np
    import threadpoolctl

    import harness
    import synth
    from oracle import formats, moe
    from oracle.lru import LayerLRU

    L, B = wl.layers, wl.batch
    t0 = time.perf_counter()
    misses = distinct = 0
    for l in range(L):
        sim = LayerLRU(wl.experts, wl.resident)
        if has_prefill:
            sim.step(routing["prefill_ids"][l].ravel())
        for s in range(steps):
            ids = routing["decode_ids"][s, l].ravel()
            misses += sum(w.count for w in sim.step(ids))
            distinct += len(set(ids.tolist()))
    t_sim = time.perf_counter() - t0
    plan_ok = (misses == M and distinct == D)
    log("oracle LRU simulator: %d layer-steps in %.2fs, plans %s" % (L * steps, t_sim,
                                                                     "match" if plan_ok else "DIFFER"))
    # (step, layer) pairs, layer by layer so a cut-off sample still spans the
    # window's steps; a layer's expert tensors are generated once, untimed (they
    # are inputs), in parallel threads
    from concurrent.futures import ThreadPoolExecutor
    t_moe, worst, done = 0.0, 0.0, []
    wall0 = time.perf_counter()
    xs = {s: formats.bf16_to_f32(synth.hidden_states(wl, s, B)) for s in sample_steps}
    pool = ThreadPoolExecutor(harness.host_threads())
    for l in range(L):
        if t_moe >= budget_s or time.perf_counter() - wall0 >= 4 * budget_s:
            break
        used = sorted({int(e) for s in sample_steps for e in np.unique(routing["decode_ids"][s, l])})
        canon = dict(zip(used, pool.map(lambda e: synth.expert_tensors(wl, l, e), used)))
        for s in sample_steps:
            if t_moe >= budget_s:
                break
            ids, w = routing["decode_ids"][s, l], routing["decode_w"][s, l]
            t1 = time.perf_counter()
            ref = moe.moe_layer(xs[s], ids, w, lambda e: formats.dequant_expert(wl.wtype, *canon[e]))
            t_moe += time.perf_counter() - t1
            done.append((s, l))
            if s in samples:
                got = harness.bf16_to_f32(samples[s][l])
                worst = max(worst, float(np.abs(got - ref).max() / np.abs(ref).max()))
        log("oracle: %d (step, layer) pairs, %.1fs of oracle time" % (len(done), t_moe))
    pool.shutdown()
    # one thread: the first (step, layer) pairs again, BLAS limited to one thread,
    # for about a quarter of the budget
    t_one, one = 0.0, 0
    with threadpoolctl.threadpool_limits(1):
        for (s, l) in done:
            if t_one >= budget_s / 4:
                break
            canon = {int(e): synth.expert_tensors(wl, l, int(e)) for e in np.unique(routing["decode_ids"][s, l])}
            t1 = time.perf_counter()
            moe.moe_layer(xs[s], routing["decode_ids"][s, l], routing["decode_w"][s, l],
                          lambda e: formats.dequant_expert(wl.wtype, *canon[e]))
            t_one += time.perf_counter() - t1
            one += 1
    log("oracle, one thread: %d (step, layer) pairs in %.2fs" % (one, t_one))
    pre_worst, pre_cpu = None, None
    if has_prefill and "prefill" in samples:
        # the whole prefill chunk through as many layers as the budget allows
        # (the first and the last at least), timed; expert tensors untimed
        xp = formats.bf16_to_f32(synth.hidden_states(wl, -1, wl.prefill_tokens))
        pre_worst, t_pre, pre_layers = 0.0, 0.0, []
        order = [0, L - 1] + [l for l in range(1, L - 1)]
        pool = ThreadPoolExecutor(harness.host_threads())
        for l in order:
            if len(pre_layers) >= 2 and t_pre >= budget_s:
                break
            ids, w = routing["prefill_ids"][l], routing["prefill_w"][l]
            used = [int(e) for e in np.unique(ids)]
            canon = dict(zip(used, pool.map(lambda e: synth.expert_tensors(wl, l, e), used)))
            t1 = time.perf_counter()
            ref = moe.moe_layer(xp, ids, w, lambda e: formats.dequant_expert(wl.wtype, *canon[e]))
            t_pre += time.perf_counter() - t1
            pre_layers.append(l)
            got = harness.bf16_to_f32(samples["prefill"][l])
            pre_worst = max(pre_worst, float(np.abs(got - ref).max() / np.abs(ref).max()))
            log("oracle prefill layer %d: %.1fs of oracle time so far" % (l, t_pre))
        pool.shutdown()
        log("oracle prefill, %d layers: max rel err %.2e" % (len(pre_layers), pre_worst))
        pre_cpu = {"value": round(wl.prefill_tokens / (t_pre / len(pre_layers) * L), 3), "unit": "tok/s",
                   "sample": "the whole %d-token prefill chunk through layers %s (of %d), fp32 unpaged oracle" % (
                       wl.prefill_tokens, pre_layers, L)}
    threads = max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1)
    tokens = B * len(done) / L                      # a token passes all L layers
    t_total = t_moe + t_sim * (len(done) / L) / steps
    log("oracle MoE: %d (step, layer) pairs in %.2fs" % (len(done), t_moe))
    tol = {"bf16": 1e-2, "fp8": 1e-2, "int4": 2e-2, "int8": 1e-2, "mxfp4": 1e-2}[wl.wtype]
    cpu = {"value": round(tokens / t_total, 5) if t_total > 0 else None, "unit": "tok/s", "cores": threads,
           "kind": "oracle",
           "sample": "%d (step, layer) pairs from decode steps %s (batch %d) through the fp32 unpaged oracle, "
                     "plus the LRU simulator over all %d steps x %d layers; host %s, %d cpus, BLAS on %d threads"
                     % (len(done), sample_steps, B, steps, L, cpu_model(), os.cpu_count(), threads),
           "single_thread": {"value": round(B * one / L / t_one, 5) if t_one > 0 else None, "unit": "tok/s",
                             "cores": 1, "sample": "the first %d of those (step, layer) pairs, BLAS on one thread"
                             % one}}
    if pre_cpu:
        cpu["prefill"] = pre_cpu
    parity = {"pairs": len(done), "max_rel_err": worst, "tol": tol,
              "ok": bool(worst <= tol and (pre_worst is None or pre_worst <= tol)) if samples else None,
              "plans_match_simulator": plan_ok}
    if pre_worst is not None:
        parity["prefill_layers"] = pre_layers
        parity["prefill_max_rel_err"] = pre_worst
    return cpu, parity


PMC_KERNELS = ("step_a_kernel", "down_sum_kernel", "wave_a_kernel", "gemv_down_kernel", "page_in_kernel")
# The down launches of a host-planned step: the fused down projection + top-k
# sum when the step is one wave, the plain down kernel per wave otherwise.
HOST_DOWN = "down_sum_kernel+gemv_down_kernel"


def source_hash():
    """Hash of the library's kernel and orchestration sources: memory-traffic
    counters taken on one build stay valid only while this is unchanged."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "host_paged_expert_amd", "csrc", "*"))):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def alg_bytes(kernel, wtype, hidden, inter, D, M, launches):
    """Algorithmic memory bytes (reads + writes) per launch of a kernel over a
    window with D distinct and M paged-in experts: the page-in launches read M
    expert blobs over the link, write them into slots and read the resident
    experts' gate/up weights; the down launches read every distinct expert's
    down weights.  Activations (< 1%) are left out."""
    w13, w2, s13, s2 = part_bytes(wtype, hidden, inter)
    blob = w13 + w2 + s13 + s2
    if kernel in ("step_a_kernel", "wave_a_kernel"):
        tot = 2 * M * blob + (D - M) * (w13 + s13)
    elif kernel == "page_in_kernel":
        tot = 2 * M * blob
    else:
        tot = D * (w2 + s2)
    return tot / max(launches, 1)


def pmc_summary(fetch_csv, write_csv, bench_json, out_json):
    """Per-launch memory traffic of the path's kernels from two rocprofv3 --pmc
    runs of the same bench command (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch), each scaled by what the same counter reads for a plain 256 MiB
    device-to-device copy run first (--copy-reference 256), against the
    algorithmic bytes of that run's window (bench_json: its JSON line)."""
    import collections
    import csv

    def load(path):
        agg = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return agg
    f, w = load(fetch_csv), load(write_csv)
    ref = 256 * 1024.0
    fs = ref / max(f["__amd_rocclr_copyBuffer"])
    ws = ref / max(w["__amd_rocclr_copyBuffer"])
    run = json.loads(open(bench_json).read().strip().splitlines()[-1])
    cfg, win = run["config"], run["window"]
    out = {"source_sha256_16": source_hash(), "workload": cfg["workload"], "fetch_scale": round(fs, 4),
           "write_scale": round(ws, 4), "window": {"distinct": win["distinct"], "page_ins": win["page_ins"]},
           "kernels": {}}
    if cfg.get("path") == "host-planned" and cfg.get("pagein") == "kernel":
        groups = [("wave_a_kernel", ("wave_a_kernel",)), (HOST_DOWN, ("down_sum_kernel", "gemv_down_kernel"))]
    else:
        groups = [(name, (name,)) for name in PMC_KERNELS]
    for name, members in groups:
        keys = [k for k in f if any(m in k for m in members)]
        if not keys:
            continue
        fv = [v for k in keys for v in f[k]]
        wv = [v for k in keys for v in w.get(k, [])]
        rd = sum(fv) / len(fv) * fs * 1024
        wr = sum(wv) / max(len(wv), 1) * ws * 1024
        alg = alg_bytes(name, cfg["wtype"], cfg["hidden"], cfg["inter"], win["distinct"], win["page_ins"], len(fv))
        out["kernels"][name] = {"launches": len(fv), "read_bytes_per_launch": round(rd),
                                "write_bytes_per_launch": round(wr), "alg_bytes_per_launch": round(alg),
                                "traffic_over_alg": round((rd + wr) / alg, 4) if alg else None}
    json.dump(out, open(out_json, "w"), indent=1)
    print(json.dumps(out, indent=1))


def traffic_for(kernel, workload, alg_per_launch):
    """Read + write bytes per launch implied by the committed counter summary
    for this workload (its traffic / algorithmic ratio times this run's
    algorithmic bytes), or None if there is none or the sources changed."""
    try:
        t = json.load(open(os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)))
    except (OSError, ValueError):
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k or t.get("source_sha256_16") != source_hash() or not k.get("traffic_over_alg"):
        return None
    return round(alg_per_launch * k["traffic_over_alg"])


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
