"""bench.py's host-side accounting on the CPU: expert part sizes, algorithmic
bytes per launch, and the memory-traffic summary of two counter runs (here
from synthetic counter files; no GPU)."""
import csv
import json

import pytest

import bench
from oracle import sizes


@pytest.mark.parametrize("wtype,H,I", [("bf16", 2048, 768), ("fp8", 2048, 768), ("int4", 2048, 768),
                                       ("int8", 2048, 768), ("mxfp4", 2880, 2880), ("fp8", 384, 640)])
def test_part_bytes_sum_to_the_oracle_expert_size(wtype, H, I):
    assert sum(bench.part_bytes(wtype, H, I)) == sizes.expert_bytes(wtype, H, I)


def test_algorithmic_bytes_per_launch():
    w13, w2, s13, s2 = bench.part_bytes("fp8", 2048, 768)
    S = w13 + w2 + s13 + s2
    D, M, n = 10, 4, 3
    # page-in launches: M blobs over the link and into slots, plus the resident experts' gate/up
    assert bench.alg_bytes("step_a_kernel", "fp8", 2048, 768, D, M, n) == (2 * M * S + (D - M) * (w13 + s13)) / n
    assert bench.alg_bytes("wave_a_kernel", "fp8", 2048, 768, D, M, n) == (2 * M * S + (D - M) * (w13 + s13)) / n
    assert bench.alg_bytes("page_in_kernel", "fp8", 2048, 768, D, M, n) == 2 * M * S / n
    # down launches: every distinct expert's down weights once
    for k in ("down_sum_kernel", "gemv_down_kernel", bench.HOST_DOWN):
        assert bench.alg_bytes(k, "fp8", 2048, 768, D, M, n) == D * (w2 + s2) / n


def _counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Value"])
        for name, v in rows:
            w.writerow([name, v])


def _summary(tmp_path, cfg, fetch, write, window):
    _counters(tmp_path / "f.csv", [("__amd_rocclr_copyBuffer", 131072.0)] + fetch)   # a 256 MiB copy reads as half
    _counters(tmp_path / "w.csv", [("__amd_rocclr_copyBuffer", 262144.0)] + write)
    (tmp_path / "b.json").write_text("[bench] log line\n" + json.dumps({"config": cfg, "window": window}) + "\n")
    bench.pmc_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "b.json"),
                      str(tmp_path / "o.json"))
    return json.loads((tmp_path / "o.json").read_text())


def test_traffic_summary_of_a_captured_workload(tmp_path):
    cfg = dict(workload="x", wtype="bf16", hidden=2048, inter=768, path="captured", pagein="kernel")
    out = _summary(tmp_path, cfg,
                   [("void pe::step_a_kernel<0, 1>(...)", 1000.0), ("void pe::step_a_kernel<0, 1>(...)", 3000.0),
                    ("void pe::down_sum_kernel<0, 1, true>(...)", 100.0)],
                   [("void pe::step_a_kernel<0, 1>(...)", 500.0), ("void pe::step_a_kernel<0, 1>(...)", 700.0),
                    ("void pe::down_sum_kernel<0, 1, true>(...)", 4.0)],
                   dict(distinct=16, page_ins=2))
    assert out["fetch_scale"] == 2.0 and out["write_scale"] == 1.0
    a, b = out["kernels"]["step_a_kernel"], out["kernels"]["down_sum_kernel"]
    assert a["launches"] == 2 and a["read_bytes_per_launch"] == 2000 * 2 * 1024
    assert a["write_bytes_per_launch"] == 600 * 1024
    alg = bench.alg_bytes("step_a_kernel", "bf16", 2048, 768, 16, 2, 2)
    assert a["alg_bytes_per_launch"] == round(alg)
    assert a["traffic_over_alg"] == round((2000 * 2 * 1024 + 600 * 1024) / alg, 4)
    assert b["launches"] == 1 and b["read_bytes_per_launch"] == 100 * 2 * 1024


def test_traffic_summary_groups_a_host_planned_steps_down_launches(tmp_path):
    cfg = dict(workload="x", wtype="int4", hidden=2048, inter=768, path="host-planned", pagein="kernel")
    out = _summary(tmp_path, cfg,
                   [("void pe::wave_a_kernel<2, 4>(...)", 900.0), ("void pe::down_sum_kernel<2, 4, true>(...)", 100.0),
                    ("void pe::gemv_down_kernel<2, 4>(...)", 300.0), ("pe::topk_sum_kernel(...)", 7.0)],
                   [("void pe::wave_a_kernel<2, 4>(...)", 90.0), ("void pe::down_sum_kernel<2, 4, true>(...)", 1.0),
                    ("void pe::gemv_down_kernel<2, 4>(...)", 3.0)],
                   dict(distinct=24, page_ins=5))
    assert set(out["kernels"]) == {"wave_a_kernel", bench.HOST_DOWN}
    dn = out["kernels"][bench.HOST_DOWN]
    assert dn["launches"] == 2 and dn["read_bytes_per_launch"] == 200 * 2 * 1024
    assert dn["alg_bytes_per_launch"] == round(bench.alg_bytes(bench.HOST_DOWN, "int4", 2048, 768, 24, 5, 2))


def test_committed_traffic_applies_only_to_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    t = {"source_sha256_16": bench.source_hash(), "kernels": {"step_a_kernel": {"traffic_over_alg": 1.25}}}
    (tmp_path / "profiles" / "traffic_w.json").write_text(json.dumps(t))
    assert bench.traffic_for("step_a_kernel", "w", 1000.0) == 1250
    assert bench.traffic_for("down_sum_kernel", "w", 1000.0) is None
    assert bench.traffic_for("step_a_kernel", "other", 1000.0) is None
    t["source_sha256_16"] = "0" * 16
    (tmp_path / "profiles" / "traffic_w.json").write_text(json.dumps(t))
    assert bench.traffic_for("step_a_kernel", "w", 1000.0) is None


def test_other_workloads_run_only_when_no_workload_is_named(monkeypatch):
    def args_of(argv):
        monkeypatch.setattr("sys.argv", ["bench.py"] + argv)
        return bench.parse()
    default = bench.others_for(args_of([]), [])
    assert default == [n for n in bench.OTHER_WORKLOADS]
    assert "decode_bf16_k40_b1" not in default
    argv = ["--workload", "decode_fp8_k40_b4"]
    assert bench.others_for(args_of(argv), argv) == []
    argv = ["--workload=decode_bf16_k40_b1", "--steps", "16"]
    assert bench.others_for(args_of(argv), argv) == []
    argv = ["--others", "decode_int4_k26_b4,decode_bf16_k40_b1"]
    assert bench.others_for(args_of(argv), argv) == ["decode_int4_k26_b4"]
    argv = ["--dma"]
    assert bench.others_for(args_of(argv), argv) == []
    synth = pytest.importorskip("synth")
    for n in bench.OTHER_WORKLOADS:
        assert n in synth.WORKLOADS
