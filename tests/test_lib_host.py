"""libpe on the CPU: it loads, exports every symbol include/pe.h declares, and
its host-only logic (expert sizes, the host wave planner, argument checks)
agrees with the oracle.  No kernel runs here."""
import os
import re

import numpy as np
import pytest

import host_paged_expert_amd as pe
from oracle import sizes
from oracle.lru import LayerLRU

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "pe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(pe_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 17
    L = pe.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(pe.SIGNATURES)


@pytest.mark.parametrize("wtype", ["bf16", "fp8", "int4", "int8", "mxfp4"])
@pytest.mark.parametrize("H,I", [(2048, 768), (256, 128), (1024, 512)])
def test_expert_bytes_match_oracle(wtype, H, I):
    alg, copied = pe.pe_expert_bytes(wtype, H, I)
    assert alg == sizes.expert_bytes(wtype, H, I)
    assert copied >= alg and copied - alg < 4 * 256 and copied % 256 == 0


def test_expert_bytes_pages_sizes():
    assert pe.pe_expert_bytes("int4", 2048, 768)[0] == 2_433_024     # the blog's 2.43 MB
    assert pe.pe_expert_bytes("fp8", 2048, 768)[0] == 4_719_744      # the blog's 4.72 MB


def test_expert_bytes_rejects_bad_shapes():
    with pytest.raises(pe.PEError):
        pe.pe_expert_bytes("fp8", 2048, 700)
    with pytest.raises(pe.PEError):
        pe.pe_expert_bytes("int4", 2880, 2880)          # group-128 formats need multiples of 128
    with pytest.raises(pe.PEError):
        pe.pe_expert_bytes("mxfp4", 2880 + 32, 2880)    # MXFP4 needs multiples of 64
    assert pe.pe_expert_bytes("mxfp4", 2880, 2880)[0] == sizes.expert_bytes("mxfp4", 2880, 2880)
    with pytest.raises(pe.PEError):
        pe.pe_expert_bytes(7, 2048, 768)


def test_strerror_and_last_error():
    assert pe.pe_strerror(pe.PE_ERR_NOT_CAPTURABLE).startswith("host-planned")
    assert pe.pe_strerror(12345) == "unknown status"
    with pytest.raises(pe.PEError) as ei:
        pe.pe_expert_bytes("int4", -1, 768)
    assert "positive" in pe.pe_last_error()
    assert ei.value.code == pe.PE_ERR_INVALID_ARG


def _sim_state(sim):
    return np.array(sim.slot_expert, np.int32), np.array(sim.last_use, np.uint32), sim.tick


def _run_trace(E, K, k, trace):
    sim = LayerLRU(E, K)
    se, lu, tick = np.full(K, -1, np.int32), np.zeros(K, np.uint32), 1
    for ids in trace:
        T = len(ids) // k
        max_waves = -(-min(T * k, E) // K)
        r = pe.pe_plan_host(E, K, k, ids, se, lu, tick, max_waves)
        waves = sim.step(ids)
        assert len(r["waves"]) == len(waves)
        for g, w in zip(r["waves"], waves):
            assert g["count"] == w.count
            assert g["experts"].tolist() == w.plan_experts
            assert g["slots"].tolist() == w.plan_slots
            assert g["evicted"].tolist() == w.evicted
        se, lu, tick = r["slot_expert"], r["last_use"], r["tick"]
        s_se, s_lu, s_tick = _sim_state(sim)
        assert np.array_equal(se, s_se) and np.array_equal(lu, s_lu) and tick == s_tick
        # slot map: the slot of each entry's expert in its wave, -1 for invalid ids
        want = [next((w.slot_of[e] for w in waves if e in w.slot_of), -1) if 0 <= e < E else -1 for e in ids]
        assert r["slot_of"].tolist() == want


@pytest.mark.parametrize("E,K,k,T", [(8, 4, 2, 1), (8, 2, 2, 3), (16, 5, 3, 4), (128, 40, 8, 1),
                                     (128, 26, 8, 4), (128, 92, 8, 64), (64, 7, 4, 9)])
def test_host_planner_matches_simulator(E, K, k, T):
    rng = np.random.default_rng(E * 1000 + K * 10 + T)
    trace = []
    for s in range(80):
        tt = int(rng.integers(1, T + 1))
        trace.append(np.concatenate([rng.choice(E, k, replace=False) for _ in range(tt)]).astype(np.int32))
    _run_trace(E, K, k, trace)


def test_host_planner_ignores_invalid_ids():
    trace = [np.array([3, -1, 9, 2], np.int32), np.array([8, 8, 5, 100], np.int32)]
    _run_trace(8, 3, 2, trace)


def test_host_planner_rejects_too_few_waves():
    with pytest.raises(pe.PEError):
        pe.pe_plan_host(16, 2, 2, np.arange(8, dtype=np.int32), np.full(2, -1), np.zeros(2), 1, 2)


def test_create_validates_before_touching_the_gpu():
    # invalid configurations are rejected with a message, whatever the machine has
    for args in [dict(num_resident=1), dict(num_resident=9), dict(top_k=0), dict(wtype=5),
                 dict(hidden=100, wtype="fp8"), dict(max_tokens=0), dict(flags=64)]:
        kw = dict(num_layers=1, num_experts=8, top_k=2, num_resident=4, hidden=64, inter=128, max_tokens=4)
        kw.update(args)
        with pytest.raises(pe.PEError) as ei:
            pe.pe_create(**kw)
        assert ei.value.code == pe.PE_ERR_INVALID_ARG


def test_suggest_k_matches_sizing_rule_and_docs_example():
    """The docs' "Choosing K" rule: per-slot bytes = blob bytes x MoE layers."""
    slot = sizes.slot_bytes("int4", 2048, 768, 48)
    assert pe.pe_suggest_k("int4", 2048, 768, 48, 128, 8, 92 * slot) == 92
    assert pe.pe_suggest_k("int4", 2048, 768, 48, 128, 8, 92 * slot - 1) == 91
    assert pe.pe_suggest_k("bf16", 2048, 768, 48, 128, 8, 1e15) == 128
    for budget in (1e9, 5e9, 20e9, 60e9):
        want = sizes.suggest_k(budget, sizes.slot_bytes("fp8", 2048, 768, 48), 128)
        _, copied = pe.pe_expert_bytes("fp8", 2048, 768)
        got = pe.pe_suggest_k("fp8", 2048, 768, 48, 128, 8, budget) if want >= 8 else None
        if got is not None:
            assert abs(got - want) <= 1 and got == min(128, int(budget // (copied * 48)))
    with pytest.raises(pe.PEError):
        pe.pe_suggest_k("bf16", 2048, 768, 48, 128, 8, 1e9)       # fewer than top_k slots


def _header_text():
    src = open(os.path.join(ROOT, "include", "pe.h")).read()
    return re.sub(r"/\*.*?\*/", "", src, flags=re.S)


def test_binding_constants_match_the_header():
    defs = dict(re.findall(r"^#define\s+(PE_\w+)\s+(-?\d+)u?\s*$", _header_text(), flags=re.M))
    names = [n for n in defs if n.startswith(("PE_OK", "PE_ERR_", "PE_W_", "PE_FLAG_"))]
    assert len(names) >= 15
    for n in names:
        assert getattr(pe, n) == int(defs[n]), n
    stages = sorted((int(v), n) for n, v in defs.items() if n.startswith("PE_STAGE_"))
    assert [n[len("PE_STAGE_"):].lower() for _, n in stages] == list(pe.STAGES)
    assert int(defs["PE_NUM_STAGES"]) == len(pe.STAGES)


def _struct_fields(name):
    body = re.search(r"typedef struct \{((?:(?!typedef struct).)*?)\}\s*" + name + r";", _header_text(),
                     flags=re.S).group(1)
    return re.findall(r"^\s*(int|unsigned|uint64_t)\s+(\w+);", body, flags=re.M)


def test_binding_structs_match_the_header():
    import ctypes
    from host_paged_expert_amd import _binding
    ct = {"int": ctypes.c_int, "unsigned": ctypes.c_uint, "uint64_t": ctypes.c_uint64}
    for name, cls in (("pe_config", _binding.pe_config), ("pe_stats", _binding.pe_stats)):
        want = [(f, ct[t]) for t, f in _struct_fields(name)]
        assert len(want) >= 9, name
        assert list(cls._fields_) == want, name
