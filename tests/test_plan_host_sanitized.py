"""The host wave planner (csrc/pe_plan_host.cpp), built on its own with g++
under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU), over random
traces: no memory or undefined-behaviour error, and every step's plans, slot
map and LRU state equal the oracle's simulator; the work lists hold every
valid entry once, grouped by expert in ascending entry order."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.lru import LayerLRU

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "tests", "native", "plan_host_driver.cpp"),
       os.path.join(ROOT, "host_paged_expert_amd", "csrc", "pe_plan_host.cpp")]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("san") / "plan_host_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g"] + SAN + SRC + ["-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def _run(driver, E, K, k, max_tokens, trace):
    lines = ["%d %d %d %d %d" % (E, K, k, max_tokens, len(trace))]
    for ids in trace:
        lines.append("%d %s" % (len(ids) // k, " ".join(str(int(v)) for v in ids)))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env,
                         timeout=120)
    assert res.returncode == 0, res.stderr[-4000:]
    assert "runtime error" not in res.stderr and "Sanitizer" not in res.stderr, res.stderr[-4000:]
    return res.stdout.splitlines()


def _ints(part):
    return [int(v) for v in part.split()]


@pytest.mark.parametrize("E,K,k,max_tokens", [(8, 2, 2, 3), (16, 5, 3, 6), (128, 26, 8, 8), (128, 92, 8, 64),
                                              (1024, 32, 8, 9), (64, 7, 4, 40)])
def test_sanitized_host_planner_matches_simulator(driver, E, K, k, max_tokens):
    rng = np.random.default_rng(E + 7 * K + 31 * k)
    trace = []
    for s in range(60):
        T = int(rng.integers(1, max_tokens + 1))
        rows = [rng.choice(E, k, replace=False) for _ in range(T)]
        ids = np.concatenate(rows).astype(np.int64)
        if s % 7 == 3:
            ids[rng.integers(0, ids.size)] = -1 if s % 2 else E + 5     # an invalid id
        if s % 11 == 5:
            ids[:k] = ids[0]                                           # one expert at every position
        trace.append(ids)
    out = _run(driver, E, K, k, max_tokens, trace)
    assert len(out) == len(trace)
    sim = LayerLRU(E, K)
    for ids, line in zip(trace, out):
        parts = line.split("|")
        rc, nw = _ints(parts[0])
        waves = sim.step(ids)
        assert rc == 0 and nw == len(waves)
        for w, wv in enumerate(waves):
            v = _ints(parts[1 + w])
            c = v[0]
            assert c == wv.count
            assert (v[1:1 + c], v[1 + c:1 + 2 * c], v[1 + 2 * c:1 + 3 * c]) == \
                (wv.plan_experts, wv.plan_slots, wv.evicted)
        rest = parts[1 + nw:]
        want = [next((wv.slot_of[e] for wv in waves if e in wv.slot_of), -1) if 0 <= e < E else -1
                for e in (int(v) for v in ids)]
        assert _ints(rest[0]) == want
        assert _ints(rest[1]) == sim.slot_expert and _ints(rest[2]) == sim.last_use and _ints(rest[3]) == [sim.tick]
        entries, used_off = _ints(rest[4]), _ints(rest[5])
        valid = [i for i, e in enumerate(ids) if 0 <= e < E]
        assert sorted(entries) == valid
        for u in range(len(used_off) - 1):
            seg = entries[used_off[u]:used_off[u + 1]]
            assert seg == sorted(seg) and len({int(ids[i]) for i in seg}) == 1


def test_sanitized_host_planner_at_the_most_waves(driver):
    """Steps whose entries are all distinct experts need the most waves the
    layout holds (ceil(max_tokens * k / K)); the arrays are sized for exactly
    that, and the sanitizers see every access."""
    E, K, k, T = 64, 4, 4, 3
    trace = [np.arange(12), np.arange(12, 24), np.arange(5, 17), np.arange(4)]
    out = _run(driver, E, K, k, T, trace)
    sim = LayerLRU(E, K)
    for ids, line in zip(trace, out):
        rc, nw = _ints(line.split("|")[0])
        assert rc == 0 and nw == len(sim.step(ids))
    assert [int(l.split()[1]) for l in out] == [3, 3, 3, 1]
