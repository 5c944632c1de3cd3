"""Generators behind `synth`: weights, hidden states and routing.

Bulk normal draws and the synthetic quantisers run in `gen.c` (built into
`libsynth.so` with gcc); routing is small and uses numpy.
"""
import ctypes
import os
import subprocess
import threading

import numpy as np

from .workloads import Workload

MASTER_SEED = 0
WEIGHT_SIGMA = 0.02
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None
_lib_lock = threading.Lock()


def build_lib(force: bool = False) -> str:
    """Compile gen.c into libsynth.so next to it (gcc, -O3)."""
    src = os.path.join(_HERE, "gen.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-Wall", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _L():
    global _lib
    if _lib is None:
        with _lib_lock:
            if _lib is None:
                if not os.path.exists(_LIB_PATH):
                    build_lib()
                lib = ctypes.CDLL(_LIB_PATH)
                u64, sz, f32, vp, i32 = ctypes.c_uint64, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p, ctypes.c_int
                lib.synth_mix64.argtypes = [u64]
                lib.synth_mix64.restype = u64
                lib.synth_normal.argtypes = [u64, sz, f32, vp]
                lib.synth_normal_bf16.argtypes = [u64, sz, f32, vp]
                lib.synth_round_bf16.argtypes = [vp, sz, vp]
                lib.synth_f16_from_f32.argtypes = [vp, sz, vp]
                lib.synth_e4m3_from_f32.argtypes = [vp, sz, vp]
                lib.synth_quant_fp8_b128.argtypes = [vp, i32, i32, vp, vp]
                lib.synth_quant_int4_g128.argtypes = [vp, i32, i32, vp, vp]
                lib.synth_quant_int8_g128.argtypes = [vp, i32, i32, vp, vp]
                lib.synth_quant_mxfp4_b32.argtypes = [vp, i32, i32, vp, vp]
                _lib = lib
    return _lib


_M64 = (1 << 64) - 1


def _mix64(z: int) -> int:
    """SplitMix64 output function on a Python int (same as synth_mix64)."""
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def _key(*parts) -> int:
    k = _mix64(0x5EED0F5EED ^ MASTER_SEED)
    for p in parts:
        if isinstance(p, str):
            p = int.from_bytes(p.encode(), "little") & _M64
        k = _mix64(k ^ (int(p) & _M64))
    return k


def normal(key: int, n: int, sigma: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    _L().synth_normal(key, n, sigma, out.ctypes.data)
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _L().synth_round_bf16(x.ctypes.data, x.size, out.ctypes.data)
    return out


def f16_from_f32(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _L().synth_f16_from_f32(x.ctypes.data, x.size, out.ctypes.data)
    return out


def e4m3_from_f32(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    _L().synth_e4m3_from_f32(x.ctypes.data, x.size, out.ctypes.data)
    return out


# ---------------------------------------------------------------- weights

def expert_key(hidden: int, inter: int, layer: int, expert: int, tensor: str) -> int:
    """Stream key of one expert tensor ("w13" or "w2"); shared by all formats,
    so bf16, FP8 and int4 experts quantise the same fp32 draws."""
    return _key("expert", hidden, inter, layer, expert, tensor)


def expert_draws(hidden: int, inter: int, layer: int, expert: int):
    """fp32 N(0, 0.02^2) draws: W13 [2I, H] (gate rows 0..I-1, up rows I..2I-1), W2 [H, I]."""
    w13 = normal(expert_key(hidden, inter, layer, expert, "w13"), 2 * inter * hidden, WEIGHT_SIGMA)
    w2 = normal(expert_key(hidden, inter, layer, expert, "w2"), hidden * inter, WEIGHT_SIGMA)
    return w13.reshape(2 * inter, hidden), w2.reshape(hidden, inter)


def expert_tensors(wl: Workload, layer: int, expert: int):
    """Canonical tensors of one expert in the workload's format.

    bf16: (W13 u16 [2I,H], W2 u16 [H,I], None, None)            bf16 bits, RNE of the draws
    fp8:  (Q13 u8 [2I,H], Q2 u8 [H,I], S13 f32 [2I/128,H/128], S2 f32 [H/128,I/128])
          e4m3fn codes and per-128x128-block fp32 multipliers
    int4: (Q13 u8 [2I,H/2], Q2 u8 [H,I/2], S13 u16 [2I,H/128], S2 u16 [H,I/128])
          nibbles q (w = (q-8)*s; element 2i in the low nibble of byte i), fp16 scale bits
    int8: (Q13 u8 [2I,H], Q2 u8 [H,I], S13 u16 [2I,H/128], S2 u16 [H,I/128])
          bytes q (w = (q-128)*s), fp16 scale bits
    mxfp4: (Q13 u8 [2I,H/2], Q2 u8 [H,I/2], S13 u8 [2I,H/32], S2 u8 [H,I/32])
          E2M1 codes packed like int4, E8M0 block scales (w = e2m1(q) * 2^(s-127))
    """
    H, I = wl.hidden, wl.inter
    L = _L()
    if wl.wtype == "bf16":
        w13 = np.empty((2 * I, H), np.uint16)
        w2 = np.empty((H, I), np.uint16)
        L.synth_normal_bf16(expert_key(H, I, layer, expert, "w13"), w13.size, WEIGHT_SIGMA, w13.ctypes.data)
        L.synth_normal_bf16(expert_key(H, I, layer, expert, "w2"), w2.size, WEIGHT_SIGMA, w2.ctypes.data)
        return w13, w2, None, None
    f13, f2 = expert_draws(H, I, layer, expert)
    if wl.wtype == "fp8":
        q13 = np.empty((2 * I, H), np.uint8)
        q2 = np.empty((H, I), np.uint8)
        s13 = np.empty((2 * I // 128, H // 128), np.float32)
        s2 = np.empty((H // 128, I // 128), np.float32)
        L.synth_quant_fp8_b128(f13.ctypes.data, 2 * I, H, q13.ctypes.data, s13.ctypes.data)
        L.synth_quant_fp8_b128(f2.ctypes.data, H, I, q2.ctypes.data, s2.ctypes.data)
        return q13, q2, s13, s2
    if wl.wtype == "int4":
        q13 = np.empty((2 * I, H // 2), np.uint8)
        q2 = np.empty((H, I // 2), np.uint8)
        s13 = np.empty((2 * I, H // 128), np.uint16)
        s2 = np.empty((H, I // 128), np.uint16)
        L.synth_quant_int4_g128(f13.ctypes.data, 2 * I, H, q13.ctypes.data, s13.ctypes.data)
        L.synth_quant_int4_g128(f2.ctypes.data, H, I, q2.ctypes.data, s2.ctypes.data)
        return q13, q2, s13, s2
    if wl.wtype == "int8":
        q13 = np.empty((2 * I, H), np.uint8)
        q2 = np.empty((H, I), np.uint8)
        s13 = np.empty((2 * I, H // 128), np.uint16)
        s2 = np.empty((H, I // 128), np.uint16)
        L.synth_quant_int8_g128(f13.ctypes.data, 2 * I, H, q13.ctypes.data, s13.ctypes.data)
        L.synth_quant_int8_g128(f2.ctypes.data, H, I, q2.ctypes.data, s2.ctypes.data)
        return q13, q2, s13, s2
    if wl.wtype == "mxfp4":
        q13 = np.empty((2 * I, H // 2), np.uint8)
        q2 = np.empty((H, I // 2), np.uint8)
        s13 = np.empty((2 * I, H // 32), np.uint8)
        s2 = np.empty((H, I // 32), np.uint8)
        L.synth_quant_mxfp4_b32(f13.ctypes.data, 2 * I, H, q13.ctypes.data, s13.ctypes.data)
        L.synth_quant_mxfp4_b32(f2.ctypes.data, H, I, q2.ctypes.data, s2.ctypes.data)
        return q13, q2, s13, s2
    raise ValueError("unknown weight type %r" % wl.wtype)


# ---------------------------------------------------------------- activations

def hidden_states(wl: Workload, step: int, tokens: int) -> np.ndarray:
    """bf16 bits [tokens, H] of N(0,1) draws; one tensor per step, fed to every layer."""
    x = normal(_key("x", wl.name, step), tokens * wl.hidden, 1.0)
    return round_bf16(x).reshape(tokens, wl.hidden)


# ---------------------------------------------------------------- routing

def _popularity_logits(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    """[L, E] log-popularity: Zipf(s) over a seeded per-layer permutation (uniform if s = 0)."""
    E = wl.experts
    logp = np.zeros((wl.layers, E), np.float64)
    if wl.zipf_s > 0:
        ranks = np.arange(1, E + 1, dtype=np.float64)
        w = -wl.zipf_s * np.log(ranks)
        for l in range(wl.layers):
            perm = rng.permutation(E)
            logp[l, perm] = w
    return logp


def _gumbel(rng, shape):
    u = rng.random(shape)
    u = np.where(u <= 0.0, np.finfo(np.float64).tiny, u)
    return -np.log(-np.log(u))


def _draw_distinct(logp, rng, k):
    """k ids per row without replacement, proportional to exp(logp): the top-k
    of logp + Gumbel noise in descending order (same law as k sequential draws)."""
    keys = logp + _gumbel(rng, logp.shape)
    return np.argsort(-keys, axis=-1, kind="stable")[..., :k].astype(np.int32)


def decode_routing(wl: Workload, steps: int = None, batch: int = None, start_ids: np.ndarray = None,
                   logp: np.ndarray = None, rng: np.random.Generator = None) -> np.ndarray:
    """E-wide routed ids [steps, L, batch, k] int32 for decode.

    Each of the `batch` tokens is an independent chain.  Step 0 draws k distinct
    ids by popularity (or continues from `start_ids` [L, batch, k]).  At each later
    step every position keeps its previous id with probability keep_p; the other
    positions are redrawn, in position order, by popularity restricted to experts
    not already in the token's new set (so a position may redraw its own old id).
    """
    steps = wl.steps if steps is None else steps
    batch = wl.batch if batch is None else batch
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([MASTER_SEED, _key("route", wl.name) & 0xFFFFFFFF])))
    if logp is None:
        logp = _popularity_logits(wl, rng)
    L, E, k = wl.layers, wl.experts, wl.top_k
    out = np.empty((steps, L, batch, k), np.int32)
    lp = np.broadcast_to(logp[:, None, :], (L, batch, E))
    if start_ids is None:
        prev = _draw_distinct(lp, rng, k)
        first = 0
        out[0] = prev
        first = 1
    else:
        prev = np.asarray(start_ids, np.int32).reshape(L, batch, k)
        first = 0
    for s in range(first, steps):
        keep = rng.random((L, batch, k)) < wl.keep_p
        keys = lp + _gumbel(rng, (L, batch, E))
        # experts kept by this token are not available for redraws
        kept_mask = np.zeros((L, batch, E), bool)
        li, bi, ji = np.nonzero(keep)
        kept_mask[li, bi, prev[li, bi, ji]] = True
        keys = np.where(kept_mask, -np.inf, keys)
        cand = np.argsort(-keys, axis=-1, kind="stable")[..., :k].astype(np.int32)
        # the r-th non-kept position (in position order) takes the r-th candidate
        rank = np.cumsum(~keep, axis=-1) - 1
        drawn = np.take_along_axis(cand, np.clip(rank, 0, k - 1), axis=-1)
        cur = np.where(keep, prev, drawn).astype(np.int32)
        out[s] = cur
        prev = cur
    return out


def prefill_routing(wl: Workload, tokens: int = None, logp: np.ndarray = None, rng=None) -> np.ndarray:
    """[L, tokens, k] int32: per token k distinct ids drawn by per-layer Zipf popularity."""
    tokens = wl.prefill_tokens if tokens is None else tokens
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([MASTER_SEED, _key("route", wl.name) & 0xFFFFFFFF])))
    if logp is None:
        logp = _popularity_logits(wl, rng)
    lp = np.broadcast_to(logp[:, None, :], (wl.layers, tokens, wl.experts))
    return _draw_distinct(lp, rng, wl.top_k)


def router_weights(wl: Workload, shape, stream: str = "w") -> np.ndarray:
    """fp32 router weights [..., k]: softmax of N(0,1) logits over the k chosen ids,
    then divided by their fp32 sum."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([MASTER_SEED, _key("rw", wl.name, stream) & 0xFFFFFFFF])))
    logits = rng.standard_normal(tuple(shape) + (wl.top_k,)).astype(np.float32)
    e = np.exp(logits - logits.max(axis=-1, keepdims=True)).astype(np.float32)
    w = (e / e.sum(axis=-1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return (w / w.sum(axis=-1, keepdims=True, dtype=np.float32)).astype(np.float32)


def routing_for(wl: Workload):
    """All routing of a workload.

    Returns dict with:
      decode_ids [steps, L, B, k] int32, decode_w [steps, L, B, k] fp32, and for
      prefill workloads also prefill_ids [L, T, k], prefill_w [L, T, k]; the
      decode continuation then starts from the last prefill token's ids with the
      same per-layer popularity.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([MASTER_SEED, _key("route", wl.name) & 0xFFFFFFFF])))
    logp = _popularity_logits(wl, rng)
    out = {}
    if wl.routing == "prefill_zipf":
        pids = prefill_routing(wl, logp=logp, rng=rng)
        out["prefill_ids"] = pids
        out["prefill_w"] = router_weights(wl, (wl.layers, wl.prefill_tokens), "prefill")
        start = pids[:, -1:, :]
        out["decode_ids"] = decode_routing(wl, start_ids=start, logp=logp, rng=rng)
    else:
        out["decode_ids"] = decode_routing(wl, logp=logp, rng=rng)
    out["decode_w"] = router_weights(wl, (wl.steps, wl.layers, wl.batch), "decode")
    return out
