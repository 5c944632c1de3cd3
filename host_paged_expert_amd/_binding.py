"""ctypes binding of libpe (include/pe.h): argument marshalling only.

Every function keeps the C name.  Pointer arguments accept an int address,
a torch tensor (its data_ptr()) or a numpy array (its buffer); `stream`
accepts a torch stream, an int hipStream_t or None.  Non-zero status codes
raise PEError with the library's message.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpe.so")

PE_OK = 0
PE_ERR_INVALID_ARG = -1
PE_ERR_UNSUPPORTED = -2
PE_ERR_OOM_HOST_PIN = -3
PE_ERR_OOM_DEVICE = -4
PE_ERR_HIP = -5
PE_ERR_NOT_CAPTURABLE = -6

PE_W_BF16 = 0
PE_W_FP8_B128 = 1
PE_W_INT4_G128 = 2
PE_W_INT8_G128 = 3
PE_W_MXFP4_B32 = 4
WTYPES = {"bf16": PE_W_BF16, "fp8": PE_W_FP8_B128, "int4": PE_W_INT4_G128, "int8": PE_W_INT8_G128,
          "mxfp4": PE_W_MXFP4_B32}

PE_FLAG_PAGEIN_DMA = 1
PE_FLAG_FORCE_HOST_PLAN = 2
PE_FLAG_UNPAGED = 4
PE_FLAG_PLAN_LOG = 8
PE_STATIC_SCRATCH_BYTES = 16 << 20


class pe_config(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int), ("num_experts", ctypes.c_int), ("top_k", ctypes.c_int),
                ("num_resident", ctypes.c_int), ("hidden", ctypes.c_int), ("inter", ctypes.c_int),
                ("max_tokens", ctypes.c_int), ("device", ctypes.c_int), ("wtype", ctypes.c_int),
                ("flags", ctypes.c_uint), ("plan_log_steps", ctypes.c_int)]


class pe_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("steps", "device_planned", "host_planned", "waves", "page_ins",
                                               "page_in_bytes", "distinct", "entries", "bad_ids")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class PEError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("libpe error %d: %s" % (code, msg))
        self.code = code


# Every symbol include/pe.h declares, with its ctypes signature.
_vp, _i, _u32p, _i32p, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = {
    "pe_create": (_i, [ctypes.POINTER(pe_config), ctypes.POINTER(ctypes.c_void_p)]),
    "pe_destroy": (None, [_vp]),
    "pe_load_expert": (_i, [_vp, _i, _i, _vp, _vp, _vp, _vp]),
    "pe_forward": (_i, [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp]),
    "pe_reset_lru": (_i, [_vp, _i, _vp]),
    "pe_expert_bytes": (_i, [_i, _i, _i, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    "pe_suggest_k": (_i, [_i, _i, _i, _i, _i, _i, ctypes.c_double]),
    "pe_max_captured_batch": (_i, [_vp]),
    "pe_max_waves": (_i, [_vp]),
    "pe_get_lru_state": (_i, [_vp, _i, _vp, _vp, _vp, _vp]),
    "pe_get_plan": (_i, [_vp, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "pe_get_slot_map": (_i, [_vp, _i, _vp, _i, _vp]),
    "pe_plan_log_record_words": (_i, [_vp]),
    "pe_get_plan_log": (_i, [_vp, _i, _vp, _i, _vp, _vp]),
    "pe_forward_static": (_i, [_vp, _i, _vp, _vp, _vp, _i, _vp, _vp]),
    "pe_get_stats": (_i, [_vp, ctypes.POINTER(pe_stats)]),
    "pe_reset_stats": (_i, [_vp]),
    "pe_link_probe": (_i, [_vp, _sz, _i, _i, ctypes.POINTER(ctypes.c_double), _vp]),
    "pe_plan_host": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "pe_set_timing": (_i, [_vp, _i]),
    "pe_get_timing": (_i, [_vp, _vp, _vp]),
    "pe_strerror": (ctypes.c_char_p, [_i]),
    "pe_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """Load libpe.so (built in-tree); raise if it is missing: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libpe.so is not built (%s); run host_paged_expert_amd/build.py" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc):
    if rc != PE_OK:
        raise PEError(rc, lib().pe_last_error().decode(errors="replace"))
    return rc


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if hasattr(t, "ctypes"):
        return t.ctypes.data
    raise TypeError("cannot take a pointer of %r" % type(t))


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


# ---------------------------------------------------------------- entry points

def pe_create(num_layers, num_experts, top_k, num_resident, hidden, inter, max_tokens, wtype="bf16",
              device=0, flags=0, plan_log_steps=0):
    cfg = pe_config(num_layers, num_experts, top_k, num_resident, hidden, inter, max_tokens, device,
                    WTYPES[wtype] if isinstance(wtype, str) else wtype, flags, plan_log_steps)
    out = ctypes.c_void_p()
    _check(lib().pe_create(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def pe_destroy(ctx):
    lib().pe_destroy(ctx)


def pe_load_expert(ctx, layer, expert, w13, w2, s13=None, s2=None):
    return _check(lib().pe_load_expert(ctx, layer, expert, _ptr(w13), _ptr(w2), _ptr(s13), _ptr(s2)))


def pe_forward(ctx, layer, x, topk_ids, topk_w, T, out, stream=None):
    return _check(lib().pe_forward(ctx, layer, _ptr(x), _ptr(topk_ids), _ptr(topk_w), T, _ptr(out),
                                   _stream(stream)))


def pe_forward_rc(ctx, layer, x, topk_ids, topk_w, T, out, stream=None):
    """pe_forward returning the status code instead of raising."""
    return lib().pe_forward(ctx, layer, _ptr(x), _ptr(topk_ids), _ptr(topk_w), T, _ptr(out), _stream(stream))


def pe_forward_static(ctx, layer, x, topk_ids, topk_w, T, out, stream=None):
    return _check(lib().pe_forward_static(ctx, layer, _ptr(x), _ptr(topk_ids), _ptr(topk_w), T, _ptr(out),
                                          _stream(stream)))


def pe_reset_lru(ctx, layer=-1, stream=None):
    return _check(lib().pe_reset_lru(ctx, layer, _stream(stream)))


def pe_expert_bytes(wtype, hidden, inter):
    a, c = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().pe_expert_bytes(WTYPES[wtype] if isinstance(wtype, str) else wtype, hidden, inter,
                                 ctypes.byref(a), ctypes.byref(c)))
    return a.value, c.value


def pe_suggest_k(wtype, hidden, inter, num_layers, num_experts, top_k, budget_bytes):
    v = lib().pe_suggest_k(WTYPES[wtype] if isinstance(wtype, str) else wtype, hidden, inter, num_layers,
                           num_experts, top_k, float(budget_bytes))
    if v < 0:
        _check(v)
    return v


def pe_max_captured_batch(ctx):
    v = lib().pe_max_captured_batch(ctx)
    if v < 0:
        _check(v)
    return v


def pe_max_waves(ctx):
    v = lib().pe_max_waves(ctx)
    if v < 0:
        _check(v)
    return v


def pe_get_lru_state(ctx, layer, K, stream=None):
    import numpy as np
    se = np.empty(K, np.int32)
    lu = np.empty(K, np.uint32)
    tick = ctypes.c_uint32()
    _check(lib().pe_get_lru_state(ctx, layer, se.ctypes.data, lu.ctypes.data, ctypes.addressof(tick),
                                  _stream(stream)))
    return se, lu, tick.value


def pe_get_plan(ctx, layer, wave, K, stream=None):
    import numpy as np
    cnt, nw = ctypes.c_int32(), ctypes.c_int32()
    ex, sl, ev = (np.empty(K, np.int32) for _ in range(3))
    _check(lib().pe_get_plan(ctx, layer, wave, ctypes.addressof(cnt), ex.ctypes.data, sl.ctypes.data,
                             ev.ctypes.data, ctypes.addressof(nw), _stream(stream)))
    c = cnt.value
    return {"count": c, "experts": ex[:c].copy(), "slots": sl[:c].copy(), "evicted": ev[:c].copy(),
            "n_waves": nw.value}


def pe_get_slot_map(ctx, layer, T, top_k, stream=None):
    import numpy as np
    out = np.empty(T * top_k, np.int32)
    _check(lib().pe_get_slot_map(ctx, layer, out.ctypes.data, T, _stream(stream)))
    return out


def pe_plan_log_record_words(ctx):
    v = lib().pe_plan_log_record_words(ctx)
    if v < 0:
        _check(v)
    return v


def pe_get_plan_log(ctx, layer, max_records, stream=None):
    """The layer's most recent plan-log records, oldest first, as an int32
    array [n, record_words] (layout in include/pe.h)."""
    import numpy as np
    rw = pe_plan_log_record_words(ctx)
    buf = np.zeros((max(max_records, 1), rw), np.int32)
    n = ctypes.c_int()
    _check(lib().pe_get_plan_log(ctx, layer, buf.ctypes.data, max_records, ctypes.byref(n), _stream(stream)))
    return buf[:n.value]


def parse_plan_record(rec, K, max_waves, max_entries):
    """Split one plan-log record into its fields (layout in include/pe.h)."""
    MW = max_waves
    o = 4
    nw = int(rec[o]); o += 1
    counts = rec[o:o + MW]; o += MW
    ex = rec[o:o + MW * K].reshape(MW, K); o += MW * K
    sl = rec[o:o + MW * K].reshape(MW, K); o += MW * K
    ev = rec[o:o + MW * K].reshape(MW, K); o += MW * K
    T = int(rec[1])
    slot_of = rec[o:o + max_entries]; o += max_entries
    waves = [{"count": int(counts[w]), "experts": ex[w, :counts[w]].copy(), "slots": sl[w, :counts[w]].copy(),
              "evicted": ev[w, :counts[w]].copy()} for w in range(nw)]
    return {"seq": int(rec[0]), "T": T, "tick": int(rec[2]) & 0xFFFFFFFF, "n_waves": nw, "waves": waves,
            "slot_of": slot_of.copy(), "slot_expert": rec[o:o + K].copy(),
            "last_use": rec[o + K:o + 2 * K].astype(np.int64) & 0xFFFFFFFF}


def pe_get_stats(ctx):
    st = pe_stats()
    _check(lib().pe_get_stats(ctx, ctypes.byref(st)))
    return st.as_dict()


def pe_reset_stats(ctx):
    return _check(lib().pe_reset_stats(ctx))


def pe_link_probe(ctx, nbytes, use_kernel, reps=5, stream=None):
    v = ctypes.c_double()
    _check(lib().pe_link_probe(ctx, nbytes, int(use_kernel), reps, ctypes.byref(v), _stream(stream)))
    return v.value


def pe_plan_host(num_experts, num_resident, top_k, topk_ids, slot_expert, last_use, tick, max_waves):
    """Run the host wave planner on a caller-held state (numpy in, numpy out)."""
    import numpy as np
    ids = np.ascontiguousarray(topk_ids, np.int32).reshape(-1)
    T = ids.size // top_k
    se = np.ascontiguousarray(slot_expert, np.int32).copy()
    lu = np.ascontiguousarray(last_use, np.uint32).copy()
    tk = ctypes.c_uint32(tick)
    nw = ctypes.c_int32()
    K = num_resident
    counts = np.zeros(max_waves, np.int32)
    ex, sl, ev = (np.zeros(max_waves * K, np.int32) for _ in range(3))
    slot_of = np.zeros(T * top_k, np.int32)
    _check(lib().pe_plan_host(num_experts, K, top_k, T, ids.ctypes.data, se.ctypes.data, lu.ctypes.data,
                              ctypes.addressof(tk), max_waves, ctypes.addressof(nw), counts.ctypes.data,
                              ex.ctypes.data, sl.ctypes.data, ev.ctypes.data, slot_of.ctypes.data))
    waves = []
    for w in range(nw.value):
        c = counts[w]
        waves.append({"count": int(c), "experts": ex[w * K:w * K + c].copy(), "slots": sl[w * K:w * K + c].copy(),
                      "evicted": ev[w * K:w * K + c].copy()})
    return {"waves": waves, "slot_expert": se, "last_use": lu, "tick": tk.value, "slot_of": slot_of}


STAGES = ("plan", "page_in", "gate_up", "down", "topk_sum")


def pe_set_timing(ctx, enable):
    return _check(lib().pe_set_timing(ctx, int(enable)))


def pe_get_timing(ctx):
    """{stage: (launches, total_ms)} since timing was enabled."""
    import numpy as np
    n = np.zeros(len(STAGES), np.uint64)
    ms = np.zeros(len(STAGES), np.float64)
    _check(lib().pe_get_timing(ctx, n.ctypes.data, ms.ctypes.data))
    return {s: (int(n[i]), float(ms[i])) for i, s in enumerate(STAGES)}


def pe_strerror(code):
    return lib().pe_strerror(code).decode()


def pe_last_error():
    return lib().pe_last_error().decode(errors="replace")
