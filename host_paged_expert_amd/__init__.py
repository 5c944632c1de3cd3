"""Paged-expert MoE layer for one AMD Instinct MI355X (gfx950).

The work is done by libpe.so (C ABI in include/pe.h, HIP kernels in csrc/).
This package is its thin ctypes binding plus `PagedMoE`, a small convenience
owner of one context.  PyTorch is used by callers only for device memory and
streams.
"""
from ._binding import (  # noqa: F401
    LIB_PATH, PEError, lib,
    PE_OK, PE_ERR_INVALID_ARG, PE_ERR_UNSUPPORTED, PE_ERR_OOM_HOST_PIN, PE_ERR_OOM_DEVICE, PE_ERR_HIP,
    PE_ERR_NOT_CAPTURABLE, PE_W_BF16, PE_W_FP8_B128, PE_W_INT4_G128, PE_W_INT8_G128, PE_W_MXFP4_B32,
    WTYPES,
    PE_FLAG_PAGEIN_DMA, PE_FLAG_FORCE_HOST_PLAN, PE_FLAG_UNPAGED, PE_FLAG_PLAN_LOG, PE_STATIC_SCRATCH_BYTES,
    SIGNATURES,
    pe_create, pe_destroy, pe_load_expert, pe_forward, pe_forward_rc, pe_forward_static, pe_reset_lru,
    pe_expert_bytes, pe_plan_log_record_words, pe_get_plan_log, parse_plan_record,
    pe_suggest_k, pe_max_captured_batch, pe_max_waves, pe_get_lru_state, pe_get_plan, pe_get_slot_map, pe_get_stats,
    pe_reset_stats, pe_link_probe, pe_plan_host, pe_strerror, pe_last_error,
    pe_set_timing, pe_get_timing, STAGES,
)


class PagedMoE:
    """Owns one libpe context; methods forward to the pe_* entry points."""

    def __init__(self, num_layers, num_experts, top_k, num_resident, hidden, inter, max_tokens,
                 wtype="bf16", device=0, flags=0, plan_log_steps=0):
        self.L, self.E, self.k, self.H, self.I = num_layers, num_experts, top_k, hidden, inter
        self.K = num_experts if flags & PE_FLAG_UNPAGED else num_resident
        self.wtype, self.flags, self.max_tokens, self.device = wtype, flags, max_tokens, device
        self.plan_log_steps = plan_log_steps
        self.ctx = pe_create(num_layers, num_experts, top_k, num_resident, hidden, inter, max_tokens,
                             wtype, device, flags, plan_log_steps)

    def close(self):
        if self.ctx:
            pe_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def load_expert(self, layer, expert, w13, w2, s13=None, s2=None):
        return pe_load_expert(self.ctx, layer, expert, w13, w2, s13, s2)

    def _check_step(self, x, topk_ids, topk_w, out, T):
        """Raise before the call if the tensors do not match what the library reads
        and writes: x / out bf16 [>=T, H], topk_ids int32 and topk_w fp32 [>=T, k],
        all contiguous on this context's device."""
        import torch
        dev = torch.device("cuda", self.device)
        for name, t, dt, cols in (("x", x, torch.bfloat16, self.H), ("out", out, torch.bfloat16, self.H),
                                  ("topk_ids", topk_ids, torch.int32, self.k),
                                  ("topk_w", topk_w, torch.float32, self.k)):
            if not isinstance(t, torch.Tensor):
                raise TypeError("%s must be a torch tensor" % name)
            if t.dtype != dt or t.device != dev or not t.is_contiguous():
                raise ValueError("%s must be a contiguous %s tensor on %s (got %s on %s%s)" % (
                    name, dt, dev, t.dtype, t.device, "" if t.is_contiguous() else ", not contiguous"))
            if t.dim() != 2 or t.shape[1] != cols or t.shape[0] < T:
                raise ValueError("%s must have shape [>=%d, %d], got %s" % (name, T, cols, tuple(t.shape)))
        if not 0 <= T <= self.max_tokens:
            raise ValueError("T=%d outside [0, %d]" % (T, self.max_tokens))

    def forward(self, layer, x, topk_ids, topk_w, out, stream=None, T=None):
        T = x.shape[0] if T is None else T
        self._check_step(x, topk_ids, topk_w, out, T)
        return pe_forward(self.ctx, layer, x, topk_ids, topk_w, T, out, stream)

    def forward_static(self, layer, x, topk_ids, topk_w, out, stream=None, T=None):
        T = x.shape[0] if T is None else T
        self._check_step(x, topk_ids, topk_w, out, T)
        return pe_forward_static(self.ctx, layer, x, topk_ids, topk_w, T, out, stream)

    def plan_log(self, layer, max_records=None, stream=None):
        """Parsed plan-log records of `layer`, oldest first."""
        rows = pe_get_plan_log(self.ctx, layer, self.plan_log_steps if max_records is None else max_records,
                               stream)
        mw, ne = pe_max_waves(self.ctx), self.max_tokens * self.k
        return [parse_plan_record(r, self.K, mw, ne) for r in rows]

    def reset_lru(self, layer=-1, stream=None):
        return pe_reset_lru(self.ctx, layer, stream)

    def lru_state(self, layer, stream=None):
        return pe_get_lru_state(self.ctx, layer, self.K, stream)

    def plan(self, layer, wave, stream=None):
        return pe_get_plan(self.ctx, layer, wave, self.K, stream)

    def slot_map(self, layer, T, stream=None):
        return pe_get_slot_map(self.ctx, layer, T, self.k, stream)

    def stats(self):
        return pe_get_stats(self.ctx)

    def reset_stats(self):
        return pe_reset_stats(self.ctx)

    def set_timing(self, enable):
        return pe_set_timing(self.ctx, enable)

    def timing(self):
        return pe_get_timing(self.ctx)

    @property
    def max_captured_batch(self):
        return pe_max_captured_batch(self.ctx)

    @property
    def max_waves(self):
        return pe_max_waves(self.ctx)
