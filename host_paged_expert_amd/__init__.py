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
    PE_FLAG_PAGEIN_DMA, PE_FLAG_FORCE_HOST_PLAN, PE_FLAG_UNPAGED, SIGNATURES,
    pe_create, pe_destroy, pe_load_expert, pe_forward, pe_forward_rc, pe_reset_lru, pe_expert_bytes,
    pe_suggest_k, pe_max_captured_batch, pe_max_waves, pe_get_lru_state, pe_get_plan, pe_get_slot_map, pe_get_stats,
    pe_reset_stats, pe_link_probe, pe_plan_host, pe_strerror, pe_last_error,
    pe_set_timing, pe_get_timing, STAGES,
)


class PagedMoE:
    """Owns one libpe context; methods forward to the pe_* entry points."""

    def __init__(self, num_layers, num_experts, top_k, num_resident, hidden, inter, max_tokens,
                 wtype="bf16", device=0, flags=0):
        self.L, self.E, self.k, self.H, self.I = num_layers, num_experts, top_k, hidden, inter
        self.K = num_experts if flags & PE_FLAG_UNPAGED else num_resident
        self.wtype, self.flags, self.max_tokens = wtype, flags, max_tokens
        self.ctx = pe_create(num_layers, num_experts, top_k, num_resident, hidden, inter, max_tokens,
                             wtype, device, flags)

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

    def forward(self, layer, x, topk_ids, topk_w, out, stream=None, T=None):
        T = x.shape[0] if T is None else T
        return pe_forward(self.ctx, layer, x, topk_ids, topk_w, T, out, stream)

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
