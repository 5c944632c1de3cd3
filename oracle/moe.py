"""The unpaged MoE layer.  TEST INFRASTRUCTURE (oracle).

The docs page states that paging leaves the layer's output unchanged ("Why
Paged Experts?") and that the merged entries are summed over top-k as the
unpaged kernel sums them (step 4 of "A step: waves, page-in, merge").  So the
reference result is the ordinary routed MoE layer

    out[t] = sum_{j=0}^{k-1}  w[t,j] * W2_e ( silu(W1_e x_t) * (W3_e x_t) ),  e = ids[t,j]

with W13_e = [W1_e ; W3_e] (gate rows first), no biases, silu(g) = g / (1 + exp(-g)).
Arithmetic is fp32 (products and sums in fp32, as numpy/BLAS sgemm do),
over the dequantised weights.  The top-k sum runs sequentially in j order.
Tokens routed to one expert are evaluated together, in ascending (t, j)
order, with one matmul per projection.
"""
import numpy as np


def silu(g: np.ndarray) -> np.ndarray:
    return g / (np.asarray(1.0, g.dtype) + np.exp(-g))


def expert_ffn(x: np.ndarray, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """SwiGLU expert: x [m, H] -> [m, H].  W13 [2I, H], W2 [H, I]."""
    dt = x.dtype
    inter = w2.shape[1]
    gu = x @ w13.T.astype(dt, copy=False)
    g, u = gu[:, :inter], gu[:, inter:]
    h = silu(g) * u
    return h @ w2.T.astype(dt, copy=False)


def moe_entries(x, ids, w, expert_weights, dtype=np.float32, select=None, num_experts=None):
    """Per-entry weighted expert outputs merged[t, j, :] = w[t,j] * FFN_e(x_t).

    x: [T, H] fp32 (already widened from bf16); ids: [T, k] int; w: [T, k] fp32;
    expert_weights(e) -> (W13 [2I,H], W2 [H,I]) fp32.  `select(e)` (optional)
    restricts evaluation to experts for which it is True; other entries stay 0
    and are reported in the returned mask as not written.
    Ids outside [0, num_experts) are not evaluated (their entries stay 0).
    """
    x = np.asarray(x, dtype)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype)
    T, k = ids.shape
    H = x.shape[1]
    merged = np.zeros((T, k, H), dtype)
    written = np.zeros((T, k), bool)
    for e in np.unique(ids):
        if e < 0 or (num_experts is not None and e >= num_experts):
            continue
        if select is not None and not select(int(e)):
            continue
        tt, jj = np.nonzero(ids == e)          # ascending (t, j)
        w13, w2 = expert_weights(int(e))
        y = expert_ffn(x[tt], np.asarray(w13, dtype), np.asarray(w2, dtype))
        merged[tt, jj] = w[tt, jj][:, None] * y
        written[tt, jj] = True
    return merged, written


def topk_sum(merged: np.ndarray) -> np.ndarray:
    """out[t] = ((merged[t,0] + merged[t,1]) + ...) + merged[t,k-1], in the merged dtype."""
    out = merged[:, 0].copy()
    for j in range(1, merged.shape[1]):
        out = out + merged[:, j]
    return out


def moe_layer(x, ids, w, expert_weights, dtype=np.float32, num_experts=None):
    """The unpaged layer output [T, H] in `dtype` (fp32 per the method)."""
    merged, _ = moe_entries(x, ids, w, expert_weights, dtype, num_experts=num_experts)
    return topk_sum(merged)
