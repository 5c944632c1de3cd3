"""Pins for oracle/moe.py (the unpaged MoE layer)."""
import numpy as np
import scipy.special
import torch

from oracle import moe


def _experts(E, H, I, seed=0, scale=0.05):
    rng = np.random.default_rng(seed)
    return [((rng.standard_normal((2 * I, H)) * scale).astype(np.float32),
             (rng.standard_normal((H, I)) * scale).astype(np.float32)) for _ in range(E)]


def _routing(T, k, E, seed=1):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    return ids, w / w.sum(1, keepdims=True)


def _dense_then_select_f64(x, ids, w, ex):
    """Brute force in another formulation: every expert on every token in fp64
    (explicit loops over the intermediate dimension), then pick and weight."""
    x = x.astype(np.float64)
    T, H = x.shape
    E = len(ex)
    full = np.zeros((E, T, H))
    for e, (w13, w2) in enumerate(ex):
        I = w2.shape[1]
        for t in range(T):
            acc = np.zeros(H)
            for i in range(I):
                g = float(np.dot(w13[i].astype(np.float64), x[t]))
                u = float(np.dot(w13[I + i].astype(np.float64), x[t]))
                h = g * scipy.special.expit(g) * u
                acc += h * w2[:, i].astype(np.float64)
            full[e, t] = acc
    out = np.zeros((T, H))
    for t in range(T):
        for j in range(ids.shape[1]):
            out[t] += float(w[t, j]) * full[ids[t, j], t]
    return out


def test_vs_dense_brute_force_fp64():
    E, H, I, T, k = 6, 32, 24, 5, 3
    ex = _experts(E, H, I)
    ids, w = _routing(T, k, E)
    x = np.random.default_rng(2).standard_normal((T, H)).astype(np.float32)
    got = moe.moe_layer(x, ids, w, lambda e: ex[e])
    ref = _dense_then_select_f64(x, ids, w, ex)
    assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max()
    # and the fp64 path of the oracle agrees to rounding
    got64 = moe.moe_layer(x, ids, w, lambda e: ex[e], dtype=np.float64)
    assert np.abs(got64 - ref).max() <= 1e-12 * np.abs(ref).max()


def test_single_expert_is_dense_swiglu_mlp():
    """E = 1, k = 1, w = 1 reduces to a dense SwiGLU MLP (torch F.silu, fp64)."""
    H, I, T = 16, 12, 4
    (w13, w2), = _experts(1, H, I, seed=5)
    x = np.random.default_rng(6).standard_normal((T, H)).astype(np.float32)
    got = moe.moe_layer(x, np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32), lambda e: (w13, w2), dtype=np.float64)
    tx, t13, t2 = (torch.from_numpy(a).double() for a in (x, w13, w2))
    g, u = (tx @ t13.T).split(I, dim=1)
    ref = (torch.nn.functional.silu(g) * u) @ t2.T
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_one_hot_input_picks_a_column():
    H, I = 8, 5
    (w13, w2), = _experts(1, H, I, seed=7)
    c = 3
    x = np.zeros((1, H), np.float64)
    x[0, c] = 1.0
    got = moe.moe_layer(x, np.zeros((1, 1), np.int32), np.ones((1, 1)), lambda e: (w13, w2), dtype=np.float64)
    g = w13[:I, c].astype(np.float64)
    u = w13[I:, c].astype(np.float64)
    ref = w2.astype(np.float64) @ (g / (1 + np.exp(-g)) * u)
    assert np.allclose(got[0], ref, rtol=1e-13)


def test_linear_in_router_weights_and_zero():
    E, H, I, T, k = 4, 16, 8, 3, 2
    ex = _experts(E, H, I, seed=8)
    ids, w = _routing(T, k, E, seed=9)
    x = np.random.default_rng(10).standard_normal((T, H)).astype(np.float32)
    a = moe.moe_layer(x, ids, w, lambda e: ex[e])
    b = moe.moe_layer(x, ids, 2 * w, lambda e: ex[e])
    assert np.array_equal(b, 2 * a)                  # scaling by 2 is exact in fp32
    z = moe.moe_layer(x, ids, np.zeros_like(w), lambda e: ex[e])
    assert not z.any()
    zx = moe.moe_layer(np.zeros_like(x), ids, w, lambda e: ex[e])
    assert not zx.any()


def test_each_entry_uses_its_own_expert_and_weight():
    """Moving one entry's weight to 1 and the rest to 0 isolates that expert."""
    E, H, I = 5, 12, 6
    ex = _experts(E, H, I, seed=11)
    x = np.random.default_rng(12).standard_normal((1, H)).astype(np.float32)
    ids = np.array([[4, 1, 3]], np.int32)
    for j in range(3):
        w = np.zeros((1, 3), np.float32)
        w[0, j] = 1.0
        got = moe.moe_layer(x, ids, w, lambda e: ex[e], dtype=np.float64)
        single = moe.moe_layer(x, np.array([[ids[0, j]]]), np.ones((1, 1)), lambda e: ex[e], dtype=np.float64)
        assert np.array_equal(got, single)


def test_silu_special_values():
    g = np.array([0.0, 30.0, -30.0, 1.0, -1.0], np.float64)
    s = moe.silu(g)
    assert s[0] == 0.0 and abs(s[1] - 30.0) < 1e-9 and abs(s[2]) < 1e-9
    assert np.allclose(s, g * scipy.special.expit(g), rtol=1e-15)


def test_topk_sum_is_sequential_in_j():
    """fp32: (1e8 + 1) - 1e8 = 0 in j order, while another order would give 1."""
    merged = np.array([[[1e8], [1.0], [-1e8]]], np.float32)
    assert moe.topk_sum(merged)[0, 0] == 0.0
    assert moe.topk_sum(merged[:, [0, 2, 1]])[0, 0] == 1.0


def test_invalid_ids_contribute_nothing():
    E, H, I = 3, 8, 4
    ex = _experts(E, H, I, seed=13)
    x = np.random.default_rng(14).standard_normal((2, H)).astype(np.float32)
    ids = np.array([[0, 7], [-1, 2]], np.int32)
    w = np.ones((2, 2), np.float32)
    got = moe.moe_layer(x, ids, w, lambda e: ex[e], num_experts=E)
    ref = moe.moe_layer(x, np.array([[0], [2]]), np.ones((2, 1), np.float32), lambda e: ex[e])
    assert np.array_equal(got, ref)
