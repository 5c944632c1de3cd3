"""Pins for oracle/formats.py: e4m3fn, int4, int8, MXFP4 and bf16 decoding."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.e4m3_to_f32(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_closed_form_points():
    v = formats.e4m3_to_f32(np.array([0x7E, 0x01, 0x07, 0x08, 0x38, 0xB8, 0x00, 0x80, 0x40], np.uint8))
    assert v[0] == 448.0                       # largest finite: 1.75 * 2^8
    assert v[1] == 2.0 ** -9                   # smallest subnormal
    assert v[2] == 7 * 2.0 ** -9
    assert v[3] == 2.0 ** -6                   # smallest normal
    assert v[4] == 1.0 and v[5] == -1.0
    assert v[6] == 0.0 and np.signbit(v[7])
    assert v[8] == 2.0


def test_e4m3_encoder_roundtrip_and_vs_torch():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = formats.e4m3_to_f32(codes)
    assert np.array_equal(synth.e4m3_from_f32(vals), codes)
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * 60).astype(np.float32)
    x = np.clip(x, -440, 440)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(synth.e4m3_from_f32(x), ref)


def test_f16_encoder_vs_numpy():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(50000).astype(np.float32) * s for s in (1e-6, 1e-3, 1.0, 1e3, 1e5)])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(synth.f16_from_f32(x), ref)


def test_bf16_decode_vs_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 65536, 10000, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]        # finite only
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(formats.bf16_to_f32(bits), ref)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -1.0 - 2 ** -8], np.float32)
    got = formats.bf16_to_f32(synth.round_bf16(x))
    assert np.array_equal(got, np.array([1.0, 1.0 + 2 ** -6, 1.0, -1.0], np.float32))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got, ref)


def test_int4_unpack_vs_bit_extraction():
    rng = np.random.default_rng(4)
    qp = rng.integers(0, 256, (3, 64), dtype=np.uint8)
    q = formats.unpack_int4(qp)
    for r in range(3):
        for c in range(128):
            byte = int(qp[r, c // 2])
            nib = (byte >> (4 * (c % 2))) & 0xF
            assert q[r, c] == nib


def test_int4_dequant_error_within_half_step():
    wl = synth.workload("decode_int4_k26_b4", hidden=256, inter=128)
    f13, f2 = synth.expert_draws(wl.hidden, wl.inter, 0, 1)
    q13, q2, s13, s2 = synth.expert_tensors(wl, 0, 1)
    for f, q, s in ((f13, q13, s13), (f2, q2, s2)):
        w = formats.dequant_int4_g128(q, s)
        step = np.repeat(formats.f16_to_f32(s), 128, axis=1)
        assert np.all(np.abs(w - f) <= step / 2 * (1 + 1e-6))
        assert formats.unpack_int4(q).min() >= 1        # symmetric: -8 is never used


def test_int8_dequant_vs_elementwise():
    """Each weight decoded on its own: the byte as an integer minus 128, times the
    fp16 scale of its row and 128-column group read with Python's own half codec."""
    import struct
    rng = np.random.default_rng(8)
    q = rng.integers(0, 256, (3, 256), dtype=np.uint8)
    s = np.array([[0x3C00, 0x2E66], [0x1400, 0xB800], [0x0001, 0x7BFF]], np.uint16)   # 1, 0.1, tiny, -0.5, subnormal, max
    w = formats.dequant_int8_g128(q, s)
    for r in range(3):
        for c in range(256):
            sc = struct.unpack("<e", struct.pack("<H", int(s[r, c // 128])))[0]
            assert w[r, c] == np.float32((int(q[r, c]) - 128) * sc)


def test_int8_dequant_error_within_half_step():
    wl = synth.workload("decode_int8_k40_b4", hidden=256, inter=128)
    f13, f2 = synth.expert_draws(wl.hidden, wl.inter, 0, 1)
    q13, q2, s13, s2 = synth.expert_tensors(wl, 0, 1)
    for f, q, s in ((f13, q13, s13), (f2, q2, s2)):
        w = formats.dequant_int8_g128(q, s)
        step = np.repeat(formats.f16_to_f32(s), 128, axis=1)
        assert np.all(np.abs(w - f) <= step / 2 * (1 + 1e-6))
        qi = q.astype(np.int64) - 128
        assert qi.min() >= -127                          # symmetric: -128 is never used
        # each group's largest magnitude lands on the last code (up to the fp16 rounding of s)
        gmax = np.abs(qi).reshape(q.shape[0], -1, 128).max(axis=2)
        assert np.all(gmax >= 126)


def test_fp8_dequant_error_within_rounding():
    wl = synth.workload("decode_fp8_k40_b4", hidden=256, inter=128)
    f13, f2 = synth.expert_draws(wl.hidden, wl.inter, 0, 1)
    q13, q2, s13, s2 = synth.expert_tensors(wl, 0, 1)
    for f, q, s in ((f13, q13, s13), (f2, q2, s2)):
        w = formats.dequant_fp8_b128(q, s)
        sc = np.repeat(np.repeat(s, 128, 0), 128, 1)
        # e4m3 keeps 3 mantissa bits: relative error <= 2^-4 for normals, absolute <= 2^-10*s below 2^-6
        assert np.all(np.abs(w - f) <= np.maximum(np.abs(f) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-6))
        # every block's largest magnitude maps to 448
        blk = np.abs(formats.e4m3_to_f32(q)).reshape(q.shape[0] // 128, 128, q.shape[1] // 128, 128).max(axis=(1, 3))
        assert np.all(blk == 448.0)


# OCP microscaling spec, FP4 E2M1 value table: codes 0..7 are +0, 0.5, 1, 1.5,
# 2, 3, 4, 6 and codes 8..15 the same magnitudes negated.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_all_codes_match_the_spec_table():
    got = formats.e2m1_to_f32(np.arange(16))
    assert got.tolist() == E2M1_TABLE
    assert np.signbit(got[8]) and not np.signbit(got[0])


def test_e8m0_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = formats.e8m0_to_f32(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float32).numpy()
    assert np.array_equal(got, ref, equal_nan=True)
    assert got[127] == 1.0 and got[128] == 2.0 and got[126] == 0.5 and np.isnan(got[255])


def test_mxfp4_dequant_vs_elementwise():
    """Each weight decoded on its own from the spec's value table: the nibble
    (low nibble first) times 2 to the power of its 32-column block's byte - 127."""
    rng = np.random.default_rng(9)
    qp = rng.integers(0, 256, (3, 32), dtype=np.uint8)        # 3 rows x 64 columns
    s = np.array([[127, 120], [130, 0], [252, 1]], np.uint8)
    w = formats.dequant_mxfp4_b32(qp, s)
    for r in range(3):
        for c in range(64):
            nib = (int(qp[r, c // 2]) >> (4 * (c % 2))) & 0xF
            want = np.float32(E2M1_TABLE[nib] * 2.0 ** (int(s[r, c // 32]) - 127))
            assert w[r, c] == want, (r, c)


def test_mxfp4_quantiser_rounds_to_the_nearest_grid_point():
    """The synthetic MXFP4 tensors against the spec's scale rule: each block's
    E8M0 exponent is floor(log2(amax)) - 2, and every weight decodes to the E2M1
    grid point nearest to w / 2^X (saturating at 6), times 2^X."""
    wl = synth.workload("decode_mxfp4_k16_b1", hidden=256, inter=128)
    f13, f2 = synth.expert_draws(wl.hidden, wl.inter, 0, 1)
    q13, q2, s13, s2 = synth.expert_tensors(wl, 0, 1)
    grid = np.array(sorted(set(abs(v) for v in E2M1_TABLE)))
    for f, q, s in ((f13, q13, s13), (f2, q2, s2)):
        w = formats.dequant_mxfp4_b32(q, s)
        amax = np.abs(f).reshape(f.shape[0], -1, 32).max(axis=2)
        assert np.array_equal(s.astype(np.int64), np.floor(np.log2(amax)).astype(np.int64) - 2 + 127)
        sc = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
        a = np.minimum(np.abs(f) / sc, 6.0)
        dist = np.abs(a[..., None] - grid)
        best = dist.min(axis=-1)
        got = np.abs(w) / sc
        # the decoded magnitude is a nearest grid point (ties may go either way here)
        assert np.all(np.abs(a - got) <= best + 1e-12)
        assert np.all((np.sign(w) == np.sign(f)) | (w == 0))


def test_dequant_expert_shapes():
    for name in ("decode_bf16_k40_b1", "decode_fp8_k40_b4", "decode_int4_k26_b4", "decode_int8_k40_b4",
                 "decode_mxfp4_k16_b1"):
        wl = synth.workload(name, hidden=256, inter=128)
        w13, w2 = formats.dequant_expert(wl.wtype, *synth.expert_tensors(wl, 1, 2))
        assert w13.shape == (256, 256) and w2.shape == (256, 128)
        assert w13.dtype == np.float32
        assert 0.015 < w13.std() < 0.025
