"""Expert weight formats decoded to fp32.  TEST INFRASTRUCTURE (oracle).

The docs page ("Supported Configurations and Limitations") lists unquantized
bf16, block-quantized FP8 with 128x128 weight blocks, and GPTQ int4.  The
canonical tensors (as produced by `synth.expert_tensors`) are:

- bf16: raw bf16 bits.
- block FP8: OCP e4m3fn codes q[n, c] and fp32 multipliers s[n/128, c/128];
  w = e4m3(q) * s.
- int4: symmetric group-128 along the input dimension, no zero points:
  w = (q - 8) * s[n, c/128] with q a nibble (element 2i in the low nibble of
  byte i of the row) and s an IEEE fp16 scale.  This is the reading that
  reproduces the blog's 2.43 MB per expert.
- int8: the docs page also names GPTQ int8.  Read as int4's scheme with 8-bit
  codes: symmetric group-128 along the input dimension, one byte per weight,
  w = (q - 128) * s[n, c/128] with s an IEEE fp16 scale.
- MXFP4 (the blog names it among the added formats and runs gpt-oss-20b with
  it): OCP microscaling, blocks of 32 weights along the input dimension, each
  an FP4 E2M1 code, sharing one E8M0 scale: w = e2m1(q[n, c]) * 2^(e[n, c/32]
  - 127).  Codes are packed two per byte like int4 (element 2i in the low
  nibble of byte i).
"""
import numpy as np


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 is the top half of an fp32: widen by a 16-bit shift."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float32)


def e4m3_to_f32(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit float E4M3 ("fn" variant): sign bit, 4 exponent bits with bias 7,
    3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); no infinities; the
    codes S.1111.111 are NaN; the largest finite magnitude is 448."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = (m / 8.0) * 2.0 ** (1 - 7)
    nor = (1.0 + m / 8.0) * np.power(2.0, e - 7)
    val = sign * np.where(e == 0, sub, nor)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return val.astype(np.float32)


def dequant_fp8_b128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """[R, C] e4m3 codes times the fp32 multiplier of their 128x128 block."""
    w = e4m3_to_f32(q)
    R, C = w.shape
    assert s.shape == (R // 128, C // 128)
    scale = np.repeat(np.repeat(np.asarray(s, np.float32), 128, axis=0), 128, axis=1)
    return (w * scale).astype(np.float32)


def unpack_int4(qp: np.ndarray) -> np.ndarray:
    """[R, C/2] packed bytes -> [R, C] nibbles, element 2i = low nibble of byte i."""
    qp = np.asarray(qp, np.uint8)
    R, half = qp.shape
    out = np.empty((R, 2 * half), np.int64)
    out[:, 0::2] = qp & 0xF
    out[:, 1::2] = qp >> 4
    return out


def dequant_int4_g128(qp: np.ndarray, s: np.ndarray) -> np.ndarray:
    """w[n, c] = (q[n, c] - 8) * fp16 scale[n, c // 128]."""
    q = unpack_int4(qp)
    R, C = q.shape
    sf = f16_to_f32(s)
    assert sf.shape == (R, C // 128)
    scale = np.repeat(sf, 128, axis=1)
    return ((q - 8).astype(np.float32) * scale).astype(np.float32)


def dequant_int8_g128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """w[n, c] = (q[n, c] - 128) * fp16 scale[n, c // 128], q one byte per weight."""
    qi = np.asarray(q, np.uint8).astype(np.int64)
    R, C = qi.shape
    sf = f16_to_f32(s)
    assert sf.shape == (R, C // 128)
    scale = np.repeat(sf, 128, axis=1)
    return ((qi - 128).astype(np.float32) * scale).astype(np.float32)


def e2m1_to_f32(codes: np.ndarray) -> np.ndarray:
    """OCP 4-bit float E2M1: sign bit, 2 exponent bits with bias 1, 1 mantissa
    bit; exponent 0 is subnormal (m/2); no infinities or NaN; largest 6."""
    c = np.arange(16)                      # the value of each of the 16 codes, then a lookup
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    val = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.power(2.0, e - 1))
    return (sign * val).astype(np.float32)[np.asarray(codes, np.int64) & 0xF]


def e8m0_to_f32(codes: np.ndarray) -> np.ndarray:
    """OCP E8M0 scale: 2^(e - 127); e = 255 is NaN."""
    e = np.asarray(codes, np.int64)
    return np.where(e == 255, np.nan, np.power(2.0, e - 127)).astype(np.float32)


def dequant_mxfp4_b32(qp: np.ndarray, s: np.ndarray) -> np.ndarray:
    """w[n, c] = e2m1(q[n, c]) * 2^(s[n, c // 32] - 127), q packed two per byte."""
    q = unpack_int4(qp)
    R, C = q.shape
    assert s.shape == (R, C // 32)
    scale = np.repeat(e8m0_to_f32(s), 32, axis=1)
    return (e2m1_to_f32(q) * scale).astype(np.float32)


def dequant_expert(wtype: str, t13, t2, s13=None, s2=None):
    """Canonical expert tensors -> (W13 fp32 [2I, H], W2 fp32 [H, I])."""
    if wtype == "bf16":
        return bf16_to_f32(t13), bf16_to_f32(t2)
    if wtype == "fp8":
        return dequant_fp8_b128(t13, s13), dequant_fp8_b128(t2, s2)
    if wtype == "int4":
        return dequant_int4_g128(t13, s13), dequant_int4_g128(t2, s2)
    if wtype == "int8":
        return dequant_int8_g128(t13, s13), dequant_int8_g128(t2, s2)
    if wtype == "mxfp4":
        return dequant_mxfp4_b32(t13, s13), dequant_mxfp4_b32(t2, s2)
    raise ValueError(wtype)
