/*
 * Seeded synthetic inputs for the paged-expert MoE layer: normal draws for
 * expert weights and hidden states, bf16 rounding, and the two synthetic
 * weight quantisers (128x128 block e4m3, group-128 symmetric int4).
 *
 * This file is input generation shared by the GPU library's tests/bench and
 * by the CPU oracle.  It holds none of the method's arithmetic: no expert FFN,
 * no dequantisation, no planning.  The quantisers only turn fp32 draws into
 * (code, scale) pairs; decoding those codes is done independently by each side.
 *
 * Random source: the SplitMix64 output function (Steele, Lea & Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014) applied to a
 * Weyl sequence key + (p+1)*golden_gamma, one 64-bit word per pair p of
 * outputs; each word gives two uniforms that the Box-Muller transform
 * (Box & Muller 1958) turns into two standard normals.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stddef.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_mix64(uint64_t z) { return mix64(z); }

static inline uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }

/* fp32 -> bf16 bits, round to nearest even (inputs here are finite). */
void synth_round_bf16(const float* in, size_t n, uint16_t* out);

/* Standard normal pair p of stream `key` (Box-Muller on one SplitMix64 word). */
static inline void normal_pair(uint64_t key, uint64_t p, float* z0, float* z1) {
  const float two_pi = 6.28318530717958647692f;
  const float inv24 = 1.0f / 16777216.0f;
  uint64_t z = mix64(key + (p + 1) * GOLDEN_GAMMA);
  float u1 = (float)((z >> 40) + 1) * inv24;               /* (0, 1] */
  float u2 = (float)(z & 0xFFFFFFu) * inv24;               /* [0, 1) */
  float r = sqrtf(-2.0f * logf(u1));
  float th = two_pi * u2;
  *z0 = r * cosf(th);
  *z1 = r * sinf(th);
}

/* out[i] = sigma * (draw i of stream `key`), i in [0, n): draw 2p and 2p+1 are pair p. */
void synth_normal(uint64_t key, size_t n, float sigma, float* out) {
  for (size_t p = 0; 2 * p < n; ++p) {
    float a, b;
    normal_pair(key, p, &a, &b);
    out[2 * p] = sigma * a;
    if (2 * p + 1 < n) out[2 * p + 1] = sigma * b;
  }
}


/* fp32 -> bf16 bits, round to nearest even (inputs here are finite). */
void synth_round_bf16(const float* in, size_t n, uint16_t* out) {
  for (size_t i = 0; i < n; ++i) {
    uint32_t u = f32_bits(in[i]);
    out[i] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  }
}

/* synth_normal followed by bf16 rounding, through a stack buffer (chunks hold
 * whole pairs, so the values equal those of synth_normal). */
void synth_normal_bf16(uint64_t key, size_t n, float sigma, uint16_t* out) {
  float buf[4096];
  for (size_t done = 0; done < n; done += 4096) {
    size_t m = n - done < 4096 ? n - done : 4096;
    for (size_t q = 0; 2 * q < m; ++q) {
      float a, b;
      normal_pair(key, done / 2 + q, &a, &b);
      buf[2 * q] = sigma * a;
      if (2 * q + 1 < m) buf[2 * q + 1] = sigma * b;
    }
    synth_round_bf16(buf, m, out + done);
  }
}

/* fp32 -> IEEE binary16 bits, round to nearest even, with subnormals and overflow. */
static uint16_t f16_from_f32(float x) {
  uint32_t u = f32_bits(x);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x7F800000u) return sign | (a > 0x7F800000u ? 0x7E00u : 0x7C00u);
  if (a >= 0x477FF000u) return sign | 0x7C00u;            /* >= 65520 rounds to inf */
  if (a < 0x38800000u) {                                   /* < 2^-14: subnormal */
    float f; memcpy(&f, &a, 4);
    return sign | (uint16_t)nearbyintf(f * 16777216.0f);   /* units of 2^-24 */
  }
  uint32_t e = (a >> 23) - 127u + 15u;
  uint32_t mant = a & 0x7FFFFFu;
  uint32_t r = (e << 10) | (mant >> 13);
  uint32_t rem = mant & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) r++;
  return sign | (uint16_t)r;
}

void synth_f16_from_f32(const float* in, size_t n, uint16_t* out) {
  for (size_t i = 0; i < n; ++i) out[i] = f16_from_f32(in[i]);
}

/* fp32 -> OCP e4m3fn code (bias 7, no inf, max 448), round to nearest even,
 * saturating to +-448.  NaN maps to 0x7F. */
static uint8_t e4m3_from_f32(float x) {
  uint8_t sign = (uint8_t)((f32_bits(x) >> 24) & 0x80u);
  float a = fabsf(x);
  if (a != a) return (uint8_t)(sign | 0x7Fu);
  if (a >= 448.0f) return (uint8_t)(sign | 0x7Eu);
  if (a < 0.015625f) {                                     /* below 2^-6: step 2^-9 */
    return (uint8_t)(sign | (uint8_t)nearbyintf(a * 512.0f));  /* 8 -> 0x08 = 2^-6 */
  }
  int e;
  float f = frexpf(a, &e);                                 /* a = f * 2^e, f in [0.5, 1) */
  int E = e - 1 + 7;
  float mr = nearbyintf((f * 2.0f - 1.0f) * 8.0f);
  if (mr == 8.0f) { mr = 0.0f; E += 1; }
  if (E > 15 || (E == 15 && mr > 6.0f)) return (uint8_t)(sign | 0x7Eu);
  return (uint8_t)(sign | (uint8_t)(E << 3) | (uint8_t)mr);
}

void synth_e4m3_from_f32(const float* in, size_t n, uint8_t* out) {
  for (size_t i = 0; i < n; ++i) out[i] = e4m3_from_f32(in[i]);
}

/* Block-FP8 quantiser for a row-major [rows, cols] fp32 matrix, 128x128 blocks:
 * s = amax(block)/448 (1 if the block is all zero), q = e4m3(w / s).
 * q: [rows, cols] codes; s: [rows/128, cols/128] fp32 multipliers. */
void synth_quant_fp8_b128(const float* w, int rows, int cols, uint8_t* q, float* s) {
  int br = rows / 128, bc = cols / 128;
  for (int i = 0; i < br; ++i)
    for (int j = 0; j < bc; ++j) {
      float amax = 0.0f;
      for (int r = 0; r < 128; ++r)
        for (int c = 0; c < 128; ++c) {
          float a = fabsf(w[(size_t)(i * 128 + r) * cols + j * 128 + c]);
          if (a > amax) amax = a;
        }
      float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
      s[(size_t)i * bc + j] = sc;
      for (int r = 0; r < 128; ++r)
        for (int c = 0; c < 128; ++c) {
          size_t o = (size_t)(i * 128 + r) * cols + j * 128 + c;
          q[o] = e4m3_from_f32(w[o] / sc);
        }
    }
}

/* Symmetric group-128 int4 quantiser along the input (column) dimension:
 * s = fp16(amax(group)/7) (1 if all zero), q = clamp(rne(w/s), -8, 7) + 8 using
 * the fp16-rounded s.  Packed two per byte along a row, element 2i in the low
 * nibble of byte i.  q: [rows, cols/2] bytes; s: [rows, cols/128] fp16 bits. */
void synth_quant_int4_g128(const float* w, int rows, int cols, uint8_t* q, uint16_t* s) {
  int ng = cols / 128;
  for (int r = 0; r < rows; ++r) {
    const float* row = w + (size_t)r * cols;
    uint8_t* qrow = q + (size_t)r * (cols / 2);
    for (int g = 0; g < ng; ++g) {
      float amax = 0.0f;
      for (int c = 0; c < 128; ++c) { float a = fabsf(row[g * 128 + c]); if (a > amax) amax = a; }
      uint16_t sh = amax > 0.0f ? f16_from_f32(amax / 7.0f) : (uint16_t)0x3C00u;
      s[(size_t)r * ng + g] = sh;
      /* decode the fp16 scale exactly (it is a normal number here or 1.0) */
      uint32_t e = (sh >> 10) & 0x1Fu, m = sh & 0x3FFu;
      float sf = e ? ldexpf((float)(1024u + m), (int)e - 25) : ldexpf((float)m, -24);
      for (int c = 0; c < 128; c += 2) {
        float v0 = nearbyintf(row[g * 128 + c] / sf), v1 = nearbyintf(row[g * 128 + c + 1] / sf);
        int i0 = (int)fminf(fmaxf(v0, -8.0f), 7.0f) + 8, i1 = (int)fminf(fmaxf(v1, -8.0f), 7.0f) + 8;
        qrow[(g * 128 + c) / 2] = (uint8_t)(i0 | (i1 << 4));
      }
    }
  }
}

/* Symmetric group-128 int8 quantiser along the input (column) dimension:
 * s = fp16(amax(group)/127) (1 if all zero), q = clamp(rne(w/s), -128, 127) + 128
 * using the fp16-rounded s.  q: [rows, cols] bytes; s: [rows, cols/128] fp16 bits. */
void synth_quant_int8_g128(const float* w, int rows, int cols, uint8_t* q, uint16_t* s) {
  int ng = cols / 128;
  for (int r = 0; r < rows; ++r) {
    const float* row = w + (size_t)r * cols;
    uint8_t* qrow = q + (size_t)r * cols;
    for (int g = 0; g < ng; ++g) {
      float amax = 0.0f;
      for (int c = 0; c < 128; ++c) { float a = fabsf(row[g * 128 + c]); if (a > amax) amax = a; }
      uint16_t sh = amax > 0.0f ? f16_from_f32(amax / 127.0f) : (uint16_t)0x3C00u;
      s[(size_t)r * ng + g] = sh;
      uint32_t e = (sh >> 10) & 0x1Fu, m = sh & 0x3FFu;
      float sf = e ? ldexpf((float)(1024u + m), (int)e - 25) : ldexpf((float)m, -24);
      for (int c = 0; c < 128; ++c) {
        float v = nearbyintf(row[g * 128 + c] / sf);
        qrow[g * 128 + c] = (uint8_t)((int)fminf(fmaxf(v, -128.0f), 127.0f) + 128);
      }
    }
  }
}

/* OCP FP4 E2M1 code of v: round to nearest, ties to the even code (mantissa bit
 * 0), saturating at +-6; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
static uint8_t e2m1_from_f32(float v) {
  static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  uint8_t sign = signbit(v) ? 8u : 0u;
  float a = fabsf(v);
  if (a >= 6.0f) return (uint8_t)(sign | 7u);
  int best = 0;
  for (int i = 1; i < 8; ++i) {
    float d = fabsf(a - mag[i]), db = fabsf(a - mag[best]);
    if (d < db || (d == db && (i & 1) == 0)) best = i;
  }
  return (uint8_t)(sign | (uint8_t)best);
}

/* MXFP4 quantiser (OCP microscaling) along the input (column) dimension, blocks
 * of 32: shared exponent X = floor(log2(amax(block))) - 2 (E2M1's largest
 * exponent), scale 2^X stored as the E8M0 byte X + 127 (127 for an all-zero
 * block), q = e2m1(w / 2^X).  q: [rows, cols/2] bytes, element 2i in the low
 * nibble of byte i; s: [rows, cols/32] E8M0 bytes. */
void synth_quant_mxfp4_b32(const float* w, int rows, int cols, uint8_t* q, uint8_t* s) {
  int nb = cols / 32;
  for (int r = 0; r < rows; ++r) {
    const float* row = w + (size_t)r * cols;
    uint8_t* qrow = q + (size_t)r * (cols / 2);
    for (int b = 0; b < nb; ++b) {
      float amax = 0.0f;
      for (int c = 0; c < 32; ++c) { float a = fabsf(row[b * 32 + c]); if (a > amax) amax = a; }
      int e = 127;
      if (amax > 0.0f) {
        int ex;
        frexpf(amax, &ex);              /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
        e = ex - 1 - 2 + 127;
        if (e < 0) e = 0;
        if (e > 254) e = 254;
      }
      s[(size_t)r * nb + b] = (uint8_t)e;
      float sc = ldexpf(1.0f, e - 127);
      for (int c = 0; c < 32; c += 2) {
        uint8_t lo = e2m1_from_f32(row[b * 32 + c] / sc), hi = e2m1_from_f32(row[b * 32 + c + 1] / sc);
        qrow[(b * 32 + c) / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}
