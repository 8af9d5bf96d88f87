/*
 * qk_oracle.c - plain scalar CPU oracle for ggml block-quantized GEMV.
 *
 * TEST INFRASTRUCTURE ONLY (see qk_oracle.h): used by tests, the smoke check
 * and the benchmark's CPU-baseline leg, never by the product path.
 *
 * Built with -O2 -ffp-contract=off and the default x86-64 ISA, so every float
 * operation below is one IEEE binary32 (or binary64) operation, rounded to
 * nearest even, in the order written.  Integer sums are exact int32.
 */
#include "qk_oracle.h"

#include <float.h>
#include <math.h>
#include <string.h>


/* ------------------------------------------------------------------------- */
/* Type table.                                                                */
/* [candle] GgmlDType table: block elements / block bytes                    */
/*   Q4_0 32/18, Q4_1 32/20, Q5_0 32/22, Q5_1 32/24, Q8_0 32/34, Q2K 256/84, */
/*   Q3K 256/110, Q4K 256/144, Q5K 256/176, Q6K 256/210, Q8K 256/292.         */
/* [sipllm] Design, "type_nbytes(t, n) = n / block_size * type_size".        */
/* ------------------------------------------------------------------------- */

int64_t orc_block_elems(int type) {
  switch (type) {
    case ORC_Q4_0:
    case ORC_Q4_1:
    case ORC_Q5_0:
    case ORC_Q5_1:
    case ORC_Q8_0:
    case ORC_Q8_1:
      return 32;
    case ORC_Q2_K:
    case ORC_Q3_K:
    case ORC_Q4_K:
    case ORC_Q5_K:
    case ORC_Q6_K:
    case ORC_Q8_K:
      return 256;
    default:
      return 0;
  }
}

int64_t orc_block_bytes(int type) {
  switch (type) {
    case ORC_Q4_0: return 18;
    case ORC_Q4_1: return 20;
    case ORC_Q5_0: return 22;
    case ORC_Q5_1: return 24;
    case ORC_Q8_0: return 34;
    case ORC_Q8_1: return 36; /* reading: d f16, s f16, 32 int8 codes */
    case ORC_Q2_K: return 84;
    case ORC_Q3_K: return 110;
    case ORC_Q4_K: return 144;
    case ORC_Q5_K: return 176;
    case ORC_Q6_K: return 210;
    case ORC_Q8_K: return 292;
    default: return 0;
  }
}

/* A row is whole blocks with nothing between them ([cl] Example 9). */
int64_t orc_row_bytes(int type, int64_t n) {
  int64_t be = orc_block_elems(type);
  if (be == 0 || n < 0 || n % be != 0) return 0;
  return n / be * orc_block_bytes(type);
}

/* Weight -> activation pairing: [candle] VecDotType table (Q4_0, Q5_0, Q8_0
 * pair with Q8_0; Q4_1, Q5_1 with Q8_1; the K-quants with Q8K); [cl] Example 11;
 * [rml] "Quantized dot products".  Q8_1 is an activation format only ([candle]
 * 块结构: it never appears in a GGUF file), so it has no pairing as a weight. */
int orc_act_type(int weight_type) {
  switch (weight_type) {
    case ORC_Q4_0:
    case ORC_Q5_0:
    case ORC_Q8_0:
      return ORC_Q8_0;
    case ORC_Q4_1:
    case ORC_Q5_1:
      return ORC_Q8_1;
    case ORC_Q2_K:
    case ORC_Q3_K:
    case ORC_Q4_K:
    case ORC_Q5_K:
    case ORC_Q6_K:
      return ORC_Q8_K;
    default:
      return -1;
  }
}

/* ------------------------------------------------------------------------- */
/* IEEE 754 binary16 <-> binary32, from the format's definition:             */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 is    */
/* zero/subnormal (fraction * 2^-24), exponent 31 is inf/NaN.  Conversion    */
/* to binary16 rounds to nearest, ties to even, overflows to infinity.       */
/* [cl] Example 2 uses Float.floatToFloat16 (that rounding); [candle]        */
/* "一些边界值": a d below the smallest subnormal becomes 0, above 65504      */
/* becomes inf.                                                              */
/* ------------------------------------------------------------------------- */

float orc_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int frac = h & 1023;
  double v;
  if (e == 0) {
    v = ldexp((double)frac, -24);
  } else if (e == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + frac), e - 25);
  }
  return (float)(sign ? -v : v);
}

/* Round a non-negative double holding an exact binary32 value to the nearest
 * integer, ties to even. */
static double orc_rint_even(double v) {
  double f = floor(v);
  double r = v - f; /* exact: v has at most 24 significant bits */
  if (r > 0.5) return f + 1.0;
  if (r < 0.5) return f;
  return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

uint16_t orc_f32_to_f16(float f) {
  uint16_t sign = signbit(f) ? 0x8000 : 0;
  if (isnan(f)) return sign | 0x7E00;
  double a = fabs((double)f);
  if (isinf(f)) return sign | 0x7C00;
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: value = m * 2^-24, m in [0, 1024]; m == 1024 is the
     * smallest normal, whose encoding (exponent 1, fraction 0) is also 1024. */
    double m = orc_rint_even(a * ldexp(1.0, 24));
    return sign | (uint16_t)m;
  }
  int e2;
  (void)frexp(a, &e2);           /* a = fr * 2^e2, fr in [0.5, 1) */
  int e = e2 - 1;                /* a in [2^e, 2^(e+1)) */
  double m = orc_rint_even(ldexp(a, 10 - e)); /* in [1024, 2048] */
  if (m == 2048.0) {
    m = 1024.0;
    e += 1;
  }
  if (e > 15) return sign | 0x7C00;
  return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

/* ------------------------------------------------------------------------- */
/* Activation / weight quantizers.                                           */
/* ------------------------------------------------------------------------- */

/* C roundf (halves away from zero) of x*id, saturated to int8 the way
 * [candle]'s `as i8` cast does; NaN becomes 0 ([candle] "一些边界值": a NaN
 * value is ignored by amax and its own code becomes 0). */
static int8_t orc_code_q8(float v) {
  if (isnan(v)) return 0;
  float r = roundf(v);
  if (r > 127.0f) return 127;
  if (r < -128.0f) return -128;
  return (int8_t)r;
}

/* The truncating conversion of the Q4_0 / Q4_1 / Q5_0 codes: the (int) cast of
 * [cl] Examples 5, 7 and 8's listings, which truncates toward zero, saturates at
 * the int32 limits and turns NaN into 0.  A value outside 0..16.5 reaches it only
 * when 1/d overflows to infinity (a block whose scale is below 2^-128). */
static int32_t orc_trunc_sat(float v) {
  if (isnan(v)) return 0;
  if (v >= 2147483648.0f) return INT32_MAX;
  if (v <= -2147483648.0f) return INT32_MIN;
  return (int32_t)v;
}

/* Largest |x| over a block, NaN ignored (fmaxf returns the other operand). */
static float orc_amax(const float* x, int64_t len) {
  float amax = 0.0f;
  for (int64_t j = 0; j < len; ++j) amax = fmaxf(amax, fabsf(x[j]));
  return amax;
}

static void orc_put_u16(uint8_t* p, uint16_t v) {
  p[0] = (uint8_t)(v & 0xFF);
  p[1] = (uint8_t)(v >> 8);
}
static uint16_t orc_get_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static int16_t orc_get_i16(const uint8_t* p) { return (int16_t)orc_get_u16(p); }
static float orc_get_f32(const uint8_t* p) {
  uint32_t u = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
               ((uint32_t)p[3] << 24);
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static void orc_put_f32(uint8_t* p, float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  p[0] = (uint8_t)u;
  p[1] = (uint8_t)(u >> 8);
  p[2] = (uint8_t)(u >> 16);
  p[3] = (uint8_t)(u >> 24);
}

/* quantize_row_q8_0 reference ([cl] Example 2, four steps per 32-block;
 * [candle] BlockQ8_0::from_float): amax; d = amax / 127; id = 1/d or 0 when
 * d is 0; store d as f16; code = roundf(x * id) with the unrounded f32 id.
 * Block bytes: d f16 little-endian at 0, 32 int8 codes at 2 ([cl] Example 1). */
int orc_quantize_q8_0(const float* x, uint8_t* out, int64_t n) {
  if (n < 0 || n % 32 != 0) return ORC_BAD_SHAPE;
  for (int64_t b = 0; b < n / 32; ++b) {
    const float* xb = x + 32 * b;
    uint8_t* ob = out + 34 * b;
    float amax = orc_amax(xb, 32);
    float d = amax / 127.0f;
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    orc_put_u16(ob, orc_f32_to_f16(d));
    for (int j = 0; j < 32; ++j) ob[2 + j] = (uint8_t)orc_code_q8(xb[j] * id);
  }
  return ORC_OK;
}

/* quantize_row_q8_1 (reading; [candle] VecDotType table names BlockQ8_1 as the
 * activation block of the _1 types, 块结构 says the _1 blocks add one f16 to the _0
 * layout): d and the codes exactly as quantize_row_q8_0 above, then
 * s = sum of the 32 codes times the unrounded f32 d, stored as f16 (a NaN product,
 * from an infinite d, as 0x7E00).  Block bytes: d f16 at 0, s f16 at 2, codes at 4. */
int orc_quantize_q8_1(const float* x, uint8_t* out, int64_t n) {
  if (n < 0 || n % 32 != 0) return ORC_BAD_SHAPE;
  for (int64_t b = 0; b < n / 32; ++b) {
    const float* xb = x + 32 * b;
    uint8_t* ob = out + 36 * b;
    float amax = orc_amax(xb, 32);
    float d = amax / 127.0f;
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    int sum = 0;
    for (int j = 0; j < 32; ++j) {
      int8_t q = orc_code_q8(xb[j] * id);
      ob[4 + j] = (uint8_t)q;
      sum += q;
    }
    orc_put_u16(ob, orc_f32_to_f16(d));
    /* d is infinite only for a block holding an infinity; its codes are then all 0
     * and the product is NaN, stored as the quiet NaN 0x7E00 whatever sign the
     * host's NaN carries. */
    float p = (float)sum * d;
    orc_put_u16(ob + 2, isnan(p) ? (uint16_t)0x7E00 : orc_f32_to_f16(p));
  }
  return ORC_OK;
}

/* quantize_row_q8_K: [candle] BlockQ8K layout (d f32 at 0, 256 int8 qs at 4,
 * 16 int16 bsums at 260, each the sum of 16 consecutive qs).  The pages give
 * no scale rule for it; the Q8_0 rule over 256 elements is taken (d = amax/127
 * kept in f32, ties away from zero). */
int orc_quantize_q8_K(const float* x, uint8_t* out, int64_t n) {
  if (n < 0 || n % 256 != 0) return ORC_BAD_SHAPE;
  for (int64_t b = 0; b < n / 256; ++b) {
    const float* xb = x + 256 * b;
    uint8_t* ob = out + 292 * b;
    float amax = orc_amax(xb, 256);
    float d = amax / 127.0f;
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    orc_put_f32(ob, d);
    int8_t q[256];
    for (int j = 0; j < 256; ++j) {
      q[j] = orc_code_q8(xb[j] * id);
      ob[4 + j] = (uint8_t)q[j];
    }
    for (int k = 0; k < 16; ++k) {
      int s = 0;
      for (int i = 0; i < 16; ++i) s += q[16 * k + i];
      orc_put_u16(ob + 260 + 2 * k, (uint16_t)(int16_t)s);
    }
  }
  return ORC_OK;
}

/* quantize_row_q4_0 reference ([rml] "A worked example: Q4_0"; [cl] Example
 * 5): max = the first value of largest magnitude, sign kept (strict <); d =
 * max / -8; id = 1/d or 0; code = min(15, trunc_sat(x*id + 8.5)); byte j holds
 * element j in its low nibble and element j+16 in its high nibble. */
int orc_quantize_q4_0(const float* x, uint8_t* out, int64_t n) {
  if (n < 0 || n % 32 != 0) return ORC_BAD_SHAPE;
  for (int64_t b = 0; b < n / 32; ++b) {
    const float* xb = x + 32 * b;
    uint8_t* ob = out + 18 * b;
    float amax = 0.0f, max = 0.0f;
    for (int j = 0; j < 32; ++j) {
      if (amax < fabsf(xb[j])) {
        amax = fabsf(xb[j]);
        max = xb[j];
      }
    }
    float d = max / -8.0f;
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    orc_put_u16(ob, orc_f32_to_f16(d));
    for (int j = 0; j < 16; ++j) {
      float v0 = xb[j] * id + 8.5f;
      float v1 = xb[j + 16] * id + 8.5f;
      int32_t c0 = orc_trunc_sat(v0);
      int32_t c1 = orc_trunc_sat(v1);
      if (c0 > 15) c0 = 15;
      if (c1 > 15) c1 = 15;
      ob[2 + j] = (uint8_t)((c0 & 15) | ((c1 & 15) << 4));
    }
  }
  return ORC_OK;
}

/* quantize_row_q4_1 ([cl] Example 7): d = (max - min) / 15, id = 1/d (0 when
 * d is 0), both d and m = min stored as f16; code = min(15, trunc_sat((x - min)
 * * id + 0.5)) from the unrounded f32 d and min; nibbles ordered as Q4_0. */
int orc_quantize_q4_1(const float* x, uint8_t* out, int64_t n) {
  if (n < 0 || n % 32 != 0) return ORC_BAD_SHAPE;
  for (int64_t b = 0; b < n / 32; ++b) {
    const float* xb = x + 32 * b;
    uint8_t* ob = out + 20 * b;
    float mn = FLT_MAX, mx = -FLT_MAX;
    for (int j = 0; j < 32; ++j) {
      if (xb[j] < mn) mn = xb[j];
      if (xb[j] > mx) mx = xb[j];
    }
    float d = (mx - mn) / 15.0f;
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    orc_put_u16(ob, orc_f32_to_f16(d));
    orc_put_u16(ob + 2, orc_f32_to_f16(mn));
    for (int j = 0; j < 16; ++j) {
      float v0 = (xb[j] - mn) * id + 0.5f;
      float v1 = (xb[j + 16] - mn) * id + 0.5f;
      int32_t c0 = orc_trunc_sat(v0);
      int32_t c1 = orc_trunc_sat(v1);
      if (c0 > 15) c0 = 15;
      if (c1 > 15) c1 = 15;
      ob[4 + j] = (uint8_t)((c0 & 15) | ((c1 & 15) << 4));
    }
  }
  return ORC_OK;
}

/* quantize_row_q5_0 ([cl] Example 8): max = the first element of largest
 * magnitude (as Q4_0), d = max / -16, code = min(31, trunc_sat(x * id + 16.5));
 * the low 4 bits go to nibbles ordered as Q4_0, bit 4 of code e to bit e of
 * the 32-bit word qh (little-endian at byte 2). */
int orc_quantize_q5_0(const float* x, uint8_t* out, int64_t n) {
  if (n < 0 || n % 32 != 0) return ORC_BAD_SHAPE;
  for (int64_t b = 0; b < n / 32; ++b) {
    const float* xb = x + 32 * b;
    uint8_t* ob = out + 22 * b;
    float amax = 0.0f, max = 0.0f;
    for (int j = 0; j < 32; ++j) {
      if (amax < fabsf(xb[j])) {
        amax = fabsf(xb[j]);
        max = xb[j];
      }
    }
    float d = max / -16.0f;
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    uint32_t qh = 0;
    for (int e = 0; e < 32; ++e) {
      float v = xb[e] * id + 16.5f;
      int32_t c = orc_trunc_sat(v);
      if (c > 31) c = 31;
      qh |= (((uint32_t)c >> 4) & 1u) << e;
      if (e < 16) {
        ob[6 + e] = (uint8_t)(c & 0x0F);
      } else {
        ob[6 + e - 16] |= (uint8_t)((c & 0x0F) << 4);
      }
    }
    orc_put_u16(ob, orc_f32_to_f16(d));
    for (int k = 0; k < 4; ++k) ob[2 + k] = (uint8_t)(qh >> (8 * k));
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Element decoders: the code q of element e of one block, and its scales.   */
/* ------------------------------------------------------------------------- */

/* Q4_0 ([cl] Example 5 picture and Example 6): byte j low nibble is element
 * j, high nibble is element j+16; the stored nibble means code - 8. */
static int orc_q4_0_code(const uint8_t* blk, int e) {
  const uint8_t* qs = blk + 2;
  int nib = (e < 16) ? (qs[e] & 0x0F) : (qs[e - 16] >> 4);
  return nib - 8;
}

/* Q4_1 ([cl] Example 7): nibbles ordered as Q4_0 (qs at byte 4), code 0..15,
 * value code * d + m. */
static int orc_q4_1_code(const uint8_t* blk, int e) {
  const uint8_t* qs = blk + 4;
  return (e < 16) ? (qs[e] & 0x0F) : (qs[e - 16] >> 4);
}

/* Q5_0 ([cl] Example 8): low 4 bits as Q4_0 (qs at byte 6), bit 4 is bit e of
 * qh (bytes 2-5, little-endian); the 5-bit code means code - 16. */
static int orc_q5_0_code(const uint8_t* blk, int e) {
  const uint8_t* qs = blk + 6;
  uint32_t qh = (uint32_t)blk[2] | ((uint32_t)blk[3] << 8) | ((uint32_t)blk[4] << 16) |
                ((uint32_t)blk[5] << 24);
  int low4 = (e < 16) ? (qs[e] & 0x0F) : (qs[e - 16] >> 4);
  int bit4 = (int)((qh >> e) & 1u);
  return (low4 | (bit4 << 4)) - 16;
}

/* Q5_1 ([candle] GgmlDType table: 32 elements in 24 bytes; 块结构 prose: the _1
 * types add an f16 min m to the _0 block): d f16 @0, m f16 @2, qh u32 @4, qs[16]
 * @8 (GGUF order; the pages do not give it).  Code as Q5_0's (low 4 bits ordered
 * as Q4_0, bit 4 = bit e of qh), unsigned 0..31, value code * d + m as Q4_1. */
static int orc_q5_1_code(const uint8_t* blk, int e) {
  const uint8_t* qs = blk + 8;
  uint32_t qh = (uint32_t)blk[4] | ((uint32_t)blk[5] << 8) | ((uint32_t)blk[6] << 16) |
                ((uint32_t)blk[7] << 24);
  int low4 = (e < 16) ? (qs[e] & 0x0F) : (qs[e - 16] >> 4);
  return low4 | (int)(((qh >> e) & 1u) << 4);
}

/* Q2_K (parity unpinned: the pages give 256 elements in 84 bytes and that the
 * K-quants carry small integer sub-block scales times an f16 d; the field order and
 * bit arrangement are GGUF's, assumed here): scales[16] @0, qs[64] @16, d f16 @80,
 * dmin f16 @82.  Sub-block j is elements 16j .. 16j+15; scales[j] holds its scale in
 * the low nibble and its min in the high nibble.  Element e: half h = e / 128,
 * r = e % 128, group g = r / 32, l = r % 32; its code (0..3) is bits 2g, 2g+1 of
 * qs[32h + l].  Value d * sc_j * code - dmin * m_j, as Q4_K's with 2-bit codes. */
static int orc_q2_K_code(const uint8_t* blk, int e) {
  int h = e / 128, r = e % 128, g = r / 32, l = r % 32;
  return (blk[16 + 32 * h + l] >> (2 * g)) & 3;
}

static void orc_q2_K_scale_min(const uint8_t* blk, int j, int* sc, int* m) {
  *sc = blk[j] & 0x0F;
  *m = blk[j] >> 4;
}

/* Q3_K (parity unpinned as Q2_K: 256 elements in 110 bytes; GGUF arrangement):
 * hmask[32] @0, qs[64] @32, scales[12] @96, d f16 @108.  Element e (h, r, g, l as
 * Q2_K): low 2 bits are bits 2g, 2g+1 of qs[32h + l], bit 2 is bit 4h + g of
 * hmask[l]; the 3-bit code means code - 4 (-4..3).  Sub-block j (16 elements) has a
 * 6-bit scale meaning scale - 32: its low 4 bits are the low nibble of scales[j]
 * (j < 8) or the high nibble of scales[j - 8] (j >= 8), its high 2 bits are bits
 * 2(j/4), 2(j/4)+1 of scales[8 + j % 4].  Value d * (scale - 32) * (code - 4). */
static int orc_q3_K_code(const uint8_t* blk, int e) {
  int h = e / 128, r = e % 128, g = r / 32, l = r % 32;
  int low2 = (blk[32 + 32 * h + l] >> (2 * g)) & 3;
  int hbit = (blk[l] >> (4 * h + g)) & 1;
  return (low2 | (hbit << 2)) - 4;
}

static int orc_q3_K_scale(const uint8_t* blk, int j) {
  const uint8_t* s = blk + 96;
  int low4 = (j < 8) ? (s[j] & 0x0F) : (s[j - 8] >> 4);
  int high2 = (s[8 + j % 4] >> (2 * (j / 4))) & 3;
  return (low4 | (high2 << 4)) - 32;
}

/* Q4_K sub-block (scale, min) pair, get_scale_min_k4:
 * [candle] 块结构: "the first 4 sub-blocks' scale and min are the low 6 bits of
 * the first 8 bytes; the last 4 keep their low 4 bits in the last 4 bytes and
 * borrow their high 2 bits from the top 2 bits of the first 8 bytes".
 * [rml] "Unpacking the packed fields", element-200 trace, fixes j = 6:
 * scale = (s[10] & 0xF) | ((s[2] >> 6) << 4), min = (s[10] >> 4) | ((s[6] >> 6) << 4).
 * So scale j<4 = s[j] & 63 and min j<4 = s[j+4] & 63; for j>=4 the scale
 * takes the low nibble of s[j+4] and the top bits of s[j-4], the min the high
 * nibble of s[j+4] and the top bits of s[j]. */
static void orc_q4_K_scale_min(const uint8_t* s, int j, int* sc, int* m) {
  if (j < 4) {
    *sc = s[j] & 63;
    *m = s[j + 4] & 63;
  } else {
    *sc = (s[j + 4] & 0x0F) | ((s[j - 4] >> 6) << 4);
    *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
  }
}

/* Q4_K code of element e ([rml] element-200 trace): chunk c = e / 64, position
 * p = e % 64; p < 32 -> low nibble of qs[32c + p]; otherwise the high nibble of
 * qs[32c + p - 32].  Field offsets follow [candle]'s BlockQ4K field order:
 * d f16 @0, dmin f16 @2, scales[12] @4, qs[128] @16. */
static int orc_q4_K_code(const uint8_t* blk, int e) {
  const uint8_t* qs = blk + 16;
  int c = e / 64, p = e % 64;
  return (p < 32) ? (qs[32 * c + p] & 0x0F) : (qs[32 * c + p - 32] >> 4);
}

/* Q5_K ([candle] GgmlDType table: 256 elements in 176 bytes; 块结构 prose:
 * like Q4K it carries an f16 d and dmin and eight 32-element sub-blocks whose
 * scale and min are 6-bit integers, value d * sc_j * q - dmin * m_j).  176 bytes
 * leave, after d, dmin, the 12 bytes of eight 6-bit (scale, min) pairs and the
 * 128 bytes of low nibbles, 32 bytes: one fifth bit per element.  The pages give
 * neither the field order nor which bit belongs to which element; this takes the
 * GGUF arrangement (parity unpinned): d f16 @0, dmin f16 @2, scales[12] @4 packed
 * as Q4_K's, qh[32] @16, qs[128] @48.  Element e, chunk c = e / 64, p = e % 64:
 * low 4 bits as Q4_K's (qs[32c + p % 32], low nibble for p < 32, else high),
 * bit 4 = bit (2c + (p >= 32)) of qh[p % 32]. */
static int orc_q5_K_code(const uint8_t* blk, int e) {
  const uint8_t* qh = blk + 16;
  const uint8_t* qs = blk + 48;
  int c = e / 64, p = e % 64;
  int low4 = (p < 32) ? (qs[32 * c + p] & 0x0F) : (qs[32 * c + p - 32] >> 4);
  int bit4 = (qh[p % 32] >> (2 * c + (p >= 32 ? 1 : 0))) & 1;
  return low4 | (bit4 << 4);
}

/* Q6_K ([candle] BlockQ6K: ql[128] @0 low 4 bits, qh[64] @128 high 2 bits,
 * scales int8[16] @192, d f16 @208; 16-element sub-block j has value
 * d * sc[j] * (q - 32)).  The pages do not give which ql nibble and which qh
 * bit pair belong to element e; this takes the GGUF arrangement (parity
 * unpinned): half h = e / 128, r = e % 128, group g = r / 32, l = r % 32;
 * low4 = nibble (g < 2 ? low : high) of ql[64h + l + 32 (g & 1)];
 * high2 = (qh[32h + l] >> 2g) & 3. */
static int orc_q6_K_code(const uint8_t* blk, int e) {
  const uint8_t* ql = blk;
  const uint8_t* qh = blk + 128;
  int h = e / 128, r = e % 128, g = r / 32, l = r % 32;
  uint8_t lb = ql[64 * h + l + 32 * (g & 1)];
  int low4 = (g < 2) ? (lb & 0x0F) : (lb >> 4);
  int high2 = (qh[32 * h + l] >> (2 * g)) & 3;
  return low4 | (high2 << 4);
}

/* ------------------------------------------------------------------------- */
/* DequantizeRow ([rml] "Dequantization": one block at a time, shaped like    */
/* the format; [sipllm] dequantize_row(t, src, dst, n)).                     */
/* ------------------------------------------------------------------------- */

int orc_dequantize(int type, const uint8_t* src, float* dst, int64_t n) {
  int64_t be = orc_block_elems(type), bb = orc_block_bytes(type);
  if (be == 0) return ORC_BAD_TYPE;
  if (n < 0 || n % be != 0) return ORC_BAD_SHAPE;
  for (int64_t b = 0; b < n / be; ++b) {
    const uint8_t* blk = src + bb * b;
    float* y = dst + be * b;
    switch (type) {
      case ORC_Q8_0: { /* [cl] Example 1: value = qs[j] * d */
        float d = orc_f16_to_f32(orc_get_u16(blk));
        for (int j = 0; j < 32; ++j) y[j] = (float)(int8_t)blk[2 + j] * d;
        break;
      }
      case ORC_Q4_0: { /* [cl] Example 6: value = (nibble - 8) * d */
        float d = orc_f16_to_f32(orc_get_u16(blk));
        for (int e = 0; e < 32; ++e) y[e] = (float)orc_q4_0_code(blk, e) * d;
        break;
      }
      case ORC_Q4_1: { /* [cl] Example 7: value = code * d + m */
        float d = orc_f16_to_f32(orc_get_u16(blk));
        float m = orc_f16_to_f32(orc_get_u16(blk + 2));
        for (int e = 0; e < 32; ++e) y[e] = (float)orc_q4_1_code(blk, e) * d + m;
        break;
      }
      case ORC_Q5_1: { /* as Q4_1 with the 5-bit code: value = code * d + m */
        float d = orc_f16_to_f32(orc_get_u16(blk));
        float m = orc_f16_to_f32(orc_get_u16(blk + 2));
        for (int e = 0; e < 32; ++e) y[e] = (float)orc_q5_1_code(blk, e) * d + m;
        break;
      }
      case ORC_Q5_0: { /* [cl] Example 8: value = (code - 16) * d */
        float d = orc_f16_to_f32(orc_get_u16(blk));
        for (int e = 0; e < 32; ++e) y[e] = (float)orc_q5_0_code(blk, e) * d;
        break;
      }
      case ORC_Q2_K: { /* d * sc_j * q - dmin * m_j, 16-element j (reading above) */
        float d = orc_f16_to_f32(orc_get_u16(blk + 80));
        float dmin = orc_f16_to_f32(orc_get_u16(blk + 82));
        for (int e = 0; e < 256; ++e) {
          int sc, m;
          orc_q2_K_scale_min(blk, e / 16, &sc, &m);
          y[e] = d * (float)sc * (float)orc_q2_K_code(blk, e) - dmin * (float)m;
        }
        break;
      }
      case ORC_Q3_K: { /* d * (scale_j - 32) * (code - 4), 16-element j */
        float d = orc_f16_to_f32(orc_get_u16(blk + 108));
        for (int e = 0; e < 256; ++e)
          y[e] = d * (float)orc_q3_K_scale(blk, e / 16) * (float)orc_q3_K_code(blk, e);
        break;
      }
      case ORC_Q4_K: { /* [rml] trace: x = d * scale * q - dmin * min */
        float d = orc_f16_to_f32(orc_get_u16(blk));
        float dmin = orc_f16_to_f32(orc_get_u16(blk + 2));
        for (int e = 0; e < 256; ++e) {
          int sc, m;
          orc_q4_K_scale_min(blk + 4, e / 32, &sc, &m);
          int q = orc_q4_K_code(blk, e);
          y[e] = d * (float)sc * (float)q - dmin * (float)m;
        }
        break;
      }
      case ORC_Q5_K: { /* as Q4_K with the 5-bit code */
        float d = orc_f16_to_f32(orc_get_u16(blk));
        float dmin = orc_f16_to_f32(orc_get_u16(blk + 2));
        for (int e = 0; e < 256; ++e) {
          int sc, m;
          orc_q4_K_scale_min(blk + 4, e / 32, &sc, &m);
          int q = orc_q5_K_code(blk, e);
          y[e] = d * (float)sc * (float)q - dmin * (float)m;
        }
        break;
      }
      case ORC_Q6_K: { /* [candle] BlockQ6K: d * sc[j] * (q - 32) */
        float d = orc_f16_to_f32(orc_get_u16(blk + 208));
        const int8_t* sc = (const int8_t*)(blk + 192);
        for (int e = 0; e < 256; ++e) {
          int q = orc_q6_K_code(blk, e);
          y[e] = d * (float)sc[e / 16] * (float)(q - 32);
        }
        break;
      }
      case ORC_Q8_1: { /* d * q, as Q8_0 (test helper: activations) */
        float d = orc_f16_to_f32(orc_get_u16(blk));
        for (int j = 0; j < 32; ++j) y[j] = (float)(int8_t)blk[4 + j] * d;
        break;
      }
      case ORC_Q8_K: { /* [candle] BlockQ8K: d * q (test helper: activations) */
        float d = orc_get_f32(blk);
        for (int j = 0; j < 256; ++j) y[j] = d * (float)(int8_t)blk[4 + j];
        break;
      }
      default:
        return ORC_BAD_TYPE;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* VecDot ([rml] "Quantized dot products", "Kernels and references": every    */
/* product inside a block is an exact int32 sum, computed here element by     */
/* element as VecDotRef does; only the block scales are float).              */
/* ------------------------------------------------------------------------- */

/* Integer quantities kept per weight block: one s for Q8_0, Q4_0, Q5_0, Q4_1,
 * Q5_1, Q3_K, Q6_K; the pair (S_q, S_m) for Q2_K, Q4_K and Q5_K (scale sum and min
 * sum). */
int64_t orc_sums_per_block(int weight_type) {
  switch (weight_type) {
    case ORC_Q8_0:
    case ORC_Q4_0:
    case ORC_Q5_0:
    case ORC_Q4_1:
    case ORC_Q5_1:
    case ORC_Q3_K:
    case ORC_Q6_K:
      return 1;
    case ORC_Q2_K:
    case ORC_Q4_K:
    case ORC_Q5_K:
      return 2;
    default:
      return 0;
  }
}

/* Exact per-block integer sums of one weight row against its paired act row. */
static int orc_block_ints(int wt, const uint8_t* wb, const uint8_t* xb, int32_t* out) {
  switch (wt) {
    case ORC_Q8_0: { /* [cl] Example 10 step 1: s = sum of the 32 code products */
      int32_t s = 0;
      for (int j = 0; j < 32; ++j) s += (int32_t)(int8_t)wb[2 + j] * (int32_t)(int8_t)xb[2 + j];
      out[0] = s;
      return ORC_OK;
    }
    case ORC_Q4_0: { /* [cl] Example 11: low nibble x a_j, high nibble x a_{j+16} */
      int32_t s = 0;
      for (int e = 0; e < 32; ++e) s += (int32_t)orc_q4_0_code(wb, e) * (int32_t)(int8_t)xb[2 + e];
      out[0] = s;
      return ORC_OK;
    }
    case ORC_Q5_0: { /* as Q4_0, with the 5-bit code (minus 16) of each element */
      int32_t s = 0;
      for (int e = 0; e < 32; ++e) s += (int32_t)orc_q5_0_code(wb, e) * (int32_t)(int8_t)xb[2 + e];
      out[0] = s;
      return ORC_OK;
    }
    case ORC_Q4_1:
    case ORC_Q5_1: { /* s = sum of code x a over the 32 elements (codes 0..15 / 0..31,
                      * unsigned: the minimum is added by the float step) */
      int32_t s = 0;
      for (int e = 0; e < 32; ++e) {
        int q = (wt == ORC_Q4_1) ? orc_q4_1_code(wb, e) : orc_q5_1_code(wb, e);
        s += (int32_t)q * (int32_t)(int8_t)xb[4 + e];
      }
      out[0] = s;
      return ORC_OK;
    }
    case ORC_Q4_K:
    case ORC_Q5_K: {
      /* S_q = sum_j sc_j * (sum_{e in j} q_e a_e);  S_m = sum_j m_j * (sum_{e in j} a_e).
       * [rml]: the sub-block min term is min * sum(a); the reference sums it
       * element by element, the kernels take sum(a) over 32 activations as two
       * stored 16-sums (bsums).  Both routes are computed and must agree. */
      const uint8_t* a = xb + 4;
      int32_t sq = 0, sm = 0, sm_bsums = 0;
      for (int j = 0; j < 8; ++j) {
        int sc, m;
        orc_q4_K_scale_min(wb + 4, j, &sc, &m);
        int32_t s = 0, sa = 0;
        for (int e = 32 * j; e < 32 * j + 32; ++e) {
          int q = (wt == ORC_Q4_K) ? orc_q4_K_code(wb, e) : orc_q5_K_code(wb, e);
          s += (int32_t)q * (int32_t)(int8_t)a[e];
          sa += (int32_t)(int8_t)a[e];
        }
        sq += sc * s;
        sm += m * sa;
        int32_t bs = (int32_t)orc_get_i16(xb + 260 + 2 * (2 * j)) +
                     (int32_t)orc_get_i16(xb + 260 + 2 * (2 * j + 1));
        sm_bsums += m * bs;
      }
      if (sm != sm_bsums) return ORC_INCONSISTENT;
      out[0] = sq;
      out[1] = sm;
      return ORC_OK;
    }
    case ORC_Q2_K: {
      /* S_q = sum_j sc_j (sum_{e in j} q_e a_e), S_m = sum_j m_j (sum_{e in j} a_e) over
       * the 16-element sub-blocks; sum a over one sub-block is one stored bsum of the
       * Q8_K block ([candle] 块结构: bsums serve the min term).  Both routes are
       * computed and must agree. */
      const uint8_t* a = xb + 4;
      int32_t sq = 0, sm = 0, sm_bsums = 0;
      for (int j = 0; j < 16; ++j) {
        int sc, m;
        orc_q2_K_scale_min(wb, j, &sc, &m);
        int32_t s = 0, sa = 0;
        for (int e = 16 * j; e < 16 * j + 16; ++e) {
          s += (int32_t)orc_q2_K_code(wb, e) * (int32_t)(int8_t)a[e];
          sa += (int32_t)(int8_t)a[e];
        }
        sq += sc * s;
        sm += m * sa;
        sm_bsums += m * (int32_t)orc_get_i16(xb + 260 + 2 * j);
      }
      if (sm != sm_bsums) return ORC_INCONSISTENT;
      out[0] = sq;
      out[1] = sm;
      return ORC_OK;
    }
    case ORC_Q3_K: { /* S = sum_j (scale_j - 32) * sum_{e in j} (code_e - 4) a_e */
      const uint8_t* a = xb + 4;
      int32_t S = 0;
      for (int j = 0; j < 16; ++j) {
        int32_t s = 0;
        for (int e = 16 * j; e < 16 * j + 16; ++e) s += (int32_t)orc_q3_K_code(wb, e) * (int32_t)(int8_t)a[e];
        S += (int32_t)orc_q3_K_scale(wb, j) * s;
      }
      out[0] = S;
      return ORC_OK;
    }
    case ORC_Q6_K: { /* S = sum_j sc_j * sum_{e in j} (q_e - 32) a_e, 16-element j */
      const uint8_t* a = xb + 4;
      const int8_t* sc = (const int8_t*)(wb + 192);
      int32_t S = 0;
      for (int j = 0; j < 16; ++j) {
        int32_t s = 0;
        for (int e = 16 * j; e < 16 * j + 16; ++e)
          s += (int32_t)(orc_q6_K_code(wb, e) - 32) * (int32_t)(int8_t)a[e];
        S += (int32_t)sc[j] * s;
      }
      out[0] = S;
      return ORC_OK;
    }
    default:
      return ORC_BAD_TYPE;
  }
}

/* The one float step per block ([rml] "Kernels and references": kernels and
 * references share it).  Q8_0/Q4_0: c = s * (dw * dx) with both f16 scales
 * ([cl] Example 10 step 2).  Q4_1, Q5_1 against Q8_1: every weight value is
 * code * dw + mw and every activation dx * a, so the block's sum is
 * dw dx sum(code a) + mw dx sum(a) = s * (dw * dx) + mw * sx, with sx the Q8_1
 * block's stored f16 dx * sum(a).  Q4_K, Q5_K: c = (dx*d) * S_q - (dx*dmin) * S_m.
 * Q2_K as Q4_K, Q3_K as Q6_K (each with its own d / dmin offsets).
 * Q6_K: c = (dx*d) * S.  dx of Q8_K is f32 ([candle] BlockQ8K). */
static float orc_block_float(int wt, const uint8_t* wb, const uint8_t* xb, const int32_t* s) {
  switch (wt) {
    case ORC_Q8_0:
    case ORC_Q4_0:
    case ORC_Q5_0: {
      float dw = orc_f16_to_f32(orc_get_u16(wb));
      float dx = orc_f16_to_f32(orc_get_u16(xb));
      return (float)s[0] * (dw * dx);
    }
    case ORC_Q4_1:
    case ORC_Q5_1: {
      float dw = orc_f16_to_f32(orc_get_u16(wb));
      float mw = orc_f16_to_f32(orc_get_u16(wb + 2));
      float dx = orc_f16_to_f32(orc_get_u16(xb));
      float sx = orc_f16_to_f32(orc_get_u16(xb + 2));
      return (float)s[0] * (dw * dx) + mw * sx;
    }
    case ORC_Q4_K:
    case ORC_Q5_K: {
      float dx = orc_get_f32(xb);
      float d = orc_f16_to_f32(orc_get_u16(wb));
      float dmin = orc_f16_to_f32(orc_get_u16(wb + 2));
      return (dx * d) * (float)s[0] - (dx * dmin) * (float)s[1];
    }
    case ORC_Q6_K: {
      float dx = orc_get_f32(xb);
      float d = orc_f16_to_f32(orc_get_u16(wb + 208));
      return (dx * d) * (float)s[0];
    }
    case ORC_Q2_K: { /* as Q4_K, d and dmin at bytes 80 and 82 */
      float dx = orc_get_f32(xb);
      float d = orc_f16_to_f32(orc_get_u16(wb + 80));
      float dmin = orc_f16_to_f32(orc_get_u16(wb + 82));
      return (dx * d) * (float)s[0] - (dx * dmin) * (float)s[1];
    }
    case ORC_Q3_K: { /* as Q6_K, d at byte 108 */
      float dx = orc_get_f32(xb);
      float d = orc_f16_to_f32(orc_get_u16(wb + 108));
      return (dx * d) * (float)s[0];
    }
    default:
      return NAN;
  }
}

/* The magnitude a block contributes to the tolerance scale: the sum of the
 * absolute values of the float terms its step adds ([cl] Example 10 measures
 * error against the sum of |a*b| over the terms).  One term for Q8_0, Q4_0,
 * Q5_0, Q3_K and Q6_K; for Q4_1 and Q5_1 the code term s*(dw*dx) and the minimum
 * term mw*sx; for Q2_K, Q4_K and Q5_K the scale term (dx*d)*S_q and the min term
 * (dx*dmin)*S_m.  Two-term steps can cancel in c while each term is rounded on
 * its own. */
static double orc_block_l1(int wt, const uint8_t* wb, const uint8_t* xb, const int32_t* s, float c) {
  if (wt == ORC_Q4_1 || wt == ORC_Q5_1) {
    float dw = orc_f16_to_f32(orc_get_u16(wb));
    float mw = orc_f16_to_f32(orc_get_u16(wb + 2));
    float dx = orc_f16_to_f32(orc_get_u16(xb));
    float sx = orc_f16_to_f32(orc_get_u16(xb + 2));
    return fabs((double)((float)s[0] * (dw * dx))) + fabs((double)(mw * sx));
  }
  if (wt != ORC_Q4_K && wt != ORC_Q5_K && wt != ORC_Q2_K) return fabs((double)c);
  int off = (wt == ORC_Q2_K) ? 80 : 0; /* d, dmin */
  float dx = orc_get_f32(xb);
  float d = orc_f16_to_f32(orc_get_u16(wb + off));
  float dmin = orc_f16_to_f32(orc_get_u16(wb + off + 2));
  return fabs((double)((dx * d) * (float)s[0])) + fabs((double)((dx * dmin) * (float)s[1]));
}

int orc_block_sums(int wt, const uint8_t* w, const uint8_t* xq, int64_t n, int32_t* sums) {
  int at = orc_act_type(wt);
  if (at < 0) return ORC_BAD_PAIR;
  int64_t be = orc_block_elems(wt), bw = orc_block_bytes(wt), bx = orc_block_bytes(at);
  if (n < 0 || n % be != 0) return ORC_BAD_SHAPE;
  int64_t k = orc_sums_per_block(wt);
  for (int64_t b = 0; b < n / be; ++b) {
    int rc = orc_block_ints(wt, w + bw * b, xq + bx * b, sums + k * b);
    if (rc != ORC_OK) return rc;
  }
  return ORC_OK;
}

/* VecDot(weight, w, x, n): y = sum over blocks of the float step, accumulated
 * in f32 in block order ([cl] Example 10: `sumf += ...`).  l1 (optional)
 * receives, in f64, the sum over blocks of the absolute float terms of each step
 * (|c_b| for the one-term formats, |scale term| + |min term| for Q4_K and Q5_K):
 * the scale the output tolerance is taken against ([cl] Example 10 reports error
 * against the sum of |a*b|). */
int orc_vec_dot(int wt, const uint8_t* w, const uint8_t* xq, int64_t n, float* out, double* l1) {
  int at = orc_act_type(wt);
  if (at < 0) return ORC_BAD_PAIR;
  int64_t be = orc_block_elems(wt), bw = orc_block_bytes(wt), bx = orc_block_bytes(at);
  if (n < 0 || n % be != 0) return ORC_BAD_SHAPE;
  float sumf = 0.0f;
  double sabs = 0.0;
  int32_t s[2];
  for (int64_t b = 0; b < n / be; ++b) {
    int rc = orc_block_ints(wt, w + bw * b, xq + bx * b, s);
    if (rc != ORC_OK) return rc;
    float c = orc_block_float(wt, w + bw * b, xq + bx * b, s);
    sumf += c;
    sabs += orc_block_l1(wt, w + bw * b, xq + bx * b, s, c);
  }
  *out = sumf;
  if (l1) *l1 = sabs;
  return ORC_OK;
}

/* GEMV ([sipllm] matmul_quant: W is [n_out, n_in] row-major, whole blocks per
 * row; the activation is quantized once and reused by every row).  xq holds
 * ncols activation rows of n_in elements each; y is [ncols][n_out]. */
int orc_gemv(int wt, const uint8_t* W, int64_t n_out, int64_t n_in, const uint8_t* xq,
             int64_t ncols, float* y, double* l1) {
  int at = orc_act_type(wt);
  if (at < 0) return ORC_BAD_PAIR;
  int64_t rw = orc_row_bytes(wt, n_in), rx = orc_row_bytes(at, n_in);
  if (rw == 0 || n_out < 0 || ncols < 0) return ORC_BAD_SHAPE;
  for (int64_t c = 0; c < ncols; ++c) {
    for (int64_t r = 0; r < n_out; ++r) {
      int rc = orc_vec_dot(wt, W + rw * r, xq + rx * c, n_in, y + c * n_out + r,
                           l1 ? l1 + c * n_out + r : NULL);
      if (rc != ORC_OK) return rc;
    }
  }
  return ORC_OK;
}

/* The per-block integer sums of a whole GEMV: orc_block_sums for every (column,
 * row), laid out [ncols][n_out][n_in / block][sums per block]. */
int orc_gemv_block_sums(int wt, const uint8_t* W, int64_t n_out, int64_t n_in, const uint8_t* xq,
                        int64_t ncols, int32_t* sums) {
  int at = orc_act_type(wt);
  if (at < 0) return ORC_BAD_PAIR;
  int64_t rw = orc_row_bytes(wt, n_in), rx = orc_row_bytes(at, n_in);
  if (rw == 0 || n_out < 0 || ncols < 0) return ORC_BAD_SHAPE;
  int64_t per_row = (n_in / orc_block_elems(wt)) * orc_sums_per_block(wt);
  for (int64_t c = 0; c < ncols; ++c) {
    for (int64_t r = 0; r < n_out; ++r) {
      int rc = orc_block_sums(wt, W + rw * r, xq + rx * c, n_in, sums + (c * n_out + r) * per_row);
      if (rc != ORC_OK) return rc;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* The gated activation between an FFN's gate / up and down projections.      */
/* The pages stop at the products; the 7B-shape layers that the FFN workload   */
/* follows combine them as SwiGLU: h = silu(g) * u with silu(v) = v * sigmoid(v) */
/* = v / (1 + e^-v).  Evaluated in double from the f32 gate and up outputs.    */
/* ------------------------------------------------------------------------- */

int orc_swiglu(const float* g, const float* u, int64_t n, double* h) {
  if (n < 0) return ORC_BAD_SHAPE;
  for (int64_t i = 0; i < n; ++i) {
    double v = (double)g[i];
    h[i] = v / (1.0 + exp(-v)) * (double)u[i];
  }
  return ORC_OK;
}
