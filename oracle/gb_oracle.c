/*
 * gb_oracle.c — the CPU oracle (test infrastructure; see gb_oracle.h).
 *
 * Written from the definitions, one element at a time, for a reader to check
 * by eye.  Rounding decisions are made by comparing the exact value with the
 * exact midpoint of its two neighbouring codes (both held exactly in double);
 * nothing here is a fast bit trick.
 *
 * How each function is pinned to something other than itself (the CPU tests
 * named in brackets):
 *   or_reduce_sum         k copies of 1.0 give k; the README's four-rank
 *                         simulation example gives 10.0; exact integer sums;
 *                         a rank-order case where the left fold differs from
 *                         any other order; exact rational brute force
 *                         [test_oracle_sum.py, test_golden.py].
 *   or_bf16_encode_one    torch's float32->bfloat16 cast on every non-NaN
 *                         float32 (all 2^32 bit patterns); round trip of all
 *                         2^16 codes; even code at every midpoint
 *                         [test_oracle_bf16.py].  The NaN rule is this
 *                         library's convention: parity unpinned for NaN.
 *   or_e4m3_*             torch's float8_e4m3fn decode of all 256 codes;
 *                         torch's saturating cast (clamp to +-448, then cast)
 *                         on every non-NaN float32; exact brute force over
 *                         the 253 finite codes [test_oracle_fp8.py].
 *   or_block_absmax,      brute force over permutations; the block's largest
 *   or_block_scale        element encodes to 448; the power-of-two scale is
 *                         the smallest that fits (checked against exact
 *                         powers) [test_oracle_fp8.py].
 *   or_fp8_quantize_one   exact rational division then exact nearest-code
 *                         search [test_oracle_fp8.py]; half-ulp bound.
 *   or_decode_accumulate  equals the plain sum on exactly representable
 *                         data; error bound; k=1 equals the decode
 *                         [test_oracle_decode.py].
 *   or_bucket_allreduce   equals the whole-buffer encode + decode when
 *                         buckets are multiples of 256 [test_oracle_decode.py].
 *   or_reduce (AVG, MAX,  AVG: exact rational RN(sum / d) on exact sums; k
 *   MIN)                  copies of x averaged over k give x.  MAX/MIN:
 *                         brute force against an exact order with the
 *                         IEEE 754-2019 zero and NaN rules; rank-permutation
 *                         invariance [test_oracle_ops.py].
 *   or_reduce_typed       f16 / bf16 sums and averages against torch's CPU
 *                         half and bfloat16 arithmetic and exact rational
 *                         rounding; f64 against exact rationals; integer
 *                         sums against numpy's wrapping arithmetic; MAX/MIN
 *                         by brute force [test_oracle_dtypes.py].
 *   or_encode_typed,      bfloat16 input through the bf16 codec is the
 *   or_decode_sum_typed,  identity; every other input equals the binary32
 *   or_bucket_allreduce_  path fed by torch's / numpy's own conversions, and
 *   typed                 the typed total equals torch's rounding of the
 *                         binary32 total; no codec is the typed SUM
 *                         [test_oracle_typed_codec.py].
 *   or_encode_*_ef        with a zero residual the payload is the plain
 *                         encode; the bf16 residual is exact and within half
 *                         an ulp; exact rational step-by-step simulation with
 *                         brute-force rounding; over repeated steps the
 *                         running mean of the decoded values converges to the
 *                         input, which fails for a wrong sign or a dropped
 *                         feedback term [test_oracle_ef.py].
 *   canonical NaN         every NaN the float32 arithmetic delivers is
 *                         0x7FC00000 whatever the host's default NaN: cases
 *                         built from invalid operations (negative default
 *                         NaN on x86) and from NaNs of both signs with
 *                         payloads, copies keeping their bits
 *                         [test_oracle_nan.py].
 * The pages fix none of the NaN and Inf conventions (NaN sign and payload,
 * Inf scale); they are readings taken here, stated at each function and
 * pinned to their own definitions: parity with the pages unpinned for
 * non-finite inputs.
 */
#include "gb_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* No contraction into fused multiply-add: the build passes -ffp-contract=off. */

static uint32_t float_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  return u;
}

static float bits_float(uint32_t u) {
  float x;
  memcpy(&x, &u, sizeof x);
  return x;
}

/* ------------------------------------------------------------------------
 * Canonical NaN (reading taken).  README "Bridge compression": every rank
 * ends with the same bits, whichever vendor's GPU ran the kernels.  IEEE
 * 754-2019 fixes neither the sign nor the payload of the NaN an operation
 * delivers: an invalid operation (0 * Inf, Inf - Inf) gives the platform's
 * default NaN, positive on AMD GPUs and negative on x86, and which input
 * NaN an operation passes on is only a recommendation (6.2.3), so those
 * bits would depend on the machine.  Every NaN that the float32 arithmetic
 * of this method delivers -- a rank-order sum, an AVG quotient, a MAX or
 * MIN, a decoded-and-added total, the error-feedback value y = x + residual
 * and the new residual -- is therefore stored as the one quiet NaN
 * 0x7FC00000 (sign 0, only the quiet bit of the fraction set).  A result
 * that no arithmetic produced keeps its bits: a sum or MAX / MIN of one rank
 * is a copy, and the decode of one bf16 payload (no accumulation) is the
 * exact widening of its codes; so do the conversions, an encoder's code for
 * a NaN input keeping the NaN's own sign and payload bits as stated where
 * it is defined.
 * --------------------------------------------------------------------- */
#define OR_CANONICAL_NAN 0x7FC00000u

static float canonical(float v) { return isnan(v) ? bits_float(OR_CANONICAL_NAN) : v; }

/* ------------------------------------------------------------------------
 * Fixed-order sum.  README "How it works": the leaders all-reduce the island
 * sums, so the leader holds the SUM of the k contributions; "API": all_reduce
 * with SUM.  The pages leave the order open (the Rust bridges add in ring
 * order, Gloo in its own); reading taken: a left fold over ranks 0..k-1
 * starting from rank 0's value (not from +0, so a sum of -0 values stays -0).
 * --------------------------------------------------------------------- */
void or_reduce_sum(float* out, const float* const* x, int k, size_t n) {
  for (size_t i = 0; i < n; i++) {
    float acc = x[0][i];
    for (int r = 1; r < k; r++) {
      acc = acc + x[r][i];
    }
    out[i] = k == 1 ? acc : canonical(acc);
  }
}

/* ------------------------------------------------------------------------
 * bf16.  README "Bridge compression": the bf16 payload is half the size of
 * float32.  bf16 is binary32
 * with the low 16 bits of the encoding dropped: 1 sign, 8 exponent and 7
 * fraction bits.  Encoding takes the nearest bf16 value, the even code at a
 * midpoint; values beyond the largest finite bf16 round to Inf exactly as
 * IEEE rounding with an unbounded exponent would (the code after the largest
 * finite one, 0x7F80, stands for 2^128 in that comparison).
 * --------------------------------------------------------------------- */
float or_bf16_decode_one(uint16_t c) { return bits_float((uint32_t)c << 16); }

/* Magnitude value of a non-negative bf16 code, exact in double. */
static double bf16_magnitude(uint32_t code) {
  if (code == 0x7F80u) return ldexp(1.0, 128); /* rounding boundary of Inf */
  return (double)bits_float(code << 16);
}

uint16_t or_bf16_encode_one(float x) {
  uint32_t u = float_bits(x);
  if (isnan(x)) {
    /* Reading taken: keep sign and top payload bits, force the quiet bit. */
    return (uint16_t)((u >> 16) | 0x0040u);
  }
  uint32_t sign = (u >> 16) & 0x8000u;
  uint32_t mag = u & 0x7FFFFFFFu;
  uint32_t below = mag >> 16; /* largest bf16 magnitude code <= |x| */
  if ((mag & 0xFFFFu) == 0) return (uint16_t)(sign | below); /* exact */
  uint32_t above = below + 1; /* smallest bf16 magnitude code > |x| */
  double m = fabs((double)x);
  double mid = (bf16_magnitude(below) + bf16_magnitude(above)) / 2.0;
  uint32_t code;
  if (m < mid) {
    code = below;
  } else if (m > mid) {
    code = above;
  } else {
    code = (below % 2 == 0) ? below : above;
  }
  return (uint16_t)(sign | code);
}

void or_encode_bf16(uint16_t* codes, const float* x, size_t n) {
  for (size_t i = 0; i < n; i++) codes[i] = or_bf16_encode_one(x[i]);
}

/* ------------------------------------------------------------------------
 * OCP E4M3.  README "Bridge compression": fp8 is OCP E4M3.  Per the OCP 8-bit
 * floating point format: 1 sign bit, 4 exponent bits with bias 7, 3 fraction
 * bits; exponent field 0 holds subnormals f * 2^-9; no infinities; the codes
 * S.1111.111 are NaN, so the largest finite magnitude is 0x7E = 1.75 * 2^8 =
 * 448.  Magnitude codes 0..0x7E are increasing in value.
 * --------------------------------------------------------------------- */
static double e4m3_magnitude(unsigned code) { /* code in 0..0x7E */
  unsigned e = code >> 3;
  unsigned f = code & 7u;
  if (e == 0) return ldexp((double)f, -9);
  return ldexp(1.0 + (double)f / 8.0, (int)e - 7);
}

float or_e4m3_decode_one(uint8_t c) {
  unsigned mag = c & 0x7Fu;
  int negative = (c & 0x80u) != 0;
  if (mag == 0x7Fu) return negative ? -NAN : NAN;
  float v = (float)e4m3_magnitude(mag); /* exact: 4 significant bits */
  return negative ? -v : v;
}

uint8_t or_e4m3_encode_one(float v, int negative) {
  unsigned sign = negative ? 0x80u : 0u;
  if (isnan(v)) return (uint8_t)(0x7Fu | sign);
  double m = fabs((double)v);
  /* Saturate (reading taken): every magnitude at or above 448, Inf included,
   * gives 448, so a finite input never becomes NaN. */
  if (m >= 448.0) return (uint8_t)(0x7Eu | sign);
  /* Binary search for the largest code `below` with value <= m. */
  unsigned lo = 0, hi = 0x7E; /* value(lo) <= m < value(hi) */
  while (hi - lo > 1) {
    unsigned mid = (lo + hi) / 2;
    if (e4m3_magnitude(mid) <= m) {
      lo = mid;
    } else {
      hi = mid;
    }
  }
  unsigned below = lo, above = lo + 1;
  double midpoint = (e4m3_magnitude(below) + e4m3_magnitude(above)) / 2.0;
  unsigned code;
  if (m < midpoint) {
    code = below;
  } else if (m > midpoint) {
    code = above;
  } else {
    code = (below % 2 == 0) ? below : above;
  }
  return (uint8_t)(code | sign);
}

void or_e4m3_encode_array(uint8_t* codes, const float* v, size_t n) {
  for (size_t i = 0; i < n; i++) {
    codes[i] = or_e4m3_encode_one(v[i], signbit(v[i]) != 0);
  }
}

void or_e4m3_decode_array(float* v, const uint8_t* codes, size_t n) {
  for (size_t i = 0; i < n; i++) v[i] = or_e4m3_decode_one(codes[i]);
}

/* ------------------------------------------------------------------------
 * Block scale.  README "Bridge compression": one scale per 256 values, with
 * the precision stated relative to the largest value of the block, so the
 * scale comes from the block's largest magnitude a.  NaN elements are skipped (reading taken);
 * an Inf element makes a = Inf.
 *   ABSMAX_DIV_448: s = RN(a / 448), so the largest element lands on 448.
 *   POW2 (the README's scale that is a power of two): the smallest 2^e, e >= -149 so
 *   that 2^e is a float, with a <= 448 * 2^e: nothing saturates.
 * Zero block: s = 0 (ABSMAX_DIV_448; the quotient step is then skipped) and
 * s = 1 (POW2).  Inf block: s = Inf in both modes.
 * --------------------------------------------------------------------- */
float or_block_absmax(const float* x, size_t len) {
  float a = 0.0f;
  for (size_t i = 0; i < len; i++) {
    float m = fabsf(x[i]);
    if (!isnan(m) && m > a) a = m;
  }
  return a;
}

float or_block_scale(float a, int mode) {
  if (mode == OR_SCALE_ABSMAX_DIV_448) return a / 448.0f;
  /* OR_SCALE_POW2.  No block's absmax is NaN (NaN elements are skipped); a
   * NaN argument gives NaN rather than a search that never ends. */
  if (isnan(a)) return a;
  if (a == 0.0f) return 1.0f;
  if (isinf(a)) return INFINITY;
  for (int e = -149;; e++) {
    if ((double)a <= 448.0 * ldexp(1.0, e)) return ldexpf(1.0f, e);
  }
}

uint8_t or_fp8_quantize_one(float x, float s) {
  int negative = signbit(x) != 0;
  if (isnan(x)) return or_e4m3_encode_one(x, negative);
  float v = (s == 0.0f) ? x : x / s; /* correctly rounded binary32 divide */
  return or_e4m3_encode_one(v, negative);
}

void or_encode_fp8(uint8_t* codes, float* scales, const float* x, size_t n,
                   int mode) {
  size_t nblocks = (n + 255) / 256;
  for (size_t b = 0; b < nblocks; b++) {
    size_t start = b * 256;
    size_t len = (n - start < 256) ? n - start : 256;
    float s = or_block_scale(or_block_absmax(x + start, len), mode);
    scales[b] = s;
    for (size_t i = 0; i < len; i++) {
      codes[start + i] = or_fp8_quantize_one(x[start + i], s);
    }
  }
}

/* ------------------------------------------------------------------------
 * Decode and accumulate.  README "Bridge compression": after the bridge step
 * the leaders dequantize the payloads and add them in float32, and every rank
 * ends with the same bits.  Reading taken: every rank's payload is decoded
 * (the leader's own included) and added in rank order; an fp8 value is
 * RN(code value * scale), rounded before the add (no fused multiply-add).
 * --------------------------------------------------------------------- */
static float decoded_value(const void* codes, const float* scales, size_t i,
                           int codec) {
  if (codec == OR_CODEC_NONE) return ((const float*)codes)[i];
  if (codec == OR_CODEC_BF16) {
    return or_bf16_decode_one(((const uint16_t*)codes)[i]);
  }
  float q = or_e4m3_decode_one(((const uint8_t*)codes)[i]);
  float s = scales[i / 256];
  return q * s;
}

void or_decode_accumulate(float* acc, const void* const* codes,
                          const float* const* scales, int k, size_t n,
                          int codec, int accumulate) {
  for (size_t i = 0; i < n; i++) {
    const float* sc0 = scales ? scales[0] : NULL;
    float a;
    int r0;
    if (accumulate) {
      a = acc[i];
      r0 = 0;
    } else {
      a = decoded_value(codes[0], sc0, i, codec);
      r0 = 1;
    }
    for (int r = r0; r < k; r++) {
      const float* sc = scales ? scales[r] : NULL;
      float v = decoded_value(codes[r], sc, i, codec);
      a = a + v;
    }
    /* one bf16 or uncompressed payload, nothing added: a widening or a copy */
    int copied = k == 1 && !accumulate && codec != OR_CODEC_FP8;
    acc[i] = copied ? a : canonical(a);
  }
}

/* ------------------------------------------------------------------------
 * Bucket stream.  README "DistributedDataParallel": each gradient bucket is
 * one all_reduce.  Per bucket: encode each rank's slice (blocks restart at
 * the bucket start), then decode and accumulate the k payloads into out.
 * --------------------------------------------------------------------- */
void or_bucket_allreduce(float* out, void* const* codes, float* const* scales,
                         const float* const* x, int k, size_t n,
                         size_t bucket_elems, int codec, int mode) {
  const float* xs[64];
  const void* cs[64];
  const float* ss[64];
  size_t scale_base = 0;
  for (size_t start = 0; start < n; start += bucket_elems) {
    size_t len = (n - start < bucket_elems) ? n - start : bucket_elems;
    for (int r = 0; r < k; r++) xs[r] = x[r] + start;
    if (codec == OR_CODEC_NONE) {
      or_reduce_sum(out + start, xs, k, len);
      continue;
    }
    for (int r = 0; r < k; r++) {
      if (codec == OR_CODEC_BF16) {
        uint16_t* c = (uint16_t*)codes[r] + start;
        or_encode_bf16(c, xs[r], len);
        cs[r] = c;
        ss[r] = NULL;
      } else {
        uint8_t* c = (uint8_t*)codes[r] + start;
        or_encode_fp8(c, scales[r] + scale_base, xs[r], len, mode);
        cs[r] = c;
        ss[r] = scales[r] + scale_base;
      }
    }
    or_decode_accumulate(out + start, cs, codec == OR_CODEC_FP8 ? ss : NULL, k,
                         len, codec, 0);
    scale_base += (len + 255) / 256;
  }
}

/* ------------------------------------------------------------------------
 * Error feedback.  README "Bridge compression": each bridge member keeps an
 * error-feedback residual per buffer, so the rounding error of one step is
 * carried into the next instead of accumulating.  Reading taken (the usual
 * error-feedback step, in binary32): y = x + residual; the payload encodes y
 * exactly as the plain encoders do (for fp8 the block scale comes from y);
 * the new residual is y minus the value the payload decodes to.
 * --------------------------------------------------------------------- */
void or_encode_bf16_ef(uint16_t* codes, float* residual, const float* x, size_t n) {
  for (size_t i = 0; i < n; i++) {
    float y = canonical(x[i] + residual[i]);
    codes[i] = or_bf16_encode_one(y);
    residual[i] = canonical(y - or_bf16_decode_one(codes[i]));
  }
}

void or_encode_fp8_ef(uint8_t* codes, float* scales, float* residual,
                      const float* x, size_t n, int mode) {
  size_t nblocks = (n + 255) / 256;
  float y[256];
  for (size_t b = 0; b < nblocks; b++) {
    size_t start = b * 256;
    size_t len = (n - start < 256) ? n - start : 256;
    for (size_t i = 0; i < len; i++) y[i] = canonical(x[start + i] + residual[start + i]);
    float s = or_block_scale(or_block_absmax(y, len), mode);
    scales[b] = s;
    for (size_t i = 0; i < len; i++) {
      uint8_t c = or_fp8_quantize_one(y[i], s);
      codes[start + i] = c;
      float decoded = or_e4m3_decode_one(c) * s;
      residual[start + i] = canonical(y[i] - decoded);
    }
  }
}

void or_bucket_allreduce_ef(float* out, void* const* codes,
                            float* const* scales, float* const* residuals,
                            const float* const* x, int k, size_t n,
                            size_t bucket_elems, int codec, int mode) {
  const void* cs[64];
  const float* ss[64];
  size_t scale_base = 0;
  for (size_t start = 0; start < n; start += bucket_elems) {
    size_t len = (n - start < bucket_elems) ? n - start : bucket_elems;
    for (int r = 0; r < k; r++) {
      if (codec == OR_CODEC_BF16) {
        uint16_t* c = (uint16_t*)codes[r] + start;
        or_encode_bf16_ef(c, residuals[r] + start, x[r] + start, len);
        cs[r] = c;
        ss[r] = NULL;
      } else {
        uint8_t* c = (uint8_t*)codes[r] + start;
        or_encode_fp8_ef(c, scales[r] + scale_base, residuals[r] + start,
                         x[r] + start, len, mode);
        cs[r] = c;
        ss[r] = scales[r] + scale_base;
      }
    }
    or_decode_accumulate(out + start, cs, codec == OR_CODEC_FP8 ? ss : NULL, k,
                         len, codec, 0);
    scale_base += (len + 255) / 256;
  }
}

/* ------------------------------------------------------------------------
 * Other reductions.  README "API": all_reduce takes SUM, AVG, MAX or MIN;
 * AVG is a SUM divided by the world size, identically on every rank.  The
 * world size is the number of ranks in the job, not the number k of island
 * sums the leader adds, so it is an explicit divisor d (reading taken).
 *   AVG:  out = RN(sum / RN(d)), sum the fixed-order SUM.
 *   MAX:  IEEE 754-2019 maximum over ranks (reading taken: the README leaves
 *         NaN to the backends): NaN if any value is NaN, otherwise the
 *         largest, with +0 above -0.
 *   MIN:  likewise the smallest, with -0 below +0.
 * --------------------------------------------------------------------- */
static float max2019(float a, float b) {
  if (isnan(a) || isnan(b)) return NAN;
  if (a > b) return a;
  if (b > a) return b;
  /* equal: they differ only if one is +0 and the other -0 */
  return signbit(a) ? b : a;
}

static float min2019(float a, float b) {
  if (isnan(a) || isnan(b)) return NAN;
  if (a < b) return a;
  if (b < a) return b;
  return signbit(a) ? a : b;
}

void or_reduce(float* out, const float* const* x, int k, size_t n, int op,
               int divisor) {
  if (op == OR_OP_SUM || op == OR_OP_AVG) {
    or_reduce_sum(out, x, k, n);
    if (op == OR_OP_AVG) {
      float d = (float)divisor;
      for (size_t i = 0; i < n; i++) out[i] = canonical(out[i] / d);
    }
    return;
  }
  for (size_t i = 0; i < n; i++) {
    float acc = x[0][i];
    for (int r = 1; r < k; r++) {
      acc = (op == OR_OP_MAX) ? max2019(acc, x[r][i]) : min2019(acc, x[r][i]);
    }
    out[i] = k == 1 ? acc : canonical(acc);
  }
}

/* ------------------------------------------------------------------------
 * Other element types.  README "API": tensors may be float16, bfloat16,
 * float32, float64, int8, uint8, int32 or int64, and all_reduce takes SUM,
 * AVG, MAX or MIN, with AVG only for floating-point types.  Readings taken:
 *   floating-point SUM is a left fold over ranks, each addition rounded to
 *   the element type (nearest, ties to even, IEEE overflow to Inf); AVG is
 *   RN_type(sum / d); MAX / MIN are the IEEE 754-2019 maximum / minimum;
 *   integer SUM wraps modulo 2^bits (two's complement); integer MAX / MIN are
 *   the ordinary order.
 * Each half-precision result is computed in binary64 and rounded once to the
 * type: the exact sum or quotient of two half-precision values, rounded to
 * binary64 (53 bits >= 2p + 2 with p = 11 or 8), rounds to the same value as
 * the exact result would (Figueroa, "When is double rounding innocuous?").
 * --------------------------------------------------------------------- */
enum { OR_T_F32 = 0, OR_T_F16 = 1, OR_T_BF16 = 2, OR_T_F64 = 3,
       OR_T_I8 = 4, OR_T_U8 = 5, OR_T_I32 = 6, OR_T_I64 = 7 };

/* Value of an IEEE half (1-5-10) code. */
static double f16_value(uint16_t c) {
  int e = (c >> 10) & 31;
  int f = c & 1023;
  double sign = (c & 0x8000) ? -1.0 : 1.0;
  if (e == 31) return f ? NAN : sign * INFINITY;
  if (e == 0) return sign * ldexp((double)f, -24);
  return sign * ldexp(1024.0 + f, e - 25);
}

/* Nearest value with p significant bits and least normal exponent emin
 * (subnormals below), ties to the even significand, rounding as if the
 * exponent were unbounded and giving Inf when that reaches 2^(emax+1).  v is
 * finite. */
static double round_format(double v, int p, int emin, int emax) {
  if (v == 0.0) return v;
  double a = fabs(v);
  int e;
  frexp(a, &e);          /* a = m * 2^e, m in [0.5, 1) */
  e = e - 1;             /* 2^e <= a < 2^(e+1) */
  if (e < emin) e = emin;
  double quantum = ldexp(1.0, e - (p - 1));
  double m = a / quantum; /* exact: a power-of-two scaling */
  double lo = floor(m);
  double rem = m - lo;
  double q = lo;
  if (rem > 0.5 || (rem == 0.5 && fmod(lo, 2.0) == 1.0)) q = lo + 1.0;
  double r = q * quantum;
  if (r >= ldexp(1.0, emax + 1)) return copysign(INFINITY, v);  /* IEEE overflow */
  return copysign(r, v);
}

static uint16_t f16_code(double v) {  /* v is an f16 value, NaN or +-Inf */
  if (isnan(v)) return 0x7E00;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isinf(a)) return sign | 0x7C00;
  if (a < ldexp(1.0, -14)) return sign | (uint16_t)(a / ldexp(1.0, -24));
  int e;
  double m = frexp(a, &e);  /* a = m * 2^e, m in [0.5, 1) */
  return sign | (uint16_t)((e - 1 + 15) << 10) | (uint16_t)((m * 2.0 - 1.0) * 1024.0);
}

/* Value of element i of an array of the given type, as binary64 (exact for
 * every type here except int64 beyond 2^53, which the integer path avoids). */
static double value_at(const void* a, size_t i, int t) {
  switch (t) {
    case OR_T_F32: return ((const float*)a)[i];
    case OR_T_F16: return f16_value(((const uint16_t*)a)[i]);
    case OR_T_BF16: return or_bf16_decode_one(((const uint16_t*)a)[i]);
    case OR_T_F64: return ((const double*)a)[i];
    default: return 0.0;
  }
}

static double round_to_type(double v, int t) {
  if (isnan(v) || isinf(v)) return v;
  switch (t) {
    case OR_T_F32: return (double)(float)v;  /* one binary32 rounding */
    case OR_T_F16: return round_format(v, 11, -14, 15);
    case OR_T_BF16: return round_format(v, 8, -126, 127);
    default: return v;
  }
}

static void store_at(void* a, size_t i, int t, double v) {
  switch (t) {
    case OR_T_F32: ((float*)a)[i] = (float)v; break;
    case OR_T_F16: ((uint16_t*)a)[i] = f16_code(v); break;
    case OR_T_BF16: ((uint16_t*)a)[i] = or_bf16_encode_one((float)v); break;
    case OR_T_F64: ((double*)a)[i] = v; break;
    default: break;
  }
}

static double max2019d(double a, double b) {
  if (isnan(a) || isnan(b)) return NAN;
  if (a > b) return a;
  if (b > a) return b;
  return signbit(a) ? b : a;
}

static double min2019d(double a, double b) {
  if (isnan(a) || isnan(b)) return NAN;
  if (a < b) return a;
  if (b < a) return b;
  return signbit(a) ? a : b;
}

static void reduce_float(void* out, const void* const* x, int k, size_t n, int t,
                         int op, int divisor) {
  for (size_t i = 0; i < n; i++) {
    double acc = value_at(x[0], i, t);
    for (int r = 1; r < k; r++) {
      double v = value_at(x[r], i, t);
      if (op == OR_OP_SUM || op == OR_OP_AVG) {
        acc = round_to_type(acc + v, t);  /* binary64 add (or binary32 for f32 below) */
      } else if (op == OR_OP_MAX) {
        acc = max2019d(acc, v);
      } else {
        acc = min2019d(acc, v);
      }
    }
    if (op == OR_OP_AVG) acc = round_to_type(acc / (double)divisor, t);
    store_at(out, i, t, acc);
  }
}

static void reduce_int(void* out, const void* const* x, int k, size_t n, int t,
                       int op) {
  for (size_t i = 0; i < n; i++) {
    int64_t v[64] = {0};
    for (int r = 0; r < k; r++) {
      switch (t) {
        case OR_T_I8: v[r] = ((const int8_t*)x[r])[i]; break;
        case OR_T_U8: v[r] = ((const uint8_t*)x[r])[i]; break;
        case OR_T_I32: v[r] = ((const int32_t*)x[r])[i]; break;
        default: v[r] = ((const int64_t*)x[r])[i]; break;
      }
    }
    uint64_t sum = (uint64_t)v[0];  /* unsigned: wraps modulo 2^64 */
    int64_t best = v[0];
    for (int r = 1; r < k; r++) {
      sum += (uint64_t)v[r];
      if (op == OR_OP_MAX && v[r] > best) best = v[r];
      if (op == OR_OP_MIN && v[r] < best) best = v[r];
    }
    uint64_t res = (op == OR_OP_SUM) ? sum : (uint64_t)best;
    switch (t) {  /* keep the low bits: wraps modulo 2^bits */
      case OR_T_I8: ((uint8_t*)out)[i] = (uint8_t)res; break;
      case OR_T_U8: ((uint8_t*)out)[i] = (uint8_t)res; break;
      case OR_T_I32: ((uint32_t*)out)[i] = (uint32_t)res; break;
      default: ((uint64_t*)out)[i] = res; break;
    }
  }
}

void or_reduce_typed(void* out, const void* const* x, int k, size_t n, int dtype,
                     int op, int divisor) {
  if (dtype == OR_T_F32) {
    /* binary32 adds, exactly as or_reduce */
    or_reduce((float*)out, (const float* const*)x, k, n, op, divisor);
  } else if (dtype == OR_T_F16 || dtype == OR_T_BF16 || dtype == OR_T_F64) {
    reduce_float(out, x, k, n, dtype, op, divisor);
  } else {
    reduce_int(out, x, k, n, dtype, op);
  }
}

/* ------------------------------------------------------------------------
 * Bridge compression of float16, bfloat16 and float64 tensors.  README
 * "Bridge compression": the bridged policies compress floating-point SUM and
 * AVG; leaders quantize their island's sum, and the payloads are dequantized
 * and added in float32.  Readings taken: an island sum of another floating
 * type is first taken to binary32 (exact from float16 and bfloat16; one
 * rounding to nearest-even from float64) and then encoded exactly as a
 * binary32 array; the float32 total is rounded once to the tensor's type
 * (nearest, ties to even, IEEE overflow to Inf).  Without a codec the stream
 * is the exact SUM of that type (or_reduce_typed).
 * --------------------------------------------------------------------- */
/* A NaN keeps its sign and the top bits of its payload and comes out quiet
 * (IEEE 754-2019, 6.2.3, the preferred NaN propagation of a format
 * conversion); bfloat16 widens bit for bit, as the bf16 codec decodes. */
static float quiet_nan_f32(uint32_t sign, uint32_t payload23) {
  return bits_float(sign | 0x7FC00000u | (payload23 & 0x3FFFFFu));
}

static float typed_to_f32(const void* a, size_t i, int t) {
  switch (t) {
    case OR_T_F32: return ((const float*)a)[i];
    case OR_T_F16: {
      uint16_t c = ((const uint16_t*)a)[i];
      if ((c & 0x7C00) == 0x7C00 && (c & 0x03FF)) {  /* NaN: 10 payload bits */
        return quiet_nan_f32((uint32_t)(c & 0x8000) << 16, (uint32_t)(c & 0x03FF) << 13);
      }
      return (float)f16_value(c);  /* exact */
    }
    case OR_T_BF16: return or_bf16_decode_one(((const uint16_t*)a)[i]);
    default: {
      double d = ((const double*)a)[i];
      if (isnan(d)) {  /* top 23 of the 52 payload bits */
        uint64_t u;
        memcpy(&u, &d, sizeof u);
        return quiet_nan_f32((uint32_t)(u >> 32) & 0x80000000u, (uint32_t)((u >> 29) & 0x7FFFFFu));
      }
      return (float)d;  /* one binary32 rounding */
    }
  }
}

static void f32_to_typed(void* a, size_t i, int t, float v) {
  switch (t) {
    case OR_T_F32: ((float*)a)[i] = v; break;
    case OR_T_F16: ((uint16_t*)a)[i] = f16_code(round_to_type((double)v, OR_T_F16)); break;
    case OR_T_BF16: ((uint16_t*)a)[i] = or_bf16_encode_one(v); break;
    default: ((double*)a)[i] = (double)v; break;  /* exact */
  }
}

/* The binary32 total that a total of type t is rounded from: a NaN total of
 * another type is always the canonical NaN's rounding (0x7E00, 0x7FC0,
 * 0x7FF8000000000000), the decode of one bf16 payload included, so that no
 * NaN payload is narrowed (reading taken, with the canonical NaN above). */
static float typed_total(float v, int t) { return t == OR_T_F32 ? v : canonical(v); }

static float* typed_array_to_f32(const void* x, size_t n, int t) {
  float* f = (float*)malloc((n ? n : 1) * sizeof(float));
  for (size_t i = 0; i < n; i++) f[i] = typed_to_f32(x, i, t);
  return f;
}

void or_encode_typed(int codec, int dtype, void* codes, float* scales, const void* x,
                     size_t n, int mode) {
  float* f = typed_array_to_f32(x, n, dtype);
  if (codec == OR_CODEC_BF16) or_encode_bf16((uint16_t*)codes, f, n);
  else or_encode_fp8((uint8_t*)codes, scales, f, n, mode);
  free(f);
}

void or_decode_sum_typed(void* out, int dtype, const void* const* codes,
                         const float* const* scales, int k, size_t n, int codec) {
  float* f = (float*)malloc((n ? n : 1) * sizeof(float));
  or_decode_accumulate(f, codes, scales, k, n, codec, 0);
  for (size_t i = 0; i < n; i++) f32_to_typed(out, i, dtype, typed_total(f[i], dtype));
  free(f);
}

void or_bucket_allreduce_typed(void* out, void* const* codes, float* const* scales,
                               const void* const* x, int k, size_t n, size_t bucket_elems,
                               int codec, int mode, int dtype) {
  if (codec == OR_CODEC_NONE) {
    or_reduce_typed(out, x, k, n, dtype, OR_OP_SUM, 1);
    return;
  }
  float* f[64];
  for (int r = 0; r < k; r++) f[r] = typed_array_to_f32(x[r], n, dtype);
  float* sum = (float*)malloc((n ? n : 1) * sizeof(float));
  or_bucket_allreduce(sum, codes, scales, (const float* const*)f, k, n, bucket_elems, codec, mode);
  for (size_t i = 0; i < n; i++) f32_to_typed(out, i, dtype, typed_total(sum[i], dtype));
  free(sum);
  for (int r = 0; r < k; r++) free(f[r]);
}

/* Error feedback over the other floating types (reading: the error-feedback
 * step of the README's "Bridge compression" runs in binary32 whatever the
 * gradient's type, as the codecs do; the residual is binary32; only the
 * conversion of the gradient on the way in and of the total on the way out
 * depend on the type). */
void or_encode_ef_typed(int codec, int dtype, void* codes, float* scales, float* residual,
                        const void* x, size_t n, int mode) {
  float* f = typed_array_to_f32(x, n, dtype);
  if (codec == OR_CODEC_BF16) or_encode_bf16_ef((uint16_t*)codes, residual, f, n);
  else or_encode_fp8_ef((uint8_t*)codes, scales, residual, f, n, mode);
  free(f);
}

void or_bucket_allreduce_ef_typed(void* out, void* const* codes, float* const* scales,
                                  float* const* residuals, const void* const* x, int k,
                                  size_t n, size_t bucket_elems, int codec, int mode,
                                  int dtype) {
  float* f[64];
  for (int r = 0; r < k; r++) f[r] = typed_array_to_f32(x[r], n, dtype);
  float* sum = (float*)malloc((n ? n : 1) * sizeof(float));
  or_bucket_allreduce_ef(sum, codes, scales, residuals, (const float* const*)f, k, n, bucket_elems,
                         codec, mode);
  for (size_t i = 0; i < n; i++) f32_to_typed(out, i, dtype, typed_total(sum[i], dtype));
  free(sum);
  for (int r = 0; r < k; r++) free(f[r]);
}
