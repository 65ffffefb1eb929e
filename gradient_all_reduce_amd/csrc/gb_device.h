// gb_device.h — device helpers shared by the kernel sources of libgbreduce
// (gb_reduce.hip, gb_codec_bf16.hip, gb_codec_fp8.hip, gb_ef.hip), for
// gfx950 (AMD Instinct MI355X, CDNA4).  Everything here has internal linkage:
// each kernel source compiles its own copy, and the sources build in
// parallel.
//
// All of this work streams HBM: a few integer and float operations per 4-byte
// element, no reuse, no contraction (so no MFMA).  The kernels are shaped for
// that:
//   * every lane moves 16-byte vectors of 4-byte values (8 bytes of 2-byte
//     values, 4-byte words of fp8 codes), and each load or store instruction
//     of a 16-lane row covers one contiguous run, so requests coalesce into
//     whole cache lines; float64 has lane maps of its own that keep this;
//   * loads and stores carry the non-temporal hint: each byte is touched once,
//     so nothing is worth keeping in L2 or the last-level cache;
//   * a lane issues all of its loads (every rank) before it computes, and the
//     k contributions of an element are combined in registers: reduce, encode
//     and decode-accumulate are fused where the call allows it;
//   * the fp8 block maximum is reduced across the 16 lanes of one DPP row (four
//     row-local DPP steps, no LDS, no barrier): a 256-value block is one row of
//     16 lanes holding 16 values each, a wavefront works on 4 blocks and a
//     256-lane workgroup on 16 (the fused pass over 4 ranks of float32
//     gradients, with error feedback also of float16 and bfloat16 ones, and
//     the decode of 4 payloads into float32 instead spread one block over a
//     wavefront from a few million values, 4 values per lane, and take the
//     row maxima's maximum with 4 lane reads);
//   * E4M3 conversion uses gfx950's packed converters (v_cvt_pk_fp8_f32 to
//     encode two values per instruction, v_cvt_pk_f32_fp8 to decode two);
//   * large launches take their groups in a permuted order (group_index) that
//     spreads the workgroups in flight over several regions of the stream,
//     one contiguous chunk per XCD for the vector kernels.
//
// Arithmetic follows the gpubridge README, "How it works" (sum of island sums)
// and "Bridge compression" (bf16; OCP E4M3 with one scale per 256 values;
// decode and add in float32).  Every rounding is IEEE binary32
// round-to-nearest-even with subnormals kept, and nothing is contracted into a
// fused multiply-add (built with -ffp-contract=off), so results do not depend
// on the launch shape.
#pragma once

#include <hip/hip_runtime.h>

#include "gb_internal.h"

namespace gb {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

struct OutTable {
  void* p[kLaunchRanks];
};

constexpr int kThreads = 256;  // 4 wavefronts of 64 lanes

__device__ __forceinline__ uint32_t fbits(float x) { return __float_as_uint(x); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __uint_as_float(u); }

// Canonical NaN (README "Bridge compression": every rank ends with the same
// bits, whichever vendor's GPU ran the kernels).  The sign and payload of
// the NaN an operation delivers are the platform's (an invalid operation
// gives +NaN here and -NaN on x86 hosts; which input NaN an add passes on
// may follow the compiler's operand order), so every NaN that the float32
// arithmetic of the method delivers -- a sum of two or more terms, an AVG
// quotient, a MAX or MIN over two or more ranks, a decoded fp8 value and
// every decoded-and-added total, the error-feedback value and residual -- is
// stored as the quiet NaN 0x7FC00000.  A copy (one source, or the decode of
// one bf16 payload with nothing added) keeps its bits.  One compare and
// select per stored value.
constexpr uint32_t kCanonicalNan = 0x7FC00000u;
__device__ __forceinline__ float canon(float v) { return v != v ? bitsf(kCanonicalNan) : v; }
__device__ __forceinline__ f4 canon4(f4 v) { return f4{canon(v.x), canon(v.y), canon(v.z), canon(v.w)}; }

// ---------------------------------------------------------------------------
// Streaming memory access (non-temporal) with guarded variants for the ragged
// end of a buffer.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f4 load4(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
}
__device__ __forceinline__ void store4(float* p, f4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p));
}

// Elements [i, i + 4) of p, zero at and beyond n.
__device__ __forceinline__ f4 load4_any(const float* p, size_t i, size_t n) {
  if (i + 4 <= n) return load4(p + i);
  f4 v = {0.0f, 0.0f, 0.0f, 0.0f};
  if (i < n) v.x = p[i];
  if (i + 1 < n) v.y = p[i + 1];
  if (i + 2 < n) v.z = p[i + 2];
  return v;
}
// Stores the elements of [i, i + 4) that lie below n.
__device__ __forceinline__ void store4_any(float* p, size_t i, size_t n, f4 v) {
  if (i + 4 <= n) {
    store4(p + i, v);
    return;
  }
  if (i < n) p[i] = v.x;
  if (i + 1 < n) p[i + 1] = v.y;
  if (i + 2 < n) p[i + 2] = v.z;
}

// 4 fp8 codes of elements [i, i + 4) as one little-endian word, clipped to n.
__device__ __forceinline__ uint32_t load_codes4(const uint8_t* codes, size_t i, size_t n) {
  if (i + 4 <= n) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(codes + i));
  uint32_t w = 0;
  for (int e = 0; e < 3; e++) {
    if (i + e < n) w |= (uint32_t)codes[i + e] << (8 * e);
  }
  return w;
}
__device__ __forceinline__ void store_codes4(uint8_t* codes, size_t i, size_t n, uint32_t w) {
  if (i + 4 <= n) {
    __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(codes + i));
    return;
  }
  for (int e = 0; e < 3; e++) {
    if (i + e < n) codes[i + e] = (uint8_t)(w >> (8 * e));
  }
}

// 4 bf16 codes of elements [i, i + 4) as 2 words, clipped to n.
__device__ __forceinline__ u2 load_bf16_4(const uint16_t* codes, size_t i, size_t n) {
  if (i + 4 <= n) return __builtin_nontemporal_load(reinterpret_cast<const u2*>(codes + i));
  uint32_t w[2] = {0u, 0u};
  for (int e = 0; e < 3; e++) {
    if (i + e < n) w[e >> 1] |= (uint32_t)codes[i + e] << (16 * (e & 1));
  }
  return u2{w[0], w[1]};
}
__device__ __forceinline__ void store_bf16_4(uint16_t* codes, size_t i, size_t n, u2 w) {
  if (i + 4 <= n) {
    __builtin_nontemporal_store(w, reinterpret_cast<u2*>(codes + i));
    return;
  }
  const uint32_t ws[2] = {w.x, w.y};
  for (int e = 0; e < 3; e++) {
    if (i + e < n) codes[i + e] = (uint16_t)(ws[e >> 1] >> (16 * (e & 1)));
  }
}

// The same accesses with the bounds test resolved at compile time: FULL means
// the caller knows the whole workgroup's range lies below n, so no access is
// guarded (one straight run of loads, no divergent branches).
template <bool FULL>
__device__ __forceinline__ f4 load4_at(const float* p, size_t i, size_t n) {
  return FULL ? load4(p + i) : load4_any(p, i, n);
}
template <bool FULL>
__device__ __forceinline__ void store4_at(float* p, size_t i, size_t n, f4 v) {
  if (FULL) store4(p + i, v);
  else store4_any(p, i, n, v);
}
template <bool FULL>
__device__ __forceinline__ uint32_t load_codes4_at(const uint8_t* codes, size_t i, size_t n) {
  return FULL ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(codes + i)) : load_codes4(codes, i, n);
}
template <bool FULL>
__device__ __forceinline__ void store_codes4_at(uint8_t* codes, size_t i, size_t n, uint32_t w) {
  if (FULL) __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(codes + i));
  else store_codes4(codes, i, n, w);
}
template <bool FULL>
__device__ __forceinline__ u2 load_bf16_4_at(const uint16_t* codes, size_t i, size_t n) {
  return FULL ? __builtin_nontemporal_load(reinterpret_cast<const u2*>(codes + i)) : load_bf16_4(codes, i, n);
}
template <bool FULL>
__device__ __forceinline__ void store_bf16_4_at(uint16_t* codes, size_t i, size_t n, u2 w) {
  if (FULL) __builtin_nontemporal_store(w, reinterpret_cast<u2*>(codes + i));
  else store_bf16_4(codes, i, n, w);
}

// ---------------------------------------------------------------------------
// bf16: nearest value, ties to the even code (the carry of the rounding add
// runs into the exponent, which gives IEEE overflow to Inf); a NaN keeps its
// sign and top payload bits with the quiet bit set.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t bf16_code(float x) {
  const uint32_t u = fbits(x);
  const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? ((u >> 16) | 0x40u) : r;
}

__device__ __forceinline__ u2 bf16_pack4(f4 x) {
  return u2{bf16_code(x.x) | (bf16_code(x.y) << 16), bf16_code(x.z) | (bf16_code(x.w) << 16)};
}
// bf16 -> fp32 is exact: the code is the top half of the binary32 pattern.
__device__ __forceinline__ f4 bf16_unpack4(u2 w) {
  return f4{bitsf(w.x << 16), bitsf(w.x & 0xFFFF0000u), bitsf(w.y << 16), bitsf(w.y & 0xFFFF0000u)};
}

// ---------------------------------------------------------------------------
// Element types of the codec kernels' inputs and outputs (README "Bridge
// compression": floating-point tensors; their payloads are added in
// float32).  ET is GB_DTYPE_F32, F16, BF16 or F64.  A load gives elements
// [i, i + 4) as binary32 (exact from the halves, rounded once to nearest-even
// from float64; zero at and beyond n); a store rounds binary32 once to the
// type (nearest-even, IEEE overflow; exact to float64).
// ---------------------------------------------------------------------------
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef double d2v __attribute__((ext_vector_type(2)));

template <int ET, bool FULL>
__device__ __forceinline__ f4 load_vals4_at(const void* p, size_t i, size_t n) {
  if constexpr (ET == GB_DTYPE_F32) {
    return load4_at<FULL>(static_cast<const float*>(p), i, n);
  } else if constexpr (ET == GB_DTYPE_BF16) {
    return bf16_unpack4(load_bf16_4_at<FULL>(static_cast<const uint16_t*>(p), i, n));
  } else if constexpr (ET == GB_DTYPE_F16) {
    const h4 h = __builtin_bit_cast(h4, load_bf16_4_at<FULL>(static_cast<const uint16_t*>(p), i, n));
    return f4{(float)h.x, (float)h.y, (float)h.z, (float)h.w};
  } else {
    const double* d = static_cast<const double*>(p) + i;
    d2v lo, hi;
    if (FULL || i + 4 <= n) {
      lo = __builtin_nontemporal_load(reinterpret_cast<const d2v*>(d));
      hi = __builtin_nontemporal_load(reinterpret_cast<const d2v*>(d + 2));
    } else {
      lo = d2v{i < n ? d[0] : 0.0, i + 1 < n ? d[1] : 0.0};
      hi = d2v{i + 2 < n ? d[2] : 0.0, 0.0};
    }
    return f4{(float)lo.x, (float)lo.y, (float)hi.x, (float)hi.y};
  }
}

template <int ET, bool FULL>
__device__ __forceinline__ void store_vals4_at(void* p, size_t i, size_t n, f4 v) {
  if constexpr (ET == GB_DTYPE_F32) {
    store4_at<FULL>(static_cast<float*>(p), i, n, v);
  } else if constexpr (ET == GB_DTYPE_BF16) {
    store_bf16_4_at<FULL>(static_cast<uint16_t*>(p), i, n, bf16_pack4(v));
  } else if constexpr (ET == GB_DTYPE_F16) {
    // The binary32 values must exist before they are rounded to float16: left
    // alone, the compiler may fold the product or sum that made them into one
    // mixed-precision fma rounding straight to float16 (one rounding instead
    // of the two the definition has, and +0 for a -0 product).  The empty asm
    // pins them in registers and emits nothing.
    asm volatile("" : "+v"(v));
    const h4 h = {(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
    store_bf16_4_at<FULL>(static_cast<uint16_t*>(p), i, n, __builtin_bit_cast(u2, h));
  } else {
    double* d = static_cast<double*>(p) + i;
    const d2v lo = {(double)v.x, (double)v.y}, hi = {(double)v.z, (double)v.w};
    if (FULL || i + 4 <= n) {
      __builtin_nontemporal_store(lo, reinterpret_cast<d2v*>(d));
      __builtin_nontemporal_store(hi, reinterpret_cast<d2v*>(d + 2));
    } else {
      if (i < n) d[0] = lo.x;
      if (i + 1 < n) d[1] = lo.y;
      if (i + 2 < n) d[2] = hi.x;
    }
  }
}

// float64 pairs and pairs of fp8 codes: 16 and 2 bytes per lane, clipped to n.
template <bool FULL>
__device__ __forceinline__ d2v load_f64x2_at(const double* d, size_t e, size_t n) {
  if (FULL || e + 2 <= n) return __builtin_nontemporal_load(reinterpret_cast<const d2v*>(d + e));
  return d2v{e < n ? d[e] : 0.0, 0.0};
}
template <bool FULL>
__device__ __forceinline__ void store_f64x2_at(double* d, size_t e, size_t n, d2v v) {
  if (FULL || e + 2 <= n) __builtin_nontemporal_store(v, reinterpret_cast<d2v*>(d + e));
  else if (e < n) d[e] = v.x;
}
// float32 pairs: the binary32 residual of a float64 gradient follows the
// gradient's lane map.
template <bool FULL>
__device__ __forceinline__ f2 load_f32x2_at(const float* p, size_t e, size_t n) {
  if (FULL || e + 2 <= n) return __builtin_nontemporal_load(reinterpret_cast<const f2*>(p + e));
  return f2{e < n ? p[e] : 0.0f, 0.0f};
}
template <bool FULL>
__device__ __forceinline__ void store_f32x2_at(float* p, size_t e, size_t n, f2 v) {
  if (FULL || e + 2 <= n) __builtin_nontemporal_store(v, reinterpret_cast<f2*>(p + e));
  else if (e < n) p[e] = v.x;
}
// Codes of elements [e, e + 2), the low byte first.
template <bool FULL>
__device__ __forceinline__ uint32_t load_codes2_at(const uint8_t* c, size_t e, size_t n) {
  if (FULL || e + 2 <= n) return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(c + e));
  return e < n ? (uint32_t)c[e] : 0u;
}
template <bool FULL>
__device__ __forceinline__ void store_codes2_at(uint8_t* c, size_t e, size_t n, uint32_t h) {
  if (FULL || e + 2 <= n) __builtin_nontemporal_store((uint16_t)h, reinterpret_cast<uint16_t*>(c + e));
  else if (e < n) c[e] = (uint8_t)h;
}

// ---------------------------------------------------------------------------
// fp8: OCP E4M3 (bias 7, largest finite 448 = 0x7E, S.1111.111 = NaN), one
// fp32 scale per 256-value block.
// ---------------------------------------------------------------------------
// Largest non-NaN magnitude of a lane's 16 values, as a bit pattern: the
// unsigned maximum of |x| bit patterns orders like the magnitudes, in any
// order of evaluation.  A NaN among the 16 shows as a pattern above Inf's;
// only then are the values scanned again with the NaNs counted as 0.
__device__ __forceinline__ uint32_t lane_absmax16(const f4 (&x)[4]) {
  uint32_t a = 0u;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    a = max(a, max(fbits(x[j].x) & 0x7FFFFFFFu, fbits(x[j].y) & 0x7FFFFFFFu));
    a = max(a, max(fbits(x[j].z) & 0x7FFFFFFFu, fbits(x[j].w) & 0x7FFFFFFFu));
  }
  if (a > 0x7F800000u) {
    a = 0u;
#pragma unroll
    for (int j = 0; j < 4; j++) {
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const uint32_t m = fbits(x[j][e]) & 0x7FFFFFFFu;
        a = max(a, m > 0x7F800000u ? 0u : m);
      }
    }
  }
  return a;
}

// Maximum over the 16 lanes of this lane's DPP row; every lane of the row
// receives it.  Requires all 64 lanes active.
__device__ __forceinline__ uint32_t row_max16(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  return v;
}

// Scale of a block whose largest non-NaN magnitude has bit pattern `abits`.
//   ABSMAX_DIV_448: RN(a / 448) (correctly rounded divide; 0 for a = 0).
//   POW2: the smallest 2^e, e >= -149, with a <= 448 * 2^e.  Writing
//   a = m * 2^q with m in [1, 2): e = q - 8 when m <= 1.75 (448 = 1.75 * 2^8),
//   else q - 7.  1 for a = 0, Inf for a = Inf.
__device__ __forceinline__ float block_scale(uint32_t abits, int mode) {
  if (mode == GB_SCALE_ABSMAX_DIV_448) return bitsf(abits) / 448.0f;
  if (abits == 0u) return 1.0f;
  if (abits >= 0x7F800000u) return bitsf(0x7F800000u);
  int q;
  uint32_t frac;
  const uint32_t ef = abits >> 23;
  if (ef != 0u) {
    q = (int)ef - 127;
    frac = abits & 0x7FFFFFu;
  } else {  // subnormal a: normalise on its leading one
    const int p = 31 - __clz(abits);
    q = p - 149;
    frac = (abits << (23 - p)) & 0x7FFFFFu;
  }
  int e = q - 8 + (frac > 0x600000u ? 1 : 0);
  e = e < -149 ? -149 : e;
  return e >= -126 ? bitsf((uint32_t)(e + 127) << 23) : bitsf(1u << (e + 149));
}

// 1/s in binary64, and 1 for s = 0 (a zero block skips the division).
__device__ __forceinline__ double scale_reciprocal(float s) {
  return s == 0.0f ? 1.0 : 1.0 / (double)s;
}

// RN32(x / s) computed as RN32(RN64(x * RN64(1/s))).  Exact: for binary32 x
// and s the quotient is never closer than 2^-48 (relative) to a binary32
// rounding midpoint, while the binary64 route is within about 2^-52 of it, so
// both round to the same binary32 value; below 2^-126 both give values that
// encode to E4M3 zero.  An s of 0 gives rinv = 1 (v = x); s = Inf gives
// rinv = 0, i.e. x / Inf = +-0 and Inf / Inf = NaN, as IEEE division does.
__device__ __forceinline__ f4 quotient4(f4 x, double rinv) {
  return f4{(float)((double)x.x * rinv), (float)((double)x.y * rinv), (float)((double)x.z * rinv),
            (float)((double)x.w * rinv)};
}

// E4M3 codes of 4 quotients v, packed little-endian, sign bits from the
// inputs x.  The hardware converter rounds to nearest even and agrees with the
// E4M3 definition for every |v| <= 448 * (1 + 2^-23) (checked over all such
// binary32 values); above that it does not saturate, so callers bring larger
// quotients back to +-448 first (see clamp448).  It returns 0xFF for any NaN,
// so the sign bit is replaced by x's: NaN codes become 0x7F | sign.
__device__ __forceinline__ uint32_t e4m3_pack4(f4 v, f4 x) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(v.x, v.y, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(v.z, v.w, w, true);
  const uint32_t s01 = __builtin_amdgcn_perm(fbits(x.y), fbits(x.x), 0x0C0C0703u);  // x.x, x.y top bytes -> bytes 0, 1
  const uint32_t s23 = __builtin_amdgcn_perm(fbits(x.w), fbits(x.z), 0x07030C0Cu);  // x.z, x.w top bytes -> bytes 2, 3
  return ((uint32_t)w & 0x7F7F7F7Fu) | ((s01 | s23) & 0x80808080u);
}

// Saturation of quotients to +-448, NaN kept.  Only a block whose scale is
// subnormal needs it: a normal s = RN(a / 448) is within 2^-24 of a / 448, so
// |x / s| <= a / s rounds to at most 448 * (1 + 2^-23), and a power-of-two
// scale is at least a / 448.  A subnormal s carries an absolute rounding
// error that can put a / s anywhere above 448.
__device__ __forceinline__ f4 clamp448(f4 v) {
  f4 c;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const float t = fminf(fmaxf(v[e], -448.0f), 448.0f);
    c[e] = v[e] != v[e] ? v[e] : t;
  }
  return c;
}

// Values of 4 packed E4M3 codes (exact; NaN codes give NaN).
__device__ __forceinline__ f4 e4m3_unpack4(uint32_t w) {
  const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  return f4{lo.x, lo.y, hi.x, hi.y};
}

// Elements of a 256-value block owned by a lane: 4 vectors, vector j at
// element offset (16 j + col) * 4 of the block, so every load or store
// instruction of a row covers 256 contiguous bytes of fp32 (64 of codes).
__device__ __forceinline__ size_t lane_elem(size_t block, int j, uint32_t col) {
  return block * kBlock + (size_t)(16 * j + col) * 4;
}

// Lane maps of a block's 256 values.  A lane of row col holds 16 values of
// the block as 4 vectors of 4; the map says which, chosen per element type
// so that every access of a row instruction is one contiguous run:
//   kMapNarrow: vector j is the 4 consecutive values at lane_elem(block, j,
//     col) (16 bytes of 4-byte values per access);
//   kMapWide (2-byte types): vectors 2m and 2m + 1 are the 8 consecutive
//     values at wide_elem(block, 2m, col), moved by one 16-byte access (and
//     their codes by one 8-byte access) instead of two 8-byte ones;
//   kMapPair (float64): vector j is two pairs of values 32 apart, at
//     pair_elem(block, j, col) and 32 further, each pair one 16-byte access
//     (4 consecutive doubles would be 32 bytes per lane at half density).
// Which lane holds which values of a block changes no result: the block
// maximum is taken over the whole row, and every value and code keeps its own
// position in memory.
enum : int { kMapNarrow = 0, kMapWide = 1, kMapPair = 2 };
template <int ET>
__host__ __device__ constexpr int codec_map() {
  return ET == GB_DTYPE_F64 ? kMapPair : (ET == GB_DTYPE_F16 || ET == GB_DTYPE_BF16) ? kMapWide : kMapNarrow;
}
// The error-feedback kernels keep the float32 residual on the gradient's map;
// the wide map would read it at half density, so 2-byte gradients stay narrow.
template <int ET>
__host__ __device__ constexpr int ef_map() {
  return ET == GB_DTYPE_F64 ? kMapPair : kMapNarrow;
}

__device__ __forceinline__ size_t wide_elem(size_t block, int j, uint32_t col) {
  return block * kBlock + (size_t)(128 * (j >> 1) + 8 * col + 4 * (j & 1));
}
__device__ __forceinline__ size_t pair_elem(size_t block, int j, uint32_t col) {
  return block * kBlock + (size_t)(64 * j + 2 * col);
}
template <int MAP>
__device__ __forceinline__ size_t vec_elem(size_t block, int j, uint32_t col) {
  return MAP == kMapWide ? wide_elem(block, j, col) : lane_elem(block, j, col);
}

typedef uint32_t u4w __attribute__((ext_vector_type(4)));

// 8 consecutive 2-byte values at element e as two binary32 vectors, and back.
template <int ET>
__device__ __forceinline__ void load8_half(const void* p, size_t e, f4& a, f4& b) {
  const u4w w = __builtin_nontemporal_load(reinterpret_cast<const u4w*>(static_cast<const uint16_t*>(p) + e));
  if constexpr (ET == GB_DTYPE_BF16) {
    a = bf16_unpack4(u2{w.x, w.y});
    b = bf16_unpack4(u2{w.z, w.w});
  } else {
    const h4 ha = __builtin_bit_cast(h4, u2{w.x, w.y}), hb = __builtin_bit_cast(h4, u2{w.z, w.w});
    a = f4{(float)ha.x, (float)ha.y, (float)ha.z, (float)ha.w};
    b = f4{(float)hb.x, (float)hb.y, (float)hb.z, (float)hb.w};
  }
}
template <int ET>
__device__ __forceinline__ void store8_half(void* p, size_t e, f4 a, f4 b) {
  u2 wa, wb;
  if constexpr (ET == GB_DTYPE_BF16) {
    wa = bf16_pack4(a);
    wb = bf16_pack4(b);
  } else {
    // as in store_vals4_at: the binary32 values must exist before rounding
    asm volatile("" : "+v"(a));
    asm volatile("" : "+v"(b));
    const h4 ha = {(_Float16)a.x, (_Float16)a.y, (_Float16)a.z, (_Float16)a.w};
    const h4 hb = {(_Float16)b.x, (_Float16)b.y, (_Float16)b.z, (_Float16)b.w};
    wa = __builtin_bit_cast(u2, ha);
    wb = __builtin_bit_cast(u2, hb);
  }
  __builtin_nontemporal_store(u4w{wa.x, wa.y, wb.x, wb.y}, reinterpret_cast<u4w*>(static_cast<uint16_t*>(p) + e));
}

// A lane's 4 vectors of a block as binary32 (converted as load_vals4_at
// converts), their store, and their codes (4 per word, value 0 in the low
// byte), placed by map MAP.
template <int ET, int MAP, bool FULL>
__device__ __forceinline__ void load_block(const void* p, size_t block, uint32_t col, size_t n, f4 (&x)[4]) {
  if constexpr (MAP == kMapPair) {
    const double* d = static_cast<const double*>(p);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const size_t e = pair_elem(block, j, col);
      const d2v lo = load_f64x2_at<FULL>(d, e, n), hi = load_f64x2_at<FULL>(d, e + 32, n);
      x[j] = f4{(float)lo.x, (float)lo.y, (float)hi.x, (float)hi.y};
    }
  } else if constexpr (MAP == kMapWide && FULL) {
#pragma unroll
    for (int m = 0; m < 2; m++) load8_half<ET>(p, wide_elem(block, 2 * m, col), x[2 * m], x[2 * m + 1]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; j++) x[j] = load_vals4_at<ET, FULL>(p, vec_elem<MAP>(block, j, col), n);
  }
}
template <int ET, int MAP, bool FULL>
__device__ __forceinline__ void store_block(void* p, size_t block, uint32_t col, size_t n, const f4 (&v)[4]) {
  if constexpr (MAP == kMapPair) {
    double* d = static_cast<double*>(p);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const size_t e = pair_elem(block, j, col);
      store_f64x2_at<FULL>(d, e, n, d2v{(double)v[j].x, (double)v[j].y});
      store_f64x2_at<FULL>(d, e + 32, n, d2v{(double)v[j].z, (double)v[j].w});
    }
  } else if constexpr (MAP == kMapWide && FULL) {
#pragma unroll
    for (int m = 0; m < 2; m++) store8_half<ET>(p, wide_elem(block, 2 * m, col), v[2 * m], v[2 * m + 1]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; j++) store_vals4_at<ET, FULL>(p, vec_elem<MAP>(block, j, col), n, v[j]);
  }
}
template <int MAP, bool FULL>
__device__ __forceinline__ void load_block_codes(const uint8_t* c, size_t block, uint32_t col, size_t n,
                                                 uint32_t (&w)[4]) {
  if constexpr (MAP == kMapPair) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const size_t e = pair_elem(block, j, col);
      w[j] = load_codes2_at<FULL>(c, e, n) | (load_codes2_at<FULL>(c, e + 32, n) << 16);
    }
  } else if constexpr (MAP == kMapWide && FULL) {
#pragma unroll
    for (int m = 0; m < 2; m++) {
      const u2 v = __builtin_nontemporal_load(reinterpret_cast<const u2*>(c + wide_elem(block, 2 * m, col)));
      w[2 * m] = v.x;
      w[2 * m + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; j++) w[j] = load_codes4_at<FULL>(c, vec_elem<MAP>(block, j, col), n);
  }
}
template <int MAP, bool FULL>
__device__ __forceinline__ void store_block_codes(uint8_t* c, size_t block, uint32_t col, size_t n,
                                                  const uint32_t (&w)[4]) {
  if constexpr (MAP == kMapPair) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const size_t e = pair_elem(block, j, col);
      store_codes2_at<FULL>(c, e, n, w[j] & 0xFFFFu);
      store_codes2_at<FULL>(c, e + 32, n, w[j] >> 16);
    }
  } else if constexpr (MAP == kMapWide && FULL) {
#pragma unroll
    for (int m = 0; m < 2; m++) {
      __builtin_nontemporal_store(u2{w[2 * m], w[2 * m + 1]}, reinterpret_cast<u2*>(c + wide_elem(block, 2 * m, col)));
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; j++) store_codes4_at<FULL>(c, vec_elem<MAP>(block, j, col), n, w[j]);
  }
}

// A float32 array (an error-feedback residual) on the narrow or pair map.
template <int MAP, bool FULL>
__device__ __forceinline__ void load_block_f32(const float* p, size_t block, uint32_t col, size_t n, f4 (&x)[4]) {
  static_assert(MAP != kMapWide, "residuals use the narrow or the pair map");
#pragma unroll
  for (int j = 0; j < 4; j++) {
    if constexpr (MAP == kMapPair) {
      const size_t e = pair_elem(block, j, col);
      const f2 lo = load_f32x2_at<FULL>(p, e, n), hi = load_f32x2_at<FULL>(p, e + 32, n);
      x[j] = f4{lo.x, lo.y, hi.x, hi.y};
    } else {
      x[j] = load4_at<FULL>(p, lane_elem(block, j, col), n);
    }
  }
}
template <int MAP, bool FULL>
__device__ __forceinline__ void store_block_f32(float* p, size_t block, uint32_t col, size_t n, const f4 (&v)[4]) {
  static_assert(MAP != kMapWide, "residuals use the narrow or the pair map");
#pragma unroll
  for (int j = 0; j < 4; j++) {
    if constexpr (MAP == kMapPair) {
      const size_t e = pair_elem(block, j, col);
      store_f32x2_at<FULL>(p, e, n, f2{v[j].x, v[j].y});
      store_f32x2_at<FULL>(p, e + 32, n, f2{v[j].z, v[j].w});
    } else {
      store4_at<FULL>(p, lane_elem(block, j, col), n, v[j]);
    }
  }
}

// Encodes a lane's 16 values of one block (all 64 lanes must be active):
// returns the block scale and writes the 4 packed code words to w.
__device__ __forceinline__ float encode_block16(const f4 (&x)[4], int mode, uint32_t (&w)[4]) {
  const float s = block_scale(row_max16(lane_absmax16(x)), mode);
  const double rinv = scale_reciprocal(s);
  const bool subnormal_scale = s > 0.0f && s < 0x1p-126f;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    f4 v = quotient4(x[j], rinv);
    if (subnormal_scale) v = clamp448(v);
    w[j] = e4m3_pack4(v, x[j]);
  }
  return s;
}

// The same for a block spread over one whole wavefront, 4 values per lane:
// the lane maximum as lane_absmax16 takes it, the block maximum from the 4
// row maxima.  Requires all 64 lanes active.
__device__ __forceinline__ uint32_t lane_absmax4(f4 x) {
  uint32_t a = max(max(fbits(x.x) & 0x7FFFFFFFu, fbits(x.y) & 0x7FFFFFFFu),
                   max(fbits(x.z) & 0x7FFFFFFFu, fbits(x.w) & 0x7FFFFFFFu));
  if (a > 0x7F800000u) {
    a = 0u;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const uint32_t m = fbits(x[e]) & 0x7FFFFFFFu;
      a = max(a, m > 0x7F800000u ? 0u : m);
    }
  }
  return a;
}
__device__ __forceinline__ uint32_t wave_max64(uint32_t v) {
  v = row_max16(v);
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}
__device__ __forceinline__ float encode_block4(f4 x, int mode, uint32_t& w) {
  const float s = block_scale(wave_max64(lane_absmax4(x)), mode);
  const double rinv = scale_reciprocal(s);
  f4 v = quotient4(x, rinv);
  if (s > 0.0f && s < 0x1p-126f) v = clamp448(v);
  w = e4m3_pack4(v, x);
  return s;
}

// Every kernel below runs one of two instantiations of its body per
// workgroup: FULL when the workgroup's whole range lies below n (all but the
// last workgroup of a launch), with no bounds test on any access, and the
// guarded one otherwise.  The choice is uniform across the workgroup.
constexpr size_t kVecPerGroup = (size_t)kThreads * 4;       // 1024 values: one 4-vector per lane
constexpr size_t kBlocksPerGroup = kThreads / 16;          // 16 fp8 blocks: one per 16-lane row

// Order in which a launch's workgroups take their groups.  Workgroups are
// dispatched in index order, round-robin over the 8 XCDs (index w runs on
// XCD w % 8), so the ones in flight at any time form a window of consecutive
// indices.  Within each run of Fronts * Spacing workgroups, index w takes
// group (w % Fronts) * Spacing + w / Fronts of that run: the window then
// sweeps Fronts regions of the stream Spacing groups apart instead of one
// contiguous region, and with 8 fronts each XCD streams a contiguous chunk of
// its own.  The tail of the grid that does not fill a whole run keeps the
// identity order, and so does every grid of fewer than MinRuns runs: the map
// is a permutation of [0, gridDim.x), and neither the grid nor any result
// depends on it.
//
// Measured on MI355X with every buffer at four different offsets: at 1e9
// values per rank the kernels over 1024-value vector groups move 2-7% more
// bytes per second with 8 fronts 256 groups (1 MiB of float32) apart, and
// the kernels over 4096-value fp8 groups 2-5% more with 4 fronts 256 groups
// (4 MiB of float32) apart; neighbouring spacings gain less or lose.  Below
// each order's MinRuns (16 runs, about 3.4e7 values, for the vector kernels;
// 8 runs, 1.7e7, for the reductions and the fused bf16 passes over float32;
// 4 runs, 8.4e6, for the bf16 decode into float32; 96 runs, about 4e8, for
// the fp8 kernels) the gain is not there and bucket-sized launches of a few
// million values lose up to 8%.
template <size_t Fronts, size_t Spacing, size_t MinRuns>
struct GroupOrder {
  static constexpr size_t fronts = Fronts, spacing = Spacing, min_runs = MinRuns;
};
using VecOrder = GroupOrder<8, 256, 16>;
// The reductions (the float32 sums and ops, and the typed reductions: 4 KiB
// of each source per workgroup) take the same order from 8 runs, 64 MiB per
// rank: from 8 to 16 runs it moves 1.3-5.2% more bytes per second than index
// order, for every element type and for 2 and 4 ranks.
using ReduceOrder = GroupOrder<8, 256, 8>;
// The fused bf16-codec passes over float32 gradients take it from 8 runs too
// (+3-7.5% between 8 and 16 runs; the plain bf16 decode loses there).
using FusedVecOrder = GroupOrder<8, 256, 8>;
using BlockOrder = GroupOrder<4, 256, 96>;
// The bf16 decode into float32 takes the vector order from 4 runs (2^23
// values of each payload): 4-rank decodes of 2^23 and 2^24 values moved
// 19-20% more bytes per second than in index order, and nothing changed
// from 2^26 up, where it was already permuted.
using DecodeBf16Order = GroupOrder<8, 256, 4>;
// The wide 4-rank sum (4 vectors per lane, 4096-value groups): 8 fronts 64
// groups apart, so each front still starts 1 MiB of float32 after the
// previous one, in every launch it is used for.
using WideSumOrder = GroupOrder<8, 64, 1>;

// The group of workgroup w of a grid of `grid` workgroups (also a bucket's
// share of a batched launch, w counted from the bucket's first workgroup).
template <class Order>
__device__ __forceinline__ size_t group_index_in(size_t w, size_t grid) {
  constexpr size_t F = Order::fronts, D = Order::spacing, run = F * D;
  if (grid < Order::min_runs * run || w >= grid / run * run) return w;
  return w / run * run + (w % F) * D + (w % run) / F;
}

template <class Order>
__device__ __forceinline__ size_t group_index() {
  return group_index_in<Order>(blockIdx.x, gridDim.x);
}

template <class Order>
__device__ __forceinline__ bool group_full(size_t per_group, size_t n) {
  return (group_index<Order>() + 1) * per_group <= n;
}

// A lane's 4 values of a 1024-value vector group sg (the bf16 codec's unit):
// 4 consecutive values at 4 t for a 1-, 2- or 4-byte type; for float64 two
// pairs, at 2 t and 512 values further, so that each 16-byte access of a
// wavefront covers 1 KiB contiguous (4 consecutive doubles would be 32 bytes
// per lane at half density) and each 4-byte code access 256 bytes.  Which
// lane holds which values changes no result.
template <int ET>
__device__ __forceinline__ size_t group_first(size_t sg, uint32_t t) {
  return sg * kVecPerGroup + (size_t)t * (ET == GB_DTYPE_F64 ? 2 : 4);
}
template <bool FULL>
__device__ __forceinline__ uint32_t load_bf16_2_at(const uint16_t* c, size_t e, size_t n) {
  if (FULL || e + 2 <= n) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(c + e));
  return e < n ? (uint32_t)c[e] : 0u;
}
template <bool FULL>
__device__ __forceinline__ void store_bf16_2_at(uint16_t* c, size_t e, size_t n, uint32_t w) {
  if (FULL || e + 2 <= n) __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(c + e));
  else if (e < n) c[e] = (uint16_t)w;
}
template <int ET, bool FULL>
__device__ __forceinline__ f4 load_group_vec(const void* p, size_t sg, uint32_t t, size_t n) {
  const size_t e = group_first<ET>(sg, t);
  if constexpr (ET != GB_DTYPE_F64) {
    return load_vals4_at<ET, FULL>(p, e, n);
  } else {
    const double* d = static_cast<const double*>(p);
    const d2v lo = load_f64x2_at<FULL>(d, e, n), hi = load_f64x2_at<FULL>(d, e + 512, n);
    return f4{(float)lo.x, (float)lo.y, (float)hi.x, (float)hi.y};
  }
}
template <int ET, bool FULL>
__device__ __forceinline__ void store_group_vec(void* p, size_t sg, uint32_t t, size_t n, f4 v) {
  const size_t e = group_first<ET>(sg, t);
  if constexpr (ET != GB_DTYPE_F64) {
    store_vals4_at<ET, FULL>(p, e, n, v);
  } else {
    double* d = static_cast<double*>(p);
    store_f64x2_at<FULL>(d, e, n, d2v{(double)v.x, (double)v.y});
    store_f64x2_at<FULL>(d, e + 512, n, d2v{(double)v.z, (double)v.w});
  }
}
// The 4 bf16 codes of those values, value 0 in the low half of word 0.
template <int ET, bool FULL>
__device__ __forceinline__ u2 load_group_bf16(const uint16_t* c, size_t sg, uint32_t t, size_t n) {
  const size_t e = group_first<ET>(sg, t);
  if constexpr (ET != GB_DTYPE_F64) return load_bf16_4_at<FULL>(c, e, n);
  else return u2{load_bf16_2_at<FULL>(c, e, n), load_bf16_2_at<FULL>(c, e + 512, n)};
}
template <int ET, bool FULL>
__device__ __forceinline__ void store_group_bf16(uint16_t* c, size_t sg, uint32_t t, size_t n, u2 w) {
  const size_t e = group_first<ET>(sg, t);
  if constexpr (ET != GB_DTYPE_F64) {
    store_bf16_4_at<FULL>(c, e, n, w);
  } else {
    store_bf16_2_at<FULL>(c, e, n, w.x);
    store_bf16_2_at<FULL>(c, e + 512, n, w.y);
  }
}
template <int MAP, bool FULL>
__device__ __forceinline__ f4 load_group_f32(const float* p, size_t sg, uint32_t t, size_t n) {
  const size_t e = group_first<MAP>(sg, t);
  if constexpr (MAP != GB_DTYPE_F64) {
    return load4_at<FULL>(p, e, n);
  } else {
    const f2 lo = load_f32x2_at<FULL>(p, e, n), hi = load_f32x2_at<FULL>(p, e + 512, n);
    return f4{lo.x, lo.y, hi.x, hi.y};
  }
}
template <int MAP, bool FULL>
__device__ __forceinline__ void store_group_f32(float* p, size_t sg, uint32_t t, size_t n, f4 v) {
  const size_t e = group_first<MAP>(sg, t);
  if constexpr (MAP != GB_DTYPE_F64) {
    store4_at<FULL>(p, e, n, v);
  } else {
    store_f32x2_at<FULL>(p, e, n, f2{v.x, v.y});
    store_f32x2_at<FULL>(p, e + 512, n, f2{v.z, v.w});
  }
}

// ---------------------------------------------------------------------------
// Launch helpers.
// ---------------------------------------------------------------------------

// AVG of a float32 total fused into a bucket pass (README "API": AVG is the
// SUM divided by the world size; a compressed AVG is the decode-and-add,
// then the division): DIV 0 leaves the total, 1 multiplies it by the exact
// reciprocal of a power-of-two divisor (the quotient rounded once, as a
// divide), 2 divides it (IEEE binary32 division, correctly rounded).
template <int DIV, int NV>
__device__ __forceinline__ void avg_total(f4 (&a)[NV], float d, float inv) {
  if (DIV == 0) return;
#pragma unroll
  for (int j = 0; j < NV; j++) {
#pragma unroll
    for (int e = 0; e < 4; e++) a[j][e] = DIV == 1 ? a[j][e] * inv : a[j][e] / d;
  }
}

// Dynamic LDS reserved per workgroup: an occupancy cap.  No kernel uses LDS;
// reserving 48, 64 or 81 KiB of the 160 KiB a compute unit has caps it at 3,
// 2 or 1 such workgroups.  A kernel that keeps many bytes of loads in flight
// per lane moves more bytes per second with fewer workgroups at once (fewer
// concurrent streams of requests at the memory); one with few bytes per lane
// loses under any cap.  Each rule below was measured on MI355X against the
// other caps in one process, with the same bits; sizes are values per rank.
constexpr unsigned kThreePerCuLds = 48u << 10;
constexpr unsigned kTwoPerCuLds = 64u << 10;
constexpr unsigned kOnePerCuLds = 81u << 10;
// Two per unit over k >= 4 ranks (also the fused sum-and-encode fp8 pass).
__host__ __device__ constexpr unsigned heavy_lds(int k) { return k >= 4 ? kTwoPerCuLds : 0u; }
// One per unit over k >= 4 ranks.
__host__ __device__ constexpr unsigned ef_lds(int k) { return k >= 4 ? kOnePerCuLds : 0u; }

// Fused fp8 pass (16k bytes of loads per lane for float32 gradients): 2 per
// unit, about 4% ahead of the 5 its registers allow at 1e9 values.  Float64
// gradients (32k bytes per lane) at 1: 5% ahead at 5e8, level at 6.7e7.
// Half-precision gradients keep half the float32 bytes in flight: uncapped
// below 2^26 values (float16 5.8% and bfloat16 2.3% ahead at one bucket),
// and at 2 from there up, as float32.
template <int ET>
__host__ __device__ constexpr unsigned fused_fp8_lds(int k, size_t n) {
  if (ET == GB_DTYPE_F64) return ef_lds(k);
  if ((ET == GB_DTYPE_F16 || ET == GB_DTYPE_BF16) && n < ((size_t)1 << 26)) return 0u;
  return heavy_lds(k);
}

// Fused fp8 pass over float32 gradients of large buffers: 128-lane
// workgroups (8 blocks, two wavefronts each) in index order, from 2^27
// values per rank over 3 to 8 ranks and from 2^28 over 2, capped at 2 per
// unit over k >= 4 ranks and at 3 over 2 or 3.  Measured on MI355X against
// the 256-lane kernel (2 per unit; 4 fronts from about 4e8 values) in one
// process, same bits: 2-9% more bytes per second at 2^27, 2^28 and 6.3e8
// values for 3, 4, 6 and 8 ranks, 1-2% at 1e9 over 4, and 4-6% over 2 ranks
// from 2^28; the 256-lane workgroup at 1 per unit (the same 4 wavefronts per
// unit) and every permuted order of the 128-lane one did worse, and so did
// the 128-lane shape at bucket sizes (6,553,600 values) and up to 2^26.
//
// Float64 gradients take the 128-lane shape at 2 per unit from 3 * 2^21
// values, up to 3 ranks at every size and over more only below 2^29: from
// one bucket to 2^28 values 1.3-10.9% more bytes per second over 2, 3, 4, 6
// and 8 ranks; at 1e9 +8% over 2 ranks and +4.7% over 3, level over 4
// (+0.0% and +1.2% in two runs) and -1.7 to -2.4% over 6 and 8; at 2^20
// values it lost up to 10%, and at 2^22 4-5% over 2 and 3 ranks.  Measured
// on MI355X against the library's 256-lane kernel in one process, same
// bits; in the benchmark's bucket stream over 4 ranks, against the library
// without the rule on the same machine: +3.7-4.0% at 1.25e8 values per
// rank, and one call per 6,553,600-value bucket +6.4% on one stream and
// +2.7% over two.  Float16 and bfloat16 gradients keep the 256-lane kernel:
// uncapped 128-lane workgroups gained up to 9.6% between 2^22 and 2^26
// values in one process, but the benchmark's one call per bucket (6,553,600
// values) gained 1% on one stream and lost 2-3% over two and four.
constexpr int kHalfThreads = 128;
template <int ET>
__host__ __device__ constexpr bool fused_fp8_half(int k, size_t n) {
  if (ET == GB_DTYPE_F64) return n >= ((size_t)3 << 21) && (k <= 3 || n < ((size_t)1 << 29));
  if (ET == GB_DTYPE_F16 || ET == GB_DTYPE_BF16) return false;
  if (k == 4) return false;  // fused_fp8_wave below takes 4 ranks
  return (k >= 3 && n >= ((size_t)1 << 27)) || (k == 2 && n >= ((size_t)1 << 28));
}
template <int ET>
__host__ __device__ constexpr unsigned fused_fp8_half_lds(int k) {
  return ET == GB_DTYPE_F64 ? kTwoPerCuLds : (k >= 4 ? kTwoPerCuLds : kThreePerCuLds);
}

// Fused fp8 pass over float32 gradients of 4 ranks from 2^22 values per
// rank: one block per 64-lane workgroup (4 values per lane, so each load
// and store of a rank covers its 1 KiB, or 256 bytes of codes, in one
// piece) in index order, capped at 20 per unit (8 KiB of LDS each).  The
// block scale then costs its maximum, exact divide and reciprocal once per
// 256 values rather than once per 1,024, which at 13 per unit left the pass
// bound by that chain; at 20 per unit it is not.  Measured in the
// benchmark's bucket stream over 4 ranks, against the 128-lane kernel on
// the same machine, two machines, same bits: +2.5% and +4.5-5.5% at 1e9
// values, +4.8-5.0% at 5e8, +0.6-1.4% at 2.5e8.  Against the 256-lane
// kernel, three runs each on two machines: at 1.25e8 values -0.1 to -1.4%
// and +0.2 to +2.7%; one call per 6,553,600-value bucket +0.4 to +3.1% on
// one stream, -0.6 to +2.0% over two and +2.8 to +5.1% over four.  In one
// process it gained -0.4% to +4.4% at 1e9 values on three machines, lost
// 4-9% over 2 ranks and was level over 8 at 2^28, so the rule is for 4
// ranks only.
__host__ __device__ constexpr bool fused_fp8_wave(int k, size_t n) {
  return k == 4 && n >= ((size_t)1 << 22);
}
constexpr unsigned kFp8WaveLds = 8u << 10;

// The fp8 pass with error feedback over float32 gradients of 4 ranks in the
// same shape from 2^22 values per rank, at 6 per unit (24 KiB of LDS each;
// 32 bytes of each rank per lane in flight, source and residual).  In one
// process at 2^30 values, against the 256-lane kernel, same bits: uncapped
// and 20 or 13 per unit lost 1-6%, 10 per unit gained 2-3.5%, 8 per unit
// 5.5-6%, 6 per unit 6.7-7.1%, and 5 per unit lost 16%.  In the benchmark,
// against the 256-lane kernel on the same machine, two runs each, same
// bits: +8.9-9.1% at 1e9 values per rank on two machines, +5.5-8.2% at
// 5e8, +11.7-13.3% at 2.5e8, +11.2-13.0% at 1.25e8, and one call per
// 6,553,600-value bucket +4.3-5.1% (8 such buckets batched +0.6-2.8%).
//
// Bfloat16 and float16 gradients (24 bytes of each rank per lane in flight)
// take it too, at 8 per unit (20 KiB): in one process, same bits, against
// the 256-lane kernel, bfloat16 +4.5% at 2^30 values (10 per unit the
// same, 13 per unit +3%, 6 per unit -8.5%) and float16 +18.4% at 2^28 (10
// per unit +18%, 13 per unit +15.6%, 6 per unit +5%).  In the benchmark,
// against the 256-lane kernel on the same machine, two runs each, same
// bits: bfloat16 +4.6-5.6% at 1e9 values, +11.0-12.7% at 1.25e8, one call
// per 6,553,600-value bucket +4.9-6.3%, 8 such buckets batched +3.3-3.7%;
// float16 +3.8-6.7% at 1e9 values, +5.2-6.0% per bucket, +3.9-4.2%
// batched.  Float64 gradients lost 1.5-3.5% at every cap and keep the
// 256-lane kernel.
template <int ET>
__host__ __device__ constexpr bool fused_fp8_ef_wave(int k, size_t n) {
  return ET != GB_DTYPE_F64 && k == 4 && n >= ((size_t)1 << 22);
}
template <int ET>
__host__ __device__ constexpr unsigned fused_fp8_ef_wave_lds() {
  return ET == GB_DTYPE_F32 ? 24u << 10 : 20u << 10;
}

// The fp8 decode of 4 payloads into a float32 total in the same shape from
// 2^24 values, uncapped (the scales are uniform across a workgroup, so each
// is one load per wavefront).  In one process at 2^26 and 2^28 values: +5%
// and +10% against the 256-lane kernel uncapped or capped up to 6 KiB, and
// -2% to -28% at 8 and 12 KiB.  In the benchmark, against the 256-lane
// kernel on the same machine, two runs each, same bits: +8.8-10.8% at 2^26,
// +5.0-9.5% at 2^25, +8.4-11.7% at 2^24; level at 2^23 (-1.7% and +1.2%,
// launches of about 9 us).
__host__ __device__ constexpr bool decode_fp8_wave(int k, size_t n) {
  return k == 4 && n >= ((size_t)1 << 24);
}

// Fused fp8 pass with error feedback (21 streams at k = 4: sources and
// residuals read; codes, scales, residuals and the sum written): 1 per unit
// from 2^28 values up, 2-4% ahead of 2 or uncapped at 5e8 and 1e9 over every
// gradient type; uncapped below, 1-8% ahead, at one bucket too.
__host__ __device__ constexpr unsigned fused_fp8_ef_lds(int k, size_t n) {
  return n >= ((size_t)1 << 28) ? ef_lds(k) : 0u;
}

// fp8 decode-accumulate over k >= 4 payloads, by the type it writes: a
// float32 total at 3 per unit, 5% ahead of 2 from 6.55e6 to 2.5e8 values and
// level at 1e9; a half-precision total uncapped, 21-26% ahead of 2; a
// float64 total at 2.
template <int ET>
__host__ __device__ constexpr unsigned decode_fp8_lds(int k) {
  if (k < 4) return 0u;
  return ET == GB_DTYPE_F32 ? kThreePerCuLds : (ET == GB_DTYPE_F64 ? kTwoPerCuLds : 0u);
}

// Fused bf16 pass with error feedback (17 streams at k = 4): 1 per unit,
// for float32 gradients 2-4% ahead of 2 at every size from one bucket to 1e9
// values, for float64 and bfloat16 gradients up to 1.5% and 2% from 6.7e7
// up; float16 gradients at 2, 3% ahead of 1 at 1e9 and up to 2% ahead of
// uncapped from 3.3e7 up.
template <int ET>
__host__ __device__ constexpr unsigned fused_bf16_ef_lds(int k) {
  return ET == GB_DTYPE_F16 ? heavy_lds(k) : ef_lds(k);
}

// Fused bf16 pass over float32 gradients from 3 ranks: 64-lane workgroups
// (one wavefront, 256 values) in index order, uncapped below 3 * 2^21 values
// per rank and from there capped by rank count, at 13 per unit over 3
// ranks, 10 over 4, 8 over 5 or 6 and 6 over 7 or 8.  Measured on MI355X
// against the 256-lane kernel (its rules below) in one process, same bits:
// from one 25 MiB bucket (6,553,600 values) to 1e9 values, 2.5-8.6% more
// bytes per second over 3 ranks, 3.3-8.8% over 4, 5.8-10.8% over 5 and 6,
// 5-13% over 7 and 8; uncapped from 2^21 to 2^22 values 1-11%; about level
// at 2^20 and below.  The caps lose below 3 * 2^21 values, and two ranks
// gain nothing consistent, so they keep the 256-lane kernel.
constexpr int kWaveThreads = 64;
__host__ __device__ constexpr bool fused_bf16_wave(int k) { return k >= 3; }
// Workgroups of a 64-lane launch over n values (4 per 1024-value vector
// group), or 0 beyond the largest grid, where the 256-lane kernel runs.
__host__ __device__ constexpr size_t wave_grid_for(size_t n) {
  return (n + kVecPerGroup - 1) / kVecPerGroup * 4 <= kMaxGrid ? (n + kVecPerGroup - 1) / kVecPerGroup * 4 : 0;
}
static_assert(wave_grid_for((size_t)1 << 38) != 0, "a 64-lane grid up to 2^38 values");
static_assert(wave_grid_for(GB_MAX_N) == 0, "the largest calls fall back to 256-lane workgroups");
static_assert(GB_MAX_N / kVecPerGroup <= kMaxGrid, "and those fit a 256-lane grid");
// A 64-lane workgroup's place in the 256-lane vector groups: workgroup w
// (counted from its buffer's first) holds lanes 64 (w mod 4) ..
// 64 (w mod 4) + 63 of vector group w / 4, so every value is where a
// 256-lane workgroup puts it.
struct WaveLane {
  size_t sg;
  uint32_t t;
};
__device__ __forceinline__ WaveLane wave_lane(size_t w) {
  return WaveLane{w >> 2, ((uint32_t)(w & 3u) << 6) + threadIdx.x};
}
__host__ __device__ constexpr unsigned fused_bf16_wave_lds(int k, size_t n) {
  if (n < ((size_t)3 << 21)) return 0u;
  return k <= 3 ? (12u << 10) : k == 4 ? (16u << 10) : k <= 6 ? (20u << 10) : (24u << 10);
}
// The same 64-lane pass over float16 and bfloat16 gradients (half the bytes
// of a float32 lane in flight per rank): over 5 to 8 ranks from 2^22 values
// per rank, over 4 from 2^29; capped at 13 per unit over 4 or 5 ranks, 10
// over 6 or 7 and 8 over 8.  Measured on MI355X against the 256-lane kernel
// in one process, same bits, both types alike, on two machines.  At 1e9
// values +0.8-10% more bytes per second over every rank count from 4 to 8
// (one run -0.4% over 5), and over 4 ranks from 2^29 +0.2-5.3%.  Over 5 to 8
// ranks at 2^22-2^23 values +1-7%.  Between 6,553,600 values and 2^26 one
// machine gained 2-18% and the other was level (-4.4 to +6.3%).  Over 4
// ranks below 2^28 the second machine lost up to 6.8%, at 2^20 values every
// 64-lane shape lost 2-13%, and over 2 or 3 ranks nothing gained at every
// size.
// Over 4 ranks of float16 and bfloat16 gradients from 2^22 values the
// pass instead takes 8 values per lane (16-byte loads) in 64-lane
// workgroups at 10 per unit (16 KiB of LDS each).  In one process at 2^26
// and 2^30 values, same bits: +3.9-6.1% against the library's kernels at
// 10 per unit, less at 13 and below (uncapped -3 to -5%).  In the
// benchmark, against them on the same machine, two runs each: bfloat16
// +3.0-3.2% at 1e9 values and +5.4-5.6% at 1.25e8, float16 +0.9-1.2% at
// 1e9; one call per 6,553,600-value bucket +7.1-7.3% for both.
__host__ __device__ constexpr bool fused_bf16_eight(int k, size_t n) { return k == 4 && n >= ((size_t)1 << 22); }
constexpr unsigned kBf16EightLds = 16u << 10;
__host__ __device__ constexpr bool fused_bf16_half_wave(int k, size_t n) {
  return (k == 4 && n >= ((size_t)1 << 29)) || (k >= 5 && n >= ((size_t)1 << 22));
}
__host__ __device__ constexpr unsigned fused_bf16_half_wave_lds(int k) {
  return k <= 5 ? (12u << 10) : k <= 7 ? (16u << 10) : (20u << 10);
}

// Fused bf16 pass with error feedback over float32 gradients: 64-lane
// workgroups in index order at every size, capped by rank count (each lane
// keeps 32 bytes of every rank in flight: gradient and residual), at 13 per
// unit over 1 rank, 10 over 2, 6 over 3 or 4 and 5 over 5 to 8.  Measured on
// MI355X against the 256-lane kernel (its rule below) in one process, same
// bits: 4-24% more bytes per second from one 25 MiB bucket to 1e9 values
// over every rank count from 1 to 8 (4 ranks: +14.5% at a bucket, +12% at
// 1e9), and 2-19% at 2^20 and 2^22 values.
//
// Float16 and bfloat16 gradients (24 bytes of every rank in flight per lane:
// 8 of gradient, 16 of residual) take the 64-lane shape over 4 to 8 ranks at
// every size and over 2 or 3 from 2^22 values, capped at 13 per unit over 2
// ranks, 10 over 3, 8 over 4 and 6 over 5 to 8.  Float64 gradients (48
// bytes) take it over 2 and 4 to 8 ranks at every size and over 1 or 3 from
// 2^22 values, at 13 per unit over 1 rank, 10 over 2 and 6 over 3 to 8.
// Measured on MI355X against the 256-lane kernel (its rule below) in one
// process, same bits, from 2^20 values to 1e9 (1 to 4 ranks) or 2^26 (5 to 8
// ranks): bfloat16 +2.3-18.7% (4 to 8 ranks +4-18.7%), float16 +0.6-10.4%,
// float64 +0.9-12.9%.  Over 1 to 3 ranks at 2^20 values every 64-lane shape
// lost up to 7%; one rank of a 2-byte type gained only from 2^26 values
// (1-3%) and keeps the 256-lane kernel.
template <int ET>
__host__ __device__ constexpr bool fused_bf16_ef_wave(int k, size_t n) {
  if (ET == GB_DTYPE_F64) return (k == 1 || k == 3) ? n >= ((size_t)1 << 22) : true;
  if (ET == GB_DTYPE_F16 || ET == GB_DTYPE_BF16) return k >= 4 || (k >= 2 && n >= ((size_t)1 << 22));
  return true;
}
template <int ET>
__host__ __device__ constexpr unsigned fused_bf16_ef_wave_lds(int k) {
  if (ET == GB_DTYPE_F64) return k <= 1 ? (12u << 10) : k == 2 ? (16u << 10) : (24u << 10);
  if (ET == GB_DTYPE_F16 || ET == GB_DTYPE_BF16) {
    return k <= 2 ? (12u << 10) : k == 3 ? (16u << 10) : k == 4 ? (20u << 10) : (24u << 10);
  }
  return k <= 1 ? (12u << 10) : k == 2 ? (16u << 10) : k <= 4 ? (24u << 10) : (32u << 10);
}

// Plain fused bf16 pass: from 2^25 values up, float32 gradients at 3 per
// unit (2-4% ahead) and float64 gradients at 2 (1-5% ahead); both lose about
// 3% at bucket sizes, which stay uncapped.  Half-precision gradients are
// never capped: 22% behind at 2, and at 3 nothing that holds below 2.5e8.
template <int ET>
__host__ __device__ constexpr unsigned fused_bf16_lds(int k, size_t n) {
  if (k < 4 || n < ((size_t)1 << 25)) return 0u;
  return ET == GB_DTYPE_F32 ? kThreePerCuLds : (ET == GB_DTYPE_F64 ? kTwoPerCuLds : 0u);
}

size_t ceil_div(size_t a, size_t b) { return (a + b - 1) / b; }

// Workgroups for one lane per `per_lane` values, or 0 if too many.
size_t grid_for(size_t n, size_t per_lane) {
  const size_t g = ceil_div(ceil_div(n, per_lane), (size_t)kThreads);
  return g > kMaxGrid ? 0 : g;
}

#define GB_DISPATCH_K(k, CALL) \
  switch (k) {                 \
    case 1: CALL(1); break;    \
    case 2: CALL(2); break;    \
    case 3: CALL(3); break;    \
    case 4: CALL(4); break;    \
    case 5: CALL(5); break;    \
    case 6: CALL(6); break;    \
    case 7: CALL(7); break;    \
    case 8: CALL(8); break;    \
    default: return hipErrorInvalidValue; \
  }

// Switch on a codec kernel's element type (return CALL(ET)).
#define GB_DISPATCH_ET(et, CALL)                      \
  (void)hipGetLastError();                             \
  switch (et) {                                        \
    case GB_DTYPE_F32: return CALL(GB_DTYPE_F32);      \
    case GB_DTYPE_F16: return CALL(GB_DTYPE_F16);      \
    case GB_DTYPE_BF16: return CALL(GB_DTYPE_BF16);    \
    case GB_DTYPE_F64: return CALL(GB_DTYPE_F64);      \
    default: return hipErrorInvalidValue;              \
  }

}  // namespace
}  // namespace gb
