// gb_kernels.hip — HIP kernels of libgbreduce for gfx950 (AMD Instinct
// MI355X, CDNA4).
//
// All of this work streams HBM: a few integer and float operations per 4-byte
// element, no reuse, no contraction (so no MFMA).  The kernels are shaped for
// that:
//   * every lane moves 16-byte vectors (4-byte words for fp8 codes), and each
//     load or store instruction of a 16-lane row covers 256 contiguous bytes,
//     so requests coalesce into whole cache lines;
//   * loads and stores carry the non-temporal hint: each byte is touched once,
//     so nothing is worth keeping in L2 or the last-level cache;
//   * a lane issues all of its loads (every rank) before it computes, and the
//     k contributions of an element are combined in registers: reduce, encode
//     and decode-accumulate are fused where the call allows it;
//   * the fp8 block maximum is reduced across the 16 lanes of one DPP row (four
//     row-local DPP steps, no LDS, no barrier): a 256-value block is one row of
//     16 lanes holding 16 values each, a wavefront works on 4 blocks and a
//     256-lane workgroup on 16;
//   * E4M3 conversion uses gfx950's packed converters (v_cvt_pk_fp8_f32 to
//     encode two values per instruction, v_cvt_pk_f32_fp8 to decode two).
//
// Arithmetic follows the gpubridge README, "How it works" (sum of island sums)
// and "Bridge compression" (bf16; OCP E4M3 with one scale per 256 values;
// decode and add in float32).  Every rounding is IEEE binary32
// round-to-nearest-even with subnormals kept, and nothing is contracted into a
// fused multiply-add (built with -ffp-contract=off), so results do not depend
// on the launch shape.
#include <hip/hip_runtime.h>

#include "gb_internal.h"

namespace gb {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

struct OutTable {
  void* p[GB_MAX_K];
};

constexpr int kThreads = 256;  // 4 wavefronts of 64 lanes

__device__ __forceinline__ uint32_t fbits(float x) { return __float_as_uint(x); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __uint_as_float(u); }

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

// Every kernel below runs one of two instantiations of its body per
// workgroup: FULL when the workgroup's whole range lies below n (all but the
// last workgroup of a launch), with no bounds test on any access, and the
// guarded one otherwise.  The choice is uniform across the workgroup.
constexpr size_t kVecPerGroup = (size_t)kThreads * 4;       // 1024 values: one 4-vector per lane
constexpr size_t kBlocksPerGroup = kThreads / 16;          // 16 fp8 blocks: one per 16-lane row

__device__ __forceinline__ bool group_full(size_t per_group, size_t n) {
  return ((size_t)blockIdx.x + 1) * per_group <= n;
}

// ===========================================================================
// Fixed-order sum: dst = [dst +] src0 + src1 + ... + src(K-1), one 4-value
// vector per lane.
// ===========================================================================
template <int K, bool ACC, bool FULL>
__device__ __forceinline__ void reduce_sum_body(float* dst, const PtrTable& src, size_t n) {
  const size_t i = ((size_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (!FULL && i >= n) return;
  f4 x[K];
  f4 a;
#pragma unroll
  for (int r = 0; r < K; r++) x[r] = load4_at<FULL>(static_cast<const float*>(src.p[r]), i, n);
  if (ACC) a = load4_at<FULL>(dst, i, n);
  f4 s = ACC ? a + x[0] : x[0];
#pragma unroll
  for (int r = 1; r < K; r++) s = s + x[r];
  store4_at<FULL>(dst, i, n, s);
}

template <int K, bool ACC>
__global__ __launch_bounds__(kThreads) void reduce_sum_kernel(float* dst, PtrTable src, size_t n) {
  if (group_full(kVecPerGroup, n)) reduce_sum_body<K, ACC, true>(dst, src, n);
  else reduce_sum_body<K, ACC, false>(dst, src, n);
}

// ===========================================================================
// AVG, MAX and MIN over K sources (README "API": all_reduce takes SUM, AVG,
// MAX or MIN; AVG is the SUM divided by the world size).  AVG divides the
// fixed-order sum by d with a correctly rounded binary32 divide; MAX and MIN
// are the IEEE 754-2019 maximum and minimum (NaN propagates, -0 < +0), which
// gfx950 executes as v_maximum3_f32 / v_minimum3_f32.
// ===========================================================================
template <int K, int OP, bool FULL, bool P2>
__device__ __forceinline__ void reduce_op_body(float* dst, const PtrTable& src, size_t n, float d, float inv) {
  const size_t i = ((size_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (!FULL && i >= n) return;
  f4 x[K];
#pragma unroll
  for (int r = 0; r < K; r++) x[r] = load4_at<FULL>(static_cast<const float*>(src.p[r]), i, n);
  f4 s = x[0];
#pragma unroll
  for (int r = 1; r < K; r++) {
    if (OP == GB_OP_AVG) s = s + x[r];
    if (OP == GB_OP_MAX) s = __builtin_elementwise_maximum(s, x[r]);
    if (OP == GB_OP_MIN) s = __builtin_elementwise_minimum(s, x[r]);
  }
  // a power-of-two d: s * (1/d) is the exact quotient rounded once, as s / d
  if (OP == GB_OP_AVG) s = P2 ? s * inv : s / d;
  store4_at<FULL>(dst, i, n, s);
}

template <int K, int OP>
__global__ __launch_bounds__(kThreads) void reduce_op_kernel(float* dst, PtrTable src, size_t n, float d, float inv) {
  const bool full = group_full(kVecPerGroup, n);
  if (OP == GB_OP_AVG && inv != 0.0f) {
    if (full) reduce_op_body<K, OP, true, true>(dst, src, n, d, inv);
    else reduce_op_body<K, OP, false, true>(dst, src, n, d, inv);
  } else {
    if (full) reduce_op_body<K, OP, true, false>(dst, src, n, d, inv);
    else reduce_op_body<K, OP, false, false>(dst, src, n, d, inv);
  }
}

// ===========================================================================
// Reductions over the README's other element types ("API": float16,
// bfloat16, float64, int8, uint8, int32, int64).  Each lane owns 16 bytes of
// every source (8 halves, 2 doubles, 16 / 4 / 2 integers).  Half-precision
// sums add in binary32 and round back to the type after every add (exact:
// 24 >= 2p + 2 bits, so the second rounding cannot go wrong; Figueroa, "When
// is double rounding innocuous?").  The AVG divisor is any integer up to 2^24,
// not a half value, so that argument does not cover the quotient: it is
// formed in binary32 rounded to odd, after which one rounding to the type is
// the correctly rounded quotient (Boldo and Melquiond, "Emulation of FMA and
// correctly rounded sums: proved algorithms using rounding to odd").  Doubles
// divide natively.  MAX / MIN are IEEE 754-2019 for floating types and the
// plain order for integers; integer sums wrap.  A power-of-two divisor
// multiplies by its exact reciprocal instead of dividing: the product is the
// same once-rounded quotient, at a fraction of a divide's instructions.
// ===========================================================================
typedef uint32_t w4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef double d2 __attribute__((ext_vector_type(2)));

template <bool FULL>
__device__ __forceinline__ w4 load16_at(const void* p, size_t byte, size_t nbytes) {
  if (FULL || byte + 16 <= nbytes) {
    return __builtin_nontemporal_load(reinterpret_cast<const w4*>(static_cast<const char*>(p) + byte));
  }
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  const unsigned char* b = static_cast<const unsigned char*>(p) + byte;
  for (int i = 0; i < 16; i++) {
    if (byte + i < nbytes) w[i >> 2] |= (uint32_t)b[i] << (8 * (i & 3));
  }
  return w4{w[0], w[1], w[2], w[3]};
}
template <bool FULL>
__device__ __forceinline__ void store16_at(void* p, size_t byte, size_t nbytes, w4 v) {
  if (FULL || byte + 16 <= nbytes) {
    __builtin_nontemporal_store(v, reinterpret_cast<w4*>(static_cast<char*>(p) + byte));
    return;
  }
  unsigned char* b = static_cast<unsigned char*>(p) + byte;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  for (int i = 0; i < 16; i++) {
    if (byte + i < nbytes) b[i] = (unsigned char)(w[i >> 2] >> (8 * (i & 3)));
  }
}

__device__ __forceinline__ float round_f16(float x) { return (float)(_Float16)x; }
__device__ __forceinline__ float round_bf16(float x) { return bitsf(bf16_code(x) << 16); }

template <int DT>
constexpr bool kHalfType = DT == GB_DTYPE_F16 || DT == GB_DTYPE_BF16;

// The 8 values of a 16-byte group of halves, as binary32 (exact).
template <int DT>
__device__ __forceinline__ void unpack_half8(w4 v, float f[8]) {
  if (DT == GB_DTYPE_F16) {
    const h8 h = __builtin_bit_cast(h8, v);
#pragma unroll
    for (int e = 0; e < 8; e++) f[e] = (float)h[e];
  } else {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; e++) {
      f[2 * e] = bitsf(w[e] << 16);
      f[2 * e + 1] = bitsf(w[e] & 0xFFFF0000u);
    }
  }
}

// Codes of 8 binary32 values that are each exactly a value of the type (or
// NaN with the type's payload), so packing rounds nothing.
template <int DT>
__device__ __forceinline__ w4 pack_half8(const float f[8]) {
  if (DT == GB_DTYPE_F16) {
    h8 h;
#pragma unroll
    for (int e = 0; e < 8; e++) h[e] = (_Float16)f[e];
    return __builtin_bit_cast(w4, h);
  }
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; e++) w[e] = (fbits(f[2 * e]) >> 16) | (fbits(f[2 * e + 1]) & 0xFFFF0000u);
  return w4{w[0], w[1], w[2], w[3]};
}

__device__ __forceinline__ float round_half(float x, bool f16) { return f16 ? round_f16(x) : round_bf16(x); }

// a = op(a, v) over 8 half values held as binary32; a SUM rounds to the type
// after every add.
template <int DT, int OP>
__device__ __forceinline__ void fold_half8(float a[8], w4 v) {
  float b[8];
  unpack_half8<DT>(v, b);
#pragma unroll
  for (int e = 0; e < 8; e++) {
    if (OP == GB_OP_SUM || OP == GB_OP_AVG) a[e] = round_half(a[e] + b[e], DT == GB_DTYPE_F16);
    else if (OP == GB_OP_MAX) a[e] = __builtin_elementwise_maximum(a[e], b[e]);
    else a[e] = __builtin_elementwise_minimum(a[e], b[e]);
  }
}

// Four 8-bit lanes of a dword.  SUM wraps each byte: the low seven bits add
// without crossing lanes and the top bit is their carry xor both top bits.
// MAX / MIN split the even and odd bytes into 16-bit halves (each 0..255)
// and take packed 16-bit unsigned max / min; int8 is first biased by 0x80,
// which maps its order onto uint8's.
typedef uint16_t us2 __attribute__((ext_vector_type(2)));
template <bool SIGNED, int OP>
__device__ __forceinline__ uint32_t combine_bytes(uint32_t a, uint32_t b) {
  if (OP == GB_OP_SUM) return ((a & 0x7F7F7F7Fu) + (b & 0x7F7F7F7Fu)) ^ ((a ^ b) & 0x80808080u);
  if (SIGNED) { a ^= 0x80808080u; b ^= 0x80808080u; }
  const us2 ae = __builtin_bit_cast(us2, a & 0x00FF00FFu), be = __builtin_bit_cast(us2, b & 0x00FF00FFu);
  const us2 ao = __builtin_bit_cast(us2, (a >> 8) & 0x00FF00FFu), bo = __builtin_bit_cast(us2, (b >> 8) & 0x00FF00FFu);
  const us2 re = OP == GB_OP_MAX ? __builtin_elementwise_max(ae, be) : __builtin_elementwise_min(ae, be);
  const us2 ro = OP == GB_OP_MAX ? __builtin_elementwise_max(ao, bo) : __builtin_elementwise_min(ao, bo);
  uint32_t r = __builtin_bit_cast(uint32_t, re) | (__builtin_bit_cast(uint32_t, ro) << 8);
  if (SIGNED) r ^= 0x80808080u;
  return r;
}

// One 16-byte group: acc = op(acc, v) element by element, in the type.
// One 16-byte group of a type other than the half-precision ones:
// acc = op(acc, v) element by element, in the type.
template <int DT, int OP>
__device__ __forceinline__ w4 combine16(w4 acc, w4 v) {
  if (DT == GB_DTYPE_F64) {
    d2 a = __builtin_bit_cast(d2, acc), b = __builtin_bit_cast(d2, v);
    if (OP == GB_OP_SUM || OP == GB_OP_AVG) a = a + b;
    else if (OP == GB_OP_MAX) a = __builtin_elementwise_maximum(a, b);
    else a = __builtin_elementwise_minimum(a, b);
    return __builtin_bit_cast(w4, a);
  } else if (DT == GB_DTYPE_I32) {
    typedef int32_t i4 __attribute__((ext_vector_type(4)));
    const i4 a = __builtin_bit_cast(i4, acc), b = __builtin_bit_cast(i4, v);
    if (OP == GB_OP_SUM) return acc + v;  // unsigned: wraps
    return __builtin_bit_cast(w4, OP == GB_OP_MAX ? __builtin_elementwise_max(a, b) : __builtin_elementwise_min(a, b));
  } else if (DT == GB_DTYPE_I64) {
    typedef int64_t l2 __attribute__((ext_vector_type(2)));
    typedef uint64_t ul2 __attribute__((ext_vector_type(2)));
    const l2 a = __builtin_bit_cast(l2, acc), b = __builtin_bit_cast(l2, v);
    if (OP == GB_OP_SUM) return __builtin_bit_cast(w4, __builtin_bit_cast(ul2, acc) + __builtin_bit_cast(ul2, v));
    return __builtin_bit_cast(w4, OP == GB_OP_MAX ? __builtin_elementwise_max(a, b) : __builtin_elementwise_min(a, b));
  } else {  // 8-bit: four lanes of a dword at a time
    const uint32_t wa[4] = {acc.x, acc.y, acc.z, acc.w}, wb[4] = {v.x, v.y, v.z, v.w};
    uint32_t r[4];
#pragma unroll
    for (int e = 0; e < 4; e++) r[e] = combine_bytes<DT == GB_DTYPE_I8, OP>(wa[e], wb[e]);
    return w4{r[0], r[1], r[2], r[3]};
  }
}

// a / d in binary32 rounded to odd: the nearest quotient q, replaced by its
// neighbour towards the exact quotient when q is inexact and its last
// significand bit is even.  The sign of the residual q*d - a gives the side;
// one fma gets that sign right, since the exact residual is a multiple of
// the least subnormal and so never rounds to zero.  Inf and NaN quotients
// pass through: their residual is NaN.
template <bool P2>
__device__ __forceinline__ float div_round_odd(float a, float d, float inv) {
  // a power-of-two d: a * (1/d) is the exact quotient rounded once, as a / d
  const float q = P2 ? a * inv : a / d;
  const float r = __builtin_fmaf(q, d, -a);
  uint32_t b = fbits(q);
  if ((r < 0.0f || r > 0.0f) && !(b & 1u)) {
    const bool grow = (r > 0.0f) == (a < 0.0f);  // |q| below |a / d|
    b = grow ? b + 1u : b - 1u;
  }
  return bitsf(b);
}

// Divisor of an AVG: d in binary32 and binary64, and for a power of two its
// exact reciprocal (1 / d is then a power of two in range of both formats).
struct Divisor {
  float f, inv_f;
  double d, inv_d;
};

template <bool P2>
__device__ __forceinline__ d2 divide_f64x2(d2 a, const Divisor& dv) {
  return P2 ? a * dv.inv_d : a / dv.d;  // one rounding either way
}

template <int DT, bool P2>
__device__ __forceinline__ void divide_half8(float a[8], const Divisor& dv) {
#pragma unroll
  for (int e = 0; e < 8; e++) a[e] = round_half(div_round_odd<P2>(a[e], dv.f, dv.inv_f), DT == GB_DTYPE_F16);
}

template <int DT, int K, int OP, bool FULL, bool P2>
__device__ __forceinline__ void reduce_typed_body(void* dst, const PtrTable& src, size_t nbytes, const Divisor& dv) {
  const size_t byte = ((size_t)blockIdx.x * kThreads + threadIdx.x) * 16;
  if (!FULL && byte >= nbytes) return;
  // Loads: all K at once in a full workgroup; rank by rank in the one ragged
  // workgroup, so that its byte-wise loads keep few registers live (the
  // kernel's register count, and so every workgroup's occupancy, is the
  // larger of the two paths').
  w4 x[FULL ? K : 1];
  if (FULL) {
#pragma unroll
    for (int r = 0; r < K; r++) x[r] = load16_at<true>(src.p[r], byte, nbytes);
  } else {
    x[0] = load16_at<false>(src.p[0], byte, nbytes);
  }
  w4 out;
  if constexpr (kHalfType<DT>) {
    float a[8];
    unpack_half8<DT>(x[0], a);
    if (FULL) {
#pragma unroll
      for (int r = 1; r < K; r++) fold_half8<DT, OP>(a, x[r]);
    } else {
#pragma unroll 1
      for (int r = 1; r < K; r++) fold_half8<DT, OP>(a, load16_at<false>(src.p[r], byte, nbytes));
    }
    if (OP == GB_OP_AVG) divide_half8<DT, P2>(a, dv);
    out = pack_half8<DT>(a);
  } else {
    out = x[0];
    if (FULL) {
#pragma unroll
      for (int r = 1; r < K; r++) out = combine16<DT, OP>(out, x[r]);
    } else {
#pragma unroll 1
      for (int r = 1; r < K; r++) out = combine16<DT, OP>(out, load16_at<false>(src.p[r], byte, nbytes));
    }
    if (DT == GB_DTYPE_F64 && OP == GB_OP_AVG) {
      out = __builtin_bit_cast(w4, divide_f64x2<P2>(__builtin_bit_cast(d2, out), dv));
    }
  }
  store16_at<FULL>(dst, byte, nbytes, out);
}

template <int DT, int K, int OP>
__global__ __launch_bounds__(kThreads) void reduce_typed_kernel(void* dst, PtrTable src, size_t nbytes, Divisor dv,
                                                                 int pow2) {
  const bool full = group_full((size_t)kThreads * 16, nbytes);
  if (OP == GB_OP_AVG && pow2) {
    if (full) reduce_typed_body<DT, K, OP, true, true>(dst, src, nbytes, dv);
    else reduce_typed_body<DT, K, OP, false, true>(dst, src, nbytes, dv);
  } else {
    if (full) reduce_typed_body<DT, K, OP, true, false>(dst, src, nbytes, dv);
    else reduce_typed_body<DT, K, OP, false, false>(dst, src, nbytes, dv);
  }
}

// ===========================================================================
// bf16 encode and decode-accumulate: one 4-value vector per lane, so each
// instruction of a wavefront loads 1 KiB of fp32 and stores 512 bytes of
// codes (or the reverse), contiguously.
// ===========================================================================
template <int ET, bool FULL>
__device__ __forceinline__ void encode_bf16_body(uint16_t* codes, const void* src, size_t n) {
  const size_t i = ((size_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (!FULL && i >= n) return;
  store_bf16_4_at<FULL>(codes, i, n, bf16_pack4(load_vals4_at<ET, FULL>(src, i, n)));
}

template <int ET>
__global__ __launch_bounds__(kThreads) void encode_bf16_kernel(uint16_t* codes, const void* src, size_t n) {
  if (group_full(kVecPerGroup, n)) encode_bf16_body<ET, true>(codes, src, n);
  else encode_bf16_body<ET, false>(codes, src, n);
}

template <int K, bool ACC, int ET, bool FULL>
__device__ __forceinline__ void decode_bf16_body(void* acc, const PtrTable& codes, size_t n) {
  const size_t i = ((size_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (!FULL && i >= n) return;
  u2 w[K];
#pragma unroll
  for (int r = 0; r < K; r++) w[r] = load_bf16_4_at<FULL>(static_cast<const uint16_t*>(codes.p[r]), i, n);
  f4 a;
  if (ACC) a = load_vals4_at<ET, FULL>(acc, i, n);
#pragma unroll
  for (int r = 0; r < K; r++) {
    const f4 v = bf16_unpack4(w[r]);
    a = (!ACC && r == 0) ? v : a + v;
  }
  store_vals4_at<ET, FULL>(acc, i, n, a);
}

template <int K, bool ACC, int ET>
__global__ __launch_bounds__(kThreads) void decode_bf16_kernel(void* acc, PtrTable codes, size_t n) {
  if (group_full(kVecPerGroup, n)) decode_bf16_body<K, ACC, ET, true>(acc, codes, n);
  else decode_bf16_body<K, ACC, ET, false>(acc, codes, n);
}

// ===========================================================================
// fp8 encode: one DPP row per 256-value block.
// ===========================================================================
template <int ET, bool FULL>
__device__ __forceinline__ void encode_fp8_body(uint8_t* codes, float* scales, const void* src, size_t n,
                                                int mode) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t col = lane & 15u;
  const size_t block = (size_t)blockIdx.x * kBlocksPerGroup + (threadIdx.x >> 4);
  f4 x[4];
#pragma unroll
  for (int j = 0; j < 4; j++) x[j] = load_vals4_at<ET, FULL>(src, lane_elem(block, j, col), n);
  uint32_t w[4];
  const float s = encode_block16(x, mode, w);  // all 64 lanes take part
  if (!FULL && block * kBlock >= n) return;
  if (col == 0u) scales[block] = s;
#pragma unroll
  for (int j = 0; j < 4; j++) store_codes4_at<FULL>(codes, lane_elem(block, j, col), n, w[j]);
}

template <int ET>
__global__ __launch_bounds__(kThreads) void encode_fp8_kernel(uint8_t* codes, float* scales, const void* src,
                                                               size_t n, int mode) {
  if (group_full(kBlocksPerGroup * kBlock, n)) encode_fp8_body<ET, true>(codes, scales, src, n, mode);
  else encode_fp8_body<ET, false>(codes, scales, src, n, mode);
}

// ===========================================================================
// fp8 decode-accumulate over K payloads: one DPP row per block, each rank's
// block scale read once per lane.
// ===========================================================================
template <int K, bool ACC, int ET, bool FULL>
__device__ __forceinline__ void decode_fp8_body(void* acc, const PtrTable& codes, const PtrTable& scales,
                                                size_t n) {
  const uint32_t col = threadIdx.x & 15u;
  const size_t block = (size_t)blockIdx.x * kBlocksPerGroup + (threadIdx.x >> 4);
  if (!FULL && block * kBlock >= n) return;
  uint32_t w[K][4];
  float s[K];
#pragma unroll
  for (int r = 0; r < K; r++) {
    const uint8_t* c = static_cast<const uint8_t*>(codes.p[r]);
#pragma unroll
    for (int j = 0; j < 4; j++) w[r][j] = load_codes4_at<FULL>(c, lane_elem(block, j, col), n);
    s[r] = static_cast<const float*>(scales.p[r])[block];
  }
  f4 a[4];
  if (ACC) {
#pragma unroll
    for (int j = 0; j < 4; j++) a[j] = load_vals4_at<ET, FULL>(acc, lane_elem(block, j, col), n);
  }
#pragma unroll
  for (int r = 0; r < K; r++) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const f4 v = e4m3_unpack4(w[r][j]) * s[r];
      a[j] = (!ACC && r == 0) ? v : a[j] + v;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; j++) store_vals4_at<ET, FULL>(acc, lane_elem(block, j, col), n, a[j]);
}

template <int K, bool ACC, int ET>
__global__ __launch_bounds__(kThreads) void decode_fp8_kernel(void* acc, PtrTable codes, PtrTable scales,
                                                               size_t n) {
  if (group_full(kBlocksPerGroup * kBlock, n)) decode_fp8_body<K, ACC, ET, true>(acc, codes, scales, n);
  else decode_fp8_body<K, ACC, ET, false>(acc, codes, scales, n);
}

// ===========================================================================
// Fused fp8 bucket pass: read each rank's block once, write its payload
// (codes, scale), decode those codes and add them in rank order.
// ===========================================================================
template <int K, int ET, bool FULL>
__device__ __forceinline__ void fused_fp8_body(void* out, const PtrTable& src, const OutTable& codes,
                                               const OutTable& scales, size_t n, int mode) {
  const uint32_t col = threadIdx.x & 15u;
  const size_t block = (size_t)blockIdx.x * kBlocksPerGroup + (threadIdx.x >> 4);
  f4 x[K][4];
#pragma unroll
  for (int r = 0; r < K; r++) {
#pragma unroll
    for (int j = 0; j < 4; j++) x[r][j] = load_vals4_at<ET, FULL>(src.p[r], lane_elem(block, j, col), n);
  }
  const bool live = FULL || block * kBlock < n;
  f4 a[4];
#pragma unroll
  for (int r = 0; r < K; r++) {
    uint32_t w[4];
    const float s = encode_block16(x[r], mode, w);  // all 64 lanes take part
    uint8_t* c = static_cast<uint8_t*>(codes.p[r]);
    if (live) {
      if (col == 0u) static_cast<float*>(scales.p[r])[block] = s;
#pragma unroll
      for (int j = 0; j < 4; j++) store_codes4_at<FULL>(c, lane_elem(block, j, col), n, w[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const f4 v = e4m3_unpack4(w[j]) * s;
      a[j] = r == 0 ? v : a[j] + v;
    }
  }
  if (!live) return;
#pragma unroll
  for (int j = 0; j < 4; j++) store_vals4_at<ET, FULL>(out, lane_elem(block, j, col), n, a[j]);
}

template <int K, int ET>
__global__ __launch_bounds__(kThreads) void fused_fp8_kernel(void* out, PtrTable src, OutTable codes,
                                                              OutTable scales, size_t n, int mode) {
  if (group_full(kBlocksPerGroup * kBlock, n)) fused_fp8_body<K, ET, true>(out, src, codes, scales, n, mode);
  else fused_fp8_body<K, ET, false>(out, src, codes, scales, n, mode);
}

// ===========================================================================
// Fused bf16 bucket pass, one 4-value vector per lane.
// ===========================================================================
template <int K, int ET, bool FULL>
__device__ __forceinline__ void fused_bf16_body(void* out, const PtrTable& src, const OutTable& codes, size_t n) {
  const size_t i = ((size_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (!FULL && i >= n) return;
  f4 x[K];
#pragma unroll
  for (int r = 0; r < K; r++) x[r] = load_vals4_at<ET, FULL>(src.p[r], i, n);
  f4 a;
#pragma unroll
  for (int r = 0; r < K; r++) {
    const u2 w = bf16_pack4(x[r]);
    store_bf16_4_at<FULL>(static_cast<uint16_t*>(codes.p[r]), i, n, w);
    const f4 v = bf16_unpack4(w);
    a = r == 0 ? v : a + v;
  }
  store_vals4_at<ET, FULL>(out, i, n, a);
}

template <int K, int ET>
__global__ __launch_bounds__(kThreads) void fused_bf16_kernel(void* out, PtrTable src, OutTable codes, size_t n) {
  if (group_full(kVecPerGroup, n)) fused_bf16_body<K, ET, true>(out, src, codes, n);
  else fused_bf16_body<K, ET, false>(out, src, codes, n);
}

// ===========================================================================
// Error feedback (README "Bridge compression": each bridge member keeps a
// residual per buffer).  y = x + residual is encoded exactly as above, and
// the residual becomes y minus the value the payload decodes to (rounded
// binary32 subtraction; exact for bf16).  The residual is read and written
// in place by the lane that owns the value.
// ===========================================================================
template <bool FULL>
__device__ __forceinline__ void encode_bf16_ef_body(uint16_t* codes, float* res, const float* src, size_t n) {
  const size_t i = ((size_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (!FULL && i >= n) return;
  const f4 y = load4_at<FULL>(src, i, n) + load4_at<FULL>(res, i, n);
  const u2 w = bf16_pack4(y);
  store_bf16_4_at<FULL>(codes, i, n, w);
  store4_at<FULL>(res, i, n, y - bf16_unpack4(w));
}

__global__ __launch_bounds__(kThreads) void encode_bf16_ef_kernel(uint16_t* codes, float* res, const float* src,
                                                                   size_t n) {
  if (group_full(kVecPerGroup, n)) encode_bf16_ef_body<true>(codes, res, src, n);
  else encode_bf16_ef_body<false>(codes, res, src, n);
}

template <bool FULL>
__device__ __forceinline__ void encode_fp8_ef_body(uint8_t* codes, float* scales, float* res, const float* src,
                                                   size_t n, int mode) {
  const uint32_t col = threadIdx.x & 15u;
  const size_t block = (size_t)blockIdx.x * kBlocksPerGroup + (threadIdx.x >> 4);
  f4 x[4], r[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    x[j] = load4_at<FULL>(src, lane_elem(block, j, col), n);
    r[j] = load4_at<FULL>(res, lane_elem(block, j, col), n);
  }
#pragma unroll
  for (int j = 0; j < 4; j++) x[j] = x[j] + r[j];  // y
  uint32_t w[4];
  const float s = encode_block16(x, mode, w);  // all 64 lanes take part
  if (!FULL && block * kBlock >= n) return;
  if (col == 0u) scales[block] = s;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    store_codes4_at<FULL>(codes, lane_elem(block, j, col), n, w[j]);
    store4_at<FULL>(res, lane_elem(block, j, col), n, x[j] - e4m3_unpack4(w[j]) * s);
  }
}

__global__ __launch_bounds__(kThreads) void encode_fp8_ef_kernel(uint8_t* codes, float* scales, float* res,
                                                                  const float* src, size_t n, int mode) {
  if (group_full(kBlocksPerGroup * kBlock, n)) encode_fp8_ef_body<true>(codes, scales, res, src, n, mode);
  else encode_fp8_ef_body<false>(codes, scales, res, src, n, mode);
}

template <int K, bool FULL>
__device__ __forceinline__ void fused_fp8_ef_body(float* out, const PtrTable& src, const OutTable& resid,
                                                  const OutTable& codes, const OutTable& scales, size_t n,
                                                  int mode) {
  const uint32_t col = threadIdx.x & 15u;
  const size_t block = (size_t)blockIdx.x * kBlocksPerGroup + (threadIdx.x >> 4);
  f4 y[K][4];
#pragma unroll
  for (int r = 0; r < K; r++) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      y[r][j] = load4_at<FULL>(static_cast<const float*>(src.p[r]), lane_elem(block, j, col), n) +
                load4_at<FULL>(static_cast<const float*>(resid.p[r]), lane_elem(block, j, col), n);
    }
  }
  const bool live = FULL || block * kBlock < n;
  f4 a[4];
#pragma unroll
  for (int r = 0; r < K; r++) {
    uint32_t w[4];
    const float s = encode_block16(y[r], mode, w);  // all 64 lanes take part
    uint8_t* c = static_cast<uint8_t*>(codes.p[r]);
    float* rp = static_cast<float*>(resid.p[r]);
    if (live && col == 0u) static_cast<float*>(scales.p[r])[block] = s;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const f4 v = e4m3_unpack4(w[j]) * s;
      if (live) {
        store_codes4_at<FULL>(c, lane_elem(block, j, col), n, w[j]);
        store4_at<FULL>(rp, lane_elem(block, j, col), n, y[r][j] - v);
      }
      a[j] = r == 0 ? v : a[j] + v;
    }
  }
  if (!live) return;
#pragma unroll
  for (int j = 0; j < 4; j++) store4_at<FULL>(out, lane_elem(block, j, col), n, a[j]);
}

template <int K>
__global__ __launch_bounds__(kThreads) void fused_fp8_ef_kernel(float* out, PtrTable src, OutTable resid,
                                                                 OutTable codes, OutTable scales, size_t n,
                                                                 int mode) {
  if (group_full(kBlocksPerGroup * kBlock, n)) fused_fp8_ef_body<K, true>(out, src, resid, codes, scales, n, mode);
  else fused_fp8_ef_body<K, false>(out, src, resid, codes, scales, n, mode);
}

template <int K, bool FULL>
__device__ __forceinline__ void fused_bf16_ef_body(float* out, const PtrTable& src, const OutTable& resid,
                                                   const OutTable& codes, size_t n) {
  const size_t i = ((size_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (!FULL && i >= n) return;
  f4 y[K];
#pragma unroll
  for (int r = 0; r < K; r++) {
    y[r] = load4_at<FULL>(static_cast<const float*>(src.p[r]), i, n) +
           load4_at<FULL>(static_cast<const float*>(resid.p[r]), i, n);
  }
  f4 a;
#pragma unroll
  for (int r = 0; r < K; r++) {
    const u2 w = bf16_pack4(y[r]);
    const f4 v = bf16_unpack4(w);
    store_bf16_4_at<FULL>(static_cast<uint16_t*>(codes.p[r]), i, n, w);
    store4_at<FULL>(static_cast<float*>(resid.p[r]), i, n, y[r] - v);
    a = r == 0 ? v : a + v;
  }
  store4_at<FULL>(out, i, n, a);
}

template <int K>
__global__ __launch_bounds__(kThreads) void fused_bf16_ef_kernel(float* out, PtrTable src, OutTable resid,
                                                                  OutTable codes, size_t n) {
  if (group_full(kVecPerGroup, n)) fused_bf16_ef_body<K, true>(out, src, resid, codes, n);
  else fused_bf16_ef_body<K, false>(out, src, resid, codes, n);
}

// ---------------------------------------------------------------------------
// Launch helpers.
// ---------------------------------------------------------------------------
constexpr size_t kMaxGrid = ((size_t)1 << 31) - 1;

// Dynamic LDS reserved per workgroup by the kernels that keep the most bytes
// in flight.  No kernel uses LDS: reserving 64 KiB of the 160 KiB a compute
// unit has caps it at 2 such workgroups.  A fused fp8 pass over k >= 4 ranks
// keeps 16k bytes of loads in flight per lane; measured on MI355X at 1e9
// values per rank, 2 workgroups per compute unit move about 4% more bytes
// per second than the 5 its registers allow (fewer concurrent streams of
// requests at the memory), while 1 per unit is worse.  Kernels with fewer
// bytes per lane lose heavily under any cap and get none.
constexpr unsigned kHeavyLds = 64u << 10;
__host__ __device__ constexpr unsigned heavy_lds(int k) { return k >= 4 ? kHeavyLds : 0u; }

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

}  // namespace

hipError_t launch_reduce_sum(float* dst, const PtrTable& srcs, int k, size_t n, bool accumulate,
                             hipStream_t stream) {
  const size_t grid = grid_for(n, 4);
  if (grid == 0) return hipErrorInvalidValue;
  (void)hipGetLastError();
#define GB_CALL(K)                                                                     \
  if (accumulate) reduce_sum_kernel<K, true><<<grid, kThreads, 0, stream>>>(dst, srcs, n); \
  else reduce_sum_kernel<K, false><<<grid, kThreads, 0, stream>>>(dst, srcs, n);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

hipError_t launch_reduce_op(float* dst, const PtrTable& srcs, int k, size_t n, int op, int divisor,
                            hipStream_t stream) {
  const size_t grid = grid_for(n, 4);
  if (grid == 0) return hipErrorInvalidValue;
  const float d = (float)divisor;
  const float inv = (divisor & (divisor - 1)) == 0 ? 1.0f / d : 0.0f;  // 0: divide
  (void)hipGetLastError();
#define GB_CALL(K)                                                                                \
  if (op == GB_OP_AVG) reduce_op_kernel<K, GB_OP_AVG><<<grid, kThreads, 0, stream>>>(dst, srcs, n, d, inv);      \
  else if (op == GB_OP_MAX) reduce_op_kernel<K, GB_OP_MAX><<<grid, kThreads, 0, stream>>>(dst, srcs, n, d, inv); \
  else if (op == GB_OP_MIN) reduce_op_kernel<K, GB_OP_MIN><<<grid, kThreads, 0, stream>>>(dst, srcs, n, d, inv); \
  else reduce_sum_kernel<K, false><<<grid, kThreads, 0, stream>>>(dst, srcs, n);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

namespace {
// K and op dispatch for one element type; integer types have no AVG.
template <int DT>
hipError_t launch_typed(void* dst, const PtrTable& srcs, int k, size_t nbytes, int op, const Divisor& dv, int pow2,
                        hipStream_t stream) {
  const size_t grid = ceil_div(nbytes, (size_t)kThreads * 16);
  if (grid == 0 || grid > kMaxGrid) return hipErrorInvalidValue;
  constexpr bool kFloat = DT == GB_DTYPE_F16 || DT == GB_DTYPE_BF16 || DT == GB_DTYPE_F64;
  if (!kFloat && op == GB_OP_AVG) return hipErrorInvalidValue;
#define GB_LAUNCH(K, OP) reduce_typed_kernel<DT, K, OP><<<grid, kThreads, 0, stream>>>(dst, srcs, nbytes, dv, pow2)
#define GB_CALL(K)                                  \
  if (op == GB_OP_SUM) GB_LAUNCH(K, GB_OP_SUM);     \
  else if (op == GB_OP_MAX) GB_LAUNCH(K, GB_OP_MAX); \
  else if (op == GB_OP_MIN) GB_LAUNCH(K, GB_OP_MIN); \
  else if constexpr (kFloat) GB_LAUNCH(K, GB_OP_AVG);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
#undef GB_LAUNCH
  return hipGetLastError();
}
}  // namespace

hipError_t launch_reduce_typed(void* dst, const PtrTable& srcs, int k, size_t n, int dtype, int op, int divisor,
                               hipStream_t stream) {
  static const size_t elem_bytes[] = {4, 2, 2, 8, 1, 1, 4, 8};
  if (dtype <= GB_DTYPE_F32 || dtype > GB_DTYPE_I64 || divisor < 1) return hipErrorInvalidValue;
  const size_t nbytes = n * elem_bytes[dtype];
  const int pow2 = (divisor & (divisor - 1)) == 0;
  const Divisor dv = {(float)divisor, 1.0f / (float)divisor, (double)divisor, 1.0 / (double)divisor};
  (void)hipGetLastError();
  switch (dtype) {
    case GB_DTYPE_F16: return launch_typed<GB_DTYPE_F16>(dst, srcs, k, nbytes, op, dv, pow2, stream);
    case GB_DTYPE_BF16: return launch_typed<GB_DTYPE_BF16>(dst, srcs, k, nbytes, op, dv, pow2, stream);
    case GB_DTYPE_F64: return launch_typed<GB_DTYPE_F64>(dst, srcs, k, nbytes, op, dv, pow2, stream);
    case GB_DTYPE_I8: return launch_typed<GB_DTYPE_I8>(dst, srcs, k, nbytes, op, dv, pow2, stream);
    case GB_DTYPE_U8: return launch_typed<GB_DTYPE_U8>(dst, srcs, k, nbytes, op, dv, pow2, stream);
    case GB_DTYPE_I32: return launch_typed<GB_DTYPE_I32>(dst, srcs, k, nbytes, op, dv, pow2, stream);
    default: return launch_typed<GB_DTYPE_I64>(dst, srcs, k, nbytes, op, dv, pow2, stream);
  }
}

namespace {
// One launcher body per element type ET; the exported launchers switch on
// the type.  Accumulation into the output is offered for float32 only.
template <int ET>
hipError_t encode_bf16_t(uint16_t* codes, const void* src, size_t n, hipStream_t stream) {
  const size_t grid = grid_for(n, 4);
  if (grid == 0) return hipErrorInvalidValue;
  encode_bf16_kernel<ET><<<grid, kThreads, 0, stream>>>(codes, src, n);
  return hipGetLastError();
}

template <int ET>
hipError_t encode_fp8_t(uint8_t* codes, float* scales, const void* src, size_t n, int scale_mode,
                        hipStream_t stream) {
  const size_t grid = grid_for(n, 16);  // 16 values per lane: a 256-lane group does 16 blocks
  if (grid == 0) return hipErrorInvalidValue;
  encode_fp8_kernel<ET><<<grid, kThreads, 0, stream>>>(codes, scales, src, n, scale_mode);
  return hipGetLastError();
}

template <int ET>
hipError_t decode_bf16_t(void* acc, const PtrTable& codes, int k, size_t n, bool accumulate, hipStream_t stream) {
  const size_t grid = grid_for(n, 4);
  if (grid == 0) return hipErrorInvalidValue;
  if (accumulate && ET != GB_DTYPE_F32) return hipErrorInvalidValue;
#define GB_CALL(K)                                                                                      \
  if constexpr (ET == GB_DTYPE_F32) {                                                                   \
    if (accumulate) decode_bf16_kernel<K, true, ET><<<grid, kThreads, 0, stream>>>(acc, codes, n);        \
    else decode_bf16_kernel<K, false, ET><<<grid, kThreads, 0, stream>>>(acc, codes, n);                  \
  } else {                                                                                              \
    decode_bf16_kernel<K, false, ET><<<grid, kThreads, 0, stream>>>(acc, codes, n);                       \
  }
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

template <int ET>
hipError_t decode_fp8_t(void* acc, const PtrTable& codes, const PtrTable& scales, int k, size_t n,
                        bool accumulate, hipStream_t stream) {
  const size_t grid = grid_for(n, 16);
  if (grid == 0) return hipErrorInvalidValue;
  if (accumulate && ET != GB_DTYPE_F32) return hipErrorInvalidValue;
#define GB_CALL(K)                                                                                               \
  if constexpr (ET == GB_DTYPE_F32) {                                                                            \
    if (accumulate) decode_fp8_kernel<K, true, ET><<<grid, kThreads, heavy_lds(K), stream>>>(acc, codes, scales, n); \
    else decode_fp8_kernel<K, false, ET><<<grid, kThreads, heavy_lds(K), stream>>>(acc, codes, scales, n);          \
  } else {                                                                                                       \
    decode_fp8_kernel<K, false, ET><<<grid, kThreads, heavy_lds(K), stream>>>(acc, codes, scales, n);             \
  }
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

template <int ET>
hipError_t fused_bf16_t(void* out, const PtrTable& srcs, const OutTable& c, int k, size_t n, hipStream_t stream) {
  const size_t grid = grid_for(n, 4);
  if (grid == 0) return hipErrorInvalidValue;
#define GB_CALL(K) fused_bf16_kernel<K, ET><<<grid, kThreads, 0, stream>>>(out, srcs, c, n);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

template <int ET>
hipError_t fused_fp8_t(void* out, const PtrTable& srcs, const OutTable& c, const OutTable& s, int k, size_t n,
                       int scale_mode, hipStream_t stream) {
  const size_t grid = grid_for(n, 16);
  if (grid == 0) return hipErrorInvalidValue;
#define GB_CALL(K) fused_fp8_kernel<K, ET><<<grid, kThreads, heavy_lds(K), stream>>>(out, srcs, c, s, n, scale_mode);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

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

hipError_t launch_encode_bf16(uint16_t* codes, const void* src, size_t n, int dtype, hipStream_t stream) {
#define GB_CALL(ET) encode_bf16_t<ET>(codes, src, n, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

hipError_t launch_encode_fp8(uint8_t* codes, float* scales, const void* src, size_t n, int scale_mode, int dtype,
                             hipStream_t stream) {
#define GB_CALL(ET) encode_fp8_t<ET>(codes, scales, src, n, scale_mode, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

hipError_t launch_decode_bf16(void* acc, const PtrTable& codes, int k, size_t n, bool accumulate, int dtype,
                              hipStream_t stream) {
#define GB_CALL(ET) decode_bf16_t<ET>(acc, codes, k, n, accumulate, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

hipError_t launch_decode_fp8(void* acc, const PtrTable& codes, const PtrTable& scales, int k, size_t n,
                             bool accumulate, int dtype, hipStream_t stream) {
#define GB_CALL(ET) decode_fp8_t<ET>(acc, codes, scales, k, n, accumulate, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

hipError_t launch_fused_bf16(void* out, const PtrTable& srcs, uint16_t* const* codes, int k, size_t n, int dtype,
                             hipStream_t stream) {
  OutTable c = {};
  for (int r = 0; r < k; r++) c.p[r] = codes[r];
#define GB_CALL(ET) fused_bf16_t<ET>(out, srcs, c, k, n, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

hipError_t launch_fused_fp8(void* out, const PtrTable& srcs, uint8_t* const* codes, float* const* scales, int k,
                            size_t n, int scale_mode, int dtype, hipStream_t stream) {
  OutTable c = {}, s = {};
  for (int r = 0; r < k; r++) {
    c.p[r] = codes[r];
    s.p[r] = scales[r];
  }
#define GB_CALL(ET) fused_fp8_t<ET>(out, srcs, c, s, k, n, scale_mode, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

hipError_t launch_encode_bf16_ef(uint16_t* codes, float* residual, const float* src, size_t n,
                                 hipStream_t stream) {
  const size_t grid = grid_for(n, 4);
  if (grid == 0) return hipErrorInvalidValue;
  (void)hipGetLastError();
  encode_bf16_ef_kernel<<<grid, kThreads, 0, stream>>>(codes, residual, src, n);
  return hipGetLastError();
}

hipError_t launch_encode_fp8_ef(uint8_t* codes, float* scales, float* residual, const float* src, size_t n,
                                int scale_mode, hipStream_t stream) {
  const size_t grid = grid_for(n, 16);
  if (grid == 0) return hipErrorInvalidValue;
  (void)hipGetLastError();
  encode_fp8_ef_kernel<<<grid, kThreads, 0, stream>>>(codes, scales, residual, src, n, scale_mode);
  return hipGetLastError();
}

hipError_t launch_fused_bf16_ef(float* out, const PtrTable& srcs, float* const* residuals,
                                uint16_t* const* codes, int k, size_t n, hipStream_t stream) {
  OutTable c = {}, rs = {};
  for (int r = 0; r < k; r++) {
    c.p[r] = codes[r];
    rs.p[r] = residuals[r];
  }
  const size_t grid = grid_for(n, 4);
  if (grid == 0) return hipErrorInvalidValue;
  (void)hipGetLastError();
#define GB_CALL(K) fused_bf16_ef_kernel<K><<<grid, kThreads, 0, stream>>>(out, srcs, rs, c, n);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

hipError_t launch_fused_fp8_ef(float* out, const PtrTable& srcs, float* const* residuals, uint8_t* const* codes,
                               float* const* scales, int k, size_t n, int scale_mode, hipStream_t stream) {
  OutTable c = {}, s = {}, rs = {};
  for (int r = 0; r < k; r++) {
    c.p[r] = codes[r];
    s.p[r] = scales[r];
    rs.p[r] = residuals[r];
  }
  const size_t grid = grid_for(n, 16);
  if (grid == 0) return hipErrorInvalidValue;
  (void)hipGetLastError();
#define GB_CALL(K) fused_fp8_ef_kernel<K><<<grid, kThreads, heavy_lds(K), stream>>>(out, srcs, rs, c, s, n, scale_mode);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

}  // namespace gb
