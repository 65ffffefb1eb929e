// gb_kernels.hip — HIP kernels of libgbreduce for gfx950 (AMD Instinct
// MI355X, CDNA4).
//
// All of this work streams HBM: a few integer and float operations per 4-byte
// element, no reuse, no contraction (so no MFMA).  The kernels are shaped for
// that:
//   * every lane moves 16-byte vectors, and each load instruction of a 64-lane
//     wavefront covers whole 256-byte runs, so requests coalesce;
//   * a lane issues all of its loads (every rank, several vectors) before it
//     computes, keeping many bytes in flight per compute unit;
//   * the k contributions of an element are read once and combined in
//     registers (reduce, encode and decode-accumulate are fused where the
//     call allows it);
//   * the fp8 block maximum is reduced across the 16 lanes of one DPP row
//     (four row-local DPP steps, no LDS and no barrier): a 256-value block is
//     one row of 16 lanes holding 16 values each, so a wavefront works on 4
//     blocks and a 256-lane workgroup on 16.
//
// Arithmetic follows the gpubridge README, "How it works" (sum of island sums)
// and "Bridge compression" (bf16; OCP E4M3 with one scale per 256 values;
// decode and add in float32).  Every rounding is IEEE binary32
// round-to-nearest-even with subnormals kept, and nothing is contracted into
// a fused multiply-add (built with -ffp-contract=off), so results are
// independent of the launch shape.
#include <hip/hip_runtime.h>

#include "gb_internal.h"

namespace gb {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

struct OutTable {
  void* p[GB_MAX_K];
};

constexpr int kThreads = 256;  // 4 wavefronts of 64 lanes

__device__ __forceinline__ uint32_t fbits(float x) { return __float_as_uint(x); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __uint_as_float(u); }

__device__ __forceinline__ f4 load4(const float* p) {
  return *reinterpret_cast<const f4*>(p);
}
__device__ __forceinline__ void store4(float* p, f4 v) {
  *reinterpret_cast<f4*>(p) = v;
}

// Elements [i, min(i + 4, n)) of p, zero beyond n.  Requires i < n.
__device__ __forceinline__ f4 load4_tail(const float* p, size_t i, size_t n) {
  f4 v = {0.0f, 0.0f, 0.0f, 0.0f};
  v.x = p[i];
  if (i + 1 < n) v.y = p[i + 1];
  if (i + 2 < n) v.z = p[i + 2];
  if (i + 3 < n) v.w = p[i + 3];
  return v;
}
__device__ __forceinline__ f4 load4_any(const float* p, size_t i, size_t n) {
  if (i + 4 <= n) return load4(p + i);
  if (i < n) return load4_tail(p, i, n);
  return f4{0.0f, 0.0f, 0.0f, 0.0f};
}
__device__ __forceinline__ void store4_any(float* p, size_t i, size_t n, f4 v) {
  if (i + 4 <= n) {
    store4(p + i, v);
    return;
  }
  if (i < n) p[i] = v.x;
  if (i + 1 < n) p[i + 1] = v.y;
  if (i + 2 < n) p[i + 2] = v.z;
}

// ---------------------------------------------------------------------------
// bf16: nearest value, ties to the even code (carry into the exponent gives
// the IEEE overflow to Inf); NaN keeps sign and top payload, quiet bit set.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t bf16_code(float x) {
  const uint32_t u = fbits(x);
  const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? ((u >> 16) | 0x40u) : r;
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return bitsf(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return bitsf(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// fp8 (OCP E4M3, bias 7, largest finite 448 = 0x7E, S.1111.111 = NaN).
// ---------------------------------------------------------------------------
// |x| as an unsigned integer, NaN counted as 0: the integer maximum of these
// is the bit pattern of the largest non-NaN magnitude, in any order.
__device__ __forceinline__ uint32_t magnitude_bits(float x) {
  const uint32_t m = fbits(x) & 0x7FFFFFFFu;
  return m > 0x7F800000u ? 0u : m;
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
__device__ __forceinline__ float quotient(float x, double rinv) {
  return (float)((double)x * rinv);
}

// E4M3 code of v (already divided by the scale), the sign bit taken from x.
// |v| >= 2^-6: round the binary32 fraction to 3 bits (ties to even, the carry
// runs into the exponent), re-bias the exponent from 127 to 7 (120 << 3 =
// 960), saturate at 0x7E.  |v| < 2^-6: the subnormal code is rint(|v| * 2^9),
// the integer rounding done by adding 2^23.  NaN gives 0x7F.
__device__ __forceinline__ uint32_t e4m3_code(float v, float x) {
  const uint32_t m = fbits(v) & 0x7FFFFFFFu;
  uint32_t c;
  if (m >= 0x3C800000u) {
    const uint32_t r = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20;
    c = min(r - 960u, 0x7Eu);
  } else {
    const float t = bitsf(m) * 512.0f;
    c = fbits(t + 8388608.0f) - 0x4B000000u;
  }
  c = m > 0x7F800000u ? 0x7Fu : c;
  return c | ((fbits(x) >> 24) & 0x80u);
}

// Value of an E4M3 code: the 7 magnitude bits placed at binary32 bits 26..20
// read as a binary32 number and scaled by 2^120 (exact, subnormal codes
// included), NaN for 0x7F, sign from bit 7.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t m = c & 0x7Fu;
  float v = bitsf(m << 20) * 0x1p120f;
  v = m == 0x7Fu ? __builtin_nanf("") : v;
  return bitsf(fbits(v) | ((c & 0x80u) << 24));
}

__device__ __forceinline__ uint32_t byte_of(uint32_t w, int e) { return (w >> (8 * e)) & 0xFFu; }

// Elements of a 256-value block owned by a lane: 4 vectors, vector j at
// element offset (16 j + col) * 4 of the block, so every load or store
// instruction of a row covers 256 contiguous bytes of fp32 (64 of codes).
__device__ __forceinline__ size_t lane_elem(size_t block, int j, uint32_t col) {
  return block * kBlock + (size_t)(16 * j + col) * 4;
}

// Stores 4 codes of elements [i, i+4), clipped to n.
__device__ __forceinline__ void store_codes4(uint8_t* codes, size_t i, size_t n, uint32_t w) {
  if (i + 4 <= n) {
    *reinterpret_cast<uint32_t*>(codes + i) = w;
    return;
  }
  for (int e = 0; e < 3; e++) {
    if (i + e < n) codes[i + e] = (uint8_t)byte_of(w, e);
  }
}
__device__ __forceinline__ uint32_t load_codes4(const uint8_t* codes, size_t i, size_t n) {
  if (i + 4 <= n) return *reinterpret_cast<const uint32_t*>(codes + i);
  uint32_t w = 0;
  for (int e = 0; e < 3; e++) {
    if (i + e < n) w |= (uint32_t)codes[i + e] << (8 * e);
  }
  return w;
}

// ===========================================================================
// Fixed-order sum: dst = (ACC ? dst : 0-term-free) + src0 + src1 + ...
// Each lane owns U 4-element vectors, 256 vectors apart.
// ===========================================================================
template <int K, int U, bool ACC>
__global__ __launch_bounds__(kThreads) void reduce_sum_kernel(float* dst, PtrTable src, size_t n) {
  const size_t v0 = (size_t)blockIdx.x * (kThreads * U) + threadIdx.x;
  f4 x[U][K];
  f4 a[U];
  const bool full = (v0 + (size_t)(U - 1) * kThreads + 1) * 4 <= n;
  if (full) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const size_t i = (v0 + (size_t)u * kThreads) * 4;
#pragma unroll
      for (int r = 0; r < K; r++) x[u][r] = load4(static_cast<const float*>(src.p[r]) + i);
      if (ACC) a[u] = load4(dst + i);
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      f4 s = ACC ? a[u] + x[u][0] : x[u][0];
#pragma unroll
      for (int r = 1; r < K; r++) s = s + x[u][r];
      store4(dst + (v0 + (size_t)u * kThreads) * 4, s);
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < U; u++) {
    const size_t i = (v0 + (size_t)u * kThreads) * 4;
#pragma unroll
    for (int r = 0; r < K; r++) x[u][r] = load4_any(static_cast<const float*>(src.p[r]), i, n);
    if (ACC) a[u] = load4_any(dst, i, n);
  }
#pragma unroll
  for (int u = 0; u < U; u++) {
    f4 s = ACC ? a[u] + x[u][0] : x[u][0];
#pragma unroll
    for (int r = 1; r < K; r++) s = s + x[u][r];
    store4_any(dst, (v0 + (size_t)u * kThreads) * 4, n, s);
  }
}

// ===========================================================================
// bf16 encode: each lane owns U groups of 8 values (two 16-byte loads, one
// 16-byte store of codes), groups 256 apart.
// ===========================================================================
__device__ __forceinline__ u4 bf16_pack8(f4 lo, f4 hi) {
  u4 w;
  w.x = bf16_code(lo.x) | (bf16_code(lo.y) << 16);
  w.y = bf16_code(lo.z) | (bf16_code(lo.w) << 16);
  w.z = bf16_code(hi.x) | (bf16_code(hi.y) << 16);
  w.w = bf16_code(hi.z) | (bf16_code(hi.w) << 16);
  return w;
}

__device__ __forceinline__ void store_bf16_8(uint16_t* codes, size_t i, size_t n, u4 w) {
  if (i + 8 <= n) {
    *reinterpret_cast<u4*>(codes + i) = w;
    return;
  }
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  for (int e = 0; e < 8; e++) {
    if (i + e < n) codes[i + e] = (uint16_t)(ws[e >> 1] >> (16 * (e & 1)));
  }
}
__device__ __forceinline__ u4 load_bf16_8(const uint16_t* codes, size_t i, size_t n) {
  if (i + 8 <= n) return *reinterpret_cast<const u4*>(codes + i);
  uint32_t ws[4] = {0u, 0u, 0u, 0u};
  for (int e = 0; e < 8; e++) {
    if (i + e < n) ws[e >> 1] |= (uint32_t)codes[i + e] << (16 * (e & 1));
  }
  return u4{ws[0], ws[1], ws[2], ws[3]};
}

template <int U>
__global__ __launch_bounds__(kThreads) void encode_bf16_kernel(uint16_t* codes, const float* src, size_t n) {
  const size_t g0 = (size_t)blockIdx.x * (kThreads * U) + threadIdx.x;
  f4 lo[U], hi[U];
#pragma unroll
  for (int u = 0; u < U; u++) {
    const size_t i = (g0 + (size_t)u * kThreads) * 8;
    lo[u] = load4_any(src, i, n);
    hi[u] = load4_any(src, i + 4, n);
  }
#pragma unroll
  for (int u = 0; u < U; u++) {
    const size_t i = (g0 + (size_t)u * kThreads) * 8;
    if (i < n) store_bf16_8(codes, i, n, bf16_pack8(lo[u], hi[u]));
  }
}

// ===========================================================================
// bf16 decode-accumulate over K payloads, groups of 8 values per lane.
// ===========================================================================
template <int K, bool ACC>
__global__ __launch_bounds__(kThreads) void decode_bf16_kernel(float* acc, PtrTable codes, size_t n) {
  const size_t g = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t i = g * 8;
  if (i >= n) return;
  u4 w[K];
#pragma unroll
  for (int r = 0; r < K; r++) w[r] = load_bf16_8(static_cast<const uint16_t*>(codes.p[r]), i, n);
  f4 lo, hi;
  if (ACC) {
    lo = load4_any(acc, i, n);
    hi = load4_any(acc, i + 4, n);
  }
#pragma unroll
  for (int r = 0; r < K; r++) {
    const f4 vlo = {bf16_lo(w[r].x), bf16_hi(w[r].x), bf16_lo(w[r].y), bf16_hi(w[r].y)};
    const f4 vhi = {bf16_lo(w[r].z), bf16_hi(w[r].z), bf16_lo(w[r].w), bf16_hi(w[r].w)};
    if (!ACC && r == 0) {
      lo = vlo;
      hi = vhi;
    } else {
      lo = lo + vlo;
      hi = hi + vhi;
    }
  }
  store4_any(acc, i, n, lo);
  store4_any(acc, i + 4, n, hi);
}

// ===========================================================================
// fp8 encode: one DPP row per 256-value block, G groups of 4 blocks per
// wavefront, all loads issued first.
// ===========================================================================
template <int G>
__global__ __launch_bounds__(kThreads) void encode_fp8_kernel(uint8_t* codes, float* scales,
                                                               const float* src, size_t n,
                                                               int mode) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t col = lane & 15u;
  const uint32_t row = lane >> 4;
  const size_t wave = (size_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const size_t nblocks = (n + kBlock - 1) / kBlock;
  f4 x[G][4];
#pragma unroll
  for (int g = 0; g < G; g++) {
    const size_t block = (wave * G + g) * 4 + row;
#pragma unroll
    for (int j = 0; j < 4; j++) x[g][j] = load4_any(src, lane_elem(block, j, col), n);
  }
#pragma unroll
  for (int g = 0; g < G; g++) {
    const size_t block = (wave * G + g) * 4 + row;
    uint32_t am = 0u;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      am = max(am, magnitude_bits(x[g][j].x));
      am = max(am, magnitude_bits(x[g][j].y));
      am = max(am, magnitude_bits(x[g][j].z));
      am = max(am, magnitude_bits(x[g][j].w));
    }
    am = row_max16(am);
    const float s = block_scale(am, mode);
    const double rinv = scale_reciprocal(s);
    if (block < nblocks) {
      if (col == 0u) scales[block] = s;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const f4 v = x[g][j];
        const uint32_t w = e4m3_code(quotient(v.x, rinv), v.x) |
                           (e4m3_code(quotient(v.y, rinv), v.y) << 8) |
                           (e4m3_code(quotient(v.z, rinv), v.z) << 16) |
                           (e4m3_code(quotient(v.w, rinv), v.w) << 24);
        store_codes4(codes, lane_elem(block, j, col), n, w);
      }
    }
  }
}

// ===========================================================================
// fp8 decode-accumulate over K payloads: one DPP row per block, the scale of
// a rank's block read once per row.
// ===========================================================================
template <int K, bool ACC>
__global__ __launch_bounds__(kThreads) void decode_fp8_kernel(float* acc, PtrTable codes,
                                                               PtrTable scales, size_t n) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t col = lane & 15u;
  const uint32_t row = lane >> 4;
  const size_t block = ((size_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * 4 + row;
  const size_t nblocks = (n + kBlock - 1) / kBlock;
  if (block >= nblocks) return;
  uint32_t w[K][4];
  float s[K];
#pragma unroll
  for (int r = 0; r < K; r++) {
    const uint8_t* c = static_cast<const uint8_t*>(codes.p[r]);
#pragma unroll
    for (int j = 0; j < 4; j++) w[r][j] = load_codes4(c, lane_elem(block, j, col), n);
    s[r] = static_cast<const float*>(scales.p[r])[block];
  }
  f4 a[4];
  if (ACC) {
#pragma unroll
    for (int j = 0; j < 4; j++) a[j] = load4_any(acc, lane_elem(block, j, col), n);
  }
#pragma unroll
  for (int r = 0; r < K; r++) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const f4 v = {e4m3_value(byte_of(w[r][j], 0)) * s[r], e4m3_value(byte_of(w[r][j], 1)) * s[r],
                    e4m3_value(byte_of(w[r][j], 2)) * s[r], e4m3_value(byte_of(w[r][j], 3)) * s[r]};
      a[j] = (!ACC && r == 0) ? v : a[j] + v;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; j++) store4_any(acc, lane_elem(block, j, col), n, a[j]);
}

// ===========================================================================
// Fused fp8 bucket pass: read each rank's block once, write its payload
// (codes, scale), decode those codes and add them in rank order.
// ===========================================================================
template <int K>
__global__ __launch_bounds__(kThreads) void fused_fp8_kernel(float* out, PtrTable src, OutTable codes,
                                                              OutTable scales, size_t n, int mode) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t col = lane & 15u;
  const uint32_t row = lane >> 4;
  const size_t block = ((size_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * 4 + row;
  const size_t nblocks = (n + kBlock - 1) / kBlock;
  f4 x[K][4];
#pragma unroll
  for (int r = 0; r < K; r++) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      x[r][j] = load4_any(static_cast<const float*>(src.p[r]), lane_elem(block, j, col), n);
    }
  }
  f4 a[4];
#pragma unroll
  for (int r = 0; r < K; r++) {
    uint32_t am = 0u;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      am = max(am, magnitude_bits(x[r][j].x));
      am = max(am, magnitude_bits(x[r][j].y));
      am = max(am, magnitude_bits(x[r][j].z));
      am = max(am, magnitude_bits(x[r][j].w));
    }
    am = row_max16(am);
    const float s = block_scale(am, mode);
    const double rinv = scale_reciprocal(s);
    uint8_t* c = static_cast<uint8_t*>(codes.p[r]);
    if (block < nblocks && col == 0u) static_cast<float*>(scales.p[r])[block] = s;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const f4 xv = x[r][j];
      const uint32_t c0 = e4m3_code(quotient(xv.x, rinv), xv.x);
      const uint32_t c1 = e4m3_code(quotient(xv.y, rinv), xv.y);
      const uint32_t c2 = e4m3_code(quotient(xv.z, rinv), xv.z);
      const uint32_t c3 = e4m3_code(quotient(xv.w, rinv), xv.w);
      if (block < nblocks) store_codes4(c, lane_elem(block, j, col), n, c0 | (c1 << 8) | (c2 << 16) | (c3 << 24));
      const f4 v = {e4m3_value(c0) * s, e4m3_value(c1) * s, e4m3_value(c2) * s, e4m3_value(c3) * s};
      a[j] = r == 0 ? v : a[j] + v;
    }
  }
  if (block >= nblocks) return;
#pragma unroll
  for (int j = 0; j < 4; j++) store4_any(out, lane_elem(block, j, col), n, a[j]);
}

// ===========================================================================
// Fused bf16 bucket pass, groups of 8 values per lane.
// ===========================================================================
template <int K>
__global__ __launch_bounds__(kThreads) void fused_bf16_kernel(float* out, PtrTable src, OutTable codes,
                                                               size_t n) {
  const size_t g = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t i = g * 8;
  if (i >= n) return;
  f4 lo[K], hi[K];
#pragma unroll
  for (int r = 0; r < K; r++) {
    lo[r] = load4_any(static_cast<const float*>(src.p[r]), i, n);
    hi[r] = load4_any(static_cast<const float*>(src.p[r]), i + 4, n);
  }
  f4 alo, ahi;
#pragma unroll
  for (int r = 0; r < K; r++) {
    const u4 w = bf16_pack8(lo[r], hi[r]);
    store_bf16_8(static_cast<uint16_t*>(codes.p[r]), i, n, w);
    const f4 vlo = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
    const f4 vhi = {bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
    alo = r == 0 ? vlo : alo + vlo;
    ahi = r == 0 ? vhi : ahi + vhi;
  }
  store4_any(out, i, n, alo);
  store4_any(out, i + 4, n, ahi);
}

// ---------------------------------------------------------------------------
// Launch helpers.
// ---------------------------------------------------------------------------
constexpr size_t kMaxGrid = (size_t)1 << 31;

size_t ceil_div(size_t a, size_t b) { return (a + b - 1) / b; }

hipError_t finish_launch() { return hipGetLastError(); }

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
  // Vectors per lane: enough 16-byte loads in flight per lane without
  // running out of registers.
  const int u = k <= 2 ? 4 : (k <= 4 ? 2 : 1);
  const size_t grid = ceil_div(ceil_div(n, 4), (size_t)kThreads * u);
  if (grid >= kMaxGrid) return hipErrorInvalidValue;
  (void)hipGetLastError();
#define GB_CALL(K)                                                                                     \
  if (u == 4) {                                                                                        \
    if (accumulate) reduce_sum_kernel<K, 4, true><<<grid, kThreads, 0, stream>>>(dst, srcs, n);        \
    else reduce_sum_kernel<K, 4, false><<<grid, kThreads, 0, stream>>>(dst, srcs, n);                  \
  } else if (u == 2) {                                                                                 \
    if (accumulate) reduce_sum_kernel<K, 2, true><<<grid, kThreads, 0, stream>>>(dst, srcs, n);        \
    else reduce_sum_kernel<K, 2, false><<<grid, kThreads, 0, stream>>>(dst, srcs, n);                  \
  } else {                                                                                             \
    if (accumulate) reduce_sum_kernel<K, 1, true><<<grid, kThreads, 0, stream>>>(dst, srcs, n);        \
    else reduce_sum_kernel<K, 1, false><<<grid, kThreads, 0, stream>>>(dst, srcs, n);                  \
  }
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return finish_launch();
}

hipError_t launch_encode_bf16(uint16_t* codes, const float* src, size_t n, hipStream_t stream) {
  constexpr int U = 2;
  const size_t grid = ceil_div(ceil_div(n, 8), (size_t)kThreads * U);
  if (grid >= kMaxGrid) return hipErrorInvalidValue;
  (void)hipGetLastError();
  encode_bf16_kernel<U><<<grid, kThreads, 0, stream>>>(codes, src, n);
  return finish_launch();
}

hipError_t launch_encode_fp8(uint8_t* codes, float* scales, const float* src, size_t n, int scale_mode,
                             hipStream_t stream) {
  constexpr int G = 2;
  const size_t grid = ceil_div(ceil_div(n, kBlock), (size_t)16 * G);
  if (grid >= kMaxGrid) return hipErrorInvalidValue;
  (void)hipGetLastError();
  encode_fp8_kernel<G><<<grid, kThreads, 0, stream>>>(codes, scales, src, n, scale_mode);
  return finish_launch();
}

hipError_t launch_decode_bf16(float* acc, const PtrTable& codes, int k, size_t n, bool accumulate,
                              hipStream_t stream) {
  const size_t grid = ceil_div(ceil_div(n, 8), (size_t)kThreads);
  if (grid >= kMaxGrid) return hipErrorInvalidValue;
  (void)hipGetLastError();
#define GB_CALL(K)                                                                          \
  if (accumulate) decode_bf16_kernel<K, true><<<grid, kThreads, 0, stream>>>(acc, codes, n); \
  else decode_bf16_kernel<K, false><<<grid, kThreads, 0, stream>>>(acc, codes, n);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return finish_launch();
}

hipError_t launch_decode_fp8(float* acc, const PtrTable& codes, const PtrTable& scales, int k, size_t n,
                             bool accumulate, hipStream_t stream) {
  const size_t grid = ceil_div(ceil_div(n, kBlock), (size_t)16);
  if (grid >= kMaxGrid) return hipErrorInvalidValue;
  (void)hipGetLastError();
#define GB_CALL(K)                                                                                   \
  if (accumulate) decode_fp8_kernel<K, true><<<grid, kThreads, 0, stream>>>(acc, codes, scales, n);   \
  else decode_fp8_kernel<K, false><<<grid, kThreads, 0, stream>>>(acc, codes, scales, n);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return finish_launch();
}

hipError_t launch_fused_bf16(float* out, const PtrTable& srcs, uint16_t* const* codes, int k, size_t n,
                             hipStream_t stream) {
  OutTable c = {};
  for (int r = 0; r < k; r++) c.p[r] = codes[r];
  const size_t grid = ceil_div(ceil_div(n, 8), (size_t)kThreads);
  if (grid >= kMaxGrid) return hipErrorInvalidValue;
  (void)hipGetLastError();
#define GB_CALL(K) fused_bf16_kernel<K><<<grid, kThreads, 0, stream>>>(out, srcs, c, n);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return finish_launch();
}

hipError_t launch_fused_fp8(float* out, const PtrTable& srcs, uint8_t* const* codes, float* const* scales,
                            int k, size_t n, int scale_mode, hipStream_t stream) {
  OutTable c = {}, s = {};
  for (int r = 0; r < k; r++) {
    c.p[r] = codes[r];
    s.p[r] = scales[r];
  }
  const size_t grid = ceil_div(ceil_div(n, kBlock), (size_t)16);
  if (grid >= kMaxGrid) return hipErrorInvalidValue;
  (void)hipGetLastError();
#define GB_CALL(K) fused_fp8_kernel<K><<<grid, kThreads, 0, stream>>>(out, srcs, c, s, n, scale_mode);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return finish_launch();
}

}  // namespace gb
