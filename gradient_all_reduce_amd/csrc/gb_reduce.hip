// gb_reduce.hip — the fixed-order sum and the other reductions (AVG, MAX,
// MIN; every element type) of libgbreduce.
#include "gb_device.h"

namespace gb {
namespace {

// ===========================================================================
// Fixed-order sum: dst = [dst +] src0 + src1 + ... + src(K-1), one 4-value
// vector per lane.
// ===========================================================================
template <int K, bool ACC, bool FULL>
__device__ __forceinline__ void reduce_sum_body(float* dst, const PtrTable& src, size_t n) {
  const size_t i = (group_index<ReduceOrder>() * kThreads + threadIdx.x) * 4;
  if (!FULL && i >= n) return;
  f4 x[K];
  f4 a;
#pragma unroll
  for (int r = 0; r < K; r++) x[r] = load4_at<FULL>(static_cast<const float*>(src.p[r]), i, n);
  if (ACC) a = load4_at<FULL>(dst, i, n);
  f4 s = ACC ? a + x[0] : x[0];
#pragma unroll
  for (int r = 1; r < K; r++) s = s + x[r];
  if (K > 1 || ACC) s = canon4(s);  // one source alone is a copy
  store4_at<FULL>(dst, i, n, s);
}

template <int K, bool ACC>
__global__ __launch_bounds__(kThreads) void reduce_sum_kernel(float* dst, PtrTable src, size_t n) {
  if (group_full<ReduceOrder>(kVecPerGroup, n)) reduce_sum_body<K, ACC, true>(dst, src, n);
  else reduce_sum_body<K, ACC, false>(dst, src, n);
}

// The same sum of 4 sources over a large buffer, shaped wider: 4 vectors per
// lane, 1024 values apart, so a workgroup takes 4096 values of each source
// (every load and store instruction of the workgroup still one contiguous
// 4 KiB run), in WideSumOrder, launched one workgroup per compute unit.
// Every lane loads all 16 of its vectors before it stores, so dst may be
// src[0].  Measured on MI355X against reduce_sum_kernel<4> in one process,
// with the same sums: +7% at 2^28 and 2^30 values per rank (6.48-6.49 TB/s
// against 6.04-6.05); at 2^26 the narrow kernel was ahead (6.55 against
// 6.40), so the wide one starts at 2^28.
constexpr size_t kWideSumVecs = 4;
constexpr size_t kWideSumMin = (size_t)1 << 28;

template <bool FULL>
__device__ __forceinline__ void reduce_sum4_wide_body(float* dst, const PtrTable& src, size_t n, size_t g) {
  const size_t base = g * kVecPerGroup * kWideSumVecs + (size_t)threadIdx.x * 4;
  f4 x[4][kWideSumVecs];
#pragma unroll
  for (int r = 0; r < 4; r++) {
#pragma unroll
    for (size_t u = 0; u < kWideSumVecs; u++) {
      x[r][u] = load4_at<FULL>(static_cast<const float*>(src.p[r]), base + u * kVecPerGroup, n);
    }
  }
#pragma unroll
  for (size_t u = 0; u < kWideSumVecs; u++) {
    const f4 s = canon4(((x[0][u] + x[1][u]) + x[2][u]) + x[3][u]);
    store4_at<FULL>(dst, base + u * kVecPerGroup, n, s);
  }
}

__global__ __launch_bounds__(kThreads) void reduce_sum4_wide_kernel(float* dst, PtrTable src, size_t n) {
  const size_t g = group_index<WideSumOrder>();
  if ((g + 1) * kVecPerGroup * kWideSumVecs <= n) reduce_sum4_wide_body<true>(dst, src, n, g);
  else reduce_sum4_wide_body<false>(dst, src, n, g);
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
  const size_t i = (group_index<ReduceOrder>() * kThreads + threadIdx.x) * 4;
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
  if (OP == GB_OP_AVG || K > 1) s = canon4(s);
  store4_at<FULL>(dst, i, n, s);
}

template <int K, int OP>
__global__ __launch_bounds__(kThreads) void reduce_op_kernel(float* dst, PtrTable src, size_t n, float d, float inv) {
  const bool full = group_full<ReduceOrder>(kVecPerGroup, n);
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
  // With a power-of-two d the product is exact unless it is a binary32
  // subnormal, so only those lanes need the residual; the block is skipped
  // when no lane of the wavefront does.
  if (!P2 || __builtin_fabsf(q) < 0x1p-126f) {
    const float r = __builtin_fmaf(q, d, -a);
    uint32_t b = fbits(q);
    if ((r < 0.0f || r > 0.0f) && !(b & 1u)) {
      const bool grow = (r > 0.0f) == (a < 0.0f);  // |q| below |a / d|
      b = grow ? b + 1u : b - 1u;
    }
    return bitsf(b);
  }
  return q;
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
  const size_t byte = (group_index<ReduceOrder>() * kThreads + threadIdx.x) * 16;
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
  const bool full = group_full<ReduceOrder>((size_t)kThreads * 16, nbytes);
  if (OP == GB_OP_AVG && pow2) {
    if (full) reduce_typed_body<DT, K, OP, true, true>(dst, src, nbytes, dv);
    else reduce_typed_body<DT, K, OP, false, true>(dst, src, nbytes, dv);
  } else {
    if (full) reduce_typed_body<DT, K, OP, true, false>(dst, src, nbytes, dv);
    else reduce_typed_body<DT, K, OP, false, false>(dst, src, nbytes, dv);
  }
}

}  // namespace

hipError_t launch_reduce_sum(float* dst, const PtrTable& srcs, int k, size_t n, bool accumulate,
                             hipStream_t stream) {
  const size_t grid = grid_for(n, 4);
  if (grid == 0) return hipErrorInvalidValue;
  (void)hipGetLastError();
  if (k == 4 && !accumulate && n >= kWideSumMin) {
    const size_t wide = grid_for(n, 4 * kWideSumVecs);
    if (wide == 0) return hipErrorInvalidValue;
    reduce_sum4_wide_kernel<<<wide, kThreads, kOnePerCuLds, stream>>>(dst, srcs, n);
    return hipGetLastError();
  }
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

}  // namespace gb
