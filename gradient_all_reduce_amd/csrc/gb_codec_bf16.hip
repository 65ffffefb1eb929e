// gb_codec_bf16.hip — the bf16 bridge codec of libgbreduce: encode,
// decode-and-accumulate and the fused bucket pass, over every codec element type.
#include "gb_device.h"

namespace gb {
namespace {

// ===========================================================================
// bf16 encode and decode-accumulate: one 4-value vector per lane, so each
// instruction of a wavefront loads 1 KiB of fp32 and stores 512 bytes of
// codes (or the reverse), contiguously.
// ===========================================================================
// V 4-value vectors per lane, 1024 values apart, so each load or store
// instruction of the workgroup stays contiguous.  Two vectors per lane move
// 3-7% more bytes per second than one from 2^23 values up (fewer, fuller
// workgroups for the same bytes in flight); below that one vector is faster.
template <int ET, int V, bool FULL>
__device__ __forceinline__ void encode_bf16_body(uint16_t* codes, const void* src, size_t n) {
  const size_t sg0 = group_index<VecOrder>() * V;  // the workgroup's first 1024-value vector group
  const uint32_t t = threadIdx.x;
  f4 x[V];
#pragma unroll
  for (int v = 0; v < V; v++) {
    if (FULL || group_first<ET>(sg0 + v, t) < n) x[v] = load_group_vec<ET, FULL>(src, sg0 + v, t, n);
  }
#pragma unroll
  for (int v = 0; v < V; v++) {
    if (FULL || group_first<ET>(sg0 + v, t) < n) store_group_bf16<ET, FULL>(codes, sg0 + v, t, n, bf16_pack4(x[v]));
  }
}

template <int ET, int V>
__global__ __launch_bounds__(kThreads) void encode_bf16_kernel(uint16_t* codes, const void* src, size_t n) {
  if (group_full<VecOrder>(kVecPerGroup * V, n)) encode_bf16_body<ET, V, true>(codes, src, n);
  else encode_bf16_body<ET, V, false>(codes, src, n);
}

// Island sum then bf16 encode in one pass: the rank-order float32 sum of K
// sources, encoded as above and stored too when SUM (all sources are loaded
// before anything is stored, so the sum may overwrite the first source).
template <int K, bool SUM, bool FULL>
__device__ __forceinline__ void reduce_encode_bf16_body(float* sum, uint16_t* codes, const PtrTable& src,
                                                        size_t n) {
  const size_t i = (group_index<VecOrder>() * kThreads + threadIdx.x) * 4;
  if (!FULL && i >= n) return;
  f4 x[K];
#pragma unroll
  for (int r = 0; r < K; r++) x[r] = load4_at<FULL>(static_cast<const float*>(src.p[r]), i, n);
  f4 a = x[0];
#pragma unroll
  for (int r = 1; r < K; r++) a = a + x[r];
  if (K > 1) a = canon4(a);
  store_bf16_4_at<FULL>(codes, i, n, bf16_pack4(a));
  if (SUM) store4_at<FULL>(sum, i, n, a);
}

template <int K, bool SUM>
__global__ __launch_bounds__(kThreads) void reduce_encode_bf16_kernel(float* sum, uint16_t* codes, PtrTable src,
                                                                       size_t n) {
  if (group_full<VecOrder>(kVecPerGroup, n)) reduce_encode_bf16_body<K, SUM, true>(sum, codes, src, n);
  else reduce_encode_bf16_body<K, SUM, false>(sum, codes, src, n);
}

template <int K, bool ACC, int ET, bool FULL>
__device__ __forceinline__ void decode_bf16_body(void* acc, const PtrTable& codes, size_t n, size_t sg) {
  const uint32_t t = threadIdx.x;
  if (!FULL && group_first<ET>(sg, t) >= n) return;
  u2 w[K];
#pragma unroll
  for (int r = 0; r < K; r++) w[r] = load_group_bf16<ET, FULL>(static_cast<const uint16_t*>(codes.p[r]), sg, t, n);
  f4 a;
  if (ACC) a = load_group_vec<ET, FULL>(acc, sg, t, n);
#pragma unroll
  for (int r = 0; r < K; r++) {
    const f4 v = bf16_unpack4(w[r]);
    a = (!ACC && r == 0) ? v : a + v;
  }
  // one payload alone into float32 is an exact widening; a total of another
  // type is rounded from the canonical NaN, so no NaN payload is narrowed
  if (K > 1 || ACC || ET != GB_DTYPE_F32) a = canon4(a);
  store_group_vec<ET, FULL>(acc, sg, t, n, a);
}

template <int K, bool ACC, int ET>
__global__ __launch_bounds__(kThreads) void decode_bf16_kernel(void* acc, PtrTable codes, size_t n) {
  const size_t sg = ET == GB_DTYPE_F32 ? group_index<DecodeBf16Order>() : group_index<VecOrder>();
  if ((sg + 1) * kVecPerGroup <= n) decode_bf16_body<K, ACC, ET, true>(acc, codes, n, sg);
  else decode_bf16_body<K, ACC, ET, false>(acc, codes, n, sg);
}

// ===========================================================================
// Fused bf16 bucket pass, one 4-value vector per lane.
// ===========================================================================
// The same pass over 4 ranks of float16 or bfloat16 gradients with 8
// consecutive values per lane (one 16-byte load of each rank): workgroup w
// takes values [512 w, 512 w + 512).  Every result is per value, so the
// bits are those of every other lane map.
template <int ET, bool FULL>
__device__ __forceinline__ void fused_bf16_eight_body(void* out, const PtrTable& src, const OutTable& codes,
                                                      size_t n, size_t e) {
  constexpr int K = 4;
  f4 x[K][2];
#pragma unroll
  for (int r = 0; r < K; r++) {
    if (FULL) {
      load8_half<ET>(src.p[r], e, x[r][0], x[r][1]);
    } else {
      x[r][0] = load_vals4_at<ET, false>(src.p[r], e, n);
      x[r][1] = load_vals4_at<ET, false>(src.p[r], e + 4, n);
    }
  }
  f4 a[2];
#pragma unroll
  for (int r = 0; r < K; r++) {
    const u2 w0 = bf16_pack4(x[r][0]), w1 = bf16_pack4(x[r][1]);
    uint16_t* c = static_cast<uint16_t*>(codes.p[r]);
    if (FULL) {
      __builtin_nontemporal_store(u4w{w0.x, w0.y, w1.x, w1.y}, reinterpret_cast<u4w*>(c + e));
    } else {
      store_bf16_4_at<false>(c, e, n, w0);
      store_bf16_4_at<false>(c, e + 4, n, w1);
    }
    const f4 v0 = bf16_unpack4(w0), v1 = bf16_unpack4(w1);
    a[0] = r == 0 ? v0 : a[0] + v0;
    a[1] = r == 0 ? v1 : a[1] + v1;
  }
  if (FULL) {
    store8_half<ET>(out, e, canon4(a[0]), canon4(a[1]));
  } else {
    store_vals4_at<ET, false>(out, e, n, canon4(a[0]));
    store_vals4_at<ET, false>(out, e + 4, n, canon4(a[1]));
  }
}

template <int ET>
__global__ __launch_bounds__(64) void fused_bf16_eight_kernel(void* out, PtrTable src, OutTable codes, size_t n) {
  const size_t e = ((size_t)blockIdx.x * 64 + threadIdx.x) * 8;
  if (((size_t)blockIdx.x + 1) * 512 <= n) fused_bf16_eight_body<ET, true>(out, src, codes, n, e);
  else if (e < n) fused_bf16_eight_body<ET, false>(out, src, codes, n, e);
}

// The batch in the same shape: bucket b takes workgroups [first[b],
// first[b + 1]), two per 1024-value vector group; lanes past the bucket's
// end do nothing.
template <int ET>
__global__ __launch_bounds__(64) void fused_bf16_eight_batch_kernel(BucketBatch t) {
  constexpr int K = 4;
  const size_t w = blockIdx.x;
  uint32_t b = 0;
  for (uint32_t i = 1; i < t.count; i++) b += w >= t.first[i] ? 1u : 0u;
  const size_t wl = w - t.first[b], n = t.n[b], e = (wl * 64 + threadIdx.x) * 8;
  if (e >= n) return;
  PtrTable src;
  OutTable codes;
#pragma unroll
  for (int r = 0; r < K; r++) {
    src.p[r] = t.src[b][r];
    codes.p[r] = t.codes[b][r];
  }
  if ((wl + 1) * 512 <= n) fused_bf16_eight_body<ET, true>(t.out[b], src, codes, n, e);
  else fused_bf16_eight_body<ET, false>(t.out[b], src, codes, n, e);
}
// Lane t of vector group sg (t in [0, 256)).
template <int K, int ET, bool FULL, int DIV = 0>
__device__ __forceinline__ void fused_bf16_body(void* out, const PtrTable& src, const OutTable& codes, size_t n,
                                                size_t sg, uint32_t t, float d = 1.0f, float inv = 0.0f) {
  if (!FULL && group_first<ET>(sg, t) >= n) return;
  f4 x[K];
#pragma unroll
  for (int r = 0; r < K; r++) x[r] = load_group_vec<ET, FULL>(src.p[r], sg, t, n);
  f4 a;
#pragma unroll
  for (int r = 0; r < K; r++) {
    const u2 w = bf16_pack4(x[r]);
    store_group_bf16<ET, FULL>(static_cast<uint16_t*>(codes.p[r]), sg, t, n, w);
    const f4 v = bf16_unpack4(w);
    a = r == 0 ? v : a + v;
  }
  f4 q[1] = {a};
  avg_total<DIV>(q, d, inv);
  if (K > 1 || DIV != 0 || ET != GB_DTYPE_F32) q[0] = canon4(q[0]);
  store_group_vec<ET, FULL>(out, sg, t, n, q[0]);
}

template <int K, int ET>
__global__ __launch_bounds__(kThreads) void fused_bf16_kernel(void* out, PtrTable src, OutTable codes, size_t n) {
  // float32 gradients in the permuted order; the others move more bytes
  // per second in index order (1-7%, up to 21% with error feedback over
  // bfloat16), measured on three machines
  const size_t sg = ET == GB_DTYPE_F32 ? group_index<FusedVecOrder>() : (size_t)blockIdx.x;
  if ((sg + 1) * kVecPerGroup <= n) fused_bf16_body<K, ET, true>(out, src, codes, n, sg, threadIdx.x);
  else fused_bf16_body<K, ET, false>(out, src, codes, n, sg, threadIdx.x);
}

// The same pass in 64-lane workgroups of 256 values (wave_lane), taken in
// index order: float32 gradients from 3 ranks (fused_bf16_wave), float16
// and bfloat16 ones from 5 ranks and 2^22 values or 4 ranks and 2^29
// (fused_bf16_half_wave).  A
// buffer's last vector group may leave up to 3 workgroups with no values;
// they return.
template <int K, int ET>
__global__ __launch_bounds__(kWaveThreads) void fused_bf16_wave_kernel(void* out, PtrTable src, OutTable codes,
                                                                       size_t n) {
  static_assert(ET == GB_DTYPE_F32 || ET == GB_DTYPE_F16 || ET == GB_DTYPE_BF16, "4-byte or 2-byte gradients");
  const size_t w = blockIdx.x;
  const WaveLane l = wave_lane(w);
  if ((w + 1) * (kVecPerGroup / 4) <= n) fused_bf16_body<K, ET, true>(out, src, codes, n, l.sg, l.t);
  else fused_bf16_body<K, ET, false>(out, src, codes, n, l.sg, l.t);
}

// Several buckets in one launch (gradients of element type ET), as the fp8
// batch: each workgroup finds its bucket, then takes that bucket's vector
// group.
template <int K, int ET, int DIV>
__global__ __launch_bounds__(kThreads) void fused_bf16_batch_kernel(BucketBatch t, float d, float inv) {
  const size_t w = blockIdx.x;
  uint32_t b = 0;
  for (uint32_t i = 1; i < t.count; i++) b += w >= t.first[i] ? 1u : 0u;
  PtrTable src;
  OutTable codes;
#pragma unroll
  for (int r = 0; r < K; r++) {
    src.p[r] = t.src[b][r];
    codes.p[r] = t.codes[b][r];
  }
  // a large bucket of float32 gradients takes the permuted order of a
  // whole-buffer launch, as there
  const size_t wl = w - t.first[b], n = t.n[b];
  const size_t sg = ET == GB_DTYPE_F32 ? group_index_in<FusedVecOrder>(wl, t.first[b + 1] - t.first[b]) : wl;
  if ((sg + 1) * kVecPerGroup <= n) fused_bf16_body<K, ET, true, DIV>(t.out[b], src, codes, n, sg, threadIdx.x, d, inv);
  else fused_bf16_body<K, ET, false, DIV>(t.out[b], src, codes, n, sg, threadIdx.x, d, inv);
}

// The batch over float32 gradients in 64-lane workgroups (fused_bf16_wave):
// bucket b takes workgroups [first[b], first[b + 1]), four per vector group.
template <int K, int DIV>
__global__ __launch_bounds__(kWaveThreads) void fused_bf16_wave_batch_kernel(BucketBatch t, float d, float inv) {
  const size_t w = blockIdx.x;
  uint32_t b = 0;
  for (uint32_t i = 1; i < t.count; i++) b += w >= t.first[i] ? 1u : 0u;
  PtrTable src;
  OutTable codes;
#pragma unroll
  for (int r = 0; r < K; r++) {
    src.p[r] = t.src[b][r];
    codes.p[r] = t.codes[b][r];
  }
  const size_t wl = w - t.first[b], n = t.n[b];
  const WaveLane l = wave_lane(wl);
  if ((wl + 1) * (kVecPerGroup / 4) <= n) {
    fused_bf16_body<K, GB_DTYPE_F32, true, DIV>(t.out[b], src, codes, n, l.sg, l.t, d, inv);
  } else {
    fused_bf16_body<K, GB_DTYPE_F32, false, DIV>(t.out[b], src, codes, n, l.sg, l.t, d, inv);
  }
}

// Launcher bodies, one per element type ET.
template <int ET>
hipError_t encode_bf16_t(uint16_t* codes, const void* src, size_t n, hipStream_t stream) {
  if (n >= ((size_t)1 << 23)) {
    const size_t grid = grid_for(n, 8);
    if (grid == 0) return hipErrorInvalidValue;
    encode_bf16_kernel<ET, 2><<<grid, kThreads, 0, stream>>>(codes, src, n);
  } else {
    const size_t grid = grid_for(n, 4);
    if (grid == 0) return hipErrorInvalidValue;
    encode_bf16_kernel<ET, 1><<<grid, kThreads, 0, stream>>>(codes, src, n);
  }
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
hipError_t fused_bf16_t(void* out, const PtrTable& srcs, const OutTable& c, int k, size_t n, hipStream_t stream) {
  if constexpr (ET == GB_DTYPE_F16 || ET == GB_DTYPE_BF16) {
    // one workgroup per 512 values; beyond the largest grid the kernels below run
    const size_t eight_grid = ceil_div(n, 512);
    if (fused_bf16_eight(k, n) && eight_grid <= kMaxGrid) {
      fused_bf16_eight_kernel<ET><<<eight_grid, 64, kBf16EightLds, stream>>>(out, srcs, c, n);
      return hipGetLastError();
    }
  }
  if constexpr (ET == GB_DTYPE_F32 || ET == GB_DTYPE_F16 || ET == GB_DTYPE_BF16) {
    const size_t wave_grid = wave_grid_for(n);
    const bool wave = ET == GB_DTYPE_F32 ? fused_bf16_wave(k) : fused_bf16_half_wave(k, n);
    if (wave && wave_grid != 0) {
      const unsigned lds = ET == GB_DTYPE_F32 ? fused_bf16_wave_lds(k, n) : fused_bf16_half_wave_lds(k);
#define GB_CALL(K) fused_bf16_wave_kernel<K, ET><<<wave_grid, kWaveThreads, lds, stream>>>(out, srcs, c, n);
      GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
      return hipGetLastError();
    }
  }
  const size_t grid = grid_for(n, 4);
  if (grid == 0) return hipErrorInvalidValue;
#define GB_CALL(K) fused_bf16_kernel<K, ET><<<grid, kThreads, fused_bf16_lds<ET>(K, n), stream>>>(out, srcs, c, n);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

}  // namespace

hipError_t launch_encode_bf16(uint16_t* codes, const void* src, size_t n, int dtype, hipStream_t stream) {
#define GB_CALL(ET) encode_bf16_t<ET>(codes, src, n, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

hipError_t launch_decode_bf16(void* acc, const PtrTable& codes, int k, size_t n, bool accumulate, int dtype,
                              hipStream_t stream) {
#define GB_CALL(ET) decode_bf16_t<ET>(acc, codes, k, n, accumulate, stream)
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

namespace {
// A batched launch takes the fused pass's cap for its largest bucket.
template <int ET, int DIV>
hipError_t fused_bf16_batch_t(BucketBatch& t, size_t grid, int k, float d, float inv, hipStream_t stream) {
  size_t largest = 0;
  for (uint32_t b = 0; b < t.count; b++) largest = t.n[b] > largest ? t.n[b] : largest;
  if constexpr (ET == GB_DTYPE_F16 || ET == GB_DTYPE_BF16) {
    // two 64-lane workgroups of 8 values per lane per vector group, as the
    // whole-buffer launch takes its largest bucket: 16-bucket batches of
    // 6,553,600-value buckets over 4 ranks moved 2.1-2.6% (bfloat16) and
    // 0.3-0.6% (float16) more bytes per second than the 256-lane batch
    // kernel, in the benchmark on one machine, same bits
    if (fused_bf16_eight(k, largest) && grid <= kMaxGrid / 2) {
      for (int b = 0; b <= kBatchBuckets; b++) t.first[b] *= 2;
      fused_bf16_eight_batch_kernel<ET><<<2 * grid, 64, kBf16EightLds, stream>>>(t);
      return hipGetLastError();
    }
  }
  if constexpr (ET == GB_DTYPE_F32) {
    // four 64-lane workgroups per vector group, uncapped: 16-bucket batches
    // of whole 25 MiB buckets and of 819,200-value ones over 4 ranks moved
    // 3% and 1% more bytes per second than the 256-lane batch kernel, and
    // lost 1-17% under any cap (the whole-buffer kernel's included)
    if (fused_bf16_wave(k) && grid <= kMaxGrid / 4) {
      for (int b = 0; b <= kBatchBuckets; b++) t.first[b] *= 4;
#define GB_CALL(K) fused_bf16_wave_batch_kernel<K, DIV><<<4 * grid, kWaveThreads, 0, stream>>>(t, d, inv);
      GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
      return hipGetLastError();
    }
  }
#define GB_CALL(K) fused_bf16_batch_kernel<K, ET, DIV><<<grid, kThreads, fused_bf16_lds<ET>(K, largest), stream>>>(t, d, inv);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fused_bf16_batch(BucketBatch& t, int k, int dtype, int divisor, hipStream_t stream) {
  if (t.count == 0 || t.count > (uint32_t)kBatchBuckets) return hipErrorInvalidValue;
  size_t grid = 0;
  for (uint32_t b = 0; b < t.count; b++) {
    t.first[b] = grid;
    grid += batch_groups(GB_CODEC_BF16, t.n[b]);
  }
  for (int b = (int)t.count; b <= kBatchBuckets; b++) t.first[b] = grid;
  if (grid == 0 || grid > kMaxGrid) return hipErrorInvalidValue;
  if (divisor != 1) {  // float32 totals only
    if (dtype != GB_DTYPE_F32) return hipErrorInvalidValue;
    (void)hipGetLastError();
    const float d = (float)divisor, inv = (divisor & (divisor - 1)) == 0 ? 1.0f / d : 0.0f;
    return inv != 0.0f ? fused_bf16_batch_t<GB_DTYPE_F32, 1>(t, grid, k, d, inv, stream)
                       : fused_bf16_batch_t<GB_DTYPE_F32, 2>(t, grid, k, d, inv, stream);
  }
#define GB_CALL(ET) fused_bf16_batch_t<ET, 0>(t, grid, k, 1.0f, 0.0f, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

hipError_t launch_reduce_encode_bf16(float* sum, uint16_t* codes, const PtrTable& srcs, int k, size_t n,
                                    hipStream_t stream) {
  const size_t grid = grid_for(n, 4);
  if (grid == 0) return hipErrorInvalidValue;
  (void)hipGetLastError();
#define GB_CALL(K)                                                                                     \
  if (sum != nullptr) reduce_encode_bf16_kernel<K, true><<<grid, kThreads, 0, stream>>>(sum, codes, srcs, n); \
  else reduce_encode_bf16_kernel<K, false><<<grid, kThreads, 0, stream>>>(sum, codes, srcs, n);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

}  // namespace gb
