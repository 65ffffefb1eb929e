// gb_ef.hip — the error-feedback encoders and bucket passes of libgbreduce.
#include "gb_device.h"

namespace gb {
namespace {

// ===========================================================================
// Error feedback (README "Bridge compression": each bridge member keeps a
// residual per buffer).  y = x + residual is encoded exactly as above, and
// the residual becomes y minus the value the payload decodes to (rounded
// binary32 subtraction; exact for bf16).  The residual is binary32 whatever
// the gradient's element type ET: x is converted to binary32 as the codecs
// convert it, and the decoded total is rounded once to ET.  The residual is
// read and written in place by the lane that owns the value, through the
// gradient's lane map.
// ===========================================================================
template <int ET, bool FULL>
__device__ __forceinline__ void encode_bf16_ef_body(uint16_t* codes, float* res, const void* src, size_t n) {
  const size_t sg = group_index<VecOrder>();
  const uint32_t t = threadIdx.x;
  if (!FULL && group_first<ET>(sg, t) >= n) return;
  const f4 y = canon4(load_group_vec<ET, FULL>(src, sg, t, n) + load_group_f32<ET, FULL>(res, sg, t, n));
  const u2 w = bf16_pack4(y);
  store_group_bf16<ET, FULL>(codes, sg, t, n, w);
  store_group_f32<ET, FULL>(res, sg, t, n, canon4(y - bf16_unpack4(w)));
}

template <int ET>
__global__ __launch_bounds__(kThreads) void encode_bf16_ef_kernel(uint16_t* codes, float* res, const void* src,
                                                                   size_t n) {
  if (group_full<VecOrder>(kVecPerGroup, n)) encode_bf16_ef_body<ET, true>(codes, res, src, n);
  else encode_bf16_ef_body<ET, false>(codes, res, src, n);
}

template <int ET, bool FULL>
__device__ __forceinline__ void encode_fp8_ef_body(uint8_t* codes, float* scales, float* res, const void* src,
                                                   size_t n, int mode) {
  const uint32_t col = threadIdx.x & 15u;
  const size_t block = group_index<BlockOrder>() * kBlocksPerGroup + (threadIdx.x >> 4);
  constexpr int MAP = ef_map<ET>();
  f4 x[4], r[4];
  load_block<ET, MAP, FULL>(src, block, col, n, x);
  load_block_f32<MAP, FULL>(res, block, col, n, r);
#pragma unroll
  for (int j = 0; j < 4; j++) x[j] = canon4(x[j] + r[j]);  // y
  uint32_t w[4];
  const float s = encode_block16(x, mode, w);  // all 64 lanes take part
  if (!FULL && block * kBlock >= n) return;
  if (col == 0u) scales[block] = s;
#pragma unroll
  for (int j = 0; j < 4; j++) r[j] = canon4(x[j] - e4m3_unpack4(w[j]) * s);
  store_block_codes<MAP, FULL>(codes, block, col, n, w);
  store_block_f32<MAP, FULL>(res, block, col, n, r);
}

template <int ET>
__global__ __launch_bounds__(kThreads) void encode_fp8_ef_kernel(uint8_t* codes, float* scales, float* res,
                                                                  const void* src, size_t n, int mode) {
  if (group_full<BlockOrder>(kBlocksPerGroup * kBlock, n)) encode_fp8_ef_body<ET, true>(codes, scales, res, src, n, mode);
  else encode_fp8_ef_body<ET, false>(codes, scales, res, src, n, mode);
}

template <int K, int ET, bool FULL, int DIV = 0>
__device__ __forceinline__ void fused_fp8_ef_body(void* out, const PtrTable& src, const OutTable& resid,
                                                  const OutTable& codes, const OutTable& scales, size_t n,
                                                  int mode, size_t g, float dv = 1.0f, float inv = 0.0f) {
  const uint32_t col = threadIdx.x & 15u;
  const size_t block = g * kBlocksPerGroup + (threadIdx.x >> 4);
  constexpr int MAP = ef_map<ET>();
  f4 y[K][4];
#pragma unroll
  for (int r = 0; r < K; r++) {
    f4 q[4];
    load_block<ET, MAP, FULL>(src.p[r], block, col, n, y[r]);
    load_block_f32<MAP, FULL>(static_cast<const float*>(resid.p[r]), block, col, n, q);
#pragma unroll
    for (int j = 0; j < 4; j++) y[r][j] = canon4(y[r][j] + q[j]);
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
    f4 d[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const f4 v = e4m3_unpack4(w[j]) * s;
      d[j] = canon4(y[r][j] - v);
      a[j] = r == 0 ? v : a[j] + v;
    }
    if (live) {
      store_block_codes<MAP, FULL>(c, block, col, n, w);
      store_block_f32<MAP, FULL>(rp, block, col, n, d);
    }
  }
  if (!live) return;
  avg_total<DIV>(a, dv, inv);
#pragma unroll
  for (int j = 0; j < 4; j++) a[j] = canon4(a[j]);
  store_block<ET, MAP, FULL>(out, block, col, n, a);
}

template <int K, int ET>
__global__ __launch_bounds__(kThreads) void fused_fp8_ef_kernel(void* out, PtrTable src, OutTable resid,
                                                                 OutTable codes, OutTable scales, size_t n,
                                                                 int mode) {
  const size_t g = group_index<BlockOrder>();
  if ((g + 1) * kBlocksPerGroup * kBlock <= n) fused_fp8_ef_body<K, ET, true>(out, src, resid, codes, scales, n, mode, g);
  else fused_fp8_ef_body<K, ET, false>(out, src, resid, codes, scales, n, mode, g);
}

template <int K, int ET, bool FULL, int DIV = 0>
__device__ __forceinline__ void fused_bf16_ef_body(void* out, const PtrTable& src, const OutTable& resid,
                                                   const OutTable& codes, size_t n, size_t sg, uint32_t t,
                                                   float dv = 1.0f, float inv = 0.0f) {
  if (!FULL && group_first<ET>(sg, t) >= n) return;
  f4 y[K];
#pragma unroll
  for (int r = 0; r < K; r++) {
    y[r] = canon4(load_group_vec<ET, FULL>(src.p[r], sg, t, n) +
                  load_group_f32<ET, FULL>(static_cast<const float*>(resid.p[r]), sg, t, n));
  }
  f4 a;
#pragma unroll
  for (int r = 0; r < K; r++) {
    const u2 w = bf16_pack4(y[r]);
    const f4 v = bf16_unpack4(w);
    store_group_bf16<ET, FULL>(static_cast<uint16_t*>(codes.p[r]), sg, t, n, w);
    store_group_f32<ET, FULL>(static_cast<float*>(resid.p[r]), sg, t, n, canon4(y[r] - v));
    a = r == 0 ? v : a + v;
  }
  f4 q[1] = {a};
  avg_total<DIV>(q, dv, inv);
  if (K > 1 || DIV != 0 || ET != GB_DTYPE_F32) q[0] = canon4(q[0]);
  store_group_vec<ET, FULL>(out, sg, t, n, q[0]);
}

template <int K, int ET>
__global__ __launch_bounds__(kThreads) void fused_bf16_ef_kernel(void* out, PtrTable src, OutTable resid,
                                                                  OutTable codes, size_t n) {
  // float32 gradients (here only beyond the largest 64-lane grid) in the
  // permuted order; the others (here below the 64-lane thresholds or beyond
  // the largest 64-lane grid) move more bytes per second in index order
  // (1-7%, up to 21% with error feedback over bfloat16), measured on three
  // machines
  const size_t sg = ET == GB_DTYPE_F32 ? group_index<FusedVecOrder>() : (size_t)blockIdx.x;
  if ((sg + 1) * kVecPerGroup <= n) fused_bf16_ef_body<K, ET, true>(out, src, resid, codes, n, sg, threadIdx.x);
  else fused_bf16_ef_body<K, ET, false>(out, src, resid, codes, n, sg, threadIdx.x);
}

// The same pass in 64-lane workgroups of 256 values (wave_lane), taken in
// index order, where fused_bf16_ef_wave says.  A float64 lane holds values
// 2t, 2t + 1, 2t + 512 and 2t + 513 of its vector group, so its workgroup
// lies below n only when the whole group does.
template <int K, int ET>
__global__ __launch_bounds__(kWaveThreads) void fused_bf16_ef_wave_kernel(void* out, PtrTable src, OutTable resid,
                                                                          OutTable codes, size_t n) {
  const size_t w = blockIdx.x;
  const WaveLane l = wave_lane(w);
  const bool full = ET == GB_DTYPE_F64 ? (l.sg + 1) * kVecPerGroup <= n : (w + 1) * (kVecPerGroup / 4) <= n;
  if (full) {
    fused_bf16_ef_body<K, ET, true>(out, src, resid, codes, n, l.sg, l.t);
  } else {
    fused_bf16_ef_body<K, ET, false>(out, src, resid, codes, n, l.sg, l.t);
  }
}

// The pass over float32, float16 or bfloat16 gradients of 4 ranks with one
// block per wavefront: workgroup b is block b, lane l its values 4l to
// 4l + 3 of every source and residual.  The block maximum and so every bit
// are those of the 16-lane map.
template <int ET, bool FULL, int DIV = 0>
__device__ __forceinline__ void fused_fp8_ef_wave_body(void* out, const PtrTable& src, const OutTable& resid,
                                                       const OutTable& codes, const OutTable& scales, size_t n,
                                                       int mode, size_t block, float dv = 1.0f, float inv = 0.0f) {
  constexpr int K = 4;
  const size_t e = block * kBlock + 4 * (size_t)threadIdx.x;
  f4 y[K];
#pragma unroll
  for (int r = 0; r < K; r++) {
    y[r] = canon4(load_vals4_at<ET, FULL>(src.p[r], e, n) +
                  load4_at<FULL>(static_cast<const float*>(resid.p[r]), e, n));
  }
  f4 a[1];
#pragma unroll
  for (int r = 0; r < K; r++) {
    uint32_t w;
    const float s = encode_block4(y[r], mode, w);  // all 64 lanes take part
    if (threadIdx.x == 0u) static_cast<float*>(scales.p[r])[block] = s;
    const f4 v = e4m3_unpack4(w) * s;
    a[0] = r == 0 ? v : a[0] + v;
    store_codes4_at<FULL>(static_cast<uint8_t*>(codes.p[r]), e, n, w);
    store4_at<FULL>(static_cast<float*>(resid.p[r]), e, n, canon4(y[r] - v));
  }
  avg_total<DIV>(a, dv, inv);
  store_vals4_at<ET, FULL>(out, e, n, canon4(a[0]));
}

template <int ET>
__global__ __launch_bounds__(64) void fused_fp8_ef_wave_kernel(void* out, PtrTable src, OutTable resid,
                                                               OutTable codes, OutTable scales, size_t n, int mode) {
  const size_t block = blockIdx.x;  // the grid has one workgroup per block, so block * kBlock < n
  if ((block + 1) * kBlock <= n) fused_fp8_ef_wave_body<ET, true>(out, src, resid, codes, scales, n, mode, block);
  else fused_fp8_ef_wave_body<ET, false>(out, src, resid, codes, scales, n, mode, block);
}

// The batch in the same shape: bucket b takes workgroups [first[b],
// first[b + 1]), 16 per 4096-value group, and those past the bucket's last
// block return at once (uniformly per workgroup).
template <int ET, int DIV>
__global__ __launch_bounds__(64) void fused_fp8_ef_wave_batch_kernel(BucketBatchEf t, int mode, float dv, float inv) {
  constexpr int K = 4;
  const size_t w = blockIdx.x;
  uint32_t b = 0;
  for (uint32_t i = 1; i < t.count; i++) b += w >= t.first[i] ? 1u : 0u;
  const size_t block = w - t.first[b], n = t.n[b];
  if (block * kBlock >= n) return;
  PtrTable src;
  OutTable resid, codes, scales;
#pragma unroll
  for (int r = 0; r < K; r++) {
    src.p[r] = t.src[b][r];
    resid.p[r] = t.resid[b][r];
    codes.p[r] = t.codes[b][r];
    scales.p[r] = t.scales[b][r];
  }
  void* out = t.out[b];
  if ((block + 1) * kBlock <= n) fused_fp8_ef_wave_body<ET, true, DIV>(out, src, resid, codes, scales, n, mode, block, dv, inv);
  else fused_fp8_ef_wave_body<ET, false, DIV>(out, src, resid, codes, scales, n, mode, block, dv, inv);
}

// Several buckets in one launch, with their residuals: each workgroup finds
// its bucket from the table of first workgroups and takes that bucket's
// group: in index order within a bucket, or in the whole-buffer launch's
// order for a bucket large enough.
template <int K, int ET, int DIV>
__global__ __launch_bounds__(kThreads) void fused_fp8_ef_batch_kernel(BucketBatchEf t, int mode, float dv, float inv) {
  const size_t w = blockIdx.x;
  uint32_t b = 0;
  for (uint32_t i = 1; i < t.count; i++) b += w >= t.first[i] ? 1u : 0u;
  PtrTable src;
  OutTable resid, codes, scales;
#pragma unroll
  for (int r = 0; r < K; r++) {
    src.p[r] = t.src[b][r];
    resid.p[r] = t.resid[b][r];
    codes.p[r] = t.codes[b][r];
    scales.p[r] = t.scales[b][r];
  }
  // a bucket large enough takes the permuted order of a whole-buffer launch
  const size_t g = group_index_in<BlockOrder>(w - t.first[b], t.first[b + 1] - t.first[b]), n = t.n[b];
  if ((g + 1) * kBlocksPerGroup * kBlock <= n)
    fused_fp8_ef_body<K, ET, true, DIV>(t.out[b], src, resid, codes, scales, n, mode, g, dv, inv);
  else fused_fp8_ef_body<K, ET, false, DIV>(t.out[b], src, resid, codes, scales, n, mode, g, dv, inv);
}

template <int K, int ET, int DIV>
__global__ __launch_bounds__(kThreads) void fused_bf16_ef_batch_kernel(BucketBatchEf t, float dv, float inv) {
  const size_t w = blockIdx.x;
  uint32_t b = 0;
  for (uint32_t i = 1; i < t.count; i++) b += w >= t.first[i] ? 1u : 0u;
  PtrTable src;
  OutTable resid, codes;
#pragma unroll
  for (int r = 0; r < K; r++) {
    src.p[r] = t.src[b][r];
    resid.p[r] = t.resid[b][r];
    codes.p[r] = t.codes[b][r];
  }
  const size_t wl = w - t.first[b], n = t.n[b];
  const size_t sg = ET == GB_DTYPE_F32 ? group_index_in<FusedVecOrder>(wl, t.first[b + 1] - t.first[b]) : wl;
  if ((sg + 1) * kVecPerGroup <= n) {
    fused_bf16_ef_body<K, ET, true, DIV>(t.out[b], src, resid, codes, n, sg, threadIdx.x, dv, inv);
  } else {
    fused_bf16_ef_body<K, ET, false, DIV>(t.out[b], src, resid, codes, n, sg, threadIdx.x, dv, inv);
  }
}

// The batch in 64-lane workgroups: bucket b takes workgroups
// [first[b], first[b + 1]), four per vector group; a float64 workgroup is
// whole only with its vector group, as in the whole-buffer kernel.
template <int K, int ET, int DIV>
__global__ __launch_bounds__(kWaveThreads) void fused_bf16_ef_wave_batch_kernel(BucketBatchEf t, float dv, float inv) {
  const size_t w = blockIdx.x;
  uint32_t b = 0;
  for (uint32_t i = 1; i < t.count; i++) b += w >= t.first[i] ? 1u : 0u;
  PtrTable src;
  OutTable resid, codes;
#pragma unroll
  for (int r = 0; r < K; r++) {
    src.p[r] = t.src[b][r];
    resid.p[r] = t.resid[b][r];
    codes.p[r] = t.codes[b][r];
  }
  const size_t wl = w - t.first[b], n = t.n[b];
  const WaveLane l = wave_lane(wl);
  const bool full = ET == GB_DTYPE_F64 ? (l.sg + 1) * kVecPerGroup <= n : (wl + 1) * (kVecPerGroup / 4) <= n;
  if (full) {
    fused_bf16_ef_body<K, ET, true, DIV>(t.out[b], src, resid, codes, n, l.sg, l.t, dv, inv);
  } else {
    fused_bf16_ef_body<K, ET, false, DIV>(t.out[b], src, resid, codes, n, l.sg, l.t, dv, inv);
  }
}

// The table's first workgroups and the grid; 0 if the table is empty or too large.
size_t batch_grid(BucketBatchEf& t, int codec) {
  if (t.count == 0 || t.count > (uint32_t)kBatchBucketsEf) return 0;
  size_t grid = 0;
  for (uint32_t b = 0; b < t.count; b++) {
    t.first[b] = grid;
    grid += batch_groups(codec, t.n[b]);
  }
  for (int b = (int)t.count; b <= kBatchBucketsEf; b++) t.first[b] = grid;
  return grid > kMaxGrid ? 0 : grid;
}

// A batched launch takes each pass's cap for its largest bucket.
template <int ET, int DIV>
hipError_t fused_fp8_ef_batch_t(BucketBatchEf& t, int k, int scale_mode, float dv, float inv, hipStream_t stream) {
  const size_t grid = batch_grid(t, GB_CODEC_FP8_E4M3_B256);
  if (grid == 0) return hipErrorInvalidValue;
  size_t largest = 0;
  for (uint32_t b = 0; b < t.count; b++) largest = t.n[b] > largest ? t.n[b] : largest;
  if constexpr (ET != GB_DTYPE_F64) {
    // sixteen 64-lane workgroups per group, as the whole-buffer launch takes
    // its largest bucket
    if (fused_fp8_ef_wave<ET>(k, largest) && grid <= kMaxGrid / 16) {
      for (int b = 0; b <= kBatchBucketsEf; b++) t.first[b] *= 16;
      fused_fp8_ef_wave_batch_kernel<ET, DIV><<<16 * grid, 64, fused_fp8_ef_wave_lds<ET>(), stream>>>(t, scale_mode, dv,
                                                                                                       inv);
      return hipGetLastError();
    }
  }
#define GB_CALL(K) \
  fused_fp8_ef_batch_kernel<K, ET, DIV><<<grid, kThreads, fused_fp8_ef_lds(K, largest), stream>>>(t, scale_mode, dv, inv);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

template <int ET, int DIV>
hipError_t fused_bf16_ef_batch_t(BucketBatchEf& t, int k, float dv, float inv, hipStream_t stream) {
  const size_t grid = batch_grid(t, GB_CODEC_BF16);
  if (grid == 0) return hipErrorInvalidValue;
  size_t largest = 0;
  for (uint32_t b = 0; b < t.count; b++) largest = t.n[b] > largest ? t.n[b] : largest;
  // four 64-lane workgroups per vector group, at the whole-buffer kernel's
  // rule and cap for the largest bucket: 8-bucket batches over 4 ranks
  // (whole 25 MiB buckets of float32 gradients, 6,553,600-value buckets of
  // the other types, and buckets of 819,200 values) moved more bytes per
  // second than the 256-lane batch kernel at its cap: float32 +19-21%,
  // bfloat16 +27-32%, float64 +13-15%, float16 level (+0.6-0.9%)
  if (fused_bf16_ef_wave<ET>(k, largest) && grid <= kMaxGrid / 4) {
    for (int b = 0; b <= kBatchBucketsEf; b++) t.first[b] *= 4;
#define GB_CALL(K)                                                                                               \
  fused_bf16_ef_wave_batch_kernel<K, ET, DIV><<<4 * grid, kWaveThreads, fused_bf16_ef_wave_lds<ET>(K), stream>>>(t, dv, \
                                                                                                              inv);
    GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
    return hipGetLastError();
  }
#define GB_CALL(K) \
  fused_bf16_ef_batch_kernel<K, ET, DIV><<<grid, kThreads, fused_bf16_ef_lds<ET>(K), stream>>>(t, dv, inv);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

template <int ET>
hipError_t encode_bf16_ef_t(uint16_t* codes, float* residual, const void* src, size_t n, hipStream_t stream) {
  const size_t grid = grid_for(n, 4);
  if (grid == 0) return hipErrorInvalidValue;
  encode_bf16_ef_kernel<ET><<<grid, kThreads, 0, stream>>>(codes, residual, src, n);
  return hipGetLastError();
}

template <int ET>
hipError_t encode_fp8_ef_t(uint8_t* codes, float* scales, float* residual, const void* src, size_t n,
                           int scale_mode, hipStream_t stream) {
  const size_t grid = grid_for(n, 16);
  if (grid == 0) return hipErrorInvalidValue;
  encode_fp8_ef_kernel<ET><<<grid, kThreads, 0, stream>>>(codes, scales, residual, src, n, scale_mode);
  return hipGetLastError();
}

template <int ET>
hipError_t fused_bf16_ef_t(void* out, const PtrTable& srcs, const OutTable& rs, const OutTable& c, int k, size_t n,
                           hipStream_t stream) {
  const size_t wave_grid = wave_grid_for(n);
  if (fused_bf16_ef_wave<ET>(k, n) && wave_grid != 0) {
#define GB_CALL(K)                                                                                       \
  fused_bf16_ef_wave_kernel<K, ET><<<wave_grid, kWaveThreads, fused_bf16_ef_wave_lds<ET>(K), stream>>>(out, srcs, rs, \
                                                                                                      c, n);
    GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
    return hipGetLastError();
  }
  const size_t grid = grid_for(n, 4);
  if (grid == 0) return hipErrorInvalidValue;
#define GB_CALL(K) \
  fused_bf16_ef_kernel<K, ET><<<grid, kThreads, fused_bf16_ef_lds<ET>(K), stream>>>(out, srcs, rs, c, n);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

template <int ET>
hipError_t fused_fp8_ef_t(void* out, const PtrTable& srcs, const OutTable& rs, const OutTable& c, const OutTable& s,
                          int k, size_t n, int scale_mode, hipStream_t stream) {
  if constexpr (ET != GB_DTYPE_F64) {
    // one workgroup per block; beyond the largest grid the 256-lane kernel runs
    const size_t wave_grid = ceil_div(n, kBlock);
    if (fused_fp8_ef_wave<ET>(k, n) && wave_grid <= kMaxGrid) {
      fused_fp8_ef_wave_kernel<ET><<<wave_grid, 64, fused_fp8_ef_wave_lds<ET>(), stream>>>(out, srcs, rs, c, s, n,
                                                                                          scale_mode);
      return hipGetLastError();
    }
  }
  const size_t grid = grid_for(n, 16);
  if (grid == 0) return hipErrorInvalidValue;
#define GB_CALL(K) fused_fp8_ef_kernel<K, ET><<<grid, kThreads, fused_fp8_ef_lds(K, n), stream>>>(out, srcs, rs, c, s, n, scale_mode);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

}  // namespace

hipError_t launch_encode_bf16_ef(uint16_t* codes, float* residual, const void* src, size_t n, int dtype,
                                 hipStream_t stream) {
#define GB_CALL(ET) encode_bf16_ef_t<ET>(codes, residual, src, n, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

hipError_t launch_encode_fp8_ef(uint8_t* codes, float* scales, float* residual, const void* src, size_t n,
                                int scale_mode, int dtype, hipStream_t stream) {
#define GB_CALL(ET) encode_fp8_ef_t<ET>(codes, scales, residual, src, n, scale_mode, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

hipError_t launch_fused_bf16_ef(void* out, const PtrTable& srcs, float* const* residuals, uint16_t* const* codes,
                                int k, size_t n, int dtype, hipStream_t stream) {
  OutTable c = {}, rs = {};
  for (int r = 0; r < k; r++) {
    c.p[r] = codes[r];
    rs.p[r] = residuals[r];
  }
#define GB_CALL(ET) fused_bf16_ef_t<ET>(out, srcs, rs, c, k, n, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

hipError_t launch_fused_fp8_ef_batch(BucketBatchEf& t, int k, int scale_mode, int dtype, int divisor,
                                     hipStream_t stream) {
  if (divisor != 1) {  // float32 totals only
    if (dtype != GB_DTYPE_F32) return hipErrorInvalidValue;
    (void)hipGetLastError();
    const float dv = (float)divisor, inv = (divisor & (divisor - 1)) == 0 ? 1.0f / dv : 0.0f;
    return inv != 0.0f ? fused_fp8_ef_batch_t<GB_DTYPE_F32, 1>(t, k, scale_mode, dv, inv, stream)
                       : fused_fp8_ef_batch_t<GB_DTYPE_F32, 2>(t, k, scale_mode, dv, inv, stream);
  }
#define GB_CALL(ET) fused_fp8_ef_batch_t<ET, 0>(t, k, scale_mode, 1.0f, 0.0f, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

hipError_t launch_fused_bf16_ef_batch(BucketBatchEf& t, int k, int dtype, int divisor, hipStream_t stream) {
  if (divisor != 1) {  // float32 totals only
    if (dtype != GB_DTYPE_F32) return hipErrorInvalidValue;
    (void)hipGetLastError();
    const float dv = (float)divisor, inv = (divisor & (divisor - 1)) == 0 ? 1.0f / dv : 0.0f;
    return inv != 0.0f ? fused_bf16_ef_batch_t<GB_DTYPE_F32, 1>(t, k, dv, inv, stream)
                       : fused_bf16_ef_batch_t<GB_DTYPE_F32, 2>(t, k, dv, inv, stream);
  }
#define GB_CALL(ET) fused_bf16_ef_batch_t<ET, 0>(t, k, 1.0f, 0.0f, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

hipError_t launch_fused_fp8_ef(void* out, const PtrTable& srcs, float* const* residuals, uint8_t* const* codes,
                               float* const* scales, int k, size_t n, int scale_mode, int dtype, hipStream_t stream) {
  OutTable c = {}, s = {}, rs = {};
  for (int r = 0; r < k; r++) {
    c.p[r] = codes[r];
    s.p[r] = scales[r];
    rs.p[r] = residuals[r];
  }
#define GB_CALL(ET) fused_fp8_ef_t<ET>(out, srcs, rs, c, s, k, n, scale_mode, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

}  // namespace gb
