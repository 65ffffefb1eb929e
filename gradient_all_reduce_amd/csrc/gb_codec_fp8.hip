// gb_codec_fp8.hip — the fp8 (OCP E4M3, one scale per 256 values) bridge
// codec of libgbreduce: encode, decode-and-accumulate and the fused bucket
// pass, over every codec element type.
#include "gb_device.h"

namespace gb {
namespace {

// ===========================================================================
// fp8 encode: one DPP row per 256-value block.
// ===========================================================================
template <int ET, bool FULL>
__device__ __forceinline__ void encode_fp8_body(uint8_t* codes, float* scales, const void* src, size_t n,
                                                int mode) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t col = lane & 15u;
  const size_t block = group_index<BlockOrder>() * kBlocksPerGroup + (threadIdx.x >> 4);
  constexpr int MAP = codec_map<ET>();
  f4 x[4];
  load_block<ET, MAP, FULL>(src, block, col, n, x);
  uint32_t w[4];
  const float s = encode_block16(x, mode, w);  // all 64 lanes take part
  if (!FULL && block * kBlock >= n) return;
  if (col == 0u) scales[block] = s;
  store_block_codes<MAP, FULL>(codes, block, col, n, w);
}

template <int ET>
__global__ __launch_bounds__(kThreads) void encode_fp8_kernel(uint8_t* codes, float* scales, const void* src,
                                                               size_t n, int mode) {
  if (group_full<BlockOrder>(kBlocksPerGroup * kBlock, n)) encode_fp8_body<ET, true>(codes, scales, src, n, mode);
  else encode_fp8_body<ET, false>(codes, scales, src, n, mode);
}

// ===========================================================================
// Island sum then fp8 encode in one pass: the rank-order float32 sum of K
// sources, encoded exactly as the encoder above encodes a float32 array, and
// stored too when SUM.  Every source is loaded before anything is stored, so
// the sum may overwrite the first source.
// ===========================================================================
template <int K, bool SUM, bool FULL>
__device__ __forceinline__ void reduce_encode_fp8_body(float* sum, uint8_t* codes, float* scales,
                                                       const PtrTable& src, size_t n, int mode) {
  const uint32_t col = threadIdx.x & 15u;
  const size_t block = group_index<BlockOrder>() * kBlocksPerGroup + (threadIdx.x >> 4);
  f4 x[K][4];
#pragma unroll
  for (int r = 0; r < K; r++) {
#pragma unroll
    for (int j = 0; j < 4; j++) x[r][j] = load4_at<FULL>(static_cast<const float*>(src.p[r]), lane_elem(block, j, col), n);
  }
  f4 a[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    a[j] = x[0][j];
#pragma unroll
    for (int r = 1; r < K; r++) a[j] = a[j] + x[r][j];
    if (K > 1) a[j] = canon4(a[j]);
  }
  uint32_t w[4];
  const float s = encode_block16(a, mode, w);  // all 64 lanes take part
  if (!FULL && block * kBlock >= n) return;
  if (col == 0u) scales[block] = s;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    store_codes4_at<FULL>(codes, lane_elem(block, j, col), n, w[j]);
    if (SUM) store4_at<FULL>(sum, lane_elem(block, j, col), n, a[j]);
  }
}

template <int K, bool SUM>
__global__ __launch_bounds__(kThreads) void reduce_encode_fp8_kernel(float* sum, uint8_t* codes, float* scales,
                                                                      PtrTable src, size_t n, int mode) {
  if (group_full<BlockOrder>(kBlocksPerGroup * kBlock, n)) reduce_encode_fp8_body<K, SUM, true>(sum, codes, scales, src, n, mode);
  else reduce_encode_fp8_body<K, SUM, false>(sum, codes, scales, src, n, mode);
}

// ===========================================================================
// fp8 decode-accumulate over K payloads: one DPP row per block, each rank's
// block scale read once per lane.
// ===========================================================================
template <int K, bool ACC, int ET, bool FULL>
__device__ __forceinline__ void decode_fp8_body(void* acc, const PtrTable& codes, const PtrTable& scales,
                                                size_t n) {
  const uint32_t col = threadIdx.x & 15u;
  const size_t block = group_index<BlockOrder>() * kBlocksPerGroup + (threadIdx.x >> 4);
  constexpr int MAP = codec_map<ET>();
  if (!FULL && block * kBlock >= n) return;
  uint32_t w[K][4];
  float s[K];
#pragma unroll
  for (int r = 0; r < K; r++) {
    load_block_codes<MAP, FULL>(static_cast<const uint8_t*>(codes.p[r]), block, col, n, w[r]);
    s[r] = static_cast<const float*>(scales.p[r])[block];
  }
  f4 a[4];
  if (ACC) load_block<ET, MAP, FULL>(acc, block, col, n, a);
#pragma unroll
  for (int r = 0; r < K; r++) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const f4 v = e4m3_unpack4(w[r][j]) * s[r];
      a[j] = (!ACC && r == 0) ? v : a[j] + v;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; j++) a[j] = canon4(a[j]);
  store_block<ET, MAP, FULL>(acc, block, col, n, a);
}

template <int K, bool ACC, int ET>
__global__ __launch_bounds__(kThreads) void decode_fp8_kernel(void* acc, PtrTable codes, PtrTable scales,
                                                               size_t n) {
  if (group_full<BlockOrder>(kBlocksPerGroup * kBlock, n)) decode_fp8_body<K, ACC, ET, true>(acc, codes, scales, n);
  else decode_fp8_body<K, ACC, ET, false>(acc, codes, scales, n);
}

// The decode of 4 payloads into a float32 total with one block per
// wavefront: workgroup b is block b, lane l its values 4l to 4l + 3; the
// scales are uniform across the workgroup.
template <bool ACC, bool FULL>
__device__ __forceinline__ void decode_fp8_wave_body(float* acc, const PtrTable& codes, const PtrTable& scales,
                                                     size_t n, size_t block) {
  constexpr int K = 4;
  const size_t e = block * kBlock + 4 * (size_t)threadIdx.x;
  uint32_t w[K];
  float s[K];
#pragma unroll
  for (int r = 0; r < K; r++) {
    w[r] = load_codes4_at<FULL>(static_cast<const uint8_t*>(codes.p[r]), e, n);
    s[r] = static_cast<const float*>(scales.p[r])[block];
  }
  f4 a;
  if (ACC) a = load4_at<FULL>(acc, e, n);
#pragma unroll
  for (int r = 0; r < K; r++) {
    const f4 v = e4m3_unpack4(w[r]) * s[r];
    a = (!ACC && r == 0) ? v : a + v;
  }
  store4_at<FULL>(acc, e, n, canon4(a));
}

template <bool ACC>
__global__ __launch_bounds__(64) void decode_fp8_wave_kernel(float* acc, PtrTable codes, PtrTable scales, size_t n) {
  const size_t block = blockIdx.x;  // the grid has one workgroup per block, so block * kBlock < n
  if ((block + 1) * kBlock <= n) decode_fp8_wave_body<ACC, true>(acc, codes, scales, n, block);
  else decode_fp8_wave_body<ACC, false>(acc, codes, scales, n, block);
}

// ===========================================================================
// Fused fp8 bucket pass: read each rank's block once, write its payload
// (codes, scale), decode those codes and add them in rank order.
// ===========================================================================
// T lanes per workgroup: group g is its T / 16 blocks.
template <int K, int ET, bool FULL, int DIV = 0, int T = kThreads>
__device__ __forceinline__ void fused_fp8_body(void* out, const PtrTable& src, const OutTable& codes,
                                               const OutTable& scales, size_t n, int mode, size_t g,
                                               float d = 1.0f, float inv = 0.0f) {
  const uint32_t col = threadIdx.x & 15u;
  const size_t block = g * (T / 16) + (threadIdx.x >> 4);
  constexpr int MAP = codec_map<ET>();
  f4 x[K][4];
#pragma unroll
  for (int r = 0; r < K; r++) load_block<ET, MAP, FULL>(src.p[r], block, col, n, x[r]);
  const bool live = FULL || block * kBlock < n;
  f4 a[4];
#pragma unroll
  for (int r = 0; r < K; r++) {
    uint32_t w[4];
    const float s = encode_block16(x[r], mode, w);  // all 64 lanes take part
    uint8_t* c = static_cast<uint8_t*>(codes.p[r]);
    if (live) {
      if (col == 0u) static_cast<float*>(scales.p[r])[block] = s;
      store_block_codes<MAP, FULL>(c, block, col, n, w);
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const f4 v = e4m3_unpack4(w[j]) * s;
      a[j] = r == 0 ? v : a[j] + v;
    }
  }
  if (!live) return;
  avg_total<DIV>(a, d, inv);
#pragma unroll
  for (int j = 0; j < 4; j++) a[j] = canon4(a[j]);
  store_block<ET, MAP, FULL>(out, block, col, n, a);
}

template <int K, int ET>
__global__ __launch_bounds__(kThreads) void fused_fp8_kernel(void* out, PtrTable src, OutTable codes,
                                                              OutTable scales, size_t n, int mode) {
  const size_t g = group_index<BlockOrder>();
  if ((g + 1) * kBlocksPerGroup * kBlock <= n) fused_fp8_body<K, ET, true>(out, src, codes, scales, n, mode, g);
  else fused_fp8_body<K, ET, false>(out, src, codes, scales, n, mode, g);
}

// The same pass in 128-lane workgroups (8 blocks) taken in index order, at
// the sizes fused_fp8_half names for float32 and float64 gradients.  Both
// lane maps place a block by its index alone, so the bits are those of the
// 256-lane kernel.
template <int K, int ET>
__global__ __launch_bounds__(kHalfThreads) void fused_fp8_half_kernel(void* out, PtrTable src, OutTable codes,
                                                                      OutTable scales, size_t n, int mode) {
  constexpr size_t per_group = (kHalfThreads / 16) * kBlock;
  const size_t g = blockIdx.x;
  if ((g + 1) * per_group <= n) {
    fused_fp8_body<K, ET, true, 0, kHalfThreads>(out, src, codes, scales, n, mode, g);
  } else {
    fused_fp8_body<K, ET, false, 0, kHalfThreads>(out, src, codes, scales, n, mode, g);
  }
}

// The pass over float32 gradients with one block per wavefront: workgroup b
// is block b, lane l its values 4l to 4l + 3, so each load or store of a
// rank covers 1 KiB (256 bytes of codes) in one piece.  The block maximum
// and so every bit are those of the 16-lane map.
template <int K, bool FULL, int DIV = 0>
__device__ __forceinline__ void fused_fp8_wave_body(float* out, const PtrTable& src, const OutTable& codes,
                                                    const OutTable& scales, size_t n, int mode, size_t block,
                                                    float d = 1.0f, float inv = 0.0f) {
  const size_t e = block * kBlock + 4 * (size_t)threadIdx.x;
  f4 x[K];
#pragma unroll
  for (int r = 0; r < K; r++) x[r] = load4_at<FULL>(static_cast<const float*>(src.p[r]), e, n);
  f4 a[1];
#pragma unroll
  for (int r = 0; r < K; r++) {
    uint32_t w;
    const float s = encode_block4(x[r], mode, w);  // all 64 lanes take part
    if (threadIdx.x == 0u) static_cast<float*>(scales.p[r])[block] = s;
    store_codes4_at<FULL>(static_cast<uint8_t*>(codes.p[r]), e, n, w);
    const f4 v = e4m3_unpack4(w) * s;
    a[0] = r == 0 ? v : a[0] + v;
  }
  avg_total<DIV>(a, d, inv);
  store4_at<FULL>(out, e, n, canon4(a[0]));
}

template <int K>
__global__ __launch_bounds__(64) void fused_fp8_wave_kernel(float* out, PtrTable src, OutTable codes,
                                                            OutTable scales, size_t n, int mode) {
  const size_t block = blockIdx.x;  // the grid has one workgroup per block, so block * kBlock < n
  if ((block + 1) * kBlock <= n) fused_fp8_wave_body<K, true>(out, src, codes, scales, n, mode, block);
  else fused_fp8_wave_body<K, false>(out, src, codes, scales, n, mode, block);
}

// The batch over float32 gradients in the same shape: bucket b takes
// workgroups [first[b], first[b + 1]), 16 per 4096-value group, and those
// past the bucket's last block return at once (uniformly per workgroup).
template <int K, int DIV>
__global__ __launch_bounds__(64) void fused_fp8_wave_batch_kernel(BucketBatch t, int mode, float d, float inv) {
  const size_t w = blockIdx.x;
  uint32_t b = 0;
  for (uint32_t i = 1; i < t.count; i++) b += w >= t.first[i] ? 1u : 0u;
  const size_t block = w - t.first[b], n = t.n[b];
  if (block * kBlock >= n) return;
  PtrTable src;
  OutTable codes, scales;
#pragma unroll
  for (int r = 0; r < K; r++) {
    src.p[r] = t.src[b][r];
    codes.p[r] = t.codes[b][r];
    scales.p[r] = t.scales[b][r];
  }
  float* out = static_cast<float*>(t.out[b]);
  if ((block + 1) * kBlock <= n) fused_fp8_wave_body<K, true, DIV>(out, src, codes, scales, n, mode, block, d, inv);
  else fused_fp8_wave_body<K, false, DIV>(out, src, codes, scales, n, mode, block, d, inv);
}

// Several buckets in one launch (gradients of element type ET): each
// workgroup finds its bucket from the table of first workgroups, then runs
// the fused pass over that bucket's group: in index order within a bucket,
// or in BlockOrder for a bucket large enough, as a whole-buffer launch.
template <int K, int ET, int DIV>
__global__ __launch_bounds__(kThreads) void fused_fp8_batch_kernel(BucketBatch t, int mode, float d, float inv) {
  const size_t w = blockIdx.x;
  uint32_t b = 0;
  for (uint32_t i = 1; i < t.count; i++) b += w >= t.first[i] ? 1u : 0u;
  PtrTable src;
  OutTable codes, scales;
#pragma unroll
  for (int r = 0; r < K; r++) {
    src.p[r] = t.src[b][r];
    codes.p[r] = t.codes[b][r];
    scales.p[r] = t.scales[b][r];
  }
  // a bucket large enough takes the permuted order of a whole-buffer launch
  const size_t g = group_index_in<BlockOrder>(w - t.first[b], t.first[b + 1] - t.first[b]), n = t.n[b];
  if ((g + 1) * kBlocksPerGroup * kBlock <= n) fused_fp8_body<K, ET, true, DIV>(t.out[b], src, codes, scales, n, mode, g, d, inv);
  else fused_fp8_body<K, ET, false, DIV>(t.out[b], src, codes, scales, n, mode, g, d, inv);
}

// Launcher bodies, one per element type ET.  Accumulation into the output
// is offered for float32 only.
template <int ET>
hipError_t encode_fp8_t(uint8_t* codes, float* scales, const void* src, size_t n, int scale_mode,
                        hipStream_t stream) {
  const size_t grid = grid_for(n, 16);  // 16 values per lane: a 256-lane group does 16 blocks
  if (grid == 0) return hipErrorInvalidValue;
  encode_fp8_kernel<ET><<<grid, kThreads, 0, stream>>>(codes, scales, src, n, scale_mode);
  return hipGetLastError();
}

template <int ET>
hipError_t decode_fp8_t(void* acc, const PtrTable& codes, const PtrTable& scales, int k, size_t n,
                        bool accumulate, hipStream_t stream) {
  const size_t grid = grid_for(n, 16);
  if (grid == 0) return hipErrorInvalidValue;
  if (accumulate && ET != GB_DTYPE_F32) return hipErrorInvalidValue;
  if constexpr (ET == GB_DTYPE_F32) {
    // one workgroup per block; beyond the largest grid the 256-lane kernel runs
    const size_t wave_grid = ceil_div(n, kBlock);
    if (decode_fp8_wave(k, n) && wave_grid <= kMaxGrid) {
      float* a = static_cast<float*>(acc);
      if (accumulate) decode_fp8_wave_kernel<true><<<wave_grid, 64, 0, stream>>>(a, codes, scales, n);
      else decode_fp8_wave_kernel<false><<<wave_grid, 64, 0, stream>>>(a, codes, scales, n);
      return hipGetLastError();
    }
  }
#define GB_CALL(K)                                                                                               \
  if constexpr (ET == GB_DTYPE_F32) {                                                                            \
    if (accumulate) decode_fp8_kernel<K, true, ET><<<grid, kThreads, decode_fp8_lds<ET>(K), stream>>>(acc, codes, scales, n); \
    else decode_fp8_kernel<K, false, ET><<<grid, kThreads, decode_fp8_lds<ET>(K), stream>>>(acc, codes, scales, n);          \
  } else {                                                                                                       \
    decode_fp8_kernel<K, false, ET><<<grid, kThreads, decode_fp8_lds<ET>(K), stream>>>(acc, codes, scales, n);             \
  }
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

template <int ET>
hipError_t fused_fp8_t(void* out, const PtrTable& srcs, const OutTable& c, const OutTable& s, int k, size_t n,
                       int scale_mode, hipStream_t stream) {
  if constexpr (ET == GB_DTYPE_F32) {
    // one workgroup per block; beyond the largest grid (above 2^39 - 2^8
    // values) the 256-lane kernel runs
    const size_t wave_grid = ceil_div(n, kBlock);
    if (fused_fp8_wave(k, n) && wave_grid <= kMaxGrid) {
      // the rule holds for 4 ranks only, so only that instantiation exists
      fused_fp8_wave_kernel<4><<<wave_grid, 64, kFp8WaveLds, stream>>>(static_cast<float*>(out), srcs, c, s, n,
                                                                      scale_mode);
      return hipGetLastError();
    }
  }
  if constexpr (ET == GB_DTYPE_F32 || ET == GB_DTYPE_F64) {
    if (fused_fp8_half<ET>(k, n)) {
      const size_t half_grid = ceil_div(n, (kHalfThreads / 16) * kBlock);
      if (half_grid > kMaxGrid) return hipErrorInvalidValue;
#define GB_CALL(K)                                                                                   \
  fused_fp8_half_kernel<K, ET><<<half_grid, kHalfThreads, fused_fp8_half_lds<ET>(K), stream>>>(out, srcs, c, s, n, \
                                                                                              scale_mode);
      GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
      return hipGetLastError();
    }
  }
  const size_t grid = grid_for(n, 16);
  if (grid == 0) return hipErrorInvalidValue;
#define GB_CALL(K) fused_fp8_kernel<K, ET><<<grid, kThreads, fused_fp8_lds<ET>(K, n), stream>>>(out, srcs, c, s, n, scale_mode);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

}  // namespace

hipError_t launch_encode_fp8(uint8_t* codes, float* scales, const void* src, size_t n, int scale_mode, int dtype,
                             hipStream_t stream) {
#define GB_CALL(ET) encode_fp8_t<ET>(codes, scales, src, n, scale_mode, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

hipError_t launch_decode_fp8(void* acc, const PtrTable& codes, const PtrTable& scales, int k, size_t n,
                             bool accumulate, int dtype, hipStream_t stream) {
#define GB_CALL(ET) decode_fp8_t<ET>(acc, codes, scales, k, n, accumulate, stream)
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

size_t batch_groups(int codec, size_t n) {
  return codec == GB_CODEC_BF16 ? ceil_div(n, kVecPerGroup) : ceil_div(n, kBlocksPerGroup * kBlock);
}

namespace {
// A batched launch takes the fused pass's cap for its largest bucket.
template <int ET, int DIV>
hipError_t fused_fp8_batch_t(BucketBatch& t, size_t grid, int k, int scale_mode, float d, float inv,
                             hipStream_t stream) {
  size_t largest = 0;
  for (uint32_t b = 0; b < t.count; b++) largest = t.n[b] > largest ? t.n[b] : largest;
  if constexpr (ET == GB_DTYPE_F32) {
    // sixteen 64-lane workgroups per group, as the whole-buffer launch takes
    // its largest bucket
    if (fused_fp8_wave(k, largest) && grid <= kMaxGrid / 16) {
      for (int b = 0; b <= kBatchBuckets; b++) t.first[b] *= 16;
      fused_fp8_wave_batch_kernel<4, DIV><<<16 * grid, 64, kFp8WaveLds, stream>>>(t, scale_mode, d, inv);
      return hipGetLastError();
    }
  }
#define GB_CALL(K) \
  fused_fp8_batch_kernel<K, ET, DIV><<<grid, kThreads, fused_fp8_lds<ET>(K, largest), stream>>>(t, scale_mode, d, inv);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fused_fp8_batch(BucketBatch& t, int k, int scale_mode, int dtype, int divisor,
                                  hipStream_t stream) {
  if (t.count == 0 || t.count > (uint32_t)kBatchBuckets) return hipErrorInvalidValue;
  size_t grid = 0;
  for (uint32_t b = 0; b < t.count; b++) {
    t.first[b] = grid;
    grid += batch_groups(GB_CODEC_FP8_E4M3_B256, t.n[b]);
  }
  for (int b = (int)t.count; b <= kBatchBuckets; b++) t.first[b] = grid;
  if (grid == 0 || grid > kMaxGrid) return hipErrorInvalidValue;
  if (divisor != 1) {  // float32 totals only
    if (dtype != GB_DTYPE_F32) return hipErrorInvalidValue;
    (void)hipGetLastError();
    const float d = (float)divisor, inv = (divisor & (divisor - 1)) == 0 ? 1.0f / d : 0.0f;
    return inv != 0.0f ? fused_fp8_batch_t<GB_DTYPE_F32, 1>(t, grid, k, scale_mode, d, inv, stream)
                       : fused_fp8_batch_t<GB_DTYPE_F32, 2>(t, grid, k, scale_mode, d, inv, stream);
  }
#define GB_CALL(ET) fused_fp8_batch_t<ET, 0>(t, grid, k, scale_mode, 1.0f, 0.0f, stream)
  GB_DISPATCH_ET(dtype, GB_CALL)
#undef GB_CALL
}

hipError_t launch_reduce_encode_fp8(float* sum, uint8_t* codes, float* scales, const PtrTable& srcs, int k,
                                   size_t n, int scale_mode, hipStream_t stream) {
  const size_t grid = grid_for(n, 16);
  if (grid == 0) return hipErrorInvalidValue;
  (void)hipGetLastError();
#define GB_CALL(K)                                                                                              \
  if (sum != nullptr)                                                                                           \
    reduce_encode_fp8_kernel<K, true><<<grid, kThreads, heavy_lds(K), stream>>>(sum, codes, scales, srcs, n,     \
                                                                                scale_mode);                    \
  else                                                                                                          \
    reduce_encode_fp8_kernel<K, false><<<grid, kThreads, heavy_lds(K), stream>>>(sum, codes, scales, srcs, n,    \
                                                                                 scale_mode);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

}  // namespace gb
