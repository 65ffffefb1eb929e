// gb_ef.hip — the error-feedback encoders and bucket passes of libgbreduce.
#include "gb_device.h"

namespace gb {
namespace {

// ===========================================================================
// Error feedback (README "Bridge compression": each bridge member keeps a
// residual per buffer).  y = x + residual is encoded exactly as above, and
// the residual becomes y minus the value the payload decodes to (rounded
// binary32 subtraction; exact for bf16).  The residual is read and written
// in place by the lane that owns the value.
// ===========================================================================
template <bool FULL>
__device__ __forceinline__ void encode_bf16_ef_body(uint16_t* codes, float* res, const float* src, size_t n) {
  const size_t i = (group_index<VecOrder>() * kThreads + threadIdx.x) * 4;
  if (!FULL && i >= n) return;
  const f4 y = load4_at<FULL>(src, i, n) + load4_at<FULL>(res, i, n);
  const u2 w = bf16_pack4(y);
  store_bf16_4_at<FULL>(codes, i, n, w);
  store4_at<FULL>(res, i, n, y - bf16_unpack4(w));
}

__global__ __launch_bounds__(kThreads) void encode_bf16_ef_kernel(uint16_t* codes, float* res, const float* src,
                                                                   size_t n) {
  if (group_full<VecOrder>(kVecPerGroup, n)) encode_bf16_ef_body<true>(codes, res, src, n);
  else encode_bf16_ef_body<false>(codes, res, src, n);
}

template <bool FULL>
__device__ __forceinline__ void encode_fp8_ef_body(uint8_t* codes, float* scales, float* res, const float* src,
                                                   size_t n, int mode) {
  const uint32_t col = threadIdx.x & 15u;
  const size_t block = group_index<BlockOrder>() * kBlocksPerGroup + (threadIdx.x >> 4);
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
  if (group_full<BlockOrder>(kBlocksPerGroup * kBlock, n)) encode_fp8_ef_body<true>(codes, scales, res, src, n, mode);
  else encode_fp8_ef_body<false>(codes, scales, res, src, n, mode);
}

template <int K, bool FULL>
__device__ __forceinline__ void fused_fp8_ef_body(float* out, const PtrTable& src, const OutTable& resid,
                                                  const OutTable& codes, const OutTable& scales, size_t n,
                                                  int mode) {
  const uint32_t col = threadIdx.x & 15u;
  const size_t block = group_index<BlockOrder>() * kBlocksPerGroup + (threadIdx.x >> 4);
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
  if (group_full<BlockOrder>(kBlocksPerGroup * kBlock, n)) fused_fp8_ef_body<K, true>(out, src, resid, codes, scales, n, mode);
  else fused_fp8_ef_body<K, false>(out, src, resid, codes, scales, n, mode);
}

template <int K, bool FULL>
__device__ __forceinline__ void fused_bf16_ef_body(float* out, const PtrTable& src, const OutTable& resid,
                                                   const OutTable& codes, size_t n) {
  const size_t i = (group_index<VecOrder>() * kThreads + threadIdx.x) * 4;
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
  if (group_full<VecOrder>(kVecPerGroup, n)) fused_bf16_ef_body<K, true>(out, src, resid, codes, n);
  else fused_bf16_ef_body<K, false>(out, src, resid, codes, n);
}

}  // namespace

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
#define GB_CALL(K) fused_bf16_ef_kernel<K><<<grid, kThreads, heavy_lds(K), stream>>>(out, srcs, rs, c, n);
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
#define GB_CALL(K) fused_fp8_ef_kernel<K><<<grid, kThreads, ef_lds(K), stream>>>(out, srcs, rs, c, s, n, scale_mode);
  GB_DISPATCH_K(k, GB_CALL)
#undef GB_CALL
  return hipGetLastError();
}

}  // namespace gb
