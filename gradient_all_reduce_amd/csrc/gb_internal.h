// gb_internal.h — launchers shared by the C-ABI layer (gb_api.cpp) and the
// HIP kernel sources (gb_*.hip).  Not installed; the public ABI is
// include/gbreduce.h.
//
// Every launcher assumes its arguments were validated by gb_api.cpp: pointers
// non-null and aligned as the ABI requires, 1 <= k <= kLaunchRanks, n > 0.  Each
// returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include <chrono>

#include "gbreduce.h"

namespace gb {

// Ranks one kernel launch reads (its rank count is a template parameter);
// calls with more ranks fold the rest in further launches.
constexpr int kLaunchRanks = 8;

// Largest grid (workgroups) of one launch.
constexpr size_t kMaxGrid = ((size_t)1 << 31) - 1;

// Up to kLaunchRanks device pointers, passed to kernels by value.
struct PtrTable {
  const void* p[kLaunchRanks];
};

// Values per fp8 scale block, and blocks per workgroup in the block kernels
// (a 256-lane workgroup = 4 wavefronts x 4 rows of 16 lanes, one row per
// block).
constexpr size_t kBlock = GB_BLOCK;

hipError_t launch_reduce_sum(float* dst, const PtrTable& srcs, int k, size_t n,
                             bool accumulate, hipStream_t stream);
// op = GB_OP_SUM, GB_OP_AVG (sum / divisor), GB_OP_MAX or GB_OP_MIN.
hipError_t launch_reduce_op(float* dst, const PtrTable& srcs, int k, size_t n, int op, int divisor,
                            hipStream_t stream);
// Any element type but fp32 (GB_DTYPE_*); integer types with SUM, MAX, MIN.
hipError_t launch_reduce_typed(void* dst, const PtrTable& srcs, int k, size_t n, int dtype, int op, int divisor,
                               hipStream_t stream);
// The codec launchers take the element type of the values they read or
// write (dtype: GB_DTYPE_F32, F16, BF16 or F64); accumulate needs F32.
hipError_t launch_encode_bf16(uint16_t* codes, const void* src, size_t n, int dtype, hipStream_t stream);
hipError_t launch_encode_fp8(uint8_t* codes, float* scales, const void* src, size_t n, int scale_mode, int dtype,
                             hipStream_t stream);
hipError_t launch_decode_bf16(void* acc, const PtrTable& codes, int k, size_t n, bool accumulate, int dtype,
                              hipStream_t stream);
hipError_t launch_decode_fp8(void* acc, const PtrTable& codes, const PtrTable& scales, int k, size_t n,
                             bool accumulate, int dtype, hipStream_t stream);
// One pass over [0, n) of k sources: encode each source into its payload
// (codes[r], scales[r]) and write the decoded rank-order sum to out.
hipError_t launch_fused_bf16(void* out, const PtrTable& srcs, uint16_t* const* codes, int k, size_t n, int dtype,
                             hipStream_t stream);
hipError_t launch_fused_fp8(void* out, const PtrTable& srcs, uint8_t* const* codes, float* const* scales, int k,
                            size_t n, int scale_mode, int dtype, hipStream_t stream);

// Up to kBatchBuckets separately allocated buckets in one fused launch, each
// with its own sources, output and payloads, passed to the kernel by value
// (about 3.5 KiB of kernel arguments).  The caller
// fills count, n, out, src, codes and scales (scales for fp8 only); the
// launcher fills first: bucket b takes workgroups [first[b], first[b + 1]).
// 16 buckets per launch move 4-6% more bytes per second than 8 for buckets of
// 819,200 values (one GPU's 1/8 share of a 25 MiB bucket), 1-2% fewer for
// whole 25 MiB buckets, where one call over a contiguous buffer does better.
constexpr int kBatchBuckets = 16;
struct BucketBatch {
  uint32_t count;
  size_t first[kBatchBuckets + 1];
  size_t n[kBatchBuckets];
  void* out[kBatchBuckets];
  const void* src[kBatchBuckets][kLaunchRanks];
  void* codes[kBatchBuckets][kLaunchRanks];
  float* scales[kBatchBuckets][kLaunchRanks];
};
static_assert(sizeof(BucketBatch) <= 4000, "a batch must fit the 4 KiB of kernel arguments");
// The error-feedback form also carries each rank's residual, so it takes 8
// buckets per launch to stay within the kernel arguments.
constexpr int kBatchBucketsEf = 8;
struct BucketBatchEf {
  uint32_t count;
  size_t first[kBatchBucketsEf + 1];
  size_t n[kBatchBucketsEf];
  void* out[kBatchBucketsEf];
  const void* src[kBatchBucketsEf][kLaunchRanks];
  void* codes[kBatchBucketsEf][kLaunchRanks];
  float* scales[kBatchBucketsEf][kLaunchRanks];
  float* resid[kBatchBucketsEf][kLaunchRanks];
};
static_assert(sizeof(BucketBatchEf) <= 4000, "a batch must fit the 4 KiB of kernel arguments");

// Workgroups of one bucket of n values in a batched launch of codec
// (GB_CODEC_BF16 or GB_CODEC_FP8_E4M3_B256).
size_t batch_groups(int codec, size_t n);
// Every bucket has 0 < n, and the workgroups of all buckets fit one grid.
// divisor 1 leaves each total; any other divisor (1 .. 2^24, float32
// totals only) stores RN(total / divisor), the AVG of the job's world size.
hipError_t launch_fused_fp8_batch(BucketBatch& batch, int k, int scale_mode, int dtype, int divisor,
                                  hipStream_t stream);
hipError_t launch_fused_bf16_batch(BucketBatch& batch, int k, int dtype, int divisor, hipStream_t stream);
hipError_t launch_fused_fp8_ef_batch(BucketBatchEf& batch, int k, int scale_mode, int dtype, int divisor,
                                     hipStream_t stream);
hipError_t launch_fused_bf16_ef_batch(BucketBatchEf& batch, int k, int dtype, int divisor, hipStream_t stream);

// The rank-order float32 sum of k sources encoded in one pass (sum stored too
// when not NULL).
hipError_t launch_reduce_encode_bf16(float* sum, uint16_t* codes, const PtrTable& srcs, int k, size_t n,
                                    hipStream_t stream);
hipError_t launch_reduce_encode_fp8(float* sum, uint8_t* codes, float* scales, const PtrTable& srcs, int k,
                                   size_t n, int scale_mode, hipStream_t stream);

// Error-feedback variants over gradients of element type dtype (binary32
// residuals): residual (or residuals[r]) is read and rewritten.
hipError_t launch_encode_bf16_ef(uint16_t* codes, float* residual, const void* src, size_t n, int dtype,
                                 hipStream_t stream);
hipError_t launch_encode_fp8_ef(uint8_t* codes, float* scales, float* residual, const void* src, size_t n,
                                int scale_mode, int dtype, hipStream_t stream);
hipError_t launch_fused_bf16_ef(void* out, const PtrTable& srcs, float* const* residuals, uint16_t* const* codes,
                                int k, size_t n, int dtype, hipStream_t stream);
hipError_t launch_fused_fp8_ef(void* out, const PtrTable& srcs, float* const* residuals, uint8_t* const* codes,
                               float* const* scales, int k, size_t n, int scale_mode, int dtype, hipStream_t stream);

// gb_bucket_allreduce_local with its failures reported under the name fn:
// validation (workspace included), then the launches.
gb_status bucket_allreduce_local(const char* fn, float* out, const float* const* srcs, int k, size_t n,
                                 size_t bucket_elems, int codec, int scale_mode, void* workspace,
                                 size_t workspace_bytes, void* stream);
// Records a failure for gb_last_error() and returns s.
gb_status fail_status(gb_status s, const char* msg);

// Per-call hooks, switched on by two environment variables read once, at
// the first call of the process (set and not "0" means on):
//   GB_TRACE  one line per call on stderr: the entry point, k, n and the
//             codec where it takes them, the stream, the status (with the
//             message of a failure) and the host time the call took;
//   GB_DEBUG  after a call that returned GB_OK, wait for its stream; an error
//             the stream reports (a kernel of the call, or earlier work on
//             the stream, failed) turns the status into GB_ERR_HIP.  A stream
//             under graph capture is not waited for.
// Off (the default), a call pays one test of a cached flag.
constexpr size_t kNoSize = ~(size_t)0;  // no n to report
bool call_hooks_on();
gb_status finish_call(const char* fn, void* stream, int k, size_t n, int codec, gb_status s, double host_us);

// Runs an entry point's body under the hooks; fn is the entry point's name.
template <class Body>
gb_status traced_call(const char* fn, void* stream, int k, size_t n, int codec, Body&& body) {
  if (!call_hooks_on()) return body(fn);
  const auto t0 = std::chrono::steady_clock::now();
  const gb_status s = body(fn);
  const double us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
  return finish_call(fn, stream, k, n, codec, s, us);
}

}  // namespace gb
