// stub_hip.cpp — host stand-ins for the kernel launchers and the HIP runtime
// calls that the C ABI layer (gradient_all_reduce_amd/csrc/gb_api.cpp) makes,
// so that layer can be built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer and driven on a machine without a GPU.  Test
// infrastructure: nothing here runs in the library.
//
// Every launcher checks the promises the ABI layer makes to the kernels (n >
// 0, 1 <= k <= 8, every pointer it passes non-null, a batch of 1..16 buckets
// each with values), counts the launch and returns hipSuccess, or the
// injected error on the chosen launch.  Pointers are never dereferenced: the
// drivers pass fabricated addresses.  hipPointerGetAttributes reports the
// addresses from kPinnedBase up as pinned host memory.  hipStreamSynchronize
// and hipStreamIsCapturing count waits and report what the driver sets, for
// the GB_DEBUG hook.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>

#include "../../gradient_all_reduce_amd/csrc/gb_internal.h"

namespace {

long g_launches = 0, g_copies = 0, g_fail_at = 0, g_syncs = 0;
int g_sync_fails = 0, g_capturing = 0;
hipError_t g_fail_error = hipErrorLaunchFailure;
constexpr uintptr_t kPinnedBase = (uintptr_t)0x700000000000ull;

[[noreturn]] void broken(const char* what, const char* why) {
  std::fprintf(stderr, "stub: %s: %s\n", what, why);
  std::abort();
}

hipError_t launch(const char* what, size_t n, int k) {
  if (n == 0) broken(what, "launched with n = 0");
  if (k < 1 || k > gb::kLaunchRanks) broken(what, "launched with k outside 1..8");
  ++g_launches;
  return g_fail_at != 0 && g_launches == g_fail_at ? g_fail_error : hipSuccess;
}

void need(const void* p, const char* what) {
  if (p == nullptr) broken(what, "a pointer the kernel reads or writes is NULL");
}

void need_table(const gb::PtrTable& t, int k, const char* what) {
  for (int r = 0; r < k; r++) need(t.p[r], what);
}

template <class Batch>
hipError_t launch_batch(const char* what, const Batch& b, int k, int cap) {
  if (b.count < 1 || b.count > (uint32_t)cap) broken(what, "batch of the wrong size");
  for (uint32_t i = 0; i < b.count; i++) {
    if (b.n[i] == 0) broken(what, "an empty bucket in a batch");
    need(b.out[i], what);
    for (int r = 0; r < k; r++) need(b.src[i][r], what);
  }
  return launch(what, b.n[0], k);
}

int g_stream_object, g_event_object;

}  // namespace

extern "C" {
void stub_reset(void) { g_launches = g_copies = g_fail_at = 0; }
void stub_fail_at(long nth) { g_fail_at = nth; }
long stub_launches(void) { return g_launches; }
long stub_copies(void) { return g_copies; }
unsigned long long stub_pinned_base(void) { return (unsigned long long)kPinnedBase; }
// hipStreamSynchronize reports an error while on != 0; the stream reads as
// under graph capture while capturing != 0.
void stub_sync_fails(int on) { g_sync_fails = on; }
void stub_capturing(int capturing) { g_capturing = capturing; }
long stub_syncs(void) { return g_syncs; }
}

namespace gb {

hipError_t launch_reduce_sum(float* dst, const PtrTable& srcs, int k, size_t n, bool, hipStream_t) {
  need(dst, "reduce_sum");
  need_table(srcs, k, "reduce_sum");
  return launch("reduce_sum", n, k);
}
hipError_t launch_reduce_op(float* dst, const PtrTable& srcs, int k, size_t n, int, int, hipStream_t) {
  need(dst, "reduce_op");
  need_table(srcs, k, "reduce_op");
  return launch("reduce_op", n, k);
}
hipError_t launch_reduce_typed(void* dst, const PtrTable& srcs, int k, size_t n, int, int, int, hipStream_t) {
  need(dst, "reduce_typed");
  need_table(srcs, k, "reduce_typed");
  return launch("reduce_typed", n, k);
}
hipError_t launch_encode_bf16(uint16_t* codes, const void* src, size_t n, int, hipStream_t) {
  need(codes, "encode_bf16");
  need(src, "encode_bf16");
  return launch("encode_bf16", n, 1);
}
hipError_t launch_encode_fp8(uint8_t* codes, float* scales, const void* src, size_t n, int, int, hipStream_t) {
  need(codes, "encode_fp8");
  need(scales, "encode_fp8");
  need(src, "encode_fp8");
  return launch("encode_fp8", n, 1);
}
hipError_t launch_decode_bf16(void* acc, const PtrTable& codes, int k, size_t n, bool, int, hipStream_t) {
  need(acc, "decode_bf16");
  need_table(codes, k, "decode_bf16");
  return launch("decode_bf16", n, k);
}
hipError_t launch_decode_fp8(void* acc, const PtrTable& codes, const PtrTable& scales, int k, size_t n, bool, int,
                             hipStream_t) {
  need(acc, "decode_fp8");
  need_table(codes, k, "decode_fp8");
  need_table(scales, k, "decode_fp8");
  return launch("decode_fp8", n, k);
}
hipError_t launch_fused_bf16(void* out, const PtrTable& srcs, uint16_t* const* codes, int k, size_t n, int,
                             hipStream_t) {
  need(out, "fused_bf16");
  need_table(srcs, k, "fused_bf16");
  for (int r = 0; r < k; r++) need(codes[r], "fused_bf16");
  return launch("fused_bf16", n, k);
}
hipError_t launch_fused_fp8(void* out, const PtrTable& srcs, uint8_t* const* codes, float* const* scales, int k,
                            size_t n, int, int, hipStream_t) {
  need(out, "fused_fp8");
  need_table(srcs, k, "fused_fp8");
  for (int r = 0; r < k; r++) {
    need(codes[r], "fused_fp8");
    need(scales[r], "fused_fp8");
  }
  return launch("fused_fp8", n, k);
}
size_t batch_groups(int codec, size_t n) { return codec == GB_CODEC_BF16 ? (n + 1023) / 1024 : (n + 4095) / 4096; }
hipError_t launch_fused_fp8_batch(BucketBatch& b, int k, int, int, int, hipStream_t) {
  return launch_batch("fused_fp8_batch", b, k, kBatchBuckets);
}
hipError_t launch_fused_bf16_batch(BucketBatch& b, int k, int, int, hipStream_t) {
  return launch_batch("fused_bf16_batch", b, k, kBatchBuckets);
}
hipError_t launch_fused_fp8_ef_batch(BucketBatchEf& b, int k, int, int, int, hipStream_t) {
  return launch_batch("fused_fp8_ef_batch", b, k, kBatchBucketsEf);
}
hipError_t launch_fused_bf16_ef_batch(BucketBatchEf& b, int k, int, int, hipStream_t) {
  return launch_batch("fused_bf16_ef_batch", b, k, kBatchBucketsEf);
}
hipError_t launch_reduce_encode_bf16(float*, uint16_t* codes, const PtrTable& srcs, int k, size_t n, hipStream_t) {
  need(codes, "reduce_encode_bf16");
  need_table(srcs, k, "reduce_encode_bf16");
  return launch("reduce_encode_bf16", n, k);
}
hipError_t launch_reduce_encode_fp8(float*, uint8_t* codes, float* scales, const PtrTable& srcs, int k, size_t n, int,
                                   hipStream_t) {
  need(codes, "reduce_encode_fp8");
  need(scales, "reduce_encode_fp8");
  need_table(srcs, k, "reduce_encode_fp8");
  return launch("reduce_encode_fp8", n, k);
}
hipError_t launch_encode_bf16_ef(uint16_t* codes, float* residual, const void* src, size_t n, int, hipStream_t) {
  need(codes, "encode_bf16_ef");
  need(residual, "encode_bf16_ef");
  need(src, "encode_bf16_ef");
  return launch("encode_bf16_ef", n, 1);
}
hipError_t launch_encode_fp8_ef(uint8_t* codes, float* scales, float* residual, const void* src, size_t n, int, int,
                                hipStream_t) {
  need(codes, "encode_fp8_ef");
  need(scales, "encode_fp8_ef");
  need(residual, "encode_fp8_ef");
  need(src, "encode_fp8_ef");
  return launch("encode_fp8_ef", n, 1);
}
hipError_t launch_fused_bf16_ef(void* out, const PtrTable& srcs, float* const* residuals, uint16_t* const* codes,
                                int k, size_t n, int, hipStream_t) {
  need(out, "fused_bf16_ef");
  need_table(srcs, k, "fused_bf16_ef");
  for (int r = 0; r < k; r++) {
    need(residuals[r], "fused_bf16_ef");
    need(codes[r], "fused_bf16_ef");
  }
  return launch("fused_bf16_ef", n, k);
}
hipError_t launch_fused_fp8_ef(void* out, const PtrTable& srcs, float* const* residuals, uint8_t* const* codes,
                               float* const* scales, int k, size_t n, int, int, hipStream_t) {
  need(out, "fused_fp8_ef");
  need_table(srcs, k, "fused_fp8_ef");
  for (int r = 0; r < k; r++) {
    need(residuals[r], "fused_fp8_ef");
    need(codes[r], "fused_fp8_ef");
    need(scales[r], "fused_fp8_ef");
  }
  return launch("fused_fp8_ef", n, k);
}

}  // namespace gb

extern "C" {

const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "injected failure"; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* event, unsigned) {
  *event = reinterpret_cast<hipEvent_t>(&g_event_object);
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t) { return hipSuccess; }
hipError_t hipStreamCreateWithFlags(hipStream_t* stream, unsigned) {
  *stream = reinterpret_cast<hipStream_t>(&g_stream_object);
  return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t) { return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned) { return hipSuccess; }
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t) {
  if (dst == nullptr || src == nullptr || bytes == 0) broken("hipMemcpyAsync", "empty or NULL copy");
  ++g_copies;
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) {
  ++g_syncs;
  return g_sync_fails ? hipErrorIllegalAddress : hipSuccess;
}
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* status) {
  *status = g_capturing ? hipStreamCaptureStatusActive : hipStreamCaptureStatusNone;
  return hipSuccess;
}
hipError_t hipPointerGetAttributes(hipPointerAttribute_t* attributes, const void* ptr) {
  if (reinterpret_cast<uintptr_t>(ptr) < kPinnedBase) return hipErrorInvalidValue;
  attributes->type = hipMemoryTypeHost;
  return hipSuccess;
}

}  // extern "C"
