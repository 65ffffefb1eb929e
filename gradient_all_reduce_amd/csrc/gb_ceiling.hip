// gb_ceiling.hip — the memory ceiling of one MI355X, measured: the program
// behind bench.py's `memory_ceiling` object and its rocprofv3 summaries.
// It is not part of libgbreduce.
//
// Every kernel here moves 16-byte non-temporal vectors through HBM with no
// arithmetic worth the name, in one of the shapes the library's kernels
// could take, so the fastest of them bounds what a streaming kernel of that
// read/write mix can reach on this chip:
//   copy      1 GiB or 4 GiB read and written: U vectors per lane (U = 1, 2,
//             4), index order or the 8-front order of the vector kernels;
//   copy_lds  the same with the loads going straight into LDS
//             (global_load_lds_dwordx4, gfx950) and out of it to the stores;
//   read      read only (the sum of each lane's values is stored only if it
//             takes an impossible value), 4 vectors per lane, 2 per CU;
//   write     write only, 1 vector per lane;
//   replica   the memory pattern of the fused fp8 bucket pass over 4 ranks,
//             with the encode replaced by taking each value's top byte: 4
//             float32 sources read, 4 code streams, 4 scale streams and the
//             float32 total written, in the pass's lane map and in the shape
//             it takes at this size (one block per 64-lane workgroup, in
//             index order, 20 per compute unit);
//   replica_ef the same for the fp8 pass with error feedback: 4 sources and
//             4 float32 residuals read; codes, scales, the 4 residuals and
//             the total written (21 streams), in that pass's shape at this
//             size (one block per 64-lane workgroup, 6 per CU).
// The buffers hold gradient-like values (every float32 a hash of its index,
// spread over +-1e-3; the write kernel stores varying bits too), because
// what the bits are changes how fast HBM moves them: a buffer of zeros
// copies several percent faster.  One copy of a zero-filled buffer is
// measured beside the others as that contrast (zeros_copy_u1), and is not a
// ceiling.
// Then the fixed cost of a launch itself: 153 launches, back to back on one
// stream, of a kernel whose body does nothing, from the stream and replayed
// from a HIP graph, for grids of 1 workgroup, of the 1,600 of one 6,553,600-
// value bucket, and of 25,600.
// Each line of output is one variant: its bytes per launch and the median
// and best GB/s over timed launches (hipEvents), or the median microseconds
// per launch; the last line is one JSON object: {"median_gbs": {...},
// "launch_us": {...}}.  Usage: gb_ceiling [size_gib] [reps].
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <utility>
#include <vector>

#include "gb_device.h"

namespace {

using gb::f4;
using gb::kThreads;

#define CK(call)                                                                              \
  do {                                                                                        \
    hipError_t e_ = (call);                                                                   \
    if (e_ != hipSuccess) {                                                                   \
      std::fprintf(stderr, "gb_ceiling: %s failed: %s\n", #call, hipGetErrorString(e_));      \
      std::exit(1);                                                                           \
    }                                                                                         \
  } while (0)

// The workgroup's group: index order, or 8 fronts 256 groups apart.
template <bool FRONTS>
__device__ __forceinline__ size_t group() {
  return FRONTS ? gb::group_index_in<gb::GroupOrder<8, 256, 1>>(blockIdx.x, gridDim.x) : (size_t)blockIdx.x;
}

// TAG only names a second instantiation (the zero-data contrast) apart.
template <int U, bool FRONTS, int TAG = 0>
__global__ __launch_bounds__(kThreads) void copy_kernel(const f4* __restrict__ src, f4* __restrict__ dst) {
  const size_t base = group<FRONTS>() * kThreads * U + threadIdx.x;
  f4 v[U];
#pragma unroll
  for (int u = 0; u < U; u++) v[u] = __builtin_nontemporal_load(src + base + (size_t)u * kThreads);
#pragma unroll
  for (int u = 0; u < U; u++) __builtin_nontemporal_store(v[u], dst + base + (size_t)u * kThreads);
}

// Loads land in LDS at M0 + 16 * lane: each wave passes its own 1 KiB slice
// of a vector's 4 KiB row as the base.
template <int U>
__global__ __launch_bounds__(kThreads) void copy_lds_kernel(const f4* __restrict__ src, f4* __restrict__ dst) {
  __shared__ f4 buf[U * kThreads];
  const size_t base = (size_t)blockIdx.x * kThreads * U + threadIdx.x;
  const unsigned wave = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < U; u++) {
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + base + (size_t)u * kThreads),
                                     (__attribute__((address_space(3))) void*)&buf[u * kThreads + wave * 64],
                                     16, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);  // every load of this wave has landed
#pragma unroll
  for (int u = 0; u < U; u++) __builtin_nontemporal_store(buf[u * kThreads + threadIdx.x], dst + base + (size_t)u * kThreads);
}

template <int U>
__global__ __launch_bounds__(kThreads) void read_kernel(const f4* __restrict__ src, float* sink) {
  const size_t base = (size_t)blockIdx.x * kThreads * U + threadIdx.x;
  f4 v[U];
#pragma unroll
  for (int u = 0; u < U; u++) v[u] = __builtin_nontemporal_load(src + base + (size_t)u * kThreads);
  float a = 0.0f;
#pragma unroll
  for (int u = 0; u < U; u++) a += (v[u].x + v[u].y) + (v[u].z + v[u].w);
  if (a == -1.25f) sink[0] = a;  // never true: every value read lies within +-1e-3
}

// Stores only if the grid has more lanes than it can (never).
__global__ __launch_bounds__(kThreads) void empty_kernel(float* sink) {
  if (threadIdx.x >= kThreads) sink[0] = 1.0f;
}

// Small positive floats whose low 23 bits come from a hash of the index.
__global__ __launch_bounds__(kThreads) void write_kernel(f4* __restrict__ dst, uint32_t seed) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const uint32_t h = (uint32_t)i * 2654435761u ^ seed;
  const uint32_t e = 0x3A000000u;
  const f4 v = {gb::bitsf(e | (h >> 9)), gb::bitsf(e | ((h * 3u) >> 9)), gb::bitsf(e | ((h * 5u) >> 9)),
                gb::bitsf(e | ((h * 7u) >> 9))};
  __builtin_nontemporal_store(v, dst + i);
}

// Gradient-like contents for a buffer of nvec vectors (grid-stride, any grid).
__global__ void fill_gradient_like(f4* p, size_t nvec, uint32_t seed) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += (size_t)gridDim.x * blockDim.x) {
    float x[4];
    for (int j = 0; j < 4; j++) {
      uint32_t h = (uint32_t)(4 * i + j) * 2654435761u ^ seed;
      h ^= h >> 15;
      h *= 2246822519u;
      h ^= h >> 13;
      h *= 3266489917u;
      h ^= h >> 16;
      x[j] = ((float)(h & 0xFFFFFFu) / 16777216.0f - 0.5f) * 2e-3f;
    }
    p[i] = f4{x[0], x[1], x[2], x[3]};
  }
}

// The fused fp8 pass's memory pattern (4 ranks, float32): lane map,
// workgroup size, order and cap of the library's kernel for large buffers
// (one 256-value block per 64-lane workgroup, 4 values per lane), the
// encode replaced by the top byte of each value and the scale by the
// block's first value.
__global__ __launch_bounds__(64) void replica_kernel(gb::PtrTable src, gb::OutTable codes, gb::OutTable scales,
                                                     float* __restrict__ out) {
  const size_t block = blockIdx.x, e = block * gb::kBlock + 4 * (size_t)threadIdx.x;
  f4 x[4];
#pragma unroll
  for (int r = 0; r < 4; r++) x[r] = gb::load4(static_cast<const float*>(src.p[r]) + e);
  f4 a;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const f4 v = x[r];
    const uint32_t w = (gb::fbits(v.x) >> 24) | ((gb::fbits(v.y) >> 24) << 8) | ((gb::fbits(v.z) >> 24) << 16) |
                       ((gb::fbits(v.w) >> 24) << 24);
    if (threadIdx.x == 0u) static_cast<float*>(scales.p[r])[block] = v.x;
    __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(codes.p[r]) + e));
    a = r == 0 ? v : a + v;
  }
  gb::store4(out + e, a);
}

// The error-feedback fp8 pass's memory pattern (4 ranks, float32), in the
// shape the pass takes for large buffers (one block per 64-lane workgroup,
// 4 values per lane, 6 per compute unit): the value is gradient plus
// residual, its top bytes stand in for the codes, the block's first value
// for the scale and half the value for the new residual.
__global__ __launch_bounds__(64) void replica_ef_kernel(gb::PtrTable src, gb::OutTable resid, gb::OutTable codes,
                                                        gb::OutTable scales, float* __restrict__ out) {
  const size_t block = blockIdx.x, e = block * gb::kBlock + 4 * (size_t)threadIdx.x;
  f4 y[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    y[r] = gb::load4(static_cast<const float*>(src.p[r]) + e) + gb::load4(static_cast<const float*>(resid.p[r]) + e);
  }
  f4 a;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const f4 v = y[r];
    const uint32_t w = (gb::fbits(v.x) >> 24) | ((gb::fbits(v.y) >> 24) << 8) | ((gb::fbits(v.z) >> 24) << 16) |
                       ((gb::fbits(v.w) >> 24) << 24);
    if (threadIdx.x == 0u) static_cast<float*>(scales.p[r])[block] = v.x;
    __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(codes.p[r]) + e));
    gb::store4(static_cast<float*>(resid.p[r]) + e, v * 0.5f);
    a = r == 0 ? v : a + v;
  }
  gb::store4(out + e, a);
}

struct Result {
  std::string name;
  double bytes, med_gbs, best_gbs;
};
std::vector<Result> g_results;

template <class F>
void measure(const std::string& name, double bytes, int reps, F launch) {
  hipEvent_t a, b;
  CK(hipEventCreate(&a));
  CK(hipEventCreate(&b));
  launch();
  launch();
  CK(hipGetLastError());
  CK(hipDeviceSynchronize());
  std::vector<float> ms;
  for (int i = 0; i < reps; i++) {
    CK(hipEventRecord(a, nullptr));
    launch();
    CK(hipEventRecord(b, nullptr));
    CK(hipEventSynchronize(b));
    float t = 0.0f;
    CK(hipEventElapsedTime(&t, a, b));
    ms.push_back(t);
  }
  CK(hipGetLastError());
  std::sort(ms.begin(), ms.end());
  const Result r{name, bytes, bytes / (ms[ms.size() / 2] * 1e6), bytes / (ms[0] * 1e6)};
  g_results.push_back(r);
  std::printf("%-28s %12.0f bytes  median %7.1f GB/s  best %7.1f GB/s\n", name.c_str(), bytes, r.med_gbs, r.best_gbs);
  std::fflush(stdout);
  CK(hipEventDestroy(a));
  CK(hipEventDestroy(b));
}

std::vector<std::pair<std::string, double>> g_launch_us;

// Median microseconds per launch of `count` empty launches of `grid`
// workgroups on `s`, issued one by one (graph = false) or replayed from one
// captured graph.
void launch_cost(hipStream_t s, float* sink, unsigned grid, bool graph, int reps) {
  constexpr int count = 153;
  hipGraphExec_t exec = nullptr;
  if (graph) {
    hipGraph_t g;
    CK(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    for (int i = 0; i < count; i++) empty_kernel<<<grid, kThreads, 0, s>>>(sink);
    CK(hipStreamEndCapture(s, &g));
    CK(hipGraphInstantiate(&exec, g, nullptr, nullptr, 0));
    CK(hipGraphDestroy(g));
  }
  auto launch = [&] {
    if (graph) CK(hipGraphLaunch(exec, s));
    else
      for (int i = 0; i < count; i++) empty_kernel<<<grid, kThreads, 0, s>>>(sink);
  };
  hipEvent_t a, b;
  CK(hipEventCreate(&a));
  CK(hipEventCreate(&b));
  launch();
  launch();
  CK(hipGetLastError());
  CK(hipStreamSynchronize(s));
  std::vector<float> ms;
  for (int i = 0; i < reps; i++) {
    CK(hipEventRecord(a, s));
    launch();
    CK(hipEventRecord(b, s));
    CK(hipEventSynchronize(b));
    float t = 0.0f;
    CK(hipEventElapsedTime(&t, a, b));
    ms.push_back(t);
  }
  CK(hipGetLastError());
  std::sort(ms.begin(), ms.end());
  const double us = ms[ms.size() / 2] * 1e3 / count;
  const std::string name = std::string(graph ? "graph_" : "stream_") + std::to_string(grid) + "wg";
  g_launch_us.emplace_back(name, us);
  std::printf("launch %-21s %8.2f us per launch (median of %d x %d)\n", name.c_str(), us, reps, count);
  std::fflush(stdout);
  CK(hipEventDestroy(a));
  CK(hipEventDestroy(b));
  if (exec) CK(hipGraphExecDestroy(exec));
}

}  // namespace

int main(int argc, char** argv) {
  const size_t gib = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 4;
  const int reps = argc > 2 ? std::atoi(argv[2]) : 10;
  if (gib < 1 || gib > 16 || reps < 1 || reps > 1000) {
    std::fprintf(stderr, "usage: gb_ceiling [size_gib 1..16] [reps 1..1000]\n");
    return 2;
  }
  const size_t bytes = gib << 30, nvec = bytes / 16, nval = bytes / 4;
  // five float32 buffers of `bytes` (4 sources and an output), 4 code
  // streams of nval bytes, 4 scale streams
  const size_t nblk = nval / 256;
  // four gradient-like sources; the fifth buffer (the replica's output)
  // starts zeroed and is the zero-data contrast's source
  f4 *buf[5];
  for (int i = 0; i < 5; i++) {
    CK(hipMalloc(&buf[i], bytes));
    if (i < 4) fill_gradient_like<<<4096, kThreads>>>(buf[i], nvec, 0x9E3779B9u * (i + 1));
    else CK(hipMemset(buf[i], 0, bytes));
  }
  CK(hipGetLastError());
  uint8_t* codes;
  float *scales, *sink;
  CK(hipMalloc(&codes, 4 * nval));
  CK(hipMalloc(&scales, 4 * nblk * sizeof(float)));
  CK(hipMalloc(&sink, 256));
  CK(hipDeviceSynchronize());
  std::printf("gb_ceiling: buffers of %zu GiB, %d timed launches per variant\n", gib, reps);

  const double copy_bytes = 2.0 * bytes;
  const std::string sz = std::to_string(gib) + "GiB";
  // grids: nvec / (256 U) workgroups; nvec is a multiple of 2^26, so every grid divides exactly
  measure("copy_u1_" + sz, copy_bytes, reps, [&] { copy_kernel<1, false><<<nvec / kThreads, kThreads>>>(buf[0], buf[1]); });
  measure("copy_u1_fronts_" + sz, copy_bytes, reps, [&] { copy_kernel<1, true><<<nvec / kThreads, kThreads>>>(buf[0], buf[1]); });
  measure("copy_u2_" + sz, copy_bytes, reps, [&] { copy_kernel<2, false><<<nvec / (2 * kThreads), kThreads>>>(buf[0], buf[1]); });
  measure("copy_u4_" + sz, copy_bytes, reps, [&] { copy_kernel<4, false><<<nvec / (4 * kThreads), kThreads>>>(buf[0], buf[1]); });
  measure("copy_u4_fronts_" + sz, copy_bytes, reps, [&] { copy_kernel<4, true><<<nvec / (4 * kThreads), kThreads>>>(buf[0], buf[1]); });
  measure("copy_lds_u1_" + sz, copy_bytes, reps, [&] { copy_lds_kernel<1><<<nvec / kThreads, kThreads>>>(buf[0], buf[1]); });
  measure("copy_lds_u4_" + sz, copy_bytes, reps, [&] { copy_lds_kernel<4><<<nvec / (4 * kThreads), kThreads>>>(buf[0], buf[1]); });
  measure("read_u4_2percu_" + sz, (double)bytes, reps,
          [&] { read_kernel<4><<<nvec / (4 * kThreads), kThreads, gb::kTwoPerCuLds>>>(buf[0], sink); });
  measure("write_u1_" + sz, (double)bytes, reps, [&] { write_kernel<<<nvec / kThreads, kThreads>>>(buf[1], 0x85EBCA6Bu); });
  measure("zeros_copy_u1_" + sz, copy_bytes, reps,
          [&] { copy_kernel<1, false, 1><<<nvec / kThreads, kThreads>>>(buf[4], buf[1]); });
  fill_gradient_like<<<4096, kThreads>>>(buf[1], nvec, 0x9E3779B9u * 2);  // rank 1 of the replica again
  CK(hipGetLastError());
  gb::PtrTable st = {};
  gb::OutTable ct = {}, sct = {};
  for (int r = 0; r < 4; r++) {
    st.p[r] = buf[r];
    ct.p[r] = codes + (size_t)r * nval;
    sct.p[r] = scales + (size_t)r * nblk;
  }
  const double replica_bytes = (double)nval * (16.0 + 4.0 + 16.0 / 256 + 4.0);
  static_assert(gb::fused_fp8_wave(4, (size_t)1 << 28), "the replica's shape is the pass's from 2^28 values");
  measure("fused_fp8_replica_" + sz, replica_bytes, reps, [&] {
    replica_kernel<<<nblk, 64, gb::kFp8WaveLds>>>(st, ct, sct, reinterpret_cast<float*>(buf[4]));
  });
  // the error-feedback pattern: four gradient-like residual buffers more
  f4* res[4];
  gb::OutTable rt = {};
  for (int r = 0; r < 4; r++) {
    CK(hipMalloc(&res[r], bytes));
    fill_gradient_like<<<4096, kThreads>>>(res[r], nvec, 0x85EBCA6Bu * (r + 3));
    rt.p[r] = res[r];
  }
  CK(hipGetLastError());
  const double replica_ef_bytes = (double)nval * (16.0 + 16.0 + 4.0 + 16.0 / 256 + 16.0 + 4.0);
  static_assert(gb::fused_fp8_ef_wave<GB_DTYPE_F32>(4, (size_t)1 << 28), "the replica's shape is the pass's at this size");
  measure("fused_fp8_ef_replica_" + sz, replica_ef_bytes, reps, [&] {
    replica_ef_kernel<<<nblk, 64, gb::fused_fp8_ef_wave_lds<GB_DTYPE_F32>()>>>(st, rt, ct, sct,
                                                                             reinterpret_cast<float*>(buf[4]));
  });
  for (auto& p : res) CK(hipFree(p));

  hipStream_t s;
  CK(hipStreamCreate(&s));
  for (unsigned grid : {1u, 1600u, 25600u}) {
    launch_cost(s, sink, grid, false, reps);
    launch_cost(s, sink, grid, true, reps);
  }
  CK(hipStreamDestroy(s));

  std::printf("{\"median_gbs\": {");
  for (size_t i = 0; i < g_results.size(); i++) {
    std::printf("%s\"%s\": %.1f", i ? ", " : "", g_results[i].name.c_str(), g_results[i].med_gbs);
  }
  std::printf("}, \"launch_us\": {");
  for (size_t i = 0; i < g_launch_us.size(); i++) {
    std::printf("%s\"%s\": %.2f", i ? ", " : "", g_launch_us[i].first.c_str(), g_launch_us[i].second);
  }
  std::printf("}}\n");
  for (auto& p : buf) CK(hipFree(p));
  CK(hipFree(codes));
  CK(hipFree(scales));
  CK(hipFree(sink));
  return 0;
}
