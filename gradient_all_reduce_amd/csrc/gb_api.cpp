// gb_api.cpp — the C ABI of libgbreduce (include/gbreduce.h): argument
// validation, workspace layout and kernel launch.  Nothing is enqueued unless
// every argument is valid; no call allocates device memory.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "gb_internal.h"

namespace {

thread_local char g_last_error[512] = "";

gb_status fail(gb_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

gb_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return GB_OK;
  return fail(GB_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t nblocks(size_t n) { return (n + GB_BLOCK - 1) / GB_BLOCK; }

size_t code_bytes(int codec, size_t n) {
  switch (codec) {
    case GB_CODEC_NONE: return 4 * n;
    case GB_CODEC_BF16: return 2 * n;
    case GB_CODEC_FP8_E4M3_B256: return n;
    default: return 0;
  }
}

bool known_codec(int codec) {
  return codec == GB_CODEC_NONE || codec == GB_CODEC_BF16 || codec == GB_CODEC_FP8_E4M3_B256;
}
bool known_mode(int mode) { return mode == GB_SCALE_ABSMAX_DIV_448 || mode == GB_SCALE_POW2; }

gb_status check_k(int k, const char* fn) {
  if (k < 1 || k > GB_MAX_K) {
    return fail(GB_ERR_INVALID_ARG, "%s: k = %d is outside 1..%d", fn, k, GB_MAX_K);
  }
  return GB_OK;
}

gb_status check_n(size_t n, const char* fn) {
  if (n > GB_MAX_N) return fail(GB_ERR_INVALID_ARG, "%s: n = %zu exceeds GB_MAX_N = %zu", fn, n, GB_MAX_N);
  return GB_OK;
}

gb_status check_array(const void* p, size_t align, const char* fn, const char* name) {
  if (p == nullptr) return fail(GB_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
  if (!aligned(p, align)) {
    return fail(GB_ERR_MISALIGNED, "%s: %s = %p is not %zu-byte aligned", fn, name, p, align);
  }
  return GB_OK;
}

gb_status check_table(const void* const* table, int k, size_t align, const char* fn, const char* name) {
  if (table == nullptr) return fail(GB_ERR_INVALID_ARG, "%s: %s array is NULL", fn, name);
  for (int r = 0; r < k; r++) {
    char label[64];
    std::snprintf(label, sizeof label, "%s[%d]", name, r);
    gb_status s = check_array(table[r], align, fn, label);
    if (s != GB_OK) return s;
  }
  return GB_OK;
}

// ---------------------------------------------------------------------------
// Overlapping buffers.  Every buffer a call writes (outputs, and the buffers
// it reads and rewrites: residuals, workspaces, staging buffers) must share
// no byte with any other buffer of the call, except where the ABI lets one
// output be one input exactly (out == srcs[0]: same address, same length);
// inputs may overlap one another.  A partial overlap would let one lane's
// store reach the values another lane has still to read.  The spans are
// sorted, so a batch of thousands of buckets costs O(N log N); a call with
// few buffers keeps them in fixed storage and allocates nothing.
// ---------------------------------------------------------------------------
struct Span {
  uintptr_t lo = 0, hi = 0;  // bytes [lo, hi)
  const char* name = "";
  long i = -1, j = -1;  // indices shown with the name, -1 if none
};

class Spans {
 public:
  void add(const void* p, size_t bytes, const char* name, long i = -1, long j = -1) {
    if (p == nullptr || bytes == 0) return;
    Span s;
    s.lo = reinterpret_cast<uintptr_t>(p);
    s.hi = s.lo + bytes;
    s.name = name;
    s.i = i;
    s.j = j;
    if (n_ < kInline) {
      inline_[n_] = s;
    } else {
      if (n_ == kInline) heap_.assign(inline_, inline_ + kInline);
      heap_.push_back(s);
    }
    n_++;
  }
  // An input, left out when it is exactly the output `alias` may be.
  void add_input(const void* p, size_t bytes, const void* alias, const char* name, long i = -1, long j = -1) {
    if (p != nullptr && p == alias) return;
    add(p, bytes, name, i, j);
  }
  Span* data() { return n_ <= kInline ? inline_ : heap_.data(); }
  size_t size() const { return n_; }

 private:
  static constexpr size_t kInline = 48;
  Span inline_[kInline];
  std::vector<Span> heap_;
  size_t n_ = 0;
};

void span_label(const Span& s, char* buf, size_t size) {
  if (s.j >= 0) std::snprintf(buf, size, "%s[%ld * k + %ld]", s.name, s.i, s.j);
  else if (s.i >= 0) std::snprintf(buf, size, "%s[%ld]", s.name, s.i);
  else std::snprintf(buf, size, "%s", s.name);
}

gb_status overlap_error(const char* fn, const Span& a, const Span& b) {
  char la[64], lb[64];
  span_label(a, la, sizeof la);
  span_label(b, lb, sizeof lb);
  return fail(GB_ERR_INVALID_ARG, "%s: %s overlaps %s (bytes %#zx..%#zx and %#zx..%#zx)", fn, la, lb, (size_t)a.lo,
              (size_t)a.hi, (size_t)b.lo, (size_t)b.hi);
}

bool by_start(const Span& a, const Span& b) { return a.lo < b.lo; }

// outs: every buffer the call writes; ins: the buffers it only reads, the
// exactly aliased input already left out.
gb_status check_disjoint(const char* fn, Spans& outs, Spans& ins) {
  Span* o = outs.data();
  Span* in = ins.data();
  const size_t no = outs.size(), ni = ins.size();
  std::sort(o, o + no, by_start);
  size_t far = 0;  // the output reaching furthest so far
  for (size_t a = 1; a < no; a++) {
    if (o[a].lo < o[far].hi) return overlap_error(fn, o[far], o[a]);
    if (o[a].hi > o[far].hi) far = a;
  }
  // the outputs are now disjoint and in order, so their ends increase too:
  // the inputs starting before an output's end only grow from one output to
  // the next, and the one of them reaching furthest decides
  std::sort(in, in + ni, by_start);
  size_t q = 0;
  long reach = -1;
  for (size_t a = 0; a < no; a++) {
    for (; q < ni && in[q].lo < o[a].hi; q++) {
      if (reach < 0 || in[q].hi > in[reach].hi) reach = (long)q;
    }
    if (reach >= 0 && in[reach].hi > o[a].lo) return overlap_error(fn, o[a], in[reach]);
  }
  return GB_OK;
}

// dst against k sources of `bytes` each; dst may be srcs[0].
gb_status check_sum_overlaps(const char* fn, const void* dst, const void* const* srcs, int k, size_t bytes) {
  Spans outs, ins;
  outs.add(dst, bytes, "dst");
  for (int r = 0; r < k; r++) ins.add_input(srcs[r], bytes, r == 0 ? dst : nullptr, "srcs", r);
  return check_disjoint(fn, outs, ins);
}

// An output of out_bytes against k payloads (code arrays of code_bytes, and
// for fp8 scale arrays of scale_bytes).
gb_status check_decode_overlaps(const char* fn, const void* out, size_t out_bytes, const void* const* codes,
                                const float* const* scales, int k, size_t code_bytes, size_t scale_bytes) {
  Spans outs, ins;
  outs.add(out, out_bytes, "acc");
  for (int r = 0; r < k; r++) {
    ins.add(codes[r], code_bytes, "codes", r);
    if (scales != nullptr) ins.add(scales[r], scale_bytes, "scales", r);
  }
  return check_disjoint(fn, outs, ins);
}

// An encoder's payload (and error-feedback residual) against its source.
gb_status check_encode_overlaps(const char* fn, const void* codes, size_t code_bytes, const void* scales,
                                size_t scale_bytes, const void* residual, size_t n, const void* src, size_t src_bytes) {
  Spans outs, ins;
  outs.add(codes, code_bytes, "codes");
  outs.add(scales, scale_bytes, "scales");
  outs.add(residual, 4 * n, "residual");
  ins.add(src, src_bytes, "src");
  return check_disjoint(fn, outs, ins);
}

size_t dtype_size(int dtype) {
  switch (dtype) {
    case GB_DTYPE_F16:
    case GB_DTYPE_BF16: return 2;
    case GB_DTYPE_F64:
    case GB_DTYPE_I64: return 8;
    case GB_DTYPE_I8:
    case GB_DTYPE_U8: return 1;
    default: return 4;
  }
}

// ---------------------------------------------------------------------------
// More ranks than one launch reads (kLaunchRanks).  Every reduction here is a
// left fold over ranks, so it continues across launches from the stored
// partial result: a later launch reads the output as its first operand (or
// accumulates into it) and folds the next ranks in.  Each step of the fold
// rounds exactly as in one launch (the partial is a value of the output's
// type), so the bits are the same.  AVG divides only in the last launch.
// ---------------------------------------------------------------------------
constexpr int kR = gb::kLaunchRanks;

int group_size(int k, int g) { return k - g < kR ? k - g : kR; }

gb::PtrTable slice(const void* const* table, int first, int count) {
  gb::PtrTable t = {};
  for (int r = 0; r < count; r++) t.p[r] = table[first + r];
  return t;
}

// dst = [dst +] srcs[0] + ... + srcs[k-1], float32, in rank order.
hipError_t sum_groups(float* dst, const void* const* srcs, int k, size_t n, bool accumulate, hipStream_t st) {
  hipError_t e = hipSuccess;
  for (int g = 0; g < k && e == hipSuccess; g += kR) {
    const int m = group_size(k, g);
    e = gb::launch_reduce_sum(dst, slice(srcs, g, m), m, n, accumulate || g > 0, st);
  }
  return e;
}

// SUM / AVG / MAX / MIN over k ranks of element type dtype into dst: the
// first launch takes kR ranks, each further one dst and up to kR - 1 ranks.
hipError_t op_groups(void* dst, const void* const* srcs, int k, size_t n, int dtype, int op, int divisor,
                     hipStream_t st) {
  auto launch = [&](const gb::PtrTable& t, int m, int o) {
    return dtype == GB_DTYPE_F32 ? gb::launch_reduce_op(static_cast<float*>(dst), t, m, n, o, divisor, st)
                                 : gb::launch_reduce_typed(dst, t, m, n, dtype, o, divisor, st);
  };
  if (k <= kR) return launch(slice(srcs, 0, k), k, op);
  const int fold_op = op == GB_OP_AVG ? GB_OP_SUM : op;
  hipError_t e = launch(slice(srcs, 0, kR), kR, fold_op);
  for (int g = kR; g < k && e == hipSuccess; g += kR - 1) {
    const int m = k - g < kR - 1 ? k - g : kR - 1;
    gb::PtrTable t = {};
    t.p[0] = dst;
    for (int r = 0; r < m; r++) t.p[1 + r] = srcs[g + r];
    e = launch(t, m + 1, g + m == k ? op : fold_op);
  }
  return e;
}

// Decode k payloads and add them in rank order into the float32 acc (or,
// with k <= kR, into dst of dtype, rounded once).
hipError_t decode_groups(void* acc, const void* const* codes, const float* const* scales, int k, size_t n,
                         int codec, bool accumulate, int dtype, hipStream_t st) {
  if (codec == GB_CODEC_NONE) return sum_groups(static_cast<float*>(acc), codes, k, n, accumulate, st);
  hipError_t e = hipSuccess;
  for (int g = 0; g < k && e == hipSuccess; g += kR) {
    const int m = group_size(k, g);
    const bool a = accumulate || g > 0;
    if (codec == GB_CODEC_BF16) {
      e = gb::launch_decode_bf16(acc, slice(codes, g, m), m, n, a, dtype, st);
    } else {
      e = gb::launch_decode_fp8(acc, slice(codes, g, m), slice(reinterpret_cast<const void* const*>(scales), g, m), m,
                                n, a, dtype, st);
    }
  }
  return e;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// ---------------------------------------------------------------------------
// Per-device state of the staged (pipelined) calls: two copy streams, at the
// default priority, so that consecutive chunks' copies go to two DMA queues
// and the fixed cost of one copy overlaps the transfer of the other, and the
// events that order them against the caller's stream.  Created on a device's
// first staged call and kept until the process ends.  A staged call holds
// the device's lock while it enqueues, so calls from several host threads
// interleave whole, never chunk by chunk.
// ---------------------------------------------------------------------------
constexpr int kCopyStreams = 2;
struct StagingContext {
  std::mutex mu;
  bool ready = false;
  hipStream_t copy[kCopyStreams] = {};
  hipEvent_t ev_copy[kCopyStreams] = {};  // copy stream -> compute stream
  hipEvent_t ev_compute = nullptr;        // compute stream -> copy stream
};
constexpr int kMaxDevices = 64;
StagingContext g_staging[kMaxDevices];

gb_status staging_context(const char* fn, StagingContext** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GB_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(GB_ERR_HIP, "%s: device %d out of range", fn, dev);
  *out = &g_staging[dev];
  return GB_OK;
}

// Creates the context's streams and events; call with c->mu held.  On a
// failure whatever was created is destroyed again, so a later call starts
// from nothing.
gb_status staging_ready(const char* fn, StagingContext* c) {
  if (c->ready) return GB_OK;
  hipError_t e = hipEventCreateWithFlags(&c->ev_compute, hipEventDisableTiming);
  for (int i = 0; i < kCopyStreams && e == hipSuccess; i++) {
    e = hipStreamCreateWithFlags(&c->copy[i], hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_copy[i], hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    for (int i = 0; i < kCopyStreams; i++) {
      if (c->ev_copy[i] != nullptr) (void)hipEventDestroy(c->ev_copy[i]);
      if (c->copy[i] != nullptr) (void)hipStreamDestroy(c->copy[i]);
      c->ev_copy[i] = nullptr;
      c->copy[i] = nullptr;
    }
    if (c->ev_compute != nullptr) (void)hipEventDestroy(c->ev_compute);
    c->ev_compute = nullptr;
    return fail(GB_ERR_HIP, "%s: creating the copy streams: %s", fn, hipGetErrorString(e));
  }
  c->ready = true;
  return GB_OK;
}

// Host buffers of the staged calls must be pinned (page-locked and mapped
// for the device), so the copies are asynchronous DMA.
gb_status check_pinned(const void* p, size_t align, const char* fn, const char* name) {
  gb_status s = check_array(p, align, fn, name);
  if (s != GB_OK) return s;
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) (void)hipGetLastError();  // an unknown host pointer leaves an error behind
  if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
    return fail(GB_ERR_INVALID_ARG, "%s: %s = %p is not pinned host memory", fn, name, p);
  }
  return GB_OK;
}

// Element types the codec calls read and write (README "Bridge compression"
// applies to floating-point tensors).
bool codec_dtype(int dtype) {
  return dtype == GB_DTYPE_F32 || dtype == GB_DTYPE_F16 || dtype == GB_DTYPE_BF16 || dtype == GB_DTYPE_F64;
}

size_t code_size(int codec) { return codec == GB_CODEC_BF16 ? 2 : (codec == GB_CODEC_FP8_E4M3_B256 ? 1 : 4); }

}  // namespace

extern "C" {

int gb_version(void) { return GB_VERSION; }

const char* gb_status_string(int status) {
  switch (status) {
    case GB_OK: return "GB_OK";
    case GB_ERR_INVALID_ARG: return "GB_ERR_INVALID_ARG";
    case GB_ERR_MISALIGNED: return "GB_ERR_MISALIGNED";
    case GB_ERR_UNSUPPORTED: return "GB_ERR_UNSUPPORTED";
    case GB_ERR_WORKSPACE: return "GB_ERR_WORKSPACE";
    case GB_ERR_HIP: return "GB_ERR_HIP";
    default: return "unknown status";
  }
}

const char* gb_last_error(void) { return g_last_error; }

size_t gb_payload_bytes(int codec, size_t n) {
  if (!known_codec(codec) || n > GB_MAX_N) return 0;
  return code_bytes(codec, n) + (codec == GB_CODEC_FP8_E4M3_B256 ? 4 * nblocks(n) : 0);
}

gb_status gb_bucket_workspace_layout(int codec, int k, size_t n, size_t bucket_elems,
                                     size_t* codes_stride, size_t* scales_offset,
                                     size_t* scales_stride, size_t* total) {
  const char* fn = "gb_bucket_workspace_layout";
  if (!known_codec(codec)) return fail(GB_ERR_UNSUPPORTED, "%s: unknown codec %d", fn, codec);
  gb_status s = check_k(k, fn);
  if (s != GB_OK) return s;
  if ((s = check_n(n, fn)) != GB_OK) return s;
  if (bucket_elems == 0 || bucket_elems % GB_BLOCK != 0) {
    return fail(GB_ERR_INVALID_ARG, "%s: bucket_elems = %zu is not a positive multiple of %d", fn,
                bucket_elems, GB_BLOCK);
  }
  if (!codes_stride || !scales_offset || !scales_stride || !total) {
    return fail(GB_ERR_INVALID_ARG, "%s: an output pointer is NULL", fn);
  }
  if (codec == GB_CODEC_NONE) {
    *codes_stride = *scales_offset = *scales_stride = *total = 0;
    return GB_OK;
  }
  const size_t cs = round_up(code_bytes(codec, n), 256);
  const size_t ss = codec == GB_CODEC_FP8_E4M3_B256 ? round_up(4 * nblocks(n), 256) : 0;
  *codes_stride = cs;
  *scales_offset = (size_t)k * cs;
  *scales_stride = ss;
  *total = (size_t)k * (cs + ss);
  return GB_OK;
}

size_t gb_bucket_workspace_bytes(int codec, int k, size_t n, size_t bucket_elems) {
  size_t cs, so, ss, total;
  char saved[sizeof g_last_error];
  std::memcpy(saved, g_last_error, sizeof saved);
  gb_status s = gb_bucket_workspace_layout(codec, k, n, bucket_elems, &cs, &so, &ss, &total);
  std::memcpy(g_last_error, saved, sizeof saved);  // a size query reports no failure
  return s == GB_OK ? total : 0;
}

gb_status gb_reduce_sum(float* dst, const float* const* srcs, int k, size_t n, void* stream) {
  return gb::traced_call("gb_reduce_sum", stream, k, n, -1, [&](const char* fn) -> gb_status {
    gb_status s = check_k(k, fn);
    if (s != GB_OK) return s;
    if (n > GB_MAX_N) return check_n(n, fn);
    if (n == 0) return GB_OK;
    if ((s = check_array(dst, GB_ALIGN, fn, "dst")) != GB_OK) return s;
    const void* const* sp = reinterpret_cast<const void* const*>(srcs);
    if ((s = check_table(sp, k, GB_ALIGN, fn, "srcs")) != GB_OK) return s;
    if ((s = check_sum_overlaps(fn, dst, sp, k, 4 * n)) != GB_OK) return s;
    return from_hip(sum_groups(dst, sp, k, n, false, as_stream(stream)), fn);
  });
}

gb_status gb_reduce(float* dst, const float* const* srcs, int k, size_t n, int op, int divisor, void* stream) {
  return gb::traced_call("gb_reduce", stream, k, n, -1, [&](const char* fn) -> gb_status {
    if (op != GB_OP_SUM && op != GB_OP_AVG && op != GB_OP_MAX && op != GB_OP_MIN) {
      return fail(GB_ERR_UNSUPPORTED, "%s: unknown op %d", fn, op);
    }
    if (op == GB_OP_AVG && (divisor < 1 || divisor > (1 << 24))) {
      return fail(GB_ERR_INVALID_ARG, "%s: AVG divisor %d is outside 1..2^24", fn, divisor);
    }
    gb_status s = check_k(k, fn);
    if (s != GB_OK) return s;
    if (n > GB_MAX_N) return check_n(n, fn);
    if (n == 0) return GB_OK;
    if ((s = check_array(dst, GB_ALIGN, fn, "dst")) != GB_OK) return s;
    const void* const* sp = reinterpret_cast<const void* const*>(srcs);
    if ((s = check_table(sp, k, GB_ALIGN, fn, "srcs")) != GB_OK) return s;
    if ((s = check_sum_overlaps(fn, dst, sp, k, 4 * n)) != GB_OK) return s;
    return from_hip(op_groups(dst, sp, k, n, GB_DTYPE_F32, op, divisor, as_stream(stream)), fn);
  });
}

gb_status gb_reduce_typed(void* dst, const void* const* srcs, int k, size_t n, int dtype, int op, int divisor,
                          void* stream) {
  return gb::traced_call("gb_reduce_typed", stream, k, n, -1, [&](const char* fn) -> gb_status {
    if (dtype < GB_DTYPE_F32 || dtype > GB_DTYPE_I64) {
      return fail(GB_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
    }
    if (op != GB_OP_SUM && op != GB_OP_AVG && op != GB_OP_MAX && op != GB_OP_MIN) {
      return fail(GB_ERR_UNSUPPORTED, "%s: unknown op %d", fn, op);
    }
    if (op == GB_OP_AVG && dtype >= GB_DTYPE_I8) {
      return fail(GB_ERR_UNSUPPORTED, "%s: AVG needs a floating-point dtype", fn);
    }
    if (op == GB_OP_AVG && (divisor < 1 || divisor > (1 << 24))) {
      return fail(GB_ERR_INVALID_ARG, "%s: AVG divisor %d is outside 1..2^24", fn, divisor);
    }
    gb_status s = check_k(k, fn);
    if (s != GB_OK) return s;
    if (n > GB_MAX_N) return check_n(n, fn);
    if (n == 0) return GB_OK;
    if ((s = check_array(dst, GB_ALIGN, fn, "dst")) != GB_OK) return s;
    if ((s = check_table(srcs, k, GB_ALIGN, fn, "srcs")) != GB_OK) return s;
    if ((s = check_sum_overlaps(fn, dst, srcs, k, dtype_size(dtype) * n)) != GB_OK) return s;
    return from_hip(op_groups(dst, srcs, k, n, dtype, op, divisor, as_stream(stream)), fn);
  });
}

gb_status gb_encode_bf16(uint16_t* codes, const float* src, size_t n, void* stream) {
  return gb::traced_call("gb_encode_bf16", stream, -1, n, -1, [&](const char* fn) -> gb_status {
    if (n > GB_MAX_N) return check_n(n, fn);
    if (n == 0) return GB_OK;
    gb_status s;
    if ((s = check_array(codes, GB_ALIGN, fn, "codes")) != GB_OK) return s;
    if ((s = check_array(src, GB_ALIGN, fn, "src")) != GB_OK) return s;
    if ((s = check_encode_overlaps(fn, codes, 2 * n, nullptr, 0, nullptr, n, src, 4 * n)) != GB_OK) return s;
    return from_hip(gb::launch_encode_bf16(codes, src, n, GB_DTYPE_F32, as_stream(stream)), fn);
  });
}

gb_status gb_encode_fp8_e4m3_blockscaled(uint8_t* codes, float* scales, const float* src, size_t n,
                                         int scale_mode, void* stream) {
  return gb::traced_call("gb_encode_fp8_e4m3_blockscaled", stream, -1, n, -1, [&](const char* fn) -> gb_status {
    if (!known_mode(scale_mode)) return fail(GB_ERR_UNSUPPORTED, "%s: unknown scale mode %d", fn, scale_mode);
    if (n > GB_MAX_N) return check_n(n, fn);
    if (n == 0) return GB_OK;
    gb_status s;
    if ((s = check_array(codes, GB_ALIGN, fn, "codes")) != GB_OK) return s;
    if ((s = check_array(scales, 4, fn, "scales")) != GB_OK) return s;
    if ((s = check_array(src, GB_ALIGN, fn, "src")) != GB_OK) return s;
    if ((s = check_encode_overlaps(fn, codes, n, scales, 4 * nblocks(n), nullptr, n, src, 4 * n)) != GB_OK) return s;
    return from_hip(gb::launch_encode_fp8(codes, scales, src, n, scale_mode, GB_DTYPE_F32, as_stream(stream)), fn);
  });
}

gb_status gb_decode_accumulate(float* acc, const void* const* codes, const float* const* scales, int k,
                               size_t n, int codec, int accumulate, void* stream) {
  return gb::traced_call("gb_decode_accumulate", stream, k, n, codec, [&](const char* fn) -> gb_status {
    if (!known_codec(codec)) return fail(GB_ERR_UNSUPPORTED, "%s: unknown codec %d", fn, codec);
    gb_status s = check_k(k, fn);
    if (s != GB_OK) return s;
    if (accumulate != 0 && accumulate != 1) {
      return fail(GB_ERR_INVALID_ARG, "%s: accumulate = %d is not 0 or 1", fn, accumulate);
    }
    if (n > GB_MAX_N) return check_n(n, fn);
    if (n == 0) return GB_OK;
    if ((s = check_array(acc, GB_ALIGN, fn, "acc")) != GB_OK) return s;
    if ((s = check_table(codes, k, GB_ALIGN, fn, "codes")) != GB_OK) return s;
    if (codec == GB_CODEC_FP8_E4M3_B256 &&
        (s = check_table(reinterpret_cast<const void* const*>(scales), k, 4, fn, "scales")) != GB_OK) {
      return s;
    }
    if ((s = check_decode_overlaps(fn, acc, 4 * n, codes, codec == GB_CODEC_FP8_E4M3_B256 ? scales : nullptr, k,
                                   code_bytes(codec, n), 4 * nblocks(n))) != GB_OK) {
      return s;
    }
    return from_hip(decode_groups(acc, codes, scales, k, n, codec, accumulate != 0, GB_DTYPE_F32, as_stream(stream)),
                    fn);
  });
}

gb_status gb_encode(int codec, int dtype, void* codes, float* scales, const void* src, size_t n, int scale_mode,
                    void* stream) {
  return gb::traced_call("gb_encode", stream, -1, n, codec, [&](const char* fn) -> gb_status {
    if (codec != GB_CODEC_BF16 && codec != GB_CODEC_FP8_E4M3_B256) {
      return fail(GB_ERR_UNSUPPORTED, "%s: codec %d is not bf16 or fp8", fn, codec);
    }
    if (!codec_dtype(dtype)) return fail(GB_ERR_UNSUPPORTED, "%s: dtype %d is not a floating-point type", fn, dtype);
    const bool fp8 = codec == GB_CODEC_FP8_E4M3_B256;
    if (fp8 && !known_mode(scale_mode)) return fail(GB_ERR_UNSUPPORTED, "%s: unknown scale mode %d", fn, scale_mode);
    if (n > GB_MAX_N) return check_n(n, fn);
    if (n == 0) return GB_OK;
    gb_status s;
    if ((s = check_array(codes, GB_ALIGN, fn, "codes")) != GB_OK) return s;
    if (fp8 && (s = check_array(scales, 4, fn, "scales")) != GB_OK) return s;
    if ((s = check_array(src, GB_ALIGN, fn, "src")) != GB_OK) return s;
    if ((s = check_encode_overlaps(fn, codes, code_bytes(codec, n), fp8 ? scales : nullptr, 4 * nblocks(n), nullptr, n,
                                   src, dtype_size(dtype) * n)) != GB_OK) {
      return s;
    }
    hipStream_t st = as_stream(stream);
    if (fp8) {
      return from_hip(gb::launch_encode_fp8(static_cast<uint8_t*>(codes), scales, src, n, scale_mode, dtype, st), fn);
    }
    return from_hip(gb::launch_encode_bf16(static_cast<uint16_t*>(codes), src, n, dtype, st), fn);
  });
}

gb_status gb_decode_sum(int dtype, void* dst, const void* const* codes, const float* const* scales, int k,
                        size_t n, int codec, void* stream) {
  return gb::traced_call("gb_decode_sum", stream, k, n, codec, [&](const char* fn) -> gb_status {
    if (!known_codec(codec)) return fail(GB_ERR_UNSUPPORTED, "%s: unknown codec %d", fn, codec);
    if (!codec_dtype(dtype)) return fail(GB_ERR_UNSUPPORTED, "%s: dtype %d is not a floating-point type", fn, dtype);
    if (codec == GB_CODEC_NONE && dtype != GB_DTYPE_F32) {
      return fail(GB_ERR_UNSUPPORTED, "%s: uncompressed payloads are float32; reduce other types exactly with "
                  "gb_reduce_typed", fn);
    }
    gb_status s = check_k(k, fn);
    if (s != GB_OK) return s;
    if (k > kR && dtype != GB_DTYPE_F32) {
      return fail(GB_ERR_INVALID_ARG, "%s: k = %d: a %s total is rounded once from float32, which holds up to %d "
                  "payloads per call; sum more into a float32 buffer", fn, k, "non-float32", kR);
    }
    if (n > GB_MAX_N) return check_n(n, fn);
    if (n == 0) return GB_OK;
    if ((s = check_array(dst, GB_ALIGN, fn, "dst")) != GB_OK) return s;
    if ((s = check_table(codes, k, GB_ALIGN, fn, "codes")) != GB_OK) return s;
    if (codec == GB_CODEC_FP8_E4M3_B256 &&
        (s = check_table(reinterpret_cast<const void* const*>(scales), k, 4, fn, "scales")) != GB_OK) {
      return s;
    }
    if ((s = check_decode_overlaps(fn, dst, dtype_size(dtype) * n, codes,
                                   codec == GB_CODEC_FP8_E4M3_B256 ? scales : nullptr, k, code_bytes(codec, n),
                                   4 * nblocks(n))) != GB_OK) {
      return s;
    }
    return from_hip(decode_groups(dst, codes, scales, k, n, codec, false, dtype, as_stream(stream)), fn);
  });
}

gb_status gb_reduce_encode(float* sum, void* codes, float* scales, const float* const* srcs, int k, size_t n,
                           int codec, int scale_mode, void* stream) {
  return gb::traced_call("gb_reduce_encode", stream, k, n, codec, [&](const char* fn) -> gb_status {
    if (codec != GB_CODEC_BF16 && codec != GB_CODEC_FP8_E4M3_B256) {
      return fail(GB_ERR_UNSUPPORTED, "%s: codec %d is not bf16 or fp8", fn, codec);
    }
    const bool fp8 = codec == GB_CODEC_FP8_E4M3_B256;
    if (fp8 && !known_mode(scale_mode)) return fail(GB_ERR_UNSUPPORTED, "%s: unknown scale mode %d", fn, scale_mode);
    gb_status s = check_k(k, fn);
    if (s != GB_OK) return s;
    if (k > kR && sum == nullptr) {
      return fail(GB_ERR_INVALID_ARG, "%s: k = %d: more than %d sources are summed into sum first, which is NULL", fn,
                  k, kR);
    }
    if (n > GB_MAX_N) return check_n(n, fn);
    if (n == 0) return GB_OK;
    if ((s = check_array(codes, GB_ALIGN, fn, "codes")) != GB_OK) return s;
    if (fp8 && (s = check_array(scales, 4, fn, "scales")) != GB_OK) return s;
    if (sum != nullptr && (s = check_array(sum, GB_ALIGN, fn, "sum")) != GB_OK) return s;
    const void* const* sp = reinterpret_cast<const void* const*>(srcs);
    if ((s = check_table(sp, k, GB_ALIGN, fn, "srcs")) != GB_OK) return s;
    {
      Spans outs, ins;
      outs.add(sum, 4 * n, "sum");
      outs.add(codes, code_bytes(codec, n), "codes");
      if (fp8) outs.add(scales, 4 * nblocks(n), "scales");
      for (int r = 0; r < k; r++) ins.add_input(sp[r], 4 * n, r == 0 ? sum : nullptr, "srcs", r);
      if ((s = check_disjoint(fn, outs, ins)) != GB_OK) return s;
    }
    hipStream_t st = as_stream(stream);
    hipError_t e;
    if (k <= kR) {
      const gb::PtrTable t = slice(sp, 0, k);
      e = fp8 ? gb::launch_reduce_encode_fp8(sum, static_cast<uint8_t*>(codes), scales, t, k, n, scale_mode, st)
              : gb::launch_reduce_encode_bf16(sum, static_cast<uint16_t*>(codes), t, k, n, st);
    } else {
      // the rank-order sum first (further launches continue the fold), then its payload
      e = sum_groups(sum, sp, k, n, false, st);
      if (e == hipSuccess) {
        e = fp8 ? gb::launch_encode_fp8(static_cast<uint8_t*>(codes), scales, sum, n, scale_mode, GB_DTYPE_F32, st)
                : gb::launch_encode_bf16(static_cast<uint16_t*>(codes), sum, n, GB_DTYPE_F32, st);
      }
    }
    return from_hip(e, fn);
  });
}

gb_status gb_encode_staged(int codec, int scale_mode, void* codes_dev, float* scales_dev, void* codes_host,
                           float* scales_host, const float* src, size_t n, size_t chunk_elems, void* stream) {
  return gb::traced_call("gb_encode_staged", stream, -1, n, codec, [&](const char* fn) -> gb_status {
    if (codec != GB_CODEC_BF16 && codec != GB_CODEC_FP8_E4M3_B256) {
      return fail(GB_ERR_UNSUPPORTED, "%s: codec %d is not bf16 or fp8", fn, codec);
    }
    const bool fp8 = codec == GB_CODEC_FP8_E4M3_B256;
    if (fp8 && !known_mode(scale_mode)) return fail(GB_ERR_UNSUPPORTED, "%s: unknown scale mode %d", fn, scale_mode);
    if (chunk_elems == 0 || chunk_elems % GB_BLOCK != 0) {
      return fail(GB_ERR_INVALID_ARG, "%s: chunk_elems = %zu is not a positive multiple of %d", fn, chunk_elems,
                  GB_BLOCK);
    }
    if (n > GB_MAX_N) return check_n(n, fn);
    if (n == 0) return GB_OK;
    gb_status s;
    if ((s = check_array(src, GB_ALIGN, fn, "src")) != GB_OK) return s;
    if ((s = check_array(codes_dev, GB_ALIGN, fn, "codes_dev")) != GB_OK) return s;
    if ((s = check_pinned(codes_host, 4, fn, "codes_host")) != GB_OK) return s;
    if (fp8) {
      if ((s = check_array(scales_dev, 4, fn, "scales_dev")) != GB_OK) return s;
      if ((s = check_pinned(scales_host, 4, fn, "scales_host")) != GB_OK) return s;
    }
    {
      Spans outs, ins;
      const size_t cbytes = code_bytes(codec, n), sbytes = fp8 ? 4 * nblocks(n) : 0;
      outs.add(codes_dev, cbytes, "codes_dev");
      outs.add(codes_host, cbytes, "codes_host");
      outs.add(fp8 ? scales_dev : nullptr, sbytes, "scales_dev");
      outs.add(fp8 ? scales_host : nullptr, sbytes, "scales_host");
      ins.add(src, 4 * n, "src");
      if ((s = check_disjoint(fn, outs, ins)) != GB_OK) return s;
    }
    StagingContext* c;
    if ((s = staging_context(fn, &c)) != GB_OK) return s;
    std::lock_guard<std::mutex> lock(c->mu);
    if ((s = staging_ready(fn, c)) != GB_OK) return s;
    hipStream_t st = as_stream(stream);
    const size_t cb = code_size(codec);
    char* cd = static_cast<char*>(codes_dev);
    char* ch = static_cast<char*>(codes_host);
    hipError_t e = hipSuccess;
    size_t chunk = 0;
    for (size_t o = 0, l = 0; o < n && e == hipSuccess; o += l, chunk++) {
      l = n - o < chunk_elems ? n - o : chunk_elems;
      hipStream_t cs = c->copy[chunk % kCopyStreams];
      e = fp8 ? gb::launch_encode_fp8(reinterpret_cast<uint8_t*>(cd + o), scales_dev + o / GB_BLOCK, src + o, l,
                                      scale_mode, GB_DTYPE_F32, st)
              : gb::launch_encode_bf16(reinterpret_cast<uint16_t*>(cd + 2 * o), src + o, l, GB_DTYPE_F32, st);
      if (e == hipSuccess) e = hipEventRecord(c->ev_compute, st);
      if (e == hipSuccess) e = hipStreamWaitEvent(cs, c->ev_compute, 0);
      if (e == hipSuccess) e = hipMemcpyAsync(ch + cb * o, cd + cb * o, cb * l, hipMemcpyDeviceToHost, cs);
    }
    // the scales (4 bytes per 256 values) go in one copy once all are written
    if (e == hipSuccess && fp8) {
      const size_t cs_last = (chunk - 1) % kCopyStreams;
      e = hipMemcpyAsync(scales_host, scales_dev, 4 * ((n + GB_BLOCK - 1) / GB_BLOCK), hipMemcpyDeviceToHost,
                         c->copy[cs_last]);
    }
    for (int i = 0; i < kCopyStreams && e == hipSuccess; i++) {
      e = hipEventRecord(c->ev_copy[i], c->copy[i]);
      if (e == hipSuccess) e = hipStreamWaitEvent(st, c->ev_copy[i], 0);
    }
    return from_hip(e, fn);
  });
}

gb_status gb_decode_accumulate_staged(float* acc, const void* const* codes_host, const float* const* scales_host,
                                      void* const* codes_dev, float* const* scales_dev, int k, size_t n,
                                      size_t chunk_elems, int codec, int accumulate, void* stream) {
  return gb::traced_call("gb_decode_accumulate_staged", stream, k, n, codec, [&](const char* fn) -> gb_status {
    if (!known_codec(codec)) return fail(GB_ERR_UNSUPPORTED, "%s: unknown codec %d", fn, codec);
    gb_status s = check_k(k, fn);
    if (s != GB_OK) return s;
    if (accumulate != 0 && accumulate != 1) {
      return fail(GB_ERR_INVALID_ARG, "%s: accumulate = %d is not 0 or 1", fn, accumulate);
    }
    if (chunk_elems == 0 || chunk_elems % GB_BLOCK != 0) {
      return fail(GB_ERR_INVALID_ARG, "%s: chunk_elems = %zu is not a positive multiple of %d", fn, chunk_elems,
                  GB_BLOCK);
    }
    if (n > GB_MAX_N) return check_n(n, fn);
    if (n == 0) return GB_OK;
    const bool fp8 = codec == GB_CODEC_FP8_E4M3_B256;
    if ((s = check_array(acc, GB_ALIGN, fn, "acc")) != GB_OK) return s;
    if (codes_host == nullptr || codes_dev == nullptr || (fp8 && (scales_host == nullptr || scales_dev == nullptr))) {
      return fail(GB_ERR_INVALID_ARG, "%s: a pointer array is NULL", fn);
    }
    for (int r = 0; r < k; r++) {
      char name[32];
      std::snprintf(name, sizeof name, "codes_host[%d]", r);
      if ((s = check_pinned(codes_host[r], 4, fn, name)) != GB_OK) return s;
      std::snprintf(name, sizeof name, "codes_dev[%d]", r);
      if ((s = check_array(codes_dev[r], GB_ALIGN, fn, name)) != GB_OK) return s;
      if (fp8) {
        std::snprintf(name, sizeof name, "scales_host[%d]", r);
        if ((s = check_pinned(scales_host[r], 4, fn, name)) != GB_OK) return s;
        std::snprintf(name, sizeof name, "scales_dev[%d]", r);
        if ((s = check_array(scales_dev[r], 4, fn, name)) != GB_OK) return s;
      }
    }
    {
      Spans outs, ins;
      const size_t cbytes = code_bytes(codec, n), sbytes = 4 * nblocks(n);
      outs.add(acc, 4 * n, "acc");
      for (int r = 0; r < k; r++) {
        outs.add(codes_dev[r], cbytes, "codes_dev", r);
        ins.add(codes_host[r], cbytes, "codes_host", r);
        if (fp8) {
          outs.add(scales_dev[r], sbytes, "scales_dev", r);
          ins.add(scales_host[r], sbytes, "scales_host", r);
        }
      }
      if ((s = check_disjoint(fn, outs, ins)) != GB_OK) return s;
    }
    StagingContext* c;
    if ((s = staging_context(fn, &c)) != GB_OK) return s;
    std::lock_guard<std::mutex> lock(c->mu);
    if ((s = staging_ready(fn, c)) != GB_OK) return s;
    hipStream_t st = as_stream(stream);
    const size_t cb = code_size(codec);
    // copies into the device staging buffers start after the caller's earlier
    // work on `stream`, which may still read them
    hipError_t e = hipEventRecord(c->ev_compute, st);
    for (int i = 0; i < kCopyStreams && e == hipSuccess; i++) e = hipStreamWaitEvent(c->copy[i], c->ev_compute, 0);
    // every rank's scales (4 bytes per 256 values) first, in one copy each on
    // the first copy stream, ahead of chunk 0, which the compute stream waits for
    for (int r = 0; r < k && e == hipSuccess && fp8; r++) {
      e = hipMemcpyAsync(scales_dev[r], scales_host[r], 4 * ((n + GB_BLOCK - 1) / GB_BLOCK), hipMemcpyHostToDevice,
                         c->copy[0]);
    }
    size_t chunk = 0;
    for (size_t o = 0, l = 0; o < n && e == hipSuccess; o += l, chunk++) {
      l = n - o < chunk_elems ? n - o : chunk_elems;
      const int ci = (int)(chunk % kCopyStreams);
      const void* cp[GB_MAX_K];
      const float* sp[GB_MAX_K];
      for (int r = 0; r < k && e == hipSuccess; r++) {
        char* dst = static_cast<char*>(codes_dev[r]) + cb * o;
        e = hipMemcpyAsync(dst, static_cast<const char*>(codes_host[r]) + cb * o, cb * l, hipMemcpyHostToDevice,
                           c->copy[ci]);
        cp[r] = dst;
        sp[r] = fp8 ? scales_dev[r] + o / GB_BLOCK : nullptr;
      }
      if (e == hipSuccess) e = hipEventRecord(c->ev_copy[ci], c->copy[ci]);
      if (e == hipSuccess) e = hipStreamWaitEvent(st, c->ev_copy[ci], 0);
      if (e != hipSuccess) break;
      e = decode_groups(acc + o, cp, sp, k, l, codec, accumulate != 0, GB_DTYPE_F32, st);
    }
    return from_hip(e, fn);
  });
}

}  // extern "C"

namespace {

// The workspace of a bucket-stream call: at least `need` bytes, 256-byte
// aligned (unused, and may be NULL, for codec NONE).
gb_status check_workspace(const char* fn, int codec, const void* workspace, size_t workspace_bytes, size_t need) {
  if (codec == GB_CODEC_NONE) return GB_OK;
  if (workspace == nullptr || workspace_bytes < need) {
    return fail(GB_ERR_WORKSPACE, "%s: workspace %p of %zu bytes, %zu needed", fn, workspace, workspace_bytes, need);
  }
  if (!aligned(workspace, 256)) {
    return fail(GB_ERR_MISALIGNED, "%s: workspace = %p is not 256-byte aligned", fn, workspace);
  }
  return GB_OK;
}

// Validation shared by the two bucket-stream calls; on success fills the
// workspace layout and the source table.
gb_status check_bucket(const char* fn, void* out, const void* const* srcs, int k, size_t n,
                       size_t bucket_elems, int codec, int scale_mode, void* workspace, size_t workspace_bytes,
                       size_t* cs, size_t* so, size_t* ss) {
  if (!known_codec(codec)) return fail(GB_ERR_UNSUPPORTED, "%s: unknown codec %d", fn, codec);
  if (codec == GB_CODEC_FP8_E4M3_B256 && !known_mode(scale_mode)) {
    return fail(GB_ERR_UNSUPPORTED, "%s: unknown scale mode %d", fn, scale_mode);
  }
  size_t need;
  gb_status s = gb_bucket_workspace_layout(codec, k, n, bucket_elems, cs, so, ss, &need);
  if (s != GB_OK) {
    // re-label the failure with this function's name (from a copy: fail()
    // writes the buffer the message is read from)
    char msg[sizeof g_last_error];
    std::snprintf(msg, sizeof msg, "%s", g_last_error + std::strlen("gb_bucket_workspace_layout: "));
    return fail(s, "%s: %s", fn, msg);
  }
  if (n == 0) return GB_OK;
  if ((s = check_array(out, GB_ALIGN, fn, "out")) != GB_OK) return s;
  if ((s = check_table(srcs, k, GB_ALIGN, fn, "srcs")) != GB_OK) return s;
  return check_workspace(fn, codec, workspace, workspace_bytes, need);
}

// A single-buffer bucket stream: out (esize bytes per value, may be
// srcs[0]), the k residuals and the workspace's k payloads (cs + ss bytes
// each) against the k sources.
gb_status check_bucket_overlaps(const char* fn, const void* out, const void* const* srcs, float* const* residuals,
                                int k, size_t n, size_t esize, int codec, const void* workspace, size_t cs, size_t ss) {
  Spans outs, ins;
  outs.add(out, esize * n, "out");
  if (codec != GB_CODEC_NONE) outs.add(workspace, (size_t)k * (cs + ss), "workspace");
  for (int r = 0; r < k; r++) {
    if (residuals != nullptr) outs.add(residuals[r], 4 * n, "residuals", r);
    ins.add_input(srcs[r], esize * n, r == 0 ? out : nullptr, "srcs", r);
  }
  return check_disjoint(fn, outs, ins);
}

// The bucket stream over the whole buffer (all buckets start on block
// boundaries, so one launch covers them; rank r's payload lands where a
// whole-buffer encode would put it).  The first kLaunchRanks ranks go through
// the fused pass (encode, decode, add; with error feedback when residuals is
// not NULL); the remaining ranks are encoded one by one into the workspace
// and their payloads decoded and added in rank order.  Without a codec: the
// exact SUM of the element type.
hipError_t bucket_groups(void* out, const void* const* srcs, float* const* residuals, int k, size_t n, int codec,
                         int mode, int dtype, char* codes0, size_t cs, char* scales0, size_t ss, hipStream_t st) {
  if (codec == GB_CODEC_NONE) {
    return dtype == GB_DTYPE_F32 ? sum_groups(static_cast<float*>(out), srcs, k, n, false, st)
                                 : op_groups(out, srcs, k, n, dtype, GB_OP_SUM, 1, st);
  }
  const bool bf16 = codec == GB_CODEC_BF16;
  void* code[GB_MAX_K];
  float* scale[GB_MAX_K];
  for (int r = 0; r < k; r++) {
    code[r] = codes0 + (size_t)r * cs;
    scale[r] = reinterpret_cast<float*>(scales0 + (size_t)r * ss);
  }
  const int m = k < kR ? k : kR;
  const gb::PtrTable t = slice(srcs, 0, m);
  hipError_t e;
  if (residuals != nullptr && bf16) {
    e = gb::launch_fused_bf16_ef(out, t, residuals, reinterpret_cast<uint16_t* const*>(code), m, n, dtype, st);
  } else if (residuals != nullptr) {
    e = gb::launch_fused_fp8_ef(out, t, residuals, reinterpret_cast<uint8_t* const*>(code), scale, m, n, mode, dtype,
                                st);
  } else if (bf16) {
    e = gb::launch_fused_bf16(out, t, reinterpret_cast<uint16_t* const*>(code), m, n, dtype, st);
  } else {
    e = gb::launch_fused_fp8(out, t, reinterpret_cast<uint8_t* const*>(code), scale, m, n, mode, dtype, st);
  }
  // more than kR ranks: float32 gradients only (checked by the callers)
  for (int r = kR; r < k && e == hipSuccess; r++) {
    const void* x = srcs[r];
    if (residuals != nullptr) {
      e = bf16 ? gb::launch_encode_bf16_ef(static_cast<uint16_t*>(code[r]), residuals[r], x, n, GB_DTYPE_F32, st)
               : gb::launch_encode_fp8_ef(static_cast<uint8_t*>(code[r]), scale[r], residuals[r], x, n, mode,
                                          GB_DTYPE_F32, st);
    } else {
      e = bf16 ? gb::launch_encode_bf16(static_cast<uint16_t*>(code[r]), x, n, GB_DTYPE_F32, st)
               : gb::launch_encode_fp8(static_cast<uint8_t*>(code[r]), scale[r], x, n, mode, GB_DTYPE_F32, st);
    }
  }
  if (k > kR && e == hipSuccess) {
    e = decode_groups(out, const_cast<const void* const*>(code + kR), const_cast<const float* const*>(scale + kR),
                      k - kR, n, codec, true, GB_DTYPE_F32, st);
  }
  return e;
}

}  // namespace

namespace gb {

gb_status fail_status(gb_status s, const char* msg) { return fail(s, "%s", msg); }

namespace {

bool env_on(const char* name) {
  const char* v = std::getenv(name);
  return v != nullptr && *v != '\0' && std::strcmp(v, "0") != 0;
}

struct Hooks {
  bool trace, debug;
};

const Hooks& hooks() {
  static const Hooks h{env_on("GB_TRACE"), env_on("GB_DEBUG")};
  return h;
}

}  // namespace

bool call_hooks_on() {
  const Hooks& h = hooks();
  return h.trace || h.debug;
}

gb_status finish_call(const char* fn, void* stream, int k, size_t n, int codec, gb_status s, double host_us) {
  const Hooks& h = hooks();
  const char* note = "";
  if (h.debug && s == GB_OK) {
    const hipStream_t st = as_stream(stream);
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(st, &capture);
    if (e == hipSuccess && capture != hipStreamCaptureStatusNone) {
      note = " (stream under capture: not waited for)";
    } else {
      if (e == hipSuccess) e = hipStreamSynchronize(st);
      if (e != hipSuccess) {
        s = fail(GB_ERR_HIP, "%s: GB_DEBUG: the stream reported HIP error %d (%s) after the call", fn, (int)e,
                 hipGetErrorString(e));
      }
    }
  }
  if (h.trace) {
    char args[96] = "";
    int used = 0;
    if (k >= 0) used += std::snprintf(args + used, sizeof args - used, " k=%d", k);
    if (n != kNoSize) used += std::snprintf(args + used, sizeof args - used, " n=%zu", n);
    if (codec >= 0) std::snprintf(args + used, sizeof args - used, " codec=%d", codec);
    std::fprintf(stderr, "gbreduce: %s%s stream=%p -> %s%s%s%s (%.1f us on the host)\n", fn, args, stream,
                 gb_status_string(s), s != GB_OK ? ": " : "", s != GB_OK ? g_last_error : "", note, host_us);
    std::fflush(stderr);
  }
  return s;
}

gb_status bucket_allreduce_local(const char* fn, float* out, const float* const* srcs, int k, size_t n,
                                 size_t bucket_elems, int codec, int scale_mode, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  size_t cs, so, ss;
  const void* const* sp = reinterpret_cast<const void* const*>(srcs);
  gb_status s = check_bucket(fn, out, sp, k, n, bucket_elems, codec, scale_mode, workspace, workspace_bytes, &cs,
                             &so, &ss);
  if (s != GB_OK || n == 0) return s;
  if ((s = check_bucket_overlaps(fn, out, sp, nullptr, k, n, 4, codec, workspace, cs, ss)) != GB_OK) return s;
  // One launch covers every bucket: a partly idle GPU at the end of each
  // bucket is avoided, and the result equals one call per bucket bit for bit.
  char* ws = static_cast<char*>(workspace);
  return from_hip(bucket_groups(out, sp, nullptr, k, n, codec, scale_mode, GB_DTYPE_F32, ws, cs, ws + so, ss,
                                as_stream(stream)),
                  fn);
}

}  // namespace gb

extern "C" {

gb_status gb_bucket_allreduce_local(float* out, const float* const* srcs, int k, size_t n,
                                    size_t bucket_elems, int codec, int scale_mode, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return gb::traced_call("gb_bucket_allreduce_local", stream, k, n, codec, [&](const char* fn) {
    return gb::bucket_allreduce_local(fn, out, srcs, k, n, bucket_elems, codec, scale_mode, workspace,
                                      workspace_bytes, stream);
  });
}

gb_status gb_bucket_allreduce_local_typed(int dtype, void* out, const void* const* srcs, int k, size_t n,
                                          size_t bucket_elems, int codec, int scale_mode, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  return gb::traced_call("gb_bucket_allreduce_local_typed", stream, k, n, codec, [&](const char* fn) -> gb_status {
    if (!codec_dtype(dtype)) return fail(GB_ERR_UNSUPPORTED, "%s: dtype %d is not a floating-point type", fn, dtype);
    size_t cs, so, ss;
    gb_status s = check_bucket(fn, out, srcs, k, n, bucket_elems, codec, scale_mode, workspace, workspace_bytes, &cs,
                               &so, &ss);
    if (s != GB_OK) return s;
    if (k > kR && dtype != GB_DTYPE_F32 && codec != GB_CODEC_NONE) {
      return fail(GB_ERR_INVALID_ARG, "%s: k = %d: a compressed non-float32 total is rounded once from float32, "
                  "which holds up to %d ranks per call", fn, k, kR);
    }
    if (n == 0) return GB_OK;
    s = check_bucket_overlaps(fn, out, srcs, nullptr, k, n, dtype_size(dtype), codec, workspace, cs, ss);
    if (s != GB_OK) {
      return s;
    }
    char* ws = static_cast<char*>(workspace);
    return from_hip(bucket_groups(out, srcs, nullptr, k, n, codec, scale_mode, dtype, ws, cs, ws + so, ss,
                                  as_stream(stream)),
                    fn);
  });
}

}  // extern "C"

namespace {

// The sizes of a batch: 1..GB_MAX_BATCH buckets of at most GB_MAX_N values
// whose sizes, each rounded up to a multiple of GB_BLOCK, add up to at most
// GB_MAX_N (the workspace's virtual buffer); *total receives that sum.
gb_status check_batch_sizes(const char* fn, const size_t* ns, int nbuckets, size_t* total) {
  if (nbuckets < 1 || nbuckets > GB_MAX_BATCH) {
    return fail(GB_ERR_INVALID_ARG, "%s: nbuckets = %d is outside 1..%d", fn, nbuckets, GB_MAX_BATCH);
  }
  if (ns == nullptr) return fail(GB_ERR_INVALID_ARG, "%s: ns is NULL", fn);
  size_t t = 0;
  for (int b = 0; b < nbuckets; b++) {
    if (ns[b] > GB_MAX_N) {
      return fail(GB_ERR_INVALID_ARG, "%s: ns[%d] = %zu exceeds GB_MAX_N = %zu", fn, b, ns[b], GB_MAX_N);
    }
    t += round_up(ns[b], GB_BLOCK);
    if (t > GB_MAX_N) {
      return fail(GB_ERR_INVALID_ARG, "%s: the bucket sizes, each rounded up to a multiple of %d, exceed GB_MAX_N",
                  fn, GB_BLOCK);
    }
  }
  *total = t;
  return GB_OK;
}

}  // namespace

extern "C" {

size_t gb_bucket_batch_workspace_bytes(int codec, int k, const size_t* ns, int nbuckets) {
  char saved[sizeof g_last_error];
  std::memcpy(saved, g_last_error, sizeof saved);
  size_t total = 0, cs, so, ss, bytes = 0;
  gb_status s = check_batch_sizes("gb_bucket_batch_workspace_bytes", ns, nbuckets, &total);
  if (s == GB_OK) s = gb_bucket_workspace_layout(codec, k, total, GB_BLOCK, &cs, &so, &ss, &bytes);
  std::memcpy(g_last_error, saved, sizeof saved);  // a size query reports no failure
  return s == GB_OK ? bytes : 0;
}

}  // extern "C"

namespace {

// The batched bucket stream, with error feedback when residuals is not NULL
// (a host array of nbuckets * k residual pointers, bucket-major).
gb_status bucket_batch(const char* fn, int dtype, void* const* outs, const void* const* srcs,
                       float* const* residuals, const size_t* ns, int nbuckets, int k, int codec, int scale_mode,
                       int divisor, void* workspace, size_t workspace_bytes, void* stream) {
  const bool ef = residuals != nullptr;
  if (!codec_dtype(dtype)) return fail(GB_ERR_UNSUPPORTED, "%s: dtype %d is not a floating-point type", fn, dtype);
  if (!known_codec(codec)) return fail(GB_ERR_UNSUPPORTED, "%s: unknown codec %d", fn, codec);
  if (ef && codec == GB_CODEC_NONE) {
    return fail(GB_ERR_UNSUPPORTED, "%s: error feedback needs a lossy codec (bf16 or fp8)", fn);
  }
  if (codec == GB_CODEC_FP8_E4M3_B256 && !known_mode(scale_mode)) {
    return fail(GB_ERR_UNSUPPORTED, "%s: unknown scale mode %d", fn, scale_mode);
  }
  if (divisor < 1 || divisor > (1 << 24)) {
    return fail(GB_ERR_INVALID_ARG, "%s: divisor %d is outside 1..2^24", fn, divisor);
  }
  gb_status s = check_k(k, fn);
  if (s != GB_OK) return s;
  if (k > kR && dtype != GB_DTYPE_F32 && codec != GB_CODEC_NONE) {
    return fail(GB_ERR_INVALID_ARG, "%s: k = %d: a compressed non-float32 total is rounded once from float32, "
                "which holds up to %d ranks per call", fn, k, kR);
  }
  size_t total;
  if ((s = check_batch_sizes(fn, ns, nbuckets, &total)) != GB_OK) return s;
  if (total == 0) return GB_OK;
  if (outs == nullptr || srcs == nullptr) return fail(GB_ERR_INVALID_ARG, "%s: outs or srcs is NULL", fn);
  for (int b = 0; b < nbuckets; b++) {
    if (ns[b] == 0) continue;
    char name[48];
    std::snprintf(name, sizeof name, "outs[%d]", b);
    if ((s = check_array(outs[b], GB_ALIGN, fn, name)) != GB_OK) return s;
    std::snprintf(name, sizeof name, "srcs[%d * k + r]", b);
    if ((s = check_table(srcs + (size_t)b * k, k, GB_ALIGN, fn, name)) != GB_OK) return s;
    if (ef) {
      std::snprintf(name, sizeof name, "residuals[%d * k + r]", b);
      const void* const* rp = reinterpret_cast<const void* const*>(residuals + (size_t)b * k);
      if ((s = check_table(rp, k, GB_ALIGN, fn, name)) != GB_OK) return s;
    }
  }
  size_t cs = 0, so = 0, ss = 0, need = 0;
  if ((s = gb_bucket_workspace_layout(codec, k, total, GB_BLOCK, &cs, &so, &ss, &need)) != GB_OK) return s;
  if ((s = check_workspace(fn, codec, workspace, workspace_bytes, need)) != GB_OK) return s;
  {
    // every bucket's output and residuals, and the workspace, against each
    // other and against every source (outs[b] may be srcs[b * k])
    const size_t esize = dtype_size(dtype);
    Spans written, read;
    if (codec != GB_CODEC_NONE) written.add(workspace, need, "workspace");
    for (int b = 0; b < nbuckets; b++) {
      if (ns[b] == 0) continue;
      written.add(outs[b], esize * ns[b], "outs", b);
      for (int r = 0; r < k; r++) {
        const size_t i = (size_t)b * k + r;
        if (ef) written.add(residuals[i], 4 * ns[b], "residuals", b, r);
        read.add_input(srcs[i], esize * ns[b], r == 0 ? outs[b] : nullptr, "srcs", b, r);
      }
    }
    if ((s = check_disjoint(fn, written, read)) != GB_OK) return s;
  }
  hipStream_t st = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  const size_t csz = code_size(codec);
  hipError_t e = hipSuccess;
  // AVG of a compressed total: the decode-and-add, then the division, fused
  // for float32 totals; other types divide their total in a second pass
  auto divide = [&](void* out, size_t n) {
    const void* one[1] = {out};
    return op_groups(out, one, 1, n, dtype, GB_OP_AVG, divisor, st);
  };
  size_t o = 0;  // the bucket's first value in the workspace's virtual buffer
  if (codec == GB_CODEC_NONE) {
    // the exact SUM (or AVG) of the type, one bucket at a time
    for (int b = 0; b < nbuckets && e == hipSuccess; b++) {
      if (ns[b] == 0) continue;
      e = op_groups(outs[b], srcs + (size_t)b * k, k, ns[b], dtype, divisor == 1 ? GB_OP_SUM : GB_OP_AVG, divisor,
                    st);
    }
    return from_hip(e, fn);
  }
  if (k > kR) {
    // one bucket at a time, exactly as the single-buffer calls (float32 only)
    for (int b = 0; b < nbuckets && e == hipSuccess; b++) {
      if (ns[b] == 0) continue;
      e = bucket_groups(outs[b], srcs + (size_t)b * k, ef ? residuals + (size_t)b * k : nullptr, k, ns[b], codec,
                        scale_mode, dtype, ws + o * csz, cs, ws + so + 4 * (o / GB_BLOCK), ss, st);
      if (e == hipSuccess && divisor != 1) e = divide(outs[b], ns[b]);
      o += round_up(ns[b], GB_BLOCK);
    }
    return from_hip(e, fn);
  }
  const int fused_divisor = dtype == GB_DTYPE_F32 ? divisor : 1;
  // several buckets per launch, as many as the table and one grid hold
  gb::BucketBatch t = {};
  gb::BucketBatchEf te = {};
  const uint32_t cap = (uint32_t)(ef ? gb::kBatchBucketsEf : gb::kBatchBuckets);
  uint32_t count = 0;
  size_t groups = 0;
  auto flush = [&]() {
    if (count == 0 || e != hipSuccess) return;
    if (ef) {
      te.count = count;
      e = codec == GB_CODEC_BF16 ? gb::launch_fused_bf16_ef_batch(te, k, dtype, fused_divisor, st)
                                 : gb::launch_fused_fp8_ef_batch(te, k, scale_mode, dtype, fused_divisor, st);
      te = gb::BucketBatchEf{};
    } else {
      t.count = count;
      e = codec == GB_CODEC_BF16 ? gb::launch_fused_bf16_batch(t, k, dtype, fused_divisor, st)
                                 : gb::launch_fused_fp8_batch(t, k, scale_mode, dtype, fused_divisor, st);
      t = gb::BucketBatch{};
    }
    count = 0;
    groups = 0;
  };
  for (int b = 0; b < nbuckets && e == hipSuccess; b++) {
    if (ns[b] == 0) continue;
    const size_t g = gb::batch_groups(codec, ns[b]);
    if (count == cap || groups + g > gb::kMaxGrid) flush();
    const uint32_t i = count++;
    for (int r = 0; r < k; r++) {
      const void* x = srcs[(size_t)b * k + r];
      void* c = ws + (size_t)r * cs + o * csz;
      float* sc = reinterpret_cast<float*>(ws + so + (size_t)r * ss + 4 * (o / GB_BLOCK));
      if (ef) {
        te.src[i][r] = x;
        te.codes[i][r] = c;
        te.scales[i][r] = sc;
        te.resid[i][r] = residuals[(size_t)b * k + r];
      } else {
        t.src[i][r] = x;
        t.codes[i][r] = c;
        t.scales[i][r] = sc;
      }
    }
    if (ef) {
      te.n[i] = ns[b];
      te.out[i] = outs[b];
    } else {
      t.n[i] = ns[b];
      t.out[i] = outs[b];
    }
    groups += g;
    o += round_up(ns[b], GB_BLOCK);
  }
  flush();
  if (fused_divisor != divisor) {
    for (int b = 0; b < nbuckets && e == hipSuccess; b++) {
      if (ns[b] != 0) e = divide(outs[b], ns[b]);
    }
  }
  return from_hip(e, fn);
}

}  // namespace

extern "C" {

gb_status gb_bucket_allreduce_local_batch(int dtype, void* const* outs, const void* const* srcs, const size_t* ns,
                                          int nbuckets, int k, int codec, int scale_mode, int divisor,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  return gb::traced_call("gb_bucket_allreduce_local_batch", stream, k, gb::kNoSize, codec, [&](const char* fn) {
    return bucket_batch(fn, dtype, outs, srcs, nullptr, ns, nbuckets, k, codec, scale_mode, divisor, workspace,
                        workspace_bytes, stream);
  });
}

gb_status gb_bucket_allreduce_local_batch_ef(int dtype, void* const* outs, const void* const* srcs,
                                             float* const* residuals, const size_t* ns, int nbuckets, int k,
                                             int codec, int scale_mode, int divisor, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  return gb::traced_call("gb_bucket_allreduce_local_batch_ef", stream, k, gb::kNoSize, codec, [&](const char* fn) {
    if (residuals == nullptr) return fail(GB_ERR_INVALID_ARG, "%s: residuals is NULL", fn);
    return bucket_batch(fn, dtype, outs, srcs, residuals, ns, nbuckets, k, codec, scale_mode, divisor, workspace,
                        workspace_bytes, stream);
  });
}

gb_status gb_encode_bf16_ef(uint16_t* codes, float* residual, const float* src, size_t n, void* stream) {
  return gb::traced_call("gb_encode_bf16_ef", stream, -1, n, -1, [&](const char* fn) -> gb_status {
    if (n > GB_MAX_N) return check_n(n, fn);
    if (n == 0) return GB_OK;
    gb_status s;
    if ((s = check_array(codes, GB_ALIGN, fn, "codes")) != GB_OK) return s;
    if ((s = check_array(residual, GB_ALIGN, fn, "residual")) != GB_OK) return s;
    if ((s = check_array(src, GB_ALIGN, fn, "src")) != GB_OK) return s;
    if ((s = check_encode_overlaps(fn, codes, 2 * n, nullptr, 0, residual, n, src, 4 * n)) != GB_OK) return s;
    return from_hip(gb::launch_encode_bf16_ef(codes, residual, src, n, GB_DTYPE_F32, as_stream(stream)), fn);
  });
}

gb_status gb_encode_fp8_e4m3_blockscaled_ef(uint8_t* codes, float* scales, float* residual, const float* src,
                                            size_t n, int scale_mode, void* stream) {
  return gb::traced_call("gb_encode_fp8_e4m3_blockscaled_ef", stream, -1, n, -1, [&](const char* fn) -> gb_status {
    if (!known_mode(scale_mode)) return fail(GB_ERR_UNSUPPORTED, "%s: unknown scale mode %d", fn, scale_mode);
    if (n > GB_MAX_N) return check_n(n, fn);
    if (n == 0) return GB_OK;
    gb_status s;
    if ((s = check_array(codes, GB_ALIGN, fn, "codes")) != GB_OK) return s;
    if ((s = check_array(scales, 4, fn, "scales")) != GB_OK) return s;
    if ((s = check_array(residual, GB_ALIGN, fn, "residual")) != GB_OK) return s;
    if ((s = check_array(src, GB_ALIGN, fn, "src")) != GB_OK) return s;
    if ((s = check_encode_overlaps(fn, codes, n, scales, 4 * nblocks(n), residual, n, src, 4 * n)) != GB_OK) return s;
    return from_hip(gb::launch_encode_fp8_ef(codes, scales, residual, src, n, scale_mode, GB_DTYPE_F32,
                                             as_stream(stream)),
                    fn);
  });
}

gb_status gb_bucket_allreduce_local_ef(float* out, const float* const* srcs, float* const* residuals, int k,
                                       size_t n, size_t bucket_elems, int codec, int scale_mode, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return gb::traced_call("gb_bucket_allreduce_local_ef", stream, k, n, codec, [&](const char* fn) -> gb_status {
    if (codec == GB_CODEC_NONE) {
      return fail(GB_ERR_UNSUPPORTED, "%s: error feedback needs a lossy codec (bf16 or fp8)", fn);
    }
    size_t cs, so, ss;
    const void* const* sp = reinterpret_cast<const void* const*>(srcs);
    gb_status s = check_bucket(fn, out, sp, k, n, bucket_elems, codec, scale_mode, workspace, workspace_bytes, &cs,
                               &so, &ss);
    if (s != GB_OK || n == 0) return s;
    if ((s = check_table(reinterpret_cast<const void* const*>(residuals), k, GB_ALIGN, fn, "residuals")) != GB_OK) {
      return s;
    }
    if ((s = check_bucket_overlaps(fn, out, sp, residuals, k, n, 4, codec, workspace, cs, ss)) != GB_OK) return s;
    char* ws = static_cast<char*>(workspace);
    return from_hip(bucket_groups(out, sp, residuals, k, n, codec, scale_mode, GB_DTYPE_F32, ws, cs, ws + so, ss,
                                  as_stream(stream)),
                    fn);
  });
}

gb_status gb_encode_ef(int codec, int dtype, void* codes, float* scales, float* residual, const void* src, size_t n,
                       int scale_mode, void* stream) {
  return gb::traced_call("gb_encode_ef", stream, -1, n, codec, [&](const char* fn) -> gb_status {
    if (codec != GB_CODEC_BF16 && codec != GB_CODEC_FP8_E4M3_B256) {
      return fail(GB_ERR_UNSUPPORTED, "%s: codec %d is not bf16 or fp8", fn, codec);
    }
    if (!codec_dtype(dtype)) return fail(GB_ERR_UNSUPPORTED, "%s: dtype %d is not a floating-point type", fn, dtype);
    const bool fp8 = codec == GB_CODEC_FP8_E4M3_B256;
    if (fp8 && !known_mode(scale_mode)) return fail(GB_ERR_UNSUPPORTED, "%s: unknown scale mode %d", fn, scale_mode);
    if (n > GB_MAX_N) return check_n(n, fn);
    if (n == 0) return GB_OK;
    gb_status s;
    if ((s = check_array(codes, GB_ALIGN, fn, "codes")) != GB_OK) return s;
    if (fp8 && (s = check_array(scales, 4, fn, "scales")) != GB_OK) return s;
    if ((s = check_array(residual, GB_ALIGN, fn, "residual")) != GB_OK) return s;
    if ((s = check_array(src, GB_ALIGN, fn, "src")) != GB_OK) return s;
    if ((s = check_encode_overlaps(fn, codes, code_bytes(codec, n), fp8 ? scales : nullptr, 4 * nblocks(n), residual, n,
                                   src, dtype_size(dtype) * n)) != GB_OK) {
      return s;
    }
    hipStream_t st = as_stream(stream);
    if (fp8) {
      return from_hip(gb::launch_encode_fp8_ef(static_cast<uint8_t*>(codes), scales, residual, src, n, scale_mode,
                                               dtype, st),
                      fn);
    }
    return from_hip(gb::launch_encode_bf16_ef(static_cast<uint16_t*>(codes), residual, src, n, dtype, st), fn);
  });
}

gb_status gb_bucket_allreduce_local_ef_typed(int dtype, void* out, const void* const* srcs, float* const* residuals,
                                             int k, size_t n, size_t bucket_elems, int codec, int scale_mode,
                                             void* workspace, size_t workspace_bytes, void* stream) {
  return gb::traced_call("gb_bucket_allreduce_local_ef_typed", stream, k, n, codec, [&](const char* fn) -> gb_status {
    if (!codec_dtype(dtype)) return fail(GB_ERR_UNSUPPORTED, "%s: dtype %d is not a floating-point type", fn, dtype);
    if (codec == GB_CODEC_NONE) {
      return fail(GB_ERR_UNSUPPORTED, "%s: error feedback needs a lossy codec (bf16 or fp8)", fn);
    }
    size_t cs, so, ss;
    gb_status s = check_bucket(fn, out, srcs, k, n, bucket_elems, codec, scale_mode, workspace, workspace_bytes, &cs,
                               &so, &ss);
    if (s != GB_OK) return s;
    if (k > kR && dtype != GB_DTYPE_F32) {
      return fail(GB_ERR_INVALID_ARG, "%s: k = %d: a compressed non-float32 total is rounded once from float32, "
                  "which holds up to %d ranks per call", fn, k, kR);
    }
    if (n == 0) return GB_OK;
    if ((s = check_table(reinterpret_cast<const void* const*>(residuals), k, GB_ALIGN, fn, "residuals")) != GB_OK) {
      return s;
    }
    if ((s = check_bucket_overlaps(fn, out, srcs, residuals, k, n, dtype_size(dtype), codec, workspace, cs, ss)) !=
        GB_OK) {
      return s;
    }
    char* ws = static_cast<char*>(workspace);
    return from_hip(bucket_groups(out, srcs, residuals, k, n, codec, scale_mode, dtype, ws, cs, ws + so, ss,
                                  as_stream(stream)),
                    fn);
  });
}

}  // extern "C"
