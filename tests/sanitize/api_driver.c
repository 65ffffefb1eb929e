/*
 * api_driver.c — drives the C ABI layer of libgbreduce (gb_api.cpp, built
 * with g++ against the host stand-ins of stub_hip.cpp) under AddressSanitizer
 * and UndefinedBehaviorSanitizer, on a machine without a GPU.  Test
 * infrastructure.  Every pointer is a fabricated address that nothing
 * dereferences; what is checked is the host code: validation, the refusal of
 * overlapping buffers, the planning of launches (how many, with what
 * arguments: the stand-ins abort on a launch the kernels could not take), and
 * the GB_ERR_HIP path when a launch fails at any point of a call.
 *
 * Exit status 0 when every check passes; each failed check prints a line.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gbreduce.h"

void stub_reset(void);
void stub_fail_at(long nth);
long stub_launches(void);
long stub_copies(void);
unsigned long long stub_pinned_base(void);
void stub_sync_fails(int on);
void stub_capturing(int capturing);
long stub_syncs(void);

static int failures, checks;

#define P(a) ((void*)(uintptr_t)(a))
#define F(a) ((float*)(uintptr_t)(a))

static void expect(int got, int want, const char* needle, long launches, const char* what) {
  checks++;
  const char* err = gb_last_error();
  if (got != want || (needle != NULL && strstr(err, needle) == NULL) || (launches >= 0 && stub_launches() != launches)) {
    fprintf(stderr, "FAIL %s: status %d (want %d), %ld launches (want %ld), detail \"%s\" (want \"%s\")\n", what,
            got, want, stub_launches(), launches, err, needle ? needle : "");
    failures++;
  }
}

/* Fabricated device addresses, 256-byte aligned and far apart. */
enum { MB = 1 << 20 };
static uintptr_t dev(int i) { return (uintptr_t)0x100000000ull + (uintptr_t)i * 64 * MB; }

static void validation(void) {
  const void* one[1] = {P(dev(1))};
  stub_reset();
  expect(gb_reduce_sum(F(dev(0)), (const float* const*)one, 0, 10, NULL), GB_ERR_INVALID_ARG, "k = 0", 0, "k = 0");
  expect(gb_reduce_sum(F(dev(0)), (const float* const*)one, 17, 10, NULL), GB_ERR_INVALID_ARG, "k = 17", 0, "k = 17");
  expect(gb_reduce_sum(NULL, (const float* const*)one, 1, 10, NULL), GB_ERR_INVALID_ARG, "dst is NULL", 0, "NULL dst");
  expect(gb_reduce_sum(F(dev(0) + 4), (const float* const*)one, 1, 10, NULL), GB_ERR_MISALIGNED, "dst", 0,
         "misaligned dst");
  expect(gb_reduce_sum(F(dev(0)), (const float* const*)one, 1, GB_MAX_N + 1, NULL), GB_ERR_INVALID_ARG, "GB_MAX_N",
         0, "n too large");
  expect(gb_reduce_sum(NULL, NULL, 1, 0, NULL), GB_OK, NULL, 0, "n = 0");
  expect(gb_decode_accumulate(F(dev(0)), one, NULL, 1, 10, 7, 0, NULL), GB_ERR_UNSUPPORTED, "codec", 0, "codec");
  expect(gb_bucket_allreduce_local(F(dev(0)), (const float* const*)one, 1, 1000, 300, 2, 0, P(dev(2)), MB, NULL),
         GB_ERR_INVALID_ARG, "bucket_elems", 0, "bucket_elems");
  expect(gb_bucket_allreduce_local(F(dev(0)), (const float* const*)one, 1, 1000, 256, 2, 0, P(dev(2)), 100, NULL),
         GB_ERR_WORKSPACE, "needed", 0, "workspace too small");
  /* sizes never wrap */
  checks++;
  if (gb_payload_bytes(GB_CODEC_FP8_E4M3_B256, GB_MAX_N + 1) != 0 ||
      gb_bucket_workspace_bytes(GB_CODEC_BF16, 16, GB_MAX_N, GB_MAX_N) != 16 * 2 * GB_MAX_N) {
    fprintf(stderr, "FAIL size queries at GB_MAX_N\n");
    failures++;
  }
}

static void overlaps(void) {
  const size_t n = 1000; /* 4000 bytes of float32 */
  stub_reset();
  {
    const void* s[2] = {P(dev(0) + 16), P(dev(1))};
    expect(gb_reduce_sum(F(dev(0)), (const float* const*)s, 2, n, NULL), GB_ERR_INVALID_ARG, "dst overlaps srcs[0]",
           0, "dst partly over srcs[0]");
  }
  {
    const void* s[2] = {P(dev(1)), P(dev(0))};
    expect(gb_reduce_sum(F(dev(0)), (const float* const*)s, 2, n, NULL), GB_ERR_INVALID_ARG, "srcs[1]", 0,
           "dst == srcs[1]");
  }
  {
    const void* s[2] = {P(dev(0)), P(dev(0))};
    expect(gb_reduce_sum(F(dev(0)), (const float* const*)s, 2, n, NULL), GB_ERR_INVALID_ARG, "srcs[1]", 0,
           "dst == srcs[0] == srcs[1]");
  }
  {
    const void* s[2] = {P(dev(1)), P(dev(1) + 64)}; /* sources may overlap each other */
    expect(gb_reduce_sum(F(dev(0)), (const float* const*)s, 2, n, NULL), GB_OK, NULL, 1, "overlapping sources");
  }
  stub_reset();
  expect(gb_encode_bf16((uint16_t*)P(dev(0) + 1024), F(dev(0)), n, NULL), GB_ERR_INVALID_ARG, "codes overlaps src",
         0, "bf16 codes over src");
  expect(gb_encode_fp8_e4m3_blockscaled((uint8_t*)P(dev(0)), F(dev(0) + 512), F(dev(1)), n, 0, NULL),
         GB_ERR_INVALID_ARG, "codes overlaps scales", 0, "fp8 codes over scales");
  {
    const void* c[3] = {P(dev(1)), P(dev(2)), P(dev(0) + 2992)};
    expect(gb_decode_accumulate(F(dev(0)), c, NULL, 3, n, GB_CODEC_BF16, 0, NULL), GB_ERR_INVALID_ARG,
           "acc overlaps codes[2]", 0, "acc over a payload");
  }
  {
    const void* s[2] = {P(dev(0)), P(dev(1))};
    expect(gb_bucket_allreduce_local(F(dev(0)), (const float* const*)s, 2, n, 256, 2, 0, P(dev(1) + 2048), MB, NULL),
           GB_ERR_INVALID_ARG, "workspace overlaps srcs[1]", 0, "workspace over a source");
    float* res[2] = {F(dev(3)), F(dev(0) + 256)};
    expect(gb_bucket_allreduce_local_ef(F(dev(0)), (const float* const*)s, res, 2, n, 256, 2, 0, P(dev(4)), MB, NULL),
           GB_ERR_INVALID_ARG, "residuals[1]", 0, "residual over out");
    expect(gb_reduce_encode(F(dev(0)), P(dev(1) + 256), NULL, (const float* const*)s, 2, n, GB_CODEC_BF16, 0, NULL),
           GB_ERR_INVALID_ARG, "codes overlaps srcs[1]", 0, "reduce_encode codes over a source");
  }
  {
    const void* s[2] = {P(dev(0)), P(dev(1) + 16)}; /* float64: 8000 bytes each */
    expect(gb_reduce_typed(P(dev(1)), s, 2, n, GB_DTYPE_F64, GB_OP_SUM, 1, NULL), GB_ERR_INVALID_ARG, "srcs[1]", 0,
           "typed dst over srcs[1]");
  }
  {
    const uintptr_t pin = (uintptr_t)stub_pinned_base();
    expect(gb_encode_staged(GB_CODEC_FP8_E4M3_B256, 0, P(dev(1)), F(dev(2)), P(pin), F(pin + 512), F(dev(0)), n,
                            256, NULL),
           GB_ERR_INVALID_ARG, "codes_host overlaps scales_host", 0, "staged host payload");
  }
  {
    /* a batch: outs[3] overlaps srcs[1 * k + 2] */
    enum { NB = 5, K = 3 };
    void* outs[NB];
    const void* srcs[NB * K];
    size_t ns[NB];
    for (int b = 0; b < NB; b++) {
      outs[b] = P(dev(1 + b));
      ns[b] = n;
      for (int r = 0; r < K; r++) srcs[b * K + r] = P(dev(10 + b * K + r));
    }
    outs[3] = P(dev(10 + 1 * K + 2) + 16);
    expect(gb_bucket_allreduce_local_batch(GB_DTYPE_F32, outs, srcs, ns, NB, K, GB_CODEC_FP8_E4M3_B256, 0, 1,
                                           P(dev(40)), 64 * MB, NULL),
           GB_ERR_INVALID_ARG, "srcs[1 * k + 2]", 0, "batch output over another bucket's source");
  }
}

static void allowed_aliases(void) {
  const size_t n = 5000;
  const void* s[3] = {P(dev(0)), P(dev(1)), P(dev(2))};
  stub_reset();
  expect(gb_reduce_sum(F(dev(0)), (const float* const*)s, 3, n, NULL), GB_OK, NULL, 1, "in place sum");
  expect(gb_bucket_allreduce_local(F(dev(0)), (const float* const*)s, 3, n, 256, 2, 0, P(dev(5)), 4 * MB, NULL),
         GB_OK, NULL, 2, "in place bucket stream");
  expect(gb_reduce_encode(F(dev(0)), P(dev(6)), F(dev(7)), (const float* const*)s, 3, n, GB_CODEC_FP8_E4M3_B256, 1,
                          NULL),
         GB_OK, NULL, 3, "in place island sum");
}

/* The largest batch: 4096 buckets of 16 ranks (65,536 sources), every
 * output its bucket's first source; the overlap check's spans leave their
 * fixed storage for the heap. */
static void largest_batch(void) {
  enum { NB = GB_MAX_BATCH, K = 16 };
  void** outs = malloc(sizeof(void*) * NB);
  const void** srcs = malloc(sizeof(void*) * NB * K);
  size_t* ns = malloc(sizeof(size_t) * NB);
  for (int b = 0; b < NB; b++) {
    ns[b] = 1 + (size_t)(b % 7) * 300;
    for (int r = 0; r < K; r++) srcs[b * K + r] = P(dev(1) + ((size_t)b * K + r) * 64 * 1024);
    outs[b] = (void*)srcs[b * K];
  }
  stub_reset();
  size_t need = gb_bucket_batch_workspace_bytes(GB_CODEC_FP8_E4M3_B256, K, ns, NB);
  int st = gb_bucket_allreduce_local_batch(GB_DTYPE_F32, outs, srcs, ns, NB, K, GB_CODEC_FP8_E4M3_B256, 0, 1,
                                           P(dev(200)), need, NULL);
  expect(st, GB_OK, NULL, -1, "largest batch");
  checks++;
  if (stub_launches() < NB) { /* more than 8 ranks: one bucket at a time, several launches each */
    fprintf(stderr, "FAIL largest batch: %ld launches\n", stub_launches());
    failures++;
  }
  srcs[4000 * K + 9] = (const void*)((uintptr_t)outs[17] + 64); /* one overlap deep in the list */
  stub_reset();
  st = gb_bucket_allreduce_local_batch(GB_DTYPE_F32, outs, srcs, ns, NB, K, GB_CODEC_FP8_E4M3_B256, 0, 1,
                                       P(dev(200)), need, NULL);
  expect(st, GB_ERR_INVALID_ARG, "srcs[4000 * k + 9]", 0, "one overlap among 65,536 sources");
  free(outs);
  free((void*)srcs);
  free(ns);
}

/* A launch that fails at any point of a call: GB_ERR_HIP with the runtime's
 * detail, and no launch after the failed one. */
static void launch_failures(void) {
  const size_t n = 100000;
  const void* s[12];
  float* res[12];
  for (int r = 0; r < 12; r++) {
    s[r] = P(dev(1 + r));
    res[r] = F(dev(20 + r));
  }
  struct {
    const char* name;
    int codec;
    int ef;
  } calls[] = {{"sum", -1, 0}, {"bf16 stream", GB_CODEC_BF16, 0}, {"fp8 stream", GB_CODEC_FP8_E4M3_B256, 0},
               {"fp8 stream with feedback", GB_CODEC_FP8_E4M3_B256, 1}};
  for (size_t c = 0; c < sizeof calls / sizeof calls[0]; c++) {
    /* first the number of launches of the whole call (12 ranks: several) */
    long total;
    int st;
    stub_reset();
#define CALL()                                                                                                     \
  (calls[c].codec < 0                                                                                              \
       ? gb_reduce_sum(F(dev(0)), (const float* const*)s, 12, n, NULL)                                            \
       : calls[c].ef ? gb_bucket_allreduce_local_ef(F(dev(0)), (const float* const*)s, res, 12, n, 4096,           \
                                                    calls[c].codec, 0, P(dev(40)), 64 * MB, NULL)                 \
                     : gb_bucket_allreduce_local(F(dev(0)), (const float* const*)s, 12, n, 4096, calls[c].codec, 0, \
                                                 P(dev(40)), 64 * MB, NULL))
    st = CALL();
    total = stub_launches();
    expect(st, GB_OK, NULL, -1, calls[c].name);
    checks++;
    if (total < 2) {
      fprintf(stderr, "FAIL %s: %ld launches for 12 ranks\n", calls[c].name, total);
      failures++;
    }
    for (long at = 1; at <= total; at++) {
      char what[96];
      snprintf(what, sizeof what, "%s, launch %ld of %ld fails", calls[c].name, at, total);
      stub_reset();
      stub_fail_at(at);
      expect(CALL(), GB_ERR_HIP, "injected failure", at, what);
    }
#undef CALL
  }
  stub_reset();
}

static void staged(void) {
  const uintptr_t pin = (uintptr_t)stub_pinned_base();
  const size_t n = 1 << 20, chunk = 1 << 18;
  stub_reset();
  expect(gb_encode_staged(GB_CODEC_FP8_E4M3_B256, 0, P(dev(1)), F(dev(2)), P(pin), F(pin + 64 * MB), F(dev(0)), n,
                          chunk, NULL),
         GB_OK, NULL, 4, "staged encode");
  checks++;
  if (stub_copies() != 5) { /* 4 chunks of codes and the scales */
    fprintf(stderr, "FAIL staged encode: %ld copies\n", stub_copies());
    failures++;
  }
  const void* ch[2] = {P(pin), P(pin + 8 * MB)};
  const float* sh[2] = {F(pin + 16 * MB), F(pin + 24 * MB)};
  void* cd[2] = {P(dev(3)), P(dev(4))};
  float* sd[2] = {F(dev(5)), F(dev(6))};
  stub_reset();
  expect(gb_decode_accumulate_staged(F(dev(0)), ch, sh, cd, sd, 2, n, chunk, GB_CODEC_FP8_E4M3_B256, 0, NULL), GB_OK,
         NULL, 4, "staged decode");
  expect(gb_decode_accumulate_staged(F(dev(0)), ch, sh, cd, sd, 2, n, chunk, GB_CODEC_FP8_E4M3_B256, 0, NULL), GB_OK,
         NULL, 8, "staged decode again (streams kept)");
  const void* not_pinned[2] = {P(dev(7)), P(pin)};
  expect(gb_decode_accumulate_staged(F(dev(0)), not_pinned, sh, cd, sd, 2, n, chunk, GB_CODEC_FP8_E4M3_B256, 0,
                                     NULL),
         GB_ERR_INVALID_ARG, "not pinned", 8, "pageable host payload");
}

static void expect_syncs(long before, long want, const char* what) {
  checks++;
  if (stub_syncs() - before != want) {
    fprintf(stderr, "FAIL %s: %ld stream waits (want %ld)\n", what, stub_syncs() - before, want);
    failures++;
  }
}

/* Run with GB_DEBUG=1 and GB_TRACE=1 in the environment: a call that
 * enqueued work waits for its stream once; an error the stream reports
 * becomes GB_ERR_HIP; a stream under capture and a refused call are not
 * waited for.  The trace lines go to stderr for the caller to check. */
static void hooks(void) {
  const void* one[1] = {P(dev(1))};
  long before = stub_syncs();
  stub_reset();
  expect(gb_reduce_sum(F(dev(0)), (const float* const*)one, 1, 10, NULL), GB_OK, NULL, 1, "debug: a sum");
  expect_syncs(before, 1, "debug: a sum");
  before = stub_syncs();
  expect(gb_bucket_allreduce_local(F(dev(0)), (const float* const*)one, 1, 1000, 256, GB_CODEC_FP8_E4M3_B256, 0,
                                   P(dev(2)), MB, NULL),
         GB_OK, NULL, 2, "debug: a bucket call");
  expect_syncs(before, 1, "debug: a bucket call");
  stub_sync_fails(1);
  before = stub_syncs();
  expect(gb_reduce_sum(F(dev(0)), (const float* const*)one, 1, 10, NULL), GB_ERR_HIP, "GB_DEBUG", 3,
         "debug: the stream reports an error");
  expect_syncs(before, 1, "debug: the stream reports an error");
  stub_sync_fails(0);
  stub_capturing(1);
  before = stub_syncs();
  expect(gb_reduce_sum(F(dev(0)), (const float* const*)one, 1, 10, NULL), GB_OK, NULL, 4, "debug: under capture");
  expect_syncs(before, 0, "debug: under capture");
  stub_capturing(0);
  before = stub_syncs();
  expect(gb_reduce_sum(F(dev(0)), (const float* const*)one, 0, 10, NULL), GB_ERR_INVALID_ARG, "k = 0", 4,
         "debug: a refused call");
  expect_syncs(before, 0, "debug: a refused call");
}

int main(int argc, char** argv) {
  if (argc > 1 && strcmp(argv[1], "hooks") == 0) {
    hooks();
  } else {
    const long before = stub_syncs();
    validation();
    overlaps();
    allowed_aliases();
    largest_batch();
    launch_failures();
    staged();
    expect_syncs(before, 0, "no GB_DEBUG: no call waits for its stream");
  }
  printf("api_driver: %d checks, %d failed\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
