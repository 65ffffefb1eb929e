/*
 * oracle_driver.c — runs every function of the CPU oracle (oracle/gb_oracle.c)
 * under AddressSanitizer and UndefinedBehaviorSanitizer, on sizes around the
 * 256-value block (empty, ragged, several blocks, several buckets) and on
 * inputs that mix gradient-like values with every special value the codecs
 * meet: signed zeros, subnormals, the largest floats, infinities, NaNs with
 * payloads.  Test infrastructure.  Values are checked elsewhere (the pins);
 * here a few identities catch a run that went wrong, and the sanitizers
 * catch any out-of-bounds access, integer overflow, bad shift or
 * out-of-range conversion.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gb_oracle.h"

static int failures, checks;

static uint32_t rng_state = 12345u;
static uint32_t next_u32(void) { /* xorshift32 */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 17;
  rng_state ^= rng_state << 5;
  return rng_state;
}

static float bits_f(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static const uint32_t kSpecial[] = {0x00000000u, 0x80000000u, 0x00000001u, 0x807FFFFFu, 0x00800000u, 0x7F7FFFFFu,
                                    0xFF7FFFFFu, 0x7F800000u, 0xFF800000u, 0x7FC00000u, 0xFFC0ABCDu, 0x7FA00001u,
                                    0x43E00000u, 0xC3E80000u, 0x3F800000u, 0x33800000u};

static void fill(float* x, size_t n) {
  for (size_t i = 0; i < n; i++) {
    uint32_t r = next_u32();
    if (r % 50 == 0) x[i] = bits_f(kSpecial[(r >> 8) % (sizeof kSpecial / sizeof kSpecial[0])]);
    else x[i] = ((float)(int32_t)(r >> 8) / 8388608.0f) * 1e-3f;
  }
}

static void check(int ok, const char* what, size_t n) {
  checks++;
  if (!ok) {
    fprintf(stderr, "FAIL %s (n = %zu)\n", what, n);
    failures++;
  }
}

static void run(size_t n, int k) {
  const size_t nb = (n + 255) / 256, m = n ? n : 1, mb = nb ? nb : 1;
  float* x[8];
  float* res[8];
  void* codes[8];
  float* scales[8];
  for (int r = 0; r < k; r++) {
    x[r] = malloc(4 * m);
    res[r] = malloc(4 * m);
    codes[r] = malloc(4 * m);
    scales[r] = malloc(4 * mb);
    fill(x[r], n);
    fill(res[r], n);
  }
  float* out = malloc(4 * m);
  float* acc = malloc(4 * m);
  uint16_t* c16 = malloc(2 * m);
  uint8_t* c8 = malloc(m);
  float* sc = malloc(4 * mb);

  or_reduce_sum(out, (const float* const*)x, k, n);
  for (int op = 0; op < 4; op++) or_reduce(out, (const float* const*)x, k, n, op, 3);

  or_encode_bf16(c16, x[0], n);
  int ok = 1;
  for (size_t i = 0; i < n; i++) ok &= or_bf16_encode_one(or_bf16_decode_one(c16[i])) == c16[i];
  check(ok, "bf16 codes round-trip", n);
  or_encode_fp8(c8, sc, x[0], n, 0);
  or_encode_fp8(c8, sc, x[0], n, 1);
  or_e4m3_encode_array(c8, x[0], n);
  or_e4m3_decode_array(acc, c8, n);
  for (int mode = 0; mode < 2; mode++) {
    for (int codec = 0; codec < 3; codec++) {
      or_bucket_allreduce(out, codes, scales, (const float* const*)x, k, n, 512, codec, mode);
      for (int a = 0; a < 2; a++) {
        or_decode_accumulate(acc, (const void* const*)codes, (const float* const*)scales, k, n, codec, a);
      }
    }
    for (int codec = 1; codec < 3; codec++) {
      or_bucket_allreduce_ef(out, codes, scales, res, (const float* const*)x, k, n, 256, codec, mode);
      or_encode_bf16_ef(c16, res[0], x[1 % k], n);
      or_encode_fp8_ef(c8, sc, res[0], x[1 % k], n, mode);
    }
  }
  for (size_t i = 0; i < n; i++) {
    (void)or_block_scale(fabsf(x[0][i]), (int)(i & 1));
    (void)or_fp8_quantize_one(x[0][i], x[k - 1][i]);
  }
  (void)or_block_absmax(x[0], n);

  /* other element types, their bit patterns drawn from the float32 arrays */
  for (int dt = 0; dt < 8; dt++) {
    for (int op = 0; op < 4; op++) {
      if (op == 1 && dt >= 4) continue;
      const size_t nt = (dt == 3 || dt == 7) ? n / 2 : n; /* 8-byte types: half as many in the same bytes */
      or_reduce_typed(out, (const void* const*)x, k, nt, dt, op, 7);
    }
  }
  for (int dt = 0; dt < 4; dt++) {
    const size_t nt = dt == 3 ? n / 2 : n; /* float64 arrays: half as many values in the same bytes */
    for (int codec = 1; codec < 3; codec++) {
      or_encode_typed(codec, dt, codes[0], scales[0], x[0], nt, 0);
      or_decode_sum_typed(out, dt, (const void* const*)codes, (const float* const*)scales, k, nt, codec);
      or_encode_ef_typed(codec, dt, codes[0], scales[0], res[0], x[0], nt, 1);
    }
    for (int codec = 0; codec < 3; codec++) {
      or_bucket_allreduce_typed(out, codes, scales, (const void* const*)x, k, nt, 256, codec, 0, dt);
      if (codec) or_bucket_allreduce_ef_typed(out, codes, scales, res, (const void* const*)x, k, nt, 256, codec, 1, dt);
    }
  }

  for (int r = 0; r < k; r++) {
    free(x[r]);
    free(res[r]);
    free(codes[r]);
    free(scales[r]);
  }
  free(out);
  free(acc);
  free(c16);
  free(c8);
  free(sc);
}

int main(void) {
  static const size_t sizes[] = {0, 1, 3, 255, 256, 257, 511, 1000, 4096 + 7};
  for (size_t i = 0; i < sizeof sizes / sizeof sizes[0]; i++) {
    for (int k = 1; k <= 8; k += 3) run(sizes[i], k);
  }
  /* every E4M3 code decodes and re-encodes to itself (NaN codes to a NaN code) */
  int ok = 1;
  for (unsigned c = 0; c < 256; c++) {
    float v = or_e4m3_decode_one((uint8_t)c);
    uint8_t back = or_e4m3_encode_one(v, (c & 0x80u) != 0);
    ok &= isnan(v) ? (back & 0x7Fu) == 0x7Fu : back == c;
  }
  check(ok, "E4M3 codes round-trip", 256);
  printf("oracle_driver: %d checks, %d failed\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
