/*
 * gb_oracle.h — plain, slow CPU oracle of the leader-side arithmetic of a
 * reduce-bridge-broadcast all-reduce with bf16 / fp8 bridge compression.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load it.  It shares no code, header,
 * table or constant with the GPU library: it is the independent definition
 * the GPU results are checked against.
 *
 * Everything is host memory, scalar C, IEEE binary32 with round-to-nearest-
 * even, no fused multiply-add (built with -ffp-contract=off) and no
 * flush-to-zero.
 *
 * Source of each step: the gpubridge README, sections "How it works" (the
 * leaders' sum of island sums), "API" (all_reduce SUM), "Bridge compression"
 * (bf16; OCP E4M3 with one scale per 256 values; decode and add in float32)
 * and "DistributedDataParallel" (one all_reduce per gradient bucket).
 * Where those passages leave a step open, the reading taken is stated at the
 * function.  Parity status of every function is listed in the file header of
 * gb_oracle.c.
 */
#ifndef GB_ORACLE_H
#define GB_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Codec numbers and scale-mode numbers of this oracle. */
enum { OR_CODEC_NONE = 0, OR_CODEC_BF16 = 1, OR_CODEC_FP8 = 2 };
enum { OR_SCALE_ABSMAX_DIV_448 = 0, OR_SCALE_POW2 = 1 };
enum { OR_OP_SUM = 0, OR_OP_AVG = 1, OR_OP_MAX = 2, OR_OP_MIN = 3 };

/* out[i] = left fold over ranks 0..k-1 of x[r][i], starting from x[0][i]. */
void or_reduce_sum(float* out, const float* const* x, int k, size_t n);

/* bf16: nearest value, ties to the even code; NaN -> (bits>>16)|0x40. */
uint16_t or_bf16_encode_one(float x);
float or_bf16_decode_one(uint16_t c);
void or_encode_bf16(uint16_t* codes, const float* x, size_t n);

/* OCP E4M3 of a value already divided by its scale: nearest, ties to the
 * even code, saturating at 448; `negative` gives the sign bit. NaN -> 0x7F|sign. */
uint8_t or_e4m3_encode_one(float v, int negative);
/* Value of an E4M3 code (NaN for 0x7F / 0xFF). */
float or_e4m3_decode_one(uint8_t c);
/* The two above over arrays (scale 1; the sign bit is each value's own). */
void or_e4m3_encode_array(uint8_t* codes, const float* v, size_t n);
void or_e4m3_decode_array(float* v, const uint8_t* codes, size_t n);

/* Largest non-NaN magnitude of a block (+0 when empty or all NaN). */
float or_block_absmax(const float* x, size_t len);
/* Scale of a block with largest magnitude a, per scale mode. */
float or_block_scale(float a, int mode);
/* Code of one element x of a block with scale s. */
uint8_t or_fp8_quantize_one(float x, float s);

/* Block-scaled fp8 encode of n values: codes[n], scales[ceil(n/256)]. */
void or_encode_fp8(uint8_t* codes, float* scales, const float* x, size_t n,
                   int mode);

/* Decode each rank's payload and add in rank order (see gb_oracle.c). */
void or_decode_accumulate(float* acc, const void* const* codes,
                          const float* const* scales, int k, size_t n,
                          int codec, int accumulate);

/* One bucket stream: per bucket, encode every rank's bucket into its payload
 * (codes[r], scales[r] for fp8; codes[r] for bf16; unused for none), then
 * decode and accumulate the k payloads into out. Blocks restart at every
 * bucket; scales of consecutive buckets are stored back to back. */
void or_bucket_allreduce(float* out, void* const* codes, float* const* scales,
                         const float* const* x, int k, size_t n,
                         size_t bucket_elems, int codec, int mode);

/* SUM, AVG (SUM / divisor, the world size), MAX or MIN over k ranks. */
void or_reduce(float* out, const float* const* x, int k, size_t n, int op,
               int divisor);

/* Element types of or_reduce_typed. */
enum { OR_DTYPE_F32 = 0, OR_DTYPE_F16 = 1, OR_DTYPE_BF16 = 2, OR_DTYPE_F64 = 3,
       OR_DTYPE_I8 = 4, OR_DTYPE_U8 = 5, OR_DTYPE_I32 = 6, OR_DTYPE_I64 = 7 };
/* SUM / AVG / MAX / MIN over k arrays of one element type (AVG: floating
 * types only). */
void or_reduce_typed(void* out, const void* const* x, int k, size_t n, int dtype,
                     int op, int divisor);

/* Error feedback: y = x + residual is encoded, and residual becomes
 * y - decode(payload).  residual is read and written (caller-owned). */
void or_encode_bf16_ef(uint16_t* codes, float* residual, const float* x, size_t n);
void or_encode_fp8_ef(uint8_t* codes, float* scales, float* residual,
                      const float* x, size_t n, int mode);
/* The bucket stream with error feedback (bf16 or fp8): each rank's residual
 * residuals[r][n] is updated as its buckets are encoded. */
void or_bucket_allreduce_ef(float* out, void* const* codes,
                            float* const* scales, float* const* residuals,
                            const float* const* x, int k, size_t n,
                            size_t bucket_elems, int codec, int mode);

/* Bridge codecs over float16 / bfloat16 / float64 arrays (f16 and bf16 as raw
 * 16-bit codes): the values go to binary32 first, then through the binary32
 * encoders; the decoded binary32 total is rounded once to the type. */
void or_encode_typed(int codec, int dtype, void* codes, float* scales, const void* x,
                     size_t n, int mode);
void or_decode_sum_typed(void* out, int dtype, const void* const* codes,
                         const float* const* scales, int k, size_t n, int codec);
void or_bucket_allreduce_typed(void* out, void* const* codes, float* const* scales,
                               const void* const* x, int k, size_t n, size_t bucket_elems,
                               int codec, int mode, int dtype);

/* Error feedback over float16 / bfloat16 / float64 (or float32) arrays: the
 * values go to binary32 as above, the binary32 error-feedback step runs on
 * them with the binary32 residual, and the decoded binary32 total is rounded
 * once to the type. */
void or_encode_ef_typed(int codec, int dtype, void* codes, float* scales, float* residual,
                        const void* x, size_t n, int mode);
void or_bucket_allreduce_ef_typed(void* out, void* const* codes, float* const* scales,
                                  float* const* residuals, const void* const* x, int k,
                                  size_t n, size_t bucket_elems, int codec, int mode,
                                  int dtype);

#ifdef __cplusplus
}
#endif

#endif /* GB_ORACLE_H */
