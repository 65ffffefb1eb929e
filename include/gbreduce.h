/*
 * gbreduce.h — C ABI of libgbreduce, the leader-side arithmetic of a
 * reduce-bridge-broadcast all-reduce on one AMD Instinct MI355X (gfx950).
 *
 * Source of the method: the gpubridge README ("How it works"; "Collective
 * policies" and its "Bridge compression" paragraph; "API").  In
 * reduce-bridge-broadcast each island reduces onto its leader, the leaders
 * combine the island sums over a CPU bridge, and each leader broadcasts the
 * total to its island.  The leader's share of that work is what this library
 * computes, with every contribution already resident in device memory:
 *
 *   - the elementwise fp32 SUM of k contributions in fixed rank order;
 *   - the opt-in bf16 bridge compression (encode; decode and add in fp32);
 *   - the opt-in fp8 bridge compression: OCP E4M3 codes with one fp32 scale
 *     per 256 values (encode; decode and add in fp32);
 *   - the DDP bucket stream of all three in one pass.
 *
 * and, around them: AVG, MAX and MIN; the README's other element types,
 * reduced exactly or through the codecs; an error-feedback residual per
 * buffer; the bucket stream over buckets held in separate buffers, several
 * per launch; and the staged (pipelined) steps through pinned host memory.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Element arrays (fp32 inputs and outputs, bf16 and fp8 code arrays) are
 *    DEVICE pointers, 16-byte aligned; scale arrays are device pointers,
 *    4-byte aligned.  Pointer ARRAYS (srcs, codes, scales) are HOST arrays of
 *    k device pointers; they are copied into the launch, so the caller may
 *    reuse them as soon as the call returns.
 *  - The caller owns every buffer.  Calls allocate no device memory.
 *  - Calls are asynchronous: work is enqueued on `stream` (a hipStream_t;
 *    NULL is the null stream) and the call returns.  Buffers must stay alive
 *    and untouched until the stream has passed the work (the duty the
 *    README's "Async collectives" section places on tensors in flight).
 *  - Validation happens before anything is enqueued: a call that returns an
 *    error enqueued nothing and wrote nothing.
 *  - Overlap: every buffer a call writes (outputs, payloads, workspaces,
 *    residuals, staging buffers) shares no byte with any other buffer of the
 *    call, except the in-place aliases each call documents (out == srcs[0]:
 *    the same address and length); inputs may overlap one another.  Any
 *    other overlap is GB_ERR_INVALID_ARG, naming the two buffers.  n == 0 is GB_OK and enqueues
 *    nothing.  The calls never abort or exit the process.
 *  - Failures return a gb_status; gb_last_error() then holds a one-line
 *    detail for the calling thread.
 *  - Two environment variables, read once at the first call of the process
 *    (set and not "0" means on), add per-call hooks to every call that takes
 *    a stream:  GB_TRACE prints one line per call on stderr (entry point,
 *    k, n and codec where the call takes them, stream, status and the
 *    failure's detail, host time);  GB_DEBUG waits for the stream after a
 *    call that returned GB_OK and returns GB_ERR_HIP if the stream reports
 *    an error (from the call's kernels, or from earlier work on the stream),
 *    except on a stream under graph capture, which is not waited for.  Both
 *    are off by default.
 *  - Arithmetic is IEEE binary32 with round-to-nearest-even, subnormals kept
 *    and no fused multiply-add: every sum is a left fold over ranks
 *    0, 1, ..., k-1 starting from rank 0's value, so a result does not depend
 *    on the launch configuration and is bit-reproducible.
 *  - NaN (README "Bridge compression": every rank ends with the same bits,
 *    whichever vendor's GPU ran the kernels).  Every NaN that the float32
 *    arithmetic delivers -- a sum of two or more terms, an AVG quotient, a
 *    MAX or MIN over two or more values, a decoded-and-added total, the
 *    error-feedback value and residual -- is stored as the quiet NaN
 *    0x7FC00000, whatever the operands' NaN signs and payloads, and a NaN
 *    total of another element type as that NaN's rounding (float16 0x7E00,
 *    bfloat16 0x7FC0, float64 0x7FF8000000000000).  A copy keeps its bits:
 *    k = 1 sums, MAX and MIN, and the decode of one bf16 payload into
 *    float32.  An encoder's code for a NaN input keeps the input's sign.
 *    The exact reductions of gb_reduce_typed over float16, bfloat16 and
 *    float64 are excepted: their NaN results are some quiet NaN.
 *  - The codecs apply to floating-point SUM (and to AVG as a decode followed
 *    by the division), as the README's compression does; MAX, MIN and the
 *    integer types are reduced exactly, never compressed.
 *  - n is at most GB_MAX_N; a larger n is GB_ERR_INVALID_ARG.
 */
#ifndef GBREDUCE_H
#define GBREDUCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GB_VERSION 1
/* Values per fp8 scale block (README "Bridge compression": one scale per
 * 256 values). */
#define GB_BLOCK 256
/* Largest number of contributions (ranks or islands) one call sums.  A
 * kernel launch reads up to 8; a call with more folds the rest in further
 * launches, continuing the same rank-order fold from the stored partial
 * result (the same bits as one pass), at 8 more bytes of traffic per value
 * per extra launch. */
#define GB_MAX_K 16
/* Required byte alignment of element arrays. */
#define GB_ALIGN 16
/* Largest element count any call accepts: 2^39 values (2 TiB of fp32 per
 * buffer, beyond the memory of any one GPU), so that no size or offset the
 * library computes from n can wrap. */
#define GB_MAX_N ((size_t)1 << 39)
/* Largest number of buckets one gb_bucket_allreduce_local_batch call takes;
 * their sizes, each rounded up to a multiple of 256, add up to at most
 * GB_MAX_N. */
#define GB_MAX_BATCH 4096

typedef enum gb_status {
  GB_OK = 0,
  GB_ERR_INVALID_ARG = 1, /* null pointer with n > 0, n > GB_MAX_N, k out of range, bad flag, bad bucket size,
                             overlapping buffers */
  GB_ERR_MISALIGNED = 2,  /* an element array is not 16-byte aligned, or a scale array not 4-byte */
  GB_ERR_UNSUPPORTED = 3, /* unknown codec or scale mode */
  GB_ERR_WORKSPACE = 4,   /* workspace pointer null or smaller than required */
  GB_ERR_HIP = 5          /* the HIP runtime refused a launch; detail in gb_last_error() */
} gb_status;

/* Bridge payload codecs ("Bridge compression": off, bf16 or fp8). */
typedef enum gb_codec {
  GB_CODEC_NONE = 0,        /* payload is the fp32 values themselves          */
  GB_CODEC_BF16 = 1,        /* n uint16 codes                                 */
  GB_CODEC_FP8_E4M3_B256 = 2 /* n uint8 OCP E4M3 codes + ceil(n/256) fp32 scales */
} gb_codec;

/* How the fp8 scale s of a block is derived from the block's largest
 * magnitude a (NaN elements ignored; a = +0 for an all-zero block).
 * Every element of the block is encoded as E4M3(RN(x / s)), saturating to
 * +-448, and decodes as RN(E4M3value * s). */
typedef enum gb_scale_mode {
  /* s = RN(a / 448): the block's largest element encodes to +-448.
   * A zero block stores s = 0 and encodes each element as +-0. */
  GB_SCALE_ABSMAX_DIV_448 = 0,
  /* s = 2^e with e the smallest integer >= -149 such that a <= 448 * 2^e,
   * i.e. the README's scale that is a power of two.
   * A zero block stores s = 1. */
  GB_SCALE_POW2 = 1
} gb_scale_mode;

/* Reductions of gb_reduce (README "API": all_reduce with SUM, AVG, MAX or
 * MIN).  The bridge codecs apply to SUM and AVG only. */
typedef enum gb_op {
  GB_OP_SUM = 0,
  GB_OP_AVG = 1, /* the SUM divided by the world size (an explicit divisor) */
  GB_OP_MAX = 2, /* IEEE 754-2019 maximum: NaN if any value is NaN; +0 > -0 */
  GB_OP_MIN = 3  /* IEEE 754-2019 minimum: NaN if any value is NaN; -0 < +0 */
} gb_op;

/* Element types of gb_reduce_typed (README "API": the dtypes every backend
 * supports).  The bridge codecs apply to float32 only. */
typedef enum gb_dtype {
  GB_DTYPE_F32 = 0,
  GB_DTYPE_F16 = 1,  /* IEEE binary16 */
  GB_DTYPE_BF16 = 2, /* bfloat16: top half of binary32 */
  GB_DTYPE_F64 = 3,
  GB_DTYPE_I8 = 4,
  GB_DTYPE_U8 = 5,
  GB_DTYPE_I32 = 6,
  GB_DTYPE_I64 = 7
} gb_dtype;

/*
 * gb_reduce_sum — the leader's sum of island sums (README "How it works":
 * leaders all-reduce the island sums, each leader then holds the total).
 *   dst[i] = RN(...RN(RN(srcs[0][i] + srcs[1][i]) + srcs[2][i]) ... + srcs[k-1][i])
 * for i in [0, n).  k = 1 copies srcs[0].
 *   dst   device fp32[n], written; may equal srcs[0] (in place), must not
 *         otherwise overlap any source.
 *   srcs  host array of k device fp32[n] pointers, read only.
 *   k     1 .. GB_MAX_K.
 * The sum is written once, straight into dst: this is also the leader's copy
 * of the total into the buffer its island broadcast reads.
 */
gb_status gb_reduce_sum(float* dst, const float* const* srcs, int k, size_t n,
                        void* stream);

/*
 * gb_reduce — the leader's uncompressed all_reduce of the island results with
 * any of the README's reductions:
 *   SUM  dst[i] = the fixed-order sum (exactly gb_reduce_sum);
 *   AVG  dst[i] = RN(sum[i] / RN(divisor)): divisor is the job's world size
 *        (the number of ranks, not k), 1 .. 2^24; identical on every rank;
 *   MAX  dst[i] = IEEE 754-2019 maximum over the k values (rank order does not
 *        matter; a NaN anywhere gives NaN);
 *   MIN  dst[i] = IEEE 754-2019 minimum.
 * divisor is ignored except for AVG.  A compressed AVG is
 * gb_decode_accumulate followed by gb_reduce(acc, {acc}, 1, n, GB_OP_AVG, d).
 * Arguments, aliasing and errors as gb_reduce_sum; GB_ERR_UNSUPPORTED for an
 * unknown op, GB_ERR_INVALID_ARG for an AVG divisor outside 1 .. 2^24.
 */
gb_status gb_reduce(float* dst, const float* const* srcs, int k, size_t n,
                    int op, int divisor, void* stream);

/*
 * gb_reduce_typed — gb_reduce over any of the README's element types, on
 * arrays of n elements of `dtype` (void pointers, 16-byte aligned):
 *   SUM  floating types: left fold over ranks, every add rounded to the type
 *        (nearest, ties to even, IEEE overflow to Inf); integer types: wraps
 *        modulo 2^bits;
 *   AVG  floating types only (GB_ERR_UNSUPPORTED for integers):
 *        RN_type(sum / divisor), divisor 1 .. 2^24;
 *   MAX, MIN  IEEE 754-2019 for floating types, the ordinary order for
 *        integers (uint8 unsigned).
 * GB_DTYPE_F32 is exactly gb_reduce.  Arguments, aliasing and errors as
 * gb_reduce; GB_ERR_UNSUPPORTED for an unknown dtype.
 */
gb_status gb_reduce_typed(void* dst, const void* const* srcs, int k, size_t n,
                          int dtype, int op, int divisor, void* stream);

/*
 * gb_encode_bf16 — bf16 bridge compression of one fp32 payload
 * (README "Bridge compression": half the bytes of float32).
 *   codes[i] = nearest bf16 to src[i], ties to the even code; values beyond
 *              the bf16 range round to +-Inf as IEEE rounding does;
 *              subnormals are kept; a NaN keeps its sign and top 7 payload
 *              bits with the quiet bit forced on: (bits >> 16) | 0x0040.
 *   codes device uint16[n], written.   src device fp32[n], read only.
 */
gb_status gb_encode_bf16(uint16_t* codes, const float* src, size_t n,
                         void* stream);

/*
 * gb_encode_fp8_e4m3_blockscaled — fp8 bridge compression of one fp32
 * payload (README "Bridge compression": OCP E4M3 with one scale per 256
 * values, about 3.9x fewer bytes than fp32).
 * Block b covers elements [256b, min(256b + 256, n)); the last block may be
 * partial and its scale covers only the elements present.
 *   scales[b] = s_b, from the block's largest non-NaN magnitude per scale_mode.
 *   codes[i]  = E4M3(v) with v = RN(src[i] / s_b) (v = src[i] when s_b == 0):
 *               nearest OCP E4M3 value (bias 7, largest finite 448, no Inf),
 *               ties to the even code, |v| > 448 saturating to 448 (0x7E);
 *               the sign bit is src[i]'s sign (so -0 encodes as 0x80); a NaN
 *               src[i], or a NaN quotient (an Inf element in a block whose
 *               scale is Inf), encodes as 0x7F | sign.
 *   codes  device uint8[n], written (16-byte aligned).
 *   scales device fp32[ceil(n/256)], written (4-byte aligned).
 *   src    device fp32[n], read only.
 * The payload on the bridge is codes followed by scales: gb_payload_bytes().
 */
gb_status gb_encode_fp8_e4m3_blockscaled(uint8_t* codes, float* scales,
                                         const float* src, size_t n,
                                         int scale_mode, void* stream);

/*
 * gb_decode_accumulate — decode every leader's payload and add in float32
 * after the bridge step (README "Bridge compression": dequantize and add in
 * float32, so every rank ends with the same bits).
 *   v_r[i]  = codes[r][i] as fp32                        (GB_CODEC_NONE)
 *           = bf16 codes[r][i] widened to fp32 (exact)   (GB_CODEC_BF16)
 *           = RN(E4M3value(codes[r][i]) * scales[r][i/256]) (GB_CODEC_FP8_E4M3_B256)
 *   accumulate == 0:  acc[i] = RN(...RN(v_0[i] + v_1[i]) ... + v_{k-1}[i])
 *   accumulate == 1:  acc[i] = RN(...RN(acc[i] + v_0[i]) ... + v_{k-1}[i])
 * The product and the sum are rounded separately (never fused).
 *   acc    device fp32[n], written (and read when accumulate == 1); must not
 *          overlap any payload.
 *   codes  host array of k device pointers: fp32[n], uint16[n] or uint8[n].
 *   scales host array of k device fp32[ceil(n/256)] pointers for fp8;
 *          ignored (may be NULL) for the other codecs.
 *   k      1 .. GB_MAX_K.   accumulate 0 or 1.
 */
gb_status gb_decode_accumulate(float* acc, const void* const* codes,
                               const float* const* scales, int k, size_t n,
                               int codec, int accumulate, void* stream);

/*
 * gb_bucket_allreduce_local — the leader arithmetic of one DDP-style bucket
 * stream (README "DistributedDataParallel": each gradient bucket is one
 * all_reduce), with all k contributions resident on this GPU.
 * The n-element buffers are cut into consecutive buckets of bucket_elems
 * elements (the last one partial).  For each bucket, in order, on `stream`:
 *   codec NONE : out = fixed-order sum of the k buckets (as gb_reduce_sum);
 *   codec BF16 : each rank's bucket is bf16-encoded into the workspace, then
 *                out = decode-and-accumulate of the k payloads (accumulate 0);
 *   codec FP8  : each rank's bucket is E4M3-encoded with per-256 scales into
 *                the workspace, then out = decode-and-accumulate.
 * Each value is read from srcs once: encode and decode of a bucket are one
 * pass, and the decoded values are the ones stored payloads decode to.
 * Buckets start on 256-value boundaries, so they are processed together in
 * one launch whose workgroups take them in order; the result equals one call
 * per bucket bit for bit.  A caller that holds only some buckets (a DDP hook
 * as buckets become ready) calls once per bucket with n = that bucket.
 *   out          device fp32[n], written; may equal srcs[0].
 *   srcs         host array of k device fp32[n] pointers, read only.
 *   bucket_elems a positive multiple of 256 (so fp8 blocks never straddle a
 *                bucket and each bucket starts 16-byte aligned).
 *   workspace    device buffer of at least gb_bucket_workspace_bytes(); it
 *                receives every rank's payload for the whole buffer, laid out
 *                as gb_bucket_workspace_layout() reports (unused for NONE,
 *                may then be NULL with workspace_bytes 0).
 * Because every bucket starts on a 256-element boundary, rank r's payload in
 * the workspace equals what gb_encode_bf16 / gb_encode_fp8_e4m3_blockscaled
 * writes for the whole of srcs[r].
 */
gb_status gb_bucket_allreduce_local(float* out, const float* const* srcs,
                                    int k, size_t n, size_t bucket_elems,
                                    int codec, int scale_mode,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);

/* Size of the static device scratch of gb_bucket_allreduce_local_noalloc:
 * 64 MiB per GPU, enough for the payloads of a 25 MiB DDP bucket
 * (6,553,600 float32 values) from up to 10 ranks with the fp8 codec or 5
 * with bf16. */
#define GB_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * gb_bucket_allreduce_local_noalloc — gb_bucket_allreduce_local for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, result
 * and errors, without the workspace: the payloads go to a static device
 * array of GB_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on until the process ends.  The call allocates nothing, device or
 * host; its first call on a device looks up that device's array address
 * once.
 *   - GB_ERR_WORKSPACE, with nothing enqueued, when
 *     gb_bucket_workspace_bytes(codec, k, n, bucket_elems) exceeds
 *     GB_NOALLOC_SCRATCH_BYTES (codec NONE needs no scratch).
 *   - The payloads are not returned: the array keeps the last call's
 *     contents and every call on one GPU shares it, so calls that overlap on
 *     one GPU (on different streams, or concurrently from several threads)
 *     race.  Nothing in the array needs to start at zero: a call writes every
 *     payload byte it reads.
 */
gb_status gb_bucket_allreduce_local_noalloc(float* out, const float* const* srcs,
                                            int k, size_t n, size_t bucket_elems,
                                            int codec, int scale_mode,
                                            void* stream);

/*
 * gb_bucket_allreduce_local_batch — the bucket stream over nbuckets buckets
 * that live in separate buffers, as a DDP hook holds them (README "API",
 * the ddp_comm_hook entry, and its "DistributedDataParallel" section: each
 * gradient bucket is averaged by one async all_reduce).  Bucket b of ns[b] values has
 * its own k sources srcs[b * k + r] and its own output outs[b], of element
 * type dtype (GB_DTYPE_F32, F16, BF16 or F64), and gives, bit for bit, what
 * gb_bucket_allreduce_local_typed gives for it alone with bucket_elems >=
 * ns[b]: fp8 blocks restart at each bucket.  A compressed total of another
 * type than float32 holds up to 8 ranks, as there.  With k <= 8 and
 * a bf16 or fp8 codec, up to 16 buckets run in one launch, so buckets that
 * are ready together keep the GPU full where one small bucket per launch
 * cannot; otherwise the buckets run one after another.  A large bucket takes
 * the workgroup order and occupancy of a whole-buffer launch, so a batch of
 * one bucket runs as the single-buffer call does, and with a divisor gives
 * that stream's AVG.
 *   outs       host array of nbuckets device dtype[ns[b]] pointers,
 *              written; outs[b] may equal srcs[b * k]; no other overlap
 *              between any output, source or the workspace.
 *   srcs       host array of nbuckets * k device dtype pointers,
 *              bucket-major.
 *   ns         host array of nbuckets sizes, each 0 .. GB_MAX_N (a bucket
 *              of 0 values is skipped, its pointers unread).
 *   nbuckets   1 .. GB_MAX_BATCH; the sizes, each rounded up to a
 *              multiple of 256, add up to at most GB_MAX_N.
 *   divisor    1 for SUM; the job's world size (up to 2^24) for AVG, which
 *              the README compresses as the decode-and-add followed by the
 *              division: a float32 total becomes RN(total / divisor) in the
 *              same pass; a total of another type is divided as
 *              gb_reduce_typed divides it, in a second pass over the output;
 *              with codec NONE each bucket is the exact AVG of gb_reduce_typed.
 *              GB_ERR_INVALID_ARG outside 1 .. 2^24.
 *   workspace  device buffer of at least gb_bucket_batch_workspace_bytes();
 *              rank r's payload of bucket b sits where the payload of values
 *              [o_b, o_b + ns[b]) of one buffer would, in the layout
 *              gb_bucket_workspace_layout() reports for that buffer, with
 *              o_b the sum of ns[i] rounded up to a multiple of 256 over
 *              i < b (unused for NONE, may then be NULL).
 * Errors as gb_bucket_allreduce_local, checked for every bucket before
 * anything is enqueued; the host arrays may be freed on return.
 */
gb_status gb_bucket_allreduce_local_batch(int dtype, void* const* outs,
                                          const void* const* srcs,
                                          const size_t* ns, int nbuckets, int k,
                                          int codec, int scale_mode,
                                          int divisor, void* workspace,
                                          size_t workspace_bytes, void* stream);

/*
 * gb_bucket_allreduce_local_batch_ef — the batched bucket stream with error
 * feedback (README "Bridge compression": a residual per buffer carries each
 * step's rounding error into the next).  Bucket b gives, bit for bit, what
 * gb_bucket_allreduce_local_ef_typed gives for it alone, reading and
 * rewriting the binary32 residuals residuals[b * k + r] (device
 * float[ns[b]] each, bucket-major, 16-byte aligned, overlapping nothing
 * else).  Up to 8 buckets per launch.  GB_ERR_UNSUPPORTED for codec NONE;
 * everything else as gb_bucket_allreduce_local_batch, whose workspace size
 * applies.
 */
gb_status gb_bucket_allreduce_local_batch_ef(int dtype, void* const* outs,
                                             const void* const* srcs,
                                             float* const* residuals,
                                             const size_t* ns, int nbuckets,
                                             int k, int codec, int scale_mode,
                                             int divisor, void* workspace,
                                             size_t workspace_bytes,
                                             void* stream);

/* Workspace bytes of gb_bucket_allreduce_local_batch and
 * gb_bucket_allreduce_local_batch_ef (0 on invalid arguments, or for codec
 * NONE). */
size_t gb_bucket_batch_workspace_bytes(int codec, int k, const size_t* ns,
                                       int nbuckets);

/*
 * gb_reduce_encode — the leader's island sum and its bridge payload in one
 * pass (README "How it works": each island reduces onto its leader;
 * "Bridge compression": leaders quantize their island's sum before the
 * bridge step).  With the island's k contributions resident here:
 *   sum[i]   = the rank-order fold of srcs[r][i], exactly as gb_reduce_sum;
 *   payload  = codes (and, for fp8, scales) of that sum, exactly as
 *              gb_encode_bf16 / gb_encode_fp8_e4m3_blockscaled encode it.
 * Reads each source once and writes the payload (and the sum) once, instead
 * of writing the sum and reading it back.
 *   sum     device fp32[n], written; may be NULL to skip storing it when
 *           k <= 8 (a larger k sums into it first, so it is then required:
 *           GB_ERR_INVALID_ARG); may equal srcs[0].
 *   codes   device uint16[n] (GB_CODEC_BF16) or uint8[n]
 *           (GB_CODEC_FP8_E4M3_B256), written; must not overlap a source.
 *   scales  device fp32[ceil(n/256)] for fp8 (ignored for bf16).
 *   srcs    host array of k device fp32[n] pointers;  k 1 .. GB_MAX_K.
 * GB_ERR_UNSUPPORTED for codec NONE or an unknown scale mode.
 */
gb_status gb_reduce_encode(float* sum, void* codes, float* scales,
                           const float* const* srcs, int k, size_t n,
                           int codec, int scale_mode, void* stream);

/*
 * Bridge compression of float16, bfloat16 and float64 tensors (README
 * "Bridge compression": the bridged policies compress floating-point SUM and
 * AVG, and the dequantized payloads are added in float32).  The island sum,
 * of the tensor's type, is first taken to binary32 (exactly from float16 and
 * bfloat16; rounded once to nearest-even from float64) and encoded exactly
 * as a binary32 array is; the float32 total of the decoded payloads is
 * rounded once to the tensor's type (nearest, ties to even, IEEE overflow to
 * Inf; exact to float64).  dtype is GB_DTYPE_F32, F16, BF16 or F64
 * (GB_ERR_UNSUPPORTED otherwise); arrays of dtype are 16-byte aligned.
 *
 * gb_encode — codes (and, for fp8, scales) of src (dtype[n]), as
 *   gb_encode_bf16 (codec GB_CODEC_BF16; scales unused, may be NULL) or
 *   gb_encode_fp8_e4m3_blockscaled (codec GB_CODEC_FP8_E4M3_B256) would
 *   write for the binary32 values.  GB_ERR_UNSUPPORTED for codec NONE.
 */
gb_status gb_encode(int codec, int dtype, void* codes, float* scales,
                    const void* src, size_t n, int scale_mode, void* stream);

/*
 * gb_decode_sum — dst (dtype[n]) = the rank-order float32 sum of the k
 *   decoded payloads (as gb_decode_accumulate with accumulate 0), rounded once
 *   to dtype.  codes, scales, k and codec as gb_decode_accumulate; codec NONE
 *   (float32 payloads) only with dtype F32 (other types reduce exactly with
 *   gb_reduce_typed).  dst must not overlap any payload.  For a dtype other
 *   than F32, k is at most 8 (GB_ERR_INVALID_ARG beyond): the total is
 *   rounded once from float32, and the library keeps no float32 buffer of its
 *   own; sum more payloads into a float32 buffer with gb_decode_accumulate.
 */
gb_status gb_decode_sum(int dtype, void* dst, const void* const* codes,
                        const float* const* scales, int k, size_t n, int codec,
                        void* stream);

/*
 * gb_bucket_allreduce_local_typed — gb_bucket_allreduce_local over arrays of
 *   dtype: out and srcs[r] hold dtype[n].  With a codec each rank's bucket is
 *   encoded as gb_encode does (into the same workspace, of the same size, as
 *   for float32) and out = the float32 total rounded once to dtype; without
 *   one (GB_CODEC_NONE) out is the exact SUM of the type (gb_reduce_typed).
 *   out may equal srcs[0].  With a codec and a dtype other than F32, k is at
 *   most 8, as for gb_decode_sum.  Everything else as
 *   gb_bucket_allreduce_local.
 */
gb_status gb_bucket_allreduce_local_typed(int dtype, void* out,
                                          const void* const* srcs, int k,
                                          size_t n, size_t bucket_elems,
                                          int codec, int scale_mode,
                                          void* workspace,
                                          size_t workspace_bytes, void* stream);

/*
 * Error feedback (README "Bridge compression": each bridge member keeps an
 * error-feedback residual per buffer, so the rounding error of one step is
 * carried into the next instead of accumulating).  The residual is a
 * caller-owned device fp32[n] per buffer, 16-byte aligned, zero before the
 * first step; each call reads it and writes it back:
 *   y[i]        = RN(src[i] + residual[i])
 *   payload     = the plain encoder's payload of y (for fp8 the block scales
 *                 come from y)
 *   residual[i] = RN(y[i] - decoded payload value[i])   (exact for bf16)
 * The residual must not overlap src or the payload.  Non-finite values follow
 * the formulas (an Inf y gives a NaN residual).
 */
gb_status gb_encode_bf16_ef(uint16_t* codes, float* residual, const float* src,
                            size_t n, void* stream);
gb_status gb_encode_fp8_e4m3_blockscaled_ef(uint8_t* codes, float* scales,
                                            float* residual, const float* src,
                                            size_t n, int scale_mode,
                                            void* stream);

/*
 * gb_bucket_allreduce_local_ef — gb_bucket_allreduce_local with error
 * feedback: rank r's buckets are encoded from y = srcs[r] + residuals[r] and
 * residuals[r] is updated as above; out receives the rank-order sum of the
 * decoded payloads.  residuals: host array of k device fp32[n] pointers.
 * codec must be BF16 or FP8 (GB_ERR_UNSUPPORTED for NONE: there is no
 * rounding to feed back).
 */
gb_status gb_bucket_allreduce_local_ef(float* out, const float* const* srcs,
                                       float* const* residuals, int k, size_t n,
                                       size_t bucket_elems, int codec,
                                       int scale_mode, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Error feedback over float16, bfloat16 and float64 gradients (the same
 * README paragraph, over the floating types of the typed calls above).  The
 * residual stays binary32, and the step is the binary32 one above applied to
 * the gradient taken to binary32 as gb_encode takes it (exactly from float16
 * and bfloat16; rounded once from float64, that rounding not being fed
 * back):
 *   y[i]        = RN(binary32(src[i]) + residual[i])
 *   residual[i] = RN(y[i] - decoded payload value[i])
 *
 * gb_encode_ef — codes (and, for fp8, scales) of y for src of dtype[n],
 *   residual updated; codec, dtype, scales and scale_mode as gb_encode.
 *
 * gb_bucket_allreduce_local_ef_typed — gb_bucket_allreduce_local_ef over
 *   arrays of dtype: out and srcs[r] hold dtype[n], residuals[r] fp32[n];
 *   out = the float32 rank-order total of the decoded payloads rounded once
 *   to dtype (out may equal srcs[0]).  For a dtype other than F32, k is at
 *   most 8, as for gb_bucket_allreduce_local_typed.  Everything else as
 *   gb_bucket_allreduce_local_ef.
 */
gb_status gb_encode_ef(int codec, int dtype, void* codes, float* scales,
                       float* residual, const void* src, size_t n,
                       int scale_mode, void* stream);
gb_status gb_bucket_allreduce_local_ef_typed(int dtype, void* out,
                                             const void* const* srcs,
                                             float* const* residuals, int k,
                                             size_t n, size_t bucket_elems,
                                             int codec, int scale_mode,
                                             void* workspace,
                                             size_t workspace_bytes,
                                             void* stream);

/*
 * Staged (pipelined) leader steps: the README's pipelined policy cuts the
 * bridge step into chunks so that the copy of one chunk to pinned host memory
 * overlaps the work on the next ("Collective policies": pipelined
 * reduce-bridge-broadcast, and the pinned staging paragraph).  These two calls
 * do the device side of it for one GPU:
 *
 * gb_encode_staged — encode src (fp32[n]) into the device payload
 *   (codes_dev, scales_dev) chunk by chunk on `stream`, and copy each chunk's
 *   codes to the pinned host payload (codes_host) on the library's copy
 *   streams as soon as that chunk is encoded, so the copy of chunk c overlaps
 *   the encode of chunk c+1; the scales (4 bytes per 256 values) follow in
 *   one copy.  codec BF16 or FP8 (scale_mode
 *   as gb_encode_fp8_e4m3_blockscaled; scales unused and may be NULL for
 *   BF16).  The payload is exactly the one-shot encoder's.  When `stream`
 *   reaches the end of the call's work, every copy has finished.
 *
 * gb_decode_accumulate_staged — the reverse: copy each of the k payloads
 *   received in pinned host memory (codes_host[r], scales_host[r]) into the
 *   device staging payloads (codes_dev[r], scales_dev[r]) chunk by chunk on
 *   the copy streams (every rank's scales first, in one copy each), and
 *   decode-and-accumulate each chunk on `stream` as soon as its copies are
 *   done (the result is exactly gb_decode_accumulate's).
 *   The copies start only after the work already queued on `stream`.
 *
 * chunk_elems: a positive multiple of 256 (the README's default chunk is
 * 4 MiB, i.e. 1,048,576 fp32 values; a copy has a fixed cost of some
 * microseconds, so chunks of a few MiB of payload or more pay off).  Host
 * buffers must be pinned
 * (hipHostMalloc, or torch's pin_memory): GB_ERR_INVALID_ARG otherwise.
 * Device arrays are 16-byte aligned, scale arrays 4-byte; host code arrays
 * 4-byte.  The library's two copy streams and their events are created on a
 * device's
 * first staged call and kept for the life of the process; calls on one
 * device from several host threads are serialised while they enqueue.
 */
gb_status gb_encode_staged(int codec, int scale_mode, void* codes_dev,
                           float* scales_dev, void* codes_host,
                           float* scales_host, const float* src, size_t n,
                           size_t chunk_elems, void* stream);
gb_status gb_decode_accumulate_staged(float* acc, const void* const* codes_host,
                                      const float* const* scales_host,
                                      void* const* codes_dev,
                                      float* const* scales_dev, int k, size_t n,
                                      size_t chunk_elems, int codec,
                                      int accumulate, void* stream);

/* Bytes one rank's n-value payload occupies on the bridge:
 * 4n (NONE), 2n (BF16), n + 4*ceil(n/256) (FP8).  0 for an unknown codec. */
size_t gb_payload_bytes(int codec, size_t n);

/* Workspace layout of gb_bucket_allreduce_local, all offsets in bytes from
 * the workspace start:
 *   rank r's codes  at r * codes_stride             (codes_stride = the code
 *                   bytes of n values rounded up to 256);
 *   rank r's scales at scales_offset + r * scales_stride (fp8 only;
 *                   scales_stride = 4*ceil(n/256) rounded up to 256).
 * *total receives gb_bucket_workspace_bytes().  Returns GB_ERR_INVALID_ARG
 * or GB_ERR_UNSUPPORTED for arguments gb_bucket_allreduce_local would refuse
 * (null output pointers included).  Host only; touches no device. */
gb_status gb_bucket_workspace_layout(int codec, int k, size_t n,
                                     size_t bucket_elems, size_t* codes_stride,
                                     size_t* scales_offset,
                                     size_t* scales_stride, size_t* total);

/* Workspace bytes gb_bucket_allreduce_local needs; 0 for codec NONE or for
 * arguments it would refuse. */
size_t gb_bucket_workspace_bytes(int codec, int k, size_t n,
                                 size_t bucket_elems);

/* Static English name of a status ("GB_OK", ...); "unknown status" else. */
const char* gb_status_string(int status);

/* Detail of the calling thread's last failed call ("" if none yet).  Valid
 * until that thread's next libgbreduce call. */
const char* gb_last_error(void);

/* GB_VERSION of the library that is loaded. */
int gb_version(void);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* GBREDUCE_H */
