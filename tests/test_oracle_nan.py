"""Pins of the oracle's canonical-NaN reading (gpubridge README, "Bridge
compression": every rank ends with the same bits, whichever vendor's GPU ran
the kernels).  IEEE 754-2019 leaves the sign and payload of an operation's NaN
to the platform, so every NaN that the float32 arithmetic of the method
delivers is stored as the quiet NaN 0x7FC00000; a result that no arithmetic
produced (a copy of one source, the widening of one bf16 payload) keeps its
bits, and so do the encoders' codes of NaN inputs.

Each case below builds its NaN from an invalid operation (whose default NaN
on an x86 host is negative) or from two NaNs of different sign and payload,
so a missing canonicalisation shows as a wrong bit pattern, not as a
different NaN count."""
import numpy as np

from oracle import oracle as O

CANON = 0x7FC00000


def f32(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


NEG_NAN_PAYLOAD = 0xFFC0ABCD   # negative quiet NaN with payload
POS_NAN_PAYLOAD = 0x7FA00001   # positive signalling NaN with payload
INF, NINF = 0x7F800000, 0xFF800000


def u32(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def test_host_default_nan_is_not_the_canonical_one():
    """The pins below mean something only if the host's own invalid operation
    gives another pattern: Inf - Inf on this host, with numpy's float32."""
    with np.errstate(invalid="ignore"):
        got = u32(f32([INF]) - f32([INF]))[0]
    assert np.isnan(f32([got]))[0]
    # x86 hosts give 0xFFC00000; on any host the oracle's answer is fixed
    assert got in (0xFFC00000, CANON)


def test_sum_of_opposite_infinities_and_of_two_nans():
    xs = [f32([INF, NEG_NAN_PAYLOAD, NEG_NAN_PAYLOAD, 1]), f32([NINF, POS_NAN_PAYLOAD, 2, NEG_NAN_PAYLOAD])]
    assert (u32(O.reduce_sum(xs)) == [CANON, CANON, CANON, CANON]).all()


def test_one_source_is_a_copy():
    x = f32([NEG_NAN_PAYLOAD, POS_NAN_PAYLOAD, INF])
    assert (u32(O.reduce_sum([x])) == u32(x)).all()
    assert (u32(O.reduce([x], O.OP_MAX)) == u32(x)).all()


def test_ops():
    xs = [f32([NEG_NAN_PAYLOAD, INF, 0x3F800000]), f32([0x3F800000, NINF, POS_NAN_PAYLOAD])]
    want = {O.OP_AVG: [CANON, CANON, CANON], O.OP_MAX: [CANON, INF, CANON], O.OP_MIN: [CANON, NINF, CANON]}
    for op, w in want.items():
        assert (u32(O.reduce(xs, op, 2)) == w).all(), op
    # AVG of one source divides: arithmetic, so canonical
    assert u32(O.reduce([f32([NEG_NAN_PAYLOAD])], O.OP_AVG, 3))[0] == CANON


def test_fp8_decode_of_an_inf_scaled_block():
    """Code 0 in a block whose scale is Inf decodes to 0 * Inf."""
    codes = np.zeros(256, np.uint8)
    scales = f32([INF])
    out = O.decode_accumulate([codes], [scales], O.CODEC_FP8)
    assert (u32(out) == CANON).all()
    # a NaN code (0xFF: negative) decodes to the canonical NaN as well
    codes[:] = 0xFF
    out = O.decode_accumulate([codes], [f32([0x3F800000])], O.CODEC_FP8)
    assert (u32(out) == CANON).all()


def test_bf16_decode_of_one_payload_widens_and_two_payloads_add():
    c = np.array([0xFFC1, 0x7FA0, 0x7F80], np.uint16)   # -NaN with payload, sNaN, +Inf
    one = O.decode_accumulate([c], None, O.CODEC_BF16)
    assert (u32(one) == c.astype(np.uint32) << 16).all()
    d = np.array([0x3F80, 0x3F80, 0xFF80], np.uint16)    # 1, 1, -Inf
    two = O.decode_accumulate([c, d], None, O.CODEC_BF16)
    assert (u32(two) == CANON).all()
    # accumulating into a buffer is arithmetic too
    acc = f32([NEG_NAN_PAYLOAD, 0, 0])
    got = O.decode_accumulate([np.array([0x3F80, 0x7FC1, 0x7F80], np.uint16)], None, O.CODEC_BF16, acc=acc)
    assert (u32(got) == [CANON, CANON, INF]).all()


def test_error_feedback_value_and_residual():
    """y = x + residual and the new residual: Inf - Inf, and a NaN x meeting a
    NaN residual of the other sign."""
    x = f32([INF, NEG_NAN_PAYLOAD, INF, 0x3F800000])
    r = f32([NINF, POS_NAN_PAYLOAD, 0, 0])
    codes, res = O.encode_bf16_ef(x, r)
    # y = canonical NaN, canonical NaN, Inf, 1: codes 0x7FC0, 0x7FC0, Inf, 1
    assert list(codes) == [0x7FC0, 0x7FC0, 0x7F80, 0x3F80]
    # residuals: NaN - NaN, NaN - NaN, Inf - Inf (invalid), 0
    assert (u32(res) == [CANON, CANON, CANON, 0]).all()
    for mode in (O.SCALE_ABSMAX_DIV_448, O.SCALE_POW2):
        xb = np.zeros(256, np.float32)
        rb = np.zeros(256, np.float32)
        xb[:4], rb[:4] = x, r
        codes, scales, res = O.encode_fp8_ef(xb, rb, mode)
        assert u32(scales)[0] == INF            # the block holds an Inf
        # NaN y encodes with y's sign, which is + for the canonical NaN
        assert list(codes[:2]) == [0x7F, 0x7F]
        # every residual of an Inf-scaled block is NaN (Inf / Inf, 0 * Inf)
        assert (u32(res) == CANON).all(), mode


def test_typed_totals_round_the_canonical_nan():
    """A NaN total reaches float16 / bfloat16 / float64 outputs as the
    conversion of 0x7FC00000: 0x7E00, 0x7FC0, 0x7FF8000000000000."""
    xs16 = [np.array([0x7C00], np.uint16), np.array([0xFC00], np.uint16)]   # +Inf, -Inf (float16)
    for dt, want in (("f16", 0x7E00), ("bf16", 0x7FC0)):
        src = xs16 if dt == "f16" else [np.array([0x7F80], np.uint16), np.array([0xFF80], np.uint16)]
        out, _, _ = O.bucket_allreduce_typed(src, dt, 256, O.CODEC_BF16)
        assert int(out[0]) == want, dt
    x64 = [np.array([np.inf]), np.array([-np.inf])]
    out, _, _ = O.bucket_allreduce_typed(x64, "f64", 256, O.CODEC_FP8)
    assert out.view(np.uint64)[0] == 0x7FF8000000000000
