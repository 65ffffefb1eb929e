"""ctypes wrapper of the C oracle (test infrastructure only).

Every function takes and returns numpy arrays in host memory and calls
straight into oracle/libgboracle.so; no arithmetic of the method happens in
Python.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import this module.  The GPU library never does, and this module never
touches a GPU.

Codec numbers: 0 none (fp32 payload), 1 bf16, 2 fp8 E4M3 with one fp32 scale
per 256 values.  Scale modes: 0 absmax/448, 1 power of two.
"""
import ctypes
import os

import numpy as np

from . import build as _build

CODEC_NONE, CODEC_BF16, CODEC_FP8 = 0, 1, 2
OP_SUM, OP_AVG, OP_MAX, OP_MIN = 0, 1, 2, 3
DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3, "i8": 4, "u8": 5, "i32": 6, "i64": 7}
NP_DTYPES = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "f64": np.float64,
             "i8": np.int8, "u8": np.uint8, "i32": np.int32, "i64": np.int64}
SCALE_ABSMAX_DIV_448, SCALE_POW2 = 0, 1
BLOCK = 256

_lib = None
_P = ctypes.c_void_p
_S = ctypes.c_size_t
_I = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    sig = {
        "or_reduce_sum": (None, [_P, _P, _I, _S]),
        "or_bf16_encode_one": (ctypes.c_uint16, [ctypes.c_float]),
        "or_bf16_decode_one": (ctypes.c_float, [ctypes.c_uint16]),
        "or_encode_bf16": (None, [_P, _P, _S]),
        "or_e4m3_encode_one": (ctypes.c_uint8, [ctypes.c_float, _I]),
        "or_e4m3_decode_one": (ctypes.c_float, [ctypes.c_uint8]),
        "or_e4m3_encode_array": (None, [_P, _P, _S]),
        "or_e4m3_decode_array": (None, [_P, _P, _S]),
        "or_block_absmax": (ctypes.c_float, [_P, _S]),
        "or_block_scale": (ctypes.c_float, [ctypes.c_float, _I]),
        "or_fp8_quantize_one": (ctypes.c_uint8, [ctypes.c_float, ctypes.c_float]),
        "or_encode_fp8": (None, [_P, _P, _P, _S, _I]),
        "or_decode_accumulate": (None, [_P, _P, _P, _I, _S, _I, _I]),
        "or_bucket_allreduce": (None, [_P, _P, _P, _P, _I, _S, _S, _I, _I]),
        "or_reduce": (None, [_P, _P, _I, _S, _I, _I]),
        "or_reduce_typed": (None, [_P, _P, _I, _S, _I, _I, _I]),
        "or_encode_bf16_ef": (None, [_P, _P, _P, _S]),
        "or_encode_fp8_ef": (None, [_P, _P, _P, _P, _S, _I]),
        "or_bucket_allreduce_ef": (None, [_P, _P, _P, _P, _P, _I, _S, _S, _I, _I]),
        "or_encode_typed": (None, [_I, _I, _P, _P, _P, _S, _I]),
        "or_decode_sum_typed": (None, [_P, _I, _P, _P, _I, _S, _I]),
        "or_bucket_allreduce_typed": (None, [_P, _P, _P, _P, _I, _S, _S, _I, _I, _I]),
        "or_encode_ef_typed": (None, [_I, _I, _P, _P, _P, _P, _S, _I]),
        "or_bucket_allreduce_ef_typed": (None, [_P, _P, _P, _P, _P, _I, _S, _S, _I, _I, _I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _ptr_array(arrays):
    arr = (ctypes.c_void_p * len(arrays))()
    for i, a in enumerate(arrays):
        arr[i] = a.ctypes.data if a is not None else None
    return arr


def nblocks(n):
    return (n + BLOCK - 1) // BLOCK


def reduce_sum(xs):
    """Left fold over ranks of k equal-length fp32 arrays."""
    xs = [_f32(x) for x in xs]
    n = xs[0].size
    out = np.empty(n, dtype=np.float32)
    _load().or_reduce_sum(_ptr(out), _ptr_array(xs), len(xs), n)
    return out


def reduce(xs, op, divisor=1):
    """SUM, AVG (divided by `divisor`), MAX or MIN over ranks."""
    xs = [_f32(x) for x in xs]
    n = xs[0].size
    out = np.empty(n, dtype=np.float32)
    _load().or_reduce(_ptr(out), _ptr_array(xs), len(xs), n, int(op), int(divisor))
    return out


def reduce_typed(xs, dtype, op, divisor=1):
    """Reduce k arrays of element type `dtype` ("f32", "f16", "bf16", "f64",
    "i8", "u8", "i32", "i64"); f16 and bf16 arrays hold raw 16-bit codes."""
    nt = NP_DTYPES[dtype]
    xs = [np.ascontiguousarray(x, dtype=nt) for x in xs]
    n = xs[0].size
    out = np.empty(n, dtype=nt)
    _load().or_reduce_typed(_ptr(out), _ptr_array(xs), len(xs), n, DTYPES[dtype], int(op), int(divisor))
    return out


def encode_bf16(x):
    x = _f32(x)
    codes = np.empty(x.size, dtype=np.uint16)
    _load().or_encode_bf16(_ptr(codes), _ptr(x), x.size)
    return codes


def decode_bf16(codes):
    codes = np.ascontiguousarray(codes, dtype=np.uint16)
    out = np.zeros(codes.size, dtype=np.float32)
    _load().or_decode_accumulate(_ptr(out), _ptr_array([codes]), None, 1,
                                 codes.size, CODEC_BF16, 0)
    return out


def e4m3_encode(v):
    """E4M3 code of each value (scale 1), saturating, ties to even."""
    v = _f32(v)
    codes = np.empty(v.size, dtype=np.uint8)
    _load().or_e4m3_encode_array(_ptr(codes), _ptr(v), v.size)
    return codes


def e4m3_decode(codes):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.size, dtype=np.float32)
    _load().or_e4m3_decode_array(_ptr(out), _ptr(codes), codes.size)
    return out


def block_absmax(x):
    x = _f32(x)
    return np.float32(_load().or_block_absmax(_ptr(x), x.size))


def block_scale(a, mode):
    return np.float32(_load().or_block_scale(float(a), int(mode)))


def fp8_quantize_one(x, s):
    return int(_load().or_fp8_quantize_one(float(x), float(s)))


def encode_fp8(x, mode):
    """Block-scaled E4M3 encode: returns (codes uint8[n], scales fp32[B])."""
    x = _f32(x)
    codes = np.empty(x.size, dtype=np.uint8)
    scales = np.empty(nblocks(x.size), dtype=np.float32)
    _load().or_encode_fp8(_ptr(codes), _ptr(scales), _ptr(x), x.size, int(mode))
    return codes, scales


def decode_accumulate(codes, scales, codec, acc=None):
    """Decode k payloads and add in rank order.

    codes: list of k arrays (fp32 / uint16 / uint8 per codec); scales: list of
    k fp32 arrays for fp8, else None; acc: starting fp32 array (accumulate=1)
    or None (accumulate=0).
    """
    dt = {CODEC_NONE: np.float32, CODEC_BF16: np.uint16, CODEC_FP8: np.uint8}[codec]
    codes = [np.ascontiguousarray(c, dtype=dt) for c in codes]
    n = codes[0].size
    if codec == CODEC_FP8:
        scales = [_f32(s) for s in scales]
        sp = _ptr_array(scales)
    else:
        sp = None
    if acc is None:
        out = np.empty(n, dtype=np.float32)
        accumulate = 0
    else:
        out = _f32(acc).copy()
        accumulate = 1
    _load().or_decode_accumulate(_ptr(out), _ptr_array(codes), sp, len(codes), n,
                                 int(codec), accumulate)
    return out


def bucket_allreduce(xs, bucket_elems, codec, mode=SCALE_ABSMAX_DIV_448):
    """Bucket stream.  Returns (out, codes list, scales list or None)."""
    xs = [_f32(x) for x in xs]
    k = len(xs)
    n = xs[0].size
    out = np.empty(n, dtype=np.float32)
    if codec == CODEC_NONE:
        codes = [np.empty(0, dtype=np.float32) for _ in range(k)]
        scales = None
    elif codec == CODEC_BF16:
        codes = [np.empty(n, dtype=np.uint16) for _ in range(k)]
        scales = None
    else:
        codes = [np.empty(n, dtype=np.uint8) for _ in range(k)]
        nb = sum(nblocks(min(bucket_elems, n - s)) for s in range(0, n, bucket_elems))
        scales = [np.empty(nb, dtype=np.float32) for _ in range(k)]
    _load().or_bucket_allreduce(
        _ptr(out), _ptr_array(codes), _ptr_array(scales) if scales else None,
        _ptr_array(xs), k, n, int(bucket_elems), int(codec), int(mode))
    return out, codes, scales


def encode_bf16_ef(x, residual):
    """Error-feedback bf16 encode: returns (codes, new residual)."""
    x = _f32(x)
    res = _f32(residual).copy()
    codes = np.empty(x.size, dtype=np.uint16)
    _load().or_encode_bf16_ef(_ptr(codes), _ptr(res), _ptr(x), x.size)
    return codes, res


def encode_fp8_ef(x, residual, mode):
    """Error-feedback fp8 encode: returns (codes, scales, new residual)."""
    x = _f32(x)
    res = _f32(residual).copy()
    codes = np.empty(x.size, dtype=np.uint8)
    scales = np.empty(nblocks(x.size), dtype=np.float32)
    _load().or_encode_fp8_ef(_ptr(codes), _ptr(scales), _ptr(res), _ptr(x), x.size, int(mode))
    return codes, scales, res


def bucket_allreduce_ef(xs, residuals, bucket_elems, codec, mode=SCALE_ABSMAX_DIV_448):
    """Bucket stream with error feedback.  Returns (out, codes, scales or None,
    new residuals)."""
    xs = [_f32(x) for x in xs]
    res = [_f32(r).copy() for r in residuals]
    k, n = len(xs), xs[0].size
    out = np.empty(n, dtype=np.float32)
    if codec == CODEC_BF16:
        codes = [np.empty(n, dtype=np.uint16) for _ in range(k)]
        scales = None
    else:
        codes = [np.empty(n, dtype=np.uint8) for _ in range(k)]
        nb = sum(nblocks(min(bucket_elems, n - s)) for s in range(0, n, bucket_elems))
        scales = [np.empty(nb, dtype=np.float32) for _ in range(k)]
    _load().or_bucket_allreduce_ef(
        _ptr(out), _ptr_array(codes), _ptr_array(scales) if scales else None, _ptr_array(res),
        _ptr_array(xs), k, n, int(bucket_elems), int(codec), int(mode))
    return out, codes, scales, res


def _typed(x, dtype):
    return np.ascontiguousarray(x, dtype=NP_DTYPES[dtype])


def encode_typed(x, dtype, codec, mode=SCALE_ABSMAX_DIV_448):
    """Bridge encode of a float16 / bfloat16 / float64 (or float32) array:
    returns (codes, scales or None)."""
    x = _typed(x, dtype)
    n = x.size
    if codec == CODEC_BF16:
        codes, scales = np.empty(n, dtype=np.uint16), None
    else:
        codes, scales = np.empty(n, dtype=np.uint8), np.empty(nblocks(n), dtype=np.float32)
    _load().or_encode_typed(int(codec), DTYPES[dtype], _ptr(codes),
                            _ptr(scales) if scales is not None else None, _ptr(x), n, int(mode))
    return codes, scales


def decode_sum_typed(codes, scales, codec, dtype):
    """Rank-order binary32 sum of the decoded payloads, rounded once to dtype."""
    dt = {CODEC_BF16: np.uint16, CODEC_FP8: np.uint8}[codec]
    codes = [np.ascontiguousarray(c, dtype=dt) for c in codes]
    n = codes[0].size
    sp = _ptr_array([_f32(s) for s in scales]) if codec == CODEC_FP8 else None
    out = np.empty(n, dtype=NP_DTYPES[dtype])
    _load().or_decode_sum_typed(_ptr(out), DTYPES[dtype], _ptr_array(codes), sp, len(codes), n, int(codec))
    return out


def encode_ef_typed(x, residual, dtype, codec, mode=SCALE_ABSMAX_DIV_448):
    """Error-feedback encode of a float16 / bfloat16 / float64 (or float32)
    array with a binary32 residual: returns (codes, scales or None, new
    residual)."""
    x = _typed(x, dtype)
    res = _f32(residual).copy()
    n = x.size
    if codec == CODEC_BF16:
        codes, scales = np.empty(n, dtype=np.uint16), None
    else:
        codes, scales = np.empty(n, dtype=np.uint8), np.empty(nblocks(n), dtype=np.float32)
    _load().or_encode_ef_typed(int(codec), DTYPES[dtype], _ptr(codes),
                               _ptr(scales) if scales is not None else None, _ptr(res), _ptr(x), n, int(mode))
    return codes, scales, res


def bucket_allreduce_ef_typed(xs, residuals, dtype, bucket_elems, codec, mode=SCALE_ABSMAX_DIV_448):
    """Bucket stream with error feedback over arrays of dtype, binary32
    residuals.  Returns (out, codes, scales or None, new residuals)."""
    xs = [_typed(x, dtype) for x in xs]
    res = [_f32(r).copy() for r in residuals]
    k, n = len(xs), xs[0].size
    out = np.empty(n, dtype=NP_DTYPES[dtype])
    if codec == CODEC_BF16:
        codes, scales = [np.empty(n, dtype=np.uint16) for _ in range(k)], None
    else:
        codes = [np.empty(n, dtype=np.uint8) for _ in range(k)]
        nb = sum(nblocks(min(bucket_elems, n - s)) for s in range(0, n, bucket_elems))
        scales = [np.empty(nb, dtype=np.float32) for _ in range(k)]
    _load().or_bucket_allreduce_ef_typed(
        _ptr(out), _ptr_array(codes), _ptr_array(scales) if scales else None, _ptr_array(res),
        _ptr_array(xs), k, n, int(bucket_elems), int(codec), int(mode), DTYPES[dtype])
    return out, codes, scales, res


def bucket_allreduce_typed(xs, dtype, bucket_elems, codec, mode=SCALE_ABSMAX_DIV_448):
    """Bucket stream over arrays of dtype.  Returns (out, codes, scales or None)."""
    xs = [_typed(x, dtype) for x in xs]
    k, n = len(xs), xs[0].size
    out = np.empty(n, dtype=NP_DTYPES[dtype])
    if codec == CODEC_NONE:
        codes, scales = [np.empty(0, dtype=np.float32) for _ in range(k)], None
    elif codec == CODEC_BF16:
        codes, scales = [np.empty(n, dtype=np.uint16) for _ in range(k)], None
    else:
        codes = [np.empty(n, dtype=np.uint8) for _ in range(k)]
        nb = sum(nblocks(min(bucket_elems, n - s)) for s in range(0, n, bucket_elems))
        scales = [np.empty(nb, dtype=np.float32) for _ in range(k)]
    _load().or_bucket_allreduce_typed(
        _ptr(out), _ptr_array(codes), _ptr_array(scales) if scales else None, _ptr_array(xs), k, n,
        int(bucket_elems), int(codec), int(mode), DTYPES[dtype])
    return out, codes, scales
