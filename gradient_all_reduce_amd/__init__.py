"""Python binding of libgbreduce (include/gbreduce.h).

Argument marshalling only: each function takes torch tensors that live in
device memory, passes their data pointers, sizes and the current HIP stream
to the C function of the same name, and raises GbError on a failed status.
Every step of the arithmetic runs in the library's HIP kernels; there is no
other implementation to fall back to.  If the library was not built this
module raises ImportError on import.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (one runtime, one device context).
"""
import ctypes
import os

import torch

__all__ = [
    "GB_OK", "GB_ERR_INVALID_ARG", "GB_ERR_MISALIGNED", "GB_ERR_UNSUPPORTED",
    "GB_ERR_WORKSPACE", "GB_ERR_HIP", "GB_CODEC_NONE", "GB_CODEC_BF16",
    "GB_CODEC_FP8_E4M3_B256", "GB_SCALE_ABSMAX_DIV_448", "GB_SCALE_POW2",
    "GB_BLOCK", "GB_MAX_K", "GbError", "library_path", "gb_reduce_sum",
    "gb_encode_bf16", "gb_encode_fp8_e4m3_blockscaled", "gb_decode_accumulate",
    "gb_bucket_allreduce_local", "gb_payload_bytes", "gb_bucket_workspace_layout",
    "gb_bucket_workspace_bytes", "gb_status_string", "gb_last_error", "gb_version",
    "gb_encode_bf16_ef", "gb_encode_fp8_e4m3_blockscaled_ef", "gb_bucket_allreduce_local_ef",
    "gb_reduce", "GB_OP_SUM", "GB_OP_AVG", "GB_OP_MAX", "GB_OP_MIN",
    "gb_encode_staged", "gb_decode_accumulate_staged", "gb_reduce_typed", "GB_DTYPE", "GB_DTYPE_OF",
    "gb_encode", "gb_decode_sum", "gb_bucket_allreduce_local_typed", "gb_reduce_encode",
    "gb_bucket_allreduce_local_batch", "gb_bucket_allreduce_local_batch_ef", "gb_bucket_batch_workspace_bytes",
    "GB_MAX_BATCH", "gb_bucket_allreduce_local_noalloc", "GB_NOALLOC_SCRATCH_BYTES",
]

GB_OK, GB_ERR_INVALID_ARG, GB_ERR_MISALIGNED = 0, 1, 2
GB_ERR_UNSUPPORTED, GB_ERR_WORKSPACE, GB_ERR_HIP = 3, 4, 5
GB_CODEC_NONE, GB_CODEC_BF16, GB_CODEC_FP8_E4M3_B256 = 0, 1, 2
GB_SCALE_ABSMAX_DIV_448, GB_SCALE_POW2 = 0, 1
GB_OP_SUM, GB_OP_AVG, GB_OP_MAX, GB_OP_MIN = 0, 1, 2, 3
GB_BLOCK = 256
GB_MAX_K = 16
GB_MAX_N = 1 << 39  # largest element count a call accepts
GB_MAX_BATCH = 4096  # largest bucket count of gb_bucket_allreduce_local_batch
GB_NOALLOC_SCRATCH_BYTES = 64 << 20  # static payload scratch of gb_bucket_allreduce_local_noalloc
# gb_dtype of each torch element type gb_reduce_typed takes
GB_DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.float64: 3,
            torch.int8: 4, torch.uint8: 5, torch.int32: 6, torch.int64: 7}
# the same numbers by short name
GB_DTYPE_OF = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3, "i8": 4, "u8": 5, "i32": 6, "i64": 7}

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgbreduce.so")
if not os.path.exists(library_path):
    raise ImportError(
        f"libgbreduce is not built ({library_path} is missing); build it with "
        "`python gradient_all_reduce_amd/build.py` or __graft_entry__.build()")

_lib = ctypes.CDLL(library_path)

_P, _S, _I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_PP = ctypes.POINTER(ctypes.c_void_p)
_SP = ctypes.POINTER(ctypes.c_size_t)
_SIGNATURES = {
    "gb_reduce_sum": (_I, [_P, _PP, _I, _S, _P]),
    "gb_reduce": (_I, [_P, _PP, _I, _S, _I, _I, _P]),
    "gb_reduce_typed": (_I, [_P, _PP, _I, _S, _I, _I, _I, _P]),
    "gb_encode": (_I, [_I, _I, _P, _P, _P, _S, _I, _P]),
    "gb_reduce_encode": (_I, [_P, _P, _P, _PP, _I, _S, _I, _I, _P]),
    "gb_decode_sum": (_I, [_I, _P, _PP, _PP, _I, _S, _I, _P]),
    "gb_bucket_allreduce_local_typed": (_I, [_I, _P, _PP, _I, _S, _S, _I, _I, _P, _S, _P]),
    "gb_encode_bf16": (_I, [_P, _P, _S, _P]),
    "gb_encode_fp8_e4m3_blockscaled": (_I, [_P, _P, _P, _S, _I, _P]),
    "gb_decode_accumulate": (_I, [_P, _PP, _PP, _I, _S, _I, _I, _P]),
    "gb_bucket_allreduce_local": (_I, [_P, _PP, _I, _S, _S, _I, _I, _P, _S, _P]),
    "gb_bucket_allreduce_local_noalloc": (_I, [_P, _PP, _I, _S, _S, _I, _I, _P]),
    "gb_bucket_allreduce_local_batch": (_I, [_I, _PP, _PP, _SP, _I, _I, _I, _I, _I, _P, _S, _P]),
    "gb_bucket_allreduce_local_batch_ef": (_I, [_I, _PP, _PP, _PP, _SP, _I, _I, _I, _I, _I, _P, _S, _P]),
    "gb_bucket_batch_workspace_bytes": (_S, [_I, _I, _SP, _I]),
    "gb_encode_bf16_ef": (_I, [_P, _P, _P, _S, _P]),
    "gb_encode_fp8_e4m3_blockscaled_ef": (_I, [_P, _P, _P, _P, _S, _I, _P]),
    "gb_bucket_allreduce_local_ef": (_I, [_P, _PP, _PP, _I, _S, _S, _I, _I, _P, _S, _P]),
    "gb_encode_ef": (_I, [_I, _I, _P, _P, _P, _P, _S, _I, _P]),
    "gb_bucket_allreduce_local_ef_typed": (_I, [_I, _P, _PP, _PP, _I, _S, _S, _I, _I, _P, _S, _P]),
    "gb_encode_staged": (_I, [_I, _I, _P, _P, _P, _P, _P, _S, _S, _P]),
    "gb_decode_accumulate_staged": (_I, [_P, _PP, _PP, _PP, _PP, _I, _S, _S, _I, _I, _P]),
    "gb_payload_bytes": (_S, [_I, _S]),
    "gb_bucket_workspace_layout": (_I, [_I, _I, _S, _S, _SP, _SP, _SP, _SP]),
    "gb_bucket_workspace_bytes": (_S, [_I, _I, _S, _S]),
    "gb_status_string": (ctypes.c_char_p, [_I]),
    "gb_last_error": (ctypes.c_char_p, []),
    "gb_version": (_I, []),
}
for _name, (_res, _args) in _SIGNATURES.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class GbError(RuntimeError):
    """A libgbreduce call returned a failed gb_status."""

    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{gb_status_string(status)}: {detail}")


def _check(status):
    if status != GB_OK:
        raise GbError(status, gb_last_error())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _ptr_array(ts):
    arr = (ctypes.c_void_p * max(1, len(ts)))()
    for i, t in enumerate(ts):
        arr[i] = t.data_ptr() if t is not None else None
    return ctypes.cast(arr, _PP)


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _device_tensor(t, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be in device memory, not on {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_numel(ts, n, name):
    for i, t in enumerate(ts):
        if t.numel() != n:
            raise ValueError(f"{name}[{i}] has {t.numel()} elements, expected {n}")


_CODE_DTYPE = {GB_CODEC_NONE: torch.float32, GB_CODEC_BF16: torch.uint16,
               GB_CODEC_FP8_E4M3_B256: torch.uint8}


def gb_reduce_sum(dst, srcs, stream=None):
    """dst = srcs[0] + srcs[1] + ... in rank order (fp32, in place if dst is srcs[0])."""
    _device_tensor(dst, torch.float32, "dst")
    for i, s in enumerate(srcs):
        _device_tensor(s, torch.float32, f"srcs[{i}]")
    _same_numel(srcs, dst.numel(), "srcs")
    _check(_lib.gb_reduce_sum(_ptr(dst), _ptr_array(srcs), len(srcs), dst.numel(),
                              _stream(stream, dst.device)))


def gb_reduce(dst, srcs, op, divisor=1, stream=None):
    """dst = SUM, AVG (sum / divisor, the world size), MAX or MIN of srcs."""
    _device_tensor(dst, torch.float32, "dst")
    for i, s in enumerate(srcs):
        _device_tensor(s, torch.float32, f"srcs[{i}]")
    _same_numel(srcs, dst.numel(), "srcs")
    _check(_lib.gb_reduce(_ptr(dst), _ptr_array(srcs), len(srcs), dst.numel(), int(op), int(divisor),
                          _stream(stream, dst.device)))


def gb_reduce_typed(dst, srcs, op, divisor=1, stream=None):
    """gb_reduce over dst's element type (any key of GB_DTYPE); srcs share it."""
    if not isinstance(dst, torch.Tensor) or dst.dtype not in GB_DTYPE:
        raise TypeError(f"dst must be a tensor of one of {list(GB_DTYPE)}")
    _device_tensor(dst, dst.dtype, "dst")
    for i, s in enumerate(srcs):
        _device_tensor(s, dst.dtype, f"srcs[{i}]")
    _same_numel(srcs, dst.numel(), "srcs")
    _check(_lib.gb_reduce_typed(_ptr(dst), _ptr_array(srcs), len(srcs), dst.numel(), GB_DTYPE[dst.dtype],
                                int(op), int(divisor), _stream(stream, dst.device)))


def gb_reduce_encode(codec, codes, scales, srcs, sum=None, scale_mode=GB_SCALE_ABSMAX_DIV_448, stream=None):
    """The rank-order float32 sum of srcs encoded in one pass: codes (uint16
    for bf16, uint8 for fp8) and, for fp8, scales; the sum itself is stored in
    `sum` when given (required for more than 8 sources)."""
    for i, s in enumerate(srcs):
        _device_tensor(s, torch.float32, f"srcs[{i}]")
    n = srcs[0].numel() if srcs else 0
    _same_numel(srcs, n, "srcs")
    _device_tensor(codes, _CODE_DTYPE[int(codec)] if int(codec) in _CODE_DTYPE else torch.uint8, "codes")
    _same_numel([codes], n, "codes")
    if scales is not None:
        _device_tensor(scales, torch.float32, "scales")
        _same_numel([scales], (n + GB_BLOCK - 1) // GB_BLOCK, "scales")
    if sum is not None:
        _device_tensor(sum, torch.float32, "sum")
        _same_numel([sum], n, "sum")
    dev = srcs[0].device if srcs else codes.device
    _check(_lib.gb_reduce_encode(_ptr(sum), _ptr(codes), _ptr(scales), _ptr_array(srcs), len(srcs), n, int(codec),
                                 int(scale_mode), _stream(stream, dev)))


def gb_encode_bf16(codes, src, stream=None):
    """codes (uint16) = bf16 round-to-nearest-even of src (fp32)."""
    _device_tensor(codes, torch.uint16, "codes")
    _device_tensor(src, torch.float32, "src")
    _same_numel([codes], src.numel(), "codes")
    _check(_lib.gb_encode_bf16(_ptr(codes), _ptr(src), src.numel(), _stream(stream, src.device)))


def gb_encode_fp8_e4m3_blockscaled(codes, scales, src, scale_mode=GB_SCALE_ABSMAX_DIV_448,
                                   stream=None):
    """codes (uint8, E4M3) and scales (fp32, one per 256 values) of src (fp32)."""
    _device_tensor(codes, torch.uint8, "codes")
    _device_tensor(scales, torch.float32, "scales")
    _device_tensor(src, torch.float32, "src")
    n = src.numel()
    _same_numel([codes], n, "codes")
    _same_numel([scales], (n + GB_BLOCK - 1) // GB_BLOCK, "scales")
    _check(_lib.gb_encode_fp8_e4m3_blockscaled(_ptr(codes), _ptr(scales), _ptr(src), n,
                                               int(scale_mode), _stream(stream, src.device)))


def gb_decode_accumulate(acc, codes, scales, codec, accumulate=False, stream=None):
    """acc (fp32) = [acc +] decoded codes[0] + decoded codes[1] + ... in rank order."""
    _device_tensor(acc, torch.float32, "acc")
    n = acc.numel()
    dt = _CODE_DTYPE.get(int(codec))
    if dt is not None:
        for i, c in enumerate(codes):
            _device_tensor(c, dt, f"codes[{i}]")
        _same_numel(codes, n, "codes")
    if scales is not None:
        for i, s in enumerate(scales):
            _device_tensor(s, torch.float32, f"scales[{i}]")
        _same_numel(scales, (n + GB_BLOCK - 1) // GB_BLOCK, "scales")
    scale_ptrs = _ptr_array(scales) if scales is not None else None
    _check(_lib.gb_decode_accumulate(_ptr(acc), _ptr_array(codes), scale_ptrs, len(codes), n,
                                     int(codec), int(bool(accumulate)), _stream(stream, acc.device)))


def gb_bucket_allreduce_local(out, srcs, bucket_elems, codec, scale_mode=GB_SCALE_ABSMAX_DIV_448,
                              workspace=None, stream=None):
    """Bucket stream: per bucket, encode each rank, decode and add in rank order into out."""
    _device_tensor(out, torch.float32, "out")
    for i, s in enumerate(srcs):
        _device_tensor(s, torch.float32, f"srcs[{i}]")
    n = out.numel()
    _same_numel(srcs, n, "srcs")
    ws_bytes = 0
    if workspace is not None:
        _device_tensor(workspace, torch.uint8, "workspace")
        ws_bytes = workspace.numel()
    _check(_lib.gb_bucket_allreduce_local(_ptr(out), _ptr_array(srcs), len(srcs), n,
                                          int(bucket_elems), int(codec), int(scale_mode),
                                          _ptr(workspace), ws_bytes, _stream(stream, out.device)))


def gb_bucket_allreduce_local_noalloc(out, srcs, bucket_elems, codec, scale_mode=GB_SCALE_ABSMAX_DIV_448,
                                      stream=None):
    """gb_bucket_allreduce_local with the payloads in the library's static
    scratch (no workspace; at most GB_NOALLOC_SCRATCH_BYTES of payloads)."""
    _device_tensor(out, torch.float32, "out")
    for i, s in enumerate(srcs):
        _device_tensor(s, torch.float32, f"srcs[{i}]")
    n = out.numel()
    _same_numel(srcs, n, "srcs")
    _check(_lib.gb_bucket_allreduce_local_noalloc(_ptr(out), _ptr_array(srcs), len(srcs), n, int(bucket_elems),
                                                  int(codec), int(scale_mode), _stream(stream, out.device)))


def _size_array(ns):
    arr = (ctypes.c_size_t * max(1, len(ns)))(*[int(v) for v in ns])
    return ctypes.cast(arr, _SP)


def _batch_args(outs, srcs, residuals):
    if len(outs) != len(srcs):
        raise ValueError(f"{len(outs)} outputs for {len(srcs)} buckets of sources")
    if residuals is not None and len(residuals) != len(srcs):
        raise ValueError(f"{len(residuals)} buckets of residuals for {len(srcs)} buckets of sources")
    k = len(srcs[0]) if srcs else 0
    dtype = outs[0].dtype if outs else torch.float32
    if dtype not in _CODEC_TYPES:
        raise TypeError(f"outs must be tensors of one of {list(_CODEC_TYPES)}")
    ns, flat, flat_res = [], [], []
    for b, (o, ss) in enumerate(zip(outs, srcs)):
        _device_tensor(o, dtype, f"outs[{b}]")
        if len(ss) != k:
            raise ValueError(f"bucket {b} has {len(ss)} sources, bucket 0 has {k}")
        for r, t in enumerate(ss):
            _device_tensor(t, dtype, f"srcs[{b}][{r}]")
        _same_numel(ss, o.numel(), f"srcs[{b}]")
        if residuals is not None:
            if len(residuals[b]) != k:
                raise ValueError(f"bucket {b} has {len(residuals[b])} residuals for {k} sources")
            for r, t in enumerate(residuals[b]):
                _device_tensor(t, torch.float32, f"residuals[{b}][{r}]")
            _same_numel(residuals[b], o.numel(), f"residuals[{b}]")
            flat_res.extend(residuals[b])
        ns.append(o.numel())
        flat.extend(ss)
    return k, dtype, ns, flat, flat_res


def _workspace_args(workspace):
    if workspace is None:
        return _ptr(None), 0
    _device_tensor(workspace, torch.uint8, "workspace")
    return _ptr(workspace), workspace.numel()


def gb_bucket_allreduce_local_batch(outs, srcs, codec, scale_mode=GB_SCALE_ABSMAX_DIV_448,
                                    workspace=None, stream=None, divisor=1):
    """The bucket stream over separately allocated buckets: outs[b] receives
    bucket b's result from the k tensors srcs[b] (all float32, float16,
    bfloat16 or float64, of one type), as gb_bucket_allreduce_local_typed on
    that bucket alone; up to 16 buckets per launch.  divisor > 1 gives the
    AVG over that world size instead of the SUM."""
    k, dtype, ns, flat, _ = _batch_args(outs, srcs, None)
    device = outs[0].device if outs else torch.device("cuda", torch.cuda.current_device())
    _check(_lib.gb_bucket_allreduce_local_batch(GB_DTYPE[dtype], _ptr_array(outs), _ptr_array(flat),
                                                _size_array(ns), len(outs), k, int(codec), int(scale_mode),
                                                int(divisor), *_workspace_args(workspace),
                                                _stream(stream, device)))


def gb_bucket_allreduce_local_batch_ef(outs, srcs, residuals, codec, scale_mode=GB_SCALE_ABSMAX_DIV_448,
                                       workspace=None, stream=None, divisor=1):
    """gb_bucket_allreduce_local_batch with error feedback: residuals[b][r]
    (float32, one per source) is read and rewritten, as
    gb_bucket_allreduce_local_ef_typed on each bucket alone; up to 8 buckets
    per launch."""
    k, dtype, ns, flat, flat_res = _batch_args(outs, srcs, residuals)
    device = outs[0].device if outs else torch.device("cuda", torch.cuda.current_device())
    _check(_lib.gb_bucket_allreduce_local_batch_ef(GB_DTYPE[dtype], _ptr_array(outs), _ptr_array(flat),
                                                   _ptr_array(flat_res), _size_array(ns), len(outs), k,
                                                   int(codec), int(scale_mode), int(divisor),
                                                   *_workspace_args(workspace), _stream(stream, device)))


_CODEC_TYPES = (torch.float32, torch.float16, torch.bfloat16, torch.float64)


def _float_tensor(t, name):
    if not isinstance(t, torch.Tensor) or t.dtype not in _CODEC_TYPES:
        raise TypeError(f"{name} must be a tensor of one of {list(_CODEC_TYPES)}")
    _device_tensor(t, t.dtype, name)


def gb_encode(codec, codes, scales, src, scale_mode=GB_SCALE_ABSMAX_DIV_448, stream=None):
    """Bridge encode of src (float32, float16, bfloat16 or float64): codes
    (uint16 for bf16, uint8 for fp8) and, for fp8, scales (fp32)."""
    _float_tensor(src, "src")
    n = src.numel()
    _device_tensor(codes, _CODE_DTYPE[int(codec)] if int(codec) in _CODE_DTYPE else torch.uint8, "codes")
    _same_numel([codes], n, "codes")
    if scales is not None:
        _device_tensor(scales, torch.float32, "scales")
        _same_numel([scales], (n + GB_BLOCK - 1) // GB_BLOCK, "scales")
    _check(_lib.gb_encode(int(codec), GB_DTYPE[src.dtype], _ptr(codes), _ptr(scales), _ptr(src), n,
                          int(scale_mode), _stream(stream, src.device)))


def gb_decode_sum(dst, codes, scales, codec, stream=None):
    """dst (float32, float16, bfloat16 or float64) = the float32 rank-order sum
    of the decoded payloads, rounded once to dst's type."""
    _float_tensor(dst, "dst")
    n = dst.numel()
    dt = _CODE_DTYPE.get(int(codec))
    if dt is not None:
        for i, c in enumerate(codes):
            _device_tensor(c, dt, f"codes[{i}]")
        _same_numel(codes, n, "codes")
    if scales is not None:
        for i, sc in enumerate(scales):
            _device_tensor(sc, torch.float32, f"scales[{i}]")
    _check(_lib.gb_decode_sum(GB_DTYPE[dst.dtype], _ptr(dst), _ptr_array(codes),
                              _ptr_array(scales) if scales is not None else None, len(codes), n, int(codec),
                              _stream(stream, dst.device)))


def gb_bucket_allreduce_local_typed(out, srcs, bucket_elems, codec, scale_mode=GB_SCALE_ABSMAX_DIV_448,
                                    workspace=None, stream=None):
    """gb_bucket_allreduce_local over float32, float16, bfloat16 or float64
    buffers (out's type; srcs share it)."""
    _float_tensor(out, "out")
    for i, s in enumerate(srcs):
        _device_tensor(s, out.dtype, f"srcs[{i}]")
    n = out.numel()
    _same_numel(srcs, n, "srcs")
    ws_bytes = 0
    if workspace is not None:
        _device_tensor(workspace, torch.uint8, "workspace")
        ws_bytes = workspace.numel()
    _check(_lib.gb_bucket_allreduce_local_typed(GB_DTYPE[out.dtype], _ptr(out), _ptr_array(srcs), len(srcs), n,
                                                int(bucket_elems), int(codec), int(scale_mode), _ptr(workspace),
                                                ws_bytes, _stream(stream, out.device)))


def gb_encode_bf16_ef(codes, residual, src, stream=None):
    """Error-feedback bf16 encode: encodes src + residual, updates residual."""
    _device_tensor(codes, torch.uint16, "codes")
    _device_tensor(residual, torch.float32, "residual")
    _device_tensor(src, torch.float32, "src")
    _same_numel([codes, residual], src.numel(), "codes/residual")
    _check(_lib.gb_encode_bf16_ef(_ptr(codes), _ptr(residual), _ptr(src), src.numel(),
                                  _stream(stream, src.device)))


def gb_encode_fp8_e4m3_blockscaled_ef(codes, scales, residual, src, scale_mode=GB_SCALE_ABSMAX_DIV_448,
                                      stream=None):
    """Error-feedback fp8 encode: encodes src + residual, updates residual."""
    _device_tensor(codes, torch.uint8, "codes")
    _device_tensor(scales, torch.float32, "scales")
    _device_tensor(residual, torch.float32, "residual")
    _device_tensor(src, torch.float32, "src")
    n = src.numel()
    _same_numel([codes, residual], n, "codes/residual")
    _same_numel([scales], (n + GB_BLOCK - 1) // GB_BLOCK, "scales")
    _check(_lib.gb_encode_fp8_e4m3_blockscaled_ef(_ptr(codes), _ptr(scales), _ptr(residual), _ptr(src), n,
                                                  int(scale_mode), _stream(stream, src.device)))


def gb_bucket_allreduce_local_ef(out, srcs, residuals, bucket_elems, codec,
                                 scale_mode=GB_SCALE_ABSMAX_DIV_448, workspace=None, stream=None):
    """Bucket stream with error feedback: residuals[r] is updated for rank r."""
    _device_tensor(out, torch.float32, "out")
    n = out.numel()
    for name, ts in (("srcs", srcs), ("residuals", residuals)):
        for i, t in enumerate(ts):
            _device_tensor(t, torch.float32, f"{name}[{i}]")
        _same_numel(ts, n, name)
    if len(residuals) != len(srcs):
        raise ValueError("one residual per source is needed")
    ws_bytes = 0
    if workspace is not None:
        _device_tensor(workspace, torch.uint8, "workspace")
        ws_bytes = workspace.numel()
    _check(_lib.gb_bucket_allreduce_local_ef(_ptr(out), _ptr_array(srcs), _ptr_array(residuals), len(srcs), n,
                                             int(bucket_elems), int(codec), int(scale_mode), _ptr(workspace),
                                             ws_bytes, _stream(stream, out.device)))



def gb_encode_ef(codec, codes, scales, residual, src, scale_mode=GB_SCALE_ABSMAX_DIV_448, stream=None):
    """Error-feedback encode of src (float32, float16, bfloat16 or float64)
    with a float32 residual: encodes binary32(src) + residual into codes (and,
    for fp8, scales), updates residual."""
    _float_tensor(src, "src")
    n = src.numel()
    _device_tensor(codes, _CODE_DTYPE[int(codec)] if int(codec) in _CODE_DTYPE else torch.uint8, "codes")
    _device_tensor(residual, torch.float32, "residual")
    _same_numel([codes, residual], n, "codes/residual")
    if scales is not None:
        _device_tensor(scales, torch.float32, "scales")
        _same_numel([scales], (n + GB_BLOCK - 1) // GB_BLOCK, "scales")
    _check(_lib.gb_encode_ef(int(codec), GB_DTYPE[src.dtype], _ptr(codes), _ptr(scales), _ptr(residual), _ptr(src),
                             n, int(scale_mode), _stream(stream, src.device)))


def gb_bucket_allreduce_local_ef_typed(out, srcs, residuals, bucket_elems, codec,
                                       scale_mode=GB_SCALE_ABSMAX_DIV_448, workspace=None, stream=None):
    """gb_bucket_allreduce_local_ef over float32, float16, bfloat16 or float64
    gradients (out's type; srcs share it), float32 residuals."""
    _float_tensor(out, "out")
    n = out.numel()
    for i, t in enumerate(srcs):
        _device_tensor(t, out.dtype, f"srcs[{i}]")
    for i, t in enumerate(residuals):
        _device_tensor(t, torch.float32, f"residuals[{i}]")
    _same_numel(srcs, n, "srcs")
    _same_numel(residuals, n, "residuals")
    if len(residuals) != len(srcs):
        raise ValueError("one residual per source is needed")
    ws_bytes = 0
    if workspace is not None:
        _device_tensor(workspace, torch.uint8, "workspace")
        ws_bytes = workspace.numel()
    _check(_lib.gb_bucket_allreduce_local_ef_typed(GB_DTYPE[out.dtype], _ptr(out), _ptr_array(srcs),
                                                   _ptr_array(residuals), len(srcs), n, int(bucket_elems),
                                                   int(codec), int(scale_mode), _ptr(workspace), ws_bytes,
                                                   _stream(stream, out.device)))

def _host_pinned(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cpu" or not t.is_pinned():
        raise ValueError(f"{name} must be a pinned host tensor (pin_memory=True)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def gb_encode_staged(codec, codes_dev, scales_dev, codes_host, scales_host, src, chunk_elems,
                     scale_mode=GB_SCALE_ABSMAX_DIV_448, stream=None):
    """Encode src chunk by chunk, copying each chunk's payload to pinned host
    tensors while the next chunk is encoded."""
    _device_tensor(src, torch.float32, "src")
    dt = _CODE_DTYPE[int(codec)]
    _device_tensor(codes_dev, dt, "codes_dev")
    _host_pinned(codes_host, "codes_host")
    n = src.numel()
    _same_numel([codes_dev, codes_host], n, "codes")
    if scales_dev is not None:
        _device_tensor(scales_dev, torch.float32, "scales_dev")
        _host_pinned(scales_host, "scales_host")
        _same_numel([scales_dev, scales_host], (n + GB_BLOCK - 1) // GB_BLOCK, "scales")
    _check(_lib.gb_encode_staged(int(codec), int(scale_mode), _ptr(codes_dev), _ptr(scales_dev),
                                 _ptr(codes_host), _ptr(scales_host), _ptr(src), n, int(chunk_elems),
                                 _stream(stream, src.device)))


def gb_decode_accumulate_staged(acc, codes_host, scales_host, codes_dev, scales_dev, codec, chunk_elems,
                                accumulate=False, stream=None):
    """Copy k host payloads to device staging chunk by chunk while the
    previous chunk is decoded and accumulated into acc."""
    _device_tensor(acc, torch.float32, "acc")
    n = acc.numel()
    dt = _CODE_DTYPE[int(codec)]
    for i, (h, d) in enumerate(zip(codes_host, codes_dev)):
        _host_pinned(h, f"codes_host[{i}]")
        _device_tensor(d, dt, f"codes_dev[{i}]")
    _same_numel(list(codes_host) + list(codes_dev), n, "codes")
    if len(codes_host) != len(codes_dev):
        raise ValueError("one device staging buffer per host payload is needed")
    sh = sd = None
    if scales_host is not None:
        for i, (h, d) in enumerate(zip(scales_host, scales_dev)):
            _host_pinned(h, f"scales_host[{i}]")
            _device_tensor(d, torch.float32, f"scales_dev[{i}]")
        _same_numel(list(scales_host) + list(scales_dev), (n + GB_BLOCK - 1) // GB_BLOCK, "scales")
        sh, sd = _ptr_array(scales_host), _ptr_array(scales_dev)
    _check(_lib.gb_decode_accumulate_staged(_ptr(acc), _ptr_array(codes_host), sh, _ptr_array(codes_dev), sd,
                                            len(codes_host), n, int(chunk_elems), int(codec),
                                            int(bool(accumulate)), _stream(stream, acc.device)))


def gb_payload_bytes(codec, n):
    return int(_lib.gb_payload_bytes(int(codec), int(n)))


def gb_bucket_workspace_layout(codec, k, n, bucket_elems):
    """Return dict(codes_stride, scales_offset, scales_stride, total) in bytes."""
    out = [ctypes.c_size_t(0) for _ in range(4)]
    _check(_lib.gb_bucket_workspace_layout(int(codec), int(k), int(n), int(bucket_elems),
                                           *[ctypes.byref(o) for o in out]))
    return dict(zip(("codes_stride", "scales_offset", "scales_stride", "total"),
                    (o.value for o in out)))


def gb_bucket_workspace_bytes(codec, k, n, bucket_elems):
    return int(_lib.gb_bucket_workspace_bytes(int(codec), int(k), int(n), int(bucket_elems)))


def gb_bucket_batch_workspace_bytes(codec, k, ns):
    """Workspace bytes of gb_bucket_allreduce_local_batch over buckets of ns values."""
    return int(_lib.gb_bucket_batch_workspace_bytes(int(codec), int(k), _size_array(ns), len(ns)))


def gb_status_string(status):
    return _lib.gb_status_string(int(status)).decode()


def gb_last_error():
    return _lib.gb_last_error().decode()


def gb_version():
    return int(_lib.gb_version())
