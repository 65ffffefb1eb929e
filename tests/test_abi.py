"""The C-ABI library loads without a GPU, exports every symbol its header
declares, and its host-side logic (argument validation, sizes, workspace
layout, status strings) behaves as documented.  No call here reaches a
kernel: each one fails validation, or is a host-only query."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gbreduce.h")


@pytest.fixture(scope="module")
def gb():
    import gradient_all_reduce_amd as lib
    return lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gb_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for f in ["gb_reduce_sum", "gb_encode_bf16", "gb_encode_fp8_e4m3_blockscaled",
              "gb_decode_accumulate", "gb_bucket_allreduce_local"]:
        assert f in names


def test_library_exports_every_declared_symbol(gb):
    lib = ctypes.CDLL(gb.library_path)
    missing = [f for f in declared_functions() if not hasattr(lib, f)]
    assert not missing


def test_single_hip_runtime_in_process(gb):
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) <= 1, paths


def test_constants_match_header(gb):
    text = open(HEADER).read()
    for name in ["GB_BLOCK", "GB_MAX_K", "GB_VERSION"]:
        v = int(re.search(rf"#define {name} (\d+)", text).group(1))
        if name == "GB_VERSION":
            assert gb.gb_version() == v
        else:
            assert getattr(gb, name) == v
    for name in ["GB_OK", "GB_ERR_INVALID_ARG", "GB_ERR_MISALIGNED", "GB_ERR_UNSUPPORTED",
                 "GB_ERR_WORKSPACE", "GB_ERR_HIP", "GB_CODEC_NONE", "GB_CODEC_BF16",
                 "GB_CODEC_FP8_E4M3_B256", "GB_SCALE_ABSMAX_DIV_448", "GB_SCALE_POW2",
                 "GB_OP_SUM", "GB_OP_AVG", "GB_OP_MAX", "GB_OP_MIN"]:
        v = int(re.search(rf"\b{name} = (\d+)", text).group(1))
        assert getattr(gb, name) == v, name
    # element types: the header's gb_dtype, the binding's map and the oracle's numbering agree
    from oracle import oracle as O
    import torch
    names = {"F32": torch.float32, "F16": torch.float16, "BF16": torch.bfloat16, "F64": torch.float64,
             "I8": torch.int8, "U8": torch.uint8, "I32": torch.int32, "I64": torch.int64}
    for name, dt in names.items():
        v = int(re.search(rf"\bGB_DTYPE_{name} = (\d+)", text).group(1))
        assert gb.GB_DTYPE[dt] == v == O.DTYPES[name.lower()], name


def test_max_n_matches_header(gb):
    text = open(HEADER).read()
    shift = int(re.search(r"#define GB_MAX_N \(\(size_t\)1 << (\d+)\)", text).group(1))
    assert gb.GB_MAX_N == 1 << shift


def test_oversized_n_is_rejected_before_anything_else(gb):
    """n above GB_MAX_N fails as an invalid argument on every call that takes
    n, before any pointer is looked at, so no size computed from it can wrap."""
    L, big = gb._lib, gb.GB_MAX_N + 1
    calls = {
        "gb_reduce_sum": lambda: L.gb_reduce_sum(None, None, 2, big, None),
        "gb_reduce": lambda: L.gb_reduce(None, None, 2, big, 1, 2, None),
        "gb_reduce_typed": lambda: L.gb_reduce_typed(None, None, 2, big, 2, 0, 1, None),
        "gb_encode_bf16": lambda: L.gb_encode_bf16(None, None, big, None),
        "gb_encode_fp8_e4m3_blockscaled": lambda: L.gb_encode_fp8_e4m3_blockscaled(None, None, None, big, 0, None),
        "gb_decode_accumulate": lambda: L.gb_decode_accumulate(None, None, None, 2, big, 2, 0, None),
        "gb_encode": lambda: L.gb_encode(2, 0, None, None, None, big, 0, None),
        "gb_decode_sum": lambda: L.gb_decode_sum(0, None, None, None, 2, big, 2, None),
        "gb_reduce_encode": lambda: L.gb_reduce_encode(None, None, None, None, 2, big, 2, 0, None),
        "gb_encode_staged": lambda: L.gb_encode_staged(2, 0, None, None, None, None, None, big, 1 << 20, None),
        "gb_decode_accumulate_staged": lambda: L.gb_decode_accumulate_staged(None, None, None, None, None, 2, big,
                                                                             1 << 20, 2, 0, None),
        "gb_bucket_allreduce_local": lambda: L.gb_bucket_allreduce_local(None, None, 2, big, 256, 2, 0, None, 0,
                                                                         None),
        "gb_bucket_allreduce_local_typed": lambda: L.gb_bucket_allreduce_local_typed(0, None, None, 2, big, 256, 2,
                                                                                     0, None, 0, None),
        "gb_bucket_allreduce_local_ef": lambda: L.gb_bucket_allreduce_local_ef(None, None, None, 2, big, 256, 2, 0,
                                                                               None, 0, None),
        "gb_encode_bf16_ef": lambda: L.gb_encode_bf16_ef(None, None, None, big, None),
        "gb_encode_fp8_e4m3_blockscaled_ef": lambda: L.gb_encode_fp8_e4m3_blockscaled_ef(None, None, None, None, big,
                                                                                         0, None),
        "gb_encode_ef": lambda: L.gb_encode_ef(2, 2, None, None, None, None, big, 0, None),
        "gb_bucket_allreduce_local_ef_typed": lambda: L.gb_bucket_allreduce_local_ef_typed(2, None, None, None, 2, big,
                                                                                           256, 2, 0, None, 0, None),
    }
    for name, call in calls.items():
        assert call() == gb.GB_ERR_INVALID_ARG, name
        assert gb.gb_last_error().startswith(name + ":") and "exceeds GB_MAX_N" in gb.gb_last_error(), name
    for codec in (0, 1, 2):
        assert gb.gb_payload_bytes(codec, big) == 0
        assert gb.gb_payload_bytes(codec, gb.GB_MAX_N) > 0
        assert gb.gb_bucket_workspace_bytes(codec, 2, big, 256) == 0
    # the largest accepted n still sizes a workspace without wrapping
    assert gb.gb_bucket_workspace_bytes(2, 16, gb.GB_MAX_N, 256) == 16 * (gb.GB_MAX_N + 4 * gb.GB_MAX_N // 256)


def test_status_strings(gb):
    assert gb.gb_status_string(0) == "GB_OK"
    assert gb.gb_status_string(4) == "GB_ERR_WORKSPACE"
    assert gb.gb_status_string(99) == "unknown status"


def test_payload_bytes(gb):
    n = 67_108_864
    assert gb.gb_payload_bytes(gb.GB_CODEC_NONE, n) == 4 * n
    assert gb.gb_payload_bytes(gb.GB_CODEC_BF16, n) == 2 * n
    assert gb.gb_payload_bytes(gb.GB_CODEC_FP8_E4M3_B256, n) == n + 4 * (n // 256)
    assert gb.gb_payload_bytes(gb.GB_CODEC_FP8_E4M3_B256, 257) == 257 + 8
    assert gb.gb_payload_bytes(7, 10) == 0


def test_workspace_layout(gb):
    lay = gb.gb_bucket_workspace_layout(gb.GB_CODEC_FP8_E4M3_B256, 4, 1000, 256)
    assert lay == {"codes_stride": 1024, "scales_offset": 4096, "scales_stride": 256, "total": 5120}
    lay = gb.gb_bucket_workspace_layout(gb.GB_CODEC_BF16, 2, 1000, 512)
    assert lay == {"codes_stride": 2048, "scales_offset": 4096, "scales_stride": 0, "total": 4096}
    n, b = 1_000_000_000, 6_553_600
    total = gb.gb_bucket_workspace_bytes(gb.GB_CODEC_FP8_E4M3_B256, 4, n, b)
    assert total == 4 * (n + 4 * 3_906_250 + (256 - 4 * 3_906_250 % 256) % 256)
    assert gb.gb_bucket_workspace_bytes(gb.GB_CODEC_NONE, 4, n, b) == 0
    assert gb.gb_bucket_workspace_bytes(gb.GB_CODEC_FP8_E4M3_B256, 4, n, 100) == 0
    assert gb.gb_bucket_workspace_bytes(gb.GB_CODEC_FP8_E4M3_B256, 0, n, b) == 0
    with pytest.raises(gb.GbError):
        gb.gb_bucket_workspace_layout(9, 4, n, b)


# Raw calls with fake (never dereferenced) addresses: validation must reject
# them before any HIP call.
def _arr(*addrs):
    a = (ctypes.c_void_p * len(addrs))(*addrs)
    return ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))


@pytest.mark.parametrize("call,status,msg", [
    (lambda L: L.gb_reduce_sum(None, _arr(256), 0, 10, None), 1, "k = 0"),
    (lambda L: L.gb_reduce_sum(None, _arr(256), 17, 10, None), 1, "k = 17"),
    (lambda L: L.gb_reduce_sum(None, _arr(256), 1, 10, None), 1, "dst is NULL"),
    (lambda L: L.gb_reduce_sum(ctypes.c_void_p(260), _arr(256), 1, 10, None), 2, "dst"),
    (lambda L: L.gb_reduce_sum(ctypes.c_void_p(256), _arr(256, 0), 2, 10, None), 1, "srcs[1] is NULL"),
    (lambda L: L.gb_reduce_sum(ctypes.c_void_p(256), _arr(256, 264), 2, 10, None), 2, "srcs[1]"),
    (lambda L: L.gb_reduce_sum(ctypes.c_void_p(256), None, 2, 10, None), 1, "srcs array is NULL"),
    (lambda L: L.gb_encode_bf16(ctypes.c_void_p(258), ctypes.c_void_p(256), 10, None), 2, "codes"),
    (lambda L: L.gb_encode_fp8_e4m3_blockscaled(ctypes.c_void_p(256), ctypes.c_void_p(258),
                                                ctypes.c_void_p(256), 10, 0, None), 2, "scales"),
    (lambda L: L.gb_encode_fp8_e4m3_blockscaled(None, None, None, 10, 2, None), 3, "scale mode"),
    (lambda L: L.gb_decode_accumulate(ctypes.c_void_p(256), _arr(256), None, 1, 10, 5, 0, None), 3, "codec"),
    (lambda L: L.gb_decode_accumulate(ctypes.c_void_p(256), _arr(256), None, 1, 10, 1, 2, None), 1, "accumulate"),
    (lambda L: L.gb_decode_accumulate(ctypes.c_void_p(256), _arr(256), None, 1, 10, 2, 0, None), 1, "scales array"),
    (lambda L: L.gb_bucket_allreduce_local(ctypes.c_void_p(256), _arr(256), 1, 1000, 300, 0, 0,
                                           None, 0, None), 1, "bucket_elems"),
    (lambda L: L.gb_bucket_allreduce_local(ctypes.c_void_p(256), _arr(256), 1, 1000, 256, 2, 0,
                                           ctypes.c_void_p(512), 100, None), 4, "needed"),
    (lambda L: L.gb_bucket_allreduce_local(ctypes.c_void_p(256), _arr(256), 1, 1000, 256, 2, 0,
                                           ctypes.c_void_p(272), 1 << 20, None), 2, "workspace"),
    (lambda L: L.gb_bucket_allreduce_local(ctypes.c_void_p(256), _arr(256), 1, 1000, 256, 2, 5,
                                           ctypes.c_void_p(512), 1 << 20, None), 3, "scale mode"),
])
def test_validation_rejects_before_launch(gb, call, status, msg):
    assert call(gb._lib) == status
    assert msg in gb.gb_last_error()


@pytest.mark.parametrize("call,status,msg", [
    (lambda L: L.gb_reduce(ctypes.c_void_p(256), _arr(256), 1, 10, 7, 1, None), 3, "unknown op"),
    (lambda L: L.gb_reduce(ctypes.c_void_p(256), _arr(256), 1, 10, 1, 0, None), 1, "divisor"),
    (lambda L: L.gb_reduce(ctypes.c_void_p(256), _arr(256), 1, 10, 1, (1 << 24) + 1, None), 1, "divisor"),
    (lambda L: L.gb_reduce(ctypes.c_void_p(256), _arr(256), 0, 10, 2, 1, None), 1, "k = 0"),
    (lambda L: L.gb_reduce_typed(ctypes.c_void_p(256), _arr(256), 1, 10, 8, 0, 1, None), 3, "unknown dtype"),
    (lambda L: L.gb_reduce_typed(ctypes.c_void_p(256), _arr(256), 1, 10, -1, 0, 1, None), 3, "unknown dtype"),
    (lambda L: L.gb_reduce_typed(ctypes.c_void_p(256), _arr(256), 1, 10, 6, 1, 2, None), 3, "floating-point"),
    (lambda L: L.gb_reduce_typed(ctypes.c_void_p(256), _arr(256), 1, 10, 1, 4, 1, None), 3, "unknown op"),
    (lambda L: L.gb_reduce_typed(ctypes.c_void_p(256), _arr(256), 1, 10, 2, 1, 0, None), 1, "divisor"),
    (lambda L: L.gb_reduce_typed(ctypes.c_void_p(264), _arr(256), 1, 10, 4, 0, 1, None), 2, "dst"),
    (lambda L: L.gb_reduce_typed(ctypes.c_void_p(256), _arr(256, 257), 2, 10, 5, 2, 1, None), 2, "srcs[1]"),
    (lambda L: L.gb_reduce_typed(ctypes.c_void_p(256), _arr(256), 17, 10, 3, 0, 1, None), 1, "k = 17"),
    (lambda L: L.gb_decode_sum(1, ctypes.c_void_p(256), _arr(*[256] * 9), None, 9, 10, 1, None), 1,
     "rounded once from float32"),
    (lambda L: L.gb_bucket_allreduce_local_typed(2, ctypes.c_void_p(256), _arr(*[256] * 9), 9, 1000, 256, 2, 0,
                                                 ctypes.c_void_p(512), 1 << 24, None), 1, "rounded once"),
    (lambda L: L.gb_reduce_encode(None, ctypes.c_void_p(256), None, _arr(256), 1, 10, 0, 0, None), 3,
     "not bf16 or fp8"),
    (lambda L: L.gb_reduce_encode(None, ctypes.c_void_p(256), None, _arr(256), 1, 10, 2, 5, None), 3, "scale mode"),
    (lambda L: L.gb_reduce_encode(None, ctypes.c_void_p(256), None, _arr(*[256] * 9), 9, 10, 1, 0, None), 1,
     "sum first"),
    (lambda L: L.gb_reduce_encode(ctypes.c_void_p(264), ctypes.c_void_p(256), None, _arr(256), 1, 10, 1, 0, None), 2,
     "sum"),
    (lambda L: L.gb_reduce_encode(None, ctypes.c_void_p(256), ctypes.c_void_p(258), _arr(256), 1, 10, 2, 0, None), 2,
     "scales"),
    (lambda L: L.gb_encode(0, 1, None, None, None, 10, 0, None), 3, "not bf16 or fp8"),
    (lambda L: L.gb_encode(1, 6, None, None, None, 10, 0, None), 3, "not a floating-point type"),
    (lambda L: L.gb_encode(2, 2, None, None, None, 10, 3, None), 3, "scale mode"),
    (lambda L: L.gb_encode(2, 2, ctypes.c_void_p(256), ctypes.c_void_p(258), ctypes.c_void_p(256), 10, 0, None),
     2, "scales"),
    (lambda L: L.gb_encode(1, 3, ctypes.c_void_p(256), None, ctypes.c_void_p(264), 10, 0, None), 2, "src"),
    (lambda L: L.gb_decode_sum(1, ctypes.c_void_p(256), _arr(256), None, 1, 10, 0, None), 3, "uncompressed"),
    (lambda L: L.gb_decode_sum(4, ctypes.c_void_p(256), _arr(256), None, 1, 10, 1, None), 3, "floating-point"),
    (lambda L: L.gb_decode_sum(2, ctypes.c_void_p(256), _arr(256), None, 1, 10, 2, None), 1, "scales array"),
    (lambda L: L.gb_decode_sum(2, ctypes.c_void_p(256), _arr(256), None, 0, 10, 1, None), 1, "k = 0"),
    (lambda L: L.gb_bucket_allreduce_local_typed(7, ctypes.c_void_p(256), _arr(256), 1, 1000, 256, 2, 0,
                                                 ctypes.c_void_p(512), 1 << 20, None), 3, "floating-point"),
    (lambda L: L.gb_bucket_allreduce_local_typed(1, ctypes.c_void_p(256), _arr(256), 1, 1000, 300, 2, 0,
                                                 ctypes.c_void_p(512), 1 << 20, None), 1, "bucket_elems"),
    (lambda L: L.gb_bucket_allreduce_local_typed(2, ctypes.c_void_p(256), _arr(256), 1, 1000, 256, 2, 0,
                                                 ctypes.c_void_p(512), 100, None), 4, "needed"),
    (lambda L: L.gb_bucket_allreduce_local_ef(ctypes.c_void_p(256), _arr(256), _arr(512), 1, 1000, 256, 0, 0,
                                              None, 0, None), 3, "lossy codec"),
    (lambda L: L.gb_bucket_allreduce_local_ef(ctypes.c_void_p(256), _arr(256), _arr(520), 1, 1000, 256, 2, 0,
                                              ctypes.c_void_p(512), 1 << 20, None), 2, "residuals[0]"),
    (lambda L: L.gb_encode_bf16_ef(ctypes.c_void_p(256), ctypes.c_void_p(264), ctypes.c_void_p(256), 10, None),
     2, "residual"),
    (lambda L: L.gb_encode_staged(0, 0, None, None, None, None, None, 10, 256, None), 3, "not bf16 or fp8"),
    (lambda L: L.gb_encode_staged(2, 0, None, None, None, None, None, 10, 100, None), 1, "chunk_elems"),
    (lambda L: L.gb_encode_staged(2, 9, None, None, None, None, None, 10, 256, None), 3, "scale mode"),
    (lambda L: L.gb_encode_staged(2, 0, ctypes.c_void_p(264), None, None, None, ctypes.c_void_p(256), 10, 256,
                                  None), 2, "codes_dev"),
    (lambda L: L.gb_decode_accumulate_staged(ctypes.c_void_p(256), None, None, None, None, 1, 10, 256, 1, 0, None),
     1, "pointer array"),
    (lambda L: L.gb_decode_accumulate_staged(ctypes.c_void_p(256), None, None, None, None, 1, 10, 0, 1, 0, None),
     1, "chunk_elems"),
    (lambda L: L.gb_decode_accumulate_staged(ctypes.c_void_p(256), None, None, None, None, 17, 10, 256, 1, 0, None),
     1, "k = 17"),
    (lambda L: L.gb_encode_ef(0, 2, None, None, None, None, 10, 0, None), 3, "not bf16 or fp8"),
    (lambda L: L.gb_encode_ef(2, 5, None, None, None, None, 10, 0, None), 3, "not a floating-point type"),
    (lambda L: L.gb_encode_ef(2, 2, None, None, None, None, 10, 7, None), 3, "scale mode"),
    (lambda L: L.gb_encode_ef(1, 1, ctypes.c_void_p(256), None, ctypes.c_void_p(264), ctypes.c_void_p(256), 10, 0,
                              None), 2, "residual"),
    (lambda L: L.gb_encode_ef(2, 3, ctypes.c_void_p(256), None, ctypes.c_void_p(256), ctypes.c_void_p(256), 10, 0,
                              None), 1, "scales is NULL"),
    (lambda L: L.gb_bucket_allreduce_local_ef_typed(6, ctypes.c_void_p(256), _arr(256), _arr(512), 1, 1000, 256, 2,
                                                    0, ctypes.c_void_p(512), 1 << 20, None), 3, "floating-point"),
    (lambda L: L.gb_bucket_allreduce_local_ef_typed(2, ctypes.c_void_p(256), _arr(256), _arr(512), 1, 1000, 256, 0,
                                                    0, None, 0, None), 3, "lossy codec"),
    (lambda L: L.gb_bucket_allreduce_local_ef_typed(2, ctypes.c_void_p(256), _arr(*[256] * 9), _arr(*[512] * 9), 9,
                                                    1000, 256, 2, 0, ctypes.c_void_p(512), 1 << 24, None), 1,
     "k = 9"),
    (lambda L: L.gb_bucket_allreduce_local_ef_typed(1, ctypes.c_void_p(256), _arr(256), _arr(516), 1, 1000, 256, 1,
                                                    0, ctypes.c_void_p(512), 1 << 20, None), 2, "residuals[0]"),
])
def test_validation_of_the_wider_calls(gb, call, status, msg):
    assert call(gb._lib) == status
    assert msg in gb.gb_last_error()


def _sizes(*ns):
    a = (ctypes.c_size_t * len(ns))(*ns)
    return ctypes.cast(a, ctypes.POINTER(ctypes.c_size_t))


_BIG_WS = (ctypes.c_void_p(1 << 20), 1 << 30)


def _batch(L, *a, divisor=1):
    """gb_bucket_allreduce_local_batch(dtype, outs, srcs, ns, nbuckets, k, codec, scale_mode, divisor, ...)."""
    return L.gb_bucket_allreduce_local_batch(*a[:8], divisor, *a[8:])


def _batch_ef(L, *a, divisor=1):
    """gb_bucket_allreduce_local_batch_ef(dtype, outs, srcs, residuals, ns, nbuckets, k, codec, scale_mode,
    divisor, ...)."""
    return L.gb_bucket_allreduce_local_batch_ef(*a[:9], divisor, *a[9:])


@pytest.mark.parametrize("call,status,msg", [
    (lambda L: _batch(L, 0, _arr(256), _arr(256), _sizes(10), 1, 1, 5, 0, *_BIG_WS, None), 3,
     "unknown codec"),
    (lambda L: _batch(L, 0, _arr(256), _arr(256), _sizes(10), 1, 1, 2, 4, *_BIG_WS, None), 3,
     "scale mode"),
    (lambda L: _batch(L, 0, _arr(256), _arr(256), _sizes(10), 1, 0, 2, 0, *_BIG_WS, None), 1,
     "k = 0"),
    (lambda L: _batch(L, 0, _arr(256), _arr(256), _sizes(10), 0, 1, 2, 0, *_BIG_WS, None), 1,
     "nbuckets = 0"),
    (lambda L: _batch(L, 0, _arr(256), _arr(256), _sizes(10), 4097, 1, 2, 0, *_BIG_WS, None), 1,
     "nbuckets = 4097"),
    (lambda L: _batch(L, 0, _arr(256), _arr(256), None, 1, 1, 2, 0, *_BIG_WS, None), 1,
     "ns is NULL"),
    (lambda L: _batch(L, 0, _arr(256, 512), _arr(256, 512), _sizes(10, (1 << 39) + 1), 2, 1,
                                                 2, 0, *_BIG_WS, None), 1, "ns[1]"),
    (lambda L: _batch(L, 0, _arr(256, 512), _arr(256, 512), _sizes(1 << 39, 1), 2, 1, 2, 0,
                                                 *_BIG_WS, None), 1, "exceed GB_MAX_N"),
    (lambda L: _batch(L, 0, None, _arr(256), _sizes(10), 1, 1, 2, 0, *_BIG_WS, None), 1,
     "outs or srcs is NULL"),
    (lambda L: _batch(L, 0, _arr(256, 264), _arr(256, 512), _sizes(10, 10), 2, 1, 2, 0,
                                                 *_BIG_WS, None), 2, "outs[1]"),
    (lambda L: _batch(L, 0, _arr(256, 0), _arr(256, 512), _sizes(10, 10), 2, 1, 2, 0,
                                                 *_BIG_WS, None), 1, "outs[1] is NULL"),
    (lambda L: _batch(L, 0, _arr(256, 512), _arr(256, 512, 768, 1032), _sizes(10, 10), 2, 2,
                                                 2, 0, *_BIG_WS, None), 2, "srcs[1 * k + r][1]"),
    (lambda L: _batch(L, 0, _arr(256), _arr(256), _sizes(1000), 1, 1, 2, 0,
                                                 ctypes.c_void_p(1 << 20), 100, None), 4, "needed"),
    (lambda L: _batch(L, 0, _arr(256), _arr(256), _sizes(1000), 1, 1, 1, 0, None, 0, None), 4,
     "needed"),
    (lambda L: _batch(L, 0, _arr(256), _arr(256), _sizes(1000), 1, 1, 2, 0,
                                                 ctypes.c_void_p((1 << 20) + 16), 1 << 30, None), 2, "workspace"),
])
def test_validation_of_the_batched_bucket_call(gb, call, status, msg):
    assert call(gb._lib) == status
    assert msg in gb.gb_last_error()


@pytest.mark.parametrize("call,status,msg", [
    (lambda L: _batch(L, 4, _arr(256), _arr(256), _sizes(10), 1, 1, 2, 0, *_BIG_WS, None), 3,
     "floating-point"),
    (lambda L: _batch(L, 2, _arr(256), _arr(*[256] * 9), _sizes(10), 1, 9, 2, 0, *_BIG_WS,
                                                 None), 1, "rounded once"),
    (lambda L: _batch(L, 3, _arr(256), _arr(256, 264), _sizes(10), 1, 2, 1, 0, *_BIG_WS,
                                                 None), 2, "srcs[0 * k + r][1]"),
])
def test_validation_of_the_typed_batched_bucket_call(gb, call, status, msg):
    assert call(gb._lib) == status
    assert msg in gb.gb_last_error()


@pytest.mark.parametrize("call,status,msg", [
    (lambda L: _batch(L, 0, _arr(256), _arr(256), _sizes(10), 1, 1, 2, 0, *_BIG_WS, None, divisor=0), 1, "divisor 0"),
    (lambda L: _batch(L, 0, _arr(256), _arr(256), _sizes(10), 1, 1, 2, 0, *_BIG_WS, None, divisor=(1 << 24) + 1), 1,
     "divisor"),
    (lambda L: _batch_ef(L, 0, _arr(256), _arr(256), _arr(512), _sizes(10), 1, 1, 1, 0, *_BIG_WS, None,
                         divisor=-3), 1, "divisor -3"),
])
def test_validation_of_the_batched_divisor(gb, call, status, msg):
    assert call(gb._lib) == status
    assert msg in gb.gb_last_error()


@pytest.mark.parametrize("call,status,msg", [
    (lambda L: _batch_ef(L, 0, _arr(256), _arr(256), None, _sizes(10), 1, 1, 2, 0,
                                                    *_BIG_WS, None), 1, "residuals is NULL"),
    (lambda L: _batch_ef(L, 0, _arr(256), _arr(256), _arr(512), _sizes(10), 1, 1, 0, 0,
                                                    *_BIG_WS, None), 3, "lossy codec"),
    (lambda L: _batch_ef(L, 0, _arr(256, 768), _arr(256, 1024), _arr(512, 1288),
                                                    _sizes(10, 10), 2, 1, 2, 0, *_BIG_WS, None), 2,
     "residuals[1 * k + r][0]"),
    (lambda L: _batch_ef(L, 2, _arr(256), _arr(*[256] * 9), _arr(*[512] * 9), _sizes(10), 1,
                                                    9, 1, 0, *_BIG_WS, None), 1, "rounded once"),
    (lambda L: _batch_ef(L, 0, _arr(256), _arr(256), _arr(512), _sizes(1000), 1, 1, 2, 0,
                                                    ctypes.c_void_p(1 << 20), 100, None), 4, "needed"),
])
def test_validation_of_the_batched_error_feedback_call(gb, call, status, msg):
    assert call(gb._lib) == status
    assert msg in gb.gb_last_error()


def test_batched_bucket_call_skips_empty_buckets_and_sizes_its_workspace(gb):
    L = gb._lib
    # every bucket empty: nothing to do, no pointer read
    assert _batch(L, 0, None, None, _sizes(0, 0, 0), 3, 4, 2, 0, None, 0, None) == 0
    # an empty bucket's pointers are not read: only bucket 1's are checked (and misaligned here)
    assert _batch(L, 0, _arr(0, 264), _arr(0, 256), _sizes(0, 10), 2, 1, 2, 0,
                                             *_BIG_WS, None) == 2
    assert "outs[1]" in gb.gb_last_error()
    # the workspace is that of one buffer of the sizes rounded up to 256 values each
    ns = [1000, 0, 256, 513, 1]
    total = sum((v + 255) // 256 * 256 for v in ns)
    for codec in (1, 2):
        for k in (1, 4, 9):
            assert gb.gb_bucket_batch_workspace_bytes(codec, k, ns) == gb.gb_bucket_workspace_bytes(codec, k, total, 256)
    assert gb.gb_bucket_batch_workspace_bytes(0, 4, ns) == 0
    assert gb.gb_bucket_batch_workspace_bytes(2, 4, []) == 0
    assert gb.gb_bucket_batch_workspace_bytes(2, 17, ns) == 0


def test_max_batch_matches_header(gb):
    text = open(HEADER).read()
    assert gb.GB_MAX_BATCH == int(re.search(r"#define GB_MAX_BATCH (\d+)", text).group(1))


def test_zero_length_returns_ok_without_pointers(gb):
    L = gb._lib
    assert L.gb_reduce_sum(None, None, 2, 0, None) == 0
    assert L.gb_reduce_typed(None, None, 2, 0, 7, 2, 1, None) == 0
    assert L.gb_encode(2, 1, None, None, None, 0, 0, None) == 0
    assert L.gb_reduce_encode(None, None, None, None, 3, 0, 2, 0, None) == 0
    assert L.gb_decode_sum(3, None, None, None, 2, 0, 2, None) == 0
    assert L.gb_bucket_allreduce_local_typed(2, None, None, 2, 0, 256, 2, 0, None, 0, None) == 0
    assert L.gb_encode_bf16(None, None, 0, None) == 0
    assert L.gb_encode_fp8_e4m3_blockscaled(None, None, None, 0, 0, None) == 0
    assert L.gb_decode_accumulate(None, None, None, 3, 0, 2, 0, None) == 0
    assert L.gb_bucket_allreduce_local(None, None, 2, 0, 256, 2, 0, None, 0, None) == 0
    assert L.gb_encode_ef(2, 2, None, None, None, None, 0, 0, None) == 0
    assert L.gb_bucket_allreduce_local_ef_typed(2, None, None, None, 2, 0, 256, 2, 0, None, 0, None) == 0


def test_header_compiles_and_links_from_plain_c(gb, tmp_path):
    """The header is plain C (C11, no C++), and a C program linked against the
    library calls its host-only functions."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    src = tmp_path / "use_gbreduce.c"
    src.write_text(r'''
#include <stdio.h>
#include "gbreduce.h"
int main(void) {
  size_t cs = 0, so = 0, ss = 0, total = 0;
  gb_status s = gb_bucket_workspace_layout(GB_CODEC_FP8_E4M3_B256, 4, 1000, 256, &cs, &so, &ss, &total);
  printf("%d %d %zu %zu %zu %zu %zu %s\n", gb_version(), (int)s, cs, so, ss, total,
         gb_payload_bytes(GB_CODEC_FP8_E4M3_B256, 1000), gb_status_string(GB_ERR_WORKSPACE));
  return gb_reduce_sum(NULL, NULL, 0, 10, NULL) == GB_ERR_INVALID_ARG ? 0 : 1;
}
''')
    exe = tmp_path / "use_gbreduce"
    libdir = os.path.dirname(gb.library_path)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", libdir, "-l:libgbreduce.so", f"-Wl,-rpath,{libdir}"],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    v, s, cs, so, ss, total, pb, name = r.stdout.split()
    assert int(v) == gb.gb_version() and int(s) == 0
    assert (int(cs), int(ss), int(total)) == (1024, 256, 4 * (1024 + 256)) and int(so) == 4 * 1024
    assert int(pb) == 1000 + 4 * 4 and name == "GB_ERR_WORKSPACE"
