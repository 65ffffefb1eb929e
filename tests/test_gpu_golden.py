"""Whole outputs of the host-drawn workloads at full size, in the launch
configuration the benchmark times, against SHA-256 hashes of the oracle's
outputs (tests/golden/hashes.json, written by tests/golden/make_hashes.py from
the oracle alone).  Complements the sampled checks of test_gpu_full_size.py:
every byte of every output is covered."""
import hashlib
import json
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import workloads as W  # noqa: E402

DEV = "cuda:0"
HASHES = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hashes.json")))["outputs"]


@pytest.fixture(scope="module")
def gb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_all_reduce_amd as lib
    return lib


def sha(t):
    if t.dtype in (torch.uint16, torch.bfloat16):
        t = t.view(torch.int16)
    return hashlib.sha256(t.cpu().numpy().tobytes()).hexdigest()


def test_two_rank_4mib(gb):
    x = [torch.from_numpy(a).to(DEV) for a in W.normal_ranks(2, W.TWO_RANK_N)]
    s = torch.empty(W.TWO_RANK_N, device=DEV)
    c = torch.empty(W.TWO_RANK_N, dtype=torch.uint16, device=DEV)
    d = torch.empty(W.TWO_RANK_N, device=DEV)
    gb.gb_reduce_sum(s, x)
    gb.gb_encode_bf16(c, s)
    gb.gb_decode_accumulate(d, [c], None, gb.GB_CODEC_BF16)
    assert sha(s) == HASHES["two_rank_4mib/sum"]
    assert sha(c) == HASHES["two_rank_4mib/bf16_codes"]
    assert sha(d) == HASHES["two_rank_4mib/decoded"]


def test_two_island_sweep(gb):
    for n in W.SWEEP_SIZES:
        x = [torch.from_numpy(a).to(DEV) for a in W.normal_ranks(2, n)]
        out = torch.empty(n, device=DEV)
        gb.gb_reduce_sum(out, x)
        assert sha(out) == HASHES[f"two_island_sweep/sum/{n}"], n
    n = W.SWEEP_SIZES[-1]
    x = [torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16) for a in W.typed_ranks(2, n, "bf16")]
    out = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    gb.gb_reduce_typed(out, x, gb.GB_OP_SUM)
    assert sha(out) == HASHES[f"two_island_sweep/bf16_sum/{n}"]


def test_gradients_64mib_bf16(gb):
    n = W.GRAD64_N
    x = [torch.from_numpy(a).to(DEV) for a in W.gradient_ranks(4, n)]
    codes = [torch.empty(n, dtype=torch.uint16, device=DEV) for _ in range(4)]
    out = torch.empty(n, device=DEV)
    for r in range(4):
        gb.gb_encode_bf16(codes[r], x[r])
    gb.gb_decode_accumulate(out, codes, None, gb.GB_CODEC_BF16)
    for r in range(4):
        assert sha(codes[r]) == HASHES[f"gradients_64mib/bf16_codes/{r}"], r
    assert sha(out) == HASHES["gradients_64mib/decoded_sum"]


@pytest.mark.parametrize("mode,tag", [(0, "absmax_div_448"), (1, "pow2")])
def test_gradients_256mib_fp8(gb, mode, tag):
    n = W.GRAD256_N
    x = [torch.from_numpy(a).to(DEV) for a in W.gradient_ranks(4, n)]
    codes = [torch.empty(n, dtype=torch.uint8, device=DEV) for _ in range(4)]
    scales = [torch.empty(n // 256, device=DEV) for _ in range(4)]
    out = torch.empty(n, device=DEV)
    for r in range(4):
        gb.gb_encode_fp8_e4m3_blockscaled(codes[r], scales[r], x[r], mode)
    gb.gb_decode_accumulate(out, codes, scales, gb.GB_CODEC_FP8_E4M3_B256)
    for r in range(4):
        assert sha(codes[r]) == HASHES[f"gradients_256mib/{tag}/fp8_codes/{r}"], r
        assert sha(scales[r]) == HASHES[f"gradients_256mib/{tag}/scales/{r}"], r
    assert sha(out) == HASHES[f"gradients_256mib/{tag}/decoded_sum"]
