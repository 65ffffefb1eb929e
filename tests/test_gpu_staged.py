"""GPU parity of the staged (pipelined) leader steps: encode into pinned host
memory chunk by chunk, and decode-accumulate from pinned host memory chunk by
chunk.  The payloads and sums must equal the oracle's one-shot results."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from oracle import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

DEV = "cuda:0"


@pytest.fixture(scope="module")
def gb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_all_reduce_amd as lib
    return lib


def pinned(n, dtype):
    return torch.empty(n, dtype=dtype, pin_memory=True)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("n,chunk", [(1, 256), (1000, 256), (65536 + 7, 4096), (3 * 262144 + 5, 1 << 20),
                                     (3 * 262144 + 5, 256 * 1000)])
def test_encode_staged_fp8(gb, n, chunk, mode):
    x = W.gradients(n, 1100) if n >= 100 else W.normal(n, 1100)
    nb = O.nblocks(n)
    cd = torch.empty(n, dtype=torch.uint8, device=DEV)
    sd = torch.empty(nb, device=DEV)
    ch, sh = pinned(n, torch.uint8), pinned(nb, torch.float32)
    gb.gb_encode_staged(gb.GB_CODEC_FP8_E4M3_B256, cd, sd, ch, sh, torch.from_numpy(x).to(DEV), chunk, mode)
    torch.cuda.current_stream().synchronize()
    wc, ws = O.encode_fp8(x, mode)
    assert (ch.numpy() == wc).all() and (cd.cpu().numpy() == wc).all()
    assert (sh.numpy().view(np.uint32) == ws.view(np.uint32)).all()


@pytest.mark.parametrize("n,chunk", [(5, 256), (65536 + 7, 4096), (3 * 262144 + 5, 1 << 20)])
def test_encode_staged_bf16(gb, n, chunk):
    x = W.gradients(n, 1200) if n >= 100 else W.normal(n, 1200)
    cd = torch.empty(n, dtype=torch.uint16, device=DEV)
    ch = pinned(n, torch.uint16)
    gb.gb_encode_staged(gb.GB_CODEC_BF16, cd, None, ch, None, torch.from_numpy(x).to(DEV), chunk)
    torch.cuda.current_stream().synchronize()
    assert (ch.view(torch.int16).numpy().view(np.uint16) == O.encode_bf16(x)).all()


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("codec", [0, 1, 2])
@pytest.mark.parametrize("k,n,chunk", [(1, 300, 256), (3, 65536 + 7, 4096), (4, 3 * 262144 + 5, 1 << 20)])
def test_decode_accumulate_staged(gb, k, n, chunk, codec, accumulate):
    xs = W.gradient_ranks(k, n, 1300)
    nb = O.nblocks(n)
    if codec == 0:
        hosts = [torch.from_numpy(x).pin_memory() for x in xs]
        devs = [torch.empty(n, device=DEV) for _ in range(k)]
        sh = sd = None
        payloads, scales = xs, None
    elif codec == 1:
        payloads = [O.encode_bf16(x) for x in xs]
        hosts = [torch.from_numpy(p.view(np.int16)).view(torch.uint16).pin_memory() for p in payloads]
        devs = [torch.empty(n, dtype=torch.uint16, device=DEV) for _ in range(k)]
        sh = sd = None
        scales = None
    else:
        enc = [O.encode_fp8(x, 0) for x in xs]
        payloads, scales = [c for c, _ in enc], [s for _, s in enc]
        hosts = [torch.from_numpy(c).pin_memory() for c in payloads]
        devs = [torch.empty(n, dtype=torch.uint8, device=DEV) for _ in range(k)]
        sh = [torch.from_numpy(s).pin_memory() for s in scales]
        sd = [torch.empty(nb, device=DEV) for _ in range(k)]
    acc0 = W.normal(n, 7)
    acc = torch.from_numpy(acc0).to(DEV)
    gb.gb_decode_accumulate_staged(acc, hosts, sh, devs, sd, codec, chunk, accumulate)
    torch.cuda.current_stream().synchronize()
    want = O.decode_accumulate(payloads, scales, codec, acc=acc0 if accumulate else None)
    assert (acc.cpu().numpy().view(np.uint32) == want.view(np.uint32)).all()


def test_staged_rejects_pageable_host_memory(gb):
    n = 4096
    x = torch.ones(n, device=DEV)
    cd = torch.empty(n, dtype=torch.uint8, device=DEV)
    sd = torch.empty(n // 256, device=DEV)
    ch_pageable = torch.empty(n, dtype=torch.uint8)
    sh = pinned(n // 256, torch.float32)
    st = gb._lib.gb_encode_staged(2, 0, ctypes.c_void_p(cd.data_ptr()), ctypes.c_void_p(sd.data_ptr()),
                                  ctypes.c_void_p(ch_pageable.data_ptr()), ctypes.c_void_p(sh.data_ptr()),
                                  ctypes.c_void_p(x.data_ptr()), n, 256,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == gb.GB_ERR_INVALID_ARG and "pinned" in gb.gb_last_error()
    # the runtime is left without a pending error: an ordinary call still works
    gb.gb_reduce_sum(x, [x])
    torch.cuda.synchronize()
