"""Guard canaries around every buffer a call writes.

Each output (and each buffer a call reads and rewrites: an accumulated total,
an error-feedback residual, a workspace) is placed in the middle of a larger
allocation whose 4 KiB before and after it hold a poison byte.  After the call
and a synchronize, both guards must still hold the poison, and every output
must equal, byte for byte, the same call's output into plain allocations
(same inputs, same starting contents).  The sizes are ragged against each unit
the kernels work in: a 4-value vector, a 256-value fp8 block, a 1,024-value
vector group, a 4,096-value block group, and the last workgroup of a launch.
Parity of the values with the oracle is tested elsewhere; this checks that no
kernel writes outside the buffers a call is given."""
import pytest
import torch

import gradient_all_reduce_amd as gb

pytestmark = pytest.mark.gpu

GUARD = 4096
POISON = 0xA5
FILL = 0x5A
SIZES = [1, 3, 255, 257, 1023, 1025, 4095, 4097, 65537, (1 << 20) + 3]
FP8, BF16, NONE = gb.GB_CODEC_FP8_E4M3_B256, gb.GB_CODEC_BF16, gb.GB_CODEC_NONE


def nblocks(n):
    return (n + gb.GB_BLOCK - 1) // gb.GB_BLOCK


class Guarded:
    """`numel` values of `dtype` at byte GUARD of a poisoned allocation."""

    def __init__(self, numel, dtype, pinned):
        self.nbytes = numel * torch.empty(0, dtype=dtype).element_size()
        total = GUARD + self.nbytes + GUARD
        if pinned:
            self.raw = torch.empty(total, dtype=torch.uint8, pin_memory=True)
        else:
            self.raw = torch.empty(total, dtype=torch.uint8, device="cuda")
        self.raw.fill_(POISON)
        self.t = self.raw[GUARD:GUARD + self.nbytes].view(dtype)

    def intact(self):
        return (bool((self.raw[:GUARD] == POISON).all())
                and bool((self.raw[GUARD + self.nbytes:] == POISON).all()))


def allocator(guarded, guards):
    """alloc(numel, dtype, init=None, pinned=False): an output buffer, plain or
    guarded, filled with FILL bytes or a copy of init."""

    def alloc(numel, dtype, init=None, pinned=False):
        if guarded:
            g = Guarded(numel, dtype, pinned)
            guards.append(g)
            t = g.t
        elif pinned:
            t = torch.empty(numel, dtype=dtype, pin_memory=True)
        else:
            t = torch.empty(numel, dtype=dtype, device="cuda")
        if init is None:
            t.view(torch.uint8).fill_(FILL)
        else:
            t.copy_(init)
        return t

    return alloc


def check(call):
    """call(alloc) makes its outputs with alloc, runs one entry point and
    returns the buffers to compare."""
    plain = call(allocator(False, []))
    guards = []
    guarded = call(allocator(True, guards))
    torch.cuda.synchronize()
    bad = [i for i, g in enumerate(guards) if not g.intact()]
    assert not bad, f"guard bytes overwritten around output(s) {bad}"
    assert len(plain) == len(guarded)
    for i, (a, b) in enumerate(zip(plain, guarded)):
        assert torch.equal(a.view(torch.uint8).cpu(), b.view(torch.uint8).cpu()), f"output {i} differs"


def gen(seed):
    return torch.Generator(device="cuda").manual_seed(seed)


def floats(n, k, seed, dtype=torch.float32):
    g = gen(seed)
    xs = [(torch.randn(n, generator=g, device="cuda") * 1e-3).to(dtype) for _ in range(k)]
    if n > 7:
        for x in xs:  # a few values far from the rest, so blocks differ in scale
            x[::7] *= 1000
    return xs


def ints(n, k, seed, dtype):
    g = gen(seed)
    lo, hi = {torch.int8: (-128, 128), torch.uint8: (0, 256)}.get(dtype, (-(1 << 30), 1 << 30))
    return [torch.randint(lo, hi, (n,), generator=g, device="cuda", dtype=torch.int64).to(dtype) for _ in range(k)]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("k", [1, 2, 4, 9])
def test_reduce_sum(n, k):
    xs = floats(n, k, 1)

    def call(alloc):
        out = alloc(n, torch.float32)
        gb.gb_reduce_sum(out, xs)
        return [out]

    check(call)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("op,div", [(gb.GB_OP_AVG, 3), (gb.GB_OP_MAX, 1), (gb.GB_OP_MIN, 1)])
def test_reduce_op(n, op, div):
    xs = floats(n, 3, 2)

    def call(alloc):
        out = alloc(n, torch.float32)
        gb.gb_reduce(out, xs, op, div)
        return [out]

    check(call)


TYPED = [(torch.bfloat16, gb.GB_OP_SUM, 2), (torch.float16, gb.GB_OP_AVG, 3), (torch.float64, gb.GB_OP_SUM, 2),
         (torch.int8, gb.GB_OP_SUM, 4), (torch.uint8, gb.GB_OP_MAX, 2), (torch.int32, gb.GB_OP_SUM, 2),
         (torch.int64, gb.GB_OP_MIN, 3)]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype,op,k", TYPED, ids=[f"{t}-{o}-{k}" for t, o, k in TYPED])
def test_reduce_typed(n, dtype, op, k):
    xs = floats(n, k, 3, dtype) if dtype.is_floating_point else ints(n, k, 3, dtype)

    def call(alloc):
        out = alloc(n, dtype)
        gb.gb_reduce_typed(out, xs, op, 3 if op == gb.GB_OP_AVG else 1)
        return [out]

    check(call)


@pytest.mark.parametrize("n", SIZES)
def test_encode_bf16(n):
    (x,) = floats(n, 1, 4)

    def call(alloc):
        codes = alloc(n, torch.uint16)
        gb.gb_encode_bf16(codes, x)
        return [codes]

    check(call)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("mode", [gb.GB_SCALE_ABSMAX_DIV_448, gb.GB_SCALE_POW2])
def test_encode_fp8(n, mode):
    (x,) = floats(n, 1, 5)

    def call(alloc):
        codes, scales = alloc(n, torch.uint8), alloc(nblocks(n), torch.float32)
        gb.gb_encode_fp8_e4m3_blockscaled(codes, scales, x, mode)
        return [codes, scales]

    check(call)


def payloads(codec, xs, mode=gb.GB_SCALE_ABSMAX_DIV_448):
    """Each rank's payload, encoded into plain buffers (inputs of a decode)."""
    n = xs[0].numel()
    codes, scales = [], []
    for x in xs:
        if codec == FP8:
            c, s = torch.empty(n, dtype=torch.uint8, device="cuda"), torch.empty(nblocks(n), device="cuda")
            gb.gb_encode_fp8_e4m3_blockscaled(c, s, x, mode)
            scales.append(s)
        elif codec == BF16:
            c = torch.empty(n, dtype=torch.uint16, device="cuda")
            gb.gb_encode_bf16(c, x)
        else:
            c = x.clone()
        codes.append(c)
    return codes, (scales if codec == FP8 else None)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("codec,k", [(BF16, 3), (FP8, 4), (FP8, 9), (NONE, 2)])
@pytest.mark.parametrize("accumulate", [False, True])
def test_decode_accumulate(n, codec, k, accumulate):
    codes, scales = payloads(codec, floats(n, k, 6))
    (acc0,) = floats(n, 1, 7)

    def call(alloc):
        acc = alloc(n, torch.float32, init=acc0)
        gb.gb_decode_accumulate(acc, codes, scales, codec, accumulate)
        return [acc]

    check(call)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype,codec", [(torch.float16, FP8), (torch.float64, BF16), (torch.bfloat16, FP8)])
def test_encode_typed(n, dtype, codec):
    (x,) = floats(n, 1, 8, dtype)

    def call(alloc):
        codes = alloc(n, torch.uint8 if codec == FP8 else torch.uint16)
        scales = alloc(nblocks(n), torch.float32) if codec == FP8 else None
        gb.gb_encode(codec, codes, scales, x)
        return [codes] + ([scales] if scales is not None else [])

    check(call)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype,codec,k", [(torch.float16, FP8, 2), (torch.bfloat16, BF16, 3),
                                           (torch.float64, FP8, 4)])
def test_decode_sum_typed(n, dtype, codec, k):
    codes, scales = payloads(codec, floats(n, k, 9))

    def call(alloc):
        out = alloc(n, dtype)
        gb.gb_decode_sum(out, codes, scales, codec)
        return [out]

    check(call)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("codec", [BF16, FP8])
def test_reduce_encode(n, codec):
    xs = floats(n, 3, 10)

    def call(alloc):
        s = alloc(n, torch.float32)
        codes = alloc(n, torch.uint8 if codec == FP8 else torch.uint16)
        scales = alloc(nblocks(n), torch.float32) if codec == FP8 else None
        gb.gb_reduce_encode(codec, codes, scales, xs, sum=s)
        return [s, codes] + ([scales] if scales is not None else [])

    check(call)


def workspace(alloc, codec, k, n, bucket):
    need = gb.gb_bucket_workspace_bytes(codec, k, n, bucket)
    return alloc(need, torch.uint8) if need > 0 else None


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("codec", [NONE, BF16, FP8])
def test_bucket_allreduce_local(n, codec):
    xs = floats(n, 4, 11)

    def call(alloc):
        out = alloc(n, torch.float32)
        ws = workspace(alloc, codec, 4, n, 512)
        gb.gb_bucket_allreduce_local(out, xs, 512, codec, workspace=ws)
        return [out] + ([ws] if ws is not None else [])

    check(call)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype,codec", [(torch.float16, FP8), (torch.float64, BF16), (torch.bfloat16, FP8)])
def test_bucket_allreduce_local_typed(n, dtype, codec):
    xs = floats(n, 3, 12, dtype)

    def call(alloc):
        out = alloc(n, dtype)
        ws = workspace(alloc, codec, 3, n, 768)
        gb.gb_bucket_allreduce_local_typed(out, xs, 768, codec, workspace=ws)
        return [out, ws]

    check(call)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("codec", [BF16, FP8])
def test_bucket_allreduce_local_ef(n, codec):
    xs = floats(n, 4, 13)
    res0 = floats(n, 4, 14)

    def call(alloc):
        out = alloc(n, torch.float32)
        res = [alloc(n, torch.float32, init=r * 1e-3) for r in res0]
        ws = workspace(alloc, codec, 4, n, 512)
        gb.gb_bucket_allreduce_local_ef(out, xs, res, 512, codec, workspace=ws)
        return [out, ws] + res

    check(call)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype,codec", [(torch.float16, FP8), (torch.float64, BF16)])
def test_bucket_allreduce_local_ef_typed(n, dtype, codec):
    xs = floats(n, 2, 15, dtype)
    res0 = floats(n, 2, 16)

    def call(alloc):
        out = alloc(n, dtype)
        res = [alloc(n, torch.float32, init=r * 1e-3) for r in res0]
        ws = workspace(alloc, codec, 2, n, 256)
        gb.gb_bucket_allreduce_local_ef_typed(out, xs, res, 256, codec, workspace=ws)
        return [out, ws] + res

    check(call)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("codec", [BF16, FP8])
def test_encode_ef(n, codec):
    (x,) = floats(n, 1, 17)
    (r0,) = floats(n, 1, 18)

    def call(alloc):
        codes = alloc(n, torch.uint8 if codec == FP8 else torch.uint16)
        res = alloc(n, torch.float32, init=r0 * 1e-3)
        if codec == FP8:
            scales = alloc(nblocks(n), torch.float32)
            gb.gb_encode_fp8_e4m3_blockscaled_ef(codes, scales, res, x)
            return [codes, scales, res]
        gb.gb_encode_bf16_ef(codes, res, x)
        return [codes, res]

    check(call)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype,codec", [(torch.float16, FP8), (torch.float64, BF16)])
def test_encode_ef_typed(n, dtype, codec):
    (x,) = floats(n, 1, 19, dtype)
    (r0,) = floats(n, 1, 20)

    def call(alloc):
        codes = alloc(n, torch.uint8 if codec == FP8 else torch.uint16)
        scales = alloc(nblocks(n), torch.float32) if codec == FP8 else None
        res = alloc(n, torch.float32, init=r0 * 1e-3)
        gb.gb_encode_ef(codec, codes, scales, res, x)
        return [codes, res] + ([scales] if scales is not None else [])

    check(call)


def batch_sizes(n):
    return [n, max(1, n // 3), 257, 1]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("codec,divisor", [(FP8, 1), (BF16, 8), (NONE, 3)])
def test_batch(n, codec, divisor):
    ns = batch_sizes(n)
    srcs = [floats(m, 3, 21 + b) for b, m in enumerate(ns)]

    def call(alloc):
        outs = [alloc(m, torch.float32) for m in ns]
        need = gb.gb_bucket_batch_workspace_bytes(codec, 3, ns)
        ws = alloc(need, torch.uint8) if need > 0 else None
        gb.gb_bucket_allreduce_local_batch(outs, srcs, codec, workspace=ws, divisor=divisor)
        return outs + ([ws] if ws is not None else [])

    check(call)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("codec", [FP8, BF16])
def test_batch_ef(n, codec):
    ns = batch_sizes(n)
    srcs = [floats(m, 2, 31 + b) for b, m in enumerate(ns)]
    res0 = [floats(m, 2, 41 + b) for b, m in enumerate(ns)]

    def call(alloc):
        outs = [alloc(m, torch.float32) for m in ns]
        res = [[alloc(m, torch.float32, init=r * 1e-3) for r in rb] for m, rb in zip(ns, res0)]
        ws = alloc(gb.gb_bucket_batch_workspace_bytes(codec, 2, ns), torch.uint8)
        gb.gb_bucket_allreduce_local_batch_ef(outs, srcs, res, codec, workspace=ws)
        return outs + [ws] + [r for rb in res for r in rb]

    check(call)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("codec", [FP8, BF16])
def test_noalloc(n, codec):
    xs = floats(n, 4, 51)

    def call(alloc):
        out = alloc(n, torch.float32)
        gb.gb_bucket_allreduce_local_noalloc(out, xs, 512, codec)
        return [out]

    check(call)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("codec", [FP8, BF16])
def test_encode_staged(n, codec):
    (x,) = floats(n, 1, 52)
    dt = torch.uint8 if codec == FP8 else torch.uint16

    def call(alloc):
        cd, ch = alloc(n, dt), alloc(n, dt, pinned=True)
        sd = alloc(nblocks(n), torch.float32) if codec == FP8 else None
        sh = alloc(nblocks(n), torch.float32, pinned=True) if codec == FP8 else None
        gb.gb_encode_staged(codec, cd, sd, ch, sh, x, 1024)
        torch.cuda.synchronize()
        return [cd, ch] + ([sd, sh] if sd is not None else [])

    check(call)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("codec", [FP8, BF16])
@pytest.mark.parametrize("accumulate", [False, True])
def test_decode_accumulate_staged(n, codec, accumulate):
    codes, scales = payloads(codec, floats(n, 3, 53))
    codes_host = [c.cpu().pin_memory() for c in codes]
    scales_host = [s.cpu().pin_memory() for s in scales] if scales is not None else None
    (acc0,) = floats(n, 1, 54)
    dt = torch.uint8 if codec == FP8 else torch.uint16

    def call(alloc):
        acc = alloc(n, torch.float32, init=acc0)
        cd = [alloc(n, dt) for _ in codes]
        sd = [alloc(nblocks(n), torch.float32) for _ in codes] if scales is not None else None
        gb.gb_decode_accumulate_staged(acc, codes_host, scales_host, cd, sd, codec, 1024, accumulate)
        return [acc]

    check(call)
