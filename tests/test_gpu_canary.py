"""Output buffers larger than the call needs, filled with a sentinel: every
entry point writes exactly its documented output and nothing past it, on
ragged shapes (sizes that are not multiples of the kernels' tiles)."""
import numpy as np
import pytest
import torch

from helpers import to_device_bf16
import synthetic as S

pytestmark = pytest.mark.gpu

PAD = 4096          # sentinel bytes after each output
SENT = 0xA5


def lib():
    import block_scaled_bit_ufp4_amd as U
    return U


def guarded(nbytes: int):
    """A uint8 device buffer of nbytes + PAD filled with the sentinel, and a
    view of its first nbytes (16-byte aligned: torch allocations are)."""
    buf = torch.full((nbytes + PAD,), SENT, dtype=torch.uint8, device="cuda")
    return buf, buf[:nbytes]


def tail_ok(buf, nbytes):
    torch.cuda.synchronize()
    t = buf[nbytes:].cpu().numpy()
    return bool(np.all(t == SENT))


SHAPES = [(48, 80), (96, 160), (288, 224), (544, 96), (1056, 2080)]   # rows, cols; ragged against every tile
CFGS = [("e2m1", "fp32", 16, "random", "rtne"), ("e2m1", "e4m3", 16, "none", "rtne"),
        ("e2m1", "e8m0", 32, "det", "rtne"), ("e1m2", "fp32", 16, "random", "sr"), ("if4", "e4m3", 16, "none", "rtne")]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("c", CFGS)
def test_quantize_writes_nothing_past_its_outputs(shape, axis, c):
    U = lib()
    fmt, scale, block, rht, rnd = c
    R, Cc = shape
    V, L = (R, Cc) if axis == "row" else (Cc, R)
    if L % block:
        pytest.skip("block axis not a multiple of the block")
    x = S.normal(R, Cc, 1.0, seed=3)
    xd = to_device_bf16(x)
    cfg = U.Cfg(fmt, scale, block, rht=rht, rounding=rnd, axis=axis, rht_seed=5)
    ncodes = V * L // 2
    nscales = V * (L // block) * (4 if scale == "fp32" else 1)
    cbuf, codes = guarded(ncodes)
    sbuf, scales = guarded(nscales)
    tbuf, ts = guarded(4)
    q = U.QTensor(codes.view(V, L // 2), scales.view(torch.float32 if scale == "fp32" else torch.uint8).view(V, -1),
                  ts.view(torch.float32) if scale == "e4m3" else None, R, Cc, cfg)
    U.ufp4_quantize(xd, cfg, out=q)
    ref = U.ufp4_quantize(xd, cfg)
    assert tail_ok(cbuf, ncodes) and tail_ok(sbuf, nscales), (shape, axis, c)
    if scale == "e4m3":
        assert tail_ok(tbuf, 4)
    assert torch.equal(q.codes, ref.codes)
    # dequantize into a guarded fp32 and a guarded bf16 buffer
    for dt, esz in ((torch.float32, 4), (torch.bfloat16, 2)):
        ybuf, y = guarded(V * L * esz)
        U.ufp4_dequantize(q, inverse_rht=rht != "none", y=y.view(dt).view(V, L))
        assert tail_ok(ybuf, V * L * esz), dt


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("axis", ["row", "col"])
def test_rht_amax_stats_write_nothing_past_their_outputs(shape, axis):
    U = lib()
    R, Cc = shape
    V, L = (R, Cc) if axis == "row" else (Cc, R)
    x = to_device_bf16(S.normal(R, Cc, 1.0, seed=4))
    ybuf, y = guarded(V * L * 4)
    U.ufp4_rht(x, axis=axis, rht="random", seed=1, y=y.view(torch.float32).view(V, L))
    assert tail_ok(ybuf, V * L * 4)
    cfg = U.Cfg("e2m1", "e4m3", axis=axis, rht="random", rht_seed=1)
    abuf, am = guarded(4)
    wbytes = U.ufp4_workspace_size(U.OP_AMAX, R, Cc, cfg)
    wbuf, ws = guarded(wbytes)
    U.ufp4_amax(x, cfg, out=am.view(torch.float32), ws=ws)
    assert tail_ok(abuf, 4) and tail_ok(wbuf, wbytes)
    q = U.ufp4_quantize(x, cfg, amax=am.view(torch.float32))
    sbuf, sums = guarded(U.NSUMS * 8)
    swb = U.ufp4_workspace_size(U.OP_STATS, R, Cc, cfg)
    swbuf, sws = guarded(swb)
    U.ufp4_stats(x, q, sums=sums.view(torch.float64), ws=sws)
    assert tail_ok(sbuf, U.NSUMS * 8) and tail_ok(swbuf, swb)


@pytest.mark.parametrize("mode", ["mxfp4", "bf16"])
def test_gemm_writes_nothing_past_its_output(mode):
    U = lib()
    M, N, K = 512, 768, 384
    a = to_device_bf16(S.normal(M, K, 1.0, 0, "gemm_a"))
    b = to_device_bf16(S.normal(N, K, 1.0, 0, "gemm_b"))
    cfg = U.Cfg("e2m1", "e8m0", 32) if mode == "mxfp4" else U.Cfg("e1m2", "fp32")
    qa, qb = U.ufp4_quantize(a, cfg), U.ufp4_quantize(b, cfg)
    cbuf, c = guarded(M * N * 4)
    wb = U.ufp4_workspace_size(U.OP_QGEMM, M + N, K, cfg) if mode == "bf16" else 0
    wbuf, ws = guarded(wb)
    U.ufp4_qgemm(qa, qb, mode, c=c.view(torch.float32).view(M, N), ws=ws if wb else None)
    assert tail_ok(cbuf, M * N * 4) and tail_ok(wbuf, wb)
    assert torch.equal(c.view(torch.float32).view(M, N), U.ufp4_qgemm(qa, qb, mode))


def test_dequant_bf16_gemm_takes_mxfp4_operands():
    """The dequantize-to-bf16 mode accepts E8M0 operands with the workspace
    the size query gives, and equals the native product (MXFP4 values are
    exact in bf16: a 2-bit significand times a power of two)."""
    U = lib()
    M, N, K = 256, 512, 256
    a = to_device_bf16(S.normal(M, K, 1.0, 1, "gemm_a"))
    b = to_device_bf16(S.normal(N, K, 1.0, 1, "gemm_b"))
    cfg = U.Cfg("e2m1", "e8m0", 32, rht="random", rht_seed=2)
    qa, qb = U.ufp4_quantize(a, cfg), U.ufp4_quantize(b, cfg)
    z1 = U.ufp4_qgemm(qa, qb, "bf16")
    z0 = U.ufp4_qgemm(qa, qb, "mxfp4")
    torch.testing.assert_close(z1, z0, rtol=1e-6, atol=1e-4)
