"""GPU parity of the block-scaled GEMMs, the bf16 GEMM and the attenuation
sums against the oracle's binary64 products of its own dequantized operands
(relative Frobenius error within 1e-3), through the C ABI."""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import host, oracle_cfg, to_device_bf16

pytestmark = pytest.mark.gpu


def lib():
    import block_scaled_bit_ufp4_amd as U
    return U


def rel_fro(got, want):
    return float(np.linalg.norm(got.astype(np.float64) - want) / np.linalg.norm(want))


def oracle_operand(x_bits, ocfg, bf16=False):
    q = O.quantize(x_bits, ocfg)
    d = O.dequantize(q, ocfg, x_bits.shape)
    return O.bf16_round(d) if bf16 else d


SHAPES = [(256, 256, 128), (512, 256, 384), (256, 768, 1024), (512, 512, 640), (256, 512, 2560)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("rht", ["none", "random"])
def test_mxfp4_gemm_matches_oracle(M, N, K, rht):
    U = lib()
    a = S.normal(M, K, 1.0, 0, "gemm_a")
    b = S.normal(N, K, 1.0, 0, "gemm_b")
    cfg = U.Cfg("e2m1", "e8m0", 32, rht=rht, rht_seed=11)
    qa = U.ufp4_quantize(to_device_bf16(a), cfg)
    qb = U.ufp4_quantize(to_device_bf16(b), cfg)
    z = host(U.ufp4_qgemm(qa, qb, "mxfp4"))
    ocfg = oracle_cfg(cfg)
    want = O.gemm_nt(oracle_operand(a, ocfg), oracle_operand(b, ocfg))
    assert rel_fro(z, want) < 1e-3, rel_fro(z, want)
    assert rel_fro(z, want) < 1e-5  # exact products, binary32 sums


@pytest.mark.parametrize("fmt", ["e1m2", "int4", "e2m1", "if4", "e2m1_max2", "mxfp4"])
def test_dequant_bf16_gemm_matches_oracle(fmt):
    """The dequantize-to-bf16 GEMM on every operand kind, MXFP4 (E8M0 per
    32) included: the same operands the native mode takes."""
    U = lib()
    M, N, K = 256, 512, 256
    if fmt == "if4":  # Gaussian rows with uniform blocks, so both block types occur
        a, _ = S.mx_if4(M, K, seed=1, frac=0.3)
        b, _ = S.mx_if4(N, K, seed=2, frac=0.3)
        cfg = U.Cfg(fmt, "e4m3")
    elif fmt == "mxfp4":
        a = S.normal(M, K, 1.0, 1, "gemm_a")
        b = S.normal(N, K, 1.0, 1, "gemm_b")
        cfg = U.Cfg("e2m1", "e8m0", 32, rht="det")
    else:
        a = S.normal(M, K, 1.0, 1, "gemm_a")
        b = S.normal(N, K, 1.0, 1, "gemm_b")
        cfg = U.Cfg(fmt, "fp32", rht="random", rht_seed=3)
    qa = U.ufp4_quantize(to_device_bf16(a), cfg)
    qb = U.ufp4_quantize(to_device_bf16(b), cfg)
    z = host(U.ufp4_qgemm(qa, qb, "bf16"))
    ocfg = oracle_cfg(cfg)
    want = O.gemm_nt(oracle_operand(a, ocfg, bf16=True), oracle_operand(b, ocfg, bf16=True))
    assert rel_fro(z, want) < 1e-5, rel_fro(z, want)


@pytest.mark.parametrize("M,N,K", [(256, 256, 64), (512, 256, 320)])
def test_bf16_gemm_matches_oracle(M, N, K):
    U = lib()
    a = S.normal(M, K, 1.0, 2, "gemm_a")
    b = S.normal(N, K, 1.0, 2, "gemm_b")
    z = host(U.ufp4_gemm_bf16(to_device_bf16(a), to_device_bf16(b)))
    want = O.gemm_nt(S.bf16_bits_to_f32(a), S.bf16_bits_to_f32(b))
    assert rel_fro(z, want) < 1e-5



@pytest.mark.parametrize("mode,K,nt", [("mxfp4", 512, 16), ("mxfp4", 384, 16), ("bf16", 512, 16), ("bf16", 384, 16),
                                       ("plain_bf16", 320, 16), ("plain_bf16", 512, 16), ("mxfp4", 512, 17),
                                       ("plain_bf16", 320, 17)])
def test_gemm_more_tiles_than_workgroups(mode, K, nt):
    """17 x 16 = 272 output tiles of 256 x 256, more than the persistent grid's
    one workgroup per compute unit (256 on MI355X): the first workgroups go on
    to a second tile, whose first stages they fetch during the first tile's
    last steps.  K = 384 (MXFP4) and 320 (bf16) round the stage count up to a
    whole group of four; 17 x 17 = 289 tiles, not a multiple of the eight
    XCDs, take the plain grouped raster.  One sampled row in each tile row,
    all columns, so every tile is checked against the oracle."""
    U = lib()
    M, N = 17 * 256, nt * 256
    a = S.normal(M, K, 1.0, 5, "gemm_a")
    b = S.normal(N, K, 1.0, 5, "gemm_b")
    rows = np.arange(17) * 256 + np.random.default_rng(7).integers(0, 256, 17)
    import torch
    c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    if mode == "plain_bf16":
        z = host(U.ufp4_gemm_bf16(to_device_bf16(a), to_device_bf16(b), c=c))
        want = O.gemm_nt(S.bf16_bits_to_f32(a[rows]), S.bf16_bits_to_f32(b))
    else:
        cfg = U.Cfg("e2m1", "e8m0", 32, rht="random", rht_seed=2) if mode == "mxfp4" else \
            U.Cfg("e1m2", "fp32", rht="random", rht_seed=2)
        z = host(U.ufp4_qgemm(U.ufp4_quantize(to_device_bf16(a), cfg), U.ufp4_quantize(to_device_bf16(b), cfg),
                              mode, c=c))
        ocfg = oracle_cfg(cfg)
        bf = mode == "bf16"
        want = O.gemm_nt(oracle_operand(a, ocfg, bf16=bf)[rows], oracle_operand(b, ocfg, bf16=bf))
    assert rel_fro(z[rows], want) < 1e-5, rel_fro(z[rows], want)
    # every element of every tile was written (the output starts as NaN)
    assert np.isfinite(z).all()


def test_eta_sums():
    U = lib()
    import torch
    rng = np.random.default_rng(0)
    z = np.float32(rng.standard_normal((256, 512)))
    zq = np.float32(z * 0.97 + rng.standard_normal(z.shape) * 0.1)
    sums = host(U.ufp4_eta(torch.from_numpy(zq).cuda(), torch.from_numpy(z).cuda()))
    z64, q64 = z.astype(np.float64), zq.astype(np.float64)
    want = [np.sum(q64 * z64), np.sum(z64 * z64), np.sum((q64 - z64) ** 2)]
    np.testing.assert_allclose(sums, want, rtol=1e-12)


def test_if4_gemm_block_type_factors():
    """IF4 operands with both block types on both sides (uniform rows pick
    INT4, Gaussian rows FP4): the GEMM equals the oracle's product of its own
    dequantized bf16 operands, whose INT4 blocks carry the 6/7 factor, so
    INT4 x INT4 block products carry 36/49 and mixed ones 6/7 ([IF4] 4.1)."""
    U = lib()
    rng = np.random.default_rng(7)
    K = 128
    a = np.where(np.arange(256)[:, None] % 2 == 0, rng.uniform(-1, 1, (256, K)), rng.standard_normal((256, K)))
    b = np.where(np.arange(256)[:, None] % 3 == 0, rng.uniform(-1, 1, (256, K)), rng.standard_normal((256, K)))
    a_bits, b_bits = S.f32_to_bf16_bits(a.astype(np.float32)), S.f32_to_bf16_bits(b.astype(np.float32))
    cfg = U.Cfg("if4", "e4m3")
    qa, qb = U.ufp4_quantize(to_device_bf16(a_bits), cfg), U.ufp4_quantize(to_device_bf16(b_bits), cfg)
    fa = host(qa.scales) >> 7
    fb = host(qb.scales) >> 7
    assert fa.any() and (1 - fa).any() and fb.any() and (1 - fb).any()   # both types on both sides
    z = host(U.ufp4_qgemm(qa, qb, "bf16")).astype(np.float64)
    ocfg = oracle_cfg(cfg)
    da, db = oracle_operand(a_bits, ocfg, bf16=True), oracle_operand(b_bits, ocfg, bf16=True)
    assert rel_fro(z, O.gemm_nt(da, db)) < 1e-5
