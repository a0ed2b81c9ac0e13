"""Pins of the oracle's attenuation sums (eta and output SQNR of a quantized
GEMM; "当你的 GPU 学不会算账", section "复利效应的反向版本"), CPU only."""
import numpy as np

import oracle as O
import synthetic as S


def test_eta_special_cases():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((64, 48))
    # the exact product: eta 1, no error
    s = O.eta_sums(z, z)
    assert s[0] == s[1] and s[2] == 0.0
    rep = O.eta_report(s)
    assert rep["eta"] == 1.0 and rep["sqnr_db"] == float("inf")
    # a power-of-two multiple: eta is that factor exactly, the error its square
    for c in (0.5, 0.25, 2.0):
        s = O.eta_sums(c * z, z)
        assert O.eta_report(s)["eta"] == c
        assert abs(s[2] - (c - 1) ** 2 * s[1]) <= 1e-12 * s[1]


def test_eta_ignores_noise_orthogonal_to_the_product():
    """Zq = Z + R with <R, Z> = 0 exactly (integer vectors): eta = 1 and the
    SQNR is ||Z||^2 / ||R||^2."""
    z = np.array([3.0, 4.0, 0.0, 12.0, -5.0, 2.0])
    r = np.array([4.0, -3.0, 7.0, 5.0, 12.0, 0.0])
    assert np.dot(z, r) == 0.0
    s = O.eta_sums(z + r, z)
    assert s[0] == s[1] == np.dot(z, z)
    assert s[2] == np.dot(r, r)
    rep = O.eta_report(s)
    assert rep["eta"] == 1.0
    assert abs(rep["sqnr_db"] - 10 * np.log10(np.dot(z, z) / np.dot(r, r))) < 1e-12


def test_eta_sums_against_numpy_dot():
    rng = np.random.default_rng(1)
    zq = rng.standard_normal(100_003)
    z = zq * 0.97 + 0.1 * rng.standard_normal(zq.size)
    s = O.eta_sums(zq, z)
    want = [np.dot(zq, z), np.dot(z, z), np.dot(zq - z, zq - z)]
    np.testing.assert_allclose(s, want, rtol=1e-12)


def test_eta_is_the_product_of_the_operand_factors():
    """The page's identity: operands A_hat = a A + noise, B_hat = b B + noise
    with noise independent of the operands give a product whose attenuation
    is a b (up to the sampling error of the noise terms).  The reversed ratio
    <Z,Z>/<Zq,Z> would give 1/(a b)."""
    rng = np.random.default_rng(2)
    M, N, K = 128, 128, 1024
    A, B = rng.standard_normal((M, K)), rng.standard_normal((N, K))
    a, b = 0.9, 0.8
    Ah = a * A + 0.3 * rng.standard_normal((M, K))
    Bh = b * B + 0.3 * rng.standard_normal((N, K))
    eta = O.eta_report(O.eta_sums(Ah @ Bh.T, A @ B.T))["eta"]
    assert abs(eta - a * b) < 1e-2, eta


def test_eta_of_quantized_gemm_is_the_product_of_signal_factors():
    """With real quantizers: eta of the quantized product equals the product
    of the operands' signal factors (alpha = sum x_hat y / sum y^2 from the
    statistics) to about 1e-3, for NVFP4-style E2M1 (which shrinks) and E1M2
    (which does not)."""
    a = S.normal(256, 1024, 1.0, 0, "gemm_a")
    b = S.normal(256, 1024, 1.0, 0, "gemm_b")
    za = S.bf16_bits_to_f32(a).astype(np.float64)
    zb = S.bf16_bits_to_f32(b).astype(np.float64)
    z = za @ zb.T
    for fmt, scale in (("e2m1", "e4m3"), ("e1m2", "fp32")):
        cfg = O.Cfg(fmt, scale)
        qa, qb = O.quantize(a, cfg), O.quantize(b, cfg)
        da = O.dequantize(qa, cfg, a.shape).astype(np.float64)
        db = O.dequantize(qb, cfg, b.shape).astype(np.float64)
        eta = O.eta_report(O.eta_sums(da @ db.T, z))["eta"]
        alpha_a = O.finalize(O.stats(a, cfg))["alpha"]
        alpha_b = O.finalize(O.stats(b, cfg))["alpha"]
        assert abs(eta - alpha_a * alpha_b) < 2e-3, (fmt, eta, alpha_a * alpha_b)
        if fmt == "e2m1":
            assert eta < 0.997
