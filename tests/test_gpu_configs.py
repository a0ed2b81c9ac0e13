"""GPU parity at the full sizes of the five workloads, in the launch
configurations the benchmark uses: every code, scale and tensor scale of every
quantization is compared bit for bit with the CPU oracle over the whole
tensor (the oracle's view rows split over host threads), the statistics over
the whole tensor within 1e-6, and the GEMM outputs over the whole matrix with
numpy binary64 BLAS as the product of the oracle's dequantized operands.

  quantize_x     256x1024 N(0,1) with 0.1% x50 outliers; FP32 1x16, no RHT,
                 RTNE to E2M1 and E1M2
  activations    8192x8192 Student-t(3)*0.02; RHT-16 + two-level E4M3 scale,
                 E2M1 / E1M2 / INT4, with and without RHT (SQNR gain)
  llama linear   X 16384x4096, W 14336x4096, dY 16384x14336; E1M2, FP32 1x16,
                 RHT-16 everywhere, row and column (transposed) quantizations,
                 Philox SR on dY
  mxfp4 + if4    16384x8192 N(0,1) with 0.5% U(-1,1) 1x32 blocks; MXFP4 with
                 deterministic H16, IF4 without transform
  gemm           A, B 8192x8192 N(0,1); RHT-16 -> MXFP4 native GEMM and
                 E1M2 -> bf16 GEMM; attenuation eta and output SQNR
"""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import assert_bits_equal, host, oracle_cfg, to_device_bf16

pytestmark = pytest.mark.gpu


def lib():
    import block_scaled_bit_ufp4_amd as U
    return U


def check_whole(q, x_bits, cfg, amax=None):
    """Every code and scale of the quantization equals the oracle's; returns
    the oracle's result."""
    want = O.quantize_threads(x_bits, oracle_cfg(cfg), amax_value=amax)
    assert_bits_equal(host(q.codes), want.codes, f"codes {cfg}")
    assert_bits_equal(host(q.scales), want.scales, f"scales {cfg}")
    if cfg.scale == "e4m3":
        assert host(q.tensor_scale)[0] == np.float32(want.alpha), cfg
    return want


def rel(a, b):
    return abs(a - b) / max(abs(b), 1e-300)


def check_stats(got, ref):
    """The GPU's 48 statistics sums against the oracle's: counts exactly,
    sums of positive terms within 1e-6 relative, the nearly cancelling signed
    sums within 1e-6 of the sum of their magnitudes."""
    got = np.asarray(got, np.float64)
    np.testing.assert_array_equal(got[[0, 7, 8]], ref[[0, 7, 8]])
    np.testing.assert_array_equal(got[16:32], ref[16:32])
    for k in (1, 2, 5, 6):
        assert rel(got[k], ref[k]) < 1e-6, k
    for k in (3, 4):
        assert abs(got[k] - ref[k]) <= 1e-6 * ref[6], k
    # per-bucket rounding bias sums: relative to the bucket's count (each
    # term is at most half a grid step, 1 in grid units)
    assert np.all(np.abs(got[32:48] - ref[32:48]) <= 1e-6 * np.maximum(ref[16:32], 1.0))


# ---- quantize_x --------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["e2m1", "e1m2"])
def test_quantize_x_full(fmt):
    U = lib()
    x = S.quantize_x(256, 1024, seed=0)
    xd = to_device_bf16(x)
    cfg = U.Cfg(fmt, "fp32")
    q = U.ufp4_quantize(xd, cfg)
    want = check_whole(q, x, cfg)
    assert_bits_equal(host(U.ufp4_dequantize(q)), O.dequantize(want, oracle_cfg(cfg), x.shape), "dequant")
    got = host(U.ufp4_stats(xd, q))
    ref = O.stats(x, oracle_cfg(cfg))
    check_stats(got, ref)
    rg, rr = U.ufp4_stats_finalize(got), O.finalize(ref)
    assert abs(rg["sqnr_db"] - rr["sqnr_db"]) < 1e-5
    assert abs(rg["mean_err"] - rr["mean_err"]) < 1e-6 * rr["mse"] ** 0.5 + 1e-12


# ---- activations -----------------------------------------------------------------

@pytest.fixture(scope="module")
def activations():
    x = S.activations_t3(8192, 8192, seed=0)
    return x, to_device_bf16(x)


@pytest.mark.parametrize("fmt", ["e2m1", "e1m2", "int4"])
@pytest.mark.parametrize("rht", ["none", "random"])
def test_activations_two_level(activations, fmt, rht):
    U = lib()
    x, xd = activations
    cfg = U.Cfg(fmt, "e4m3", rht=rht, rht_seed=0)
    amax = U.ufp4_amax(xd, cfg)
    a_ref = O.amax_threads(x, oracle_cfg(cfg))
    assert host(amax)[0] == np.float32(a_ref)
    q = U.ufp4_quantize(xd, cfg, amax=amax)
    want = check_whole(q, x, cfg, amax=a_ref)
    assert want.alpha == np.float32(np.float32(a_ref) / np.float32(O.gridmax(fmt) * 448))
    if fmt == "e2m1" and rht == "random":
        # the whole dequantization, inverse transform included
        got = host(U.ufp4_dequantize(q, inverse_rht=True))
        assert_bits_equal(got, O.dequantize_threads(want, oracle_cfg(cfg), x.shape, inverse=True), "dequant")


def test_activations_sqnr_gain(activations):
    """Whole-tensor statistics on the GPU match the oracle's, and RHT moves
    E2M1 and E1M2 SQNR in opposite directions."""
    U = lib()
    x, xd = activations
    sq = {}
    for fmt in ("e2m1", "e1m2"):
        for rht in ("none", "random"):
            cfg = U.Cfg(fmt, "e4m3", rht=rht, rht_seed=0)
            q = U.ufp4_quantize(xd, cfg)
            got = host(U.ufp4_stats(xd, q))
            check_stats(got, O.stats_threads(x, oracle_cfg(cfg)))
            sq[fmt, rht] = U.ufp4_stats_finalize(got)["sqnr_db"]
    assert sq["e2m1", "random"] < sq["e2m1", "none"]
    assert sq["e1m2", "random"] > sq["e1m2", "none"]


# ---- llama linear ----------------------------------------------------------------

@pytest.fixture(scope="module")
def llama():
    x = S.llama_x(16384, 4096, seed=0)
    w = S.llama_w(14336, 4096, seed=0)
    dy = S.llama_dy(16384, 14336, seed=0)
    return {"x": (x, to_device_bf16(x)), "w": (w, to_device_bf16(w)), "dy": (dy, to_device_bf16(dy))}


@pytest.mark.parametrize("name,axis", [("x", "row"), ("x", "col"), ("w", "row"), ("w", "col"),
                                       ("dy", "row"), ("dy", "col")])
def test_llama_six_quantizations(llama, name, axis):
    U = lib()
    src, dev = llama[name]
    sr = name == "dy"
    cfg = U.Cfg("e1m2", "fp32", rht="random", rht_seed=0, rounding="sr" if sr else "rtne", axis=axis,
                sr_seed=0, sr_stream=1 if axis == "col" else 0)
    q = U.ufp4_quantize(dev, cfg)
    check_whole(q, src, cfg)


@pytest.mark.parametrize("fmt", ["e1m2", "e2m1"])
def test_llama_x_statistics(llama, fmt):
    U = lib()
    x, xd = llama["x"]
    cfg = U.Cfg(fmt, "fp32", rht="random", rht_seed=0)
    q = U.ufp4_quantize(xd, cfg)
    check_stats(host(U.ufp4_stats(xd, q)), O.stats_threads(x, oracle_cfg(cfg)))


# ---- mxfp4 + if4 -------------------------------------------------------------------

@pytest.fixture(scope="module")
def mx():
    x, which = S.mx_if4(16384, 8192, seed=0)
    return x, to_device_bf16(x), which


def test_mxfp4_h16(mx):
    U = lib()
    x, xd, _ = mx
    cfg = U.Cfg("e2m1", "e8m0", 32, rht="det")
    q = U.ufp4_quantize(xd, cfg)
    check_whole(q, x, cfg)


def test_if4_selection(mx):
    U = lib()
    x, xd, which = mx
    cfg = U.Cfg("if4", "e4m3")
    amax = U.ufp4_amax(xd, cfg)
    a_ref = O.amax_threads(x, oracle_cfg(cfg))
    assert host(amax)[0] == np.float32(a_ref)
    q = U.ufp4_quantize(xd, cfg, amax=amax)
    check_whole(q, x, cfg, amax=a_ref)
    flags = (host(q.scales) >> 7).reshape(-1)
    inj = flags.reshape(-1, 2)[which]
    assert inj.mean() > 0.9                       # uniform blocks pick INT4
    got = host(U.ufp4_stats(xd, q))
    check_stats(got, O.stats_threads(x, oracle_cfg(cfg), amax_value=a_ref))
    assert abs(U.ufp4_stats_finalize(got)["int4_share"] - flags.mean()) < 1e-12


# ---- GEMM ----------------------------------------------------------------------------

@pytest.fixture(scope="module")
def gemm_inputs():
    a = S.gemm_a(8192, 8192, seed=0)
    b = S.gemm_b(8192, 8192, seed=0)
    ad, bd = to_device_bf16(a), to_device_bf16(b)
    # Z = A B^T of the bf16 inputs, binary64 (numpy BLAS)
    z_ref = S.bf16_bits_to_f32(a).astype(np.float64) @ S.bf16_bits_to_f32(b).astype(np.float64).T
    return a, b, ad, bd, z_ref


@pytest.mark.parametrize("mode", ["mxfp4", "bf16"])
def test_gemm_full_size(gemm_inputs, mode):
    """The whole 8192^3 product against the binary64 product of the oracle's
    dequantized operands (bf16-rounded for the dequantize-to-bf16 path):
    relative Frobenius error below 1e-3; eta and the output SQNR against the
    oracle's (Z = A B^T of the bf16 inputs) within 1e-4; and the library's
    attenuation sums on its own outputs equal binary64 sums of the same
    matrices."""
    U = lib()
    a, b, ad, bd, z_ref = gemm_inputs
    cfg = U.Cfg("e2m1", "e8m0", 32, rht="random", rht_seed=0) if mode == "mxfp4" else \
        U.Cfg("e1m2", "fp32", rht="random", rht_seed=0)
    qa, qb = U.ufp4_quantize(ad, cfg), U.ufp4_quantize(bd, cfg)
    zq = U.ufp4_qgemm(qa, qb, mode)
    ocfg = oracle_cfg(cfg)
    oa, ob = check_whole(qa, a, cfg), check_whole(qb, b, cfg)
    da = O.dequantize_threads(oa, ocfg, a.shape)
    db = O.dequantize_threads(ob, ocfg, b.shape)
    if mode == "bf16":
        da, db = O.bf16_round(da), O.bf16_round(db)
    zq_ref = da.astype(np.float64) @ db.astype(np.float64).T
    del da, db
    got = host(zq).astype(np.float64)
    err = np.linalg.norm(got - zq_ref) / np.linalg.norm(zq_ref)
    assert err < 1e-3, err
    want = O.eta_report(O.eta_sums(zq_ref, z_ref))
    z = U.ufp4_gemm_bf16(ad, bd)
    s = host(U.ufp4_eta(zq, z))
    rep = O.eta_report(s)
    assert rel(rep["eta"], want["eta"]) < 1e-4, (rep, want)
    assert abs(rep["sqnr_db"] - want["sqnr_db"]) < 1e-4 * abs(want["sqnr_db"]), (rep, want)
    # the attenuation sums of the library equal binary64 sums over its own
    # fp32 outputs (summation order aside)
    exact = O.eta_sums(got, host(z).astype(np.float64))
    np.testing.assert_allclose(s, exact, rtol=1e-9)
    assert 0.95 < rep["eta"] < 1.0 + 5e-3
