"""The linear layer's three 4-bit GEMMs (fwd_y, bwd_dx, bwd_dw) against the
oracle, for the UFP4 recipe and the E2M1 baseline: the oracle quantizes each
operand along the GEMM's contraction axis (rows or columns, SR on dY with its
two streams), dequantizes, rounds to bf16 and multiplies in binary64. The
GPU product must be within 1e-5 relative Frobenius error of that (bf16
operands, fp32 accumulation), on small shapes in full and at the
llama-shaped sizes on sampled output rows. The autograd function reproduces
the direct calls."""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import host, oracle_cfg, sample_rows, to_device_bf16

pytestmark = pytest.mark.gpu


def L():
    import block_scaled_bit_ufp4_amd.linear as lin
    return lin


def rel_fro(got, want):
    return float(np.linalg.norm(got.astype(np.float64) - want) / np.linalg.norm(want))


def oracle_view(x_bits, cfg, rows=None):
    """bf16-rounded dequantized view rows of the oracle's quantization."""
    ocfg = oracle_cfg(cfg)
    if rows is None:
        q = O.quantize(x_bits, ocfg)
        return O.bf16_round(O.dequantize(q, ocfg, x_bits.shape))
    parts = []
    for r in rows:
        q = O.quantize(x_bits, ocfg, v0=int(r), v1=int(r) + 1)
        parts.append(O.dequantize(q, ocfg, x_bits.shape, v0=int(r), v1=int(r) + 1))
    return O.bf16_round(np.concatenate(parts))


def small_inputs(T=512, K=256, N=768, seed=4):
    x = S.llama_x(T, K, seed=seed, n_outlier_cols=4)
    w = S.llama_w(N, K, seed=seed)
    dy = S.llama_dy(T, N, seed=seed)
    return x, w, dy


@pytest.mark.parametrize("recipe", ["ufp4", "e2m1_baseline"])
def test_three_gemms_small(recipe):
    lin = L()
    r = lin.UFP4 if recipe == "ufp4" else lin.E2M1_BASELINE
    x, w, dy = small_inputs()
    xd, wd, dyd = to_device_bf16(x), to_device_bf16(w), to_device_bf16(dy)
    y = host(lin.linear_fwd(xd, wd, r))
    dx, dw = (host(t) for t in lin.linear_bwd(dyd, xd, wd, r))
    want_y = O.gemm_nt(oracle_view(x, r.cfg(r.rht_fwd, "row")), oracle_view(w, r.cfg(r.rht_fwd, "row")))
    want_dx = O.gemm_nt(oracle_view(dy, r.cfg(r.rht_dx, "row", r.sr_dy, 0)), oracle_view(w, r.cfg(r.rht_dx, "col")))
    want_dw = O.gemm_nt(oracle_view(dy, r.cfg(r.rht_dw, "col", r.sr_dy, 1)), oracle_view(x, r.cfg(r.rht_dw, "col")))
    assert y.shape == (512, 768) and dx.shape == (512, 256) and dw.shape == (768, 256)
    assert rel_fro(y, want_y) < 1e-5
    assert rel_fro(dx, want_dx) < 1e-5
    assert rel_fro(dw, want_dw) < 1e-5
    # and all three are close to the unquantized products (E1M2 closer than E2M1)
    xf, wf, dyf = (S.bf16_bits_to_f32(t).astype(np.float64) for t in (x, w, dy))
    for got, ref in ((y, xf @ wf.T), (dx, dyf @ wf), (dw, dyf.T @ xf)):
        assert rel_fro(got, ref) < 0.25


def test_autograd_matches_direct_calls():
    import torch
    lin = L()
    x, w, dy = small_inputs(seed=5)
    xd = to_device_bf16(x).requires_grad_(True)
    wd = to_device_bf16(w).requires_grad_(True)
    dyd = to_device_bf16(dy)
    y = lin.ufp4_linear(xd, wd)
    y.backward(dyd)
    with torch.no_grad():
        y0 = lin.linear_fwd(xd, wd).to(torch.bfloat16)
        dx0, dw0 = lin.linear_bwd(dyd, xd, wd)
    np.testing.assert_array_equal(host(y.detach().float()), host(y0.float()))
    np.testing.assert_array_equal(host(xd.grad.float()), host(dx0.to(torch.bfloat16).float()))
    np.testing.assert_array_equal(host(wd.grad.float()), host(dw0.to(torch.bfloat16).float()))


def test_rht_seed_cancels_in_the_product():
    """With a shared sign diagonal the rotation leaves the product unchanged
    up to quantization: the UFP4 GEMMs with RHT stay within the quantization
    error of the unquantized product, like those without."""
    lin = L()
    x, w, _ = small_inputs(seed=6)
    xd, wd = to_device_bf16(x), to_device_bf16(w)
    ref = S.bf16_bits_to_f32(x).astype(np.float64) @ S.bf16_bits_to_f32(w).astype(np.float64).T
    with_rht = host(lin.linear_fwd(xd, wd, lin.UFP4))
    without = host(lin.linear_fwd(xd, wd, lin.Recipe(rht_fwd=False)))
    assert rel_fro(with_rht, ref) < 0.2 and rel_fro(without, ref) < 0.2


@pytest.fixture(scope="module")
def llama():
    x = S.llama_x(16384, 4096, seed=0)
    w = S.llama_w(14336, 4096, seed=0)
    dy = S.llama_dy(16384, 14336, seed=0)
    return x, w, dy


@pytest.mark.parametrize("gemm", ["fwd_y", "bwd_dx", "bwd_dw"])
def test_llama_gemms_sampled_rows(llama, gemm):
    """Full-size UFP4 GEMMs; the oracle computes 8 sampled output rows."""
    lin = L()
    r = lin.UFP4
    x, w, dy = llama
    xd, wd, dyd = to_device_bf16(x), to_device_bf16(w), to_device_bf16(dy)
    if gemm == "fwd_y":
        got = lin.linear_fwd(xd, wd, r)
        a_src, a_cfg, b_src, b_cfg = x, r.cfg(True, "row"), w, r.cfg(True, "row")
    elif gemm == "bwd_dx":
        got = lin.linear_bwd(dyd, xd, wd, r)[0]
        a_src, a_cfg, b_src, b_cfg = dy, r.cfg(True, "row", True, 0), w, r.cfg(True, "col")
    else:
        got = lin.linear_bwd(dyd, xd, wd, r)[1]
        a_src, a_cfg, b_src, b_cfg = dy, r.cfg(True, "col", True, 1), x, r.cfg(True, "col")
    rows = sample_rows(got.shape[0], 8, seed=11)
    want = O.gemm_nt(oracle_view(a_src, a_cfg, rows), oracle_view(b_src, b_cfg))
    assert rel_fro(host(got)[rows], want) < 1e-5
