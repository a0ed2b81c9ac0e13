"""Pins of the oracle's Hadamard transform, sign diagonal and Philox stream
(CPU only)."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import scipy.linalg

import oracle as O
import synthetic as S

H16 = scipy.linalg.hadamard(16).astype(np.float64)


def test_fwht_is_sylvester_hadamard_over_four():
    """Column j of the transform is column j of scipy's (Sylvester-ordered)
    Hadamard matrix divided by 4, exactly."""
    for j in range(16):
        e = np.zeros(16, np.float32)
        e[j] = 1.0
        np.testing.assert_array_equal(O.fwht16(e).astype(np.float64), H16[:, j] / 4)
    np.testing.assert_array_equal(H16 @ H16.T, 16 * np.eye(16))


def test_fwht_within_fp32_bound_of_dense_product():
    rng = np.random.default_rng(0)
    for _ in range(2000):
        v = np.float32(rng.standard_normal(16) * 10.0 ** rng.uniform(-3, 3))
        want = H16 @ v.astype(np.float64) / 4
        got = O.fwht16(v).astype(np.float64)
        # four butterfly stages: each partial sum carries at most 4 roundings
        bound = 4 * 2.0 ** -24 * np.abs(v).astype(np.float64).sum() / 4 * 1.01
        assert np.max(np.abs(got - want)) <= bound


def test_fwht_is_an_involution_and_keeps_the_norm():
    rng = np.random.default_rng(1)
    for _ in range(500):
        v = np.float32(rng.standard_normal(16))
        w = O.fwht16(O.fwht16(v))
        np.testing.assert_allclose(w, v, rtol=0, atol=8 * 2.0 ** -24 * np.abs(v).max() * 4)
        y = O.fwht16(v)
        assert abs(np.sum(y.astype(np.float64) ** 2) - np.sum(v.astype(np.float64) ** 2)) \
            <= 1e-6 * np.sum(v.astype(np.float64) ** 2)
    # integer inputs stay exact: the round trip is the identity
    v = np.float32(np.arange(16) - 7)
    np.testing.assert_array_equal(O.fwht16(O.fwht16(v)), v)


def _sylvester_f32(v: np.ndarray, halves_first: bool) -> np.ndarray:
    """The Sylvester definition H_2n = [[H_n, H_n], [H_n, -H_n]] applied to
    the rows of v (float32, any power-of-two length) with float32 rounding
    at every addition.  halves_first: transform each half, then combine the
    two (H_n a + H_n b, H_n a - H_n b); otherwise combine first and transform
    the sum and the difference (H_n (a + b), H_n (a - b)).  Both equal H v in
    exact arithmetic; they round differently."""
    n = v.shape[-1]
    if n == 1:
        return v
    a, b = v[..., : n // 2], v[..., n // 2:]
    if halves_first:
        ta, tb = _sylvester_f32(a, True), _sylvester_f32(b, True)
        return np.concatenate([ta + tb, ta - tb], axis=-1)
    return np.concatenate([_sylvester_f32(a + b, False), _sylvester_f32(a - b, False)], axis=-1)


def _mixed_vectors(n: int, seed: int) -> np.ndarray:
    """16-vectors whose entries span many binades and signs, so that most
    float32 additions round."""
    rng = np.random.default_rng(seed)
    mag = 10.0 ** rng.uniform(-4, 4, size=(n, 16))
    return np.float32(rng.standard_normal((n, 16)) * mag)


def test_fwht_stage_order_matches_recursive_definition():
    """The oracle's butterflies run spans 1, 2, 4, 8 in that order.  Written
    as the recursion of the Sylvester definition, that order is "transform
    each half, then combine the halves": the oracle must equal that recursion
    (in float32, then x 1/4) bit for bit on 10^5 mixed-magnitude vectors.
    The other order (spans 8, 4, 2, 1: combine first, then transform) rounds
    differently on many of the same vectors, so the comparison can tell the
    two orders apart."""
    v = _mixed_vectors(100_000, 11)
    want = _sylvester_f32(v, halves_first=True) * np.float32(0.25)
    other = _sylvester_f32(v, halves_first=False) * np.float32(0.25)
    got = np.stack([O.fwht16(r) for r in v])
    assert want.dtype == np.float32 and got.dtype == np.float32
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    differ = np.any(other.view(np.uint32) != want.view(np.uint32), axis=1).mean()
    assert differ > 0.5, differ
    # the two recursions agree with scipy's matrix where nothing rounds
    e = np.eye(16, dtype=np.float32)
    np.testing.assert_array_equal(_sylvester_f32(e, True).astype(np.float64), H16)
    np.testing.assert_array_equal(_sylvester_f32(e, False).astype(np.float64), H16)


@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("kind", ["random", "det"])
def test_rht_view_is_signed_hadamard(axis, kind):
    x = S.normal(48, 64, 1.0, 0)
    xf = S.bf16_bits_to_f32(x).astype(np.float64)
    view = xf if axis == "row" else xf.T
    mask = O.rht_sign_mask(kind, 1234)
    d = np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(16)])
    y = O.rht_view(x, axis, kind, 1234)
    want = (view.reshape(view.shape[0], -1, 16) * d) @ H16.T / 4
    np.testing.assert_allclose(y.reshape(want.shape), want, rtol=0, atol=1e-5)
    if kind == "det":
        assert mask == 0


def test_shared_signs_keep_inner_products():
    """With one sign diagonal for both operands the rotated operands have the
    same inner products (the GEMM result is unchanged)."""
    a = S.normal(32, 128, 1.0, 0, "gemm_a")
    b = S.normal(32, 128, 1.0, 0, "gemm_b")
    ya = O.rht_view(a, "row", "random", 99).astype(np.float64)
    yb = O.rht_view(b, "row", "random", 99).astype(np.float64)
    za = S.bf16_bits_to_f32(a).astype(np.float64) @ S.bf16_bits_to_f32(b).astype(np.float64).T
    np.testing.assert_allclose(ya @ yb.T, za, rtol=0, atol=1e-4)


def test_rht_signs_differ_by_seed():
    masks = {O.rht_sign_mask("random", s) for s in range(64)}
    assert len(masks) > 60
    assert all(0 <= m < (1 << 16) for m in masks)


# ---- Philox4x32-10 against rocRAND ------------------------------------------

ROCRAND_PROBE = r"""
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  for (int i = 1; i + 2 < argc; i += 3) {
    unsigned long long seed = strtoull(argv[i], 0, 0), sub = strtoull(argv[i + 1], 0, 0),
                       q = strtoull(argv[i + 2], 0, 0);
    rocrand_device::philox4x32_10_engine e(seed, sub, 4ull * q);
    unsigned a = e(), b = e(), c = e(), d = e();
    printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def rocrand_probe():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    d = tempfile.mkdtemp()
    src = os.path.join(d, "p.cpp")
    open(src, "w").write(ROCRAND_PROBE)
    exe = os.path.join(d, "p")
    subprocess.run([hipcc, "-O1", "-x", "hip", "--offload-arch=gfx950", "-o", exe, src], check=True,
                   capture_output=True)
    return exe


def test_philox_matches_rocrand_engine(rocrand_probe):
    """rocRAND's engine(seed, subsequence, offset=4q) runs the block with
    key = seed and counter = (q lo, q hi, subsequence lo, subsequence hi).
    The SR stream takes that block's counter with stream = subsequence, and
    reads its four words 16 bits at a time, low half first: element 8q + 2j + h
    holds bits 16h..16h+15 of word j in the top half of its SR word."""
    cases = [(0, 0, 0), (0, 0, 1), (1, 0, 0), (0x1234567890, 3, 77), (2 ** 64 - 1, 1, 2 ** 40 + 5),
             (0xDEADBEEF, 0, 123456789), (7, 0x52485400, 0)]
    args = [str(v) for c in cases for v in c]
    out = subprocess.run([rocrand_probe, *args], check=True, capture_output=True, text=True).stdout.split("\n")
    for (seed, sub, q), line in zip(cases, out):
        want = [int(t) for t in line.split()]
        got = [int(v) for v in O.philox4x32_10([q & 0xFFFFFFFF, q >> 32, sub, 0],
                                                [seed & 0xFFFFFFFF, seed >> 32])]
        assert got == want, (seed, sub, q)
        halves = [(x >> (16 * h)) & 0xFFFF for x in want for h in range(2)]
        assert [O.sr_word(seed, sub, 8 * q + i) for i in range(8)] == [v << 16 for v in halves], (seed, sub, q)
    # the sign diagonal is word 0 of the counter (0,0,"RHT\0",0) block
    w = O.philox4x32_10([0, 0, 0x52485400, 0], [7, 0])
    assert O.rht_sign_mask("random", 7) == (int(w[0]) & 0xFFFF)


def test_sr_words_array_matches_scalar():
    w = O.sr_words(11, 1, 1000, 64)
    assert [int(v) for v in w] == [O.sr_word(11, 1, 1000 + i) for i in range(64)]


# ---- stochastic rounding ---------------------------------------------------

@pytest.mark.parametrize("fmt", ["e2m1", "e1m2", "int4"])
def test_sr_is_unbiased(fmt):
    """E[q] = |z| for z inside the grid range, and P(round up) = frac."""
    g = O.grid(fmt)
    n = 1 << 20
    w = O.sr_words(2024, 0, 0, n)
    rng = np.random.default_rng(7)
    for a in [0.1, 0.3, 1.2, 1.9, 2.2, 2.7, 3.3, 4.4, 5.5]:
        a = np.float32(min(a, g[7] * 0.95))
        codes = O.round_sr_array(np.full(n, a, np.float32), w, fmt)
        q = g[codes & 7]
        lo = g[g <= a].max()
        hi = g[g > a].min()
        frac = (float(a) - lo) / (hi - lo)
        sigma = (hi - lo) * np.sqrt(frac * (1 - frac) / n)
        assert abs(q.mean() - float(a)) < 5 * sigma + 1e-12
        assert set(np.unique(q)) <= {lo, hi}
    # grid points never move; saturation above the top
    for k in range(8):
        z = np.full(4096, g[k], np.float32)
        assert np.all(O.round_sr_array(z, w[:4096], fmt) == k)
    assert O.round_sr(g[7] * 3, fmt, 0) == 7
    assert O.round_sr(-1e-3, fmt, 0) & 8
    _ = rng


@pytest.mark.parametrize("fmt", ["e2m1", "e1m2", "int4"])
def test_sr_resolution_and_direction(fmt):
    """The SR decision at 16-bit resolution (the reading of IF4 page 6.1's
    random() < frac): over the 2^16 words w = j 2^16 + r, r any low 16 bits,
    exactly floor(frac 2^16) round up, and they are the largest j.  frac and
    its 16-bit floor are computed here exactly with fractions."""
    from fractions import Fraction
    g = O.grid(fmt)
    rng = np.random.default_rng(3)
    j = np.arange(1 << 16, dtype=np.uint64)
    for a in [0.1, 0.3, 0.8, 1.2, 1.7, 2.3, 2.9, 3.3, 4.4, 5.5, 6.9, 0.75, 1.0 + 2.0**-15, 2.5 - 2.0**-14]:
        a = np.float32(min(a, float(g[7]) * 0.999))
        k_lo = int(np.nonzero(g <= a)[0].max())
        frac = (Fraction(float(a)) - Fraction(float(g[k_lo]))) / (Fraction(float(g[k_lo + 1])) - Fraction(float(g[k_lo])))
        F = int(frac * 2**16)  # floor (frac >= 0)
        r = rng.integers(0, 1 << 16, size=j.size).astype(np.uint64)
        w = ((j << np.uint64(16)) | r).astype(np.uint32)
        codes = O.round_sr_array(np.full(j.size, a, np.float32), w, fmt) & 7
        assert set(np.unique(codes)) <= {k_lo, k_lo + 1}
        up = codes == k_lo + 1
        assert int(up.sum()) == F, (fmt, float(a), int(up.sum()), F)
        assert np.array_equal(up, j >= (1 << 16) - F)
    # less than 2^-16 of a step above a grid point: never up, even for the largest word
    step = float(g[1] - g[0])
    for a in [step * 2.0**-17, step * 2.0**-30, float(g[2]) + float(g[3] - g[2]) * 2.0**-17]:
        z = np.full(4, a, np.float32)
        lo = int(np.nonzero(g <= np.float32(a))[0].max())
        w = np.array([0xFFFFFFFF, 0xFFFF0000, 0x80000000, 0], np.uint32)
        assert np.all(O.round_sr_array(z, w, fmt) == lo)
