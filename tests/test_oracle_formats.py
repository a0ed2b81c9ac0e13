"""Pins of the oracle's number formats against what the pages print and
against library or textbook routines (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


def f32_range(lo, hi, stride=1):
    """Every `stride`-th binary32 bit pattern of the non-negative values in [lo, hi)."""
    a = np.float32(lo).view(np.uint32)
    b = np.float32(hi).view(np.uint32)
    return np.arange(a, b, stride, dtype=np.uint64).astype(np.uint32).view(np.float32)


def near(points, ulps=300):
    """Binary32 values within `ulps` of each point (points >= 0)."""
    out = []
    for p in points:
        u = np.int64(np.float32(p).view(np.uint32))
        out.append(np.arange(max(u - ulps, 0), u + ulps + 1, dtype=np.int64).astype(np.uint32).view(np.float32))
    return np.concatenate(out)


# ---- grids and RTNE --------------------------------------------------------

@pytest.mark.parametrize("fmt", ["e2m1", "e1m2"])
def test_grid_is_the_pages_grid(fmt):
    assert list(O.grid(fmt)) == GOLD["grids"][fmt]["values"]


def test_int4_grid_is_integers_to_seven():
    assert list(O.grid("int4")) == list(range(8))


def test_every_value_in_the_pages_tie_interval_rounds_to_two():
    g = GOLD["rtne_interval_to_2"]
    z = f32_range(g["lo"], np.nextafter(np.float32(g["hi"]), np.float32(10)))
    codes = O.round_rtne_array(z, "e2m1")
    assert np.all(O.grid("e2m1")[codes & 7] == g["value"])
    # just outside the interval the neighbours win
    assert O.grid("e2m1")[O.round_rtne(np.nextafter(np.float32(1.75), np.float32(0)), "e2m1")] == 1.5
    assert O.grid("e2m1")[O.round_rtne(np.nextafter(np.float32(2.5), np.float32(9)), "e2m1")] == 3.0


def textbook_round(a: np.ndarray, fmt: str) -> np.ndarray:
    """Round |z| the way a binary format with a short significand rounds
    (round half to even on the quotient by the local quantum), saturating at
    the largest value; returns the value.  E2M1: 1 mantissa bit, smallest
    exponent 0 (quantum 0.5 below 1); E1M2: quantum 0.5 everywhere; INT4:
    quantum 1."""
    a = a.astype(np.float64)
    if fmt == "e1m2":
        return np.minimum(np.rint(a / 0.5) * 0.5, 3.5)
    if fmt == "int4":
        return np.minimum(np.rint(a), 7.0)
    _, e = np.frexp(np.maximum(a, 1.0))          # a = f 2^e, f in [0.5, 1)
    quantum = np.where(a < 1.0, 0.5, np.ldexp(1.0, e - 2))
    return np.minimum(np.rint(a / quantum) * quantum, 6.0)


@pytest.mark.parametrize("fmt", ["e2m1", "e1m2", "int4"])
def test_rtne_matches_textbook_rounding(fmt):
    top = 16.0
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 2.25, 2.75, 3.25, 4.5, 5.5, 6.5, 7.0, 3.75, 0.5, 1.5]
    z = np.concatenate([f32_range(0.0, top, 97), near(mids), np.float32([0.0, 1e-45, 1e30, 3e38])])
    codes = O.round_rtne_array(z, fmt)
    got = O.grid(fmt)[codes & 7]
    np.testing.assert_array_equal(got, textbook_round(z, fmt))
    assert not np.any(codes & 8)
    # the sign goes into bit 3, magnitude code unchanged
    codes_neg = O.round_rtne_array(-z, fmt)
    np.testing.assert_array_equal(codes_neg, codes | 8)


def cell_average_error(fmt, k, n=1 << 16):
    """Mean of (q - a) for a uniform on the rounding cell of grid point k,
    evaluated on a fine lattice of cell midpoints."""
    g = O.grid(fmt)
    lo = (g[k - 1] + g[k]) / 2
    hi = (g[k] + g[k + 1]) / 2
    a = lo + (np.arange(n) + 0.5) * (hi - lo) / n
    codes = O.round_rtne_array(a.astype(np.float32), fmt)
    assert np.all(codes == k)
    return np.mean(g[codes] - a.astype(np.float32).astype(np.float64))


def test_shrinkage_bias_closed_form_e2m1():
    """For values uniform inside a cell, the expected rounding error is (left
    half-width - right half-width)/2: -0.125 at q=2 and -0.25 at q=4 (as the
    pages print), 0 where the neighbours are equally spaced."""
    g = O.grid("e2m1")
    for k in range(1, 7):
        closed = ((g[k] - g[k - 1]) / 2 - (g[k + 1] - g[k]) / 2) / 2
        assert abs(cell_average_error("e2m1", k) - closed) < 1e-6
    gold = GOLD["cell_bias"]["e2m1"]
    assert abs(cell_average_error("e2m1", 4) - gold["2.0"]) < 1e-6
    assert abs(cell_average_error("e2m1", 6) - gold["4.0"]) < 1e-6


def test_uniform_grid_has_no_cell_bias():
    for k in range(1, 7):
        assert abs(cell_average_error("e1m2", k) - GOLD["cell_bias"]["e1m2_interior"]) < 1e-6


# ---- restricted-range E2M1 ----------------------------------------------------
# The UFP4 page (section "UFP4：换一把尺子") tries emulating a uniform grid on
# E2M1 by capping its range (at 2.0 the points {0, .5, 1, 1.5, 2} are uniform)
# and finds every capped variant worse than the E2M1 baseline.

RESTRICTED = {"e2m1_max4": (4.0, 6), "e2m1_max3": (3.0, 5), "e2m1_max2": (2.0, 4)}


@pytest.mark.parametrize("fmt", sorted(RESTRICTED))
def test_restricted_e2m1_is_nearest_capped_point(fmt):
    """Brute force: the nearest of the E2M1 points up to the cap (ties to the
    even code), the cap for everything above it; sign in bit 3."""
    cap, kmax = RESTRICTED[fmt]
    assert O.gridmax(fmt) == cap
    np.testing.assert_array_equal(O.grid(fmt), O.grid("e2m1"))
    pts = O.grid("e2m1")[:kmax + 1]
    mids = (pts[1:] + pts[:-1]) / 2
    z = np.concatenate([f32_range(0.0, 9.0, 61), near(list(mids) + [cap, 6.0]), np.float32([1e30])])
    codes = O.round_rtne_array(z, fmt)
    a = z.astype(np.float64)
    d = np.abs(a[:, None] - pts[None, :])
    best = np.argmin(d, axis=1)
    tie = (d == d.min(axis=1, keepdims=True)).sum(axis=1) > 1
    best[tie] = [k if k % 2 == 0 else k + 1 for k in best[tie]]  # ties: the even code
    best[a >= cap] = kmax
    np.testing.assert_array_equal(codes & 7, best)
    np.testing.assert_array_equal(O.round_rtne_array(-z, fmt), codes | 8)


def test_capped_at_two_is_the_uniform_grid():
    """Capped at 2 the E2M1 codes 0..4 are the points k/2, the E1M2 codes 0..4:
    below the cap both round identically; above it E2M1 saturates."""
    z = np.concatenate([f32_range(0.0, 2.0, 211), near([0.25, 0.75, 1.25, 1.75])])
    np.testing.assert_array_equal(O.round_rtne_array(z, "e2m1_max2"), O.round_rtne_array(z, "e1m2"))
    assert set(O.round_rtne_array(np.float32([2.3, 3.0, 7.0]), "e2m1_max2")) == {4}


def test_restricted_e2m1_loses_to_the_full_grid():
    """On Gaussian blocks (what the RHT makes of a tensor) each cap costs SQNR
    against full E2M1, the more the lower the cap, while the uniform E1M2 grid
    beats both; the capped grids also shrink more than E1M2."""
    x = S.normal(512, 1024, 1.0, 2, "uniform")
    for scale in ("fp32", "e4m3"):
        sq = {f: O.finalize(O.stats(x, O.Cfg(f, scale)))
              for f in ("e2m1", "e2m1_max4", "e2m1_max3", "e2m1_max2", "e1m2")}
        db = {f: r["sqnr_db"] for f, r in sq.items()}
        assert db["e1m2"] > db["e2m1"] > db["e2m1_max4"] > db["e2m1_max3"] > db["e2m1_max2"]
        assert sq["e2m1_max2"]["mean_shrink"] < sq["e1m2"]["mean_shrink"] < 0


# ---- E4M3 / E8M0 scales ----------------------------------------------------

def test_e4m3_decode_matches_torch_for_every_finite_byte():
    b = np.arange(0x7F, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([O.e4m3_decode(int(v)) for v in b], dtype=np.float32)
    np.testing.assert_array_equal(got, ref)


def test_e4m3_encode_matches_torch_rtne_below_saturation():
    # torch's float8_e4m3fn cast is round-to-nearest-even and non-saturating;
    # below 464 (halfway from 448 to 480) the two must agree exactly.
    edges = [O.e4m3_decode(b) for b in range(1, 0x7F)]
    mids = [(O.e4m3_decode(b) + O.e4m3_decode(b + 1)) / 2 for b in range(0, 0x7E)]
    v = np.concatenate([f32_range(0.0, 464.0, 4099), near(edges, 40), near(mids, 40),
                        np.float32([0.0, 2.0 ** -10, 0.75 * 2.0 ** -9, 2.0 ** -9])])
    v = v[v < 464.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode_array(v)
    np.testing.assert_array_equal(got, ref)


def test_e4m3_saturates_at_448():
    for v in [448.0, 449.0, 463.9, 464.0, 480.0, 1e9, 3e38]:
        assert O.e4m3_encode(v) == 0x7E
    assert O.e4m3_decode(0x7E) == 448.0


def test_format_table_ranges():
    """Max/min magnitudes of the format table and NVINT4's 58.3% relative
    dynamic range follow from the grids and the scale formats."""
    e4_max, e4_min = O.e4m3_decode(0x7E), O.e4m3_decode(0x01)
    assert e4_max == 448.0 and e4_min == 2.0 ** -9
    assert O.gridmax("e2m1") * e4_max == 6 * 448
    assert O.gridmax("int4") * e4_max == 7 * 448
    assert O.grid("e2m1")[1] * e4_min == 0.5 * 2.0 ** -9
    assert O.grid("int4")[1] * e4_min == 1.0 * 2.0 ** -9
    ratio = (O.gridmax("int4") / O.grid("int4")[1]) / (O.gridmax("e2m1") / O.grid("e2m1")[1])
    assert abs(ratio - GOLD["format_table"]["nvint4"]["dyn_range"]) < 5e-4
    # E8M0: exponents -127..127, so MXFP4 spans 0.5*2^-127 .. 6*2^127
    assert O.e8m0_exponent(3e38) == 127 - 0 or O.e8m0_exponent(3e38) <= 127
    assert O.e8m0_exponent(0.0) == -127
    assert O.e8m0_exponent(2.0 ** -149) == -127


def test_e8m0_exponent_is_floor_log2_minus_two():
    rng = np.random.default_rng(5)
    v = np.float32(np.abs(rng.standard_normal(20000)) * 10.0 ** rng.uniform(-30, 30, 20000))
    v = np.concatenate([v, np.float32([2.0 ** k for k in range(-120, 120)]),
                        np.nextafter(np.float32([2.0 ** k for k in range(-120, 120)]), np.float32(0))])
    _, e = np.frexp(v.astype(np.float64))
    want = np.clip(e - 1 - 2, -127, 127)
    got = np.array([O.e8m0_exponent(float(x)) for x in v])
    np.testing.assert_array_equal(got, want)


# ---- the format table's MSE column ----------------------------------------

@pytest.mark.parametrize("name,cfg", [
    ("mxfp4", O.Cfg("e2m1", "e8m0", 32)),
    ("nvfp4", O.Cfg("e2m1", "e4m3")),
    ("nvint4", O.Cfg("int4", "e4m3")),
    ("if4", O.Cfg("if4", "e4m3")),
])
def test_format_table_mse_on_standard_normal(name, cfg):
    """The table's MSE column (x1e-3) is reproduced on N(0,1) data with the
    table's block sizes and scale formats.  Tolerance 0.1e-3: the page prints
    one decimal and does not state its data (IF4 comes out at 6.14)."""
    x = S.normal(1024, 2048, 1.0, 0, "uniform")
    r = O.finalize(O.stats(x, cfg))
    assert abs(r["mse"] * 1e3 - GOLD["format_table"][name]["mse_e3"]) < 0.1, r["mse"]


def test_format_table_mse_order():
    x = S.normal(512, 2048, 1.0, 1, "uniform")
    mse = [O.finalize(O.stats(x, c))["mse"] for c in
           (O.Cfg("e2m1", "e8m0", 32), O.Cfg("e2m1", "e4m3"), O.Cfg("int4", "e4m3"), O.Cfg("if4", "e4m3"))]
    assert mse[0] > mse[1] > mse[2] > mse[3]


# ---- bf16 rounding (GEMM operands of the dequantize-to-bf16 path) ----------

def test_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    v = np.float32(rng.standard_normal(100000) * 10.0 ** rng.uniform(-20, 20, 100000))
    ties = ((rng.integers(0, 1 << 16, 1000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    v = np.concatenate([v, ties[np.isfinite(ties)]])
    ref = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(O.bf16_round(v), ref)
