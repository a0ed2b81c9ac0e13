"""GPU parity of the quantizer, amax, transform, dequantizer and statistics
against the CPU oracle, through the C ABI (small shapes that span several
workgroup tiles with ragged tails, and corner-case inputs)."""
import itertools

import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import assert_bits_equal, host, oracle_cfg, to_device_bf16, to_device_f32

pytestmark = pytest.mark.gpu

def lib():
    import block_scaled_bit_ufp4_amd as U
    return U


def all_configs():
    out = []
    for fmt, scale, rht, rnd, axis in itertools.product(["e2m1", "e1m2", "int4"], ["fp32", "e4m3"],
                                                        ["none", "random", "det"], ["rtne", "sr"], ["row", "col"]):
        out.append(dict(format=fmt, scale=scale, block=16, rht=rht, rounding=rnd, axis=axis))
    for rht, axis in itertools.product(["none", "random", "det"], ["row", "col"]):
        out.append(dict(format="e2m1", scale="e8m0", block=32, rht=rht, rounding="rtne", axis=axis))
        out.append(dict(format="if4", scale="e4m3", block=16, rht=rht, rounding="rtne", axis=axis))
    # range-capped E2M1
    for fmt, scale, rht, axis in itertools.product(["e2m1_max4", "e2m1_max3", "e2m1_max2"], ["fp32", "e4m3"],
                                                   ["none", "random"], ["row", "col"]):
        out.append(dict(format=fmt, scale=scale, block=16, rht=rht, rounding="rtne", axis=axis))
    return out


def cfg_id(d):
    return f"{d['format']}-{d['scale']}-{d['rht']}-{d['rounding']}-{d['axis']}"


# a row length of 1056 (66 chunks), 96 rows: 12672 octets = 13 row workgroups with a
# ragged last one; for the column axis 1056 source rows = 3 row tiles (the last
# ragged) and 96 columns = 2 column tiles (the last half empty)
SHAPE = (1056, 96)


def make_input(kind: str, shape=SHAPE, seed=0):
    R, Cc = shape
    if kind == "t3":
        return S.activations_t3(R, Cc, seed=seed)
    if kind == "outliers":
        return S.llama_x(R, Cc, seed=seed)
    return S.normal(R, Cc, 1.0, seed)


def check_quant(x_bits, d, ldx_pad=0, dtype="bf16"):
    U = lib()
    cfg = U.Cfg(**d, rht_seed=1234, sr_seed=77, sr_stream=1 if d["axis"] == "col" else 0)
    ocfg = oracle_cfg(cfg)
    R, Cc = x_bits.shape
    if dtype == "bf16":
        xd = to_device_bf16(np.pad(x_bits, ((0, 0), (0, ldx_pad))))[:, :Cc] if ldx_pad else to_device_bf16(x_bits)
        xo = x_bits
    else:
        xf = S.bf16_bits_to_f32(x_bits) * np.float32(1.0 + 2 ** -12)  # use the full binary32 mantissa
        xd = to_device_f32(xf)
        xo = xf
    q = U.ufp4_quantize(xd, cfg)
    want = O.quantize(xo, ocfg)
    assert_bits_equal(host(q.codes), want.codes, "codes")
    assert_bits_equal(host(q.scales), want.scales, "scales")
    if cfg.scale == "e4m3":
        assert host(q.tensor_scale)[0] == np.float32(want.alpha)
    return U, cfg, ocfg, xd, xo, q, want


@pytest.mark.parametrize("d", all_configs(), ids=cfg_id)
def test_quantize_matches_oracle(d):
    check_quant(make_input("t3" if d["scale"] == "e4m3" else "outliers"), d)


@pytest.mark.parametrize("d", [c for c in all_configs() if c["rounding"] == "rtne" and c["rht"] != "det"], ids=cfg_id)
def test_quantize_binary32_input(d):
    check_quant(make_input("normal", seed=3), d, dtype="f32")


@pytest.mark.parametrize("axis", ["row", "col"])
def test_quantize_strided_source(axis):
    d = dict(format="e1m2", scale="fp32", block=16, rht="random", rounding="sr", axis=axis)
    check_quant(make_input("normal", seed=4), d, ldx_pad=24)


@pytest.mark.parametrize("d", [c for c in all_configs() if c["rht"] != "det" and c["rounding"] == "rtne"], ids=cfg_id)
def test_corner_case_inputs(d):
    x = S.edge_cases(64, 256)
    if d["axis"] == "col":
        x = np.ascontiguousarray(x.T)  # keep the special blocks along the quantization axis
    check_quant(x, d)


@pytest.mark.parametrize("fmt", ["e1m2", "int4", "e2m1", "if4"])
@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("rht", ["none", "random"])
def test_subnormal_block_scales(fmt, axis, rht):
    """Blocks far below the tensor's largest magnitude take E4M3 block scales
    in the subnormal range, where |y| / s can pass the grid's upper rounding
    boundary: the kernels clamp only in waves holding such a block."""
    x = S.small_blocks(256, 512, seed=2)
    if axis == "col":
        x = np.ascontiguousarray(x.T)
    d = dict(format=fmt, scale="e4m3", block=16, rht=rht, rounding="rtne", axis=axis)
    _, _, _, _, _, _, want = check_quant(x, d)
    b = want.scales & 0x7F
    assert np.any((b > 0) & (b < 8))  # the case is reached


def binary32_tiny_blocks(rows=96, cols=256, seed=0):
    """binary32 N(0,1) blocks scaled by 2^-e, e drawn per 16-element block in
    [110, 151], so many blocks lie in (or reach into) the binary32 subnormal
    range, where a single-level FP32 block scale m / gridmax is itself
    subnormal and loses precision; plus blocks whose only nonzero value is a
    few units of 2^-149."""
    rng = np.random.default_rng([seed, 97])
    e = rng.integers(110, 152, (rows, cols // 16)).repeat(16, axis=1)
    x = (rng.standard_normal((rows, cols)) * np.exp2(-e.astype(np.float64))).astype(np.float32)
    x[0, :16] = 0
    x[0, 0] = np.float32(5 * 2.0 ** -149)
    x[1, :16] = 0
    x[1, 3] = np.float32(-11 * 2.0 ** -149)
    x[2, :16] = np.float32(2.0 ** -149) * rng.integers(-40, 41, 16).astype(np.float32)
    return x


def binary32_huge_blocks(rows=96, cols=256, seed=0):
    """binary32 N(0,1) blocks scaled by 2^e, e drawn per block in [90, 120]: the
    block maxima reach about 2^122, so squares and sums of squares overflow
    binary32 while every transform stays finite (16 x 2^122 < 2^128)."""
    rng = np.random.default_rng([seed, 98])
    e = rng.integers(90, 121, (rows, cols // 16)).repeat(16, axis=1)
    return (rng.standard_normal((rows, cols)) * np.exp2(e.astype(np.float64))).astype(np.float32)


def tiny_configs():
    out = []
    for fmt, scale, rnd, rht, axis in itertools.product(["e1m2", "int4", "e2m1"], ["fp32", "e4m3"], ["rtne", "sr"],
                                                        ["none", "random"], ["row", "col"]):
        out.append(dict(format=fmt, scale=scale, block=16, rht=rht, rounding=rnd, axis=axis))
    for rht, axis in itertools.product(["none", "random"], ["row", "col"]):
        out.append(dict(format="if4", scale="e4m3", block=16, rht=rht, rounding="rtne", axis=axis))
        out.append(dict(format="e2m1", scale="e8m0", block=32, rht=rht, rounding="rtne", axis=axis))
    return out


@pytest.mark.parametrize("shift", [0, 25, None], ids=["mixed", "all_tiny", "huge"])
@pytest.mark.parametrize("d", tiny_configs(), ids=cfg_id)
def test_binary32_extreme_blocks(d, shift):
    """binary32 sources with blocks down in the subnormal range: where the block
    scale is subnormal, |y| / s can pass the grid's largest code, and the codes
    must still saturate there as the oracle's do.  With shift 25 the whole
    tensor is tiny (amax near 2^-135), so the two-level tensor scale and the
    E4M3 scales built on it are subnormal as well.  The "huge" case takes the
    other end: block maxima near 2^122, squares past the binary32 range."""
    U = lib()
    x = binary32_huge_blocks() if shift is None else binary32_tiny_blocks() * np.float32(2.0 ** -shift)
    if d["axis"] == "col":
        x = np.ascontiguousarray(x.T)
    cfg = U.Cfg(**d, rht_seed=1234, sr_seed=77, sr_stream=1 if d["axis"] == "col" else 0)
    xd = to_device_f32(x)
    q = U.ufp4_quantize(xd, cfg)
    ocfg = oracle_cfg(cfg)
    want = O.quantize(x, ocfg)
    assert_bits_equal(host(q.codes), want.codes, "codes")
    assert_bits_equal(host(q.scales), want.scales, "scales")
    # the dequantized values (also through the inverse transform) and the
    # statistics of the same blocks
    assert_bits_equal(host(U.ufp4_dequantize(q)), O.dequantize(want, ocfg, x.shape), "dequant")
    assert_bits_equal(host(U.ufp4_dequantize(q, inverse_rht=True)), O.dequantize(want, ocfg, x.shape, inverse=True),
                      "dequant inverse")
    if d["scale"] == "e4m3":
        # the tensor amax and the standalone transform of the same source
        assert host(U.ufp4_amax(xd, cfg))[0] == np.float32(O.amax(x, ocfg))
        assert_bits_equal(host(U.ufp4_rht(xd, d["axis"], d["rht"], 1234)), O.rht_view(x, d["axis"], d["rht"], 1234),
                          "rht f32")
    got = host(U.ufp4_stats(xd, q))
    ref = O.stats(x, ocfg)
    assert np.all(np.isfinite(got)), got
    compare_sums(got, ref)
    np.testing.assert_array_equal(got[[0, 7, 8] + list(range(16, 32))], ref[[0, 7, 8] + list(range(16, 32))])


@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("rht", ["none", "random", "det"])
def test_amax_and_transform(axis, rht):
    U = lib()
    x = make_input("outliers", seed=5)
    xd = to_device_bf16(x)
    cfg = U.Cfg("e2m1", "e4m3", rht=rht, axis=axis, rht_seed=99)
    got = host(U.ufp4_amax(xd, cfg))[0]
    assert got == np.float32(O.amax(x, oracle_cfg(cfg)))
    y = host(U.ufp4_rht(xd, axis, rht, 99))
    want = O.rht_view(x, axis, rht, 99)
    assert_bits_equal(y, want, "rht f32")
    yb = host(U.ufp4_rht(xd, axis, rht, 99, out_dtype=__import__("torch").bfloat16).float())
    assert_bits_equal(yb, O.bf16_round(want), "rht bf16")


@pytest.mark.parametrize("d", [c for c in all_configs() if c["rounding"] == "rtne" or c["format"] == "e1m2"],
                         ids=cfg_id)
def test_dequantize_matches_oracle(d):
    U, cfg, ocfg, xd, xo, q, want = check_quant(make_input("outliers", seed=6), d)
    shape = xo.shape
    got = host(U.ufp4_dequantize(q))
    assert_bits_equal(got, O.dequantize(want, ocfg, shape), "dequant")
    got_inv = host(U.ufp4_dequantize(q, inverse_rht=True))
    assert_bits_equal(got_inv, O.dequantize(want, ocfg, shape, inverse=True), "dequant inverse")


def compare_sums(got, want):
    for k in range(48):
        if k == 3:  # sum of signed errors nearly cancels: compare against sum |e|
            assert abs(got[3] - want[3]) <= 1e-6 * want[6] + 1e-300, k
        elif k == 4:
            assert abs(got[4] - want[4]) <= 1e-6 * want[6] + 1e-300, k
        elif k >= 32:
            assert abs(got[k] - want[k]) <= 1e-6 * max(1.0, want[k - 16]) * 8, k
        else:
            assert abs(got[k] - want[k]) <= 1e-6 * abs(want[k]) + 1e-300, (k, got[k], want[k])


@pytest.mark.parametrize("d", [c for c in all_configs() if c["rht"] != "det" and c["rounding"] == "rtne"], ids=cfg_id)
def test_stats_corner_case_inputs(d):
    """Statistics on the corner-case blocks (zeros, subnormal blocks whose scale
    is subnormal, huge and tiny magnitudes, ties) against the oracle."""
    x = S.edge_cases(64, 256)
    if d["axis"] == "col":
        x = np.ascontiguousarray(x.T)
    U, cfg, ocfg, xd, xo, q, want = check_quant(x, d)
    got = host(U.ufp4_stats(xd, q))
    ref = O.stats(xo, ocfg)
    assert np.all(np.isfinite(got)), got
    compare_sums(got, ref)
    np.testing.assert_array_equal(got[[0, 7, 8] + list(range(16, 32))], ref[[0, 7, 8] + list(range(16, 32))])


@pytest.mark.parametrize("d", all_configs()[::3] + all_configs()[-12:], ids=cfg_id)
def test_stats_match_oracle(d):
    U, cfg, ocfg, xd, xo, q, want = check_quant(make_input("t3", seed=7), d)
    got = host(U.ufp4_stats(xd, q))
    ref = O.stats(xo, ocfg)
    compare_sums(got, ref)
    np.testing.assert_array_equal(got[[0, 7, 8] + list(range(16, 32))], ref[[0, 7, 8] + list(range(16, 32))])


def test_fused_equals_unfused():
    """Quantizing the standalone binary32 transform without RHT gives the same
    bits as the fused RHT + quantize."""
    U = lib()
    x = make_input("outliers", seed=8)
    xd = to_device_bf16(x)
    for axis in ("row", "col"):
        for fmt, scale in (("e1m2", "fp32"), ("e2m1", "e4m3"), ("if4", "e4m3")):
            fused = U.ufp4_quantize(xd, U.Cfg(fmt, scale, rht="random", rht_seed=5, axis=axis))
            y = U.ufp4_rht(xd, axis, "random", 5)                       # the view, binary32
            # quantize the view along its rows
            unfused = U.ufp4_quantize(y, U.Cfg(fmt, scale, rht="none", axis="row"))
            assert_bits_equal(host(fused.codes), host(unfused.codes), f"codes {axis} {fmt}")
            assert_bits_equal(host(fused.scales), host(unfused.scales), f"scales {axis} {fmt}")


def test_repeat_runs_are_identical():
    U = lib()
    x = make_input("t3", (2048, 1024), seed=9)
    xd = to_device_bf16(x)
    for axis in ("row", "col"):
        cfg = U.Cfg("e1m2", "fp32", rht="random", rounding="sr", axis=axis, sr_seed=3)
        a = U.ufp4_quantize(xd, cfg)
        b = U.ufp4_quantize(xd, cfg)
        assert_bits_equal(host(a.codes), host(b.codes), "codes")
        assert_bits_equal(host(a.scales), host(b.scales), "scales")
        s1 = host(U.ufp4_stats(xd, a))
        s2 = host(U.ufp4_stats(xd, a))
        np.testing.assert_array_equal(s1, s2)


def test_column_axis_equals_row_axis_of_transpose_on_gpu():
    U = lib()
    x = make_input("outliers", (512, 256), seed=10)
    xd = to_device_bf16(x)
    xt = to_device_bf16(np.ascontiguousarray(x.T))
    for d in (dict(format="e1m2", rounding="sr", rht="random"), dict(format="if4", scale="e4m3"),
              dict(format="e2m1", scale="e8m0", block=32, rht="det")):
        a = U.ufp4_quantize(xd, U.Cfg(axis="col", sr_seed=4, **d))
        b = U.ufp4_quantize(xt, U.Cfg(axis="row", sr_seed=4, **d))
        assert_bits_equal(host(a.codes), host(b.codes), "codes")
        assert_bits_equal(host(a.scales), host(b.scales), "scales")


def test_empty_tensor_is_a_no_op():
    U = lib()
    import torch
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q = U.ufp4_quantize(x, U.Cfg("e2m1"))
    assert q.codes.numel() == 0
    x = torch.empty((64, 0), dtype=torch.bfloat16, device="cuda")
    q = U.ufp4_quantize(x, U.Cfg("e1m2", axis="col"))
    assert q.codes.numel() == 0


@pytest.mark.parametrize("fmt", ["e2m1", "e1m2"])
def test_unfused_rht_then_quantize_equals_fused(fmt):
    """The RHT as its own call (fp32 output) followed by a quantization
    without it gives the fused kernel's codes and scales bit for bit."""
    import torch
    import block_scaled_bit_ufp4_amd as U
    x = to_device_bf16(S.activations_t3(512, 1024, seed=3))
    fused_cfg = U.Cfg(fmt, "e4m3", rht="random", rht_seed=5)
    fused = U.ufp4_quantize(x, fused_cfg)
    y = U.ufp4_rht(x, rht="random", seed=5, out_dtype=torch.float32)
    plain = U.ufp4_quantize(y, U.Cfg(fmt, "e4m3", rht="none"))
    np.testing.assert_array_equal(host(fused.codes), host(plain.codes))
    np.testing.assert_array_equal(host(fused.scales).view(np.uint8), host(plain.scales).view(np.uint8))
    np.testing.assert_array_equal(host(fused.tensor_scale), host(plain.tensor_scale))
