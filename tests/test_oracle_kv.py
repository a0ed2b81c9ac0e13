"""Pins of the KV-cache decode oracle (oracle/kvcache.c), CPU only.

What fixes each function, independently of the oracle's own code:
  * the Walsh-Hadamard transform equals scipy's Sylvester Hadamard matrix
    times the vector (exact on small integers) and is its own inverse up to n;
  * the UE8M0 exponent follows closed forms of floor(log2 amax) - emax;
  * the E4M3 encoder equals torch's float8_e4m3fn cast (round to nearest even)
    on float32 inputs, ties included, and saturates at 448;
  * Q's MXFP8 and K's / V's MXFP4 codes equal a brute-force nearest search;
  * decode attention reduces to closed forms (a zero query averages V; a
    dominant key returns its value row), ignores tokens past the length, and
    stays within the error bound of E4M3-rounded probabilities of a plain
    numpy softmax over the dequantized operands.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle as O
import synthetic as S

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def bf16(a):
    return S.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def e4m3_torch(a32: np.ndarray) -> np.ndarray:
    """torch's RNE cast of non-negative float32 values <= 448 to E4M3FN bytes."""
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_values(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def e2m1_nearest(z: np.ndarray) -> np.ndarray:
    """Brute force: nearest E2M1 magnitude, ties to the even code, saturating."""
    a = np.abs(z.astype(np.float64))
    d = np.abs(a[..., None] - E2M1)
    best = np.argmin(d, axis=-1)
    # ties: prefer the even code
    dmin = d.min(axis=-1, keepdims=True)
    tie = (d == dmin).sum(axis=-1) > 1
    even = np.where((d == dmin) & (np.arange(8) % 2 == 0), np.arange(8), 99).min(axis=-1)
    best = np.where(tie, even, best)
    best = np.where(a >= 6.0, 7, best)
    return (best | np.where(np.signbit(z), 8, 0)).astype(np.uint8)


def floor_log2(a: float) -> int:
    return int(np.frexp(a)[1]) - 1


# ---- transform, exponent, encoder -------------------------------------------

@pytest.mark.parametrize("n", [32, 64, 128])
def test_fwht_is_the_sylvester_hadamard_matrix(n):
    rng = np.random.default_rng(n)
    x = rng.integers(-4, 5, n).astype(np.float32)
    H = scipy.linalg.hadamard(n).astype(np.float64)
    np.testing.assert_array_equal(O.fwht(x).astype(np.float64), H @ x)
    np.testing.assert_array_equal(O.fwht(O.fwht(x)), n * x)


def test_mx_exponent_closed_forms():
    assert O.mx_exponent(1.0, 2) == -2
    assert O.mx_exponent(6.0, 2) == 0
    assert O.mx_exponent(7.99, 2) == 0
    assert O.mx_exponent(8.0, 2) == 1
    assert O.mx_exponent(448.0, 8) == 0
    assert O.mx_exponent(1.0, 7) == -7
    assert O.mx_exponent(0.75, 7) == -8
    assert O.mx_exponent(0.0, 2) == -127
    assert O.mx_exponent(2.0 ** -130, 2) == -127      # clamped
    assert O.mx_exponent(2.0 ** 200, 2) == 127        # clamped


def test_e4m3_encoder_matches_torch_cast():
    rng = np.random.default_rng(1)
    a = np.float32(2.0 ** rng.uniform(-14, math.log2(448), 20000))
    codes = np.array([O.e4m3_encode_d(float(v)) for v in a], dtype=np.uint8)
    np.testing.assert_array_equal(codes, e4m3_torch(a))
    # exact midpoints between neighbouring codes go to the even code
    vals = e4m3_values(np.arange(0x7F, dtype=np.uint8))
    mids = np.float32((vals[:-1] + vals[1:]) / 2)
    codes = np.array([O.e4m3_encode_d(float(v)) for v in mids], dtype=np.uint8)
    np.testing.assert_array_equal(codes, e4m3_torch(mids))
    assert all(c % 2 == 0 for c in codes)
    assert O.e4m3_encode_d(460.0) == 0x7E and O.e4m3_encode_d(1e9) == 0x7E


# ---- Q, K, V quantizers ------------------------------------------------------

def mxfp8_brute(y: np.ndarray):
    """y float32 [D] -> (codes, scales) by the MX rule and torch's cast."""
    D = y.size
    codes = np.empty(D, np.uint8)
    scales = np.empty(D // 32, np.uint8)
    for g in range(D // 32):
        blk = y[32 * g:32 * g + 32].astype(np.float64)
        amax = np.abs(blk).max()
        e = -127 if amax == 0 else max(-127, min(127, floor_log2(amax) - 8))
        scales[g] = e + 127
        mag = np.minimum(np.abs(blk) * 2.0 ** -e, 448.0).astype(np.float32)
        codes[32 * g:32 * g + 32] = e4m3_torch(mag) | np.where(np.signbit(blk), 0x80, 0).astype(np.uint8)
    return codes, scales


def mxfp4_brute(y: np.ndarray):
    D = y.size
    nib = np.empty(D, np.uint8)
    scales = np.empty(D // 32, np.uint8)
    for g in range(D // 32):
        blk = y[32 * g:32 * g + 32].astype(np.float64)
        amax = np.abs(blk).max()
        e = -127 if amax == 0 else max(-127, min(127, floor_log2(amax) - 2))
        scales[g] = e + 127
        nib[32 * g:32 * g + 32] = e2m1_nearest(blk * 2.0 ** -e)
    return (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8), scales


def test_q_quantize_brute_force():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((24, 128)) * 2.0 ** rng.integers(-20, 20, (24, 1))
    q[0, :32] = 0
    q[1, :32] = 1.875 * 2.0 ** 3          # group max lands in [448, 512): saturation
    q = bf16(q)
    codes, scales = O.q_quantize(q, rotate=False)
    for r in range(q.shape[0]):
        c, s = mxfp8_brute(S.bf16_bits_to_f32(q[r]))
        np.testing.assert_array_equal(codes[r], c)
        np.testing.assert_array_equal(scales[r], s)
    assert codes[1, 0] == 0x7E


def test_q_quantize_rotated_integer_inputs():
    """On small integers the binary32 transform is exact: y = H q / D."""
    rng = np.random.default_rng(3)
    H = scipy.linalg.hadamard(128).astype(np.float64)
    q = rng.integers(-6, 7, (8, 128)).astype(np.float32)
    codes, scales = O.q_quantize(bf16(q), rotate=True)
    for r in range(8):
        c, s = mxfp8_brute((H @ q[r] / 128).astype(np.float32))
        np.testing.assert_array_equal(codes[r], c)
        np.testing.assert_array_equal(scales[r], s)


def test_kv_quantize_seq_brute_force():
    rng = np.random.default_rng(4)
    L, D, length, ntok = 80, 128, 77, 96
    k = bf16(rng.standard_normal((L, D)) * 2.0 ** rng.integers(-8, 8, (L, 1)))
    v = bf16(rng.standard_normal((L, D)) * 2.0 ** rng.integers(-8, 8, (1, D)))
    kc, ks, vc, vs = O.kv_quantize_seq(k, v, length, ntok, rotate=False)
    for t in range(ntok):
        y = S.bf16_bits_to_f32(k[t]) if t < length else np.zeros(D, np.float32)
        c, s = mxfp4_brute(y)
        np.testing.assert_array_equal(kc[t], c)
        np.testing.assert_array_equal(ks[t], s)
    assert (kc[length:] == 0).all() and (ks[length:] == 0).all()
    vf = np.zeros((ntok, D), np.float32)
    vf[:length] = S.bf16_bits_to_f32(v[:length])
    for d in range(D):
        c, s = mxfp4_brute(vf[:, d])
        np.testing.assert_array_equal(vc[d], c)
        np.testing.assert_array_equal(vs[d], s)


def test_k_quantize_rotated_integer_inputs():
    rng = np.random.default_rng(5)
    H = scipy.linalg.hadamard(128).astype(np.float64)
    k = rng.integers(-3, 4, (32, 128)).astype(np.float32)
    kc, ks, _, _ = O.kv_quantize_seq(bf16(k), bf16(k), 32, 32, rotate=True)
    for t in range(32):
        c, s = mxfp4_brute((H @ k[t]).astype(np.float32))
        np.testing.assert_array_equal(kc[t], c)
        np.testing.assert_array_equal(ks[t], s)


# ---- decode attention --------------------------------------------------------

def dequant_seq(q, k, v, length, rotate, fmt="fp4"):
    """Dequantized operands from the (brute-force pinned) quantizers."""
    D = q.shape[1]
    ntok = (length + 31) // 32 * 32
    qc, qs = O.q_quantize(q, rotate)
    qh = e4m3_values(qc) * 2.0 ** (qs.astype(np.int64) - 127).repeat(32, axis=1)
    kc, ks, vc, vs = O.kv_quantize_seq(k, v, length, ntok, rotate, fmt)
    def nib(codes):
        if fmt == "fp8":
            return e4m3_values(codes)
        n = np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)
        return np.where(n & 8, -1.0, 1.0) * E2M1[n & 7]
    kh = nib(kc) * 2.0 ** (ks.astype(np.int64) - 127).repeat(32, axis=1)
    vh = (nib(vc) * 2.0 ** (vs.astype(np.int64) - 127).repeat(32, axis=1)).T
    return qh, kh[:length], vh[:length]


def test_decode_zero_query_averages_v():
    """q = 0: every score is 0, every probability exactly 1, so the output is
    the mean of V over the valid tokens; V on the E2M1 grid with a 6 in each
    group is quantized exactly."""
    rng = np.random.default_rng(6)
    G, D, L, length = 3, 128, 96, 50
    v = E2M1[rng.integers(0, 8, (L, D))] * rng.choice([-1.0, 1.0], (L, D))
    v[0::32, :] = 6.0
    k = rng.standard_normal((L, D))
    out = O.kv_decode_seq(np.zeros((G, D), np.uint16), bf16(k), bf16(v), length, 0.1, rotate=True)
    np.testing.assert_allclose(out, np.tile(v[:length].mean(axis=0), (G, 1)), rtol=0, atol=1e-15)


def test_decode_dominant_key_returns_its_value():
    """One key far ahead of the rest: every other probability rounds to an
    E4M3 zero, so the output is that token's dequantized value row times
    p'/p, a factor within one E4M3 half-step of 1."""
    rng = np.random.default_rng(7)
    D, L, tstar = 128, 200, 137
    q = np.zeros((1, D))
    q[0, 5] = 1.0
    k = np.zeros((L, D))
    k[tstar, 5] = 6.0
    v = rng.standard_normal((L, D))
    qb, kb, vb = bf16(q), bf16(k), bf16(v)
    out = O.kv_decode_seq(qb, kb, vb, L, 40.0, rotate=False)[0]
    _, _, vh = dequant_seq(qb, kb, vb, L, False)
    ratio = out @ vh[tstar] / (vh[tstar] @ vh[tstar])
    np.testing.assert_allclose(out, ratio * vh[tstar], rtol=1e-13, atol=0)
    assert abs(ratio - 1) <= 2.0 ** -4


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
@pytest.mark.parametrize("rotate", [False, True])
def test_decode_within_fp8_probability_bound(rotate, fmt):
    """The output differs from a plain numpy softmax over the dequantized
    operands only by the E4M3 rounding of the probabilities: per token at
    most 2^-4 p (normal range) or 2^(E-10) (subnormal range, E the group's
    exponent floor(log2 max p) - 7)."""
    G, D, L, length, sm = 8, 128, 1000, 931, 1 / math.sqrt(128)
    q = S.kv_q(1, G, D, seed=8)[0]
    k, v = S.kv_seq(0, 0, L, D, seed=8)
    out = O.kv_decode_seq(q, k, v, length, sm, rotate, fmt)
    qh, kh, vh = dequant_seq(q, k, v, length, rotate, fmt)
    s = qh @ kh.T * sm
    p = np.exp(s - s.max(axis=1, keepdims=True))
    ref = p @ vh / p.sum(axis=1, keepdims=True)
    # bound in units where the row maximum is 1 (the output is scale-free)
    ntok = (length + 31) // 32 * 32
    pp = np.zeros((G, ntok))
    pp[:, :length] = p
    amax = pp.reshape(G, -1, 32).max(axis=2)
    E = np.floor(np.log2(amax)) - 7
    sub = 2.0 ** (E - 10)
    bound_t = np.maximum(2.0 ** -4 * p, np.repeat(sub, 32, axis=1)[:, :length])
    bound = bound_t @ np.abs(vh) / p.sum(axis=1, keepdims=True)
    err = np.abs(out - ref)
    assert (err <= bound + 1e-12).all()
    assert err.max() > 0                       # the probabilities are really rounded
    assert np.linalg.norm(out - ref) / np.linalg.norm(ref) < 5e-2   # FP8 probabilities cost ~2 %


def test_decode_ignores_tokens_past_the_length():
    rng = np.random.default_rng(9)
    G, D, L, length = 4, 128, 300, 161
    q = bf16(rng.standard_normal((G, D)))
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    k[length:] = 1e4
    v[length:] = -1e4
    a = O.kv_decode_seq(q, bf16(k), bf16(v), length, 0.09, True)
    b = O.kv_decode_seq(q, bf16(k[:length]), bf16(v[:length]), length, 0.09, True)
    np.testing.assert_array_equal(a, b)
    assert not np.any(O.kv_decode_seq(q, bf16(k), bf16(v), 0, 0.09, True))    # empty cache: zeros


def test_decode_rows_are_independent():
    q = S.kv_q(1, 6, 128, seed=10)[0]
    k, v = S.kv_seq(0, 1, 256, 128, seed=10)
    all_rows = O.kv_decode_seq(q, k, v, 256, 0.088, True)
    for r in range(6):
        np.testing.assert_array_equal(all_rows[r], O.kv_decode_seq(q[r:r + 1], k, v, 256, 0.088, True)[0])


def test_rotation_helps_keys_with_outlier_channels():
    """Keys with a few large channels: the Walsh-Hadamard rotation lowers
    the error against unquantized attention (fp64 softmax of the bf16 inputs)."""
    G, D, L, sm = 8, 128, 2048, 1 / math.sqrt(128)
    q = S.kv_q(1, G, D, seed=11)[0]
    k, v = S.kv_seq(0, 0, L, D, seed=11)
    qf, kf, vf = (S.bf16_bits_to_f32(t).astype(np.float64) for t in (q, k, v))
    s = qf @ kf.T * sm
    p = np.exp(s - s.max(axis=1, keepdims=True))
    exact = p @ vf / p.sum(axis=1, keepdims=True)
    e_rot = np.linalg.norm(O.kv_decode_seq(q, k, v, L, sm, True) - exact)
    e_raw = np.linalg.norm(O.kv_decode_seq(q, k, v, L, sm, False) - exact)
    assert e_rot < e_raw


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_comparison_bound_covers_perturbed_scores(fmt):
    """kv_decode_bounds: a decode whose scores are perturbed anywhere inside
    the allowed error (here in numpy, probabilities rounded by torch's E4M3
    cast) stays within 2e-4 mass + amb of the oracle, and the bound is zero
    where no code can move."""
    G, D, L, length, sm = 4, 128, 1024, 1000, 1 / math.sqrt(128)
    q = S.kv_q(1, G, D, seed=12)[0]
    k, v = S.kv_seq(0, 0, L, D, seed=12)
    want = O.kv_decode_seq(q, k, v, length, sm, True, fmt)
    mass, amb, nfrag = O.kv_decode_bounds(q, k, v, length, sm, True, eps_s=2.0 ** -15, fmt=fmt)
    assert (amb >= 0).all() and (mass > 0).all() and nfrag > 0
    qh, kh, vh = dequant_seq(q, k, v, length, True, fmt)
    s = qh @ kh.T
    sabs = np.abs(qh) @ np.abs(kh).T
    c = sm / math.log(2)
    rng = np.random.default_rng(13)
    ntok = (length + 31) // 32 * 32
    for _ in range(6):
        x = (s + rng.uniform(-1, 1, s.shape) * 2.0 ** -15 * sabs) * c
        p = np.exp2(x - np.ceil(x.max(axis=1, keepdims=True)))
        pp = np.zeros((G, ntok))
        pp[:, :length] = p
        E = np.floor(np.log2(pp.reshape(G, -1, 32).max(axis=2))) - 7
        scale = np.repeat(2.0 ** E, 32, axis=1)
        ph = e4m3_values(e4m3_torch((pp / scale).astype(np.float32))).reshape(G, ntok) * scale
        out = ph[:, :length] @ vh / p.sum(axis=1, keepdims=True)
        assert (np.abs(out - want) <= 2e-4 * mass + amb).all()
    # with no score error only the exponential's 2^-20 allowance remains
    _, amb0, nf0 = O.kv_decode_bounds(q, k, v, length, sm, True, eps_s=0.0, fmt=fmt)
    assert nf0 < nfrag and amb0.max() < amb.max()


# ---- the FP8 (MXFP8) cache baseline -------------------------------------------

@pytest.mark.parametrize("rotate", [False, True])
def test_fp8_cache_brute_force(rotate):
    rng = np.random.default_rng(14)
    L, D, length, ntok = 70, 128, 65, 96
    k = rng.integers(-5, 6, (L, D)).astype(np.float32) if rotate else \
        rng.standard_normal((L, D)) * 2.0 ** rng.integers(-8, 8, (L, 1))
    v = rng.standard_normal((L, D)) * 2.0 ** rng.integers(-8, 8, (1, D))
    v[3, :] = 1.9 * 2.0 ** 6            # group maxima in [448, 512) after scaling: saturation
    kb, vb = bf16(k), bf16(v)
    kc, ks, vc, vs = O.kv_quantize_seq(kb, vb, length, ntok, rotate, "fp8")
    H = scipy.linalg.hadamard(128).astype(np.float64)
    for t in range(ntok):
        y = (S.bf16_bits_to_f32(kb[t]) if t < length else np.zeros(D, np.float32)).astype(np.float64)
        c, sc = mxfp8_brute((H @ y if rotate else y).astype(np.float32))
        np.testing.assert_array_equal(kc[t], c)
        np.testing.assert_array_equal(ks[t], sc)
    vf = np.zeros((ntok, D), np.float32)
    vf[:length] = S.bf16_bits_to_f32(vb[:length])
    for d in range(D):
        c, sc = mxfp8_brute(vf[:, d])
        np.testing.assert_array_equal(vc[d], c)
        np.testing.assert_array_equal(vs[d], sc)
    assert (vc[:, 3] & 0x7F == 0x7E).any()       # some saturated code


def test_fp8_decode_zero_query_averages_v():
    """Integers in [-8, 8] with an 8 in every 32-token group are exact in
    MXFP8 (exponent -5, codes up to 256), so a zero query returns their mean."""
    rng = np.random.default_rng(15)
    G, D, L, length = 2, 128, 64, 61
    v = rng.integers(-8, 9, (L, D)).astype(np.float64)
    v[0::32, :] = 8.0
    k = rng.standard_normal((L, D))
    out = O.kv_decode_seq(np.zeros((G, D), np.uint16), bf16(k), bf16(v), length, 0.1, True, "fp8")
    np.testing.assert_allclose(out, np.tile(v[:length].mean(axis=0), (G, 1)), rtol=0, atol=1e-15)


def test_fp8_cache_is_closer_to_exact_attention():
    G, D, L, sm = 8, 128, 2048, 1 / math.sqrt(128)
    q = S.kv_q(1, G, D, seed=16)[0]
    k, v = S.kv_seq(0, 0, L, D, seed=16)
    qf, kf, vf = (S.bf16_bits_to_f32(t).astype(np.float64) for t in (q, k, v))
    s = qf @ kf.T * sm
    p = np.exp(s - s.max(axis=1, keepdims=True))
    exact = p @ vf / p.sum(axis=1, keepdims=True)
    e4 = np.linalg.norm(O.kv_decode_seq(q, k, v, L, sm, True, "fp4") - exact)
    e8 = np.linalg.norm(O.kv_decode_seq(q, k, v, L, sm, True, "fp8") - exact)
    assert e8 < e4 / 3

