"""FP4 KV-cache decode attention on the GPU against the oracle.

  * the cache quantizer's codes and exponents equal the oracle's MXFP4 (and,
    for the FP8 baseline, MXFP8) of K (rotated or not) and V bit for bit, for
    ragged lengths and strided inputs;
  * the query quantizer equals the oracle's MXFP8 bit for bit;
  * decode outputs match the oracle element by element within
    2e-4 x mass + amb, for several query-group sizes, split counts and ragged
    lengths, and at the full llama-8B-shaped size on sampled sequences.  The
    oracle computes scores, probabilities and the output in binary64, the
    kernel in fp32 on the MFMA (accumulation error of a score up to about
    2^-17 of the sum of its products' magnitudes, measured) with a few-ulp
    2^x, so a probability whose E4M3 code (or block exponent) lies within
    that distance of a rounding boundary may legitimately round the other
    way.  mass = sum p'|V'| / sum p is the scale of each output element;
    amb bounds the change from every such code (oracle.kv_decode_bounds, with
    4x margin on the score error);
  * different split counts give the same output up to fp32 summation order
    (the splits combine by exact powers of two).
"""
import math

import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import host, kv_unshuffle, to_device_bf16

pytestmark = pytest.mark.gpu


def U():
    import block_scaled_bit_ufp4_amd as lib
    return lib


def dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def rel_fro(got, want):
    n = np.linalg.norm(want)
    return float(np.linalg.norm(got.astype(np.float64) - want) / (n if n > 0 else 1.0))


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
@pytest.mark.parametrize("rotate", [True, False])
def test_cache_bits_match_oracle(rotate, fmt):
    B, Hq, Hkv, L = 3, 8, 2, 384
    lens = np.array([384, 200, 1], np.int32)
    q, k, v = S.kv_decode(B, Hq, Hkv, L, seed=1)
    cache = host(U().ufp4_kv_cache_quantize(to_device_bf16(k), to_device_bf16(v), dev_i32(lens), rotate, fmt=fmt))
    for b in range(B):
        npg = (int(lens[b]) + 127) // 128
        for h in range(Hkv):
            got = kv_unshuffle(cache, B, Hkv, L, b, h, npg, fmt)
            want = O.kv_quantize_seq(k[b, h], v[b, h], int(lens[b]), 128 * npg, rotate, fmt)
            for name, gg, ww in zip(("kcodes", "kscales", "vcodes", "vscales"), got, want):
                np.testing.assert_array_equal(gg, ww, err_msg=f"{name} b={b} h={h}")


def test_cache_from_token_major_views():
    """K, V as [B][L][Hkv][D] tensors (the projection's layout), passed as
    permuted views: same cache as from contiguous [B][Hkv][L][D]."""
    import torch
    B, Hq, Hkv, L = 2, 4, 2, 256
    lens = np.array([256, 131], np.int32)
    _, k, v = S.kv_decode(B, Hq, Hkv, L, seed=2)
    kt = to_device_bf16(np.ascontiguousarray(k.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
    vt = to_device_bf16(np.ascontiguousarray(v.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
    a = U().ufp4_kv_cache_quantize(kt, vt, dev_i32(lens), True)
    b = U().ufp4_kv_cache_quantize(to_device_bf16(k), to_device_bf16(v), dev_i32(lens), True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(a), host(b))


@pytest.mark.parametrize("rotate", [True, False])
def test_q_quantize_bits(rotate):
    rng = np.random.default_rng(3)
    q = rng.standard_normal((37, 128)) * 2.0 ** rng.integers(-30, 30, (37, 1))
    q[0] = 0
    q[1, :32] = 1.875 * 8.0            # saturation at 448
    q[2, 40] = -1e-40                   # subnormal input
    qb = S.f32_to_bf16_bits(q.astype(np.float32))
    codes, scales = U().ufp4_kv_q_quantize(to_device_bf16(qb), rotate)
    want_c, want_s = O.q_quantize(qb, rotate)
    np.testing.assert_array_equal(host(codes), want_c)
    np.testing.assert_array_equal(host(scales), want_s)


def run_decode(q, k, v, lens, Hkv, rotate, sm, pps=0, fmt="fp4"):
    L = k.shape[2]
    d_lens = dev_i32(lens)
    cache = U().ufp4_kv_cache_quantize(to_device_bf16(k), to_device_bf16(v), d_lens, rotate, fmt=fmt)
    out = U().ufp4_kv_decode(to_device_bf16(q), cache, d_lens, Hkv, L, sm, rotate, pages_per_split=pps, fmt=fmt)
    return host(out)


def check_against_oracle(out, q, k, v, lens, Hkv, rotate, sm, pairs=None, fmt="fp4"):
    """Element-wise |got - want| <= 2e-4 mass + amb; returns the largest ratio
    of the error to that bound and the largest relative Frobenius error."""
    B, Hq, _ = q.shape
    G = Hq // Hkv
    worst, worst_fro = 0.0, 0.0
    for b, h in (pairs or [(b, h) for b in range(B) for h in range(Hkv)]):
        args = (q[b, h * G:(h + 1) * G], k[b, h], v[b, h], int(lens[b]), sm, rotate)
        want = O.kv_decode_seq(*args, fmt=fmt)
        got = out[b, h * G:(h + 1) * G]
        if int(lens[b]) == 0:
            assert not np.any(got), (b, h)
            continue
        mass, amb, _ = O.kv_decode_bounds(*args, fmt=fmt)
        ratio = np.abs(got.astype(np.float64) - want) / (2e-4 * mass + amb + 1e-300)
        worst = max(worst, float(ratio.max()))
        worst_fro = max(worst_fro, rel_fro(got, want))
        assert ratio.max() <= 1.0, (b, h, np.unravel_index(np.argmax(ratio), ratio.shape), float(ratio.max()))
        assert rel_fro(got, want) < 5e-2, (b, h)
    return worst, worst_fro


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
@pytest.mark.parametrize("G", [1, 4, 8, 16])
@pytest.mark.parametrize("rotate", [True, False])
def test_decode_matches_oracle(G, rotate, fmt):
    B, Hkv, L = 3, 2, 1024
    lens = np.array([1024, 777, 129], np.int32)
    q, k, v = S.kv_decode(B, G * Hkv, Hkv, L, seed=4 + G)
    sm = 1.0 / math.sqrt(128)
    out = run_decode(q, k, v, lens, Hkv, rotate, sm, fmt=fmt)
    worst, fro = check_against_oracle(out, q, k, v, lens, Hkv, rotate, sm, fmt=fmt)
    print(f"{fmt} G={G} rotate={rotate}: error / bound {worst:.3g}, rel Frobenius {fro:.3g}")


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
@pytest.mark.parametrize("pps", [1, 2, 3, 5, 64])
def test_decode_split_counts(pps, fmt):
    """Different pages per split: every result within the oracle bar, and
    equal to the unsplit result up to fp32 summation order."""
    B, Hq, Hkv, L = 2, 8, 2, 1280
    lens = np.array([1280, 1000], np.int32)
    q, k, v = S.kv_decode(B, Hq, Hkv, L, seed=9)
    sm = 1.0 / math.sqrt(128)
    out = run_decode(q, k, v, lens, Hkv, True, sm, pps=pps, fmt=fmt)
    check_against_oracle(out, q, k, v, lens, Hkv, True, sm, fmt=fmt)
    ref = run_decode(q, k, v, lens, Hkv, True, sm, pps=64, fmt=fmt)
    assert rel_fro(out, ref.astype(np.float64)) < 1e-5


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_decode_edge_lengths(fmt):
    """Lengths 0 (zeros), 1, 127, 128, 129, and one past the capacity
    (clamped to it)."""
    B, Hq, Hkv, L = 6, 4, 1, 256
    lens = np.array([0, 1, 127, 128, 129, 300], np.int32)
    q, k, v = S.kv_decode(B, Hq, Hkv, L, seed=10)
    sm = 0.1
    out = run_decode(q, k, v, lens, Hkv, True, sm, fmt=fmt)
    check_against_oracle(out, q, k, v, np.minimum(lens, L), Hkv, True, sm, fmt=fmt)
    assert not np.any(out[0])


def test_empty_batch_is_a_no_op():
    import torch
    q = torch.zeros((0, 4, 128), dtype=torch.bfloat16, device="cuda")
    out = U().ufp4_kv_decode(q, torch.zeros(16, dtype=torch.uint8, device="cuda"),
                             torch.zeros(1, dtype=torch.int32, device="cuda"), 1, 128, 0.1)
    assert out.shape == (0, 4, 128)


@pytest.fixture(scope="module")
def llama_decode():
    B, Hq, Hkv, L = 32, 32, 8, 16384
    q, k, v = S.kv_decode(B, Hq, Hkv, L, seed=0)
    return q, k, v, S.kv_lens(B, L)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_full_size_sampled_sequences(llama_decode, fmt):
    """Llama-3-8B-shaped decode (32 sequences x 16384 tokens, 32 query and 8
    KV heads): five sampled (sequence, KV head) pairs against the oracle."""
    q, k, v, lens = llama_decode
    sm = 1.0 / math.sqrt(128)
    out = run_decode(q, k, v, lens, 8, True, sm, fmt=fmt)
    pairs = [(0, 0), (31, 7), (5, 3), (17, 1), (26, 6)]
    worst, fro = check_against_oracle(out, q, k, v, lens, 8, True, sm, pairs=pairs, fmt=fmt)
    print(f"{fmt} full size: error / bound {worst:.3g}, rel Frobenius {fro:.3g}")
    assert np.all(np.isfinite(out))
