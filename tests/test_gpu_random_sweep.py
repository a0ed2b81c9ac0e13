"""Seeded random sweeps against the oracle.  The quantizer: random view
shapes (ragged against every tile), every supported configuration, random
transform and rounding seeds and streams, input kinds from heavy-tailed to
tiny (1e-30) and sparse, bf16 and binary32 sources.  Codes, scales, tensor
scale and the dequantized values must match bit for bit.  The GEMMs: random
shapes and operand formats in both modes.  The KV decode: random shapes,
lengths, splits, rotation and cache format."""
import random

import numpy as np
import pytest

import oracle as O
import synthetic as S
from helpers import host, oracle_cfg, to_device_bf16, to_device_f32
from test_gpu_quantize import all_configs

pytestmark = pytest.mark.gpu


def _case(rng, cfgs):
    d = rng.choice(cfgs)
    B = 32 if d["scale"] == "e8m0" else 16
    if d["axis"] == "row":
        R, Cc = rng.randint(1, 300), B * rng.randint(1, 90)
    else:
        R, Cc = B * rng.randint(1, 90), 8 * rng.randint(1, 40)
    kind = rng.choice(["t3", "normal", "outliers", "tiny", "sparse"])
    seed = rng.randint(0, 10 ** 6)
    if kind == "t3":
        x = S.activations_t3(R, Cc, seed=seed)
    elif kind == "outliers":
        x = S.llama_x(R, Cc, seed=seed)
    elif kind == "tiny":
        x = S.normal(R, Cc, 1e-30, seed)
    elif kind == "sparse":
        x = S.normal(R, Cc, 1.0, seed)
        x = np.where(np.random.default_rng(seed).random((R, Cc)) < 0.3, np.uint16(0), x).astype(np.uint16)
    else:
        x = S.normal(R, Cc, 1.0, seed)
    dtype = rng.choice(["bf16", "bf16", "f32"])
    return d, x, dtype, (rng.randint(0, 2 ** 32 - 1), rng.randint(0, 2 ** 63), rng.randint(0, 3))


@pytest.mark.parametrize("master", [11, 12, 13])
def test_random_sweep_bit_exact(master):
    import block_scaled_bit_ufp4_amd as U
    rng = random.Random(master)
    cfgs = all_configs()
    for it in range(200):
        d, x, dtype, (rseed, sseed, stream) = _case(rng, cfgs)
        cfg = U.Cfg(**d, rht_seed=rseed, sr_seed=sseed, sr_stream=stream)
        ocfg = oracle_cfg(cfg)
        if dtype == "bf16":
            xd, xo = to_device_bf16(x), x
        else:
            xo = S.bf16_bits_to_f32(x) * np.float32(1.0 + 2 ** -12)
            xd = to_device_f32(xo)
        q = U.ufp4_quantize(xd, cfg)
        want = O.quantize(xo, ocfg)
        tag = f"case {it}: {d} {x.shape} {dtype} seeds {rseed} {sseed} {stream}"
        np.testing.assert_array_equal(host(q.codes), want.codes, err_msg=tag)
        np.testing.assert_array_equal(host(q.scales), want.scales, err_msg=tag)
        if cfg.scale == "e4m3":
            assert host(q.tensor_scale)[0] == np.float32(want.alpha), tag
        got = host(U.ufp4_dequantize(q))
        ref = O.dequantize(want, ocfg, xo.shape)
        np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32), err_msg=tag)


def _rel_fro(got, want):
    return float(np.linalg.norm(got.astype(np.float64) - want) / np.linalg.norm(want))


@pytest.mark.parametrize("master", [21, 22])
def test_random_gemm_sweep(master):
    """Random GEMM shapes (M, N multiples of 256, K of 128) and operand
    formats in both modes, against the oracle's binary64 product of its own
    dequantized (for the bf16 mode, bf16-rounded) operands."""
    import block_scaled_bit_ufp4_amd as U
    rng = random.Random(master)
    for it in range(8):
        M, N, K = 256 * rng.randint(1, 5), 256 * rng.randint(1, 5), 128 * rng.randint(1, 16)
        mode = rng.choice(["mxfp4", "bf16"])
        seed = rng.randint(0, 10 ** 6)
        rht = rng.choice(["none", "random", "det"])
        if mode == "mxfp4":
            cfg = U.Cfg("e2m1", "e8m0", 32, rht=rht, rht_seed=seed)
        else:
            fmt = rng.choice(["e1m2", "int4", "e2m1", "if4", "e2m1_max3"])
            scale = "e4m3" if fmt == "if4" else rng.choice(["fp32", "e4m3"])
            cfg = U.Cfg(fmt, scale, rht=rht, rht_seed=seed)
        a = S.activations_t3(M, K, seed=seed)
        b = S.normal(N, K, 1.0, seed + 1, "gemm_b")
        qa, qb = U.ufp4_quantize(to_device_bf16(a), cfg), U.ufp4_quantize(to_device_bf16(b), cfg)
        z = host(U.ufp4_qgemm(qa, qb, mode))
        ocfg = oracle_cfg(cfg)
        bf = mode == "bf16"
        opa = O.dequantize(O.quantize(a, ocfg), ocfg, a.shape)
        opb = O.dequantize(O.quantize(b, ocfg), ocfg, b.shape)
        want = O.gemm_nt(O.bf16_round(opa) if bf else opa, O.bf16_round(opb) if bf else opb)
        err = _rel_fro(z, want)
        assert err < 1e-5, f"case {it}: {mode} {cfg} {(M, N, K)}: {err}"


@pytest.mark.parametrize("master", [31, 32])
def test_random_kv_decode_sweep(master):
    """Random batches, heads, group sizes, capacities, ragged lengths (zero
    and full included), splits, rotation and cache format, against the
    oracle's decode within its bound."""
    import math
    import torch
    import block_scaled_bit_ufp4_amd as U
    from test_gpu_kv import check_against_oracle
    rng = random.Random(master)
    for it in range(5):
        B, Hkv, G = rng.randint(1, 3), rng.randint(1, 3), rng.choice([1, 2, 4, 8, 16])
        L = 128 * rng.randint(1, 12)
        lens = np.array([rng.choice([0, L, rng.randint(1, L)]) for _ in range(B)], np.int32)
        rotate, fmt, pps = rng.choice([True, False]), rng.choice(["fp4", "fp8"]), rng.choice([0, 1, 2, 3, 8])
        q, k, v = S.kv_decode(B, G * Hkv, Hkv, L, seed=rng.randint(0, 10 ** 6))
        sm = 1.0 / math.sqrt(128)
        d_lens = torch.from_numpy(lens).cuda()
        cache = U.ufp4_kv_cache_quantize(to_device_bf16(k), to_device_bf16(v), d_lens, rotate, fmt=fmt)
        out = host(U.ufp4_kv_decode(to_device_bf16(q), cache, d_lens, Hkv, L, sm, rotate, pages_per_split=pps,
                                    fmt=fmt))
        check_against_oracle(out, q, k, v, lens, Hkv, rotate, sm, fmt=fmt)
