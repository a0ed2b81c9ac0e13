"""Seeded random sweep of the quantizer against the oracle: random view
shapes (ragged against every tile), every supported configuration, random
transform and rounding seeds and streams, input kinds from heavy-tailed to
tiny (1e-30) and sparse, bf16 and binary32 sources.  Codes, scales, tensor
scale and the dequantized values must match bit for bit."""
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
