"""The launch-timing aid: a timed launch computes the same result as an
untimed one and its events bracket a positive duration; the request is used
once."""
import numpy as np
import pytest

import synthetic as S
from helpers import host, to_device_bf16

pytestmark = pytest.mark.gpu


def test_timed_quantize_matches_untimed_and_reports_duration():
    import torch
    import block_scaled_bit_ufp4_amd as U
    x = to_device_bf16(S.quantize_x(512, 1024, seed=3))
    cfg = U.Cfg("e2m1", "e4m3", rht="random", rht_seed=5)
    amax = U.ufp4_amax(x, cfg)
    plain = U.ufp4_quantize(x, cfg, amax=amax)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    U.ufp4_time_next_launch(a, b)
    timed = U.ufp4_quantize(x, cfg, amax=amax)
    torch.cuda.synchronize()
    assert a.elapsed_time(b) > 0
    np.testing.assert_array_equal(host(timed.codes), host(plain.codes))
    np.testing.assert_array_equal(host(timed.scales), host(plain.scales))
    # consumed: a later call does not touch the events again
    t0 = a.elapsed_time(b)
    U.ufp4_quantize(x, cfg, amax=amax)
    torch.cuda.synchronize()
    assert a.elapsed_time(b) == t0


def test_timed_gemm_matches_untimed():
    import torch
    import block_scaled_bit_ufp4_amd as U
    a = to_device_bf16(S.normal(256, 512, 1.0, 7, "gemm_a"))
    b = to_device_bf16(S.normal(512, 512, 1.0, 7, "gemm_b"))
    cfg = U.Cfg("e2m1", "e8m0", 32)
    qa, qb = U.ufp4_quantize(a, cfg), U.ufp4_quantize(b, cfg)
    z0 = U.ufp4_qgemm(qa, qb, "mxfp4")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    U.ufp4_time_next_launch(e0, e1)
    z1 = U.ufp4_qgemm(qa, qb, "mxfp4")
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) > 0
    np.testing.assert_array_equal(host(z1), host(z0))
