"""The allocation-free amax entry point (ufp4_amax_noalloc, the library's
built-in scratch instead of a workspace) called through the C ABI: equal to
ufp4_amax bit for bit on two calls in a row, the second with a smaller input
(the scratch keeps the first call's partials), for both axes and with and
without the transform; sizes past the scratch are refused before anything
runs."""
import ctypes as C

import numpy as np
import pytest
import torch

import synthetic as S
from helpers import to_device_bf16

pytestmark = pytest.mark.gpu


def lib():
    import block_scaled_bit_ufp4_amd as U
    return U


def noalloc(U, x, cfg, out):
    c = cfg.c()
    return U.lib().ufp4_amax_noalloc(x.data_ptr(), 0, x.shape[0], x.shape[1], x.stride(0), C.byref(c),
                                     out.data_ptr(), torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("rht", ["none", "random"])
def test_noalloc_amax_equals_workspace_amax(axis, rht):
    U = lib()
    cfg = U.Cfg("e2m1", "e4m3", rht=rht, rht_seed=3, axis=axis)
    # a larger tensor first, then a smaller one whose partials are fewer
    for (R, Cc), seed in (((4096, 2048), 1), ((272, 96), 2)):
        x = to_device_bf16(S.activations_t3(R, Cc, seed=seed))
        got = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
        assert noalloc(U, x, cfg, got) == 0
        want = U.ufp4_amax(x, cfg)
        torch.cuda.synchronize()
        assert got.item() == want.item(), (axis, rht, R, Cc)
        assert got.item() == float(x.float().abs().max()) or rht != "none"


def test_noalloc_amax_refuses_sizes_past_its_scratch():
    U = lib()
    c = U.Cfg("e2m1", "e4m3").c()
    fake = 0x10000  # never dereferenced: the size check comes first
    big = U.lib().ufp4_amax_noalloc(fake, 0, 1 << 16, (1 << 14) + 16, (1 << 14) + 16, C.byref(c), fake, None)
    assert big == -5
    ok_rows = (1 << 30) // (1 << 14)
    assert U.ufp4_workspace_size(U.OP_AMAX, ok_rows, 1 << 14, U.Cfg()) == 65536 * 4
