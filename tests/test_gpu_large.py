"""Tensors past the sizes the other tests reach: 160 copies of an 8192x8192
tile stacked along rows (10.7 G elements, 21.5 GB of bf16).  Every
quantization of the stack must be the tile's, repeated (the row quantization
tile by tile, the column quantization period by period along each view row),
which checks the quantizer at offsets far past 2^32 bytes.  The statistics
kernel takes at most 2^15 elements per thread in one launch, so on a tensor
this large it runs several launches, the later ones adding to the partial
sums: every count must be 160 times the tile's and every sum 160 times the
tile's to within summation order."""
import numpy as np
import pytest

import synthetic as S
from helpers import host, to_device_bf16

pytestmark = pytest.mark.gpu

T = 160          # tiles in the stack
R0 = C0 = 8192   # tile shape


def lib():
    import block_scaled_bit_ufp4_amd as U
    return U


@pytest.fixture(scope="module")
def tile():
    import torch
    x = to_device_bf16(S.activations_t3(R0, C0, seed=3))
    yield x
    del x
    torch.cuda.empty_cache()


def check_scaled_sums(big, one, n):
    """The 48 sums of the stack against n times the tile's."""
    big, want = np.asarray(big, np.float64), n * np.asarray(one, np.float64)
    np.testing.assert_array_equal(big[[0, 7, 8]], want[[0, 7, 8]])      # elements, blocks, INT4 blocks
    np.testing.assert_array_equal(big[16:32], want[16:32])              # code counts
    for k in (1, 2, 5, 6):
        assert abs(big[k] - want[k]) <= 1e-9 * abs(want[k]), k
    for k in (3, 4):                                                    # nearly cancelling sums
        assert abs(big[k] - want[k]) <= 1e-9 * want[6], k
    assert np.all(np.abs(big[32:48] - want[32:48]) <= 1e-9 * np.maximum(want[16:32], 1.0))


@pytest.mark.parametrize("spec", [
    dict(format="e2m1", scale="e4m3", rht="random", rht_seed=5),
    dict(format="e2m1", scale="e8m0", block=32, rht="det"),
    dict(format="e1m2", scale="fp32", rht="random", rht_seed=5, axis="col"),
])
def test_stacked_tiles(tile, spec):
    import torch
    U = lib()
    cfg = U.Cfg(**spec)
    big = tile.repeat(T, 1)
    assert big.shape == (T * R0, C0)
    amax_t = amax_b = None
    if cfg.scale == "e4m3":
        amax_t, amax_b = U.ufp4_amax(tile, cfg), U.ufp4_amax(big, cfg)
        assert host(amax_b)[0] == host(amax_t)[0]
    q_t = U.ufp4_quantize(tile, cfg, amax=amax_t)
    q_b = U.ufp4_quantize(big, cfg, amax=amax_b)
    if cfg.axis == "row":
        # view rows of the stack: T copies of the tile's
        assert torch.equal(q_b.codes.view(T, R0, -1), q_t.codes.unsqueeze(0).expand(T, -1, -1))
        assert torch.equal(q_b.scales.view(T, R0, -1), q_t.scales.unsqueeze(0).expand(T, -1, -1))
    else:
        # each view row (a source column) repeats the tile's with period R0
        assert torch.equal(q_b.codes.view(C0, T, -1), q_t.codes.unsqueeze(1).expand(-1, T, -1))
        assert torch.equal(q_b.scales.view(C0, T, -1), q_t.scales.unsqueeze(1).expand(-1, T, -1))
    if cfg.scale == "e4m3":
        assert host(q_b.tensor_scale)[0] == host(q_t.tensor_scale)[0]
    check_scaled_sums(host(U.ufp4_stats(big, q_b)), host(U.ufp4_stats(tile, q_t)), T)
    del big, q_b
    torch.cuda.empty_cache()
