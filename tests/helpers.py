"""Shared test helpers: move seeded inputs to the GPU, build matching oracle
and library configurations, compare results."""
import dataclasses

import numpy as np

import oracle as O


def oracle_cfg(cfg) -> "O.Cfg":
    return O.Cfg(**dataclasses.asdict(cfg))


def to_device_bf16(x_bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_device_f32(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def first_mismatch(a: np.ndarray, b: np.ndarray):
    idx = np.argwhere(a != b)
    if idx.size == 0:
        return None
    i = tuple(idx[0])
    return f"{len(idx)} mismatches; first at {i}: got {a[i]!r} want {b[i]!r}"


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    if got.dtype == np.float32:
        got = got.view(np.uint32)
        want = want.view(np.uint32)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    msg = first_mismatch(got, want)
    assert msg is None, f"{what}: {msg}"


def sample_rows(V: int, n: int, seed: int = 0) -> np.ndarray:
    """Sorted view rows to check at full size: the first, the last and a
    seeded spread in between."""
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(V, size=min(n, V), replace=False).tolist()) | {0, V - 1}
    return np.array(sorted(pick))
