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


KV_PAGE_BYTES = 17408


def kv_unshuffle(cache: np.ndarray, B: int, Hkv: int, L_cap: int, b: int, h: int, npages: int):
    """One sequence's pages of the FP4 KV cache in natural layout: K codes
    [T][64], K exponents [T][4], V codes [128][T/2], V exponents [128][T/32]
    for T = 128 npages.  Index logic only, from the documented page layout
    (lane l, rho = l % 16, g = l / 16; K instruction j holds channel group g
    of token 64(j/4) + 16(rho/4) + 4(j%4) + rho%4; V instruction n holds
    tokens 32g..32g+31 of channel 8 rho + n)."""
    pages = cache.reshape(B, Hkv, L_cap // 128, KV_PAGE_BYTES)[b, h, :npages]
    T = 128 * npages
    kc = np.empty((T, 64), np.uint8)
    ks = np.empty((T, 4), np.uint8)
    vc = np.empty((128, T // 2), np.uint8)
    vs = np.empty((128, T // 32), np.uint8)
    lane = np.arange(64)
    rho, g = lane % 16, lane // 16
    cols16 = 16 * g[:, None] + np.arange(16)
    for p in range(npages):
        pg = pages[p]
        kcodes = pg[:8192].reshape(8, 64, 16)
        kscl = pg[8192:8704].reshape(64, 8)
        vcodes = pg[8704:16896].reshape(8, 64, 16)
        vscl = pg[16896:].reshape(64, 8)
        for j in range(8):
            tok = 128 * p + 64 * (j // 4) + 16 * (rho // 4) + 4 * (j % 4) + rho % 4
            kc[tok[:, None], cols16] = kcodes[j]
            ks[tok, g] = kscl[:, j]
        for n in range(8):
            ch = 8 * rho + n
            vc[ch[:, None], (64 * p + 16 * g)[:, None] + np.arange(16)] = vcodes[n]
            vs[ch, 4 * p + g] = vscl[:, n]
    return kc, ks, vc, vs
