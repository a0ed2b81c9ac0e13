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


KV_PAGE_BYTES = {"fp4": 17408, "fp8": 33792}


def kv_unshuffle(cache: np.ndarray, B: int, Hkv: int, L_cap: int, b: int, h: int, npages: int, fmt: str = "fp4"):
    """One sequence's pages of the KV cache in natural layout: K codes
    [T][D cb], K exponents [T][4], V codes [128][T cb], V exponents
    [128][T/32] for T = 128 npages and cb = 1/2 (fp4) or 1 (fp8).  Index
    logic only, from the documented page layout (lane l, rho = l % 16,
    g = l / 16; K instruction j holds token 64(j/4) + 16(rho/4) + 4(j%4) +
    rho%4; V instruction n holds channel 8 rho + n).  FP4 lanes hold the 32
    consecutive positions 32g .. 32g+31 (channels of K, tokens of V); FP8 lanes
    hold positions 16g .. 16g+15 and 64+16g .. 64+16g+15, stored as the first
    halves of all 64 lanes, then the second halves; the exponent a lane stores
    is that of positions 32g .. 32g+31 in both."""
    fp8 = fmt == "fp8"
    PB = KV_PAGE_BYTES[fmt]
    pages = cache.reshape(B, Hkv, L_cap // 128, PB)[b, h, :npages]
    T = 128 * npages
    cb = 1 if fp8 else 2          # positions per byte
    lb = 32 if fp8 else 16        # bytes per lane and instruction
    kc = np.empty((T, 128 // cb), np.uint8)
    ks = np.empty((T, 4), np.uint8)
    vc = np.empty((128, T // cb), np.uint8)
    vs = np.empty((128, T // 32), np.uint8)
    lane = np.arange(64)
    rho, g = lane % 16, lane // 16
    if fp8:   # byte i of lane g -> position
        pos = np.where(np.arange(32) < 16, 16 * g[:, None] + np.arange(32), 64 + 16 * g[:, None] + np.arange(32) - 16)
    else:     # byte i of lane g -> byte of the natural row (two positions per byte)
        pos = 16 * g[:, None] + np.arange(16)
    ko, kso, vo, vso = (0, 16384, 16896, 33280) if fp8 else (0, 8192, 8704, 16896)
    for p in range(npages):
        pg = pages[p]
        if fp8:  # [instruction][half][lane][16 B] -> [instruction][lane][32 B]
            kcodes = pg[ko:ko + 16384].reshape(8, 2, 64, 16).transpose(0, 2, 1, 3).reshape(8, 64, 32)
            vcodes = pg[vo:vo + 16384].reshape(8, 2, 64, 16).transpose(0, 2, 1, 3).reshape(8, 64, 32)
        else:
            kcodes = pg[ko:ko + 8 * 64 * lb].reshape(8, 64, lb)
            vcodes = pg[vo:vo + 8 * 64 * lb].reshape(8, 64, lb)
        kscl = pg[kso:kso + 512].reshape(64, 8)
        vscl = pg[vso:vso + 512].reshape(64, 8)
        for j in range(8):
            tok = 128 * p + 64 * (j // 4) + 16 * (rho // 4) + 4 * (j % 4) + rho % 4
            kc[tok[:, None], pos] = kcodes[j]
            ks[tok, g] = kscl[:, j]
        for n in range(8):
            ch = 8 * rho + n
            vc[ch[:, None], (128 // cb) * p + pos] = vcodes[n]
            vs[ch, 4 * p + g] = vscl[:, n]
    return kc, ks, vc, vs
