"""Seeded synthetic inputs shaped like the pages' workloads.

This module serves both the CPU oracle checks and the GPU library checks, and
holds none of the quantizer's arithmetic: it only draws random numbers and
stores them as bfloat16 bit patterns (uint16).

Recipe (all tensors row-major):
  * random numbers from numpy's PCG64 ``default_rng([seed, tensor_id])``,
    drawn in float64 in row chunks of ``CHUNK`` elements, cast to float32,
    then to bfloat16 by round-to-nearest-even on the float32 bit pattern;
  * ``quantize_x``      256x1024  N(0,1), round(0.001 n) positions (drawn
                        without replacement) replaced by N(0,1)*50;
  * ``activations_t3``  8192x8192 Student-t(3) * 0.02 (heavy tails);
  * ``llama_x``         16384x4096 Student-t(4), 8 seeded columns * 40;
  * ``llama_w``         14336x4096 N(0, 0.02);
  * ``llama_dy``        16384x14336 N(0, 1e-3);
  * ``mx_if4``          16384x8192 N(0,1) with round(0.005 n / 32) aligned
                        1x32 row blocks replaced by U(-1,1);
  * ``gemm_a``/``gemm_b`` 8192x8192 N(0,1), independent streams;
  * ``kv_decode``       one decode step of attention: q [B][Hq][D] N(0,1);
                        k, v [B][Hkv][L][D], one stream per (batch entry,
                        KV head); k N(0,1) with 4 seeded channels per KV head
                        scaled by 10 (the channel outliers of keys), v N(0,1);
  * ``kv_peaked_q``     queries aimed at a few seeded tokens of their KV
                        head (the sum of 4 key rows, scaled to length
                        sqrt(D)), so the attention is peaked instead of
                        near-uniform;
  * ``kv_lens``         per-sequence lengths: all L, or ragged, uniform in
                        [1, L] with the first entry L.
Every generator takes ``rows``/``cols`` so tests can draw smaller tensors of
the same distribution.
"""
from __future__ import annotations

import hashlib

import numpy as np

CHUNK = 1 << 20

# tensor ids keep the streams of different tensors independent
TID = {"quantize_x": 1, "activations_t3": 2, "llama_x": 3, "llama_w": 4, "llama_dy": 5,
       "mx_if4": 6, "gemm_a": 7, "gemm_b": 8, "uniform": 9, "edge": 10, "kv_q": 11, "kv_k": 12,
       "kv_v": 13, "kv_lens": 14, "small_blocks": 15}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16   # no overflow for finite values
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)


def _draw(rng: np.random.Generator, n: int, fn) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    for i in range(0, n, CHUNK):
        m = min(CHUNK, n - i)
        out[i:i + m] = f32_to_bf16_bits(fn(rng, m).astype(np.float32))
    return out


def normal(rows, cols, sigma=1.0, seed=0, tensor="uniform"):
    rng = np.random.default_rng([seed, TID[tensor]])
    return _draw(rng, rows * cols, lambda g, m: g.standard_normal(m) * sigma).reshape(rows, cols)


def quantize_x(rows=256, cols=1024, seed=0):
    rng = np.random.default_rng([seed, TID["quantize_x"]])
    n = rows * cols
    x = rng.standard_normal(n)
    k = int(round(0.001 * n))
    pos = rng.choice(n, size=k, replace=False)
    x[pos] = rng.standard_normal(k) * 50.0
    return f32_to_bf16_bits(x.astype(np.float32)).reshape(rows, cols)


def activations_t3(rows=8192, cols=8192, seed=0):
    rng = np.random.default_rng([seed, TID["activations_t3"]])
    return _draw(rng, rows * cols, lambda g, m: g.standard_t(3.0, m) * 0.02).reshape(rows, cols)


def llama_x(rows=16384, cols=4096, seed=0, n_outlier_cols=8, factor=40.0):
    rng = np.random.default_rng([seed, TID["llama_x"]])
    cols_out = np.sort(rng.choice(cols, size=min(n_outlier_cols, cols), replace=False))
    gain = np.ones(cols, dtype=np.float64)
    gain[cols_out] = factor
    out = np.empty(rows * cols, dtype=np.uint16)
    rows_per = max(1, CHUNK // cols)
    for r0 in range(0, rows, rows_per):
        r1 = min(rows, r0 + rows_per)
        blk = rng.standard_t(4.0, (r1 - r0, cols)) * gain
        out[r0 * cols:r1 * cols] = f32_to_bf16_bits(blk.astype(np.float32)).ravel()
    return out.reshape(rows, cols)


def llama_w(rows=14336, cols=4096, seed=0):
    return normal(rows, cols, 0.02, seed, "llama_w")


def llama_dy(rows=16384, cols=14336, seed=0):
    return normal(rows, cols, 1e-3, seed, "llama_dy")


def mx_if4(rows=16384, cols=8192, seed=0, frac=0.005, block=32):
    rng = np.random.default_rng([seed, TID["mx_if4"]])
    n = rows * cols
    x = np.empty(n, dtype=np.uint16)
    for i in range(0, n, CHUNK):
        m = min(CHUNK, n - i)
        x[i:i + m] = f32_to_bf16_bits(rng.standard_normal(m).astype(np.float32))
    nblk = n // block
    k = int(round(frac * nblk))
    which = rng.choice(nblk, size=k, replace=False)
    u = rng.uniform(-1.0, 1.0, (k, block))
    xv = x.reshape(nblk, block)
    xv[which] = f32_to_bf16_bits(u.astype(np.float32))
    return x.reshape(rows, cols), np.sort(which)


def gemm_a(rows=8192, cols=8192, seed=0):
    return normal(rows, cols, 1.0, seed, "gemm_a")


def gemm_b(rows=8192, cols=8192, seed=0):
    return normal(rows, cols, 1.0, seed, "gemm_b")


def kv_seq(b, h, L, D=128, seed=0):
    """k, v [L][D] of batch entry b, KV head h (bf16 bits)."""
    rk = np.random.default_rng([seed, TID["kv_k"], b, h])
    k = rk.standard_normal((L, D))
    k[:, np.sort(rk.choice(D, 4, replace=False))] *= 10.0
    rv = np.random.default_rng([seed, TID["kv_v"], b, h])
    v = rv.standard_normal((L, D))
    return f32_to_bf16_bits(k.astype(np.float32)), f32_to_bf16_bits(v.astype(np.float32))


def kv_q(B, Hq, D=128, seed=0):
    rng = np.random.default_rng([seed, TID["kv_q"]])
    return f32_to_bf16_bits(rng.standard_normal((B, Hq, D)).astype(np.float32))


def kv_decode(B=32, Hq=32, Hkv=8, L=16384, D=128, seed=0):
    """q [B][Hq][D], k, v [B][Hkv][L][D] (bf16 bits)."""
    from concurrent.futures import ThreadPoolExecutor
    k = np.empty((B, Hkv, L, D), dtype=np.uint16)
    v = np.empty((B, Hkv, L, D), dtype=np.uint16)

    def fill(i):
        b, h = divmod(i, Hkv)
        k[b, h], v[b, h] = kv_seq(b, h, L, D, seed)

    with ThreadPoolExecutor(min(8, B * Hkv)) as ex:
        list(ex.map(fill, range(B * Hkv)))
    return kv_q(B, Hq, D, seed), k, v


def kv_peaked_q(k, Hq, ntop=4, gain=1.0, seed=0):
    """Queries whose attention concentrates on a few tokens: for every query
    head, the sum of ntop seeded key rows of its KV head (from k, bf16 bits
    [B][Hkv][L][D]), scaled to length gain * sqrt(D).  With the usual
    1/sqrt(D) score scale and the default gain, those tokens hold about 95 %
    of the attention over 16k tokens (about two effective tokens), as a
    retrieval-like decode step does.  Returns q [B][Hq][D] (bf16 bits)."""
    B, Hkv, L, D = k.shape
    G = Hq // Hkv
    rng = np.random.default_rng([seed, TID["kv_q"], 1])
    q = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            t = rng.choice(L, size=ntop, replace=False)
            u = bf16_bits_to_f32(k[b, h // G, t]).astype(np.float64).sum(axis=0)
            q[b, h] = u * (gain * np.sqrt(D) / np.linalg.norm(u))
    return f32_to_bf16_bits(q.astype(np.float32))


def kv_lens(B, L, seed=0, ragged=False):
    if not ragged:
        return np.full(B, L, dtype=np.int32)
    rng = np.random.default_rng([seed, TID["kv_lens"]])
    n = rng.integers(1, L + 1, B).astype(np.int32)
    n[0] = L
    return n


def edge_cases(rows=64, cols=256, seed=0):
    """bf16 bit patterns that probe the corners: exact zeros (both signs), ties
    of the scaled grid, subnormals, huge magnitudes, all-equal blocks."""
    rng = np.random.default_rng([seed, TID["edge"]])
    x = f32_to_bf16_bits(rng.standard_normal(rows * cols).astype(np.float32)).reshape(rows, cols)
    x[0, :32] = 0                                   # zero blocks
    x[0, 32:48] = 0x8000                            # negative zeros
    x[1, :16] = f32_to_bf16_bits(np.float32([6, 1, 1.5, 2, 2.5, 3, 3.5, 5, 0.25, 0.75, 1.25, 1.75,
                                             -5, -2.5, -0.25, -1.75]))
    x[1, 16:32] = f32_to_bf16_bits(np.float32([3.5] + [0.25 * i for i in range(15)]))
    x[2, :16] = rng.integers(1, 0x80, 16).astype(np.uint16)          # positive subnormals
    x[2, 16:32] = rng.integers(0x8001, 0x8080, 16).astype(np.uint16)  # negative subnormals
    x[3, :16] = f32_to_bf16_bits(np.float32(rng.standard_normal(16) * 1e37))
    x[3, 16:32] = f32_to_bf16_bits(np.full(16, 1.5, np.float32))      # all equal
    x[4, :16] = f32_to_bf16_bits(np.float32(rng.standard_normal(16) * 1e-30))
    x[4, 16:32] = f32_to_bf16_bits(np.float32(np.r_[1e-38, rng.standard_normal(15) * 1e-3]))
    x[5, :32] = f32_to_bf16_bits(np.float32(np.r_[1000.0, np.full(31, 1e-3)]))
    return x


def small_blocks(rows=256, cols=512, seed=0):
    """N(0,1) values scaled per 16-element block by 10^u, u uniform in
    [-6.5, -3.5], with x[0][0] = 1 the tensor's largest magnitude: under a
    two-level E4M3 scale most block scales land in E4M3's subnormal range."""
    rng = np.random.default_rng([seed, TID["small_blocks"]])
    x = rng.standard_normal((rows, cols))
    x = x * np.repeat(10.0 ** rng.uniform(-6.5, -3.5, (rows, cols // 16)), 16, axis=1)
    x[0, 0] = 1.0
    return f32_to_bf16_bits(x.astype(np.float32))


def digest(h: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(h).tobytes()).hexdigest()
