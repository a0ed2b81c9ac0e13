"""Python access to the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
cpu_baseline leg import this package; the HIP library never does.  Arrays are
numpy; bf16 tensors are passed as uint16 bit patterns.

The C functions cite the passages of the pages they follow.  ``orc_philox4x32_10``
is pinned against rocRAND's Philox4x32-10 engine (a library routine); every
other step is pinned by closed forms, brute force or library routines in
tests/test_oracle_*.py.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

FORMATS = {"e2m1": 0, "e1m2": 1, "int4": 2, "if4": 3, "e2m1_max4": 4, "e2m1_max3": 5, "e2m1_max2": 6}
SCALES = {"fp32": 0, "e4m3": 1, "e8m0": 2}
RHTS = {"none": 0, "random": 1, "det": 2}
ROUNDINGS = {"rtne": 0, "sr": 1}
AXES = {"row": 0, "col": 1}
NSUMS = 48


class OrcConfig(C.Structure):
    _fields_ = [("format", C.c_int32), ("scale", C.c_int32), ("block", C.c_int32), ("rht", C.c_int32),
                ("rounding", C.c_int32), ("axis", C.c_int32), ("rht_seed", C.c_uint64),
                ("sr_seed", C.c_uint64), ("sr_stream", C.c_uint32), ("reserved", C.c_uint32)]


@dataclass(frozen=True)
class Cfg:
    """A quantizer configuration in words (the same vocabulary the tests use
    for the GPU library)."""
    format: str = "e2m1"
    scale: str = "fp32"
    block: int = 16
    rht: str = "none"
    rounding: str = "rtne"
    axis: str = "row"
    rht_seed: int = 0
    sr_seed: int = 0
    sr_stream: int = 0

    def c(self) -> OrcConfig:
        return OrcConfig(FORMATS[self.format], SCALES[self.scale], self.block, RHTS[self.rht],
                         ROUNDINGS[self.rounding], AXES[self.axis], self.rht_seed, self.sr_seed,
                         self.sr_stream, 0)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(LIB_PATH)
        p, i64, u64, u32, i32 = C.c_void_p, C.c_int64, C.c_uint64, C.c_uint32, C.c_int
        L.orc_philox4x32_10.argtypes = [p, p, p]
        L.orc_sr_word.argtypes = [u64, u32, u64]
        L.orc_sr_word.restype = u32
        L.orc_rht_sign_mask.argtypes = [i32, u64]
        L.orc_rht_sign_mask.restype = u32
        L.orc_fwht16.argtypes = [p]
        L.orc_round_rtne.argtypes = [C.c_float, i32]
        L.orc_round_sr.argtypes = [C.c_float, i32, u32]
        L.orc_e4m3_encode.argtypes = [C.c_float]
        L.orc_e4m3_encode.restype = C.c_uint8
        L.orc_e4m3_decode.argtypes = [C.c_uint8]
        L.orc_e4m3_decode.restype = C.c_float
        L.orc_e8m0_exponent.argtypes = [C.c_float]
        L.orc_f32_to_bf16.argtypes = [C.c_float]
        L.orc_f32_to_bf16.restype = C.c_uint16
        L.orc_rht_view.argtypes = [p, i32, i64, i64, i64, i32, i32, u64, i64, i64, p]
        L.orc_amax.argtypes = [p, i32, i64, i64, i64, C.POINTER(OrcConfig)]
        L.orc_amax.restype = C.c_float
        L.orc_quantize.argtypes = [p, i32, i64, i64, i64, C.POINTER(OrcConfig), C.c_float, i64, i64, p, p]
        L.orc_quantize.restype = C.c_float
        L.orc_dequantize.argtypes = [C.POINTER(OrcConfig), i64, i64, p, p, C.c_float, i32, i64, i64, p]
        L.orc_stats.argtypes = [p, i32, i64, i64, i64, C.POINTER(OrcConfig), C.c_float, i64, i64, p]
        L.orc_gemm_nt_f32.argtypes = [p, p, i64, i64, i64, i64, p]
        L.orc_eta_sums.argtypes = [p, p, i64, p]
        L.orc_round_rtne_array.argtypes = [p, i64, i32, p]
        L.orc_round_sr_array.argtypes = [p, p, i64, i32, p]
        L.orc_e4m3_encode_array.argtypes = [p, i64, p]
        L.orc_f32_to_bf16_array.argtypes = [p, i64, p]
        L.orc_sr_word_array.argtypes = [u64, u32, u64, i64, p]
        L.orc_gridmax.argtypes = [i32]
        L.orc_gridmax.restype = C.c_float
        L.orc_grid_value.argtypes = [i32, i32]
        L.orc_grid_value.restype = C.c_double
        L.orc_fwht_f32.argtypes = [p, i32]
        L.orc_mx_exponent.argtypes = [C.c_double, i32]
        L.orc_mx_exponent.restype = i32
        L.orc_e4m3_encode_d.argtypes = [C.c_double]
        L.orc_e4m3_encode_d.restype = C.c_uint8
        L.orc_q_quantize.argtypes = [p, i32, i32, p, p]
        L.orc_k_quantize_row.argtypes = [p, i32, i32, i32, p, p]
        L.orc_kv_quantize_seq.argtypes = [p, p, i64, i64, i64, i32, i32, i32, p, p, p, p]
        L.orc_kv_decode_seq.argtypes = [p, i32, p, p, i64, i64, i32, C.c_float, i32, i32, p]
        L.orc_kv_decode_seq.restype = i32
        L.orc_kv_decode_bounds.argtypes = [p, i32, p, p, i64, i64, i32, C.c_float, i32, i32, C.c_double, p, p, p]
        L.orc_kv_decode_bounds.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _src(x: np.ndarray):
    if x.dtype == np.uint16:
        return 0
    if x.dtype == np.float32:
        return 1
    raise TypeError("oracle inputs are bf16 bit patterns (uint16) or float32")


# ---- scalar helpers --------------------------------------------------------

def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    o = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(o))
    return o


def sr_word(seed, stream, n):
    return int(lib().orc_sr_word(seed, stream, n))


def rht_sign_mask(kind: str, seed: int) -> int:
    return int(lib().orc_rht_sign_mask(RHTS[kind], seed))


def fwht16(v) -> np.ndarray:
    a = np.array(v, dtype=np.float32).copy()
    assert a.shape == (16,)
    lib().orc_fwht16(_ptr(a))
    return a


def round_rtne(z: float, fmt: str) -> int:
    return int(lib().orc_round_rtne(float(np.float32(z)), FORMATS[fmt]))


def round_sr(z: float, fmt: str, w: int) -> int:
    return int(lib().orc_round_sr(float(np.float32(z)), FORMATS[fmt], w))


def e4m3_encode(v: float) -> int:
    return int(lib().orc_e4m3_encode(float(np.float32(v))))


def e4m3_decode(b: int) -> float:
    return float(lib().orc_e4m3_decode(b))


def e8m0_exponent(m: float) -> int:
    return int(lib().orc_e8m0_exponent(float(np.float32(m))))


def f32_to_bf16(f: float) -> int:
    return int(lib().orc_f32_to_bf16(float(np.float32(f))))


def gridmax(fmt: str) -> float:
    return float(lib().orc_gridmax(FORMATS[fmt]))


def grid(fmt: str) -> np.ndarray:
    return np.array([lib().orc_grid_value(FORMATS[fmt], k) for k in range(8)])


# ---- tensor operations -----------------------------------------------------

def view_shape(x: np.ndarray, axis: str):
    R, Cc = x.shape
    return (R, Cc) if axis == "row" else (Cc, R)


def rht_view(x: np.ndarray, axis: str = "row", rht: str = "random", seed: int = 0, v0: int = 0, v1=None):
    x = np.ascontiguousarray(x)
    V, L = view_shape(x, axis)
    v1 = V if v1 is None else v1
    y = np.empty((v1 - v0, L), dtype=np.float32)
    rc = lib().orc_rht_view(_ptr(x), _src(x), x.shape[0], x.shape[1], x.shape[1], AXES[axis], RHTS[rht], seed,
                            v0, v1, _ptr(y))
    if rc:
        raise ValueError("bad shape")
    return y


def amax(x: np.ndarray, cfg: Cfg) -> float:
    x = np.ascontiguousarray(x)
    c = cfg.c()
    return float(np.float32(lib().orc_amax(_ptr(x), _src(x), x.shape[0], x.shape[1], x.shape[1], C.byref(c))))


@dataclass
class QResult:
    codes: np.ndarray      # uint8 [V][L/2]
    scales: np.ndarray     # float32 or uint8 [V][L/B]
    alpha: float           # tensor scale (E4M3 two-level), else 0
    amax: float


def quantize(x: np.ndarray, cfg: Cfg, v0: int = 0, v1=None, amax_value=None) -> QResult:
    """Quantize view rows [v0, v1) (all by default).  Arrays cover the whole
    view; rows outside the range stay zero."""
    x = np.ascontiguousarray(x)
    V, L = view_shape(x, cfg.axis)
    v1 = V if v1 is None else v1
    c = cfg.c()
    if cfg.scale == "e4m3" and amax_value is None:
        amax_value = amax(x, cfg)
    amax_value = 0.0 if amax_value is None else float(amax_value)
    codes = np.zeros((V, L // 2), dtype=np.uint8)
    scales = np.zeros((V, L // cfg.block), dtype=np.float32 if cfg.scale == "fp32" else np.uint8)
    alpha = lib().orc_quantize(_ptr(x), _src(x), x.shape[0], x.shape[1], x.shape[1], C.byref(c), amax_value,
                               v0, v1, _ptr(codes), _ptr(scales))
    if alpha < 0:
        raise ValueError(f"unsupported configuration {cfg}")
    return QResult(codes, scales, float(np.float32(alpha)), amax_value)


def dequantize(q: QResult, cfg: Cfg, shape, inverse: bool = False, v0: int = 0, v1=None) -> np.ndarray:
    R, Cc = shape
    V, L = (R, Cc) if cfg.axis == "row" else (Cc, R)
    v1 = V if v1 is None else v1
    out = np.empty((v1 - v0, L), dtype=np.float32)
    c = cfg.c()
    rc = lib().orc_dequantize(C.byref(c), R, Cc, _ptr(np.ascontiguousarray(q.codes)),
                              _ptr(np.ascontiguousarray(q.scales)), q.alpha, int(inverse), v0, v1, _ptr(out))
    if rc:
        raise ValueError("bad configuration")
    return out


def stats(x: np.ndarray, cfg: Cfg, v0: int = 0, v1=None, amax_value=None) -> np.ndarray:
    x = np.ascontiguousarray(x)
    V, L = view_shape(x, cfg.axis)
    v1 = V if v1 is None else v1
    if cfg.scale == "e4m3" and amax_value is None:
        amax_value = amax(x, cfg)
    sums = np.zeros(NSUMS, dtype=np.float64)
    c = cfg.c()
    rc = lib().orc_stats(_ptr(x), _src(x), x.shape[0], x.shape[1], x.shape[1], C.byref(c),
                         0.0 if amax_value is None else float(amax_value), v0, v1, _ptr(sums))
    if rc:
        raise ValueError("bad configuration")
    return sums


def gemm_nt(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Z = A B^T in binary64 (A: M x K rows to compute, B: N x K), float32 in."""
    A = np.ascontiguousarray(A, dtype=np.float32)
    B = np.ascontiguousarray(B, dtype=np.float32)
    M, K = A.shape
    N = B.shape[0]
    Z = np.empty((M, N), dtype=np.float64)
    lib().orc_gemm_nt_f32(_ptr(A), _ptr(B), N, K, 0, M, _ptr(Z))
    return Z


def eta_sums(zq: np.ndarray, z: np.ndarray) -> np.ndarray:
    """(<Zq,Z>, <Z,Z>, ||Zq-Z||^2) in binary64, summed in index order."""
    zq = np.ascontiguousarray(zq, dtype=np.float64).ravel()
    z = np.ascontiguousarray(z, dtype=np.float64).ravel()
    assert zq.size == z.size
    out = np.zeros(3, dtype=np.float64)
    lib().orc_eta_sums(_ptr(zq), _ptr(z), zq.size, _ptr(out))
    return out


def eta_report(sums) -> dict:
    """eta = <Zq,Z>/<Z,Z> and the output SQNR 10 log10(<Z,Z>/||Zq-Z||^2)."""
    s = np.asarray(sums, dtype=np.float64)
    return {"eta": s[0] / s[1] if s[1] > 0 else float("nan"),
            "sqnr_db": 10.0 * np.log10(s[1] / s[2]) if s[2] > 0 else float("inf")}


# ---- row-partitioned forms (threads) ----------------------------------------
# The rows of a quantization view are independent once the tensor amax is
# known, and the C functions run outside the interpreter lock, so whole
# full-size tensors are checked by splitting the view rows over host threads.
# Each thread writes its own rows of the shared output arrays.

def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _row_ranges(V: int, threads: int):
    threads = max(1, min(threads, V)) if V else 1
    return [(i * V // threads, (i + 1) * V // threads) for i in range(threads)]


def _run_parallel(fn, ranges):
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(len(ranges)) as ex:
        return list(ex.map(lambda r: fn(*r), ranges))


def amax_threads(x: np.ndarray, cfg: Cfg, threads: int = 0) -> float:
    """Tensor amax, the max of the amaxes of row (or column) slices."""
    x = np.ascontiguousarray(x)
    V, _ = view_shape(x, cfg.axis)
    parts = _row_ranges(V, threads or default_threads())
    if cfg.axis == "row":
        slices = [np.ascontiguousarray(x[a:b]) for a, b in parts]
    else:
        slices = [np.ascontiguousarray(x[:, a:b]) for a, b in parts]
    return float(max(_run_parallel(lambda s: amax(s, cfg), [(s,) for s in slices])))


def quantize_threads(x: np.ndarray, cfg: Cfg, amax_value=None, threads: int = 0) -> QResult:
    """quantize() of the whole view, its rows split over host threads."""
    x = np.ascontiguousarray(x)
    V, L = view_shape(x, cfg.axis)
    if cfg.scale == "e4m3" and amax_value is None:
        amax_value = amax_threads(x, cfg, threads)
    amax_value = 0.0 if amax_value is None else float(amax_value)
    c = cfg.c()
    codes = np.zeros((V, L // 2), dtype=np.uint8)
    scales = np.zeros((V, L // cfg.block), dtype=np.float32 if cfg.scale == "fp32" else np.uint8)
    alphas = _run_parallel(
        lambda v0, v1: lib().orc_quantize(_ptr(x), _src(x), x.shape[0], x.shape[1], x.shape[1], C.byref(c),
                                          amax_value, v0, v1, _ptr(codes), _ptr(scales)),
        _row_ranges(V, threads or default_threads()))
    if min(alphas) < 0:
        raise ValueError(f"unsupported configuration {cfg}")
    return QResult(codes, scales, float(np.float32(alphas[0])), amax_value)


def dequantize_threads(q: QResult, cfg: Cfg, shape, inverse: bool = False, threads: int = 0) -> np.ndarray:
    R, Cc = shape
    V, L = (R, Cc) if cfg.axis == "row" else (Cc, R)
    out = np.empty((V, L), dtype=np.float32)
    c = cfg.c()
    codes = np.ascontiguousarray(q.codes)
    scales = np.ascontiguousarray(q.scales)
    rcs = _run_parallel(
        lambda v0, v1: lib().orc_dequantize(C.byref(c), R, Cc, _ptr(codes), _ptr(scales), q.alpha, int(inverse),
                                            v0, v1, _ptr(out[v0:v1])),
        _row_ranges(V, threads or default_threads()))
    if any(rcs):
        raise ValueError("bad configuration")
    return out


def stats_threads(x: np.ndarray, cfg: Cfg, amax_value=None, threads: int = 0) -> np.ndarray:
    """stats() of the whole view: the sums of each thread's rows, added."""
    x = np.ascontiguousarray(x)
    V, _ = view_shape(x, cfg.axis)
    if cfg.scale == "e4m3" and amax_value is None:
        amax_value = amax_threads(x, cfg, threads)
    parts = _run_parallel(lambda v0, v1: stats(x, cfg, v0, v1, amax_value),
                          _row_ranges(V, threads or default_threads()))
    return np.sum(parts, axis=0)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even), returned as float32 values."""
    flat = np.ascontiguousarray(a, dtype=np.float32).ravel()
    out = np.empty(flat.size, dtype=np.uint16)
    lib().orc_f32_to_bf16_array(_ptr(flat), flat.size, _ptr(out))
    return (out.astype(np.uint32) << 16).view(np.float32).reshape(a.shape)


def round_rtne_array(z: np.ndarray, fmt: str) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.float32).ravel()
    out = np.empty(z.size, dtype=np.uint8)
    lib().orc_round_rtne_array(_ptr(z), z.size, FORMATS[fmt], _ptr(out))
    return out


def round_sr_array(z: np.ndarray, w: np.ndarray, fmt: str) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.float32).ravel()
    w = np.ascontiguousarray(w, dtype=np.uint32).ravel()
    out = np.empty(z.size, dtype=np.uint8)
    lib().orc_round_sr_array(_ptr(z), _ptr(w), z.size, FORMATS[fmt], _ptr(out))
    return out


def e4m3_encode_array(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    lib().orc_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def sr_words(seed: int, stream: int, n0: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    lib().orc_sr_word_array(seed, stream, n0, n, _ptr(out))
    return out


def finalize(s: np.ndarray) -> dict:
    """Report derived from the sums (SQNR, alpha, mean errors, per-bucket
    bias, INT4 share), binary64."""
    n = s[0]
    rep = {
        "n": n,
        "sqnr_db": 10.0 * np.log10(s[1] / s[2]) if s[2] > 0 else float("inf"),
        "alpha": s[5] / s[1] if s[1] > 0 else float("nan"),
        "mean_err": s[3] / n if n else 0.0,
        "mean_shrink": s[4] / n if n else 0.0,
        "mse": s[2] / n if n else 0.0,
        "int4_share": s[8] / s[7] if s[7] else 0.0,
        "counts": s[16:32].reshape(2, 8).copy(),
        "bucket_bias": np.divide(s[32:48], s[16:32], out=np.full(16, np.nan), where=s[16:32] > 0).reshape(2, 8),
    }
    return rep


# ---- FP4 KV-cache decode attention (kvcache.c) ----------------------------

def fwht(v) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform (binary32 butterflies)."""
    a = np.array(v, dtype=np.float32).copy()
    lib().orc_fwht_f32(_ptr(a), a.size)
    return a


def mx_exponent(amax: float, emax: int) -> int:
    return int(lib().orc_mx_exponent(float(amax), emax))


def e4m3_encode_d(a: float) -> int:
    return int(lib().orc_e4m3_encode_d(float(a)))


def q_quantize(q: np.ndarray, rotate: bool):
    """MXFP8 of query rows q[..., D] (bf16 bits): (E4M3 bytes [..., D],
    biased exponents [..., D/32])."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    D = q.shape[-1]
    rows = q.reshape(-1, D)
    codes = np.empty(rows.shape, dtype=np.uint8)
    scales = np.empty((rows.shape[0], D // 32), dtype=np.uint8)
    for i in range(rows.shape[0]):
        r = np.ascontiguousarray(rows[i])
        lib().orc_q_quantize(_ptr(r), D, int(rotate), _ptr(codes[i]), _ptr(scales[i]))
    return codes.reshape(q.shape), scales.reshape(q.shape[:-1] + (D // 32,))


KV_FORMATS = {"fp4": 0, "fp8": 1}


def kv_quantize_seq(k: np.ndarray, v: np.ndarray, length: int, ntok: int, rotate: bool, fmt: str = "fp4"):
    """The KV cache of one sequence, natural layout: k, v bf16 bits [T][D]
    (T >= length).  Returns kcodes [ntok][D cb], kscales [ntok][D/32],
    vcodes [D][ntok cb], vscales [D][ntok/32] with cb = 1/2 (fp4) or 1 (fp8)."""
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    assert k.shape == v.shape and ntok % 32 == 0 and ntok >= length
    D = k.shape[1]
    fp8 = KV_FORMATS[fmt]
    cb = 1 if fp8 else 2
    kc = np.empty((ntok, D // cb), dtype=np.uint8)
    ks = np.empty((ntok, D // 32), dtype=np.uint8)
    vc = np.empty((D, ntok // cb), dtype=np.uint8)
    vs = np.empty((D, ntok // 32), dtype=np.uint8)
    lib().orc_kv_quantize_seq(_ptr(k), _ptr(v), D, int(length), int(ntok), D, int(rotate), fp8,
                              _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs))
    return kc, ks, vc, vs


def kv_decode_seq(q: np.ndarray, k: np.ndarray, v: np.ndarray, length: int, sm_scale: float,
                  rotate: bool, fmt: str = "fp4") -> np.ndarray:
    """Decode attention of one sequence: q bf16 bits [G][D], k, v [T][D]
    (T >= length); binary64 output [G][D]."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    G, D = q.shape
    out = np.empty((G, D), dtype=np.float64)
    rc = lib().orc_kv_decode_seq(_ptr(q), G, _ptr(k), _ptr(v), D, int(length), D, float(sm_scale), int(rotate),
                                 KV_FORMATS[fmt], _ptr(out))
    if rc:
        raise ValueError("bad decode shape" if rc == -1 else "out of memory")
    return out


def kv_decode_bounds(q: np.ndarray, k: np.ndarray, v: np.ndarray, length: int, sm_scale: float, rotate: bool,
                     eps_s: float = 2.0 ** -15, fmt: str = "fp4"):
    """(mass [G][D], ambiguity bound [G][D], number of fragile tokens) for
    comparing a binary32 decode with kv_decode_seq."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    G, D = q.shape
    mass = np.empty((G, D), dtype=np.float64)
    amb = np.empty((G, D), dtype=np.float64)
    frag = C.c_int64(0)
    rc = lib().orc_kv_decode_bounds(_ptr(q), G, _ptr(k), _ptr(v), D, int(length), D, float(sm_scale), int(rotate),
                                    KV_FORMATS[fmt], float(eps_s), _ptr(mass), _ptr(amb), C.byref(frag))
    if rc:
        raise ValueError("bad decode shape" if rc == -1 else "out of memory")
    return mass, amb, int(frag.value)
