"""Python binding of libufp4, the MI355X (gfx950) 4-bit block quantizer.

Thin marshalling over the C ABI declared in include/ufp4.h: every function
here has the C entry point's name, turns torch tensors into device pointers,
passes torch's current HIP stream, and raises on a non-zero return code.
torch supplies device memory and streams only; all computation runs in the
library's kernels.  The library must have been built (``build()`` in
__graft_entry__.py, or block_scaled_bit_ufp4_amd/build.py): importing this
package without it raises ImportError.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass, field
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libufp4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libufp4.so not built at {LIB_PATH}; run block_scaled_bit_ufp4_amd/build.py")

FORMATS = {"e2m1": 0, "e1m2": 1, "int4": 2, "if4": 3, "e2m1_max4": 4, "e2m1_max3": 5, "e2m1_max2": 6}
SCALES = {"fp32": 0, "e4m3": 1, "e8m0": 2}
RHTS = {"none": 0, "random": 1, "det": 2}
ROUNDINGS = {"rtne": 0, "sr": 1}
AXES = {"row": 0, "col": 1}
GEMM_MODES = {"mxfp4": 0, "bf16": 1}
OP_STATS, OP_QGEMM, OP_ETA, OP_AMAX = 0, 1, 2, 3
NSUMS = 48
BF16, F32 = 0, 1


class Ufp4Error(RuntimeError):
    pass


class ufp4_config(C.Structure):
    _fields_ = [("format", C.c_int32), ("scale", C.c_int32), ("block", C.c_int32), ("rht", C.c_int32),
                ("rounding", C.c_int32), ("axis", C.c_int32), ("rht_seed", C.c_uint64),
                ("sr_seed", C.c_uint64), ("sr_stream", C.c_uint32), ("reserved", C.c_uint32)]


class ufp4_qtensor(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("tensor_scale", C.c_void_p),
                ("rows", C.c_int64), ("cols", C.c_int64), ("cfg", ufp4_config)]


class ufp4_stats_report(C.Structure):
    _fields_ = [("n", C.c_double), ("sqnr_db", C.c_double), ("alpha", C.c_double), ("mse", C.c_double),
                ("mean_err", C.c_double), ("mean_shrink", C.c_double), ("int4_share", C.c_double),
                ("counts", (C.c_double * 8) * 2), ("bucket_bias", (C.c_double * 8) * 2)]


_lib = C.CDLL(LIB_PATH)
_p, _i64, _u64, _i32, _sz = C.c_void_p, C.c_int64, C.c_uint64, C.c_int, C.c_size_t
_lib.ufp4_rht.argtypes = [_p, _i32, _i64, _i64, _i64, _i32, _i32, _u64, _p, _i32, _i64, _p]
_lib.ufp4_amax.argtypes = [_p, _i32, _i64, _i64, _i64, C.POINTER(ufp4_config), _p, _p, _sz, _p]
_lib.ufp4_amax_noalloc.argtypes = [_p, _i32, _i64, _i64, _i64, C.POINTER(ufp4_config), _p, _p]
_lib.ufp4_quantize.argtypes = [_p, _i32, _i64, _i64, _i64, C.POINTER(ufp4_config), _p, C.POINTER(ufp4_qtensor), _p]
_lib.ufp4_dequantize.argtypes = [C.POINTER(ufp4_qtensor), _i32, _p, _i32, _i64, _p]
_lib.ufp4_stats.argtypes = [_p, _i32, _i64, C.POINTER(ufp4_qtensor), _p, _p, _sz, _p]
_lib.ufp4_stats_finalize.argtypes = [_p, C.POINTER(ufp4_stats_report)]
_lib.ufp4_stats_finalize.restype = None
_lib.ufp4_qgemm.argtypes = [C.POINTER(ufp4_qtensor), C.POINTER(ufp4_qtensor), _i32, _p, _i64, _p, _sz, _p]
_lib.ufp4_gemm_bf16.argtypes = [_p, _p, _i64, _i64, _i64, _i64, _i64, _p, _i64, _p]
_lib.ufp4_eta.argtypes = [_p, _p, _i64, _i64, _i64, _p, _p, _sz, _p]
_lib.ufp4_workspace_size.argtypes = [_i32, _i64, _i64, C.POINTER(ufp4_config)]
_lib.ufp4_workspace_size.restype = _sz
_lib.ufp4_strerror.argtypes = [_i32]
_lib.ufp4_strerror.restype = C.c_char_p
_lib.ufp4_last_hip_error.restype = _i32
_lib.ufp4_version.restype = _i32
_lib.ufp4_time_next_launch.argtypes = [_p, _p]
_lib.ufp4_kv_cache_bytes.argtypes = [_i64, _i64, _i64, _i64, _i32]
_lib.ufp4_kv_cache_bytes.restype = _sz
_lib.ufp4_kv_cache_quantize.argtypes = [_p, _p, _i64, _i64, _i64, _i64, _i32, _i64, _i64, _i64, _p, _i32, _p, _p]
_lib.ufp4_kv_q_quantize.argtypes = [_p, _i64, _i64, _i32, _p, _p, _p]
_lib.ufp4_kv_decode_workspace_size.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64]
_lib.ufp4_kv_decode_workspace_size.restype = _sz
_lib.ufp4_kv_decode.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i64, C.c_float, _i32, _i64, _p, _p, _sz,
                                _p]

EXPORTS = ["ufp4_rht", "ufp4_amax", "ufp4_amax_noalloc", "ufp4_quantize", "ufp4_dequantize", "ufp4_stats", "ufp4_stats_finalize",
           "ufp4_qgemm", "ufp4_gemm_bf16", "ufp4_eta", "ufp4_workspace_size", "ufp4_strerror",
           "ufp4_last_hip_error", "ufp4_version", "ufp4_time_next_launch", "ufp4_kv_cache_bytes",
           "ufp4_kv_cache_quantize", "ufp4_kv_q_quantize", "ufp4_kv_decode_workspace_size", "ufp4_kv_decode"]


def lib():
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = _lib.ufp4_strerror(rc).decode()
        if rc == -6:
            msg += f" (hipError {_lib.ufp4_last_hip_error()})"
        raise Ufp4Error(f"{what}: {msg} [{rc}]")


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported element type {t.dtype}")


def _ld(t: torch.Tensor) -> int:
    if t.dim() == 2 and t.numel() == 0:
        return max(8, (t.shape[1] + 7) // 8 * 8)
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


@dataclass(frozen=True)
class Cfg:
    """Quantizer options in words; .c() gives the ABI struct."""
    format: str = "e2m1"
    scale: str = "fp32"
    block: int = 16
    rht: str = "none"
    rounding: str = "rtne"
    axis: str = "row"
    rht_seed: int = 0
    sr_seed: int = 0
    sr_stream: int = 0

    def c(self) -> ufp4_config:
        return ufp4_config(FORMATS[self.format], SCALES[self.scale], self.block, RHTS[self.rht],
                           ROUNDINGS[self.rounding], AXES[self.axis], self.rht_seed, self.sr_seed,
                           self.sr_stream, 0)

    def view_shape(self, rows: int, cols: int):
        return (rows, cols) if self.axis == "row" else (cols, rows)


@dataclass
class QTensor:
    """Device buffers of one quantization (view layout, see ufp4.h)."""
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: Optional[torch.Tensor]
    rows: int
    cols: int
    cfg: Cfg
    _keep: list = field(default_factory=list, repr=False)

    def c(self) -> ufp4_qtensor:
        return ufp4_qtensor(self.codes.data_ptr(), self.scales.data_ptr(),
                            self.tensor_scale.data_ptr() if self.tensor_scale is not None else None,
                            self.rows, self.cols, self.cfg.c())


def alloc_qtensor(rows: int, cols: int, cfg: Cfg, device="cuda") -> QTensor:
    V, L = cfg.view_shape(rows, cols)
    codes = torch.empty((V, L // 2), dtype=torch.uint8, device=device)
    if cfg.scale == "fp32":
        scales = torch.empty((V, L // cfg.block), dtype=torch.float32, device=device)
    else:
        scales = torch.empty((V, L // cfg.block), dtype=torch.uint8, device=device)
    ts = torch.zeros(1, dtype=torch.float32, device=device) if cfg.scale == "e4m3" else None
    return QTensor(codes, scales, ts, rows, cols, cfg)


# ---- the C entry points ---------------------------------------------------------

def ufp4_rht(x: torch.Tensor, axis: str = "row", rht: str = "random", seed: int = 0,
             out_dtype=torch.float32, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    R, Cc = x.shape
    V, L = (R, Cc) if axis == "row" else (Cc, R)
    if y is None:
        y = torch.empty((V, L), dtype=out_dtype, device=x.device)
    rc = _lib.ufp4_rht(x.data_ptr(), _dtype_code(x), R, Cc, _ld(x), AXES[axis], RHTS[rht], seed, y.data_ptr(),
                       _dtype_code(y), _ld(y), _stream(stream))
    _check(rc, "ufp4_rht")
    return y


def ufp4_amax(x: torch.Tensor, cfg: Cfg, out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    if ws is None:
        ws = torch.empty(ufp4_workspace_size(OP_AMAX, x.shape[0], x.shape[1], cfg), dtype=torch.uint8,
                         device=x.device)
    c = cfg.c()
    rc = _lib.ufp4_amax(x.data_ptr(), _dtype_code(x), x.shape[0], x.shape[1], _ld(x), C.byref(c), out.data_ptr(),
                        ws.data_ptr(), ws.numel(), _stream(stream))
    _check(rc, "ufp4_amax")
    return out


def ufp4_amax_noalloc(x: torch.Tensor, cfg: Cfg, out: torch.Tensor, stream=None) -> torch.Tensor:
    """ufp4_amax with the library's built-in scratch instead of a workspace
    (out: a device float the caller allocated)."""
    c = cfg.c()
    rc = _lib.ufp4_amax_noalloc(x.data_ptr(), _dtype_code(x), x.shape[0], x.shape[1], _ld(x), C.byref(c),
                                out.data_ptr(), _stream(stream))
    _check(rc, "ufp4_amax_noalloc")
    return out


def ufp4_quantize(x: torch.Tensor, cfg: Cfg, amax: Optional[torch.Tensor] = None, out: Optional[QTensor] = None,
                  stream=None) -> QTensor:
    """Quantize x.  For E4M3 scales pass amax (from ufp4_amax), or it is
    computed here first."""
    R, Cc = x.shape
    if out is None:
        out = alloc_qtensor(R, Cc, cfg, x.device)
    if cfg.scale == "e4m3" and amax is None:
        amax = ufp4_amax(x, cfg, stream=stream)
    c = cfg.c()
    q = out.c()
    rc = _lib.ufp4_quantize(x.data_ptr(), _dtype_code(x), R, Cc, _ld(x), C.byref(c),
                            amax.data_ptr() if amax is not None else None, C.byref(q), _stream(stream))
    _check(rc, "ufp4_quantize")
    out.rows, out.cols, out.cfg = R, Cc, cfg
    return out


def ufp4_dequantize(q: QTensor, inverse_rht: bool = False, dtype=torch.float32, y: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    V, L = q.cfg.view_shape(q.rows, q.cols)
    if y is None:
        y = torch.empty((V, L), dtype=dtype, device=q.codes.device)
    qc = q.c()
    rc = _lib.ufp4_dequantize(C.byref(qc), int(inverse_rht), y.data_ptr(), _dtype_code(y), _ld(y), _stream(stream))
    _check(rc, "ufp4_dequantize")
    return y


def ufp4_workspace_size(op: int, rows: int, cols: int, cfg: Optional[Cfg] = None) -> int:
    c = cfg.c() if cfg is not None else None
    return int(_lib.ufp4_workspace_size(op, rows, cols, C.byref(c) if c is not None else None))


def ufp4_stats(x: torch.Tensor, q: QTensor, sums: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    if sums is None:
        sums = torch.empty(NSUMS, dtype=torch.float64, device=x.device)
    need = ufp4_workspace_size(OP_STATS, q.rows, q.cols, q.cfg)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    qc = q.c()
    rc = _lib.ufp4_stats(x.data_ptr(), _dtype_code(x), _ld(x), C.byref(qc), sums.data_ptr(), ws.data_ptr(),
                         ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "ufp4_stats")
    return sums


def ufp4_stats_finalize(sums) -> dict:
    import numpy as np
    s = np.ascontiguousarray(sums.detach().cpu().numpy() if isinstance(sums, torch.Tensor) else sums,
                             dtype=np.float64)
    r = ufp4_stats_report()
    _lib.ufp4_stats_finalize(s.ctypes.data_as(C.c_void_p), C.byref(r))
    return {"n": r.n, "sqnr_db": r.sqnr_db, "alpha": r.alpha, "mse": r.mse, "mean_err": r.mean_err,
            "mean_shrink": r.mean_shrink, "int4_share": r.int4_share,
            "counts": np.array([[r.counts[t][k] for k in range(8)] for t in range(2)]),
            "bucket_bias": np.array([[r.bucket_bias[t][k] for k in range(8)] for t in range(2)])}


def ufp4_qgemm(a: QTensor, b: QTensor, mode: str = "mxfp4", c: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    M, K = a.cfg.view_shape(a.rows, a.cols)
    N = b.cfg.view_shape(b.rows, b.cols)[0]
    if c is None:
        c = torch.empty((M, N), dtype=torch.float32, device=a.codes.device)
    need = ufp4_workspace_size(OP_QGEMM, M + N, K, a.cfg) if mode == "bf16" else 0
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=a.codes.device)
    ac, bc = a.c(), b.c()
    rc = _lib.ufp4_qgemm(C.byref(ac), C.byref(bc), GEMM_MODES[mode], c.data_ptr(), _ld(c),
                         ws.data_ptr() if ws is not None else None,
                         ws.numel() if ws is not None else 0, _stream(stream))
    _check(rc, "ufp4_qgemm")
    return c


def ufp4_gemm_bf16(a: torch.Tensor, b: torch.Tensor, c: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    M, K = a.shape
    N = b.shape[0]
    if c is None:
        c = torch.empty((M, N), dtype=torch.float32, device=a.device)
    rc = _lib.ufp4_gemm_bf16(a.data_ptr(), b.data_ptr(), M, N, K, _ld(a), _ld(b), c.data_ptr(), _ld(c),
                             _stream(stream))
    _check(rc, "ufp4_gemm_bf16")
    return c


def ufp4_eta(zq: torch.Tensor, z: torch.Tensor, sums: Optional[torch.Tensor] = None,
             ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    M, N = z.shape
    if sums is None:
        sums = torch.empty(3, dtype=torch.float64, device=z.device)
    need = ufp4_workspace_size(OP_ETA, M, N)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=z.device)
    rc = _lib.ufp4_eta(zq.data_ptr(), z.data_ptr(), M, N, _ld(z), sums.data_ptr(), ws.data_ptr(), ws.numel(),
                       _stream(stream))
    _check(rc, "ufp4_eta")
    return sums


def ufp4_strerror(code: int) -> str:
    return _lib.ufp4_strerror(code).decode()


def ufp4_last_hip_error() -> int:
    return int(_lib.ufp4_last_hip_error())


def ufp4_version() -> int:
    return int(_lib.ufp4_version())


def ufp4_time_next_launch(start=None, stop=None) -> None:
    """Make the next kernel the library launches from this thread timestamp
    its own dispatch on two torch.cuda.Event objects (created with
    enable_timing=True); start.elapsed_time(stop) is then that kernel's
    duration.  No arguments clears a pending request."""
    handles = []
    for e in (start, stop):
        if e is None:
            handles.append(None)
            continue
        if not e.cuda_event:
            e.record()  # torch creates the underlying event lazily
        handles.append(e.cuda_event)
    _check(_lib.ufp4_time_next_launch(handles[0], handles[1]), "ufp4_time_next_launch")


# ---- FP4 KV cache and decode attention -------------------------------------

KV_PAGE_TOKENS = 128
KV_FORMATS = {"fp4": 0, "fp8": 1}
KV_PAGE_BYTES = {"fp4": 17408, "fp8": 33792}


def ufp4_kv_cache_bytes(B: int, Hkv: int, L_cap: int, D: int = 128, fmt: str = "fp4") -> int:
    return int(_lib.ufp4_kv_cache_bytes(B, Hkv, L_cap, D, KV_FORMATS[fmt]))


def ufp4_kv_cache_quantize(k: torch.Tensor, v: torch.Tensor, lens: torch.Tensor, rotate: bool = True,
                           cache: Optional[torch.Tensor] = None, stream=None, fmt: str = "fp4") -> torch.Tensor:
    """k, v: bf16 [B][Hkv][L_cap][128] views with unit channel stride (any
    batch/head/token strides); lens: int32 [B] on the device; fmt "fp4" or
    the "fp8" baseline.  Returns the uint8 cache (ufp4_kv_cache_bytes)."""
    B, Hkv, L_cap, D = k.shape
    if v.shape != k.shape or v.stride() != k.stride() or k.stride(3) != 1:
        raise ValueError("k and v must have the same shape and strides, channels contiguous")
    if cache is None:
        cache = torch.empty(max(1, ufp4_kv_cache_bytes(B, Hkv, L_cap, D, fmt)), dtype=torch.uint8, device=k.device)
    rc = _lib.ufp4_kv_cache_quantize(k.data_ptr(), v.data_ptr(), B, Hkv, L_cap, D, KV_FORMATS[fmt], k.stride(0),
                                     k.stride(1), k.stride(2), lens.data_ptr(), int(rotate), cache.data_ptr(),
                                     _stream(stream))
    _check(rc, "ufp4_kv_cache_quantize")
    return cache


def ufp4_kv_q_quantize(q: torch.Tensor, rotate: bool = True, stream=None):
    """q: bf16 [..., 128] contiguous -> (E4M3 codes uint8 [..., 128], exponents uint8 [..., 4])."""
    D = q.shape[-1]
    rows = q.numel() // D
    codes = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    scales = torch.empty(q.shape[:-1] + (D // 32,), dtype=torch.uint8, device=q.device)
    rc = _lib.ufp4_kv_q_quantize(q.data_ptr(), rows, D, int(rotate), codes.data_ptr(), scales.data_ptr(),
                                 _stream(stream))
    _check(rc, "ufp4_kv_q_quantize")
    return codes, scales


def ufp4_kv_decode_workspace_size(B: int, Hq: int, Hkv: int, L_cap: int, pages_per_split: int = 0,
                                  D: int = 128) -> int:
    return int(_lib.ufp4_kv_decode_workspace_size(B, Hq, Hkv, D, L_cap, pages_per_split))


def ufp4_kv_decode(q: torch.Tensor, cache: torch.Tensor, lens: torch.Tensor, Hkv: int, L_cap: int,
                   sm_scale: float, rotate: bool = True, pages_per_split: int = 0,
                   out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None,
                   fmt: str = "fp4") -> torch.Tensor:
    """One decode step: q bf16 [B][Hq][128] contiguous -> fp32 [B][Hq][128],
    against a cache of format fmt ("fp4", or the "fp8" baseline)."""
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    need = ufp4_kv_decode_workspace_size(B, Hq, Hkv, L_cap, pages_per_split, D)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    rc = _lib.ufp4_kv_decode(q.data_ptr(), cache.data_ptr(), lens.data_ptr(), B, Hq, Hkv, D, KV_FORMATS[fmt], L_cap,
                             float(sm_scale), int(rotate), pages_per_split, out.data_ptr(),
                             ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
                             _stream(stream))
    _check(rc, "ufp4_kv_decode")
    return out

