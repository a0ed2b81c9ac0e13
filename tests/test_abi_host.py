"""The C-ABI library loads without a GPU, exports every declared entry point,
and rejects bad arguments on the host before any HIP call (CPU only)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import block_scaled_bit_ufp4_amd as U
import oracle as O

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ufp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ufp4_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 12
    lib = C.CDLL(U.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(U.EXPORTS)


def test_strerror_and_version():
    assert U.ufp4_strerror(0) == "ok"
    for code in range(-6, 0):
        assert U.ufp4_strerror(code) and U.ufp4_strerror(code) != "unknown error code"
    assert U.ufp4_strerror(-99) == "unknown error code"
    assert U.ufp4_version() >= 1
    assert U.ufp4_last_hip_error() == 0


FAKE = 0x10000  # aligned non-null address; never dereferenced on these paths


def quant(cfg, rows, cols, ld, x=FAKE, codes=FAKE, scales=FAKE, ts=FAKE, amax=FAKE):
    c = cfg.c()
    q = U.ufp4_qtensor(codes, scales, ts, 0, 0, U.ufp4_config())
    return U.lib().ufp4_quantize(x, 0, rows, cols, ld, C.byref(c), amax, C.byref(q), None)


@pytest.mark.parametrize("cfg,rows,cols,ld,code", [
    (U.Cfg("e2m1"), 16, 24, 24, -2),                       # row length not a multiple of 16
    (U.Cfg("e2m1", "e8m0", 32), 16, 48, 48, -2),           # not a multiple of 32
    (U.Cfg("e2m1", axis="col"), 24, 16, 16, -2),           # column axis: rows multiple of 16
    (U.Cfg("e2m1", axis="col"), 32, 12, 16, -2),           # column axis: cols multiple of 8
    (U.Cfg("e2m1"), 16, 32, 16, -2),                       # ld < cols
    (U.Cfg("e2m1"), 16, 32, 36, -3),                       # ld not a multiple of 8
    (U.Cfg("e1m2", "e8m0", 32), 16, 32, 32, -4),           # E8M0 only with E2M1
    (U.Cfg("if4", "fp32"), 16, 32, 32, -4),                # IF4 needs the E4M3 scale
    (U.Cfg("if4", "e4m3", rounding="sr"), 16, 32, 32, -4), # SR with IF4 not on the pages
    (U.Cfg("e2m1", "e8m0", 32, rounding="sr"), 16, 32, 32, -4),
    (U.Cfg("e2m1", "fp32", 32), 16, 32, 32, -4),           # FP32 scale uses 16-blocks
    (U.Cfg("e2m1", block=8), 16, 32, 32, -1),
    (U.Cfg("e2m1_max2", rounding="sr"), 16, 32, 32, -4),   # capped E2M1: RTNE only
    (U.Cfg("e2m1_max4", "e8m0", 32), 16, 32, 32, -4),      # capped E2M1: no E8M0
])
def test_quantize_validation(cfg, rows, cols, ld, code):
    assert quant(cfg, rows, cols, ld) == code


def test_quantize_null_and_alignment():
    cfg = U.Cfg("e2m1")
    assert quant(cfg, 16, 32, 32, x=0) == -1
    assert quant(cfg, 16, 32, 32, codes=0) == -1
    assert quant(cfg, 16, 32, 32, x=FAKE + 2) == -3
    assert quant(U.Cfg("e2m1", "e4m3"), 16, 32, 32, amax=0) == -1
    assert quant(U.Cfg("e2m1", "e4m3"), 16, 32, 32, ts=0) == -1
    bad = U.Cfg("e2m1").c()
    bad.reserved = 1
    q = U.ufp4_qtensor(FAKE, FAKE, FAKE, 0, 0, U.ufp4_config())
    assert U.lib().ufp4_quantize(FAKE, 0, 16, 32, 32, C.byref(bad), FAKE, C.byref(q), None) == -1
    bad = U.Cfg("e2m1").c()
    bad.format = 9
    assert U.lib().ufp4_quantize(FAKE, 0, 16, 32, 32, C.byref(bad), FAKE, C.byref(q), None) == -1


def test_other_calls_validate():
    L = U.lib()
    assert L.ufp4_rht(FAKE, 0, 16, 24, 24, 0, 1, 0, FAKE, 1, 24, None) == -2
    assert L.ufp4_rht(FAKE, 0, 16, 32, 32, 0, 1, 0, FAKE, 1, 16, None) == -2
    assert L.ufp4_rht(FAKE, 0, 16, 32, 32, 0, 7, 0, FAKE, 1, 32, None) == -1
    cfg = U.Cfg("e2m1").c()
    assert L.ufp4_amax(FAKE, 0, 16, 32, 32, C.byref(cfg), None, FAKE, 64, None) == -1
    assert L.ufp4_amax(FAKE, 0, 16, 32, 32, C.byref(cfg), FAKE, None, 0, None) == -5
    q = U.ufp4_qtensor(FAKE, FAKE, None, 16, 24, U.Cfg("e2m1").c())
    assert L.ufp4_dequantize(C.byref(q), 0, FAKE, 1, 24, None) == -2
    q = U.ufp4_qtensor(FAKE, FAKE, None, 16, 32, U.Cfg("e2m1").c())
    assert L.ufp4_stats(FAKE, 0, 32, C.byref(q), FAKE, None, 0, None) == -5
    a = U.ufp4_qtensor(FAKE, FAKE, None, 256, 128, U.Cfg("e2m1", "e8m0", 32).c())
    b = U.ufp4_qtensor(FAKE, FAKE, None, 256, 256, U.Cfg("e2m1", "e8m0", 32).c())
    assert L.ufp4_qgemm(C.byref(a), C.byref(b), 0, FAKE, 256, None, 0, None) == -2     # K differs
    b = U.ufp4_qtensor(FAKE, FAKE, None, 200, 128, U.Cfg("e2m1", "e8m0", 32).c())
    assert L.ufp4_qgemm(C.byref(a), C.byref(b), 0, FAKE, 256, None, 0, None) == -2     # N not a multiple of 256
    b = U.ufp4_qtensor(FAKE, FAKE, None, 256, 128, U.Cfg("e1m2").c())
    assert L.ufp4_qgemm(C.byref(a), C.byref(b), 0, FAKE, 256, None, 0, None) == -4     # native path needs MXFP4
    b = U.ufp4_qtensor(FAKE, FAKE, None, 256, 128, U.Cfg("e2m1", "e8m0", 32, rht="random", rht_seed=3).c())
    assert L.ufp4_qgemm(C.byref(a), C.byref(b), 0, FAKE, 256, None, 0, None) == -4     # different transforms
    a2 = U.ufp4_qtensor(FAKE, FAKE, None, 256, 128, U.Cfg("e1m2").c())
    b2 = U.ufp4_qtensor(FAKE, FAKE, None, 256, 128, U.Cfg("e1m2").c())
    assert L.ufp4_qgemm(C.byref(a2), C.byref(b2), 1, FAKE, 256, None, 0, None) == -5   # workspace
    assert L.ufp4_gemm_bf16(FAKE, FAKE, 256, 256, 48, 48, 48, FAKE, 256, None) == -2
    assert L.ufp4_eta(FAKE, FAKE, 4, 6, 6, FAKE, FAKE, 1 << 20, None) == -2
    assert L.ufp4_eta(FAKE, FAKE, 4, 8, 8, FAKE, FAKE, 16, None) == -5


def test_empty_inputs_are_no_ops():
    cfg = U.Cfg("e2m1")
    assert quant(cfg, 0, 32, 32) == 0


def test_workspace_sizes():
    assert U.ufp4_workspace_size(U.OP_STATS, 100, 64) == 2048 * 48 * 8      # one row of 48 sums per workgroup
    assert U.ufp4_workspace_size(U.OP_ETA, 100, 64) == 1024 * 3 * 8
    assert U.ufp4_workspace_size(U.OP_AMAX, 8192, 8192, U.Cfg()) == 4096 * 4      # one per 1024 chunks
    assert U.ufp4_workspace_size(U.OP_AMAX, 16384, 4096, U.Cfg(axis="col")) == 64 * 32 * 4
    assert U.ufp4_workspace_size(U.OP_QGEMM, 512, 256, U.Cfg("e1m2")) == 512 * 256 * 2
    # the dequantize-to-bf16 mode needs the same for MXFP4 operands
    assert U.ufp4_workspace_size(U.OP_QGEMM, 512, 256, U.Cfg("e2m1", "e8m0", 32)) == 512 * 256 * 2
    assert U.ufp4_workspace_size(U.OP_QGEMM, 512, 256, None) == 512 * 256 * 2


def test_gemm_rejects_row_offsets_past_32_bits():
    """The GEMM kernels address 256 operand rows with 32-bit buffer offsets;
    a row stride that makes them wrap is refused before any launch."""
    L = U.lib()
    big = (1 << 32) // 512 + 8          # bf16 elements: 256 rows x 2 B span > 4 GiB
    assert L.ufp4_gemm_bf16(FAKE, FAKE, 256, 256, 64, big - big % 8, 64, FAKE, 256, None) == -2
    assert L.ufp4_gemm_bf16(FAKE, FAKE, 256, 256, 64, 64, big - big % 8, FAKE, 256, None) == -2



def test_stats_finalize_matches_oracle_report():
    rng = np.random.default_rng(0)
    s = rng.uniform(1, 100, 48)
    s[0], s[7], s[8] = 4096, 256, 64
    s[16:32] = rng.integers(0, 300, 16)
    s[20] = 0
    a = U.ufp4_stats_finalize(s)
    b = O.finalize(s)
    for k in ("sqnr_db", "alpha", "mse", "mean_err", "mean_shrink", "int4_share"):
        assert a[k] == pytest.approx(b[k], rel=1e-15), k
    np.testing.assert_array_equal(a["counts"], b["counts"])
    np.testing.assert_allclose(a["bucket_bias"], b["bucket_bias"], rtol=1e-15)
    assert np.isnan(a["bucket_bias"][0, 4])


def test_time_next_launch_needs_both_events_or_none():
    import ctypes
    import block_scaled_bit_ufp4_amd as U
    lib = U.lib()
    fake = ctypes.c_void_p(0x1000)
    assert lib.ufp4_time_next_launch(fake, None) == -1
    assert lib.ufp4_time_next_launch(None, fake) == -1
    assert lib.ufp4_time_next_launch(None, None) == 0   # clears; launches nothing


def test_kv_calls_validate():
    L = U.lib()
    assert U.ufp4_kv_cache_bytes(2, 2, 256) == 2 * 2 * 2 * 17408
    assert U.ufp4_kv_cache_bytes(2, 2, 256, fmt="fp8") == 2 * 2 * 2 * 33792
    assert U.ufp4_kv_cache_bytes(2, 2, 100) == 0                       # capacity not a multiple of 128
    assert U.ufp4_kv_cache_bytes(2, 2, 256, 64) == 0                   # head dim 128 only
    assert L.ufp4_kv_cache_bytes(2, 2, 256, 128, 2) == 0               # unknown format
    assert U.ufp4_kv_cache_bytes(1, 1, 128 * 70000) == 0               # one sequence's pages over 2 GiB
    q = L.ufp4_kv_cache_quantize
    assert q(FAKE, FAKE, 1, 1, 100, 128, 0, 0, 0, 128, FAKE, 1, FAKE, None) == -2
    assert q(FAKE, FAKE, 1, 1, 128, 64, 0, 0, 0, 128, FAKE, 1, FAKE, None) == -4
    assert q(FAKE, FAKE, 1, 1, 128, 128, 0, 0, 0, 120, FAKE, 1, FAKE, None) == -2   # token stride < D
    assert q(FAKE, FAKE, 1, 1, 128, 128, 0, 0, 0, 130, FAKE, 1, FAKE, None) == -3   # stride not a multiple of 8
    assert q(FAKE + 2, FAKE, 1, 1, 128, 128, 0, 0, 0, 128, FAKE, 1, FAKE, None) == -3
    assert q(FAKE, FAKE, 1, 1, 128, 128, 0, 0, 0, 128, None, 1, FAKE, None) == -1
    assert q(FAKE, FAKE, 1, 1, 128, 128, 0, 0, 0, 128, FAKE, 2, FAKE, None) == -1
    assert q(FAKE, FAKE, 1, 1, 128, 128, 5, 0, 0, 128, FAKE, 1, FAKE, None) == -1   # unknown format
    assert q(None, None, 0, 1, 128, 128, 0, 0, 0, 128, None, 1, None, None) == 0    # empty batch
    assert L.ufp4_kv_q_quantize(FAKE, 4, 64, 1, FAKE, FAKE, None) == -4
    assert L.ufp4_kv_q_quantize(FAKE, 4, 128, 1, FAKE + 4, FAKE, None) == -3
    d = L.ufp4_kv_decode
    assert d(FAKE, FAKE, FAKE, 1, 6, 4, 128, 0, 128, 0.1, 1, 0, FAKE, None, 0, None) == -2    # Hq % Hkv
    assert d(FAKE, FAKE, FAKE, 1, 32, 1, 128, 0, 128, 0.1, 1, 0, FAKE, None, 0, None) == -4   # 32 query rows per KV head
    assert d(FAKE, FAKE, FAKE, 1, 4, 1, 128, 0, 128, float("inf"), 1, 0, FAKE, None, 0, None) == -1
    assert d(FAKE, FAKE, FAKE, 1, 4, 1, 128, 0, 128, 0.1, 1, -1, FAKE, None, 0, None) == -1
    assert d(FAKE, FAKE, FAKE, 1, 4, 1, 128, 3, 128, 0.1, 1, 0, FAKE, None, 0, None) == -1    # unknown format
    assert d(FAKE, FAKE, FAKE, 1, 4, 1, 128, 0, 1024, 0.1, 1, 2, FAKE, None, 0, None) == -5   # 4 splits need a workspace


def test_kv_decode_workspace_sizes():
    # one split: no workspace; four splits of 2 pages: B * Hq * 4 * (128 + 2) floats
    assert U.ufp4_kv_decode_workspace_size(1, 4, 1, 256) == 0
    assert U.ufp4_kv_decode_workspace_size(1, 4, 1, 1024, pages_per_split=2) == 1 * 4 * 4 * 130 * 4
    # automatic split: about 256 workgroups of at least 8 pages; 256 sequences
    # of 128 pages need no split, 4 sequences are cut into 16 splits of 8 pages
    assert U.ufp4_kv_decode_workspace_size(32, 32, 8, 16384) == 0
    assert U.ufp4_kv_decode_workspace_size(1, 16, 4, 16384) == 1 * 16 * 16 * 130 * 4


def test_package_without_the_library_fails_loudly(tmp_path):
    """A copy of the package without libufp4.so refuses to import (no CPU
    fallback exists to route to)."""
    import shutil
    import subprocess
    import sys
    src = os.path.dirname(os.path.abspath(U.__file__))
    dst = tmp_path / "block_scaled_bit_ufp4_amd"
    dst.mkdir()
    for name in os.listdir(src):
        if name.endswith(".py"):
            shutil.copy(os.path.join(src, name), dst / name)
    assert not (dst / "libufp4.so").exists()
    r = subprocess.run([sys.executable, "-c", "import block_scaled_bit_ufp4_amd"], cwd=str(tmp_path),
                       env={**os.environ, "PYTHONPATH": str(tmp_path)}, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libufp4.so not built" in r.stderr
