"""Reentrancy and graph capture.  The library's calls allocate nothing and
record no memset, so a captured sequence (tensor amax, quantize with RTNE and
with stochastic rounding, column quantize, dequantize, statistics, both GEMM
modes, KV-cache quantize and a split KV decode) replays to the eager results
bit for bit, replay after replay, with unrelated eager work and
synchronizations between the replays."""
import numpy as np
import pytest

import synthetic as S
from helpers import host, to_device_bf16

pytestmark = pytest.mark.gpu


def _outputs(U, torch, x, a, b, kv):
    """Preallocated outputs and workspaces, and the call sequence writing
    them (every call gets its buffers, so nothing is allocated inside)."""
    R, C = x.shape
    c_e2m1 = U.Cfg("e2m1", "e4m3", rht="random", rht_seed=3)
    c_sr = U.Cfg("e1m2", "fp32", rht="random", rht_seed=3, rounding="sr", sr_seed=11)
    c_col = U.Cfg("e1m2", "fp32", rht="random", rht_seed=3, axis="col")
    c_mx = U.Cfg("e2m1", "e8m0", 32, rht="random", rht_seed=4)
    c_bf = U.Cfg("e1m2", "fp32", rht="random", rht_seed=4)
    M, K = a.shape
    N = b.shape[0]
    o = {
        "amax": torch.zeros(1, dtype=torch.float32, device="cuda"),
        "amax_ws": torch.empty(U.ufp4_workspace_size(U.OP_AMAX, R, C, c_e2m1), dtype=torch.uint8, device="cuda"),
        "q_e2m1": U.alloc_qtensor(R, C, c_e2m1),
        "q_sr": U.alloc_qtensor(R, C, c_sr),
        "q_col": U.alloc_qtensor(R, C, c_col),
        "deq": torch.empty((R, C), dtype=torch.float32, device="cuda"),
        "sums": torch.empty(U.NSUMS, dtype=torch.float64, device="cuda"),
        "qa_mx": U.alloc_qtensor(M, K, c_mx), "qb_mx": U.alloc_qtensor(N, K, c_mx),
        "qa_bf": U.alloc_qtensor(M, K, c_bf), "qb_bf": U.alloc_qtensor(N, K, c_bf),
        "z_mx": torch.empty((M, N), dtype=torch.float32, device="cuda"),
        "z_bf": torch.empty((M, N), dtype=torch.float32, device="cuda"),
        "gemm_ws": torch.empty(U.ufp4_workspace_size(U.OP_QGEMM, M + N, K, c_bf), dtype=torch.uint8,
                               device="cuda"),
    }
    o["stats_ws"] = torch.empty(U.ufp4_workspace_size(U.OP_STATS, R, C, c_e2m1), dtype=torch.uint8, device="cuda")
    q, k, v, lens, Hkv, L = kv
    B, Hq, D = q.shape
    o["cache"] = torch.empty(U.ufp4_kv_cache_bytes(B, Hkv, L, D), dtype=torch.uint8, device="cuda")
    o["attn"] = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    o["kv_ws"] = torch.empty(max(16, U.ufp4_kv_decode_workspace_size(B, Hq, Hkv, L, pages_per_split=8)),
                             dtype=torch.uint8, device="cuda")

    def run():
        U.ufp4_amax(x, c_e2m1, out=o["amax"], ws=o["amax_ws"])
        U.ufp4_quantize(x, c_e2m1, amax=o["amax"], out=o["q_e2m1"])
        U.ufp4_quantize(x, c_sr, out=o["q_sr"])
        U.ufp4_quantize(x, c_col, out=o["q_col"])
        U.ufp4_dequantize(o["q_e2m1"], inverse_rht=True, y=o["deq"])
        U.ufp4_stats(x, o["q_e2m1"], sums=o["sums"], ws=o["stats_ws"])
        U.ufp4_quantize(a, c_mx, out=o["qa_mx"])
        U.ufp4_quantize(b, c_mx, out=o["qb_mx"])
        U.ufp4_qgemm(o["qa_mx"], o["qb_mx"], "mxfp4", c=o["z_mx"])
        U.ufp4_quantize(a, c_bf, out=o["qa_bf"])
        U.ufp4_quantize(b, c_bf, out=o["qb_bf"])
        U.ufp4_qgemm(o["qa_bf"], o["qb_bf"], "bf16", c=o["z_bf"], ws=o["gemm_ws"])
        U.ufp4_kv_cache_quantize(k, v, lens, True, cache=o["cache"])
        U.ufp4_kv_decode(q, o["cache"], lens, Hkv, L, 0.088, True, pages_per_split=8, out=o["attn"],
                         ws=o["kv_ws"])

    return o, run


def _snapshot(o):
    snap = {}
    for name, t in o.items():
        if name.endswith("_ws"):
            continue
        if hasattr(t, "codes"):
            snap[name + ".codes"] = host(t.codes)
            snap[name + ".scales"] = host(t.scales)
            if t.tensor_scale is not None:
                snap[name + ".tensor_scale"] = host(t.tensor_scale)
        else:
            snap[name] = host(t)
    return snap


def _scramble(o):
    """Overwrite every output eagerly, so a replay that skipped a call would
    leave visible garbage."""
    for name, t in o.items():
        if name.endswith("_ws"):
            continue
        for u in ([t.codes, t.scales] + ([t.tensor_scale] if t.tensor_scale is not None else [])
                  if hasattr(t, "codes") else [t]):
            if u.dtype.is_floating_point:
                u.fill_(-7.0)
            else:
                u.fill_(0x5A)


def test_graph_replays_match_eager():
    import torch
    import block_scaled_bit_ufp4_amd as U
    x = to_device_bf16(S.activations_t3(512, 1024, seed=21))
    a = to_device_bf16(S.normal(256, 512, 1.0, 22, "gemm_a"))
    b = to_device_bf16(S.normal(512, 512, 1.0, 22, "gemm_b"))
    # two sequences of up to 16 pages, 8 pages per split: two splits and the
    # combine pass
    B, Hq, Hkv, L, D = 2, 8, 2, 2048, 128
    qh, kh, vh = S.kv_decode(B, Hq, Hkv, L, D, seed=23)
    kv = (to_device_bf16(qh), to_device_bf16(kh), to_device_bf16(vh),
          torch.tensor([L, 1400], dtype=torch.int32, device="cuda"), Hkv, L)
    o, run = _outputs(U, torch, x, a, b, kv)
    run()
    torch.cuda.synchronize()
    want = _snapshot(o)

    _scramble(o)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        _scramble(o)
        y = torch.randn(512, 512, device="cuda") @ torch.randn(512, 512, device="cuda")  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(o)
        assert float(y.abs().sum()) > 0
        for name in want:
            g_, w_ = got[name], want[name]
            if name == "cache":
                # pages past a sequence's length are not written (the decode
                # never reads them): compare the written pages only
                pb = U.KV_PAGE_BYTES["fp4"]
                npages = L // 128
                lens_h = host(kv[3])
                keep = np.zeros((B, Hkv, npages), dtype=bool)
                for bi in range(B):
                    keep[bi, :, :(int(lens_h[bi]) + 127) // 128] = True
                g_ = g_.reshape(B, Hkv, npages, pb)[keep]
                w_ = w_.reshape(B, Hkv, npages, pb)[keep]
            np.testing.assert_array_equal(g_, w_, err_msg=f"replay {rep}: {name}")


def test_concurrent_streams_and_threads_match_sequential():
    """Calls are reentrant: different quantizations and GEMMs issued at once on
    two streams, from two host threads, give the sequential results bit for
    bit (the library keeps no state between calls besides a per-thread
    last error)."""
    import threading
    import torch
    import block_scaled_bit_ufp4_amd as U
    x = to_device_bf16(S.activations_t3(1024, 2048, seed=31))
    a = to_device_bf16(S.normal(512, 1024, 1.0, 32, "gemm_a"))
    b = to_device_bf16(S.normal(512, 1024, 1.0, 32, "gemm_b"))
    jobs = [
        lambda st: U.ufp4_quantize(x, U.Cfg("e2m1", "e4m3", rht="random", rht_seed=1),
                                   amax=U.ufp4_amax(x, U.Cfg("e2m1", "e4m3", rht="random", rht_seed=1), stream=st),
                                   stream=st).codes,
        lambda st: U.ufp4_quantize(x, U.Cfg("e1m2", "fp32", rht="random", rht_seed=1, rounding="sr", sr_seed=5,
                                            axis="col"), stream=st).codes,
        lambda st: U.ufp4_qgemm(U.ufp4_quantize(a, U.Cfg("e2m1", "e8m0", 32), stream=st),
                                U.ufp4_quantize(b, U.Cfg("e2m1", "e8m0", 32), stream=st), "mxfp4", stream=st),
        lambda st: U.ufp4_quantize(x, U.Cfg("if4", "e4m3"), stream=st).scales,
    ]
    torch.cuda.synchronize()
    want = []
    for job in jobs:
        want.append(host(job(torch.cuda.current_stream())))
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [None] * len(jobs)

    def worker(w):
        torch.cuda.set_device(0)
        st = streams[w]
        with torch.cuda.stream(st):
            for i in range(w, len(jobs), 2):
                for _ in range(3):  # overlapping repeats on the same stream
                    got[i] = job_out = jobs[i](st)
                got[i] = job_out
        st.synchronize()

    threads = [threading.Thread(target=worker, args=(w,)) for w in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for i in range(len(jobs)):
        np.testing.assert_array_equal(host(got[i]), want[i], err_msg=f"job {i}")
