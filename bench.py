"""Benchmark of the exact fused attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--cpu-baseline on|off] [--copy-calibration]
                    [--mfma-ceiling on|off] [--extras on|off]

One step is one pass of the whole path over one batch of synthetic input:
  * the fused causal forward (fa_fwd) on B=8, H=16, Nq=Nk=8192, d=128, bf16, K scaled x2;
  * one-token split-KV decode (fa_decode_split + fa_decode_combine) on B=16, H=32,
    Nk=32768, d=128, bf16, 64 splits.
Inputs are generated on the host from the seeded recipe, copied to HBM once, and stay
resident; the timed region holds only kernel launches.  Every launch is bracketed by HIP
events on the stream it runs on, so per-kernel average durations come from the GPU clock.

The printed JSON line carries:
  value        forward TFLOP/s = 4*B*H*Nq*Nk*d / 2 (causal) / mean fa_fwd duration
  roofline     the forward kernel against the dense bf16 MFMA peak (2516.6 TFLOP/s); beside it,
               the sustained matrix-core rate this GPU holds under a long run of back-to-back
               bf16 MFMAs on N(0,1) operands (libfa_calib.so), which sits below the nominal
               peak because the engine clock settles under 2.4 GHz
  decode       decode KV-read GB/s (K and V read once) with its own HBM roofline
  cpu_baseline the float64 reference implementation timed on the host cores on a sample
               of the same workload (a reported baseline only)
  extras       the other entry points, timed separately after the steps (not part of
               `value`): the backward (fa_bwd) on the headline prefill, a bottom-right causal,
               grouped-K/V-head prefill chunk (fa_fwd_ex, FLOPs counted over the visible
               query-key pairs) and a grouped-K/V-head decode (fa_decode_split_ex +
               fa_decode_combine, GB/s of K/V bytes read once)
HBM traffic measured with rocprofv3 counters is read from profiles/ when the summary there
was taken on the current kernel sources, else reported as null.
"""
from __future__ import annotations

import argparse
import hashlib
import math
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import roofline  # noqa: E402  (MI355X peaks and the algorithmic work and byte models)

PEAK_BF16_TFLOPS = roofline.PEAK_BF16_MFMA_TFLOPS
PEAK_FP8_TFLOPS = roofline.PEAK_FP8_MFMA_TFLOPS
PEAK_HBM_GBS = roofline.PEAK_HBM_GBS
PREFILL = "prefill_b8h16_n8192_d128_causal"
DECODE = "decode_b16h32_nk32768_d128"
FWD_SOURCES = ["exact_attention_126_amd/csrc/fa_fwd.hip", "exact_attention_126_amd/csrc/fa_device.h",
               "exact_attention_126_amd/csrc/fa_tile_layout.h"]
DEC_SOURCES = ["exact_attention_126_amd/csrc/fa_decode.hip", "exact_attention_126_amd/csrc/fa_device.h"]


def sources_sha(paths) -> str:
    """Hash of the kernel sources with // comments and whitespace removed, so that editing a
    comment does not invalidate counter figures taken on the same code."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p)) as f:
            for ln in f:
                code = ln.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode())
    return h.hexdigest()[:16]


def read_traffic(name: str, paths) -> dict | None:
    """Counter-derived HBM bytes per launch from profiles/<name>, if it matches the sources."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith((" ", "#", "|", "`")):
                k, v = ln.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("sources_sha256_16") != sources_sha(paths):
        return None
    try:
        return {"bytes": float(kv["traffic_bytes_per_launch"]), "read": float(kv["read_bytes_per_launch"]),
                "write": float(kv["write_bytes_per_launch"])}
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------- CPU baseline (oracle)
def _oracle_prefill_head(args):
    import threadpoolctl
    import oracle
    from synth import inputs as si
    from synth.workloads import get
    w = get(PREFILL)
    b, h = args
    with threadpoolctl.threadpool_limits(1):
        q, k, v = (si.head_block_f32(w, x, b, h) for x in "qkv")
        t0 = time.perf_counter()
        oracle.attention_head(q, k, v, w.scale, w.causal)
        return time.perf_counter() - t0


def _oracle_decode_head(args):
    import threadpoolctl
    import oracle
    from synth import inputs as si
    from synth.workloads import get
    w = get(DECODE)
    b, h = args
    with threadpoolctl.threadpool_limits(1):
        q, k, v = (si.head_block_f32(w, x, b, h) for x in "qkv")
        t0 = time.perf_counter()
        oracle.attention_head(q, k, v, w.scale, False)
        return time.perf_counter() - t0


def cpu_baseline():
    """Time the float64 reference on the host cores, on whole heads of the two workloads.

    Runs before anything touches the GPU: the worker processes are forked from a process
    that has not initialised the HIP runtime.  Each worker uses one BLAS thread."""
    import multiprocessing as mp
    from synth.workloads import get
    cores = min(16, len(os.sched_getaffinity(0)))
    wp, wd = get(PREFILL), get(DECODE)
    n_pre = 2 * cores  # whole heads of batch 0 (and 1 on a wide host)
    pre_heads = [(i // wp.H, i % wp.H) for i in range(n_pre)]
    dec_heads = [(i // wd.H, i % wd.H) for i in range(4 * cores)]
    ctx = mp.get_context("fork")
    with ctx.Pool(cores) as pool:
        t0 = time.perf_counter()
        pool.map(_oracle_prefill_head, pre_heads, chunksize=1)
        t_pre = time.perf_counter() - t0
        t0 = time.perf_counter()
        pool.map(_oracle_decode_head, dec_heads, chunksize=1)
        t_dec = time.perf_counter() - t0
    flops = 4.0 * len(pre_heads) * wp.Nq * wp.Nk * wp.d / 2
    kv_bytes = 2 * len(dec_heads) * wd.Nk * wd.d * wd.elt_bytes
    prefill = {"value": flops / t_pre / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
               "sample": f"{len(pre_heads)} of {wp.B * wp.H} heads of {PREFILL} (whole heads; float64; the "
                         f"reference builds the full masked score matrix, counted at the causal FLOP formula), "
                         f"{t_pre:.2f} s wall"}
    decode = {"value": kv_bytes / t_dec / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
              "sample": f"{len(dec_heads)} of {wd.B * wd.H} heads of {DECODE} (float64), {t_dec:.2f} s wall"}
    return prefill, decode


# ----------------------------------------------------------------- GPU part
def sustained_mfma_ceiling(torch, warm_s: float = 0.3, reps: int = 20) -> dict | None:
    """Sustained dense bf16 MFMA TFLOP/s: one wave per SIMD issues v_mfma_f32_32x32x16_bf16 back to back on
    seeded N(0,1) bf16 operands (the value distribution of the workload's Q, K, V) for warm_s
    seconds, then `reps` launches are timed with HIP events; the kernel also reports its shader
    clock (s_memtime against the 100 MHz s_memrealtime).  None if libfa_calib.so is not built."""
    import ctypes
    path = os.path.join(ROOT, "exact_attention_126_amd", "libfa_calib.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.fa_calib_src_bytes.argtypes = [ctypes.c_int]
    lib.fa_calib_src_bytes.restype = ctypes.c_size_t
    lib.fa_calib_out_floats.argtypes = [ctypes.c_int]
    lib.fa_calib_out_floats.restype = ctypes.c_size_t
    lib.fa_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_calib_mfma.restype = ctypes.c_int
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    niter = 40000
    nb, nf = lib.fa_calib_src_bytes(grid), lib.fa_calib_out_floats(grid)
    g = torch.Generator(device="cuda").manual_seed(7)
    src = torch.randn(nb // 2, generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty(nf, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2 * grid, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()

    def launch():
        rc = lib.fa_calib_mfma(src.data_ptr(), nb, out.data_ptr(), nf, clk.data_ptr(), grid, niter, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"fa_calib_mfma failed ({rc})")

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for _ in range(10):
            launch()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = grid * 4.0 * 4.0 * niter * 32768.0  # 4 waves per workgroup, 4 * niter MFMAs per wave
    c = clk.cpu().tolist()
    ghz = sum(c[2 * i] / (c[2 * i + 1] * 10.0) for i in range(grid)) / grid
    return {"value": round(flops / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s", "clock_ghz": round(ghz, 3),
            "operands": "bf16 N(0,1), seeded", "warm_s": warm_s}


def time_backward(torch, fa, si, w, dev, o, lse, reps: int = 10) -> dict:
    """fa_bwd on the headline prefill (its q, k, v and the o, lse of the timed forward) with a seeded
    N(0,1) dO; TFLOP/s counted as 2.5x the forward's FLOPs (the five products of the gradients
    against the forward's two), the usual convention, though the kernels compute seven."""
    stream = torch.cuda.current_stream()
    do = to_device(w, si.make_tensor(w, "do"))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.Nq) // 4, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(dev["q"]), torch.empty_like(dev["k"]), torch.empty_like(dev["v"])
    mask = fa.FA_MASK_CAUSAL if w.causal else fa.FA_MASK_NONE
    call = lambda: fa.fa_bwd(dev["q"], dev["k"], dev["v"], o, do, lse, dq, dk, dv, ws, mask, w.scale, stream=stream)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = 2.5 * 4.0 * w.B * w.H * w.Nq * w.Nk * w.d / (2 if w.causal else 1) / (ms * 1e-3) / 1e12
    del do, ws, dq, dk, dv
    return {"workload": w.name, "entry": "fa_bwd (dQ, dK, dV)", "value": round(tf, 1),
            "unit": "TFLOP/s (2.5x forward FLOPs)", "ms": round(ms, 4), "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}


def time_extras(torch, fa, si, get, reps: int = 20, min_window_ms: float = 20.0) -> dict:
    """The extended entry points on their own workloads, each timed over at least `reps` launches
    after a warm-up, with HIP events on the current stream.  A kernel that `reps` launches keep busy
    for less than `min_window_ms` is timed again over enough launches to fill that window: a window
    of a millisecond or two mostly measures how far the clock has ramped up."""
    stream = torch.cuda.current_stream()

    def timed(fn, n, warm):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()

        def window(k):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(k):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)

        ms = window(n)
        if ms < min_window_ms:
            n = min(50 * n, math.ceil(n * min_window_ms / max(ms, 1e-3)))
            ms = window(n)
        return ms / n

    out = {}
    # the other forward workloads: the tiny fp32 case, the short d = 64 batch and the long context
    for name in ("tiny_f32_n128_d64", "batch_b4h16_n2048_d64", "long_b1h32_n16384_d128_causal"):
        w = get(name)
        if w.dtype == "f32":
            dev = {x: torch.from_numpy(si.make_tensor(w, x)).cuda() for x in "qkv"}
        else:
            dev = {x: to_device(w, si.make_tensor(w, x)) for x in "qkv"}
        o = torch.empty_like(dev["q"])
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
        n = 10 * reps if w.dtype == "f32" else reps
        ms = timed(lambda: fa.fa_fwd(dev["q"], dev["k"], dev["v"], o, lse, causal=w.causal, scale=w.scale,
                                     stream=stream), n, n)
        tf = 4.0 * w.B * w.H * w.Nq * w.Nk * w.d / (2 if w.causal else 1) / (ms * 1e-3) / 1e12
        out[name] = {"workload": w.name, "entry": "fa_fwd (" + ("fp32" if w.dtype == "f32" else "bf16") +
                     (", causal)" if w.causal else ")"), "value": round(tf, 2), "unit": "TFLOP/s", "ms": round(ms, 4),
                     "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}
        if w.d == 64 and w.dtype == "bf16":
            # d = 64: per 64 keys a wave's MFMA work is 16 MFMAs (512 cycles; the kernel runs 128-key tiles,
            # 32 MFMAs each) while its softmax is about 154 VALU instructions (counted, 308 per 128-key tile,
            # profiles/counters_fwd_valu_issue_*), 616 cycles at one wave64 instruction per 4 cycles: the VALU
            # issue roof is 512 / 616 of the matrix-core peak
            valu_roof = PEAK_BF16_TFLOPS * 512 / (154 * 4)
            out[name]["roofline"] = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                                     "valu_issue_roof": round(valu_roof, 1),
                                     "frac_of_valu_issue_roof": round(tf / valu_roof, 4)}
        del dev, o, lse
    w = get("chunk_prefill_b1h32kv8_nq2048_nk16384_d128")
    dev = {x: to_device(w, si.make_tensor(w, x)) for x in "qkv"}
    o = torch.empty_like(dev["q"])
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    ms = timed(lambda: fa.fa_fwd_ex(dev["q"], dev["k"], dev["v"], o, lse, fa.FA_MASK_CAUSAL_BOTTOM_RIGHT, w.scale,
                                    stream=stream), 2 * reps, 2 * reps)
    pairs = sum(min(w.Nk, i + w.diag + 1) for i in range(w.Nq))  # visible (query, key) pairs per head
    tf = 4.0 * w.B * w.H * pairs * w.d / (ms * 1e-3) / 1e12
    out["chunked_prefill"] = {"workload": w.name, "entry": "fa_fwd_ex (bottom-right causal, H_kv=8)",
                              "value": round(tf, 1), "unit": "TFLOP/s", "ms": round(ms, 4),
                              "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}
    del dev, o, lse
    # the element-mask forward on packed documents (causal inside each document)
    import numpy as np
    from synth import masks
    w = get("masked_docs_b4h16_n8192_d128")
    allowed = masks.element_mask(w)
    pairs = masks.visible_pairs(allowed)
    blocks = allowed.reshape(w.Nq // 256, 256, w.Nk // 64, 64)
    t_any, t_all = blocks.any(axis=(1, 3)), blocks.all(axis=(1, 3))
    md = torch.from_numpy(masks.pack_bits(allowed).view(np.int64)).cuda()
    dev = {x: to_device(w, si.make_tensor(w, x)) for x in "qkv"}
    o = torch.empty_like(dev["q"])
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_fwd_masked_workspace_bytes(w.Nq, w.Nk), dtype=torch.uint8, device="cuda")
    ms = timed(lambda: fa.fa_fwd_masked(dev["q"], dev["k"], dev["v"], o, lse, md, ws, w.scale, stream=stream),
               reps, 3)
    tf = 4.0 * w.B * w.H * pairs * w.d / (ms * 1e-3) / 1e12
    out["masked_documents"] = {
        "workload": w.name, "entry": "fa_fwd_masked (tile classification + forward)", "value": round(tf, 1),
        "unit": "TFLOP/s (4 d FLOP per visible query-key pair)", "ms": round(ms, 4),
        "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
        "visible_fraction": round(pairs / (w.Nq * w.Nk), 4),
        "tiles_256x64": {"empty": int((~t_any).sum()), "full": int(t_all.sum()), "partial": int((t_any & ~t_all).sum())}}
    del dev, o, lse, ws, md
    w = get("decode_gqa_b16h32kv8_nk32768_d128")
    dev = {x: to_device(w, si.make_tensor(w, x)) for x in "qkv"}
    ws = fa.decode_workspace(dev["q"], w.num_splits)
    o = torch.empty_like(dev["q"])
    lse = torch.empty((w.B, w.H, 1), dtype=torch.float32, device="cuda")
    ms_s = timed(lambda: fa.fa_decode_split_ex(dev["q"], dev["k"], dev["v"], ws, w.num_splits, w.scale,
                                               stream=stream), reps, 3)
    ms_c = timed(lambda: fa.fa_decode_combine(ws, o, lse, w.num_splits, stream=stream), reps, 3)
    kv = 2.0 * w.B * w.kv_heads * w.Nk * w.d * w.elt_bytes
    gbs = kv / ((ms_s + ms_c) * 1e-3) / 1e9
    out["decode_gqa"] = {"workload": w.name, "entry": "fa_decode_split_ex + fa_decode_combine (H_kv=8)",
                         "value": round(gbs, 1), "unit": "GB/s (K/V bytes read once)",
                         "split_ms": round(ms_s, 4), "combine_ms": round(ms_c, 4),
                         "pct_of_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2)}
    del dev, ws, o, lse
    w = get("prefill_fp8_b8h16_n8192_d128_causal")
    t8 = {}
    for x in "qkv":
        codes, scales = si.make_kv_fp8(w, x)
        t8[x], t8[x + "s"] = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
        del codes
    o = torch.empty((w.B, w.H, w.Nq, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    ms = timed(lambda: fa.fa_fwd_fp8(t8["q"], t8["k"], t8["v"], t8["qs"], t8["ks"], t8["vs"], o, lse,
                                     fa.FA_MASK_CAUSAL, w.scale, stream=stream), reps, 3)
    flops = 4.0 * w.B * w.H * w.d * (w.Nq * (w.Nq + 1) / 2)  # visible (query, key) pairs, 4d FLOP each
    tf = flops / (ms * 1e-3) / 1e12
    out["prefill_fp8"] = {"workload": w.name, "entry": "fa_fwd_fp8 (E4M3 Q, K, V; causal)", "value": round(tf, 1),
                          "unit": "TFLOP/s", "ms": round(ms, 4),
                          "pct_of_fp8_peak": round(100 * tf / PEAK_FP8_TFLOPS, 2),
                          "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}
    del t8, o, lse
    w = get("decode_fp8kv_b16h32_nk32768_d128")
    q = to_device(w, si.make_tensor(w, "q"))
    kv = {}
    for x in "kv":
        codes, scales = si.make_kv_fp8(w, x)
        kv[x], kv[x + "s"] = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
        del codes
    ws = fa.decode_workspace(q, w.num_splits)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, 1), dtype=torch.float32, device="cuda")
    ms_s = timed(lambda: fa.fa_decode_split_fp8kv(q, kv["k"], kv["v"], kv["ks"], kv["vs"], ws, w.num_splits, w.scale,
                                                  stream=stream), reps, 3)
    ms_c = timed(lambda: fa.fa_decode_combine(ws, o, lse, w.num_splits, stream=stream), reps, 3)
    nbytes = 2.0 * w.B * w.kv_heads * w.Nk * w.d  # one byte per code
    gbs = nbytes / ((ms_s + ms_c) * 1e-3) / 1e9
    out["decode_fp8kv"] = {"workload": w.name, "entry": "fa_decode_split_fp8kv + fa_decode_combine (E4M3 K/V)",
                           "value": round(gbs, 1), "unit": "GB/s (E4M3 K/V bytes read once)",
                           "split_ms": round(ms_s, 4), "combine_ms": round(ms_c, 4),
                           "pct_of_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2)}
    del q, kv, ws, o, lse
    return out


def to_device(w, x):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--extras", choices=["on", "off"], default="on",
                    help="after the timed steps, time the extended entry points on their own workloads")
    ap.add_argument("--mfma-ceiling", choices=["on", "off"], default="on",
                    help="after the timed steps, measure the sustained bf16 MFMA rate (libfa_calib.so)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device-to-device copy (reference point for HBM counters)")
    ap.add_argument("--kernel-only", metavar="WORKLOAD[:bwd]", default=None,
                    help="for profiler runs: launch fa_fwd on one forward workload --warmup + --steps times (with "
                         "':bwd', fa_fwd once and then fa_bwd that many times) and exit, with no timing and no "
                         "JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path shards over "
              f"(batch, head) with no communication, so N GPUs run N independent copies of this step).",
              file=sys.stderr)
        sys.exit(2)

    from synth import inputs as si
    from synth.workloads import get

    if args.kernel_only:
        import torch
        import exact_attention_126_amd as fa
        name, _, what = args.kernel_only.partition(":")
        w = get(name)
        if w.is_decode or w.q_dtype or w.kv_dtype or w.mask_rule or w.kv_heads != w.H or w.causal_align != "top_left":
            sys.exit(f"--kernel-only takes a plain forward workload (fa_fwd), not {w.name}")
        if w.dtype == "f32":
            dev = {x: torch.from_numpy(si.make_tensor(w, x)).cuda() for x in "qkv"}
        else:
            dev = {x: to_device(w, si.make_tensor(w, x)) for x in "qkv"}
        o = torch.empty_like(dev["q"])
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
        if what == "bwd":
            fa.fa_fwd(dev["q"], dev["k"], dev["v"], o, lse, causal=w.causal, scale=w.scale)
            do = to_device(w, si.make_tensor(w, "do"))
            for _ in range(args.warmup + args.steps):
                fa.attention_backward(dev["q"], dev["k"], dev["v"], o, lse, do, causal=w.causal, scale=w.scale)
        else:
            for _ in range(args.warmup + args.steps):
                fa.fa_fwd(dev["q"], dev["k"], dev["v"], o, lse, causal=w.causal, scale=w.scale)
        torch.cuda.synchronize()
        print(f"[bench] --kernel-only {args.kernel_only}: {args.warmup + args.steps} launches", file=sys.stderr)
        return

    cpu_pre = cpu_dec = None
    if args.cpu_baseline == "on":
        print("[bench] timing the float64 reference on host cores ...", file=sys.stderr, flush=True)
        cpu_pre, cpu_dec = cpu_baseline()
        print(f"[bench] cpu baseline: {cpu_pre['value']:.4f} TFLOP/s, {cpu_dec['value']:.2f} GB/s "
              f"on {cpu_pre['cores']} cores", file=sys.stderr, flush=True)

    import torch
    import exact_attention_126_amd as fa

    wp, wd = get(PREFILL), get(DECODE)
    t0 = time.perf_counter()
    dp = {x: to_device(wp, si.make_tensor(wp, x)) for x in "qkv"}
    dd = {}
    for x in "qkv":
        dd[x] = to_device(wd, si.make_tensor(wd, x))
    print(f"[bench] inputs generated and resident in HBM in {time.perf_counter() - t0:.1f} s",
          file=sys.stderr, flush=True)

    o = torch.empty_like(dp["q"])
    lse = torch.empty((wp.B, wp.H, wp.Nq), dtype=torch.float32, device="cuda")
    od = torch.empty_like(dd["q"])
    lsed = torch.empty((wd.B, wd.H, 1), dtype=torch.float32, device="cuda")
    ws = fa.decode_workspace(dd["q"], wd.num_splits)
    stream = torch.cuda.current_stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def step(rec=None):
        e = [ev() for _ in range(4)] if rec is not None else None
        if e: e[0].record(stream)
        fa.fa_fwd(dp["q"], dp["k"], dp["v"], o, lse, causal=True, scale=wp.scale, stream=stream)
        if e: e[1].record(stream)
        fa.fa_decode_split(dd["q"], dd["k"], dd["v"], ws, wd.num_splits, wd.scale, stream=stream)
        if e: e[2].record(stream)
        fa.fa_decode_combine(ws, od, lsed, wd.num_splits, stream=stream)
        if e: e[3].record(stream)
        if rec is not None:
            rec.append(e)

    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] copy calibration: 1 GiB read + 1 GiB written by one device copy", file=sys.stderr, flush=True)
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rec = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    t_fwd = [a.elapsed_time(b) for a, b, _, _ in rec]
    t_split = [b.elapsed_time(c) for _, b, c, _ in rec]
    t_comb = [c.elapsed_time(d) for _, _, c, d in rec]
    ms_fwd = sum(t_fwd) / len(t_fwd)
    ms_split = sum(t_split) / len(t_split)
    ms_comb = sum(t_comb) / len(t_comb)
    flops = 4.0 * wp.B * wp.H * wp.Nq * wp.Nk * wp.d / 2
    tflops = flops / (ms_fwd * 1e-3) / 1e12
    kv_bytes = 2.0 * wd.B * wd.H * wd.Nk * wd.d * wd.elt_bytes
    dec_gbs = kv_bytes / ((ms_split + ms_comb) * 1e-3) / 1e9
    split_gbs = kv_bytes / (ms_split * 1e-3) / 1e9

    bwd = time_backward(torch, fa, si, wp, dp, o, lse) if args.extras == "on" else None
    del dp, dd, o, lse, od, lsed, ws
    extras = time_extras(torch, fa, si, get) if args.extras == "on" else None
    if extras is not None:
        extras["backward"] = bwd
    ceiling = sustained_mfma_ceiling(torch) if args.mfma_ceiling == "on" else None
    tr_f = read_traffic("fwd_bf16_prefill_b8h16_n8192_d128_causal_hbm_traffic.txt", FWD_SOURCES)
    tr_d = read_traffic("decode_split_b16h32_nk32768_d128_hbm_traffic.txt", DEC_SOURCES)
    line = {
        "metric": "fwd attention TFLOP/s & % bf16 MFMA peak at N=8K d=128; decode KV GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded PCG64 N(0,1), rounded to bf16)",
        "config": {"workload": f"{PREFILL} + {DECODE}", "prefill": "B=8 H=16 Nq=Nk=8192 d=128 causal, K x2",
                   "decode": "B=16 H=32 Nq=1 Nk=32768 d=128, 64 splits", "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "fwd_ms": round(ms_fwd, 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "kernel": "fwd_bf16_kernel<128, causal>",
                     "traffic": None if tr_f is None else tr_f["bytes"],
                     "sustained_mfma": ceiling,
                     "frac_of_sustained": None if ceiling is None else round(tflops / ceiling["value"], 4)},
        "decode": {"value": round(dec_gbs, 1), "unit": "GB/s", "pct_of_hbm_peak": round(100 * dec_gbs / PEAK_HBM_GBS, 2),
                   "split_ms": round(ms_split, 4), "combine_ms": round(ms_comb, 4),
                   "roofline": {"bound": "hbm", "achieved": round(split_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(split_gbs / PEAK_HBM_GBS, 4), "kernel": "decode_split_kernel<bf16, 128>",
                                "traffic": None if tr_d is None else tr_d["bytes"]},
                   "cpu_baseline": cpu_dec},
        "cpu_baseline": cpu_pre,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
