#!/usr/bin/env python3
"""Benchmark of one MLA decode step (absorbed-MQA form) on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic inputs:
the split-KV attention kernel over the paged latent cache followed by the LSE
combine (mla_decode_fwd_split + mla_decode_fwd_combine on one stream, which is
what mla_decode_fwd launches).  The split plan is made once per step for all
layers of a model, so it is timed separately and reported as ``plan_us``.

Default workload: batch 16, s_q 1, 16 heads, 65536-token contexts over a
shuffled pool of 64-token bf16 pages (about 1.2 GB of cache), values N(0,1).
Prints ONE JSON line on stdout; progress goes to stderr.  ``extras`` holds the
timings of the library's other entry points; ``--flush-mib`` adds per-step
timings taken after a last-level-cache flush.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


def read_probe_gbs(dev, stream, reps: int = 10):
    """Streaming-read rate of this GPU: a plain kernel (libmla_read_probe.so, built beside the
    decode library) reads 1 GiB once per launch; GB/s of bytes read.  None if it is not built."""
    import ctypes

    import torch

    import mla_decode_attention_amd as mla
    path = os.path.join(os.path.dirname(mla.LIB_PATH), "libmla_read_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.mla_read_probe_out_words.restype = ctypes.c_int
    lib.mla_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_longlong,
                                   ctypes.c_void_p]
    words = lib.mla_read_probe_out_words()
    if words <= 0:
        return None
    buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    out = torch.empty(words, dtype=torch.int32, device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    run = lambda: lib.mla_read_probe(buf.data_ptr(), buf.numel(), out.data_ptr(), words, sp)
    for _ in range(3):
        if run() != 0:
            return None
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    chunk = 18 * 1024
    return (buf.numel() // chunk) * chunk * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9

def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def source_code_digest(texts) -> str:
    """sha256 of C++ sources with comments and whitespace removed: an edit of a comment keeps the
    measurements taken on that code valid, any change of code does not."""
    import re
    h = hashlib.sha256()
    for txt in texts:
        txt = re.sub(r"/\*.*?\*/", " ", txt, flags=re.S)
        txt = re.sub(r"//[^\n]*", " ", txt)
        h.update(" ".join(txt.split()).encode())
    return h.hexdigest()[:16]


def kernel_source_digest() -> str:
    texts = []
    for f in ("mla_decode_kernels.h", "mla_plan_kernel.h", "mla_sv_kernel.h", "mla_decode.hip"):
        with open(os.path.join(ROOT, "mla_decode_attention_amd", "csrc", f)) as fh:
            texts.append(fh.read())
    return source_code_digest(texts)


def measured_traffic(workload: str):
    """HBM bytes per split-kernel launch from committed rocprofv3 PMC runs, if they match this source."""
    path = os.path.join(ROOT, "profiles", f"traffic_split_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_digest") != kernel_source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def c_calls(mla, fn):
    """Run fn once through the binding and return the C-ABI calls it made (function, marshalled
    arguments), for replay in timed loops: the binding's argument checks cost host time comparable
    to the shorter kernels, and a replayed call costs only the ctypes call itself."""
    calls = []
    real_lib = mla.lib

    class _Recorder:
        def __getattr__(self, name):
            f = getattr(real_lib(), name)

            def call(*args):
                calls.append((f, args))
                return f(*args)
            return call
    mla.lib = lambda: _Recorder()
    try:
        fn()
    finally:
        mla.lib = real_lib

    def replay():
        for f, a in calls:
            status = f(*a)
            if status != 0:
                raise RuntimeError(f"C call failed with status {status}")
    return replay


def cpu_baseline(case, o_gpu, lse_gpu, n_seqs: int, threads: int, min_seconds: float):
    """Time the fp64 oracle on the host cores over the first n_seqs sequences (all their query rows),
    repeating the sample until at least min_seconds of CPU work have been timed."""
    import numpy as np

    import oracle
    from mla_decode_attention_amd import workloads as W

    n_seqs = max(1, min(n_seqs, case.batch))
    rows = np.arange(n_seqs * case.s_q * case.heads, dtype=np.int64)
    oracle.default()   # load (and if needed build) outside the timed region
    reps, dt = 0, 0.0
    while reps == 0 or dt < min_seconds:
        t0 = time.perf_counter()
        ro, rl = oracle.mla_decode(case.q, case.cache, case.block_table, case.seqlens, case.softmax_scale,
                                   case.causal, rows=rows, threads=threads)
        dt += time.perf_counter() - t0
        reps += 1
    sample_bytes = W.algorithmic_bytes(case.seqlens[:n_seqs], n_seqs, case.s_q, case.heads)
    # per-core figure: one thread over the first sequence's rows
    rows1 = np.arange(case.s_q * case.heads, dtype=np.int64)
    t0 = time.perf_counter()
    oracle.mla_decode(case.q, case.cache, case.block_table, case.seqlens, case.softmax_scale, case.causal,
                      rows=rows1, threads=1)
    dt1 = time.perf_counter() - t0
    bytes1 = W.algorithmic_bytes(case.seqlens[:1], 1, case.s_q, case.heads)
    err = np.abs(o_gpu.reshape(case.rows, -1)[rows] - ro)
    rl_ok = np.isfinite(rl)
    parity = dict(rows=int(rows.size), o_maxabs=float(err.max()), o_rmse=float(np.sqrt(np.mean(err ** 2))),
                  lse_rel=float(np.max(np.abs(lse_gpu.reshape(-1)[rows][rl_ok] - rl[rl_ok])
                                       / np.maximum(1.0, np.abs(rl[rl_ok])))))
    return dict(value=sample_bytes * reps / dt / 1e12, unit="TB/s", cores=threads, kind="oracle",
                sample=f"{n_seqs} of {case.batch} sequences, all {case.s_q * case.heads} query rows each "
                       f"({rows.size} rows, {sample_bytes / 1e6:.1f} MB algorithmic), run {reps}x, "
                       f"fp64 C oracle (OpenMP)",
                seconds=round(dt, 2), cpu_model=_cpu_model(), host_cpus=os.cpu_count(),
                per_core_value=bytes1 / dt1 / 1e12,
                per_core_sample=f"1 thread, 1 sequence ({rows1.size} rows, {bytes1 / 1e6:.1f} MB algorithmic), "
                                f"{dt1:.2f} s"), parity


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def flushed_medians(scratch, kind: str, steps: int, split_c, combine_c, stream):
    """Median step (split + combine) and split-kernel durations in ms, each launch timed alone
    right after the scratch went through the cache: kind "read" sums it (clean lines), "write"
    fills it (dirty lines).  The step and the split are timed in separate loops, so that no event
    sits between the split and the combine of a timed step."""
    import numpy as np
    import torch

    def flush(k):
        if kind == "write":
            scratch.fill_(float(k))
        else:
            scratch.sum()

    def timed(body):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for k in range(steps):
            flush(k)
            ev[k][0].record(stream)
            body()
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))

    def step():
        split_c()
        combine_c()

    return timed(step), timed(split_c)


def measure_workload(mla, name: str, dev, steps: int, warmup: int, parity_rows: int, flush_mib: int = 512):
    """One of the other configured workloads, timed like the headline: step (split + combine) and
    split-kernel durations, algorithmic TB/s and MFMA utilisation, the same per step after a cache
    flush, and raw parity of the first parity_rows query rows against the fp64 oracle (reported,
    not asserted)."""
    import numpy as np
    import torch

    from mla_decode_attention_amd import workloads as W
    from mla_decode_attention_amd.inputs import bf16_bits_to_f32
    stream = torch.cuda.current_stream()
    case = W.build(name)
    q = torch.from_numpy(case.q.view(np.int16)).to(dev).view(torch.bfloat16)
    cache = torch.from_numpy(case.cache.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(case.block_table).to(dev)
    sl = torch.from_numpy(case.seqlens).to(dev)
    b, s_q, h = case.batch, case.s_q, case.heads
    ws = torch.empty(mla.workspace_size(b, s_q, h), dtype=torch.uint8, device=dev)
    out = torch.empty((b, s_q, h, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((b, s_q, h), dtype=torch.float32, device=dev)
    mla.plan(sl, s_q, h, ws)
    split_c = c_calls(mla, lambda: mla.fwd_split(q, cache, bt, sl, case.softmax_scale, case.causal, ws))
    combine_c = c_calls(mla, lambda: mla.fwd_combine(sl, bt.shape[1], s_q, h, ws, out, lse))
    for _ in range(warmup):
        split_c()
        combine_c()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        split_c()
        combine_c()
    e1.record(stream)
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) * 1e3 / steps
    ea = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    eb = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for k in range(steps):
        ea[k].record(stream)
        split_c()
        eb[k].record(stream)
        combine_c()
    torch.cuda.synchronize()
    split_us = float(np.mean([ea[k].elapsed_time(eb[k]) for k in range(steps)])) * 1e3
    # each step alone after 512 MiB (twice the last-level cache) went through the cache, so shapes
    # whose keys fit that cache are timed reading them from HBM too: "read" leaves clean lines (as a
    # model's other reads would), "write" dirty ones that must be written back as they are evicted
    scratch = torch.empty(flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    flushed = {}
    for kind in ("read", "write"):
        f_step, f_split = flushed_medians(scratch, kind, steps, split_c, combine_c, stream)
        flushed[kind] = (f_step * 1e3, f_split * 1e3)
    del scratch
    nbytes = W.algorithmic_bytes(case.seqlens, b, s_q, h)
    flops = W.algorithmic_flops(case.seqlens, s_q, h, case.causal)
    kv_q = int(case.seqlens.astype(np.int64).sum()) * W.ROW_BYTES + b * s_q * h * 576 * 2
    rec = {"us_per_step": round(step_us, 2), "split_avg_us": round(split_us, 2),
           "TB/s": round(nbytes / step_us / 1e6, 4), "pct_of_hbm_peak": round(100 * nbytes / step_us / 1e3 / HBM_PEAK_GBS, 2),
           "split_GB/s": round(kv_q / split_us / 1e3, 1),
           "mfma_util_step": round(flops / step_us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
           "mfma_util_split": round(flops / split_us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
           "flushed": {kind: {"flush_mib": flush_mib, "median_us_per_step": round(fs, 2),
                              "median_split_us": round(fp, 2), "TB/s": round(nbytes / fs / 1e6, 4),
                              "mfma_util_step": round(flops / fs / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4)}
                       for kind, (fs, fp) in flushed.items()},
           "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
           "config": {"batch": b, "s_q": s_q, "heads": h, "causal": bool(case.causal),
                      "context": [int(case.seqlens.min()), int(case.seqlens.max())]}}
    try:
        import oracle
        rows = np.arange(min(parity_rows, case.rows), dtype=np.int64)
        og = bf16_bits_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
        lg = lse.cpu().numpy().astype(np.float64).reshape(-1)[rows]
        ro, rl = oracle.mla_decode(case.q, case.cache, case.block_table, case.seqlens, case.softmax_scale,
                                   case.causal, rows=rows)
        err = np.abs(og.reshape(case.rows, -1)[rows] - ro)
        rec["parity_sampled_rows"] = {
            "rows": int(rows.size), "o_maxabs": float(err.max()), "o_rmse": float(np.sqrt(np.mean(err ** 2))),
            "o_maxabs_over_max1_maxO": float(err.max() / max(1.0, np.abs(ro).max())),
            "lse_rel": float(np.max(np.abs(lg - rl) / np.maximum(1.0, np.abs(rl))))}
    except Exception as exc:   # the timing stands without the check
        rec["parity_sampled_rows"] = f"skipped: {exc}"
    del q, cache, ws
    torch.cuda.empty_cache()
    return rec


def measure_extras(mla, case, dev, q, cache, bt, sl, steps: int):
    """Time the library's other entry points: a top-2048 sparse decode over the same cache (with a
    parity check of sampled query tokens against the fp64 oracle), the absorption and
    un-absorption products, the GQA path on the MTP shape beside the latent path on the same
    lengths (with sampled parity), and the cache append with rotary embedding of the new tokens."""
    import numpy as np
    import torch

    from mla_decode_attention_amd.inputs import make_append_inputs, make_sparse_indices
    stream = torch.cuda.current_stream()
    b, s_q, h = case.batch, case.s_q, case.heads

    def timed(fn):
        replay = c_calls(mla, fn)
        for _ in range(3):
            replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    out = {}
    topk = 2048
    ind = make_sparse_indices(case, topk, seed=8)
    ind_d = torch.from_numpy(ind).to(dev)
    ws = torch.empty(mla.sparse_workspace_size(b, s_q, h, topk), dtype=torch.uint8, device=dev)
    o = torch.empty((b, s_q, h, 512), dtype=torch.bfloat16, device=dev)
    l = torch.empty((b, s_q, h), dtype=torch.float32, device=dev)
    mla.sparse_plan(b, s_q, h, topk, ws)
    us = timed(lambda: mla.sparse_fwd(q, cache, bt, sl, ind_d, case.softmax_scale, ws, o, l))
    nbytes = int((ind >= 0).sum()) * 1152 + b * s_q * h * 576 * 2
    rec = {"us": round(us, 2), "topk": topk, "bytes": nbytes, "GB/s": round(nbytes / us / 1e3, 1),
           "frac_of_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4), "bound": "hbm"}
    try:
        import oracle
        from mla_decode_attention_amd.inputs import bf16_bits_to_f32
        og = bf16_bits_to_f32(o.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
        lg = l.cpu().numpy().astype(np.float64)
        sel = [0, b - 1]
        ro, rl = oracle.sparse_decode(case.q[sel], case.cache, case.block_table[sel], case.seqlens[sel], ind[sel],
                                      case.softmax_scale)
        err = np.abs(og[sel] - ro)
        rec["parity_sampled_tokens"] = {"tokens": len(sel) * s_q, "o_maxabs": float(err.max()),
                                        "lse_rel": float(np.max(np.abs(lg[sel] - rl) / np.maximum(1, np.abs(rl))))}
    except Exception as exc:   # the timing stands without the check
        rec["parity_sampled_tokens"] = f"skipped: {exc}"
    out["sparse_topk2048"] = rec
    from mla_decode_attention_amd.inputs import make_absorb_inputs
    qn, qr, wuk, wuv = (torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
                        for x in make_absorb_inputs(b, s_q, h, seed=9))
    qa = torch.empty((b, s_q, h, 576), dtype=torch.bfloat16, device=dev)
    ol = torch.randn((b, s_q, h, 512), device=dev).to(torch.bfloat16)
    oo = torch.empty((b, s_q, h, 128), dtype=torch.bfloat16, device=dev)
    us_a = timed(lambda: mla.absorb_q(qn, qr, wuk, qa))
    us_u = timed(lambda: mla.unabsorb_o(ol, wuv, oo))
    wbytes = h * 512 * 128 * 2
    out["absorb_q"] = {"us": round(us_a, 2), "weight_bytes": wbytes, "GB/s": round(wbytes / us_a / 1e3, 1),
                       "bound": "launch / HBM (weights)"}
    out["unabsorb_o"] = {"us": round(us_u, 2), "weight_bytes": wbytes, "GB/s": round(wbytes / us_u / 1e3, 1),
                         "bound": "launch / HBM (weights)"}
    # GQA path of GQLA on the MTP-shaped workload (one group: 16 heads, two causal query tokens,
    # L ~ U{8192..16384}), beside the absorbed path on the same lengths
    from mla_decode_attention_amd import workloads as W
    from mla_decode_attention_amd.inputs import make_case as _mk
    spec = dict(W.WORKLOADS["mtp_b16_h16_sq2_L8K-16K"])
    spec.pop("outlier_frac", None)
    spec.pop("outlier_scale", None)
    gcase = _mk("gqa_b16_sq2_L8K-16K", row_dims=320, q_dims=192, **spec)
    gq = torch.from_numpy(gcase.q.view(np.int16)).to(dev).view(torch.bfloat16)
    gc = torch.from_numpy(gcase.cache.view(np.int16)).to(dev).view(torch.bfloat16)
    gbt = torch.from_numpy(gcase.block_table).to(dev)
    gsl = torch.from_numpy(gcase.seqlens).to(dev)
    gws = torch.empty(mla.gqa_workspace_size(gcase.batch, 2, 16), dtype=torch.uint8, device=dev)
    go = torch.empty((gcase.batch, 2, 16, 128), dtype=torch.bfloat16, device=dev)
    gl = torch.empty((gcase.batch, 2, 16), dtype=torch.float32, device=dev)
    mla.gqa_plan(gsl, 2, 16, gws)
    us_g = timed(lambda: mla.gqa_fwd(gq, gc, gbt, gsl, gcase.softmax_scale, True, gws, go, gl))
    gbytes = int(gcase.seqlens.astype(np.int64).sum()) * 640 + gcase.batch * 2 * 16 * 192 * 2
    grec = {"us": round(us_g, 2), "bytes": gbytes, "GB/s": round(gbytes / us_g / 1e3, 1),
            "frac_of_hbm_peak": round(gbytes / us_g / 1e3 / HBM_PEAK_GBS, 4), "bound": "hbm",
            "config": "b16 s_q2 causal, 16 heads of one group, d_h 128, L ~ U{8192..16384}"}
    try:
        import oracle.gqa as OG
        from mla_decode_attention_amd.inputs import bf16_bits_to_f32
        og = bf16_bits_to_f32(go.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
        sel = [0, gcase.batch - 1]
        ro, rl = OG.gqa_decode(gcase.q[sel], gcase.cache, gcase.block_table[sel], gcase.seqlens[sel],
                               gcase.softmax_scale, True)
        grec["parity_sampled_sequences"] = {"sequences": 2, "o_maxabs": float(np.abs(og[sel] - ro).max())}
    except Exception as exc:
        grec["parity_sampled_sequences"] = f"skipped: {exc}"
    out["gqa_mtp_b16_sq2_L8K-16K"] = grec
    del gq, gc, gws
    mcase = W.build("mtp_b16_h16_sq2_L8K-16K")
    mq = torch.from_numpy(mcase.q.view(np.int16)).to(dev).view(torch.bfloat16)
    mc = torch.from_numpy(mcase.cache.view(np.int16)).to(dev).view(torch.bfloat16)
    mbt = torch.from_numpy(mcase.block_table).to(dev)
    msl = torch.from_numpy(mcase.seqlens).to(dev)
    mws = torch.empty(mla.workspace_size(mcase.batch, 2, 16), dtype=torch.uint8, device=dev)
    mo = torch.empty((mcase.batch, 2, 16, 512), dtype=torch.bfloat16, device=dev)
    ml_ = torch.empty((mcase.batch, 2, 16), dtype=torch.float32, device=dev)
    mla.plan(msl, 2, 16, mws)
    us_m = timed(lambda: mla.fwd(mq, mc, mbt, msl, mcase.softmax_scale, True, mws, mo, ml_))
    mbytes = int(mcase.seqlens.astype(np.int64).sum()) * 1152 + mcase.batch * 2 * 16 * 576 * 2
    out["mla_absorbed_same_lengths"] = {"us": round(us_m, 2), "bytes": mbytes, "GB/s": round(mbytes / us_m / 1e3, 1)}
    del mq, mc, mws
    # the append writes the new tokens' rows into the cache: measured after the sparse check
    lat, rope = make_append_inputs(case, seed=7)
    lat_d = torch.from_numpy(lat.view(np.int16)).to(dev).view(torch.bfloat16)
    rope_d = torch.from_numpy(rope.view(np.int16)).to(dev).view(torch.bfloat16)
    q2 = q.clone()
    us = timed(lambda: mla.cache_append_rope(lat_d, rope_d, q2, cache, bt, sl))
    nbytes = b * s_q * (512 * 2 + 64 * 2 + 576 * 2) + b * s_q * h * 64 * 2 * 2
    out["append_rope"] = {"us": round(us, 2), "bytes": nbytes, "GB/s": round(nbytes / us / 1e3, 1),
                          "bound": "launch", "tokens": b * s_q}

    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline long-context one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=16)
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (default: min(16, usable cores))")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum timed oracle work")
    ap.add_argument("--no-extras", action="store_true", help="skip the timings of the other entry points (extras)")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="also time each step alone after overwriting this many MiB of scratch memory, so the "
                         "cache is read from HBM and not from the last-level cache (256 MB on MI355X)")
    ap.add_argument("--flush-kind", choices=("write", "read"), default="write",
                    help="how --flush-mib evicts the cache: overwrite the scratch (leaves dirty lines) or read it")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this size (for scaling PMC byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import mla_decode_attention_amd as mla
    from mla_decode_attention_amd import workloads as W
    from mla_decode_attention_amd.inputs import bf16_bits_to_f32

    name = args.workload or W.HEADLINE
    if not os.path.exists(mla.LIB_PATH):
        from mla_decode_attention_amd import build as hip_build
        hip_build.build()
    mla.lib()
    dev = torch.device("cuda:0")
    log(f"workload {name}: generating inputs")
    case = W.build(name)
    q = torch.from_numpy(case.q.view(np.int16)).to(dev).view(torch.bfloat16)
    cache = torch.from_numpy(case.cache.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(case.block_table).to(dev)
    sl = torch.from_numpy(case.seqlens).to(dev)
    b, s_q, h = case.batch, case.s_q, case.heads
    ws = torch.empty(mla.workspace_size(b, s_q, h), dtype=torch.uint8, device=dev)
    out = torch.empty((b, s_q, h, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((b, s_q, h), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    log(f"inputs on device: cache {cache.numel() * 2 / 1e9:.3f} GB, workspace {ws.numel() / 1e6:.1f} MB")

    # plan (once per decode step for every layer): timed on its own
    # Every timed loop below replays the C-ABI calls the binding makes (see c_calls).
    torch.cuda.synchronize()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    plan_c = c_calls(mla, lambda: mla.plan(sl, s_q, h, ws))
    p0.record(stream)
    for _ in range(10):
        plan_c()
    p1.record(stream)
    torch.cuda.synchronize()
    plan_us = p0.elapsed_time(p1) * 1e3 / 10

    split_c = c_calls(mla, lambda: mla.fwd_split(q, cache, bt, sl, case.softmax_scale, case.causal, ws))
    combine_c = c_calls(mla, lambda: mla.fwd_combine(sl, bt.shape[1], s_q, h, ws, out, lse))

    def step():
        split_c()
        combine_c()

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(K):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / K

    # Dominant-kernel duration: the same K steps again, with events on the launch stream
    # bracketing every split-kernel launch.
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    for k in range(K):
        ev_a[k].record(stream)
        split_c()
        ev_b[k].record(stream)
        combine_c()
    torch.cuda.synchronize()
    split_ms = [ev_a[k].elapsed_time(ev_b[k]) for k in range(K)]
    split_avg_ms = float(np.mean(split_ms))
    log(f"step {ms_per_step * 1e3:.1f} us (split kernel {split_avg_ms * 1e3:.1f} us avg, "
        f"median {np.median(split_ms) * 1e3:.1f} us), plan {plan_us:.1f} us")

    # context: a plain device-to-device copy of 1 GiB (torch's copy kernel), the streaming rate a
    # simple kernel gets on this GPU (read + write bytes per second)
    src = torch.empty(256 << 20, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 4 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    log(f"device copy probe: {copy_gbs:.0f} GB/s (read + write)")
    read_gbs = read_probe_gbs(dev, stream)
    if read_gbs is not None:
        log(f"streaming-read probe: {read_gbs:.0f} GB/s")

    flushed = None
    if args.flush_mib > 0:
        # each step alone, after flush_mib MiB went through the cache (outside the timed region)
        scratch = torch.empty(args.flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        f_step, f_split = flushed_medians(scratch, args.flush_kind, K, split_c, combine_c, stream)
        del scratch
        flushed = {"flush_mib": args.flush_mib, "flush_kind": args.flush_kind, "steps": K, "median_us_per_step": round(f_step * 1e3, 2),
                   "median_split_us": round(f_split * 1e3, 2)}
        log(f"flushed: step median {f_step * 1e3:.1f} us, split median {f_split * 1e3:.1f} us")

    step_bytes = W.algorithmic_bytes(case.seqlens, b, s_q, h)
    step_flops = W.algorithmic_flops(case.seqlens, s_q, h, case.causal)
    kv_q_bytes = int(case.seqlens.astype(np.int64).sum()) * W.ROW_BYTES + b * s_q * h * 576 * 2
    tbs = step_bytes / (ms_per_step * 1e-3) / 1e12
    split_gbs = kv_q_bytes / (split_avg_ms * 1e-3) / 1e9
    mfma_util = step_flops / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS
    split_flops = step_flops   # every FLOP of the step is in the split kernel
    split_name = "split_kernel" if s_q * h <= 16 else "split_sv_kernel"
    if flushed is not None:
        flushed["TB/s"] = round(step_bytes / (flushed["median_us_per_step"] * 1e-6) / 1e12, 4)
        flushed["split_GB/s"] = round(kv_q_bytes / (flushed["median_split_us"] * 1e-6) / 1e9, 1)

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.calib_copy_mib} MiB done")
        del src, dst

    o_gpu = bf16_bits_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    lse_gpu = lse.cpu().numpy().astype(np.float64)

    extras = None
    if not args.no_extras:
        log("extras: sparse top-k, absorption, GQA path, cache append")
        try:
            extras = measure_extras(mla, case, dev, q, cache, bt, sl, K)
        except Exception as exc:   # the headline line stands without them
            extras = {"error": f"{type(exc).__name__}: {exc}"}
        log(f"extras: {extras}")
        # the other configured workloads, timed the same way
        wl = {}
        for other, prow in (("paged_b16_h16_L4096", 16), ("mtp_b16_h16_sq2_L8K-16K", 32),
                            ("allheads_b8_h128_L32768", 128)):
            if other == name:
                continue
            log(f"extras: workload {other}")
            try:
                wl[other] = measure_workload(mla, other, dev, K, args.warmup, prow)
            except Exception as exc:
                wl[other] = {"error": f"{type(exc).__name__}: {exc}"}
            log(f"extras: {other}: {wl[other]}")
        extras["workloads"] = wl

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        try:
            usable = len(os.sched_getaffinity(0))
        except AttributeError:
            usable = os.cpu_count() or 1
        threads = args.cpu_threads or min(16, usable)
        log(f"cpu baseline: fp64 oracle on {threads} threads, {args.cpu_sample_seqs} sequences")
        try:
            cpu, parity = cpu_baseline(case, o_gpu, lse_gpu, args.cpu_sample_seqs, threads, args.cpu_seconds)
            log(f"cpu baseline {cpu['seconds']:.1f} s -> {cpu['value']:.3e} TB/s; parity {parity}")
        except Exception as exc:   # reported in the line instead of losing it
            cpu = {"error": f"{type(exc).__name__}: {exc}", "kind": "oracle"}
            log(f"cpu baseline failed: {cpu['error']}")

    line = {
        "metric": "MLA decode achieved HBM TB/s (% of peak) + us/step, b16 h16 64K ctx",
        "value": round(tbs, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100 * tbs * 1e3 / HBM_PEAK_GBS, 2),
        "mfma_util": round(mfma_util, 4),
        "plan_us": round(plan_us, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 latent cache and queries; no model weights)",
        "config": {"workload": name, "batch": b, "s_q": s_q, "heads": h,
                   "context": int(case.seqlens.max()), "page_size": 64, "d_k": 576, "d_v": 512,
                   "causal": bool(case.causal), "algorithmic_bytes": step_bytes, "algorithmic_flops": step_flops},
        "roofline": {"bound": "hbm", "kernel": split_name, "achieved": round(split_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(split_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(name), "avg_launch_us": round(split_avg_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": kv_q_bytes,
                     "mfma_frac": round(split_flops / (split_avg_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "median_launch_us": round(float(np.median(split_ms)) * 1e3, 2),
                     "copy_probe_GB/s": round(copy_gbs, 1), "frac_of_copy_probe": round(split_gbs / copy_gbs, 4),
                     "read_probe_GB/s": None if read_gbs is None else round(read_gbs, 1),
                     "frac_of_read_probe": None if read_gbs is None else round(split_gbs / read_gbs, 4)},
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
        "extras": extras,
    }
    if flushed is not None:
        line["flushed"] = flushed
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
