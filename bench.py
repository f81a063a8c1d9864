"""Benchmark of absorbed-MQA MLA decode on one MI355X (gfx950).

One step = one mla_decode_partial call over the whole batch: the device
planner, the split-KV decode kernel (paged latent KV streamed HBM -> LDS,
QK^T and PV on MFMA, online softmax) and the split combine.  Inputs are
synthetic and already resident in HBM when the timed region starts; the cache
rotates over several copies so that repeated steps do not re-read it from the
256 MB Infinity Cache.

Headline workload (default): the long-context, low-concurrency decode (batch
4, q_len 2 causal, 128 heads, 576/512 latent dims, seq_len 131072, bf16,
64-token pages, automatic split-KV).  The same JSON line carries keyed
sub-records for the fp8-cache decode (batch 128, ragged 1k-16k), one DCP
rank's share (batch 32, 512 heads, 8192 local tokens, plus the merge of its 4
shard partials), the DeepSeek-V3-shape decode (batch 64, 128 heads, 4096) and
the long-context decode at 256 and 64 splits per sequence.  Each record has
its decode kernel's roofline (median of >= 50 event-timed launches, separate
from the timed steps) and the fp64 oracle timed on the host's cores.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config c5] [--num-splits 0]
                    [--no-sub-records] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA decode KV-cache GB/s + TFLOP/s (fraction of MI355X HBM/MFMA roofline)"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
FLOP_PER_ROW_TOKEN = 2 * (576 + 512)
KERNEL_SRC = os.path.join(ROOT, "mla_latent_decode_absorbed_amd", "csrc", "mla_kernels.hip")
# rocprofv3 counter summaries (HBM traffic, MFMA/LDS utilisation) of the decode
# kernel on a workload, used while the kernel sources hash to the profiled ones
PMC_FILES = {"c2": os.path.join(ROOT, "profiles", "decode_kernel_c2_pmc.json"),
             "c3": os.path.join(ROOT, "profiles", "decode_kernel_c3_pmc.json"),
             "c4": os.path.join(ROOT, "profiles", "decode_fp8_kernel_c4_pmc.json"),
             "c5": os.path.join(ROOT, "profiles", "decode_kernel_c5_pmc.json")}

WORKLOAD_NAMES = {
    "c2": "DeepSeek-V3-shape decode on one unsharded cache: batch 64, q_len 1, 128 heads, "
          "576 (512 latent + 64 rope) per token, seq_len 4096, bf16 cache, 64-token pages",
    "c3": "one DCP rank's share: batch 32, q_len 1, 512 heads (128 x 4), 8192 local tokens of "
          "32768, bf16 cache, 64-token pages",
    "c4": "fp8 e4m3 cache: batch 128, q_len 1, 128 heads, seq_len uniform in [1024, 16384]",
    "c5": "long context: batch 4, q_len 2 (causal), 128 heads, seq_len 131072, bf16 cache",
}


class HipEvents:
    """hipEvent_t pairs from the HIP runtime (the library records them on the stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        ev = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev: int) -> None:
        self.hip.hipEventDestroy(ctypes.c_void_p(ev))


def kernel_source_hash() -> str:
    """sha256 (16 hex) of the kernel sources (every kernel and the shared
    header): the stored counter file is used only while this matches."""
    h = hashlib.sha256()
    for path in (KERNEL_SRC, os.path.join(os.path.dirname(KERNEL_SRC), "mla_internal.h")):
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def workload_accounting(inp) -> dict:
    """Algorithmic bytes and flops of one step (valid tokens only)."""
    import numpy as np
    sl = inp.seq_lens.cpu().numpy().astype(np.int64)
    B, T, H = inp.batch, inp.q_len, inp.heads
    e = 2 if inp.dtype == "bf16" else 1
    tokens = int(sl.sum())
    if inp.causal and T > 1:
        vis = sum(max(int(n) - (T - 1 - t), 0) for n in sl for t in range(T))
    else:
        vis = tokens * T
    rows = B * T * H
    kv_bytes = tokens * 576 * e
    q_bytes = rows * 576 * e
    bt_bytes = int(((sl + 63) // 64).sum()) * 4 + B * 4
    out_bytes = rows * 512 * 4 + rows * 4
    flops = vis * H * FLOP_PER_ROW_TOKEN
    return dict(kv_bytes=kv_bytes, q_bytes=q_bytes, bt_bytes=bt_bytes, out_bytes=out_bytes,
                flops=flops, rows=rows, tokens=tokens)


def oracle_threads() -> int:
    """Threads the oracle's BLAS runs on (threadpoolctl's view), else the host's CPUs."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [os.cpu_count()]))
    except Exception:
        return int(os.cpu_count() or 1)


def cpu_baseline(inp, budget_s: float = 20.0) -> dict:
    """The fp64 oracle on this host's cores over whole requests of the same workload
    (as many as fit a ~budget_s time box, at least one)."""
    import numpy as np
    import torch
    from oracle import bf16_bits_to_f64, decode_partial_ref, e4m3_bits_to_f64
    bt_all = inp.block_table.cpu().numpy()
    sl_all = inp.seq_lens.cpu().numpy()
    dec = bf16_bits_to_f64 if inp.dtype == "bf16" else e4m3_bits_to_f64
    view = (lambda x: x.view(torch.int16)) if inp.dtype == "bf16" else (lambda x: x)
    done_bytes, done_flops, done_req, spent = 0, 0, 0, 0.0
    e = 2 if inp.dtype == "bf16" else 1
    T = inp.q_len
    for b in range(inp.batch):
        n = int(sl_all[b])
        pages = bt_all[b][: (n + 63) // 64]
        kv_host = view(inp.kv_cache[torch.as_tensor(pages, dtype=torch.long, device=inp.kv_cache.device)]).cpu().numpy()
        q_host = view(inp.q[b:b + 1]).cpu().numpy()
        t0 = time.perf_counter()
        q64 = dec(q_host)
        kv64 = dec(kv_host)
        decode_partial_ref(q64, kv64, np.arange(len(pages))[None, :], np.array([n]), inp.scale,
                           kv_scale=inp.kv_scale_value, causal=inp.causal)
        spent += time.perf_counter() - t0
        done_bytes += n * 576 * e
        vis = sum(max(n - (T - 1 - t), 0) for t in range(T)) if inp.causal and T > 1 else n * T
        done_flops += vis * inp.heads * FLOP_PER_ROW_TOKEN
        done_req += 1
        if spent >= budget_s:
            break
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s",
            "tflops": round(done_flops / spent / 1e12, 5), "cores": oracle_threads(), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{done_req} of {inp.batch} requests (whole requests, all heads), "
                      f"{done_bytes / 1e6:.1f} MB of KV, {spent:.2f} s of fp64 numpy on the host"}


def bench_query_prep(args) -> int:
    """mla_query_prep (W_UK_T absorption + rope concat, bf16 or e4m3 storage) on
    the query rows and heads of a decode workload, P = 128.  The weights rotate
    over copies totalling more than the 256 MB Infinity Cache (one layer's
    weights are read once per decode step).  Prints ONE JSON line."""
    import torch
    import mla_latent_decode_absorbed_amd as mla
    import workloads

    dev = torch.device("cuda:0")
    c = workloads.QPREP_CONFIGS[args.config]
    R, H, P = c["rows"], c["heads"], 128
    fp8 = args.config == "c4"
    inp = workloads.make_query_prep_inputs(R, H, P, seed=args.seed or 0, device=dev, fp8=fp8)
    w_bytes = inp.w_uk.numel() * 2
    n_w = max(2, -(-(300 << 20) // w_bytes))
    ws = [inp.w_uk] + [inp.w_uk.clone() for _ in range(n_w - 1)]
    out = torch.empty((R, H, 576), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
    e = 1 if fp8 else 2
    alg = w_bytes + R * H * P * 2 + R * H * 64 * 2 + R * H * 576 * e + (4 if fp8 else 0)
    flops = 2 * R * H * P * 512
    torch.cuda.synchronize()

    # checked once through the binding, then called with pre-built arguments so
    # that the loop times the GPU, not the per-call argument marshalling
    mla.query_prep(inp.q_nope, inp.q_pe, inp.w_uk, out, q_scale=inp.q_scale)
    desc = mla.QueryPrepDesc(R, H, P, mla.FP8_E4M3 if fp8 else mla.BF16)
    stream = torch.cuda.current_stream().cuda_stream
    call = mla.lib.mla_query_prep
    qs_ptr = inp.q_scale.data_ptr() if fp8 else None
    args_of = [(ctypes.byref(desc), inp.q_nope.data_ptr(), inp.q_pe.data_ptr(), w.data_ptr(), qs_ptr,
                out.data_ptr(), stream) for w in ws]

    def step(i):
        if call(*args_of[i % n_w]) != mla.OK:
            raise RuntimeError("mla_query_prep failed")

    ms, kern_ms, n_warm = _time_launches(step, args)
    achieved = alg / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": "MLA query preparation GB/s (fraction of MI355X HBM roofline)",
        "value": round(alg / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": n_warm,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) query, N(0,1/P) W_UK_T, bf16)",
        "config": {"workload": f"{args.config} query rows and heads: rows {R}, heads {H}, P {P}, "
                               f"out {'e4m3 (q_scale 1/64)' if fp8 else 'bf16'}",
                   "rows": R, "heads": H, "nope_dim": P, "weight_copies_rotated": n_w},
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel_ms": round(kern_ms, 5),
                     "algorithmic_bytes_per_launch": alg},
    }
    if not args.no_cpu_baseline:
        import numpy as np
        from oracle import bf16_bits_to_f64, query_prep_ref
        f64 = lambda t: bf16_bits_to_f64(t.view(torch.int16).cpu().numpy())
        qn, qp, w = f64(inp.q_nope), f64(inp.q_pe), f64(inp.w_uk)
        done, spent = 0, 0.0
        while done < R and spent < 20.0:
            t = time.perf_counter()
            query_prep_ref(qn[done:done + 1], qp[done:done + 1], w)
            spent += time.perf_counter() - t
            done += 1
        per_row = (H * P * 2 + H * 64 * 2 + H * 576 * e)
        res["cpu_baseline"] = {"value": round((w_bytes * done / R + per_row * done) / spent / 1e9, 4),
                               "unit": "GB/s", "cores": oracle_threads(), "cpu_model": cpu_model(), "kind": "oracle",
                               "sample": f"{done} of {R} rows (all heads), {spent:.2f} s of fp64 numpy"}
    print(json.dumps(res), flush=True)
    return 0


def _time_launches(step, args):
    """Warm-up (at least W calls and --warmup-seconds), then K calls timed by
    the wall clock between synchronisations, then a separate loop of
    --event-launches (>= 50) calls each bracketed by torch events on the
    current stream; returns (ms per call by the wall clock, median event-timed
    ms, warm-up calls run)."""
    import torch
    step(0)
    torch.cuda.synchronize()
    n_warm, t_w = 1, time.perf_counter()
    while n_warm < args.warmup or time.perf_counter() - t_w < args.warmup_seconds:
        step(n_warm)
        n_warm += 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_ev = max(args.event_launches, 50)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    for i, (a, b) in enumerate(evs):
        a.record()
        step(i)
        b.record()
    torch.cuda.synchronize()
    return wall * 1e3 / args.steps, median([a.elapsed_time(b) for a, b in evs]), n_warm


def bench_up_project(args) -> int:
    """mla_up_project (latent output through W_UV, v_head_dim 128) on the rows
    and heads of a decode workload: fp32 latent input, bf16 output.  The
    weights rotate over copies totalling more than the 256 MB Infinity Cache.
    Prints ONE JSON line."""
    import torch
    import mla_latent_decode_absorbed_amd as mla
    import workloads

    dev = torch.device("cuda:0")
    c = workloads.QPREP_CONFIGS[args.config]
    R, H, Vd = c["rows"], c["heads"], 128
    inp = workloads.make_up_project_inputs(R, H, Vd, seed=args.seed or 0, device=dev)
    w_bytes = inp.w_uv.numel() * 2
    n_w = max(2, -(-(300 << 20) // w_bytes))
    ws = [inp.w_uv] + [inp.w_uv.clone() for _ in range(n_w - 1)]
    out = torch.empty((R, H, Vd), dtype=torch.bfloat16, device=dev)
    alg = w_bytes + R * H * 512 * 4 + R * H * Vd * 2
    flops = 2 * R * H * 512 * Vd
    mla.up_project(inp.o_lat, inp.w_uv, out)           # checked once through the binding
    desc = mla.UpProjectDesc(R, H, Vd, mla.F32, mla.BF16)
    stream = torch.cuda.current_stream().cuda_stream
    call = mla.lib.mla_up_project
    args_of = [(ctypes.byref(desc), inp.o_lat.data_ptr(), w.data_ptr(), out.data_ptr(), stream) for w in ws]

    def step(i):
        if call(*args_of[i % n_w]) != mla.OK:
            raise RuntimeError("mla_up_project failed")

    ms, kern_ms, n_warm = _time_launches(step, args)
    achieved = alg / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": "MLA output up-projection GB/s (fraction of MI355X HBM roofline)",
        "value": round(alg / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": n_warm,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) fp32 latent output, N(0,1/512) W_UV, bf16)",
        "config": {"workload": f"{args.config} rows and heads: rows {R}, heads {H}, v_head_dim {Vd}, "
                               "fp32 in, bf16 out",
                   "rows": R, "heads": H, "v_head_dim": Vd, "weight_copies_rotated": n_w},
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel_ms": round(kern_ms, 5),
                     "algorithmic_bytes_per_launch": alg},
    }
    if not args.no_cpu_baseline:
        from oracle import bf16_bits_to_f64, up_project_ref
        x = inp.o_lat.double().cpu().numpy()
        w = bf16_bits_to_f64(inp.w_uv.view(torch.int16).cpu().numpy())
        done, spent = 0, 0.0
        while done < R and spent < 20.0:
            t = time.perf_counter()
            up_project_ref(x[done:done + 1], w)
            spent += time.perf_counter() - t
            done += 1
        per_row = H * 512 * 4 + H * Vd * 2
        res["cpu_baseline"] = {"value": round((w_bytes * done / R + per_row * done) / spent / 1e9, 4),
                               "unit": "GB/s", "cores": oracle_threads(), "cpu_model": cpu_model(), "kind": "oracle",
                               "sample": f"{done} of {R} rows (all heads), {spent:.2f} s of fp64 numpy"}
    print(json.dumps(res), flush=True)
    return 0


def bench_gather(args) -> int:
    """mla_gather_cache of each request's first min(seq_len, 2048) cache tokens
    (a chunked-prefill context chunk) out of the workload's paged cache into a
    contiguous bf16 buffer (e4m3 caches dequantised).  Prints ONE JSON line."""
    import numpy as np
    import torch
    import mla_latent_decode_absorbed_amd as mla
    import workloads

    dev = torch.device("cuda:0")
    kw = dict(shard_only=0) if args.config == "c3" else {}
    inp = workloads.make_config(args.config, seed=args.seed, device=dev, poison=False, extra_pages=0, **kw)
    sl = inp.seq_lens.cpu().numpy()
    lens = np.minimum(sl, 2048).astype(np.int32)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
    starts = torch.zeros(len(sl), dtype=torch.int32, device=dev)
    total = int(lens.sum())
    out = torch.empty((total, 576), dtype=torch.bfloat16, device=dev)
    e = 2 if inp.dtype == "bf16" else 1
    alg = total * 576 * (e + 2) + int(((lens + 63) // 64).sum()) * 4 + (2 * len(sl) + 1) * 4
    copies = [inp.kv_cache] + [inp.kv_cache.clone() for _ in range(max(args.copies, 1) - 1)]
    mla.gather_cache(inp.kv_cache, inp.block_table, starts, cu, total, out, kv_scale=inp.kv_scale)
    call = mla.lib.mla_gather_cache
    stream = torch.cuda.current_stream().cuda_stream
    kvs = inp.kv_scale.data_ptr() if inp.kv_scale is not None else None
    dt = mla.BF16 if inp.dtype == "bf16" else mla.FP8_E4M3
    B, maxp = inp.block_table.shape
    args_of = [(c.data_ptr(), dt, kvs, inp.block_table.data_ptr(), B, c.shape[0], maxp, starts.data_ptr(),
                cu.data_ptr(), ctypes.c_int64(total), out.data_ptr(), stream) for c in copies]

    def step(i):
        if call(*args_of[i % len(copies)]) != mla.OK:
            raise RuntimeError("mla_gather_cache failed")

    ms, kern_ms, n_warm = _time_launches(step, args)
    achieved = alg / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": "MLA context gather GB/s (fraction of MI355X HBM roofline)",
        "value": round(alg / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": n_warm,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": inp.dtype, "data": "synthetic (seeded N(0,1) latent cache, shuffled 64-token pages)",
        "config": {"workload": f"{args.config}: first min(seq_len, 2048) tokens of each of {B} requests "
                               f"({total} rows) out of the {inp.dtype} paged cache into bf16",
                   "rows": total, "cache_copies_rotated": len(copies)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel_ms": round(kern_ms, 5),
                     "algorithmic_bytes_per_launch": alg},
    }
    if not args.no_cpu_baseline:
        from oracle import gather_cache_ref
        cache = inp.kv_cache.cpu()
        cache = cache.view(torch.int16).numpy().view(np.uint16) if inp.dtype == "bf16" else cache.numpy()
        bt = inp.block_table.cpu().numpy()
        st = np.zeros(len(sl), dtype=np.int64)
        done, spent, rows_done = 0, 0.0, 0
        while done < B and spent < 20.0:
            t = time.perf_counter()
            gather_cache_ref(cache, bt[done:done + 1], st[done:done + 1], lens[done:done + 1], inp.dtype,
                             inp.kv_scale_value)
            spent += time.perf_counter() - t
            rows_done += int(lens[done])
            done += 1
        res["cpu_baseline"] = {"value": round(rows_done * 576 * (e + 2) / spent / 1e9, 4), "unit": "GB/s",
                               "cores": int(os.cpu_count() or 1), "kind": "oracle",
                               "sample": f"{done} of {B} requests ({rows_done} rows), {spent:.2f} s of numpy"}
    print(json.dumps(res), flush=True)
    return 0


def probe_peaks() -> int:
    """Achievable figures of this GPU next to the published peaks the rooflines
    use: a 4 GiB device-to-device copy (HBM read + write), a 4 GiB reduction
    (HBM read), and 8192^3 dense GEMMs in bf16 and (when torch offers it) fp8
    through hipBLASLt."""
    import torch

    dev = torch.device("cuda:0")

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    res = {"probe": "achievable peaks", "published": {"hbm_gbs": HBM_PEAK_GBS, "mfma_tflops": MFMA_PEAK_TFLOPS}}
    src = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src), 10)
    res["hbm_copy_gbs"] = round(2 * src.numel() / t / 1e9, 1)        # bytes read + written
    del dst
    f = src.view(torch.float32)
    t = timed(lambda: f.sum(), 10)
    res["hbm_read_gbs"] = round(src.numel() / t / 1e9, 1)              # a 4 GiB reduction: reads only
    del src, f
    n = 8192
    a = torch.randn((n, n), device=dev).to(torch.bfloat16)
    b = torch.randn((n, n), device=dev).to(torch.bfloat16)
    t = timed(lambda: torch.mm(a, b), 20)
    res["bf16_gemm_tflops"] = round(2 * n ** 3 / t / 1e12, 1)
    try:
        a8, b8 = a.to(torch.float8_e4m3fn), b.t().contiguous().to(torch.float8_e4m3fn).t()
        one = torch.ones((), device=dev)
        t = timed(lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one, out_dtype=torch.bfloat16), 20)
        res["fp8_gemm_tflops"] = round(2 * n ** 3 / t / 1e12, 1)
    except Exception as exc:                                              # not offered by this torch build
        res["fp8_gemm_tflops"] = None
        res["fp8_note"] = f"torch._scaled_mm unavailable: {type(exc).__name__}"
    print(json.dumps(res), flush=True)
    return 0


def bench_merge_up_project(args) -> int:
    """mla_merge_up_project on one DCP rank's shape: 4 shard partials of 32
    tokens x 512 heads (fp32 [4][16384][512] + LSEs) merged and mapped through
    W_UV (v_head_dim 128, bf16 out), against mla_merge_states followed by
    mla_up_project on the same inputs.  Prints ONE JSON line."""
    import torch
    import mla_latent_decode_absorbed_amd as mla
    import workloads

    dev = torch.device("cuda:0")
    n, R, H, Vd = 4, 32, 512, 128
    g = torch.Generator(device=dev).manual_seed(args.seed or 3)
    outs = torch.randn((n, R, H, 512), generator=g, device=dev)
    lses = torch.randn((n, R, H), generator=g, device=dev)
    w = workloads.make_up_project_inputs(1, H, Vd, seed=args.seed or 3, device=dev).w_uv
    ws = [w] + [w.clone() for _ in range(4)]                   # 5 x 67 MB of weights rotated
    out = torch.empty((R, H, Vd), dtype=torch.bfloat16, device=dev)
    merged = torch.empty((R * H, 512), dtype=torch.float32, device=dev)
    mlse = torch.empty(R * H, dtype=torch.float32, device=dev)
    alg = n * R * H * (512 * 4 + 4) + H * Vd * 512 * 2 + R * H * Vd * 2
    mla.merge_up_project(outs, lses, n, w, out)                 # checked once through the binding
    desc = mla.UpProjectDesc(R, H, Vd, mla.F32, mla.BF16)
    stream = torch.cuda.current_stream().cuda_stream
    fused_args = [(outs.data_ptr(), lses.data_ptr(), n, ctypes.byref(desc), x.data_ptr(), out.data_ptr(), None,
                   stream) for x in ws]

    def fused(i):
        if mla.lib.mla_merge_up_project(*fused_args[i % len(ws)]) != mla.OK:
            raise RuntimeError("mla_merge_up_project failed")

    def unfused(i):
        mla.merge_states(outs.view(n, R * H, 512), lses.view(n, R * H), n, R * H, merged, mlse)
        mla.up_project(merged.view(R, H, 512), ws[i % len(ws)], out)

    ms, kern_ms, n_warm = _time_launches(fused, args)
    ms_u, kern_u, _ = _time_launches(unfused, args)
    achieved = alg / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": "MLA DCP merge + W_UV up-projection GB/s (fraction of MI355X HBM roofline)",
        "value": round(alg / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": n_warm,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) fp32 partials and LSEs, N(0,1/512) W_UV, bf16)",
        "config": {"workload": f"one DCP rank's merge: {n} shard partials of {R} tokens x {H} heads, "
                               f"v_head_dim {Vd}, bf16 out", "partials": n, "rows": R, "heads": H,
                   "v_head_dim": Vd, "weight_copies_rotated": len(ws)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel_ms": round(kern_ms, 5),
                     "algorithmic_bytes_per_launch": alg},
        "unfused": {"what": "mla_merge_states then mla_up_project (the merged latent through HBM)",
                    "ms_events": round(kern_u, 5), "ms_per_step": round(ms_u, 5)},
    }
    if not args.no_cpu_baseline:
        import numpy as np
        from oracle import bf16_bits_to_f64, merge_ref, up_project_ref
        o64 = outs.double().cpu().numpy().reshape(n, R * H, 512)
        l64 = lses.double().cpu().numpy().reshape(n, R * H)
        w64 = bf16_bits_to_f64(w.view(torch.int16).cpu().numpy())
        done, spent = 0, 0.0
        while done < R and spent < 20.0:
            t = time.perf_counter()
            om, _ = merge_ref(o64[:, done * H:(done + 1) * H], l64[:, done * H:(done + 1) * H])
            up_project_ref(om.reshape(1, H, 512), w64)
            spent += time.perf_counter() - t
            done += 1
        per_row = H * (n * (512 * 4 + 4) + Vd * 2)
        res["cpu_baseline"] = {"value": round((H * Vd * 512 * 2 * done / R + per_row * done) / spent / 1e9, 4),
                               "unit": "GB/s", "cores": oracle_threads(), "cpu_model": cpu_model(), "kind": "oracle",
                               "sample": f"{done} of {R} tokens (all heads), {spent:.2f} s of fp64 numpy"}
    print(json.dumps(res), flush=True)
    return 0


def cpu_model() -> str | None:
    """The host CPU's model name (first /proc/cpuinfo entry), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def make_workload(name: str, seed, dev):
    import workloads
    kw = dict(shard_only=0) if name == "c3" else {}
    return workloads.make_config(name, seed=seed, device=dev, poison=False, extra_pages=0, **kw)


def decode_roofline(acc, dtype: str, kern_ms: float) -> dict:
    """The decode kernel's roofline: the binding roof of the workload's
    arithmetic intensity (FLOP per byte of KV + q against the peaks' ratio),
    the algorithmic bytes or flops per launch over the kernel's time."""
    peak_tf = MFMA_PEAK_TFLOPS[dtype]
    ai = acc["flops"] / (acc["kv_bytes"] + acc["q_bytes"])
    k_bytes = acc["kv_bytes"] + acc["q_bytes"] + acc["bt_bytes"]
    if ai < peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9):
        achieved = k_bytes / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = acc["flops"] / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(achieved / peak_tf, 4)}
    roof["kernel_ms"] = round(kern_ms, 5)
    roof["algorithmic_bytes_per_launch"] = k_bytes
    roof["algorithmic_flops_per_launch"] = acc["flops"]
    return roof


def stored_counters(name: str, num_splits: int, seed) -> tuple:
    """(HBM bytes per launch, utilisation counters) of the decode kernel on a
    workload from its rocprofv3 summary, while the kernel sources hash to the
    profiled ones; (None, None) otherwise."""
    pmc_file = PMC_FILES.get(name)
    if not pmc_file or not os.path.exists(pmc_file) or num_splits != 0 or seed is not None:
        return None, None
    pmc = json.load(open(pmc_file))
    if pmc.get("kernel_source_sha256_16") != kernel_source_hash():
        return None, None
    return pmc.get("hbm_bytes_per_launch"), {k: pmc.get(k) for k in (
        "MfmaUtil_percent", "LdsUtil_percent", "LdsBankConflict_per_access", "mfma_flops_per_launch")}


def decode_record(name: str, inp, args, hev, num_splits: int, steps: int, cpu_budget: float) -> dict:
    """One workload through mla_decode_partial: warm-up, `steps` whole steps
    timed by the wall clock between synchronisations, then a separate loop of
    `--event-launches` calls whose decode kernel is bracketed by HIP events on
    the stream it runs on (median duration).  Inputs are resident in HBM; the
    cache rotates over `--copies` copies."""
    import torch
    import mla_latent_decode_absorbed_amd as mla

    dev = inp.q.device
    acc = workload_accounting(inp)
    desc = mla.make_desc(inp.batch, inp.q_len, inp.heads, inp.kv_cache.shape[0], inp.block_table.shape[1],
                         kv_dtype=mla.BF16 if inp.dtype == "bf16" else mla.FP8_E4M3,
                         causal=1 if inp.causal else 0, num_splits=num_splits)
    dec = mla.Decoder(desc, device=dev)
    copies = [inp.kv_cache] + [inp.kv_cache.clone() for _ in range(max(args.copies, 1) - 1)]
    out = torch.empty((inp.batch, inp.q_len, inp.heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((inp.batch, inp.q_len, inp.heads), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, events=None):
        dec(inp.q, copies[i % len(copies)], inp.block_table, inp.seq_lens, inp.scale,
            kv_scale=inp.kv_scale, out=out, lse=lse, stream=stream, events=events)

    # warm-up: at least W steps and at least --warmup-seconds of back-to-back
    # work (the first call, module load and first touch, excluded), so that
    # clocks have settled before the timed region
    step(0)
    torch.cuda.synchronize()
    n_warm, t_w = 1, time.perf_counter()
    while n_warm < args.warmup or time.perf_counter() - t_w < args.warmup_seconds:
        step(n_warm)
        n_warm += 1
        if n_warm % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / steps

    n_ev = max(args.event_launches, 50)
    evs = [(hev.create(), hev.create()) for _ in range(n_ev)]
    for i in range(n_ev):
        step(i, events=evs[i])
    torch.cuda.synchronize()
    kern = [hev.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        hev.destroy(a)
        hev.destroy(b)
    kern_ms = median(kern)

    # pieces per request the planner chose (the workspace's first 4 B int32:
    # pieces, first piece, first page, 0); a request of more than one piece
    # goes through fp32 partials
    req_info = dec.workspace[: 16 * inp.batch].view(torch.int32).view(inp.batch, 4).cpu()
    info = req_info[:, 0]
    balanced_plan = bool((req_info[:, 2] != 0).any())
    partial_rows = int(sum(int(sp) for sp in info.tolist() if sp > 1) * inp.q_len * inp.heads)
    partial_bytes = partial_rows * (512 * 2 + 4)       # bf16 partial row + fp32 lse

    peak_tf = MFMA_PEAK_TFLOPS[inp.dtype]
    kv_gbs = acc["kv_bytes"] / (ms_per_step * 1e-3) / 1e9
    tflops = acc["flops"] / (ms_per_step * 1e-3) / 1e12
    total_gbs = (acc["kv_bytes"] + acc["q_bytes"] + acc["bt_bytes"] + acc["out_bytes"]) / (ms_per_step * 1e-3) / 1e9
    roof = decode_roofline(acc, inp.dtype, kern_ms)
    traffic, counters = stored_counters(name, num_splits, args.seed)
    roof["traffic"] = traffic
    roof["counters"] = counters
    roof["kernel_ms_min_max"] = [round(min(kern), 5), round(max(kern), 5)]
    roof["event_timed_launches"] = n_ev
    rec = {
        "workload": f"{name}: {WORKLOAD_NAMES[name]}",
        "num_splits": num_splits or "auto",
        "value": round(kv_gbs, 2), "unit": "GB/s", "steps": steps, "warmup_steps_run": n_warm,
        "ms_per_step": round(ms_per_step, 5), "dtype": inp.dtype,
        "tflops": round(tflops, 2),
        "fractions": {"hbm_kv_only": round(kv_gbs / HBM_PEAK_GBS, 4),
                      "hbm_all_algorithmic_bytes": round(total_gbs / HBM_PEAK_GBS, 4),
                      "mfma": round(tflops / peak_tf, 4),
                      "binding_roof": round(max(acc["kv_bytes"] / (HBM_PEAK_GBS * 1e9),
                                                acc["flops"] / (peak_tf * 1e12)) / (ms_per_step * 1e-3), 4)},
        "roofline": roof,
        "split_partials": {"plan": "balanced page ranges" if balanced_plan else "common chunk",
                           "splits_per_request_min_max": [int(info.min()), int(info.max())],
                           "partial_bytes_written_and_read": 2 * partial_bytes,
                           "overhead_vs_kv_bytes": round(2 * partial_bytes / acc["kv_bytes"], 4)},
        "shape": {"batch": inp.batch, "q_len": inp.q_len, "heads": inp.heads,
                  "seq_lens_total": acc["tokens"], "cache_copies_rotated": len(copies)},
    }
    if cpu_budget > 0:
        rec["cpu_baseline"] = cpu_baseline(inp, budget_s=cpu_budget)
    rec["_decoder"] = (dec, out, lse, stream, copies)
    return rec


def dcp_merge_record(args, inp0, rec0, cpu_budget: float) -> dict:
    """One DCP rank's share, 4 shards: mla_merge_states of the 4 shard partials
    (n = 4, 16,384 rows) with its own roofline (HBM: 4 x 2052 B in and 2052 B
    out per row; median of >= 50 event-timed calls), and all 4 shard decodes
    plus that merge, for information.  Shards 1-3 are built like shard 0."""
    import numpy as np
    import torch
    import mla_latent_decode_absorbed_amd as mla
    import workloads

    dev = inp0.q.device
    dec, out0, lse0, stream, _ = rec0["_decoder"]
    shards = [inp0] + [workloads.make_config("c3", seed=args.seed, device=dev, poison=False, extra_pages=0,
                                             shard_only=r) for r in (1, 2, 3)]
    rows = inp0.batch * inp0.q_len * inp0.heads
    outs = torch.empty((4, rows, 512), dtype=torch.float32, device=dev)
    lses = torch.empty((4, rows), dtype=torch.float32, device=dev)
    mo = torch.empty((rows, 512), dtype=torch.float32, device=dev)
    ml = torch.empty(rows, dtype=torch.float32, device=dev)

    def all_shards():
        for r, sh in enumerate(shards):
            dec(sh.q, sh.kv_cache, sh.block_table, sh.seq_lens, sh.scale, out=outs[r].view_as(out0),
                lse=lses[r].view_as(lse0), stream=stream)
        mla.merge_states(outs, lses, 4, rows, mo, ml, stream=stream)

    def merge_only():
        mla.merge_states(outs, lses, 4, rows, mo, ml, stream=stream)

    all_shards()
    torch.cuda.synchronize()
    for _ in range(5):
        merge_only()
    n_ev = max(args.event_launches, 50)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    for a, b in evs:
        a.record(stream)
        merge_only()
        b.record(stream)
    torch.cuda.synchronize()
    merge_ms = median([a.elapsed_time(b) for a, b in evs])
    for _ in range(2):
        all_shards()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(10):
        all_shards()
    b.record(stream)
    torch.cuda.synchronize()
    merge_bytes = 4 * rows * 2052 + rows * 2052
    achieved = merge_bytes / (merge_ms * 1e-3) / 1e9
    res = {"what": "mla_merge_states of the 4 shard partials (n = 4, 16,384 rows; 4 x 2052 B in and 2052 B "
                   "out per row); and the 4 shard decodes plus that merge",
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel_ms": round(merge_ms, 5),
                        "algorithmic_bytes_per_launch": merge_bytes, "event_timed_launches": n_ev},
           "four_shards_and_merge_ms": round(a.elapsed_time(b) / 10, 5)}
    if cpu_budget > 0:
        from oracle import merge_ref
        o64 = outs.double().cpu().numpy()
        l64 = lses.double().cpu().numpy()
        done, spent = 0, 0.0
        while done < rows and spent < cpu_budget:
            t = time.perf_counter()
            merge_ref(o64[:, done:done + 512], l64[:, done:done + 512])
            spent += time.perf_counter() - t
            done += 512
        res["cpu_baseline"] = {"value": round(done * 2052 * 5 / spent / 1e9, 4), "unit": "GB/s",
                               "cores": oracle_threads(), "cpu_model": cpu_model(), "kind": "oracle",
                               "sample": f"{done} of {rows} rows (blocks of 512), {spent:.2f} s of fp64 numpy"}
    return res


def plan_reuse_timings(args, inp, rec) -> dict:
    """The same decode with the split plan made once per step and reused by
    every layer: mla_decode_plan alone, and one layer's decode on the stored
    plan (mla_decode_partial_planned: decode + combine, no planning), each
    averaged over back-to-back launches, for information."""
    import torch
    dec, out, lse, stream, copies = rec["_decoder"]

    def plan():
        dec.plan(inp.seq_lens, stream=stream)

    def layer(i):
        dec.planned(inp.q, copies[i % len(copies)], inp.block_table, inp.seq_lens, inp.scale,
                    kv_scale=inp.kv_scale, out=out, lse=lse, stream=stream)

    res = {}
    for name, fn, reps in (("plan_ms", lambda i: plan(), 50), ("layer_decode_on_stored_plan_ms", layer, 50)):
        for i in range(5):
            fn(i)
        plan()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(reps):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        res[name] = round(a.elapsed_time(b) / reps, 5)
    return res


def bench_decode(args) -> int:
    """The headline line: mla_decode_partial on the --config workload (default:
    the long-context bf16 decode), with keyed sub-records for the fp8 cache
    decode, one DCP rank's share (plus its 4-shard merge), the DeepSeek-V3-shape
    decode and the long-context decode at 256 and 64 splits per sequence."""
    import torch

    dev = torch.device("cuda:0")
    hev = HipEvents()
    t_setup = time.perf_counter()
    inp = make_workload(args.config, args.seed, dev)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    head = decode_record(args.config, inp, args, hev, args.num_splits, args.steps,
                         0.0 if args.no_cpu_baseline else 20.0)
    res = {
        "metric": METRIC,
        "value": head["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "warmup_steps_run": head["warmup_steps_run"], "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"],
        "data": "synthetic (seeded N(0,1) query and latent cache, shuffled 64-token pages)",
        "config": {"workload": head["workload"], "batch": inp.batch, "q_len": inp.q_len, "heads": inp.heads,
                   "seq_lens_total": head["shape"]["seq_lens_total"], "num_splits": head["num_splits"],
                   "cache_copies_rotated": head["shape"]["cache_copies_rotated"]},
        "tflops": head["tflops"], "fractions": head["fractions"], "roofline": head["roofline"],
        "split_partials": head["split_partials"], "setup_s": round(setup_s, 2),
    }
    res["plan_reuse"] = plan_reuse_timings(args, inp, head)
    if "cpu_baseline" in head:
        res["cpu_baseline"] = head["cpu_baseline"]
    if args.config == "c3" and args.num_splits == 0:
        res["dcp_rank_merge"] = dcp_merge_record(args, inp, head, 0.0 if args.no_cpu_baseline else 5.0)
    del head["_decoder"]
    del inp
    torch.cuda.empty_cache()

    if not args.no_sub_records:
        subs = {}
        plan = [("c4", "c4", 0), ("c3", "c3", 0), ("c2", "c2", 0)]
        if args.config == "c5":
            plan += [("c5_splits256", "c5", 256), ("c5_splits64", "c5", 64)]
        for key, name, ns in plan:
            if name == args.config and ns == args.num_splits:
                continue
            sub_inp = make_workload(name, args.seed, dev)
            rec = decode_record(name, sub_inp, args, hev, ns, args.sub_steps,
                                0.0 if (args.no_cpu_baseline or ns) else 5.0)
            if name == "c3" and ns == 0:
                rec["dcp_rank_merge"] = dcp_merge_record(args, sub_inp, rec, 0.0 if args.no_cpu_baseline else 3.0)
            del rec["_decoder"]
            subs[key] = rec
            del sub_inp
            torch.cuda.empty_cache()
        res["sub_records"] = subs
    print(json.dumps(res), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="minimum wall time of the untimed warm-up (clocks settle)")
    ap.add_argument("--config", default="c5", choices=sorted(WORKLOAD_NAMES),
                    help="headline workload (default c5, the long-context bf16 decode)")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--copies", type=int, default=3, help="cache copies rotated over the steps")
    ap.add_argument("--event-launches", type=int, default=60,
                    help="event-timed decode launches per workload (median; at least 50)")
    ap.add_argument("--sub-steps", type=int, default=50, help="whole steps timed per sub-record")
    ap.add_argument("--no-sub-records", action="store_true",
                    help="only the headline workload (no fp8 / DCP-rank / DeepSeek-V3-shape / split records)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--probe-peaks", action="store_true",
                    help="print achievable HBM copy bandwidth and dense bf16/fp8 GEMM rates of this "
                         "GPU (torch's copy kernel and hipBLASLt) as one JSON line, and exit")
    ap.add_argument("--op", default="decode", choices=["decode", "qprep", "upproj", "gather", "mergeup"],
                    help="decode (default): mla_decode_partial; qprep: mla_query_prep on the "
                         "workload's query rows and heads; upproj: mla_up_project of its latent output; "
                         "gather: mla_gather_cache of each request's first 2048 cache tokens; "
                         "mergeup: mla_merge_up_project of 4 DCP shard partials (one DCP rank's shape)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "DCP shards are materialised on one device, so run with --gpus 1.", file=sys.stderr)
        return 2

    if args.probe_peaks:
        return probe_peaks()
    if args.op == "qprep":
        return bench_query_prep(args)
    if args.op == "upproj":
        return bench_up_project(args)
    if args.op == "gather":
        return bench_gather(args)
    if args.op == "mergeup":
        return bench_merge_up_project(args)

    return bench_decode(args)


if __name__ == "__main__":
    sys.exit(main())
