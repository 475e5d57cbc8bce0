"""Benchmark of the batch-invariant chunked attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one monolithic prefill over the dense workload (B=1, Hq=Hkv=32,
N=8192, D=128, bf16): Q tile staging, the 64-key block stream, QK^T, masking,
online softmax, PV, the 512-key chunk merge, finalisation and the bounded
store all run inside that one launch.  The line printed reports its
throughput in TFLOP/s (4*D FLOP per visible (query, key) pair per head), the
roofline of that kernel (HIP events on the stream it is launched on, against
the 2.5 PFLOP/s dense bf16 MFMA peak) and the fp64 CPU oracle timed on a
bounded sample of the same workload.  The other workloads (causal GQA varlen
prefill, split-KV paged decode with its merge, fp8 D=192 prefill) are timed
after it and reported under "secondary", decode against the 8 TB/s HBM peak,
followed by the batch-invariant GEMM on four tensor-parallel layer shapes
(torch.matmul, i.e. hipBLASLt, timed beside it as context; it does not follow
the batch-invariant contract).  Inputs are seeded, synthetic and resident in
HBM before timing starts.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "attention TFLOP/s (prefill) + decode HBM GB/s, fraction of MI355X peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--pmc-pass", nargs="?", const="traffic", choices=["traffic", "prefill"],
                    help="one launch per kernel for counter runs: 'traffic' (default; a "
                         "256 MiB copy, the dense prefill, decode, GEMM) or 'prefill'")
    ap.add_argument("--pmc-summary", nargs="+", metavar=("KIND", "CSV"),
                    help="summarise rocprofv3 counter CSVs of a --pmc-pass KIND run")
    return ap.parse_args()


def _source_hash() -> str:
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "deterministic_flash_attention_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def counted_traffic(kernel: str):
    """HBM bytes per dispatch measured with rocprofv3 counters (profiles/hbm_traffic.json),
    or None when the kernel sources changed since the counters were taken."""
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != _source_hash() or kernel not in rec.get("kernels", {}):
        return None
    return rec["kernels"][kernel]["hbm_bytes"]


def timed(fn, steps: int, warmup: int, min_warm_s: float = 0.3):
    """Warm up (at least `warmup` calls and about `min_warm_s` seconds of work,
    so the GPU clocks have ramped), then run `steps` calls back to back.
    Returns (per-call ms from HIP events recorded on the launch stream around
    each call, wall seconds of the whole timed region between two device
    synchronisations).  Both figures come from the same calls."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < min_warm_s:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in evs], wall


def prefill_workload(cfg, causal, dtype, seed=0):
    import synth
    import torch
    inp = synth.prefill_inputs(seed, cfg["seqlens"], cfg["hq"], cfg["hkv"], cfg["d"], causal,
                               dtype=dtype)
    dev = torch.device("cuda")
    t = dict(q=inp.q.to(dev), k=inp.k.to(dev), v=inp.v.to(dev), cq=inp.cu_seqlens_q.to(dev),
             ck=inp.cu_seqlens_k.to(dev))
    return inp, t


def run_prefill_fn(inp, t, schedule, window=(-1, -1)):
    import torch
    import deterministic_flash_attention_amd as dfa
    tq, hq, d = inp.q.shape
    o = torch.empty(tq, hq, d, dtype=torch.bfloat16, device="cuda")
    ms, mk = max(inp.seqlens_q), max(inp.seqlens_k)
    desc = (inp.q_scale, inp.k_scale, inp.v_scale)

    def fn():
        dfa.attn_prefill_fwd(t["q"], t["k"], t["v"], t["cq"], t["ck"], ms, mk, inp.scale,
                             inp.causal, schedule, o=o, descales=desc, window=window)
    return fn, o


# ---------------------------------------------------------------- secondary lines
# Each secondary line is set up once (inputs resident in HBM) and exposes one or
# more named callables; the lines are then timed in REPS interleaved repetitions
# (repetition r of every line before repetition r + 1 of any), ITERS timed calls
# each, and report the median of the repetition means and the minimum call.
REPS, ITERS, WARMUP = 3, 20, 3


class Line:
    def __init__(self, fns, finish):
        self.fns = fns          # name -> callable (one launch sequence per call)
        self.finish = finish    # dict name -> stats -> entry dict
        self.times = {k: [] for k in fns}


def stats(rep_ms):
    """rep_ms: list over repetitions of per-call ms lists."""
    import statistics
    means = [sum(r) / len(r) for r in rep_ms]
    return {"ms_median": statistics.median(means), "ms_min": min(min(r) for r in rep_ms),
            "ms_rep_means": [round(m, 5) for m in means]}


def prefill_line(name, cfg, causal, dtype, peak, peak_note, window=(-1, -1), traffic=None):
    import oracle
    inp, t = prefill_workload(cfg, causal, dtype)
    fn, _ = run_prefill_fn(inp, t, 0, window)
    flops = oracle.attention_flops(cfg["seqlens"], cfg["seqlens"], cfg["hq"], cfg["d"], causal,
                                   window=window)

    def finish(st):
        s = st["run"]
        tf = flops / (s["ms_median"] * 1e-3) / 1e12
        return {
            "workload": name, "causal": causal, "dtype": dtype, "seqlens": cfg["seqlens"],
            "window": list(window), "hq": cfg["hq"], "hkv": cfg["hkv"], "d": cfg["d"],
            "flop": flops, **s, "value": tf, "unit": "TFLOP/s",
            "tflops_at_min": flops / (s["ms_min"] * 1e-3) / 1e12,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s",
                         "frac": tf / peak, "traffic": counted_traffic(traffic) if traffic else None,
                         "peak_note": peak_note},
        }
    return Line({"run": fn}, finish)


def decode_bytes(inp) -> int:
    """Algorithmic HBM bytes of one decode step: K and V of every visible token
    (Hkv heads, D elements, element size), Q in, O out (bf16), the used page-table
    entries and the context lengths."""
    es = 1 if inp.dtype == "fp8" else 2
    ctx = inp.context_lens.long()
    pages = (ctx + inp.page_size - 1) // inp.page_size
    b, hq, d = inp.q.shape
    kv = int(ctx.sum()) * inp.hkv * d * es * 2
    return kv + b * hq * d * es + b * hq * d * 2 + 4 * int(pages.sum()) + 4 * b


def decode_line(dtype="bf16"):
    """The paged decode workload (bf16, or an e4m3 cache with per-tensor scales),
    cache pages stored heads-outer ("HND": each kv head's 16 page rows contiguous,
    5% faster than tokens-outer "NHD", timed beside it; the same bits)."""
    import torch
    import deterministic_flash_attention_amd as dfa
    import synth
    cfg = synth.PAGED_DECODE
    inp = synth.decode_inputs(0, cfg["batch"], cfg["hq"], cfg["hkv"], cfg["d"],
                              ctx_min=cfg["ctx_min"], ctx_max=cfg["ctx_max"],
                              spare_pages=cfg["spare_pages"], poison=False, dtype=dtype)
    dev = torch.device("cuda")
    q = inp.q.to(dev)
    kc = inp.k_cache.permute(0, 2, 1, 3).contiguous().to(dev)
    vc = inp.v_cache.permute(0, 2, 1, 3).contiguous().to(dev)
    kc_nhd, vc_nhd = inp.k_cache.to(dev), inp.v_cache.to(dev)
    pt, cl = inp.page_table.to(dev), inp.context_lens.to(dev)
    b, hq, d = inp.q.shape
    mc = int(inp.context_lens.max())
    cmax = dfa.attn_num_chunks(mc)
    part = torch.empty(dfa.attn_partials_bytes(b, hq, cmax, d) // 4, dtype=torch.float32, device=dev)
    o = torch.empty(b, hq, d, dtype=torch.bfloat16, device=dev)
    desc = (inp.q_scale, inp.k_scale, inp.v_scale)

    def split():
        dfa.attn_decode_split_fwd(q, kc, vc, pt, cl, mc, inp.scale, dfa.SPLIT, partials=part,
                                  descales=desc, kv_layout="HND")

    def merge():
        dfa.attn_chunk_merge(part, b, hq, cmax, d, o, v_descale=desc[2])

    def step():
        split()
        merge()

    def step_nhd():
        dfa.attn_decode_split_fwd(q, kc_nhd, vc_nhd, pt, cl, mc, inp.scale, dfa.SPLIT,
                                  partials=part, descales=desc, kv_layout="NHD")
        merge()

    nbytes = decode_bytes(inp)
    part_bytes = int((inp.context_lens.long() + 511).div(512, rounding_mode="floor").sum()) * hq * (d + 2) * 4

    def finish(st):
        gbs = lambda ms: nbytes / (ms * 1e-3) / 1e9  # noqa: E731
        a_split, a_step = st["split"]["ms_median"], st["step"]["ms_median"]
        return {
            "workload": "paged_decode" if dtype == "bf16" else "paged_decode_fp8", "dtype": dtype,
            "batch": b, "hq": hq, "hkv": inp.hkv, "d": d, "kv_layout": "HND",
            "sum_context": int(inp.context_lens.sum()), "bytes": nbytes,
            "ms_split": a_split, "ms_merge": st["merge"]["ms_median"], "ms_step": a_step,
            "ms_step_min": st["step"]["ms_min"], "ms_split_min": st["split"]["ms_min"],
            "ms_step_rep_means": st["step"]["ms_rep_means"],
            "value": gbs(a_step), "unit": "GB/s",
            "partials_bytes_written": part_bytes,
            "roofline": {"bound": "hbm", "achieved": gbs(a_split), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": gbs(a_split) / PEAK_HBM_GBS,
                         "traffic": counted_traffic(f"decode_split_{dtype}"),
                         "kernel": "decode split"},
            "step_frac_of_hbm": gbs(a_step) / PEAK_HBM_GBS,
            "step_frac_of_hbm_nhd": gbs(st["step_nhd"]["ms_median"]) / PEAK_HBM_GBS,
        }
    return Line({"split": split, "merge": merge, "step": step, "step_nhd": step_nhd}, finish)


def extend_setup():
    import torch
    import synth
    cfg = synth.MIXED_EXTEND
    inp = synth.extend_inputs(0, cfg["ctx_lens"], cfg["q_lens"], cfg["hq"], cfg["hkv"], cfg["d"],
                              spare_pages=cfg["spare_pages"], poison=False)
    dev = torch.device("cuda")
    t = dict(q=inp.q.to(dev), cq=inp.cu_seqlens_q.to(dev), kc=inp.k_cache.to(dev),
             vc=inp.v_cache.to(dev), pt=inp.page_table.to(dev), cl=inp.context_lens.to(dev))
    return cfg, inp, t


def extend_line():
    """The mixed prefill / extend / decode batch over a paged cache, one
    monolithic launch of attn_paged_extend_fwd per step, with the workspace
    that spreads the decode rows' chunks over the launch's idle workgroups
    (zero-filled once, outside the timed region; every launch leaves its
    counters at zero).  The same launch without the workspace is timed
    beside it ("single_tile")."""
    import torch
    import deterministic_flash_attention_amd as dfa
    import oracle
    cfg, inp, t = extend_setup()
    o = torch.empty_like(t["q"])
    mq, mc = max(inp.q_lens), max(inp.ctx_lens)
    nbytes = dfa.attn_extend_workspace_bytes(len(inp.q_lens), cfg["hq"], cfg["hkv"],
                                             dfa.attn_num_chunks(mc), cfg["d"])
    ws = torch.zeros((nbytes + 3) // 4, dtype=torch.float32, device="cuda")

    def fn():
        dfa.attn_paged_extend_fwd(t["q"], t["cq"], t["kc"], t["vc"], t["pt"], t["cl"], mq, mc,
                                  inp.scale, True, dfa.MONOLITHIC, o=o, partials=ws)

    def fn_single():
        dfa.attn_paged_extend_fwd(t["q"], t["cq"], t["kc"], t["vc"], t["pt"], t["cl"], mq, mc,
                                  inp.scale, True, dfa.MONOLITHIC, o=o)
    flops = oracle.attention_flops(inp.q_lens, inp.ctx_lens, cfg["hq"], cfg["d"], True)

    def finish(st):
        s = st["run"]
        tf = flops / (s["ms_median"] * 1e-3) / 1e12
        return {
            "workload": "mixed_paged_extend", "causal": True, "dtype": "bf16",
            "ctx_lens": inp.ctx_lens, "q_lens": inp.q_lens, "hq": cfg["hq"], "hkv": cfg["hkv"],
            "d": cfg["d"], "flop": flops, **s, "value": tf, "unit": "TFLOP/s",
            "workspace_bytes": nbytes,
            "single_tile_ms_median": st["single"]["ms_median"],
            "single_tile_tflops": flops / (st["single"]["ms_median"] * 1e-3) / 1e12,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                         "traffic": counted_traffic("mixed_paged_extend"),
                         "kernel": "prefill_kernel<128, bf16, paged, monolithic, chunk spread>"},
        }
    return Line({"run": fn, "single": fn_single}, finish)


def gemm_line(name, m, n, k):
    """C = A W^T for one layer shape: monolithic schedule for large M, split over
    the 1024-wide chunks plus the combine pass for decode-sized M.  Large M is
    priced against the bf16 MFMA peak (2 M N K FLOP), decode-sized M against
    HBM (the weight, A and C bytes).  torch.matmul (hipBLASLt, not batch
    invariant) is timed beside it as context."""
    import torch
    import deterministic_flash_attention_amd as dfa
    import synth
    inp = synth.gemm_inputs(0, m, n, k)
    a, w = inp.a.cuda(), inp.w.cuda()
    c = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    split = m <= 64
    sched = dfa.SPLIT if split else dfa.MONOLITHIC
    ws = torch.empty(max(dfa.det_gemm_workspace_bytes(m, n, k) // 4, 4), dtype=torch.float32,
                     device="cuda")
    wt = w.t()

    def fn():
        dfa.det_gemm_fwd(a, w, c, dfa.WEIGHT_NK, sched, -1, ws)

    def ref():
        torch.matmul(a, wt)
    flops = 2 * m * n * k
    nbytes = 2 * (m * k + n * k + m * n)

    def finish(st):
        s = st["run"]
        avg = s["ms_median"]
        tf = flops / (avg * 1e-3) / 1e12
        gbs = nbytes / (avg * 1e-3) / 1e9
        if split:
            roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": gbs / PEAK_HBM_GBS, "traffic": counted_traffic(f"gemm_{name}"),
                    "kernel": "gemm split + combine (one step)"}
        else:
            roof = {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": tf / PEAK_BF16_TFLOPS, "traffic": counted_traffic(f"gemm_{name}"),
                    "kernel": "gemm monolithic"}
        return {
            "workload": f"gemm_{name}", "m": m, "n": n, "k": k, "dtype": "bf16",
            "schedule": "split" if split else "monolithic", "flop": flops, "bytes": nbytes,
            **s, "value": tf, "unit": "TFLOP/s", "gb_s": gbs, "roofline": roof,
            "context_torch_matmul_ms_min": st["torch_matmul"]["ms_min"],
        }
    return Line({"run": fn, "torch_matmul": ref}, finish)


def secondary_lines():
    import synth
    mixed = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
    lines = [
        prefill_line("causal_gqa_varlen", synth.CAUSAL_VARLEN, True, "bf16", PEAK_BF16_TFLOPS,
                     "bf16 dense MFMA", traffic="prefill_causal_varlen_bf16"),
        decode_line("bf16"),
        decode_line("fp8"),
        extend_line(),
        prefill_line("sliding_window_1024", synth.DENSE_PREFILL, True, "bf16", PEAK_BF16_TFLOPS,
                     "bf16 dense MFMA", window=(1024, -1), traffic="sliding_window_1024"),
    ]
    for causal in (False, True):
        lines.append(prefill_line("fp8_wide_head", synth.FP8_WIDE, causal, "fp8", mixed,
                                  "QK^T on fp8 MFMA, PV on bf16 MFMA: half the FLOPs at each peak",
                                  traffic="prefill_fp8_d192_" + ("causal" if causal else "dense")))
    for name, m, n, k in synth.GEMM_SHAPES:
        lines.append(gemm_line(name, m, n, k))
    return lines


def run_secondary():
    lines = secondary_lines()
    for rep in range(REPS):
        for ln in lines:
            for name, fn in ln.fns.items():
                ms, _ = timed(fn, ITERS, WARMUP if rep == 0 else 1, min_warm_s=0.3 if rep == 0 else 0.05)
                ln.times[name].append(ms)
    out = []
    for ln in lines:
        e = ln.finish({k: stats(v) for k, v in ln.times.items()})
        if e["workload"] == "fp8_wide_head":
            e["frac_of_bf16_peak"] = e["value"] / PEAK_BF16_TFLOPS
            e["frac_of_fp8_peak"] = e["value"] / PEAK_FP8_TFLOPS
        out.append(e)
    return out


def cpu_baseline(target_s: float = 12.0):
    """The fp64 oracle on a bounded row sample of the dense workload: as many
    query rows as fit about target_s seconds, all 32 heads, every key."""
    import numpy as np
    import oracle
    import synth
    cfg = synth.DENSE_PREFILL
    inp = synth.prefill_inputs(0, cfg["seqlens"], cfg["hq"], cfg["hkv"], cfg["d"], False)
    q, k, v = synth.to_f64(inp.q), synth.to_f64(inp.k), synth.to_f64(inp.v)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        pass
    n = cfg["seqlens"][0]
    oracle.attention(q, k, v, [0, n], [0, n], cfg["hq"], cfg["hkv"], inp.scale, False,
                     rows=np.arange(16))
    t0 = time.perf_counter()
    oracle.attention(q, k, v, [0, n], [0, n], cfg["hq"], cfg["hkv"], inp.scale, False,
                     rows=np.arange(128))
    t1 = time.perf_counter() - t0
    nrows = int(min(n, max(128, 128 * target_s / max(t1, 1e-3))))
    rows = np.linspace(0, n - 1, nrows).astype(np.int64)
    t0 = time.perf_counter()
    oracle.attention(q, k, v, [0, n], [0, n], cfg["hq"], cfg["hkv"], inp.scale, False, rows=rows)
    dt = time.perf_counter() - t0
    flops = 4 * cfg["d"] * cfg["hq"] * nrows * n
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s",
            "cores": threads or len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{nrows} of {n} query rows x {cfg['hq']} heads x {n} keys of the dense "
                      f"workload, fp64 NumPy/BLAS, {dt:.1f} s",
            "seconds": dt, "host_cpus": len(os.sched_getaffinity(0))}


def pmc_pass(kind: str):
    """Launches for counter runs (rocprofv3 --pmc), one dispatch per kernel in a
    fixed order printed to stdout.  "traffic": a copy of known size (256 MiB read,
    256 MiB written) that calibrates FETCH_SIZE / WRITE_SIZE, then the prefill
    workloads (dense, causal GQA varlen, fp8 D=192 dense and causal, the sliding
    window, the mixed paged batch), the bf16 and e4m3 decode split and merge, and
    the four GEMM shapes.
    "prefill": the prefill workloads whose SQ counters the profiles quote
    (dense, causal GQA varlen, fp8 D=192 dense and causal, the mixed paged batch,
    the sliding window)."""
    import torch
    import deterministic_flash_attention_amd as dfa
    import synth
    dfa.load_library()
    order = []

    def run(label, fn):
        fn()
        torch.cuda.synchronize()
        order.append(label)
    if kind == "traffic":
        src = torch.ones(128 << 20, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        run("copy_256MiB", lambda: dst.copy_(src))
        for label, cfg, causal, dt, win in (
                ("prefill_dense_bf16", synth.DENSE_PREFILL, False, "bf16", (-1, -1)),
                ("prefill_causal_varlen_bf16", synth.CAUSAL_VARLEN, True, "bf16", (-1, -1)),
                ("prefill_fp8_d192_dense", synth.FP8_WIDE, False, "fp8", (-1, -1)),
                ("prefill_fp8_d192_causal", synth.FP8_WIDE, True, "fp8", (-1, -1)),
                ("sliding_window_1024", synth.DENSE_PREFILL, True, "bf16", (1024, -1))):
            inp, t = prefill_workload(cfg, causal, dt)
            run(label, run_prefill_fn(inp, t, dfa.MONOLITHIC, win)[0])
            del inp, t
        ln = extend_line()
        run("mixed_paged_extend", ln.fns["run"])
        del ln
        for dt in ("bf16", "fp8"):
            ln = decode_line(dt)
            run(f"decode_split_{dt}", ln.fns["split"])
            run(f"merge_d128_{dt}", ln.fns["merge"])
            del ln
        for name, m, n, k in synth.GEMM_SHAPES:
            inp_g = synth.gemm_inputs(0, m, n, k)
            a, w = inp_g.a.cuda(), inp_g.w.cuda()
            run(f"gemm_{name}", lambda: dfa.gemm(a, w))
    elif kind == "prefill":
        mixed = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
        lines = [("prefill_dense_bf16", prefill_line("dense", synth.DENSE_PREFILL, False, "bf16",
                                                     PEAK_BF16_TFLOPS, "")),
                 ("prefill_causal_varlen_bf16", prefill_line("causal", synth.CAUSAL_VARLEN, True,
                                                             "bf16", PEAK_BF16_TFLOPS, "")),
                 ("prefill_fp8_d192_dense", prefill_line("fp8", synth.FP8_WIDE, False, "fp8",
                                                         mixed, "")),
                 ("prefill_fp8_d192_causal", prefill_line("fp8", synth.FP8_WIDE, True, "fp8",
                                                          mixed, "")),
                 ("mixed_paged_extend", extend_line()),
                 ("sliding_window_1024", prefill_line("win", synth.DENSE_PREFILL, True, "bf16",
                                                      PEAK_BF16_TFLOPS, "", window=(1024, -1)))]
        for label, ln in lines:
            run(label, ln.fns["run"])
    else:
        raise ValueError(kind)
    print("pmc pass dispatch order: " + ", ".join(order))


# Library dispatches of each counter pass, in launch order (see pmc_pass).
PMC_LABELS = {
    "traffic": ["prefill_dense_bf16", "prefill_causal_varlen_bf16", "prefill_fp8_d192_dense",
                "prefill_fp8_d192_causal", "sliding_window_1024", "mixed_paged_extend",
                "decode_split_bf16", "merge_d128_bf16", "decode_split_fp8",
                "merge_d128_fp8", "gemm_gate_up", "gemm_down", "gemm_qkv_decode",
                "gemm_qkv_decode_combine", "gemm_gate_up_decode", "gemm_gate_up_decode_combine"],
    "prefill": ["prefill_dense_bf16", "prefill_causal_varlen_bf16", "prefill_fp8_d192_dense",
                "prefill_fp8_d192_causal", "mixed_paged_extend", "sliding_window_1024"],
}


def pmc_summary(kind: str, csv_paths):
    """Counter values per labelled dispatch from rocprofv3 counter_collection CSVs
    of `bench.py --pmc-pass KIND`.  For "traffic" (one CSV with FETCH_SIZE, one
    with WRITE_SIZE) it also writes profiles/hbm_traffic.json: KiB per dispatch
    scaled by what the same counter reads for the 256 MiB copy."""
    import csv
    per = {}
    for path in csv_paths:
        disp = {}
        for r in csv.DictReader(open(path)):
            d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "grid": r["Grid_Size"],
                                                       "vgpr": r["VGPR_Count"], "lds": r["LDS_Block_Size"],
                                                       "c": {}})
            d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        ids = sorted(disp)
        lib = [i for i in ids if "detattn::" in disp[i]["name"]]
        labels = PMC_LABELS[kind]
        assert len(lib) == len(labels), f"{path}: {len(lib)} library dispatches, expected {len(labels)}"
        for i, lab in zip(lib, labels):
            e = per.setdefault(lab, {"kernel": disp[i]["name"].split("(")[0].replace("void ", ""),
                                     "grid": disp[i]["grid"], "vgpr": disp[i]["vgpr"],
                                     "lds": disp[i]["lds"], "counters": {}})
            e["counters"].update(disp[i]["c"])
        copies = [i for i in ids if "copyBuffer" in disp[i]["name"] and int(disp[i]["grid"]) == 131072]
        if copies:
            per.setdefault("copy_256MiB", {"counters": {}})["counters"].update(disp[copies[0]]["c"])
    if kind == "traffic":
        cf = per["copy_256MiB"]["counters"]["FETCH_SIZE"]
        cw = per["copy_256MiB"]["counters"]["WRITE_SIZE"]
        out = {"source_hash": _source_hash(), "fetch_scale": 256 * 1024 / cf,
               "write_scale": 256 * 1024 / cw, "copy_fetch_kib": cf, "copy_write_kib": cw,
               "kernels": {}}
        for lab in PMC_LABELS["traffic"]:
            if lab.endswith("_combine"):
                continue
            f = per[lab]["counters"]["FETCH_SIZE"]
            w = per[lab]["counters"]["WRITE_SIZE"]
            comb = per.get(lab + "_combine")
            if comb:  # a decode-sized GEMM step is the split kernel plus its combine pass
                f += comb["counters"]["FETCH_SIZE"]
                w += comb["counters"]["WRITE_SIZE"]
            out["kernels"][lab] = {"fetch_kib": f, "write_kib": w,
                                   "hbm_bytes": f * 1024 * out["fetch_scale"] + w * 1024 * out["write_scale"]}
        out["note"] = ("HBM bytes per dispatch from two rocprofv3 --pmc runs (FETCH_SIZE, then "
                       "WRITE_SIZE, KiB per dispatch) of `python3 bench.py --pmc-pass traffic`, each "
                       "scaled by what the same counter reads for a 256 MiB device copy in the same "
                       "run (bench.py --pmc-summary traffic). source_hash covers "
                       "deterministic_flash_attention_amd/csrc/*; bench.py reports traffic only while "
                       "it matches.")
        json.dump(out, open(os.path.join(ROOT, "profiles", "hbm_traffic.json"), "w"), indent=1)
    print(json.dumps(per, indent=1))


def main():
    args = parse()
    if args.pmc_pass:
        pmc_pass(args.pmc_pass)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1:])
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path to time.", file=sys.stderr)
        sys.exit(2)
    import torch
    import deterministic_flash_attention_amd as dfa
    import oracle
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if not os.path.exists(dfa.library_path()):
        from deterministic_flash_attention_amd import build
        build.build()
    dfa.load_library()

    cfg = synth.DENSE_PREFILL
    inp, t = prefill_workload(cfg, False, "bf16")
    fn, _ = run_prefill_fn(inp, t, dfa.MONOLITHIC)
    flops = oracle.attention_flops(cfg["seqlens"], cfg["seqlens"], cfg["hq"], cfg["d"], False)
    # K steps timed back to back after the warm-up; HIP events around each
    # step (on the launch stream) give the kernel time for the roofline.
    ms_kernel, wall = timed(fn, args.steps, args.warmup)
    ms_step = wall * 1e3 / args.steps
    value = flops * args.steps / wall / 1e12
    k_avg = sum(ms_kernel) / len(ms_kernel)
    achieved = flops / (k_avg * 1e-3) / 1e12

    secondary = [] if args.no_secondary else run_secondary()
    cpu = None if args.no_cpu_baseline else cpu_baseline()
    props = torch.cuda.get_device_properties(0)
    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dense_prefill", "batch": 1, "seq_len": cfg["seqlens"][0],
                   "num_heads_q": cfg["hq"], "num_heads_kv": cfg["hkv"], "head_dim": cfg["d"],
                   "causal": False, "schedule": "monolithic", "block_keys": 64, "chunk_keys": 512,
                   "inputs": "N(0,1) unscaled, seed 0"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": counted_traffic("prefill_dense_bf16"),
                     "kernel": "prefill_kernel<128, bf16, monolithic>",
                     "kernel_ms_mean": round(k_avg, 4), "kernel_ms_min": round(min(ms_kernel), 4)},
        "cpu_baseline": cpu,
        "secondary": secondary,
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
