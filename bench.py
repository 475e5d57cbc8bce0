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
    ap.add_argument("--pmc-pass", action="store_true",
                    help="one launch of each kernel plus a 256 MiB copy, for counter runs")
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


def prefill_entry(name, cfg, causal, dtype, iters, warmup, peak, peak_note, window=(-1, -1)):
    import oracle
    inp, t = prefill_workload(cfg, causal, dtype)
    fn, _ = run_prefill_fn(inp, t, 0, window)
    ms, _ = timed(fn, iters, warmup)
    flops = oracle.attention_flops(cfg["seqlens"], cfg["seqlens"], cfg["hq"], cfg["d"], causal,
                                   window=window)
    avg = sum(ms) / len(ms)
    tf = flops / (avg * 1e-3) / 1e12
    return {
        "workload": name, "causal": causal, "dtype": dtype, "seqlens": cfg["seqlens"],
        "window": list(window),
        "hq": cfg["hq"], "hkv": cfg["hkv"], "d": cfg["d"], "flop": flops,
        "ms_mean": avg, "ms_min": min(ms), "value": tf, "unit": "TFLOP/s",
        "roofline": {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s",
                     "frac": tf / peak, "traffic": None, "peak_note": peak_note},
    }


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


def decode_entry(iters, warmup, dtype="bf16"):
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

    def both():
        split()
        merge()
    ms_split, _ = timed(split, iters, warmup)
    ms_merge, _ = timed(merge, iters, warmup)
    ms_step, _ = timed(both, iters, warmup)
    kc_nhd, vc_nhd = inp.k_cache.to(dev), inp.v_cache.to(dev)

    def both_nhd():
        dfa.attn_decode_split_fwd(q, kc_nhd, vc_nhd, pt, cl, mc, inp.scale, dfa.SPLIT,
                                  partials=part, descales=desc, kv_layout="NHD")
        merge()
    ms_step_nhd, _ = timed(both_nhd, iters, warmup)
    del kc_nhd, vc_nhd
    nbytes = decode_bytes(inp)
    a_split = sum(ms_split) / iters
    a_step = sum(ms_step) / iters
    gbs_step = nbytes / (a_step * 1e-3) / 1e9
    gbs_split = nbytes / (a_split * 1e-3) / 1e9
    part_bytes = int((inp.context_lens.long() + 511).div(512, rounding_mode="floor").sum()) * hq * (d + 2) * 4
    return {
        "workload": "paged_decode" if dtype == "bf16" else "paged_decode_fp8", "dtype": dtype,
        "batch": b, "hq": hq, "hkv": inp.hkv, "d": d, "kv_layout": "HND",
        "step_frac_of_hbm_nhd": nbytes / (sum(ms_step_nhd) / iters * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "sum_context": int(inp.context_lens.sum()), "bytes": nbytes,
        "ms_split": a_split, "ms_merge": sum(ms_merge) / iters, "ms_step": a_step,
        "value": gbs_step, "unit": "GB/s",
        "partials_bytes_written": part_bytes,
        "roofline": {"bound": "hbm", "achieved": gbs_split, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs_split / PEAK_HBM_GBS,
                     "traffic": counted_traffic(f"decode_split_{dtype}"),
                     "kernel": "decode split"},
        "step_frac_of_hbm": gbs_step / PEAK_HBM_GBS,
    }


def extend_entry(iters, warmup):
    """The mixed prefill / extend / decode batch over a paged cache, one
    monolithic launch of attn_paged_extend_fwd per step."""
    import torch
    import deterministic_flash_attention_amd as dfa
    import oracle
    import synth
    cfg = synth.MIXED_EXTEND
    inp = synth.extend_inputs(0, cfg["ctx_lens"], cfg["q_lens"], cfg["hq"], cfg["hkv"], cfg["d"],
                              spare_pages=cfg["spare_pages"], poison=False)
    dev = torch.device("cuda")
    q, cq = inp.q.to(dev), inp.cu_seqlens_q.to(dev)
    kc, vc = inp.k_cache.to(dev), inp.v_cache.to(dev)
    pt, cl = inp.page_table.to(dev), inp.context_lens.to(dev)
    o = torch.empty_like(q)
    mq, mc = max(inp.q_lens), max(inp.ctx_lens)

    def fn():
        dfa.attn_paged_extend_fwd(q, cq, kc, vc, pt, cl, mq, mc, inp.scale, True, dfa.MONOLITHIC,
                                  o=o)
    ms, _ = timed(fn, iters, warmup)
    flops = oracle.attention_flops(inp.q_lens, inp.ctx_lens, cfg["hq"], cfg["d"], True)
    avg = sum(ms) / len(ms)
    tf = flops / (avg * 1e-3) / 1e12
    return {
        "workload": "mixed_paged_extend", "causal": True, "dtype": "bf16",
        "ctx_lens": inp.ctx_lens, "q_lens": inp.q_lens, "hq": cfg["hq"], "hkv": cfg["hkv"],
        "d": cfg["d"], "flop": flops, "ms_mean": avg, "ms_min": min(ms), "value": tf,
        "unit": "TFLOP/s",
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS, "traffic": None,
                     "kernel": "prefill_kernel<128, bf16, paged, monolithic>"},
    }


def gemm_entry(name, m, n, k, iters, warmup):
    """C = A W^T for one layer shape: monolithic schedule for large M, split over
    the 1024-wide chunks plus the combine pass for decode-sized M.  Large M is
    priced against the bf16 MFMA peak (2 M N K FLOP), decode-sized M against
    HBM (the weight, A and C bytes)."""
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

    def fn():
        dfa.det_gemm_fwd(a, w, c, dfa.WEIGHT_NK, sched, -1, ws)
    ms, _ = timed(fn, iters, warmup)
    wt = w.t()
    ms_ref, _ = timed(lambda: torch.matmul(a, wt), iters, warmup)
    avg = sum(ms) / len(ms)
    flops = 2 * m * n * k
    tf = flops / (avg * 1e-3) / 1e12
    nbytes = 2 * (m * k + n * k + m * n)
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
        "ms_mean": avg, "ms_min": min(ms), "value": tf, "unit": "TFLOP/s", "gb_s": gbs,
        "roofline": roof,
        "context_torch_matmul_ms_min": min(ms_ref),
    }


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


def pmc_pass():
    """One launch of each kernel and a copy of known size (256 MiB read, 256 MiB
    written) whose counters calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch
    import deterministic_flash_attention_amd as dfa
    import synth
    dfa.load_library()
    src = torch.ones(128 << 20, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    inp, t = prefill_workload(synth.DENSE_PREFILL, False, "bf16")
    fn, _ = run_prefill_fn(inp, t, dfa.MONOLITHIC)
    fn()
    decode_entry(1, 0)
    decode_entry(1, 0, dtype="fp8")
    for name, m, n, k in synth.GEMM_SHAPES:
        inp_g = synth.gemm_inputs(0, m, n, k)
        dfa.gemm(inp_g.a.cuda(), inp_g.w.cuda())
    torch.cuda.synchronize()
    print("pmc pass done")


def main():
    args = parse()
    if args.pmc_pass:
        pmc_pass()
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

    secondary = []
    if not args.no_secondary:
        secondary.append(prefill_entry("causal_gqa_varlen", synth.CAUSAL_VARLEN, True, "bf16",
                                       20, 3, PEAK_BF16_TFLOPS, "bf16 dense MFMA"))
        secondary.append(decode_entry(20, 3))
        secondary.append(decode_entry(20, 3, dtype="fp8"))
        secondary.append(extend_entry(20, 3))
        secondary.append(prefill_entry("sliding_window_1024", synth.DENSE_PREFILL, True, "bf16",
                                       20, 3, PEAK_BF16_TFLOPS, "bf16 dense MFMA",
                                       window=(1024, -1)))
        mixed = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
        for causal in (False, True):
            e = prefill_entry("fp8_wide_head", synth.FP8_WIDE, causal, "fp8", 20, 3, mixed,
                              "QK^T on fp8 MFMA, PV on bf16 MFMA: half the FLOPs at each peak")
            e["frac_of_bf16_peak"] = e["value"] / PEAK_BF16_TFLOPS
            secondary.append(e)
        for name, m, n, k in synth.GEMM_SHAPES:
            secondary.append(gemm_entry(name, m, n, k, 20, 3))
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
