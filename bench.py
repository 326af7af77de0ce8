#!/usr/bin/env python3
"""Benchmark of the sparse MLA forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_fp8]

A step is one sparse_mla_fwd call (the whole hot path: gather, widening, QK,
softmax, PV, epilogue, and the combine kernel when the plan splits) over the
workload's seeded synthetic inputs, already resident in HBM. Before each timed
step a 1 GiB buffer is written (untimed) so the call starts with cold caches
(the MI355X MALL is 256 MB and would otherwise hold most of the pool). Device
time per call comes from HIP events recorded on the stream the library
launches on. Rank 0 prints one JSON line.

Headline workload: fp8 decode, 128 requests x (5+1) rows = 768 rows, 16 heads,
576-wide rows, pool 262144 x 576 e4m3fn + per-tensor scale, top-k 2048 (the
decode shape the HBM-roofline target is set on). Every configuration of the
method's workload table (tiny, the bf16 and fp8 decodes, the two 64-head
prefills) is timed on its own under "configs", with its roofline fraction (HBM
for the decodes and the tiny call, bf16 MFMA for the prefills) and the fp64
oracle timed beside it on the host (the tiny call and the decodes in full, the
prefills on every 64th row, scaled to the whole call). The two decodes are
timed again with their heads split over two GPUs (32 heads: one GPU's share)
under "head_share", as two-segment calls (a seeded 128-slot sliding window over
a second pool with its own scale, next to the same workload's one-segment
time; the fp8 prefill too, whose 64-head kernel composes the two segments
through the combine kernel) under "two_segment", and with the output epilogue (inverse RoPE of the
last 64 columns and an MXFP8 store) fused into the forward's store, next to
the plain forward followed by the separate epilogue pass, under "epilogue".
The headline decode is timed again on a pool that does not fit the MALL (each
request's top-k from its own 16384-row context of a 1.2 GB pool) under
"sensitivity". The indexer that produces index rows (fp8 MQA logits over
[ks, ke) windows, then a per-row top-k) is timed on the shapes of its own
kernel-time table under "indexer".
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
CSRC = os.path.join(ROOT, "sparse_mla_attention_05_amd", "csrc")


def attention_kernel(plan, d_qk, fp8):
    """(kernel name as rocprofv3 shows it, source file) of the attention
    kernel a plan launches without an output epilogue (the instance with
    `false` last); mirrors the dispatch in csrc/kernels.hip."""
    hb, v = plan["head_block"], plan["variant"]
    if hb == 16 and fp8 and v == 0:
        return f"smla::decode_kernel<{d_qk}, false>", "decode.hip"
    if hb == 64 and v != 1:
        if fp8 and v == 0:
            return f"smla::prefill_fp8_kernel<{d_qk}, false>", "prefill_fp8.hip"
        if fp8 and v == 3:
            return f"smla::prefill_mx_kernel<{d_qk}, false, false, false>", "prefill_mx.hip"
        return f"smla::prefill_kernel<{d_qk}, {str(fp8).lower()}, false>", "prefill.hip"
    return f"smla::fwd_kernel (staged tile, {hb} heads)", "kernels.hip"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_fp8")
    ap.add_argument("--variant", type=int, default=0,
                    help="kernel instance for the --workload timing (0: the planner's choice); "
                         "used to profile an opt-in kernel")
    ap.add_argument("--configs", default="tiny,decode_bf16,decode_fp8,prefill_fp8,prefill_glm",
                    help="comma list of the configurations timed on their own, each with its "
                         "roofline fraction and the oracle beside it ('' for none)")
    ap.add_argument("--head-share", default="decode_bf16_h32,decode_fp8_h32",
                    help="decode workloads with 32 heads (one GPU's share of a two-way head "
                         "split) ('' for none)")
    ap.add_argument("--two-segment", default="decode_bf16,decode_fp8,prefill_fp8",
                    help="comma list of workloads also timed with a sliding-window second "
                         "segment ('' for none)")
    ap.add_argument("--window", type=int, default=128, help="slots of that second segment")
    ap.add_argument("--indexer", default="ix_causal_8k_8k,ix_causal_4k_32k,ix_causal_2k_64k,"
                    "ix_causal_1k_128k,ix_multi_4k_32k",
                    help="indexer workloads timed (fp8 MQA logits, then the top-k)")
    ap.add_argument("--epilogue", default="decode_bf16,decode_fp8",
                    help="workloads also timed with the fused inverse-RoPE + MXFP8 store")
    ap.add_argument("--sensitivity", default="decode_fp8_ctx",
                    help="decode workloads whose pool does not fit the MALL, reported next to "
                         "the headline ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm", action="store_true", help="skip the cache flush between steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (to calibrate HBM byte counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain copy kernel of known size: 1 GiB read + 1 GiB written, 3 times.
    Its FETCH_SIZE / WRITE_SIZE under rocprofv3 --pmc give the factor that
    turns those counters into HBM bytes."""
    import torch
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": a.numel() * 4,
                      "copy_calibration_bytes_written": b.numel() * 4}), flush=True)


def algorithmic(inp):
    """Algorithmic bytes and flops of one call.

    bytes = gathered KV (one pool row per valid slot) + q + indices + out + lse;
    flops = 2 * H * (valid slots) * (D_qk + 512)."""
    R, H, D = inp.q.shape
    K = inp.indices.shape[1]
    valid = int((inp.indices >= 0).sum())
    eb = 1 if inp.workload.kv_dtype == "fp8" else 2
    kv = valid * D * eb
    other = R * H * D * 2 + R * K * 4 + R * H * 512 * 2 + R * H * 4
    flops = 2 * H * valid * (D + 512)
    return dict(kv_bytes=kv, bytes=kv + other, flops=flops, valid_slots=valid)


def source_digest(src):
    with open(os.path.join(CSRC, src), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counters_from_profiles(kernel_src, workload):
    """The committed rocprofv3 --pmc summary of a kernel on a workload, if it
    was taken on the current source of the kernel; else None."""
    stem = kernel_src.rsplit(".", 1)[0]
    path = os.path.join(ROOT, "profiles", f"{stem}_kernel_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
        if d.get("kernel_source_sha256_16") != source_digest(kernel_src):
            return None
        return d
    except Exception:
        return None


def time_workload(name, steps, warmup, cold, window=0, epi=None, variant=0):
    """Time one workload; with `window` > 0 as a two-segment call whose second
    segment is a seeded sliding window of that many slots over its own pool;
    with epi = "fused" the forward's store applies the inverse RoPE and the
    MXFP8 store, with epi = "unfused" the plain forward is followed by the
    separate epilogue pass. A nonzero `variant` asks the planner for that
    kernel instance (plain calls only)."""
    import torch
    from sparse_mla_attention_05_amd import _lib
    from sparse_mla_attention_05_amd.inputs import (make_epilogue_inputs, make_extra_segment,
                                                    make_inputs)

    inp = make_inputs(name)
    dev = torch.device("cuda:0")
    q, pool, idx = inp.q.to(dev), inp.pool.to(dev), inp.indices.to(dev)
    scale = inp.kv_scale.to(dev) if inp.kv_scale is not None else None
    R, H = q.shape[0], q.shape[1]
    out = torch.empty((R, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev) if cold else None  # 1 GiB
    stream = torch.cuda.current_stream(dev)
    ex = None
    if window > 0:
        ex = make_extra_segment(inp, window, seed=1000 + inp.workload.seed, value_std=0.7)
        xpool, xidx = ex.pool.to(dev), ex.indices.to(dev)
        xscale = ex.kv_scale.to(dev) if ex.kv_scale is not None else None
        p1, p2, _ = _lib.sparse_mla_plan2(q, pool, idx, xpool, xidx)
        plan = {"main": p1, "extra": p2}

        def call():
            _lib.sparse_mla_fwd2(q, pool, scale, idx, xpool, xscale, xidx, inp.sm_scale, out, lse,
                                 stream=stream)
    elif epi is not None:
        plan = _lib.sparse_mla_plan(q, pool, idx)
        e = make_epilogue_inputs(R, seed=inp.workload.seed)
        pos, cs = e.positions.to(dev), e.cos_sin.to(dev)
        codes = torch.empty((R, H, 512), dtype=torch.float8_e4m3fn, device=dev)
        scales = torch.empty((R, H, 16), dtype=torch.float8_e8m0fnu, device=dev)
        if epi == "fused":
            def call():
                _lib.sparse_mla_fwd_epi(q, pool, scale, idx, inp.sm_scale, codes, lse,
                                        rope_positions=pos, rope_cos_sin=cs, out_scale=scales,
                                        stream=stream)
        else:
            def call():
                _lib.sparse_mla_fwd(q, pool, scale, idx, inp.sm_scale, out, lse, stream=stream)
                _lib.sparse_mla_out_epilogue(out, codes, rope_positions=pos, rope_cos_sin=cs,
                                             out_scale=scales, stream=stream)
    elif variant:
        plan = _lib.sparse_mla_plan(q, pool, idx, variant=variant)

        def call():
            _lib.sparse_mla_fwd_ex(q, pool, scale, idx, inp.sm_scale, out, lse, stream=stream,
                                   variant=variant)
    else:
        plan = _lib.sparse_mla_plan(q, pool, idx)

        def call():
            _lib.sparse_mla_fwd(q, pool, scale, idx, inp.sm_scale, out, lse, stream=stream)

    # Warm until the device clock has settled: at least `warmup` calls and
    # WARM_SECONDS of back-to-back work (the clock ramps over tens of ms:
    # successive calls of a cold device run up to ~15 % slower).
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < WARM_SECONDS:
        call()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    times = []
    t0 = time.perf_counter()
    for _ in range(steps):
        if flush is not None:
            flush.fill_(1.0)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)  # us
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # warm: back-to-back calls, one event pair around all of them
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    warm_us = e0.elapsed_time(e1) * 1e3 / steps
    alg = algorithmic(inp)
    if ex is not None:
        eb = 1 if inp.workload.kv_dtype == "fp8" else 2
        xv = int((ex.indices >= 0).sum())
        xk = xv * inp.workload.d_qk * eb
        alg = dict(kv_bytes=alg["kv_bytes"] + xk, bytes=alg["bytes"] + xk + ex.indices.numel() * 4,
                   flops=alg["flops"] + 2 * H * xv * (inp.workload.d_qk + 512),
                   valid_slots=alg["valid_slots"] + xv)
    return dict(inp=inp, plan=plan, times=times, wall=wall, warm_us=warm_us, alg=alg)


MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA, TFLOP/s
WARM_SECONDS = 0.15  # back-to-back work before a timing starts


def time_indexer(name, steps, warmup):
    """Cold device time of the indexer logits (clean) and of the top-k over
    them, for one workload."""
    import torch
    from sparse_mla_attention_05_amd import _lib
    from sparse_mla_attention_05_amd.inputs import make_indexer_inputs

    inp = make_indexer_inputs(name)
    dev = torch.device("cuda:0")
    q, k, sc, w = inp.q.to(dev), inp.k.to(dev), inp.kv_scale.to(dev), inp.w.to(dev)
    ks, ke = inp.ks.to(dev), inp.ke.to(dev)
    M, N = q.shape[0], k.shape[0]
    logits = torch.empty((M, N), dtype=torch.float32, device=dev)
    topk = inp.workload.topk
    idx = torch.empty((M, topk), dtype=torch.int32, device=dev)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    calls = {
        "logits": lambda: _lib.sparse_mla_indexer_logits(q, k, sc, w, ks, ke, logits, True, stream=stream),
        "topk": lambda: _lib.sparse_mla_indexer_topk(logits, ks, ke, topk, idx, stream=stream),
    }
    res = {}
    for key, call in calls.items():
        # warm until the device clock has settled (as time_workload does)
        t0 = time.perf_counter()
        n = 0
        while n < warmup or time.perf_counter() - t0 < WARM_SECONDS:
            call()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
        times = []
        for _ in range(steps):
            flush.fill_(1.0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        res[key] = statistics.median(times)
    lo = inp.ks.clamp(0, N).long()
    hi = torch.maximum(inp.ke.clamp(0, N).long(), lo)
    pairs = int((hi - lo).sum())
    flops = 2 * pairs * inp.workload.heads * inp.workload.dim
    tf = flops / (res["logits"] * 1e-6) / 1e12
    return {"workload": name, "rows": M, "keys": N, "requests": inp.workload.requests,
            "logits_us": round(res["logits"], 1), "topk_us": round(res["topk"], 1), "topk": topk,
            "window_pairs": pairs, "tflops": round(tf, 1),
            "mfma_fp8_frac": round(tf / MFMA_FP8_PEAK_TFLOPS, 4),
            "logits_write_tbs": round(M * N * 4 / (res["logits"] * 1e-6) / 1e12, 2)}


def host_cores():
    """(physical cores, logical CPUs) of the host."""
    logical = os.cpu_count() or 1
    try:
        import psutil
        return psutil.cpu_count(logical=False) or logical, logical
    except Exception:
        return logical, logical


def cpu_baseline(inp, stride=1):
    """Time the fp64 oracle as it stands on the call's rows (every
    `stride`-th row when stride > 1, the time then scaled by the row count to
    one whole call)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    R = inp.q.shape[0]
    rows = np.arange(0, R, stride)
    t0 = time.perf_counter()
    for lo in range(0, len(rows), 64):  # chunks bound the gathered rows held at once
        oracle.sparse_mla_fwd_torch(inp.q, inp.pool, inp.kv_scale, inp.indices, inp.sm_scale,
                                    rows=rows[lo:lo + 64])
    el = time.perf_counter() - t0
    cores, logical = host_cores()
    if stride == 1:
        sample = f"all {R} rows in {el:.2f} s"
    else:
        sample = (f"every {stride}th row ({len(rows)} of {R}) in {el:.2f} s, scaled by "
                  f"{R}/{len(rows)} to the whole call (rows cost the same: equal top-k)")
    return {"value": round(el / len(rows) * R * 1e6, 1), "unit": "us/call", "cores": cores,
            "threads": threads, "logical_cpus": logical, "kind": "oracle", "sample": sample}


def config_record(name, r, bound, cpu=None):
    """One configuration's figures from a time_workload result."""
    us = statistics.median(r["times"])
    w = r["inp"].workload
    alg = r["alg"]
    tf = alg["flops"] / (us * 1e-6) / 1e12
    gbs = alg["bytes"] / (us * 1e-6) / 1e9
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    rec = {"workload": name, "description": w.description, "us_per_call": round(us, 2),
           "us_min": round(min(r["times"]), 2), "warm_us_per_call": round(r["warm_us"], 2),
           "gathered_kv_tbs": round(alg["kv_bytes"] / (us * 1e-6) / 1e12, 3),
           "alg_tbs": round(gbs / 1e3, 3), "tflops": round(tf, 2), "roofline": roof,
           "kernel": attention_kernel(r["plan"], w.d_qk, w.kv_dtype == "fp8")[0], "plan": r["plan"]}
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    return rec


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the sparse MLA forward runs on one GPU (it has no cross-GPU "
              "path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    from sparse_mla_attention_05_amd import _lib
    _lib.load()  # fails loudly if the HIP library is not built

    cold = not args.warm
    cpu_on = not args.no_cpu_baseline
    head = time_workload(args.workload, args.steps, args.warmup, cold, variant=args.variant)
    times = head["times"]
    us = statistics.median(times)
    alg = head["alg"]
    w = head["inp"].workload
    kname, ksrc = attention_kernel(head["plan"], w.d_qk, w.kv_dtype == "fp8")
    # the plan is one launch of the attention kernel (splits == 1), so the
    # event time of a call is that kernel's launch duration
    achieved = alg["bytes"] / (us * 1e-6) / 1e9
    ctr = counters_from_profiles(ksrc, w.name)
    line = {
        "metric": "sparse MLA us/call; HBM TB/s (decode) and MFMA TFLOP/s (prefill), 1 GPU",
        "value": round(us, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 MFMA, fp32 accumulate/softmax, fp8 e4m3fn KV" if w.kv_dtype == "fp8"
                 else "bf16 MFMA, fp32 accumulate/softmax, bf16 KV",
        "data": "synthetic (seeded, CPU-generated; no dataset or weights)",
        "config": {
            "workload": w.name, "description": w.description, "rows": w.rows, "heads": w.heads,
            "d_qk": w.d_qk, "topk": w.topk, "pool_rows": w.pool_rows, "kv_dtype": w.kv_dtype,
            "timing": "cold (1 GiB write before each call), median of device event times",
            "plan": head["plan"],
        },
        "gathered_kv_tbs": round(alg["kv_bytes"] / (us * 1e-6) / 1e12, 3),
        "alg_tbs": round(alg["bytes"] / (us * 1e-6) / 1e12, 3),
        "tflops": round(alg["flops"] / (us * 1e-6) / 1e12, 2),
        "us_min": round(min(times), 2),
        "us_mean": round(statistics.mean(times), 2),
        "warm_us_per_call": round(head["warm_us"], 2),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": ctr.get("hbm_bytes_per_launch") if ctr else None,
            "traffic_kind": "L2-to-fabric bytes per launch: FETCH_SIZE x 2 + WRITE_SIZE (factors "
                            "from a 1 GiB copy); MALL hits included",
            "dram_destined_read_bytes": ctr.get("dram_destined_read_bytes_per_launch") if ctr else None,
            "bytes_per_launch": alg["bytes"],
            "kernel": kname,
            "call_event_us": round(us, 2),
        },
    }
    configs = []
    for name in [s_ for s_ in args.configs.split(",") if s_]:
        prefill = name.startswith("prefill")
        r = head if name == args.workload else time_workload(
            name, max(3, args.steps // 2) if prefill else args.steps, 2 if prefill else 3, cold)
        cpu = cpu_baseline(r["inp"], stride=64 if prefill else 1) if cpu_on else None
        configs.append(config_record(name, r, "mfma" if prefill else "hbm", cpu))
        if name == args.workload and cpu is not None:
            line["cpu_baseline"] = cpu
        if r is not head:
            del r
    if configs:
        line["configs"] = configs
    if cpu_on and "cpu_baseline" not in line:
        line["cpu_baseline"] = cpu_baseline(head["inp"], stride=1)
    share = []
    for name in [s_ for s_ in args.head_share.split(",") if s_]:
        r = time_workload(name, args.steps, 3, cold)
        share.append(config_record(name, r, "hbm"))
        del r
    if share:
        line["head_share"] = share
    sens = []
    for name in [s_ for s_ in args.sensitivity.split(",") if s_]:
        r = time_workload(name, args.steps, 3, cold)
        sus = statistics.median(r["times"])
        ws = r["inp"].workload
        sc = counters_from_profiles(attention_kernel(r["plan"], ws.d_qk, ws.kv_dtype == "fp8")[1],
                                    name)
        sens.append({"workload": name, "description": ws.description,
                     "us_per_call": round(sus, 1), "warm_us_per_call": round(r["warm_us"], 1),
                     "alg_tbs": round(r["alg"]["bytes"] / (sus * 1e-6) / 1e12, 2),
                     "hbm_frac": round(r["alg"]["bytes"] / (sus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "l2_fabric_bytes": sc.get("hbm_bytes_per_launch") if sc else None,
                     "dram_destined_read_bytes": sc.get("dram_destined_read_bytes_per_launch") if sc else None,
                     "plan": r["plan"]})
        del r
    if sens:
        line["sensitivity"] = sens
    two = []
    for name in [s_ for s_ in args.two_segment.split(",") if s_]:
        prefill = name.startswith("prefill")
        k = max(3, args.steps // 2) if prefill else args.steps
        r = time_workload(name, k, 3, cold, window=args.window)
        one = time_workload(name, k, 3, cold)
        tus = statistics.median(r["times"])
        ous = statistics.median(one["times"])
        rec = {"workload": name, "window": args.window, "us_per_call": round(tus, 1),
               "one_segment_us_per_call": round(ous, 1),
               "gathered_kv_tbs": round(r["alg"]["kv_bytes"] / (tus * 1e-6) / 1e12, 2)}
        if prefill:
            rec["mfma_frac"] = round(r["alg"]["flops"] / (tus * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        else:
            rec["hbm_frac"] = round(r["alg"]["bytes"] / (tus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        rec.update({"warm_us_per_call": round(r["warm_us"], 1), "plan": r["plan"]})
        two.append(rec)
        del r, one
    if two:
        line["two_segment"] = two
    epis = []
    for name in [s_ for s_ in args.epilogue.split(",") if s_]:
        res = {m: time_workload(name, args.steps, 3, cold, epi=m)
               for m in ("fused", "unfused", None)}
        us_ = {m: statistics.median(r["times"]) for m, r in res.items()}
        epis.append({"workload": name, "epilogue": "inverse RoPE (64 columns) + MXFP8 store",
                     "us_fused": round(us_["fused"], 1), "us_unfused": round(us_["unfused"], 1),
                     "us_plain_bf16": round(us_[None], 1),
                     "fused_vs_unfused": round(us_["fused"] / us_["unfused"] - 1.0, 4),
                     "warm_us_fused": round(res["fused"]["warm_us"], 1),
                     "warm_us_unfused": round(res["unfused"]["warm_us"], 1)})
        del res
    if epis:
        line["epilogue"] = epis
    ixs = [time_indexer(name, max(5, args.steps // 2), 2)
           for name in [s_ for s_ in args.indexer.split(",") if s_]]
    if ixs:
        line["indexer"] = ixs
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
