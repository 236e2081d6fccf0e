#!/usr/bin/env python3
"""Throughput of single-token GQA decode on one MI355X: KV bytes streamed per second.

A step is one gqa_decode over one batch of the Llama-70B-shaped layer (B32 Hq64 Hkv8 d128 L8192,
seq_lens ~ U[6000, 8192], bf16) with inputs resident in HBM.  The KV bytes of a step are
sum_b seq_lens[b] * Hkv * 2 * d * 2 (one K and one V row per cached token and KV head).  Several
copies of the cache are rotated so that no step finds its cache in the 256 MB last-level cache.

With --paged BS the same workload is laid out in pages of BS positions placed by a seeded random
permutation (gqa_decode_paged); the KV bytes counted are the same.  With --append a step first writes
the new token's K and V rows (bf16, converted to the cache format: fp8 caches quantise) at position
seq_lens[b] - 1 of every sequence, then decodes; the KV bytes counted are the same.

With --prefill NAME (prefill-8b, prefill-70b) it instead times causal GQA prefill (gqa_prefill) and
reports matmul TFLOP/s against the bf16 matrix-core peak.

Prints one JSON line on stdout (diagnostics go to stderr).
"""
import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV GB/s and % HBM roofline for GQA decode (Hq=64,Hkv=8,d=128,bf16)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of an MI355X
# rocprofv3 counter summaries, keyed by (workload, page size) (page size 0 = dense cache)
TRAFFIC_SUMMARY = {(3, 0): os.path.join(ROOT, "profiles", "gqa_decode_llama70b_traffic.md"),
                   (3, 16): os.path.join(ROOT, "profiles", "gqa_decode_paged16_llama70b_traffic.md"),
                   (5, 0): os.path.join(ROOT, "profiles", "gqa_decode_long_fp8_trace_traffic_counters.md"),
                   (2, 0): os.path.join(ROOT, "profiles", "gqa_decode_llama3_8b_trace_traffic_counters.md")}
KERNEL_SOURCES = [os.path.join(ROOT, "grouped_query_attention_04_amd", "csrc", f)
                  for f in ("gqa_device.h", "gqa_kernels.h", "gqa_api.hip")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(wid, workgroups, paged=0):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on this
    workload, layout and launch configuration with the kernel sources as they are now; else None."""
    path = TRAFFIC_SUMMARY.get((wid, paged))
    if workgroups != 0 or path is None or not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo (empty when unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(case, groups_b, paged=None):
    """Time the fp64 oracle on every query head of batch entries [0, groups_b): once on one thread,
    once with the rows cut over every CPU this process may use (the same C code per row)."""
    from oracle import ref

    rows = [(b, h) for b in range(groups_b) for h in range(case["Hq"])]
    sl = case["seq_lens"].numpy()

    def run(threads):
        t0 = time.perf_counter()
        if paged is None:
            ref.decode_rows(case["q"], case["k"], case["v"], sl, case["scale"], rows, case["q_dtype"],
                            case["kv_dtype"], case["k_descale"], case["v_descale"], threads=threads)
        else:
            ref.decode_paged(case["q"], paged["k_pages"], paged["v_pages"], paged["block_table"].numpy(), sl,
                             case["scale"], rows, case["q_dtype"], case["kv_dtype"], case["k_descale"],
                             case["v_descale"], threads=threads)
        return time.perf_counter() - t0

    cores = ref.host_threads()
    dt_all = run(cores)
    dt_one = run(1)
    elt = 1 if case["kv_dtype"] == "fp8_e4m3" else (4 if case["kv_dtype"] == "f32" else 2)
    kv_bytes = int(sl[:groups_b].sum()) * case["Hkv"] * 2 * case["d"] * elt
    return {"value": round(kv_bytes / dt_all / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"all {case['Hq']} query heads of batch entries 0..{groups_b - 1} "
                      f"({groups_b * case['Hkv']} of {case['B'] * case['Hkv']} (batch, KV head) groups, "
                      f"{kv_bytes / 1e6:.1f} MB of KV): {dt_all:.2f} s with the rows cut over {cores} threads, "
                      f"{dt_one:.1f} s on one",
            "single_thread": {"value": round(kv_bytes / dt_one / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "seconds": round(dt_one, 2)},
            "cpu_model": cpu_model() or "unnamed", "cpus_online": os.cpu_count()}


def prefill_cpu_baseline(case, nrows=4000):
    """Time the fp64 oracle on a sample of causal prefill rows, as TFLOP/s: on one thread and with
    the rows cut over every CPU this process may use."""
    from oracle import ref

    import numpy as np

    w = case["workload"]
    random_rows = []
    gen = np.random.default_rng(7)
    for _ in range(nrows):
        random_rows.append((int(gen.integers(w.B)), int(gen.integers(w.Hq)), int(gen.integers(w.S))))
    flops = sum(4 * w.d * (i + 1) for _, _, i in random_rows)

    def run(threads):
        t0 = time.perf_counter()
        ref.prefill(case["q"], case["k"], case["v"], case["scale"], "bf16", True, rows=random_rows,
                    threads=threads)
        return time.perf_counter() - t0

    cores = ref.host_threads()
    dt_all = run(cores)
    dt_one = run(1)
    return {"value": round(flops / dt_all / 1e12, 8), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{nrows} random (batch, head, position) rows of the same prompt, "
                      f"{flops / 1e9:.2f} GFLOP: {dt_all:.2f} s on {cores} threads, {dt_one:.1f} s on one",
            "single_thread": {"value": round(flops / dt_one / 1e12, 8), "unit": "TFLOP/s", "cores": 1,
                              "seconds": round(dt_one, 2)},
            "cpu_model": cpu_model() or "unnamed", "cpus_online": os.cpu_count()}


def launch_stats(step, stream, nsteps, per_block=10):
    """Per-step device time of back-to-back launches, from HIP events on the launch stream around
    blocks of `per_block` launches: median, p10 and p90 over the blocks (microseconds).  One event
    pair per block keeps the events' own cost out of the per-launch figure."""
    import torch

    nblocks = max(10, nsteps // per_block)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nblocks)]
    i = 0
    for a, b in ev:
        a.record(stream)
        for _ in range(per_block):
            step(i)
            i += 1
        b.record(stream)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 / per_block for a, b in ev)
    n = len(us)
    return {"median": round(us[n // 2], 3), "p10": round(us[n // 10], 3), "p90": round(us[(9 * n) // 10], 3),
            "blocks": n, "launches_per_block": per_block}


def end_to_end_us(step, n=50):
    """Host time of one call issued and completed alone (launch included): median over n calls."""
    import torch

    t = []
    for i in range(n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        step(i)
        torch.cuda.synchronize()
        t.append((time.perf_counter() - t0) * 1e6)
    t.sort()
    return round(t[len(t) // 2], 2)


def bench_prefill(args):
    import torch

    import grouped_query_attention_04_amd as gqa
    import workloads

    w = workloads.PREFILL_WORKLOADS[args.prefill]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"prefill {args.prefill}: {w.name}; generating inputs")
    case = workloads.make_prefill(args.prefill)
    q, k, v = (case[n].to(dev) for n in ("q", "k", "v"))
    out = torch.empty_like(q)
    shape = gqa.PrefillShape(w.B, w.Hq, w.Hkv, w.S, w.d, gqa.BF16, gqa.BF16, 1)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    shape_ref = ctypes.byref(shape)
    scale = float(case["scale"])

    def step():
        rc = gqa.lib.gqa_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), scale, out.data_ptr(), shape_ref, sh)
        if rc:
            raise RuntimeError(gqa.status_string(rc))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    value = w.flops / (ms_per_step * 1e-3) / 1e12
    lt = launch_stats(lambda i: step(), stream, args.steps, per_block=5)
    achieved = w.flops / (lt["median"] * 1e-6) / 1e12
    log(f"step {ms_per_step * 1e3:.1f} us wall ({value:.1f} TFLOP/s); per launch median {lt['median']:.1f} us "
        f"(p10 {lt['p10']:.1f}, p90 {lt['p90']:.1f}); "
        f"{achieved:.1f} TFLOP/s = {100 * achieved / MFMA_BF16_PEAK_TFLOPS:.1f}% of the bf16 MFMA peak")
    result = {
        "metric": "causal GQA prefill TFLOP/s (bf16)", "value": round(value, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "S": w.S,
                   "causal": True, "flops_per_step": w.flops, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None},
        "launch_us": lt,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of the same prompt")
        result["cpu_baseline"] = prefill_cpu_baseline(case)
    print(json.dumps(result), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="3", help="workload id (1, 2, 3, 4-mha, 4-gqa, 4-mqa, 5, 3-tp8, 3-d64)")
    ap.add_argument("--copies", type=int, default=0, help="cache copies rotated (0 = enough for 2 GiB)")
    ap.add_argument("--workgroups", type=int, default=0, help="workgroups (0 = library choice)")
    ap.add_argument("--prefill", default="", metavar="NAME",
                    help="time causal prefill instead (prefill-8b or prefill-70b)")
    ap.add_argument("--append", action="store_true",
                    help="each step appends the new token's K/V rows before the decode")
    ap.add_argument("--fused", action="store_true",
                    help="with --append: one launch stores the new rows and decodes (gqa_decode_append)")
    ap.add_argument("--paged", type=int, default=0, metavar="BS",
                    help="lay the cache out in pages of BS positions (0 = dense cache)")
    ap.add_argument("--mean-lengths", action="store_true",
                    help="give every sequence the workload's mean length (a stable trend line)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-batches", type=int, default=32)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain torch copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: libgqa has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        return 2

    if args.prefill:
        return bench_prefill(args)

    import torch

    import grouped_query_attention_04_amd as gqa
    import workloads

    wid = int(args.workload) if args.workload.isdigit() else args.workload
    w = workloads.WORKLOADS[wid]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"workload {wid}: {w.name}; generating inputs")
    case = workloads.make(wid)
    if args.mean_lengths:
        n = int(round(float(case["seq_lens"].double().mean())))
        case["seq_lens"] = torch.full_like(case["seq_lens"], n)
        log(f"every sequence set to the mean length {n}")
    elt = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[w.kv_dtype]
    sl = case["seq_lens"]
    kv_bytes = int(sl.sum()) * w.Hkv * 2 * w.d * elt
    paged = None
    if args.paged:
        paged = workloads.paginate(case, args.paged, seed=w.seed + 100)
        kc, vc = paged["k_pages"], paged["v_pages"]
    else:
        kc, vc = case["k"], case["v"]
    alloc = 2 * kc.numel() * elt
    copies = args.copies or max(2, -(-(2 << 30) // alloc))

    q = case["q"].to(dev)
    seq = sl.to(dev)
    ks = [kc.to(dev) for _ in range(copies)]
    vs = [vc.to(dev) for _ in range(copies)]
    od = workloads.TORCH_DTYPES[w.out_dtype]
    out = torch.empty(w.B, w.Hq, w.d, dtype=od, device=dev)
    code = {"f32": gqa.F32, "bf16": gqa.BF16, "fp8_e4m3": gqa.FP8_E4M3}
    if paged:
        table = paged["block_table"].to(dev)
        shape = gqa.make_paged_shape(w.B, w.Hq, w.Hkv, w.d, args.paged, table.shape[1], paged["num_blocks"],
                                     code[w.q_dtype], code[w.kv_dtype], code[w.out_dtype],
                                     num_workgroups=args.workgroups)
    else:
        shape = gqa.make_shape(w.B, w.Hq, w.Hkv, w.L, w.d, code[w.q_dtype], code[w.kv_dtype],
                               code[w.out_dtype], num_workgroups=args.workgroups)
    ws = gqa.new_workspace(shape, dev)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    shape_ref = ctypes.byref(shape)
    kptr = [t.data_ptr() for t in ks]
    vptr = [t.data_ptr() for t in vs]
    scale = float(case["scale"])

    if args.append:
        g = torch.Generator().manual_seed(w.seed + 200)
        k_new = torch.randn(w.B, w.Hkv, w.d, generator=g).to(torch.bfloat16).to(dev)
        v_new = torch.randn(w.B, w.Hkv, w.d, generator=g).to(torch.bfloat16).to(dev)
        positions = (sl - 1).clamp(min=-1).to(torch.int32).to(dev)
        ashape = shape

    if args.fused and not args.append:
        print("--fused times the fused append and decode: give --append too", file=sys.stderr)
        return 2

    def step(i):
        if args.fused:
            if paged:
                rc = gqa.lib.gqa_decode_append_paged(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                                     kptr[i % copies], vptr[i % copies], table.data_ptr(),
                                                     seq.data_ptr(), scale, out.data_ptr(), shape_ref, None,
                                                     ws.data_ptr(), ws.numel(), sh)
            else:
                rc = gqa.lib.gqa_decode_append(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), kptr[i % copies],
                                               vptr[i % copies], seq.data_ptr(), scale, out.data_ptr(), shape_ref,
                                               None, ws.data_ptr(), ws.numel(), sh)
            if rc:
                raise RuntimeError(gqa.status_string(rc))
            return
        if args.append:
            if paged:
                rc = gqa.lib.gqa_append_kv_paged(k_new.data_ptr(), v_new.data_ptr(), gqa.BF16, kptr[i % copies],
                                                 vptr[i % copies], table.data_ptr(), ctypes.byref(ashape),
                                                 positions.data_ptr(), None, sh)
            else:
                rc = gqa.lib.gqa_append_kv(k_new.data_ptr(), v_new.data_ptr(), gqa.BF16, kptr[i % copies],
                                           vptr[i % copies], ctypes.byref(ashape), positions.data_ptr(), None, sh)
            if rc:
                raise RuntimeError(gqa.status_string(rc))
        if paged:
            rc = gqa.lib.gqa_decode_paged(q.data_ptr(), kptr[i % copies], vptr[i % copies], table.data_ptr(),
                                          seq.data_ptr(), scale, out.data_ptr(), shape_ref, ws.data_ptr(),
                                          ws.numel(), sh)
        else:
            rc = gqa.lib.gqa_decode(q.data_ptr(), kptr[i % copies], vptr[i % copies], seq.data_ptr(), scale,
                                    out.data_ptr(), shape_ref, ws.data_ptr(), ws.numel(), sh)
        if rc:
            raise RuntimeError(gqa.status_string(rc))

    log(f"{copies} cache copies of {alloc / 2**20:.0f} MiB; KV bytes per step {kv_bytes / 1e6:.1f} MB; "
        f"workgroups {args.workgroups or 'auto'}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K back-to-back steps between two device synchronisations (host clock), with one
    # HIP event pair on the launch stream around the whole region
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(args.steps):
        step(i)
    r1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    region_us = r0.elapsed_time(r1) * 1e3 / args.steps

    # per-launch device time for the roofline figure: the median over blocks of back-to-back launches
    lt = launch_stats(step, stream, max(args.steps, 200))
    lt["region_avg"] = round(region_us, 3)
    achieved = kv_bytes / (lt["median"] * 1e-6) / 1e9
    e2e = end_to_end_us(step)
    log(f"step {ms_per_step * 1e3:.1f} us wall ({value:.0f} GB/s); per launch median {lt['median']:.1f} us "
        f"(p10 {lt['p10']:.1f}, p90 {lt['p90']:.1f}; timed-region average {region_us:.1f}); "
        f"{achieved:.0f} GB/s = {100 * achieved / HBM_PEAK_GBS:.1f}% of 8 TB/s; one call alone, launch included, "
        f"{e2e:.1f} us")

    # achievable streaming-read bandwidth on one cache copy, for context
    sink = torch.empty(gqa.lib.gqa_stream_read_sink_words(), dtype=torch.int32, device=dev)
    for i in range(3):
        gqa.stream_read(ks[i % copies], sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(10):
        gqa.stream_read(ks[i % copies], sink)
        gqa.stream_read(vs[i % copies], sink)
    e1.record(stream)
    torch.cuda.synchronize()
    calib = 20 * ks[0].numel() * elt / (e0.elapsed_time(e1) * 1e-3) / 1e9
    log(f"calibration: non-temporal streaming read of the cache copies {calib:.0f} GB/s")

    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.calib_copy_mib} MiB done")

    traffic = None if args.mean_lengths else recorded_traffic(wid, args.workgroups, args.paged)
    layout = f"paged, {args.paged} positions per page, random page placement" if paged else "dense"
    if args.append:
        layout += ("; each step appends the new token's K/V (bf16 rows) and decodes, in one launch" if args.fused
                   else "; each step appends the new token's K/V (bf16 rows) then decodes")
        traffic = None
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.kv_dtype, "data": "synthetic",
        "config": {"workload": w.name + (" mean lengths" if args.mean_lengths else "") + (f" paged bs{args.paged}" if paged else "") + (
                       (" fused append+decode" if args.fused else " append+decode") if args.append else ""),
                   "cache_layout": layout,
                   "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "L": w.L,
                   "seq_lens": f"sum {int(sl.sum())} (min {int(sl.min())}, max {int(sl.max())})",
                   "kv_bytes_per_step": kv_bytes, "cache_copies": copies,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "launch_us": lt,
        "end_to_end_us": e2e,
        "calibration_read_gbs": round(calib, 1),
        # measured HBM bytes per launch over the algorithmic KV bytes: ~1.0 means the cache is read
        # once for all query heads of a group; about G would mean the heads re-read it
        "traffic_per_kv_byte": None if traffic is None else round(traffic / kv_bytes, 4),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of the same workload")
        result["cpu_baseline"] = cpu_baseline(case, min(args.cpu_sample_batches, w.B), paged)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
