"""Benchmark: MXFP4-KV absorbed-MLA decode on one MI355X.

A step is one decode call (split-K decode kernel + reduce kernel when some
sequence is split) over one batch of synthetic inputs already resident in
HBM. Default workload: B=256 sequences x 8192 tokens (641.7 MB of packed KV +
E8M0 scales). Prints one JSON line with the metric (KV-cache GB/s), us/call,
the roofline of the decode kernel (HIP-event timing on the launch stream) and
the CPU oracle timed on a bounded sample as a reported baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import torch

from mla_mxfp4_kv_amd import binding, synth

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRC = {
    "mxfp4": os.path.join(ROOT, "mla_mxfp4_kv_amd", "csrc", "mla_kernels.hip"),
    "fp8": os.path.join(ROOT, "mla_mxfp4_kv_amd", "csrc", "mla_dense_kernels.hip"),
    "bf16": os.path.join(ROOT, "mla_mxfp4_kv_amd", "csrc", "mla_dense_kernels.hip"),
    "mxfp4_24": os.path.join(ROOT, "mla_mxfp4_kv_amd", "csrc", "mla_mxfp4_24_kernels.hip"),
}
KERNEL_NAME = {"mxfp4": "mla_decode_kernel<false, false, false>", "fp8": "mla_decode_dense_kernel<true, false>",
               "bf16": "mla_decode_dense_kernel<false, false>", "mxfp4_24": "mla_decode_mxfp4_24_kernel"}
GATHER_KERNEL_NAME = {"mxfp4": "mla_decode_kernel<true, false, false>", "fp8": "mla_decode_dense_kernel<true, true>",
                      "bf16": "mla_decode_dense_kernel<false, true>"}
PAGE_TABLE_KERNEL_NAME = dict(GATHER_KERNEL_NAME, mxfp4="mla_decode_kernel<true, true, false>")
STARTS_KERNEL_NAME = dict(KERNEL_NAME, mxfp4="mla_decode_kernel<false, false, true>")


def kernel_source_hash(fmt: str = "mxfp4") -> str:
    with open(KERNEL_SRC[fmt], "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _profile_name(workload: str, fmt: str) -> str:
    return f"decode_{workload}" if fmt == "mxfp4" else f"decode_{fmt}_{workload}"


def measured_traffic(workload: str, fmt: str = "mxfp4"):
    """HBM bytes per decode launch from the committed rocprofv3 counter
    summary of this workload, if it was taken on the current kernel source
    (else None)."""
    path = os.path.join(ROOT, "profiles", f"{_profile_name(workload, fmt)}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash(fmt):
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profiled_kernel_us(workload: str, fmt: str = "mxfp4"):
    """Average duration of the decode kernel in the committed rocprofv3 trace
    summary of this workload, if it was taken on the current kernel source
    (else None)."""
    path = os.path.join(ROOT, "profiles", f"{_profile_name(workload, fmt)}_kernel_trace.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash(fmt):
        return None
    try:
        return float(fields["decode_kernel_avg_us"])
    except (KeyError, ValueError):
        return None


def read_probe_gbs(nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Read bandwidth a plain device reduction over ``nbytes`` reaches on this
    box (HIP events), the practical ceiling the decode's stream is compared
    with."""
    words = torch.ones(nbytes // 8, dtype=torch.int64, device="cuda")
    words.sum()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        words.sum()
    e1.record()
    torch.cuda.synchronize()
    gbs = nbytes / (e0.elapsed_time(e1) * 1e-3 / reps) / 1e9
    del words
    return gbs


def copy_probe(nbytes: int, reps: int) -> int:
    """Plain device-to-device copy of a known size (calibrates the
    FETCH_SIZE / WRITE_SIZE counters against bytes actually moved) and a
    read-only pass over it, each timed with HIP events: the bandwidth a
    plain copy / read reaches on this machine."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    words = src.view(torch.int64)
    words.sum()
    torch.cuda.synchronize()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    for _ in range(reps):
        words.sum()
    e2.record()
    torch.cuda.synchronize()
    copy_s = e0.elapsed_time(e1) * 1e-3 / reps
    read_s = e1.elapsed_time(e2) * 1e-3 / reps
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps,
                      "copy_gbs_read_plus_write": round(2 * nbytes / copy_s / 1e9, 1),
                      "read_gbs": round(nbytes / read_s / 1e9, 1)}), flush=True)
    return 0
QO_BYTES_PER_SEQ = 16 * 576 * 2 + 16 * 512 * 2
PARTIAL_BYTES = 16 * (512 + 1) * 4


def algorithmic_bytes(words, total_tokens, fmt="mxfp4", gather=False, pages=None):
    """Bytes the decode must move: KV (+ scales), Q, output, each split
    partial written once and read once, and with a gathered cache the
    4-byte row index of every token (or, through a page table, the 4-byte
    entry of every page: ``pages`` entries)."""
    num_partials = words[9]
    batch = words[2]
    index = 4 * pages if pages is not None else (4 * total_tokens if gather else 0)
    return (synth.kv_bytes(total_tokens, fmt) + batch * QO_BYTES_PER_SEQ
            + 2 * num_partials * PARTIAL_BYTES + index)


def cpu_baseline(w, q, packed, scales, lens, budget_s, fmt="mxfp4", kv_scale=None):
    """Time the fp64 oracle (as it stands) on whole sequences of the same
    workload until about ``budget_s`` seconds of CPU work."""
    import numpy as np
    from oracle import dense_ref, mxfp4_24_ref, mxfp4_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = torch.get_num_threads()
    cpu_count = os.cpu_count()
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = cpu_count
    qb = q.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    ind = [0]
    for n in lens:
        ind.append(ind[-1] + n)
    done_tokens = 0
    n_seq = 0
    oracle_s = 0.0
    for b in range(len(lens)):
        lo, hi = ind[b], ind[b + 1]
        if fmt in ("mxfp4", "mxfp4_24"):
            pk = packed[lo:hi].cpu().numpy()
            sc = scales[lo:hi].cpu().numpy()
            t0 = time.perf_counter()          # device->host copies are not timed
            if fmt == "mxfp4":
                mxfp4_ref.mla_decode_ref_seq(qb[b], pk, sc, w.sm_scale)
            else:
                mxfp4_24_ref.mla_decode_ref_24_seq(qb[b], pk, sc, w.sm_scale)
        elif fmt == "fp8":
            rows = packed[lo:hi].cpu().numpy()
            t0 = time.perf_counter()
            dense_ref.mla_decode_ref_fp8_seq(qb[b], rows, kv_scale, w.sm_scale)
        else:
            rows = packed[lo:hi].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
            t0 = time.perf_counter()
            dense_ref.mla_decode_ref_bf16_seq(qb[b], rows, w.sm_scale)
        oracle_s += time.perf_counter() - t0
        done_tokens += hi - lo
        n_seq += 1
        if oracle_s >= budget_s:
            break
    gbs = synth.kv_bytes(done_tokens, fmt) / oracle_s / 1e9
    return {
        "value": round(gbs, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "cpu_count": cpu_count,
        "affinity_cores": affinity,
        "blas_threads": int(threads),
        "kind": "oracle",
        "sample": f"first {n_seq} of {len(lens)} sequences ({done_tokens} tokens) of {w.name} ({fmt} cache), "
                  f"{oracle_s:.1f} s, us/call extrapolated "
                  f"{oracle_s / done_tokens * sum(lens) * 1e6:.0f}",
    }


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="b256_kv8192", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--kv-format", default="mxfp4", choices=["mxfp4", "fp8", "bf16", "mxfp4_24"],
                    help="cache format: the MXFP4 path (18 scales per token), the 24-scale MXFP4 "
                         "layout, or the fp8 / bf16 sibling decodes")
    ap.add_argument("--gather", type=int, default=0, metavar="PAGE",
                    help="scatter the rows over the pool in pages of PAGE rows (seeded shuffle) and "
                         "decode through per-token kv_indices (the *_paged entry points)")
    ap.add_argument("--page-table", type=int, default=0, metavar="PAGE",
                    help="store every sequence in pages of PAGE rows (the last one partial), pages "
                         "shuffled over the pool (seeded), and decode through the page table (the "
                         "*_page_table entry points)")
    ap.add_argument("--groups", type=int, default=0, metavar="G",
                    help="G 16-head query entries per sequence over its shared rows (8: 128 heads; "
                         "q_seq_len tokens: G = q_seq_len), the *_starts entry points")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the cpu_baseline (0 = skip)")
    ap.add_argument("--cold", action="store_true",
                    help="time the K steps with cold caches (a 1 GB read before every call evicts L2 and "
                         "MALL; the read leaves clean lines, so the decode pays no write-backs). Without it "
                         "the K steps run back to back and a cold pass of K calls is reported beside them")
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="seconds of untimed decode calls before the warm-up steps: a fresh process first "
                         "runs through the GPU's clock/power transient (calls 2-8 fast, the next ~30 ~40%% "
                         "slower, steady after ~300), which a short warm-up would otherwise time")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache pass")
    ap.add_argument("--graph", action="store_true",
                    help="time the K steps as one HIP-graph replay of K captured calls (no host launch cost "
                         "between calls: what a serving loop that replays graphs sees); without it the calls "
                         "are launched from Python one by one, which bounds small workloads by the host")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures the decode kernel on one GPU; runs over several GPUs are not "
              "implemented (the decode would shard by sequence: each GPU plans and decodes its own). Use --gpus 1.",
              file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a HIP GPU", file=sys.stderr)
        return 2
    if args.copy_probe:
        return copy_probe(args.copy_probe, max(1, args.steps))

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fmt = args.kv_format
    print(f"[bench] generating {w.name} ({fmt} cache)", file=sys.stderr, flush=True)
    if fmt in ("mxfp4", "mxfp4_24"):
        q, packed, scales, indptr, lens = synth.make_inputs(w, device=dev, block=24 if fmt == "mxfp4_24" else 32)
        kv_scale_host = None
    else:
        # `packed` holds the cache rows, `scales` the fp8 per-tensor scale
        q, packed, scales, indptr, lens = synth.make_dense_inputs(w, fmt, device=dev)
        kv_scale_host = float(scales[0]) if fmt == "fp8" else None
    total = int(indptr[-1])
    t_plan = time.perf_counter()
    dec = binding.MlaDecode(indptr.tolist(), device=dev)
    plan_first_ms = (time.perf_counter() - t_plan) * 1e3   # includes the library's one-time HIP set-up
    t_plan = time.perf_counter()
    binding.plan(indptr.tolist(), dec.workspace)            # the steady-state host plan of this indptr
    plan_ms = (time.perf_counter() - t_plan) * 1e3
    words, _ = binding.plan_host(indptr.tolist(), binding.num_cus())
    out = torch.empty(w.batch, 16, 512, dtype=torch.bfloat16, device=dev)
    kv_indices = None
    if args.gather:
        page = args.gather
        if total % page:
            print(f"--gather {page}: the token count {total} is not a multiple of the page", file=sys.stderr)
            return 2
        g = torch.Generator().manual_seed(1234)
        perm = torch.randperm(total // page, generator=g).to(torch.int32)
        kv_indices = (perm.repeat_interleave(page) * page
                      + torch.arange(page, dtype=torch.int32).repeat(total // page)).to(dev)
        pool_p = torch.empty_like(packed)
        pool_p[kv_indices.long()] = packed
        if fmt == "mxfp4":
            pool_s = torch.empty_like(scales)
            pool_s[kv_indices.long()] = scales
            scales = pool_s
        packed = pool_p
        binding.check_kv_indices(kv_indices, indptr.tolist(), packed.shape[0],
                                 packed.shape[1] * packed.element_size())
        torch.cuda.synchronize()
    page_table = None
    groups = None
    if args.groups:
        if args.gather or args.page_table:
            print("--groups works on the contiguous cache only", file=sys.stderr)
            return 2
        groups = binding.MlaDecodeGroups(indptr.tolist(), args.groups, device=dev)
        gq = torch.Generator(device="cpu").manual_seed(w.seed + 1)
        q = (torch.randn(groups.batch, 16, 576, generator=gq) * w.q_std).to(torch.bfloat16).to(dev)
        out = torch.empty(groups.batch, 16, 512, dtype=torch.bfloat16, device=dev)
        dec = groups.plan
        words, _ = binding.plan_host(dec.indptr_host, groups.num_cus)

        def call():
            binding.decode_starts(fmt, q, packed, scales, groups.kv_start, dec.kv_indptr, out, w.sm_scale,
                                  dec.workspace)
    elif args.page_table:
        if args.gather:
            print("--gather and --page-table are exclusive", file=sys.stderr)
            return 2
        ps = args.page_table
        lens_t = torch.tensor([int(n) for n in lens], dtype=torch.int64)
        npages = (lens_t + ps - 1) // ps
        pi = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(npages, 0)])
        last = torch.where(npages > 0, lens_t - (npages - 1) * ps, torch.zeros_like(lens_t))
        g = torch.Generator().manual_seed(1234)
        pages = torch.randperm(int(pi[-1]), generator=g).to(torch.int32)
        # token -> pool row: page of the token's run within its sequence
        seq = torch.repeat_interleave(torch.arange(w.batch), lens_t)
        rel = torch.arange(total) - torch.as_tensor(indptr.tolist()[:-1], dtype=torch.int64)[seq]
        rows = pages[pi[seq] + rel // ps].to(torch.int64) * ps + rel % ps
        rows = rows.to(dev)
        pool_p = torch.empty((int(pi[-1]) * ps,) + tuple(packed.shape[1:]), dtype=packed.dtype, device=dev)
        pool_p[rows] = packed
        if fmt == "mxfp4":
            pool_s = torch.empty((pool_p.shape[0], scales.shape[1]), dtype=scales.dtype, device=dev)
            pool_s[rows] = scales
            scales = pool_s
        packed = pool_p
        page_table = binding.MlaDecodePageTable(pi.tolist(), last.tolist(), ps, device=dev)
        pages_dev = pages.to(dev)
        binding.check_page_table(pages_dev, pi.tolist(), last.tolist(), ps, packed.shape[0],
                                 packed.shape[1] * packed.element_size())
        torch.cuda.synchronize()
        dec = page_table.plan

        def call():
            binding.decode_page_table(fmt, q, packed, scales, pages_dev, page_table.page_indptr, ps,
                                      dec.kv_indptr, out, w.sm_scale, dec.workspace)
    elif kv_indices is not None and fmt == "mxfp4":
        def call():
            binding.decode_mxfp4_paged(q, packed, scales, kv_indices, dec.kv_indptr, out, w.sm_scale,
                                       dec.workspace)
    elif kv_indices is not None and fmt == "fp8":
        def call():
            binding.decode_fp8_paged(q, packed, scales, kv_indices, dec.kv_indptr, out, w.sm_scale, dec.workspace)
    elif kv_indices is not None:
        def call():
            binding.decode_bf16_paged(q, packed, kv_indices, dec.kv_indptr, out, w.sm_scale, dec.workspace)
    elif fmt == "mxfp4":
        def call():
            dec(q, packed, scales, out=out, sm_scale=w.sm_scale)
    elif fmt == "mxfp4_24":
        if args.gather or args.page_table or args.groups:
            print("the 24-scale layout is decoded from contiguous rows only", file=sys.stderr)
            return 2

        def call():
            dec.mxfp4_24(q, packed, scales, out=out, sm_scale=w.sm_scale)
    elif fmt == "fp8":
        def call():
            dec.fp8(q, packed, scales, out=out, sm_scale=w.sm_scale)
    else:
        def call():
            dec.bf16(q, packed, out=out, sm_scale=w.sm_scale)
    flush_buf = None if args.no_cold and not args.cold else torch.ones(1 << 27, dtype=torch.int64, device=dev)
    flush = flush_buf if args.cold else None

    settle_calls = 0
    if args.settle_s > 0:
        print(f"[bench] settling clocks for {args.settle_s} s", file=sys.stderr, flush=True)
        t_end = time.perf_counter() + args.settle_s
        while time.perf_counter() < t_end:
            for _ in range(10):
                call()
            settle_calls += 10
            torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    graph = None
    if args.graph:
        if flush is not None:
            print("--graph and --cold are exclusive", file=sys.stderr)
            return 2
        # capture on a side stream (the decode launches on the current stream)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                call()
        graph.replay()
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
    if graph is not None:
        ev_a = torch.cuda.Event(enable_timing=True)
        ev_b = torch.cuda.Event(enable_timing=True)
        ev_a.record(stream)
        graph.replay()
        ev_b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        avg_us = ev_a.elapsed_time(ev_b) * 1e3 / args.steps
    elif flush is None:
        # back-to-back calls, one event pair around the whole timed region
        ev_a = torch.cuda.Event(enable_timing=True)
        ev_b = torch.cuda.Event(enable_timing=True)
        ev_a.record(stream)
        for _ in range(args.steps):
            call()
        ev_b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        avg_us = ev_a.elapsed_time(ev_b) * 1e3 / args.steps
    else:
        # cold caches: the flush before each call is kept out of its event pair
        ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        for i in range(args.steps):
            flush.sum()
            ev0[i].record(stream)
            call()
            ev1[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        avg_us = statistics.fmean(a.elapsed_time(b) * 1e3 for a, b in zip(ev0, ev1))

    # spread of single calls (an event pair around each call), after the timed region
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        if flush is not None:
            flush.sum()
        ev0[i].record(stream)
        call()
        ev1[i].record(stream)
    torch.cuda.synchronize()
    call_us = [a.elapsed_time(b) * 1e3 for a, b in zip(ev0, ev1)]
    med_us = statistics.median(call_us)
    # the other cache state: cold calls beside a warm timed region, or
    # back-to-back calls beside a cold one
    other = None
    if flush_buf is not None and not args.cold:
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        for i in range(args.steps):
            flush_buf.sum()
            e0[i].record(stream)
            call()
            e1[i].record(stream)
        torch.cuda.synchronize()
        cold_us = sorted(a.elapsed_time(b) * 1e3 for a, b in zip(e0, e1))
        other = {"mode": "cold (1 GB read before each call)", "us_per_call_mean": round(statistics.fmean(cold_us), 2),
                 "us_per_call_median": round(statistics.median(cold_us), 2),
                 "us_p10_p90": [round(cold_us[int(0.1 * (len(cold_us) - 1))], 2),
                                round(cold_us[int(0.9 * (len(cold_us) - 1))], 2)]}
    elif args.cold:
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea.record(stream)
        for _ in range(args.steps):
            call()
        eb.record(stream)
        torch.cuda.synchronize()
        other = {"mode": "warm (back to back)", "us_per_call_mean": round(ea.elapsed_time(eb) * 1e3 / args.steps, 2)}
    read_gbs = read_probe_gbs() if not args.groups else None
    ms_per_step = wall / args.steps * 1e3
    kvb = synth.kv_bytes(total, fmt)
    # whole-job throughput (wall clock over the timed steps); with --cold the
    # wall clock includes the flushes, so the event time is used instead
    step_s = (avg_us * 1e-6) if args.cold else (wall / args.steps)
    value = kvb / step_s / 1e9
    alg = algorithmic_bytes(words, total, fmt, kv_indices is not None,
                            page_table.page_indptr_host[-1] if page_table is not None else None)
    achieved = alg / (avg_us * 1e-6) / 1e9

    prof_us = None if (args.gather or args.page_table or args.groups) else profiled_kernel_us(w.name, fmt)
    cpu = None
    if args.cpu_budget > 0 and not args.groups:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, q, packed, scales, lens, args.cpu_budget, fmt, kv_scale_host)

    line = {
        "metric": "KV-cache HBM GB/s (us/call), MXFP4 MLA decode" if fmt == "mxfp4"
                  else "KV-cache HBM GB/s (us/call), MXFP4 (24 scales per token) MLA decode" if fmt == "mxfp4_24"
                  else f"KV-cache HBM GB/s (us/call), {fmt} MLA decode",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(avg_us, 2),
        "single_call_us_median": round(med_us, 2),
        "single_call_us_p10_p90": [round(sorted(call_us)[int(0.1 * (len(call_us) - 1))], 2),
                                round(sorted(call_us)[int(0.9 * (len(call_us) - 1))], 2)],
        "plan_ms": round(plan_ms, 3),
        "plan_first_call_ms": round(plan_first_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"mxfp4": "bf16 (MXFP4 e2m1/E8M0 KV; latent QK on the scaled fp4 x e4m3 hi+lo MFMA, whose "
                           "128-wide steps sum within 1.2e-4 x sum|terms| (pinned) and add up in fp32; rope QK "
                           "and P V on the bf16 MFMA, fp32 accumulate; P rounded to bf16)",
                  "fp8": "bf16 (fp8 e4m3 KV + per-tensor scale, fp32 accumulate)",
                  "bf16": "bf16 (bf16 KV, fp32 accumulate)",
                  "mxfp4_24": "bf16 (MXFP4 e2m1 KV with 24 E8M0 scales per token, decoded to bf16 for both "
                              "bf16 MFMA products, fp32 accumulate)"}[fmt],
        "data": "synthetic",
        "cold": bool(args.cold),
        "timing": "HIP-graph replay of the K calls" if args.graph else
                  ("per-call event pairs, cold caches" if args.cold else "back-to-back calls launched from Python"),
        "config": {
            "workload": w.name,
            "kv_format": fmt,
            "gather_page_rows": args.gather or None,
            "page_table_rows": args.page_table or None,
            "query_groups": args.groups or None,
            "batch": w.batch,
            "kv_len": w.kv_len if w.kv_len is not None else f"U{list(w.ragged)}",
            "total_tokens": total,
            "heads": 16,
            "qk_dim": 576,
            "v_dim": 512,
            "kv_bytes": kvb,
            "num_partials": words[9],
            "num_slots": words[7],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if (args.gather or args.page_table or args.groups) else measured_traffic(w.name, fmt),
            "kernel": (PAGE_TABLE_KERNEL_NAME[fmt] if args.page_table
                       else GATHER_KERNEL_NAME[fmt] if args.gather
                       else STARTS_KERNEL_NAME[fmt] if args.groups else KERNEL_NAME[fmt]),
            "bytes_per_launch": alg,
            "kv_frac": round(kvb / (avg_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_source_sha256": kernel_source_hash(fmt),
            # the event time covers the whole call: the decode kernel alone
            # when no sequence is split (no reduce launch), else decode + reduce
            "time_source": "HIP events on the decode stream, " + (
                "decode kernel only (no reduce launch in this plan)" if words[10] == 0
                else "decode + reduce kernels"),
            "read_probe_gbs": round(read_gbs, 1) if read_gbs else None,
            "frac_of_read_probe": round(achieved / read_gbs, 4) if read_gbs else None,
            "profiled_kernel_us": prof_us,
            "profiled_frac": round(alg / (prof_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) if prof_us else None,
        },
        "other_cache_state": other,
        "clock_settle": {"seconds": args.settle_s, "calls": settle_calls},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
