"""Benchmark of the scheduled-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the whole hot path on one batch of synthetic input that
is already resident in HBM: the GPU schedule build from lane (0, 0)'s keys
(centroids, distances, MST + elder rule + top-k + CSR) followed by the
scheduled attention forward over every lane.  Prints ONE JSON line.

value = visited-block flops (4 * 64 * 64 * D per visited block and lane, full
tiles) / step time, in TFLOP/s.  The attention kernel is also timed on its own
(HIP events on the stream it runs on, around every launch in the timed region)
for the roofline entry, and the same kernel over the dense causal CSR gives the
sparse-vs-dense-CSR speedup.  The fp64 CPU oracle is timed on a bounded sample
of the same workload (cpu_baseline), and the lanes it computes are compared with
the output of the last timed step (parity: max abs error, max |O|, CSR equality);
the bench exits non-zero when that check fails.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scheduled-attn fwd effective TFLOP/s (% MFMA peak) + sparse/dense-CSR speedup"
PEAK_TFLOPS = {"fp16": 2500.0, "bf16": 2500.0}  # MI355X dense MFMA, published
PARITY_BAR = {"fp16": 2e-3, "bf16": 1e-2}  # max abs error of the output against the fp64 oracle
# sources of the attention forward kernels (their files and the shared device helpers)
ATTN_SOURCES = [os.path.join(ROOT, "block_sparse_causal_amd", "csrc", f)
                for f in ("attention_fwd.hip", "attention_fwd_duo.hip", "mfma_tile.h")]


def _kernel_hash() -> str:
    h = hashlib.sha256()
    for path in ATTN_SOURCES:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _profile_fields(name: str):
    """key: value lines of a committed rocprofv3 summary under profiles/, or None
    when it is missing or was taken on another attention kernel source."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256_16") != _kernel_hash():
        return None
    return fields


def _traffic(workload: str):
    """HBM bytes per attention launch from a committed rocprofv3 --pmc summary,
    only if it was taken on the current kernel source."""
    fields = _profile_fields(f"attention_fwd_{workload}_pmc.txt")
    try:
        return float(fields["hbm_bytes_per_launch"]) if fields else None
    except (KeyError, ValueError):
        return None


def _sq_counters(workload: str):
    """Matrix-core and VALU counters of the attention kernel from a committed
    rocprofv3 --pmc summary (per launch), only if it was taken on the current
    kernel source."""
    fields = _profile_fields(f"attention_fwd_{workload}_sq.txt")
    if not fields:
        return None
    keys = ("mfma_busy_frac", "clock_ghz", "valu_insts_per_mfma", "trans_insts_per_mfma",
            "wait_inst_frac", "kernel_us")
    try:
        return {key: float(fields[key]) for key in keys}
    except (KeyError, ValueError):
        return None


def _cpu_baseline(w, q, k, v, budget_s: float, gpu_out=None, gpu_csr=None):
    """Time the oracle on the host: schedule build (all pairs) + dense masked
    attention lane by lane until the time budget is used (at least one lane).

    When the GPU's output of the timed launch (and its CSR) is given, the oracle
    lanes just computed are also compared with it: max abs error, max |O|, and
    whether the GPU-built CSR equals the oracle's bit for bit."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    ql, kl, vl = (t.reshape(-1, w.S, w.D) for t in (q, k, v))
    t0 = time.perf_counter()
    if w.dense:
        rp, ci = oracle.dense_causal_schedule(w.nb)
    else:
        rp, ci, _ = oracle.build_schedule(kl[0], 64, w.sink, w.local_radius, w.topk)
    lanes = 0
    outs = []
    for lane in range(ql.shape[0]):
        outs.append(oracle.masked_attention(ql[lane], kl[lane], vl[lane], rp, ci, 64))
        lanes += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    parity = None
    if gpu_out is not None:
        got = gpu_out.reshape(-1, w.S, w.D)[:lanes].double().numpy()
        want = np.stack(outs)
        grp, gci = gpu_csr
        parity = {
            "max_abs_err": float(np.abs(got - want).max()),
            "max_abs_out": float(np.abs(want).max()),
            "lanes_checked": lanes,
            "rows_per_lane": w.S,
            "csr_bit_exact": bool(np.array_equal(grp, rp) and np.array_equal(gci, ci)),
        }
    flops = lanes * int(ci.shape[0]) * 4 * 64 * 64 * w.D
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"schedule build + {lanes} of {ql.shape[0]} lanes (all {w.S} rows each) in {dt:.1f} s; "
                  f"visited-block flops of those lanes / wall time; host has {os.cpu_count()} cpus",
        "seconds": dt,
        "lanes": lanes,
        "parity": parity,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy 10 times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        return 2

    import torch

    import block_sparse_causal_amd as tsa
    import workloads

    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_launch": 256 << 20,
                          "copy_calibration_bytes_written_per_launch": 256 << 20}))
        return 0

    name = args.workload or workloads.BENCH_WORKLOAD
    w = workloads.WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q_cpu, k_cpu, v_cpu = workloads.make_qkv(w)
    q, k, v = (t.to(dev) for t in (q_cpu, k_cpu, v_cpu))
    keys = k.reshape(-1, w.S, w.D)[0]
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)

    if w.dense:
        bufs = None
        rp, ci = tsa.dense_causal_schedule(w.nb, dev)

        def step():
            tsa.dense_causal_schedule(w.nb, dev)
    else:
        bufs = tsa.ScheduleBuffers(w.S, w.D, w.sink, w.local_radius, w.topk, dev)
        rp, ci = bufs.row_ptr, bufs.col_idx

        def step():
            tsa.build_schedule_into(keys, bufs)

    # The attention launches of every timed loop go through a prepared call: one C
    # ABI call each (about 7 us of host time, against 14 us through the binding),
    # so the host stays well ahead of the GPU.
    attention = tsa.prepare_scheduled_attention(q, k, v, rp, ci, out)

    print(f"# workload {name}: shape {w.shape} {w.dtype}; warmup {args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
        attention()
    torch.cuda.synchronize()
    nnz = int(rp[-1].item())
    lanes = w.lanes
    flops = lanes * nnz * 4 * 64 * 64 * w.D
    diag = w.nb
    flops_exact = lanes * 4 * w.D * (64 * 64 * (nnz - diag) + diag * (64 * 65 // 2))

    # Step pass: exactly K steps, events only at the two ends.  An event recorded
    # between two launches costs the GPU a few microseconds of idle time, so the
    # step pass carries none.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step()
        attention()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = start.elapsed_time(end) / args.steps
    print(f"# timed {args.steps} steps in {wall:.3f} s wall", file=sys.stderr, flush=True)

    # Kernel pass: the same K steps again, with events on the kernels' stream
    # before the schedule build, between it and the attention kernel, and after
    # that kernel.  Their means give the build time and the attention kernel's
    # launch duration behind the roofline figures.
    ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev_s[i].record(stream)
        step()
        ev_a[i].record(stream)
        attention()
        ev_b[i].record(stream)
    torch.cuda.synchronize()
    attn_ms_each = sorted(a.elapsed_time(b) for a, b in zip(ev_a, ev_b))
    attn_ms = sum(attn_ms_each) / len(attn_ms_each)
    build_ms = sum(s.elapsed_time(a) for s, a in zip(ev_s, ev_a)) / args.steps
    # The output and CSR of the last timed step, checked against the oracle below.
    timed_out = out.cpu()
    timed_csr = (rp.cpu().numpy(), ci[:nnz].cpu().numpy())

    # Same kernel over the dense causal CSR at the same shape (like-for-like
    # baseline), measured the way the kernel pass measures the workload's CSR:
    # each launch follows a schedule build, between two events.  Launch for
    # launch this is the regime of the timed steps; back-to-back launches of one
    # kernel run at a lower clock under sustained load (at the batched workload
    # the same topology-CSR launch takes about 71 us after a build and about 83
    # us after another attention launch).
    drp, dci = tsa.dense_causal_schedule(w.nb, dev)
    dense_attention = tsa.prepare_scheduled_attention(q, k, v, drp, dci, out)
    for _ in range(max(3, args.warmup // 2)):
        step()
        dense_attention()
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step()
        ev_a[i].record(stream)
        dense_attention()
        ev_b[i].record(stream)
    torch.cuda.synchronize()
    dense_ms = sum(a.elapsed_time(b) for a, b in zip(ev_a, ev_b)) / args.steps
    sparse_ms = attn_ms

    def in_step_ms(fn, reps_=None):
        """Mean time of fn launched after a schedule build, between two events."""
        n = reps_ or max(5, args.steps // 2)
        for _ in range(3):
            step()
            fn()
        e_a = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        e_b = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            step()
            e_a[i].record(stream)
            fn()
            e_b[i].record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in zip(e_a, e_b)) / n
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(5, args.steps // 2)
    # The per-row top-k scope of the builder: its build time, and the kernel over
    # its schedule, timed the same way.
    per_row = None
    if not w.dense:
        pbufs = tsa.ScheduleBuffers(w.S, w.D, w.sink, w.local_radius, w.topk, dev, per_row=True)
        for _ in range(3):
            tsa.build_schedule_into(keys, pbufs)
        torch.cuda.synchronize()
        d0.record(stream)
        for _ in range(reps):
            tsa.build_schedule_into(keys, pbufs)
        d1.record(stream)
        torch.cuda.synchronize()
        pr_build_ms = d0.elapsed_time(d1) / reps
        pr_nnz = int(pbufs.row_ptr[-1].item())
        pr_attention = tsa.prepare_scheduled_attention(q, k, v, pbufs.row_ptr, pbufs.col_idx, out)
        pr_ms = in_step_ms(pr_attention)
        per_row = {"nnz_blocks": pr_nnz, "builder_ms": round(pr_build_ms, 5), "attention_ms": round(pr_ms, 5),
                   "attention_tflops": round(lanes * pr_nnz * 4 * 64 * 64 * w.D / (pr_ms * 1e-3) / 1e12, 3)}
    # The fixed-segment CSR (512-token segments) at the same shape, timed the same way.
    seg = None
    if w.S % 512 == 0:
        srp, sci = tsa.segment_schedule(w.nb, 512 // 64, dev)
        seg_nnz = int(sci.shape[0])
        seg_attention = tsa.prepare_scheduled_attention(q, k, v, srp, sci, out)
        seg_ms = in_step_ms(seg_attention)
        seg = {"segment_tokens": 512, "nnz_blocks": seg_nnz, "ms": round(seg_ms, 5),
               "tflops": round(lanes * seg_nnz * 4 * 64 * 64 * w.D / (seg_ms * 1e-3) / 1e12, 3)}
    # The same workload with a schedule over 128-row blocks (sink, window and top-k
    # taken at the same token counts, rounded up), refined to the 64-row CSR the
    # attention kernel takes: builder, refinement and attention, timed the same way.
    coarse = None
    if not w.dense:
        cb = 128
        csink, crad, ctop = -(-w.sink // 2), -(-w.local_radius // 2), max(1, w.topk // 2)
        cbufs = tsa.ScheduleBuffers(w.S, w.D, csink, crad, ctop, dev, block=cb)
        for _ in range(3):
            tsa.build_schedule_into(keys, cbufs)
        torch.cuda.synchronize()
        d0.record(stream)
        for _ in range(reps):
            tsa.build_schedule_into(keys, cbufs)
        d1.record(stream)
        torch.cuda.synchronize()
        c_build_ms = d0.elapsed_time(d1) / reps
        c_nnz = int(cbufs.row_ptr[-1].item())
        crp, cci = tsa.refine_schedule(cbufs.row_ptr, cbufs.col_idx[:c_nnz], w.S, cb)
        torch.cuda.synchronize()
        d0.record(stream)
        for _ in range(reps):
            tsa.refine_schedule(cbufs.row_ptr, cbufs.col_idx[:c_nnz], w.S, cb)
        d1.record(stream)
        torch.cuda.synchronize()
        c_refine_ms = d0.elapsed_time(d1) / reps
        f_nnz = int(cci.shape[0])
        c_attention = tsa.prepare_scheduled_attention(q, k, v, crp, cci, out)
        c_ms = in_step_ms(c_attention)
        coarse = {"block": cb, "sink": csink, "local_radius": crad, "topk": ctop, "nnz_blocks": c_nnz,
                  "nnz_blocks_64": f_nnz, "builder_ms": round(c_build_ms, 5),
                  "refine_ms": round(c_refine_ms, 5), "refine_note": "host-synchronising call (reads nnz)",
                  "attention_ms": round(c_ms, 5),
                  "attention_tflops": round(lanes * f_nnz * 4 * 64 * 64 * w.D / (c_ms * 1e-3) / 1e12, 3)}
    # Backward pass over the same schedule: the forward with lse and the column
    # view once, then back-to-back backward calls (dq kernel, then dk/dv kernel).
    # Algorithmic work: 5 block products per visited block (S recomputed once, dP,
    # dV, dQ, dK), 2.5x the forward's.
    dout = workloads.random_normal(w.shape, w.dtype, 99).to(dev)
    o_l, lse = tsa.scheduled_attention(q, k, v, rp, ci, return_lse=True)
    for _ in range(3):
        tsa.schedule_transpose(rp, ci)
    torch.cuda.synchronize()
    d0.record(stream)
    for _ in range(reps):
        cp, ri = tsa.schedule_transpose(rp, ci)
    d1.record(stream)
    torch.cuda.synchronize()
    tr_ms = d0.elapsed_time(d1) / reps
    for _ in range(3):
        grads = tsa.scheduled_attention_backward(q, k, v, o_l, dout, lse, rp, ci, cp, ri)
    torch.cuda.synchronize()
    d0.record(stream)
    for _ in range(reps):
        grads = tsa.scheduled_attention_backward(q, k, v, o_l, dout, lse, rp, ci, cp, ri)
    d1.record(stream)
    torch.cuda.synchronize()
    bwd_ms = d0.elapsed_time(d1) / reps
    if not all(bool(torch.isfinite(g).all()) for g in grads):
        print("non-finite gradient", file=sys.stderr)
        return 1
    bwd_tflops = 2.5 * flops / (bwd_ms * 1e-3) / 1e12
    backward = {"ms": round(bwd_ms, 5), "tflops": round(bwd_tflops, 3),
                "frac_of_peak": round(bwd_tflops / PEAK_TFLOPS[w.dtype], 4),
                "flops_per_block": "5 products of 64x64xD (2.5x forward)",
                "transpose_ms": round(tr_ms, 5), "transpose_note": "host-synchronising call (reads nnz)"}
    if not bool(torch.isfinite(out).all()):
        print("non-finite output", file=sys.stderr)
        return 1

    peak = PEAK_TFLOPS[w.dtype]
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    value = flops / (step_ms * 1e-3) / 1e12
    traffic = _traffic(name)
    nnz_dense = w.nb * (w.nb + 1) // 2
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": name,
            "shape": list(w.shape),
            "block": 64,
            "sink": None if w.dense else w.sink,
            "local_radius": None if w.dense else w.local_radius,
            "topk": None if w.dense else w.topk,
            "schedule": "dense causal CSR" if w.dense else "topology (GPU-built each step)",
            "nnz_blocks": nnz,
            "dense_blocks": nnz_dense,
            "parallelism": "single GPU",
        },
        "frac_of_peak": round(value / peak, 4),
        "attention_ms": round(attn_ms, 5),
        "attention_ms_min": round(attn_ms_each[0], 5),
        "builder_ms": round(build_ms, 5),
        "attention_tflops": round(attn_tflops, 3),
        "attention_frac_of_peak": round(attn_tflops / peak, 4),
        "attention_tflops_causal_exact": round(flops_exact / (attn_ms * 1e-3) / 1e12, 3),
        "dense_csr_ms": round(dense_ms, 5),
                "sparse_vs_dense_csr_speedup": round(dense_ms / sparse_ms, 3),
        "ideal_speedup": round(nnz_dense / nnz, 3),
        "dense_csr_tflops": round(lanes * nnz_dense * 4 * 64 * 64 * w.D / (dense_ms * 1e-3) / 1e12, 3),
        "segment_csr": seg,
        "per_row_topk": per_row,
        "block_128": coarse,
        "backward": backward,
        "roofline": {
            "bound": "mfma",
            "achieved": round(attn_tflops, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / peak, 4),
            "traffic": traffic,
        },
        "cpu_baseline": None,
        # per-launch SQ counters of the attention kernel (profiles/attention_fwd_<workload>_sq.txt):
        # MFMA-busy fraction of all SIMD cycles at the measured clock, and instruction mix
        "counters": _sq_counters(name),
    }
    bad = None
    if not args.no_cpu_baseline:
        print(f"# timing the fp64 oracle for about {args.cpu_budget:.0f} s", file=sys.stderr, flush=True)
        cb = _cpu_baseline(w, q_cpu, k_cpu, v_cpu, args.cpu_budget, timed_out, timed_csr)
        result["cpu_baseline"] = {key: cb[key] for key in ("value", "unit", "cores", "kind", "sample")}
        result["cpu_baseline"]["value"] = round(cb["value"], 6)
        par = cb["parity"]
        par["bar"] = PARITY_BAR[w.dtype]
        result["parity"] = par
        if par["max_abs_err"] > par["bar"] or not par["csr_bit_exact"]:
            bad = f"timed output fails the oracle check: {par}"
    print(json.dumps(result), flush=True)
    if bad:
        print(bad, file=sys.stderr, flush=True)
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
