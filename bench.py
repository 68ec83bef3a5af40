#!/usr/bin/env python3
"""Benchmark of the decomposed AllGather->GEMM and GEMM->ReduceScatter on one MI355X.

One step = the tensor-parallel MLP hot path of one layer on N virtual ranks:
AllGather->GEMM (column-parallel fc1 over the gathered sequence shards)
followed by GEMM->ReduceScatter (row-parallel fc2 back to sequence shards),
both decomposed into per-shard partial GEMMs overlapped with SDMA ring hops.

Prints ONE JSON line:
  value        whole-step TFLOP/s (algorithmic FLOPs of both ops / wall time)
  roofline     the dominant kernel (the batched step GEMM) against the bf16
               dense MFMA peak, from HIP events around every launch of it on
               the compute stream during the timed steps
  overlap      per op: decomposed time over max(GEMM-only, copy-only) time.
               GEMM-only: the monolithic GEMM alone (the naive schedule's);
               copy-only: the smaller of the naive collective alone and the
               decomposed hops' busy time.  Also the GEMM and hop busy times
               inside the decomposed run and the fraction of hop time hidden
               under GEMMs, from the same events
  cpu_baseline the CPU oracle timed on a bounded sample of the same workload

Inputs are seeded synthetic tensors (activations N(0,1), weights
N(0, 0.02^2), bf16) resident in HBM before the timed region.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOADS = {
    # Llama-3-8B MLP: d = 4096, ffn = 14336, 4096 tokens, N = 8 (f/N = 1792)
    "llama3-8b-mlp": dict(N=8, T=4096, d=4096, f=14336),
    # GPT-3 175B MLP: d = 12288, ffn = 49152, 2048 tokens, N = 8 (f/N = 6144)
    "gpt3-175b-mlp": dict(N=8, T=2048, d=12288, f=49152),
    # the tiny check: d = 256, ffn = 1024, 256 tokens, N = 4
    "tiny": dict(N=4, T=256, d=256, f=1024),
}
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def union_length(intervals):
    total, end = 0.0, -1e300
    for a, b in sorted(intervals):
        if b <= end:
            continue
        total += b - max(a, end)
        end = b
    return total


def algorithmic_bytes(op_rec, jobs, out_size):
    """Bytes a GEMM launch must move at least once: A, B (once per run of
    b_share jobs that read the same weights), C, and the fp32 addends."""
    total = 0
    share = max(1, op_rec.b_share)
    for j in jobs[op_rec.first_job:op_rec.first_job + op_rec.n_jobs]:
        total += op_rec.rows * op_rec.depth * 2 + op_rec.cols * op_rec.depth * 2 // share
        total += op_rec.rows * op_rec.cols * (4 if j.c_dtype == 1 else 2)
        total += op_rec.rows * op_rec.cols * 4 * ((j.in0_buf >= 0) + (j.in1_buf >= 0))
    return total


def addends_per_job(op_rec, jobs):
    """How many fp32 addends (arrived buckets) each job of a GEMM launch reads."""
    return max((j.in0_buf >= 0) + (j.in1_buf >= 0) for j in jobs[op_rec.first_job:op_rec.first_job + op_rec.n_jobs])


def launch_label(name, jobs, nadd):
    """A GEMM launch shape's name: op, jobs per launch, fp32 addends per job."""
    return "%s%d_add%d" % (name, jobs, nadd)


def profiled_traffic(workload, label):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (profiles/gemm_step_<workload>.md: FETCH_SIZE and WRITE_SIZE
    scaled by calibration kernels), or None when that summary was taken on
    other kernel source than the one built now or holds no such launch."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemm_step_%s.md" % workload)
    src = os.path.join(ROOT, "collective_matmul_decomposition_amd", "csrc", "kernels.hip")
    try:
        lines = open(path).read().splitlines()
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    kv = dict(l.strip().split("=", 1) for l in lines if "=" in l and " " not in l.strip())
    if kv.get("kernel_source_sha256") != sha:
        return None
    v = kv.get("traffic_bytes_%s" % label)
    return int(v) if v else None


def rs_hop(args):
    """The RS hop kind a run uses: add-and-forward exists for the ring RS with an fp32 bucket only."""
    ok = args.rs_op == "rs" and args.dir in ("uni", "bi") and args.rs_bucket == "f32"
    return args.rs_hop if ok else "copy"


_STREAMS = {}


def streams(n_comm):
    """The compute stream and n_comm comm streams.  One set for the whole run,
    created at its start: torch hands out streams from a pool round-robin, and
    the runtime spreads streams over the process's few hardware queues by
    creation order, so streams made anew for every measurement landed on
    different queues from run to run (a backward's bulk stream could share
    the compute stream's queue and serialise behind it)."""
    import torch
    if not _STREAMS:
        _STREAMS["compute"] = torch.cuda.Stream()
        _STREAMS["comm"] = [torch.cuda.Stream() for _ in range(3)]
    if n_comm > len(_STREAMS["comm"]):
        _STREAMS["comm"] += [torch.cuda.Stream() for _ in range(n_comm - len(_STREAMS["comm"]))]
    return _STREAMS["compute"], _STREAMS["comm"][:n_comm]


def measure(args, workload, steps, warmup, with_naive, with_trace):
    import torch
    from collective_matmul_decomposition_amd import _native as nat
    from collective_matmul_decomposition_amd import buffers
    from collective_matmul_decomposition_amd import inputs as gen

    wl = WORKLOADS[workload]
    N, T, d, f = wl["N"], wl["T"], wl["d"], wl["f"]
    m, fN = T // N, f // N
    n_comm = args.n_comm
    tile = tuple(int(v) for v in args.tile.split("x"))

    def make_plans(skip="none"):
        pa = nat.cm_ring_plan(op="ag", n_ranks=N, m=m, k=d, n=fN, dir=args.dir, chunks=args.chunks_ag,
                              out_dtype="bf16", n_comm=n_comm, tile=tile, copy_engine=args.copy_engine, skip=skip,
                              group=args.group)
        pr = nat.cm_ring_plan(op=args.rs_op, n_ranks=N, m=m, k=fN, n=d, dir=args.dir, chunks=args.chunks_rs,
                              out_dtype="bf16", n_comm=n_comm, tile=tile, copy_engine=args.copy_engine,
                              bucket=args.rs_bucket, hop=rs_hop(args), skip=skip, group=args.group)
        return pa, pr

    plan_ag, plan_rs = make_plans(args.skip)
    # the engine each op's hops run on (the planner's choice when the request says auto)
    hops_on = {k: "cu" if p.desc.copy_engine == nat.CM_COPY_CU else "sdma" for k, p in (("ag", plan_ag), ("rs", plan_rs))}
    log("%s plans: AG chunks=%d tile=%dx%d ws=%.0fMB launches %s | RS(%s) chunks=%d tile=%dx%d ws=%.0fMB "
        "launches %s | n_comm=%d | hops on %s" % (
            workload, plan_ag.chunks, plan_ag.tile_m, plan_ag.tile_n, plan_ag.ws_bytes / 1e6,
            list(plan_ag.group_len[:plan_ag.n_launches]), args.rs_op, plan_rs.chunks, plan_rs.tile_m, plan_rs.tile_n,
            plan_rs.ws_bytes / 1e6, list(plan_rs.group_len[:plan_rs.n_launches]), n_comm, hops_on))

    x, w1 = gen.ag_inputs_torch(N, m, d, fN, "normal", 0, "cuda")
    h, w2 = gen.rs_inputs_torch(N, m, fN, d, "normal", 0, "cuda")
    y1, ws1 = buffers.alloc_outputs(plan_ag)
    y2, ws2 = buffers.alloc_outputs(plan_rs)
    buffers.check_inputs(plan_ag, x, w1, y1, ws1)
    buffers.check_inputs(plan_rs, h, w2, y2, ws2)
    compute, comm = streams(n_comm)
    compute.wait_stream(torch.cuda.current_stream())  # inputs were written on the current stream
    flops_op = 2.0 * N * T * d * fN  # each op: N ranks x [T x d] . [d x f/N]
    flops_step = 2 * flops_op

    def step(tr_ag=None, tr_rs=None, pa=plan_ag, pr=plan_rs):
        nat.cm_ag_gemm(pa, x, w1, y1, ws1, compute, comm, tr_ag)
        nat.cm_gemm_rs(pr, h, w2, y2, ws2, compute, comm, tr_rs)

    ops_ag, jobs_ag = nat.cm_plan_program(plan_ag)
    ops_rs, jobs_rs = nat.cm_plan_program(plan_rs)
    cap_ag = sum(1 for o in ops_ag if o.kind in (nat.CM_OPK_GEMM, nat.CM_OPK_COPY, nat.CM_OPK_REDUCE))
    cap_rs = sum(1 for o in ops_rs if o.kind in (nat.CM_OPK_GEMM, nat.CM_OPK_COPY, nat.CM_OPK_REDUCE))
    # one trace pair per timed step: each call's graph records its own events
    traces = [(nat.Trace(cap_ag), nat.Trace(cap_rs)) for _ in range(steps)] if with_trace else None

    # warm-up; with traces, every timed step's graphs (one per trace) are built here
    for i in range(max(warmup, steps) if with_trace else warmup):
        if with_trace:
            step(*traces[i % steps])
        else:
            step()
    torch.cuda.synchronize()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if with_trace:
            step(*traces[i])
        else:
            step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / steps
    value = flops_step / (wall / steps) / 1e12
    log("%s timed: %.3f ms/step, %.1f TFLOP/s" % (workload, ms_per_step, value))
    res = {"value": value, "ms_per_step": ms_per_step, "N": N, "T": T, "d": d, "f": f, "fN": fN, "m": m,
           "plan_ag": plan_ag, "plan_rs": plan_rs, "n_comm": n_comm, "hops_on": hops_on,
           "tensors": (x, w1, y1, h, w2, y2)}

    if with_trace:
        gemm_stats = {}  # launch shape -> [durations]
        per_op = {"ag": [], "rs": []}

        def launch_keys(ops, jobs, name):
            keys = []
            for o in ops:
                if o.kind == nat.CM_OPK_GEMM:
                    keys.append((name, o.rows, o.cols, o.depth, o.n_jobs, o.tile_m, o.tile_n,
                                 addends_per_job(o, jobs), algorithmic_bytes(o, jobs, 2)))
            return keys

        keys = {"ag": launch_keys(ops_ag, jobs_ag, "ag"), "rs": launch_keys(ops_rs, jobs_rs, "rs")}
        # the last timed step's operations, start and end relative to each op's first one
        kind_name = {nat.CM_OPK_GEMM: "gemm", nat.CM_OPK_COPY: "copy", nat.CM_OPK_REDUCE: "add"}
        timeline = {}
        for name, i in (("ag", 0), ("rs", 1)):
            spans = traces[-1][i].read()[0]
            t0s = min(q[4] for q in spans)
            timeline[name] = [[kind_name.get(q[0], str(q[0])), q[1], q[2], round(q[4] - t0s, 1), round(q[5] - t0s, 1)]
                              for q in sorted(spans, key=lambda q: q[4])]
        res["timeline"] = timeline
        if getattr(args, "timeline", False):
            for name in ("ag", "rs"):
                log("%s timeline (kind, stream, step, start us, end us): %s" % (name, timeline[name]))
        for tr_ag, tr_rs in traces:
            for name, tr in (("ag", tr_ag), ("rs", tr_rs)):
                spans, total = tr.read()
                g = [s for s in spans if s[0] == nat.CM_OPK_GEMM]
                assert len(g) == len(keys[name])
                for key, s in zip(keys[name], g):
                    gemm_stats.setdefault(key, []).append(s[5] - s[4])
                G = union_length([(s[4], s[5]) for s in g])
                C = union_length([(s[4], s[5]) for s in spans if s[0] in (nat.CM_OPK_COPY, nat.CM_OPK_REDUCE)])
                per_op[name].append((total, G, C))
        # the dominant kernel: the launch shape with the most total time
        (name, rows, cols, depth, jobs, tm, tn, nadd, abytes), durs = max(gemm_stats.items(),
                                                                        key=lambda kv: sum(kv[1]))
        dom_key = (name, rows, cols, depth, jobs, tm, tn, nadd, abytes)
        flops_launch = 2.0 * rows * cols * depth * jobs
        avg_us = float(np.mean(durs))
        intensity = flops_launch / abytes
        ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
        if intensity >= ridge:
            achieved = flops_launch / (avg_us * 1e-6) / 1e12
            roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
        else:
            achieved = abytes / (avg_us * 1e-6) / 1e9
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBPS, 4)}
        roof.update({"traffic": None,
                     "kernel": "gemm_jobs_kernel<%d,%d,...> (%s step: %d jobs of [%dx%d].[%dx%d]^T%s)" % (
                         tm, tn, name.upper(), jobs, rows, depth, cols, depth,
                         ", + %d fp32 addend(s)" % nadd if nadd else ""),
                     "launch": launch_label(name, jobs, nadd),
                     "avg_launch_us": round(avg_us, 2), "launches": len(durs),
                     "flops_per_launch": flops_launch, "algorithmic_bytes_per_launch": abytes,
                     "intensity_flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": round(ridge, 1),
                     "mfma_tflops": round(flops_launch / (avg_us * 1e-6) / 1e12, 1),
                     "hbm_gbps": round(abytes / (avg_us * 1e-6) / 1e9, 1)})
        roof["traffic"] = profiled_traffic(workload, launch_label(name, jobs, nadd))
        res["roofline"] = roof
        res["gemm_launches"] = {
            "%s %dx%dx%d x%d tile %dx%d%s" % (nm, r, c, dd, j, a, b, " +%d addend" % na if na else ""): {
                "launch": launch_label(nm, j, na), "avg_us": round(float(np.mean(dl)), 2), "count": len(dl),
                "tflops": round(2.0 * r * c * dd * j / (np.mean(dl) * 1e-6) / 1e12, 1), "algorithmic_bytes": ab}
            for (nm, r, c, dd, j, a, b, na, ab), dl in gemm_stats.items()}
        # the GEMM launches of one step in program order (for splitting a profiler's trace)
        res["step_launches"] = [launch_label(k[0], k[4], k[7]) for k in keys["ag"] + keys["rs"]]
        ov = {}
        for name, plan in (("ag", plan_ag), ("rs", plan_rs)):
            arr = np.array(per_op[name])
            D, G, C = np.median(arr[:, 0]), np.median(arr[:, 1]), np.median(arr[:, 2])
            elt = 2 if name == "ag" or args.rs_bucket == "bf16" else 4
            ring_bytes = N * (N - 1) * m * d * elt
            ov[name] = {"decomposed_us": round(D, 1), "gemm_busy_us": round(G, 1), "hop_busy_us": round(C, 1),
                        "overlap_efficiency_inrun": round(D / max(G, C), 3),
                        "hidden_fraction_inrun": round((G + C - D) / C, 3) if C > 0 else None,
                        "tflops": round(flops_op / (D * 1e-6) / 1e12, 1), "ring_bytes": ring_bytes,
                        "hop_GBps": round(ring_bytes / (C * 1e-6) / 1e9, 1) if C > 0 else None,
                        "chunks": plan.chunks}
        res["overlap"] = ov

        gemm_alone_stats = {}  # launch shape -> durations with the hops skipped
        # G and C alone: the same programs (same launches, copies and edges)
        # with the hops, or the compute-stream launches, replaced by empty
        # operations, timed per op inside alternating AG/RS steps as D is
        alone = {"ag": {}, "rs": {}}
        reps = max(5, steps // 2)
        if not (args.no_alone or args.skip != "none"):
            # their own outputs and workspaces: a call in a measurement mode leaves
            # meaningless values, and y1 / y2 hold the step's results for the checks
            ys1, wss1 = buffers.alloc_outputs(plan_ag)
            ys2, wss2 = buffers.alloc_outputs(plan_rs)

            def step_alone(ta, tb, pa, pr):
                nat.cm_ag_gemm(pa, x, w1, ys1, wss1, compute, comm, ta)
                nat.cm_gemm_rs(pr, h, w2, ys2, wss2, compute, comm, tb)

            for skip in ("hops", "gemms"):
                pa, pr = make_plans(skip)
                tr = [(nat.Trace(cap_ag), nat.Trace(cap_rs)) for _ in range(reps)]
                for _ in range(2):  # the first round builds each trace's graphs
                    for ta, tb in tr:
                        step_alone(ta, tb, pa, pr)
                    torch.cuda.synchronize()
                for name, i in (("ag", 0), ("rs", 1)):
                    alone[name][skip] = float(np.median([t[i].read()[1] for t in tr]))
                if skip == "hops":
                    # each launch's duration with the GEMMs alone (same programs, hops empty)
                    for name, i in (("ag", 0), ("rs", 1)):
                        for t in tr:
                            g = [q for q in t[i].read()[0] if q[0] == nat.CM_OPK_GEMM]
                            for key, q in zip(keys[name], g):
                                gemm_alone_stats.setdefault(key, []).append(q[5] - q[4])
                for ta, tb in tr:
                    ta.close()
                    tb.close()
            del ys1, wss1, ys2, wss2
            # the dominant launch's roofline with the GEMMs alone: no hop (SDMA copy or
            # add kernel) shares the device, which is what a profiler reproduces exactly
            da = gemm_alone_stats.get(dom_key)
            flops_launch = 2.0 * dom_key[1] * dom_key[2] * dom_key[3] * dom_key[4]
            abytes = dom_key[8]
            if da:
                avg_a = float(np.mean(da))
                ra = dict(roof)
                if ra["bound"] == "mfma":
                    ra["achieved"] = round(flops_launch / (avg_a * 1e-6) / 1e12, 1)
                else:
                    ra["achieved"] = round(abytes / (avg_a * 1e-6) / 1e9, 1)
                ra["frac"] = round(ra["achieved"] / ra["peak"], 4)
                ra["avg_launch_us"] = round(avg_a, 2)
                ra["launches"] = len(da)
                ra["mfma_tflops"] = round(flops_launch / (avg_a * 1e-6) / 1e12, 1)
                ra["hbm_gbps"] = round(abytes / (avg_a * 1e-6) / 1e9, 1)
                ra["measured"] = "GEMM-alone measurement mode (hops skipped, same programs)"
                res["roofline_gemm_alone"] = ra
            for name, plan in (("ag", plan_ag), ("rs", plan_rs)):
                o = ov[name]
                D, Ga, Ca = o["decomposed_us"], alone[name]["hops"], alone[name]["gemms"]
                elt = 2 if name == "ag" or args.rs_bucket == "bf16" else 4
                # overlap efficiency = D / max(GEMM-only, copy-only); hidden
                # fraction = (G + C - D) / C, with G and C the op's parts alone
                o.update({"gemm_alone_us": round(Ga, 1), "copy_alone_us": round(Ca, 1),
                          "bound_by": "gemm" if Ga >= Ca else "copy",
                          "overlap_efficiency": round(D / max(Ga, Ca), 3),
                          "hidden_fraction": round((Ga + Ca - D) / Ca, 3) if Ca > 0 else None,
                          # each hop byte is read and written once in HBM
                          "hop_GBps_alone": round(o["ring_bytes"] / (Ca * 1e-6) / 1e9, 1) if Ca > 0 else None,
                          "hop_hbm_frac_alone": round(2 * o["ring_bytes"] / (Ca * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)
                          if Ca > 0 else None})
                log("%s alone: G %.1f us (hops skipped), C %.1f us (GEMMs skipped), D %.1f us -> D/max(G,C) %.3f, "
                    "hidden (G+C-D)/C %.3f" % (name, Ga, Ca, D, o["overlap_efficiency"],
                                                o["hidden_fraction"] or 0.0))

    if with_naive:
        # the naive schedule with the engine the decomposed AllGather uses, then with the other one
        first = hops_on["ag"]
        pa = nat.cm_ring_plan(op="ag", n_ranks=N, m=m, k=d, n=fN, sched="naive", out_dtype="bf16", n_comm=n_comm,
                              copy_engine=first)
        pr = nat.cm_ring_plan(op="rs", n_ranks=N, m=m, k=fN, n=d, sched="naive", out_dtype="bf16", n_comm=n_comm,
                              copy_engine=first)
        yn1, wsn1 = buffers.alloc_outputs(pa)
        yn2, wsn2 = buffers.alloc_outputs(pr)

        def naive_step():
            nat.cm_ag_gemm(pa, x, w1, yn1, wsn1, compute, comm)
            nat.cm_gemm_rs(pr, h, w2, yn2, wsn2, compute, comm)
        for _ in range(2):
            naive_step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ns = max(3, steps // 2)
        for _ in range(ns):
            naive_step()
        torch.cuda.synchronize()
        nwall = (time.perf_counter() - t0) / ns
        res["naive"] = {"ms_per_step": round(nwall * 1e3, 3), "tflops": round(flops_step / nwall / 1e12, 1),
                        "speedup_of_decomposed": round(nwall * 1e3 / ms_per_step, 3), "copy_engine": first}
        # the same naive schedule with the other engine: its collective moves one
        # rank's shard per copy, where the engines differ most
        other = "cu" if first == "sdma" else "sdma"
        pa2 = nat.cm_ring_plan(op="ag", n_ranks=N, m=m, k=d, n=fN, sched="naive", out_dtype="bf16", n_comm=n_comm,
                               copy_engine=other)
        pr2 = nat.cm_ring_plan(op="rs", n_ranks=N, m=m, k=fN, n=d, sched="naive", out_dtype="bf16", n_comm=n_comm,
                               copy_engine=other)

        def naive_other():
            nat.cm_ag_gemm(pa2, x, w1, yn1, wsn1, compute, comm)
            nat.cm_gemm_rs(pr2, h, w2, yn2, wsn2, compute, comm)
        for _ in range(2):
            naive_other()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(ns):
            naive_other()
        torch.cuda.synchronize()
        owall = (time.perf_counter() - t0) / ns
        res["naive"]["other_copy_engine"] = {"copy_engine": other, "ms_per_step": round(owall * 1e3, 3),
                                             "speedup_of_decomposed": round(owall * 1e3 / ms_per_step, 3)}
        res["naive"]["speedup_over_faster_naive"] = round(min(nwall, owall) * 1e3 / ms_per_step, 3)
        log("naive: %.3f ms (%s), %.3f ms (%s) -> decomposed is x%.2f faster than the faster one" % (
            nwall * 1e3, first, owall * 1e3, other, res["naive"]["speedup_over_faster_naive"]))
        if with_trace and "overlap" in res:
            # GEMM-only and copy-only times: the naive schedule runs the
            # monolithic GEMM and the collective one after the other, so each
            # runs alone; the overlap efficiency is the decomposed time over
            # the larger of the two
            caps = [sum(1 for o in nat.cm_plan_program(p)[0]
                        if o.kind in (nat.CM_OPK_GEMM, nat.CM_OPK_COPY, nat.CM_OPK_REDUCE)) for p in (pa, pr)]
            ntr = [(nat.Trace(caps[0]), nat.Trace(caps[1])) for _ in range(3)]
            for _ in range(2):
                for ta, tb in ntr:
                    nat.cm_ag_gemm(pa, x, w1, yn1, wsn1, compute, comm, ta)
                    nat.cm_gemm_rs(pr, h, w2, yn2, wsn2, compute, comm, tb)
                torch.cuda.synchronize()
            alone = {"ag": [], "rs": []}
            for ta, tb in ntr:
                for name, tr in (("ag", ta), ("rs", tb)):
                    spans, _total = tr.read()
                    alone[name].append((union_length([(q[4], q[5]) for q in spans if q[0] == nat.CM_OPK_GEMM]),
                                        union_length([(q[4], q[5]) for q in spans
                                                      if q[0] in (nat.CM_OPK_COPY, nat.CM_OPK_REDUCE)])))
                    tr.close()
            for name, ov in res["overlap"].items():
                Ga, Cn = (float(np.median([a[i] for a in alone[name]])) for i in (0, 1))
                D = ov["decomposed_us"]
                # copy-only: the naive collective alone, or the decomposed
                # ring's own hops, whose busy time beside the GEMMs bounds
                # theirs alone from above; the smaller of the two
                Ca = min(Cn, ov["hop_busy_us"])
                ov.update({"monolithic_gemm_us": round(Ga, 1), "naive_collective_us": round(Cn, 1),
                           "overlap_efficiency_vs_naive": round(D / max(Ga, Ca), 3)})
                if "gemm_alone_us" in ov:
                    # the cost of cutting the GEMM into per-step partial GEMMs: G / M
                    ov["g_over_m"] = round(ov["gemm_alone_us"] / Ga, 3)
                log("%s: decomposed %.1f us; monolithic GEMM %.1f us, copy-only %.1f us (naive collective %.1f) -> "
                    "efficiency %.3f (in-run busy: GEMM %.1f, hops %.1f -> %.3f)" % (
                        name, D, Ga, Ca, Cn, ov["overlap_efficiency_vs_naive"], ov["gemm_busy_us"], ov["hop_busy_us"],
                        ov["overlap_efficiency_inrun"]))
        del yn1, wsn1, yn2, wsn2
    return res


def measure_op(op, N, m, k, n, chunks, ring, n_comm, reps, copy_engine="sdma"):
    """One op alone (no step around it): decomposed time D from the wall clock
    of `reps` graph replays, GEMM-busy G and hop-busy C from the trace of the
    same replays, and the naive (all hops, then the monolithic GEMM) time."""
    import torch
    from collective_matmul_decomposition_amd import _native as nat
    from collective_matmul_decomposition_amd import buffers
    from collective_matmul_decomposition_amd import inputs as gen
    mk = gen.ag_inputs_torch if op == "ag" else gen.rs_inputs_torch
    x, w = mk(N, m, k, n, "normal", 0, "cuda")
    compute, comm = streams(n_comm)
    compute.wait_stream(torch.cuda.current_stream())
    fn = nat.cm_ag_gemm if op == "ag" else nat.cm_gemm_rs
    flops = 2.0 * N * (N * m) * k * n
    out = {"op": op, "N": N, "m": m, "k": k, "n": n, "ring": ring, "n_comm": n_comm, "copy_engine": copy_engine}
    for sched in ("decomposed", "naive"):
        plan = nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, dir=ring, chunks=chunks, sched=sched,
                                out_dtype="bf16", n_comm=n_comm, copy_engine=copy_engine)
        y, ws = buffers.alloc_outputs(plan)
        out["hops_on_" + sched] = "cu" if plan.desc.copy_engine == nat.CM_COPY_CU else "sdma"
        ops, _ = nat.cm_plan_program(plan)
        cap = sum(1 for o in ops if o.kind in (nat.CM_OPK_GEMM, nat.CM_OPK_COPY, nat.CM_OPK_REDUCE))
        traces = [nat.Trace(cap) for _ in range(reps)]
        for tr in traces:  # builds (and warms) one graph per trace
            fn(plan, x, w, y, ws, compute, comm, tr)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for tr in traces:
            fn(plan, x, w, y, ws, compute, comm, tr)
        torch.cuda.synchronize()
        wall_us = (time.perf_counter() - t0) / reps * 1e6
        Gs, Cs, Ts = [], [], []
        for tr in traces:
            spans, total = tr.read()
            Gs.append(union_length([(q[4], q[5]) for q in spans if q[0] == nat.CM_OPK_GEMM]))
            Cs.append(union_length([(q[4], q[5]) for q in spans if q[0] in (nat.CM_OPK_COPY, nat.CM_OPK_REDUCE)]))
            Ts.append(total)
            tr.close()
        G, C, D = float(np.median(Gs)), float(np.median(Cs)), float(np.median(Ts))
        if sched == "decomposed":
            out.update({"chunks": plan.chunks, "tile": "%dx%d" % (plan.tile_m, plan.tile_n),
                        "declined_by_cost_model": bool(plan.declined),
                        "decomposed_us": round(D, 1), "wall_us": round(wall_us, 1), "gemm_busy_us": round(G, 1),
                        "hop_busy_us": round(C, 1), "overlap_efficiency": round(D / max(G, C), 3),
                        "hidden_fraction": round((G + C - D) / C, 3) if C > 0 else None,
                        "tflops": round(flops / (D * 1e-6) / 1e12, 1)})
        else:
            # the naive schedule runs the monolithic GEMM and the collective
            # one after the other: its GEMM time is the GEMM-only time; the
            # copy-only time is the smaller of its collective's time and the
            # decomposed hops' busy time (an upper bound on those hops alone)
            out.update({"naive_us": round(D, 1), "monolithic_gemm_us": round(G, 1),
                        "speedup_over_naive": round(D / out["decomposed_us"], 3),
                        "gemm_only_us": round(G, 1), "naive_collective_us": round(C, 1),
                        "copy_only_us": round(min(C, out["hop_busy_us"]), 1),
                        "overlap_efficiency_busy": out["overlap_efficiency"],
                        "overlap_efficiency": round(out["decomposed_us"] / max(G, min(C, out["hop_busy_us"])), 3)})
        del y, ws
    del x, w
    torch.cuda.empty_cache()
    return out


def measure_share(workload, reps):
    """One rank's share of the step: virtual rank 0's fc1 (AllGather->GEMM)
    and fc2 (GEMM->ReduceScatter) ring steps at their real shapes, as one GPU
    of the N-GPU group runs them.  Each step's GEMM is split along K (S
    slices, the planner's choice) and one reduce launch sums the partials; the
    hops bring in the neighbour's shard / bucket (N(0, 0.5^2) buckets for
    fc2).  Op time D: wall clock of `reps` graph replays without the trace,
    with the hops on the SDMA engines and on compute units (the faster is
    reported); compute-only time: the same program with its hops replaced by
    empty operations (every edge kept); per-launch times from a traced run."""
    import torch
    from collective_matmul_decomposition_amd import _native as nat
    from collective_matmul_decomposition_amd import buffers
    from collective_matmul_decomposition_amd import inputs as gen
    W = WORKLOADS[workload]
    N, T, d, f = W["N"], W["T"], W["d"], W["f"]
    m, fN = T // N, f // N
    out = {"workload": workload, "rank": 0, "virtual_ranks": N,
           "what": "virtual rank 0's ring steps at real shape (one GPU's share of the N-rank group); split-K step "
                   "GEMMs + one reduce launch per step; hops bring in the neighbour's shard / bucket"}
    total_flops, total_us = 0.0, 0.0
    compute, _ = streams(1)
    compute.wait_stream(torch.cuda.current_stream())

    def wall(fn, plan, x, w, y, ws, comm, n):
        # best of three batches of n calls (one op is about half a millisecond)
        for _ in range(3):
            fn(plan, x, w, y, ws, compute, comm, None)
        torch.cuda.synchronize()
        best = None
        for _ in range(3):
            t0 = time.perf_counter()
            for _ in range(n):
                fn(plan, x, w, y, ws, compute, comm, None)
            torch.cuda.synchronize()
            t = (time.perf_counter() - t0) / n * 1e6
            best = t if best is None else min(best, t)
        return best

    for name, op, k, n in (("fc1", "ag", d, fN), ("fc2", "rs", fN, d)):
        if op == "ag":
            x, w = gen.ag_inputs_torch(N, m, k, n, "normal", 0, "cuda")
        else:
            x, w = gen.rs_inputs_torch(N, m, k, n, "normal", 0, "cuda")
            x = x[:1].contiguous()
        w = w[:1].contiguous()
        fn = nat.cm_ag_gemm if op == "ag" else nat.cm_gemm_rs
        comm = streams(1)[1]
        D = {}
        for ce in ("sdma", "cu"):
            plan = nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, share=1, out_dtype="bf16", n_comm=1,
                                    copy_engine=ce)
            y, ws = buffers.alloc_outputs(plan)
            if op == "rs":
                peer = gen.peer_buckets(N, m, n, "normal", 0)
                ws[:peer.nbytes].copy_(torch.from_numpy(peer.view(np.uint8).reshape(-1)))
            D[ce] = wall(fn, plan, x, w, y, ws, comm, reps)
            del y, ws
        best = min(D, key=D.get)
        # compute only: the same program with its hops replaced by empty
        # operations (every edge kept)
        p1 = nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, share=1, out_dtype="bf16", n_comm=1,
                              copy_engine=best, skip="hops")
        y1, ws1 = buffers.alloc_outputs(p1)
        if op == "rs":
            ws1[:peer.nbytes].copy_(torch.from_numpy(peer.view(np.uint8).reshape(-1)))
        g_only = wall(fn, p1, x, w, y1, ws1, comm, reps)
        del y1, ws1
        # per-launch breakdown (the trace's timing events slow the op down)
        plan = nat.cm_ring_plan(op=op, n_ranks=N, m=m, k=k, n=n, share=1, out_dtype="bf16", n_comm=1, copy_engine=best)
        y, ws = buffers.alloc_outputs(plan)
        ops, _ = nat.cm_plan_program(plan)
        cap = sum(1 for o in ops if o.kind in (nat.CM_OPK_GEMM, nat.CM_OPK_COPY, nat.CM_OPK_REDUCE))
        traces = [nat.Trace(cap) for _ in range(reps)]
        for _ in range(2):
            for tr in traces:
                fn(plan, x, w, y, ws, compute, comm, tr)
            torch.cuda.synchronize()
        g_each, r_each, c_each = [], [], []
        for tr in traces:
            spans, _total = tr.read()
            g_each += [q[5] - q[4] for q in spans if q[0] == nat.CM_OPK_GEMM]
            r_each += [q[5] - q[4] for q in spans if q[0] == nat.CM_OPK_REDUCE]
            c_each += [q[5] - q[4] for q in spans if q[0] == nat.CM_OPK_COPY]
            tr.close()
        g_us, r_us = float(np.median(g_each)), float(np.median(r_each))
        c_us = float(np.median(c_each)) if c_each else 0.0
        C = c_us * (N - 1)
        Db = D[best]
        flops = 2.0 * N * m * k * n  # rank 0's work in one op
        hop_bytes = m * k * 2 if op == "ag" else m * n * 4
        out[name] = {
            "op": op, "step_gemm": "[%dx%d].[%dx%d]" % (m, k, k, n), "split_k": plan.split,
            "tile": "%dx%d" % (plan.tile_m, plan.tile_n),
            "workgroups_per_step": plan.split * (-(-m // plan.tile_m)) * (-(-n // plan.tile_n)),
            "op_us": round(Db, 1), "op_us_sdma_hops": round(D["sdma"], 1), "op_us_cu_hops": round(D["cu"], 1),
            "hops_on": best, "tflops": round(flops / (Db * 1e-6) / 1e12, 1),
            "pct_of_bf16_peak": round(100 * flops / (Db * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "compute_only_us": round(g_only, 1),
            "gemm_us_per_step": round(g_us, 1), "gemm_tflops": round(2.0 * m * k * n / (g_us * 1e-6) / 1e12, 1),
            "reduce_us_per_step": round(r_us, 1),
            "hop_us_per_step": round(c_us, 1) if c_each else None,
            "hop_GBps": round(hop_bytes / (c_us * 1e-6) / 1e9, 1) if c_each else None,
            "overlap_efficiency": round(Db / max(g_only, C), 3),
            "hidden_fraction": round((g_only + C - Db) / C, 3) if C > 0 else None,
            "weight_shard_MB": round(n * k * 2 / 1e6, 1),
        }
        total_flops += flops
        total_us += Db
        log("share %s: %s split %d tile %s: op %.1f us (hops on %s; sdma %.1f, cu %.1f) -> %.1f TFLOP/s; compute "
            "only %.1f us; GEMM %.1f us/step = %.1f TFLOP/s, reduce %.1f us/step, hop %.1f us/step, hidden %s" % (
                name, out[name]["step_gemm"], plan.split, out[name]["tile"], Db, best, D["sdma"], D["cu"],
                out[name]["tflops"], g_only, g_us, out[name]["gemm_tflops"], r_us, c_us, out[name]["hidden_fraction"]))
        del x, w, y, ws
        torch.cuda.empty_cache()
    out["step_us"] = round(total_us, 1)
    out["tflops"] = round(total_flops / (total_us * 1e-6) / 1e12, 1)
    out["pct_of_bf16_peak"] = round(100 * out["tflops"] / PEAK_BF16_TFLOPS, 2)
    return out


def run_sweep(name, reps, copy_engine):
    """The small-chunk regime grid (d = 2048, ffn 8192, 1024 tokens, N in
    {2, 4, 8}, chunks in {1, 2, 4}, AG / RS / pipeline-chunk RS) or the four
    GEMM + collective pairs of the SP transformer layer (N = 8, 4096 tokens,
    d = 8192, ffn 28672); one JSON line per case."""
    cases = []
    if name == "c4":
        T, d, f = 1024, 2048, 8192
        for op in ("ag", "rs", "rs_pipe"):
            for N in (2, 4, 8):
                for c in (1, 2, 4):
                    k, n = (d, f // N) if op == "ag" else (f // N, d)
                    cases.append((op, N, T // N, k, n, c))
    else:
        N, m = 8, 512
        cases = [("ag", N, m, 8192, 3072, 0), ("rs_pipe", N, m, 1024, 8192, 4), ("ag", N, m, 8192, 3584, 0),
                 ("rs", N, m, 3584, 8192, 0)]
    for op, N, m, k, n, c in cases:
        r = measure_op(op, N, m, k, n, c, "uni", 1, reps, copy_engine)
        r["sweep"] = name
        log("%-4s %-7s N=%d c=%d [%dx%d].[%dx%d]^T: D %.1f us (G %.1f, C %.1f, eff %.2f, hidden %s) naive %.1f us -> x%.2f" % (
            copy_engine, op, N, r["chunks"], m, k, n, k, r["decomposed_us"], r["gemm_busy_us"], r["hop_busy_us"],
            r["overlap_efficiency"], r["hidden_fraction"], r["naive_us"], r["speedup_over_naive"]))
        print(json.dumps(r), flush=True)


LAYER = dict(N=8, T=4096, d=8192, heads=64, head_dim=128, ffn=28672)  # the full SP layer (4096 tokens, d 8192)


def measure_layer(args, steps, warmup):
    """The sequence-parallel transformer-layer forward on N = 8 virtual ranks
    (AG->QKV, causal attention, out-proj->pipeline-chunk RS, LayerNorm on the
    shard, AG->fc1+GELU, fc2->RS): whole-layer wall time over `steps` calls,
    then each stage alone between events on the compute stream."""
    import torch
    from collective_matmul_decomposition_amd import _native as nat
    from collective_matmul_decomposition_amd import buffers
    from collective_matmul_decomposition_amd import inputs as gen
    L = LAYER
    N, T, d, D, f = L["N"], L["T"], L["d"], L["head_dim"], L["ffn"]
    m, H, fN = T // N, L["heads"] // N, f // N
    HD = H * D
    ring = args.dir if args.dir != "bi" else "uni"
    plan = nat.cm_plan_layer(n_ranks=N, m=m, d=d, heads=H, ffn=fN, dir=ring, n_comm=args.n_comm,
                             copy_engine=args.layer_copy_engine, ag_chunks=1, rs_chunks=1, proj_chunks=0)
    engines = {s: ("cu" if getattr(plan, s).desc.copy_engine == nat.CM_COPY_CU else "sdma")
               for s in ("qkv", "proj", "fc1", "fc2")}
    x, wqkv, wo, w1, w2 = gen.layer_inputs_torch(N, m, d, H, D, fN, "normal", 0, "cuda")
    out = torch.empty((N, m, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device="cuda")
    compute, comm = streams(args.n_comm)
    compute.wait_stream(torch.cuda.current_stream())
    for _ in range(warmup):
        nat.cm_layer_forward(plan, x, wqkv, wo, w1, w2, out, ws, compute, comm)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        nat.cm_layer_forward(plan, x, wqkv, wo, w1, w2, out, ws, compute, comm)
    torch.cuda.synchronize()
    layer_ms = (time.perf_counter() - t0) * 1e3 / steps
    gemm_fl = {"qkv": 2.0 * N * T * d * 3 * HD, "proj": 2.0 * N * T * HD * d, "fc1": 2.0 * N * T * d * fN,
               "fc2": 2.0 * N * T * fN * d}
    attn_fl = 2.0 * N * H * D * T * (T + 1)  # causal: q.k and p.v over the T(T+1)/2 visible pairs
    total_fl = sum(gemm_fl.values()) + attn_fl
    # each stage alone, between events on the compute stream (the same calls
    # cm_layer_forward makes, on the same workspace regions)
    base = ws.data_ptr()
    reg = {k: base + getattr(plan, "off_" + k) for k in ("qkv", "attn", "proj", "ln", "fc1", "ops")}
    opbytes = plan.ws_bytes - plan.off_ops
    stages = [
        ("qkv", lambda: nat.cm_ag_gemm(plan.qkv, x, wqkv, reg["qkv"], reg["ops"], compute, comm, ws_bytes=opbytes)),
        ("attention", lambda: nat.cm_attention(reg["qkv"], reg["attn"], N, T, H, D, True, compute)),
        ("proj", lambda: nat.cm_gemm_rs(plan.proj, reg["attn"], wo, reg["proj"], reg["ops"], compute, comm,
                                        ws_bytes=opbytes)),
        ("layernorm", lambda: nat.cm_layernorm(reg["proj"], reg["ln"], N * m, d, plan.desc.ln_eps, None, None,
                                               compute)),
        ("fc1", lambda: nat.cm_ag_gemm(plan.fc1, reg["ln"], w1, reg["fc1"], reg["ops"], compute, comm,
                                       ws_bytes=opbytes)),
        ("fc2", lambda: nat.cm_gemm_rs(plan.fc2, reg["fc1"], w2, out, reg["ops"], compute, comm, ws_bytes=opbytes)),
    ]
    reps = max(3, steps)
    times = {}
    for name, fn in stages:
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(compute)
            fn()
            b.record(compute)
        torch.cuda.synchronize()
        times[name] = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3  # us
    st = {}
    for name in ("qkv", "proj", "fc1", "fc2"):
        st[name] = {"us": round(times[name], 1), "tflops": round(gemm_fl[name] / (times[name] * 1e-6) / 1e12, 1)}
    attn_t = times["attention"]
    st["attention"] = {"us": round(attn_t, 1), "tflops": round(attn_fl / (attn_t * 1e-6) / 1e12, 1),
                       "roofline": {"bound": "mfma", "achieved": round(attn_fl / (attn_t * 1e-6) / 1e12, 1),
                                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                    "frac": round(attn_fl / (attn_t * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                    "flops": attn_fl}}
    ln_bytes = N * m * d * (4 + 2)  # fp32 in, bf16 out
    ln_t = times["layernorm"]
    st["layernorm"] = {"us": round(ln_t, 1),
                       "roofline": {"bound": "hbm", "achieved": round(ln_bytes / (ln_t * 1e-6) / 1e9, 1),
                                    "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                    "frac": round(ln_bytes / (ln_t * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                                    "bytes": ln_bytes}}
    log("layer: %.3f ms, %.1f TFLOP/s; %s" % (layer_ms, total_fl / (layer_ms * 1e-3) / 1e12,
                                             ", ".join("%s %.0f us" % (k, v) for k, v in times.items())))
    res = {"workload": "sp-layer-fwd (N=8, 4096 tokens, d=8192, 64 heads x 128, ffn 28672)",
           "ms": round(layer_ms, 4), "tflops": round(total_fl / (layer_ms * 1e-3) / 1e12, 1),
           "pct_of_bf16_peak": round(100 * total_fl / (layer_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
           "flops": total_fl, "ring": ring, "proj_chunks": plan.proj.chunks,
           "copy_engine": args.layer_copy_engine, "hops_on": engines, "stages": st,
           "stage_sum_ms": round(sum(times.values()) / 1e3, 4)}
    del x, wqkv, wo, w1, w2, out, ws
    torch.cuda.empty_cache()
    return res


def measure_backward(args, workload, steps, warmup):
    """The backward of the workload's two linears (fc1: column-parallel, the
    forward was AllGather->GEMM; fc2: row-parallel, the forward was
    GEMM->ReduceScatter), bf16 gradients: wall time per call with the weight
    gradient's AllGather on the bulk stream (bulk overlap) and in the serial
    order, and with the transposed weights passed in."""
    import torch
    from collective_matmul_decomposition_amd import _native as nat
    from collective_matmul_decomposition_amd import buffers
    from collective_matmul_decomposition_amd import inputs as gen
    wl = WORKLOADS[workload]
    N, T, d, f = wl["N"], wl["T"], wl["d"], wl["f"]
    m, fN = T // N, f // N
    compute, comm = streams(3)
    compute.wait_stream(torch.cuda.current_stream())
    out = {"workload": workload}
    for kind, k, n in (("col", d, fN), ("row", fN, d)):
        act, w, grad = gen.backward_inputs_torch(kind, N, m, k, n, "normal", 0, "cuda")
        wt = w.transpose(1, 2).contiguous()
        dact = torch.empty((N, m, k) if kind == "col" else (N, T, k), dtype=torch.bfloat16, device="cuda")
        dw = torch.empty((N, n, k), dtype=torch.bfloat16, device="cuda")
        flops = 2 * 2.0 * N * T * n * k  # input gradient + weight gradient
        r = {}
        for label, bulk, wtp in (("bulk", True, None), ("serial", False, None), ("bulk_wt_given", True, wt)):
            plan = nat.cm_plan_backward(kind=kind, n_ranks=N, m=m, k=k, n=n, chunks=1, n_comm=1, bulk=bulk,
                                        dx_dtype="bf16", dw_dtype="bf16", copy_engine=args.copy_engine)
            ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device="cuda")
            call = lambda: nat.cm_linear_backward(plan, act, w, wtp, grad, dact, dw, ws, compute, comm)
            for _ in range(warmup):
                call()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                call()
            torch.cuda.synchronize()
            us = (time.perf_counter() - t0) / steps * 1e6
            r[label + "_us"] = round(us, 1)
            if label == "bulk":
                r["tflops"] = round(flops / (us * 1e-6) / 1e12, 1)
            del ws
        r["bulk_speedup_over_serial"] = round(r["serial_us"] / r["bulk_us"], 3)
        r["flops"] = flops
        out["fc1_col" if kind == "col" else "fc2_row"] = r
        log("backward %s: bulk %.0f us (%.0f TFLOP/s), serial %.0f us, W^T given %.0f us" % (
            kind, r["bulk_us"], r["tflops"], r["serial_us"], r["bulk_wt_given_us"]))
        del act, w, grad, wt, dact, dw
        torch.cuda.empty_cache()
    tot = out["fc1_col"]["bulk_us"] + out["fc2_row"]["bulk_us"]
    out["mlp_backward_ms"] = round(tot / 1e3, 4)
    out["mlp_backward_tflops"] = round((out["fc1_col"]["flops"] + out["fc2_row"]["flops"]) / (tot * 1e-6) / 1e12, 1)
    return out


def sampled_parity(res, rs_bucket="f32"):
    import oracle
    from collective_matmul_decomposition_amd import inputs as gen
    x, w1, y1, h, w2, y2 = res["tensors"]
    N, T, m = res["N"], res["T"], res["m"]
    xa, w1a = gen.torch_bf16_to_bits(x), gen.torch_bf16_to_bits(w1)
    ha, w2a = gen.torch_bf16_to_bits(h), gen.torch_bf16_to_bits(w2)
    rng = np.random.default_rng(0)
    rk, rw = rng.integers(0, N, 4), rng.integers(0, T, 4)
    ref, mag = oracle.ag_gemm_rows(xa, w1a, rk, rw, with_mag=True)
    got = gen.bf16_bits_to_f32(gen.torch_bf16_to_bits(y1)[rk, rw]).astype(np.float64)
    worst_ag = float((np.abs(got - ref) / (1e-5 * mag + 2.0 ** -8 * np.abs(ref))).max())
    qo, qr = rng.integers(0, N, 4), rng.integers(0, m, 4)
    if rs_bucket == "bf16":
        ref, mag, rmag = oracle.gemm_rs_bf16_bucket_rows(ha, w2a, qo, qr, with_mag=True)
        mag = mag + 2.0 ** -7 / 1e-5 * rmag  # each bucket rounding: up to one bf16 spacing
    else:
        ref, mag = oracle.gemm_rs_rows(ha, w2a, qo, qr, with_mag=True)
    got = gen.bf16_bits_to_f32(gen.torch_bf16_to_bits(y2)[qo, qr]).astype(np.float64)
    worst_rs = float((np.abs(got - ref) / (1e-5 * mag + 2.0 ** -8 * np.abs(ref))).max())
    return {"ag": round(worst_ag, 4), "rs": round(worst_rs, 4)}, (xa, w1a, ha, w2a)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(res, arrays, seconds):
    """The oracle timed on the host's cores on a row sample of the step; then
    the same rows (with the |a||b| magnitudes, untimed) are checked against
    the GPU's step output."""
    import oracle
    from collective_matmul_decomposition_amd import inputs as gen
    xa, w1a, ha, w2a = arrays
    x, w1, y1, h, w2, y2 = res["tensors"]
    N, T, m, d, fN = res["N"], res["T"], res["m"], res["d"], res["fN"]
    rng = np.random.default_rng(1)
    cores = oracle.threads()
    t0 = time.perf_counter()
    oracle.ag_gemm_rows(xa, w1a, np.zeros(cores, np.int32), np.arange(cores, dtype=np.int32))
    per_row = (time.perf_counter() - t0) / cores
    rows_ag = int(max(cores, min(N * T, seconds / max(per_row, 1e-9))))
    sel_ag = rng.choice(N * T, rows_ag, replace=False)
    ra, rr = (sel_ag // T).astype(np.int32), (sel_ag % T).astype(np.int32)
    t0 = time.perf_counter()
    ref_ag = oracle.ag_gemm_rows(xa, w1a, ra, rr)
    t_ag = time.perf_counter() - t0
    rows_rs = max(cores, rows_ag // N)
    sel = rng.choice(N * m, min(rows_rs, N * m), replace=False)
    qo, qr = (sel // m).astype(np.int32), (sel % m).astype(np.int32)
    t0 = time.perf_counter()
    ref_rs = oracle.gemm_rs_rows(ha, w2a, qo, qr)
    t_rs = time.perf_counter() - t0
    fl = 2.0 * rows_ag * d * fN + 2.0 * len(sel) * N * fN * d
    # parity of the same rows: |gpu - oracle| <= 1e-5 * sum|a||b| + 2^-8 |oracle| (bf16 outputs)
    _, mag_ag = oracle.ag_gemm_rows(xa, w1a, ra, rr, with_mag=True)
    _, mag_rs = oracle.gemm_rs_rows(ha, w2a, qo, qr, with_mag=True)
    got_ag = gen.bf16_bits_to_f32(gen.torch_bf16_to_bits(y1)[ra, rr]).astype(np.float64)
    got_rs = gen.bf16_bits_to_f32(gen.torch_bf16_to_bits(y2)[qo, qr]).astype(np.float64)
    w_ag = float((np.abs(got_ag - ref_ag) / (1e-5 * mag_ag + 2.0 ** -8 * np.abs(ref_ag))).max())
    w_rs = float((np.abs(got_rs - ref_rs) / (1e-5 * mag_rs + 2.0 ** -8 * np.abs(ref_rs))).max())
    log("cpu baseline: %d AG + %d RS rows in %.1f s on %d cores; their parity err/bound: AG %.4f, RS %.4f" % (
        rows_ag, len(sel), t_ag + t_rs, cores, w_ag, w_rs))
    return {"value": round(fl / (t_ag + t_rs) / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "%d of %d AG output rows and %d of %d RS output rows of the step (fp64, all %d rank "
                      "contributions each), %.1f s" % (rows_ag, N * T, len(sel), N * m, N, t_ag + t_rs),
            "parity": {"ag_rows": rows_ag, "rs_rows": int(len(sel)), "max_err_over_bound_ag": round(w_ag, 4),
                       "max_err_over_bound_rs": round(w_rs, 4),
                       "passed": bool(w_ag <= 1.0 and w_rs <= 1.0)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt3-175b-mlp", choices=sorted(WORKLOADS))
    ap.add_argument("--secondary", default="llama3-8b-mlp", help="second workload reported beside (or 'none')")
    ap.add_argument("--dir", default="uni", choices=["uni", "bi", "direct"])
    ap.add_argument("--rs-op", default="rs", choices=["rs", "rs_pipe"])
    ap.add_argument("--chunks-ag", type=int, default=0)
    ap.add_argument("--chunks-rs", type=int, default=1, help="RS column chunks (0: cost model)")
    ap.add_argument("--n-comm", type=int, default=1, help="comm streams (copy lanes) per op")
    ap.add_argument("--copy-engine", default="auto", choices=["sdma", "cu", "auto"],
                    help="what moves the ring hops (auto: the planner chooses per op)")
    ap.add_argument("--layer-copy-engine", default="auto", choices=["sdma", "cu", "auto"],
                    help="what moves the layer's ring hops (auto: the planner chooses per stage)")
    ap.add_argument("--no-alt-copy", action="store_true", help="skip the run with the other copy engine")
    ap.add_argument("--rs-bucket", default="f32", choices=["f32", "bf16"],
                    help="element type of the circulating RS bucket (bf16: half the hop bytes, outside the "
                         "fp32-bucket error bound)")
    ap.add_argument("--no-alt-bucket", action="store_true", help="skip the run with the other RS bucket type")
    ap.add_argument("--no-alt-hop", action="store_true", help="skip the run with the other RS hop kind")
    ap.add_argument("--rs-hop", default="add", choices=["copy", "add"],
                    help="RS ring hop: a copy with the addition in the GEMM epilogue, or an add-and-forward "
                         "launch that lets each step's GEMM start without waiting for the previous hop")
    ap.add_argument("--tile", default="0x0")
    ap.add_argument("--group", type=int, default=0,
                    help="steps per GEMM launch (0: cost model, 1: one step per launch, g: at most g)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time")
    ap.add_argument("--no-naive", action="store_true")
    ap.add_argument("--no-bi", action="store_true", help="skip the run on the bidirectional ring")
    ap.add_argument("--bi-n-comm", type=int, default=1,
                    help="comm streams of the bidirectional-ring run (2: one per direction; measured slower)")
    ap.add_argument("--no-alone", action="store_true", help="skip timing G and C alone (the measurement modes)")
    ap.add_argument("--skip", default="none", choices=["none", "hops", "gemms"],
                    help="time the step itself in a measurement mode (hops or GEMMs replaced by empty "
                         "operations; for profiling the GEMM launches alone)")
    ap.add_argument("--no-layer", action="store_true", help="skip the sequence-parallel layer forward")
    ap.add_argument("--no-share", action="store_true", help="skip one rank's share (rank 0's steps at real shape)")
    ap.add_argument("--no-backward", action="store_true", help="skip the MLP backward (bulk overlap)")
    ap.add_argument("--no-c4", action="store_true", help="skip the small-chunk grid (d 2048, N 2/4/8, chunks 1/2/4)")
    ap.add_argument("--no-trace", action="store_true", help="time without the per-launch events")
    ap.add_argument("--timeline", action="store_true",
                    help="log the last timed step's operations (GEMM launches, copies, adds) with their times")
    ap.add_argument("--sweep", choices=["c4", "c5"], help="instead of the step: the small-chunk grid (c4) or the "
                    "layer's GEMM + collective pairs (c5), one JSON line per case")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the N-rank tensor-parallel group is emulated as virtual ranks on a "
              "single MI355X; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from collective_matmul_decomposition_amd import _native as nat
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    nat.lib()
    streams(3)  # the run's streams, first, so they take the same hardware queues in every run

    if args.sweep:
        run_sweep(args.sweep, max(3, args.steps // 2), args.copy_engine)
        return

    if args.calib_copy_mib:
        # plain kernels of known traffic, for scaling the FETCH_SIZE / WRITE_SIZE
        # counters: a fill that writes the buffer, then an fp32 -> bf16 copy
        # kernel that reads it once (and writes half as many bytes)
        nbytes = args.calib_copy_mib << 20
        a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        # a second fill of the same size evicts `a` from the last-level cache,
        # so the copy below reads all of it from HBM
        flush = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(2.0)
        b = a.to(torch.bfloat16)
        torch.cuda.synchronize()
        del a, b, flush
    res = measure(args, args.workload, args.steps, args.warmup, not args.no_naive, not args.no_trace)
    parity, cpu = None, None
    if args.skip == "none":  # in a measurement mode the outputs are not computed
        parity, arrays = sampled_parity(res, args.rs_bucket if args.rs_op == "rs" else "f32")
        cpu = None if args.no_cpu_baseline else cpu_baseline(res, arrays, args.cpu_seconds)
    del res["tensors"]
    torch.cuda.empty_cache()
    alt = None
    if not args.no_alt_copy:
        # the same step with the other engine moving the hops
        alt_args = argparse.Namespace(**vars(args))
        alt_args.copy_engine = "cu" if res["hops_on"]["ag"] == "sdma" else "sdma"
        ra = measure(alt_args, args.workload, args.steps, args.warmup, False, not args.no_trace)
        alt = {"copy_engine": alt_args.copy_engine, "value": round(ra["value"], 2), "unit": "TFLOP/s",
               "ms_per_step": round(ra["ms_per_step"], 4), "overlap": ra.get("overlap"),
               "gemm_launches": ra.get("gemm_launches")}
        del ra
        torch.cuda.empty_cache()
    alt_bucket = None
    if not args.no_alt_bucket and args.rs_op == "rs":
        alt_args = argparse.Namespace(**vars(args))
        alt_args.rs_bucket = "bf16" if args.rs_bucket == "f32" else "f32"
        rb = measure(alt_args, args.workload, args.steps, args.warmup, False, not args.no_trace)
        alt_bucket = {"rs_bucket": alt_args.rs_bucket, "rs_hop": rs_hop(alt_args), "value": round(rb["value"], 2),
                      "unit": "TFLOP/s",
                      "ms_per_step": round(rb["ms_per_step"], 4), "overlap": rb.get("overlap")}
        del rb
        torch.cuda.empty_cache()
    alt_hop = None
    if not args.no_alt_hop and rs_hop(args) == args.rs_hop:
        alt_args = argparse.Namespace(**vars(args))
        alt_args.rs_hop = "copy" if args.rs_hop == "add" else "add"
        rh = measure(alt_args, args.workload, args.steps, args.warmup, False, not args.no_trace)
        alt_hop = {"rs_hop": alt_args.rs_hop, "value": round(rh["value"], 2), "unit": "TFLOP/s",
                   "ms_per_step": round(rh["ms_per_step"], 4), "overlap": rh.get("overlap"),
                   "gemm_launches": rh.get("gemm_launches")}
        del rh
        torch.cuda.empty_cache()
    bi = None
    if not args.no_bi and args.dir != "bi":
        # the same step on the bidirectional ring
        bi_args = argparse.Namespace(**vars(args))
        bi_args.dir = "bi"
        bi_args.n_comm = args.bi_n_comm  # one comm lane (copy engine queue) per direction
        rb = measure(bi_args, args.workload, args.steps, args.warmup, False, not args.no_trace)
        def bi_row(rb):
            return {"ring": "bi", "n_comm_streams": bi_args.n_comm, "value": round(rb["value"], 2),
                    "unit": "TFLOP/s", "ms_per_step": round(rb["ms_per_step"], 4), "hops_on": rb["hops_on"],
                    "steps_per_launch_ag": list(rb["plan_ag"].group_len[:rb["plan_ag"].n_launches]),
                    "steps_per_launch_rs": list(rb["plan_rs"].group_len[:rb["plan_rs"].n_launches]),
                    "pct_of_bf16_peak": round(100 * rb["value"] / PEAK_BF16_TFLOPS, 2), "overlap": rb.get("overlap"),
                    "gemm_launches": rb.get("gemm_launches")}
        bi = bi_row(rb)
        del rb
        torch.cuda.empty_cache()
        if bi["hops_on"]["ag"] != "sdma":
            # the bidirectional ring with its AllGather hops on the SDMA engines as well
            bi_args.copy_engine = "sdma"
            rb = measure(bi_args, args.workload, args.steps, args.warmup, False, not args.no_trace)
            bi["sdma_hops"] = bi_row(rb)
            del rb
            torch.cuda.empty_cache()
    secondary = None
    if args.secondary != "none" and args.secondary != args.workload:
        s2 = measure(args, args.secondary, max(5, args.steps // 2), 2, not args.no_naive, not args.no_trace)
        secondary = {"workload": args.secondary, "value": round(s2["value"], 2), "unit": "TFLOP/s",
                     "ms_per_step": round(s2["ms_per_step"], 4), "hops_on": s2["hops_on"],
                     "pct_of_bf16_peak": round(100 * s2["value"] / PEAK_BF16_TFLOPS, 2),
                     "roofline": s2.get("roofline"), "overlap": s2.get("overlap"), "naive": s2.get("naive")}
        del s2
        torch.cuda.empty_cache()
        if not args.no_alt_copy:
            # the same step with the other engine moving the hops (at these small hops it matters)
            alt_args = argparse.Namespace(**vars(args))
            alt_args.copy_engine = "cu" if secondary["hops_on"]["ag"] == "sdma" else "sdma"
            s3 = measure(alt_args, args.secondary, max(5, args.steps // 2), 2, False, not args.no_trace)
            secondary["alt_copy_engine"] = {"copy_engine": alt_args.copy_engine, "value": round(s3["value"], 2),
                                            "ms_per_step": round(s3["ms_per_step"], 4), "overlap": s3.get("overlap")}
            del s3
            torch.cuda.empty_cache()

    share = None if args.no_share else measure_share(args.workload, max(10, args.steps))
    layer = None if args.no_layer else measure_layer(args, max(5, args.steps // 2), 2)
    backward = None if args.no_backward else measure_backward(args, args.workload, max(5, args.steps // 2), 2)
    c4 = None
    if not args.no_c4:
        # the small-chunk regime grid (d = 2048, ffn 8192, 1024 tokens, N in {2, 4, 8}, chunks in {1, 2, 4}):
        # where per-chunk GEMMs are too small to hide the hops and the launch overhead
        c4 = []
        T4, d4, f4 = 1024, 2048, 8192
        for op in ("ag", "rs", "rs_pipe"):
            for N4 in (2, 4, 8):
                for c in (1, 2, 4):
                    k4, n4 = (d4, f4 // N4) if op == "ag" else (f4 // N4, d4)
                    r = measure_op(op, N4, T4 // N4, k4, n4, c, "uni", 1, 3, args.copy_engine)
                    c4.append({key: r[key] for key in ("op", "N", "chunks", "decomposed_us", "gemm_busy_us",
                                                       "hop_busy_us", "hidden_fraction", "naive_us",
                                                       "speedup_over_naive", "declined_by_cost_model")})
        log("c4 sweep: %s" % "; ".join("%s N=%d c=%d D %.0f naive x%.2f" % (
            r["op"], r["N"], r["chunks"], r["decomposed_us"], r["speedup_over_naive"]) for r in c4))
        torch.cuda.empty_cache()

    out = {
        "metric": "AG-GEMM / GEMM-RS TFLOP/s + % bf16 MFMA peak + overlap efficiency, 1 GPU",
        "value": round(res["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "virtual_ranks": res["N"], "tokens": res["T"], "hidden": res["d"],
                   "ffn": res["f"], "ffn_per_rank": res["fN"], "ring": args.dir, "rs_variant": args.rs_op,
                   "n_comm_streams": res["n_comm"], "copy_engine": args.copy_engine, "hops_on": res["hops_on"], "rs_bucket": args.rs_bucket,
                   "rs_hop": rs_hop(args), "measurement_mode": args.skip,
                   "chunks_ag": res["plan_ag"].chunks,
                   "chunks_rs": res["plan_rs"].chunks,
                   "steps_per_launch_ag": list(res["plan_ag"].group_len[:res["plan_ag"].n_launches]),
                   "steps_per_launch_rs": list(res["plan_rs"].group_len[:res["plan_rs"].n_launches]),
                   "step": "AllGather->GEMM (fc1) then GEMM->ReduceScatter (fc2), decomposed, bf16 in / fp32 "
                           "accumulate / bf16 out"},
        "pct_of_bf16_peak": round(100 * res["value"] / PEAK_BF16_TFLOPS, 2),
        "roofline": res.get("roofline"),
        "roofline_gemm_alone": res.get("roofline_gemm_alone"),
        "cpu_baseline": cpu,
        "overlap": res.get("overlap"),
        "gemm_launches": res.get("gemm_launches"),
        "naive": res.get("naive"),
        "parity_sampled_err_over_bound": parity,
        "bi": bi,
        "alt_copy_engine": alt,
        "alt_rs_bucket": alt_bucket,
        "alt_rs_hop": alt_hop,
        "step_launches": res.get("step_launches"),
        "timeline": res.get("timeline"),
        "secondary": secondary,
        "one_rank_share": share,
        "layer": layer,
        "backward": backward,
        "c4_sweep": c4,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
