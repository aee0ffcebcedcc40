"""Benchmark: zigzag ring context-parallel attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One timed step = one call of the library's hot path over the workload's share:
for the default workload, rank 0's share of a causal 32768-token sequence at
cp 8 (zigzag chunks {0, 15}, 32 heads x 128, bf16): 8 ring steps, each with the
next step's K/V received into the other slot while the step computes,
blockwise MFMA attention with the LSE merge in the epilogue, and the final
scatter of O/LSE to token positions.  Inputs are resident in HBM before timing
starts.  Other schedule modes (side-stream receive, separate merge kernel,
serialized) are timed alongside and reported under "modes_ms".

Prints ONE JSON line.  `value` is effective TFLOP/s over mask-valid FLOPs
(4 * head_dim per valid (query, key) pair per head).
"""

import argparse
import json
import os
import platform
import sys
import time

import numpy as np
import torch

DEFAULT_WORKLOAD = "causal_s32768_cp8_zigzag_h32_d128_bf16_rank0"
METRIC = "effective causal attn TFLOP/s (valid FLOPs) + % bf16 MFMA peak; zigzag imbalance"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="keep warming up (untimed calls) until this long has passed, so clocks have ramped")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip imbalance / mode / parity side measurements")
    ap.add_argument("--cpu-seconds", type=float, default=40.0,
                    help="bound on the oracle's CPU time (the 32k/cp8 rank-0 share takes about 25 s)")
    ap.add_argument("--recv", choices=["kernel", "memcpy", "fused", "hybrid"], default=None, help="ring receive path (default: library's)")
    ap.add_argument("--recv-blocks", type=int, default=None, help="grid bound of the receive copy kernel")
    ap.add_argument("--serialize", action="store_true", help="run the whole schedule on one stream")
    ap.add_argument("--graph", action="store_true", help="graph mode: each call replays a recorded HIP graph")
    ap.add_argument("--merge", choices=["fused", "separate"], default="fused",
                    help="LSE merge in the attention epilogue (default) or in the separate merge/finalize kernels")
    ap.add_argument("--backward", action="store_true",
                    help="also time the share's backward (on by default with the extras)")
    ap.add_argument("--no-key-split", action="store_true", help="never split a step's keys over two workgroups")
    ap.add_argument("--no-fused-ring", action="store_true",
                    help="one launch of the step kernel per ring step instead of one per rank")
    ap.add_argument("--fused-ring-staged", action="store_true",
                    help="fused ring with every receive done before the launch (for counter collection, "
                         "which runs one kernel at a time)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one layout gather of q (a plain copy of known size) before timing, "
                         "as the reference for hardware traffic counters")
    return ap.parse_args()


def share_pairs(plan, w):
    ranks = range(w.cp) if w.rank is None else [w.rank]
    return sum(plan.valid_work(r, s, 128, 64)[1] for r in ranks for s in range(w.cp))


def run_call(plan, w, bufs, stream):
    q, k, v, out, lse = bufs
    if w.rank is None:
        plan.full_forward(q, k, v, out, lse, stream=stream)
    else:
        plan.rank_forward(q, k, v, out, lse, w.rank, stream=stream)


def time_calls(plan, w, bufs, stream, steps, warmup, warmup_seconds=0.0):
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < warmup_seconds:
        run_call(plan, w, bufs, stream)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        run_call(plan, w, bufs, stream)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    time_calls.last = {"median": float(np.median(per)), "min": float(np.min(per))}
    return ev[0].elapsed_time(ev[steps]) / steps


def step_kernel_times(plan, w, bufs, stream, reps, graph=False, queued=1):
    """Per-(rank, step) attention-kernel ms from the library's own HIP events
    (recorded by eager calls: graph mode records no step events).  queued > 1:
    each sample is the last of that many calls queued back to back, so the
    launch runs as in the timed loop rather than on a GPU left idle by the
    host's wait for the previous call's events."""
    plan.set_graph(False)
    plan.set_step_timing(True)
    acc = None
    for _ in range(reps):
        for _ in range(queued):
            run_call(plan, w, bufs, stream)
        t = np.array(plan.last_step_times())
        acc = t if acc is None else acc + t
    plan.set_step_timing(False)
    plan.set_graph(graph)
    return acc / reps


def kernel_launches(plan, w, bufs, stream, reps):
    """The attention launches of one call of the plan's default schedule:
    (kind, per-launch ms list), from the library's HIP step events recorded
    on the launching stream right around each launch: one per ring step, or
    one per rank for a call that ran fused (CP_ATTN_OPT_FUSED_RING, reported
    under step 0)."""
    run_call(plan, w, bufs, stream)
    torch.cuda.synchronize()
    fused = plan.fused_ring_active()
    times = step_kernel_times(plan, w, bufs, stream, reps, queued=4)
    ranks = range(w.cp) if w.rank is None else [w.rank]
    return ("fused_ring" if fused else "per_step"), [times[r][s] for r in ranks for s in range(w.cp) if times[r][s] > 0]


PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                       "attn_step_bf16_d128_causal_s32768_cp8_rank0.md")
KERNEL_SOURCES = ("attn_bf16.hip", "epilogue.h", "kernels.h", "lds_dma.h")


def recorded_traffic(workload):
    """HBM bytes per launch of the step kernel from the committed rocprofv3 summary,
    or None when the kernel source has changed since the counters were taken."""
    if workload != DEFAULT_WORKLOAD or not os.path.exists(PROFILE):
        return None
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "ring_context_parallelism_amd", "csrc")
    for f in KERNEL_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    fields = {}
    with open(PROFILE) as fh:
        for line in fh:
            if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "kernel_source_sha256"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != h.hexdigest():
        return None
    return int(fields["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in fields else None


def cpu_baseline(w, q, k, v, out, lse, target_s):
    """The fp64 oracle on the same share, timed on the host: every row of the
    share (at most 4096) for one head per worker thread, BLAS held to one
    thread per worker (numpy releases the GIL in BLAS and its ufuncs), waves of
    heads until every head is done or target_s has passed.  Its results are
    also compared with the GPU's output of the timed call (parity over the
    rows and heads it covered)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from ring_context_parallelism_amd.inputs import to_numpy_f64
    from threadpoolctl import threadpool_limits
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    workers = max(1, min(avail, 16))  # at most 16 worker threads
    ranks = range(w.cp) if w.rank is None else [w.rank]
    rows = np.concatenate([oracle.rank_positions(w.seq_len, w.cp, r, w.layout) for r in ranks])
    rows = rows[:: max(1, rows.size // 4096)][:4096]
    kpos = np.arange(w.seq_len)
    rows_t = torch.from_numpy(rows)

    def one_head(h):
        qh = to_numpy_f64(q[rows_t, h:h + 1])
        kh = to_numpy_f64(k[:, h:h + 1])
        vh = to_numpy_f64(v[:, h:h + 1])
        return h, oracle.attention(qh, kh, vh, causal=w.causal, q_pos=rows, k_pos=kpos)

    results = {}
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(workers) as ex:
        t0 = time.perf_counter()
        h = 0
        while h < w.heads and (h == 0 or time.perf_counter() - t0 < target_s):
            wave = range(h, min(w.heads, h + workers))
            for hh, res in ex.map(one_head, wave):
                results[hh] = res
            h = wave.stop
        t_cpu = time.perf_counter() - t0
    pairs = int((rows + 1).sum()) if w.causal else rows.size * w.seq_len
    flops = oracle.valid_flops(pairs, len(results), w.head_dim)
    out_c = out.cpu()
    lse_c = lse.cpu()
    d_o = d_l = 0.0
    for h, (o_ref, l_ref) in results.items():
        o_got = out_c[rows_t, h:h + 1].to(torch.float64).numpy()
        l_got = lse_c[h, rows_t].to(torch.float64).numpy()
        d_o = max(d_o, float(np.max(np.abs(o_got - o_ref))))
        d_l = max(d_l, float(np.max(np.abs(l_got - l_ref[0]))))
    whole = rows.size == sum(oracle.rank_positions(w.seq_len, w.cp, r, w.layout).size for r in ranks)
    return {"value": flops / t_cpu / 1e12, "unit": "TFLOP/s", "cores": int(workers), "kind": "oracle",
            "sample": (f"{'the whole share: ' if whole else ''}{rows.size} rows x {len(results)} of {w.heads} "
                       f"heads, every valid key, fp64 numpy, one head per thread on {workers} threads "
                       f"(BLAS 1 thread each; host reports {os.cpu_count()} CPUs, {avail} usable); "
                       f"{flops / 1e9:.1f} GFLOP in {t_cpu:.1f} s"),
            "parity": {"rows": int(rows.size), "heads": len(results), "max_abs_dO": d_o, "max_abs_dLSE": d_l}}


def imbalance_section(stream):
    """Zigzag vs contiguous at 16384 tokens, cp 4: plan tiles and measured step times."""
    import ring_context_parallelism_amd as R
    from ring_context_parallelism_amd.inputs import WORKLOADS, workload_qkv
    res = {}
    for layout in ("zigzag", "contiguous"):
        w = WORKLOADS[f"causal_s16384_cp4_{layout}_h16_d128_bf16"]
        p = R.Plan(w.seq_len, w.cp, w.heads, w.head_dim, w.causal, w.layout)
        p.set_fused_ring(False)  # per-step times: the one-launch-per-step schedule
        tiles = [[p.valid_work(r, s, 128, 64)[0] for s in range(w.cp)] for r in range(w.cp)]
        q, k, v = (t.cuda() for t in workload_qkv(w))
        out = torch.empty_like(q)
        lse = torch.empty(w.heads, w.seq_len, device="cuda")
        bufs = (q, k, v, out, lse)
        p.set_counters(True)
        run_call(p, w, bufs, stream)
        dev_tiles, (tr, tk) = p.last_tile_counts()
        p.set_counters(False)
        plan_fine = [[w.heads * p.valid_work(r, s, tr, tk)[0] for s in range(w.cp)] for r in range(w.cp)]
        times = step_kernel_times(p, w, bufs, stream, 3)
        ms = time_calls(p, w, bufs, stream, 5, 1)
        def imb(tab):
            t = np.asarray(tab, dtype=np.float64)
            mx, mean = t.max(axis=0), t.mean(axis=0)
            return [round(float(a / b), 4) if b > 0 else 1.0 for a, b in zip(mx, mean)], round(
                float(mx.sum() / mean.sum()), 4)
        per_t, agg_t = imb(tiles)
        per_m, agg_m = imb(times)
        res[layout] = {"tiles_128x64": tiles, "tile_imbalance_per_step": per_t, "tile_imbalance": agg_t,
                       f"device_tiles_{tr}x{tk}_all_heads": dev_tiles,
                       "device_tiles_match_plan": dev_tiles == plan_fine,
                       "step_ms": [[round(float(x), 4) for x in row] for row in times],
                       "time_imbalance_per_step": per_m, "time_imbalance": agg_m,
                       "full_forward_ms": round(ms, 4)}
        p.close()
        del q, k, v, out, lse, bufs
        torch.cuda.empty_cache()
    return res


def workload_section(name, stream, steps, graph_too=False):
    """One of the other workloads, timed like the headline: calls per second
    over its share, effective TFLOP/s of the valid pairs, the step kernel's
    mean launch time from the library's step events and its fraction of the
    bf16 peak, (graph_too) the same calls replayed from a HIP graph, and, for
    a share of every rank, the ranks in lockstep (every rank's ring step in
    one launch, CP_ATTN_OPT_LOCKSTEP)."""
    import ring_context_parallelism_amd as R
    from ring_context_parallelism_amd.inputs import WORKLOADS, workload_qkv
    w = WORKLOADS[name]
    p = R.Plan(w.seq_len, w.cp, w.heads, w.head_dim, w.causal, w.layout, dtype=w.torch_dtype)
    q, k, v = (t.cuda() for t in workload_qkv(w))
    out = torch.empty_like(q)
    lse = torch.empty(w.heads, w.seq_len, device="cuda")
    bufs = (q, k, v, out, lse)
    pairs = share_pairs(p, w)
    flops = 4 * w.head_dim * w.heads * pairs
    ms = time_calls(p, w, bufs, stream, steps, 3, 0.3)
    med = time_calls.last["median"]
    kind, launches = kernel_launches(p, w, bufs, stream, 3)
    avg = float(np.mean(launches))
    kern = flops / len(launches) / (avg * 1e-3) / 1e12
    res = {"workload": name, "share": "all ranks" if w.rank is None else f"rank {w.rank}", "valid_flops": flops,
           "ms_per_call": round(ms, 5), "ms_per_call_median": round(med, 5),
           "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "frac_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "step_kernel": {"schedule": kind, "launches_per_call": len(launches), "avg_launch_ms": round(avg, 5),
                           "tflops": round(kern, 2), "frac_bf16_peak": round(kern / PEAK_BF16_TFLOPS, 4)}}
    if kind == "fused_ring":
        p.set_fused_ring(False)
        sms = time_calls(p, w, bufs, stream, steps, 3, 0.3)
        p.set_fused_ring(True)
        res["one_launch_per_step_ms_per_call"] = round(sms, 5)
    if graph_too:
        p.set_graph(True)
        gms = time_calls(p, w, bufs, stream, steps, 3, 0.3)
        p.set_graph(False)
        res["graph_replay_ms_per_call"] = round(gms, 5)
        res["graph_replay_median_ms"] = round(time_calls.last["median"], 5)
    if w.rank is None:
        p.set_lockstep(True)
        lms = time_calls(p, w, bufs, stream, steps, 3, 0.3)
        p.set_lockstep(False)
        res["lockstep"] = {"ms_per_call": round(lms, 5), "ms_per_call_median": round(time_calls.last["median"], 5),
                           "tflops": round(flops / (lms * 1e-3) / 1e12, 2),
                           "frac_bf16_peak": round(flops / (lms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "launches_per_call": w.cp}
    p.close()
    del q, k, v, out, lse, bufs
    torch.cuda.empty_cache()
    return res


def rank_step_imbalance(plan, w, bufs, stream, reps=3):
    """Every rank's share of the timed workload, one rank_forward call each:
    per-(rank, step) step-kernel ms of the one-launch-per-step schedule,
    per-step max/mean over ranks, and the valid 128x64 tile counts (the
    plan's balance); then every rank's share measured whole: back to back
    with the fused ring, back to back one launch per step, and in lockstep;
    and each rank's fused call alone."""
    plan.set_fused_ring(False)
    times = []
    for r in range(w.cp):
        plan.set_step_timing(True)
        acc = None
        for _ in range(reps):
            plan.rank_forward(*bufs, r, stream=stream)
            t = np.array(plan.last_step_times())[r]
            acc = t if acc is None else acc + t
        plan.set_step_timing(False)
        times.append(acc / reps)
    t = np.asarray(times)
    per = [round(float(t[:, s].max() / t[:, s].mean()), 4) for s in range(w.cp)]
    tiles = [[plan.valid_work(r, s, 128, 64)[0] for s in range(w.cp)] for r in range(w.cp)]
    # A ring runs in lockstep: step s of the job takes the slowest rank's
    # step s.  Per GPU, the job's valid FLOPs (all ranks, divided by cp) over
    # the sum of those maxima of the step kernels' times.
    all_pairs = sum(plan.valid_work(r, s, 128, 64)[1] for r in range(w.cp) for s in range(w.cp))
    lockstep_ms = float(t.max(axis=0).sum())
    lockstep_tflops = 4 * w.head_dim * w.heads * all_pairs / w.cp / (lockstep_ms * 1e-3) / 1e12
    rank0_ms = float(t[0].sum())
    # measured: every rank's share on this GPU, back to back and in lockstep
    # (every rank's ring step in one launch), whole calls
    flops_all = 4 * w.head_dim * w.heads * all_pairs
    full = {}
    for mode in ("per_step", "lockstep", "fused"):
        plan.set_lockstep(mode == "lockstep")
        plan.set_fused_ring(mode == "fused")
        for _ in range(2):
            plan.full_forward(*bufs, stream=stream)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            plan.full_forward(*bufs, stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        full[mode] = ev[0].elapsed_time(ev[1]) / reps
    plan.set_lockstep(False)
    plan.set_fused_ring(True)
    # each rank's fused call alone: a ring whose ranks each run one fused
    # launch moves at the slowest rank's call
    rank_ms = []
    for r in range(w.cp):
        for _ in range(2):
            plan.rank_forward(*bufs, r, stream=stream)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        n = max(reps, 10)
        ev[0].record(stream)
        for _ in range(n):
            plan.rank_forward(*bufs, r, stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        rank_ms.append(ev[0].elapsed_time(ev[1]) / n)
    measured = {"fused_ring_rank_ms": [round(x, 5) for x in rank_ms],
                "fused_ring_max_over_rank0": round(max(rank_ms) / rank_ms[0], 4),
                "fused_ring_max_over_mean": round(max(rank_ms) / (sum(rank_ms) / len(rank_ms)), 4),
                "fused_ring_slowest_rank_tflops_per_gpu": round(flops_all / w.cp / (max(rank_ms) * 1e-3) / 1e12, 2),
                "all_ranks_fused_ring_ms": round(full["fused"], 5),
                "fused_ring_tflops_per_gpu": round(flops_all / (full["fused"] * 1e-3) / 1e12, 2),
                "all_ranks_back_to_back_ms": round(full["per_step"], 5), "all_ranks_lockstep_ms": round(full["lockstep"], 5),
                "lockstep_ms_per_rank": round(full["lockstep"] / w.cp, 5),
                "lockstep_tflops_per_gpu": round(flops_all / (full["lockstep"] * 1e-3) / 1e12, 2),
                "lockstep_frac_bf16_peak": round(flops_all / (full["lockstep"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "note": "one GPU runs every rank; per GPU of a cp-GPU ring, the same rate"}
    return {"workload": w.name, "step_ms": [[round(float(x), 4) for x in row] for row in t],
            "measured_lockstep": measured,
            "lockstep_step_kernel_ms": round(lockstep_ms, 5), "rank0_step_kernel_ms": round(rank0_ms, 5),
            "lockstep_over_rank0": round(lockstep_ms / rank0_ms, 4),
            "lockstep_tflops_per_gpu": round(lockstep_tflops, 2),
            "lockstep_frac_bf16_peak": round(lockstep_tflops / PEAK_BF16_TFLOPS, 4),
            "time_imbalance_per_step": per, "max_step_imbalance": max(per),
            "time_imbalance": round(float(t.max(axis=0).sum() / t.mean(axis=0).sum()), 4),
            "tiles_128x64": tiles}


def sampled_parity(w, q, k, v, out, lse):
    import oracle
    from ring_context_parallelism_amd.inputs import to_numpy_f64
    ranks = range(w.cp) if w.rank is None else [w.rank]
    rng = np.random.default_rng(w.seed)
    rows = np.concatenate([oracle.rank_positions(w.seq_len, w.cp, r, w.layout) for r in ranks])
    rows = np.unique(np.concatenate([rows[:2], rows[-2:], rng.choice(rows, 24, replace=False)]))
    oc, lc = out.cpu(), lse.cpu()
    d_o = d_l = 0.0
    for h in sorted({0, w.heads - 1}):
        o_ref, l_ref = oracle.attention(to_numpy_f64(q[torch.from_numpy(rows), h:h + 1]),
                                        to_numpy_f64(k[:, h:h + 1]), to_numpy_f64(v[:, h:h + 1]),
                                        causal=w.causal, q_pos=rows)
        d_o = max(d_o, float(np.abs(oc[rows, h:h + 1].double().numpy() - o_ref).max()))
        d_l = max(d_l, float(np.abs(lc[h, rows].double().numpy() - l_ref[0]).max()))
    return {"rows": int(rows.size), "heads": 2, "max_abs_dO": d_o, "max_abs_dLSE": d_l}


def backward_section(plan, w, bufs, stream, reps):
    """One rank's backward on the timed workload: time per call, TFLOP/s at the
    usual 2.5x of the forward's valid FLOPs (five products of 2 head_dim flops
    per valid pair), and dQ of sampled rows against the fp64 oracle."""
    import oracle
    from ring_context_parallelism_amd.inputs import make_qkv, to_numpy_f64
    q, k, v, out, lse = bufs
    dout_cpu = make_qkv(w.seq_len, w.heads, w.head_dim, w.dtype, w.seed + 7)[0]
    dout = dout_cpu.cuda()
    run_call(plan, w, bufs, stream)  # out and lse of the share
    shape = (w.seq_len, w.heads, w.head_dim)
    dq = torch.zeros(shape, device="cuda", dtype=torch.float32)
    dk = torch.zeros(shape, device="cuda", dtype=torch.float32)
    dv = torch.zeros(shape, device="cuda", dtype=torch.float32)
    args = (q, k, v, out, lse, dout, dq, dk, dv, w.rank)
    plan.rank_backward(*args, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed():
        e0.record(stream)
        for _ in range(reps):
            plan.rank_backward(*args, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    plan.set_backward_key_kernel("four")  # one wave per 32-key column, for comparison
    plan.rank_backward(*args, stream=stream)
    ms_four = timed()
    plan.set_backward_key_kernel("eight")
    flops = 2.5 * 4 * w.head_dim * w.heads * share_pairs(plan, w)
    fused_ms = {}
    for mode in (0, 2, 1):  # the last one (the default schedule) writes dq last
        plan.set_backward_fused(mode)
        plan.rank_backward(*args, stream=stream)
        fused_ms[mode] = timed()
    ms = fused_ms[1]
    tflops = flops / (ms * 1e-3) / 1e12
    # dQ of sampled rows of the share (written by the last call in full)
    rows = oracle.rank_positions(w.seq_len, w.cp, w.rank, w.layout)
    sample = rows[np.linspace(0, rows.size - 1, 8).astype(np.int64)]
    q_cpu, k_cpu, v_cpu = (t.cpu() for t in (q, k, v))
    ref = oracle.query_gradients(*(to_numpy_f64(t) for t in (q_cpu, k_cpu, v_cpu, dout_cpu)), sample, causal=w.causal)
    got = dq.cpu().double().numpy()[sample]
    rel = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    return {"ms_per_call": round(ms, 5), "tflops": round(tflops, 2),
            "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4), "valid_flops": flops,
            "four_wave_key_kernel_ms_per_call": round(ms_four, 5),
            "schedules": {name: {"ms_per_call": round(fused_ms[m], 5),
                                 "tflops": round(flops / (fused_ms[m] * 1e-3) / 1e12, 2),
                                 "frac_bf16_peak": round(flops / (fused_ms[m] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
                          for name, m in (("per_step", 0), ("fused_dq", 1), ("all_gather_form", 2))},
            "flop_convention": "2.5 x forward valid flops",
            "parity_dq_sampled_rows": {"rows": sample.tolist(), "max_rel_err": rel, "tol": 2e-2, "ok": rel <= 2e-2}}


def documents_section(w, bufs, stream, reps):
    """Document masks on the timed workload's share (seeded document lengths,
    uniform on [1, 2 mean - 1]): time per call, TFLOP/s of the valid pairs
    (same document and causal), and sampled rows against the fp64 oracle."""
    import oracle
    import ring_context_parallelism_amd as R
    from ring_context_parallelism_amd.inputs import make_documents, to_numpy_f64
    q, k, v, out, lse = bufs
    rows = oracle.rank_positions(w.seq_len, w.cp, w.rank, w.layout)
    sample = rows[np.linspace(0, rows.size - 1, 12).astype(np.int64)]
    qn, kn, vn = (to_numpy_f64(t.cpu()) for t in (q, k, v))
    res = {}
    for mean in (8192, 1024):
        docs = make_documents(w.seq_len, mean, seed=w.seed + mean)
        p = R.Plan(w.seq_len, w.cp, w.heads, w.head_dim, w.causal, w.layout, dtype=w.torch_dtype)
        p.set_documents(docs)
        pairs = sum(p.valid_work(w.rank, s, 128, 64)[1] for s in range(w.cp))
        p.rank_forward(q, k, v, out, lse, w.rank, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            p.rank_forward(q, k, v, out, lse, w.rank, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        flops = 4 * w.head_dim * w.heads * pairs
        o_ref, l_ref = oracle.attention(qn[sample], kn, vn, causal=w.causal, q_pos=sample, doc_starts=docs)
        d_o = float(np.max(np.abs(out.cpu()[sample].double().numpy() - o_ref)))
        d_l = float(np.max(np.abs(lse.cpu()[:, sample].double().numpy() - l_ref)))
        res[f"mean_doc_len_{mean}"] = {
            "documents": len(docs), "valid_pairs_per_head": pairs, "ms_per_call": round(ms, 5),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "parity_sampled": {"rows": sample.tolist(), "max_abs_dO": d_o, "max_abs_dLSE": d_l,
                               "ok": d_o <= 2e-2 and d_l <= 1e-3}}
        p.close()
    return res


def ulysses_section(plan, w, bufs, stream, reps):
    """Ulysses variant on the timed workload: the all-to-all of Q, K, V to head
    ownership (every rank at once on one GPU), rank 0's attention over all
    tokens of its head slice, the all-to-all of O back."""
    q, k, v, out, lse = bufs
    cp, heads, dim = w.cp, w.heads, w.head_dim
    if heads % cp:
        return None
    g = heads // cp
    n_seq = cp * plan.local_rows()
    seq_l = [torch.empty((n_seq, heads, dim), device="cuda", dtype=q.dtype) for _ in range(3)]
    for src, dst in zip((q, k, v), seq_l):
        plan.layout_gather(src, dst, stream=stream)
    head_l = [torch.empty((cp, w.seq_len, g, dim), device="cuda", dtype=q.dtype) for _ in range(3)]
    out_h = torch.empty((cp, w.seq_len, g, dim), device="cuda", dtype=q.dtype)
    lse_h = torch.empty((heads, w.seq_len), device="cuda", dtype=torch.float32)
    out_s = torch.empty((n_seq, heads, dim), device="cuda", dtype=q.dtype)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def a2a_in():
        for s_l, h_l in zip(seq_l, head_l):
            plan.ulysses_a2a(s_l, h_l, True, stream=stream)

    ms_in = timed(a2a_in)
    ms_rank0 = timed(lambda: plan.ulysses_forward(head_l[0][0], head_l[1][0], head_l[2][0], out_h[0], lse_h[:g],
                                                  stream=stream))

    def all_ranks():
        for r in range(cp):
            plan.ulysses_forward(head_l[0][r], head_l[1][r], head_l[2][r], out_h[r], lse_h[r * g:(r + 1) * g],
                                 stream=stream)
    ms_all = timed(all_ranks)
    ms_out = timed(lambda: plan.ulysses_a2a(out_h, out_s, False, stream=stream))
    pairs = w.seq_len * (w.seq_len + 1) // 2 if w.causal else w.seq_len * w.seq_len
    rank_flops = 4 * dim * g * pairs
    tensor_bytes = w.seq_len * heads * dim * q.element_size()
    return {"heads_per_rank": g, "a2a_qkv_ms": round(ms_in, 5), "a2a_out_ms": round(ms_out, 5),
            "a2a_gbps": round(2 * tensor_bytes / (ms_out * 1e-3) / 1e9, 1),
            "rank0_attention_ms": round(ms_rank0, 5),
            "rank0_attention_tflops": round(rank_flops / (ms_rank0 * 1e-3) / 1e12, 2),
            "all_ranks_attention_ms": round(ms_all, 5),
            "note": "one GPU: each all-to-all moves every rank's data (a rank's part is 1/cp of it)"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the one-GPU ring schedule has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import ring_context_parallelism_amd as R
    from ring_context_parallelism_amd.inputs import WORKLOADS, sha256_of, workload_qkv

    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    q_cpu, k_cpu, v_cpu = workload_qkv(w)
    q, k, v = (t.cuda() for t in (q_cpu, k_cpu, v_cpu))
    out = torch.empty_like(q)
    lse = torch.empty(w.heads, w.seq_len, device="cuda", dtype=torch.float32)
    bufs = (q, k, v, out, lse)
    plan = R.Plan(w.seq_len, w.cp, w.heads, w.head_dim, w.causal, w.layout, dtype=w.torch_dtype)
    if args.recv is not None:
        plan.set_recv(args.recv)
    if args.recv_blocks is not None:
        plan.set_recv_blocks(args.recv_blocks)
    if args.serialize:
        plan.set_serialize(True)
    if args.graph:
        plan.set_graph(True)
    if args.merge == "separate":
        plan.set_merge(True)
    if args.no_key_split:
        plan.set_key_split(False)
    if args.no_fused_ring:
        plan.set_fused_ring(False)
    if args.fused_ring_staged:
        plan.set_fused_ring("staged")

    if args.copy_probe:
        probe = torch.empty_like(q)
        plan.layout_gather(q, probe)
        torch.cuda.synchronize()
        print(f"[bench] copy probe: layout gather of {q.numel() * q.element_size()} bytes", file=sys.stderr)
        del probe
    pairs = share_pairs(plan, w)
    flops = 4 * w.head_dim * w.heads * pairs
    ms = time_calls(plan, w, bufs, stream, args.steps, args.warmup, args.warmup_seconds)
    call_stats = dict(time_calls.last)
    tflops = flops / (ms * 1e-3) / 1e12
    print(f"[bench] {w.name}: {ms:.4f} ms/step, {tflops:.1f} TFLOP/s", file=sys.stderr, flush=True)

    # dominant kernel: the attention step kernel, timed with HIP events on its own stream
    plan.set_graph(False)
    kind, launches = kernel_launches(plan, w, bufs, stream, min(args.steps, 10))
    plan.set_graph(args.graph)
    avg_ms = float(np.mean(launches))
    flops_per_launch = flops / len(launches)
    achieved = flops_per_launch / (avg_ms * 1e-3) / 1e12
    kname = "attn_step_bf16" if w.dtype == "bf16" else "attn_step_f32"
    roofline = {"kernel": kname + ("_fused_ring" if kind == "fused_ring" else ""), "bound": "mfma",
                "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": recorded_traffic(w.name),
                "avg_launch_ms": round(avg_ms, 5), "launches_per_step": len(launches),
                "valid_flops_per_launch": flops_per_launch}

    result = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic: i.i.d. N(0,1) Q/K/V, seeded, CPU-drawn",
        "config": {"workload": w.name, "seq_len": w.seq_len, "cp_size": w.cp, "layout": w.layout,
                   "causal": w.causal, "rank": w.rank, "heads": w.heads, "head_dim": w.head_dim,
                   "ring_steps": w.cp, "valid_flops": flops, "seed": w.seed,
                   "inputs_sha256": sha256_of(q_cpu, k_cpu, v_cpu)},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
    }
    result["ms_per_call_median"] = round(call_stats["median"], 5)
    result["ms_per_call_min"] = round(call_stats["min"], 5)

    if not args.no_extras:
        # same share, other schedule modes (exposed copy / merge cost)
        plan.set_serialize(True)
        ms_serial = time_calls(plan, w, bufs, stream, max(3, args.steps // 4), 1)
        plan.set_serialize(False)
        plan.set_merge(True)
        ms_sep = time_calls(plan, w, bufs, stream, max(3, args.steps // 4), 1)
        plan.set_merge(False)
        plan.set_recv("kernel")
        ms_blocks = {}
        for nb in (64, 128, 256, 512, 1024):
            plan.set_recv_blocks(nb)
            ms_blocks[nb] = round(time_calls(plan, w, bufs, stream, max(3, args.steps // 4), 1), 5)
        plan.set_recv_blocks(-1 if args.recv_blocks is None else args.recv_blocks)
        recv_ms = {}
        for mode in ("memcpy", "fused", "hybrid", "kernel"):
            plan.set_recv(mode)
            recv_ms[mode] = round(time_calls(plan, w, bufs, stream, max(3, args.steps // 4), 1), 5)
        plan.set_recv(args.recv or "kernel")
        plan.set_graph(not args.graph)
        ms_graph_other = round(time_calls(plan, w, bufs, stream, max(3, args.steps // 4), 1), 5)
        plan.set_graph(args.graph)
        ms_allgather = None
        if w.rank is not None:
            # the same share in one launch against the whole K/V (no ring steps, no merge)
            ag_calls = max(3, args.steps // 4)
            plan.allgather_forward(*bufs, w.rank, stream=stream)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(ag_calls):
                plan.allgather_forward(*bufs, w.rank, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ms_allgather = round(e0.elapsed_time(e1) / ag_calls, 5)
        plan.set_fused_ring(False)
        ms_per_step_launches = round(time_calls(plan, w, bufs, stream, max(3, args.steps // 4), 1), 5)
        plan.set_fused_ring("staged" if args.fused_ring_staged else not args.no_fused_ring)
        result["modes_ms"] = {"default_receive": args.recv or "kernel",
                              "dominant_launch": kind,
                              "one_launch_per_step": ms_per_step_launches,
                              "graph_mode": bool(args.graph),
                              ("eager_calls" if args.graph else "graph_replay"): ms_graph_other,
                              "allgather_single_launch": ms_allgather,
                              "overlapped_fused_merge": round(ms, 5), "serialized_fused_merge": round(ms_serial, 5),
                              "overlapped_separate_merge": round(ms_sep, 5),
                              "receive_kernel_grid_blocks_ms": ms_blocks,
                              "receive_mode_ms": recv_ms,
                              # serial order also gives each receive the full copy grid (it overlaps
                              # no step kernel there), so this difference is not the copy time that
                              # the overlap hides; it is what the overlapped schedule saves
                              "serial_minus_overlapped_ms": round(ms_serial - ms, 5)}
        run_call(plan, w, bufs, stream)
        torch.cuda.synchronize()
        result["parity_sampled"] = sampled_parity(w, q_cpu, k_cpu, v_cpu, out, lse)
        result["imbalance"] = imbalance_section(stream)
        if w.rank is not None:
            plan.set_graph(False)
            result["imbalance"]["all_ranks_timed_workload"] = rank_step_imbalance(plan, w, bufs, stream)
            plan.set_graph(args.graph)
        result["imbalance"]["zigzag_step_time_imbalance"] = result["imbalance"]["zigzag"]["time_imbalance"]

    if not args.no_extras:
        result["other_workloads"] = [
            workload_section("causal_s8192_cp4_zigzag_h32_d128_bf16", stream, max(5, args.steps // 2), graph_too=True),
            workload_section("bidir_s65536_cp16_contiguous_h8_d128_bf16_rank0", stream, max(5, args.steps // 2)),
        ]
        print("[bench] other workloads: " + "; ".join(f"{o['workload']}: {o['ms_per_call']} ms, {o['tflops']} TFLOP/s"
                                                    for o in result["other_workloads"]), file=sys.stderr, flush=True)
        result["ulysses"] = ulysses_section(plan, w, bufs, stream, max(3, args.steps // 4))
        if w.rank is not None and w.causal:
            result["documents"] = documents_section(w, bufs, stream, max(3, args.steps // 4))

    if (args.backward or not args.no_extras) and w.rank is not None:
        plan.set_graph(False)
        result["backward"] = backward_section(plan, w, bufs, stream, max(3, args.steps // 4))
        plan.set_graph(args.graph)
        print(f"[bench] backward: {result['backward']['ms_per_call']} ms/call, "
              f"{result['backward']['tflops']} TFLOP/s", file=sys.stderr, flush=True)

    if not args.no_cpu_baseline:
        run_call(plan, w, bufs, stream)
        torch.cuda.synchronize()
        result["cpu_baseline"] = cpu_baseline(w, q_cpu, k_cpu, v_cpu, out, lse, args.cpu_seconds)
        result["parity_oracle_share"] = result["cpu_baseline"].pop("parity")

    props = torch.cuda.get_device_properties(0)
    result["env"] = {"gpu": props.name, "arch": getattr(props, "gcnArchName", ""), "cus": props.multi_processor_count,
                     "torch": torch.__version__, "hip": torch.version.hip, "host": platform.node(),
                     "host_cpus": os.cpu_count()}
    plan.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
