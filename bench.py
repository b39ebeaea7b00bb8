"""Benchmark of the DSpark draft / confidence / schedule / verify path on one GPU.

One step = one decode round over a batch of synthetic inputs already resident in
HBM: dsp_draft_step (all gamma positions), dsp_confidence, dsp_schedule, dsp_verify, as
Round.run issues them: with the streaming draft, dsp_confidence and dsp_schedule on a
second stream while the last position is drafted (they read no token of it), the rest in
order on one stream.  A workload without scheduling (every position verified)
has no consumer for the confidence head: its round is dsp_draft_step + dsp_verify with
l_r = gamma set once, and dsp_confidence and dsp_schedule are timed in a loop of their
own for the per-entry-point breakdown.  The throughput (`value`) times K rounds replayed
from HIP graphs, one graph captured per round (its own round index and input
set), so kernel launch gaps are not counted; a second, eager pass over the same
K rounds times every entry point with HIP events on the launch stream and gives
the roofline of the dominant one.  Prints one JSON line, with the CPU oracle
timed on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4] [--mode greedy]

Besides the headline workload it times the other workloads (per_workload) and the
entry points outside the round (extended).
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from draft_sampling_lossless_markov_amd import dsp  # noqa: E402
from draft_sampling_lossless_markov_amd.engine import Round  # noqa: E402
from draft_sampling_lossless_markov_amd.workloads import (BENCH_LAYOUT, WORKLOADS,  # noqa: E402
                                                          make_inputs)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
# sources of the draft-step kernels; the profiled HBM traffic is reported only
# while they are byte-for-byte the profiled ones
DRAFT_SOURCES = ("draft_sampling_lossless_markov_amd/build.py",
                 "draft_sampling_lossless_markov_amd/csrc/draft.hip",
                 "draft_sampling_lossless_markov_amd/csrc/draft_run.h",
                 "draft_sampling_lossless_markov_amd/csrc/draft_pass.h",
                 "draft_sampling_lossless_markov_amd/csrc/draft_pass_wide.h",
                 "draft_sampling_lossless_markov_amd/csrc/tile_pass.h",
                 "draft_sampling_lossless_markov_amd/csrc/bias_tile.h",
                 "draft_sampling_lossless_markov_amd/csrc/dsp_device.h",
                 "draft_sampling_lossless_markov_amd/csrc/dsp_launch.h")
METRIC = "verified draft positions/sec (draft+verify) and % of MI355X HBM roofline"
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, vendor figure
HEADLINE_WORKLOAD = 4            # the largest single-GPU configuration
PER_WORKLOAD = ((1, "sampling"), (2, "sampling"), (3, "sampling"), (4, "greedy"))
UNIT = "verified draft positions/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def round_bytes(wl, inp, len_sum, n_rej, greedy):
    """Algorithmic HBM bytes of one round: logit rows streamed once (draft base
    rows, verified and bonus target rows, the p and base rows re-read for each
    residual draw), W2 once, hidden states (read by the confidence head, only
    where a scheduler consumes it) and embedding rows once."""
    s = inp["base"].element_size()
    R, g, V, r, d = inp["R"], inp["gamma"], inp["V"], inp["r"], inp["d"]
    rows = R * g + (R + len_sum) + (0 if greedy else 2 * n_rej)
    hid = d if wl.mode != 0 else 0
    return s * V * rows + 2 * r * V + 2 * R * g * (hid + r)


def draft_call_bytes(inp):
    """Compulsory bytes of one dsp_draft_step call over all gamma positions: the
    gamma [R, V] base slices, all of W2 once (every vocabulary column needs its
    bias), the gathered E rows and the per-request outputs."""
    s = inp["base"].element_size()
    R, g, V, r = inp["R"], inp["gamma"], inp["V"], inp["r"]
    return g * s * R * V + 2 * r * V + g * (2 * R * r + R * 16)


def probe_draft_path(call):
    """'persistent' when the persistent draft launch serves this workload (what
    DSP_PATH_AUTO then runs), else 'streaming'."""
    try:
        call(dsp.DSP_PATH_PERSISTENT)
        path = "persistent"
    except dsp.DspError:
        path = "streaming"
    torch.cuda.synchronize()
    return path


def draft_sources_digest():
    import hashlib
    h = hashlib.sha256()
    for rel in DRAFT_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_file(workload):
    short = workload.split("-r256")[0]
    return os.path.join(ROOT, "profiles", f"draft_call_traffic_{short}.txt")


def profiled_traffic(workload, path):
    """HBM bytes of one dsp_draft_step call (FETCH_SIZE and WRITE_SIZE of its
    kernels, scaled by a plain copy) from the committed profile, or None when that
    profile is of other kernel sources, another workload or another draft path."""
    try:
        kv = dict(line.split(None, 1) for line in open(traffic_file(workload)).read().splitlines()
                  if line and not line.startswith("#"))
    except OSError:
        return None
    if (kv.get("workload", "").strip() != workload
            or kv.get("draft_path", "").strip() != path
            or kv.get("sources_sha256", "").strip() != draft_sources_digest()):
        return None
    return int(kv["draft_call_bytes"])


def steps_of(wl):
    """The entry points of one round of workload wl."""
    return "draft + confidence + verify" if wl.mode != 0 else "draft + verify"


def cpu_baseline(wl, inp, temp, budget_s):
    """The oracle as it stands, one thread, on whole requests of set 0 until about
    budget_s seconds of CPU work; every position of a sampled request verified."""
    import oracle
    E = oracle.bf16_bits(inp["E"])
    W2 = oracle.bf16_bits(inp["W2"])
    anchor = inp["anchor"].cpu().numpy()
    w, T = inp["w"].cpu().numpy(), inp["T"].cpu().numpy()
    off = None if inp["offset"] is None else inp["offset"].cpu().numpy()
    g = inp["gamma"]
    done, positions, spent = 0, 0, 0.0
    while spent < budget_s and done < inp["R"]:
        n = done
        sl = slice(n, n + 1)
        base = oracle.host_logits(inp["base"][sl])
        target = oracle.host_logits(inp["target"][sl])
        h = oracle.bf16_bits(inp["h"][sl])
        t0 = time.perf_counter()
        tok, q, _, _ = oracle.draft(base, E, W2, anchor[sl], np.array([n], np.int32), temp, 0, 0)
        if wl.mode != 0:
            oracle.confidence(h, E, anchor[sl], tok, w, T, None if off is None else off[sl])
        oracle.verify(target, base, E, W2, anchor[sl], tok, q, np.array([g], np.int32),
                      np.array([n], np.int32), temp, 0, 0)
        spent += time.perf_counter() - t0
        done += 1
        positions += g
    return {"value": positions / spent, "unit": UNIT, "cores": 1, "kind": "oracle",
            "sample": f"{done} of {inp['R']} requests of one round of {wl.name} "
                      f"({steps_of(wl)} of all {g} positions each), "
                      f"{spent:.1f} s on one host thread"}


def cpu_baseline_threads(wl, inp, temp, budget_s):
    """The same oracle calls, requests sharded over the host threads this process may
    use, at most 16 (the oracle is plain C called through ctypes, which releases the GIL),
    on whole requests of set 0: host copies prepared first, wall time measured."""
    import concurrent.futures as cf
    import oracle
    E = oracle.bf16_bits(inp["E"])
    W2 = oracle.bf16_bits(inp["W2"])
    anchor = inp["anchor"].cpu().numpy()
    w, T = inp["w"].cpu().numpy(), inp["T"].cpu().numpy()
    off = None if inp["offset"] is None else inp["offset"].cpu().numpy()
    g, R = inp["gamma"], inp["R"]
    # the host threads this process may use, at most 16 (a GPU's share of its host)
    threads = min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count())
    n_req = min(R, max(threads, 1) * 4)
    rows = [(oracle.host_logits(inp["base"][n:n + 1]), oracle.host_logits(inp["target"][n:n + 1]),
             oracle.bf16_bits(inp["h"][n:n + 1])) for n in range(n_req)]

    def one(n):
        base, target, h = rows[n]
        sl = slice(n, n + 1)
        tok, q, _, _ = oracle.draft(base, E, W2, anchor[sl], np.array([n], np.int32), temp, 0, 0)
        if wl.mode != 0:
            oracle.confidence(h, E, anchor[sl], tok, w, T, None if off is None else off[sl])
        oracle.verify(target, base, E, W2, anchor[sl], tok, q, np.array([g], np.int32),
                      np.array([n], np.int32), temp, 0, 0)
        return g

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        positions = sum(ex.map(one, range(n_req)))
    wall = time.perf_counter() - t0
    return {"value": positions / wall, "unit": UNIT, "cores": threads, "kind": "oracle",
            "sample": f"{n_req} of {R} requests of one round of {wl.name} ({steps_of(wl)} "
                      f"of all {g} positions each) sharded over {threads} host threads, "
                      f"{wall:.1f} s wall"}


def host_cpu():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_bandwidth(nbytes=1 << 30, reps=5):
    """Achieved bandwidth of a plain device-to-device copy (bytes read + written per
    second): the second denominator of the roofline."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def measure(wl, mode, args, steps, warmup, with_cpu, log_prefix=""):
    """Time one workload: K graph-replayed rounds (value), an eager pass with per-entry-
    point events, the draft call's roofline and the bias GEMM's MFMA rate."""
    greedy = mode == "greedy"
    temp = 0.0 if greedy else wl.temperature
    log(f"{log_prefix}workload {wl.name}, {mode}, building {args.sets} input sets")
    sets = [make_inputs(wl, s, device="cuda", layout=BENCH_LAYOUT) for s in range(args.sets)]
    inp0 = sets[0]
    R, g, V, r = inp0["R"], inp0["gamma"], inp0["V"], inp0["r"]
    rd = Round(R, g, V, r)
    stream = torch.cuda.current_stream()
    seed = 0

    def draft(i, s=stream, flags=dsp.DSP_PATH_AUTO):
        inp = sets[i % len(sets)]
        dsp.dsp_draft_step(inp["base"], inp["E"], inp["W2"], inp["anchor"], rd.tok, rd.q,
                           rd.stats, 0, temp, seed, i, rd.ws_draft, s, n_steps=g, flags=flags)

    # with the scheduler off every position is verified: l_r = gamma, set once
    scheduled = wl.mode != 0
    if not scheduled:
        rd.schedule(inp0)
        torch.cuda.synchronize()

    def one_round(i, ev=None, s=stream):
        inp = sets[i % len(sets)]
        if ev is not None:
            ev[0].record(s)
        draft(i, s)
        if ev is not None:
            ev[1].record(s)
        if scheduled:
            rd.confidence(inp, s)
        if ev is not None:
            ev[2].record(s)
        if scheduled:
            rd.schedule(inp, stream=s)
        if ev is not None:
            ev[3].record(s)
        rd.verify(inp, temp, seed, i, s)
        if ev is not None:
            ev[4].record(s)

    draft_path = probe_draft_path(lambda f: draft(0, flags=f))
    log(f"{log_prefix}draft path: {draft_path}")

    for i in range(warmup):
        one_round(i)
    torch.cuda.synchronize()
    K = steps

    # eager pass: per entry point event timing (roofline, breakdown)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e_start.record(stream)
    for i in range(K):
        one_round(warmup + i, evs[i])
    e_end.record(stream)
    torch.cuda.synchronize()
    eager_ms_per_step = e_start.elapsed_time(e_end) / K
    rd.check()

    # throughput pass: the same K rounds replayed from one captured graph each
    if args.eager:
        ms_per_step = eager_ms_per_step
        timing = "eager launches"
        round_ms = np.array([evs[i][0].elapsed_time(evs[i][4]) for i in range(K)])
    else:
        # the round as Round.run issues it: with the scheduler on and the streaming
        # draft, the confidence head and the scheduler on a second stream while the
        # last position is drafted (outputs identical to the calls in order; the
        # persistent draft runs all positions in one launch, and splitting it
        # costs more than the overlap saves)
        overlap = scheduled and draft_path == "streaming"
        cap = torch.cuda.Stream()
        graphs = []
        for i in range(K):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=cap):
                if overlap:
                    rd.run(sets[(warmup + i) % len(sets)], temp, seed, warmup + i, stream=cap,
                           overlap=True)
                else:
                    one_round(warmup + i, s=cap)
            graphs.append(gr)
        for gr in graphs[:2]:
            gr.replay()
        torch.cuda.synchronize()
        t_ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        t_ev[0].record(stream)
        for i, gr in enumerate(graphs):
            gr.replay()
            t_ev[i + 1].record(stream)
        torch.cuda.synchronize()
        ms_per_step = t_ev[0].elapsed_time(t_ev[K]) / K
        round_ms = np.array([t_ev[i].elapsed_time(t_ev[i + 1]) for i in range(K)])
        timing = ("HIP graph replay, one graph per round" +
                  ("; confidence and scheduler on a second stream during the last draft position"
                   if overlap else ""))
        rd.check()
        del graphs

    # per entry point (event-bracketed) average durations, in ms
    draft_ms = np.array([evs[i][0].elapsed_time(evs[i][1]) for i in range(K)])
    conf_ms = np.array([evs[i][1].elapsed_time(evs[i][2]) for i in range(K)])
    sched_ms = np.array([evs[i][2].elapsed_time(evs[i][3]) for i in range(K)])
    ver_ms = np.array([evs[i][3].elapsed_time(evs[i][4]) for i in range(K)])
    if not scheduled:
        # not in the round: timed in a loop of their own (the schedule in the
        # workload's mode, which sets l_r = gamma again)
        ce = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
        for i in range(K):
            inp = sets[(warmup + i) % len(sets)]
            ce[i][0].record(stream)
            rd.confidence(inp, stream)
            ce[i][1].record(stream)
            rd.schedule(inp, stream=stream)
            ce[i][2].record(stream)
        torch.cuda.synchronize()
        conf_ms = np.array([ce[i][0].elapsed_time(ce[i][1]) for i in range(K)])
        sched_ms = np.array([ce[i][1].elapsed_time(ce[i][2]) for i in range(K)])

    # replay the timed rounds (deterministic) to count verified positions
    len_sum = rej = 0
    for i in range(K):
        one_round(warmup + i)
        L = rd.len.cpu().numpy()
        na = rd.n_accept.cpu().numpy()
        len_sum += int(L.sum())
        rej += int((na < L).sum())
    rd.check()
    len_per_round = len_sum / K
    rej_per_round = rej / K
    value = len_per_round / (ms_per_step * 1e-3)
    A = round_bytes(wl, inp0, len_per_round, rej_per_round, greedy)

    call_bytes = draft_call_bytes(inp0)
    if args.eager:
        draft_avg_s = float(draft_ms.mean()) * 1e-3
        draft_timing = "eager launches, events around each call"
    else:
        # K draft calls captured back to back in one graph, replayed with events
        # on the launch stream: the calls' kernels back to back (what the kernel
        # trace's durations add up to)
        cap = torch.cuda.Stream()
        gd = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gd, stream=cap):
            for i in range(K):
                draft(warmup + i, s=cap)
        gd.replay()
        torch.cuda.synchronize()
        d0 = torch.cuda.Event(enable_timing=True)
        d1 = torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        gd.replay()
        d1.record(stream)
        torch.cuda.synchronize()
        rd.check()
        draft_avg_s = d0.elapsed_time(d1) / K * 1e-3
        draft_timing = "one graph of K draft calls back to back"
        del gd
    achieved = call_bytes / draft_avg_s / 1e9
    traffic = profiled_traffic(wl.name, draft_path)
    kernels = ("run_clear_kernel + draft_run_kernel (one persistent launch, all gamma positions)"
               if draft_path == "persistent" else
               "draft_pass_wide_kernel + draft_pick_kernel per position")
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": f"dsp_draft_step, {g} positions: {kernels}",
            "bytes_per_launch": int(call_bytes), "avg_launch_us": round(draft_avg_s * 1e6, 2),
            "timing": draft_timing}
    # the Markov-bias contraction [R x r] . [r x V] per draft position, bf16 MFMA
    bias_flop = 2.0 * R * r * V * g
    mfma = {"flop_per_call": bias_flop,
            "achieved_tflops": round(bias_flop / draft_avg_s / 1e12, 1),
            "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "utilisation": round(bias_flop / draft_avg_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "what": "2 R r V flop per draft position over the whole draft call's time"}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": UNIT, "n_gpus": 1, "steps": K,
        "warmup": warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if inp0["base"].dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "R": R, "gamma": g, "V": V, "r": r, "d": inp0["d"],
                   "mode": mode, "scheduler": "on" if wl.mode == 1 else "off (every position verified)",
                   "round": ("dsp_draft_step + dsp_confidence + dsp_schedule + dsp_verify" if scheduled
                             else "dsp_draft_step + dsp_verify (no scheduler: the confidence head has "
                                  "no consumer; l_r = gamma)"),
                   "base_layout": BENCH_LAYOUT + "-major [gamma, R, V]",
                   "draft_path": draft_path,
                   "parallelism": "single GPU"},
        "round_roofline": {"algorithmic_bytes": int(A), "t_roof_us": round(A / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
                           "frac": round(A / (HBM_PEAK_GBS * 1e9) / (ms_per_step * 1e-3), 4)},
        "entry_points_us": {"in_round": (["draft_step_all_positions", "confidence", "schedule", "verify"]
                                         if scheduled else ["draft_step_all_positions", "verify"]),
                            "draft_step_all_positions": round(float(draft_ms.mean()) * 1e3, 2),
                            "confidence": round(float(conf_ms.mean()) * 1e3, 2),
                            "schedule": round(float(sched_ms.mean()) * 1e3, 2),
                            "verify": round(float(ver_ms.mean()) * 1e3, 2)},
        "verified_per_round": len_per_round, "drafted_per_round": R * g,
        "rejections_per_round": rej_per_round,
        "timing": timing, "eager_ms_per_step": round(eager_ms_per_step, 5),
        "roofline": roof,
        "bias_gemm_mfma": mfma,
        "round_us_percentiles": {"p10": round(float(np.percentile(round_ms, 10)) * 1e3, 2),
                                 "median": round(float(np.median(round_ms)) * 1e3, 2),
                                 "p90": round(float(np.percentile(round_ms, 90)) * 1e3, 2)},
    }
    if with_cpu:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(wl, inp0, temp, args.cpu_seconds)
        result["cpu_baseline_threads"] = cpu_baseline_threads(wl, inp0, temp, args.cpu_seconds)
        result["cpu_host"] = {"model": host_cpu(), "threads": len(os.sched_getaffinity(0))}
    del sets, inp0, rd
    torch.cuda.empty_cache()
    return result


def _time_calls(fn, reps, stream):
    """Average ms of fn() over reps calls back to back, events on the launch stream."""
    fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def measure_extended(reps=5):
    """The entry points outside the round, at the large-batch workload's sizes (R 2048,
    gamma 8, V 262144, r 256, bf16, sampling): the capacity-barrier scheduler, the
    exact acceptance probability of every draft position, the recurrent head's draft
    step, and sequential temperature scaling with its calibration error on a held-out
    set of 65536 samples of 8 positions."""
    from draft_sampling_lossless_markov_amd.workloads import calibration_set, rnn_matrix
    wl = WORKLOADS[4]
    inp = make_inputs(wl, 0, device="cuda", layout=BENCH_LAYOUT)
    R, g, V, r = inp["R"], inp["gamma"], inp["V"], inp["r"]
    rd = Round(R, g, V, r)
    stream = torch.cuda.current_stream()
    temp, seed = wl.temperature, 0
    out = {"workload": wl.name, "mode": "sampling"}
    rd.draft(inp, temp, seed, 0)
    rd.confidence(inp)
    c_hist = rd.c.roll(1, dims=0).contiguous()   # another round's confidences
    torch.cuda.synchronize()

    # prefix schedulers (latency-bound: one workgroup sorts R gamma candidates)
    t_sync = _time_calls(lambda: rd.schedule(inp), 20, stream)
    t_async = _time_calls(lambda: rd.schedule_async(inp, c_hist), 20, stream)
    out["schedule_us"] = round(t_sync * 1e3, 2)
    out["schedule_async_us"] = round(t_async * 1e3, 2)

    # exact acceptance probability: target rows 0..gamma-1 and the draft rows
    # streamed once, W2 once, the per-entry outputs
    alpha = torch.zeros(R, g, dtype=torch.float64, device="cuda")
    ws_tv = torch.zeros(dsp.dsp_workspace_size(dsp.DSP_WS_TV, R, g, V, r), dtype=torch.uint8,
                        device="cuda")
    t_tv = _time_calls(lambda: dsp.dsp_tv_accept(inp["target"], inp["base"], inp["E"], inp["W2"],
                                                 inp["anchor"], rd.tok, rd.stats, alpha, temp,
                                                 ws_tv), reps, stream)
    tv_bytes = 2 * (2 * R * g * V) + 2 * r * V + 8 * R * g
    out["tv_accept"] = {"us": round(t_tv * 1e3, 1), "algorithmic_bytes": tv_bytes,
                        "achieved_GBs": round(tv_bytes / (t_tv * 1e-3) / 1e9, 1),
                        "frac_of_hbm_peak": round(tv_bytes / (t_tv * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del ws_tv, alpha

    # recurrent head: the Markov draft call against the recurrent one
    A = rnn_matrix(r, 0).cuda()
    S = torch.zeros(R, g, r, dtype=torch.bfloat16, device="cuda")
    t_markov = _time_calls(lambda: dsp.dsp_draft_step(inp["base"], inp["E"], inp["W2"], inp["anchor"],
                                                      rd.tok, rd.q, rd.stats, 0, temp, seed, 0,
                                                      rd.ws_draft, n_steps=g,
                                                      flags=dsp.DSP_PATH_STREAMING), reps, stream)
    t_rnn = _time_calls(lambda: dsp.dsp_draft_step_rnn(inp["base"], inp["E"], inp["W2"], A,
                                                       inp["anchor"], rd.tok, rd.q, rd.stats, S, 0,
                                                       temp, seed, 0, rd.ws_draft, n_steps=g),
                        reps, stream)
    rnn_bytes = draft_call_bytes(inp) + 2 * r * r + 2 * (2 * R * g * r)
    out["rnn_draft"] = {"us": round(t_rnn * 1e3, 1), "markov_streaming_us": round(t_markov * 1e3, 1),
                        "overhead": round(t_rnn / t_markov - 1.0, 4),
                        "achieved_GBs": round(rnn_bytes / (t_rnn * 1e-3) / 1e9, 1),
                        "frac_of_hbm_peak": round(rnn_bytes / (t_rnn * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del S, A, rd, inp
    torch.cuda.empty_cache()

    # sequential temperature scaling: 2 grid stages x 256 candidates x N samples
    # per position, each a cumulative-survival cross-entropy in fp64
    N, gc = 65536, 8
    z, acc = calibration_set(N, gc, 0, device="cuda")
    T = torch.zeros(gc, dtype=torch.float32, device="cuda")
    ws = torch.zeros(dsp.dsp_workspace_size(dsp.DSP_WS_STS, N, gc, 1, 1), dtype=torch.uint8,
                     device="cuda")
    t_fit = _time_calls(lambda: dsp.dsp_sts_fit(z, acc, 1.0 / 16, 16.0, T, None, ws), 3, stream)
    ece = torch.zeros(1, dtype=torch.float64, device="cuda")
    ws_e = torch.zeros(dsp.dsp_workspace_size(dsp.DSP_WS_ECE, 0, 0, 0, 0), dtype=torch.uint8,
                       device="cuda")
    t_ece = _time_calls(lambda: dsp.dsp_ece(z, acc, T, 15, ece, ws_e), 10, stream)
    ece_after = float(ece.item())
    dsp.dsp_ece(z, acc, None, 15, ece, ws_e)
    evals = N * gc * 2 * 256
    out["sts_fit"] = {"N": N, "gamma": gc, "ms": round(t_fit, 3),
                      "loss_evaluations_per_s": round(evals / (t_fit * 1e-3), 1),
                      "ece_us": round(t_ece * 1e3, 2),
                      "ece_before": round(float(ece.item()), 5), "ece_after": round(ece_after, 5),
                      "T": [round(float(x), 4) for x in T.cpu()]}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=HEADLINE_WORKLOAD)
    ap.add_argument("--mode", choices=["sampling", "greedy"], default=None)
    ap.add_argument("--sets", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-workload", action="store_true",
                    help="time only the headline workload")
    ap.add_argument("--no-extended", action="store_true",
                    help="skip the entry points outside the round (async scheduler, exact "
                         "acceptance, recurrent head, temperature scaling)")
    ap.add_argument("--eager", action="store_true",
                    help="time the rounds as eager launches instead of graph replays")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy five times (the known-size "
                         "reference for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "copies": 5}), flush=True)
        return

    if args.gpus != 1:
        print(f"bench.py measures the one-GPU path only; --gpus {args.gpus} is not supported "
              "(the path shards by request; see the multi-GPU design notes)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    dsp.lib()
    wl = WORKLOADS[args.workload]
    mode = args.mode or wl.modes[-1]
    result = measure(wl, mode, args, args.steps, args.warmup, not args.no_cpu_baseline)
    if not args.no_per_workload and args.workload == HEADLINE_WORKLOAD and args.mode is None:
        per = {}
        for wid, m in PER_WORKLOAD:
            w2 = WORKLOADS[wid]
            r2 = measure(w2, m, args, max(10, args.steps // 2), max(3, args.warmup // 2), False,
                         log_prefix="  ")
            per[f"{w2.name}/{m}"] = {k: r2[k] for k in (
                "value", "unit", "ms_per_step", "round_roofline", "roofline", "bias_gemm_mfma",
                "entry_points_us", "verified_per_round", "round_us_percentiles")}
            per[f"{w2.name}/{m}"]["draft_path"] = r2["config"]["draft_path"]
        result["per_workload"] = per
    if not args.no_extended and args.workload == HEADLINE_WORKLOAD and args.mode is None:
        log("entry points outside the round")
        result["extended"] = measure_extended()
    copy_gbs = copy_bandwidth()
    A = result["round_roofline"]["algorithmic_bytes"]
    result["copy_bandwidth"] = {"GBs": round(copy_gbs, 1),
                                "round_frac_of_copy": round(A / (copy_gbs * 1e9) / (result["ms_per_step"] * 1e-3), 4),
                                "what": "1 GiB device-to-device copy, bytes read + written per second"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
