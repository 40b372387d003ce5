"""Throughput of the partial-attention + LSE-merge hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads a,b,...] [--no-cpu-baseline]

A step is one CP rank's whole share of one batch: every partial attention the
rank computes, then the merge of all partials (other ranks' partials already
resident in HBM where the schedule has them; in decode the merge is folded
into the rank's own decode launches). Inputs are seeded synthetic tensors
resident in HBM before timing starts.

Headline (`value`): the largest workload, the Llama-3-8B-shaped 128K-token
cp=4 rank-1 pass-KV share (1 sequence of 131072 tokens, zigzag into 8 chunks,
32/8 heads, d=128, bf16; 4 partial attentions + 4-way merge): algorithmic
TFLOP/s = 4 * d * hq * (visible causal pairs) / step time. The other
full-size workloads are reported under "workloads" (TFLOP/s for prefill,
GB/s for decode and for every merge).

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "partial-attn+merge TFLOP/s and % bf16 MFMA peak (prefill); GB/s (decode)"
HEADLINE = "llama3_8b_128k_cp4_rank1"
DEFAULT_WORKLOADS = [HEADLINE, "qwen2.5_3b_cp2_rank0", "chunked_prefill_passq_cp4", "allgather_decode_cp2"]
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
XGMI_LINK_BYTES_PER_S = 153e9  # one MI355X xGMI link
# dominant kernel of the headline step and the committed counter summary of it
ATTN_KERNEL_SOURCES = ("attn_pp.hip", "attn_pp_common.h", "device_common.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_llama3_8b_128k_traffic.md")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_llama3_8b_128k_counters.md")


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ work counts (host integers)


def pass_kv_pairs(inp, step: int) -> int:
    """Visible (query, key) pairs of one pass-KV step: per query, the keys of
    its sequence's shard with position <= its own."""
    qp, cu = inp["q_positions_host"], inp["cu_q_host"]
    st = inp["steps"][step]
    kp, cuk = st["k_positions_host"], st["cu_k_host"]
    total = 0
    for b in range(len(cu) - 1):
        total += int(np.searchsorted(kp[cuk[b]:cuk[b + 1]], qp[cu[b]:cu[b + 1]], side="right").sum())
    return total


def paged_pairs(inp, rank: int) -> int:
    qp, cu = inp["q_positions_host"], inp["cu_q_host"]
    rk = inp["ranks"][rank]
    l2g, cul = rk["local_to_global_host"], rk["cu_local_host"]
    total = 0
    for b in range(len(cu) - 1):
        total += int(np.searchsorted(l2g[cul[b]:cul[b + 1]], qp[cu[b]:cu[b + 1]], side="right").sum())
    return total


def merge_bytes(w, rows: int, n_parts: int, out_bytes: int) -> int:
    return n_parts * rows * (w.d * 4 + 4) + rows * (w.d * out_bytes + 4)


# ------------------------------------------------------------------ GPU timing


def bench_workload(name: str, steps: int, warmup: int, next_rows: bool = True) -> dict:
    import torch

    import context_partial_attention_amd as cpa
    from context_partial_attention_amd import harness
    from context_partial_attention_amd.workloads import WORKLOADS

    w = WORKLOADS[name]
    t_build = time.perf_counter()
    inp = harness.build(w, device="cuda", keep_full=False)
    run = harness.Runner(inp)
    torch.cuda.synchronize()
    log(f"[bench] {name}: inputs built in {time.perf_counter() - t_build:.1f} s")
    stream = torch.cuda.current_stream()
    if w.kind == "pass_kv":
        # every pass-KV step is this rank's work; all shards are resident, so
        # the steps run as one batched launch (heaviest tiles first)
        own = list(range(w.cp))
        launches = [run.partials_batched]
    else:
        own = [w.rank]  # this rank's paged shard; the other ranks' partials are resident
        for r in range(w.cp):
            if r != w.rank:
                run.partial(r)
        # the received partials are merged inside the rank's own launches
        # (decode: split kernel + merge kernel; pass-Q: the prefill kernel's
        # epilogue), no merge launch; the rank's own partial is written once,
        # for the separate merge timed below for comparison
        run.partial(w.rank)
        if run.fold_supported():
            launches = [lambda: run.rank_fold(own=False)]
        else:
            launches = [lambda: run.partial(w.rank)]
    merge_in_step = w.kind == "pass_kv" or not run.fold_supported()

    def step():
        for f in launches:
            f()
        if merge_in_step:
            run.merge()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the step runs as a captured HIP graph (its kernels are plain launches on
    # the stream: no memsets, no allocations), which removes the host launch
    # overhead between its kernels. The timed loop replays a graph holding
    # `per_graph` consecutive steps (the largest divisor of `steps` up to 64),
    # as a model's forward pass holds its attention layers in one graph: each
    # graph launch opens a dispatch gap of ~8-20 us on the stream.
    per_graph = max(d for d in range(1, 65) if steps % d == 0)
    graph1 = run.capture(step)
    graph = graph1 if per_graph == 1 else run.capture(lambda: [step() for _ in range(per_graph)])
    for _ in range(max(1, warmup // per_graph)):
        graph.replay()
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    # (1) the step: events only at the two ends of the timed region (an event
    # recorded between two kernels opens a dispatch gap of ~10 us on the stream)
    g0, g1 = ev(), ev()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record(stream)
    for _ in range(steps // per_graph):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    gpu_ms = g0.elapsed_time(g1)
    # (2) each launch of the step on its own: `steps` back-to-back launches
    # between one pair of events on the launch stream, mean per launch
    def per_launch_ms(f):
        a, b = ev(), ev()
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(steps):
            f()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    # per-step spread: the one-step graph replayed between its own pair of
    # events each time (these include the graph launch and the dispatch gap
    # an event opens)
    pairs_ev = [(ev(), ev()) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in pairs_ev:
        a.record(stream)
        graph1.replay()
        b.record(stream)
    torch.cuda.synchronize()
    rep_ms = [a.elapsed_time(b) for a, b in pairs_ev]

    part_ms = [per_launch_ms(f) for f in launches]
    merge_ms = per_launch_ms(run.merge)

    # (3) cold caches for the HBM-bound launches (merge; decode partial): a
    # read of a 1 GiB buffer before every launch evicts the 256 MB Infinity
    # Cache and the L2s without leaving dirty lines behind. Timed as the
    # difference between `steps` rounds of (flush, launch) and of the flush
    # alone, both back to back between one pair of events.
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=stream.device)
    flush_out = torch.empty((), dtype=torch.float32, device=stream.device)

    def cold_launch_ms(f):
        def rounds(with_f):
            a, b = ev(), ev()
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(steps):
                torch.sum(flush_buf, dim=0, out=flush_out)
                if with_f:
                    f()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / steps

        rounds(True)
        return max(rounds(True) - rounds(False), 1e-6)

    merge_cold_ms = cold_launch_ms(run.merge)

    rows = inp["q"].shape[0] * w.hq
    mbytes = merge_bytes(w, rows, w.cp, 2 if run.merged_dtype == torch.bfloat16 else 4)
    res = {
        "kind": w.kind,
        "description": w.description,
        "steps": steps,
        "ms_per_step": wall_ms / steps,
        "gpu_ms_per_step": gpu_ms / steps,
        "steps_per_graph": per_graph,
        "step_ms_median_own_events": float(np.median(rep_ms)),
        "step_ms_min_own_events": float(np.min(rep_ms)),
        "partial_ms": part_ms,
        "merge_ms": merge_ms,
        "merge_GBps": mbytes / (merge_ms * 1e-3) / 1e9,
        "merge_hbm_frac": mbytes / (merge_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "merge_bytes": int(mbytes),
        "merge_cold_ms": merge_cold_ms,
        "merge_cold_GBps": mbytes / (merge_cold_ms * 1e-3) / 1e9,
        "merge_cold_hbm_frac": mbytes / (merge_cold_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }
    if w.kind == "pass_kv":
        pairs = [pass_kv_pairs(inp, i) for i in own]
    else:
        pairs = [paged_pairs(inp, i) for i in own]
    flops = [4 * w.d * w.hq * p for p in pairs]
    res["pairs_per_partial"] = pairs
    res["flops_per_step"] = int(sum(flops))
    if w.kind in ("pass_kv", "pass_q"):
        res["TFLOPs"] = sum(flops) / (res["ms_per_step"] * 1e-3) / 1e12
        res["pct_bf16_peak"] = 100 * res["TFLOPs"] / PEAK_BF16_TFLOPS
        res["partial_TFLOPs"] = sum(flops) / (sum(part_ms) * 1e-3) / 1e12
        res["partial_pct_bf16_peak"] = 100 * res["partial_TFLOPs"] / PEAK_BF16_TFLOPS
        # the pass choice's rate model with this run's partial-attention rate
        # and one xGMI link per exchanged shard: which shard to pass, and
        # whether its transfer hides under the step's compute
        if w.kind == "pass_kv":
            q_lens, kv_lens = list(inp["lens"]), list(inp["lens"])
        else:
            q_lens, kv_lens = [w.new] * len(inp["lens"]), list(inp["lens"])
        res["pass_choice"] = dict(cpa.pass_cost(q_lens, kv_lens, w.hq, w.hkv, w.d, 2, w.cp, XGMI_LINK_BYTES_PER_S,
                                                res["partial_TFLOPs"] * 1e12),
                                  link_bytes_per_s=XGMI_LINK_BYTES_PER_S,
                                  mfma_flops_per_s=res["partial_TFLOPs"] * 1e12)
    else:
        # decode step (the rank's split and merge launches): K and V of every
        # visible local token, q, the cp-1 received partials (fp32 O + LSE)
        # and the merged O and LSE
        kv_bytes = 2 * w.hkv * w.d * 2 * pairs[0]  # one query per sequence: pairs == visible tokens
        nq = inp["q"].shape[0]
        out_bytes = 2 if run.merged_dtype == torch.bfloat16 else 4
        io_bytes = (nq * w.hq * w.d * 2 + (w.cp - 1) * nq * w.hq * (w.d * 4 + 4)
                    + nq * w.hq * (w.d * out_bytes + 4))
        step_bytes = kv_bytes + io_bytes
        res["step_bytes"] = int(step_bytes)
        res["partial_GBps"] = step_bytes / (res["partial_ms"][0] * 1e-3) / 1e9
        res["partial_hbm_frac"] = res["partial_GBps"] / PEAK_HBM_GBS
        cold = cold_launch_ms(launches[0])
        res["partial_cold_ms"] = cold
        res["partial_cold_GBps"] = step_bytes / (cold * 1e-3) / 1e9
        res["partial_cold_hbm_frac"] = res["partial_cold_GBps"] / PEAK_HBM_GBS
        res["GBps"] = step_bytes / (res["ms_per_step"] * 1e-3) / 1e9
        res["hbm_frac"] = res["GBps"] / PEAK_HBM_GBS
    if not merge_in_step:
        # the separate cp-way merge launch the fold replaces, timed on its own
        # for comparison (not part of the step)
        for k in [k for k in res if k.startswith("merge_")]:
            res["unfolded_" + k] = res.pop(k)
    if w.kind == "pass_kv":
        res["seq_lens"] = inp["lens"]
        if next_rows and w.dtype == torch.bfloat16 and (w.hq // w.hkv) % 2 == 0:
            # next row (fused merge): every resident shard walked in one launch,
            # the merged (O, LSE) written directly; same algorithmic work
            fw_ms = per_launch_ms(run.merged_walk)
            res["fused_walk_ms"] = fw_ms
            res["fused_walk_TFLOPs"] = sum(flops) / (fw_ms * 1e-3) / 1e12
            res["fused_walk_pct_bf16_peak"] = 100 * res["fused_walk_TFLOPs"] / PEAK_BF16_TFLOPS
            # the same shards one at a time, each folded into a running (O, LSE)
            # as a ring exchange would deliver them (cpa_partial_attn_accumulate)
            ra_ms = per_launch_ms(run.ring_accumulate)
            res["ring_accumulate_ms"] = ra_ms
            res["ring_accumulate_TFLOPs"] = sum(flops) / (ra_ms * 1e-3) / 1e12
    del run, inp, flush_buf, flush_out
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ traffic from committed counters


def _code_only(text: str) -> str:
    """Source text without comments, trailing blanks or empty lines, so that a
    comment edit does not mark the counters of an unchanged kernel stale."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def _source_digest() -> str:
    """Digest of the prefill kernel's code and of the flags it is compiled
    with: counters taken on another build of it do not describe this one."""
    from context_partial_attention_amd import build as _build

    h = hashlib.sha256()
    for f in ATTN_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "context_partial_attention_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    h.update(" ".join(_build.HIP_FLAGS + _build.FILE_FLAGS.get(ATTN_KERNEL_SOURCES[0], [])).encode())
    return h.hexdigest()[:16]


def committed_traffic():
    """HBM bytes per launch of the partial-attention kernel on the headline
    workload, from the committed rocprofv3 counter summary; None when it is
    missing or was taken from a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_digest") != _source_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def committed_clock():
    """Shader clock (GHz) during the headline launch, from the committed
    rocprofv3 counter summary (GRBM_GUI_ACTIVE per XCC over the traced launch
    time); None when it is missing or was taken from a different kernel
    source. The clock a run holds under sustained matrix load varies from box
    to box, so this is context for the roofline fraction, not a measurement of
    this run."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    text = open(COUNTERS_FILE).read()
    dig = re.search(r"kernel_source_digest: `([0-9a-f]+)`", text)
    clk = re.search(r"shader clock during the launch = .* = ([0-9.]+) GHz", text)
    if not dig or dig.group(1) != _source_digest() or not clk:
        return None
    return float(clk.group(1))


# ------------------------------------------------------------------ CPU baseline (oracle)


def cpu_baseline(name: str, budget_s: float = 15.0, block_rows: int = 64) -> dict:
    """Times the oracle on the host on a bounded sample of a pass-KV workload:
    blocks of `block_rows` consecutive query rows of the rank's zigzag shard,
    taken at evenly spread offsets through the shard (cheap early rows and
    expensive late ones alike), each with all heads against every step's KV
    shard plus the merge, until about `budget_s` of CPU work. The rate counts
    the algorithmic FLOPs (visible pairs) of the rows done."""
    import torch
    from threadpoolctl import threadpool_info

    import oracle
    from context_partial_attention_amd.workloads import WORKLOADS, draw_sequence, seq_lengths

    w = WORKLOADS[name]
    lens = seq_lengths(w)
    mine = oracle.zigzag_partition(lens, w.cp, w.rank)
    cu, qpos_all, src_all = mine["cu_seqlens"], mine["positions"], mine["src_index"]
    n_rows = int(cu[-1])
    starts = [int(x) for x in np.linspace(0, max(0, n_rows - block_rows), 16).round()]
    # shard tensors of every sequence, fp64 on the host (values drawn on the CPU:
    # the timing does not depend on them)
    data = {}
    def seq_data(b):
        if b not in data:
            L = lens[b]
            q, k, v = draw_sequence(w, b, L, L, device="cpu")
            steps = []
            for s in range(w.cp):
                part = oracle.zigzag_partition([L], w.cp, (w.rank - s) % w.cp)
                kp = part["positions"]
                steps.append((k[kp].float().numpy().astype(np.float64), v[kp].float().numpy().astype(np.float64),
                              kp))
            data[b] = (q, steps)
        return data[b]

    done_flops, elapsed, blocks = 0, 0.0, 0
    for a in starts:
        b = int(np.searchsorted(cu, a, side="right") - 1)
        e = min(a + block_rows, int(cu[b + 1]))
        q_seq, steps = seq_data(b)
        qp = qpos_all[a:e]
        qb = q_seq[torch.as_tensor(qp)].float().numpy().astype(np.float64)
        t0 = time.perf_counter()
        parts = [oracle.partial_attn(qb, qp, [0, e - a], k, v, kp, [0, len(kp)], w.scale) for k, v, kp in steps]
        oracle.lse_merge([p[0] for p in parts], [p[1] for p in parts])
        elapsed += time.perf_counter() - t0
        done_flops += 4 * w.d * w.hq * sum(int(np.searchsorted(kp, qp, side="right").sum()) for _, _, kp in steps)
        blocks += 1
        if elapsed >= budget_s:
            break
    del src_all, torch
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": done_flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{blocks} blocks of {block_rows} consecutive query rows at evenly spread offsets of rank "
                  f"{w.rank}'s zigzag shard of the {name} workload (sequence lengths {lens}), all {w.hq} heads, "
                  f"against all {w.cp} pass-KV steps' KV shards, plus the merge; fp64 NumPy; "
                  f"{done_flops / 1e9:.1f} GFLOP of visible pairs in {elapsed:.1f} s",
        "seconds": elapsed,
        "cpu": platform.processor() or platform.machine(),
    }


# ------------------------------------------------------------------ main


def environment() -> dict:
    """Software versions and the device. (The clock levels sysfs lists after
    a run are not the clock the work ran at; the roofline carries the clock
    measured by the committed counters instead.)"""
    import torch

    props = torch.cuda.get_device_properties(0)
    env = {
        "torch": torch.__version__,
        "hip": torch.version.hip,
        "device": props.name,
        "arch": getattr(props, "gcnArchName", None),
        "compute_units": props.multi_processor_count,
        "host_cpus": len(os.sched_getaffinity(0)),
    }
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    return env


def power_probe(seconds: float = 5.0):
    """Board power and shader clock (sysfs, sampled every 0.1 s) while one
    piece of work repeats for `seconds`: a 8192^3 bf16 matrix product
    (torch.matmul) with N(0, 1) operands and with zero operands, then the
    step of every workload. One JSON line per piece. The product is the
    reference for the dense bf16 rate the chip sustains at its power limit."""
    import glob
    import threading

    import torch

    from context_partial_attention_amd import harness
    from context_partial_attention_amd.workloads import WORKLOADS

    def first(pattern):
        f = sorted(glob.glob(pattern))
        return f[0] if f else None

    pw = first("/sys/class/drm/card*/device/hwmon/hwmon*/power1_average") or \
        first("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input")
    sclk = first("/sys/class/drm/card*/device/pp_dpm_sclk")
    temps = {}  # label -> file
    for f in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/temp*_input")):
        try:
            label = open(f.replace("_input", "_label")).read().strip()
        except OSError:
            label = os.path.basename(f)
        temps.setdefault(label, f)

    def read_temps():
        out = {}
        for label, f in temps.items():
            try:
                out[label] = int(open(f).read()) / 1000.0
            except (OSError, ValueError):
                pass
        return out

    def sample():
        w = mhz = None
        try:
            w = int(open(pw).read()) / 1e6 if pw else None
        except (OSError, ValueError):
            pass
        try:
            for line in open(sclk) if sclk else []:
                if "*" in line:
                    mhz = int(line.split(":")[1].strip().lower().split("mhz")[0])
        except (OSError, ValueError, IndexError):
            pass
        return w, mhz

    def run(label, fn, flops=None):
        samples, tsamples, done = [], [], threading.Event()

        def sampler():
            while not done.is_set():
                samples.append(sample())
                tsamples.append(read_temps())
                time.sleep(0.1)

        fn()
        torch.cuda.synchronize()
        th = threading.Thread(target=sampler)
        n, t0 = 0, time.time()
        th.start()
        while time.time() < t0 + seconds:
            fn()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        el = time.time() - t0
        done.set()
        th.join()
        # the first second is the ramp from idle
        steady = samples[len(samples) // 5:]
        ws = sorted(x[0] for x in steady if x[0] is not None)
        cs = sorted(x[1] for x in steady if x[1] is not None)
        out = {"work": label, "calls": n, "seconds": round(el, 2), "ms_per_call": round(el / n * 1e3, 4),
               "power_W_median": ws[len(ws) // 2] if ws else None, "sclk_MHz_median": cs[len(cs) // 2] if cs else None}
        if flops:
            out["TFLOPs"] = round(flops * n / el / 1e12, 1)
        steady_t = tsamples[len(tsamples) // 5:]
        for lab in temps:
            v = sorted(t[lab] for t in steady_t if lab in t)
            if v:
                out[f"temp_{lab}_C_median"] = v[len(v) // 2]
        print(json.dumps(out), flush=True)

    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    c = torch.empty_like(a)
    run("matmul bf16 8192^3, N(0,1) operands", lambda: torch.matmul(a, b, out=c), 2 * 8192 ** 3)
    a.zero_()
    b.zero_()
    run("matmul bf16 8192^3, zero operands", lambda: torch.matmul(a, b, out=c), 2 * 8192 ** 3)
    del a, b, c
    for name in DEFAULT_WORKLOADS:
        w = WORKLOADS[name]
        inp = harness.build(w, device="cuda", keep_full=False)
        r = harness.Runner(inp)
        if w.kind == "pass_kv":
            run(f"{name}: batched partials + merge", r.step)
        else:  # the other ranks' partials arrive once; the rank's own launch folds them in
            for i in range(w.cp):
                if i != w.rank:
                    r.partial(i)
            run(f"{name}: the rank's own launch with the fold", r.rank_fold)
        del r, inp
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workloads", type=str, default=",".join(DEFAULT_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the fused-merge walk and running-merge timings (profiling the partials kernel alone)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device-to-device copy of 256 MiB (x4) to scale HBM byte counters")
    ap.add_argument("--power-probe", action="store_true",
                    help="only sample board power and shader clock under a bf16 matmul and each workload's step")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}); "
              "the whole-job value is the one GPU's throughput at --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import context_partial_attention_amd as cpa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cpa.load_library()
    if args.calibrate_copy:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_per_dispatch": n, "dispatches": 4}), flush=True)
        return
    if args.power_probe:
        power_probe()
        return
    names = [n for n in args.workloads.split(",") if n]
    if HEADLINE not in names:
        names = [HEADLINE] + names
    results = {}
    for name in names:
        log(f"[bench] {name}: {args.warmup} warmup + {args.steps} timed steps")
        results[name] = bench_workload(name, args.steps, args.warmup, next_rows=not args.no_next_rows)
        log(f"[bench] {name}: {json.dumps({k: v for k, v in results[name].items() if k != 'description'})}")
    h = results[HEADLINE]
    from context_partial_attention_amd.workloads import WORKLOADS

    hw = WORKLOADS[HEADLINE]
    # dominant kernel of the headline: the batched partial-attention launch
    part_ms = float(np.mean(h["partial_ms"]))
    flops_per_launch = h["flops_per_step"] / len(h["partial_ms"])
    achieved = flops_per_launch / (part_ms * 1e-3) / 1e12
    traffic = committed_traffic()
    clock = committed_clock()
    line = {
        "metric": METRIC,
        "value": h["TFLOPs"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_bf16_mfma_peak": h["pct_bf16_peak"],
        "config": {
            "workload": HEADLINE,
            "seq_lens": h["seq_lens"],
            "cp": hw.cp,
            "rank": hw.rank,
            "hq": hw.hq,
            "hkv": hw.hkv,
            "d": hw.d,
            "step": f"{hw.cp} pass-KV partial attentions (one batched launch) + {hw.cp}-way LSE merge (bf16 out); "
                    f"the timed loop replays a captured HIP graph of {h['steps_per_graph']} consecutive steps",
        },
        "roofline": {
            "kernel": f"attn_pp_kernel<{hw.d}, contiguous, fp32 out, partials>, all {hw.cp} pass-KV steps in one "
                      "launch (event time includes its launch-order pre-pass)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "avg_launch_ms": part_ms,
            "flops_per_launch": flops_per_launch,
            # from the committed counters (same kernel source), not this run:
            # the shader clock under this launch's load and the dense bf16 rate
            # of 1024 SIMDs x 1024 FLOP per clock at that clock
            "profiled_shader_clock_ghz": clock,
            "mfma_peak_at_profiled_clock": 1024 * 1024 * clock * 1e-3 if clock else None,
        },
        "workloads": {k: v for k, v in results.items() if k != HEADLINE},
        # not the step above: the fused-merge walk (cpa_partial_attn_merged) on
        # the same workload, merged output without fp32 partials or a merge pass
        "fused_merge": {
            "ms": h.get("fused_walk_ms"),
            "TFLOPs": h.get("fused_walk_TFLOPs"),
            "pct_bf16_peak": h.get("fused_walk_pct_bf16_peak"),
            "ring_accumulate_ms": h.get("ring_accumulate_ms"),
            "ring_accumulate_TFLOPs": h.get("ring_accumulate_TFLOPs"),
        },
        # the headline step's two parts: the batched partial launch and the
        # HBM-bound 4-way merge (warm and with caches evicted first)
        "step_parts": {k: h.get(k) for k in ("partial_ms", "merge_ms", "merge_bytes", "merge_GBps", "merge_hbm_frac",
                                             "merge_cold_ms", "merge_cold_GBps", "merge_cold_hbm_frac")},
    }
    line["environment"] = environment()
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(HEADLINE)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
