"""Throughput of the batched speculative-sampling verifier on one MI355X.

One step = one spec_verify call (statistics of every position, the
first-rejection scan, residual mass and the correction or bonus draw) over
one synthetic batch already resident in HBM.  Default workload: the largest
of the single-GPU batches, B=256 rows, K=7 drafts, V=201,088 bf16 logits,
T=1.0, dense draft, low draft agreement.  Inputs rotate over enough
identical copies that the 256 MB Infinity Cache cannot serve a step's reads
from the previous steps.

Prints one JSON line: verified draft positions per second (B*K per step);
the dominant kernel's achieved HBM bandwidth against the 8 TB/s peak
(``roofline``) and the whole call's (``whole_call``); per-call p10/p50/p90;
the fp64 CPU oracle's rate on a bounded sample of the same workload
(``cpu_baseline``) and how the timed call's outputs compare with it.

    python bench.py [--steps K] [--warmup W] [--config C] [--no-cpu]

Warm-up: W untimed calls before each timed pass.  By default W is sized so
that the warm-up keeps the GPU busy for about WARMUP_S seconds (estimated
from a few calls), which brings the clocks to their steady state; a GPU
that has been idle while the host generated the inputs runs a short burst
several percent slower.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft positions/sec at 1 GPU + achieved HBM GB/s vs peak"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
WARMUP_S = 0.3


def warmup_calls(args, step, torch) -> int:
    """W: args.warmup if given, else enough calls to fill about WARMUP_S
    seconds (the calls made to estimate it are among the W).  Runs the first
    warm-up pass."""
    if args.warmup is not None:
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        return args.warmup
    probe = 5
    for i in range(probe):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(probe):
        step(i)
    torch.cuda.synchronize()
    per_call = (time.perf_counter() - t0) / probe
    w = max(20, min(20000, int(WARMUP_S / max(per_call, 1e-6)) + 1))
    for i in range(2 * probe, w):
        step(i)
    torch.cuda.synchronize()
    return max(w, 2 * probe)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rejection_sampling_verifier_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(d) -> dict:
    """Bytes the method must move: every target logit once, every draft logit
    of a sampling row once (greedy rows never read the draft), plus tokens,
    uniforms, temperatures and outputs."""
    B, Kp1, V = d["target"].shape
    K = Kp1 - 1
    esz = d["target"].itemsize
    n_sampling = int((d["temperature"] > 0).sum())
    logits = B * Kp1 * V * esz + n_sampling * K * V * esz
    small = B * K * 4 + B * Kp1 * 4 + B * 4 + B * Kp1 * 4 + B * 4
    return {"stats_kernel": logits, "m_min": logits + small}


def traffic_from_profiles(workload: str, kernel: str = "stats_kernel"):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*(\w+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def call_traffic_from_profiles(workload: str):
    """HBM bytes read and written per spec_verify call (every kernel of the
    call) from the committed counter summary, if it was taken on the current
    kernel source."""
    path = os.path.join(ROOT, "profiles", f"stats_kernel_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*(\w+)", text)
    if not m_hash or m_hash.group(1) != kernel_source_hash():
        return None
    per = {k: (float(r), float(w)) for k, r, w in
           re.findall(r"^(\w+_kernel): \d+ dispatches; read ([0-9.]+) B, written ([0-9.]+) B", text, re.M)}
    if "stats_kernel" not in per or "finish_kernel" not in per:
        return None
    return {"read": sum(r for r, _ in per.values()), "written": sum(w for _, w in per.values()),
            "kernels": sorted(per)}


# Threads of the CPU baseline: the host CPU share of one GPU on the
# measurement machines (16), whatever os.cpu_count() reports there.
CPU_THREADS = 16


def host_cpu() -> dict:
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"logical_cpus": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0)), "model": model}


def cpu_baseline(d, budget_s: float, runs: int = 3):
    """The fp64 oracle, as it is, over rows in a thread pool.  `runs` timed
    runs, each of whole passes over the batch for about budget_s / runs
    seconds; the rate is the median run's.  Also returns the first pass's
    oracle results (for comparison with the GPU outputs)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    B, Kp1, _ = d["target"].shape
    K = Kp1 - 1
    threads = max(1, min(CPU_THREADS, len(os.sched_getaffinity(0))))

    def one(b):
        return oracle.verify(d["target"], d["draft"], d["tokens"], d["uniforms"], d["temperature"],
                             d["topk"], d["dtype"], rows=[b])[0]

    rates, first, passes, secs = [], None, 0, 0.0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for _ in range(runs):
            rows_done = 0
            t0 = time.perf_counter()
            while True:
                res = list(ex.map(one, range(B)))
                first = first or res
                rows_done += B
                if time.perf_counter() - t0 >= budget_s / runs:
                    break
            dt = time.perf_counter() - t0
            rates.append(rows_done * K / dt)
            passes += rows_done // B
            secs += dt
    rates.sort()
    hc = host_cpu()
    return {"value": rates[len(rates) // 2], "unit": "positions/s", "cores": threads, "kind": "oracle",
            "runs": [round(r, 1) for r in rates],
            "host": hc,
            "sample": f"median of {runs} runs; {passes} full passes over the {B}-row batch "
                      f"({passes * B * K} positions) in {secs:.1f} s, rows spread over {threads} threads "
                      f"(the CPU share of one GPU; the host reports {hc['logical_cpus']} logical CPUs)"}, first


def oracle_comparison(out, nacc, ref, uniforms) -> dict:
    """How the timed call's outputs compare with the oracle: rows equal, and
    the rows with a decision within 1e-5 of its threshold (near), where the
    other side is also correct."""
    import numpy as np

    equal = near = near_equal = 0
    for b, r in enumerate(ref):
        same = int(nacc[b]) == r.n and list(out[b]) == list(r.tokens)
        is_near = False
        if not r.greedy:
            K = r.margins.shape[0]
            for i in range(min(r.n + 1, K)):
                if r.margins[i] <= 1e-5 and r.margins[i] <= 1e-4 * max(r.p_d[i], float(uniforms[b, i]) * r.q_d[i]):
                    is_near = True
            is_near = is_near or r.gap <= 1e-5
        equal += same
        near += is_near
        near_equal += same and is_near
    return {"rows": len(ref), "rows_equal": equal, "near_rows": near, "near_rows_equal": near_equal,
            "firm_rows_differing": len(ref) - near - (equal - near_equal),
            "mean_accepted_oracle": round(float(np.mean([r.n for r in ref])), 4)}


def copy_calibration(nbytes: int, reps: int):
    """Plain device-to-device copies of a known size (for counter scaling)."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=None,
                    help=f"untimed calls before each timed pass (default: about {WARMUP_S} s of calls)")
    ap.add_argument("--config", type=int, default=2,
                    help="workload index (2 = the default bench line: B256 K7 V201088)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run plain copies of this many MiB (counter calibration)")
    ap.add_argument("--kl", action="store_true",
                    help="time spec_verify_kl (verification plus KL(p||q) per position; whole-call "
                         "rate only)")
    ap.add_argument("--early-exit", action="store_true",
                    help="time spec_verify_early_exit (reads each row's logits up to its first rejection)")
    ap.add_argument("--tree", type=int, default=-1,
                    help="time spec_verify_tree on this draft-tree workload instead (0 = 61-node tree)")
    ap.add_argument("--streams", type=int, default=1,
                    help="independent batches in flight: consecutive calls alternate over this many streams, "
                         "each with its own workspace and outputs (1: one call after the other)")
    ap.add_argument("--relaxed", default="",
                    help="ALPHA,MAX_RANK,MIN_PROB: time the lossy relaxed acceptance rule instead "
                         "(whole-call rate only; per-kernel times come from a rocprofv3 trace)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(rows shard across GPUs without communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    import rejection_sampling_verifier_amd as rsv

    if args.tree >= 0:
        tree_main(args, W, rsv, np, torch)
        return

    case = W.CONFIGS[args.config]
    t0 = time.perf_counter()
    d = W.make(case)
    print(f"[bench] generated {case.name} in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    by = algorithmic_bytes(d)
    copies = max(1, -(-(2 * MALL_BYTES) // by["m_min"]) + (1 if by["m_min"] < 2 * MALL_BYTES else 0))
    copies = min(copies, 8)

    def upload(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if a.dtype == np.uint16:
            t = t.view(torch.bfloat16)
        return t.to(dev)

    base = {k: upload(d[k]) for k in ("target", "draft", "tokens", "uniforms", "temperature")}
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]
    B, Kp1, V = base["target"].shape
    K = Kp1 - 1
    dt_code = rsv.SV_BF16 if d["dtype"] == "bf16" else rsv.SV_F32
    # One stream, workspace and output set per batch in flight.
    ns = max(1, args.streams)
    main_stream = torch.cuda.current_stream(dev)
    streams = [main_stream] + [torch.cuda.Stream(dev) for _ in range(ns - 1)]

    def buffers():
        return {"ws": rsv.new_workspace(B, K, V, d["topk"], dt_code, dev),
                "out": torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                "nacc": torch.empty((B,), dtype=torch.int32, device=dev),
                "kl": torch.empty((B, K), dtype=torch.float32, device=dev) if args.kl else None,
                "ee_ws": (rsv.new_early_exit_workspace(B, K, V, dt_code, dev, d["topk"])
                          if args.early_exit else None)}

    bufs = [buffers() for _ in range(ns)]
    nacc = bufs[0]["nacc"]

    rule = None
    if args.relaxed:
        a_, r_, p_ = args.relaxed.split(",")
        rule = dict(alpha=float(a_), max_rank=int(r_), min_prob=float(p_))

    def step(i, timer=None):
        x = sets[i % copies]
        k = 0 if timer is not None else i % ns  # per-kernel timing runs on one stream
        stream, bf = streams[k], bufs[k]
        out, nacc, ws, ee_ws, kl_buf = bf["out"], bf["nacc"], bf["ws"], bf["ee_ws"], bf["kl"]
        if args.early_exit and timer is None:
            rsv.verify_early_exit(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"],
                                  d["topk"], out_tokens=out, num_accepted=nacc, workspace=ee_ws,
                                  stream=stream.cuda_stream)
            return
        if args.kl and timer is None:
            rsv.verify_kl(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"], d["topk"],
                          out_tokens=out, num_accepted=nacc, kl=kl_buf, workspace=ws, stream=stream.cuda_stream)
            return
        if rule is not None and timer is None:
            rsv.verify_relaxed(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"],
                               d["topk"], **rule, out_tokens=out, num_accepted=nacc, workspace=ws,
                               stream=stream.cuda_stream)
            return
        fn = timer.run if timer is not None else rsv.verify
        fn(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"], d["topk"],
           out_tokens=out, num_accepted=nacc, workspace=ws, stream=stream.cuda_stream)

    args.warmup = warmup_calls(args, step, torch)

    # Timed region 1: plain calls, bracketed by events and wall clock, with
    # nothing else enqueued between them.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(main_stream)
    for s_ in streams[1:]:
        s_.wait_event(ev0)
    for i in range(args.steps):
        step(i)
    for s_ in streams[1:]:
        main_stream.wait_stream(s_)
    ev1.record(main_stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # The per-call spread (one stream): the same calls with an event after
    # each, in a pass of their own -- an event between two calls delays the
    # next one by a few microseconds, so it stays out of the timed region.
    spread = None
    if ns == 1:
        per_call = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        for i in range(args.warmup):
            step(i)
        per_call[0].record(main_stream)
        for i in range(args.steps):
            step(i)
            per_call[i + 1].record(main_stream)
        torch.cuda.synchronize()
        ts = [per_call[i].elapsed_time(per_call[i + 1]) for i in range(args.steps)]
        q = np.percentile(np.array(ts), [10, 50, 90])
        spread = {"p10": round(float(q[0]), 5), "p50": round(float(q[1]), 5), "p90": round(float(q[2]), 5),
                  "note": "from a separate pass with an event after every call, which adds a few us per call"}
    accepted = float(nacc.float().mean().item())

    # Timed region 2: the same calls, each kernel's dispatch carrying a
    # start/stop event pair on the stream it runs on, for per-kernel times.
    # The host-side set-up above leaves the GPU idle for a moment: the same
    # W untimed calls first, enqueued right before the timed ones.
    timers = [rsv.StageTimer() for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    for i in range(args.steps):
        step(i, timers[i])
    torch.cuda.synchronize()
    stages = np.array([t.stage_ms() for t in timers])
    for t in timers:
        t.close()
    stage_ms = stages.mean(axis=0)
    n_launch = rsv.launches(B, K, V, d["topk"], dt_code)
    if n_launch < 3:
        stage_ms[1] = 0.0  # no merge kernel: its two events are recorded back to back
    stats_ms = float(stage_ms[0])

    positions = B * K
    value = positions / (ms_per_step * 1e-3)
    roof_kernel, roof_bytes, roof_ms = "stats_kernel", by["stats_kernel"], stats_ms
    achieved = roof_bytes / (roof_ms * 1e-3) / 1e9
    if args.early_exit:
        # Algorithmic bytes: the logits of the positions each row reaches
        # (targets 0..n, drafts 0..min(n, K-1) of sampling rows); a truncated
        # draft is selected before the walk, so all K drafts of a sampling
        # row are read.  The residual re-read is extra traffic.
        n_acc = nacc.cpu().numpy().astype(np.int64)
        esz = d["target"].itemsize
        samp = d["temperature"] > 0
        drafts = np.full_like(n_acc, K) if int(d["topk"]) > 0 else np.minimum(n_acc + 1, K)
        rows = np.minimum(n_acc + 1, K + 1) + np.where(samp, drafts, 0)
        roof_kernel, roof_bytes, roof_ms = "early_exit_kernel", int(rows.sum()) * V * esz, ms_per_step
        achieved = roof_bytes / (roof_ms * 1e-3) / 1e9
    traffic = traffic_from_profiles(f"B{B}K{K}V{V}", roof_kernel)
    plain = not (args.early_exit or args.kl or rule is not None)
    call_traffic = call_traffic_from_profiles(f"B{B}K{K}V{V}") if plain else None
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": case.name, "B": B, "K": K, "V": V, "logits": d["dtype"],
                   "temperature": float(case.temperature), "greedy_rows": case.greedy_rows,
                   "topk_draft": case.topk, "input_copies": copies,
                   "acceptance": "lossless" if rule is None else f"relaxed {rule}",
                   "kl_per_position": bool(args.kl), "early_exit": bool(args.early_exit),
                   "streams": ns},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None if args.early_exit else traffic, "kernel": roof_kernel,
                     "bytes_per_launch": roof_bytes, "avg_launch_ms": round(roof_ms, 5)},
        "whole_call": {"achieved": round(by["m_min"] / (ms_per_step * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                       "unit": "GB/s", "frac": round(by["m_min"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                       "bytes": by["m_min"], "ms": round(ms_per_step, 5),
                       "note": "algorithmic bytes of the whole call (every logit it must read once, tokens, "
                               "uniforms, temperatures, outputs) over the per-call time of all its kernels"},
        # The call's HBM traffic from the committed counter summary (FETCH_SIZE and
        # WRITE_SIZE of every kernel of the call, calibrated), while the kernel
        # sources are those it was taken on; null otherwise.
        "whole_call_counters": None if call_traffic is None else {
            "read_bytes": round(call_traffic["read"]), "written_bytes": round(call_traffic["written"]),
            "GBps": round((call_traffic["read"] + call_traffic["written"]) / (ms_per_step * 1e-3) / 1e9, 1),
            "frac": round((call_traffic["read"] + call_traffic["written"]) / (ms_per_step * 1e-3) / 1e9
                          / HBM_PEAK_GBPS, 4),
            "read_over_m_min": round(call_traffic["read"] / by["m_min"], 4),
            "kernels": call_traffic["kernels"]},
        "ms_per_call_spread": spread,
        "m_min_bytes": by["m_min"],
        "kernel_ms": {"stats_kernel": round(float(stage_ms[0]), 5),
                      "merge_kernel": round(float(stage_ms[1]), 5),
                      "finish_kernel": round(float(stage_ms[2]), 5)},
        "launches_per_call": n_launch,
        "wall_ms_per_step": round(wall_ms / args.steps, 5),
        "mean_accepted": round(accepted, 4),
        "kernel_ms_rule": "lossless",
        "kernel_source_hash": kernel_source_hash(),
    }
    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb << 20, 5)
    if not args.no_cpu:
        print("[bench] timing the CPU oracle ...", file=sys.stderr, flush=True)
        line["cpu_baseline"], ref = cpu_baseline(d, args.cpu_seconds)
        if rule is None:
            o = bufs[0]["out"].cpu().numpy()
            n_ = bufs[0]["nacc"].cpu().numpy()
            line["oracle_comparison"] = oracle_comparison(o, n_, ref, d["uniforms"])
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def tree_algorithmic_bytes(d) -> dict:
    """Every target logit once, and the draft logits of every node with
    children of a sampling row once, plus tokens, parents, uniforms,
    temperatures and outputs."""
    import numpy as np

    B, N, V = d["target"].shape
    esz = d["target"].itemsize
    internal = 0
    for b in range(B):
        if d["temperature"][b] > 0:
            internal += np.unique(d["parents"][b, 1:][d["parents"][b, 1:] >= 0]).size
    logits = B * N * V * esz + internal * V * esz
    small = 3 * B * N * 4 + B * 4 + 2 * B * N * 4 + B * 4
    return {"stats_kernel": logits, "m_min": logits + small, "internal_nodes": internal}


def tree_cpu_baseline(d, budget_s: float, runs: int = 3):
    """The oracle's tree walk, as it is, over rows in a thread pool: the
    median of `runs` timed runs of whole passes over the batch."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    B, N, _ = d["target"].shape
    threads = max(1, min(CPU_THREADS, len(os.sched_getaffinity(0))))

    def one(b):
        return oracle.verify_tree(d["target"], d["draft"], d["tokens"], d["parents"], d["uniforms"],
                                  d["temperature"], d.get("topk", 0), d["dtype"], rows=[b])

    rates, passes, secs = [], 0, 0.0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for _ in range(runs):
            rows_done = 0
            t0 = time.perf_counter()
            while True:
                list(ex.map(one, range(B)))
                rows_done += B
                if time.perf_counter() - t0 >= budget_s / runs:
                    break
            dt = time.perf_counter() - t0
            rates.append(rows_done * (N - 1) / dt)
            passes += rows_done // B
            secs += dt
    rates.sort()
    hc = host_cpu()
    return {"value": rates[len(rates) // 2], "unit": "nodes/s", "cores": threads, "kind": "oracle",
            "runs": [round(r, 1) for r in rates], "host": hc,
            "sample": f"median of {runs} runs; {passes} full passes over the {B}-row batch "
                      f"({passes * B * (N - 1)} draft nodes) in {secs:.1f} s, rows spread over {threads} threads "
                      f"(the CPU share of one GPU; the host reports {hc['logical_cpus']} logical CPUs)"}


def tree_main(args, W, rsv, np, torch):
    """One step = one spec_verify_tree call over a batch of draft trees."""
    case = W.TREE_CONFIGS[args.tree]
    t0 = time.perf_counter()
    d = W.make_tree(case)
    print(f"[bench] generated {case.name} in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    by = tree_algorithmic_bytes(d)
    copies = min(8, max(1, -(-(2 * MALL_BYTES) // by["m_min"]) + (1 if by["m_min"] < 2 * MALL_BYTES else 0)))

    def upload(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if a.dtype == np.uint16:
            t = t.view(torch.bfloat16)
        return t.to(dev)

    keys = ("target", "draft", "tokens", "parents", "uniforms", "temperature")
    base = {k: upload(d[k]) for k in keys}
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]
    B, N, V = base["target"].shape
    dt_code = rsv.SV_BF16 if d["dtype"] == "bf16" else rsv.SV_F32
    ws = rsv.new_tree_workspace(B, N, V, dt_code, dev, case.topk)
    out = torch.empty((B, N), dtype=torch.int32, device=dev)
    nodes = torch.empty((B, N), dtype=torch.int32, device=dev)
    nacc = torch.empty((B,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, timer=None):
        x = sets[i % copies]
        fn = timer.run if timer is not None else rsv.verify_tree
        fn(x["target"], x["draft"], x["tokens"], x["parents"], x["uniforms"], x["temperature"], case.topk,
           out_tokens=out, out_nodes=nodes, num_accepted=nacc, workspace=ws,
           stream=stream.cuda_stream)

    args.warmup = warmup_calls(args, step, torch)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    accepted = float(nacc.float().mean().item())

    timers = [rsv.TreeTimer() for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.warmup):  # the GPU is idle after the host-side set-up
        step(i)
    for i in range(args.steps):
        step(i, timers[i])
    torch.cuda.synchronize()
    stages = np.array([t.stage_ms() for t in timers])
    for t in timers:
        t.close()
    stats_ms, walk_ms = (float(v) for v in stages.mean(axis=0))

    # Residual passes per row (rejected siblings), from one probed call.
    x = sets[0]
    _, _, na, probs, _ = rsv.verify_tree(x["target"], x["draft"], x["tokens"], x["parents"], x["uniforms"],
                                         x["temperature"], case.topk, probes=True, workspace=ws)
    torch.cuda.synchronize()
    tested = (~torch.isnan(probs[:, :, 0])).sum(dim=1).cpu().numpy()
    passes = tested - na.cpu().numpy()

    value = B * (N - 1) / (ms_per_step * 1e-3)
    achieved = by["stats_kernel"] / (stats_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": case.name, "B": B, "nodes": N, "V": V, "logits": d["dtype"],
                   "temperature": float(case.temperature), "internal_nodes_read": by["internal_nodes"],
                   "topk_draft": case.topk,
                   "input_copies": copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "tree_stats_kernel", "bytes_per_launch": by["stats_kernel"],
                     "avg_launch_ms": round(stats_ms, 5)},
        "effective_GBps_whole_call": round(by["m_min"] / (ms_per_step * 1e-3) / 1e9, 1),
        "m_min_bytes": by["m_min"],
        "kernel_ms": {"tree_stats_kernel": round(stats_ms, 5), "tree_finish_kernel": round(walk_ms, 5)},
        "wall_ms_per_step": round(wall_ms / args.steps, 5),
        "mean_accepted": round(accepted, 4),
        "mean_residual_passes": round(float(passes.mean()), 3),
        "max_residual_passes": int(passes.max()),
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu:
        print("[bench] timing the CPU oracle ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = tree_cpu_baseline(d, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
