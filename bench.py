#!/usr/bin/env python3
"""Benchmark of DSpark's per-round token path on one MI355X.

Metric: verified draft positions per second, B * gamma / t_step, where one
step is one round of the gated path -- dspark_markov_draft followed by
dspark_verify -- over one batch of the V=151936, r=256, gamma=7, B=256,
T=0.7 synthetic workload (bf16 Markov weights, float32 logits), with the
inputs resident in HBM.  The round counter changes every step, so the drafts
and the accepted lengths change while the input bytes stay fixed.  Each
step runs after a 512 MiB write that evicts the memory-side cache (as the
target's forward pass does between rounds) and is timed alone with HIP events
on the launch stream; the value is the median step, with p10 and p90 beside
it and the back-to-back warm-cache rate as an extra field.

The draft is the device-resident one (all positions in one launch, from the
vocabulary-major copy of W2 prepared once outside the timed region) wherever
the library can run it, else one tile pass and one selection per position;
--per-position forces the latter.

Printed (one JSON line): the metric, the fraction of the 8 TB/s HBM peak that
the step's compulsory bytes reach, the roofline of the dominant kernel (the
resident draft, or the per-position draft's tile pass, timed live with HIP
events on its own stream), the analytical
dspark_survival time and the scheduled round (confidence head, prefix
scheduler, verification at its lengths; both reported beside the gated
path), the RNN-head draft at the same sizes beside the Markov draft, and the
float64 oracle
timed on the host cores on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload NAME]
"""

import argparse
import hashlib
import json
import multiprocessing
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

HBM_PEAK = 8.0e12            # bytes/s, MI355X published peak
MFMA_BF16_PEAK = 2.5e15      # dense bf16 FLOP/s, MI355X published peak
METRIC = "verified draft positions/sec, V=151936 γ=7 B=256; % of HBM roofline"
TILE_COLS = 128              # vocabulary columns per tile of the tile pass
PMC_FILES = {"tile_pass_sample": os.path.join(ROOT, "profiles", "tile_pass_sample_v151936_b256_pmc.json"),
             "draft_resident": os.path.join(ROOT, "profiles", "draft_resident_v151936_b256_pmc.json")}
KERNEL_SRC = {"tile_pass_sample": os.path.join(ROOT, "draft_sampling_verification_bias_amd", "csrc", "tile_pass.hip"),
              "draft_resident": os.path.join(ROOT, "draft_sampling_verification_bias_amd", "csrc", "resident.hip")}


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a bounded sample of requests
# ---------------------------------------------------------------------------
_CTX = {}


def _oracle_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def _oracle_round(task):
    import oracle
    b, rnd = task
    wl, W1f, W2f = _CTX["wl"], _CTX["W1f"], _CTX["W2f"]
    d = oracle.markov_draft(wl.U, W1f, W2f, wl.x0, wl.T, wl.seeds, rnd, requests=[b])
    v = oracle.verify(wl.U, W1f, W2f, wl.x0, d["tokens"], wl.tgt, wl.T, wl.seeds, rnd, requests=[b])
    return int(v["accept_len"][b])


def cpu_baseline(wl, nreq, nrounds):
    """The oracle's draft + verify of requests 0..nreq-1 over nrounds rounds."""
    import oracle
    _CTX["wl"] = wl
    _CTX["W1f"] = oracle.weights_as_f64(wl.W1, wl.wdtype)
    _CTX["W2f"] = oracle.weights_as_f64(wl.W2, wl.wdtype)
    tasks = [(b, 1000 + i) for i in range(nrounds) for b in range(nreq)]
    workers = max(1, min(16, len(os.sched_getaffinity(0)), len(tasks)))
    ctx = multiprocessing.get_context("fork")
    with ctx.Pool(workers, initializer=_oracle_worker_init) as pool:
        pool.map(int, range(workers))  # start the workers before timing
        t0 = time.perf_counter()
        pool.map(_oracle_round, tasks, chunksize=1)
        t1 = time.perf_counter()
    secs = t1 - t0
    visible, model = host_cpus()
    return {"value": len(tasks) * wl.gamma / secs, "unit": "positions/s", "cores": workers, "kind": "oracle",
            "host_cores_visible": visible, "cpu_model": model,
            "sample": "draft+verify of requests 0..%d of %s over %d rounds (float64 numpy, %d worker processes x "
                      "1 thread on %d visible cores, %.1f s wall)" % (nreq - 1, wl.name, nrounds, workers, visible,
                                                                      secs)}


def host_cpus():
    """Cores this process may run on, and the CPU model name."""
    visible = len(os.sched_getaffinity(0))
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return visible, model


# ---------------------------------------------------------------------------
def tile_pass_bytes(B, gamma, V, r):
    """Algorithmic bytes of one draft tile-pass launch (one block position):
    the U_k rows, the launch's share of W2 -- read once per round, so r V / gamma
    of its 2-byte values per position -- the gathered W1 rows and the
    per-(row, tile) summaries.  Re-reads of W2 at every position are not
    algorithmic bytes."""
    ntiles = (V + TILE_COLS - 1) // TILE_COLS
    return 4 * B * V + 2 * r * V / gamma + 2 * B * r + 8 * B * ntiles


def resident_draft_bytes(B, gamma, V, r):
    """Algorithmic bytes of one device-resident draft launch (all gamma
    positions): every U row, W2 once (from its vocabulary-major copy), the W1
    rows of the previous tokens and the three outputs."""
    return 4 * B * gamma * V + 2 * r * V + 2 * r * B * gamma + 12 * B * gamma


def step_bytes(B, gamma, V, r, accept_len):
    """Compulsory bytes of one round (draft + verify): all U rows, target rows
    1..n_b+1 of each request, W2 once, the W1 rows gathered by the draft and by
    the residual of the rejecting requests."""
    n = accept_len.astype(np.int64)
    rej = int((n < gamma).sum())
    return 4 * B * gamma * V + 4 * V * int((n + 1).sum()) + 2 * r * V + 2 * r * (B * gamma + rej)


def code_digest(path):
    """sha256 of a kernel source's code: the text with // comments, trailing
    blanks and empty lines removed, so that edits of comments alone keep it."""
    lines = []
    with open(path) as f:
        for line in f:
            i = line.find("//")
            if i >= 0:
                line = line[:i]
            line = line.rstrip()
            if line.strip():
                lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def pmc_traffic(kname, workload):
    """HBM bytes per launch of a kernel from its committed counter summary, or
    None if there is none for this workload or the kernel's code changed since
    it was taken."""
    path = PMC_FILES.get(kname)
    if path is None or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("workload") != workload:
        return None
    if rec.get("code_sha256") != code_digest(KERNEL_SRC[kname]):
        return None
    return rec.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="v151936_b256_t07", choices=workloads.NAMES)
    ap.add_argument("--cpu-sample", type=int, default=256, help="requests in the oracle baseline (0: skip)")
    ap.add_argument("--cpu-rounds", type=int, default=6, help="rounds of those requests in the oracle baseline")
    ap.add_argument("--survival-steps", type=int, default=10)
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="MiB written before every step to evict the memory-side cache (0: no eviction)")
    ap.add_argument("--warm-steps", type=int, default=20,
                    help="extra back-to-back steps without eviction, reported as 'warm' (0: skip)")
    ap.add_argument("--schedule-steps", type=int, default=20,
                    help="timed calls of the prefix scheduler and of verification with its lengths (0: skip)")
    ap.add_argument("--rnn-steps", type=int, default=10,
                    help="timed calls of the RNN-head draft beside the Markov draft (0: skip)")
    ap.add_argument("--per-position", action="store_true",
                    help="draft with one tile pass and one selection launch per position (default: all "
                         "positions in one device-resident launch from the W2T copy, where it applies)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="copy this many MiB device to device once before timing (a reference kernel of known "
                         "traffic for hardware counter runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the path is sharded by request with no exchange between "
              "GPUs, and runs with more than one GPU are not part of this build (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    log("building workload %s" % args.workload)
    wl = workloads.make(args.workload)
    B, gamma, V, r, T = wl.B, wl.gamma, wl.V, wl.r, wl.T

    cpu = None
    if args.cpu_sample > 0:
        log("timing the oracle on %d requests" % args.cpu_sample)
        cpu = cpu_baseline(wl, min(args.cpu_sample, B), max(1, args.cpu_rounds))
        log("oracle: %.1f positions/s on %d cores" % (cpu["value"], cpu["cores"]))

    import torch
    import draft_sampling_verification_bias_amd as dsp

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    U = torch.from_numpy(wl.U).to(dev)
    tgt = torch.from_numpy(wl.tgt).to(dev)
    if wl.wdtype == "bf16":
        W1 = torch.from_numpy(wl.W1.view(np.int16)).to(dev).view(torch.bfloat16)
        W2 = torch.from_numpy(wl.W2.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        W1, W2 = torch.from_numpy(wl.W1).to(dev), torch.from_numpy(wl.W2).to(dev)
    x0 = torch.from_numpy(wl.x0).to(dev)
    seeds = torch.from_numpy(wl.seeds.view(np.int64)).to(dev).view(torch.uint64)
    del wl.U, wl.tgt
    # The Markov projection is also held vocabulary-major: a constant weight
    # layout prepared once per model, outside the timed region.
    W2T = dsp.transpose_w2(W2) if T > 0 else None
    # the draft uses the copy at every temperature (it holds W2 on chip from it)
    W2T_d = dsp.transpose_w2(W2) if (W2T is None and wl.wdtype == "bf16") else W2T
    if args.per_position:
        W2T_d = None

    ws_d = torch.empty(dsp.workspace_size(dsp.OP_DRAFT, B, gamma, V, r), dtype=torch.uint8, device=dev)
    ws_v = torch.empty(dsp.workspace_size(dsp.OP_VERIFY, B, gamma, V, r), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(dsp.workspace_size(dsp.OP_SURVIVAL, B, gamma, V, r), dtype=torch.uint8, device=dev)
    dout = (torch.empty((B, gamma), dtype=torch.int32, device=dev),
            torch.empty((B, gamma), dtype=torch.float32, device=dev),
            torch.empty((B, gamma), dtype=torch.float32, device=dev))
    nsteps = args.steps
    vouts = [(torch.empty((B,), dtype=torch.int32, device=dev),
              torch.empty((B, gamma + 1), dtype=torch.int32, device=dev),
              torch.empty((B, gamma), dtype=torch.float32, device=dev)) for _ in range(max(nsteps, 1))]
    stream = torch.cuda.current_stream(dev)

    def step(i, rnd):
        dsp.markov_draft(U, W1, W2, x0, T, seeds, rnd, out=dout, workspace=ws_d, stream=stream, W2T=W2T_d)
        dsp.verify(U, W1, W2, x0, dout[0], dout[1], tgt, T, seeds, rnd, out=vouts[i % len(vouts)], W2T=W2T,
                   workspace=ws_v, stream=stream)

    if args.copy_probe_mb > 0:
        src = torch.ones(args.copy_probe_mb << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Every step runs after a write of flush_mb MiB that evicts the 256 MB
    # memory-side cache, as the target model's forward pass does between
    # rounds in real use; the write is outside the step's timed interval (HIP
    # events on the launch stream around the step alone).
    scratch = torch.empty(args.flush_mb << 18, dtype=torch.float32, device=dev) if args.flush_mb > 0 else None

    def run_steps(n, rnd0):
        ev = []
        for i in range(n):
            if scratch is not None:
                scratch.fill_(float(i))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step(i, rnd0 + i)
            e1.record(stream)
            ev.append((e0, e1))
        return ev

    log("warmup %d steps" % args.warmup)
    run_steps(args.warmup, 0)
    torch.cuda.synchronize()

    log("timing %d steps" % nsteps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    events = run_steps(nsteps, 1000)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    times = np.array([a.elapsed_time(b) for a, b in events])
    med = float(np.median(times))

    # The same steps again with a HIP event pair around every kernel launch
    # (recorded by the library on the launch stream) for the per-kernel
    # durations.
    log("timing %d steps with per-kernel events" % nsteps)
    dsp.profile_enable(True)
    torch.cuda.synchronize()
    p0 = time.perf_counter()
    run_steps(nsteps, 1000)
    torch.cuda.synchronize()
    p1 = time.perf_counter()
    prof = dsp.profile_read()
    dsp.profile_enable(False)

    # Back to back without the cache-evicting writes (warm memory-side cache).
    warm = None
    if args.warm_steps > 0:
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for i in range(args.warm_steps):
            step(i, 1000 + i)
        torch.cuda.synchronize()
        wms = (time.perf_counter() - w0) / args.warm_steps * 1e3
        warm = {"ms_per_step": wms, "value": B * gamma / (wms * 1e-3), "steps": args.warm_steps}
    del scratch

    lens = np.stack([vouts[i][0].cpu().numpy() for i in range(nsteps)])
    bytes_steps = [step_bytes(B, gamma, V, r, lens[i]) for i in range(nsteps)]
    mean_bytes = float(np.mean(bytes_steps))
    hbm_frac = mean_bytes / (med * 1e-3) / HBM_PEAK
    # tokens a round emits over all requests: the accepted draft tokens plus
    # each request's correction or bonus token
    emitted = float((lens + 1).sum(axis=1).mean()) / (med * 1e-3)

    # dominant kernel: the device-resident draft (one launch per step) when it
    # runs, else the per-position draft tile pass (sample mode at T > 0,
    # argmax mode at T = 0)
    if "draft_resident" in prof:
        kname = "draft_resident"
        k_bytes = resident_draft_bytes(B, gamma, V, r)
    else:
        kname = "tile_pass_sample" if T > 0 else "tile_pass_greedy"
        k_bytes = tile_pass_bytes(B, gamma, V, r)
    launches, kms = prof.get(kname, (0, 0.0))
    k_avg_s = kms / max(launches, 1) / 1e3
    achieved = k_bytes / k_avg_s if k_avg_s > 0 else 0.0
    traffic = pmc_traffic(kname, args.workload)
    roofline = {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": achieved / HBM_PEAK, "traffic": traffic, "kernel": kname,
                "avg_launch_us": k_avg_s * 1e6, "bytes_per_launch": k_bytes,
                "traffic_over_bytes": (traffic / k_bytes) if traffic else None}
    if kname != "draft_resident":
        roofline["bytes_per_launch_w2_every_launch"] = k_bytes + 2 * r * V * (1 - 1 / gamma)
    kernels = {k: {"launches": n, "avg_us": ms / n * 1e3, "ms_per_step": ms / nsteps} for k, (n, ms) in prof.items()}

    # survival (analytical), timed beside the gated path
    surv_ms = None
    if args.survival_steps > 0:
        cst = torch.empty((B, gamma), dtype=torch.float32, device=dev)
        sv = torch.empty((B, gamma), dtype=torch.float32, device=dev)
        dsp.markov_draft(U, W1, W2, x0, T, seeds, 1000, out=dout, workspace=ws_d, stream=stream)
        for _ in range(2):
            dsp.survival(U, W1, W2, x0, dout[0], dout[2], tgt, T, out=(cst, sv), workspace=ws_s, stream=stream)
        torch.cuda.synchronize()
        s0 = time.perf_counter()
        for _ in range(args.survival_steps):
            dsp.survival(U, W1, W2, x0, dout[0], dout[2], tgt, T, out=(cst, sv), workspace=ws_s, stream=stream)
        torch.cuda.synchronize()
        surv_ms = (time.perf_counter() - s0) / args.survival_steps * 1e3

    # The scheduled round of the pages' production flow, reported beside the
    # gated path: the draft with its fused confidence head (Eq. 7, synthetic
    # hidden states of width 4096 and per-position temperatures), survival
    # products of the confidences, prefix scheduler with a synthetic profiled
    # throughput table, verification at the scheduled lengths.  The same
    # drafted round is also verified whole for comparison.
    sched = None
    if args.schedule_steps > 0:
        d_hidden = 4096
        h_np, w_np, sts_np = workloads.confidence_inputs(B, gamma, d_hidden, r)
        hd, wd_, stsd = (torch.from_numpy(h_np).to(dev), torch.from_numpy(w_np).to(dev),
                         torch.from_numpy(sts_np).to(dev))
        conf = torch.empty((B, gamma), dtype=torch.float32, device=dev)
        sv = torch.empty((B, gamma), dtype=torch.float32, device=dev)
        half, power = 4.0 * B, 2.0
        sps = torch.from_numpy(workloads.sps_curve(B * (gamma + 1), half, power)).to(dev)
        lengths = torch.empty((B,), dtype=torch.int32, device=dev)
        theta = torch.empty((1,), dtype=torch.float64, device=dev)
        vo = vouts[0]

        head = (hd, wd_, stsd)
        dcout = (dout[0], dout[1], dout[2], conf)

        def draft_conf(rnd):
            dsp.markov_draft(U, W1, W2, x0, T, seeds, rnd, out=dcout, workspace=ws_d, stream=stream, W2T=W2T_d,
                             conf_head=head)

        def plan():
            dsp.survival(None, None, None, None, None, None, None, T, conf=conf, out=(None, sv), stream=stream)
            dsp.schedule(sv, sps, out=(lengths, theta), stream=stream)

        def verify_at(lens_arg, rnd):
            dsp.verify(U, W1, W2, x0, dout[0], dout[1], tgt, T, seeds, rnd, out=vo, W2T=W2T, workspace=ws_v,
                       stream=stream, lengths=lens_arg)

        def timed(fn):
            fn(0)
            torch.cuda.synchronize()
            t = time.perf_counter()
            for i in range(args.schedule_steps):
                fn(i)
            torch.cuda.synchronize()
            return (time.perf_counter() - t) / args.schedule_steps * 1e3

        # the same per-position launches with and without the confidence head
        # (a draft that returns confidences does not take the resident loop)
        draft_ms = timed(lambda i: dsp.markov_draft(U, W1, W2, x0, T, seeds, 2000, out=dout, workspace=ws_d,
                                                    stream=stream))
        draft_conf_ms = timed(lambda i: draft_conf(2000))
        plan_ms = timed(lambda i: plan())
        full_ms = timed(lambda i: verify_at(None, 2000))
        full_len = vo[0].cpu().numpy()
        sch_ms = timed(lambda i: verify_at(lengths, 2000))
        sch_len = vo[0].cpu().numpy()

        def round_scheduled(i):
            draft_conf(3000 + i)
            plan()
            verify_at(lengths, 3000 + i)

        round_ms = timed(round_scheduled)
        lens_h = lengths.cpu().numpy()
        sched = {"flow": "draft with the fused confidence head (d=%d, STS), survival of the confidences, "
                         "schedule, verify at the scheduled lengths" % d_hidden,
                 "draft_ms": draft_ms, "draft_with_confidence_ms": draft_conf_ms,
                 "sps": "1/(1+(n/%g)^%g), n = verified tokens" % (half, power),
                 "plan_ms": plan_ms, "mean_length": float(lens_h.mean()),
                 "theta_best": float(theta.cpu().numpy()[0]),
                 "verify_full_ms": full_ms, "verify_scheduled_ms": sch_ms,
                 "mean_accept_len_full": float(full_len.mean()), "mean_accept_len_scheduled": float(sch_len.mean()),
                 "round_scheduled_ms": round_ms}

    # Block sampling with the RNN head (Eq. 6) at the same sizes, timed beside
    # the Markov draft: synthetic cell projection and hidden-state part.
    rnn = None
    if args.rnn_steps > 0 and wl.wdtype == "bf16":
        Wp_np, hp_np = workloads.rnn_inputs(B, gamma, r)
        Wp_d, hp_d = torch.from_numpy(Wp_np).to(dev), torch.from_numpy(hp_np).to(dev)
        ws_r = torch.empty(dsp.workspace_size(dsp.OP_RNN_DRAFT, B, gamma, V, r), dtype=torch.uint8, device=dev)
        rout = dout + (None,)

        def rnn_step(i):
            dsp.rnn_draft(U, W1, W2, Wp_d, hp_d, x0, T, seeds, 4000 + i, out=rout, workspace=ws_r, stream=stream)

        def markov_step(i):
            dsp.markov_draft(U, W1, W2, x0, T, seeds, 4000 + i, out=dout, workspace=ws_d, stream=stream, W2T=W2T_d)

        def per_call_ms(fn):
            fn(0)
            torch.cuda.synchronize()
            t = time.perf_counter()
            for i in range(args.rnn_steps):
                fn(i)
            torch.cuda.synchronize()
            return (time.perf_counter() - t) / args.rnn_steps * 1e3

        rnn_ms = per_call_ms(rnn_step)
        markov_ms = per_call_ms(markov_step)
        dsp.profile_enable(True)
        for i in range(args.rnn_steps):
            rnn_step(i)
        torch.cuda.synchronize()
        rprof = dsp.profile_read()
        dsp.profile_enable(False)
        rnn = {"draft_ms": rnn_ms, "markov_draft_ms": markov_ms,
               "positions_per_s": B * gamma / (rnn_ms * 1e-3),
               "kernels": {k: {"launches": n, "avg_us": ms / n * 1e3, "ms_per_call": ms / args.rnn_steps}
                           for k, (n, ms) in rprof.items()}}
        del ws_r, Wp_d, hp_d

    flops = 2.0 * r * V * (B * gamma + float((lens < gamma).sum()) / nsteps)
    out = {
        "metric": METRIC,
        "value": B * gamma / (med * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": nsteps,
        "warmup": args.warmup,
        "ms_per_step": med,
        "ms_per_step_p10": float(np.percentile(times, 10)),
        "ms_per_step_p90": float(np.percentile(times, 90)),
        "timing": "median over the timed steps, each after a %d MiB cache-evicting write (HIP events on the launch "
                  "stream around the step)" % args.flush_mb,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "V": V, "r": r, "gamma": gamma, "T": T,
                   "weights": wl.wdtype, "logits": "f32",
                   "draft": "device-resident" if "draft_resident" in prof else "per-position"},
        "hbm_fraction": hbm_frac,
        "bytes_per_step": mean_bytes,
        "mfma_fraction": flops / (med * 1e-3) / MFMA_BF16_PEAK,
        "emitted_tokens_per_s": emitted,
        "mean_accept_len": float(lens.mean()),
        "roofline": roofline,
        "kernels": kernels,
        "wall_ms_per_step_with_flush": (t1 - t0) / nsteps * 1e3,
        "wall_ms_per_step_with_events": (p1 - p0) / nsteps * 1e3,
        "warm": warm,
        "survival_ms": surv_ms,
        "schedule": sched,
        "rnn_draft": rnn,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
