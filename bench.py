#!/usr/bin/env python3
"""KDA prefill + decode throughput on one MI355X.

The headline step is one ``kda_chunk_fwd`` over the 1M-token workload: one
sequence of T = 1,048,576 tokens on H = 16 heads (one GPU's head share),
K = V = 128, bf16 inputs, fp32 state, zero initial state, final state
returned, all inputs resident in HBM, in the plan the library picks.
``value`` is prefill tokens/s (B*T / step time).  The same JSON line carries,
each measured the same way in its own timed region:

* ``prefill_32k_x8``: 8 sequences of 32,768 tokens on 32 heads from a random
  fp32 initial state, 20 % of the (head, channel) gates pinned at the clamp
  floor, final state returned;
* ``prefill_8k``: one 8,192-token sequence on 32 heads (with its fused output
  gate and its backward beside it);
* ``decode``: 256 sequences x 32 heads, 512 MiB fp32 state, 64 successive
  one-token steps (and a 4-token verify).

For every prefill workload: ``roofline`` is the dominant kernel of the call
(its algorithmic bytes per launch over its average launch duration, measured
with HIP events that the library records on the launch stream,
kda_profile_start); ``roofline_call`` is the whole call against its
algorithmic bytes (1,282 B per head-token plus the states), the binding
roofline of the path; ``mfma`` is its algorithmic flops against the bf16 MFMA
peak; ``traffic`` is the counter-measured HBM bytes per launch of the dominant
kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE scaled by a plain-copy calibration,
read from profiles/<workload>_traffic.json while the kernel sources still have
the hash recorded there); ``cpu_baseline`` is the fp64 oracle on the host
cores on a bounded sample of the same workload.

Before each workload's warm-up steps its step runs untimed for --settle-ms
(an idle GPU needs about 30 ms of work to reach its steady clocks).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS]
       [--workloads prefill_1m,prefill_32k_x8,prefill_8k] [--extra]
       [--no-cpu-baseline] [--no-decode] [--no-backward] [--no-gate] [--cpu-seconds S]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
MALL_BYTES = 256 << 20         # last-level (Infinity) cache

METRIC = "KDA prefill tokens/s (MFMA % peak) + decode tokens/s (HBM GB/s %)"
PREFILL_WORKLOADS = ("prefill_1m", "prefill_32k_x8", "prefill_8k")

# launches that write o (and read S0 / write S_T): the path's algorithmic
# bytes are attributed to them; the two-pass plan's intra-chunk pass gets the
# input reads; a segmented fused call splits them: its first launch runs
# segment 0 with output (all of that segment's bytes) beside the summaries of
# segments 1 .. n_seg - 2 (k, g, v and beta read, two states written per
# segment), its output launch the other segments; the two-pass summaries
# (which read the intra-chunk workspace), scans and copies are plan overhead
# (zero)
OUTPUT_LAUNCHES = ("chunk_output", "state_output", "fused_output", "token_fwd")


def prefill_bytes(B, T, H, K, V, in_bytes=2, s0=False, final=True):
    """Algorithmic HBM bytes of one prefill call: q, k, g (K each), v, beta
    and o per head-token, plus the initial / final state per (b, h)."""
    per_ht = in_bytes * (3 * K + V + 1) + in_bytes * V
    return B * T * H * per_ht + B * H * K * V * 4 * (int(s0) + int(final))


def prefill_flops(B, T, H, K, V, C=64):
    """Algorithmic flops per head-token of the chunk form at C = 64 with the
    triangular products counted as half: C (3K + 2V) + 6 K V."""
    return B * T * H * (C * (3 * K + 2 * V) + 6 * K * V)


def decode_bytes(N, H, K, V, in_bytes=2):
    """Per step: state read + write (8 K V) and the token vectors."""
    return N * H * (8 * K * V + in_bytes * (3 * K + V + 1) + in_bytes * V)


def fused_segments(n_chunks, n_seg):
    """(chunks of segment 0, chunks of each later segment) of a segmented
    fused call: the library's split, segment 0 about 3.5 % shorter than the
    others when that leaves the last segment non-empty."""
    cps = (n_chunks + n_seg - 1) // n_seg
    if n_seg <= 1:
        return cps, cps
    d = (cps * 35 + 500) // 1000
    c0 = cps - d
    if d > 0 and c0 >= 1:
        rest = (n_chunks - c0 + n_seg - 2) // (n_seg - 1)
        if c0 + (n_seg - 2) * rest < n_chunks:
            return c0, rest
    return cps, cps


def kernel_bytes(name, B, T, H, K, V, in_bytes, s0, final, two_pass, n_seg=1):
    """Algorithmic bytes of one launch named `name` (see OUTPUT_LAUNCHES)."""
    ht = B * T * H
    states = B * H * K * V * 4 * (int(s0) + int(final))
    reads = ht * in_bytes * (3 * K + V + 1)
    writes = ht * in_bytes * V
    if name == "intra_chunk":
        return reads
    n_chunks = (T + 63) // 64
    cps0, cps = fused_segments(n_chunks, n_seg)
    t0 = min(cps0 * 64, T)                                # tokens of segment 0
    per_tok = in_bytes * (3 * K + V + 1) + in_bytes * V
    if name == "fused_output" and n_seg > 1:
        return B * (T - t0) * H * per_tok + B * H * K * V * 4 * int(final)
    if name in OUTPUT_LAUNCHES:
        return writes + states + (0 if two_pass else reads)
    if name == "fused_summary" and n_seg > 1:
        covered = min((cps0 + (n_seg - 2) * cps) * 64, T) - t0   # tokens of the summarised segments
        return (B * t0 * H * per_tok + B * H * K * V * 4 * int(s0) +
                B * covered * H * in_bytes * (2 * K + V + 1) + 2 * B * H * (n_seg - 1) * K * V * 4)
    return 0


def recorded_traffic(workload, kernel, plan):
    """Counter-derived HBM bytes per launch of `kernel` in `workload`, if the
    committed record was taken on the current kernel sources and plan."""
    path = os.path.join(PROFILES, "%s_traffic.json" % workload)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, "no counter record for this workload"
    from gated_delta_rule_66_amd.traffic import kernel_source_hash
    if rec.get("source_sha256") != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    if list(rec.get("plan", [])) != list(plan):
        return None, "plan differs from the one profiled"
    k = rec.get("kernels", {}).get(kernel)
    if not k:
        return None, "kernel not in the counter record"
    return k["hbm_bytes_per_launch"], rec.get("note", "")


def host_cpu():
    """Model name and core counts of the host (the oracle's machine)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"model": model, "cpu_count": os.cpu_count(), "affinity_cpus": affinity}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-passes", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="untimed run of each step before its warm-up steps, so that the GPU has left its "
                         "idle clock state (the first ~30 ms of work run up to 10%% slower)")
    ap.add_argument("--workloads", default=",".join(PREFILL_WORKLOADS),
                    help="prefill workloads to time, the first being the headline")
    ap.add_argument("--extra", action="store_true", help="also time a packed variable-length batch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-gate", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="target duration of each workload's oracle sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run only a plain device copy of this size (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: measures one GPU only; --gpus %d is not supported "
              "(heads and batch rows would shard across GPUs without communication)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    workloads = [w for w in args.workloads.split(",") if w]
    for w in workloads:
        if w not in PREFILL_WORKLOADS:
            print("bench.py: unknown workload %s" % w, file=sys.stderr)
            sys.exit(2)

    import torch
    import gated_delta_rule_66_amd as kda
    from gated_delta_rule_66_amd.inputs import CONFIGS, make_decode_config, make_prefill_config

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": 5}))
        return

    kda.load_library()   # fails loudly if the HIP library is missing
    stream = torch.cuda.current_stream(dev)

    def settle(fn, ms):
        """Run fn untimed for about ms milliseconds of GPU work."""
        if ms <= 0:
            return
        fn()
        torch.cuda.synchronize()
        t = time.time()
        fn()
        torch.cuda.synchronize()
        one = max(time.time() - t, 1e-5)
        for _ in range(int(ms * 1e-3 / one) + 1):
            fn()
        torch.cuda.synchronize()

    def time_calls(fn, warmup, steps):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps   # ms per call

    def time_launches(fn, steps):
        """Per-kernel average duration (ms) and launch count per call, from
        the events the library records around each launch."""
        torch.cuda.synchronize()
        kda.profile_start(64 * steps + 64)
        for _ in range(steps):
            fn()
        rec = kda.profile_stop(64 * steps + 64)
        per = {}
        for name, ms in rec:
            per.setdefault(name, []).append(ms)
        return {n: {"avg_ms": sum(v) / len(v), "launches_per_call": len(v) / steps} for n, v in per.items()}

    def describe(c):
        return "KDA prefill B=%d T=%d H=%d K=V=%d bf16 in, fp32 state, %s, final state out%s" % (
            c.B, c.T, c.H, c.K, "S0~N(0,0.02)" if c.s0_std is not None else "S0=0",
            ", %d%% of (head, channel) gates pinned at the floor" % round(100 * c.pinned_frac)
            if c.pinned_frac else "")

    # ------------------------------------------------------------ prefill workloads
    def bench_prefill(name):
        c = CONFIGS[name]
        x = make_prefill_config(c, dev)
        B, T, H, K, V = c.B, c.T, c.H, c.K, c.V
        plan = kda.chunk_plan(B, T, H, K, V, c.dtype)
        o = torch.empty((B, T, H, V), dtype=c.dtype, device=dev)
        sT = torch.empty((B, H, K, V), dtype=torch.float32, device=dev)
        ws_n = kda.chunk_workspace_size(B, T, H, K, V, c.dtype)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

        def step():
            kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], True, None,
                          out=o, final_state=sT, workspace=ws)

        settle(step, args.settle_ms)
        ms = time_calls(step, args.warmup, args.steps)
        kernels = time_launches(step, args.steps)
        has_s0 = c.s0_std is not None
        nbytes = prefill_bytes(B, T, H, K, V, 2, s0=has_s0, final=True)
        nflops = prefill_flops(B, T, H, K, V)
        gbs = nbytes / (ms * 1e-3) / 1e9
        tflops = nflops / (ms * 1e-3) / 1e12
        dom = max(kernels, key=lambda n: kernels[n]["avg_ms"] * kernels[n]["launches_per_call"])
        dom_ms = kernels[dom]["avg_ms"]
        dom_bytes = kernel_bytes(dom, B, T, H, K, V, 2, has_s0, True, plan[2] == 2, plan[0])
        dom_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9
        traffic, traffic_note = recorded_traffic(name, dom, plan)
        working_set = nbytes + ws_n
        res = {
            "workload": describe(c),
            "global_batch": B, "seq_len": T, "heads": H,
            "plan": {"n_seg": plan[0], "v_block": plan[1], "split": plan[2]},
            "ms": ms,
            "tokens_per_s": B * T / (ms * 1e-3),
            "head_tokens_per_s": B * T * H / (ms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": dom_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dom_gbs / HBM_PEAK_GBS, "traffic": traffic,
                         "kernel": dom, "kernel_avg_ms": dom_ms,
                         "algorithmic_bytes_per_launch": dom_bytes, "traffic_note": traffic_note},
            "roofline_call": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_call": nbytes},
            "mfma": {"achieved_tflops": tflops, "peak_tflops": BF16_PEAK_TFLOPS,
                     "frac": tflops / BF16_PEAK_TFLOPS, "algorithmic_flops_per_call": nflops},
            "kernels": kernels,
            "workspace_bytes": ws_n,
            "cache_note": ("inputs, outputs and workspace (%.0f MB) partly fit the 256 MB last-level cache; "
                           "it is not flushed between repetitions" % (working_set / 1e6))
            if working_set < 2 * MALL_BYTES else
            "working set %.1f GB, far above the 256 MB last-level cache" % (working_set / 1e9),
        }
        extras = {}
        if name == "prefill_8k" and not args.no_gate:
            # the same call with the output gate fused into the store of o, beside
            # the ungated call followed by a separate elementwise o * sigmoid(gate)
            gen = torch.Generator(device=dev)
            gen.manual_seed(11)
            z = torch.randn((B, T, H, V), generator=gen, device=dev).to(c.dtype)

            def gated_step():
                kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], True, tuple(plan),
                              out=o, final_state=sT, workspace=ws, gate=z)

            def unfused_step():
                step()
                o.mul_(torch.sigmoid(z))

            settle(gated_step, args.settle_ms)
            ms_gated = time_calls(gated_step, 2, args.steps)
            ms_plain = time_calls(step, 2, args.steps)
            ms_unfused = time_calls(unfused_step, 2, args.steps)
            extras["gate"] = {"ms": ms_gated, "tokens_per_s": B * T / (ms_gated * 1e-3), "ms_ungated": ms_plain,
                              "ms_unfused": ms_unfused}
            del z
        del x, o, sT, ws
        torch.cuda.empty_cache()
        if name == "prefill_8k" and not args.no_backward:
            xb = make_prefill_config(c, dev)
            gen = torch.Generator(device=dev)
            gen.manual_seed(12)
            d_o = torch.randn((B, T, H, V), generator=gen, device=dev).to(c.dtype)
            ws_b = torch.empty(max(kda.chunk_bwd_workspace_size(B, T, H, K, V, c.dtype), 1), dtype=torch.uint8,
                               device=dev)

            def bwd_step():
                kda.chunk_bwd(xb["q"], xb["k"], xb["v"], xb["g"], xb["beta"], xb["s0"], d_o, None, workspace=ws_b)

            settle(bwd_step, args.settle_ms)
            ms_b = time_calls(bwd_step, 1, 3)
            # algorithmic bytes: the forward's inputs and dL/do read, the five gradients written
            b_bytes = B * T * H * 2 * (2 * (3 * K + V + 1) + V)
            extras["backward"] = {
                "workload": "gradients of the 8K prefill (dq, dk, dv, dg, dbeta; zero S0, no dL/dS_T)",
                "ms": ms_b, "tokens_per_s": B * T / (ms_b * 1e-3),
                "achieved_gbs": b_bytes / (ms_b * 1e-3) / 1e9,
                "hbm_frac": b_bytes / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "kernels": time_launches(bwd_step, 2),
                "workspace_bytes": ws_b.numel()}
            del xb, d_o, ws_b
            torch.cuda.empty_cache()
        res.update(extras)
        return res

    # ------------------------------------------------------------ CPU oracle baseline
    def cpu_baseline(name):
        """The fp64 oracle on the host cores, on a bounded sample of the
        workload: the first Ts tokens of batch row 0, all H heads, drawn by the
        same recipe (its cost is linear in tokens x heads and independent of
        the values), repeated to about --cpu-seconds; tokens/s of the whole
        workload = Ts * reps / wall time."""
        import oracle
        c = CONFIGS[name]
        nthreads = oracle.oracle_max_threads()

        def sample(ts):
            xs = make_prefill_config(c, dev, T=ts, B=1)
            inp = [xs[n].cpu() for n in ("q", "k", "v", "g", "beta")]
            return inp, (xs["s0"].cpu() if xs["s0"] is not None else None)

        def run(inp, s0, reps):
            t0 = time.perf_counter()
            for _ in range(reps):
                oracle.oracle_fwd(*inp, s0, want_state=False, nthreads=nthreads)
            return time.perf_counter() - t0

        # at most about a million head-tokens per sample (host memory), at
        # least enough for every thread to hold a (head, 16-column) chain
        ts = min(c.T, max(64, (1 << 20) // c.H // 64 * 64))
        inp, s0 = sample(min(ts, 1024))
        t_small = run(inp, s0, 1) / min(ts, 1024)
        reps = max(1, int(round(args.cpu_seconds / max(t_small * ts, 1e-9))))
        inp, s0 = sample(ts)
        dt = run(inp, s0, reps)
        chains = c.H * (c.V // 16)
        return {
            "value": ts * reps / dt,
            "unit": "tokens/s",
            "cores": min(nthreads, chains),
            "kind": "oracle",
            "sample": "fp64 token-by-token oracle (C, OpenMP, %d threads over %d (head, 16-column) chains) on "
                      "the first %d tokens of one sequence, all %d heads, drawn by the workload's recipe, run "
                      "%d time(s): %.1f s wall; its cost is linear in tokens x heads, so tokens/s of the whole "
                      "workload = %d x %d / wall" % (min(nthreads, chains), chains, ts, c.H, reps, dt, ts, reps),
            "host": host_cpu(),
        }

    def progress(msg):
        print("[bench] " + msg, file=sys.stderr, flush=True)

    results = {}
    for w in workloads:
        progress("%s: timing" % w)
        results[w] = bench_prefill(w)
        progress("%s: %.4f ms per call, plan %s" % (w, results[w]["ms"], results[w]["plan"]))
        if not args.no_cpu_baseline:
            results[w]["cpu_baseline"] = cpu_baseline(w)
            progress("%s: oracle %.0f tokens/s" % (w, results[w]["cpu_baseline"]["value"]))

    # ------------------------------------------------------------ decode workload
    dec = None
    if not args.no_decode:
        progress("decode_256x32: timing")
        dcfg = CONFIGS["decode_256x32"]
        d = make_decode_config(dcfg, dev)
        pristine = d["state"]
        state = pristine.clone()
        od = torch.empty((dcfg.N, dcfg.H, dcfg.V), dtype=dcfg.dtype, device=dev)

        def decode_pass():
            for t in range(dcfg.steps):
                kda.recurrent_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t], state, out=od)

        settle(decode_pass, args.settle_ms)
        state.copy_(pristine)
        ms_pass = time_calls(decode_pass, 1, args.decode_passes)
        dk = time_launches(decode_pass, 1)["decode_step"]
        ms_step = ms_pass / dcfg.steps
        dec_bytes = decode_bytes(dcfg.N, dcfg.H, dcfg.K, dcfg.V)
        dec_gbs = dec_bytes / (ms_step * 1e-3) / 1e9
        dec = {"workload": "256 seq x 32 heads, K=V=128, fp32 state 512 MiB, 64 steps, bf16 tokens",
               "tokens_per_s": dcfg.N / (ms_step * 1e-3), "ms_per_step": ms_step, "achieved_gbs": dec_gbs,
               "hbm_frac": dec_gbs / HBM_PEAK_GBS, "bytes_per_step": dec_bytes,
               "kernel_avg_ms": dk["avg_ms"],
               "kernel_gbs": dec_bytes / (dk["avg_ms"] * 1e-3) / 1e9}
        dec_traffic, dec_note = recorded_traffic("decode_256x32", "decode_step", [0, 0, 0])
        dec["traffic"] = dec_traffic
        dec["traffic_gbs"] = None if dec_traffic is None else dec_traffic / (dk["avg_ms"] * 1e-3) / 1e9
        if dec_traffic is None:
            dec["traffic_note"] = dec_note
        # multi-token verification: the first 4 tokens of every sequence in one
        # call, state read and written once, against 4 single steps
        TV = 4
        tok = lambda t: t[:TV].transpose(0, 1).contiguous()
        dv = {n: tok(d[n]) for n in ("q", "k", "v", "g", "beta")}
        ov = torch.empty((dcfg.N, TV, dcfg.H, dcfg.V), dtype=dcfg.dtype, device=dev)
        state.copy_(pristine)
        ms_verify = time_calls(lambda: kda.recurrent_steps(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], state,
                                                           out=ov), 2, 10)
        verify_bytes = decode_bytes(dcfg.N, dcfg.H, dcfg.K, dcfg.V) + \
            (TV - 1) * (dec_bytes - 8 * dcfg.N * dcfg.H * dcfg.K * dcfg.V)
        dec["verify"] = {"tokens_per_sequence": TV, "ms": ms_verify,
                         "tokens_per_s": dcfg.N * TV / (ms_verify * 1e-3),
                         "achieved_gbs": verify_bytes / (ms_verify * 1e-3) / 1e9,
                         "speedup_vs_single_steps": TV * ms_step / ms_verify}
        del d, pristine, state, od, dv, ov
        torch.cuda.empty_cache()

    extra = {}
    if args.extra:
        # packed variable-length batch: 256 sequences of lengths drawn
        # uniformly from [1, 2048], 32 heads, K = V = 128, per-sequence states
        gen = torch.Generator().manual_seed(7)
        lengths = torch.randint(1, 2049, (256,), generator=gen)
        cu = torch.zeros(257, dtype=torch.int32)
        cu[1:] = torch.cumsum(lengths, 0).to(torch.int32)
        Tt, Hv = int(cu[-1]), 32
        xv = make_prefill_config(CONFIGS["prefill_8k"], dev, T=Tt, B=1, H=Hv)
        sq = lambda t: t[0]
        s0v = torch.zeros((256, Hv, 128, 128), dtype=torch.float32, device=dev)
        ov = torch.empty((Tt, Hv, 128), dtype=torch.bfloat16, device=dev)
        sv = torch.empty_like(s0v)
        wsv = torch.empty(kda.chunk_fwd_varlen_workspace_size(256, Tt, Hv, 128, 128, torch.bfloat16),
                          dtype=torch.uint8, device=dev)
        cud = cu.to(dev)
        fnv = lambda: kda.chunk_fwd_varlen(sq(xv["q"]), sq(xv["k"]), sq(xv["v"]), sq(xv["g"]), sq(xv["beta"]),
                                           cud, s0v, out=ov, final_state=sv, workspace=wsv)
        msv = time_calls(fnv, 2, 5)
        nbv = prefill_bytes(1, Tt, Hv, 128, 128, 2, s0=True, final=True) + 256 * Hv * 128 * 128 * 8 - \
            Hv * 128 * 128 * 8
        extra["varlen"] = {
            "workload": "packed batch of 256 sequences, lengths U[1, 2048] (%d tokens), H=32, K=V=128 bf16, "
                        "per-sequence initial and final states" % Tt,
            "ms": round(msv, 4),
            "tokens_per_s": Tt / (msv * 1e-3),
            "hbm_frac": nbv / (msv * 1e-3) / 1e9 / HBM_PEAK_GBS,
        }
        del xv, s0v, ov, sv, wsv
        torch.cuda.empty_cache()

    head = results[workloads[0]]
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: %s" % (workloads[0], head["workload"]),
                   "global_batch": head["global_batch"], "seq_len": head["seq_len"], "heads": head["heads"],
                   "plan": head["plan"], "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "roofline_call": head["roofline_call"],
        "mfma": head["mfma"],
        "kernels": head["kernels"],
        "cpu_baseline": head.get("cpu_baseline"),
    }
    for key in ("gate", "backward"):
        if key in head:
            line[key] = head[key]
    for w in workloads[1:]:
        line[w] = results[w]
    line["decode"] = dec
    if extra:
        line["extra"] = extra
    print(json.dumps(line))


if __name__ == "__main__":
    main()
