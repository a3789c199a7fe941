#!/usr/bin/env python3
"""KDA prefill + decode throughput on one MI355X.

A step is one ``kda_chunk_fwd`` over the 8K-token workload (B=1, H=32,
T=8192, K=V=128, bf16 inputs, fp32 state, zero initial state, final state
returned), with all inputs resident in HBM.  ``value`` is prefill tokens/s
(B*T / step time).  Before its W warm-up steps the step runs untimed for
--settle-ms (50 ms): an idle GPU needs about 30 ms of work to reach its
steady clocks, and the first calls run up to 10 % slower.  The same line carries the decode workload (256
sequences x 32 heads, 512 MiB fp32 state, 64 successive one-token steps), the
roofline of the dominant launch, and the fp64 CPU oracle timed on a bounded
sample of the prefill workload.

The roofline object describes the dominant kernel of the prefill step: its
algorithmic bytes per launch (1,282 B per head-token it processes plus the
states it must read or write) over its average duration, measured with HIP
events that the library records on the launch stream (kda_profile_start).
``traffic`` is the HBM traffic per launch from rocprofv3 FETCH_SIZE and
WRITE_SIZE counters, scaled by a plain-copy calibration; it is read from
profiles/prefill_8k_traffic.json and reported only while the kernel
source still has the hash recorded there.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS] [--extra]
       [--no-cpu-baseline] [--no-decode] [--no-backward] [--cpu-seconds S]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_8k_traffic.json")

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA

METRIC = "KDA prefill tokens/s (MFMA % peak) + decode tokens/s (HBM GB/s %)"


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


def recorded_traffic(kernel, plan):
    """Counter-derived HBM bytes per launch of `kernel`, if the committed
    measurement was taken on the current kernel sources and plan."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, "no counter record"
    from gated_delta_rule_66_amd.traffic import kernel_source_hash
    if rec.get("source_sha256") != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    if list(rec.get("plan", [])) != list(plan):
        return None, "plan differs from the one profiled"
    k = rec.get("kernels", {}).get(kernel)
    if not k:
        return None, "kernel not in the counter record"
    return k["hbm_bytes_per_launch"], rec.get("note", "")


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-passes", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="untimed run of the prefill step before its warm-up steps, so that the GPU "
                         "has left its idle clock state (the first ~30 ms of work run up to 10%% slower)")
    ap.add_argument("--extra", action="store_true", help="also time the 32K x 256-chain and 1M-token workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the oracle sample (heads of the 8K workload)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run only a plain device copy of this size (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: measures one GPU only; --gpus %d is not supported "
              "(heads and batch rows would shard across GPUs without communication)" % args.gpus,
              file=sys.stderr)
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

    # ------------------------------------------------------------ prefill, 8K workload
    cfg = CONFIGS["prefill_8k"]
    x = make_prefill_config(cfg, dev)
    B, T, H, K, V = cfg.B, cfg.T, cfg.H, cfg.K, cfg.V
    plan = kda.chunk_plan(B, T, H, K, V, cfg.dtype)
    o = torch.empty((B, T, H, V), dtype=cfg.dtype, device=dev)
    sT = torch.empty((B, H, K, V), dtype=torch.float32, device=dev)
    ws_n = kda.chunk_workspace_size(B, T, H, K, V, cfg.dtype)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

    def prefill_step():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], True, None,
                      out=o, final_state=sT, workspace=ws)

    settle(prefill_step, args.settle_ms)
    ms = time_calls(prefill_step, args.warmup, args.steps)
    kernels = time_launches(prefill_step, args.steps)
    tok_s = B * T / (ms * 1e-3)
    nbytes = prefill_bytes(B, T, H, K, V, 2, s0=False, final=True)
    nflops = prefill_flops(B, T, H, K, V)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tflops = nflops / (ms * 1e-3) / 1e12

    # algorithmic bytes per launch of each kernel: the path's 1,282 B per
    # head-token (q, k, g, v, beta in; o out) plus the states, attributed to
    # the kernel that moves them; workspace traffic (segment summaries, the
    # per-chunk records of the two-pass plan) is overhead and counts zero
    in_bytes = B * T * H * 2 * (3 * K + V + 1)
    out_bytes = B * T * H * 2 * V + B * H * K * V * 4
    per_kernel_bytes = {
        "chunk_output": nbytes, "chunk_summary": 0, "segment_scan": 0, "copy_state": 0,
        "intra_chunk": in_bytes, "state_output": out_bytes, "state_summary": 0,
    }
    dom = max(kernels, key=lambda n: kernels[n]["avg_ms"] * kernels[n]["launches_per_call"])
    dom_ms = kernels[dom]["avg_ms"]
    dom_bytes = per_kernel_bytes.get(dom, 0)
    dom_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic, traffic_note = recorded_traffic(dom, plan)

    # the same call with the output gate fused into the store of o, beside the
    # ungated call followed by a separate elementwise o * sigmoid(gate)
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    z = torch.randn((B, T, H, V), generator=gen, device=dev).to(cfg.dtype)

    def gated_step():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], True, None,
                      out=o, final_state=sT, workspace=ws, gate=z)

    def unfused_step():
        prefill_step()
        o.mul_(torch.sigmoid(z))

    # the three variants back to back, after a settle run, in the same conditions
    settle(gated_step, args.settle_ms)
    ms_gated = time_calls(gated_step, 2, args.steps)
    ms_plain = time_calls(prefill_step, 2, args.steps)
    ms_unfused = time_calls(unfused_step, 2, args.steps)
    gate = {"ms": ms_gated, "tokens_per_s": B * T / (ms_gated * 1e-3), "ms_ungated": ms_plain,
            "ms_unfused": ms_unfused}
    del x, o, sT, ws, z
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ backward, 8K workload
    bwd = None
    if not args.no_backward:
        x = make_prefill_config(cfg, dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(12)
        d_o = torch.randn((B, T, H, V), generator=gen, device=dev).to(cfg.dtype)
        ws_b = torch.empty(max(kda.chunk_bwd_workspace_size(B, T, H, K, V, cfg.dtype), 1), dtype=torch.uint8,
                           device=dev)

        def bwd_step():
            kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], d_o, None, workspace=ws_b)

        settle(bwd_step, args.settle_ms)
        ms_b = time_calls(bwd_step, 1, 3)
        # algorithmic bytes: the forward's inputs and dL/do read, the five gradients written
        b_bytes = B * T * H * 2 * (2 * (3 * K + V + 1) + V)
        bwd = {"workload": "gradients of the 8K prefill (dq, dk, dv, dg, dbeta; zero S0, no dL/dS_T)",
               "ms": ms_b, "tokens_per_s": B * T / (ms_b * 1e-3),
               "achieved_gbs": b_bytes / (ms_b * 1e-3) / 1e9,
               "hbm_frac": b_bytes / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS,
               "workspace_bytes": ws_b.numel()}
        del x, d_o, ws_b
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ decode workload
    dec = None
    if not args.no_decode:
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
        # HBM bytes per decode launch from the same counter record as the
        # prefill's (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None
        dec_traffic, dec_note = recorded_traffic("decode_step", plan)
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
        for name in ("prefill_32k_x8", "prefill_1m"):
            c = CONFIGS[name]
            xe = make_prefill_config(c, dev)
            oe = torch.empty((c.B, c.T, c.H, c.V), dtype=c.dtype, device=dev)
            se = torch.empty((c.B, c.H, c.K, c.V), dtype=torch.float32, device=dev)
            n_ws = kda.chunk_workspace_size(c.B, c.T, c.H, c.K, c.V, c.dtype)
            wse = torch.empty(max(n_ws, 1), dtype=torch.uint8, device=dev)
            fn = lambda: kda.chunk_fwd(xe["q"], xe["k"], xe["v"], xe["g"], xe["beta"], xe["s0"], True,
                                       None, out=oe, final_state=se, workspace=wse)
            mse = time_calls(fn, 2, 5)
            nb = prefill_bytes(c.B, c.T, c.H, c.K, c.V, 2, s0=c.s0_std is not None, final=True)
            nf = prefill_flops(c.B, c.T, c.H, c.K, c.V)
            extra[name] = {
                "workload": "B=%d T=%d H=%d K=V=%d bf16%s" % (c.B, c.T, c.H, c.K,
                                                             ", S0~N(0,0.02), 20%% channels at g=-5"
                                                             if c.pinned_frac else ""),
                "plan": list(kda.chunk_plan(c.B, c.T, c.H, c.K, c.V, c.dtype)),
                "ms": round(mse, 4),
                "tokens_per_s": c.B * c.T / (mse * 1e-3),
                "hbm_frac": nb / (mse * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "mfma_frac": nf / (mse * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            }
            del xe, oe, se, wse
            torch.cuda.empty_cache()
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

    # ------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nthreads = oracle.oracle_max_threads()

        def oracle_inputs(nh):
            xs = make_prefill_config(cfg, dev, H=nh)   # same recipe, first nh heads' draws
            return [xs[n].cpu() for n in ("q", "k", "v", "g", "beta")]

        def run_oracle(inp, reps):
            t0 = time.perf_counter()
            for _ in range(reps):
                oracle.oracle_fwd(*inp, None, nthreads=nthreads)
            return time.perf_counter() - t0

        # the oracle parallelises over (b, h, 16-column block) chains: size the
        # sample (heads, then repetitions of the whole workload) so that every
        # thread has chains and the run lasts about cpu_seconds
        chains1 = V // 16
        t1 = run_oracle(oracle_inputs(1), 1)
        per_chain = t1 / -(-chains1 // nthreads)
        rounds = max(1, int(args.cpu_seconds / max(per_chain, 1e-9)))
        nh = max(1, min(H, rounds * nthreads // chains1))
        inp = oracle_inputs(nh)
        t_one = run_oracle(inp, 1)
        reps = max(1, int(round(args.cpu_seconds / max(t_one, 1e-9)))) if nh == H else 1
        dt = run_oracle(inp, reps) if reps > 1 else t_one
        chains = nh * chains1
        cpu = {
            "value": B * T * nh * reps / dt / H,       # tokens/s of all H heads
            "unit": "tokens/s",
            "cores": min(nthreads, chains),
            "kind": "oracle",
            "sample": "fp64 token-by-token oracle (C, OpenMP, %d threads) on %d of %d heads of the 8K "
                      "workload (B=1, T=%d, K=V=128), run %d time(s): %.1f s wall; tokens/s scaled to "
                      "all %d heads" % (min(nthreads, chains), nh, H, T, reps, dt, H),
        }

    line = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "KDA prefill B=1 T=8192 H=32 K=V=128 bf16 in, fp32 state, S0=0, final state out",
                   "global_batch": B, "seq_len": T, "heads": H,
                   "plan": {"n_seg": plan[0], "v_block": plan[1], "split": plan[2]},
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": dom_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": dom_gbs / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "kernel": dom, "kernel_avg_ms": dom_ms,
                     "algorithmic_bytes_per_launch": dom_bytes,
                     "traffic_note": traffic_note},
        "roofline_call": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_call": nbytes},
        "mfma": {"achieved_tflops": tflops, "peak_tflops": BF16_PEAK_TFLOPS, "frac": tflops / BF16_PEAK_TFLOPS,
                 "algorithmic_flops_per_call": nflops},
        "kernels": kernels,
        "gate": gate,
        "backward": bwd,
        "decode": dec,
        "cpu_baseline": cpu,
    }
    if extra:
        line["extra"] = extra
    print(json.dumps(line))


if __name__ == "__main__":
    main()
