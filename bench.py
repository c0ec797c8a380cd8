#!/usr/bin/env python3
"""Benchmark of the SWAN hybrid-cache decode step on one MI355X.

Workload (default): batch 16, 32 query / 8 kv heads (GQA 4), d_h = 128,
context 32768 at the first step, dense buffer R = 256, k = 32 kept
coordinates, 16 consecutive decode steps.  Inputs are seeded synthetic
tensors of that shape (raw keys and queries N(0,1), values N(0,1) in the
stored basis, random orthogonal P_QK); the initial hybrid cache is built on
the GPU from a 32767-token history with swan_prefill_convert.

A timed step is the whole hot path: swan_project_append (projection and
append/evict in one launch; on a paged pool swan_project_append_paged, which
also carries the step's block-table writes and copy-on-write copies) ->
swan_decode_split -> swan_decode_reduce, all inputs already resident in HBM.
After the decode measurements the prefill conversion of the same history
(swan_prefill_convert, the step before decoding) is timed too, against the
fp64 matrix-core roofline of its double-precision key projection.
Prints one JSON line (rank 0).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_F64_PEAK_TFLOPS = 78.6  # MI355X dense fp64 matrix, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "split_kernel_traffic.json")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def cpu_baseline(w, seqs: list[int], seconds: float, max_steps: int = 4096, threads: int | None = None):
    """The float64 oracle on a sample of the workload: the chosen sequences,
    all kv heads, consecutive decode steps from the workload's first step
    until about `seconds` of stepping (prefill excluded), on `threads` host
    threads (default: all).  Returns (KV tokens/s, threads, seconds, sample
    description)."""
    import oracle
    from decode_attention_compressed_02_amd import workloads as wl

    sub = w.scaled(B=len(seqs), ctx=tuple(w.ctx[b] for b in seqs))
    oc = oracle.OracleCache.for_workload(sub, sub.n_cap() + max_steps)
    Tm = max(sub.history_len(b) for b in range(sub.B))
    K = np.zeros((sub.B, sub.H_kv, Tm, 128), np.float32)
    V = np.zeros_like(K)
    for i, b in enumerate(seqs):
        kb, vb = wl.history(w, b)
        K[i, :, :kb.shape[1]], V[i, :, :vb.shape[1]] = kb, vb
    P = wl.projection_qk(w).astype(np.float64)
    threads = threads or oracle.default_threads()
    t0 = time.time()
    oc.prefill(K, V, np.array([sub.history_len(b) for b in range(sub.B)], np.int64), P, w.rope_base, threads)
    log(f"oracle prefill of the sample in {time.time() - t0:.1f}s")
    del K, V
    tokens, secs, steps = 0, 0.0, 0
    while secs < seconds and steps < max_steps:
        q, kr, vn, pos = wl.step_inputs(w, steps)
        q, kr, vn, pos = q[seqs], kr[seqs], vn[seqs], pos[seqs].astype(np.int64)
        t = time.perf_counter()
        oc.step(q, kr, vn, pos, P, w.rope_base, threads)
        secs += time.perf_counter() - t
        tokens += int(np.sum(pos + 1))
        steps += 1
    used = min(threads, sub.B * sub.H_kv)
    desc = (f"sequences {seqs} of {w.B} (all {w.H_kv} kv heads), steps 0..{steps - 1}: "
            f"project + append/evict + decode in float64")
    return tokens / secs, used, secs, desc


def host_cpu():
    """(CPU model, hardware threads this process may run on) of the host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:
        threads = os.cpu_count() or 1
    return model, threads


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=16)
    ap.add_argument("--warmup", type=int, default=16,
                    help="untimed steps right before the timed ones (replaying the step sequence)")
    ap.add_argument("--settle-steps", type=int, default=400,
                    help="steps run back to back, timed in chunks and reported, before the warm-up of the "
                         "timed steps: the GPU's power management needs some tens of ms of sustained load "
                         "before kernels run at their steady speed (0 = no settle phase)")
    ap.add_argument("--config", type=int, default=3, help="workload number (1-5); 3 is the headline")
    ap.add_argument("--split-tokens", type=int, default=0, help="work rows per wave (0 = automatic)")
    ap.add_argument("--layers", type=int, default=1,
                    help="layers stacked along the batch (each the workload's batch, drawn from its own seed): "
                         "one launch of each kernel serves all of them")
    ap.add_argument("--values", choices=("fp16", "fp8"), default="fp16",
                    help="storage of the sparse values (fp8: E4M3, one byte each)")
    ap.add_argument("--kv-share", type=float, default=0.0,
                    help="keys keep this share of the workload's k + k coordinates and values the rest "
                         "(e.g. 0.6: TopK_R 0.6 / TopV_R 0.4 of the same budget); 0 = equal")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as HIP graph replays (one captured graph per step's inputs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=16, help="sequences in the oracle sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle stepping time of the sample")
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="split launches timed one at a time after a 1 GiB cache-evicting fill (median); 0 = skip")
    ap.add_argument("--no-stream-ceiling", action="store_true",
                    help="skip the streaming-read measurement of the GPU's attainable HBM read rate")
    ap.add_argument("--prefill-reps", type=int, default=5,
                    help="swan_prefill_convert launches over the workload's history timed back to back "
                         "after the decode measurements (one layer only; 0 = skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run plain device copies of this size (for calibrating HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the SWAN decode step here runs on a single MI355X "
              "(no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_attention_compressed_02_amd import accounting as acc
    from decode_attention_compressed_02_amd import swan as S
    from decode_attention_compressed_02_amd import workloads as wl
    from decode_attention_compressed_02_amd.state import build_decoder, step_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    S.lib()
    w = wl.config(args.config)
    base_name = w.name.replace(f" {w.steps} steps", "")
    if args.values == "fp8":
        w = w.scaled(value_format=1)
    if args.kv_share > 0:
        kk = int(round(2 * w.k * args.kv_share))
        w = w.scaled(k=kk, k_v=2 * w.k - kk)
    vbytes = 1 if w.value_format else 2
    if args.steps > w.steps:
        w = w.scaled(steps=args.steps)
    if args.layers > 1:
        w = w.scaled(layers=args.layers)
    L = max(1, w.layers)
    dec = build_decoder(w, args.split_tokens, keep_history=args.prefill_reps > 0)
    log(f"device {torch.cuda.get_device_name(0)}; dims {dec.dims}")

    # step inputs for every step, resident in HBM before timing
    inputs, pos_host = [], []
    for s in range(args.steps):
        q, kr, vn, pos = step_inputs(w, s)
        inputs.append(tuple(torch.from_numpy(a).cuda() for a in (q, kr, vn, pos)) + (int(pos.max()),))
        pos_host.append(pos)
    paged = w.block_size > 0
    if paged:
        import copy
        pool0 = copy.deepcopy(dec.pool)
    max_pos_all = max(x[4] for x in inputs)
    dec.ensure_workspace(max_pos_all)
    kb0, vb0 = dec.cache.k_buf.clone(), dec.cache.v_buf.clone()
    nsplit = S.swan_decode_num_splits(dec.dims, inputs[0][4])

    stream = torch.cuda.current_stream()

    def run_step(x, ev=None, ph=None):
        q, kr, vn, pos, mp = x
        if paged:  # host bookkeeping, then table update + projection + append in one launch
            dec.project_append_paged(q, kr, vn, pos, ph)
        else:
            dec.project_append(q, kr, vn, pos, mp)
        if ev is not None:
            ev[0].record(stream)
        S.swan_decode_split(dec.dims, dec.cache.struct(), pos, mp, dec.q_hat, dec.workspace)
        if ev is not None:
            ev[1].record(stream)
        S.swan_decode_reduce(dec.dims, pos, mp, dec.workspace, dec.o_hat)

    def restore():
        # back to the initial state: the steps only changed the ring and rows
        # past n (and, paged, the pool's tables and counts)
        dec.cache.k_buf.copy_(kb0)
        dec.cache.v_buf.copy_(vb0)
        if paged:
            dec.pool = copy.deepcopy(pool0)
            dec._bt_version = -1
            dec.sync_table()

    def split_launch():
        q, kr, vn, pos, mp = inputs[args.steps - 1]
        S.swan_decode_split(dec.dims, dec.cache.struct(), pos, mp, dec.q_hat, dec.workspace)

    def back_to_back(launch, reps=20):
        """Per-launch time (ms) of `reps` launches enqueued back to back between two events."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    graphs = None

    def timed_steps(warmup):
        """`warmup` untimed steps replaying the step sequence from the initial
        state, then the args.steps timed steps from it: wall seconds."""
        for s in range(warmup):
            if s % args.steps == 0:
                restore()
            run_step(inputs[s % args.steps], ph=pos_host[s % args.steps])
        torch.cuda.synchronize()
        restore()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            if graphs is None:
                run_step(inputs[s], ph=pos_host[s])
            else:
                if paged:  # host bookkeeping stays eager; its table writes travel by value
                    dec.prepare_step(pos_host[s])
                graphs[s].replay()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    tokens = sum(int(inputs[s][3].sum().item()) + inputs[s][3].numel() for s in range(args.steps))  # sum (pos + 1)
    # algorithmic bytes of the split kernel per launch, per timed step
    split_bytes, dec_bytes, flops = [], [], []
    for s in range(args.steps):
        pos = inputs[s][3].cpu().numpy()
        n = [max(0, int(p) + 1 - w.R) for p in pos]
        f = [min(int(p) + 1, w.R) for p in pos]
        split_bytes.append(acc.split_kernel_bytes(n, w.H_kv, w.N_h, f, w.k, value_bytes=vbytes, k_v=w.k_v))
        dec_bytes.append(acc.decode_bytes(n, w.H_kv, w.N_h, f, w.k, value_bytes=vbytes, k_v=w.k_v))
        flops.append(acc.decode_flops(n, w.H_kv, w.N_h, f, w.k, k_v=w.k_v))
    last_bytes = float(split_bytes[-1])

    # 1. the timed steps without a settle phase (only the warm-up before them)
    wall_u = timed_steps(args.warmup)
    split_b2b_u = back_to_back(split_launch)
    unsettled = {"warmup": args.warmup, "ms_per_step": wall_u * 1e3 / args.steps, "value": tokens / wall_u,
                 "step_frac_of_peak": float(np.mean(dec_bytes)) / wall_u * args.steps / 1e9 / HBM_PEAK_GBS,
                 "split_kernel_ms_back_to_back": split_b2b_u,
                 "roofline_frac": last_bytes / (split_b2b_u * 1e-3) / 1e9 / HBM_PEAK_GBS}
    log(f"without a settle phase: {unsettled['ms_per_step'] * 1e3:.1f} us a step, split pass "
        f"{split_b2b_u * 1e3:.1f} us back to back")

    # 2. the settle phase: whole steps back to back, in chunks of the step
    # sequence (restored before each), each chunk timed between two events
    settle = None
    if args.settle_steps > 0:
        chunks, done = [], 0
        while done < args.settle_steps:
            restore()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for s in range(args.steps):
                run_step(inputs[s], ph=pos_host[s])
            e1.record(stream)
            chunks.append((e0, e1))
            done += args.steps
        torch.cuda.synchronize()
        per_step = [a.elapsed_time(b) * 1e3 / args.steps for a, b in chunks]
        settle = {"steps": done, "chunk_steps": args.steps, "ms": sum(per_step) * args.steps / 1e3,
                  "per_step_us_by_chunk": [round(x, 1) for x in per_step]}
        log(f"settle phase: {done} steps, {per_step[0]:.1f} -> {per_step[-1]:.1f} us a step")

    if args.graph:  # capturing records the launches and runs nothing: the state is unchanged
        from decode_attention_compressed_02_amd.cache import StepGraph
        restore()
        graphs = [StepGraph(dec, *inputs[s][:4], max_pos=max_pos_all) for s in range(args.steps)]
        torch.cuda.synchronize()

    # 3. the timed steps (the reported value): warm-up, then the steps
    wall = timed_steps(args.warmup)
    ms_step = wall * 1e3 / args.steps
    value = tokens / wall

    # the split pass's duration inside a step, from a replay of the same steps
    # with events around it (event markers add a few microseconds of launch
    # gap each, so this replay is not the timed one); it ends in the same state
    restore()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for s in range(args.steps):
        run_step(inputs[s], evs[s], ph=pos_host[s])
    torch.cuda.synchronize()
    split_ms = [a.elapsed_time(b) for a, b in evs]
    split_avg_ms = float(np.mean(split_ms))

    # the split kernel alone, launched back to back on the same stream over
    # the state the last step left (decode does not modify the cache): its
    # per-launch time is the kernel's duration plus the launch gap, without
    # the wait for the preceding kernels of a step
    split_b2b_ms = back_to_back(split_launch)
    achieved = last_bytes / (split_b2b_ms * 1e-3) / 1e9

    # the whole decode (split + reduce) back to back: t_decode
    def decode_launch():
        q, kr, vn, pos, mp = inputs[args.steps - 1]
        S.swan_decode_split(dec.dims, dec.cache.struct(), pos, mp, dec.q_hat, dec.workspace)
        S.swan_decode_reduce(dec.dims, pos, mp, dec.workspace, dec.o_hat)
    decode_ms = back_to_back(decode_launch)
    last_tokens = int(inputs[args.steps - 1][3].sum().item()) + inputs[args.steps - 1][3].numel()

    # the split kernel from a cold last-level cache: before every other one of
    # these launches a 1 GiB fill evicts the L2s and the 256 MB MALL, so a
    # cache that fits the MALL (e.g. 202 MB) is streamed from HBM; events
    # bracket the launch only, and the launches without the fill give the
    # warm figure of the same protocol
    split_cold_ms = split_single_ms = None
    if args.cold_reps > 0:
        flush = torch.empty(2 ** 30, dtype=torch.uint8, device="cuda")
        times = {True: [], False: []}
        for i in range(2 * args.cold_reps):
            evict = i % 2 == 0
            if evict:
                flush.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            split_launch()
            b.record(stream)
            torch.cuda.synchronize()
            times[evict].append(a.elapsed_time(b))
        del flush
        split_cold_ms, split_single_ms = float(np.median(times[True])), float(np.median(times[False]))

    # the attainable HBM read rate on this GPU: a plain streaming read of the
    # split kernel's byte count, at a few grid sizes (the best is the ceiling)
    stream_read = None
    if not args.no_stream_ceiling:
        nb = int(last_bytes) // 16 * 16
        buf = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)
        sink = torch.empty(4096 * 64, dtype=torch.int32, device="cuda")
        best = None
        for waves in (1024, 2048, 4096):
            launch = lambda: S.swan_measure_stream_read(buf, waves, sink)
            back_to_back(launch, 3)
            ms = back_to_back(launch)
            gbs = nb / (ms * 1e-3) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, waves, ms)
        del buf, sink
        stream_read = {"GBps": best[0], "waves": best[1], "ms": best[2], "bytes": nb,
                       "frac_of_peak": best[0] / HBM_PEAK_GBS}

    traffic = traffic_ea = None
    if os.path.exists(TRAFFIC_FILE):
        from decode_attention_compressed_02_amd.profiling import kernel_source_hash
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if (tr.get("kernel_source_sha") == kernel_source_hash() and tr.get("workload") == w.name
                and tr.get("value_format", 0) == w.value_format and not w.k_v and L == 1):
            traffic = tr.get("hbm_bytes_per_launch")
            cc = tr.get("cross_check")
            if cc:  # DRAM read requests in 32-byte units, plus the same writes
                traffic_ea = cc["ea_read_bytes_per_launch"] + tr["write_bytes_per_launch"]

    # the prefill conversion of the workload's own history (the step before
    # decoding; it rebuilds the cache the decode steps started from): its
    # double-precision key projection runs on the fp64 matrix cores, so its
    # roofline is their rate, published and measured with the same grid of
    # independent products (swan_measure_mfma_f64)
    prefill = None
    if args.prefill_reps > 0 and getattr(dec, "history", None) is not None:
        lens, Tm, K, V = dec.history
        T = [int(x) for x in lens.cpu()]
        th = sum(T) * w.H_kv
        pf_flops = 2.0 * 128 * 128 * th
        kv_v = w.k_v or w.k
        n_rows = sum(max(0, t - w.R) for t in T) * w.H_kv
        pf_bytes = (th * 2 * 128 * 4 + n_rows * (w.k + kv_v) * (1 + vbytes)
                    + sum(min(t, w.R) for t in T) * w.H_kv * 2 * 128 * 2)
        launch = lambda: dec.prefill(lens, Tm, K, V)
        back_to_back(launch, 1)
        pf_ms = back_to_back(launch, args.prefill_reps)
        mf_waves, mf_iters = 16384, 1024
        sink = torch.empty(mf_waves * 64, dtype=torch.float64, device="cuda")
        mf = lambda: S.swan_measure_mfma_f64(1.0, mf_waves, mf_iters, sink)
        back_to_back(mf, 2)
        mf_ms = back_to_back(mf, 5)
        mf_tflops = mf_waves * mf_iters * 16384 / (mf_ms * 1e-3) / 1e12
        del sink
        pf_tflops = pf_flops / (pf_ms * 1e-3) / 1e12
        prefill = {"kernel": "k_prefill", "ms": pf_ms, "reps": args.prefill_reps, "history_tokens": sum(T),
                   "token_heads": th, "tokens_per_s": sum(T) / (pf_ms * 1e-3),
                   "bytes_per_launch": pf_bytes, "GBps": pf_bytes / (pf_ms * 1e-3) / 1e9,
                   "roofline": {"bound": "mfma", "achieved": pf_tflops, "peak": MFMA_F64_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": pf_tflops / MFMA_F64_PEAK_TFLOPS,
                                "algorithmic_flops_per_launch": pf_flops,
                                "measured_ceiling_TFLOPs": mf_tflops,
                                "frac_of_measured_ceiling": pf_tflops / mf_tflops}}
        log(f"prefill conversion: {pf_ms:.3f} ms ({pf_tflops:.1f} TFLOP/s fp64 projection, "
            f"{100 * pf_tflops / MFMA_F64_PEAK_TFLOPS:.1f}% of peak; fp64 matrix cores sustain {mf_tflops:.1f})")
        del dec.history, K, V

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * 2 ** 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                "kernel": "k_split", "algorithmic_bytes_per_launch": last_bytes}
    if traffic_ea is not None:
        roofline["traffic_dram_request_count"] = traffic_ea
    if stream_read:
        roofline["measured_ceiling_GBps"] = stream_read["GBps"]
        roofline["frac_of_measured_ceiling"] = achieved / stream_read["GBps"]
    result = {
        "metric": "decode-attn KV tokens/sec and achieved HBM GB/s (% of peak) per step",
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) raw keys/queries, stored-basis values, random orthogonal P_QK)",
        "config": {"workload": f"workload {args.config}: {base_name}" + (", fp8 values" if w.value_format else "")
                   + (f", k_K {w.k} / k_V {w.k_v}" if w.k_v else "")
                   + (f", {L} layers stacked in one batch" if L > 1 else "")
                   + f", {args.steps} consecutive decode steps timed",
                   "B": w.B, "N_h": w.N_h, "H_kv": w.H_kv,
                   "d_h": w.d_h, "ctx_first_step": int(w.ctx[0]), "R": w.R, "k": w.k, "k_v": w.k_v or w.k,
                   "layers": L,
                   "storage": f"{'fp8 E4M3' if w.value_format else 'fp16'} values, uint8 indices, fp16 dense buffer",
                   "split_waves": nsplit,
                   "split_tokens": dec.dims.split_tokens or "auto",
                   "launch": "HIP graph per step" if args.graph else "eager"},
        "settle": settle,
        "unsettled": unsettled,
        "step_hbm_GBps": float(np.mean(dec_bytes)) / (ms_step * 1e-3) / 1e9,
        "step_frac_of_peak": float(np.mean(dec_bytes)) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "head_tokens_per_s": value * w.H_kv,
        "ms_per_step_per_layer": ms_step / L,
        "decode_ms_back_to_back": decode_ms,
        "decode_kv_tokens_per_s": last_tokens / (decode_ms * 1e-3),
        "decode_frac_of_peak": float(dec_bytes[-1]) / (decode_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "split_kernel_ms_in_step": split_avg_ms,
        "split_kernel_ms_back_to_back": split_b2b_ms,
        "split_kernel_ms_single_launch": split_single_ms,
        "split_kernel_ms_cold_cache": split_cold_ms,
        "split_cold_cache_GBps": (last_bytes / (split_cold_ms * 1e-3) / 1e9) if split_cold_ms else None,
        "stream_read": stream_read,
        "decode_gflops_per_step": float(np.mean(flops)) / 1e9,
        "roofline": roofline,
        "prefill": prefill,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        model, threads = host_cpu()
        seqs = list(range(min(args.cpu_seqs, w.B)))
        v, cores, secs, desc = cpu_baseline(w, seqs, args.cpu_seconds)
        result["cpu_baseline"] = {"value": v, "unit": "KV tokens/s", "cores": cores, "kind": "oracle",
                                  "sample": desc, "seconds": secs, "host_cpu": model, "host_threads": threads}
        # the same oracle on one thread, over one sequence (all kv heads)
        v1, _, secs1, desc1 = cpu_baseline(w, seqs[:1], args.cpu_seconds / 4, threads=1)
        result["cpu_baseline_1_thread"] = {"value": v1, "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
                                           "sample": desc1, "seconds": secs1, "host_cpu": model}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
