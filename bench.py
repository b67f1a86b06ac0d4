"""Benchmark of the gated delta-rule hot path on one MI355X.

A step is one chunkwise-parallel prefill (dr_chunk_fwd) over the KDA prefill
workload: B=4, T=4096, H=16, d_k=d_v=128, bf16 q/k/v, fp32 gates and states,
inputs resident in HBM. The call launches two kernels back to back on the
stream (chunk preparation, then the sequential state pass); the roofline
figure is the call's algorithmic bytes over its event-timed duration, and the
measured HBM traffic is given per kernel beside it. Two full input sets alternate so the 256 MB Infinity
Cache cannot hold a step's inputs from the previous one. `value` is tokens/s
(B*T tokens per step). The decode step (dr_decode_step) is timed in its own loop
on 512 sequences x 32 heads with the 1 GiB fp32 state updated in place, and is
reported as state GB/s under "decode". Further legs time the snapshots, the
fused input preparation, the backward pass and the two-transitions-per-token
variant (prefill and decode) on the same shapes.

Prints one JSON line. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
SETTLE_CALLS = 100           # untimed prefill calls before the warm-up steps (see main)
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


def prefill_work(B, T, H, dk, dv, C=64, in_bytes=2, gate_bytes=4, n_states=None, alpha_bytes=4):
    """Algorithmic bytes and useful FLOPs of one prefill call.
    Bytes per token-head: q, k, v inputs + alpha (fp32, or bf16 pre-activations) + gates +
    o (fp32); plus the initial and final state of every (sequence, head). FLOPs: the
    chunkwise form's useful (triangular) work per full chunk-head, pro rata per token."""
    th = B * T * H
    per_th = (2 * dk + dv) * in_bytes + alpha_bytes * dk + gate_bytes + 4 * dv
    n_states = B if n_states is None else n_states
    bytes_ = th * per_th + 2 * n_states * H * dk * dv * 4
    f_chunk = 2 * (C * (C - 1) // 2 * dk + C * (C + 1) // 2 * dk + C * (C - 1) * (C - 2) // 6
                   + C * (C - 1) // 2 * dk + C * (C - 1) // 2 * dv + 3 * C * dk * dv + C * (C + 1) // 2 * dv)
    flops = th * f_chunk / C
    return bytes_, flops


def decode_bytes(N, H, dk, dv, in_bytes=2, gate_bytes=4):
    """State read + write, plus the token's q, k, v, alpha, gates and o, per step."""
    return N * H * (8 * dk * dv + (2 * dk + dv) * in_bytes + 4 * dk + gate_bytes + 4 * dv)


# the prefill kernels' sources (both passes and what they include)
PREFILL_SOURCES = ("prefill.hip", "prefill_state.hip", "prefill.hpp", "common.hpp")


def kernel_source_digest():
    """sha256 of the prefill kernel's sources with comments and whitespace removed, and of their
    per-file compiler options: a stored traffic measurement is used only while it matches the
    code that is being timed (an edit of a comment leaves it valid, any change of code or of
    its build options does not)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in PREFILL_SOURCES:
        with open(os.path.join(ROOT, "delta_rule_linear_chunked_amd", "csrc", f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)  # block comments
        src = re.sub(r"//[^\n]*", " ", src)                # line comments
        h.update(" ".join(src.split()).encode())
    # the per-file compiler options change the kernels as much as their sources do
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_dr_build", os.path.join(os.path.dirname(os.path.abspath(__file__)), "delta_rule_linear_chunked_amd", "_build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    h.update(repr(sorted((f, build.FILE_FLAGS.get(f, [])) for f in PREFILL_SOURCES)).encode())
    return h.hexdigest()


def copy_calibration(dev, mib=512, reps=5):
    """A plain device-to-device copy of known size (the reference for HBM counters and the
    measured copy bandwidth)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"bytes_read_per_copy": n * 4, "bytes_written_per_copy": n * 4, "copies": reps + 1,
            "ms_per_copy": ms, "copy_GBps": 2 * n * 4 / (ms * 1e-3) / 1e9}


def gpu_clocks():
    """The GPU's shader and memory clock levels as the kernel driver lists them in sysfs (the
    current level is marked with '*'); read from files, so no other program is started."""
    import glob
    out = {}
    for card in sorted(glob.glob("/sys/class/drm/card*/device")):
        for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
            try:
                with open(os.path.join(card, name)) as fh:
                    levels = [ln.strip() for ln in fh if ln.strip()]
            except OSError:
                continue
            out.setdefault(os.path.basename(os.path.dirname(card)), {})[name] = levels
    return out or None


def run_conditions():
    """Host CPU model, the CPUs this process may use and the date."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        ncpu = os.cpu_count()
    return {"host_cpu_model": model or platform.processor() or platform.machine(), "host_cpus_usable": ncpu,
            "date_utc": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime())}


_CPU_WL = {}   # the workload the forked oracle workers read (set before the pool is made)
_PRESETS = {}  # workloads the CPU baseline generated, kept for the GPU legs of the same run


def _pin_worker(counter, cpus):
    """Pool initializer: pin this worker process to a core of its own (the i-th worker started takes
    the i-th usable core)."""
    with counter.get_lock():
        i = counter.value
        counter.value += 1
    try:
        os.sched_setaffinity(0, {cpus[i % len(cpus)]})
    except (AttributeError, OSError):  # pragma: no cover
        pass


def _pinned_worker(heads):
    """Run the oracle's step recurrence over the given heads of the current workload in this (pinned)
    worker; returns (seconds, token-heads)."""
    import oracle
    wl = _CPU_WL["wl"]
    h = list(heads)
    g = lambda x: None if x is None else np.ascontiguousarray(x[:, :, h])  # noqa: E731
    args_ = (g(wl.q), g(wl.k), g(wl.v), g(wl.alpha), g(wl.erase), g(wl.write))
    S0 = None if wl.S0 is None else np.ascontiguousarray(wl.S0[:, h])
    t0 = time.perf_counter()
    oracle.step_recurrence(*args_, wl.variant, S0=S0, cu_seqlens=wl.cu_seqlens)
    return time.perf_counter() - t0, wl.q.shape[0] * wl.q.shape[1] * len(h)


def cpu_baseline(full=False):
    """The fp64 oracle as it is (never tuned), on the host cores, in two modes: one process pinned to
    one core (numpy limited to one thread), and the heads split over as many pinned processes as
    there are usable cores. Every workload runs whole in the multi-process mode; on one core the
    KDA prefill runs on 4 of its 16 heads and the varlen and long-context workloads on 1 (all of
    them with ``full``). Rates are tokens/s of the whole workload (token-heads/s divided by its 16
    heads). Decode: one oracle step of 1/16 of the decode workload on one core."""
    import multiprocessing as mp
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    import oracle
    import synth
    ctx = threadpool_limits(1) if threadpool_limits else None
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    cpus = sorted(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else list(range(os.cpu_count() or 1))
    H = 16
    out = {}
    for name, sample_heads in (("kda_prefill", 4), ("rda_varlen", 1), ("gdn2_varlen", 1), ("ckda_long", 1)):
        _CPU_WL["wl"] = _PRESETS[name] = synth.preset(name)
        ctx_fork = mp.get_context("fork")
        workers = min(len(cpus), H)
        pool = ctx_fork.Pool(workers, initializer=_pin_worker, initargs=(ctx_fork.Value("i", 0), cpus))
        try:
            nh = H if full else sample_heads
            dt, th = pool.apply(_pinned_worker, (range(nh),))
            one = {"tokens_per_s": th / dt / H, "seconds": dt, "cores": 1,
                   "sample": "whole workload" if nh == H else f"{nh} of {H} heads, every sequence"}
            # one head per task, the pool's processes pinned to distinct cores: the rate is all
            # token-heads over the wall time of the whole map (rounds of tasks where there are more
            # heads than cores)
            tw = time.perf_counter()
            res = pool.map(_pinned_worker, [range(i, i + 1) for i in range(H)], chunksize=1)
            span = time.perf_counter() - tw
            many = {"tokens_per_s": sum(r[1] for r in res) / span / H, "seconds": span,
                    "cores": workers, "sample": "whole workload, one head per task"}
            out[name] = {"one_core": one, "all_cores": many}
        finally:
            pool.close()
            pool.join()
            _CPU_WL.clear()
    # decode: one step of 32 of the 512 sequences (x 32 heads), the fp64 state of the subset
    # (128 MiB) updated once
    wd = synth.make_decode("kda", 32, 32, 128, 128, steps=1, in_dtype="bf16", seed=1005)
    S = wd.S0.astype(np.float64)
    t1 = time.perf_counter()
    oracle.decode_step(S, wd.q[0], wd.k[0], wd.v[0], wd.alpha[0], wd.erase[0], None, "kda")
    dd = time.perf_counter() - t1
    if ctx is not None:
        ctx.__exit__(None, None, None)
    cond = run_conditions()
    _PRESETS.pop("kda_prefill", None)  # the GPU legs draw their own KDA inputs
    k2 = out["kda_prefill"]["one_core"]
    nh = H if full else 4
    return {"value": k2["tokens_per_s"], "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{nh} of the 16 heads of the KDA prefill workload (4 x 4096 tokens, fp64 step recurrence) "
                      f"in {k2['seconds']:.1f} s in one process pinned to one core of {cond['host_cpu_model']}; "
                      f"rate scaled to the whole workload's tokens",
            "modes": out,
            "decode": {"value": 32 * 32 / dd, "unit": "head-steps/s", "cores": 1,
                       "sample": f"one KDA decode step of 32 sequences x 32 heads (1/16 of the decode "
                                 f"workload, fp64 state) in {dd:.2f} s on one core"},
            "conditions": cond}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="run the oracle on every head of every workload on one core too (minutes)")
    ap.add_argument("--no-strided", action="store_true",
                    help="skip the prefill on q, k, v given as views of one fused projection")
    ap.add_argument("--no-recurrence", action="store_true",
                    help="skip the GPU step recurrence (the decode kernel token by token) beside the prefill")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-states", action="store_true", help="skip the snapshot and slot-pool timings")
    ap.add_argument("--no-prep", action="store_true", help="skip the fused input preparation timing")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward (gradient) timing")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the timings of the varlen (RDA, GDN-2) and long-context (CKDA) prefill workloads")
    ap.add_argument("--no-product", action="store_true",
                    help="skip the two-transitions-per-token variant's prefill and decode timings")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the plain copy used to scale the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only; --gpus must be 1 (the path runs per GPU with no "
              "communication, see the sharding notes)", file=sys.stderr)
        sys.exit(2)

    # run conditions first, then the oracle's CPU baseline in processes forked before anything
    # touches the GPU
    conditions = run_conditions()
    cpu = None if (args.no_cpu_baseline or args.calibrate_copy) else cpu_baseline(full=args.cpu_full)

    import torch
    import delta_rule_linear_chunked_amd as drl
    import synth

    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        print(json.dumps({"copy_calibration": copy_calibration(dev)}))
        return
    drl.load_library()

    def t(x, bf16=False):
        if x is None:
            return None
        y = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        return y.to(torch.bfloat16) if bf16 else y

    # ------------------------------------------------------------------ prefill
    B, T, H, D = 4, 4096, 16, 128
    sets = []
    for seed in (1002, 2002):
        wl = synth.make_prefill("kda", B, T, H, D, D, in_dtype="bf16", seed=seed)
        sets.append(dict(q=t(wl.q, True), k=t(wl.k, True), v=t(wl.v, True), alpha=t(wl.alpha),
                         erase=t(wl.erase), S0=t(wl.S0)))
        del wl
    o = torch.empty((B, T, H, D), dtype=torch.float32, device=dev)
    S_T = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)

    def step(i):
        s = sets[i % 2]
        drl.dr_chunk_fwd(s["q"], s["k"], s["v"], s["alpha"], s["erase"], None, "kda", s["S0"], None, o, S_T)

    # The GPU idled while the CPU baseline and the inputs were made. Per-call times measured from
    # idle: the first few calls are fast, calls 5-25 run about 10% slower while the GPU's power
    # management reacts to the load, and from about call 30 on the time holds steady (plain copies
    # do not bring this about). So SETTLE_CALLS untimed calls run first, then the W warm-up steps,
    # then the K timed steps; the line reports SETTLE_CALLS.
    for i in range(SETTLE_CALLS):
        step(i)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    # the timed steps run back to back with events only at the ends of the loop (an event
    # between every pair of calls adds a few microseconds per call); a second loop with an
    # event after every call gives the per-call percentiles
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    ms_step = total_ms / args.steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])  # ms per call
    clocks_after_timing = gpu_clocks()
    tokens = B * T
    value = tokens / (ms_step * 1e-3)
    alg_bytes, flops = prefill_work(B, T, H, D, D)
    achieved_gbs = alg_bytes / (ms_step * 1e-3) / 1e9
    plan = drl.chunk_fwd_plan(B, T, H, D, D)

    # the same tokens through the step recurrence on the GPU: the decode kernel applied once per
    # token (4096 launches over the 64 (sequence, head) states, bf16 inputs, fp32 state), timed as
    # an eager loop and as one replayed HIP graph, with its error against the chunked call
    recurrence = None
    if not args.no_recurrence:
        s = sets[0]
        per_tok = {name: s[name].transpose(0, 1).contiguous() for name in ("q", "k", "v", "alpha", "erase")}
        S_rec = torch.empty_like(S_T)
        o_rec = torch.empty((T, B, H, D), dtype=torch.float32, device=dev)

        def recur():
            S_rec.copy_(s["S0"])
            for t_ in range(T):
                drl.dr_decode_step(per_tok["q"][t_], per_tok["k"][t_], per_tok["v"][t_], per_tok["alpha"][t_],
                                   per_tok["erase"][t_], None, "kda", S_rec, o_rec[t_])

        recur()
        step(0)  # the chunked call on the same inputs (sets[0])
        torch.cuda.synchronize()
        o_r = o_rec.transpose(0, 1)
        rms_o = o.pow(2).mean().sqrt().item()
        rms_s = S_T.pow(2).mean().sqrt().item()
        err_o = (o_r - o).abs().max().item() / rms_o
        err_s = (S_rec - S_T).abs().max().item() / rms_s
        reps = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            recur()
        e1.record(stream)
        torch.cuda.synchronize()
        eager_ms = e0.elapsed_time(e1) / reps
        graph_ms = None
        try:
            g = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream(dev)
            cap.wait_stream(stream)
            with torch.cuda.stream(cap):
                recur()  # one eager pass on the capture stream first
            stream.wait_stream(cap)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                recur()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(o_rec.transpose(0, 1), o_r):
                raise RuntimeError("graph replay differs from the eager recurrence")
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            graph_ms = e0.elapsed_time(e1) / reps
            del g
        except Exception as exc:  # noqa: BLE001 - the graph timing is optional; say why it is missing
            graph_ms = f"not timed: {exc}"
        best = min(eager_ms, graph_ms) if isinstance(graph_ms, float) else eager_ms
        recurrence = {
            "workload": "the KDA prefill's tokens (4 x 4096, 16 heads, d=128, bf16 inputs, fp32 state) through "
                        "dr_decode_step once per token",
            "ms_eager_loop": eager_ms, "ms_graph_replay": graph_ms, "tokens_per_s": tokens / (best * 1e-3),
            "chunked_speedup": best / ms_step,
            "err_o_vs_chunked": err_o, "err_S_T_vs_chunked": err_s,
            "err_metric": "max |recurrence - chunked| / RMS(chunked), on o and on S_T"}
        del per_tok, S_rec, o_rec, o_r

    # q, k, v as views of one fused [B, T, 3, H, d] projection (read through their strides, no copy)
    strided = None
    if not args.no_strided:
        fused_sets = [torch.stack([s_["q"], s_["k"], s_["v"]], dim=2).contiguous() for s_ in sets]

        def fstep(i):
            s_, f_ = sets[i % 2], fused_sets[i % 2]
            drl.dr_chunk_fwd(f_[:, :, 0], f_[:, :, 1], f_[:, :, 2], s_["alpha"], s_["erase"], None, "kda", s_["S0"],
                             None, o, S_T)

        for i in range(10):
            fstep(i)
        torch.cuda.synchronize()
        # blocks of dense and strided calls in alternation (medians of the block means), so that
        # a drift of the clocks between two loops does not pass for a cost of the strides
        blocks = {"dense": [], "strided": []}
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for rnd in range(8):
            order = (("dense", step), ("strided", fstep)) if rnd % 2 == 0 else (("strided", fstep), ("dense", step))
            for name, fn in order:
                e0.record(stream)
                for i in range(10):
                    fn(i)
                e1.record(stream)
                torch.cuda.synchronize()
                blocks[name].append(e0.elapsed_time(e1) / 10)
        fms, dms_ = float(np.median(blocks["strided"])), float(np.median(blocks["dense"]))
        strided = {"workload": "the KDA prefill with q, k, v as views of one [4, 4096, 3, 16, 128] bf16 tensor "
                               "(token stride 3 H d)", "ms_per_step": fms, "tokens_per_s": tokens / (fms * 1e-3),
                   "dense_ms_same_blocks": dms_, "vs_dense": fms / dms_,
                   "timing": "medians of 8 blocks of 10 calls each, dense and strided blocks alternating"}
        del fused_sets

    # stored-state options on the same workload: snapshots every 64 and every 1024 tokens
    states = None
    if not args.no_states:
        states = {}
        for every in (1024, 64):
            snaps = torch.empty((B * (T // every), H, D, D), dtype=torch.float32, device=dev)

            def sstep(i, every=every, snaps=snaps):
                s = sets[i % 2]
                drl.dr_chunk_fwd_ex(s["q"], s["k"], s["v"], s["alpha"], s["erase"], None, "kda", s["S0"], None,
                                    o, S_T, snapshots=snaps, snapshot_every=every)

            for i in range(3):
                sstep(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(args.steps):
                sstep(i)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            states[f"prefill_snapshot_every_{every}"] = {
                "ms_per_step": ms, "tokens_per_s": tokens / (ms * 1e-3),
                "snapshot_bytes": snaps.numel() * 4, "overhead_vs_plain": ms / ms_step - 1.0}
            del snaps

    # fused input preparation on the same shape: raw q/k (normalised in the kernel), decay as
    # bf16 pre-activation of exp(-0.1 softplus(z)), beta as pre-activation of sigmoid
    fused = None
    if not args.no_prep:
        psets = []
        for seed in (1002, 2002):
            wl = synth.make_prefill("kda", B, T, H, D, D, in_dtype="bf16", seed=seed, preact=True, alpha_dtype="bf16")
            kw = {k: v for k, v in wl.meta["prep"].items() if k != "alpha_dtype"}
            psets.append(dict(q=t(wl.q, True), k=t(wl.k, True), v=t(wl.v, True), alpha=t(wl.alpha, True),
                              erase=t(wl.erase), S0=t(wl.S0)))
            del wl

        def pstep(i):
            s = psets[i % 2]
            drl.dr_chunk_fwd_ex(s["q"], s["k"], s["v"], s["alpha"], s["erase"], None, "kda", s["S0"], None,
                                o, S_T, prep=kw)

        for i in range(3):
            pstep(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            pstep(i)
        e1.record(stream)
        torch.cuda.synchronize()
        pms = e0.elapsed_time(e1) / args.steps
        pbytes, _ = prefill_work(B, T, H, D, D, alpha_bytes=2)
        fused = {"workload": "KDA prefill B=4 T=4096 H=16 d=128, raw bf16 q/k, bf16 decay pre-activations, "
                             "beta pre-activations; normalisation and activations inside the kernels",
                 "ms_per_step": pms, "tokens_per_s": tokens / (pms * 1e-3), "alg_bytes_per_launch": pbytes,
                 "achieved_GBps": pbytes / (pms * 1e-3) / 1e9}
        del psets

    # backward (gradients of the same prefill, dO and dS_T random): checkpointing forward, then the
    # chunked MFMA path (these gates never hand the call to the walk); the exact walk alone is timed
    # beside it (DR_BWD_WALK=1)
    bwd = None
    if not args.no_backward:
        gdO = torch.randn((B, T, H, D), device=dev)
        gdS = torch.randn((B, H, D, D), device=dev)
        grads = dict(dq=torch.empty((B, T, H, D), device=dev), dk=torch.empty((B, T, H, D), device=dev),
                     dv=torch.empty((B, T, H, D), device=dev), dalpha=torch.empty((B, T, H, D), device=dev),
                     derase=torch.empty((B, T, H), device=dev), dS0=torch.empty((B, H, D, D), device=dev))

        def bstep(i):
            s = sets[i % 2]
            drl.dr_chunk_bwd(s["q"], s["k"], s["v"], s["alpha"], s["erase"], None, "kda", s["S0"], None, gdO, gdS,
                             grads["dq"], grads["dk"], grads["dv"], grads["dalpha"], grads["derase"], None, grads["dS0"])

        bsteps = max(3, args.steps // 5)
        for i in range(2):
            bstep(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(bsteps):
            bstep(i)
        e1.record(stream)
        torch.cuda.synchronize()
        bms = e0.elapsed_time(e1) / bsteps
        # the same gradients given the forward's checkpoints (a training step's forward taken with
        # snapshot_every = 64): the call then skips its own forward pass
        ckpts = [torch.empty((B * (T // 64), H, D, D), dtype=torch.float32, device=dev) for _ in sets]
        for s, c in zip(sets, ckpts):
            drl.dr_chunk_fwd_ex(s["q"], s["k"], s["v"], s["alpha"], s["erase"], None, "kda", s["S0"], None, o, S_T,
                                snapshots=c, snapshot_every=64)

        def cstep(i):
            s = sets[i % 2]
            drl.dr_chunk_bwd(s["q"], s["k"], s["v"], s["alpha"], s["erase"], None, "kda", s["S0"], None, gdO, gdS,
                             grads["dq"], grads["dk"], grads["dv"], grads["dalpha"], grads["derase"], None, grads["dS0"],
                             checkpoints=ckpts[i % 2])

        for i in range(2):
            cstep(i)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(bsteps):
            cstep(i)
        e1.record(stream)
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / bsteps
        old_walk = os.environ.get("DR_BWD_WALK")
        os.environ["DR_BWD_WALK"] = "1"
        try:
            bstep(0)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(bsteps):
                bstep(i)
            e1.record(stream)
            torch.cuda.synchronize()
            wms = e0.elapsed_time(e1) / bsteps
        finally:
            if old_walk is None:
                del os.environ["DR_BWD_WALK"]
            else:
                os.environ["DR_BWD_WALK"] = old_walk
        bwd = {"workload": "gradients of the KDA prefill (dq, dk, dv, dalpha, dbeta, dS0) for random dO and dS_T",
               "path": "checkpointing forward, then the chunked MFMA backward",
               "ms_per_step": bms, "tokens_per_s": tokens / (bms * 1e-3), "steps": bsteps,
               "vs_forward": bms / ms_step,
               "ms_per_step_given_checkpoints": cms,
               "walk_ms_per_step": wms}
        del gdO, gdS, grads, ckpts

    # two KDA transitions per token (PRODUCT2) on the same shape: 4 x 4096 tokens, 2 x 4096 steps
    prod = None
    if not args.no_product:
        p2 = []
        for seed in (1006, 2006):
            wl = synth.make_product("kda", B, T, H, D, D, in_dtype="bf16", seed=seed)
            p2.append(dict(q=t(wl.q, True), k=t(wl.k, True), v=t(wl.v, True), alpha=t(wl.alpha),
                           erase=t(wl.erase), S0=t(wl.S0)))
            del wl

        def p2step(i):
            s = p2[i % 2]
            drl.dr_chunk_fwd(s["q"], s["k"], s["v"], s["alpha"], s["erase"], None, "product2", s["S0"], None, o, S_T)

        for i in range(3):
            p2step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            p2step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        p2ms = e0.elapsed_time(e1) / args.steps
        prod = {"prefill": {"workload": "two KDA transitions per token, B=4 T=4096 H=16 d=128 bf16 (8192 steps per "
                                        "sequence)", "ms_per_step": p2ms, "tokens_per_s": tokens / (p2ms * 1e-3),
                            "vs_kda": p2ms / ms_step}}
        if not args.no_backward:
            s = p2[0]
            gdO = torch.randn((B, T, H, D), device=dev)
            g2 = dict(dq=torch.empty((B, T, H, D), device=dev), dk=torch.empty((B, T, H, 2, D), device=dev),
                      dv=torch.empty((B, T, H, 2, D), device=dev), dalpha=torch.empty((B, T, H, D), device=dev),
                      derase=torch.empty((B, T, H, 2), device=dev), dS0=torch.empty((B, H, D, D), device=dev))

            def p2b():
                drl.dr_chunk_bwd(s["q"], s["k"], s["v"], s["alpha"], s["erase"], None, "product2", s["S0"], None,
                                 gdO, None, g2["dq"], g2["dk"], g2["dv"], g2["dalpha"], g2["derase"], None, g2["dS0"])

            p2b()
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(3):
                p2b()
            e1.record(stream)
            torch.cuda.synchronize()
            p2bms = e0.elapsed_time(e1) / 3
            prod["backward"] = {"ms_per_step": p2bms, "tokens_per_s": tokens / (p2bms * 1e-3), "steps": 3}
            del gdO, g2
        del p2

    # the other prefill workloads (checked for parity elsewhere), timed for context
    others = None
    if not args.no_configs:
        others = {}
        for name, gate_bytes in (("rda_varlen", 8), ("gdn2_varlen", 4 * (D + D)), ("ckda_long", 4)):
            wl = _PRESETS.pop(name, None) or synth.preset(name)
            a = dict(q=t(wl.q, True), k=t(wl.k, True), v=t(wl.v, True), alpha=t(wl.alpha), erase=t(wl.erase),
                     write=t(wl.write), S0=t(wl.S0), cu=None if wl.cu_seqlens is None else t(wl.cu_seqlens))
            Bw, Tw = wl.q.shape[0], wl.q.shape[1]
            N = wl.num_seqs
            ow = torch.empty((Bw, Tw, H, D), dtype=torch.float32, device=dev)
            Sw = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
            variant = wl.variant
            del wl

            def ostep():
                drl.dr_chunk_fwd(a["q"], a["k"], a["v"], a["alpha"], a["erase"], a["write"], variant, a["S0"], a["cu"],
                                 ow, Sw)

            for i in range(3):
                ostep()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(10):
                ostep()
            e1.record(stream)
            torch.cuda.synchronize()
            oms = e0.elapsed_time(e1) / 10
            ob, _ = prefill_work(Bw, Tw, H, D, D, gate_bytes=gate_bytes, n_states=N)
            others[name] = {"ms_per_step": oms, "tokens_per_s": Bw * Tw / (oms * 1e-3), "sequences": N,
                            "tokens": Bw * Tw, "alg_bytes_per_launch": ob,
                            "achieved_GBps": ob / (oms * 1e-3) / 1e9,
                            "hbm_frac": ob / (oms * 1e-3) / 1e9 / HBM_PEAK_GBS}
            if not args.no_backward and name != "ckda_long":
                # the backward of the packed workloads: chunked path, and the exact walk beside it
                gdO = torch.randn((Bw, Tw, H, D), device=dev)
                gdS = torch.randn((N, H, D, D), device=dev)
                gshape = (Bw, Tw, H, D) if variant == "gdn2" else (Bw, Tw, H)
                gg = [torch.empty((Bw, Tw, H, D), device=dev) for _ in range(4)]
                ge, gw = torch.empty(gshape, device=dev), torch.empty(gshape, device=dev)
                gS0 = torch.empty((N, H, D, D), device=dev)

                def gstep():
                    drl.dr_chunk_bwd(a["q"], a["k"], a["v"], a["alpha"], a["erase"], a["write"], variant, a["S0"],
                                     a["cu"], gdO, gdS, gg[0], gg[1], gg[2], gg[3], ge, gw, gS0)

                def gtime():
                    gstep()
                    torch.cuda.synchronize()
                    e0.record(stream)
                    for i in range(5):
                        gstep()
                    e1.record(stream)
                    torch.cuda.synchronize()
                    return e0.elapsed_time(e1) / 5

                others[name]["backward_ms_per_step"] = gtime()
                old_walk = os.environ.get("DR_BWD_WALK")
                os.environ["DR_BWD_WALK"] = "1"
                try:
                    others[name]["backward_walk_ms_per_step"] = gtime()
                finally:
                    if old_walk is None:
                        del os.environ["DR_BWD_WALK"]
                    else:
                        os.environ["DR_BWD_WALK"] = old_walk
                del gdO, gdS, gg, ge, gw, gS0
            del a, ow, Sw

    traffic, kernel_traffic = None, None
    tfile = os.path.join(ROOT, "profiles", "chunk_fwd_kda_B4_T4096_H16_d128_traffic.json")
    if os.path.exists(tfile):
        tj = json.load(open(tfile))
        if tj.get("kernel_source_sha256") == kernel_source_digest():
            traffic = tj.get("bytes_per_launch")
            kernel_traffic = {k: v["bytes"] for k, v in tj.get("kernels", {}).items()}

    # matrix-core busy fraction of each prefill kernel, from rocprofv3 counters taken on this
    # workload and these kernel sources: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x CUs x 4 SIMDs)
    mfma_busy = None
    mfile = os.path.join(ROOT, "profiles", "chunk_fwd_kda_B4_T4096_H16_d128_mfma.json")
    if os.path.exists(mfile):
        mj = json.load(open(mfile))
        if mj.get("kernel_source_sha256") == kernel_source_digest():
            mfma_busy = {k: v["mfma_busy_frac"] for k, v in mj.get("kernels", {}).items()}

    # ------------------------------------------------------------------ decode
    decode = None
    if not args.no_decode:
        del sets
        torch.cuda.empty_cache()
        N, HD = 512, 32
        pool = 16
        wd = synth.make_decode("kda", N, HD, D, D, steps=pool, in_dtype="bf16", seed=1005)
        toks = [dict(q=t(wd.q[i], True), k=t(wd.k[i], True), v=t(wd.v[i], True), alpha=t(wd.alpha[i]),
                     erase=t(wd.erase[i])) for i in range(pool)]
        S = t(wd.S0)
        od = torch.empty((N, HD, D), dtype=torch.float32, device=dev)
        del wd

        def dstep(i):
            s = toks[i % pool]
            drl.dr_decode_step(s["q"], s["k"], s["v"], s["alpha"], s["erase"], None, "kda", S, od)

        # warm-up: about 40 ms of decode steps (the first steps after the prefill legs run slower
        # while the clocks settle)
        for i in range(100):
            dstep(i)
        torch.cuda.synchronize()
        # mean over back-to-back steps with events only at the ends of the loop (an event between
        # every pair of launches adds a few microseconds per step), then a second loop with an
        # event after every step for the percentiles
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.decode_steps):
            dstep(i)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / args.decode_steps
        dev_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.decode_steps + 1)]
        dev_ev[0].record(stream)
        for i in range(args.decode_steps):
            dstep(i)
            dev_ev[i + 1].record(stream)
        torch.cuda.synchronize()
        dper = np.array([dev_ev[i].elapsed_time(dev_ev[i + 1]) for i in range(args.decode_steps)])
        dbytes = decode_bytes(N, HD, D, D)
        pooled = None
        if not args.no_states:
            # the same steps through a slot pool: sequence n owns a random slot of the 1 GiB state
            perm = torch.from_numpy(np.random.default_rng(7).permutation(N).astype(np.int32)).to(dev)

            def pstep(i):
                s = toks[i % pool]
                drl.dr_decode_step_ex(s["q"], s["k"], s["v"], s["alpha"], s["erase"], None, "kda", S, od,
                                      state_idx=perm)

            for i in range(10):
                pstep(i)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(args.decode_steps):
                pstep(i)
            e1.record(stream)
            torch.cuda.synchronize()
            pms = e0.elapsed_time(e1) / args.decode_steps
            pooled = {"us_per_step": pms * 1e3, "state_GBps": dbytes / (pms * 1e-3) / 1e9,
                      "slots": N, "order": "random permutation"}
        dvariants = None
        if not args.no_configs:
            # the other variants' decode steps on the same shape and state
            dvariants = {}
            for vname in ("rda", "gdn2", "ckda"):
                wv = synth.preset(f"decode_{vname}", steps=4)
                vt = [dict(q=t(wv.q[i], True), k=t(wv.k[i], True), v=t(wv.v[i], True), alpha=t(wv.alpha[i]),
                           erase=t(wv.erase[i]), write=None if wv.write is None else t(wv.write[i])) for i in range(4)]
                del wv

                def vstep(i):
                    s_ = vt[i % 4]
                    drl.dr_decode_step(s_["q"], s_["k"], s_["v"], s_["alpha"], s_["erase"], s_["write"], vname, S, od)

                for i in range(10):
                    vstep(i)
                torch.cuda.synchronize()
                e0.record(stream)
                for i in range(args.decode_steps):
                    vstep(i)
                e1.record(stream)
                torch.cuda.synchronize()
                vus = e0.elapsed_time(e1) / args.decode_steps * 1e3
                vbytes = decode_bytes(N, HD, D, D, gate_bytes=(8 if vname == "rda" else 4 * (D + D) if vname == "gdn2" else 4))
                dvariants[vname] = {"us_per_step": vus, "state_GBps": vbytes / (vus * 1e-6) / 1e9,
                                    "hbm_frac": vbytes / (vus * 1e-6) / 1e9 / HBM_PEAK_GBS}
                del vt
        if prod is not None:
            # two transitions per token: the same state traffic, three column reductions
            wp = synth.make_product_decode("kda", N, HD, D, D, steps=4, in_dtype="bf16", seed=1006)
            ptoks = [dict(q=t(wp.q[i], True), k=t(wp.k[i], True), v=t(wp.v[i], True), alpha=t(wp.alpha[i]),
                          erase=t(wp.erase[i])) for i in range(4)]
            del wp

            def p2dstep(i):
                s = ptoks[i % 4]
                drl.dr_decode_step(s["q"], s["k"], s["v"], s["alpha"], s["erase"], None, "product2", S, od)

            for i in range(10):
                p2dstep(i)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(args.decode_steps):
                p2dstep(i)
            e1.record(stream)
            torch.cuda.synchronize()
            p2d = e0.elapsed_time(e1) / args.decode_steps
            p2bytes = dbytes + N * HD * (2 * D * 2 + 4)   # the second key, value and beta
            prod["decode"] = {"workload": "decode, two KDA transitions per token, 512 x 32 heads, d=128, 1 GiB "
                                          "fp32 state in place", "us_per_step": p2d * 1e3,
                              "state_GBps": p2bytes / (p2d * 1e-3) / 1e9,
                              "hbm_frac": p2bytes / (p2d * 1e-3) / 1e9 / HBM_PEAK_GBS}
            del ptoks
        decode = {
            "workload": "decode KDA, 512 sequences x 32 heads, d_k=d_v=128, fp32 state 1 GiB in place, bf16 q/k/v",
            "us_per_step": dms * 1e3,
            "p50_us": float(np.percentile(dper, 50) * 1e3), "p95_us": float(np.percentile(dper, 95) * 1e3),
            "p99_us": float(np.percentile(dper, 99) * 1e3), "percentiles_from": "a loop with an event after every step",
            "state_GBps": dbytes / (dms * 1e-3) / 1e9,
            "tokens_per_s": N / (dms * 1e-3),
            "hbm_frac": dbytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bytes_per_step": dbytes, "steps": args.decode_steps,
            "slot_pool": pooled,
            "other_variants": dvariants,
        }

    copy = copy_calibration(dev, mib=256, reps=3)
    props = torch.cuda.get_device_properties(dev)
    line = {
        "metric": "chunked fwd tokens/s (H=16,d=128,T=4096) + decode state GB/s, 1xMI355X",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "KDA chunked prefill B=4 T=4096 H=16 d_k=d_v=128, bf16 q/k/v, fp32 "
                               "gates/state/output, random S0, chunk 64",
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": D,
                   "dv_block": plan[1], "workgroups": plan[2]},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "dr_chunk_fwd: chunk_prep_kernel<128,bf16> then chunk_state_kernel<128,32,bf16>",
                     "alg_bytes_per_launch": alg_bytes, "traffic_per_kernel": kernel_traffic},
        "mfma": {"useful_tflops": flops / (ms_step * 1e-3) / 1e12,
                 "frac_of_bf16_peak": flops / (ms_step * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                 "useful_flop_per_launch": flops, "busy_frac_per_kernel": mfma_busy},
        "latency_ms": {"p50": float(np.percentile(per, 50)), "p95": float(np.percentile(per, 95)),
                       "p99": float(np.percentile(per, 99)), "mean": float(per.mean()),
                       "from": "a second loop with an event after every call"},
        "decode": decode,
        "step_recurrence": recurrence,
        "strided_inputs": strided,
        "stored_states": states,
        "fused_prep": fused,
        "backward": bwd,
        "product2": prod,
        "other_workloads": others,
        "measured_copy_GBps": copy["copy_GBps"],
        "run": {"gpu": props.name, "arch": getattr(props, "gcnArchName", ""),
                "cus": props.multi_processor_count, "torch": torch.__version__,
                "hip": getattr(torch.version, "hip", None), "wall_s_timed": wall, "settle_calls_before_warmup": SETTLE_CALLS, **conditions,
                "gpu_clocks_after_timing": clocks_after_timing},
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line))


if __name__ == "__main__":
    main()
