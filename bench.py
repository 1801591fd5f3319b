"""Throughput of one device's share of ZeCO causal linear attention on one MI355X.

A step is one pass of the whole per-device path over one batch of synthetic input at the
pages' per-device shape (B=1, H=16, L=16384, dk=dv=128, bf16, chunk 64, no decay), for a device
that receives the state S_recv (drawn N(0, 0.05) where the workload has one, else 0): the exact
outputs O and the outgoing state S_out = Lambda S_recv + S_loc.  The headline step computes them
with one la_chunk_fwd call from S_recv; inside it the library cuts the segment into G
sub-segments (G = 16 here, one workgroup each per head) and applies the ZeCO decomposition
between them:
  state pass       every sub-segment but the last: its local end state from zero (k, v read)
  la_state_scan    the scan over [S_recv, S_loc,1..G-1]: every sub-segment's exact incoming state
  output pass      every sub-segment from its exact incoming state: O, and S_out from the last
Alongside, the same result is timed in the pages' decomposed form (local forward of every
sub-segment from zero, the All-Scan over [S_recv, S_loc,1..G], output correction
O += (Q * cumulative decay) S_in), with the library's chained single launch (the state pass,
scan and output pass in one kernel, la_shape.fwd_schedule = 2), and with the pages' two-pass
schedule (every chunk's state stored, scanned and reloaded).
Prints one JSON line.  Per-kernel durations come from HIP events that the library records
around every kernel on the stream it launches them on (la_trace); the dominant kernel's
roofline uses its algorithmic bytes (q, k, v read + o written) over its mean duration.
Per-step statistics (median, mean, std, min) are given warm and cold (a 512 MiB buffer read
before each step evicts the 256 MB last-level cache; reading, not writing, so that the step does
not also pay for writing back someone else's dirty lines).  The head-decay and gate workloads
(B = 2 and 4) and the 1M-token 64-segment pass are timed alongside, unless --no-alongside.
Every workload is warmed up with at least ~20 ms of steps first: the GPU's clocks take about
10 ms of sustained work to settle (for the main step this runs before the --warmup steps and is
reported as clock_settle).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_output_pass_plain_B1_H16_L16k_d128.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(w, mode_bytes_gate: int):
    """Per token-head algorithmic bytes and flops of the local forward (q, k, v read, o written;
    QK^T, PV, QS and K^T V on full 64 x 64 chunk tiles)."""
    es = 2 if w.dtype == "bf16" else 4
    by = es * (2 * w.dk + 2 * w.dv) + mode_bytes_gate
    fl = 2 * w.chunk * w.dk + 2 * w.chunk * w.dv + 2 * w.dk * w.dv + 2 * w.dk * w.dv
    return by, fl


def live_correction_tokens(w, seg_len: int, nseg_corr: int, inp=None, step=None) -> int:
    """Tokens the correction actually touches.  Head decay: per segment and head, the 64-token
    tiles whose cumulative decay exp(lambda (64 i + 1)) at their first token is nonzero in fp32
    (the kernel's own test; the others' correction is exactly zero and they are skipped).  Gate
    decay: the tiles the forward flagged live in its last run (the correction skips the rest).
    No decay: every token."""
    import numpy as np

    total = w.B * w.H * seg_len * nseg_corr
    if w.mode == "gate" and step is not None and getattr(step, "live", None) is not None:
        flags = step.live[:, :, -nseg_corr:] if nseg_corr < step.live.shape[2] else step.live
        return min(total, int((flags != 0).sum().item()) * 64)
    if w.mode != "head" or inp is None:
        return total
    lam = inp["decay"].float().cpu().numpy()
    tiles = (seg_len + 63) // 64
    tau0 = (np.arange(tiles, dtype=np.float32) * 64 + 1).astype(np.float32)
    live = 0
    for h in range(w.H):
        with np.errstate(under="ignore"):
            alive = np.exp(np.float32(lam[h]) * tau0) != 0
        n = int(alive.sum())
        live += min(n * 64, seg_len)
    return w.B * live * nseg_corr


def split_plan(w):
    """(G, chunks per sub-segment) of the library's split of one segment for the bf16 matrix-core
    forward with 64-token chunks: about 256 workgroups at dk = 128 (512 below), at least four
    chunks per sub-segment (the same rule as fwd_split_plan in chunk_fwd_split.hip; used here
    for byte accounting only)."""
    units = w.B * w.H * w.nseg
    nch = -(-(w.L // w.nseg) // 64)
    g_want = -(-(256 if w.dk >= 128 else 512) // units)
    cps = min(max(4, -(-nch // g_want)), nch)
    return -(-nch // cps), cps


def kernel_roofline(w, step, kernels, inp=None):
    """Adds algorithmic bytes per launch, achieved GB/s and the fraction of the 8 TB/s peak to the
    forward's output pass, the state scan and the correction (their per-unit figures: q, k, v read
    and o written (+ g in gate mode) per token-head; P states read and written (+ their decay
    vectors); q read and o read and written per corrected token-head, plus the incoming states)."""
    es = 2 if w.dtype == "bf16" else 4
    bh = w.B * w.H
    state = w.dk * w.dv * 4
    nseg = getattr(step, "nseg", None)
    if hasattr(step, "schedule"):  # one exact call: state pass over G - 1 sub-segments, scan over G - 1
        G, cps = split_plan(w)
        fwd = w.B * w.H * w.L * (es * (2 * w.dk + 2 * w.dv) + (4 * w.dk if w.mode == "gate" else 0))
        spass = bh * (G - 1) * (cps * 64 * es * (w.dk + w.dv) + state + 4 * w.dk)
        scan = bh * (G - 1) * (2 * state + (4 * w.dk if w.mode != "none" else 0))
        for name, d in kernels.items():
            by = None if "redo" in name else fwd if name.endswith("_output_pass") else \
                spass if name.endswith("_state_pass") else scan if name == "state_scan" else None
            if by is not None and d["launches_per_step"] == 1:
                gbs = by / (d["mean_us"] * 1e-6) / 1e9
                d.update(algorithmic_bytes=by, gbps=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4))
        return
    if nseg is None:  # device step: G sub-segments, scan over G + 1 entries, every live token corrected
        P, nstates = step.G + 1, step.G
        corrected = live_correction_tokens(w, w.L // step.G, step.G, inp, step)
    else:             # segmented pass: P segments, the live tokens of segments 1.. corrected
        P, nstates = nseg, nseg - 1
        corrected = live_correction_tokens(w, w.L // nseg, nseg - 1, inp, step)
    fwd = w.B * w.H * w.L * (es * (2 * w.dk + 2 * w.dv) + (4 * w.dk if w.mode == "gate" else 0))
    scan = bh * P * (2 * state + (4 * w.dk if w.mode != "none" else 0))
    corr = corrected * es * (w.dk + 2 * w.dv) + bh * nstates * state
    for name, d in kernels.items():
        # the gate mode's redo launch reruns only flagged units (none in these workloads): no figure
        by = None if "redo" in name else fwd if name.endswith("_output_pass") else \
            scan if name == "state_scan" else corr if name.startswith("state_correct") else None
        if by is None:
            continue
        if name == "state_scan" and d["launches_per_step"] > 1:
            continue  # more than one scan per step (an internal split): no single figure
        gbs = by / (d["mean_us"] * 1e-6) / 1e9
        d.update(algorithmic_bytes=by, gbps=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4))


class BackwardStep:
    """One backward pass (la_chunk_bwd) over a workload's inputs with seeded d_o and ds_out; with
    ``want_decay`` also the decay derivative (learned decays), else the decays are held fixed.
    Outputs are allocated once."""

    def __init__(self, w, want_decay=False, forward_states=False):
        import torch

        from chunked_scan_amd.inputs import make_grads, make_inputs
        from chunked_scan_amd.pipeline import DeviceStep

        self.w = w
        self.inp = make_inputs(w, "cuda")
        self.gr = make_grads(w, device="cuda")
        self.dq = torch.empty_like(self.inp["q"])
        self.dk = torch.empty_like(self.inp["k"])
        self.dv = torch.empty_like(self.inp["v"])
        self.want_decay = want_decay and w.mode != "none"
        self.s_sub, self.sub_len = None, 0
        if forward_states:  # training order: the device step's scan buffer (s_in as S_recv) is reused
            i = self.inp
            step = DeviceStep(i["q"], i["k"], i["v"], i["decay"], i["s_in"], mode=w.mode, chunk=w.chunk,
                              gate_norm=w.gate_norm)
            step.run()
            torch.cuda.synchronize()
            self.s_sub, self.sub_len = step.states[:, :, :step.G], w.L // step.G
            self._keep = step

    def run(self, timers=None):
        from chunked_scan_amd import binding

        i, g = self.inp, self.gr
        binding.la_chunk_bwd(i["q"], i["k"], i["v"], g["d_o"], i["decay"], i["s_in"], g["ds_out"], mode=self.w.mode,
                             chunk=self.w.chunk, want_decay=self.want_decay, dq=self.dq, dk=self.dk, dv=self.dv,
                             s_sub=self.s_sub, sub_len=self.sub_len, timer=(timers or {}).get("fwd"))


def backward_legs(stream):
    """la_chunk_bwd at the plain (B=1), head-decay (B=2) and gate (B=4) shapes, decays fixed, and at
    the head-decay and gate shapes with the decay derivative (learned decays): median time, tokens/s,
    GB/s on the compulsory bytes (q, k, v, d_o and the gate read once, dq, dk, dv and dg written once)
    and per-kernel means."""
    import torch

    from chunked_scan_amd.inputs import WORKLOADS

    backward = {}
    legs = ((1, False, False), (2, False, False), (2, True, False), (3, False, False), (3, True, False),
            (1, False, True), (2, True, True), (3, True, True))
    for wid, want_decay, fstates in legs:
        wb = WORKLOADS[wid]
        dname = "dg" if wb.mode == "gate" else "d_lambda"
        key = wb.name + (f" + {dname}" if want_decay else "") + (", forward's sub-segment states" if fstates else "")
        log(f"[bench] backward: workload {wid} {key}")
        sb = BackwardStep(wb, want_decay, fstates)
        for _ in range(60):  # >= 20 ms of work: settled clocks
            sb.run()
        torch.cuda.synchronize()
        st = step_stats(sb, 30, stream)
        ks, _ = kernel_stats(sb, 30, stream, capacity=16)
        th = wb.B * wb.H * wb.L
        # algorithmic bytes per token-head of each pass (bf16, d = 128): state passes read two tensors,
        # the dq and d lambda output passes read three or four, the dk/dv output pass reads four and
        # writes two; in gate mode the dq and dk/dv passes also read the fp32 gate row (4 d bytes)
        gate = 4 * wb.dk if wb.mode == "gate" else 0
        # the gate derivative: D at every chunk's start (bf16 d x d per 64 tokens) written by the dk/dv
        # pass and read by the dq pass; chunk_bwd_dg reads q, k, dq, dk and the gate, writes dg
        dstart = 2 * wb.dk * wb.dv // 64 if (gate and want_decay) else 0
        per_th = {"chunk_bwd_dq_state_pass": 512 + gate, "chunk_bwd_dq": 1024 + gate + dstart,
                  "chunk_bwd_dkdv_state_pass": 512 + gate, "chunk_bwd_dkdv": 1536 + gate + dstart,
                  "chunk_bwd_dlam_state_pass": 512, "chunk_bwd_dlam": 1024,
                  "chunk_bwd_dg": 8 * wb.dk + 2 * gate}
        for name, d in ks.items():
            if name in per_th and d["launches_per_step"] == 1:
                by = per_th[name] * th
                g = by / (d["mean_us"] * 1e-6) / 1e9
                d.update(algorithmic_bytes=by, gbps=round(g, 1), hbm_frac=round(g / HBM_PEAK_GBS, 4))
        # compulsory bytes (bf16): q, k, v, d_o (and the fp32 gate) read once, dq, dk, dv (and dg) written once
        comp = th * 2 * (wb.dk + wb.dk + wb.dv + wb.dv) + th * 2 * (wb.dk + wb.dk + wb.dv) + th * gate
        if gate and want_decay:
            comp += th * gate
        gbs = comp / (st["median_us"] * 1e-6) / 1e9
        backward[key] = dict(
            what=("la_chunk_bwd_states" if fstates else "la_chunk_bwd") + ": dq, dk, dv, ds_in"
            + (f", {dname}" if want_decay else " (decay held fixed)")
            + (" (the states entering the sub-segments from the device step's scan)" if fstates else ""),
            B=wb.B, H=wb.H, L=wb.L, decay=wb.decay,
            tokens_per_s=round(wb.B * wb.L / (st["median_us"] * 1e-6), 1), per_step_us=st,
            compulsory_bytes=comp, gbps_on_compulsory_bytes=round(gbs, 1),
            hbm_frac_on_compulsory_bytes=round(gbs / HBM_PEAK_GBS, 4),
            kernels={n: {k: round(v, 2) for k, v in d.items()} for n, d in ks.items()})
        log(f"[bench]   backward {key}: median {st['median_us']:.1f} us, "
            f"{backward[key]['tokens_per_s']:.3e} tokens/s, {gbs:.0f} GB/s on compulsory bytes; " +
            ", ".join(f"{n} {d['mean_us']:.1f} us" for n, d in ks.items()))
        del sb
        torch.cuda.empty_cache()
    return backward


def copy_rate_gbs(mib: int = 1024, reps: int = 10) -> float:
    """This GPU's rate for a plain device-to-device copy of ``mib`` MiB (bytes read + written over
    time, median of ``reps``): context for the roofline fraction, whose peak is the datasheet's."""
    import statistics

    import torch

    a = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    del a, b
    torch.cuda.empty_cache()
    return round(2 * mib * (1 << 20) / statistics.median(ts) / 1e9, 1)


def step_stats(step, steps, stream, scratch=None):
    """Per-step times (us) with events around each step; with ``scratch``, the buffer is read
    before every step so that the step starts with a cold last-level cache."""
    import statistics

    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        if scratch is not None:
            scratch.sum()
        a.record(stream)
        step.run()
        b.record(stream)
    torch.cuda.synchronize()
    t = [1e3 * a.elapsed_time(b) for a, b in evs]
    return dict(median_us=round(statistics.median(t), 2), mean_us=round(statistics.mean(t), 2),
                std_us=round(statistics.pstdev(t), 2), min_us=round(min(t), 2))


def kernel_stats(step, steps, stream, capacity=8):
    """Mean duration of every library kernel over ``steps`` steps, from the events the library
    records around each kernel on its stream."""
    import torch

    from chunked_scan_amd import binding

    timers = [{c: binding.KernelTimer(capacity) for c in ("fwd", "cum", "scan", "corr")} for _ in range(steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        step.run(timers=timers[i])
    e1.record(stream)
    torch.cuda.synchronize()
    per_kernel = {}
    for tset in timers:
        for c in ("fwd", "cum", "scan", "corr"):
            for name, ms in tset[c].harvest():
                per_kernel.setdefault(name, []).append(ms)
    kernels = {n: dict(mean_us=1e3 * sum(v) / len(v), launches_per_step=len(v) / steps, min_us=1e3 * min(v))
               for n, v in per_kernel.items()}
    return kernels, e0.elapsed_time(e1) / steps


def epsilon(w, inp, stream, steps: int = 20):
    """The single-GPU analogue of the reviewers' overhead question on this workload: the same
    exact result (O and S_out from S_recv) four ways, each step timed with events (median us).
      decomposed        the pages' device step: local forward of every sub-segment from zero, the
                        All-Scan over [S_recv, S_loc,1..G], output correction by each S_in
      recv_first        the decomposed step with S_recv as the first sub-segment's initial state
                        (no correction of that sub-segment)
      exact_passes      one la_chunk_fwd from S_recv (state pass, scan, output pass from the exact
                        incoming states; no correction)
      exact_chained     the same in one launch with the chained state hand-off (where it exists)
      two_pass_chunk_states  la_chunk_fwd from S_recv with every chunk's state stored to HBM, scanned
                        and reloaded (the pages' two-pass schedule, one sub-segment per chunk)"""
    import torch

    from chunked_scan_amd import binding
    from chunked_scan_amd.pipeline import DeviceStep, ExactStep, RecvFirstStep

    kw = dict(mode=w.mode, chunk=w.chunk, gate_norm=w.gate_norm)
    args = (inp["q"], inp["k"], inp["v"], inp["decay"], inp["s_in"])
    chained = w.dtype == "bf16" and w.dk == w.dv == 128 and w.chunk == 64 and w.mode != "gate"
    # (the output correction takes head dims up to 128: no decomposed step at d = 256)
    forms = {"decomposed": DeviceStep(*args, **kw) if w.dk <= 128 else None,
             "recv_first": RecvFirstStep(*args, **kw) if w.dk <= 128 else None,
             "exact_passes": ExactStep(*args, schedule="passes", **kw),
             "exact_chained": ExactStep(*args, schedule="chained", **kw) if chained else None,
             "two_pass_chunk_states": ExactStep(*args, schedule="passes", subseg_chunks=1, **kw)}
    live = {k: st for k, st in forms.items() if st is not None}
    for st in live.values():  # every form's buffers touched before any is timed
        for _ in range(3):
            st.run()
    torch.cuda.synchronize()
    # two rounds over the forms, the better median of each: a form's time does not depend on
    # where in the region it falls
    out = {k: None for k in forms}
    for _ in range(2):
        for k, st in live.items():
            t = step_stats(st, steps, stream)["median_us"]
            out[k] = t if out[k] is None else min(out[k], t)
    if chained:
        binding.la_chain_status()  # raises if a chained wave gave up on a wait (NaN outputs)
    return out


def state_size_sweep(stream):
    """The falsifier's question asked on one GPU: how the decomposition's cost (the decomposed
    device step against one exact forward call, both on the same inputs) moves with the state size
    dk x dv at a fixed token count (B1 H16 L16384, bf16, no decay, S_recv drawn N(0, 0.05)), d = 32
    to 256.  Median us.  For d = 32, 64 and 128 also the exact step with 128-token chunks (the
    chunk-length variant); d = 256 has no decomposed step and no backward."""
    import math

    import torch

    from chunked_scan_amd.inputs import WORKLOADS, make_inputs
    from chunked_scan_amd.pipeline import DeviceStep, ExactStep

    out = {}
    for d in (32, 64, 128, 256):
        w = WORKLOADS[1].scaled(dk=d, dv=d, qkv_std=1.0 / math.sqrt(d), s_in_std=0.05, seed=10 + d)
        inp = make_inputs(w, "cuda")
        step = ExactStep(inp["q"], inp["k"], inp["v"], inp["decay"], inp["s_in"], mode=w.mode, chunk=w.chunk)
        for _ in range(150):  # >= 20 ms of work: settled clocks
            step.run()
        torch.cuda.synchronize()
        eps = epsilon(w, inp, stream, steps=30)
        ks, _ = kernel_stats(step, 30, stream)
        bwd = None
        if d <= 128:
            bw = BackwardStep(w)
            for _ in range(40):
                bw.run()
            torch.cuda.synchronize()
            bwd = step_stats(bw, 20, stream)["median_us"]
            del bw
        c128 = None
        if d <= 128:
            s128 = ExactStep(inp["q"], inp["k"], inp["v"], inp["decay"], inp["s_in"], mode=w.mode, chunk=128)
            for _ in range(150):
                s128.run()
            torch.cuda.synchronize()
            c128 = step_stats(s128, 30, stream)["median_us"]
            del s128
        dec = eps["decomposed"]
        out[f"d{d}"] = dict(state_bytes=4 * d * d, decomposed_step_us=dec, chunk128_step_us=c128,
                            exact_step_us=eps["exact_passes"], exact_chained_us=eps["exact_chained"],
                            decomposition_overhead_us=round(dec - eps["exact_passes"], 2) if dec else None,
                            decomposition_overhead_frac=round(dec / eps["exact_passes"] - 1, 4) if dec else None,
                            backward_us=bwd,
                            kernels={n: round(v["mean_us"], 2) for n, v in ks.items()})
        log(f"[bench] state size d={d}: " + (f"decomposed step {dec:.1f} us, " if dec else "")
            + f"one exact call {eps['exact_passes']:.1f} us"
            + (f" (128-token chunks {c128:.1f} us)" if c128 else "")
            + (f" (chained {eps['exact_chained']:.1f} us)" if eps["exact_chained"] else "")
            + (f", backward {bwd:.1f} us" if bwd else "") + "; "
            + ", ".join(f"{n} {v['mean_us']:.1f}" for n, v in ks.items()))
        del step, inp
        torch.cuda.empty_cache()
    return out


def host_cpu():
    """(threads to use, cores in this process's affinity mask, CPU model name): the oracle runs on
    every core of the affinity mask, or on the job's CPU share when OMP_NUM_THREADS states one."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = os.cpu_count() or 1
    threads = aff
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and 0 < int(share) < aff:
        threads = int(share)
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.lower().startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return threads, aff, model


def cpu_baseline(w, inp):
    import numpy as np
    import torch

    import oracle
    from oracle import HEAD, NONE, GATE

    threads, aff, model = host_cpu()
    f32 = lambda t: None if t is None else t.to("cpu", torch.float32).numpy()  # noqa: E731
    q, k, v = f32(inp["q"]), f32(inp["k"]), f32(inp["v"])
    mode = {"none": NONE, "head": HEAD, "gate": GATE}[w.mode]
    s_in = None if inp["s_in"] is None else f32(inp["s_in"]).astype(np.float64)
    oracle.build(force=False)
    # the whole workload is the sample; it is repeated until about 10 s of CPU time have passed
    reps, t0 = 0, time.perf_counter()
    while True:
        o_ref, s_ref = oracle.recurrence(q, k, v, mode, f32(inp["decay"]), s_in, threads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 100:
            break
    items = w.B * w.H * ((w.dv + 15) // 16)
    used = min(threads, items)
    return dict(value=reps * w.B * w.L / dt, unit="tokens/s", cores=used, kind="oracle",
                affinity_cores=aff, cpu_model=model,
                sample=f"whole workload (B={w.B} H={w.H} L={w.L} d={w.dk}) x {reps} repetitions, fp64 "
                       f"token-by-token recurrence in C, {dt:.1f} s on {used} threads ({aff} cores in the "
                       f"affinity mask; {model})"), (o_ref, s_ref)


def cpu_baseline_backward(w, sample_len: int = 2048):
    """The fp64 oracle's backward (token by token, whole state trajectory kept) timed on a bounded
    sample of workload ``w``: every head, the first ``sample_len`` tokens, d_o and ds_out seeded as
    on the GPU; repeated to about 5 s.  tokens/s = repetitions x B x sample_len / seconds."""
    import numpy as np
    import torch

    import oracle
    from oracle import HEAD, NONE, GATE
    from chunked_scan_amd.inputs import make_grads, make_inputs

    ws = w.scaled(L=sample_len)
    inp = make_inputs(ws, "cpu")
    gr = make_grads(ws)
    threads, aff, model = host_cpu()
    f32 = lambda t: None if t is None else t.to(torch.float32).numpy()  # noqa: E731
    mode = {"none": NONE, "head": HEAD, "gate": GATE}[w.mode]
    s_in = None if inp["s_in"] is None else f32(inp["s_in"]).astype(np.float64)
    ds_out = f32(gr["ds_out"]).astype(np.float64)
    oracle.build(force=False)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.recurrence_bwd(f32(inp["q"]), f32(inp["k"]), f32(inp["v"]), f32(gr["d_o"]), mode, f32(inp["decay"]),
                              s_in, ds_out, threads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 5.0 or reps >= 100:
            break
    used = min(threads, ws.B * ws.H)
    return dict(value=reps * ws.B * sample_len / dt, unit="tokens/s", cores=used, kind="oracle",
                affinity_cores=aff, cpu_model=model,
                sample=f"backward of B={ws.B} H={ws.H} d={ws.dk}, first {sample_len} tokens x {reps} repetitions, "
                       f"fp64 token-by-token derivatives in C, {dt:.1f} s on {used} threads ({model})")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400,
                    help="untimed steps first; the GPU's clocks take ~10 ms of sustained work to settle")
    ap.add_argument("--workload", type=int, default=1, help="index into chunked_scan_amd.inputs.WORKLOADS")
    ap.add_argument("--step", choices=("auto", "exact", "decomposed", "recv_first", "chained"), default="auto",
                    help="form of the device step (one-segment workloads): one exact la_chunk_fwd from S_recv "
                         "(the library's separate passes, or its chained single launch), or the pages' local "
                         "forward + All-Scan + output correction (recv_first: with S_recv taken in by the first "
                         "sub-segment, whose correction then drops); auto = the faster on MI355X: exact without "
                         "decay and with head decay, recv_first with the gate (its correction skips the tiles "
                         "whose cumulative decay has underflowed)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-alongside", action="store_true",
                    help="skip the decay and segmented workloads and the three-way comparison reported next "
                         "to the headline")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the backward legs (la_chunk_bwd at the plain and head-decay shapes) and exit; "
                         "prints their JSON")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this path runs on one "
              "GPU and needs no collectives).", file=sys.stderr)
        sys.exit(2)

    import torch

    from chunked_scan_amd import binding, profsum
    from chunked_scan_amd.inputs import WORKLOADS, make_inputs
    from chunked_scan_amd.pipeline import DeviceStep, ExactStep, RecvFirstStep, SegmentedForward

    def form_of(wx):
        if args.step == "auto":
            return "recv_first" if wx.mode == "gate" else "exact"
        return "exact" if args.step == "chained" and wx.mode == "gate" else args.step

    def one_segment_step(wx, ix, form):
        a = (ix["q"], ix["k"], ix["v"], ix["decay"], ix["s_in"])
        kw = dict(mode=wx.mode, chunk=wx.chunk, gate_norm=wx.gate_norm)
        if form == "decomposed":
            return DeviceStep(*a, **kw)
        if form == "recv_first":
            return RecvFirstStep(*a, **kw)
        return ExactStep(*a, schedule="chained" if form == "chained" else "auto", **kw)

    torch.cuda.set_device(0)
    if args.calib_copy_mib:  # counter runs (chunked_scan_amd.profsum) scale FETCH/WRITE_SIZE by this copy
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        torch.cuda.empty_cache()
        log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done")
    if args.backward_only:
        print(json.dumps(dict(backward=backward_legs(torch.cuda.current_stream()))))
        return
    w = WORKLOADS[args.workload]
    log(f"[bench] workload {args.workload} {w.name}: generating inputs on cuda:0")
    inp = make_inputs(w, "cuda")
    if w.nseg == 1:
        step = one_segment_step(w, inp, form_of(w))
    else:  # a sequence split into segments, all on this device: the All-Scan as a segmented scan
        if not args.no_cpu_baseline:
            raise SystemExit("the CPU baseline is timed on the one-segment device step only")
        step = SegmentedForward(inp["q"], inp["k"], inp["v"], inp["decay"], inp["s_in"], mode=w.mode,
                                nseg=w.nseg, chunk=w.chunk, gate_norm=w.gate_norm)
    stream = torch.cuda.current_stream()
    # reading this buffer evicts the 256 MB last-level cache before a "cold" step
    scratch = torch.ones(512 << 18, dtype=torch.float32, device="cuda")

    # Clocks: the GPU reaches its sustained clocks only after ~10 ms of continuous work (the plain
    # step runs ~10% slower for its first ~100 steps), so before the W warm-up steps the step runs
    # untimed for at least 20 ms of GPU time; the figure is reported as clock_settle.
    settle_ms, settle_steps = 0.0, 0
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    while settle_ms < 20.0 and settle_steps < 4000:
        s0.record(stream)
        for _ in range(10):
            step.run()
        s1.record(stream)
        s1.synchronize()
        settle_ms += s0.elapsed_time(s1)
        settle_steps += 10
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    log(f"[bench] clocks settled over {settle_steps} steps ({settle_ms:.1f} ms); warmup {args.warmup} done")

    # --- every step bracketed by its own events (warm: back to back on the same inputs)
    warm = step_stats(step, args.steps, stream)

    # --- the headline: K steps back to back as a user runs them (no per-kernel events)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step.run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step")

    # --- the same steps with HIP events around every kernel (la_trace)
    kernels, ms_traced = kernel_stats(step, args.steps, stream)
    kernel_roofline(w, step, kernels, inp)
    log("[bench] per kernel: " + ", ".join(f"{n} {d['mean_us']:.1f} us" + (f" ({d['hbm_frac']:.2f} of HBM peak)"
                                                                         if "hbm_frac" in d else "")
                                          for n, d in kernels.items()))

    # --- cold: the last-level cache evicted before every step (last: the 512 MiB reads between
    # steps change the GPU's power state for the regions after them)
    cold = step_stats(step, args.steps, stream, scratch)
    if w.nseg == 1 and form_of(w) == "chained":
        binding.la_chain_status()  # raises if a chained wave gave up on a wait (NaN outputs)
    log(f"[bench] per step: warm median {warm['median_us']:.1f} us, cold median {cold['median_us']:.1f} us")

    eps = None
    if w.nseg == 1 and not args.no_alongside:
        eps = epsilon(w, inp, stream)
        log("[bench] same result three ways (median us/step): " + ", ".join(f"{k} {v:.1f}" for k, v in eps.items()))

    alongside = {}
    if not args.no_alongside:
        for wid in (2, 3, 4):
            if wid == args.workload:
                continue
            wa = WORKLOADS[wid]
            log(f"[bench] alongside: workload {wid} {wa.name}")
            ia = make_inputs(wa, "cuda")
            if wa.nseg == 1:
                sa = one_segment_step(wa, ia, form_of(wa))
            else:
                sa = SegmentedForward(ia["q"], ia["k"], ia["v"], ia["decay"], ia["s_in"], mode=wa.mode,
                                      nseg=wa.nseg, chunk=wa.chunk, gate_norm=wa.gate_norm)
            for _ in range(4 if wa.nseg > 1 else 100):  # >= 20 ms of work: settled clocks
                sa.run()
            torch.cuda.synchronize()
            n_al = 10 if wa.nseg > 1 else 50
            st = step_stats(sa, n_al, stream)
            ks, _ = kernel_stats(sa, n_al, stream)
            kernel_roofline(wa, sa, ks, ia)
            alongside[wa.name] = dict(
                step=("segmented pass over %d segments" % wa.nseg) if wa.nseg > 1 else f"device step ({form_of(wa)})",
                B=wa.B, H=wa.H, L=wa.L, decay=wa.decay, tokens_per_s=round(wa.B * wa.L / (st["median_us"] * 1e-6), 1),
                per_step_us=st, kernels={n: {k: round(v, 2) for k, v in d.items()} for n, d in ks.items()})
            if wa.nseg == 1:  # the same result in the other forms
                alongside[wa.name]["same_result_us"] = epsilon(wa, ia, stream, steps=20)
            log(f"[bench]   {wa.name}: median {st['median_us']:.1f} us/step, "
                f"{alongside[wa.name]['tokens_per_s']:.3e} tokens/s; " +
                ", ".join(f"{n} {d['mean_us']:.1f} us" for n, d in ks.items()))
            del sa, ia
            torch.cuda.empty_cache()

    backward = {}
    sweep = {}
    if not args.no_alongside:
        backward = backward_legs(stream)
        if not args.no_cpu_baseline and WORKLOADS[1].name in backward:
            log("[bench] backward cpu_baseline (oracle, bounded sample)")
            backward[WORKLOADS[1].name]["cpu_baseline"] = cpu_baseline_backward(WORKLOADS[1])
        sweep = state_size_sweep(stream)

    tokens = w.B * w.L
    gate_bytes = 4 * w.dk if w.mode == "gate" else 0
    by_tok, fl_tok = algorithmic(w, gate_bytes)
    dom = max(kernels, key=lambda n: kernels[n]["mean_us"] * kernels[n]["launches_per_step"])
    dom_us = kernels[dom]["mean_us"]
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_sha256_16") == profsum.source_hash() and tr.get("workload") == w.name and tr.get("kernel") == dom:
            traffic = tr["bytes_per_launch"]
    alg_bytes = tokens * w.H * by_tok if dom.endswith("_output_pass") else None
    roof = None
    if alg_bytes is not None:
        achieved = alg_bytes / (dom_us * 1e-6) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic, kernel=dom,
                    kernel_mean_us=round(dom_us, 2), algorithmic_bytes=alg_bytes,
                    mfma_frac=round(tokens * w.H * fl_tok / (dom_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                    measured_copy_GBps=copy_rate_gbs())
        # the whole step against the same peak: every kernel's algorithmic bytes, and the compulsory
        # bytes (each input read once, each output written once), over the back-to-back step time
        step_bytes = sum(int(d["algorithmic_bytes"] * d["launches_per_step"]) for d in kernels.values()
                         if "algorithmic_bytes" in d)
        es = 2 if w.dtype == "bf16" else 4
        compulsory = tokens * w.H * (es * (2 * w.dk + 2 * w.dv) + (4 * w.dk if w.mode == "gate" else 0))
        step_s = ms_per_step * 1e-3
        roof["step"] = dict(algorithmic_bytes=step_bytes, frac=round(step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
                            compulsory_bytes=compulsory,
                            compulsory_frac=round(compulsory / step_s / 1e9 / HBM_PEAK_GBS, 4))

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        cpu, (o_ref, s_ref) = cpu_baseline(w, inp)
        o, s_out = step.run()
        torch.cuda.synchronize()
        import numpy as np
        err_o = float(np.max(np.abs(o.float().cpu().numpy() - o_ref)) / np.max(np.abs(o_ref)))
        err_s = float(np.max(np.abs(s_out.cpu().numpy() - s_ref[:, :, 0])) / max(np.max(np.abs(s_ref)), 1e-30))
        cpu["parity_err_o"], cpu["parity_err_s"] = err_o, err_s
        log(f"[bench] oracle {cpu['value']:.3e} tokens/s; full-size parity err O {err_o:.2e} S {err_s:.2e}")

    out = {
        "metric": "tokens/s per GPU, linear-attn fwd (L=16k,H=16,dk=128) + % MFMA/HBM peak",
        "value": round(tokens / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": ({"exact": f"{w.name}: device step = exact O and S_out from S_recv in one la_chunk_fwd "
                                          f"call (sub-segment state pass, scan with S_recv as its first entry, "
                                          f"output pass from the exact incoming states)",
                                 "chained": f"{w.name}: device step = exact O and S_out from S_recv in one chained "
                                            f"launch (state pass, flag hand-off scan, output pass)",
                                 "decomposed": f"{w.name}: device step = local chunked fwd + All-Scan state combine "
                                               f"+ output correction",
                                 "recv_first": f"{w.name}: device step = local chunked fwd with S_recv taken in by the "
                                               f"first sub-segment + All-Scan state combine + output correction of "
                                               f"the others"}[form_of(w)]) if w.nseg == 1 else
                               (f"{w.name}: {w.nseg} segments on one device = local chunked fwd + segmented "
                                f"state scan + output correction"), "B": w.B, "H": w.H, "L": w.L, "dk": w.dk, "dv": w.dv,
                   "chunk": w.chunk, "decay": w.decay, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_step_us": {"warm": warm, "cold": cold},
        "kernels": {n: {k: round(v, 2) for k, v in d.items()} for n, d in kernels.items()},
        "ms_per_step_with_kernel_events": round(ms_traced, 5),
        "clock_settle": {"steps": settle_steps, "ms": round(settle_ms, 2)},
        "overhead_one_gpu_us": eps,
        "alongside": alongside,
        "backward": backward,
        "state_size_sweep": sweep,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
