"""Benchmark: striped ring-attention forward on one MI355X.

One step = original-order Q, K, V -> striped device layout -> all N ring
rounds -> O and LSE back in original order. With --order device (the default
at 262,144 and 786,432 tokens) the step runs the explicit gather kernels:
stripe_permute Q, K, V; the ring on device-layout tensors, each device's
stripe contiguous as on a real ring; unstripe O and LSE. With --order
original (the default at the shorter lengths) it is one launch: the ring
kernel addresses device d's j-th token at its position j*N + d, so the
stripe permutation and its inverse are folded into its row addressing. The
other form is timed alongside either way. Inputs are resident in
HBM before the timed region. The ring runs with the fused schedule by
default (one launch walks every (round, key tile) pair, the log-sum-exp
merge done online); the per-round schedule (one launch per ring round, merge
fused in its epilogue) and the contiguous layout are timed alongside. Prints
one JSON line.

value  = useful causal TFLOP/s of the whole step: 4*Dh flops per live causal
         pair, B*H*S*(S+1)/2 pairs per step (masked pairs inside partial
         tiles and skipped tiles are not counted).
roofline = the ring attention kernel (the dominant kernel): useful flops of
         every launch in the timed region / the sum of their durations, from
         HIP events recorded on the launch stream around each launch, against
         the bf16 dense MFMA peak.
Timing: the default warm-up and step counts depend on the workload (Short:
300 untimed, then 300 timed steps) so that the timed region runs at the
GPU's sustained clocks; each secondary section is preceded by at least
~0.15 s of the same work, and short kernels are timed behind queued GPU work.
cpu_baseline = the CPU oracle (fp64 numpy causal attention, oracle.attention_rows)
         on a bounded sample of the same workload: 64-row blocks of one head
         at fixed, evenly spaced positions, visited in a fixed order until
         about --cpu-seconds of work; its useful TFLOP/s is extrapolated to the
         whole forward by useful-pair count.
The default workload is the longest one (786,432 tokens, 32 heads, 16 ring
devices, forward plus backward): --steps and --warmup count its forward
launches; the backward is timed in the same run over a few calls and
reported with its own roofline fraction, and the secondary sections (other
schedule, contiguous layout, device order, simulated ring) use few steps.
"""

import argparse
import hashlib
import json
import statistics
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "useful causal attn TFLOP/s + % bf16 MFMA peak; striped vs contiguous max/mean"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published

FWD_KERNEL_SOURCES = ("attn_fwd.hip", "kernel_common.h", "sra_internal.h")
# HBM traffic of one fused forward launch (striped, tensors in the order
# named) per workload, from rocprofv3 FETCH_SIZE and WRITE_SIZE passes scaled
# by the same counters on the stripe-permute copy kernel of known size;
# filled in from the counter summaries under profiles/ and valid only for the
# kernel sources they were taken on.
TRAFFIC = [
    {"workload": "very_long", "order": "device",
     "kernel_sources_sha256": "951c1a8b95bee521cb70eb772cc448b5370a07eb045a792c7e4754302ce77b22",
     "bytes_per_launch": 2027301211163,
     "fetch_bytes_per_launch": 2020054931994, "write_bytes_per_launch": 7246279168,
     "copy_scale": {"FETCH_SIZE": 1.99999, "WRITE_SIZE": 1.00000}},
    {"workload": "very_long", "order": "original",
     "kernel_sources_sha256": "951c1a8b95bee521cb70eb772cc448b5370a07eb045a792c7e4754302ce77b22",
     "bytes_per_launch": 5340605878429,
     "fetch_bytes_per_launch": 5333423112820, "write_bytes_per_launch": 7182765609,
     "copy_scale": {"FETCH_SIZE": 1.99999, "WRITE_SIZE": 1.00000}},
]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default per workload: about 0.1-1 s of timed GPU work)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before them (default per workload: past the clock ramp)")
    ap.add_argument("--workload", default="very_long",
                    help="tiny/short/mid/long/very_long (default: very_long, the longest single-GPU shape)")
    ap.add_argument("--seq", type=int, default=None,
                    help="override the workload's sequence length (the JSON then names the workload '<name>+override')")
    ap.add_argument("--heads", type=int, default=None, help="override the workload's head count")
    ap.add_argument("--layout", default="striped", choices=["striped", "contiguous"])
    ap.add_argument("--schedule", default="fused", choices=["fused", "per_round"],
                    help="ring schedule of the timed step (the other one is timed alongside)")
    ap.add_argument("--order", default=None, choices=["original", "device"],
                    help="original: q, k, v, o, lse in token order, the stripe permutation folded into the ring "
                         "kernel's row addressing (one launch per step); device: gather into the striped "
                         "device layout, ring, gather back (the other one is timed alongside). Default per "
                         "workload: device for Long and Very long, original otherwise")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time for cpu_baseline")
    ap.add_argument("--sec-steps", type=int, default=None,
                    help="timed steps of each secondary section (default per workload)")
    ap.add_argument("--bwd-steps", type=int, default=None, help="timed backward calls (default per workload)")
    ap.add_argument("--no-compare", action="store_true", help="skip the other-schedule and contiguous runs")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-critical-path", action="store_true",
                    help="skip the per-(device, round) timing of the simulated ring")
    return ap.parse_args()


# Default (timed steps, warm-up steps) per workload. After an idle period the
# GPU's clocks take ~50 ms of back-to-back work to reach their sustained level
# (a Short forward launch takes 330-380 us over its first 40 launches, then a
# steady ~300 us for as long as it runs), so the warm-up spans >= 100 ms and
# the timed region measures the sustained rate.
DEFAULT_STEPS = {"short": (300, 300), "mid": (10, 4), "long": (3, 1), "very_long": (5, 1)}
# Timed steps of each secondary section (other schedule, layout or order; the
# simulated ring's repetitions) and timed backward calls, at most. A Very long
# forward takes ~4.4 s and its backward ~16 s, so these stay small there.
SECONDARY_CAP = {"short": 300, "mid": 10, "long": 3, "very_long": 2}
BACKWARD_CAP = {"short": 100, "mid": 10, "long": 3, "very_long": 2}
RING_SIM_REPS = {"long": 1, "very_long": 1}
# Default order of the timed step. At 262,144 and 786,432 tokens the ring
# kernel on device-layout tensors (each device's stripe contiguous, as on a
# real ring) runs ~2% faster than with the stripe read in place, which more
# than pays for the explicit gathers (~10 ms of a ~4.4 s step at 786,432
# tokens); at the shorter lengths the gathers cost more than they save.
DEFAULT_ORDER = {"long": "device", "very_long": "device"}
WARM_SECONDS = 0.15   # back-to-back work before each secondary timed section


def note(msg):
    """Progress line on stderr (stdout carries only the JSON result)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def warm(torch, fn, seconds=WARM_SECONDS):
    """Run `fn` back to back for at least `seconds` (at least once), so the
    section that follows starts at sustained clocks instead of after host-side
    idle time."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    dt = max(time.perf_counter() - t0, 1e-5)
    for _ in range(max(0, int(seconds / dt) - 1)):
        fn()
    torch.cuda.synchronize()


def queued_ms(torch, fn, reps=20):
    """Mean GPU time of `fn` over `reps` back-to-back calls. The calls are
    enqueued behind ~2.5 ms of matrix products, so the host's enqueueing of
    short launches never leaves the GPU idle inside the timed region."""
    pad = torch.ones((4096, 4096), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    for _ in range(28):
        torch.mm(pad, pad)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def imbalance(live):
    """Per-round max/mean over devices and the aggregate sum(max)/sum(mean)."""
    import numpy as np
    live = np.asarray(live, dtype=np.float64)
    per = [float(r.max() / r.mean()) if r.mean() > 0 else None for r in live]
    agg = float(live.max(axis=1).sum() / live.mean(axis=1).sum())
    return per, agg


def blas_info():
    """numpy's BLAS library and thread count (threadpoolctl), or None."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return {"vendor": i.get("internal_api"), "version": i.get("version"),
                        "threads": i.get("num_threads"), "library": os.path.basename(i.get("filepath", ""))}
    except Exception:  # pragma: no cover
        return None
    return None


def cpu_baseline(x, seconds, block=64, n_blocks=64):
    """The oracle's useful rate on a bounded sample of the workload, extrapolated.

    Sample: head 0 of batch 0; `n_blocks` blocks of `block` consecutive query
    rows at evenly spaced positions over the sequence, visited in a fixed
    (seeded) order until about `seconds` of oracle time. Each block is one
    call of oracle.attention_rows (fp64 numpy: the block's scores against
    every key up to its last row, masked, softmax, times V). Useful flops are
    4*Dh per live causal pair of the sampled rows; the whole forward's time is
    extrapolated from that rate and the workload's pair count."""
    import numpy as np
    import oracle
    cores = len(os.sched_getaffinity(0))
    B, S, H, D = x["q"].shape
    qh, kh, vh = (x[n][:1, :, :1].cpu() for n in ("q", "k", "v"))
    blas = blas_info()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
    except Exception:  # pragma: no cover
        limiter = None
    blas_used = blas_info()
    nb = min(n_blocks, max(1, S // block))
    starts = [min(S - block, (m * S) // nb) if S >= block else 0 for m in range(nb)]
    order = np.random.default_rng(0).permutation(nb)
    done, pairs, t_total = 0, 0, 0.0
    for m in order:
        if t_total >= seconds:
            break
        i0 = starts[m]
        rows = np.arange(i0, min(S, i0 + block))
        t0 = time.perf_counter()
        oracle.attention_rows(qh, kh, vh, rows)
        t_total += time.perf_counter() - t0
        pairs += int((rows + 1).sum())
        done += 1
    if limiter is not None:
        limiter.restore_original_limits()
    rate = 4.0 * D * pairs / t_total / 1e12
    full_flops = 4.0 * D * B * H * S * (S + 1) / 2
    return {"value": rate, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} blocks of {block} consecutive query rows (head 0 of {H}, batch 0) at fixed, "
                      f"evenly spaced positions of the {S}-token sequence, {pairs} useful causal pairs, fp64 numpy "
                      f"oracle.attention_rows, {t_total:.1f} s; rate extrapolated to the whole forward by "
                      f"useful-pair count",
            "extrapolated": True, "extrapolated_full_forward_s": full_flops / (rate * 1e12),
            "blas": blas_used or blas, "cores_note": "len(os.sched_getaffinity(0)); BLAS threads limited to it"}


def queried_peak_bf16(torch):
    """Dense bf16 MFMA peak from the device's own properties: compute units x
    4 SIMDs x 1,024 bf16 flop per clock (one 32x32x16 MFMA per 32 cycles) x the
    peak engine clock that HIP reports. Reported next to the published figure."""
    import ctypes
    dev = torch.cuda.current_device()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    khz = ctypes.c_int(0)
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, dev) != 0:   # 5: hipDeviceAttributeClockRate (kHz)
            return None
    except OSError:
        return None
    return {"TFLOP/s": cus * 4096 * khz.value * 1e3 / 1e12, "compute_units": cus, "clock_mhz": khz.value / 1e3}


def kernel_source_digest():
    """sha256 over the sources the forward ring kernel is compiled from."""
    h = hashlib.sha256()
    for name in FWD_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "striped_ring_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_record(workload, sched, layout, order):
    """The counter record of the fused forward kernel for this configuration,
    or None when none covers it or the kernel's sources have changed since
    the counters were taken."""
    if sched != 1 or layout != 1:
        return None
    digest = kernel_source_digest()
    for t in TRAFFIC:
        if t["workload"] == workload and t["order"] == order and t["kernel_sources_sha256"] == digest:
            return t
    return None


def stored_traffic(workload, sched, layout, order):
    """HBM bytes per launch of the fused forward kernel, or None (see traffic_record)."""
    t = traffic_record(workload, sched, layout, order)
    return None if t is None else t["bytes_per_launch"]


def traffic_detail(workload, sched, layout, order):
    t = traffic_record(workload, sched, layout, order)
    if t is None:
        return None
    return {k: t[k] for k in ("fetch_bytes_per_launch", "write_bytes_per_launch", "copy_scale")}


def time_backward(sra, torch, x, N, layout, ordr, fwd_step, qd, kd, vd, o_dev, lse_dev, o, lse, K, useful_fwd_flops):
    """The ring backward (dQ, dK, dV) on the forward's outputs, in the step's
    order: after at least ~0.15 s of untimed calls, K calls of the three
    backward kernels, each bracketed by events on the current stream (the
    stream the kernels are launched on). Useful flops: 10*Dh per live causal
    pair (S recomputed, dP, dV, dQ, dK), i.e. 2.5x the forward's."""
    fwd_step()
    if layout == sra.STRIPED and ordr == sra.ORDER_DEVICE:
        q, k, v, out, l = qd, kd, vd, o_dev, lse_dev
        do = sra.stripe_permute(x["do"], N)
    else:
        q, k, v, out, l, do = x["q"], x["k"], x["v"], o, lse, x["do"]
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    ws = torch.empty(max(1, sra.bwd_workspace_bytes(q, N, layout)), dtype=torch.uint8, device=q.device)
    warm(torch, lambda: sra.ring_attn_bwd(q, k, v, out, l, do, N, layout, dq=dq, dk=dk, dv=dv, workspace=ws,
                                          order=ordr))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        sra.ring_attn_bwd(q, k, v, out, l, do, N, layout, dq=dq, dk=dk, dv=dv, workspace=ws, order=ordr)
        b.record()
    torch.cuda.synchronize()
    per_call = [a.elapsed_time(b) for a, b in evs]
    ms = sum(per_call) / K
    flops = 2.5 * useful_fwd_flops
    achieved = flops / (ms * 1e-3) / 1e12
    return {"ms": ms, "ms_per_call": per_call, "useful_TFLOPs": achieved,
            "pct_bf16_peak": 100 * achieved / PEAK_BF16_TFLOPS,
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": achieved / PEAK_BF16_TFLOPS, "flops_per_call": flops},
            "flops_per_live_pair": "10*head_dim", "kernels": ["bwd_delta", "bwd_dq", "bwd_dkdv"],
            "calls": K, "order": "original" if ordr == sra.ORDER_ORIGINAL else "device",
            "note": "not part of value: the headline is the forward; one call = the three backward kernels"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the N virtual ring devices are simulated as rounds on a single "
              f"MI355X, and no multi-GPU path is built (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import striped_ring_attention_amd as sra
    from striped_ring_attention_amd.inputs import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sra.load()
    w = dict(WORKLOADS[args.workload])
    over = {n: val for n, val in (("seq", args.seq), ("heads", args.heads)) if val is not None}
    w.update(over)
    wname = args.workload + ("+override" if over else "")
    if over:
        # Steps sized from the useful work at ~1 PFLOP/s: ~0.1 s of warm-up, ~0.3 s timed.
        t_est = 2.0 * w["head_dim"] * w["batch"] * w["heads"] * w["seq"] ** 2 / 1e15
        k_def, w_def = max(2, round(0.3 / t_est)), max(1, round(0.1 / t_est))
    else:
        k_def, w_def = DEFAULT_STEPS.get(args.workload, (20, 3))
    args.steps = k_def if args.steps is None else args.steps
    args.warmup = w_def if args.warmup is None else args.warmup
    if w["dtype"] != torch.bfloat16:
        print("bench.py times the bf16 workloads", file=sys.stderr)
        sys.exit(2)
    B, S, H, D, N = w["batch"], w["seq"], w["heads"], w["head_dim"], w["n_dev"]
    layout = sra.STRIPED if args.layout == "striped" else sra.CONTIGUOUS
    sched = sra.SCHEDULE_FUSED if args.schedule == "fused" else sra.SCHEDULE_PER_ROUND
    dev = torch.device("cuda:0")
    if w["seq"] % w["n_dev"] != 0:
        print(f"--seq must be a multiple of the workload's {w['n_dev']} ring devices", file=sys.stderr)
        sys.exit(2)
    x = make_inputs(w, device=dev, with_grad=not args.no_backward)
    q, k, v = x["q"], x["k"], x["v"]
    qd, kd, vd = (torch.empty_like(t) for t in (q, k, v))
    o_dev = torch.empty_like(q)
    lse_dev = torch.empty((B, S, H), dtype=torch.float32, device=dev)
    o, lse = torch.empty_like(q), torch.empty_like(lse_dev)
    ws_bytes = max(sra.fwd_workspace_bytes(q, N, lay, sc) for lay in (0, 1) for sc in (0, 1))
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)
    counts = torch.zeros(N * N, dtype=torch.int64, device=dev)

    def launches(sc):
        return N if sc == sra.SCHEDULE_PER_ROUND else 1

    if args.order is None:
        args.order = DEFAULT_ORDER.get(args.workload, "original")
    ordr = sra.ORDER_ORIGINAL if args.order == "original" else sra.ORDER_DEVICE

    def step(lay, sc, events=None, perm_events=None, cnt=None, od=None):
        od = ordr if od is None else od

        def ring(a, b, c, out, l_out):
            sra.ring_attn_fwd(a, b, c, N, lay, schedule=sc, out=out, lse=l_out, workspace=ws, live_counts=cnt,
                              round_events=events, order=od)
        if od == sra.ORDER_ORIGINAL:
            ring(q, k, v, o, lse)
        elif lay == sra.STRIPED:
            if perm_events:
                perm_events[0].record()
            for src, dst in ((q, qd), (k, kd), (v, vd)):
                sra.stripe_permute(src, N, out=dst)
            if perm_events:
                perm_events[1].record()
            ring(qd, kd, vd, o_dev, lse_dev)
            if perm_events:
                perm_events[2].record()
            sra.unstripe(o_dev, N, out=o)
            sra.unstripe(lse_dev, N, out=lse)
            if perm_events:
                perm_events[3].record()
        else:
            ring(q, k, v, o, lse)

    def new_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record()          # create the underlying HIP event before its handle is passed on
        return evs

    def timed(lay, sc, K, perm=False, od=None):
        """K steps; returns (ms per step, kernel ms per launch list per step, permutation events)."""
        nl = launches(sc)
        evs = [new_events(2 * nl) for _ in range(K)]
        pev = [new_events(4) for _ in range(K)] if perm else [None] * K
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for i in range(K):
            step(lay, sc, events=[e.cuda_event for e in evs[i]], perm_events=pev[i], od=od)
        t1.record()
        torch.cuda.synchronize()
        per_launch = [[evs[i][2 * r].elapsed_time(evs[i][2 * r + 1]) for r in range(nl)] for i in range(K)]
        return t0.elapsed_time(t1) / K, per_launch, pev

    # Warm-up (and one counted pass for the device-side census).
    step(layout, sched, cnt=counts)
    for _ in range(args.warmup):
        step(layout, sched)
    torch.cuda.synchronize()

    note(f"{wname}: census pass and {args.warmup} warm-up steps done")
    K = args.steps
    base = args.workload
    sec_K = args.sec_steps if args.sec_steps is not None else min(K, SECONDARY_CAP.get(base, K))
    bwd_K = args.bwd_steps if args.bwd_steps is not None else min(K, BACKWARD_CAP.get(base, K))
    wall0 = time.perf_counter()
    dev_striped = ordr == sra.ORDER_DEVICE and layout == sra.STRIPED
    ms_step, per_launch, perm_ev = timed(layout, sched, K, perm=dev_striped)
    wall = time.perf_counter() - wall0
    note(f"{K} timed steps done ({wall:.1f} s)")
    attn_ms = sum(sum(p) for p in per_launch) / K
    ring_ms_steps = [sum(p) for p in per_launch]   # kernel time of each timed step
    nl = launches(sched)
    useful_flops = 4.0 * D * B * H * S * (S + 1) / 2
    value = useful_flops / (ms_step * 1e-3) / 1e12
    attn_tflops = useful_flops / (attn_ms * 1e-3) / 1e12
    pairs = sra.count_live_pairs(S, N, layout).numpy() * (B * H)
    if sched == sra.SCHEDULE_PER_ROUND:
        flops_per_launch = [4.0 * D * float(pairs[r].sum()) for r in range(N)]
    else:
        flops_per_launch = [useful_flops]

    # The other order, timed alongside (striped): the explicit gather kernels
    # are timed inside the device-order step (the timed step itself when
    # --order device, else a run of its own).
    perm = {}
    other_step = None
    if layout == sra.STRIPED:
        other = sra.ORDER_ORIGINAL if dev_striped else sra.ORDER_DEVICE
        warm(torch, lambda: step(layout, sched, od=other))
        o_step, o_launch, o_perm = timed(layout, sched, sec_K, perm=not dev_striped, od=other)
        if not dev_striped:
            perm_ev = o_perm
        o_attn = sum(sum(p) for p in o_launch) / sec_K
        other_step = {"step_ms": o_step, "step_useful_TFLOPs": useful_flops / (o_step * 1e-3) / 1e12,
                      "ring_ms": o_attn, "ring_useful_TFLOPs": useful_flops / (o_attn * 1e-3) / 1e12,
                      "steps": sec_K}
    if layout == sra.STRIPED:
        n_ev = len(perm_ev)
        p_ms = sum(perm_ev[i][0].elapsed_time(perm_ev[i][1]) for i in range(n_ev)) / n_ev
        u_ms = sum(perm_ev[i][2].elapsed_time(perm_ev[i][3]) for i in range(n_ev)) / n_ev
        el = q.element_size()
        p_bytes = 3 * 2 * q.numel() * el
        u_bytes = 2 * (o.numel() * el + lse.numel() * 4)
        perm = {"stripe_permute_qkv_ms": p_ms, "stripe_permute_GBps": p_bytes / (p_ms * 1e-3) / 1e9,
                "unstripe_o_lse_ms": u_ms, "unstripe_GBps": u_bytes / (u_ms * 1e-3) / 1e9,
                "hbm_peak_GBps": PEAK_HBM_GBS, "note": "timed back to back inside the step (caches warm)"}

    note("other-order step done")
    # Cold-cache rates: the 256 MB Infinity Cache is flushed (a 1 GiB write)
    # before each repetition; median of 5.
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=q.device)

    def cold_ms(fn, reps=5):
        ts = []
        for _ in range(reps):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts)

    if layout == sra.STRIPED:
        pq_out = torch.empty_like(q)
        c_ms = cold_ms(lambda: sra.stripe_permute(q, N, out=pq_out))
        perm["stripe_permute_cold_GBps"] = 2 * q.numel() * q.element_size() / (c_ms * 1e-3) / 1e9
        perm["cold_note"] = "one tensor, Infinity Cache flushed before each of 5 runs, median"

    # Model-input step (not part of value): rotary embedding of Q and K at their
    # original positions, fused with the stripe gather (device layout).
    qr_out, kr_out = torch.empty_like(q), torch.empty_like(k)

    def rope_qk():
        sra.rope_permute(q, N, layout, out=qr_out)
        sra.rope_permute(k, N, layout, out=kr_out)

    warm(torch, rope_qk)
    r_ms = queued_ms(torch, rope_qk)
    r_bytes = 2 * 2 * q.numel() * q.element_size()
    rc_ms = cold_ms(rope_qk)
    model_input = {"rope_permute_qk_ms": r_ms, "rope_permute_GBps": r_bytes / (r_ms * 1e-3) / 1e9,
                   "rope_permute_cold_GBps": r_bytes / (rc_ms * 1e-3) / 1e9, "hbm_peak_GBps": PEAK_HBM_GBS,
                   "note": "Q and K rotated at original positions and gathered into the layout; not part of value"}

    # Unfused log-sum-exp merge of one round's fp32 partial into the running
    # (O, LSE): per row (2 Dh + 2) fp32 read and (Dh + 1) written. The driver
    # fuses this into the round kernel's epilogue; the standalone kernel is the
    # unfused form.
    g = torch.Generator(device=dev).manual_seed(7)
    m_oa = torch.randn((B, S, H, D), generator=g, device=dev)
    m_op = torch.randn((B, S, H, D), generator=g, device=dev)
    m_la = torch.randn((B, S, H), generator=g, device=dev)
    m_lp = torch.randn((B, S, H), generator=g, device=dev)
    warm(torch, lambda: sra.lse_merge(m_oa, m_la, m_op, m_lp))
    m_ms = queued_ms(torch, lambda: sra.lse_merge(m_oa, m_la, m_op, m_lp))
    m_bytes = B * S * H * (3 * D + 3) * 4
    mc_ms = cold_ms(lambda: sra.lse_merge(m_oa, m_la, m_op, m_lp))
    merge = {"lse_merge_ms": m_ms, "lse_merge_GBps": m_bytes / (m_ms * 1e-3) / 1e9,
             "lse_merge_cold_GBps": m_bytes / (mc_ms * 1e-3) / 1e9, "bytes": m_bytes, "hbm_peak_GBps": PEAK_HBM_GBS,
             "note": "standalone unfused merge of one fp32 partial, rows B*S*H; not part of value"}
    del flush, m_oa, m_op, m_la, m_lp

    note("gathers, rotary gather and merge done")
    # Imbalance: host census at 128x128 tiles and at the kernel's own tiles; device counters.
    tq, tk = sra.kernel_tiles(torch.bfloat16, D)
    imb = {}
    for lname, lay in (("contiguous", sra.CONTIGUOUS), ("striped", sra.STRIPED)):
        live128 = sra.count_live_tiles(S, N, lay, 128, 128)[0].numpy()
        livek = sra.count_live_tiles(S, N, lay, tq, tk)[0].numpy()
        per, agg = imbalance(live128)
        _, aggk = imbalance(livek)
        _, pagg = imbalance(sra.count_live_pairs(S, N, lay).numpy())
        imb[lname] = {"per_round_max_over_mean_128x128": per, "aggregate_128x128": agg,
                      f"aggregate_{tq}x{tk}_kernel_tiles": aggk, "aggregate_pairs": pagg}
    dev_counts = counts.view(N, N).cpu().numpy()
    host_counts = sra.count_live_tiles(S, N, layout, tq, tk)[0].numpy() * (B * H)
    imb["device_counters_match_host"] = bool(np.array_equal(dev_counts, host_counts))
    imb["device_per_round_max_over_mean"] = imbalance(dev_counts)[0]

    compare = None
    if not args.no_compare:
        compare = {}
        other = sra.SCHEDULE_PER_ROUND if sched == sra.SCHEDULE_FUSED else sra.SCHEDULE_FUSED
        oname = "per_round" if other == sra.SCHEDULE_PER_ROUND else "fused"
        for cname, lay, sc in ((f"{args.layout}_{oname}", layout, other),
                               ("contiguous_per_round", sra.CONTIGUOUS, sra.SCHEDULE_PER_ROUND),
                               ("contiguous_fused", sra.CONTIGUOUS, sra.SCHEDULE_FUSED)):
            if lay == layout and sc == sched:
                continue
            warm(torch, lambda: step(lay, sc))
            c_step, c_launch, _ = timed(lay, sc, sec_K)
            c_attn = sum(sum(p) for p in c_launch) / sec_K
            rec = {"ring_ms": c_attn, "ring_useful_TFLOPs": useful_flops / (c_attn * 1e-3) / 1e12,
                   "step_ms": c_step}
            if sc == sra.SCHEDULE_PER_ROUND:
                rec["round_ms"] = [sum(c_launch[i][r] for i in range(sec_K)) / sec_K for r in range(N)]
            rec["steps"] = sec_K
            compare[cname] = rec
            note(f"compare {cname} done")
        compare[f"{args.layout}_{args.schedule}"] = {"ring_ms": attn_ms, "ring_useful_TFLOPs": attn_tflops,
                                                     "step_ms": ms_step}
        if other_step is not None:
            oname = "original" if dev_striped else "device"
            compare[f"{args.layout}_{args.schedule}_{oname}_order"] = other_step

    critical = None
    if not args.no_critical_path:
        from striped_ring_attention_amd import ring_sim
        warm(torch, lambda: step(sra.CONTIGUOUS, sra.SCHEDULE_PER_ROUND))
        reps = RING_SIM_REPS.get(base, 3)
        t_c = ring_sim.time_device_rounds(q, k, v, N, sra.CONTIGUOUS, reps=reps)
        for src, dst in ((q, qd), (k, kd), (v, vd)):
            sra.stripe_permute(src, N, out=dst)
        warm(torch, lambda: step(sra.STRIPED, sra.SCHEDULE_PER_ROUND))
        t_s = ring_sim.time_device_rounds(qd, kd, vd, N, sra.STRIPED, reps=reps)
        critical = ring_sim.project(t_s, t_c, ring_sim.kv_block_bytes(B, S, H, D, N, q.element_size()))
        critical["note"] = ("one launch per (device, round) on this GPU; ring time = sum over rounds of "
                            "max(slowest device, K/V transfer at the assumed link bandwidth); prefetch time = "
                            "every block sent at the start over the direct links, round r waiting for its block")
        critical["reps"] = reps
        note("simulated ring done")

    backward = None
    if not args.no_backward:
        backward = time_backward(sra, torch, x, N, layout, ordr, lambda: step(layout, sched), qd, kd, vd, o_dev,
                                 lse_dev, o, lse, bwd_K, useful_flops)
        note("backward done")

    rec = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wname, "batch": B, "seq_len": S, "heads": H, "head_dim": D,
                   "ring_devices": N, "layout": args.layout, "schedule": args.schedule, "order": args.order,
                   "causal": True,
                   "pass": "forward"},
        "pct_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / PEAK_BF16_TFLOPS,
                     "traffic": stored_traffic(wname, sched, layout, args.order),
                     "kernel": "round_fwd_bf16_d128<fused>" if sched == sra.SCHEDULE_FUSED
                     else "round_fwd_bf16_d128<per-round>",
                     "traffic_detail": traffic_detail(wname, sched, layout, args.order),
                     "launches_per_step": nl, "avg_launch_ms": attn_ms / nl,
                     "step_kernel_ms_median_min_max": [statistics.median(ring_ms_steps), min(ring_ms_steps),
                                                       max(ring_ms_steps)],
                     "flops_per_launch": flops_per_launch,
                     "peak_queried": queried_peak_bf16(torch)},
        "imbalance": imb, "permutation": perm, "model_input": model_input, "lse_merge": merge, "compare": compare, "backward": backward,
        "critical_path": critical,
        "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
        # Step throughput over the oracle's (extrapolated) rate on the host cores.
        rec["cpu_baseline"]["gpu_over_cpu"] = value / rec["cpu_baseline"]["value"]
        note("cpu baseline done")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
