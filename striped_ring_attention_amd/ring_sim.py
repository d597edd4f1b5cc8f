"""Simulated N-device ring from one-GPU measurements.

Striped Attention summary page (research.elamur.ai), "Summary" paragraph 1:
every ring round, each device attends its queries to the K/V block it holds
and passes the block on, so a round lasts as long as its slowest device; with
contiguous chunks the causal mask leaves some devices with little or no work
in a round while others have a full block ("Key points", Imbalance). The
striped layout gives every device the same share in every round ("Summary"
paragraph 2). On one MI355X each (device d, round r) unit of work is launched
alone (``sra_ring_round_attn`` with a device filter, one GPU standing in for
one ring device) and timed; then

    ring time      = sum_r max(max_d t(d, r), t_comm)
    compute bound  = sum_r max_d t(d, r)

where t_comm is the time to pass one K/V block to the next device, overlapped
with the round's compute (a stated model, not a measurement: the pages name
no interconnect, and every simulated device runs on the same GPU). The projected speedup of
striped over contiguous is the ratio of ring times at the same shape.

A second model fits a node whose GPUs are all directly linked (an MI355X has 7
links to the 7 other GPUs of its node): instead of passing blocks around the
ring, every device sends its own block to all others at the start, one block
per link at a time, so the block of round r arrives after ceil(r / links)
transfers, and round r starts when both round r-1 has finished and its block
is in:

    prefetch time  = finish of the last round, round r on [max(end of r-1, ceil(r / links) t_comm), + max_d t(d, r)]

Host-side functions (``critical_path``, ``ring_time``, ``kv_block_bytes``,
``project``) are plain Python; ``time_device_rounds`` needs the GPU library.
"""

import argparse
import json
import statistics

DEFAULT_LINK_GBPS = 153.0   # assumed bandwidth of one device-to-device link, GB/s
DEFAULT_LINKS = 7           # direct links per GPU in an 8-GPU MI355X node


def critical_path(t):
    """sum over rounds of the slowest device's time; t[r][d]."""
    return float(sum(max(row) for row in t))


def ring_time(t, t_comm):
    """Ring time when each round's K/V transfer (t_comm) overlaps its compute."""
    return float(sum(max(max(row), t_comm) for row in t))


def prefetch_time(t, t_comm, links=DEFAULT_LINKS):
    """Time of all rounds when every remote block is sent directly at the start
    over `links` links (one block per link at a time): round r >= 1 waits for
    its block, which arrives after ceil(r / links) transfers."""
    end = 0.0
    for r, row in enumerate(t):
        arrive = -(-r // links) * t_comm if r > 0 else 0.0
        end = max(end, arrive) + max(row)
    return float(end)


def mean_path(t):
    """sum over rounds of the mean device time: the time if work were perfectly balanced."""
    return float(sum(sum(row) / len(row) for row in t))


def kv_block_bytes(batch, seq, heads, head_dim, n_dev, elem_bytes=2):
    """Bytes of one device's K and V block (what one ring hop carries)."""
    return 2 * batch * (seq // n_dev) * heads * head_dim * elem_bytes


def project(t_striped, t_contig, block_bytes, link_gbps=DEFAULT_LINK_GBPS, links=DEFAULT_LINKS):
    """Projected ring times and speedups from per-(round, device) times in ms."""
    t_comm = block_bytes / (link_gbps * 1e9) * 1e3
    out = {"t_comm_ms": t_comm, "link_GBps": link_gbps, "kv_block_bytes": block_bytes, "direct_links": links}
    for name, t in (("striped", t_striped), ("contiguous", t_contig)):
        out[name] = {"critical_path_ms": critical_path(t), "ring_ms": ring_time(t, t_comm),
                     "prefetch_ms": prefetch_time(t, t_comm, links),
                     "balanced_ms": mean_path(t),
                     "round_max_ms": [max(row) for row in t],
                     "round_max_over_mean": [max(row) / (sum(row) / len(row)) for row in t]}
    out["speedup_compute_bound"] = out["contiguous"]["critical_path_ms"] / out["striped"]["critical_path_ms"]
    out["speedup_with_comm"] = out["contiguous"]["ring_ms"] / out["striped"]["ring_ms"]
    out["speedup_with_prefetch"] = out["contiguous"]["prefetch_ms"] / out["striped"]["prefetch_ms"]
    return out


def time_device_rounds(q, k, v, n_dev, layout, reps=3):
    """t[r][d] in ms: one launch per (round, device) on device-layout q, k, v,
    bracketed by events on the current stream; median over `reps` after one
    warm-up pass.

    A short launch can take less GPU time than the host needs to enqueue it;
    an event pair around it would then also measure the host. Each timed pass
    therefore starts behind a queue of matrix products sized from the warm-up
    pass to outlast the host's enqueueing, so the launches run back to back."""
    import math
    import time
    import torch
    import striped_ring_attention_amd as sra
    B, S, H, D = q.shape
    o = torch.empty((B, S, H, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, S, H), dtype=torch.float32, device=q.device)
    pad = torch.ones((4096, 4096), dtype=torch.bfloat16, device=q.device)
    samples = [[[] for _ in range(n_dev)] for _ in range(n_dev)]
    n_pad, host_s = 0, 0.0
    for rep in range(reps + 1):
        if rep == 1:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(8):
                torch.mm(pad, pad)
            b.record()
            torch.cuda.synchronize()
            pad_ms = a.elapsed_time(b) / 8
            n_pad = math.ceil(2.0 * host_s * 1e3 / max(pad_ms, 1e-3)) + 1
        for _ in range(n_pad):
            torch.mm(pad, pad)
        t0 = time.perf_counter()
        evs = []
        for r in range(n_dev):
            for d in range(n_dev):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                sra.ring_round_attn(q, k, v, n_dev, layout, r, device=d, o_part=o, lse_part=lse)
                b.record()
                evs.append((r, d, a, b))
        host_s = time.perf_counter() - t0
        torch.cuda.synchronize()
        if rep == 0:
            continue
        for r, d, a, b in evs:
            samples[r][d].append(a.elapsed_time(b))
    return [[statistics.median(samples[r][d]) for d in range(n_dev)] for r in range(n_dev)]


def simulate(workload="long", reps=3, link_gbps=DEFAULT_LINK_GBPS, seed=None, links=DEFAULT_LINKS):
    """Times both layouts of a named workload and returns the projection."""
    import torch
    import striped_ring_attention_amd as sra
    from striped_ring_attention_amd.inputs import WORKLOADS, make_inputs
    sra.load()
    w = WORKLOADS[workload]
    over = {} if seed is None else {"seed": seed}
    x = make_inputs(workload, device="cuda", **over)
    N = w["n_dev"]
    q, k, v = x["q"], x["k"], x["v"]
    t_contig = time_device_rounds(q, k, v, N, sra.CONTIGUOUS, reps)
    qs, ks, vs = (sra.stripe_permute(t, N) for t in (q, k, v))
    del q, k, v, x
    t_striped = time_device_rounds(qs, ks, vs, N, sra.STRIPED, reps)
    B, S, H, D = qs.shape
    res = project(t_striped, t_contig, kv_block_bytes(B, S, H, D, N, qs.element_size()), link_gbps, links)
    pairs = {name: sra.count_live_pairs(S, N, lay).numpy() for name, lay in
             (("striped", sra.STRIPED), ("contiguous", sra.CONTIGUOUS))}
    ideal = {n: float(p.max(axis=1).sum()) for n, p in pairs.items()}
    res["speedup_ideal_pairs"] = ideal["contiguous"] / ideal["striped"]
    res["workload"] = {"name": workload, "batch": B, "seq": S, "heads": H, "head_dim": D, "ring_devices": N}
    res["t_ms"] = {"striped": t_striped, "contiguous": t_contig}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="long")
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--link-gbps", type=float, default=DEFAULT_LINK_GBPS)
    ap.add_argument("--links", type=int, default=DEFAULT_LINKS, help="direct links per GPU (prefetch model)")
    args = ap.parse_args()
    print(json.dumps(simulate(args.workload, args.reps, args.link_gbps, links=args.links)), flush=True)


if __name__ == "__main__":
    main()
