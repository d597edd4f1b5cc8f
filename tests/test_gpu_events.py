"""Timing events passed to sra_ring_attn_fwd (the benchmark's roofline comes
from them): each event pair brackets its launch with a positive duration, and
passing events changes no result bit."""

import sys

import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dtype,D,schedule,order", [
    (torch.bfloat16, 128, 1, 1),   # fused, original order (the benchmark's launch)
    (torch.bfloat16, 128, 1, 0),   # fused, device layout
    (torch.bfloat16, 128, 0, 0),   # one launch per round
    (torch.float32, 64, 0, 1),     # fp32 rounds: events recorded on the stream around each launch
])
def test_round_events_bracket_launches(sra, dtype, D, schedule, order):
    S, N, H = 2048, 4, 2
    say("events", dtype, D, schedule, order)
    g = torch.Generator(device="cuda").manual_seed(21)
    q, k, v = ((torch.randn((1, S, H, D), generator=g, device="cuda") * 0.5).to(dtype) for _ in range(3))
    if order == sra.ORDER_DEVICE:
        q, k, v = (sra.stripe_permute(t, N) for t in (q, k, v))
    o0, l0 = sra.ring_attn_fwd(q, k, v, N, oracle.STRIPED, schedule=schedule, order=order)
    n_launch = 1 if schedule == sra.SCHEDULE_FUSED else N
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_launch)]
    for e in evs:
        e.record()   # creates the HIP event before its handle is passed on
    o1, l1 = sra.ring_attn_fwd(q, k, v, N, oracle.STRIPED, schedule=schedule, order=order,
                               round_events=[e.cuda_event for e in evs])
    torch.cuda.synchronize()
    times = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(n_launch)]
    say("  launch ms", times)
    assert all(t > 0 for t in times)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
