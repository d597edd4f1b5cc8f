"""Original-order entry points (desc.order = SRA_ORDER_ORIGINAL): the kernels
address device d's j-th token at its position in the sequence, so no
permuted copy is made. The arithmetic is the same as on device-layout
tensors, so the results must be bit-identical to the device-layout call
followed by unstripe -- checked for both layouts, both schedules, ragged
shapes, fp32, a single round with a device filter, and the backward. One
direct check against the oracle covers the path end to end."""

import sys

import numpy as np
import pytest
import torch

import oracle
from striped_ring_attention_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(sra, x, n, layout):
    return sra.stripe_permute(x, n) if layout == oracle.STRIPED else x


def from_device(sra, y, n, layout):
    return sra.unstripe(y, n) if layout == oracle.STRIPED else y


def rand_bf16(S, H, seed, D=128):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return [(torch.randn((1, S, H, D), generator=g, device="cuda") * 0.5).to(torch.bfloat16) for _ in range(4)]


CASES = [(8192, 16, 8), (8 * 300, 3, 8), (4 * 200, 2, 4), (16, 1, 16), (640, 2, 1)]


@pytest.mark.parametrize("S,H,N", CASES)
@pytest.mark.parametrize("schedule", [0, 1])
def test_fwd_original_order_bit_identical(sra, S, H, N, schedule):
    q, k, v, _ = rand_bf16(S, H, 40 + S + N)
    for layout in (oracle.CONTIGUOUS, oracle.STRIPED):
        o1, l1 = sra.ring_attn_fwd(q, k, v, N, layout, schedule=schedule, order=sra.ORDER_ORIGINAL)
        qd, kd, vd = (to_device(sra, t, N, layout) for t in (q, k, v))
        o2, l2 = sra.ring_attn_fwd(qd, kd, vd, N, layout, schedule=schedule)
        o2, l2 = from_device(sra, o2, N, layout), from_device(sra, l2, N, layout)
        torch.cuda.synchronize()
        say(f"fwd order S={S} H={H} N={N} sched={schedule} layout={layout}")
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_original_order_fp32(sra):
    w = WORKLOADS["tiny"]
    x = make_inputs("tiny", device="cuda")
    N = w["n_dev"]
    for layout in (oracle.CONTIGUOUS, oracle.STRIPED):
        o1, l1 = sra.ring_attn_fwd(x["q"], x["k"], x["v"], N, layout, order=sra.ORDER_ORIGINAL)
        qd, kd, vd = (to_device(sra, x[n], N, layout) for n in ("q", "k", "v"))
        o2, l2 = sra.ring_attn_fwd(qd, kd, vd, N, layout)
        assert torch.equal(o1, from_device(sra, o2, N, layout))
        assert torch.equal(l1, from_device(sra, l2, N, layout))


def test_round_original_order_device_filter(sra):
    S, H, N = 8 * 300, 3, 8
    q, k, v, _ = rand_bf16(S, H, 7)
    qd, kd, vd = (sra.stripe_permute(t, N) for t in (q, k, v))
    for r, dev in ((0, 0), (3, 5), (7, 2)):
        o1, l1 = sra.ring_round_attn(q, k, v, N, oracle.STRIPED, r, device=dev, order=sra.ORDER_ORIGINAL)
        o2, l2 = sra.ring_round_attn(qd, kd, vd, N, oracle.STRIPED, r, device=dev)
        assert torch.equal(o1, sra.unstripe(o2, N)) and torch.equal(l1, sra.unstripe(l2, N))


# (32768, 32, 16) and (16000, 32, 16): the Very long ring's N and heads, so a
# device's consecutive tokens are 128 KiB apart in original order (a dK/dV
# query tile spans 4 MiB), with slabs a multiple of the tiles and ragged.
@pytest.mark.parametrize("S,H,N", [(8192, 4, 8), (8 * 300, 3, 8), (16, 1, 16), (32768, 32, 16), (16000, 32, 16)])
def test_bwd_original_order_bit_identical(sra, S, H, N):
    q, k, v, do = rand_bf16(S, H, 90 + S)
    for layout in (oracle.CONTIGUOUS, oracle.STRIPED):
        o1, l1 = sra.ring_attn_fwd(q, k, v, N, layout, schedule=sra.SCHEDULE_FUSED, order=sra.ORDER_ORIGINAL)
        g1 = sra.ring_attn_bwd(q, k, v, o1, l1, do, N, layout, order=sra.ORDER_ORIGINAL)
        qd, kd, vd, dod = (to_device(sra, t, N, layout) for t in (q, k, v, do))
        o2, l2 = sra.ring_attn_fwd(qd, kd, vd, N, layout, schedule=sra.SCHEDULE_FUSED)
        g2 = sra.ring_attn_bwd(qd, kd, vd, o2, l2, dod, N, layout)
        torch.cuda.synchronize()
        say(f"bwd order S={S} H={H} N={N} layout={layout}")
        for a, b in zip(g1, g2):
            assert torch.equal(a, from_device(sra, b, N, layout))


def test_striped_attention_matches_dense_oracle(sra):
    """striped_attention (original order in and out) against dense fp64
    causal attention, no permutation anywhere on the host side."""
    S, H, N = 4 * 300, 2, 4
    q, k, v, _ = rand_bf16(S, H, 3)
    o, lse = sra.striped_attention(q, k, v, N)
    o_ref, l_ref = oracle.dense_causal_attention(q.cpu(), k.cpu(), v.cpu())
    e_o = float(np.abs(o.double().cpu().numpy() - o_ref).max())
    e_l = float(np.abs(lse.double().cpu().numpy() - l_ref).max())
    say(f"striped_attention vs oracle: O {e_o:.3g} LSE {e_l:.3g}")
    assert e_o <= 2e-2 and e_l <= 2e-2
