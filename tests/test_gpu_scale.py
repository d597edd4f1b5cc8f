"""GPU parity on descriptor settings the other tests leave at one value:
an explicit softmax scale (instead of the default 1/sqrt(head_dim)) for the
ring forward on both schedules and layouts, the fp32 rounds and the backward,
against the oracle evaluated with the same scale (a kernel that ignored the
field would fail here); and 48 or 64 heads, i.e. token rows of 24 and 32 KiB."""

import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def err(gpu, ref):
    return float(np.abs(gpu.detach().cpu().double().numpy() - ref).max())


@pytest.mark.parametrize("scale", [0.03, 0.25])
def test_explicit_scale_bf16_forward_and_backward(sra, scale):
    S, N, H = 1024, 4, 2
    g = torch.Generator().manual_seed(77)
    x = {n: (torch.randn((1, S, H, 128), generator=g) * 0.5).to(torch.bfloat16) for n in ("q", "k", "v")}
    x["do"] = torch.randn((1, S, H, 128), generator=g).to(torch.bfloat16)
    o_ref, l_ref = oracle.dense_causal_attention(x["q"], x["k"], x["v"], scale=scale)
    ref = oracle.dense_causal_backward(x["q"], x["k"], x["v"], o_ref, l_ref, x["do"], scale=scale)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    for schedule in (sra.SCHEDULE_PER_ROUND, sra.SCHEDULE_FUSED):
        for layout in (oracle.CONTIGUOUS, oracle.STRIPED):
            say("scale", scale, "schedule", schedule, "layout", layout)
            o, lse = sra.ring_attn_fwd(q, k, v, N, layout, scale=scale, schedule=schedule,
                                       order=sra.ORDER_ORIGINAL)
            torch.cuda.synchronize()
            e_o, e_l = err(o, o_ref), err(lse, l_ref)
            say(f"  forward: O {e_o:.3g} LSE {e_l:.3g}")
            assert e_o <= 2e-2 and e_l <= 2e-2
    o, lse = sra.ring_attn_fwd(q, k, v, N, oracle.STRIPED, scale=scale, schedule=sra.SCHEDULE_FUSED,
                               order=sra.ORDER_ORIGINAL)
    grads = sra.ring_attn_bwd(q, k, v, o, lse, do, N, oracle.STRIPED, scale=scale, order=sra.ORDER_ORIGINAL)
    torch.cuda.synchronize()
    errs = [err(gr, r) for gr, r in zip(grads, ref)]
    say(f"  backward: dQ {errs[0]:.3g} dK {errs[1]:.3g} dV {errs[2]:.3g}")
    assert max(errs) <= 2e-2


def test_explicit_scale_fp32_rounds(sra):
    S, N, H, D, scale = 256, 4, 1, 64, 0.3
    g = torch.Generator().manual_seed(78)
    q, k, v = (torch.randn((1, S, H, D), generator=g) for _ in range(3))
    o_ref, l_ref = oracle.dense_causal_attention(q, k, v, scale=scale)
    for layout in (oracle.CONTIGUOUS, oracle.STRIPED):
        o, lse = sra.ring_attn_fwd(q.cuda(), k.cuda(), v.cuda(), N, layout, scale=scale,
                                   schedule=sra.SCHEDULE_PER_ROUND, order=sra.ORDER_ORIGINAL)
        torch.cuda.synchronize()
        e_o, e_l = err(o, o_ref), err(lse, l_ref)
        say(f"fp32 layout {layout}: O {e_o:.3g} LSE {e_l:.3g}")
        assert e_o <= 1e-5 and e_l <= 1e-5


@pytest.mark.parametrize("S,N,H", [(512, 4, 48), (256, 16, 64)])
def test_many_heads_forward_and_backward(sra, S, N, H):
    """Token rows of 24 and 32 KiB (48 and 64 heads): one head's consecutive
    tokens are that far apart, and 16 of them in original order with N = 16.
    Fused and per-round forwards and the backward against the dense oracle."""
    g = torch.Generator().manual_seed(79 + H)
    x = {n: (torch.randn((1, S, H, 128), generator=g) * 0.5).to(torch.bfloat16) for n in ("q", "k", "v")}
    x["do"] = torch.randn((1, S, H, 128), generator=g).to(torch.bfloat16)
    o_ref, l_ref = oracle.dense_causal_attention(x["q"], x["k"], x["v"])
    ref = oracle.dense_causal_backward(x["q"], x["k"], x["v"], o_ref, l_ref, x["do"])
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    for schedule in (sra.SCHEDULE_PER_ROUND, sra.SCHEDULE_FUSED):
        say("S", S, "N", N, "H", H, "schedule", schedule)
        o, lse = sra.ring_attn_fwd(q, k, v, N, oracle.STRIPED, schedule=schedule, order=sra.ORDER_ORIGINAL)
        torch.cuda.synchronize()
        assert err(o, o_ref) <= 2e-2 and err(lse, l_ref) <= 2e-2
    grads = sra.ring_attn_bwd(q, k, v, o, lse, do, N, oracle.STRIPED, order=sra.ORDER_ORIGINAL)
    torch.cuda.synchronize()
    errs = [err(gr, r) for gr, r in zip(grads, ref)]
    say(f"  backward: dQ {errs[0]:.3g} dK {errs[1]:.3g} dV {errs[2]:.3g}")
    assert max(errs) <= 2e-2
