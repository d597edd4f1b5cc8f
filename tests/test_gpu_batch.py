"""Batch > 1 through the attention kernels: every kernel decodes its work item
(batch, head, device, tile) and addresses rows with the batch index, so the
forward (both schedules, layouts and orders) and the backward are checked
against the dense fp64 oracle with several batches. One case has N = 3, where
the number of (batch, head, device) groups is not a multiple of 8 and the
work decode takes its plain (non-XCD-grouped) path.

Tolerance: max-abs 2e-2 (bf16) on O, LSE and the gradients.
"""

import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().cpu().double().numpy()


CASES = [(3, 8 * 96, 2, 8), (2, 3 * 300, 3, 3)]   # (B, S, H, N)


@pytest.fixture(scope="module", params=CASES, ids=lambda c: f"B{c[0]}-S{c[1]}-H{c[2]}-N{c[3]}")
def batch_case(request):
    B, S, H, N = request.param
    g = torch.Generator().manual_seed(500 + B + S)
    x = {n: (torch.randn((B, S, H, 128), generator=g) * 0.5).to(torch.bfloat16) for n in ("q", "k", "v")}
    x["do"] = torch.randn((B, S, H, 128), generator=g).to(torch.bfloat16)
    o_ref, l_ref = oracle.dense_causal_attention(x["q"], x["k"], x["v"])
    grads = oracle.dense_causal_backward(x["q"], x["k"], x["v"], o_ref, l_ref, x["do"])
    return (B, S, H, N), {n: t.cuda() for n, t in x.items()}, (o_ref, l_ref), grads


@pytest.mark.parametrize("schedule", [0, 1])
def test_batch_forward(sra, batch_case, schedule):
    (B, S, H, N), x, (o_ref, l_ref), _ = batch_case
    for layout in (oracle.CONTIGUOUS, oracle.STRIPED):
        for order in (sra.ORDER_DEVICE, sra.ORDER_ORIGINAL):
            q, k, v = x["q"], x["k"], x["v"]
            dev = order == sra.ORDER_DEVICE and layout == oracle.STRIPED
            if dev:
                q, k, v = (sra.stripe_permute(t, N) for t in (q, k, v))
            o, lse = sra.ring_attn_fwd(q, k, v, N, layout, schedule=schedule, order=order)
            if dev:
                o, lse = sra.unstripe(o, N), sra.unstripe(lse, N)
            torch.cuda.synchronize()
            e_o = float(np.abs(np64(o) - o_ref).max())
            e_l = float(np.abs(np64(lse) - l_ref).max())
            say(f"batch fwd B={B} S={S} H={H} N={N} sched={schedule} layout={layout} order={order}: "
                f"O {e_o:.3g} LSE {e_l:.3g}")
            assert e_o <= 2e-2 and e_l <= 2e-2


def test_batch_backward(sra, batch_case):
    (B, S, H, N), x, _, grads = batch_case
    for layout in (oracle.CONTIGUOUS, oracle.STRIPED):
        o, lse = sra.ring_attn_fwd(x["q"], x["k"], x["v"], N, layout, schedule=sra.SCHEDULE_FUSED,
                                   order=sra.ORDER_ORIGINAL)
        g = sra.ring_attn_bwd(x["q"], x["k"], x["v"], o, lse, x["do"], N, layout, order=sra.ORDER_ORIGINAL)
        torch.cuda.synchronize()
        errs = [float(np.abs(np64(a) - r).max()) for a, r in zip(g, grads)]
        say(f"batch bwd B={B} S={S} H={H} N={N} layout={layout}: dq {errs[0]:.3g} dk {errs[1]:.3g} dv {errs[2]:.3g}")
        assert max(errs) <= 2e-2, errs


def test_batch_per_round_grouped_order(sra):
    """Two batches with 16 query tiles per device: the one-launch-per-round
    schedule then hands out one (batch, head, device) group's tiles at a time
    per XCD. Sampled rows of every batch and head (row 0, the first and last
    rows of every device's stripe, random rows) against the oracle, for both
    layouts and orders, with the fused schedule alongside."""
    B, S, H, N = 2, 8 * 4096, 4, 8
    g = torch.Generator().manual_seed(611)
    xc = {n: (torch.randn((B, S, H, 128), generator=g) * 0.5).to(torch.bfloat16) for n in ("q", "k", "v")}
    L = S // N
    rows = {0}
    for d in range(N):
        for j in (0, 1, L - 2, L - 1):
            rows.add(j * N + d)
    rows |= set(np.random.default_rng(612).integers(0, S, 24).tolist())
    rows = np.array(sorted(rows))
    o_ref, l_ref = oracle.attention_rows(xc["q"], xc["k"], xc["v"], rows)
    x = {n: t.cuda() for n, t in xc.items()}
    for schedule in (sra.SCHEDULE_PER_ROUND, sra.SCHEDULE_FUSED):
        for layout in (oracle.CONTIGUOUS, oracle.STRIPED):
            for order in (sra.ORDER_DEVICE, sra.ORDER_ORIGINAL):
                q, k, v = x["q"], x["k"], x["v"]
                dev = order == sra.ORDER_DEVICE and layout == oracle.STRIPED
                if dev:
                    q, k, v = (sra.stripe_permute(t, N) for t in (q, k, v))
                o, lse = sra.ring_attn_fwd(q, k, v, N, layout, schedule=schedule, order=order)
                if dev:
                    o, lse = sra.unstripe(o, N), sra.unstripe(lse, N)
                torch.cuda.synchronize()
                e_o = float(np.abs(np64(o[:, rows]) - o_ref).max())
                e_l = float(np.abs(np64(lse[:, rows]) - l_ref).max())
                say(f"batch grouped B={B} S={S} H={H} N={N} sched={schedule} layout={layout} order={order}: "
                    f"O {e_o:.3g} LSE {e_l:.3g}")
                assert e_o <= 2e-2 and e_l <= 2e-2
