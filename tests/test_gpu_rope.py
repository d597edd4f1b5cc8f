"""Rotary embedding fused with the stripe gather (sra_rope_permute), against
the oracle's fp64 rotary embedding at original positions.

Tolerances: bf16 outputs may differ from the fp64 value by one bf16 rounding
(relative 2^-9, bounded here by 2^-8) plus the fp32 rotation's own error,
bounded by 1e-5 absolute; fp32 outputs by 1e-5 absolute (|x| stays below ~6
for these standard-normal inputs, and the fp32 sine and cosine of the
fp64-reduced angle are good to a few 1e-7). The end-to-end case, attention
over rotated inputs, uses the usual 2e-2 bf16 bound.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from striped_ring_attention_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_close(got, want, dtype):
    g = got.double().cpu().numpy()
    if dtype == torch.bfloat16:
        bound = np.abs(want) * 2.0 ** -8 + 1e-5
    else:
        bound = np.full(want.shape, 1e-5)
    err = np.abs(g - want)
    assert np.all(err <= bound), f"max err {err.max():.3g}, worst excess {(err - bound).max():.3g}"
    return float(err.max())


def rand(shape, dtype, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda").to(dtype)


CASES = [  # (B, S, H, D, N, dtype)
    (1, 8 * 300, 3, 128, 8, torch.bfloat16),
    (2, 4 * 96, 2, 128, 4, torch.bfloat16),
    (1, 256, 1, 64, 4, torch.float32),
    (1, 640, 2, 64, 1, torch.bfloat16),
    (1, 48, 5, 8, 16, torch.float32),
    (1, 96, 2, 256, 3, torch.bfloat16),
]


@pytest.mark.parametrize("B,S,H,D,N,dtype", CASES)
@pytest.mark.parametrize("with_pos", [False, True])
def test_rope_permute_matches_oracle(sra, B, S, H, D, N, dtype, with_pos):
    x = rand((B, S, H, D), dtype, 100 + S + D)
    pos = None
    if with_pos:
        g = torch.Generator(device="cuda").manual_seed(7)
        pos = torch.randint(0, 800_000, (B, S), generator=g, device="cuda", dtype=torch.int64)
    pos_np = None if pos is None else pos.cpu().numpy()
    for layout in (oracle.CONTIGUOUS, oracle.STRIPED):
        y = sra.rope_permute(x, N, layout, pos=pos)
        want = oracle.rope_device_layout(x.cpu(), N, layout, pos_np)
        e = check_close(y, want, dtype)
        # original order: plain rotary embedding, no permutation
        y2 = sra.rope_permute(x, N, layout, pos=pos, order=sra.ORDER_ORIGINAL)
        e2 = check_close(y2, oracle.rope(x.cpu(), pos_np), dtype)
        say(f"rope B={B} S={S} H={H} D={D} N={N} {dtype} pos={with_pos} layout={layout}: {e:.3g} {e2:.3g}")


def test_rope_in_place_original_order(sra):
    x = rand((1, 1024, 4, 128), torch.bfloat16, 3)
    want = sra.rope_permute(x, 8, oracle.STRIPED, order=sra.ORDER_ORIGINAL)
    y = x.clone()
    sra.rope_permute(y, 8, oracle.STRIPED, order=sra.ORDER_ORIGINAL, out=y)
    torch.cuda.synchronize()
    assert torch.equal(y, want)


def test_rope_base_and_large_positions(sra):
    """Other bases, and positions near 2^20 where an fp32 angle would already
    be off by ~0.03 rad: the fp64 reduction keeps the rotation accurate."""
    x = rand((1, 64, 2, 128), torch.float32, 4)
    pos = torch.arange(1_048_000, 1_048_064, device="cuda", dtype=torch.int64)[None, :]
    for base in (10000.0, 500000.0, 2.0):
        y = sra.rope_permute(x, 1, oracle.CONTIGUOUS, pos=pos, base=base)
        check_close(y, oracle.rope(x.cpu(), pos.cpu().numpy(), base), torch.float32)


def test_token_ids_stripe_bit_exact(sra):
    """Token ids and position ids (int64 rows) go through sra_stripe_permute."""
    B, S, N = 2, 8 * 96, 8
    ids = torch.randint(0, 50_000, (B, S, 1), device="cuda", dtype=torch.int64)
    got = sra.stripe_permute(ids, N).cpu().numpy()
    want = oracle.to_device_layout(ids.cpu().numpy(), N, oracle.STRIPED)
    assert np.array_equal(got, want)
    assert torch.equal(sra.unstripe(sra.stripe_permute(ids, N), N), ids)


@pytest.mark.parametrize("order", ["device", "original"])
def test_striped_attention_over_rotated_inputs(sra, order):
    """Model-input step end to end: rotate Q and K at their original
    positions (striping them), run the striped ring, and compare with dense
    causal attention of the rotated inputs."""
    x = make_inputs("short", device="cuda")
    q, k, v = x["q"][:, :2048, :4].contiguous(), x["k"][:, :2048, :4].contiguous(), x["v"][:, :2048, :4].contiguous()
    N = 8
    if order == "device":
        qd = sra.rope_permute(q, N, oracle.STRIPED)
        kd = sra.rope_permute(k, N, oracle.STRIPED)
        vd = sra.stripe_permute(v, N)
        o, lse = sra.ring_attn_fwd(qd, kd, vd, N, oracle.STRIPED, schedule=sra.SCHEDULE_FUSED)
        o, lse = sra.unstripe(o, N), sra.unstripe(lse, N)
    else:
        qr = sra.rope_permute(q, N, oracle.STRIPED, order=sra.ORDER_ORIGINAL)
        kr = sra.rope_permute(k, N, oracle.STRIPED, order=sra.ORDER_ORIGINAL)
        o, lse = sra.striped_attention(qr, kr, v, N)
    o_ref, l_ref = oracle.dense_causal_attention(oracle.rope(q.cpu()), oracle.rope(k.cpu()), v.cpu())
    e_o = float(np.abs(o.double().cpu().numpy() - o_ref).max())
    e_l = float(np.abs(lse.double().cpu().numpy() - l_ref).max())
    say(f"attention over rotated inputs ({order}): O {e_o:.3g} LSE {e_l:.3g}")
    assert e_o <= 2e-2 and e_l <= 2e-2


def test_rope_large_striped(sra):
    """A striped tensor of 512 MB (the Long workload's Q at 8 heads):
    unstriped, its output equals the original-order call bit for bit, with and
    without explicit position ids, and sampled rows match the oracle."""
    B, S, H, D, N = 1, 262144, 8, 128, 8
    x = rand((B, S, H, D), torch.bfloat16, 9)
    g = torch.Generator(device="cuda").manual_seed(10)
    for pos in (None, torch.randint(0, 1_000_000, (B, S), generator=g, device="cuda", dtype=torch.int64)):
        y = sra.rope_permute(x, N, oracle.STRIPED, pos=pos)
        y2 = sra.rope_permute(x, N, oracle.STRIPED, pos=pos, order=sra.ORDER_ORIGINAL)
        torch.cuda.synchronize()
        assert torch.equal(sra.unstripe(y, N), y2)
        rows = np.unique(np.concatenate([[0, 1, N, S - 1], np.random.default_rng(11).integers(0, S, 60)]))
        p = rows[None, :] if pos is None else pos[:, rows].cpu().numpy()
        e = check_close(y2[:, rows], oracle.rope(x[:, rows].cpu(), p), torch.bfloat16)
        say(f"large striped rope pos={'ids' if pos is not None else 'index'}: sampled rows {e:.3g}, bit-identical orders")
