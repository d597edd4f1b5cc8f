"""The allocation-free backward (sra_ring_attn_bwd_noalloc) against the
backward with a caller workspace (sra_ring_attn_bwd): two calls in a row, the
second on a smaller problem, each bit-identical to the workspace form (the
same kernels on the same statistics)."""

import sys

import pytest
import torch

import oracle
from striped_ring_attention_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(sra, seq, heads, n_dev, layout, order, seed):
    w = dict(batch=1, heads=heads, seq=seq, head_dim=128, dtype=torch.bfloat16, n_dev=n_dev,
             std=(0.5, 0.5, 0.5), do_std=1.0, seed=seed)
    x = make_inputs(w, device="cuda", with_grad=True)
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    sched = sra.SCHEDULE_FUSED
    o, lse = sra.ring_attn_fwd(q, k, v, n_dev, layout, schedule=sched, order=order)
    want = sra.ring_attn_bwd(q, k, v, o, lse, do, n_dev, layout, order=order)
    got = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
    sra.ring_attn_bwd_noalloc(q, k, v, o, lse, do, *got, n_dev, layout, order=order)
    torch.cuda.synchronize()
    return want, got


def test_noalloc_backward_matches_workspace_backward_twice(sra):
    # First call: Short's shape (131,072 rows of statistics); second: smaller.
    for seq, heads, n_dev, layout, order, seed in ((8192, 16, 8, oracle.STRIPED, 1, 51),
                                                   (2048, 4, 4, oracle.CONTIGUOUS, 0, 52)):
        say(f"noalloc backward: S={seq} H={heads} N={n_dev} layout={layout} order={order}")
        want, got = _case(sra, seq, heads, n_dev, layout, order, seed)
        for name, a, b in zip(("dq", "dk", "dv"), want, got):
            assert torch.equal(a, b), name


def test_noalloc_backward_rejects_oversized(sra):
    """More rows than the library's array holds: rejected before any work."""
    import ctypes
    d = sra.make_desc(1, 1 << 25, 2, 128, 1024, oracle.STRIPED, sra.DTYPE_BF16)
    fake = ctypes.c_void_p(1 << 20)
    st = sra.lib().sra_ring_attn_bwd_noalloc(ctypes.byref(d), fake, fake, fake, fake, fake, fake,
                                             ctypes.c_void_p(1 << 40), ctypes.c_void_p(1 << 42),
                                             ctypes.c_void_p(1 << 44), None)
    assert st == 4 and b"allocation-free" in sra.lib().sra_last_error()
