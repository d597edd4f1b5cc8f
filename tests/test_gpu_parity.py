"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances: max-abs 1e-5 for fp32 workloads and 2e-2 for bf16 workloads on
O and LSE; permutation and tile counters are bit-exact. bf16 runs compare
against the oracle evaluated in fp64 on the very same bf16 inputs.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from striped_ring_attention_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
LAYOUTS = [oracle.CONTIGUOUS, oracle.STRIPED]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().cpu().double().numpy()


def to_dev_layout(x, n_dev, layout):
    """Original order -> device layout by plain indexing (oracle's permutation table)."""
    perm = torch.from_numpy(oracle.stripe_index(x.shape[1], n_dev, layout)).to(x.device)
    return x.index_select(1, perm).contiguous()


def from_dev_layout(y, n_dev, layout):
    inv = torch.from_numpy(oracle.unstripe_index(y.shape[1], n_dev, layout)).to(y.device)
    return y.index_select(1, inv).contiguous()


def maxabs(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), "finite/-inf pattern differs"
    assert np.array_equal(a[~fin], b[~fin])
    return float(np.abs(a[fin] - b[fin]).max()) if fin.any() else 0.0


# ----------------------------------------------------------- permutation --

@pytest.mark.parametrize("shape,dtype,n_dev", [
    ((1, 8192, 16, 128), torch.bfloat16, 8),    # token rows of 4 KiB
    ((1, 8192, 16), torch.float32, 8),           # LSE rows of 64 B
    ((2, 60, 3, 5), torch.float32, 3),           # 60-byte rows: 4-byte path, batch 2
    ((1, 1536, 32, 128), torch.bfloat16, 16),    # 8 KiB rows, N = 16
    ((3, 48, 2, 8), torch.bfloat16, 48),         # N = S
    ((1, 7, 4), torch.float32, 1),               # N = 1 (identity)
    ((1, 1536, 3, 4096), torch.bfloat16, 16),    # 24 KiB rows (one row per workgroup), L = 96
    ((2, 3072, 32, 128), torch.bfloat16, 3),     # N = 3, batch 2
    ((1, 393216, 1, 8), torch.float32, 16),      # 32-byte rows, L = 24,576 (not a power of two)
    ((1, 786432, 32, 128), torch.bfloat16, 16),  # Very long Q/K/V (6.4 GB): the large-tensor launch shape
    ((1, 393216, 3, 60), torch.float32, 16),     # 720-byte rows, 283 MB: 4-byte path, large-tensor shape
])
def test_permute_bit_exact(sra, shape, dtype, n_dev):
    say("permute", shape, dtype, n_dev)
    g = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn(shape, generator=g, device="cuda").to(dtype)
    y = sra.stripe_permute(x, n_dev)
    torch.cuda.synchronize()
    perm = torch.from_numpy(oracle.stripe_index(shape[1], n_dev, oracle.STRIPED)).cuda()
    ref = x.index_select(1, perm)
    iview = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(y.view(iview), ref.view(iview))
    back = sra.unstripe(y, n_dev)
    assert torch.equal(back.view(iview), x.view(iview))


# --------------------------------------------------------- per-round path --

def _partials_case(sra, S, N, H, D, dtype, seed, layouts=LAYOUTS, per_device=False):
    g = torch.Generator().manual_seed(seed)
    q, k, v = (torch.randn((1, S, H, D), generator=g) * 0.5 for _ in range(3))
    q, k, v = (t.to(dtype) for t in (q, k, v))
    worst = 0.0
    for layout in layouts:
        qd, kd, vd = (to_dev_layout(t, N, layout) for t in (q, k, v))
        gq, gk, gv = (t.cuda() for t in (qd, kd, vd))
        L = S // N
        for r in range(N):
            if per_device:
                outs = {}
                for d in range(N):
                    outs[d] = sra.ring_round_attn(gq, gk, gv, N, layout, r, device=d)
            else:
                o_all, l_all = sra.ring_round_attn(gq, gk, gv, N, layout, r)
            torch.cuda.synchronize()
            for d in range(N):
                o_ref, l_ref = oracle.ring_partial(qd, kd, vd, N, layout, d, r)
                o_g, l_g = outs[d] if per_device else (o_all, l_all)
                o_g = np64(o_g[:, d * L:(d + 1) * L])
                l_g = np64(l_g[:, d * L:(d + 1) * L])
                e = max(maxabs(o_g, o_ref), maxabs(l_g, l_ref))
                worst = max(worst, e)
                assert e <= TOL[dtype], (layout, r, d, e)
    say(f"partials S={S} N={N} H={H} {dtype}: worst max-abs {worst:.3g}")
    return worst


def test_round_partials_fp32_tiny(sra):
    w = WORKLOADS["tiny"]
    _partials_case(sra, w["seq"], w["n_dev"], w["heads"], w["head_dim"], torch.float32, 1, per_device=True)


def test_round_partials_fp32_d128_ragged(sra):
    _partials_case(sra, 3 * 70, 3, 2, 128, torch.float32, 2)


@pytest.mark.parametrize("S,N,H", [(1024, 2, 2), (8 * 200, 8, 2), (512, 4, 3), (16, 16, 1), (130, 1, 2),
                                   (64, 1, 1), (128, 1, 1)])
def test_round_partials_bf16(sra, S, N, H):
    _partials_case(sra, S, N, H, 128, torch.bfloat16, 3 + S + N)


def test_round_single_device_selection_bf16(sra):
    _partials_case(sra, 1024, 4, 2, 128, torch.bfloat16, 5, per_device=True)


def test_lse_merge_matches_oracle(sra):
    g = torch.Generator().manual_seed(7)
    R, D = 4096, 128
    oa, ob = torch.randn(R, D, generator=g), torch.randn(R, D, generator=g)
    la, lb = torch.randn(R, generator=g) * 3, torch.randn(R, generator=g) * 3
    la[::5] = float("-inf")
    lb[::7] = float("-inf")
    oa[::5] = 0
    ob[::7] = 0
    o_ref, l_ref = oracle.lse_merge(oa.numpy(), la.numpy(), ob.numpy(), lb.numpy())
    ga, gla = oa.cuda(), la.cuda()
    sra.lse_merge(ga, gla, ob.cuda(), lb.cuda())
    torch.cuda.synchronize()
    assert maxabs(np64(ga), o_ref) <= 1e-5
    assert maxabs(np64(gla), l_ref) <= 1e-5


# ------------------------------------------------------------ full driver --

def _census(sra, S, N, layout, dtype, H, B=1):
    tq, tk = sra.kernel_tiles(dtype, 128 if dtype == torch.bfloat16 else 64)
    live, _, _ = sra.count_live_tiles(S, N, layout, tq, tk)
    return live * (H * B)


def run_full(sra, x, n_dev, layout):
    """Original-order inputs -> device layout -> ring fwd -> original order."""
    q, k, v = x["q"], x["k"], x["v"]
    if layout == oracle.STRIPED:
        qd, kd, vd = (sra.stripe_permute(t, n_dev) for t in (q, k, v))
    else:
        qd, kd, vd = q, k, v
    counts = torch.zeros(n_dev * n_dev, dtype=torch.int64, device=q.device)
    o, lse = sra.ring_attn_fwd(qd, kd, vd, n_dev, layout, live_counts=counts)
    if layout == oracle.STRIPED:
        o, lse = sra.unstripe(o, n_dev), sra.unstripe(lse, n_dev)
    torch.cuda.synchronize()
    return o, lse, counts.view(n_dev, n_dev).cpu()


def test_fwd_tiny_fp32_dense_parity(sra):
    w = WORKLOADS["tiny"]
    x = make_inputs("tiny", device="cpu")
    o_ref, l_ref = oracle.dense_causal_attention(x["q"], x["k"], x["v"])
    xg = {n: t.cuda() for n, t in x.items()}
    outs = {}
    for layout in LAYOUTS:
        o, lse, counts = run_full(sra, xg, w["n_dev"], layout)
        e_o, e_l = maxabs(np64(o), o_ref), maxabs(np64(lse), l_ref)
        say(f"tiny layout={layout}: O {e_o:.3g}  LSE {e_l:.3g}")
        assert e_o <= 1e-5 and e_l <= 1e-5
        assert torch.equal(o[:, 0], xg["v"][:, 0])                  # O_0 == V_0 exactly
        assert torch.equal(counts, _census(sra, w["seq"], w["n_dev"], layout, torch.float32, w["heads"]))
        outs[layout] = o
    assert maxabs(np64(outs[0]), np64(outs[1])) <= 1e-5             # equivariance


@pytest.fixture(scope="module")
def short_case():
    x = make_inputs("short", device="cuda")
    say("short: computing dense fp64 oracle on the host ...")
    cpu = {n: t.cpu() for n, t in x.items()}
    o_ref, l_ref = oracle.dense_causal_attention(cpu["q"], cpu["k"], cpu["v"])
    return x, o_ref, l_ref


@pytest.mark.parametrize("layout", LAYOUTS)
def test_fwd_short_bf16_dense_parity(sra, short_case, layout):
    w = WORKLOADS["short"]
    x, o_ref, l_ref = short_case
    o, lse, counts = run_full(sra, x, w["n_dev"], layout)
    e_o, e_l = maxabs(np64(o), o_ref), maxabs(np64(lse), l_ref)
    rel = e_o / float(np.abs(o_ref).max())
    say(f"short layout={layout}: O max-abs {e_o:.3g} (rel {rel:.3g})  LSE {e_l:.3g}")
    assert e_o <= 2e-2 and e_l <= 2e-2
    assert torch.equal(o[:, 0], x["v"][:, 0])
    assert torch.equal(counts, _census(sra, w["seq"], w["n_dev"], layout, torch.bfloat16, w["heads"]))


def test_fwd_short_striped_equals_contiguous(sra, short_case):
    w = WORKLOADS["short"]
    x, _, _ = short_case
    o_s, l_s, _ = run_full(sra, x, w["n_dev"], oracle.STRIPED)
    o_c, l_c, _ = run_full(sra, x, w["n_dev"], oracle.CONTIGUOUS)
    assert (o_s.float() - o_c.float()).abs().max().item() <= 2e-2
    assert (l_s - l_c).abs().max().item() <= 2e-2


def sampled_rows(S, N, n_random, seed):
    """Row 0, the first two and last two tokens of every device's stripe, and
    random rows (original positions)."""
    rows = {0}
    for d in range(N):
        L = S // N
        for j in (0, 1, L - 2, L - 1):
            rows.add(j * N + d)
    rows |= set(np.random.default_rng(seed).integers(0, S, n_random).tolist())
    return np.array(sorted(rows))


@pytest.mark.slow
def test_fwd_mid_bf16_sampled_rows(sra):
    """Mid (65,536 tokens, 32 heads, 8 devices): sampled rows on every head
    against the oracle, for the per-round schedule in both layouts and for
    the benchmark's launch (fused, striped, original order)."""
    w = WORKLOADS["mid"]
    x = make_inputs("mid", device="cuda")
    rows = sampled_rows(w["seq"], w["n_dev"], 24, 5)
    cpu = {n: x[n][:, :int(rows.max()) + 1].cpu() for n in ("q", "k", "v")}
    o_ref, l_ref = oracle.attention_rows(cpu["q"], cpu["k"], cpu["v"], rows)
    say(f"mid: {len(rows)} sampled rows x {w['heads']} heads")
    for layout in LAYOUTS:
        o, lse, counts = run_full(sra, x, w["n_dev"], layout)
        e_o, e_l = maxabs(np64(o[:, rows]), o_ref), maxabs(np64(lse[:, rows]), l_ref)
        say(f"mid layout={layout}: sampled O {e_o:.3g} LSE {e_l:.3g}")
        assert e_o <= 2e-2 and e_l <= 2e-2
        assert torch.equal(counts, _census(sra, w["seq"], w["n_dev"], layout, torch.bfloat16, w["heads"]))
    o, lse = sra.ring_attn_fwd(x["q"], x["k"], x["v"], w["n_dev"], oracle.STRIPED, schedule=sra.SCHEDULE_FUSED,
                               order=sra.ORDER_ORIGINAL)
    torch.cuda.synchronize()
    e_o, e_l = maxabs(np64(o[:, rows]), o_ref), maxabs(np64(lse[:, rows]), l_ref)
    say(f"mid fused original order: sampled O {e_o:.3g} LSE {e_l:.3g}")
    assert e_o <= 2e-2 and e_l <= 2e-2
    assert torch.equal(o[:, 0], x["v"][:, 0])


@pytest.mark.slow
def test_fwd_mid_zero_query_closed_form(sra):
    """Q = 0: every live key has weight 1/(i+1), so LSE_i = log(i+1) and O_i is
    the prefix mean of V (fp64 cumsum on the host), at the full Mid shape."""
    w = WORKLOADS["mid"]
    x = make_inputs("mid", device="cuda")
    x["q"].zero_()
    heads = [3, 30]
    S = w["seq"]
    vcpu = x["v"][:, :, heads].cpu().double().numpy()
    prefix = np.cumsum(vcpu, axis=1) / np.arange(1, S + 1, dtype=np.float64)[None, :, None, None]
    for layout in LAYOUTS:
        o, lse, _ = run_full(sra, x, w["n_dev"], layout)
        l_ref = np.log(np.arange(1, S + 1, dtype=np.float64))[None, :, None]
        e_l = float(np.abs(np64(lse) - l_ref).max())
        e_o = float(np.abs(np64(o[:, :, heads]) - prefix).max())
        say(f"mid Q=0 layout={layout}: O {e_o:.3g} LSE {e_l:.3g}")
        assert e_o <= 2e-2 and e_l <= 2e-2


# ---------------------------------------------------- fused all-rounds path --

def run_full_fused(sra, x, n_dev, layout):
    q, k, v = x["q"], x["k"], x["v"]
    if layout == oracle.STRIPED:
        q, k, v = (sra.stripe_permute(t, n_dev) for t in (q, k, v))
    counts = torch.zeros(n_dev * n_dev, dtype=torch.int64, device=q.device)
    o, lse = sra.ring_attn_fwd(q, k, v, n_dev, layout, schedule=sra.SCHEDULE_FUSED, live_counts=counts)
    if layout == oracle.STRIPED:
        o, lse = sra.unstripe(o, n_dev), sra.unstripe(lse, n_dev)
    torch.cuda.synchronize()
    return o, lse, counts.view(n_dev, n_dev).cpu()


@pytest.mark.parametrize("layout", LAYOUTS)
def test_fwd_short_bf16_fused_dense_parity(sra, short_case, layout):
    w = WORKLOADS["short"]
    x, o_ref, l_ref = short_case
    o, lse, counts = run_full_fused(sra, x, w["n_dev"], layout)
    e_o, e_l = maxabs(np64(o), o_ref), maxabs(np64(lse), l_ref)
    say(f"short fused layout={layout}: O max-abs {e_o:.3g}  LSE {e_l:.3g}")
    assert e_o <= 2e-2 and e_l <= 2e-2
    assert torch.equal(o[:, 0], x["v"][:, 0])
    assert torch.equal(counts, _census(sra, w["seq"], w["n_dev"], layout, torch.bfloat16, w["heads"]))
    o2, l2, _ = run_full(sra, x, w["n_dev"], layout)        # per-round schedule, same inputs
    assert (o.float() - o2.float()).abs().max().item() <= 2e-2
    assert (lse - l2).abs().max().item() <= 1e-4


@pytest.mark.parametrize("layout", LAYOUTS)
def test_fwd_short_original_order_fused_dense_parity(sra, short_case, layout):
    """The launch the benchmark times: Short, fused schedule, tensors in original
    token order (each device's stripe read in place). Every row and head against
    the dense fp64 oracle, and bit-identical to the device-layout path."""
    w = WORKLOADS["short"]
    x, o_ref, l_ref = short_case
    o, lse = sra.ring_attn_fwd(x["q"], x["k"], x["v"], w["n_dev"], layout, schedule=sra.SCHEDULE_FUSED,
                               order=sra.ORDER_ORIGINAL)
    torch.cuda.synchronize()
    e_o, e_l = maxabs(np64(o), o_ref), maxabs(np64(lse), l_ref)
    say(f"short fused original order layout={layout}: O max-abs {e_o:.3g}  LSE {e_l:.3g}")
    assert e_o <= 2e-2 and e_l <= 2e-2
    assert torch.equal(o[:, 0], x["v"][:, 0])
    o_d, l_d, _ = run_full_fused(sra, x, w["n_dev"], layout)
    assert torch.equal(o, o_d) and torch.equal(lse, l_d)


@pytest.mark.parametrize("S,N,H", [(8 * 200, 8, 2), (1024, 1, 2), (16, 16, 1), (4 * 300, 4, 3),
                                   (64, 1, 1), (128, 1, 2), (192, 1, 1), (2 * 96, 2, 1)])
def test_fwd_fused_small_dense_parity(sra, S, N, H):
    """Ragged shards (L not a multiple of the 256 x 64 tile), one device, one
    token per device, and workgroups with one, two or three key tiles in all
    (the first and last steps of both wave groups); both layouts."""
    g = torch.Generator().manual_seed(S + N + H)
    x = {n: (torch.randn((1, S, H, 128), generator=g) * 0.5).to(torch.bfloat16) for n in ("q", "k", "v")}
    o_ref, l_ref = oracle.dense_causal_attention(x["q"], x["k"], x["v"])
    xg = {n: t.cuda() for n, t in x.items()}
    for layout in LAYOUTS:
        o, lse, counts = run_full_fused(sra, xg, N, layout)
        e_o, e_l = maxabs(np64(o), o_ref), maxabs(np64(lse), l_ref)
        assert e_o <= 2e-2 and e_l <= 2e-2, (layout, e_o, e_l)
        assert torch.equal(counts, _census(sra, S, N, layout, torch.bfloat16, H))


@pytest.mark.parametrize("S,N,H", [(2048, 4, 2), (8 * 200, 8, 1)])
def test_fwd_rising_scores_rescale(sra, S, N, H):
    """Scores that rise along the sequence (keys grow along the queries' shared
    direction, about 3 log2 units per 64-key tile): a row's running offset has
    to be raised again and again within and across key tiles, so the weights'
    overflow check, the exact row-max path and the pending O rescale all run.
    Fused and per-round schedules, both layouts, against the dense fp64
    oracle on the same bf16 inputs."""
    g = torch.Generator().manual_seed(7 + S + N)
    u = torch.randn(128, generator=g, dtype=torch.float64)
    u /= u.norm()
    ramp = (torch.arange(S, dtype=torch.float64) / S)[None, :, None, None]
    q = 4.0 * u + 0.3 * torch.randn((1, S, H, 128), generator=g, dtype=torch.float64)
    k = 200.0 * ramp * u + 0.3 * torch.randn((1, S, H, 128), generator=g, dtype=torch.float64)
    v = 0.5 * torch.randn((1, S, H, 128), generator=g, dtype=torch.float64)
    x = {n: t.to(torch.bfloat16) for n, t in (("q", q), ("k", k), ("v", v))}
    o_ref, l_ref = oracle.dense_causal_attention(x["q"], x["k"], x["v"])
    assert float(l_ref.max()) > 40.0   # the last rows' scores are far above their first ones
    xg = {n: t.cuda() for n, t in x.items()}
    for layout in LAYOUTS:
        for name, run in (("fused", run_full_fused), ("per-round", run_full)):
            o, lse, _ = run(sra, xg, N, layout)
            e_o, e_l = maxabs(np64(o), o_ref), maxabs(np64(lse), l_ref)
            say(f"rising scores S={S} N={N} layout={layout} {name}: O max-abs {e_o:.3g}  LSE {e_l:.3g}")
            assert e_o <= 2e-2 and e_l <= 2e-2, (layout, name, e_o, e_l)
