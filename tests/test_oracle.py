"""Pins for the CPU oracle: it is checked against things other than itself.

* brute force: pure-Python loops (``math`` only, no numpy matmul) on tiny inputs;
* closed forms: Q = 0 gives lse_i = log(i+1) and a prefix mean; tile census
  formulas; per-round contiguous imbalance N/(N-r);
* invariants: row softmax sums, O_0 = V_0, permutation equivariance (striped
  result un-striped == contiguous == dense), key-shift invariance, structured
  self/previous/future-match inputs, gradient sum rules;
* a library special case: with one device the ring is plain causal attention,
  equal to torch's scaled_dot_product_attention(is_causal=True) in fp64;
* finite differences for the backward pass;
* mutation tests: a plausible mistake is planted in a copy of the oracle's
  source (on the CPU) and one of the pins above must fail on it.
"""

import math
import pathlib
import types

import numpy as np
import pytest

import oracle
from oracle import attention as oatt
from oracle import stripes as ost

ORACLE_DIR = pathlib.Path(oatt.__file__).parent


# ----------------------------------------------------------------- helpers --

def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def bf_causal(Q, K, V, scale):
    """Causal attention for one head by pure-Python loops over lists."""
    S, D = len(Q), len(Q[0])
    O, LSE = [], []
    for i in range(S):
        sc = [scale * sum(Q[i][c] * K[j][c] for c in range(D)) for j in range(i + 1)]
        m = max(sc)
        z = sum(math.exp(x - m) for x in sc)
        LSE.append(m + math.log(z))
        O.append([sum(math.exp(sc[j] - m) / z * V[j][c] for j in range(i + 1)) for c in range(D)])
    return O, LSE


def bf_masked(Q, K, V, live, scale):
    """Softmax attention over an explicit liveness matrix (list of lists of
    bools); rows with no live key give O = 0, lse = -inf."""
    O, LSE = [], []
    D = len(Q[0])
    for i in range(len(Q)):
        idx = [j for j in range(len(K)) if live[i][j]]
        if not idx:
            O.append([0.0] * D)
            LSE.append(-math.inf)
            continue
        sc = {j: scale * sum(Q[i][c] * K[j][c] for c in range(D)) for j in idx}
        m = max(sc.values())
        z = sum(math.exp(x - m) for x in sc.values())
        LSE.append(m + math.log(z))
        O.append([sum(math.exp(sc[j] - m) / z * V[j][c] for j in idx) for c in range(D)])
    return O, LSE


def explicit_position(n_dev, L, layout, dev, j):
    """Position of device ``dev``'s j-th token, straight from the layout's
    wording: contiguous chunk, or every N-th token starting at ``dev``."""
    return dev * L + j if layout == ost.CONTIGUOUS else dev + j * n_dev


# ------------------------------------------------------------ dense forward --

@pytest.mark.parametrize("S,D,H", [(1, 3, 1), (5, 1, 2), (17, 4, 2), (33, 8, 1), (300, 2, 1)])
def test_dense_matches_brute_force(S, D, H):
    q, k, v = (rand((2, S, H, D), s) for s in (1, 2, 3))
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.dense_causal_attention(q, k, v)
    for b in range(2):
        for h in range(H):
            O, LSE = bf_causal(q[b, :, h].tolist(), k[b, :, h].tolist(), v[b, :, h].tolist(), scale)
            np.testing.assert_allclose(o[b, :, h], np.array(O), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, :, h], np.array(LSE), rtol=0, atol=1e-12)


def test_explicit_scale_is_used():
    q, k, v = (rand((1, 9, 1, 4), s) for s in (4, 5, 6))
    o, lse = oracle.dense_causal_attention(q, k, v, scale=0.3)
    O, LSE = bf_causal(q[0, :, 0].tolist(), k[0, :, 0].tolist(), v[0, :, 0].tolist(), 0.3)
    np.testing.assert_allclose(o[0, :, 0], np.array(O), atol=1e-12)
    np.testing.assert_allclose(lse[0, :, 0], np.array(LSE), atol=1e-12)


def test_softmax_rows_sum_to_one():
    B, S, H, D = 1, 700, 2, 16
    q, k, v = (rand((B, S, H, D), s) for s in (7, 8, 9))
    _, lse = oracle.dense_causal_attention(q, k, v)
    sc = 1.0 / math.sqrt(D)
    for h in range(H):
        s = sc * q[0, :, h] @ k[0, :, h].T
        mask = np.tril(np.ones((S, S), dtype=bool))
        p = np.where(mask, np.exp(np.where(mask, s, 0) - lse[0, :, h][:, None]), 0.0)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_first_output_is_first_value_exactly():
    q, k, v = (rand((2, 300, 3, 32), s) for s in (10, 11, 12))
    o, lse = oracle.dense_causal_attention(q, k, v)
    assert np.array_equal(o[:, 0], v[:, 0])
    sc = 1.0 / math.sqrt(32)
    np.testing.assert_allclose(lse[:, 0], sc * (q[:, 0] * k[:, 0]).sum(-1), atol=1e-13)


def test_zero_query_closed_form():
    B, S, H, D = 1, 600, 2, 8
    q = np.zeros((B, S, H, D))
    k, v = rand((B, S, H, D), 13), rand((B, S, H, D), 14)
    o, lse = oracle.dense_causal_attention(q, k, v)
    i = np.arange(S)
    np.testing.assert_allclose(lse[0], np.log(i + 1.0)[:, None].repeat(H, 1), rtol=0, atol=1e-12)
    prefix_mean = np.cumsum(v, axis=1) / (i + 1.0)[None, :, None, None]
    np.testing.assert_allclose(o, prefix_mean, rtol=0, atol=1e-12)


def test_single_device_matches_torch_sdpa_fp64():
    torch = pytest.importorskip("torch")
    B, S, H, D = 2, 320, 3, 16
    q, k, v = (rand((B, S, H, D), s) for s in (15, 16, 17))
    o, _ = oracle.ring_attention(q, k, v, 1, ost.STRIPED)
    t = lambda a: torch.from_numpy(a).permute(0, 2, 1, 3).contiguous()  # noqa: E731
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
    ref = ref.permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def _pin_rows(mod):
    q, k, v = (rand((1, 21, 2, 3), s) for s in (21, 22, 23))
    rows = np.array([0, 1, 7, 20])
    o, lse = mod.attention_rows(q, k, v, rows)
    for h in range(2):
        O, LSE = bf_causal(q[0, :, h].tolist(), k[0, :, h].tolist(), v[0, :, h].tolist(), 1.0 / math.sqrt(3))
        np.testing.assert_allclose(o[0, :, h], np.array(O)[rows], atol=1e-12)
        np.testing.assert_allclose(lse[0, :, h], np.array(LSE)[rows], atol=1e-12)


def test_attention_rows_brute_force():
    _pin_rows(oracle)


def test_attention_rows_matches_dense():
    q, k, v = (rand((2, 520, 2, 8), s) for s in (18, 19, 20))
    o, lse = oracle.dense_causal_attention(q, k, v)
    rows = np.array([0, 1, 255, 256, 257, 519])
    orow, lrow = oracle.attention_rows(q, k, v, rows)
    np.testing.assert_allclose(orow, o[:, rows], atol=1e-12)
    np.testing.assert_allclose(lrow, lse[:, rows], atol=1e-12)


# ------------------------------------------------------- structured inputs --

def _unit_rows(shape, seed):
    u = rand(shape, seed)
    return u / np.linalg.norm(u, axis=-1, keepdims=True)


def test_self_match_recovers_values():
    B, S, H, D = 1, 2048, 1, 64
    c = math.sqrt(64.0 * math.sqrt(D))       # scale * c^2 = 64
    u = _unit_rows((B, S, H, D), 21)
    v = rand((B, S, H, D), 22)
    o, lse = oracle.dense_causal_attention(c * u, c * u, v)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-6)
    np.testing.assert_allclose(lse, 64.0, rtol=0, atol=1e-6)


def test_previous_match_and_future_mask():
    B, S, H, D = 1, 1024, 1, 64
    c = math.sqrt(64.0 * math.sqrt(D))
    u = _unit_rows((B, S + 1, H, D), 23)
    v = rand((B, S, H, D), 24)
    k = c * u[:, :S]
    # previous match: Q_i = K_{i-1} (i >= 1) -> O_i ~ V_{i-1}
    qprev = np.concatenate([k[:, :1], k[:, :-1]], axis=1)
    o, _ = oracle.dense_causal_attention(qprev, k, v)
    np.testing.assert_allclose(o[:, 1:], v[:, :-1], rtol=0, atol=1e-6)
    # future match: Q_i = K_{i+1} must not see V_{i+1}
    qnext = c * u[:, 1:]
    o, _ = oracle.dense_causal_attention(qnext, k, v)
    a, b = o[0, :-1, 0], v[0, 1:, 0]
    cos = (a * b).sum(-1) / (np.linalg.norm(a, axis=-1) * np.linalg.norm(b, axis=-1) + 1e-300)
    assert cos.max() < 0.9


def test_key_shift_invariance():
    B, S, H, D = 1, 300, 2, 8
    q, k, v = (rand((B, S, H, D), s) for s in (25, 26, 27))
    u = rand((D,), 28)
    o1, l1 = oracle.dense_causal_attention(q, k, v)
    o2, l2 = oracle.dense_causal_attention(q, k + u, v)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, (q @ u) / math.sqrt(D), atol=1e-12)


# ------------------------------------------------------------- layouts ----

@pytest.mark.parametrize("layout", [ost.CONTIGUOUS, ost.STRIPED])
@pytest.mark.parametrize("S,N", [(8, 1), (8, 2), (12, 3), (16, 4), (64, 8), (24, 24)])
def test_positions_follow_the_layout_wording(S, N, layout):
    L = S // N
    pos = oracle.positions(S, N, layout)
    assert sorted(pos.tolist()) == list(range(S))           # a bijection
    for d in range(N):
        for j in range(L):
            assert pos[d * L + j] == explicit_position(N, L, layout, d, j)
    inv = oracle.unstripe_index(S, N, layout)
    for p in range(S):
        closed = (p % N) * L + p // N if layout == ost.STRIPED else p
        assert inv[p] == closed


def test_striped_devices_hold_every_nth_token():
    S, N = 96, 8
    L = S // N
    pos = oracle.positions(S, N, ost.STRIPED)
    for d in range(N):
        mine = pos[d * L:(d + 1) * L]
        assert mine[0] == d and np.all(np.diff(mine) == N)


def test_degenerate_layouts_coincide():
    for S in (1, 7, 32):
        ident = np.arange(S)
        assert np.array_equal(oracle.positions(S, 1, ost.STRIPED), ident)
        assert np.array_equal(oracle.positions(S, S, ost.STRIPED), ident)
        assert np.array_equal(oracle.positions(S, S, ost.CONTIGUOUS), ident)


def test_layout_round_trip():
    x = rand((2, 48, 3, 5), 29)
    for layout in (ost.CONTIGUOUS, ost.STRIPED):
        for N in (1, 2, 3, 4, 6, 8, 48):
            y = oracle.to_device_layout(x, N, layout)
            assert np.array_equal(oracle.from_device_layout(y, N, layout), x)


def test_round_source_ring_order():
    N = 5
    for d in range(N):
        assert oracle.round_source(d, 0, N) == d
        # round r+1 holds what the previous device held in round r
        for r in range(N - 1):
            assert oracle.round_source(d, r + 1, N) == oracle.round_source((d - 1) % N, r, N)
        assert sorted(oracle.round_source(d, r, N) for r in range(N)) == list(range(N))


# ------------------------------------------------------------ ring rounds --

@pytest.mark.parametrize("layout", [ost.CONTIGUOUS, ost.STRIPED])
@pytest.mark.parametrize("S,N,D", [(8, 1, 4), (8, 2, 4), (12, 3, 2), (16, 4, 4), (32, 8, 8), (8, 8, 2)])
def test_ring_partial_matches_brute_force(S, N, D, layout):
    L = S // N
    q, k, v = (rand((1, S, 1, D), s) for s in (30, 31, 32))
    scale = 1.0 / math.sqrt(D)
    for d in range(N):
        for r in range(N):
            src = (d - r) % N
            o, lse = oracle.ring_partial(q, k, v, N, layout, d, r)
            live = [[explicit_position(N, L, layout, src, kk) <= explicit_position(N, L, layout, d, j)
                     for kk in range(L)] for j in range(L)]
            O, LSE = bf_masked(q[0, d * L:(d + 1) * L, 0].tolist(), k[0, src * L:(src + 1) * L, 0].tolist(),
                               v[0, src * L:(src + 1) * L, 0].tolist(), live, scale)
            np.testing.assert_allclose(o[0, :, 0], np.array(O), atol=1e-12)
            assert np.array_equal(np.isneginf(lse[0, :, 0]), np.isneginf(np.array(LSE)))
            fin = np.isfinite(np.array(LSE))
            np.testing.assert_allclose(lse[0, fin, 0], np.array(LSE)[fin], atol=1e-12)


@pytest.mark.parametrize("S,N", [(64, 1), (64, 2), (96, 3), (128, 4), (256, 8), (16, 16)])
def test_permutation_equivariance(S, N):
    B, H, D = 1, 2, 8
    q, k, v = (rand((B, S, H, D), s) for s in (33, 34, 35))
    o_ref, l_ref = oracle.dense_causal_attention(q, k, v)
    outs = {}
    for layout in (ost.CONTIGUOUS, ost.STRIPED):
        dev = [oracle.to_device_layout(t, N, layout) for t in (q, k, v)]
        o, lse = oracle.ring_attention(*dev, N, layout)
        outs[layout] = (oracle.from_device_layout(o, N, layout), oracle.from_device_layout(lse, N, layout))
        np.testing.assert_allclose(outs[layout][0], o_ref, atol=1e-12)
        np.testing.assert_allclose(outs[layout][1], l_ref, atol=1e-12)
    np.testing.assert_allclose(outs[0][0], outs[1][0], atol=1e-12)


def test_striped_empty_rows_only_at_first_token():
    """Striped, source after the query device: token 0 has no live key."""
    S, N = 32, 4
    q, k, v = (rand((1, S, 1, 4), s) for s in (36, 37, 38))
    for d in range(N):
        for r in range(N):
            src = (d - r) % N
            _, lse = oracle.ring_partial(q, k, v, N, ost.STRIPED, d, r)
            empty = np.isneginf(lse[0, :, 0])
            assert empty[0] == (src > d)
            assert not empty[1:].any()


# ------------------------------------------------------------------ merge --

def test_merge_identity_and_empty():
    o = rand((3, 5, 4), 39)
    l = rand((3, 5), 40)
    zero, ninf = np.zeros_like(o), np.full_like(l, -np.inf)
    mo, ml = oracle.lse_merge(o, l, zero, ninf)
    assert np.array_equal(mo, o) and np.array_equal(ml, l)
    mo, ml = oracle.lse_merge(zero, ninf, o, l)
    assert np.array_equal(mo, o) and np.array_equal(ml, l)
    mo, ml = oracle.lse_merge(zero, ninf, zero, ninf)
    assert np.array_equal(mo, zero) and np.all(np.isneginf(ml))


def test_merge_of_disjoint_key_sets_equals_union():
    D, nq, nk = 3, 4, 9
    Q, K, V = rand((nq, D), 41).tolist(), rand((nk, D), 42).tolist(), rand((nk, D), 43).tolist()
    sets = [[0, 2, 3], [1, 4], [5, 6, 7, 8]]
    parts = []
    for keys in sets:
        live = [[kk in keys for kk in range(nk)] for _ in range(nq)]
        O, LSE = bf_masked(Q, K, V, live, 0.7)
        parts.append((np.array(O), np.array(LSE)))
    Ou, Lu = bf_masked(Q, K, V, [[True] * nk for _ in range(nq)], 0.7)
    o, l = parts[0]
    for po, pl in parts[1:]:
        o, l = oracle.lse_merge(o, l, po, pl)
    np.testing.assert_allclose(o, np.array(Ou), atol=1e-12)
    np.testing.assert_allclose(l, np.array(Lu), atol=1e-12)
    # order does not matter
    o2, l2 = oracle.lse_merge(*oracle.lse_merge(parts[2][0], parts[2][1], parts[0][0], parts[0][1]), *parts[1])
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(l2, l, atol=1e-12)


# -------------------------------------------------------------- tile census --

def closed_form_census(S, N, layout, T):
    """Live/full/partial tiles per (r, d) for square power-of-two tiles that
    divide L, from the mask algebra: striped reduces to k <= j (source not
    after the query device) or k < j (source after it), so every (d, r) has
    T(T-1)/2 full and T partial tiles; contiguous is all-full before the
    diagonal block, triangular on it, and empty after it."""
    L = S // N
    t = L // T
    live = np.zeros((N, N), dtype=np.int64)
    full = np.zeros_like(live)
    part = np.zeros_like(live)
    for r in range(N):
        for d in range(N):
            src = (d - r) % N
            if layout == ost.STRIPED or src == d:
                full[r, d], part[r, d] = t * (t - 1) // 2, t
            elif src < d:
                full[r, d] = t * t
    live[:] = full + part
    return live, full, part


@pytest.mark.parametrize("layout", [ost.CONTIGUOUS, ost.STRIPED])
@pytest.mark.parametrize("S,N,T", [(256, 4, 16), (256, 4, 64), (512, 8, 16), (384, 3, 32), (64, 4, 4)])
def test_tile_census_closed_forms(S, N, T, layout):
    got = oracle.live_tiles(S, N, layout, T, T)
    want = closed_form_census(S, N, layout, T)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)


def test_tile_census_ragged_matches_pairwise_enumeration():
    S, N, tq, tk = 60, 3, 7, 6          # L = 20: ragged last tiles on both axes
    L = S // N
    for layout in (ost.CONTIGUOUS, ost.STRIPED):
        live, full, part = oracle.live_tiles(S, N, layout, tq, tk)
        for r in range(N):
            for d in range(N):
                src = (d - r) % N
                f = p = 0
                for a in range(0, L, tq):
                    for b in range(0, L, tk):
                        cnt = tot = 0
                        for j in range(a, min(a + tq, L)):
                            for kk in range(b, min(b + tk, L)):
                                tot += 1
                                cnt += explicit_position(N, L, layout, src, kk) <= explicit_position(N, L, layout, d, j)
                        f += cnt == tot
                        p += 0 < cnt < tot
                assert (full[r, d], part[r, d], live[r, d]) == (f, p, f + p)


def test_contiguous_imbalance_per_round_and_striped_balance():
    S, N, T = 1024, 8, 16
    for layout, expect in ((ost.CONTIGUOUS, lambda r: N / (N - r)), (ost.STRIPED, lambda r: 1.0)):
        live, _, _ = oracle.live_tiles(S, N, layout, T, T)
        for r in range(N):
            rho = live[r].max() / live[r].mean()
            assert rho == pytest.approx(expect(r), rel=1e-12)


def test_live_pairs_causal_half_and_striped_split():
    for S, N in ((64, 4), (96, 8), (60, 5)):
        L = S // N
        for layout in (ost.CONTIGUOUS, ost.STRIPED):
            pairs = oracle.live_pairs(S, N, layout)
            assert pairs.sum() == S * (S + 1) // 2            # causal: about half of S^2
        pairs = oracle.live_pairs(S, N, ost.STRIPED)
        for r in range(N):
            for d in range(N):
                src = (d - r) % N
                assert pairs[r, d] == (L * (L + 1) // 2 if src <= d else L * (L - 1) // 2)


# --------------------------------------------------------------- backward --

def _loss(q, k, v, do):
    o, _ = oracle.dense_causal_attention(q, k, v)
    return float((o * do).sum())


def test_backward_matches_finite_differences():
    B, S, H, D = 1, 6, 2, 3
    q, k, v, do = (rand((B, S, H, D), s) for s in (44, 45, 46, 47))
    o, lse = oracle.dense_causal_attention(q, k, v)
    grads = oracle.dense_causal_backward(q, k, v, o, lse, do)
    eps = 1e-6
    for which, g in enumerate(grads):
        args = [q, k, v]
        for idx in np.ndindex(*q.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            fd = (_loss(*plus, do) - _loss(*minus, do)) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-7, (which, idx, fd, g[idx])


def test_backward_matches_torch_autograd_fp64():
    torch = pytest.importorskip("torch")
    B, S, H, D = 1, 300, 2, 8
    q, k, v, do = (rand((B, S, H, D), s) for s in (48, 49, 50, 51))
    o, lse = oracle.dense_causal_attention(q, k, v)
    dq, dk, dv = oracle.dense_causal_backward(q, k, v, o, lse, do)
    tq, tk, tv = (torch.from_numpy(a).permute(0, 2, 1, 3).contiguous().requires_grad_() for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    out.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, t.grad.permute(0, 2, 1, 3).numpy(), atol=1e-11)


def test_backward_invariants_and_zero_query_closed_form():
    B, S, H, D = 1, 400, 2, 8
    q, k, v, do = (rand((B, S, H, D), s) for s in (52, 53, 54, 55))
    o, lse = oracle.dense_causal_attention(q, k, v)
    dq, dk, dv = oracle.dense_causal_backward(q, k, v, o, lse, do)
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), atol=1e-10)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-10)
    assert np.abs(dq[:, 0]).max() < 1e-14
    # Q = 0: uniform weights 1/(i+1)
    z = np.zeros_like(q)
    o, lse = oracle.dense_causal_attention(z, k, v)
    dq, dk, dv = oracle.dense_causal_backward(z, k, v, o, lse, do)
    assert np.abs(dk).max() < 1e-13
    i = np.arange(S, dtype=np.float64)
    w = do / (i + 1.0)[None, :, None, None]
    suffix = np.cumsum(w[:, ::-1], axis=1)[:, ::-1]
    np.testing.assert_allclose(dv, suffix, atol=1e-12)
    # dQ_i = scale/(i+1) [ sum_{k<=i} (V_k . dO_i) K_k - Delta_i sum_{k<=i} K_k ]
    sc = 1.0 / math.sqrt(D)
    for h in range(H):
        Kh, Vh, dOh, Oh = k[0, :, h], v[0, :, h], do[0, :, h], o[0, :, h]
        outer = np.cumsum(np.einsum("kc,ke->kce", Kh, Vh), axis=0)      # sum K_k V_k^T
        ksum = np.cumsum(Kh, axis=0)
        delta = (dOh * Oh).sum(-1)
        want = sc / (i + 1.0)[:, None] * (np.einsum("ice,ie->ic", outer, dOh) - delta[:, None] * ksum)
        np.testing.assert_allclose(dq[0, :, h], want, atol=1e-11)


def test_backward_key_rows_matches_dense():
    B, S, H, D = 1, 600, 3, 8
    q, k, v, do = (rand((B, S, H, D), s) for s in (56, 57, 58, 59))
    o, lse = oracle.dense_causal_attention(q, k, v)
    _, dk, dv = oracle.dense_causal_backward(q, k, v, o, lse, do)
    keys = np.array([300, 301, 450, 599])
    heads = [0, 2]
    dks, dvs = oracle.backward_key_rows(q, k, v, do, keys, heads)
    np.testing.assert_allclose(dks, dk[:, keys][:, :, heads], atol=1e-11)
    np.testing.assert_allclose(dvs, dv[:, keys][:, :, heads], atol=1e-11)


def test_backward_query_rows_matches_dense():
    B, S, H, D = 1, 600, 3, 8
    q, k, v, do = (rand((B, S, H, D), s) for s in (60, 61, 62, 63))
    o, lse = oracle.dense_causal_attention(q, k, v)
    dq, _, _ = oracle.dense_causal_backward(q, k, v, o, lse, do)
    rows = np.array([0, 1, 299, 300, 599])
    heads = [1, 2]
    got = oracle.backward_query_rows(q, k, v, do, rows, heads)
    np.testing.assert_allclose(got, dq[:, rows][:, :, heads], atol=1e-11)
    assert np.abs(got[:, 0]).max() < 1e-14          # dQ_0 = 0: row 0 sees only its own key


# --------------------------------------------------------- mutation tests --

def _mutant(module_file, old, new):
    """Load a copy of an oracle module with one planted mistake."""
    src = (ORACLE_DIR / module_file).read_text()
    assert src.count(old) >= 1, f"mutation anchor {old!r} not found in {module_file}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__package__"] = "oracle"
    mod.__dict__["__name__"] = "oracle.mutant"
    exec(compile(src, f"<mutant {module_file}>", "exec"), mod.__dict__)
    return mod


def _pin_dense(mod):
    q, k, v = (rand((1, 33, 2, 4), s) for s in (1, 2, 3))
    o, lse = mod.dense_causal_attention(q, k, v)
    for h in range(2):
        O, LSE = bf_causal(q[0, :, h].tolist(), k[0, :, h].tolist(), v[0, :, h].tolist(), 0.5)
        np.testing.assert_allclose(o[0, :, h], np.array(O), atol=1e-12)
        np.testing.assert_allclose(lse[0, :, h], np.array(LSE), atol=1e-12)


def _pin_ring(mod):
    S, N = 16, 4
    q, k, v = (rand((1, S, 1, 4), s) for s in (30, 31, 32))
    for layout in (ost.CONTIGUOUS, ost.STRIPED):
        L = S // N
        for d in range(N):
            for r in range(N):
                src = (d - r) % N
                o, _ = mod.ring_partial(q, k, v, N, layout, d, r)
                live = [[explicit_position(N, L, layout, src, kk) <= explicit_position(N, L, layout, d, j)
                         for kk in range(L)] for j in range(L)]
                O, _ = bf_masked(q[0, d * L:(d + 1) * L, 0].tolist(), k[0, src * L:(src + 1) * L, 0].tolist(),
                                 v[0, src * L:(src + 1) * L, 0].tolist(), live, 0.5)
                np.testing.assert_allclose(o[0, :, 0], np.array(O), atol=1e-12)


def _pin_merge(mod):
    D, nq, nk = 3, 4, 9
    Q, K, V = rand((nq, D), 41).tolist(), rand((nk, D), 42).tolist(), rand((nk, D), 43).tolist()
    a = bf_masked(Q, K, V, [[kk < 4 for kk in range(nk)] for _ in range(nq)], 0.7)
    b = bf_masked(Q, K, V, [[kk >= 4 for kk in range(nk)] for _ in range(nq)], 0.7)
    u = bf_masked(Q, K, V, [[True] * nk for _ in range(nq)], 0.7)
    o, l = mod.lse_merge(np.array(a[0]), np.array(a[1]), np.array(b[0]), np.array(b[1]))
    np.testing.assert_allclose(o, np.array(u[0]), atol=1e-12)
    np.testing.assert_allclose(l, np.array(u[1]), atol=1e-12)


def _pin_positions(mod):
    for layout in (ost.CONTIGUOUS, ost.STRIPED):
        for S, N in ((16, 4), (24, 3)):
            L = S // N
            pos = mod.positions(S, N, layout)
            for d in range(N):
                for j in range(L):
                    assert pos[d * L + j] == explicit_position(N, L, layout, d, j)


def _pin_census(mod):
    for layout in (ost.CONTIGUOUS, ost.STRIPED):
        got = mod.live_tiles(256, 4, layout, 16, 16)
        for g, w in zip(got, closed_form_census(256, 4, layout, 16)):
            assert np.array_equal(g, w)


def _pin_backward(mod):
    B, S, H, D = 1, 5, 1, 2
    q, k, v, do = (rand((B, S, H, D), s) for s in (44, 45, 46, 47))
    o, lse = oracle.dense_causal_attention(q, k, v)
    grads = mod.dense_causal_backward(q, k, v, o, lse, do)
    eps = 1e-6
    for which, g in enumerate(grads):
        for idx in np.ndindex(*q.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += eps
            fp = _loss(*args, do)
            args[which][idx] -= 2 * eps
            fm = _loss(*args, do)
            assert abs((fp - fm) / (2 * eps) - g[idx]) < 1e-7


MUTATIONS = [
    # (file, original text, planted mistake, pin that must catch it)
    ("attention.py", "s = np.where(cols <= rows, s, -np.inf)", "s = np.where(cols < rows, s, -np.inf)", _pin_dense),
    ("attention.py", "s = sc * (Q[i0:i1] @ K[:i1].T)\n                rows = np.arange(i0, i1)[:, None]\n                cols",
     "s = (Q[i0:i1] @ K[:i1].T)\n                rows = np.arange(i0, i1)[:, None]\n                cols", _pin_dense),
    ("attention.py", "o[b, i0:i1, h] = (e @ V[:i1]) / den", "o[b, i0:i1, h] = (e @ K[:i1]) / den", _pin_dense),
    ("attention.py", "lse[b, i0:i1, h] = (m + np.log(den))[:, 0]", "lse[b, i0:i1, h] = (np.log(den))[:, 0]", _pin_dense),
    ("attention.py", "live = kpos[None, :] <= qpos[:, None]", "live = kpos[None, :] < qpos[:, None]", _pin_ring),
    ("attention.py", "s = np.where(keys[None, :] <= rows[:, None], s, -np.inf)",
     "s = np.where(keys[None, :] < rows[:, None], s, -np.inf)", _pin_rows),
    ("attention.py", "K = k_dev[b, s_dev * L:(s_dev + 1) * L, h]", "K = k_dev[b, d * L:(d + 1) * L, h]", _pin_ring),
    ("attention.py", "o = (wa / tot)[..., None] * o_a + (wb / tot)[..., None] * o_b",
     "o = (wb / tot)[..., None] * o_a + (wa / tot)[..., None] * o_b", _pin_merge),
    ("attention.py", "ds = p * (dp - delta[i0:i1, None])", "ds = p * (dp + delta[i0:i1, None])", _pin_backward),
    ("attention.py", "dk[b, :i1, h] += sc * (ds.T @ Q[i0:i1])", "dk[b, :i1, h] += sc * (p.T @ Q[i0:i1])", _pin_backward),
    ("attention.py", "dq[b, i0:i1, h] = sc * (ds @ K[:i1])", "dq[b, i0:i1, h] = sc * (ds @ V[:i1])", _pin_backward),
    ("stripes.py", "pos[d * L + j] = j * n_dev + d", "pos[d * L + j] = j * n_dev + (n_dev - 1 - d)", _pin_positions),
    ("stripes.py", "return (d - r) % n_dev", "return (d + r) % n_dev", _pin_census),
]


@pytest.mark.parametrize("case", range(len(MUTATIONS)))
def test_planted_mistake_is_caught(case):
    fname, old, new, pin = MUTATIONS[case]
    mod = _mutant(fname, old, new)
    pin(oracle)                         # the real oracle passes the pin ...
    with pytest.raises(AssertionError):
        pin(mod)                        # ... the mutant fails it


# ------------------------------------------------- generated shapes (hypothesis) --

from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=40, deadline=None, derandomize=True)
@given(n_dev=st.integers(1, 6), L=st.integers(1, 5), D=st.integers(1, 4),
       layout=st.sampled_from([ost.CONTIGUOUS, ost.STRIPED]), seed=st.integers(0, 2**16),
       pick=st.integers(0, 35))
def test_generated_shapes_ring_matches_brute_force(n_dev, L, D, layout, seed, pick):
    """On generated shapes: the ring over all rounds, taken back to original
    order, equals causal attention by pure-Python loops; and one generated
    (device, round) partial equals the brute-force masked softmax over the
    keys whose position (the layout's wording) is at most the query's."""
    S = n_dev * L
    q, k, v = (rand((1, S, 1, D), seed + i) for i in range(3))
    scale = 1.0 / math.sqrt(D)
    O, LSE = bf_causal(q[0, :, 0].tolist(), k[0, :, 0].tolist(), v[0, :, 0].tolist(), scale)
    dev = [oracle.to_device_layout(t, n_dev, layout) for t in (q, k, v)]
    o, lse = oracle.ring_attention(*dev, n_dev, layout)
    o, lse = oracle.from_device_layout(o, n_dev, layout), oracle.from_device_layout(lse, n_dev, layout)
    np.testing.assert_allclose(o[0, :, 0], np.array(O), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, :, 0], np.array(LSE), rtol=0, atol=1e-12)

    d, r = pick % n_dev, (pick // n_dev) % n_dev
    src = (d - r) % n_dev
    op, lp = oracle.ring_partial(*dev, n_dev, layout, d, r)
    live = [[explicit_position(n_dev, L, layout, src, kk) <= explicit_position(n_dev, L, layout, d, j)
             for kk in range(L)] for j in range(L)]
    Op, Lp = bf_masked(dev[0][0, d * L:(d + 1) * L, 0].tolist(), dev[1][0, src * L:(src + 1) * L, 0].tolist(),
                       dev[2][0, src * L:(src + 1) * L, 0].tolist(), live, scale)
    np.testing.assert_allclose(op[0, :, 0], np.array(Op), rtol=0, atol=1e-12)
    assert np.array_equal(np.isneginf(lp[0, :, 0]), np.isneginf(np.array(Lp)))
    fin = np.isfinite(np.array(Lp))
    np.testing.assert_allclose(lp[0, fin, 0], np.array(Lp)[fin], rtol=0, atol=1e-12)
