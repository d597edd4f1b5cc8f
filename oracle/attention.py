"""Exact causal attention, its ring decomposition and its gradient, in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the method computes (Striped Attention summary page, research.elamur.ai,
"Summary" ¶2 and "Key points: Striped layout"; abstract at
pith.science/paper/2311.09431): ring attention is exact attention, and the
striped layout leaves the result unchanged because attention is
permutation-equivariant. The result is therefore plain causal softmax
attention on the original sequence. For every batch b, head h and original
position i:

    s_ik = scale * sum_c Q_ic K_kc            for k <= i (diagonal included)
    lse_i = log sum_{k <= i} exp(s_ik)        (natural log)
    O_i   = sum_{k <= i} exp(s_ik - lse_i) V_k

Readings where the pages are silent: scale defaults to 1/sqrt(D); the
diagonal is included (so O_0 = V_0); lse is a natural logarithm; a row with
no live key in a partial result has O = 0 and lse = -inf.

Tensors are [B, S, H, D] (lse: [B, S, H]); inputs of any float dtype are
widened to float64 before any arithmetic.
"""

import numpy as np

from .stripes import positions, round_source

_ROW_BLOCK = 256


def _f64(x):
    """Widen to a float64 numpy array (accepts numpy arrays or CPU torch tensors)."""
    if hasattr(x, "detach"):  # a torch tensor: widen in torch first (numpy has no bf16)
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _scale(D, scale):
    return 1.0 / np.sqrt(D) if scale is None else float(scale)


def dense_causal_attention(q, k, v, scale=None):
    """Dense causal softmax attention on the original order.

    Computed per (b, h) in blocks of 256 query rows: scores against every key
    up to the block's last row, mask k > i, max-shifted softmax, times V.
    Returns (O, lse) in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, S, H, D = q.shape
    sc = _scale(D, scale)
    o = np.zeros((B, S, H, D))
    lse = np.zeros((B, S, H))
    for b in range(B):
        for h in range(H):
            Q, K, V = q[b, :, h], k[b, :, h], v[b, :, h]
            for i0 in range(0, S, _ROW_BLOCK):
                i1 = min(S, i0 + _ROW_BLOCK)
                s = sc * (Q[i0:i1] @ K[:i1].T)
                rows = np.arange(i0, i1)[:, None]
                cols = np.arange(i1)[None, :]
                s = np.where(cols <= rows, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                den = e.sum(axis=1, keepdims=True)
                o[b, i0:i1, h] = (e @ V[:i1]) / den
                lse[b, i0:i1, h] = (m + np.log(den))[:, 0]
    return o, lse


def attention_rows(q, k, v, rows, scale=None):
    """Causal attention for selected original positions only (for shapes where
    the dense oracle is too slow). ``rows`` is a 1-D integer array.

    Returns (O[B, len(rows), H, D], lse[B, len(rows), H]) in float64. Per
    (batch, head): the scores of all selected rows against keys 0 .. max(rows)
    in one product, keys after a row's own position set to -inf, then the
    row softmax and its product with V -- the definition above, row by row.
    """
    rows = np.asarray(rows, dtype=np.int64)
    B, S, H, D = q.shape
    sc = _scale(D, scale)
    o = np.zeros((B, len(rows), H, D))
    lse = np.zeros((B, len(rows), H))
    if len(rows) == 0:
        return o, lse
    i1 = int(rows.max()) + 1
    keys = np.arange(i1)
    for b in range(B):
        for h in range(H):
            Q = _f64(q[b, rows, h])         # [R, D]
            K = _f64(k[b, :i1, h])          # [i1, D]
            V = _f64(v[b, :i1, h])
            s = sc * (Q @ K.T)
            s = np.where(keys[None, :] <= rows[:, None], s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            den = e.sum(axis=1, keepdims=True)
            o[b, :, h] = (e @ V) / den
            lse[b, :, h] = (m + np.log(den))[:, 0]
    return o, lse


def ring_partial(q_dev, k_dev, v_dev, n_dev, layout, d, r, scale=None):
    """One ring round for one device, on device-layout tensors.

    Device d's queries (slots d*L .. d*L+L-1) attend to the K/V block of
    device s = (d - r) mod N, with liveness decided by original positions
    (key position <= query position). Rows with no live key get O = 0 and
    lse = -inf. Returns (O[B, L, H, D], lse[B, L, H]) in float64, each row
    normalised over this round's keys only.
    """
    q_dev, k_dev, v_dev = _f64(q_dev), _f64(k_dev), _f64(v_dev)
    B, S, H, D = q_dev.shape
    L = S // n_dev
    sc = _scale(D, scale)
    s_dev = round_source(d, r, n_dev)
    pos = positions(S, n_dev, layout)
    qpos = pos[d * L:(d + 1) * L]
    kpos = pos[s_dev * L:(s_dev + 1) * L]
    live = kpos[None, :] <= qpos[:, None]          # [L, L]
    has_key = live.any(axis=1)
    o = np.zeros((B, L, H, D))
    lse = np.full((B, L, H), -np.inf)
    for b in range(B):
        for h in range(H):
            Q = q_dev[b, d * L:(d + 1) * L, h]
            K = k_dev[b, s_dev * L:(s_dev + 1) * L, h]
            V = v_dev[b, s_dev * L:(s_dev + 1) * L, h]
            s = np.where(live, sc * (Q @ K.T), -np.inf)
            m = np.where(has_key, s.max(axis=1), 0.0)[:, None]
            e = np.where(live, np.exp(s - m), 0.0)
            den = e.sum(axis=1, keepdims=True)
            safe = np.where(den > 0, den, 1.0)
            o[b, :, h] = np.where(has_key[:, None], (e @ V) / safe, 0.0)
            lse[b, :, h] = np.where(has_key, (m + np.log(safe))[:, 0], -np.inf)
    return o, lse


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Combine two partial results over disjoint key sets.

    With M = max(lse_a, lse_b): lse = M + log(exp(lse_a - M) + exp(lse_b - M))
    and O = exp(lse_a - lse) O_a + exp(lse_b - lse) O_b. A side with
    lse = -inf contributes nothing; if both are -inf the result is O = 0,
    lse = -inf. Returns new arrays (float64).
    """
    o_a, lse_a, o_b, lse_b = _f64(o_a), _f64(lse_a), _f64(o_b), _f64(lse_b)
    M = np.maximum(lse_a, lse_b)
    empty = np.isneginf(M)
    Ms = np.where(empty, 0.0, M)
    wa = np.exp(lse_a - Ms)
    wb = np.exp(lse_b - Ms)
    tot = wa + wb
    lse = np.where(empty, -np.inf, Ms + np.log(np.where(empty, 1.0, tot)))
    tot = np.where(empty, 1.0, tot)
    o = (wa / tot)[..., None] * o_a + (wb / tot)[..., None] * o_b
    o = np.where(empty[..., None], 0.0, o)
    return o, lse


def ring_attention(q_dev, k_dev, v_dev, n_dev, layout, scale=None):
    """All N rounds for all N devices, merged round by round (r = 0 .. N-1).

    Inputs and outputs are in device layout. Returns (O, lse) float64.
    """
    B, S, H, D = q_dev.shape
    L = S // n_dev
    o = np.zeros((B, S, H, D))
    lse = np.full((B, S, H), -np.inf)
    for d in range(n_dev):
        acc_o = np.zeros((B, L, H, D))
        acc_l = np.full((B, L, H), -np.inf)
        for r in range(n_dev):
            po, pl = ring_partial(q_dev, k_dev, v_dev, n_dev, layout, d, r, scale)
            acc_o, acc_l = lse_merge(acc_o, acc_l, po, pl)
        o[:, d * L:(d + 1) * L] = acc_o
        lse[:, d * L:(d + 1) * L] = acc_l
    return o, lse


def dense_causal_backward(q, k, v, o, lse, do, scale=None):
    """Gradient of sum(O * dO) through dense causal attention (original order).

    With P_ik = exp(s_ik - lse_i) on live pairs and Delta_i = sum_c dO_ic O_ic:
        dV = P^T dO,  dP = dO V^T,  dS = P * (dP - Delta),
        dQ = scale * dS K,  dK = scale * dS^T Q.
    ``o`` and ``lse`` are the forward's results (the oracle's own, or any
    caller-supplied values of matching shape). Returns (dQ, dK, dV) float64.
    """
    q, k, v, o, lse, do = (_f64(t) for t in (q, k, v, o, lse, do))
    B, S, H, D = q.shape
    sc = _scale(D, scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            Q, K, V = q[b, :, h], k[b, :, h], v[b, :, h]
            dO, O = do[b, :, h], o[b, :, h]
            delta = (dO * O).sum(axis=1)
            for i0 in range(0, S, _ROW_BLOCK):
                i1 = min(S, i0 + _ROW_BLOCK)
                rows = np.arange(i0, i1)[:, None]
                cols = np.arange(i1)[None, :]
                live = cols <= rows
                s = sc * (Q[i0:i1] @ K[:i1].T)
                p = np.where(live, np.exp(np.where(live, s, 0.0) - lse[b, i0:i1, h][:, None]), 0.0)
                dv[b, :i1, h] += p.T @ dO[i0:i1]
                dp = dO[i0:i1] @ V[:i1].T
                ds = p * (dp - delta[i0:i1, None])
                dq[b, i0:i1, h] = sc * (ds @ K[:i1])
                dk[b, :i1, h] += sc * (ds.T @ Q[i0:i1])
    return dq, dk, dv


def backward_key_rows(q, k, v, do, key_rows, heads, scale=None):
    """dK and dV for selected key positions and heads (for shapes where the
    dense backward is too slow).

    Key k receives gradient from every query i >= k, so this recomputes the
    forward rows i >= min(key_rows) for the chosen heads (their lse and O
    included) and accumulates dK_k, dV_k for the selected keys.
    Returns (dK[B, len(key_rows), len(heads), D], dV[...]) float64.
    """
    key_rows = np.asarray(key_rows, dtype=np.int64)
    B, S, H, D = q.shape
    sc = _scale(D, scale)
    k0 = int(key_rows.min())
    dk = np.zeros((B, len(key_rows), len(heads), D))
    dv = np.zeros_like(dk)
    for b in range(B):
        for hn, h in enumerate(heads):
            K = _f64(k[b, :, h])
            V = _f64(v[b, :, h])
            Ksel, Vsel = K[key_rows], V[key_rows]
            for i0 in range(k0, S, _ROW_BLOCK):
                i1 = min(S, i0 + _ROW_BLOCK)
                Q = _f64(q[b, i0:i1, h])
                dO = _f64(do[b, i0:i1, h])
                rows = np.arange(i0, i1)[:, None]
                s = sc * (Q @ K[:i1].T)
                s = np.where(np.arange(i1)[None, :] <= rows, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                den = e.sum(axis=1, keepdims=True)
                O = (e @ V[:i1]) / den
                lse = m + np.log(den)
                delta = (dO * O).sum(axis=1, keepdims=True)
                live = key_rows[None, :] <= rows           # [rows, nsel]
                p = np.where(live, np.exp(sc * (Q @ Ksel.T) - lse), 0.0)
                dp = dO @ Vsel.T
                ds = p * (dp - delta)
                dv[b, :, hn] += p.T @ dO
                dk[b, :, hn] += sc * (ds.T @ Q)
    return dk, dv


def backward_query_rows(q, k, v, do, rows, heads, scale=None):
    """dQ for selected query positions and heads (for shapes where the dense
    backward is too slow).

    Row i needs its own forward quantities over keys k <= i: lse_i, O_i and
    Delta_i = dO_i . O_i; then dS_ik = P_ik (dO_i . V_k - Delta_i) and
    dQ_i = scale * sum_k dS_ik K_k. Each row costs O(i * D).
    Returns dQ[B, len(rows), len(heads), D] float64.
    """
    rows = np.asarray(rows, dtype=np.int64)
    B, S, H, D = q.shape
    sc = _scale(D, scale)
    dq = np.zeros((B, len(rows), len(heads), D))
    for b in range(B):
        for hn, h in enumerate(heads):
            for n, i in enumerate(rows):
                i = int(i)
                Qi = _f64(q[b, i, h])
                dOi = _f64(do[b, i, h])
                K = _f64(k[b, :i + 1, h])
                V = _f64(v[b, :i + 1, h])
                s = sc * (K @ Qi)
                m = s.max()
                e = np.exp(s - m)
                den = e.sum()
                p = e / den
                Oi = p @ V
                delta = float(dOi @ Oi)
                ds = p * (V @ dOi - delta)
                dq[b, n, hn] = sc * (ds @ K)
    return dq
