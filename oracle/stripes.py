"""Sequence layouts over N ring devices, written out from their definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Layouts (Striped Attention summary page, research.elamur.ai, "Summary" ¶1
and ¶2, "Key points: Striped layout"; notes page, phantomic12.github.io ¶2):

* contiguous -- ring attention's original split: device ``d`` holds one
  contiguous chunk of ``L = S / N`` tokens, positions ``d*L .. d*L + L - 1``.
* striped -- device ``d`` holds every N-th token. Reading taken for the
  offset and the storage order the pages leave open: device ``d`` holds
  positions ``d, d + N, d + 2N, ...``, i.e. its ``j``-th token is position
  ``j*N + d``.

"Device layout" stores device ``d``'s ``j``-th token in slot ``d*L + j`` of
one buffer (the N virtual devices are consecutive slices). For the
contiguous layout that is the original order.

Ring rounds (summary page, "Summary" ¶1: K/V blocks circulate around the
ring): in round ``r`` device ``d`` holds the K/V block that started on device
``(d - r) mod N``. The exact result does not depend on the direction; only
rounding order does.

A key slot is live for a query slot when the key's original position is not
after the query's (causal attention, diagonal included).
"""

import numpy as np

CONTIGUOUS = 0
STRIPED = 1


def _check(seq, n_dev, layout):
    if layout not in (CONTIGUOUS, STRIPED):
        raise ValueError(f"unknown layout {layout}")
    if n_dev < 1 or seq < 1 or seq % n_dev:
        raise ValueError(f"seq={seq} must be a positive multiple of n_dev={n_dev}")


def positions(seq, n_dev, layout):
    """pos[slot] = original sequence position held in device-layout ``slot``.

    Slot ``t`` is token ``j = t mod L`` of device ``d = t // L``.
    """
    _check(seq, n_dev, layout)
    L = seq // n_dev
    pos = np.empty(seq, dtype=np.int64)
    for d in range(n_dev):
        for j in range(L):
            if layout == STRIPED:
                pos[d * L + j] = j * n_dev + d
            else:
                pos[d * L + j] = d * L + j
    return pos


def stripe_index(seq, n_dev, layout):
    """perm[slot] = original position (alias of :func:`positions`).

    Gathering ``x[perm]`` along the sequence axis moves original order into
    device layout.
    """
    return positions(seq, n_dev, layout)


def unstripe_index(seq, n_dev, layout):
    """inv[position] = slot holding that position: the inverse permutation,
    found by inverting the table (no closed form used)."""
    pos = positions(seq, n_dev, layout)
    inv = np.full(seq, -1, dtype=np.int64)
    for slot, p in enumerate(pos):
        inv[p] = slot
    return inv


def to_device_layout(x, n_dev, layout, axis=1):
    """Reorder ``x`` (sequence on ``axis``) from original order into device layout."""
    x = np.asarray(x)
    return np.take(x, stripe_index(x.shape[axis], n_dev, layout), axis=axis)


def from_device_layout(y, n_dev, layout, axis=1):
    """Inverse of :func:`to_device_layout`."""
    y = np.asarray(y)
    return np.take(y, unstripe_index(y.shape[axis], n_dev, layout), axis=axis)


def round_source(d, r, n_dev):
    """Device whose K/V block device ``d`` holds in ring round ``r``."""
    return (d - r) % n_dev


def live_mask(seq, n_dev, layout, d, r):
    """Boolean [L, L]: mask[j, k] is True when key k of the source device is
    live for query j of device d in round r (key position <= query position)."""
    pos = positions(seq, n_dev, layout)
    L = seq // n_dev
    s = round_source(d, r, n_dev)
    qpos = pos[d * L:(d + 1) * L]
    kpos = pos[s * L:(s + 1) * L]
    return kpos[None, :] <= qpos[:, None]


def live_pairs(seq, n_dev, layout):
    """pairs[r, d] = number of live (query, key) pairs device d computes in round r."""
    out = np.zeros((n_dev, n_dev), dtype=np.int64)
    for r in range(n_dev):
        for d in range(n_dev):
            out[r, d] = int(live_mask(seq, n_dev, layout, d, r).sum())
    return out


def live_tiles(seq, n_dev, layout, tile_q, tile_k):
    """Brute-force tile census from the element mask (no closed form).

    Queries of each device are cut into tiles of ``tile_q`` rows and keys of
    the source device into tiles of ``tile_k`` (the last tile of each may be
    ragged). A tile is FULL when every pair in it is live, EMPTY when none
    is, PARTIAL otherwise; live = FULL + PARTIAL.

    Returns ``(live, full, partial)``, each int64 [N, N] indexed [r, d].
    """
    L = seq // n_dev
    nq = -(-L // tile_q)
    nk = -(-L // tile_k)
    live = np.zeros((n_dev, n_dev), dtype=np.int64)
    full = np.zeros_like(live)
    partial = np.zeros_like(live)
    for r in range(n_dev):
        for d in range(n_dev):
            m = live_mask(seq, n_dev, layout, d, r)
            for a in range(nq):
                rows = m[a * tile_q:(a + 1) * tile_q]
                for b in range(nk):
                    t = rows[:, b * tile_k:(b + 1) * tile_k]
                    n_live = int(t.sum())
                    if n_live == t.size:
                        full[r, d] += 1
                    elif n_live > 0:
                        partial[r, d] += 1
            live[r, d] = full[r, d] + partial[r, d]
    return live, full, partial
