"""Rotary position embedding of the model inputs, and its stripe permutation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The striped layout is applied once, to the model's inputs before the first
layer (Striped Attention summary page, research.elamur.ai, "Summary" ¶2 and
"Key points: Striped layout"): each device then holds every N-th token of
the sequence. The pages say nothing about positional encodings. A
position-dependent encoding inside the model must still see every token's
original position, so the position ids travel with the tokens. Reading used
here: rotary embedding in the "rotate half" form. For a head vector x of
dimension D (even) at position p, each pair (c, c + D/2), c < D/2, is rotated
by the angle a_c = p * base^(-2c/D):

    y_c       = x_c cos(a_c) - x_{c+D/2} sin(a_c)
    y_{c+D/2} = x_c sin(a_c) + x_{c+D/2} cos(a_c)

Positions default to the token's index in the original sequence; explicit
position ids [B, S] (in original order) may be given instead. The device
layout of a rotated tensor holds, in slot d*L + j, the token at original
position j*N + d rotated by that token's own position.

fp64 numpy on the inputs as stored.
"""

import numpy as np

from .attention import _f64
from .stripes import stripe_index


def inv_freq(D, base=10000.0):
    """base^(-2c/D) for c = 0 .. D/2 - 1, in fp64."""
    c = np.arange(D // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * c / D)


def _positions(B, S, pos):
    if pos is None:
        return np.broadcast_to(np.arange(S, dtype=np.float64), (B, S))
    p = pos.detach().cpu().numpy() if hasattr(pos, "detach") else np.asarray(pos)
    return p.astype(np.float64)


def rope(x, pos=None, base=10000.0):
    """Rotary embedding of x [B, S, H, D] at positions pos ([B, S] or None for
    0 .. S-1); returns fp64 [B, S, H, D]."""
    X = _f64(x)
    B, S, H, D = X.shape
    if D % 2:
        raise ValueError("head dim must be even")
    a = _positions(B, S, pos)[:, :, None, None] * inv_freq(D, base)[None, None, None, :]
    cos, sin = np.cos(a), np.sin(a)
    x1, x2 = X[..., : D // 2], X[..., D // 2:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)


def rope_device_layout(x, n_dev, layout, pos=None, base=10000.0):
    """Rotary embedding and stripe gather in one: the device-layout tensor
    whose slot t holds original token perm[t], rotated by that token's
    position (its original index, or pos[b, perm[t]])."""
    X = _f64(x)
    B, S = X.shape[:2]
    perm = stripe_index(S, n_dev, layout)
    gathered_pos = _positions(B, S, pos)[:, perm]
    return rope(X[:, perm], gathered_pos, base)
