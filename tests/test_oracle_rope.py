"""Pins for the oracle's rotary embedding and its stripe composition.

The oracle's ``rope`` is checked against things other than itself:

* brute force: pure-Python loops with ``math.cos``/``math.sin`` and
  ``math.pow`` for the frequencies, on small inputs;
* special cases: position 0 is the identity; D = 2 is a plain 2-D rotation by
  the position in radians;
* invariants: every (c, c + D/2) pair keeps its length; rotations compose
  (rotating by a then by b is rotating by a + b); the dot product of two
  rotated vectors depends only on the difference of their positions, so
  causal attention over rotated Q and K is unchanged when every position is
  shifted by the same amount;
* the striped composition rotates each token by its original position:
  slot d*L + j of the device layout equals the token at j*N + d rotated by
  j*N + d, written out with explicit indices;
* mutation tests: a planted mistake in a copy of ``oracle/rotary.py`` fails
  one of the pins above.
"""

import math
import pathlib
import types

import numpy as np
import pytest

import oracle
from oracle import rotary as orope
from oracle import stripes as ost

ROPE_FILE = pathlib.Path(orope.__file__)


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def bf_rope_row(vec, p, base):
    """Pure-Python rotation of one head vector at position p."""
    D = len(vec)
    h = D // 2
    out = [0.0] * D
    for c in range(h):
        a = p * math.pow(base, -2.0 * c / D)
        out[c] = vec[c] * math.cos(a) - vec[c + h] * math.sin(a)
        out[c + h] = vec[c] * math.sin(a) + vec[c + h] * math.cos(a)
    return out


# ------------------------------------------------------------------- pins --

def _pin_brute_force(mod):
    B, S, H, D = 2, 7, 2, 8
    x = rand((B, S, H, D), 1)
    pos = np.array([[0, 3, 5, 11, 100, 4096, 786431], [7, 7, 2, 0, 1, 65536, 31]])
    for base in (10000.0, 500.0):
        for p_arg in (None, pos):
            y = mod.rope(x, p_arg, base)
            for b in range(B):
                for s in range(S):
                    p = s if p_arg is None else int(pos[b, s])
                    for h in range(H):
                        want = bf_rope_row(x[b, s, h].tolist(), p, base)
                        np.testing.assert_allclose(y[b, s, h], want, rtol=0, atol=1e-9)


def _pin_special_cases(mod):
    x = rand((1, 4, 3, 6), 2)
    y = mod.rope(x, np.zeros((1, 4), np.int64))
    assert np.array_equal(y, x)                     # position 0: identity, exactly
    x2 = rand((1, 5, 1, 2), 3)                      # D = 2: rotation by p radians
    y2 = mod.rope(x2)
    for p in range(5):
        c, s = math.cos(p), math.sin(p)
        np.testing.assert_allclose(y2[0, p, 0], [x2[0, p, 0, 0] * c - x2[0, p, 0, 1] * s,
                                                 x2[0, p, 0, 0] * s + x2[0, p, 0, 1] * c], atol=1e-12)


def _pin_striped_positions(mod):
    B, S, H, D = 2, 24, 2, 8
    x = rand((B, S, H, D), 4)
    pos = np.random.default_rng(5).integers(0, 10 ** 6, size=(B, S))
    for layout in (ost.CONTIGUOUS, ost.STRIPED):
        for N in (1, 3, 4, 8):
            L = S // N
            for p_arg in (None, pos):
                y = mod.rope_device_layout(x, N, layout, p_arg)
                for d in range(N):
                    for j in range(L):
                        t = j * N + d if layout == ost.STRIPED else d * L + j
                        for b in range(B):
                            p = t if p_arg is None else int(pos[b, t])
                            for h in range(H):
                                want = bf_rope_row(x[b, t, h].tolist(), p, 10000.0)
                                np.testing.assert_allclose(y[b, d * L + j, h], want, rtol=0, atol=1e-9)


PINS = (_pin_brute_force, _pin_special_cases, _pin_striped_positions)


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_rope_pins(pin):
    pin(orope)


def test_rope_pair_norms_are_kept():
    x = rand((2, 9, 3, 16), 6)
    y = oracle.rope(x, np.arange(18).reshape(2, 9) * 977)
    n_in = x[..., :8] ** 2 + x[..., 8:] ** 2
    n_out = y[..., :8] ** 2 + y[..., 8:] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-12)


def test_rope_composes():
    x = rand((1, 6, 2, 8), 7)
    a = np.array([[0, 5, 17, 300, 9000, 123456]])
    b = np.array([[3, 1, 40, 2, 11, 654321]])
    np.testing.assert_allclose(oracle.rope(oracle.rope(x, a), b), oracle.rope(x, a + b), atol=1e-9)


def test_rope_dot_product_depends_on_position_difference():
    D = 16
    q, k = rand((1, 1, 1, D), 8), rand((1, 1, 1, D), 9)
    for m, n in ((5, 2), (1000, 997), (786431, 786428), (40, 40), (3, 10)):
        lhs = float(np.sum(oracle.rope(q, [[m]]) * oracle.rope(k, [[n]])))
        rhs = float(np.sum(oracle.rope(q, [[m - n]]) * k))
        assert abs(lhs - rhs) < 1e-9, (m, n, lhs, rhs)


def test_attention_over_rotated_inputs_is_shift_invariant():
    """Scores of rotated Q, K depend on position differences only, so causal
    attention is unchanged when every position moves by the same amount."""
    B, S, H, D = 1, 40, 2, 8
    q, k, v = rand((B, S, H, D), 10), rand((B, S, H, D), 11), rand((B, S, H, D), 12)
    pos = np.arange(S)[None, :]
    o1, l1 = oracle.dense_causal_attention(oracle.rope(q, pos), oracle.rope(k, pos), v)
    o2, l2 = oracle.dense_causal_attention(oracle.rope(q, pos + 12345), oracle.rope(k, pos + 12345), v)
    np.testing.assert_allclose(o1, o2, atol=1e-9)
    np.testing.assert_allclose(l1, l2, atol=1e-9)


def test_striped_attention_of_rotated_inputs_is_exact():
    """Rotate at original positions and stripe; the ring over the device
    layout, un-striped, equals dense attention of the rotated inputs."""
    B, S, H, D, N = 1, 48, 2, 8, 4
    q, k, v = rand((B, S, H, D), 13), rand((B, S, H, D), 14), rand((B, S, H, D), 15)
    o_ref, l_ref = oracle.dense_causal_attention(oracle.rope(q), oracle.rope(k), v)
    for layout in (ost.CONTIGUOUS, ost.STRIPED):
        qd, kd = oracle.rope_device_layout(q, N, layout), oracle.rope_device_layout(k, N, layout)
        vd = oracle.to_device_layout(v, N, layout)
        o, l = oracle.ring_attention(qd, kd, vd, N, layout)
        np.testing.assert_allclose(oracle.from_device_layout(o, N, layout), o_ref, atol=1e-9)
        np.testing.assert_allclose(oracle.from_device_layout(l, N, layout), l_ref, atol=1e-9)


# ---------------------------------------------------------- mutation tests --

def _mutant(old, new):
    src = ROPE_FILE.read_text()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_rope_mutant")
    mod.__dict__["__package__"] = "oracle"
    mod.__dict__["__name__"] = "oracle.rope_mutant"
    exec(compile(src.replace(old, new), "<mutant rotary.py>", "exec"), mod.__dict__)
    return mod


MUTATIONS = [
    # sign of the sine term
    ("np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)",
     "np.concatenate([x1 * cos + x2 * sin, x1 * sin + x2 * cos], axis=-1)", _pin_brute_force),
    # interleaved pairs (2c, 2c+1) instead of (c, c + D/2)
    ("x1, x2 = X[..., : D // 2], X[..., D // 2:]", "x1, x2 = X[..., 0::2], X[..., 1::2]", _pin_brute_force),
    # frequency exponent off by a factor of two
    ("return np.power(float(base), -2.0 * c / D)", "return np.power(float(base), -c / D)", _pin_brute_force),
    # striped rows rotated by their slot index instead of their original position
    ("return rope(X[:, perm], gathered_pos, base)", "return rope(X[:, perm], None, base)", _pin_striped_positions),
]


@pytest.mark.parametrize("case", range(len(MUTATIONS)))
def test_planted_rope_mistake_is_caught(case):
    old, new, pin = MUTATIONS[case]
    mod = _mutant(old, new)
    pin(orope)
    with pytest.raises(AssertionError):
        pin(mod)
