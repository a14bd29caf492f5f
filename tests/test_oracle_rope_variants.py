"""Pins of the oracle's RoPE variants: partial rotary, PI, NTK, YaRN (CPU only).

[P7] "Part 7: The Modern Decoder Block" modules L7.3 and L7.4 name these
variants without formulas; the oracle follows their published definitions.
Each check below is fixed by something other than the oracle's own code: a
reduction to plain RoPE, complex multiplication, a closed form, or a property
the method is defined by.
"""

import math

import numpy as np
import pytest
import torch

from oracle import (bf16_to_f64, llama3_scaled_frequencies, rope_append, rope_attention_factor, rope_frequencies,
                    rope_rotate, yarn_frequencies)


def bf(rng, shape):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


def plain_rotation(x, pos, theta, r, layout):
    """RoPE of the first r dims written with numpy complex numbers (independent route)."""
    i = np.arange(r // 2)
    z_ang = np.exp(1j * np.asarray(pos, np.float64)[..., None] * theta ** (-2.0 * i / r))
    y = np.array(x, dtype=np.float64, copy=True)
    if layout == "interleaved":
        z = (x[..., 0:r:2] + 1j * x[..., 1:r:2]) * z_ang
        y[..., 0:r:2], y[..., 1:r:2] = z.real, z.imag
    else:
        z = (x[..., : r // 2] + 1j * x[..., r // 2: r]) * z_ang
        y[..., : r // 2], y[..., r // 2: r] = z.real, z.imag
    return y


YARN = dict(type="yarn", factor=16.0, beta_slow=1.0, beta_fast=32.0, original_max_pos=4096.0)

# ---------------------------------------------------------------- partial rotary


@pytest.mark.parametrize("layout", ["interleaved", "half"])
@pytest.mark.parametrize("d,r", [(128, 64), (64, 16), (128, 96)])
def test_partial_rotary_is_full_rope_of_the_leading_dims(layout, d, r):
    """Rotating r of d dims equals full RoPE of an r-dim head, then the tail unchanged."""
    rng = np.random.default_rng(d + r)
    B, n_q, n_kv, T, S, past = 2, 4, 2, 3, 40, [5, 30]
    q, kn, vn = bf(rng, (B, n_q, T, d)), bf(rng, (B, n_kv, T, d)), bf(rng, (B, n_kv, T, d))
    kc, vc = bf(rng, (B, n_kv, S, d)), bf(rng, (B, n_kv, S, d))
    qr, kr, vr = rope_append(q, kn, vn, kc, vc, past, 1.0e4, layout, rotary_dim=r)
    q2, k2, _ = rope_append(q[..., :r].copy(), kn[..., :r].copy(), vn[..., :r].copy(), kc[..., :r].copy(),
                            vc[..., :r].copy(), past, 1.0e4, layout)
    assert np.array_equal(qr[..., :r], q2) and np.array_equal(kr[..., :r], k2)
    assert np.array_equal(qr[..., r:], q[..., r:])
    for b in range(B):
        rows = slice(past[b], past[b] + T)
        assert np.array_equal(kr[b][:, rows, r:], kn[b][..., r:])
        assert np.array_equal(vr[b][:, rows], vn[b])
    # and the rotated part is complex multiplication at theta^(-2i/r)
    x = bf16_to_f64(q[0])
    got = rope_rotate(x, past[0] + np.arange(T)[None, :], 1.0e4, layout, None, r)
    assert np.allclose(got, plain_rotation(x, past[0] + np.arange(T)[None, :], 1.0e4, r, layout), rtol=0,
                       atol=1e-12)


def test_full_rotary_dim_is_plain_rope():
    rng = np.random.default_rng(2)
    q, kn, vn = bf(rng, (1, 2, 2, 64)), bf(rng, (1, 1, 2, 64)), bf(rng, (1, 1, 2, 64))
    kc, vc = bf(rng, (1, 1, 9, 64)), bf(rng, (1, 1, 9, 64))
    a = rope_append(q, kn, vn, kc, vc, [4], 1.0e4)
    b = rope_append(q, kn, vn, kc, vc, [4], 1.0e4, rotary_dim=64)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_partial_rotary_rejects_bad_sizes():
    with pytest.raises(ValueError):
        rope_frequencies(1.0e4, 64, rotary_dim=15)
    with pytest.raises(ValueError):
        rope_frequencies(1.0e4, 64, rotary_dim=66)


# ---------------------------------------------------------------- position interpolation


def test_linear_scaling_is_position_interpolation():
    """PI at position p equals plain RoPE at the fractional position p / s."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 128))
    pos = rng.integers(0, 32768, size=5).astype(np.float64)
    for s in (2.0, 4.0, 8.0):
        got = rope_rotate(x, pos, 5.0e5, "interleaved", dict(type="linear", factor=s))
        assert np.allclose(got, plain_rotation(x, pos / s, 5.0e5, 128, "interleaved"), rtol=0, atol=1e-9)
    same = rope_rotate(x, pos, 5.0e5, "half", dict(type="linear", factor=1.0))
    assert np.array_equal(same, rope_rotate(x, pos, 5.0e5, "half"))


# ---------------------------------------------------------------- NTK-aware


@pytest.mark.parametrize("d,r", [(128, 128), (64, 64), (128, 32)])
def test_ntk_base_change(d, r):
    theta, s = 5.0e5, 8.0
    plain = rope_frequencies(theta, d, rotary_dim=r)
    ntk = rope_frequencies(theta, d, dict(type="ntk", factor=s), rotary_dim=r)
    assert ntk[0] == 1.0  # the fastest pair keeps its frequency
    assert math.isclose(ntk[-1], plain[-1] / s, rel_tol=1e-13)  # the slowest is interpolated by s
    # still a geometric progression, now with base theta * s^(r / (r - 2))
    assert np.allclose(np.diff(np.log(ntk)), -2.0 * math.log(theta * s ** (r / (r - 2))) / r, rtol=0, atol=1e-12)
    assert np.all(ntk <= plain) and np.all(ntk >= plain / s * (1 - 1e-14))
    assert np.array_equal(rope_frequencies(theta, d, dict(type="ntk", factor=1.0), rotary_dim=r), plain)


# ---------------------------------------------------------------- YaRN


def test_yarn_limits_and_continuity():
    theta, d = 1.0e4, 128
    plain = rope_frequencies(theta, d)
    f = rope_frequencies(theta, d, YARN)
    turns = YARN["original_max_pos"] * plain / (2 * math.pi)
    fast, slow = turns > 32.0, turns < 1.0
    assert fast.any() and slow.any() and (~fast & ~slow).any()
    assert np.array_equal(f[fast], plain[fast])
    assert np.allclose(f[slow], plain[slow] / 16.0, rtol=1e-15, atol=0)
    # continuous at both ends of the ramp
    for edge in (1.0, 32.0):
        fe = 2 * math.pi * edge / YARN["original_max_pos"] * np.array([1 - 1e-9, 1.0, 1 + 1e-9])
        ratio = yarn_frequencies(fe, 16.0, 1.0, 32.0, YARN["original_max_pos"]) / fe
        assert np.ptp(ratio) < 1e-6
    # factor 1 changes nothing and leaves the logits alone
    one = dict(YARN, factor=1.0)
    assert np.allclose(rope_frequencies(theta, d, one), plain, rtol=1e-15, atol=0)
    assert rope_attention_factor(one) == 1.0


def test_yarn_ramp_agrees_with_the_llama3_rule():
    """Same cutoffs in turns-per-original-context: the two separately written rules coincide."""
    plain = rope_frequencies(5.0e5, 128)
    y = yarn_frequencies(plain, 8.0, 1.0, 4.0, 8192.0)
    l3 = llama3_scaled_frequencies(plain, 8.0, 1.0, 4.0, 8192.0)
    assert np.allclose(y, l3, rtol=1e-13, atol=0)


def test_yarn_attention_factor():
    # closed form of the YaRN paper: sqrt(1/t) = 0.1 ln s + 1
    assert math.isclose(rope_attention_factor(YARN), 0.1 * math.log(16.0) + 1.0, rel_tol=1e-15)
    assert rope_attention_factor(dict(YARN, attn_factor=1.5)) == 1.5
    for other in (None, dict(type="linear", factor=4.0), dict(type="ntk", factor=4.0)):
        assert rope_attention_factor(other) == 1.0
    # at equal positions the rotation cancels, so q.k scales by exactly m^2
    rng = np.random.default_rng(9)
    q, k = rng.standard_normal((6, 128)), rng.standard_normal((6, 128))
    pos = rng.integers(0, 60000, size=6)
    dot = np.sum(rope_rotate(q, pos, 1.0e4, "interleaved", YARN) * rope_rotate(k, pos, 1.0e4, "interleaved", YARN), -1)
    m = 0.1 * math.log(16.0) + 1.0
    assert np.allclose(dot, m * m * np.sum(q * k, -1), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("scaling,r", [(dict(type="linear", factor=4.0), None), (dict(type="ntk", factor=8.0), 64),
                                       (YARN, None), (YARN, 32)])
@pytest.mark.parametrize("layout", ["interleaved", "half"])
def test_relative_offset_invariance_of_variants(scaling, r, layout):
    """[P7] key ideas: a rotated q.k depends only on the offset, for every variant (tail dims included)."""
    rng = np.random.default_rng(12)
    worst = 0.0
    for _ in range(100):
        q, k = rng.standard_normal(128), rng.standard_normal(128)
        m, n = rng.integers(0, 30000, size=2)
        s = int(rng.integers(-min(m, n), 30000 - max(m, n)))
        a = rope_rotate(q, m, 5.0e5, layout, scaling, r) @ rope_rotate(k, n, 5.0e5, layout, scaling, r)
        b = rope_rotate(q, m + s, 5.0e5, layout, scaling, r) @ rope_rotate(k, n + s, 5.0e5, layout, scaling, r)
        worst = max(worst, abs(a - b) / (np.linalg.norm(q) * np.linalg.norm(k)))
    assert worst < 1e-11
