"""Pins of the oracle's bf16 rounding, RoPE frequencies and rotation (CPU only).

Every check here is fixed by something other than the oracle itself: exact
bit patterns, torch's own fp32 -> bf16 cast, complex multiplication, closed
forms, or properties the pages state.
"""

import math

import numpy as np
import pytest
import torch

from oracle import bf16_to_f64, f64_to_bf16, llama3_scaled_frequencies, rope_frequencies, rotate_pairs



# ---------------------------------------------------------------- bf16 rounding

def test_bf16_exact_values():
    cases = {1.0: 0x3F80, -2.0: 0xC000, 0.5: 0x3F00, 0.0: 0x0000, 3.0: 0x4040,
             1.0 + 2 ** -7: 0x3F81, 2.0 ** -126: 0x0080, 2.0 ** -133: 0x0001}
    for x, b in cases.items():
        assert int(f64_to_bf16(np.array([x]))[0]) == b, x
    assert int(f64_to_bf16(np.array([-0.0]))[0]) == 0x8000
    assert int(f64_to_bf16(np.array([np.inf]))[0]) == 0x7F80
    assert int(f64_to_bf16(np.array([np.nan]))[0]) == 0x7FC0


def test_bf16_ties_to_even_and_no_double_rounding():
    # 1 + 2^-8 lies exactly between 1 and 1 + 2^-7: ties go to the even pattern 0x3F80
    assert int(f64_to_bf16(np.array([1.0 + 2 ** -8]))[0]) == 0x3F80
    # 1 + 3*2^-8 lies between 0x3F81 and 0x3F82: tie to even -> 0x3F82
    assert int(f64_to_bf16(np.array([1.0 + 3 * 2 ** -8]))[0]) == 0x3F82
    # just above the tie: fp32 would first round it onto the tie (then to 0x3F80);
    # a single correct rounding from fp64 must give 0x3F81
    x = 1.0 + 2 ** -8 + 2 ** -30
    assert np.float32(x) == np.float32(1.0 + 2 ** -8)
    assert int(f64_to_bf16(np.array([x]))[0]) == 0x3F81
    # overflow and the largest finite bf16
    assert int(f64_to_bf16(np.array([3.3895313892515355e38]))[0]) == 0x7F7F
    assert int(f64_to_bf16(np.array([3.4e38]))[0]) == 0x7F80


def test_bf16_matches_torch_cast_on_fp32_values():
    # for numbers exact in fp32, rounding fp64 -> bf16 and torch's fp32 -> bf16 cast agree
    rng = np.random.default_rng(7)
    x32 = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                          (rng.standard_normal(5000) * 1e-39).astype(np.float32),
                          (rng.standard_normal(5000) * 1e30).astype(np.float32)])
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = f64_to_bf16(x32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_roundtrip_exact():
    allbits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bf16_to_f64(allbits)
    finite = np.isfinite(vals)
    back = f64_to_bf16(vals[finite])
    # every finite pattern maps back to itself (both zeros keep their sign)
    assert np.array_equal(back, allbits[finite])


# ---------------------------------------------------------------- frequencies

@pytest.mark.parametrize("theta,d", [(1.0e4, 64), (5.0e5, 128), (10.0, 8)])
def test_frequencies_geometric(theta, d):
    f = rope_frequencies(theta, d)
    assert f.shape == (d // 2,)
    assert f[0] == 1.0
    # log-frequencies fall on a straight line with slope -2 ln(theta) / d
    slope = np.diff(np.log(f))
    assert np.allclose(slope, -2.0 * math.log(theta) / d, rtol=0, atol=1e-12)
    # one more step of the progression lands on 1/theta
    assert math.isclose(f[-1] * theta ** (-2.0 / d), 1.0 / theta, rel_tol=1e-12)
    assert np.all(np.diff(f) < 0)


def test_frequency_scaling_limits():
    theta, d = 5.0e5, 128
    base = rope_frequencies(theta, d)
    orig = 8192.0
    # factor 1 changes nothing, whatever the cutoffs
    same = llama3_scaled_frequencies(base, 1.0, 1.0, 4.0, orig)
    assert np.allclose(same, base, rtol=1e-15, atol=0)
    sc = llama3_scaled_frequencies(base, 8.0, 1.0, 4.0, orig)
    wl = 2 * math.pi / base
    short = wl < orig / 4.0
    long_ = wl > orig / 1.0
    assert short.any() and long_.any()
    # short wavelengths (high frequencies) are untouched, long ones divided by the factor
    assert np.array_equal(sc[short], base[short])
    assert np.allclose(sc[long_], base[long_] / 8.0, rtol=1e-15, atol=0)
    # in between the scaled frequency lies between freq/factor and freq
    mid = ~short & ~long_
    assert np.all(sc[mid] <= base[mid]) and np.all(sc[mid] >= base[mid] / 8.0)


def test_frequency_scaling_continuous_at_cutoffs():
    orig, low, high, factor = 8192.0, 1.0, 4.0, 8.0
    for cut in (orig / high, orig / low):
        f_at = 2 * math.pi / cut
        eps = 1e-9
        fs = np.array([f_at * (1 + eps), f_at, f_at * (1 - eps)])
        out = llama3_scaled_frequencies(fs, factor, low, high, orig)
        ratios = out / fs
        assert np.ptp(ratios) < 1e-6
    # the ratio scaled/plain never increases as the wavelength grows
    fs = np.geomspace(10.0, 1e-6, 4000)
    r = llama3_scaled_frequencies(fs, factor, low, high, orig) / fs
    assert np.all(np.diff(r) <= 1e-15)
    assert r[0] == 1.0 and math.isclose(r[-1], 1 / factor)


# ---------------------------------------------------------------- rotation

def test_rotation_is_complex_multiplication():
    rng = np.random.default_rng(3)
    d = 16
    x = rng.standard_normal((5, d))
    ang = rng.uniform(-50, 50, size=(5, d // 2))
    got = rotate_pairs(x, ang, "interleaved")
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * ang)
    assert np.allclose(got[:, 0::2], z.real, atol=1e-13)
    assert np.allclose(got[:, 1::2], z.imag, atol=1e-13)
    # the half layout pairs dim i with dim i + d/2: same rotation on a permuted vector
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])  # interleaved -> half order
    got_half = rotate_pairs(x[:, perm], ang, "half")
    assert np.allclose(got_half, got[:, perm], atol=1e-13)


def test_rotation_direction_and_identity():
    # a quarter turn sends (1, 0) to (0, 1): counter-clockwise, multiplication by e^{+i angle}
    r = rotate_pairs(np.array([1.0, 0.0]), np.array([math.pi / 2]), "interleaved")
    assert np.allclose(r, [0.0, 1.0], atol=1e-15)
    x = np.random.default_rng(0).standard_normal(64)
    assert np.array_equal(rotate_pairs(x, np.zeros(32), "interleaved"), x)
    assert np.array_equal(rotate_pairs(x, np.zeros(32), "half"), x)


@pytest.mark.parametrize("layout", ["interleaved", "half"])
def test_rotation_keeps_pair_norms(layout):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 128))
    ang = rng.uniform(0, 8191, size=(7, 64))
    y = rotate_pairs(x, ang, layout)
    if layout == "interleaved":
        nx = x[:, 0::2] ** 2 + x[:, 1::2] ** 2
        ny = y[:, 0::2] ** 2 + y[:, 1::2] ** 2
    else:
        nx = x[:, :64] ** 2 + x[:, 64:] ** 2
        ny = y[:, :64] ** 2 + y[:, 64:] ** 2
    assert np.allclose(nx, ny, rtol=1e-12)


@pytest.mark.parametrize("layout", ["interleaved", "half"])
@pytest.mark.parametrize("scaling", [None, dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0,
                                                original_max_pos=8192.0)])
def test_relative_offset_invariance(layout, scaling):
    """Part 7 key ideas: a rotated q.k depends only on the offset between the two positions."""
    rng = np.random.default_rng(11)
    d = 128
    f = rope_frequencies(5.0e5, d, scaling)
    worst = 0.0
    for _ in range(300):
        q, k = rng.standard_normal(d), rng.standard_normal(d)
        m, n = rng.integers(0, 8192, size=2)
        s = int(rng.integers(-min(m, n), 8192 - max(m, n)))
        a = rotate_pairs(q, m * f, layout) @ rotate_pairs(k, n * f, layout)
        b = rotate_pairs(q, (m + s) * f, layout) @ rotate_pairs(k, (n + s) * f, layout)
        worst = max(worst, abs(a - b) / (np.linalg.norm(q) * np.linalg.norm(k)))
    assert worst < 1e-11
