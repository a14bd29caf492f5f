"""Plant plausible mistakes in a copy of the oracle and check that the pins catch each one.

Each mutant is the oracle's source with one edit (a wrong sign, index, offset,
operand or dropped term), loaded as a separate module on the CPU.  The pins
below are the same independent references the oracle tests use; every
mutant must fail at least one of them, while the unmodified source passes all.
"""

import importlib.util
import math
import os
import sys
import types

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "oracle", "gqa_oracle.py")).read()

MUTANTS = {
    "rotation sign": ("ra = a * c - b * s", "ra = a * c + b * s"),
    "rotation output swapped": ("rb = a * s + b * c", "rb = a * s - b * c"),
    "half pairing": ("a, b = x[..., : d // 2], x[..., d // 2:]", "a, b = x[..., d // 2:], x[..., : d // 2]"),
    "no position offset": ("pos = int(past_len[b]) + np.arange(T, dtype=np.float64)",
                           "pos = np.arange(T, dtype=np.float64)"),
    "frequency exponent": ("freq = np.power(base, -(2.0 * i) / r)", "freq = np.power(base, -(1.0 * i) / r)"),
    "partial rotary exponent uses head dim": ("freq = np.power(base, -(2.0 * i) / r)",
                                              "freq = np.power(base, -(2.0 * i) / d)"),
    "partial rotary tail zeroed": ("out = np.array(x, copy=True)\n    out[..., :r]",
                                   "out = np.zeros_like(x)\n    out[..., :r]"),
    "position interpolation multiplies": ("freq = freq / float(scaling[\"factor\"])",
                                          "freq = freq * float(scaling[\"factor\"])"),
    "ntk exponent dropped": ("base = base * float(scaling[\"factor\"]) ** (r / (r - 2.0))",
                             "base = base * float(scaling[\"factor\"])"),
    "yarn temperature dropped": ("return 0.1 * math.log(float(scaling[\"factor\"])) + 1.0", "return 1.0"),
    "yarn ramp reversed": ("return (1.0 - gamma) * freq / factor + gamma * freq",
                           "return gamma * freq / factor + (1.0 - gamma) * freq"),
    "head map modulo": ("Q = bf16_to_f64(q_rot[b, j * g:(j + 1) * g]).reshape(g * T, d)",
                        "Q = bf16_to_f64(q_rot[b, j::n_kv]).reshape(g * T, d)"),
    "mask off by one": ("vis = r <= pos", "vis = r < pos"),
    "mask ignores past": ("visible_rows(P + t, L, window, n_sink) for t in t_of_row",
                          "visible_rows(t, L, window, n_sink) for t in t_of_row"),
    "window off by one": ("vis &= (r > pos - window) | (r < n_sink)", "vis &= (r >= pos - window) | (r < n_sink)"),
    "sinks ignored": ("vis &= (r > pos - window) | (r < n_sink)", "vis &= (r > pos - window)"),
    "learned sink ignored": ("w = w / (w.sum(axis=1, keepdims=True) + np.exp(sk - top))",
                             "w = w / w.sum(axis=1, keepdims=True)"),
    "row order of score block": ("t_of_row = np.tile(np.arange(T), g)", "t_of_row = np.repeat(np.arange(T), g)"),
    "missing scale": ("s = (Q @ K.T) * scale", "s = (Q @ K.T)"),
    "keys not transposed": ("s = (Q @ K.T) * scale", "s = (Q @ K[:, ::-1].T) * scale"),
    "softmax not normalised": ("w = w / w.sum(axis=1, keepdims=True)", "w = w / w.sum(axis=1, keepdims=True).max()"),
    "value not written": ("vc[b][:, rows, :] = v_new[b]", "pass"),
    "key written unrotated": ("kc[b][:, rows, :] = k_rot", "kc[b][:, rows, :] = k_new[b]"),
    "llama3 blend linear in wavelength": (
        "s = (original_max_pos / wavelength - low_freq_factor) / (high_freq_factor - low_freq_factor)",
        "s = (long_cut - wavelength) / (long_cut - short_cut)"),
    "llama3 blend weights swapped": ("out[i] = (1.0 - s) * f / factor + s * f", "out[i] = s * f / factor + (1.0 - s) * f"),
    "yarn ramp linear in wavelength": ("gamma = np.clip((rho - alpha) / (beta - alpha), 0.0, 1.0)",
                                       "gamma = np.clip((1.0 / alpha - 1.0 / rho) / (1.0 / alpha - 1.0 / beta), 0.0, 1.0)"),
    "ties away from zero": ("y[nz] = np.ldexp(np.rint(np.ldexp(x[nz], -q)), q)",
                            "y[nz] = np.ldexp(np.trunc(np.ldexp(x[nz], -q) + np.copysign(0.5, x[nz])), q)"),
}


def load(src, name):
    mod = types.ModuleType(name)
    exec(compile(src, name, "exec"), mod.__dict__)
    return mod


def rb(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---- independent pins, each returns True when the module passes it

def pin_complex_rotation(m):
    rng = np.random.default_rng(3)
    ok = True
    for layout in ("interleaved", "half"):
        x = rng.standard_normal((4, 16))
        ang = rng.uniform(-9, 9, size=(4, 8))
        got = m.rotate_pairs(x, ang, layout)
        lo, hi = (x[:, 0::2], x[:, 1::2]) if layout == "interleaved" else (x[:, :8], x[:, 8:])
        z = (lo + 1j * hi) * np.exp(1j * ang)
        glo, ghi = (got[:, 0::2], got[:, 1::2]) if layout == "interleaved" else (got[:, :8], got[:, 8:])
        ok &= np.allclose(glo, z.real, atol=1e-12) and np.allclose(ghi, z.imag, atol=1e-12)
    return ok


def pin_frequencies(m):
    f = m.rope_frequencies(1.0e4, 64)
    return f[0] == 1.0 and np.allclose(np.diff(np.log(f)), -2 * math.log(1.0e4) / 64, atol=1e-12)


def pin_position_offset(m):
    rng = np.random.default_rng(4)
    P, d = 6, 8
    qa, ka, va = rb(rng, (1, 2, P + 1, d)), rb(rng, (1, 1, P + 1, d)), rb(rng, (1, 1, P + 1, d))
    kc, vc = rb(rng, (1, 1, 10, d)), rb(rng, (1, 1, 10, d))
    qall, kall, vall = m.rope_append(qa, ka, va, kc, vc, np.array([0]), 100.0)
    qone, kone, vone = m.rope_append(qa[:, :, P:], ka[:, :, P:], va[:, :, P:], kc, vc, np.array([P]), 100.0)
    # the unrotated key must not be what is stored (position P != 0)
    return (np.array_equal(qone[:, :, 0], qall[:, :, P]) and np.array_equal(kone[:, :, P], kall[:, :, P])
            and np.array_equal(vone[:, :, P], va[:, :, P]) and not np.array_equal(kone[:, :, P], ka[:, :, P]))


def pin_torch_cast(m):
    x32 = np.random.default_rng(5).standard_normal(4000).astype(np.float32)
    x32 = np.concatenate([x32, np.float32([1.0 + 2 ** -8, -(1.0 + 2 ** -8), 1.0 + 3 * 2 ** -8])])
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return np.array_equal(m.f64_to_bf16(x32.astype(np.float64)), ref)


def pin_sdpa(m):
    rng = np.random.default_rng(6)
    B, n_q, n_kv, T, d, past = 2, 6, 2, 3, 16, [5, 9]
    S = 14
    q, kc, vc = rb(rng, (B, n_q, T, d)), rb(rng, (B, n_kv, S, d)), rb(rng, (B, n_kv, S, d))
    got = m.attend(q, kc, vc, np.array(past), n_kv)
    g = n_q // n_kv
    for b in range(B):
        L = past[b] + T
        K = torch.from_numpy(f64(kc[b][:, :L])).repeat_interleave(g, dim=0)
        V = torch.from_numpy(f64(vc[b][:, :L])).repeat_interleave(g, dim=0)
        allowed = torch.arange(L)[None, :] <= (past[b] + torch.arange(T))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(f64(q[b])), K, V, attn_mask=allowed)
        if not np.allclose(got[b], ref.numpy(), atol=1e-12):
            return False
    return True


def pin_bruteforce(m):
    rng = np.random.default_rng(7)
    q, kc, vc = rb(rng, (1, 4, 2, 4)), rb(rng, (1, 2, 6, 4)), rb(rng, (1, 2, 6, 4))
    return np.allclose(m.attend(q, kc, vc, np.array([3]), 2), m.attend_bruteforce(q, kc, vc, np.array([3]), 2),
                       atol=1e-12)


def pin_window_rows(m):
    # hand-checked row set: position 9, window 3, two sinks
    return np.flatnonzero(m.visible_rows(9, 12, window=3, n_sink=2)).tolist() == [0, 1, 7, 8, 9]


def pin_window_slice(m):
    # decode with window W equals plain attention over the last W rows
    rng = np.random.default_rng(31)
    q, kc, vc = rb(rng, (1, 4, 1, 8)), rb(rng, (1, 2, 24, 8)), rb(rng, (1, 2, 24, 8))
    W, P = 5, 17
    win = m.attend(q, kc, vc, np.array([P]), 2, window=W)
    lo = P + 1 - W
    sl = m.attend(q, kc[:, :, lo:], vc[:, :, lo:], np.array([W - 1]), 2)
    return np.allclose(win, sl, rtol=0, atol=1e-12)


def pin_sink_closed_form(m):
    # equal keys: output = sum of the visible value rows / (rows + exp(sink - score))
    rng = np.random.default_rng(37)
    q, vc = rb(rng, (1, 2, 1, 8)), rb(rng, (1, 1, 12, 8))
    kc = np.repeat(rb(rng, (1, 1, 1, 8)), 12, axis=2)
    sinks = np.array([0.7, -0.4])
    out = m.attend(q, kc, vc, np.array([7]), 1, sink_logits=sinks)
    ok = True
    for h in range(2):
        s0 = float(f64(q[0, h, 0]) @ f64(kc[0, 0, 0])) / np.sqrt(8)
        expect = f64(vc[0, 0, :8]).sum(axis=0) / (8 + np.exp(sinks[h] - s0))
        ok &= np.allclose(out[0, h, 0], expect, rtol=0, atol=1e-12)
    return ok


def pin_partial_rotary(m):
    # rotating 16 of 32 dims equals full RoPE of a 16-dim head; the tail is copied bit for bit
    rng = np.random.default_rng(41)
    q, kn, vn = rb(rng, (1, 2, 2, 32)), rb(rng, (1, 1, 2, 32)), rb(rng, (1, 1, 2, 32))
    kc, vc = rb(rng, (1, 1, 8, 32)), rb(rng, (1, 1, 8, 32))
    ok = True
    for layout in ("interleaved", "half"):
        qr, kr, _ = m.rope_append(q, kn, vn, kc, vc, np.array([3]), 100.0, layout, rotary_dim=16)
        q2, k2, _ = m.rope_append(q[..., :16].copy(), kn[..., :16].copy(), vn[..., :16].copy(), kc[..., :16].copy(),
                                  vc[..., :16].copy(), np.array([3]), 100.0, layout)
        ok &= np.array_equal(qr[..., :16], q2) and np.array_equal(kr[..., :16], k2)
        ok &= np.array_equal(qr[..., 16:], q[..., 16:]) and np.array_equal(kr[0, :, 3:5, 16:], kn[0, :, :, 16:])
        x = rng.standard_normal((2, 32))
        ok &= np.array_equal(m.rope_rotate(x, 7, 100.0, layout, None, 16)[:, 16:], x[:, 16:])
    return ok


def pin_position_interpolation(m):
    # PI at position p = plain rotation at p / s, written with complex numbers
    x = np.random.default_rng(43).standard_normal((3, 16))
    pos = np.array([5.0, 700.0, 3001.0])
    got = m.rope_rotate(x, pos, 1.0e4, "interleaved", dict(type="linear", factor=4.0))
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * (pos / 4.0)[:, None] * 1.0e4 ** (-np.arange(8) / 8.0))
    return np.allclose(got[:, 0::2], z.real, atol=1e-10) and np.allclose(got[:, 1::2], z.imag, atol=1e-10)


def pin_ntk_lowest_frequency(m):
    plain = m.rope_frequencies(5.0e5, 64)
    ntk = m.rope_frequencies(5.0e5, 64, dict(type="ntk", factor=8.0))
    return ntk[0] == 1.0 and math.isclose(ntk[-1], plain[-1] / 8.0, rel_tol=1e-12)


def pin_yarn(m):
    sc = dict(type="yarn", factor=16.0, beta_slow=1.0, beta_fast=32.0, original_max_pos=4096.0)
    plain = m.rope_frequencies(1.0e4, 64)
    f = m.rope_frequencies(1.0e4, 64, sc)
    turns = 4096.0 * plain / (2 * math.pi)
    ok = np.array_equal(f[turns > 32], plain[turns > 32]) and np.allclose(f[turns < 1], plain[turns < 1] / 16.0)
    rng = np.random.default_rng(47)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    dot = m.rope_rotate(q, 900, 1.0e4, "half", sc) @ m.rope_rotate(k, 900, 1.0e4, "half", sc)
    return ok and math.isclose(dot, (0.1 * math.log(16.0) + 1.0) ** 2 * (q @ k), rel_tol=1e-10)


try:
    from transformers import LlamaConfig
    from transformers import modeling_rope_utils as hf_rope
except ImportError:  # the library pins below need it; the mutants only they catch are then skipped
    hf_rope = None

LIBRARY_MUTANTS = {"llama3 blend linear in wavelength", "llama3 blend weights swapped",
                   "yarn ramp linear in wavelength"}


def _hf_table(kind, fields):
    ctx = int(fields["factor"] * fields["original_max_position_embeddings"])
    cfg = LlamaConfig(hidden_size=512, num_attention_heads=4, num_key_value_heads=2, head_dim=128,
                      max_position_embeddings=ctx, rope_parameters=dict(fields, rope_type=kind, rope_theta=5.0e5))
    fn = hf_rope._compute_llama3_parameters if kind == "llama3" else hf_rope._compute_yarn_parameters
    return fn(cfg, device="cpu")[0].double().numpy()


def pin_llama3_library(m):
    # Llama 3.1's scaling (8, 1, 4, 8192) at theta 5e5, d 128 against the library's table, blend band included
    lib = _hf_table("llama3", {"factor": 8.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0,
                               "original_max_position_embeddings": 8192})
    ours = m.rope_frequencies(5.0e5, 128, dict(type="llama3", factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0,
                                               original_max_pos=8192))
    return float(np.max(np.abs(ours - lib) / lib)) <= 1e-6


def pin_yarn_library(m):
    # same band as the library's ramp; inside it, rho from the library's (log-linear) ramp gives the paper's gamma
    lib = _hf_table("yarn", {"factor": 16.0, "beta_slow": 1.0, "beta_fast": 32.0,
                             "original_max_position_embeddings": 4096, "truncate": False})
    plain = 5.0e5 ** (-np.arange(64) / 64.0)
    ours = m.rope_frequencies(5.0e5, 128, dict(type="yarn", factor=16.0, beta_slow=1.0, beta_fast=32.0,
                                               original_max_pos=4096))
    gl = (lib - plain / 16) / (plain - plain / 16)
    go = (ours - plain / 16) / (plain - plain / 16)
    band = (gl > 1e-5) & (gl < 1 - 1e-5)
    same_band = np.array_equal(band, (go > 1e-5) & (go < 1 - 1e-5))
    outside = float(np.max(np.abs(ours[~band] - lib[~band]) / lib[~band])) <= 1e-6
    inside = np.allclose(go[band], (32.0 ** gl[band] - 1.0) / 31.0, rtol=0, atol=1e-5)
    return same_band and outside and inside


LIBRARY_PINS = [pin_llama3_library, pin_yarn_library] if hf_rope is not None else []

PINS = LIBRARY_PINS + [pin_partial_rotary, pin_position_interpolation, pin_ntk_lowest_frequency, pin_yarn, pin_complex_rotation, pin_frequencies, pin_position_offset, pin_torch_cast, pin_sdpa, pin_bruteforce,
        pin_window_rows, pin_window_slice, pin_sink_closed_form]


def test_unmodified_oracle_passes_every_pin():
    m = load(SRC, "oracle_copy")
    assert all(p(m) for p in PINS)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    if name in LIBRARY_MUTANTS and not LIBRARY_PINS:
        pytest.skip("transformers is not importable: the library pins are unavailable")
    assert SRC.count(old) >= 1, f"mutation site for {name!r} not found"
    m = load(SRC.replace(old, new), "oracle_mutant")
    failed = []
    for p in PINS:
        try:
            if not p(m):
                failed.append(p.__name__)
        except Exception:
            failed.append(p.__name__ + " (raised)")
    assert failed, f"no pin caught mutant {name!r}"
