"""Pins of the oracle's sliding window, attention sinks and learned sinks (CPU only).

The window / sink rule is pinned by reductions to the already pinned causal
attention (a window covering the whole context, sinks covering it, a window
equal to full attention over the cache sliced to its last W rows), by closed
forms (a one-row window returns that value row; with equal keys the output
is the mean of the kept rows, or that mean shrunk by the learned sink's share
of the normaliser), by the explicit-loop formulation on tiny shapes, and by
the row sets the rule must produce on a small hand-checked example.
"""

import math

import numpy as np
import pytest

from oracle import attend, attend_bruteforce, bf16_to_f64, f64_to_bf16, visible_rows


def rand_bits(rng, shape, scale=1.0):
    return f64_to_bf16(rng.standard_normal(shape) * scale)


def make_case(rng, B, n_q, n_kv, T, d, S, past):
    q = rand_bits(rng, (B, n_q, T, d))
    kc = rand_bits(rng, (B, n_kv, S, d))
    vc = rand_bits(rng, (B, n_kv, S, d))
    return q, kc, vc, np.asarray(past, dtype=np.int32)


def test_visible_rows_hand_example():
    # query at position 9 of a 12-row cache, window 3, two sinks: rows 0, 1 and 7, 8, 9
    assert np.flatnonzero(visible_rows(9, 12, window=3, n_sink=2)).tolist() == [0, 1, 7, 8, 9]
    assert np.flatnonzero(visible_rows(9, 12)).tolist() == list(range(10))
    assert np.flatnonzero(visible_rows(9, 12, window=3)).tolist() == [7, 8, 9]
    assert np.flatnonzero(visible_rows(1, 12, window=3, n_sink=2)).tolist() == [0, 1]
    assert np.flatnonzero(visible_rows(0, 12, window=1)).tolist() == [0]


@pytest.mark.parametrize("B,n_q,n_kv,T,d,past,window,n_sink", [
    (1, 2, 1, 1, 4, [9], 3, 2),
    (2, 4, 2, 3, 4, [0, 6], 2, 1),
    (1, 6, 2, 4, 8, [5], 4, 0),
    (1, 2, 2, 2, 4, [3], 1, 3),
])
def test_matches_bruteforce(B, n_q, n_kv, T, d, past, window, n_sink):
    rng = np.random.default_rng(sum(past) + window * 7 + n_sink)
    q, kc, vc, pl = make_case(rng, B, n_q, n_kv, T, d, max(past) + T + 2, past)
    sinks = rng.standard_normal(n_q)
    for sl in (None, sinks):
        a = attend(q, kc, vc, pl, n_kv, window=window, n_sink=n_sink, sink_logits=sl)
        b = attend_bruteforce(q, kc, vc, pl, n_kv, window=window, n_sink=n_sink, sink_logits=sl)
        assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_window_covering_the_context_is_plain_attention():
    rng = np.random.default_rng(3)
    q, kc, vc, pl = make_case(rng, 2, 8, 2, 3, 16, 40, [20, 31])
    full = attend(q, kc, vc, pl, 2)
    assert np.array_equal(attend(q, kc, vc, pl, 2, window=34), full)
    assert np.array_equal(attend(q, kc, vc, pl, 2, window=3, n_sink=34), full)


def test_decode_window_equals_attention_over_the_sliced_cache():
    rng = np.random.default_rng(5)
    B, n_q, n_kv, d, S, W = 2, 8, 2, 16, 64, 7
    q, kc, vc, pl = make_case(rng, B, n_q, n_kv, 1, d, S, [40, 12])
    win = attend(q, kc, vc, pl, n_kv, window=W)
    for b in range(B):
        P = int(pl[b])
        lo = P + 1 - W
        sl = attend(q[b:b + 1], kc[b:b + 1, :, lo:], vc[b:b + 1, :, lo:], np.array([W - 1]), n_kv)
        assert np.allclose(win[b:b + 1], sl, rtol=0, atol=1e-13)


def test_one_row_window_returns_the_newest_value_row():
    rng = np.random.default_rng(6)
    q, kc, vc, pl = make_case(rng, 1, 4, 2, 3, 8, 20, [9])
    out = attend(q, kc, vc, pl, 2, window=1)
    for h in range(4):
        for t in range(3):
            assert np.array_equal(out[0, h, t], bf16_to_f64(vc[0, h // 2, 9 + t]))


def test_equal_keys_give_the_mean_of_the_kept_rows():
    rng = np.random.default_rng(7)
    B, n_q, n_kv, T, d, S, W, NS = 1, 4, 2, 2, 8, 30, 4, 3
    q, kc, vc, pl = make_case(rng, B, n_q, n_kv, T, d, S, [17])
    kc[:] = kc[:, :, :1, :]
    out = attend(q, kc, vc, pl, n_kv, window=W, n_sink=NS)
    for h in range(n_q):
        for t in range(T):
            pos = 17 + t
            rows = sorted(set(range(NS)) | set(range(pos - W + 1, pos + 1)))
            mean = bf16_to_f64(vc[0, h // 2, rows]).mean(axis=0)
            assert np.allclose(out[0, h, t], mean, rtol=0, atol=1e-13)


def test_learned_sink_closed_forms():
    rng = np.random.default_rng(8)
    B, n_q, n_kv, T, d, S = 1, 4, 2, 1, 8, 16
    q, kc, vc, pl = make_case(rng, B, n_q, n_kv, T, d, S, [9])
    plain = attend(q, kc, vc, pl, n_kv)
    assert np.array_equal(attend(q, kc, vc, pl, n_kv, sink_logits=np.full(n_q, -np.inf)), plain)
    # equal keys: every score is s0 = q.k0 * scale; the sink adds exp(sink - s0) rows' worth of weight
    kc[:] = kc[:, :, :1, :]
    sinks = np.array([0.5, -1.0, 2.0, 0.0])
    out = attend(q, kc, vc, pl, n_kv, sink_logits=sinks)
    scale = 1.0 / math.sqrt(d)
    for h in range(n_q):
        k0 = bf16_to_f64(kc[0, h // 2, 0])
        s0 = float(bf16_to_f64(q[0, h, 0]) @ k0) * scale
        vals = bf16_to_f64(vc[0, h // 2, :10])
        expect = vals.sum(axis=0) / (10 + math.exp(sinks[h] - s0))
        assert np.allclose(out[0, h, 0], expect, rtol=0, atol=1e-12)
