"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded inputs.

Bars: cache rows bit-exact for v and within 1 bf16 ulp for the rotated k (and
for q_rot); attention outputs within max-abs 1e-2 AND max-rel 1e-2, where the
relative error of an element is |e| / max(|ref|, 1e-2).  Every cache row the
call must not read is filled with bf16 NaN first, so a stray read shows up
as a non-finite output.
"""

import math
import sys

import numpy as np
import pytest
import torch

import gqa_attention_rope_amd as gq
from gqa_attention_rope_amd import synth
from oracle import attend, bf16_to_f64, rope_append

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCALED = synth.LLAMA3_SCALING


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ulp_key(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    return np.where(b & 0x8000, 0x8000 - b, b)


def max_ulp(a, b):
    return int(np.max(np.abs(ulp_key(a) - ulp_key(b)))) if np.size(a) else 0


def half_ulp_bf16(x):
    """Half the spacing of bf16 values at |x| (8 significant bits): the most that rounding x to bf16 moves it."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def check_out(gpu_bits, ref, name):
    """Attention outputs against the fp64 oracle: max-abs 1e-2 on the computed result, which the output
    then carries rounded once to bf16 (up to half a bf16 ulp of the reference more), and max-rel 1e-2."""
    g = bf16_to_f64(gpu_bits)
    assert np.all(np.isfinite(g)), f"{name}: non-finite outputs"
    err = np.abs(g - ref)
    rel = err / np.maximum(np.abs(ref), 1e-2)
    bad = (err > 1e-2 + half_ulp_bf16(ref)) | (rel > 1e-2)
    say(f"  {name}: max abs {err.max():.3e}  max rel {rel.max():.3e}  n={err.size}")
    if bad.any():
        i = np.flatnonzero(bad)[0]
        raise AssertionError(f"{name}: {int(bad.sum())} of {bad.size} outside; first at flat index {i}: "
                             f"ref {ref.flat[i]:.6g} got {g.flat[i]:.6g} (max abs {err.max():.3e}, "
                             f"max rel {rel.max():.3e})")


def dev(bits):
    return synth.from_bits(bits, DEV)


def past_dev(p):
    return torch.as_tensor(np.asarray(p, dtype=np.int32), device=DEV)


def make_inputs(B, n_q, n_kv, T, d, S, past, seed):
    q = synth.bits(synth.normal_bf16((B, n_q, T, d), seed))
    kn = synth.bits(synth.normal_bf16((B, n_kv, T, d), seed + 1))
    vn = synth.bits(synth.normal_bf16((B, n_kv, T, d), seed + 2))
    kc = synth.bits(synth.normal_bf16((B, n_kv, S, d), seed + 3))
    vc = synth.bits(synth.normal_bf16((B, n_kv, S, d), seed + 4))
    for b in range(B):  # rows the step must neither read nor write
        kc[b, :, past[b] + T:] = synth.NAN_BF16
        vc[b, :, past[b] + T:] = synth.NAN_BF16
    return q, kn, vn, kc, vc


def poison_unread_tiles(caches, past, W, NS):
    """Under a window of W rows with NS sinks, fill with bf16 NaN the 64-row tiles that hold no row visible to
    any query of the call: those wholly between the sink tiles and the window of the earliest query (position
    past_len, which sees rows past_len - W + 1 .. past_len).  The kernels must not read them.  Returns the
    number of rows filled per cache."""
    n = 0
    for b, P in enumerate(past):
        w0 = P - W + 1
        if W <= 0 or w0 <= NS:
            continue
        lo, hi = -(-NS // 64) * 64, (w0 // 64) * 64
        if hi > lo:
            for c in caches:
                c[b, :, lo:hi] = synth.NAN_BF16
            n += hi - lo
    return n


# ---------------------------------------------------------------- rope_append

APPEND_CASES = [
    # B, n_q, n_kv, T, d, S, past, theta, layout, scaling
    (1, 6, 2, 1, 64, 256, [255], 1.0e4, "interleaved", None),
    (1, 32, 8, 1, 128, 8192, [1000], 5.0e5, "interleaved", None),
    (3, 8, 2, 5, 128, 300, [0, 17, 290], 5.0e5, "interleaved", None),
    (2, 8, 2, 3, 128, 8192, [8000, 4096], 5.0e5, "half", None),
    (2, 16, 2, 1, 128, 8192, [8190, 5000], 5.0e5, "interleaved", SCALED),
    (2, 6, 3, 4, 64, 100, [10, 96], 1.0e4, "half", SCALED),
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=lambda c: f"B{c[0]}q{c[1]}kv{c[2]}T{c[3]}d{c[4]}{c[8]}{'S' if c[9] else ''}")
def test_rope_append_parity(case):
    B, n_q, n_kv, T, d, S, past, theta, layout, scaling = case
    say(f"rope_append {case[:8]} {layout} scaled={bool(scaling)}")
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, T, d, S, past, seed=11 + B + d)
    q_ref, kc_ref, vc_ref = rope_append(q, kn, vn, kc, vc, past, theta, layout, scaling)
    kc_d, vc_d = dev(kc), dev(vc)
    q_rot = gq.gqa_rope_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, past_dev(past), max(past), theta, layout, scaling)
    torch.cuda.synchronize()
    q_g, kc_g, vc_g = synth.bits(q_rot), synth.bits(kc_d), synth.bits(vc_d)
    assert np.array_equal(vc_g, vc_ref), "value rows must be copied bit for bit and no other row touched"
    rows = np.zeros(S, dtype=bool)
    for b in range(B):
        other = np.ones(S, dtype=bool)
        other[past[b]:past[b] + T] = False
        assert np.array_equal(kc_g[b][:, other], kc[b][:, other]), "rows outside the append must not change"
        assert max_ulp(kc_g[b][:, ~other], kc_ref[b][:, ~other]) <= 1
    assert max_ulp(q_g, q_ref) <= 1
    say(f"  q_rot bit-exact {np.mean(q_g == q_ref):.6f}, k rows bit-exact "
        f"{np.mean(kc_g == kc_ref):.6f}")


def test_rope_append_in_place_q():
    B, n_q, n_kv, T, d, S, past = 2, 8, 2, 3, 128, 64, [7, 40]
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, T, d, S, past, seed=5)
    q_ref, _, _ = rope_append(q, kn, vn, kc, vc, past, 5.0e5)
    qd = dev(q)
    out = gq.gqa_rope_append(qd, dev(kn), dev(vn), dev(kc), dev(vc), past_dev(past), max(past), 5.0e5, q_rot=qd)
    torch.cuda.synchronize()
    assert out.data_ptr() == qd.data_ptr()
    assert max_ulp(synth.bits(qd), q_ref) <= 1


LIN4 = dict(type="linear", factor=4.0)
NTK8 = dict(type="ntk", factor=8.0)
YARN16 = dict(type="yarn", factor=16.0, beta_slow=1.0, beta_fast=32.0, original_max_pos=4096.0)

VARIANT_CASES = [
    # B, n_q, n_kv, T, d, S, past, theta, layout, scaling, rotary_dim
    (2, 8, 2, 3, 128, 300, [0, 290], 1.0e4, "interleaved", None, 64),
    (2, 8, 2, 3, 128, 300, [5, 200], 1.0e4, "half", None, 32),
    (2, 6, 3, 2, 64, 100, [10, 90], 1.0e4, "half", None, 16),
    (2, 6, 3, 2, 64, 100, [10, 90], 1.0e4, "interleaved", None, 48),
    (2, 16, 2, 1, 128, 8192, [8190, 5000], 5.0e5, "interleaved", LIN4, None),
    (2, 16, 2, 4, 128, 8192, [8000, 30], 5.0e5, "half", NTK8, None),
    (1, 8, 2, 5, 64, 8192, [7000], 1.0e4, "interleaved", dict(NTK8, factor=4.0), 32),
    (2, 16, 2, 4, 128, 8192, [8000, 30], 1.0e4, "interleaved", YARN16, None),
    (1, 8, 2, 5, 128, 8192, [6000], 1.0e4, "half", dict(YARN16, attn_factor=1.3), 64),
]


@pytest.mark.parametrize("case", VARIANT_CASES,
                         ids=lambda c: f"d{c[4]}{c[8][0]}{(c[9] or {}).get('type', 'plain')}r{c[10] or c[4]}")
def test_rope_append_variants(case):
    B, n_q, n_kv, T, d, S, past, theta, layout, scaling, rdim = case
    say(f"rope_append variant {case}")
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, T, d, S, past, seed=23 + T + d)
    q_ref, kc_ref, vc_ref = rope_append(q, kn, vn, kc, vc, past, theta, layout, scaling, rotary_dim=rdim)
    kc_d, vc_d = dev(kc), dev(vc)
    q_rot = gq.gqa_rope_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, past_dev(past), max(past), theta, layout,
                               scaling, rotary_dim=rdim)
    torch.cuda.synchronize()
    q_g, kc_g, vc_g = synth.bits(q_rot), synth.bits(kc_d), synth.bits(vc_d)
    r = rdim or d
    assert np.array_equal(vc_g, vc_ref)
    assert np.array_equal(q_g[..., r:], q[..., r:]), "unrotated dims are copied bit for bit"
    assert max_ulp(q_g, q_ref) <= 1
    for b in range(B):
        rows = slice(past[b], past[b] + T)
        assert np.array_equal(kc_g[b][:, rows, r:], kn[b][..., r:])
        assert max_ulp(kc_g[b][:, rows], kc_ref[b][:, rows]) <= 1
        other = np.ones(S, dtype=bool)
        other[rows] = False
        assert np.array_equal(kc_g[b][:, other], kc[b][:, other])
    say(f"  q_rot bit-exact {np.mean(q_g == q_ref):.6f}")


def test_decode_after_yarn_partial_rotary():
    B, n_q, n_kv, d, S, past = 3, 32, 8, 128, 6000, [5999, 4100, 10]
    say("decode after YaRN + partial rotary")
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=77)
    q_ref, kc_ref, vc_ref = rope_append(q, kn, vn, kc, vc, past, 1.0e4, "half", YARN16, rotary_dim=64)
    ref = attend(q_ref, kc_ref, vc_ref, past, n_kv)
    kc_d, vc_d, pl = dev(kc), dev(vc), past_dev(past)
    q_rot = gq.gqa_rope_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, pl, max(past), 1.0e4, "half", YARN16,
                               rotary_dim=64)
    out = gq.gqa_decode_attn(q_rot, kc_d, vc_d, pl, max(past))
    torch.cuda.synchronize()
    check_out(synth.bits(out), ref, "decode after YaRN + partial rotary")


# ---------------------------------------------------------------- decode

DECODE_CASES = [
    # B, n_q, n_kv, d, S, past, theta, layout, scaling
    (1, 6, 2, 64, 256, [255], 1.0e4, "interleaved", None),            # tiny 6/2-head window
    (1, 32, 8, 128, 8192, [1000], 5.0e5, "interleaved", None),        # one Llama-3.1-8B layer
    (5, 32, 8, 128, 1100, [0, 63, 64, 65, 1098], 5.0e5, "interleaved", None),  # tile edges, L = 1
    (3, 64, 8, 128, 600, [511, 300, 599], 5.0e5, "interleaved", SCALED),       # g = 8, scaled RoPE
    (2, 8, 8, 128, 200, [150, 9], 5.0e5, "half", None),               # g = 1 (MHA)
    (2, 6, 1, 64, 300, [299, 77], 1.0e4, "interleaved", None),        # g = 6 (MQA)
    (2, 16, 1, 128, 300, [200, 1], 5.0e5, "interleaved", None),       # g = 16
    (2, 10, 2, 128, 300, [100, 257], 5.0e5, "interleaved", None),     # g = 5: one head per segment
    (2, 24, 2, 64, 200, [130, 66], 1.0e4, "half", None),              # g = 12
]


def run_decode_e2e(case, seed, wg=0, schedule=(-1, 0), slot_ratio=0):
    """rope_append + decode_attn on the GPU.  The rotated rows are checked against the oracle's (q and k
    within 1 bf16 ulp, v exact); the attention reference is the oracle on the same bf16 inputs the GPU
    attention read (its rotated q and appended rows), so a permitted 1-ulp rotation difference does not
    count against the attention tolerance."""
    B, n_q, n_kv, d, S, past, theta, layout, scaling = case
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed)
    q_ref, kc_ref, vc_ref = rope_append(q, kn, vn, kc, vc, past, theta, layout, scaling)
    kc_d, vc_d, pl = dev(kc), dev(vc), past_dev(past)
    gq.gqa_set_decode_workgroups(wg)
    gq.gqa_set_decode_schedule(*schedule)
    gq.gqa_set_decode_slot_ratio(slot_ratio)
    try:
        q_rot = gq.gqa_rope_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, pl, max(past), theta, layout, scaling)
        out = gq.gqa_decode_attn(q_rot, kc_d, vc_d, pl, max(past))
        torch.cuda.synchronize()
    finally:
        gq.gqa_set_decode_workgroups(0)
        gq.gqa_set_decode_schedule()
        gq.gqa_set_decode_slot_ratio(0)
    rows_b, rows_p = np.arange(B), np.asarray(past)
    tb, tp = torch.as_tensor(rows_b, device=DEV), torch.as_tensor(rows_p, device=DEV)
    qg = synth.bits(q_rot)
    kg_rows, vg_rows = synth.bits(kc_d[tb, :, tp]), synth.bits(vc_d[tb, :, tp])
    assert max_ulp(qg, q_ref) <= 1, "rotated q beyond 1 bf16 ulp"
    assert max_ulp(kg_rows, kc_ref[rows_b, :, rows_p]) <= 1, "rotated k row beyond 1 bf16 ulp"
    assert np.array_equal(vg_rows, vc_ref[rows_b, :, rows_p]), "appended v row differs"
    kc_ref[rows_b, :, rows_p] = kg_rows
    ref = attend(qg, kc_ref, vc_ref, past, n_kv)
    return synth.bits(out), ref, (q_rot, kc_d, vc_d, pl)


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"B{c[0]}q{c[1]}kv{c[2]}d{c[3]}P{max(c[5])}")
def test_decode_end_to_end(case):
    say(f"decode e2e {case[:6]}")
    got, ref, _ = run_decode_e2e(case, seed=100 + case[1])
    check_out(got, ref, "decode")


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"B{c[0]}q{c[1]}kv{c[2]}d{c[3]}P{max(c[5])}")
def test_decode_oracle_rope_end_to_end(case):
    """rope_append + decode_attn against the oracle doing its own RoPE and append: the reference never
    sees a GPU value (the tiny 6/2-head and one-layer Llama-3.1-8B shapes are the first two cases)."""
    B, n_q, n_kv, d, S, past, theta, layout, scaling = case
    say(f"decode e2e, oracle RoPE {case[:6]}")
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=150 + case[1])
    q_ref, kc_ref, vc_ref = rope_append(q, kn, vn, kc, vc, past, theta, layout, scaling)
    ref = attend(q_ref, kc_ref, vc_ref, past, n_kv)
    kc_d, vc_d, pl = dev(kc), dev(vc), past_dev(past)
    q_rot = gq.gqa_rope_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, pl, max(past), theta, layout, scaling)
    out = gq.gqa_decode_attn(q_rot, kc_d, vc_d, pl, max(past))
    torch.cuda.synchronize()
    check_out(synth.bits(out), ref, "decode, oracle RoPE")


@pytest.mark.parametrize("case", DECODE_CASES[:4], ids=lambda c: f"B{c[0]}q{c[1]}kv{c[2]}P{max(c[5])}")
def test_decode_kernel_isolated(case):
    """Attention alone on synthetic already-rotated q and cache rows."""
    B, n_q, n_kv, d, S, past = case[:6]
    say(f"decode isolated {case[:6]}")
    q, _, _, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=300 + n_q)
    # the new row past_len is part of the attended range here: make it finite
    kc2, vc2 = kc.copy(), vc.copy()
    for b in range(B):
        kc2[b, :, past[b]] = synth.bits(synth.normal_bf16((n_kv, d), 900 + b))
        vc2[b, :, past[b]] = synth.bits(synth.normal_bf16((n_kv, d), 950 + b))
    ref = attend(q, kc2, vc2, past, n_kv)
    out = gq.gqa_decode_attn(dev(q), dev(kc2), dev(vc2), past_dev(past), max(past))
    torch.cuda.synchronize()
    check_out(synth.bits(out), ref, "decode isolated")


def test_decode_workgroup_count_invariance_and_determinism():
    case = (4, 32, 8, 128, 2000, [1999, 3, 700, 1500], 5.0e5, "interleaved", None)
    say("decode workgroup sweep")
    outs = []
    for wg in (1, 3, 37, 256, 0):
        got, ref, _ = run_decode_e2e(case, seed=77, wg=wg)
        check_out(got, ref, f"decode wg={wg}")
        outs.append(got)
    again, _, _ = run_decode_e2e(case, seed=77, wg=0)
    assert np.array_equal(again, outs[-1]), "same launch shape must give bitwise identical results"


@pytest.mark.parametrize("wg", [0, 37])
def test_decode_schedule_invariance_and_determinism(wg):
    """All-static, all-dynamic and mixed work splits, chunk sizes 1..5: same results to the tolerance, and a
    repeated call with the same launch shape and schedule is bitwise identical."""
    case = (6, 32, 8, 128, 3000, [2999, 0, 700, 1500, 64, 2100], 5.0e5, "interleaved", None)
    say(f"decode schedule sweep wg={wg}")
    for sched in ((1000, 2), (0, 1), (0, 2), (500, 3), (700, 2), (300, 5)):
        got, ref, _ = run_decode_e2e(case, seed=91, wg=wg, schedule=sched)
        check_out(got, ref, f"decode wg={wg} schedule={sched}")
        again, _, _ = run_decode_e2e(case, seed=91, wg=wg, schedule=sched)
        assert np.array_equal(again, got), f"schedule {sched}: repeated call differs"


@pytest.mark.parametrize("wg", [0, 600, 1100])
def test_decode_slot_weighted_shares(wg):
    """Static shares weighted by dispatch slot: equal (1000), the default, steep (3000) and extreme (8000,
    where the youngest slots get empty shares) ratios, over grids of one to several dispatch rounds, with
    all-static and mixed splits: same results to the tolerance, bitwise repeatable."""
    case = (6, 32, 8, 128, 3000, [2999, 0, 700, 1500, 64, 2100], 5.0e5, "interleaved", None)
    say(f"decode slot-weighted shares wg={wg}")
    for ratio in (1000, 0, 3000, 8000):
        for sched in ((1000, 2), (700, 4)):
            got, ref, _ = run_decode_e2e(case, seed=93, wg=wg, schedule=sched, slot_ratio=ratio)
            check_out(got, ref, f"decode wg={wg} ratio={ratio} schedule={sched}")
            again, _, _ = run_decode_e2e(case, seed=93, wg=wg, schedule=sched, slot_ratio=ratio)
            assert np.array_equal(again, got), f"ratio {ratio} schedule {sched}: repeated call differs"


def test_decode_many_short_segments():
    """17600 (sequence, KV head) segments of at most one tile each: a record per segment, ragged one-row
    to 31-row contexts, outputs up to |4| and more (where a bf16 output rounds by up to 0.0156)."""
    B, n_q, n_kv, d, S = 1100, 32, 16, 64, 32
    past = [int(x) for x in np.random.default_rng(6).integers(0, 31, size=B)]
    case = (B, n_q, n_kv, d, S, past, 1.0e4, "interleaved", None)
    say(f"decode many segments B{B} n_kv{n_kv}")
    got, ref, _ = run_decode_e2e(case, seed=99)
    check_out(got, ref, "decode many segments")


def test_decode_workspace_reuse_leaves_header_zero():
    """One caller-owned workspace serves consecutive calls of different sizes; each call clears the
    scheduling header it used."""
    say("decode workspace reuse")
    B, n_q, n_kv, d, S = 4, 32, 8, 128, 2500
    ws = torch.zeros(gq.gqa_decode_workspace_bytes(B, n_q, n_kv, d, S), dtype=torch.uint8, device=DEV)
    for it, past in enumerate(([2400, 10, 999, 1800], [5, 2499, 64, 300], [1, 1, 1, 1])):
        q, _, _, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=500 + it)
        for b in range(B):  # row past_len is attended here: make it finite
            kc[b, :, past[b]] = synth.bits(synth.normal_bf16((n_kv, d), 600 + 10 * it + b))
            vc[b, :, past[b]] = synth.bits(synth.normal_bf16((n_kv, d), 700 + 10 * it + b))
        ref = attend(q, kc, vc, past, n_kv)
        out = gq.gqa_decode_attn(dev(q), dev(kc), dev(vc), past_dev(past), max(past), workspace=ws)
        torch.cuda.synchronize()
        check_out(synth.bits(out), ref, f"decode reuse call {it}")
        assert int(ws[:256].count_nonzero()) == 0, "scheduling header must be zero after a call"


def test_decode_workspace_serves_smaller_batches():
    """A decode workspace sized for six sequences serves calls of 6, 2, 5, 1 and 6 sequences in turn (the
    scheduling header sits at a fixed place and is zero after every call; the record directory and the
    records are rewritten by each call), each matching the oracle."""
    n_q, n_kv, d, S = 32, 8, 128, 3000
    ws = torch.zeros(gq.gqa_decode_workspace_bytes(6, n_q, n_kv, d, S), dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(43)
    for it, B in enumerate((6, 2, 5, 1, 6)):
        past = [int(x) for x in rng.integers(0, S - 1, size=B)]
        q, _, _, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=2300 + it)
        for b in range(B):  # row past_len is attended here: make it finite
            kc[b, :, past[b]] = synth.bits(synth.normal_bf16((n_kv, d), 2400 + 10 * it + b))
            vc[b, :, past[b]] = synth.bits(synth.normal_bf16((n_kv, d), 2500 + 10 * it + b))
        ref = attend(q, kc, vc, past, n_kv)
        out = gq.gqa_decode_attn(dev(q), dev(kc), dev(vc), past_dev(past), max(past), workspace=ws)
        torch.cuda.synchronize()
        check_out(synth.bits(out), ref, f"decode B{B} on a six-sequence workspace")
        assert int(ws[:256].count_nonzero()) == 0, "scheduling header must be zero after a call"


def test_decode_scale_argument():
    B, n_q, n_kv, d, S, past = 2, 8, 2, 128, 128, [100, 20]
    q, _, _, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=8)
    for b in range(B):
        kc[b, :, past[b]] = 0
        vc[b, :, past[b]] = 0
    ref = attend(q, kc, vc, past, n_kv, scale=0.3)
    out = gq.gqa_decode_attn(dev(q), dev(kc), dev(vc), past_dev(past), max(past), scale=0.3)
    torch.cuda.synchronize()
    check_out(synth.bits(out), ref, "decode scale=0.3")


# ---------------------------------------------------------------- prefill

PREFILL_CASES = [
    # B, n_q, n_kv, T, d, S, past, theta, layout, scaling
    (2, 8, 2, 70, 128, 256, [5, 130], 5.0e5, "interleaved", None),
    (1, 6, 2, 100, 64, 160, [33], 1.0e4, "interleaved", None),       # g = 3: 42 positions per workgroup
    (2, 4, 4, 65, 128, 200, [0, 64], 5.0e5, "half", None),           # g = 1
    (1, 32, 2, 40, 128, 100, [27], 5.0e5, "interleaved", SCALED),    # g = 16
    (3, 16, 2, 1, 128, 300, [299 - 1, 10, 200], 5.0e5, "interleaved", None),  # T = 1
    # 16 (sequence, KV head) groups: the XCD-local work map with complementary query tiles, ragged lengths
    (2, 32, 8, 45, 128, 300, [17, 250], 5.0e5, "interleaved", None),
    (2, 16, 8, 70, 64, 200, [5, 120], 1.0e4, "half", None),          # g = 2, d 64: two query tiles per group
]


def run_prefill_e2e(case, seed):
    B, n_q, n_kv, T, d, S, past, theta, layout, scaling = case
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, T, d, S, past, seed)
    q_ref, kc_ref, vc_ref = rope_append(q, kn, vn, kc, vc, past, theta, layout, scaling)
    ref = attend(q_ref, kc_ref, vc_ref, past, n_kv)
    kc_d, vc_d, pl = dev(kc), dev(vc), past_dev(past)
    q_rot = gq.gqa_rope_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, pl, max(past), theta, layout, scaling)
    out = gq.gqa_prefill_attn(q_rot, kc_d, vc_d, pl, max(past))
    torch.cuda.synchronize()
    return synth.bits(out), ref, (q_rot, kc_d, vc_d, pl)


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: f"B{c[0]}q{c[1]}kv{c[2]}T{c[3]}d{c[4]}")
def test_prefill_end_to_end(case):
    say(f"prefill e2e {case[:7]}")
    got, ref, _ = run_prefill_e2e(case, seed=500 + case[3])
    check_out(got, ref, "prefill")


def test_prefill_split_equals_whole():
    """prefill(T) == prefill(T-1) then a one-token decode at the next position."""
    B, n_q, n_kv, T, d, S, past = 2, 32, 8, 33, 128, 200, [40, 100]
    say("prefill split")
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, T, d, S, past, seed=42)
    kc_d, vc_d, pl = dev(kc), dev(vc), past_dev(past)
    q_rot = gq.gqa_rope_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, pl, max(past), 5.0e5)
    whole = gq.gqa_prefill_attn(q_rot, kc_d, vc_d, pl, max(past))
    head = gq.gqa_prefill_attn(q_rot[:, :, :T - 1].contiguous(), kc_d, vc_d, pl, max(past))
    pl_last = past_dev([p + T - 1 for p in past])
    tail = gq.gqa_decode_attn(q_rot[:, :, T - 1:].contiguous(), kc_d, vc_d, pl_last, max(past) + T - 1)
    torch.cuda.synchronize()
    w = bf16_to_f64(synth.bits(whole))
    check_out(synth.bits(head), w[:, :, :T - 1], "prefill head vs whole")
    check_out(synth.bits(tail), w[:, :, T - 1:], "decode tail vs whole")


# ---------------------------------------------------------------- full-size workloads (sampled outputs)

def full_size_decode(name, sample_b, layer_seed_offset=0):
    w = synth.WORKLOADS[name]
    B, n_q, n_kv, d, S = w["B"], w["n_q"], w["n_kv"], w["d"], w["S"]
    past = synth.past_lengths(B, w["past"], w["seed"])
    seed = w["seed"] + layer_seed_offset
    say(f"{name}: B={B} n_q={n_q} n_kv={n_kv} S={S} max past {past.max()}")
    kc = synth.normal_bf16((B, n_kv, S, d), seed + 3, DEV)
    vc = synth.normal_bf16((B, n_kv, S, d), seed + 4, DEV)
    q = synth.normal_bf16((B, n_q, 1, d), seed, DEV)
    kn = synth.normal_bf16((B, n_kv, 1, d), seed + 1, DEV)
    vn = synth.normal_bf16((B, n_kv, 1, d), seed + 2, DEV)
    synth.poison_beyond(kc, past, 1)
    synth.poison_beyond(vc, past, 1)
    sb = np.asarray(sample_b)
    # the oracle sees the sampled sequences' inputs as they are before the step
    kc_s, vc_s = synth.bits(kc[sb]), synth.bits(vc[sb])
    q_s, kn_s, vn_s = synth.bits(q[sb]), synth.bits(kn[sb]), synth.bits(vn[sb])
    pl = past_dev(past)
    q_rot = gq.gqa_rope_append(q, kn, vn, kc, vc, pl, int(past.max()), w["theta"], "interleaved", w["scaling"])
    out = gq.gqa_decode_attn(q_rot, kc, vc, pl, int(past.max()))
    torch.cuda.synchronize()
    got = synth.bits(out[sb])
    q_ref, kc_ref, vc_ref = rope_append(q_s, kn_s, vn_s, kc_s, vc_s, past[sb], w["theta"], "interleaved",
                                        w["scaling"])
    ref = attend(q_ref, kc_ref, vc_ref, past[sb], n_kv)
    check_out(got, ref, name)
    assert max_ulp(synth.bits(q_rot[sb]), q_ref) <= 1
    for i, b in enumerate(sb):
        p = int(past[b])
        assert max_ulp(synth.bits(kc[b, :, p]), kc_ref[i, :, p]) <= 1
        assert np.array_equal(synth.bits(vc[b, :, p]), vc_ref[i, :, p])
    del kc, vc
    torch.cuda.empty_cache()


def test_full_size_batched_decode_layer():
    """B=32 ragged contexts up to 8192, one layer of the 32-layer step (sampled sequences)."""
    full_size_decode("llama8b_b32_decode_32layers", sample_b=[0, 5, 13, 31])


def test_full_size_long_context_scaled_decode():
    """B=64, 64/8 heads, ragged 4096..8191, scaled RoPE: one of the 80 layer calls (sampled)."""
    full_size_decode("llama70b_shape_decode_scaled", sample_b=[0, 17, 63])


def test_full_size_long_context_scaled_decode_80_calls():
    """The 70B-shaped workload as the bench runs it: one cache pair (B=64, 64/8 heads, 2 GiB), 80
    sequential rope_append + decode_attn calls with their own new q/k/v (the bench's per-call inputs),
    each rewriting row past_len[b].  Calls 0 and 79 are compared with the oracle on sampled sequences;
    the oracle's cache for call c is the initial cache with row past_len[b] appended by call c."""
    name = "llama70b_shape_decode_scaled"
    w = synth.WORKLOADS[name]
    B, n_q, n_kv, d, S, layers = w["B"], w["n_q"], w["n_kv"], w["d"], w["S"], w["layers"]
    past = synth.past_lengths(B, w["past"], w["seed"])
    say(f"{name}: {layers} calls on one cache pair, B={B} max past {past.max()}")
    kc = torch.empty((B, n_kv, S, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    synth.fill_normal_bf16_(kc, w["seed"] * 1000)
    synth.fill_normal_bf16_(vc, w["seed"] * 1000 + 1)
    synth.poison_beyond(kc, past, 1)
    synth.poison_beyond(vc, past, 1)
    q = synth.normal_bf16((layers, B, n_q, 1, d), w["seed"] + 11, DEV)
    kn = synth.normal_bf16((layers, B, n_kv, 1, d), w["seed"] + 12, DEV)
    vn = synth.normal_bf16((layers, B, n_kv, 1, d), w["seed"] + 13, DEV)
    sb = np.array([0, 17, 63])
    kc_s, vc_s = synth.bits(kc[sb]), synth.bits(vc[sb])
    pl = past_dev(past)
    maxp = int(past.max())
    ws = torch.zeros(gq.gqa_decode_workspace_bytes(B, n_q, n_kv, d, S), dtype=torch.uint8, device=DEV)
    q_rot = torch.empty((B, n_q, 1, d), dtype=torch.bfloat16, device=DEV)
    outs = {}
    for c in range(layers):
        gq.gqa_rope_append(q[c], kn[c], vn[c], kc, vc, pl, maxp, w["theta"], "interleaved", w["scaling"],
                           q_rot=q_rot)
        out = gq.gqa_decode_attn(q_rot, kc, vc, pl, maxp, workspace=ws)
        if c in (0, layers - 1):
            outs[c] = synth.bits(out[sb])
    torch.cuda.synchronize()
    for c, got in outs.items():
        q_ref, kc_ref, vc_ref = rope_append(synth.bits(q[c][sb]), synth.bits(kn[c][sb]), synth.bits(vn[c][sb]),
                                            kc_s, vc_s, past[sb], w["theta"], "interleaved", w["scaling"])
        check_out(got, attend(q_ref, kc_ref, vc_ref, past[sb], n_kv), f"{name} call {c}")
        if c == layers - 1:  # the cache holds the last call's rows; every other row is as it started
            for i, b in enumerate(sb):
                p = int(past[b])
                assert max_ulp(synth.bits(kc[b, :, p]), kc_ref[i, :, p]) <= 1
                assert np.array_equal(synth.bits(vc[b, :, p]), vc_ref[i, :, p])
                assert np.array_equal(synth.bits(kc[b, :, :p]), kc_s[i, :, :p])
                assert np.array_equal(synth.bits(vc[b, :, :p]), vc_s[i, :, :p])
    assert int(ws[:256].count_nonzero()) == 0
    del kc, vc
    torch.cuda.empty_cache()


def test_full_size_chunked_prefill():
    w = synth.WORKLOADS["llama8b_chunked_prefill"]
    B, n_q, n_kv, T, d, S = w["B"], w["n_q"], w["n_kv"], w["T"], w["d"], w["S"]
    past = synth.past_lengths(B, w["past"], w["seed"])
    say(f"chunked prefill: B={B} T={T} P={past.tolist()}")
    seed = w["seed"]
    kc = synth.normal_bf16((B, n_kv, S, d), seed + 3, DEV)
    vc = synth.normal_bf16((B, n_kv, S, d), seed + 4, DEV)
    q = synth.normal_bf16((B, n_q, T, d), seed, DEV)
    kn = synth.normal_bf16((B, n_kv, T, d), seed + 1, DEV)
    vn = synth.normal_bf16((B, n_kv, T, d), seed + 2, DEV)
    synth.poison_beyond(kc, past, T)
    synth.poison_beyond(vc, past, T)
    sb = np.array([0, 3])
    kc_s, vc_s = synth.bits(kc[sb]), synth.bits(vc[sb])
    q_s, kn_s, vn_s = synth.bits(q[sb]), synth.bits(kn[sb]), synth.bits(vn[sb])
    pl = past_dev(past)
    q_rot = gq.gqa_rope_append(q, kn, vn, kc, vc, pl, int(past.max()), w["theta"])
    out = gq.gqa_prefill_attn(q_rot, kc, vc, pl, int(past.max()))
    torch.cuda.synchronize()
    q_ref, kc_ref, vc_ref = rope_append(q_s, kn_s, vn_s, kc_s, vc_s, past[sb], w["theta"])
    ref = attend(q_ref, kc_ref, vc_ref, past[sb], n_kv)
    check_out(synth.bits(out[sb]), ref, "chunked prefill")


# ---------------------------------------------------------------- sliding window, sinks, learned sinks

WINDOW_DECODE_CASES = [
    # B, n_q, n_kv, d, S, past, window, n_sink, learned sinks
    (4, 32, 8, 128, 3000, [2999, 0, 700, 1500], 256, 0, False),
    (4, 32, 8, 128, 3000, [2999, 0, 700, 1500], 100, 4, True),
    (4, 32, 8, 128, 3000, [2999, 10, 700, 1500], 1000, 130, False),  # sinks span three tiles
    (3, 64, 8, 128, 600, [511, 300, 599], 1, 0, False),              # one-row window, g = 8
    (2, 6, 2, 64, 300, [299, 77], 64, 64, True),                      # window meets the sinks
    (2, 6, 2, 64, 300, [299, 77], 5000, 0, True),                     # window wider than the context
]


@pytest.mark.parametrize("case", WINDOW_DECODE_CASES,
                         ids=lambda c: f"B{c[0]}q{c[1]}kv{c[2]}d{c[3]}W{c[6]}ns{c[7]}{'L' if c[8] else ''}")
def test_decode_window_and_sinks(case):
    B, n_q, n_kv, d, S, past, W, NS, learned = case
    say(f"decode window {case}")
    q, _, _, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=1100 + W)
    for b in range(B):  # row past_len is attended: make it finite
        kc[b, :, past[b]] = synth.bits(synth.normal_bf16((n_kv, d), 1200 + b))
        vc[b, :, past[b]] = synth.bits(synth.normal_bf16((n_kv, d), 1300 + b))
    sinks = np.random.default_rng(W + NS).standard_normal(n_q).astype(np.float32) if learned else None
    ref = attend(q, kc, vc, past, n_kv, window=W, n_sink=NS, sink_logits=sinks)
    say(f"  {poison_unread_tiles((kc, vc), past, W, NS)} unread rows NaN-filled")
    sk = torch.from_numpy(sinks).to(DEV) if learned else None
    for sched in ((-1, 0), (0, 1), (1000, 2)):
        gq.gqa_set_decode_schedule(*sched)
        try:
            out = gq.gqa_decode_attn(dev(q), dev(kc), dev(vc), past_dev(past), max(past), window=W, n_sink=NS,
                                     sink_logits=sk)
            torch.cuda.synchronize()
        finally:
            gq.gqa_set_decode_schedule()
        check_out(synth.bits(out), ref, f"decode window {W} sinks {NS} schedule {sched}")


WINDOW_PREFILL_CASES = [
    # B, n_q, n_kv, T, d, S, past, window, n_sink, learned sinks
    (2, 8, 2, 33, 128, 400, [20, 200], 50, 4, False),
    (2, 8, 2, 70, 128, 400, [0, 257], 64, 0, True),
    (1, 32, 8, 130, 128, 600, [300], 1, 0, False),
    (2, 6, 2, 40, 64, 300, [100, 3], 17, 70, True),
]


@pytest.mark.parametrize("case", WINDOW_PREFILL_CASES,
                         ids=lambda c: f"B{c[0]}q{c[1]}kv{c[2]}T{c[3]}d{c[4]}W{c[7]}ns{c[8]}{'L' if c[9] else ''}")
def test_prefill_window_and_sinks(case):
    B, n_q, n_kv, T, d, S, past, W, NS, learned = case
    say(f"prefill window {case}")
    q, _, _, kc, vc = make_inputs(B, n_q, n_kv, T, d, S, past, seed=1400 + W)
    sinks = np.random.default_rng(3 * W + NS).standard_normal(n_q).astype(np.float32) if learned else None
    ref = attend(q, kc, vc, past, n_kv, window=W, n_sink=NS, sink_logits=sinks)
    say(f"  {poison_unread_tiles((kc, vc), past, W, NS)} unread rows NaN-filled")
    sk = torch.from_numpy(sinks).to(DEV) if learned else None
    out = gq.gqa_prefill_attn(dev(q), dev(kc), dev(vc), past_dev(past), max(past), window=W, n_sink=NS,
                              sink_logits=sk)
    torch.cuda.synchronize()
    check_out(synth.bits(out), ref, f"prefill window {W} sinks {NS}")


# ---------------------------------------------------------------- single-launch decode step

STEP_CASES = [
    # B, n_q, n_kv, d, S, past, theta, layout, scaling, rotary_dim, window, n_sink, learned sinks
    (1, 6, 2, 64, 256, [255], 1.0e4, "interleaved", None, None, 0, 0, False),       # tiny 6/2-head window
    (1, 32, 8, 128, 8192, [1000], 5.0e5, "interleaved", None, None, 0, 0, False),   # one Llama-3.1-8B layer
    (4, 32, 8, 128, 300, [0, 63, 64, 299], 5.0e5, "interleaved", None, None, 0, 0, False),  # L = 1, tile edges
    (3, 64, 8, 128, 600, [511, 300, 599], 5.0e5, "interleaved", SCALED, None, 0, 0, False),  # g = 8, scaled
    (2, 8, 8, 128, 200, [150, 9], 5.0e5, "half", None, None, 0, 0, False),           # g = 1
    (2, 6, 1, 64, 300, [299, 77], 1.0e4, "interleaved", None, None, 0, 0, False),    # g = 6 (MQA)
    (2, 32, 1, 128, 400, [399, 5], 5.0e5, "interleaved", None, None, 0, 0, False),   # g = 32 (MQA)
    (1, 64, 1, 128, 200, [150], 5.0e5, "half", None, None, 0, 0, True),              # g = 64
    (3, 32, 8, 128, 3000, [2999, 10, 1500], 5.0e5, "interleaved", None, None, 256, 4, True),  # window + sinks
    (2, 32, 8, 128, 5000, [4999, 100], 1.0e4, "half", YARN16, 64, 0, 0, False),     # YaRN, partial rotary
    (2, 24, 2, 64, 2000, [1999, 1000], 1.0e4, "half", NTK8, None, 100, 70, False),  # g = 12, window meets sinks
]


def run_step(case, seed, ws=None, want_q_rot=True):
    B, n_q, n_kv, d, S, past, theta, layout, scaling, rdim, W, NS, learned = case
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed)
    for b in range(B):  # the row being appended: never read before it is written
        kc[b, :, past[b]] = synth.NAN_BF16
        vc[b, :, past[b]] = synth.NAN_BF16
    sinks = np.random.default_rng(seed).standard_normal(n_q).astype(np.float32) if learned else None
    q_ref, kc_ref, vc_ref = rope_append(q, kn, vn, kc, vc, past, theta, layout, scaling, rotary_dim=rdim)
    ref = attend(q_ref, kc_ref, vc_ref, past, n_kv, window=W, n_sink=NS, sink_logits=sinks)
    if poison_unread_tiles((kc, vc, kc_ref, vc_ref), past, W, NS):
        say("  unread window tiles NaN-filled")
    kc_d, vc_d, pl = dev(kc), dev(vc), past_dev(past)
    q_rot = torch.empty(B, n_q, 1, d, dtype=torch.bfloat16, device=DEV) if want_q_rot else None
    out = gq.gqa_decode_step(dev(q), dev(kn), dev(vn), kc_d, vc_d, pl, max(past), theta, layout, scaling, rdim,
                             q_rot=q_rot, workspace=ws, window=W, n_sink=NS,
                             sink_logits=torch.from_numpy(sinks).to(DEV) if learned else None)
    torch.cuda.synchronize()
    return out, ref, (q_rot, q_ref, kc_d, kc_ref, vc_d, vc_ref, kc)


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: f"B{c[0]}q{c[1]}kv{c[2]}d{c[3]}W{c[10]}"
                         f"{(c[8] or {}).get('type', 'plain') if c[8] else ''}")
def test_decode_step_parity(case):
    say(f"decode_step {case}")
    B, S, past = case[0], case[4], case[5]
    out, ref, (q_rot, q_ref, kc_d, kc_ref, vc_d, vc_ref, kc_in) = run_step(case, seed=900 + case[1] + case[3])
    check_out(synth.bits(out), ref, "decode_step")
    assert max_ulp(synth.bits(q_rot), q_ref) <= 1
    kc_g, vc_g = synth.bits(kc_d), synth.bits(vc_d)
    assert np.array_equal(vc_g, vc_ref), "value row appended bit for bit, nothing else touched"
    for b in range(B):
        other = np.ones(S, dtype=bool)
        other[past[b]] = False
        assert np.array_equal(kc_g[b][:, other], kc_in[b][:, other])
        assert max_ulp(kc_g[b][:, past[b]], kc_ref[b][:, past[b]]) <= 1


LARGE_STEP_CASES = [
    # tile bounds 8 x 8 x 32 = 2048 and 6 x 8 x 18 = 864 (window): past the split threshold of 512
    (8, 32, 8, 128, 2048, [2047, 0, 63, 64, 1000, 1500, 777, 2046], 5.0e5, "interleaved", SCALED, None, 0, 0, True),
    (6, 32, 8, 128, 3000, [2999, 10, 1500, 64, 2500, 999], 5.0e5, "half", None, None, 1000, 4, True),
]


@pytest.mark.parametrize("route", ["split", "single"])
@pytest.mark.parametrize("case", LARGE_STEP_CASES, ids=lambda c: f"B{c[0]}W{c[10]}")
def test_decode_step_large_batch_routes(case, route):
    """Batches past the tile threshold: by default the step runs as rope_append + split-K decode; with the
    threshold raised it stays one launch.  Both against the oracle doing its own RoPE and append."""
    say(f"decode_step large batch, route {route}, {case[:6]}")
    B, S, past = case[0], case[4], case[5]
    gq.gqa_set_decode_step_split_min_tiles(0 if route == "split" else 1 << 30)
    try:
        out, ref, (q_rot, q_ref, kc_d, kc_ref, vc_d, vc_ref, kc_in) = run_step(case, seed=2100 + B)
    finally:
        gq.gqa_set_decode_step_split_min_tiles(0)
    check_out(synth.bits(out), ref, f"decode_step {route}")
    assert max_ulp(synth.bits(q_rot), q_ref) <= 1
    assert np.array_equal(synth.bits(vc_d), vc_ref), "value row appended bit for bit, nothing else touched"
    kc_g = synth.bits(kc_d)
    for b in range(B):
        other = np.ones(S, dtype=bool)
        other[past[b]] = False
        assert np.array_equal(kc_g[b][:, other], kc_in[b][:, other])
        assert max_ulp(kc_g[b][:, past[b]], kc_ref[b][:, past[b]]) <= 1


def test_decode_step_split_route_repeatable():
    """The split route of the step (rope_append + split-K) gives bitwise identical results on a reused
    workspace and leaves its first 256 bytes zero."""
    case = LARGE_STEP_CASES[0]
    B, n_q, n_kv, d, S = case[0], case[1], case[2], case[3], case[4]
    ws = torch.zeros(gq.gqa_decode_step_workspace_bytes(B, n_q, n_kv, d, S), dtype=torch.uint8, device=DEV)
    out1, ref, _ = run_step(case, seed=2150, ws=ws, want_q_rot=False)
    assert int(ws[:256].view(torch.int32).abs().sum()) == 0
    out2, _, _ = run_step(case, seed=2150, ws=ws, want_q_rot=False)
    assert torch.equal(out1, out2), "repeated split-route step differs"
    check_out(synth.bits(out2), ref, "decode_step split route, second call")
    assert int(ws[:256].view(torch.int32).abs().sum()) == 0


def test_decode_step_workspace_serves_every_batch_size_and_route():
    """One workspace sized for the largest batch serves steps of several batch sizes through all routes in
    turn (split-K, single launch, forced either way; the rotated q returned or kept in the workspace); every
    call matches the oracle and leaves the first 256 bytes (single-launch counters, split-K ticket) zero."""
    n_q, n_kv, d, S = 32, 8, 128, 1200
    rng = np.random.default_rng(41)
    ws = torch.zeros(gq.gqa_decode_step_workspace_bytes(16, n_q, n_kv, d, S), dtype=torch.uint8, device=DEV)
    plan = [(16, 0), (2, 0), (16, 1 << 30), (8, 0), (2, 1), (16, 0), (8, 1 << 30)]
    try:
        for i, (B, thr) in enumerate(plan):
            past = [int(x) for x in rng.integers(0, S - 1, size=B)]
            case = (B, n_q, n_kv, d, S, past, 5.0e5, "interleaved", None, None, 0, 0, False)
            gq.gqa_set_decode_step_split_min_tiles(thr)
            say(f"  call {i}: B{B} threshold {gq.gqa_set_decode_step_split_min_tiles(thr)}")
            out, ref, _ = run_step(case, seed=2200 + i, ws=ws, want_q_rot=(i % 2 == 0))
            check_out(synth.bits(out), ref, f"decode_step call {i} B{B}")
            assert int(ws[:256].view(torch.int32).abs().sum()) == 0, "first 256 bytes must be zero after a call"
    finally:
        gq.gqa_set_decode_step_split_min_tiles(0)


def test_decode_step_repeat_calls_and_workspace_reuse():
    """Two calls on one workspace give identical bits, and the per-segment counters end at zero."""
    case = STEP_CASES[1]
    B, n_q, n_kv, d, S = case[0], case[1], case[2], case[3], case[4]
    ws = torch.zeros(gq.gqa_decode_step_workspace_bytes(B, n_q, n_kv, d, S), dtype=torch.uint8, device=DEV)
    out1, ref, _ = run_step(case, seed=5, ws=ws)
    assert int(ws[:256].view(torch.int32).abs().sum()) == 0
    out2, _, _ = run_step(case, seed=5, ws=ws)
    assert torch.equal(out1, out2)
    check_out(synth.bits(out2), ref, "decode_step second call")
    assert int(ws[:256].view(torch.int32).abs().sum()) == 0


def test_decode_step_matches_three_call_path():
    case = (2, 32, 8, 128, 3000, [2999, 1234], 5.0e5, "interleaved", SCALED)
    B, n_q, n_kv, d, S, past, theta, layout, scaling = case
    say("decode_step vs rope_append + decode_attn")
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=31)
    kc1, vc1, kc2, vc2, pl = dev(kc), dev(vc), dev(kc), dev(vc), past_dev(past)
    q_rot = gq.gqa_rope_append(dev(q), dev(kn), dev(vn), kc1, vc1, pl, max(past), theta, layout, scaling)
    o3 = gq.gqa_decode_attn(q_rot, kc1, vc1, pl, max(past))
    q_rot2 = torch.empty_like(q_rot)
    o1 = gq.gqa_decode_step(dev(q), dev(kn), dev(vn), kc2, vc2, pl, max(past), theta, layout, scaling, q_rot=q_rot2)
    torch.cuda.synchronize()
    assert torch.equal(q_rot, q_rot2)
    # bit patterns (the caches hold NaN poison beyond the appended row)
    assert np.array_equal(synth.bits(kc1), synth.bits(kc2)) and np.array_equal(synth.bits(vc1), synth.bits(vc2))
    diff = (o1.float() - o3.float()).abs().max().item()
    assert diff <= 2 ** -7, diff  # two orders of the same fp32 sums, each rounded once to bf16


def test_graph_replays_match_eager():
    """Both decode paths captured in a HIP graph: every replay equals the eager result bit for bit."""
    B, n_q, n_kv, d, S, past, theta = 2, 32, 8, 128, 2000, [1999, 700], 5.0e5
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=61)
    qd, knd, vnd, pl = dev(q), dev(kn), dev(vn), past_dev(past)
    kc1, vc1, kc2, vc2 = dev(kc), dev(vc), dev(kc), dev(vc)
    q_rot, o3, o1 = torch.empty_like(qd), torch.empty_like(qd), torch.empty_like(qd)
    ws3 = torch.zeros(gq.gqa_decode_workspace_bytes(B, n_q, n_kv, d, S), dtype=torch.uint8, device=DEV)
    ws1 = torch.zeros(gq.gqa_decode_step_workspace_bytes(B, n_q, n_kv, d, S), dtype=torch.uint8, device=DEV)

    def three():
        gq.gqa_rope_append(qd, knd, vnd, kc1, vc1, pl, max(past), theta, q_rot=q_rot)
        gq.gqa_decode_attn(q_rot, kc1, vc1, pl, max(past), out=o3, workspace=ws3)

    def one():
        gq.gqa_decode_step(qd, knd, vnd, kc2, vc2, pl, max(past), theta, out=o1, workspace=ws1)

    three()
    one()
    torch.cuda.synchronize()
    e3, e1 = o3.clone(), o1.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        three()
        one()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        three()
        one()
    for rep in range(3):
        o3.zero_()
        o1.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o3, e3) and torch.equal(o1, e1), f"replay {rep}"
        three()  # eager work between replays
        torch.cuda.synchronize()
    assert int(ws1[:256].view(torch.int32).abs().sum()) == 0 and int(ws3[:256].view(torch.int32).abs().sum()) == 0


# ---------------------------------------------------------------- wide query groups (g > 16, MQA)

WIDE_CASES = [
    # B, n_q, n_kv, d, S, past, theta, layout, scaling
    (2, 32, 1, 128, 600, [599, 0], 5.0e5, "interleaved", None),               # g = 32, L = 1
    (3, 64, 1, 128, 1100, [63, 64, 1099], 5.0e5, "interleaved", SCALED),      # g = 64, tile edges
    (2, 40, 1, 64, 300, [200, 5], 1.0e4, "half", None),                       # g = 40: padded head block
    (2, 34, 2, 128, 500, [499, 130], 5.0e5, "interleaved", None),             # g = 17
    (4, 48, 2, 64, 400, [399, 1, 64, 250], 1.0e4, "interleaved", None),       # g = 24
    (9, 256, 8, 128, 200, [199, 3, 64, 100, 150, 7, 63, 128, 77], 5.0e5, "interleaved", None),  # two launch slices
    (2, 16, 1, 128, 4200, [4100, 2100], 5.0e5, "interleaved", None),          # g = 16: 64 and 17 splits, so 64
    (2, 16, 1, 128, 1100, [1087, 500], 5.0e5, "half", None),                  # and 17 records per head merged
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: f"B{c[0]}q{c[1]}kv{c[2]}g{c[1]//c[2]}d{c[3]}")
def test_wide_group_decode(case):
    say(f"wide decode {case}")
    out, ref, _ = run_decode_e2e(case, seed=1500 + case[1])
    check_out(out, ref, "wide-group decode")


def test_wide_group_decode_window_sinks_and_paths():
    """Window, sinks and learned sinks on the wide kernel; it agrees with the split-K path; calls repeat bit for bit."""
    B, n_q, n_kv, d, S, past, W, NS = 2, 64, 1, 128, 3000, [2999, 1500], 256, 4
    say("wide decode window + paths")
    q, _, _, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=1601)
    for b in range(B):
        kc[b, :, past[b]] = synth.bits(synth.normal_bf16((n_kv, d), 1610 + b))
        vc[b, :, past[b]] = synth.bits(synth.normal_bf16((n_kv, d), 1620 + b))
    sinks = np.random.default_rng(3).standard_normal(n_q).astype(np.float32)
    sk = torch.from_numpy(sinks).to(DEV)
    ref = attend(q, kc, vc, past, n_kv, window=W, n_sink=NS, sink_logits=sinks)
    assert poison_unread_tiles((kc, vc), past, W, NS) > 0
    qd, kd, vd, pl = dev(q), dev(kc), dev(vc), past_dev(past)
    ws = torch.zeros(gq.gqa_decode_workspace_bytes(B, n_q, n_kv, d, S), dtype=torch.uint8, device=DEV)
    o1 = gq.gqa_decode_attn(qd, kd, vd, pl, max(past), workspace=ws, window=W, n_sink=NS, sink_logits=sk)
    o2 = gq.gqa_decode_attn(qd, kd, vd, pl, max(past), workspace=ws, window=W, n_sink=NS, sink_logits=sk)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert int(ws[:256].view(torch.int32).abs().sum()) == 0
    check_out(synth.bits(o1), ref, "wide-group decode under a window")
    gq.gqa_set_decode_wide_min_group(65)  # split-K path for the same call
    try:
        o3 = gq.gqa_decode_attn(qd, kd, vd, pl, max(past), workspace=ws, window=W, n_sink=NS, sink_logits=sk)
        torch.cuda.synchronize()
    finally:
        gq.gqa_set_decode_wide_min_group(0)
    check_out(synth.bits(o3), ref, "split-K decode, same shape")
    assert (o1.float() - o3.float()).abs().max().item() <= 2 ** -7


def test_wide_group_kernel_on_small_groups():
    """The wide kernel also serves g <= 16 when asked (padded head blocks)."""
    case = (3, 32, 8, 128, 700, [699, 64, 300], 5.0e5, "interleaved", None)
    say("wide kernel at g = 4")
    gq.gqa_set_decode_wide_min_group(2)
    try:
        out, ref, _ = run_decode_e2e(case, seed=1700)
    finally:
        gq.gqa_set_decode_wide_min_group(0)
    check_out(out, ref, "wide kernel, g = 4")


@pytest.mark.parametrize("case", [(2, 16, 1, 128, 300, [200, 1], 5.0e5, "interleaved", None),
                                  (2, 32, 1, 128, 600, [599, 70], 5.0e5, "half", None),
                                  (2, 64, 2, 64, 300, [299, 64], 1.0e4, "interleaved", SCALED)],
                         ids=lambda c: f"g{c[1]//c[2]}d{c[3]}")
def test_split_k_path_for_large_groups(case):
    """Groups of 16 and more default to the wide kernel; the split-K path (head chunks of 16) stays correct."""
    say(f"split-K for large groups {case}")
    gq.gqa_set_decode_wide_min_group(65)
    try:
        out, ref, _ = run_decode_e2e(case, seed=1800 + case[1])
    finally:
        gq.gqa_set_decode_wide_min_group(0)
    check_out(out, ref, "split-K, large group")


@pytest.mark.parametrize("thr", [65, 0], ids=["single_launch", "wide_route"])
def test_decode_step_large_group_both_routes(thr):
    """Large groups: the single-launch kernel (forced) and the rope_append + wide-kernel route agree with the oracle."""
    case = (2, 64, 1, 128, 900, [899, 130], 5.0e5, "half", NTK8, 64, 100, 4, True)
    say(f"decode_step large group, threshold {thr}")
    gq.gqa_set_decode_wide_min_group(thr)
    try:
        out, ref, (q_rot, q_ref, kc_d, kc_ref, vc_d, vc_ref, kc_in) = run_step(case, seed=1900)
    finally:
        gq.gqa_set_decode_wide_min_group(0)
    check_out(synth.bits(out), ref, "decode_step, large group")
    assert max_ulp(synth.bits(q_rot), q_ref) <= 1
    assert np.array_equal(synth.bits(vc_d), vc_ref)


# ---------------------------------------------------------------- launch slicing at the batch limits

def test_decode_batch_beyond_one_launch():
    """More sequences than one split-K launch takes (1024): the batch runs in slices."""
    B, n_q, n_kv, d, S = 2100, 8, 2, 64, 64
    past = [int(x) for x in np.random.default_rng(5).integers(0, S - 1, size=B)]
    say("decode B = 2100")
    q, _, _, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=2001)
    out = gq.gqa_decode_attn(dev(q), dev(kc), dev(vc), past_dev(past), max(past))
    torch.cuda.synchronize()
    got = synth.bits(out)
    pick = [0, 1, 2047, 2048, 2049, B - 1]
    ref = attend(q[pick], kc[pick], vc[pick], [past[i] for i in pick], n_kv)
    check_out(got[pick], ref, "decode, sliced batch")


def test_rope_and_prefill_batch_beyond_grid_limit():
    """More sequences than one grid dimension holds (65535): rope_append and prefill run in slices."""
    B, n_q, n_kv, T, d, S = 65537, 2, 1, 2, 64, 8
    past = [int(x) for x in np.random.default_rng(6).integers(0, S - T + 1, size=B)]
    say("rope_append + prefill B = 65537")
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, T, d, S, past, seed=2002)
    kc_d, vc_d, pl = dev(kc), dev(vc), past_dev(past)
    q_rot = gq.gqa_rope_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, pl, max(past), 1.0e4)
    out = gq.gqa_prefill_attn(q_rot, kc_d, vc_d, pl, max(past))
    torch.cuda.synchronize()
    pick = [0, 1, 65534, 65535, 65536]
    pp = [past[i] for i in pick]
    q_ref, kc_ref, vc_ref = rope_append(q[pick], kn[pick], vn[pick], kc[pick], vc[pick], pp, 1.0e4)
    assert max_ulp(synth.bits(q_rot)[pick], q_ref) <= 1
    kc_g = synth.bits(kc_d)[pick]
    for i, p in enumerate(pp):
        assert max_ulp(kc_g[i][:, p:p + T], kc_ref[i][:, p:p + T]) <= 1
    ref = attend(q_ref, kc_ref, vc_ref, pp, n_kv)
    check_out(synth.bits(out)[pick], ref, "prefill, sliced batch")


@pytest.mark.parametrize("case", [(2, 64, 1, 9, 128, 300, [120, 0], 5.0e5, "interleaved", None),
                                  (1, 32, 1, 70, 64, 400, [300], 1.0e4, "half", None),
                                  (2, 48, 2, 5, 128, 200, [64, 190], 5.0e5, "interleaved", SCALED)],
                         ids=lambda c: f"B{c[0]}q{c[1]}kv{c[2]}T{c[3]}d{c[4]}")
def test_prefill_wide_groups(case):
    """Prefill with many query heads per KV head (MQA and g = 24, 32): few positions per workgroup."""
    B, n_q, n_kv, T, d, S, past, theta, layout, scaling = case
    say(f"prefill wide group {case}")
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, T, d, S, past, seed=2100 + n_q)
    q_ref, kc_ref, vc_ref = rope_append(q, kn, vn, kc, vc, past, theta, layout, scaling)
    ref = attend(q_ref, kc_ref, vc_ref, past, n_kv)
    kc_d, vc_d, pl = dev(kc), dev(vc), past_dev(past)
    q_rot = gq.gqa_rope_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, pl, max(past), theta, layout, scaling)
    out = gq.gqa_prefill_attn(q_rot, kc_d, vc_d, pl, max(past))
    torch.cuda.synchronize()
    check_out(synth.bits(out), ref, "prefill, wide group")


def test_wide_group_decode_g16_window_learned_sinks():
    """The one-head-block path (g = 16: 16 rows per wave, row groups merged in the workgroup) under a window
    with sinks and learned sink logits; tiles no query sees hold NaN."""
    B, n_q, n_kv, d, S, past, W, NS = 3, 32, 2, 128, 3000, [2999, 700, 40], 300, 4
    say("wide decode g16 window")
    q, _, _, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=2301)
    sinks = np.random.default_rng(11).standard_normal(n_q).astype(np.float32)
    ref = attend(q, kc, vc, past, n_kv, window=W, n_sink=NS, sink_logits=sinks)
    assert poison_unread_tiles((kc, vc), past, W, NS) > 0
    out = gq.gqa_decode_attn(dev(q), dev(kc), dev(vc), past_dev(past), max(past), window=W, n_sink=NS,
                             sink_logits=torch.from_numpy(sinks).to(DEV))
    torch.cuda.synchronize()
    check_out(synth.bits(out), ref, "wide decode, g 16, window")


def test_wide_group_decode_d64_window():
    B, n_q, n_kv, d, S, past, W, NS = 3, 32, 1, 64, 2000, [1999, 40, 1000], 300, 2
    say("wide decode d64 window")
    q, _, _, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=2201)
    sinks = np.random.default_rng(7).standard_normal(n_q).astype(np.float32)
    ref = attend(q, kc, vc, past, n_kv, window=W, n_sink=NS, sink_logits=sinks)
    assert poison_unread_tiles((kc, vc), past, W, NS) > 0
    out = gq.gqa_decode_attn(dev(q), dev(kc), dev(vc), past_dev(past), max(past), window=W, n_sink=NS,
                             sink_logits=torch.from_numpy(sinks).to(DEV))
    torch.cuda.synchronize()
    check_out(synth.bits(out), ref, "wide decode, d 64, window")
