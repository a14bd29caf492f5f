"""GPU contracts beyond the values: every output and workspace write stays inside its buffer, calls on a
side stream see their default temporaries ready, and rows that a window hides contribute nothing.

Guard bands: each output (out, q_rot) and each workspace is carved out of a larger buffer whose extra
bytes on both sides hold a sentinel pattern no kernel writes.  After the call every sentinel must be
intact, including where a batch runs as several launches (beyond 2048 decode sequences, beyond the
65535-sequence grid limit of rope_append and prefill).  Values are checked against the fp64 oracle too.
"""

import sys

import numpy as np
import pytest
import torch

import gqa_attention_rope_amd as gq
from gqa_attention_rope_amd import synth
from oracle import attend, bf16_to_f64, rope_append

pytestmark = pytest.mark.gpu

DEV = "cuda"
GUARD = 4096            # elements (bf16) or bytes (workspace) of guard on each side; keeps 16-byte alignment
SENT_BF16 = 0x7FA5      # a NaN pattern: no kernel writes it (kernels write finite values or 0x7FC0)
SENT_BYTE = 0xA5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def half_ulp_bf16(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def check_out(gpu_bits, ref, name):
    g = bf16_to_f64(gpu_bits)
    assert np.all(np.isfinite(g)), f"{name}: non-finite outputs"
    err = np.abs(g - ref)
    rel = err / np.maximum(np.abs(ref), 1e-2)
    bad = (err > 1e-2 + half_ulp_bf16(ref)) | (rel > 1e-2)
    say(f"  {name}: max abs {err.max():.3e}  max rel {rel.max():.3e}  n={err.size}")
    assert not bad.any(), f"{name}: {int(bad.sum())} of {bad.size} outside the tolerance"


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
    for b in range(B):
        kc[b, :, past[b] + T:] = synth.NAN_BF16
        vc[b, :, past[b] + T:] = synth.NAN_BF16
    return q, kn, vn, kc, vc


class Guarded:
    """A bf16 tensor of ``shape`` (or a zeroed byte workspace of ``nbytes``) inside sentinel bands."""

    def __init__(self, shape=None, nbytes=None):
        if nbytes is None:
            self.n = int(np.prod(shape))
            self.big = torch.full((self.n + 2 * GUARD,), SENT_BF16, dtype=torch.int16, device=DEV)
            self.view = self.big[GUARD:GUARD + self.n].view(torch.bfloat16).view(shape)
        else:
            self.n = int(nbytes)
            self.big = torch.full((self.n + 2 * GUARD,), SENT_BYTE, dtype=torch.uint8, device=DEV)
            self.big[GUARD:GUARD + self.n] = 0
            self.view = self.big[GUARD:GUARD + self.n]
        assert self.view.data_ptr() % 16 == 0

    def intact(self):
        h = self.big.cpu().numpy()
        sent = np.uint16(SENT_BF16).view(np.int16) if h.dtype == np.int16 else np.uint8(SENT_BYTE)
        lo, hi = h[:GUARD], h[GUARD + self.n:]
        return bool(np.all(lo == sent) and np.all(hi == sent))


DECODE_GUARD_CASES = [
    # B, n_q, n_kv, d, S, past, window, n_sink
    (5, 32, 8, 128, 1100, [0, 63, 64, 65, 1098], 0, 0),   # split-K, tile edges
    (3, 64, 8, 64, 700, [699, 5, 300], 100, 4),           # split-K, g = 8, window + sinks
    (3, 64, 2, 128, 900, [899, 1, 450], 0, 0),            # wide-group kernel (g = 32)
    (2, 64, 1, 64, 500, [499, 70], 0, 0),                 # wide-group kernel, MQA
]


@pytest.mark.parametrize("case", DECODE_GUARD_CASES, ids=lambda c: f"B{c[0]}q{c[1]}kv{c[2]}d{c[3]}W{c[6]}")
def test_decode_writes_stay_inside_out_and_workspace(case):
    B, n_q, n_kv, d, S, past, W, NS = case
    say(f"decode guard bands {case}")
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=3100 + n_q + d)
    q_ref, kc_ref, vc_ref = rope_append(q, kn, vn, kc, vc, past, 5.0e5)
    ref = attend(q_ref, kc_ref, vc_ref, past, n_kv, window=W, n_sink=NS)
    kc_d, vc_d, pl = dev(kc), dev(vc), past_dev(past)
    qr = Guarded((B, n_q, 1, d))
    out = Guarded((B, n_q, 1, d))
    ws = Guarded(nbytes=gq.gqa_decode_workspace_bytes(B, n_q, n_kv, d, S))
    gq.gqa_rope_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, pl, max(past), 5.0e5, q_rot=qr.view)
    gq.gqa_decode_attn(qr.view, kc_d, vc_d, pl, max(past), out=out.view, workspace=ws.view, window=W, n_sink=NS)
    torch.cuda.synchronize()
    assert qr.intact(), "rope_append wrote outside q_rot"
    assert out.intact(), "decode wrote outside out"
    assert ws.intact(), "decode wrote outside its workspace"
    check_out(synth.bits(out.view), ref, "decode (guarded)")


@pytest.mark.parametrize("case", [(2, 8, 2, 70, 128, 400, [0, 257], 0, 0), (2, 6, 2, 40, 64, 300, [100, 3], 17, 70),
                                  (1, 64, 1, 9, 128, 300, [120], 0, 0)],
                         ids=lambda c: f"B{c[0]}q{c[1]}kv{c[2]}T{c[3]}d{c[4]}W{c[7]}")
def test_prefill_writes_stay_inside_out(case):
    B, n_q, n_kv, T, d, S, past, W, NS = case
    say(f"prefill guard bands {case}")
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, T, d, S, past, seed=3200 + T)
    q_ref, kc_ref, vc_ref = rope_append(q, kn, vn, kc, vc, past, 1.0e4)
    ref = attend(q_ref, kc_ref, vc_ref, past, n_kv, window=W, n_sink=NS)
    kc_d, vc_d, pl = dev(kc), dev(vc), past_dev(past)
    qr = Guarded((B, n_q, T, d))
    out = Guarded((B, n_q, T, d))
    gq.gqa_rope_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, pl, max(past), 1.0e4, q_rot=qr.view)
    gq.gqa_prefill_attn(qr.view, kc_d, vc_d, pl, max(past), out=out.view, window=W, n_sink=NS)
    torch.cuda.synchronize()
    assert qr.intact() and out.intact(), "write outside q_rot or out"
    check_out(synth.bits(out.view), ref, "prefill (guarded)")


@pytest.mark.parametrize("case", [(3, 32, 8, 128, 600, [599, 0, 300]), (2, 32, 1, 128, 400, [399, 5]),
                                  (1, 6, 2, 64, 256, [255])],
                         ids=lambda c: f"B{c[0]}q{c[1]}kv{c[2]}d{c[3]}")
def test_decode_step_writes_stay_inside_its_buffers(case):
    B, n_q, n_kv, d, S, past = case
    say(f"decode step guard bands {case}")
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=3300 + n_q)
    q_ref, kc_ref, vc_ref = rope_append(q, kn, vn, kc, vc, past, 5.0e5)
    ref = attend(q_ref, kc_ref, vc_ref, past, n_kv)
    kc_d, vc_d, pl = dev(kc), dev(vc), past_dev(past)
    qr = Guarded((B, n_q, 1, d))
    out = Guarded((B, n_q, 1, d))
    ws = Guarded(nbytes=gq.gqa_decode_step_workspace_bytes(B, n_q, n_kv, d, S))
    for _ in range(2):  # the second call reuses the workspace the first one left
        gq.gqa_decode_step(dev(q), dev(kn), dev(vn), kc_d, vc_d, pl, max(past), 5.0e5, out=out.view, q_rot=qr.view,
                           workspace=ws.view)
    torch.cuda.synchronize()
    assert qr.intact() and out.intact() and ws.intact(), "write outside q_rot, out or the workspace"
    check_out(synth.bits(out.view), ref, "decode step (guarded)")


def test_sliced_batches_write_inside_their_buffers():
    """Decode beyond one launch (1024 sequences) and rope_append + prefill beyond the grid limit (65535)."""
    B, n_q, n_kv, d, S = 2100, 8, 2, 64, 64
    past = [int(x) for x in np.random.default_rng(15).integers(0, S - 1, size=B)]
    say("guard bands: decode B = 2100")
    q, _, _, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=3401)
    out = Guarded((B, n_q, 1, d))
    ws = Guarded(nbytes=gq.gqa_decode_workspace_bytes(B, n_q, n_kv, d, S))
    gq.gqa_decode_attn(dev(q), dev(kc), dev(vc), past_dev(past), max(past), out=out.view, workspace=ws.view)
    torch.cuda.synchronize()
    assert out.intact() and ws.intact(), "sliced decode wrote outside out or the workspace"
    pick = [0, 2047, 2048, B - 1]
    check_out(synth.bits(out.view)[pick], attend(q[pick], kc[pick], vc[pick], [past[i] for i in pick], n_kv),
              "sliced decode (guarded)")

    B, n_q, n_kv, T, d, S = 65537, 2, 1, 2, 64, 8
    past = [int(x) for x in np.random.default_rng(16).integers(0, S - T + 1, size=B)]
    say("guard bands: rope_append + prefill B = 65537")
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, T, d, S, past, seed=3402)
    kc_d, vc_d, pl = dev(kc), dev(vc), past_dev(past)
    qr = Guarded((B, n_q, T, d))
    out = Guarded((B, n_q, T, d))
    gq.gqa_rope_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, pl, max(past), 1.0e4, q_rot=qr.view)
    gq.gqa_prefill_attn(qr.view, kc_d, vc_d, pl, max(past), out=out.view)
    torch.cuda.synchronize()
    assert qr.intact() and out.intact(), "sliced rope_append or prefill wrote outside its output"
    pick = [0, 65535, 65536]
    pp = [past[i] for i in pick]
    q_ref, kc_ref, vc_ref = rope_append(q[pick], kn[pick], vn[pick], kc[pick], vc[pick], pp, 1.0e4)
    check_out(synth.bits(out.view)[pick], attend(q_ref, kc_ref, vc_ref, pp, n_kv), "sliced prefill (guarded)")


# ---------------------------------------------------------------- explicit streams

def test_default_temporaries_on_a_side_stream():
    """Decode and the decode step on an explicit side stream, with the binding's default workspace and
    outputs, while the current stream is still busy: the temporaries are made on the side stream, so the
    kernels see a zeroed workspace header even when the allocator hands back a block that held junk."""
    B, n_q, n_kv, d, S, past = 4, 32, 8, 128, 2048, [2047, 3, 1000, 1500]
    say("side-stream decode with default temporaries")
    q, kn, vn, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=3500)
    q_ref, kc_ref, vc_ref = rope_append(q, kn, vn, kc, vc, past, 5.0e5)
    ref = attend(q_ref, kc_ref, vc_ref, past, n_kv)
    kc_d, vc_d, pl = dev(kc), dev(vc), past_dev(past)
    q_rot = gq.gqa_rope_append(dev(q), dev(kn), dev(vn), kc_d, vc_d, pl, max(past), 5.0e5)
    expect = synth.bits(gq.gqa_decode_attn(q_rot, kc_d, vc_d, pl, max(past)))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for it in range(3):
        # junk in freed blocks of the workspace's size, then a long kernel on the current stream
        junk = torch.full((gq.gqa_decode_workspace_bytes(B, n_q, n_kv, d, S),), 0xFF, dtype=torch.uint8, device=DEV)
        del junk
        big = torch.randn(4096, 4096, device=DEV)
        busy = big @ big
        out = gq.gqa_decode_attn(q_rot, kc_d, vc_d, pl, max(past), stream=side)
        side.synchronize()
        got = synth.bits(out)
        torch.cuda.synchronize()
        del busy, big
        assert np.array_equal(got, expect), f"side-stream decode differs (iteration {it})"
    check_out(expect, ref, "decode (current stream)")

    # the single-launch step on the side stream, default workspace, fresh caches each time
    for it in range(2):
        kc_s, vc_s = dev(kc), dev(vc)
        junk = torch.full((gq.gqa_decode_step_workspace_bytes(B, n_q, n_kv, d, S),), 0xFF, dtype=torch.uint8,
                          device=DEV)
        del junk
        torch.cuda.synchronize()
        big = torch.randn(4096, 4096, device=DEV)
        busy = big @ big
        out = gq.gqa_decode_step(dev(q), dev(kn), dev(vn), kc_s, vc_s, pl, max(past), 5.0e5, stream=side)
        side.synchronize()
        got = synth.bits(out)
        torch.cuda.synchronize()
        del busy, big
        check_out(got, ref, f"side-stream decode step (iteration {it})")


# ---------------------------------------------------------------- rows hidden by a window

def test_window_hidden_rows_contribute_nothing():
    """Rows between the sinks and the window start may share a 64-row tile with visible rows; whatever
    finite values they hold (here the largest bf16 magnitudes) must not change the output."""
    B, n_q, n_kv, d, S, past, W, NS = 3, 32, 8, 128, 2000, [1999, 700, 130], 100, 4
    say("window: extreme values in hidden rows")
    q, _, _, kc, vc = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=3600)
    for b in range(B):
        kc[b, :, past[b]] = synth.bits(synth.normal_bf16((n_kv, d), 3610 + b))
        vc[b, :, past[b]] = synth.bits(synth.normal_bf16((n_kv, d), 3620 + b))
    ref = attend(q, kc, vc, past, n_kv, window=W, n_sink=NS)
    big = np.uint16(0x7F7F)  # 3.39e38, the largest finite bf16
    kc2, vc2 = kc.copy(), vc.copy()
    for b in range(B):
        lo, hi = NS, past[b] - W + 1  # hidden rows [lo, hi)
        if hi > lo:
            kc2[b, :, lo:hi] = big
            vc2[b, :, lo:hi] = big ^ np.uint16(0x8000) if b % 2 else big
    assert np.array_equal(attend(q, kc2, vc2, past, n_kv, window=W, n_sink=NS), ref)
    for sched in ((-1, 0), (0, 1)):
        gq.gqa_set_decode_schedule(*sched)
        try:
            out = gq.gqa_decode_attn(dev(q), dev(kc2), dev(vc2), past_dev(past), max(past), window=W, n_sink=NS)
            torch.cuda.synchronize()
        finally:
            gq.gqa_set_decode_schedule()
        check_out(synth.bits(out), ref, f"decode window, extreme hidden rows, schedule {sched}")
    # the same through the wide-group kernel and the single-launch step's attention
    qw = synth.bits(synth.normal_bf16((B, 64, 1, d), 3630))
    kw, vw = kc2[:, :2].copy(), vc2[:, :2].copy()
    refw = attend(qw, kc[:, :2], vc[:, :2], past, 2, window=W, n_sink=NS)
    out = gq.gqa_decode_attn(dev(qw), dev(kw), dev(vw), past_dev(past), max(past), window=W, n_sink=NS)
    torch.cuda.synchronize()
    check_out(synth.bits(out), refw, "wide decode window, extreme hidden rows")

    # and through the single-launch step (rotation and append included)
    _, kn, vn, _, _ = make_inputs(B, n_q, n_kv, 1, d, S, past, seed=3640)
    q_ref, kc_ref, vc_ref = rope_append(q, kn, vn, kc, vc, past, 5.0e5)
    refs = attend(q_ref, kc_ref, vc_ref, past, n_kv, window=W, n_sink=NS)
    out = gq.gqa_decode_step(dev(q), dev(kn), dev(vn), dev(kc2), dev(vc2), past_dev(past), max(past), 5.0e5,
                             window=W, n_sink=NS)
    torch.cuda.synchronize()
    check_out(synth.bits(out), refs, "decode step window, extreme hidden rows")


# ---------------------------------------------------------------- measurement probe

def test_mfma_rate_probe_writes_its_sink_only():
    """The matrix-rate probe writes 8 words per workgroup and nothing past them: finite folded results, a
    positive clock count and 100 MHz tick count per workgroup, zeros in the two spare words."""
    wg, iters = 8, 64
    say("mfma rate probe")
    buf = torch.full((8 * wg + 64,), -1, dtype=torch.int64, device=DEV)
    gq.gqa_measure_mfma_rate(wg, iters, buf)
    torch.cuda.synchronize()
    w = buf.cpu().numpy()
    assert np.all(w[8 * wg:] == -1), "writes past the sink"
    w = w[:8 * wg].reshape(wg, 8)
    folded = w[:, :4].astype(np.uint32).view(np.float32)
    assert np.all(np.isfinite(folded))
    assert np.all(w[:, 4] > 0) and np.all(w[:, 5] > 0)
    assert np.all(w[:, 6:] == 0)
    mhz = w[:, 4].sum() / w[:, 5].sum() * 100.0
    say(f"  shader clock over the probe loop: {mhz:.0f} MHz")
    assert 100.0 < mhz < 5000.0
