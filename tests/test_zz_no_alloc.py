"""gqa_decode_attn_noalloc (the library's fixed per-GPU scratch instead of a workspace) against
gqa_decode_attn on the same inputs, called through the C ABI: bitwise equal outputs (same kernels and
launch shape), and both within the oracle's tolerance.  Three calls in a row share the one scratch
buffer; the later ones are smaller, so stale records of a larger call are present when they run.
"""

import ctypes
import sys

import numpy as np
import pytest
import torch

import gqa_attention_rope_amd as gq
from gqa_attention_rope_amd import synth
from oracle import attend, bf16_to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


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


# B, n_q, n_kv, d, S, past, seed: largest first, so each later call finds the scratch holding more records
CALLS = [
    (8, 32, 8, 128, 4096, [4095, 17, 2048, 900, 3001, 63, 64, 1500], 71),
    (4, 64, 2, 128, 1024, [1000, 5, 640, 129], 72),   # g = 32: the wide-group path
    (2, 6, 2, 64, 300, [255, 40], 73),
]


def one_call(B, n_q, n_kv, d, S, past, seed):
    say(f"noalloc decode B{B} {n_q}/{n_kv} d{d} S{S} past {past} seed {seed}")
    q = synth.bits(synth.normal_bf16((B, n_q, 1, d), seed))
    kc = synth.bits(synth.normal_bf16((B, n_kv, S, d), seed + 1))
    vc = synth.bits(synth.normal_bf16((B, n_kv, S, d), seed + 2))
    for b in range(B):  # rows the call must not read
        kc[b, :, past[b] + 1:] = synth.NAN_BF16
        vc[b, :, past[b] + 1:] = synth.NAN_BF16
    q_d, kc_d, vc_d = synth.from_bits(q, DEV), synth.from_bits(kc, DEV), synth.from_bits(vc, DEV)
    pl = torch.as_tensor(np.asarray(past, np.int32), device=DEV)
    pmax = max(past)
    ref_out = gq.gqa_decode_attn(q_d, kc_d, vc_d, pl, pmax)
    out = torch.empty_like(q_d)
    st = gq.lib().gqa_decode_attn_noalloc(ctypes.c_void_p(q_d.data_ptr()), ctypes.c_void_p(kc_d.data_ptr()),
                                          ctypes.c_void_p(vc_d.data_ptr()), ctypes.c_void_p(pl.data_ptr()), pmax,
                                          ctypes.c_void_p(out.data_ptr()), B, n_q, n_kv, d, S, 0.0, None,
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == gq.GQA_OK, gq.gqa_status_string(st)
    torch.cuda.synchronize()
    a, b = synth.bits(out), synth.bits(ref_out)
    assert np.array_equal(a, b), f"{int(np.sum(a != b))} outputs differ from gqa_decode_attn"
    check_out(a[:, :, 0], attend(q, kc, vc, np.asarray(past), n_kv)[:, :, 0], "noalloc vs oracle")


def test_noalloc_matches_decode_attn_on_consecutive_calls():
    for c in CALLS:
        one_call(*c)
    # the largest case again after the small ones: the header is cleared per call
    one_call(*CALLS[0])
