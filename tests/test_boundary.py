"""The C ABI library loads, exports what include/gqa.h declares, and rejects bad
arguments on the host before any HIP call (CPU only, no device needed)."""

import ctypes
import os
import re

import pytest

import gqa_attention_rope_amd as gq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(gq.LIB_PATH), reason="libgqa.so not built")

FAKE = 0x10000  # aligned, never dereferenced on the host
P = ctypes.c_void_p


def header_functions():
    text = open(os.path.join(ROOT, "include", "gqa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = gq.lib()
    names = header_functions()
    assert set(names) == set(gq.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


def rope(theta=5.0e5, layout=0, scaled=0, factor=8.0, low=1.0, high=4.0, orig=8192.0, rdim=0, attn=0.0):
    p = gq.GqaRopeParams()
    p.theta, p.layout, p.scaling = theta, layout, scaled
    p.rotary_dim, p.attn_factor = rdim, attn
    p.factor, p.low_freq_factor, p.high_freq_factor, p.original_max_pos = factor, low, high, orig
    return p


def append(**kw):
    a = dict(q=FAKE, q_rot=FAKE, k_new=FAKE, v_new=FAKE, kc=FAKE, vc=FAKE, pl=FAKE, maxp=10, B=2, n_q=8, n_kv=2,
             T=1, d=128, S=64, rope=rope())
    a.update(kw)
    r = a["rope"]
    return gq.lib().gqa_rope_append(P(a["q"]), P(a["q_rot"]), P(a["k_new"]), P(a["v_new"]), P(a["kc"]), P(a["vc"]),
                                    P(a["pl"]), a["maxp"], a["B"], a["n_q"], a["n_kv"], a["T"], a["d"], a["S"],
                                    None if r is None else ctypes.byref(r), None)


def decode(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, pl=FAKE, maxp=10, out=FAKE, ws=FAKE, wsb=1 << 40, B=2, n_q=8, n_kv=2, d=128,
             S=64, scale=0.0)
    a.update(kw)
    return gq.lib().gqa_decode_attn(P(a["q"]), P(a["kc"]), P(a["vc"]), P(a["pl"]), a["maxp"], P(a["out"]),
                                    P(a["ws"]), a["wsb"], a["B"], a["n_q"], a["n_kv"], a["d"], a["S"], a["scale"],
                                    None)


def prefill(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, pl=FAKE, maxp=10, out=FAKE, B=2, n_q=8, n_kv=2, T=4, d=128, S=64, scale=0.0)
    a.update(kw)
    return gq.lib().gqa_prefill_attn(P(a["q"]), P(a["kc"]), P(a["vc"]), P(a["pl"]), a["maxp"], P(a["out"]), a["B"],
                                     a["n_q"], a["n_kv"], a["T"], a["d"], a["S"], a["scale"], None)


INV, GRP, HD, RNG, WS, HIP = (gq.GQA_ERR_INVALID_ARG, gq.GQA_ERR_GROUP, gq.GQA_ERR_HEAD_DIM, gq.GQA_ERR_RANGE,
                              gq.GQA_ERR_WORKSPACE, gq.GQA_ERR_HIP)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), INV), (dict(kc=0), INV), (dict(pl=0), INV), (dict(rope=None), INV), (dict(q_rot=FAKE + 8), INV),
    (dict(B=0), INV), (dict(n_q=-1), INV), (dict(T=0), INV), (dict(S=0), INV), (dict(d=127), INV),
    (dict(n_q=6, n_kv=4), GRP), (dict(d=96), HD), (dict(d=256), HD),
    (dict(maxp=-1), RNG), (dict(maxp=64, T=1, S=64), RNG), (dict(maxp=60, T=5, S=64), RNG),
    (dict(rope=rope(theta=0.0)), INV), (dict(rope=rope(theta=float("nan"))), INV), (dict(rope=rope(layout=2)), INV),
    (dict(rope=rope(scaled=1, factor=0.0)), INV), (dict(rope=rope(scaled=1, low=4.0, high=1.0)), INV),
    (dict(rope=rope(scaled=1, orig=0.0)), INV),
    (dict(rope=rope(scaled=5)), INV), (dict(rope=rope(scaled=-1)), INV),
    (dict(rope=rope(scaled=2, factor=0.5)), INV), (dict(rope=rope(scaled=3, factor=0.9)), INV),
    (dict(rope=rope(scaled=4, factor=0.5)), INV), (dict(rope=rope(scaled=4, low=32.0, high=1.0)), INV),
    (dict(rope=rope(scaled=4, orig=-1.0)), INV), (dict(rope=rope(scaled=2, factor=float("inf"))), INV),
    (dict(rope=rope(rdim=8)), INV), (dict(rope=rope(rdim=24)), INV), (dict(rope=rope(rdim=144)), INV),
    (dict(d=64, rope=rope(rdim=80)), INV), (dict(rope=rope(rdim=-16)), INV),
    (dict(rope=rope(attn=-1.0)), INV), (dict(rope=rope(attn=float("nan"))), INV),
])
def test_rope_append_validation(kw, code):
    assert append(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), INV), (dict(out=0), INV), (dict(ws=0), INV), (dict(out=FAKE + 4), INV), (dict(pl=FAKE + 2), INV),
    (dict(B=0), INV), (dict(d=63), INV), (dict(n_q=8, n_kv=3), GRP), (dict(d=32), HD),
    (dict(maxp=64, S=64), RNG), (dict(maxp=-5), RNG), (dict(wsb=0), WS), (dict(scale=float("inf")), INV),
])
def test_decode_validation(kw, code):
    assert decode(**kw) == code


def test_decode_workspace_query():
    L = gq.lib()
    n = L.gqa_decode_workspace_bytes(32, 32, 8, 128, 8192)
    assert n > 0 and n % 16 == 0
    assert decode(wsb=L.gqa_decode_workspace_bytes(2, 8, 2, 128, 64) - 1) == WS
    assert L.gqa_decode_workspace_bytes(2, 8, 3, 128, 64) == 0
    assert L.gqa_decode_workspace_bytes(2, 8, 2, 96, 64) == 0
    # batches beyond one launch's slice reuse the workspace: size stops growing
    assert L.gqa_decode_workspace_bytes(4096, 32, 8, 128, 64) == L.gqa_decode_workspace_bytes(2048, 32, 8, 128, 64)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), INV), (dict(vc=FAKE + 1), INV), (dict(T=0), INV), (dict(n_q=8, n_kv=16), GRP), (dict(d=80), HD),
    (dict(maxp=61, T=4, S=64), RNG), (dict(scale=float("nan")), INV),
])
def test_prefill_validation(kw, code):
    assert prefill(**kw) == code


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, -6, -99):
        assert isinstance(gq.gqa_status_string(s), str) and gq.gqa_status_string(s)
    assert "multiple" in gq.gqa_status_string(gq.GQA_ERR_GROUP)


def test_valid_call_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    assert append() == HIP
    # every scaling rule with valid fields, partial rotary, an explicit attention factor
    for r in (rope(scaled=1), rope(scaled=2, factor=4.0), rope(scaled=3, factor=8.0), rope(scaled=4, high=32.0),
              rope(rdim=16), rope(rdim=112, layout=1), rope(attn=1.2), rope(scaled=2, factor=1.0, low=0.0)):
        assert append(rope=r) == HIP
    assert append(d=64, rope=rope(rdim=64)) == HIP
    assert decode() == HIP
    assert prefill() == HIP
    assert gq.gqa_status_string(HIP)


def test_python_binding_validates_before_calling():
    import torch
    with pytest.raises(ValueError):
        gq.gqa_decode_attn(torch.zeros(1, 2, 2, 64, dtype=torch.bfloat16), torch.zeros(1, 1, 8, 64),
                           torch.zeros(1, 1, 8, 64), torch.zeros(1, dtype=torch.int32), 3)
    with pytest.raises(ValueError):
        gq.gqa_prefill_attn(torch.zeros(1, 2, 2, 64, dtype=torch.float32), torch.zeros(1, 1, 8, 64),
                            torch.zeros(1, 1, 8, 64), torch.zeros(1, dtype=torch.int32), 3)


def test_decode_workgroup_override_clamps():
    assert gq.gqa_set_decode_workgroups(-3) == 0
    assert gq.gqa_set_decode_workgroups(10 ** 6) > 0
    assert gq.gqa_set_decode_workgroups(0) == 0


def test_decode_slot_ratio_clamps():
    assert gq.gqa_set_decode_slot_ratio(0) == 0  # per-variant defaults
    assert gq.gqa_set_decode_slot_ratio(1000) == 1000
    assert gq.gqa_set_decode_slot_ratio(10) == 250
    assert gq.gqa_set_decode_slot_ratio(10 ** 6) == 8000
    assert gq.gqa_set_decode_slot_ratio(-1) == 0


def test_decode_schedule_override_validates():
    assert gq.gqa_set_decode_schedule(700, 2) is None
    assert gq.gqa_set_decode_schedule(0, 1) is None
    assert gq.gqa_set_decode_schedule(1000, 64) is None
    for bad in ((1001, 2), (-5, 2), (500, 0), (500, -1)):
        with pytest.raises(ValueError):
            gq.gqa_set_decode_schedule(*bad)
    gq.gqa_set_decode_schedule()  # defaults


def opts(window=0, n_sink=0, sink=None):
    return gq.GqaAttnOpts(window, n_sink, sink)


def decode_ex(o, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, pl=FAKE, maxp=10, out=FAKE, ws=FAKE, wsb=1 << 40, B=2, n_q=8, n_kv=2, d=128,
             S=64, scale=0.0)
    a.update(kw)
    return gq.lib().gqa_decode_attn_ex(P(a["q"]), P(a["kc"]), P(a["vc"]), P(a["pl"]), a["maxp"], P(a["out"]),
                                       P(a["ws"]), a["wsb"], a["B"], a["n_q"], a["n_kv"], a["d"], a["S"], a["scale"],
                                       None if o is None else ctypes.byref(o), None)


def prefill_ex(o, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, pl=FAKE, maxp=10, out=FAKE, B=2, n_q=8, n_kv=2, T=4, d=128, S=64, scale=0.0)
    a.update(kw)
    return gq.lib().gqa_prefill_attn_ex(P(a["q"]), P(a["kc"]), P(a["vc"]), P(a["pl"]), a["maxp"], P(a["out"]),
                                        a["B"], a["n_q"], a["n_kv"], a["T"], a["d"], a["S"], a["scale"],
                                        None if o is None else ctypes.byref(o), None)


@pytest.mark.parametrize("o", [opts(window=-1), opts(n_sink=-3), opts(window=8, sink=FAKE + 2)])
def test_attention_options_validation(o):
    assert decode_ex(o) == INV
    assert prefill_ex(o) == INV


def test_attention_options_shape_checks_still_apply():
    o = opts(window=16, n_sink=4, sink=FAKE)
    assert decode_ex(o, n_q=8, n_kv=3) == GRP
    assert prefill_ex(o, d=80) == HD
    assert decode_ex(o, q=0) == INV


def test_attention_options_accepted_without_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    for o in (None, opts(), opts(window=16, n_sink=4), opts(window=1, sink=FAKE)):
        assert decode_ex(o) == HIP
        assert prefill_ex(o) == HIP


def test_python_binding_validates_attention_options():
    import torch
    assert gq._opts(0, 0, None, 8, "cpu") == (None, None)
    o, _ = gq._opts(64, 4, None, 8, "cpu")
    assert (o.window, o.n_sink, o.sink_logits) == (64, 4, None)
    sk = torch.zeros(8)
    o, keep = gq._opts(0, 0, sk, 8, "cpu")
    assert o.sink_logits == sk.data_ptr() and keep is sk
    for bad in (dict(window=-1), dict(n_sink=-1), dict(window=0, n_sink=-2),
                dict(sink_logits=torch.zeros(3)),                        # one logit per query head
                dict(sink_logits=torch.zeros(8, dtype=torch.float64)),   # float32 only
                dict(sink_logits=torch.zeros(16)[::2])):                 # contiguous only
        a = dict(window=16, n_sink=0, sink_logits=None)
        a.update(bad)
        with pytest.raises(ValueError):
            gq._opts(a["window"], a["n_sink"], a["sink_logits"], 8, "cpu")


def step(o=None, **kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, pl=FAKE, maxp=10, out=FAKE, q_rot=None, ws=FAKE,
             wsb=1 << 40, B=2, n_q=8, n_kv=2, d=128, S=64, rope=rope(), scale=0.0)
    a.update(kw)
    r = a["rope"]
    return gq.lib().gqa_decode_step(P(a["q"]), P(a["kn"]), P(a["vn"]), P(a["kc"]), P(a["vc"]), P(a["pl"]), a["maxp"],
                                    P(a["out"]), P(a["q_rot"]), P(a["ws"]), a["wsb"], a["B"], a["n_q"], a["n_kv"],
                                    a["d"], a["S"], None if r is None else ctypes.byref(r), a["scale"],
                                    None if o is None else ctypes.byref(o), None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), INV), (dict(kn=0), INV), (dict(ws=0), INV), (dict(rope=None), INV), (dict(out=FAKE + 8), INV),
    (dict(q_rot=FAKE + 4), INV), (dict(pl=FAKE + 1), INV), (dict(B=0), INV), (dict(n_q=8, n_kv=3), GRP),
    (dict(d=96), HD), (dict(maxp=64, S=64), RNG), (dict(maxp=-1), RNG), (dict(wsb=0), WS),
    (dict(n_q=130, n_kv=2), INV), (dict(scale=float("nan")), INV), (dict(rope=rope(rdim=24)), INV),
    (dict(rope=rope(scaled=4, factor=0.5)), INV), (dict(S=1 << 23, maxp=10), INV),
    (dict(B=65536), INV), (dict(n_q=65536 * 2, n_kv=65536), INV),
])
def test_decode_step_validation(kw, code):
    assert step(**kw) == code


def test_decode_step_options_and_workspace_query():
    assert step(opts(window=-1)) == INV
    assert step(opts(n_sink=-1)) == INV
    assert step(opts(window=4, sink=FAKE + 2)) == INV
    L = gq.lib()
    n = L.gqa_decode_step_workspace_bytes(2, 8, 2, 128, 64)
    assert n > 0 and n % 16 == 0
    assert step(wsb=n - 1) == WS
    assert L.gqa_decode_step_workspace_bytes(2, 8, 3, 128, 64) == 0
    assert L.gqa_decode_step_workspace_bytes(1, 130, 2, 128, 64) == 0
    assert L.gqa_decode_step_workspace_bytes(2, 128, 2, 128, 64) > 0  # g = 64, the largest group
    import torch
    if not torch.cuda.is_available():
        assert step() == HIP
        assert step(opts(window=16, n_sink=4, sink=FAKE), q_rot=FAKE) == HIP


def test_every_entry_point_checks_the_slab_size():
    """S * d * 2 must stay below 2^31: the kernels address one KV head's slab with 32-bit offsets."""
    big = dict(S=1 << 23, maxp=10)
    assert decode(**big) == INV
    assert prefill(**big) == INV
    assert append(**big) == INV
    assert step(**big) == INV


def test_wide_group_override():
    assert gq.gqa_set_decode_wide_min_group(40) == 40
    assert gq.gqa_set_decode_wide_min_group(0) == 16
    L = gq.lib()
    # the decode workspace also covers the wide-group kernel for MQA shapes
    assert L.gqa_decode_workspace_bytes(16, 64, 1, 128, 8192) >= 256 + 16 * 32 * 64 * 132 * 4


# ---------------------------------------------------------------- no-allocation decode (host-side checks)

def decode_noalloc(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, pl=FAKE, maxp=10, out=FAKE, B=2, n_q=8, n_kv=2, d=128, S=64, scale=0.0)
    a.update(kw)
    return gq.lib().gqa_decode_attn_noalloc(P(a["q"]), P(a["kc"]), P(a["vc"]), P(a["pl"]), a["maxp"], P(a["out"]),
                                            a["B"], a["n_q"], a["n_kv"], a["d"], a["S"], a["scale"], None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), INV), (dict(out=0), INV), (dict(pl=FAKE + 2), INV), (dict(out=FAKE + 8), INV), (dict(B=0), INV),
    (dict(scale=float("nan")), INV), (dict(n_q=6, n_kv=4), GRP), (dict(d=96), HD), (dict(maxp=64), RNG),
    # 1024 sequences of 64/16 heads: 90 MiB of split-K records per launch, beyond the fixed 64 MiB buffer
    (dict(B=1024, n_q=64, n_kv=16, S=8192, maxp=100), gq.GQA_ERR_SCRATCH),
])
def test_decode_noalloc_rejects_on_host(kw, code):
    assert decode_noalloc(**kw) == code
    assert gq.gqa_status_string(code)


def test_decode_noalloc_sizes_within_its_buffer():
    # the headline and long-context shapes fit the fixed buffer; the check uses the path's own record bytes
    assert gq.gqa_decode_workspace_bytes(32, 32, 8, 128, 8192) <= gq.GQA_DECODE_NOALLOC_MAX_BYTES
    assert gq.gqa_decode_workspace_bytes(64, 64, 8, 128, 8192) <= gq.GQA_DECODE_NOALLOC_MAX_BYTES
    assert "no-allocation" in gq.gqa_status_string(gq.GQA_ERR_SCRATCH)


def test_decode_noalloc_without_device_is_a_hip_error():
    # a valid call reaches the device lookup, which fails cleanly here (no GPU in this container)
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert decode_noalloc() == HIP


def test_measure_mfma_rate_checks_on_host():
    L = gq.lib()
    sink = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host checks
    assert L.gqa_measure_mfma_rate(0, 10, sink, None) == INV
    assert L.gqa_measure_mfma_rate(65536, 10, sink, None) == INV
    assert L.gqa_measure_mfma_rate(8, 0, sink, None) == INV
    assert L.gqa_measure_mfma_rate(8, (1 << 24) + 1, sink, None) == INV
    assert L.gqa_measure_mfma_rate(8, 10, None, None) == INV
    assert L.gqa_measure_mfma_rate(8, 10, ctypes.c_void_p(0x1004), None) == INV  # not 8-byte aligned


def test_measure_mfma_rate_without_device_is_a_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert gq.lib().gqa_measure_mfma_rate(8, 10, ctypes.c_void_p(0x1000), None) == HIP
