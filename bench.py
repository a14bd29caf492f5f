"""Benchmark of the GQA + RoPE KV-cache attention step on one MI355X.

A step is one decode step of a batch of 32 Llama-3.1-8B sequences through 32
layers: per layer, RoPE + cache append of the new token (gqa_rope_append),
then split-K decode attention over cache rows 0..past_len[b]
(gqa_decode_attn: the partials kernel and the combine kernel).  Contexts are
ragged, past_len ~ U[512, 8191] (seeded), caches [32, 8, 8192, 128] bf16 per
layer, 32 distinct layers (32 GiB).  All inputs are resident in HBM before
timing starts.

Printed: one JSON line.
  value = KV-read GB/s over the whole step (sum over layers and sequences of
    (past_len+1) * n_kv * d * 2 tensors * 2 B, divided by the step time);
    tokens/s = B / step time.
  decode_attention = the same KV bytes over the decode attention kernels
    alone (partials + combine per layer).
  roofline = decode attention (partials + combine): algorithmic bytes per
    layer (KV rows + q) over the two kernels' mean launch times, against
    8 TB/s; roofline.dominant_kernel = the partials kernel alone.  Launch times
    come from HIP events recorded on the launch stream around every launch
    (the library's timing hooks); the rocprofv3 kernel trace under profiles/
    gives the same figures from the profiler.  roofline.traffic = HBM bytes
    per layer from the committed rocprofv3 byte-counter summary (null once the
    decode kernel sources differ from the ones it was taken on).
  stream_read_ceiling = the library's read-only streaming kernel over a
    buffer of one layer's KV bytes (larger than the 256 MB MALL): the HBM read
    rate a plain kernel reaches on this machine.
  cpu_baseline = the fp64 oracle on a bounded sample of the same workload on
    this host, all cores and one core.

extra (skipped with --no-extra): chunked prefill TFLOP/s (B4, T512 on
past_len 2048); the 70B-shaped scaled-RoPE decode (B64, 64/8 heads, 80 calls);
small-batch decode latency (tiny 6/2-head case and one Llama-3.1-8B layer),
rope_append + decode_attn against the single-launch gqa_decode_step; and
wide-group decode (B16 64/1 and B32 32/2 heads), the wide kernel against the
split-K path on the same call.  The small-batch and wide legs time HIP graphs
of 20 calls replayed back to back, so host launch overhead is excluded.
"warm" figures replay with the inputs left in the caches by the previous call
(the small cases fit in the 256 MB MALL); "cold" ones put a 1 GiB write
between calls inside the graph and subtract a graph of the writes alone.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
HEADLINE = "llama8b_b32_decode_32layers"


COUNTERS = os.path.join(ROOT, "profiles", "decode_llama8b_b32_decode_32layers_hbm_counters.txt")
KERNEL_SOURCES = ("gqa_attention_rope_amd/csrc/decode.hip", "gqa_attention_rope_amd/csrc/common.hpp",
                  "gqa_attention_rope_amd/csrc/kernels.hpp", "gqa_attention_rope_amd/build.py")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic():
    """HBM bytes per layer of the decode attention kernels (partials, combine) from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, each counter scaled by its plain-copy calibration factor.  None when the
    kernel sources have changed since the counters were taken (or the summary is absent)."""
    try:
        with open(COUNTERS) as fh:
            recs = [json.loads(l[len("RECORD "):]) for l in fh if l.startswith("RECORD ")]
    except (OSError, ValueError):
        recs = []
    if not recs:
        return None, "no counter summary"
    if any(r.get("source_sha256_16") != kernel_source_hash() for r in recs):
        return None, "decode kernel sources changed since the counters were taken"
    out = {}
    for r in recs:
        out[r["kernel"]] = int(round(r["fetch_kib"] * 1024 * r["fetch_factor"] + r["write_kib"] * 1024 * r["write_factor"]))
    f = recs[0]
    return out, "rocprofv3 FETCH_SIZE x%g + WRITE_SIZE x%g (plain-copy calibration), bytes per launch" % (
        f["fetch_factor"], f["write_factor"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the prefill and 70B-shape figures")
    ap.add_argument("--decode-wg", type=int, default=0, help="override the split-K workgroup count")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="first run one plain device copy of this many GiB (reference for HBM byte counters)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling leg")
    ap.add_argument("--legs", default="prefill,long,small,wide",
                    help="extra legs to run (comma list of prefill, long, small, wide, batch; batch is the decode "
                         "attention batch-size sweep, not run by default)")
    return ap.parse_args()


def kv_bytes(past, n_kv, d):
    return int(sum((int(p) + 1) * n_kv * d * 2 * 2 for p in past))


def timed(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def kernel_avg(gq, fn, steps, kind):
    """Average device time of one kernel kind over `steps` more steps (HIP events on the launch stream)."""
    import torch
    torch.cuda.synchronize()
    gq.gqa_profile_reset()
    gq.gqa_profile_enable(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    gq.gqa_profile_enable(False)
    out = {k: gq.gqa_profile_read(k) for k in KINDS}
    gq.gqa_profile_reset()
    ms, n = out[kind]
    return ms / max(n, 1), out


KINDS = ("rope_append", "decode_partial", "decode_combine", "prefill", "decode_step", "decode_wide", "stream_read")


def call_kernel_us(gq, fn, reps, flush=None):
    """Per call of fn: the device time of each kernel kind it launches (HIP events around every launch, summed
    per call, median over reps calls).  With flush, a 1 GiB write runs before each call (not timed), so the
    call starts with its inputs out of the L2 and the 256 MB MALL ("cold")."""
    import numpy as np
    import torch
    per = {k: [] for k in KINDS}
    for r in range(reps):
        if flush is not None:
            flush.fill_(r & 0xff)
        torch.cuda.synchronize()
        gq.gqa_profile_reset()
        gq.gqa_profile_enable(True)
        fn()
        torch.cuda.synchronize()
        gq.gqa_profile_enable(False)
        for k in KINDS:
            ms, n = gq.gqa_profile_read(k)
            if n:
                per[k].append(ms * 1e3)
        gq.gqa_profile_reset()
    kinds = {k: round(float(np.median(v)), 2) for k, v in per.items() if v}
    return round(sum(kinds.values()), 2), kinds


def stream_ceiling(gq, dev, nbytes):
    """Best mean launch time of the library's streaming-read kernel over nbytes, across grid sizes."""
    import torch
    n = (nbytes + 15) // 16 * 16
    buf = torch.ones(n, dtype=torch.uint8, device=dev)
    sink = torch.empty(65536, dtype=torch.int32, device=dev)
    res = {}
    for wg in (512, 1024, 2048, 4096, 8192):
        for _ in range(2):
            gq.gqa_measure_stream_read(buf, sink, wg)
        ms, _ = kernel_avg(gq, lambda: gq.gqa_measure_stream_read(buf, sink, wg), 20, "stream_read")
        res[wg] = n / (ms * 1e-3) / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    best = max(res, key=res.get)
    return {"gbs": round(res[best], 1), "pct_hbm_peak": round(100 * res[best] / HBM_PEAK_GBS, 2), "bytes": n,
            "workgroups": best, "by_workgroups": {str(k): round(v, 1) for k, v in res.items()},
            "timing": "HIP events around each launch, mean of 20 launches"}


def mfma_ceiling(gq, dev, workgroups=512, iters=4000):
    """Sustained rate of the prefill kernel's matrix instruction (bf16 16x16x32 MFMA, 16384 flops) with every
    CU busy, from the library's matrix-rate probe at the prefill's occupancy (two 4-wave workgroups per CU),
    and the shader clock the probe recorded.  The measured counterpart of the datasheet peak, as the
    streaming-read ceiling is for HBM."""
    import torch
    sink = torch.zeros(8 * workgroups, dtype=torch.int64, device=dev)
    gq.gqa_measure_mfma_rate(workgroups, max(1, iters // 4), sink)
    torch.cuda.synchronize()
    best = None
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        gq.gqa_measure_mfma_rate(workgroups, iters, sink)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3
        w = sink.view(-1, 8).to(torch.float64).cpu()
        mhz = float(w[:, 4].sum() / w[:, 5].sum() * 100.0)
        if best is None or us < best[0]:
            best = (us, mhz)
    us, mhz = best
    flops = workgroups * 4 * iters * 8 * 16384
    tf = flops / (us * 1e-6) / 1e12
    return {"tflops": round(tf, 1), "frac_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "clock_mhz": round(mhz),
            "instruction": "v_mfma_f32_16x16x32_bf16, random operands", "workgroups": workgroups,
            "timing": "HIP events around one launch (best of 3)"}


def decode_workload(gq, synth, name, dev):
    import torch
    w = synth.WORKLOADS[name]
    B, n_q, n_kv, d, S, layers = w["B"], w["n_q"], w["n_kv"], w["d"], w["S"], w["layers"]
    past = synth.past_lengths(B, w["past"], w["seed"])
    # the 70B-shaped workload reuses one cache pair for all of its layer calls
    n_caches = layers if name == HEADLINE else 1
    kc = [torch.empty((B, n_kv, S, d), dtype=torch.bfloat16, device=dev) for _ in range(n_caches)]
    vc = [torch.empty((B, n_kv, S, d), dtype=torch.bfloat16, device=dev) for _ in range(n_caches)]
    for i in range(n_caches):
        synth.fill_normal_bf16_(kc[i], w["seed"] * 1000 + 2 * i)
        synth.fill_normal_bf16_(vc[i], w["seed"] * 1000 + 2 * i + 1)
    q = synth.normal_bf16((layers, B, n_q, 1, d), w["seed"] + 11, dev)
    kn = synth.normal_bf16((layers, B, n_kv, 1, d), w["seed"] + 12, dev)
    vn = synth.normal_bf16((layers, B, n_kv, 1, d), w["seed"] + 13, dev)
    q_rot = torch.empty_like(q)
    out = torch.empty_like(q)
    pl = torch.as_tensor(past, device=dev)
    maxp = int(past.max())
    ws = torch.zeros(gq.gqa_decode_workspace_bytes(B, n_q, n_kv, d, S), dtype=torch.uint8, device=dev)

    def step():
        for l in range(layers):
            c = l % n_caches
            gq.gqa_rope_append(q[l], kn[l], vn[l], kc[c], vc[c], pl, maxp, w["theta"], "interleaved", w["scaling"],
                               q_rot=q_rot[l])
            gq.gqa_decode_attn(q_rot[l], kc[c], vc[c], pl, maxp, out=out[l], workspace=ws)

    def attention_only():
        # the decode attention calls of the step alone, on the q_rot the last step left
        for l in range(layers):
            c = l % n_caches
            gq.gqa_decode_attn(q_rot[l], kc[c], vc[c], pl, maxp, out=out[l], workspace=ws)

    info = dict(w=w, B=B, n_q=n_q, n_kv=n_kv, d=d, S=S, layers=layers, past=past,
                kv_per_layer=kv_bytes(past, n_kv, d), q_bytes=B * n_q * d * 2, attention_only=attention_only)
    return step, info, (kc, vc, q, kn, vn)


def prefill_workload(gq, synth, dev):
    import torch
    w = synth.WORKLOADS["llama8b_chunked_prefill"]
    B, n_q, n_kv, T, d, S = w["B"], w["n_q"], w["n_kv"], w["T"], w["d"], w["S"]
    past = synth.past_lengths(B, w["past"], w["seed"])
    kc = synth.normal_bf16((B, n_kv, S, d), w["seed"] + 3, dev)
    vc = synth.normal_bf16((B, n_kv, S, d), w["seed"] + 4, dev)
    q = synth.normal_bf16((B, n_q, T, d), w["seed"], dev)
    kn = synth.normal_bf16((B, n_kv, T, d), w["seed"] + 1, dev)
    vn = synth.normal_bf16((B, n_kv, T, d), w["seed"] + 2, dev)
    pl = torch.as_tensor(past, device=dev)
    maxp = int(past.max())
    q_rot = gq.gqa_rope_append(q, kn, vn, kc, vc, pl, maxp, w["theta"])
    out = torch.empty_like(q_rot)

    def step():
        gq.gqa_prefill_attn(q_rot, kc, vc, pl, maxp, out=out)

    # flops over the visible (query, key) pairs only: QK^T and PV, 2 flops per multiply-add
    pairs = sum(sum(int(p) + t + 1 for t in range(T)) for p in past)
    flops = 2 * 2 * n_q * d * pairs
    return step, flops


def small_batch_workload(gq, synth, name, dev):
    """One decode step of a small workload two ways: rope_append + decode_attn, and the single-launch step."""
    import torch
    w = synth.WORKLOADS[name]
    B, n_q, n_kv, d, S = w["B"], w["n_q"], w["n_kv"], w["d"], w["S"]
    past = synth.past_lengths(B, w["past"], w["seed"])
    kc = synth.normal_bf16((B, n_kv, S, d), w["seed"] + 3, dev)
    vc = synth.normal_bf16((B, n_kv, S, d), w["seed"] + 4, dev)
    q = synth.normal_bf16((B, n_q, 1, d), w["seed"], dev)
    kn = synth.normal_bf16((B, n_kv, 1, d), w["seed"] + 1, dev)
    vn = synth.normal_bf16((B, n_kv, 1, d), w["seed"] + 2, dev)
    pl = torch.as_tensor(past, device=dev)
    maxp = int(past.max())
    q_rot, out3, out1 = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws3 = torch.zeros(gq.gqa_decode_workspace_bytes(B, n_q, n_kv, d, S), dtype=torch.uint8, device=dev)
    ws1 = torch.zeros(gq.gqa_decode_step_workspace_bytes(B, n_q, n_kv, d, S), dtype=torch.uint8, device=dev)

    def three():
        gq.gqa_rope_append(q, kn, vn, kc, vc, pl, maxp, w["theta"], "interleaved", w["scaling"], q_rot=q_rot)
        gq.gqa_decode_attn(q_rot, kc, vc, pl, maxp, out=out3, workspace=ws3)

    def one():
        gq.gqa_decode_step(q, kn, vn, kc, vc, pl, maxp, w["theta"], "interleaved", w["scaling"], out=out1,
                           workspace=ws1)

    return three, one, kv_bytes(past, n_kv, d), B


def graph_us(fn, per_graph=20, replays=20):
    """Device time per call of fn, from a HIP graph of per_graph calls replayed back to back (no host gaps)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (replays * per_graph)


def wide_group_workload(gq, synth, dev, B, n_q, n_kv, seed, cold_bytes=6.4e8):
    """Decode attention for a wide query group (g = n_q / n_kv >= 16), ragged contexts U[2048, 8191].

    Returns (warm, cold, kv bytes per call, layers): warm repeats the call on one cache pair, whose rows
    then partly stay in the 256 MB MALL; cold moves to the next of `layers` cache pairs on every call (as
    the layers of a decode step do), with enough layers that about cold_bytes of K/V lie between two reads
    of the same rows."""
    import math
    import torch
    d, S = 128, 8192
    past = synth.past_lengths(B, ("uniform", 2048, 8191), seed)
    kvb = kv_bytes(past, n_kv, d)
    layers = max(2, math.ceil(cold_bytes / kvb))
    kcs, vcs = [], []
    for l in range(layers):
        kc = torch.empty((B, n_kv, S, d), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        synth.fill_normal_bf16_(kc, seed * 1000 + 2 * l)
        synth.fill_normal_bf16_(vc, seed * 1000 + 2 * l + 1)
        kcs.append(kc)
        vcs.append(vc)
    q = synth.normal_bf16((B, n_q, 1, d), seed + 11, dev)
    pl = torch.as_tensor(past, device=dev)
    maxp = int(past.max())
    out = torch.empty_like(q)
    ws = torch.zeros(gq.gqa_decode_workspace_bytes(B, n_q, n_kv, d, S), dtype=torch.uint8, device=dev)
    nxt = [0]

    def warm():
        gq.gqa_decode_attn(q, kcs[0], vcs[0], pl, maxp, out=out, workspace=ws)

    def cold():
        l = nxt[0] % layers
        nxt[0] += 1
        gq.gqa_decode_attn(q, kcs[l], vcs[l], pl, maxp, out=out, workspace=ws)

    return warm, cold, kvb, layers


BATCH_SWEEP = (1, 2, 4, 8, 16, 32, 64, 128, 256)


def batch_sweep_workload(gq, synth, dev, B, cold_bytes=1.2e9):
    """gqa_decode_attn at the headline's shape (32/8 heads, d 128, S 8192, past_len U[512, 8191], seed 1003) for
    batch size B, each call on the next of enough cache pairs that about cold_bytes of K/V lie between two reads
    of the same rows.  Returns (call, kv bytes per call, cache pairs)."""
    import math
    import torch
    w = synth.WORKLOADS[HEADLINE]
    n_q, n_kv, d, S = w["n_q"], w["n_kv"], w["d"], w["S"]
    past = synth.past_lengths(B, w["past"], w["seed"])
    kvb = kv_bytes(past, n_kv, d)
    layers = min(32, max(2, math.ceil(cold_bytes / kvb)))
    kcs, vcs = [], []
    for l in range(layers):
        kc = torch.empty((B, n_kv, S, d), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        synth.fill_normal_bf16_(kc, 7000 + 2 * l)
        synth.fill_normal_bf16_(vc, 7001 + 2 * l)
        kcs.append(kc)
        vcs.append(vc)
    q = synth.normal_bf16((B, n_q, 1, d), w["seed"] + 11, dev)
    pl = torch.as_tensor(past, device=dev)
    maxp = int(past.max())
    out = torch.empty_like(q)
    ws = torch.zeros(gq.gqa_decode_workspace_bytes(B, n_q, n_kv, d, S), dtype=torch.uint8, device=dev)
    nxt = [0]

    def call():
        l = nxt[0] % layers
        nxt[0] += 1
        gq.gqa_decode_attn(q, kcs[l], vcs[l], pl, maxp, out=out, workspace=ws)

    return call, kvb, layers


def cpu_baseline(info, kc, vc, q, kn, vn):
    """The fp64 oracle on one layer of the headline step (all 32 sequences), with every host core this process
    may use and with one thread."""
    import numpy as np
    from gqa_attention_rope_amd import synth
    from oracle import attend, rope_append
    from threadpoolctl import threadpool_info, threadpool_limits
    affinity = len(os.sched_getaffinity(0))
    w = info["w"]
    past = info["past"]
    # host copies of layer 0 (not timed)
    kc0, vc0 = synth.bits(kc[0]), synth.bits(vc[0])
    q0, kn0, vn0 = synth.bits(q[0]), synth.bits(kn[0]), synth.bits(vn[0])

    def run(max_reps, budget_s):
        reps = 0
        t0 = time.perf_counter()
        while True:
            qr, kr, vr = rope_append(q0, kn0, vn0, kc0, vc0, past, w["theta"], "interleaved", w["scaling"])
            attend(qr, kr, vr, past, info["n_kv"])
            reps += 1
            el = time.perf_counter() - t0
            if el > budget_s or reps >= max_reps:
                return el / reps, reps

    with threadpool_limits(limits=affinity):
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        per_all, reps_all = run(3, 10.0)
    with threadpool_limits(limits=1):
        per_one, reps_one = run(1, 30.0)
    kvb = info["kv_per_layer"]
    tok = lambda per: round(info["B"] / (per * info["layers"]), 4)
    return {"value": round(kvb / per_all / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one of the 32 layers (all 32 sequences, rope_append + attend in fp64), {reps_all} rep(s), "
                      f"{per_all:.2f} s per layer with {threads} BLAS threads ({affinity} host CPUs in this "
                      f"process's affinity); tokens/s at that rate over 32 layers: {tok(per_all)}",
            "single_thread": {"value": round(kvb / per_one / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"same layer, {reps_one} rep(s), {per_one:.2f} s per layer; "
                                        f"tokens/s over 32 layers: {tok(per_one)}"}}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch
    import gqa_attention_rope_amd as gq
    from gqa_attention_rope_amd import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    gq.gqa_set_decode_workgroups(args.decode_wg)

    if args.copy_calibration_gib > 0:
        n = int(args.copy_calibration_gib * (1 << 30))
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copy calibration: {n} bytes read and {n} bytes written by one copy kernel", file=sys.stderr)
        del src, dst
        torch.cuda.empty_cache()

    step, info, tensors = decode_workload(gq, synth, HEADLINE, dev)
    print(f"# headline workload ready: B={info['B']} layers={info['layers']} mean ctx "
          f"{np.mean(info['past']) + 1:.1f}", file=sys.stderr, flush=True)
    ms, wall = timed(step, args.steps, args.warmup, stream)
    kv_step = info["kv_per_layer"] * info["layers"]
    value = kv_step / (ms * 1e-3) / 1e9
    tok_s = info["B"] / (ms * 1e-3)

    # decode attention alone: the 32 layers' gqa_decode_attn calls (partials + combine) back to back, timed
    # over at least 50 loops after at least 10 warm-up loops whatever --steps is (a secondary figure: a short
    # loop right after the step loop measured 1-3 % slow)
    attn_reps, attn_warm = max(args.steps, 50), max(args.warmup, 10)
    attn_layers_ms, _ = timed(info["attention_only"], attn_reps, attn_warm, stream)
    attn_ms = attn_layers_ms / info["layers"]
    avg_ms, per_kind = kernel_avg(gq, step, max(5, args.steps // 5), "decode_partial")
    comb_ms = per_kind["decode_combine"][0] / max(per_kind["decode_combine"][1], 1)
    alg = info["kv_per_layer"] + info["q_bytes"]
    achieved = alg / (attn_ms * 1e-3) / 1e9
    achieved_p = alg / (avg_ms * 1e-3) / 1e9
    traffic, traffic_note = counter_traffic()
    t_part = traffic.get("decode_partial_kernel<128,4,1>") if traffic else None
    t_comb = traffic.get("decode_combine_kernel<128>") if traffic else None
    t_attn = t_part + t_comb if (t_part is not None and t_comb is not None) else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": t_attn, "traffic_note": traffic_note,
                "traffic_over_alg": round(t_attn / alg, 4) if t_attn else None,
                "kernel": "decode attention per layer: decode_partial_kernel<128,4,1> + decode_combine_kernel<128>",
                "avg_launch_us": round(attn_ms * 1e3, 2), "alg_bytes_per_launch": alg,
                "timing": f"HIP events around {attn_reps} x 32 back-to-back gqa_decode_attn calls (two kernels "
                          f"each, after {attn_warm} x 32 untimed), per call",
                "dominant_kernel": {"kernel": "decode_partial_kernel<128,4,1>", "achieved": round(achieved_p, 1),
                                    "frac": round(achieved_p / HBM_PEAK_GBS, 4), "avg_launch_us": round(avg_ms * 1e3, 2),
                                    "traffic": t_part,
                                    "traffic_over_alg": round(t_part / alg, 4) if t_part else None,
                                    "timing": "HIP events on the launch stream around each launch, mean over "
                                              f"{per_kind['decode_partial'][1]} launches (adds the dispatch gap)"}}
    kinds = {k: {"avg_us": round(v[0] / max(v[1], 1) * 1e3, 2), "launches": v[1]} for k, v in per_kind.items() if v[1]}
    attn_gbs = info["kv_per_layer"] / (attn_ms * 1e-3) / 1e9
    decode_attention = {"kv_gbs": round(attn_gbs, 1), "pct_hbm_peak": round(100 * attn_gbs / HBM_PEAK_GBS, 2),
                        "us_per_layer": round(attn_ms * 1e3, 2),
                        "definition": "KV bytes per layer / time of one gqa_decode_attn call (partials + combine), "
                                      "from 32-call loops timed with HIP events"}

    line = {
        "metric": "decode attn KV-read GB/s (% of HBM peak) + tokens/s, B=32 ragged ctx<=8192",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "B": info["B"], "n_q": info["n_q"], "n_kv": info["n_kv"], "d": info["d"],
                   "max_seq": info["S"], "layers": info["layers"], "past_len": "U[512,8191], seed 1003",
                   "mean_ctx": round(float(np.mean(info["past"]) + 1), 1), "kv_bytes_per_step": kv_step},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(tok_s, 1),
        "wall_s_timed": round(wall, 3),
        "kernels": kinds,
        "kernels_timing": "HIP events on the launch stream around each launch, mean per launch; each bracket also "
                          "holds that launch's dispatch gap, so the kinds sum to more than ms_per_step / layers "
                          "(the rocprofv3 kernel durations under profiles/ do not)",
        "decode_attention": decode_attention,
        "roofline": roofline,
    }
    if not args.no_ceiling:
        line["stream_read_ceiling"] = stream_ceiling(gq, dev, info["kv_per_layer"] + info["q_bytes"])

    legs = set(x.strip() for x in args.legs.split(",") if x.strip())
    if not args.no_extra:
        extra = {}
        torch.cuda.synchronize()
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    if not args.no_extra and "prefill" in legs:
        pstep, flops = prefill_workload(gq, synth, dev)
        pms, _ = timed(pstep, 20, 3, stream)
        pavg, _ = kernel_avg(gq, pstep, 10, "prefill")
        p_warm, _ = call_kernel_us(gq, pstep, 20)
        p_cold, _ = call_kernel_us(gq, pstep, 20, flush)
        ceil = mfma_ceiling(gq, dev)
        extra["chunked_prefill"] = {"workload": "llama8b_chunked_prefill B4 T512 P2048", "ms": round(pms, 4),
                                    "tflops": round(flops / (pms * 1e-3) / 1e12, 1),
                                    "kernel_tflops": round(flops / (pavg * 1e-3) / 1e12, 1),
                                    "frac_mfma_peak": round(flops / (pavg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                                    "visible_pair_gflop": round(flops / 1e9, 2),
                                    "kernel_us_warm": p_warm, "kernel_us_cold": p_cold,
                                    "cold_tflops": round(flops / (p_cold * 1e-6) / 1e12, 1),
                                    "mfma_ceiling": ceil,
                                    "frac_measured_ceiling": round(flops / (pavg * 1e-3) / 1e12 / ceil["tflops"], 4)}
        del pstep
        torch.cuda.empty_cache()
    if not args.no_extra and "long" in legs:
        s5, info5, t5 = decode_workload(gq, synth, "llama70b_shape_decode_scaled", dev)
        ms5, _ = timed(s5, 5, 1, stream)
        kv5 = info5["kv_per_layer"] * info5["layers"]
        extra["long_context_scaled_decode"] = {
            "workload": "llama70b_shape_decode_scaled B64 64/8 heads ctx U[4096,8191] 80 calls",
            "ms_per_80_calls": round(ms5, 3), "kv_gbs": round(kv5 / (ms5 * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * kv5 / (ms5 * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "tokens_per_s": round(info5["B"] / (ms5 * 1e-3), 1)}
        del s5, t5
        torch.cuda.empty_cache()
    if not args.no_extra and "small" in legs:
        small = {}
        for name in ("tiny_decode_g3", "llama8b_layer_decode"):
            three, one, kvb, Bs = small_batch_workload(gq, synth, name, dev)
            t3, t1 = graph_us(three), graph_us(one)
            k3w, _ = call_kernel_us(gq, three, 30)
            k3c, _ = call_kernel_us(gq, three, 30, flush)
            k1w, _ = call_kernel_us(gq, one, 30)
            k1c, _ = call_kernel_us(gq, one, 30, flush)
            small[name] = {"rope_append_plus_decode_us": round(t3, 2), "single_launch_step_us": round(t1, 2),
                           "speedup": round(t3 / t1, 2), "kv_bytes": kvb,
                           "single_launch_tokens_per_s": round(Bs / (t1 * 1e-6), 1),
                           "kernel_us": {"three_call_warm": k3w, "three_call_cold": k3c,
                                         "single_launch_warm": k1w, "single_launch_cold": k1c}}
        extra["small_batch_decode"] = dict(
            small, timing="HIP graph of 20 steps replayed 20 times, per step; kernel_us: sum of the call's kernel "
                          "times (HIP events around each launch), median of 30 calls, warm = back to back, "
                          "cold = a 1 GiB write before each call")
    if not args.no_extra and "wide" in legs:
        wide = {}
        for (Bw, nqw, nkvw, seed) in ((16, 64, 1, 1006), (32, 32, 2, 1007)):
            warm, cold, kvb, layers = wide_group_workload(gq, synth, dev, Bw, nqw, nkvw, seed)
            t_cold = graph_us(cold)
            t_warm = graph_us(warm)
            gq.gqa_set_decode_wide_min_group(65)  # the split-K path on the same calls
            t_split = graph_us(cold)
            gq.gqa_set_decode_wide_min_group(0)
            wide[f"B{Bw}_{nqw}q_{nkvw}kv_g{nqw // nkvw}"] = {
                "wide_kernel_us": round(t_cold, 2), "kv_gbs": round(kvb / (t_cold * 1e-6) / 1e9, 1),
                "frac_hbm_peak": round(kvb / (t_cold * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "warm_us": round(t_warm, 2), "warm_kv_gbs": round(kvb / (t_warm * 1e-6) / 1e9, 1),
                "split_k_us": round(t_split, 2), "speedup": round(t_split / t_cold, 2), "kv_bytes": kvb,
                "cache_layers": layers}
            del warm, cold
            torch.cuda.empty_cache()
        extra["wide_group_decode"] = dict(
            wide, context="past_len U[2048,8191] seeded, d 128, S 8192",
            timing="HIP graph of 20 calls replayed 20 times, per call (partials + combine); wide_kernel_us, kv_gbs "
                   "and split_k_us: each call on the next of cache_layers cache pairs (cold, as across the layers "
                   "of a step); warm_*: every call on the same cache pair (rows partly held in the MALL)")
    if not args.no_extra and "batch" in legs:
        sweep = {}
        for Bs in BATCH_SWEEP:
            call, kvb, layers = batch_sweep_workload(gq, synth, dev, Bs)
            t = graph_us(call)
            sweep[f"B{Bs}"] = {"us": round(t, 2), "kv_gbs": round(kvb / (t * 1e-6) / 1e9, 1),
                               "frac_hbm_peak": round(kvb / (t * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "kv_bytes": kvb,
                               "cache_layers": layers}
            del call
            torch.cuda.empty_cache()
        extra["decode_batch_sweep"] = dict(
            sweep, context="gqa_decode_attn (partials + combine), 32/8 heads, d 128, S 8192, past_len U[512,8191] "
                           "seed 1003 (the headline's), batch size B",
            timing="HIP graph of 20 calls replayed 20 times, per call, each call on the next of cache_layers cache "
                   "pairs (cold)")
    if not args.no_extra:
        del flush
        torch.cuda.empty_cache()
        line["extra"] = extra
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(info, *tensors)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
