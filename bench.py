"""Benchmark of the GQA + RoPE KV-cache attention step on one MI355X.

A step is one decode step of a batch of 32 Llama-3.1-8B sequences through 32
layers: per layer, RoPE + cache append of the new token (gqa_rope_append),
then split-K decode attention over cache rows 0..past_len[b]
(gqa_decode_attn).  Contexts are ragged, past_len ~ U[512, 8191] (seeded),
caches [32, 8, 8192, 128] bf16 per layer, 32 distinct layers (32 GiB).  All
inputs are resident in HBM before timing starts.

Printed: one JSON line.  value = KV-read GB/s over the whole step
(sum over layers and sequences of (past_len+1) * n_kv * d * 2 tensors * 2 B,
divided by the step time); tokens/s = B / step time.  roofline = the decode
split-K kernel's algorithmic bytes per launch over its average launch time
(HIP events on the launch stream), against 8 TB/s; roofline.traffic = HBM bytes
per launch from the committed rocprofv3 byte-counter summary under profiles/
(null once the decode kernel sources differ from the ones it was taken on).
cpu_baseline = the fp64
oracle on a bounded sample of the same workload, on this host.

extra (skipped with --no-extra): chunked prefill TFLOP/s (B4, T512 on
past_len 2048); the 70B-shaped scaled-RoPE decode (B64, 64/8 heads, 80 calls);
small-batch decode latency (tiny 6/2-head case and one Llama-3.1-8B layer),
rope_append + decode_attn against the single-launch gqa_decode_step; and
wide-group decode (B16 64/1 and B32 32/2 heads), the wide kernel against the
split-K path on the same call.  The small-batch and wide legs time HIP graphs
of 20 calls replayed back to back, so host launch overhead is excluded.
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


COUNTERS = os.path.join(ROOT, "profiles", "decode_partial_llama8b_b32_decode_32layers_hbm_counters.txt")
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
    """HBM bytes per decode split-K launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary,
    each counter scaled by its plain-copy calibration factor.  None when the kernel sources have changed
    since the counters were taken (or the summary is absent)."""
    try:
        with open(COUNTERS) as fh:
            rec = next(json.loads(l[len("RECORD "):]) for l in fh if l.startswith("RECORD "))
    except (OSError, StopIteration, ValueError):
        return None, "no counter summary"
    if rec.get("source_sha256_16") != kernel_source_hash():
        return None, "decode kernel sources changed since the counters were taken"
    t = rec["fetch_kib"] * 1024 * rec["fetch_factor"] + rec["write_kib"] * 1024 * rec["write_factor"]
    return int(round(t)), "rocprofv3 FETCH_SIZE x%g + WRITE_SIZE x%g (plain-copy calibration), bytes per launch" % (
        rec["fetch_factor"], rec["write_factor"])


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
    out = {k: gq.gqa_profile_read(k) for k in ("rope_append", "decode_partial", "decode_combine", "prefill",
                                               "decode_step", "decode_wide")}
    gq.gqa_profile_reset()
    ms, n = out[kind]
    return ms / max(n, 1), out


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

    info = dict(w=w, B=B, n_q=n_q, n_kv=n_kv, d=d, S=S, layers=layers, past=past,
                kv_per_layer=kv_bytes(past, n_kv, d), q_bytes=B * n_q * d * 2)
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


def wide_group_workload(gq, synth, dev, B, n_q, n_kv, seed):
    """Decode attention for a wide query group (g = n_q / n_kv >= 16), ragged contexts U[2048, 8191]."""
    import torch
    d, S = 128, 8192
    past = synth.past_lengths(B, ("uniform", 2048, 8191), seed)
    kc = torch.empty((B, n_kv, S, d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    synth.fill_normal_bf16_(kc, seed * 1000)
    synth.fill_normal_bf16_(vc, seed * 1000 + 1)
    q = synth.normal_bf16((B, n_q, 1, d), seed + 11, dev)
    pl = torch.as_tensor(past, device=dev)
    maxp = int(past.max())
    out = torch.empty_like(q)
    ws = torch.zeros(gq.gqa_decode_workspace_bytes(B, n_q, n_kv, d, S), dtype=torch.uint8, device=dev)

    def call():
        gq.gqa_decode_attn(q, kc, vc, pl, maxp, out=out, workspace=ws)

    return call, kv_bytes(past, n_kv, d)


def cpu_baseline(info, kc, vc, q, kn, vn):
    """The fp64 oracle on one layer of the headline step, all 32 sequences."""
    import numpy as np
    from gqa_attention_rope_amd import synth
    from oracle import attend, rope_append
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    w = info["w"]
    past = info["past"]
    # host copies of layer 0 (not timed)
    kc0, vc0 = synth.bits(kc[0]), synth.bits(vc[0])
    q0, kn0, vn0 = synth.bits(q[0]), synth.bits(kn[0]), synth.bits(vn[0])
    reps = 0
    t0 = time.perf_counter()
    while True:
        qr, kr, vr = rope_append(q0, kn0, vn0, kc0, vc0, past, w["theta"], "interleaved", w["scaling"])
        attend(qr, kr, vr, past, info["n_kv"])
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0 or reps >= 3:
            break
    per_layer = el / reps
    gbs = info["kv_per_layer"] / per_layer / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one of the 32 layers (all 32 sequences, rope_append + attend in fp64), {reps} rep(s), "
                      f"{per_layer:.2f} s per layer; tokens/s at that rate over 32 layers: "
                      f"{info['B'] / (per_layer * info['layers']):.4f}"}


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

    avg_ms, per_kind = kernel_avg(gq, step, max(5, args.steps // 5), "decode_partial")
    alg = info["kv_per_layer"] + info["q_bytes"]
    achieved = alg / (avg_ms * 1e-3) / 1e9
    traffic, traffic_note = counter_traffic()
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_note": traffic_note,
                "traffic_over_alg": round(traffic / alg, 4) if traffic else None,
                "kernel": "decode_partial_kernel<128,4,1>", "avg_launch_us": round(avg_ms * 1e3, 2),
                "alg_bytes_per_launch": alg}
    kinds = {k: {"avg_us": round(v[0] / max(v[1], 1) * 1e3, 2), "launches": v[1]} for k, v in per_kind.items() if v[1]}

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
        "roofline": roofline,
    }

    if not args.no_extra:
        extra = {}
        torch.cuda.synchronize()
        pstep, flops = prefill_workload(gq, synth, dev)
        pms, _ = timed(pstep, 20, 3, stream)
        pavg, _ = kernel_avg(gq, pstep, 10, "prefill")
        extra["chunked_prefill"] = {"workload": "llama8b_chunked_prefill B4 T512 P2048", "ms": round(pms, 4),
                                    "tflops": round(flops / (pms * 1e-3) / 1e12, 1),
                                    "kernel_tflops": round(flops / (pavg * 1e-3) / 1e12, 1),
                                    "frac_mfma_peak": round(flops / (pavg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                                    "visible_pair_gflop": round(flops / 1e9, 2)}
        del pstep
        torch.cuda.empty_cache()
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
        small = {}
        for name in ("tiny_decode_g3", "llama8b_layer_decode"):
            three, one, kvb, Bs = small_batch_workload(gq, synth, name, dev)
            t3, t1 = graph_us(three), graph_us(one)
            small[name] = {"rope_append_plus_decode_us": round(t3, 2), "single_launch_step_us": round(t1, 2),
                           "speedup": round(t3 / t1, 2), "kv_bytes": kvb,
                           "single_launch_tokens_per_s": round(Bs / (t1 * 1e-6), 1)}
        extra["small_batch_decode"] = dict(small, timing="HIP graph of 20 steps replayed 20 times, per step")
        wide = {}
        for (Bw, nqw, nkvw, seed) in ((16, 64, 1, 1006), (32, 32, 2, 1007)):
            call, kvb = wide_group_workload(gq, synth, dev, Bw, nqw, nkvw, seed)
            t_wide = graph_us(call)
            gq.gqa_set_decode_wide_min_group(65)  # the split-K path on the same call
            t_split = graph_us(call)
            gq.gqa_set_decode_wide_min_group(0)
            wide[f"B{Bw}_{nqw}q_{nkvw}kv_g{nqw // nkvw}"] = {
                "wide_kernel_us": round(t_wide, 2), "kv_gbs": round(kvb / (t_wide * 1e-6) / 1e9, 1),
                "split_k_us": round(t_split, 2), "speedup": round(t_split / t_wide, 2), "kv_bytes": kvb}
            del call
            torch.cuda.empty_cache()
        extra["wide_group_decode"] = dict(wide, context="past_len U[2048,8191] seeded, d 128, S 8192",
                                          timing="HIP graph of 20 calls replayed 20 times, per call")
        line["extra"] = extra
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(info, *tensors)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
