"""Seeded synthetic inputs shared by the tests, the bench and smoke().

This module holds none of the attention step's arithmetic: it only draws
numbers.  Values are i.i.d. N(0, 1) draws made by torch's generator (CPU or
device) and cast to bf16 by torch; integer past lengths come from numpy's
PCG64 generator.  The HIP path and the oracle both consume what it returns.

The named workloads are the five shapes the attention step is exercised on:
a tiny 6/2-head decode, a single Llama-3.1-8B layer decode, a batched 32-layer
decode over ragged contexts, a chunked prefill, and a long-context 64/8-head
decode with Llama-3 scaled RoPE.
"""

import numpy as np
import torch

# Llama-3 scaled RoPE parameters of the 70B-shaped workload
LLAMA3_SCALING = dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0, original_max_pos=8192.0)

WORKLOADS = {
    "tiny_decode_g3": dict(B=1, n_q=6, n_kv=2, d=64, S=256, T=1, past=("fixed", 255),
                           theta=1.0e4, scaling=None, layers=1, seed=1001),
    "llama8b_layer_decode": dict(B=1, n_q=32, n_kv=8, d=128, S=8192, T=1, past=("fixed", 1000),
                                 theta=5.0e5, scaling=None, layers=1, seed=1002),
    "llama8b_b32_decode_32layers": dict(B=32, n_q=32, n_kv=8, d=128, S=8192, T=1, past=("uniform", 512, 8191),
                                        theta=5.0e5, scaling=None, layers=32, seed=1003),
    "llama8b_chunked_prefill": dict(B=4, n_q=32, n_kv=8, d=128, S=8192, T=512, past=("fixed", 2048),
                                    theta=5.0e5, scaling=None, layers=1, seed=1004),
    "llama70b_shape_decode_scaled": dict(B=64, n_q=64, n_kv=8, d=128, S=8192, T=1, past=("uniform", 4096, 8191),
                                         theta=5.0e5, scaling=LLAMA3_SCALING, layers=80, seed=1005),
}


def past_lengths(B, spec, seed):
    """Per-sequence cached lengths: ('fixed', P) or ('uniform', lo, hi) inclusive."""
    if spec[0] == "fixed":
        return np.full(B, int(spec[1]), dtype=np.int32)
    lo, hi = int(spec[1]), int(spec[2])
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, size=B).astype(np.int32)


def normal_bf16(shape, seed, device="cpu"):
    """i.i.d. N(0, 1) draws as a contiguous bf16 torch tensor on ``device``."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16).contiguous()


def fill_normal_bf16_(t, seed):
    """Fill an existing bf16 tensor in place with seeded N(0, 1) draws (in slabs, low memory)."""
    gen = torch.Generator(device=t.device)
    gen.manual_seed(int(seed))
    flat = t.view(t.shape[0], -1)
    for i in range(flat.shape[0]):
        flat[i].copy_(torch.randn(flat.shape[1], generator=gen, device=t.device, dtype=torch.float32))
    return t


def bits(t):
    """uint16 bit patterns of a bf16 tensor, as a host numpy array."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a, device="cpu"):
    """bf16 torch tensor from uint16 bit patterns."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.uint16))
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)


NAN_BF16 = 0x7FC0


def poison_beyond(cache, past_len, T):
    """Set every cache row at or beyond past_len[b] + T to bf16 NaN (in place, torch tensor)."""
    S = cache.shape[2]
    raw = cache.view(torch.int16)
    for b in range(cache.shape[0]):
        lo = int(past_len[b]) + T
        if lo < S:
            raw[b, :, lo:, :] = NAN_BF16
    return cache
