"""Pins of the oracle's scaled-RoPE frequency rules against an independent library (CPU only).

The pages name the Llama-3 scaling fields (factor 8, low and high frequency
cutoffs, original context) in "Llama 3.1 8B KV cache", *Training details that
matter*, and list Llama-3 scaling and YaRN in "Part 7: The Modern Decoder
Block", module L7.4, citing the YaRN paper.  None prints the formulas.  The
Hugging Face ``transformers`` package ships separately written frequency
initialisers for both rules; they are called here as black boxes and their
tables (fp32) compared with the oracle's fp64 ones.

Llama-3: the library's table must equal the oracle's to fp32 rounding on every
pair, the blend band included.

YaRN: the paper defines the ramp gamma as linear in rho (turns over the original
context) between alpha and beta; the library's ramp is linear in the pair index
between the two correction dims, i.e. linear in ln(rho).  The oracle keeps the
paper's definition.  The two must agree outside the band, select the same band,
and inside it the library's gamma u fixes rho = alpha (beta / alpha)^u, from
which the paper's gamma follows; the paper's gamma is also never above the
library's (a line under the concave log).
"""

import math

import numpy as np
import pytest

from oracle import rope_attention_factor, rope_frequencies

transformers = pytest.importorskip("transformers")
from transformers import LlamaConfig  # noqa: E402
from transformers import modeling_rope_utils as hf_rope  # noqa: E402

FP32_REL = 1e-6  # the library builds its table in fp32


def hf_config(theta, d, rope):
    """A model config carrying the rope fields; the context is the extended one (factor x original)."""
    ctx = int(rope["factor"] * rope["original_max_position_embeddings"])
    return LlamaConfig(hidden_size=d * 4, num_attention_heads=4, num_key_value_heads=2, head_dim=d,
                       max_position_embeddings=ctx, rope_parameters=dict(rope, rope_theta=float(theta)))


def hf_llama3(theta, d, factor, low, high, orig):
    cfg = hf_config(theta, d, {"rope_type": "llama3", "factor": factor, "low_freq_factor": low,
                               "high_freq_factor": high, "original_max_position_embeddings": orig})
    inv, att = hf_rope._compute_llama3_parameters(cfg, device="cpu")
    return inv.double().numpy(), float(att)


def hf_yarn(theta, d, factor, beta_slow, beta_fast, orig):
    cfg = hf_config(theta, d, {"rope_type": "yarn", "factor": factor, "beta_slow": beta_slow,
                               "beta_fast": beta_fast, "original_max_position_embeddings": orig,
                               "truncate": False})
    inv, att = hf_rope._compute_yarn_parameters(cfg, device="cpu")
    return inv.double().numpy(), float(att)


LLAMA3_CASES = [
    # theta, d, factor, low, high, original context
    (5.0e5, 128, 8.0, 1.0, 4.0, 8192),   # Llama 3.1 8B / 70B: the long-context decode workload
    (5.0e5, 64, 8.0, 1.0, 4.0, 8192),
    (1.0e4, 64, 4.0, 1.0, 4.0, 2048),
    (5.0e5, 128, 32.0, 1.0, 4.0, 8192),
]


@pytest.mark.parametrize("case", LLAMA3_CASES, ids=lambda c: f"theta{c[0]:g}_d{c[1]}_s{c[2]:g}")
def test_llama3_frequencies_match_library(case):
    theta, d, factor, low, high, orig = case
    lib, att = hf_llama3(theta, d, factor, low, high, orig)
    ours = rope_frequencies(theta, d, dict(type="llama3", factor=factor, low_freq_factor=low,
                                           high_freq_factor=high, original_max_pos=orig))
    plain = rope_frequencies(theta, d)
    rel = np.abs(ours - lib) / lib
    assert rel.max() <= FP32_REL, f"max rel {rel.max():.3e} at pair {int(np.argmax(rel))}"
    assert att == 1.0 and rope_attention_factor(dict(type="llama3", factor=factor)) == 1.0
    if case[:2] == (5.0e5, 128):
        # the blend band of the 8B/70B configuration really is exercised: pairs 29..34 are strictly between
        # plain/factor and plain
        band = np.flatnonzero((lib < plain * (1 - 1e-5)) & (lib > plain / factor * (1 + 1e-5)))
        assert band.tolist() == list(range(29, 35))


YARN_CASES = [
    # theta, d, factor, alpha (beta_slow), beta (beta_fast), original context
    (1.0e4, 128, 16.0, 1.0, 32.0, 4096),
    (5.0e5, 128, 16.0, 1.0, 32.0, 4096),
    (1.0e4, 64, 8.0, 1.0, 32.0, 2048),
    (5.0e5, 128, 4.0, 2.0, 16.0, 8192),
]


@pytest.mark.parametrize("case", YARN_CASES, ids=lambda c: f"theta{c[0]:g}_d{c[1]}_s{c[2]:g}_a{c[3]:g}_b{c[4]:g}")
def test_yarn_frequencies_against_library(case):
    theta, d, factor, alpha, beta, orig = case
    lib, att = hf_yarn(theta, d, factor, alpha, beta, orig)
    sc = dict(type="yarn", factor=factor, beta_slow=alpha, beta_fast=beta, original_max_pos=orig)
    ours = rope_frequencies(theta, d, sc)
    plain = rope_frequencies(theta, d)
    lo = plain / factor
    g_lib = (lib - lo) / (plain - lo)
    g_ours = (ours - lo) / (plain - lo)
    eps = 1e-5
    band_lib = (g_lib > eps) & (g_lib < 1 - eps)
    band_ours = (g_ours > eps) & (g_ours < 1 - eps)
    assert band_lib.any(), "the case must put some pairs inside the ramp"
    assert np.array_equal(band_lib, band_ours), "both rules must select the same ramp band"
    out = ~band_lib
    assert np.max(np.abs(ours[out] - lib[out]) / lib[out]) <= FP32_REL
    # inside the band: rho from the library's ramp, then the paper's gamma
    rho = alpha * (beta / alpha) ** g_lib[band_lib]
    expect = (rho - alpha) / (beta - alpha)
    assert np.max(np.abs(g_ours[band_lib] - expect)) <= 1e-5
    assert np.all(g_ours[band_lib] <= g_lib[band_lib] + 1e-6)
    # the logit temperature of the paper: sqrt(1/t) = 0.1 ln s + 1, as the library returns it
    assert math.isclose(rope_attention_factor(sc), att, rel_tol=1e-7)
