"""Plain, slow, fp64 CPU oracle for one GQA + RoPE KV-cache attention step.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Everything here is
written from the mathematics the pages state; nothing is blocked, fused or
reordered beyond what those definitions say.

Pages cited (title, then section / formula / excerpt):
  [KV]   "Llama 3.1 8B KV cache" (alijanati.com)
  [ATL]  "Llama 3 8B - KV cache" (OpenModelAtlas, decode at position 1000)
  [REP]  "Llama 3.1 8B - Repeat heads" (OpenModelAtlas)
  [EP18] "Grouped-query attention: a smaller KV cache" (mvgpt, episode 18)
  [P7]   "Part 7: The Modern Decoder Block" (openlearn course outline)

Tensor conventions (all bf16 tensors are numpy uint16 bit patterns):
  q       [B, n_q,  T, d]      new queries
  k_new   [B, n_kv, T, d]      new keys (not yet rotated)
  v_new   [B, n_kv, T, d]      new values
  k_cache [B, n_kv, S, d]      rotated keys of every position so far
  v_cache [B, n_kv, S, d]      values of every position so far
  past_len int[B]              rows already in the cache for each sequence

Parity status:
  bf16_to_f64 / f64_to_bf16   pinned (exact bit patterns, torch RNE, ties)
  rope_frequencies            pinned (closed form, geometric ratio)
  llama3_scaled_frequencies   pinned, blend band included: the pages name the
                              factor and the two cutoffs but print no formula;
                              the table matches an independently written
                              library initialiser (transformers' Llama-3 rule)
                              to fp32 rounding; limits and continuity too
  rope_frequencies linear     pinned (PI = plain RoPE at position p / s)
  rope_frequencies ntk        pinned (freq_0 = 1, lowest frequency divided by
                              exactly s, geometric progression)
  yarn_frequencies            pinned: the paper's ramp (linear in turns rho)
                              against transformers' YaRN table (linear in
                              ln rho): equal outside the ramp, the same band,
                              and inside it the paper's ramp at the rho the
                              library's ramp implies; limits, continuity, and
                              agreement with the Llama-3 rule at equal cutoffs
  rope_attention_factor       pinned (closed form 0.1 ln s + 1; equal-position
                              q.k scales by its square)
  rotate_pairs / rope_append  pinned (complex multiplication, p = 0 identity,
                              relative-offset invariance, index rule, sizes);
                              partial rotary pinned by reduction to full RoPE
                              of the leading dims and a bit-exact tail
  visible_rows (window, sinks) pinned by reduction to the full mask (window at
                              least the context, sinks covering it), the
                              one-row window (the output is that value row),
                              constant keys (the mean of the kept rows), and a
                              window equal to full attention over the sliced
                              cache; the reading of the window and sink rules
                              is the plainest one the course outline supports
  attend sink_logits          pinned by -inf (no sink), constant keys (closed
                              form of the extra denominator term)
  attend                      pinned (brute force with materialised repeat_kv
                              and the printed mask construction, torch SDPA on
                              CPU, closed forms, MHA/MQA special cases,
                              prefill = prefill + decode)
  kv_cache_bytes              pinned (every cache size the pages print)
"""

import math

import numpy as np

# ---------------------------------------------------------------------------
# bf16 <-> fp64
# ---------------------------------------------------------------------------


def bf16_to_f64(bits):
    """Exact widening of bf16 bit patterns to fp64.

    A bf16 number is the top half of an IEEE fp32 number, so shifting the
    pattern into the high 16 bits of a uint32 gives the same value as fp32.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16(x):
    """Round fp64 values to bf16 directly (round to nearest, ties to even).

    [ATL] (the generation excerpt) makes bf16 the default tensor type, and
    torch's float -> bf16 cast rounds to nearest-even.  The rounding here is
    done once, from fp64, so no double rounding through fp32 can occur.

    Method: write |x| = m * 2**e with 0.5 <= m < 1 (frexp).  bf16 keeps 8
    significant bits, so the representable numbers next to x are spaced
    2**(e-8); below the smallest normal (2**-126) the spacing is fixed at
    2**-133.  Scaling by a power of two is exact in fp64 and np.rint rounds
    half to even, so y = rint(x / q) * q is the correctly rounded value.
    """
    x = np.asarray(x, dtype=np.float64)
    y = np.array(x, dtype=np.float64, copy=True)
    nz = np.isfinite(x) & (x != 0.0)
    if np.any(nz):
        _, e = np.frexp(x[nz])
        q = np.maximum(e - 8, -133)
        y[nz] = np.ldexp(np.rint(np.ldexp(x[nz], -q)), q)
    big = np.isfinite(y) & (np.abs(y) >= 2.0 ** 128)
    y[big] = np.copysign(np.inf, y[big])
    # y is now exactly representable in bf16, hence in fp32
    with np.errstate(over="ignore", invalid="ignore"):
        f32 = y.astype(np.float32)
    u = f32.view(np.uint32)
    nan = np.isnan(x)
    out = (u >> np.uint32(16)).astype(np.uint16)
    assert np.all((u[~nan] & np.uint32(0xFFFF)) == 0), "bf16 rounding left low bits set"
    out[nan] = np.uint16(0x7FC0)
    return out


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------


SCALING_KINDS = ("llama3", "linear", "ntk", "yarn")


def rope_frequencies(theta, d, scaling=None, rotary_dim=None):
    """Per-pair rotary frequencies freq_i = theta ** (-2 i / r), i = 0 .. r/2-1.

    [KV] section "RoPE has to know where it is": the frequency of pair i is
    theta raised to minus (2i / head_dim).  r is the number of rotated dims:
    the head dimension d, or ``rotary_dim`` < d for partial rotary ([P7]
    module L7.3 names it; reading taken: the exponent uses r, as when the
    first r dims formed a head of their own).

    ``scaling`` (a dict) selects a context-extension rule ([P7] module L7.4
    lists PI, NTK, YaRN and Llama-3 scaling; the pages print none of the
    formulas, so each follows its published definition):
      type "llama3" (the default when no type is given): factor,
          low_freq_factor, high_freq_factor, original_max_pos; see
          ``llama3_scaled_frequencies``.  [KV] "Training details that matter"
          names these fields.
      type "linear" (position interpolation, Chen et al. 2023): positions are
          divided by ``factor``, i.e. every frequency is.
      type "ntk" (NTK-aware base change): the base becomes
          theta * factor ** (r / (r - 2)), which leaves freq_0 = 1 and divides
          the lowest frequency by exactly ``factor``.
      type "yarn" (Peng et al. 2023, the YaRN paper the course cites): factor,
          beta_slow (alpha), beta_fast (beta), original_max_pos; see
          ``yarn_frequencies``.  Its attention factor is applied by
          ``rope_rotate``.
    """
    r = d if rotary_dim is None else int(rotary_dim)
    if r % 2 or not 0 < r <= d:
        raise ValueError("rotary_dim must be even and in (0, d]")
    kind = None if scaling is None else scaling.get("type", "llama3")
    if kind is not None and kind not in SCALING_KINDS:
        raise ValueError(f"unknown RoPE scaling {kind!r}")
    base = float(theta)
    if kind == "ntk":
        base = base * float(scaling["factor"]) ** (r / (r - 2.0))
    i = np.arange(r // 2, dtype=np.float64)
    freq = np.power(base, -(2.0 * i) / r)
    if kind == "llama3":
        freq = llama3_scaled_frequencies(freq, scaling["factor"], scaling["low_freq_factor"],
                                         scaling["high_freq_factor"], scaling["original_max_pos"])
    elif kind == "linear":
        freq = freq / float(scaling["factor"])
    elif kind == "yarn":
        freq = yarn_frequencies(freq, scaling["factor"], scaling.get("beta_slow", 1.0),
                                scaling.get("beta_fast", 32.0), scaling["original_max_pos"])
    return freq


def llama3_scaled_frequencies(freq, factor, low_freq_factor, high_freq_factor, original_max_pos):
    """Llama-3 frequency-dependent RoPE scaling.

    Reading taken (the pages only name the fields): with wavelength
    lambda = 2 pi / freq, wavelengths shorter than original_max_pos /
    high_freq_factor keep their frequency, wavelengths longer than
    original_max_pos / low_freq_factor are divided by ``factor``, and in
    between the frequency is the mix (1 - s) freq / factor + s freq with
    s = (original_max_pos / lambda - low_freq_factor) /
        (high_freq_factor - low_freq_factor).
    s is 1 at the short cutoff and 0 at the long one, so the rule is
    continuous.  Pinned, blend band included, against the frequency table of
    an independently written library initialiser (Hugging Face transformers'
    Llama-3 rule), to fp32 rounding.
    """
    freq = np.asarray(freq, dtype=np.float64)
    out = np.empty_like(freq)
    long_cut = original_max_pos / low_freq_factor
    short_cut = original_max_pos / high_freq_factor
    for i, f in enumerate(freq):
        wavelength = 2.0 * math.pi / f
        if wavelength < short_cut:
            out[i] = f
        elif wavelength > long_cut:
            out[i] = f / factor
        else:
            s = (original_max_pos / wavelength - low_freq_factor) / (high_freq_factor - low_freq_factor)
            out[i] = (1.0 - s) * f / factor + s * f
    return out


def yarn_frequencies(freq, factor, alpha, beta, original_max_pos):
    """YaRN's "NTK-by-parts" frequencies.

    Following the YaRN paper's definition (the pages cite the paper and name
    the method, nothing more): rho = original_max_pos / lambda counts the
    turns pair i makes over the original context.  A ramp gamma(rho) is 0 for
    rho < alpha, 1 for rho > beta and (rho - alpha) / (beta - alpha) between;
    the new frequency is (1 - gamma) freq / factor + gamma freq, so pairs that
    turn many times keep their frequency and pairs that turn less than alpha
    times are interpolated fully.

    The paper's ramp is linear in rho.  The library implementations ramp
    linearly in the pair index, i.e. in ln(rho), between the same two edges;
    the oracle keeps the paper's.  Pinned against Hugging Face transformers'
    YaRN table (untruncated edges): equal outside the ramp, the same ramp
    band, and inside it the paper's gamma of the rho that the library's ramp
    value implies.
    """
    freq = np.asarray(freq, dtype=np.float64)
    rho = original_max_pos * freq / (2.0 * math.pi)
    gamma = np.clip((rho - alpha) / (beta - alpha), 0.0, 1.0)
    return (1.0 - gamma) * freq / factor + gamma * freq


def rope_attention_factor(scaling):
    """Multiplier of the rotated dims: YaRN's attention temperature, else 1.

    The YaRN paper scales the logits by 1/t with sqrt(1/t) = 0.1 ln(s) + 1;
    multiplying both the rotated q and the rotated k by sqrt(1/t) does that.
    ``attn_factor`` in ``scaling``, when given and > 0, replaces the default.
    """
    if scaling is None:
        return 1.0
    given = float(scaling.get("attn_factor", 0.0) or 0.0)
    if given > 0.0:
        return given
    if scaling.get("type", "llama3") == "yarn":
        return 0.1 * math.log(float(scaling["factor"])) + 1.0
    return 1.0


def rotate_pairs(x, angle, layout="interleaved"):
    """Rotate each (a, b) pair of the last axis of ``x`` by ``angle``.

    [P7] key ideas: every pair of query/key dimensions turns by an angle
    proportional to the position.  The rotation is multiplication of a + ib
    by e^{i angle}: (a, b) -> (a cos - b sin, a sin + b cos).  Pair i uses
    ``angle[..., i]``.  [P7] module L7.3 names two pairings:
      interleaved: dims (2i, 2i+1)       half: dims (i, i + d/2)
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    c = np.cos(angle)
    s = np.sin(angle)
    if layout == "interleaved":
        a, b = x[..., 0::2], x[..., 1::2]
    elif layout == "half":
        a, b = x[..., : d // 2], x[..., d // 2:]
    else:
        raise ValueError(f"unknown RoPE layout {layout!r}")
    ra = a * c - b * s
    rb = a * s + b * c
    out = np.empty(np.broadcast_shapes(x.shape, ra.shape[:-1] + (d,)), dtype=np.float64)
    if layout == "interleaved":
        out[..., 0::2], out[..., 1::2] = ra, rb
    else:
        out[..., : d // 2], out[..., d // 2:] = ra, rb
    return out


def rope_rotate(x, pos, theta, layout="interleaved", scaling=None, rotary_dim=None):
    """fp64 RoPE of the last axis of ``x`` (values, not bits) at positions ``pos``.

    The first r dims (r = rotary_dim or d) turn pair by pair by pos * freq_i
    and are multiplied by the attention factor; dims r .. d-1 pass through
    unchanged ([P7] module L7.3 "partial rotary"; reading taken: the half
    layout pairs dim i with i + r/2 inside the rotated part).  ``pos`` has the
    shape of x without its last axis, or broadcasts to it.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    r = d if rotary_dim is None else int(rotary_dim)
    freq = rope_frequencies(theta, d, scaling, r)
    angle = np.asarray(pos, dtype=np.float64)[..., None] * freq
    out = np.array(x, copy=True)
    out[..., :r] = rotate_pairs(x[..., :r], angle, layout) * rope_attention_factor(scaling)
    return out


def rope_append(q, k_new, v_new, k_cache, v_cache, past_len, theta, layout="interleaved", scaling=None,
                rotary_dim=None):
    """RoPE on q and the new k at offset past_len, then write k_rot and v into the cache.

    [KV] "RoPE has to know where it is": new token t of a sequence with
    past_len cached rows sits at position past_len + t.
    [ATL] cache formula: the call writes cache rows past_len .. past_len+T-1
    with the rotated keys and the values; the keys are stored after rotation.
    All other rows keep their contents.  The rotated dims of q_rot and k_rot
    are rounded to bf16 once, from fp64; dims beyond rotary_dim and v are
    copied bit for bit.

    Returns (q_rot, k_cache_out, v_cache_out) as new uint16 arrays.
    """
    q = np.asarray(q, dtype=np.uint16)
    k_new = np.asarray(k_new, dtype=np.uint16)
    v_new = np.asarray(v_new, dtype=np.uint16)
    B, n_q, T, d = q.shape
    S = k_cache.shape[2]
    r = d if rotary_dim is None else int(rotary_dim)
    q_rot = np.array(q, copy=True)
    kc = np.array(k_cache, dtype=np.uint16, copy=True)
    vc = np.array(v_cache, dtype=np.uint16, copy=True)
    for b in range(B):
        pos = int(past_len[b]) + np.arange(T, dtype=np.float64)
        if int(past_len[b]) < 0 or int(past_len[b]) + T > S:
            raise ValueError("past_len + T exceeds the cache")
        qr = rope_rotate(bf16_to_f64(q[b]), pos[None, :], theta, layout, scaling, r)
        kr = rope_rotate(bf16_to_f64(k_new[b]), pos[None, :], theta, layout, scaling, r)
        q_rot[b][..., :r] = f64_to_bf16(qr[..., :r])
        k_rot = np.array(k_new[b], copy=True)
        k_rot[..., :r] = f64_to_bf16(kr[..., :r])
        rows = int(past_len[b]) + np.arange(T)
        kc[b][:, rows, :] = k_rot
        vc[b][:, rows, :] = v_new[b]
    return q_rot, kc, vc


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------


def visible_rows(pos, L, window=0, n_sink=0):
    """Boolean mask over cache rows 0 .. L-1 seen by the query at position pos.

    Causal rule ([ATL] Transformer.forward excerpt): rows 0 .. pos.  With a
    sliding window of W > 0 rows ([P7] modules L7.5 and L7.7 name the window
    and StreamingLLM sinks; reading taken: the query sees its own row and the
    W - 1 rows before it), only rows r > pos - W stay visible, except the first
    n_sink rows (the sinks), which every query keeps seeing.
    """
    r = np.arange(L)
    vis = r <= pos
    if window > 0:
        vis &= (r > pos - window) | (r < n_sink)
    return vis


def attend(q_rot, k_cache, v_cache, past_len, n_kv, scale=None, window=0, n_sink=0, sink_logits=None):
    """Grouped-query attention of the new queries over the cache, in fp64.

    Head map ([REP] formula; [EP18] "Our six heads, three ways"): query head
    h reads KV head floor(h / g) with g = n_q / n_kv.
    Scores ([KV] "The cache itself is concatenation"): q . k / sqrt(d).
    Mask ([ATL] Transformer.forward excerpt): new row t of a sequence with
    past_len P is at position P + t and sees cache rows 0 .. P + t; with a
    window and sinks, see ``visible_rows``.
    Softmax over the visible rows, then the weighted sum of the value rows.
    A learned sink ([P7] L7.5 / L7.7 "learned sinks"; reading taken: one extra
    logit per query head that joins the softmax normaliser and carries no
    value) adds exp(sink_logits[h]) to the denominator.
    Rows at or beyond P + T are never read.

    Returns float64 [B, n_q, T, d].
    """
    q_rot = np.asarray(q_rot, dtype=np.uint16)
    B, n_q, T, d = q_rot.shape
    if n_q % n_kv:
        raise ValueError(f"n_q={n_q} is not a multiple of n_kv={n_kv}")
    g = n_q // n_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, n_q, T, d), dtype=np.float64)
    t_of_row = np.tile(np.arange(T), g)  # rows of the [g*T, L] score block are (head, t)
    for b in range(B):
        P = int(past_len[b])
        L = P + T
        for j in range(n_kv):
            K = bf16_to_f64(k_cache[b, j, :L])
            V = bf16_to_f64(v_cache[b, j, :L])
            Q = bf16_to_f64(q_rot[b, j * g:(j + 1) * g]).reshape(g * T, d)
            s = (Q @ K.T) * scale
            visible = np.stack([visible_rows(P + t, L, window, n_sink) for t in t_of_row])
            s = np.where(visible, s, -np.inf)
            if sink_logits is None:
                top = s.max(axis=1, keepdims=True)
                w = np.exp(s - top)
                w = w / w.sum(axis=1, keepdims=True)
            else:
                sk = np.repeat(np.asarray(sink_logits, dtype=np.float64)[j * g:(j + 1) * g], T)[:, None]
                top = np.maximum(s.max(axis=1, keepdims=True), sk)
                w = np.exp(s - top)
                w = w / (w.sum(axis=1, keepdims=True) + np.exp(sk - top))
            out[b, j * g:(j + 1) * g] = (w @ V).reshape(g, T, d)
    return out


def attend_bruteforce(q_rot, k_cache, v_cache, past_len, n_kv, scale=None, window=0, n_sink=0, sink_logits=None):
    """Second formulation of ``attend`` for tiny shapes: explicit loops.

    It follows the pages' own construction literally: the KV heads are
    first copied out to one per query head ([REP] repeat_kv formula:
    K_G[h] = K[floor(h / g)]), and the additive mask is built as in the [ATL]
    Transformer.forward excerpt: zeros over the past_len cached columns next
    to an upper-triangular -inf block (strictly above the diagonal) over the
    new ones.  Exponentials and sums are plain Python floats.
    """
    q = bf16_to_f64(q_rot)
    B, n_q, T, d = q.shape
    g = n_q // n_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, n_q, T, d), dtype=np.float64)
    for b in range(B):
        P = int(past_len[b])
        L = P + T
        kb = bf16_to_f64(k_cache[b][:, :L])
        vb = bf16_to_f64(v_cache[b][:, :L])
        k_rep = [kb[h // g] for h in range(n_q)]
        v_rep = [vb[h // g] for h in range(n_q)]
        new_block = [[(-math.inf if col > row else 0.0) for col in range(T)] for row in range(T)]
        mask = [[0.0] * P + new_block[row] for row in range(T)]
        if window > 0:  # rows that fell out of the window, other than the sinks
            for t in range(T):
                for r in range(L):
                    if r <= P + t - window and r >= n_sink:
                        mask[t][r] = -math.inf
        for h in range(n_q):
            for t in range(T):
                scores = []
                for r in range(L):
                    dot = 0.0
                    for c in range(d):
                        dot += q[b, h, t, c] * k_rep[h][r, c]
                    scores.append(dot * scale + mask[t][r])
                top = max(scores)
                extra = 0.0
                if sink_logits is not None:
                    top = max(top, float(sink_logits[h]))
                    extra = math.exp(float(sink_logits[h]) - top)
                weights = [math.exp(x - top) for x in scores]
                total = sum(weights) + extra
                for c in range(d):
                    acc = 0.0
                    for r in range(L):
                        acc += weights[r] * v_rep[h][r, c]
                    out[b, h, t, c] = acc / total
    return out


# ---------------------------------------------------------------------------
# sizes
# ---------------------------------------------------------------------------


def kv_cache_bytes(n_layers, n_kv, head_dim, tokens, bytes_per_number):
    """Bytes a KV cache holds: one key and one value per layer, KV head, channel and token.

    [EP18] "The cache's size, and the flags": per token the cache keeps a key
    and a value for each layer, each KV head and each channel of a head.
    """
    return 2 * n_layers * n_kv * head_dim * tokens * bytes_per_number
