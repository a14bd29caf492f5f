"""MI355X-native grouped-query attention step with RoPE over a bf16 KV cache.

Thin ctypes binding over libgqa.so (``include/gqa.h``).  The functions carry
the C ABI's names and only marshal arguments: every step of the attention
step runs in the library's HIP kernels.  torch is used for device memory and
the current stream, nothing else.  If libgqa.so is missing the first call
raises: there is no fallback path.
"""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgqa.so")

GQA_OK = 0
GQA_ERR_INVALID_ARG = -1
GQA_ERR_GROUP = -2
GQA_ERR_HEAD_DIM = -3
GQA_ERR_RANGE = -4
GQA_ERR_WORKSPACE = -5
GQA_ERR_HIP = -6
GQA_ERR_SCRATCH = -7
GQA_DECODE_NOALLOC_MAX_BYTES = 64 << 20

GQA_ROPE_INTERLEAVED = 0
GQA_ROPE_HALF = 1

# context-extension rules (gqa_rope_params.scaling)
ROPE_SCALING = {None: 0, "llama3": 1, "linear": 2, "ntk": 3, "yarn": 4}

EXPORTED = (
    "gqa_rope_append",
    "gqa_decode_workspace_bytes",
    "gqa_decode_attn",
    "gqa_decode_attn_ex",
    "gqa_decode_attn_noalloc",
    "gqa_prefill_attn",
    "gqa_prefill_attn_ex",
    "gqa_decode_step_workspace_bytes",
    "gqa_decode_step",
    "gqa_status_string",
    "gqa_measure_stream_read",
    "gqa_measure_mfma_rate",
    "gqa_profile_enable",
    "gqa_profile_read",
    "gqa_profile_reset",
    "gqa_set_decode_workgroups",
    "gqa_set_decode_schedule",
    "gqa_set_decode_slot_ratio",
    "gqa_set_decode_wide_min_group",
    "gqa_set_decode_step_split_min_tiles",
)

KERNEL_KINDS = {"rope_append": 0, "decode_partial": 1, "decode_combine": 2, "prefill": 3, "decode_step": 4,
                "decode_wide": 5, "stream_read": 6}


class GqaAttnOpts(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int), ("n_sink", ctypes.c_int), ("sink_logits", ctypes.c_void_p)]


class GqaRopeParams(ctypes.Structure):
    _fields_ = [
        ("theta", ctypes.c_double),
        ("layout", ctypes.c_int),
        ("scaling", ctypes.c_int),
        ("factor", ctypes.c_double),
        ("low_freq_factor", ctypes.c_double),
        ("high_freq_factor", ctypes.c_double),
        ("original_max_pos", ctypes.c_double),
        ("rotary_dim", ctypes.c_int),
        ("attn_factor", ctypes.c_double),
    ]


class GqaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib = None


def lib():
    """Load libgqa.so once; raise if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(hipcc, gfx950); there is no fallback implementation")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    L.gqa_rope_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                  ctypes.POINTER(GqaRopeParams), vp]
    L.gqa_rope_append.restype = i32
    L.gqa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.gqa_decode_workspace_bytes.restype = sz
    L.gqa_decode_attn.argtypes = [vp, vp, vp, vp, i32, vp, vp, sz, i32, i32, i32, i32, i32, f32, vp]
    L.gqa_decode_attn.restype = i32
    L.gqa_decode_attn_ex.argtypes = [vp, vp, vp, vp, i32, vp, vp, sz, i32, i32, i32, i32, i32, f32,
                                     ctypes.POINTER(GqaAttnOpts), vp]
    L.gqa_decode_attn_ex.restype = i32
    L.gqa_decode_attn_noalloc.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, f32,
                                          ctypes.POINTER(GqaAttnOpts), vp]
    L.gqa_decode_attn_noalloc.restype = i32
    L.gqa_prefill_attn.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, f32, vp]
    L.gqa_prefill_attn.restype = i32
    L.gqa_prefill_attn_ex.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, f32,
                                      ctypes.POINTER(GqaAttnOpts), vp]
    L.gqa_prefill_attn_ex.restype = i32
    L.gqa_decode_step_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.gqa_decode_step_workspace_bytes.restype = ctypes.c_size_t
    L.gqa_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, ctypes.c_size_t, i32, i32, i32, i32, i32,
                                  ctypes.POINTER(GqaRopeParams), f32, ctypes.POINTER(GqaAttnOpts), vp]
    L.gqa_decode_step.restype = i32
    L.gqa_measure_stream_read.argtypes = [vp, sz, vp, i32, vp]
    L.gqa_measure_stream_read.restype = i32
    L.gqa_measure_mfma_rate.argtypes = [i32, i32, vp, vp]
    L.gqa_measure_mfma_rate.restype = i32
    L.gqa_status_string.argtypes = [i32]
    L.gqa_status_string.restype = ctypes.c_char_p
    L.gqa_profile_enable.argtypes = [i32]
    L.gqa_profile_enable.restype = i32
    L.gqa_profile_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_longlong)]
    L.gqa_profile_read.restype = i32
    L.gqa_profile_reset.argtypes = []
    L.gqa_profile_reset.restype = i32
    L.gqa_set_decode_workgroups.argtypes = [i32]
    L.gqa_set_decode_workgroups.restype = i32
    L.gqa_set_decode_wide_min_group.argtypes = [i32]
    L.gqa_set_decode_wide_min_group.restype = i32
    L.gqa_set_decode_schedule.argtypes = [i32, i32]
    L.gqa_set_decode_schedule.restype = i32
    L.gqa_set_decode_slot_ratio.argtypes = [i32]
    L.gqa_set_decode_slot_ratio.restype = i32
    L.gqa_set_decode_step_split_min_tiles.argtypes = [i32]
    L.gqa_set_decode_step_split_min_tiles.restype = i32
    _lib = L
    return L


def gqa_status_string(status):
    return lib().gqa_status_string(int(status)).decode()


def _check(status):
    if status == GQA_OK:
        return
    msg = gqa_status_string(status)
    if status in (GQA_ERR_INVALID_ARG, GQA_ERR_GROUP, GQA_ERR_HEAD_DIM, GQA_ERR_RANGE, GQA_ERR_WORKSPACE,
                  GQA_ERR_SCRATCH):
        raise ValueError(f"{msg} (status {status})")
    raise GqaError(status, msg)


# ---------------------------------------------------------------- torch marshalling helpers

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Context under which the binding's temporaries are made: with an explicit stream they are
    allocated (and zero-filled) on that stream, so the caching allocator orders their reuse after
    the library's kernels and the kernels see the fill complete."""
    import contextlib
    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _bf16(t, name, shape=None):
    import torch
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _past(past_len, B):
    import torch
    if past_len.dtype != torch.int32 or not past_len.is_cuda or past_len.numel() != B:
        raise ValueError("past_len must be a device int32 tensor with B entries")
    return past_len.contiguous()


def rope_params(theta, layout="interleaved", scaling=None, rotary_dim=None):
    """gqa_rope_params from a scaling dict.

    scaling: None, or a dict whose "type" is "llama3" (the default; factor,
    low_freq_factor, high_freq_factor, original_max_pos), "linear" (factor),
    "ntk" (factor) or "yarn" (factor, beta_slow, beta_fast, original_max_pos);
    any of them may carry "attn_factor".  rotary_dim: None for all d dims.
    """
    p = GqaRopeParams()
    p.theta = float(theta)
    p.layout = {"interleaved": GQA_ROPE_INTERLEAVED, "half": GQA_ROPE_HALF}[layout]
    kind = None if not scaling else scaling.get("type", "llama3")
    if kind not in ROPE_SCALING:
        raise ValueError(f"unknown RoPE scaling {kind!r}")
    p.scaling = ROPE_SCALING[kind]
    if kind is not None:
        p.factor = float(scaling["factor"])
    if kind == "llama3":
        p.low_freq_factor = float(scaling["low_freq_factor"])
        p.high_freq_factor = float(scaling["high_freq_factor"])
        p.original_max_pos = float(scaling["original_max_pos"])
    elif kind == "yarn":
        p.low_freq_factor = float(scaling.get("beta_slow", 1.0))
        p.high_freq_factor = float(scaling.get("beta_fast", 32.0))
        p.original_max_pos = float(scaling["original_max_pos"])
    p.attn_factor = float(scaling.get("attn_factor", 0.0) or 0.0) if scaling else 0.0
    p.rotary_dim = int(rotary_dim or 0)
    return p


# ---------------------------------------------------------------- entry points

def gqa_rope_append(q, k_new, v_new, k_cache, v_cache, past_len, max_past_len, theta,
                    layout="interleaved", scaling=None, q_rot=None, stream=None, rotary_dim=None):
    """Rotate q and k_new at positions past_len[b] + t and append k_rot, v to the cache.

    q [B, n_q, T, d], k_new/v_new [B, n_kv, T, d], caches [B, n_kv, S, d] (bf16, device),
    past_len int32 [B] (device).  scaling and rotary_dim as in ``rope_params``.  Returns q_rot (a new
    tensor unless given; may be q).
    """
    import torch
    B, n_q, T, d = q.shape
    n_kv, S = k_cache.shape[1], k_cache.shape[2]
    _bf16(q, "q")
    _bf16(k_new, "k_new", (B, n_kv, T, d))
    _bf16(v_new, "v_new", (B, n_kv, T, d))
    _bf16(k_cache, "k_cache", (B, n_kv, S, d))
    _bf16(v_cache, "v_cache", (B, n_kv, S, d))
    p = rope_params(theta, layout, scaling, rotary_dim)
    with _on(stream):
        past_len = _past(past_len, B)
        if q_rot is None:
            q_rot = torch.empty_like(q)
        _bf16(q_rot, "q_rot", (B, n_q, T, d))
        _check(lib().gqa_rope_append(_ptr(q), _ptr(q_rot), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                     _ptr(v_cache), _ptr(past_len), int(max_past_len), B, n_q, n_kv, T, d, S,
                                     ctypes.byref(p), _stream(stream)))
    return q_rot


def gqa_decode_workspace_bytes(B, n_q, n_kv, d, S):
    return int(lib().gqa_decode_workspace_bytes(B, n_q, n_kv, d, S))


def _opts(window, n_sink, sink_logits, n_q, device):
    """Options struct for the _ex entry points (None when every option is off)."""
    import torch
    if window < 0 or n_sink < 0:
        raise ValueError("window and n_sink must be >= 0")
    if not window and sink_logits is None:
        return None, None
    keep = None
    ptr = None
    if sink_logits is not None:
        if not (isinstance(sink_logits, torch.Tensor) and sink_logits.dtype == torch.float32
                and sink_logits.device.type == torch.device(device).type and sink_logits.is_contiguous()
                and sink_logits.numel() == n_q):
            raise ValueError(f"sink_logits must be a contiguous float32 device tensor of {n_q} values")
        keep = sink_logits
        ptr = sink_logits.data_ptr()
    return GqaAttnOpts(int(window), int(n_sink), ptr), keep


def gqa_decode_attn(q_rot, k_cache, v_cache, past_len, max_past_len, out=None, workspace=None, scale=0.0,
                    stream=None, window=0, n_sink=0, sink_logits=None):
    """One new query per sequence attends to cache rows 0..past_len[b] (or its window and sinks);
    returns out [B, n_q, 1, d] bf16."""
    import torch
    B, n_q, T, d = q_rot.shape
    if T != 1:
        raise ValueError("decode takes exactly one new token per sequence")
    n_kv, S = k_cache.shape[1], k_cache.shape[2]
    _bf16(q_rot, "q_rot")
    _bf16(k_cache, "k_cache", (B, n_kv, S, d))
    _bf16(v_cache, "v_cache", (B, n_kv, S, d))
    opts, _keep = _opts(window, n_sink, sink_logits, n_q, q_rot.device)
    need = gqa_decode_workspace_bytes(B, n_q, n_kv, d, S)
    with _on(stream):
        past_len = _past(past_len, B)
        if out is None:
            out = torch.empty_like(q_rot)
        _bf16(out, "out", (B, n_q, 1, d))
        if workspace is None:
            # the scheduling header at the start must be zero before first use
            workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=q_rot.device)
        _check(lib().gqa_decode_attn_ex(_ptr(q_rot), _ptr(k_cache), _ptr(v_cache), _ptr(past_len),
                                        int(max_past_len), _ptr(out), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), B, n_q, n_kv, d, S,
                                        float(scale), ctypes.byref(opts) if opts else None, _stream(stream)))
    return out


def gqa_decode_attn_noalloc(q_rot, k_cache, v_cache, past_len, max_past_len, out, scale=0.0, stream=None,
                            window=0, n_sink=0, sink_logits=None):
    """gqa_decode_attn without a workspace: the library's fixed per-GPU scratch holds the split-K records.
    ``out`` [B, n_q, 1, d] bf16 must be given (nothing is allocated); past_len must already be a contiguous
    device int32 tensor.  Calls that may overlap in time on one GPU race."""
    import torch
    B, n_q, T, d = q_rot.shape
    if T != 1:
        raise ValueError("decode takes exactly one new token per sequence")
    n_kv, S = k_cache.shape[1], k_cache.shape[2]
    _bf16(q_rot, "q_rot")
    _bf16(k_cache, "k_cache", (B, n_kv, S, d))
    _bf16(v_cache, "v_cache", (B, n_kv, S, d))
    _bf16(out, "out", (B, n_q, 1, d))
    if past_len.dtype != torch.int32 or not past_len.is_cuda or past_len.numel() != B or not past_len.is_contiguous():
        raise ValueError("past_len must be a contiguous device int32 tensor with B entries")
    opts, _keep = _opts(window, n_sink, sink_logits, n_q, q_rot.device)
    _check(lib().gqa_decode_attn_noalloc(_ptr(q_rot), _ptr(k_cache), _ptr(v_cache), _ptr(past_len),
                                         int(max_past_len), _ptr(out), B, n_q, n_kv, d, S, float(scale),
                                         ctypes.byref(opts) if opts else None, _stream(stream)))
    return out


def gqa_prefill_attn(q_rot, k_cache, v_cache, past_len, max_past_len, out=None, scale=0.0, stream=None,
                     window=0, n_sink=0, sink_logits=None):
    """T new queries per sequence under the rectangular causal mask (and optional window / sinks);
    returns out [B, n_q, T, d] bf16."""
    import torch
    B, n_q, T, d = q_rot.shape
    n_kv, S = k_cache.shape[1], k_cache.shape[2]
    _bf16(q_rot, "q_rot")
    _bf16(k_cache, "k_cache", (B, n_kv, S, d))
    _bf16(v_cache, "v_cache", (B, n_kv, S, d))
    opts, _keep = _opts(window, n_sink, sink_logits, n_q, q_rot.device)
    with _on(stream):
        past_len = _past(past_len, B)
        if out is None:
            out = torch.empty_like(q_rot)
        _bf16(out, "out", (B, n_q, T, d))
        _check(lib().gqa_prefill_attn_ex(_ptr(q_rot), _ptr(k_cache), _ptr(v_cache), _ptr(past_len),
                                         int(max_past_len), _ptr(out), B, n_q, n_kv, T, d, S, float(scale),
                                         ctypes.byref(opts) if opts else None, _stream(stream)))
    return out


def gqa_decode_step_workspace_bytes(B, n_q, n_kv, d, S):
    return int(lib().gqa_decode_step_workspace_bytes(B, n_q, n_kv, d, S))


def gqa_decode_step(q, k_new, v_new, k_cache, v_cache, past_len, max_past_len, theta, layout="interleaved",
                    scaling=None, rotary_dim=None, out=None, q_rot=None, workspace=None, scale=0.0, stream=None,
                    window=0, n_sink=0, sink_logits=None):
    """One decode step in a single launch: rotate q and k_new at past_len, append k_rot and v_new to the
    caches, attend over rows 0..past_len (or the window and sinks).  Returns out [B, n_q, 1, d] bf16;
    q_rot, when given, receives the rotated q.  A workspace must start zeroed (the default one is)."""
    import torch
    B, n_q, T, d = q.shape
    if T != 1:
        raise ValueError("decode takes exactly one new token per sequence")
    n_kv, S = k_cache.shape[1], k_cache.shape[2]
    _bf16(q, "q")
    _bf16(k_new, "k_new", (B, n_kv, 1, d))
    _bf16(v_new, "v_new", (B, n_kv, 1, d))
    _bf16(k_cache, "k_cache", (B, n_kv, S, d))
    _bf16(v_cache, "v_cache", (B, n_kv, S, d))
    if q_rot is not None:
        _bf16(q_rot, "q_rot", (B, n_q, 1, d))
    need = gqa_decode_step_workspace_bytes(B, n_q, n_kv, d, S)
    p = rope_params(theta, layout, scaling, rotary_dim)
    opts, _keep = _opts(window, n_sink, sink_logits, n_q, q.device)
    with _on(stream):
        past_len = _past(past_len, B)
        if out is None:
            out = torch.empty_like(q)
        _bf16(out, "out", (B, n_q, 1, d))
        if workspace is None:
            workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
        _check(lib().gqa_decode_step(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(past_len), int(max_past_len), _ptr(out),
                                     _ptr(q_rot) if q_rot is not None else None, _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), B, n_q, n_kv, d, S,
                                     ctypes.byref(p), float(scale), ctypes.byref(opts) if opts else None,
                                     _stream(stream)))
    return out


def gqa_measure_stream_read(buf, sink, workgroups, stream=None):
    """Read all of ``buf`` (a device tensor, size a multiple of 16 bytes) once with the library's streaming
    kernel (the HBM read ceiling); ``sink`` is a device int32 tensor of at least ``workgroups`` entries."""
    _check(lib().gqa_measure_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), int(workgroups),
                                         _stream(stream)))


def gqa_measure_mfma_rate(workgroups, iters, sink, stream=None):
    """Run the library's matrix-rate probe: ``workgroups`` workgroups of 4 waves, each wave issuing
    ``iters`` x 8 bf16 16x16x32 MFMAs (16384 flops each) on random operands.  ``sink`` is a device int64
    tensor of at least 8 * workgroups entries; per workgroup, entries 4 and 5 receive wave 0's shader-clock
    cycles and 100 MHz ticks over its loop."""
    _check(lib().gqa_measure_mfma_rate(int(workgroups), int(iters), _ptr(sink), _stream(stream)))


def gqa_profile_enable(on=True):
    _check(lib().gqa_profile_enable(1 if on else 0))


def gqa_profile_reset():
    _check(lib().gqa_profile_reset())


def gqa_profile_read(kind):
    """(total device ms, launches) of one kernel kind since the last reset."""
    k = KERNEL_KINDS[kind] if isinstance(kind, str) else int(kind)
    ms = ctypes.c_double()
    n = ctypes.c_longlong()
    _check(lib().gqa_profile_read(k, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def gqa_set_decode_workgroups(n):
    return int(lib().gqa_set_decode_workgroups(int(n)))


def gqa_set_decode_schedule(static_permille=-1, chunk_tiles=0):
    """Static fraction (per mille) and dynamic chunk size of the decode split; (-1, 0) = defaults."""
    _check(lib().gqa_set_decode_schedule(int(static_permille), int(chunk_tiles)))


def gqa_set_decode_slot_ratio(ratio_permille=0):
    """Static share of each dispatch slot relative to the next younger one (per mille); 0 = the kernel
    variant's default.  Returns the override in effect (clamped to [250, 8000]; 0 for the defaults)."""
    return int(lib().gqa_set_decode_slot_ratio(int(ratio_permille)))


def gqa_set_decode_step_split_min_tiles(tiles=0):
    """Tile bound from which gqa_decode_step runs as rope_append + split-K decode (0 restores the default, 512;
    a large value keeps every step in one launch).  Returns the value in effect."""
    return int(lib().gqa_set_decode_step_split_min_tiles(int(tiles)))


def gqa_set_decode_wide_min_group(g=0):
    """Smallest group size the wide-group decode kernel takes; 0 = default, > 64 = off."""
    return int(lib().gqa_set_decode_wide_min_group(int(g)))
