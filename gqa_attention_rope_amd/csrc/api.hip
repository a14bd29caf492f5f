// C ABI of libgqa: argument validation, workspace sizing, launch, status text,
// and the optional kernel-timing hooks.  Every check runs on the host before
// any HIP call, so an invalid call launches nothing.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "gqa.h"
#include "kernels.hpp"
#include "measure.hpp"

// Decode scratch of gqa_decode_attn_noalloc: one copy per GPU, allocated when
// the code object is loaded and held until the process ends.  In host code
// this name is only a stand-in for the symbol; the device address of each
// GPU's copy comes from hipGetSymbolAddress (decode_scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[GQA_DECODE_NOALLOC_MAX_BYTES];

namespace gqa {

hipError_t device_cu_count(int* n) {
    constexpr int MAX_DEVICES = 64;
    static std::atomic<int> cache[MAX_DEVICES] = {};  // 0: not looked up yet
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < MAX_DEVICES;
    if (cached) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *n = c;
            return hipSuccess;
        }
    }
    int c = 0;
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (c < 1) c = 1;
    if (cached) cache[dev].store(c, std::memory_order_relaxed);
    *n = c;
    return hipSuccess;
}

}  // namespace gqa

namespace {

thread_local char g_hip_msg[256] = "";

int hip_status(hipError_t e) {
    snprintf(g_hip_msg, sizeof(g_hip_msg), "%s (%d)", hipGetErrorString(e), (int)e);
    return GQA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks common to every entry point.
int check_shape(int B, int n_q, int n_kv, int T, int d, int S, int max_past_len) {
    if (B <= 0 || n_q <= 0 || n_kv <= 0 || T <= 0 || d <= 0 || S <= 0) return GQA_ERR_INVALID_ARG;
    if (d & 1) return GQA_ERR_INVALID_ARG;
    if (n_q % n_kv) return GQA_ERR_GROUP;
    if (d != 64 && d != 128) return GQA_ERR_HEAD_DIM;
    if (max_past_len < 0 || (long long)max_past_len + T > (long long)S) return GQA_ERR_RANGE;
    // one KV head's cache slab is addressed with 32-bit byte offsets
    if ((long long)S * d * 2 > 0x7fffffffLL) return GQA_ERR_INVALID_ARG;
    return GQA_OK;
}

int ensure_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    int n = 0;
    e = hipGetDeviceCount(&n);
    if (e != hipSuccess) return hip_status(e);
    if (n <= 0) return hip_status(hipErrorNoDevice);
    return GQA_OK;
}

float resolve_scale(float scale, int d) { return scale > 0.f ? scale : 1.0f / sqrtf((float)d); }

// ---- kernel timing -------------------------------------------------------------
struct EvPair {
    hipEvent_t a, b;
};
bool g_prof_on = false;
std::vector<EvPair> g_prof[gqa::K_KINDS];
hipEvent_t g_pending[gqa::K_KINDS] = {};

int g_decode_wg = 0;

// ---- no-allocation decode: per-device address of `scratch` -----------------
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SCRATCH_MAX_DEVICES] = {};

// Address of the current device's copy of `scratch`, looked up once per
// device with that device current.
int decode_scratch_ptr(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hip_status(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!p) return hip_status(hipErrorInvalidSymbol);
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return GQA_OK;
}

// Zeroes the decode workspace header (the split-K ticket counter) at the start
// of every no-allocation call: the scratch holds whatever the last call on
// this GPU left, and a fill kernel (not a memset node) keeps the call
// capturable.
__global__ void clear_header_kernel(float* ws) {
    if (threadIdx.x < gqa::DECODE_WS_HEADER_FLOATS) ws[threadIdx.x] = 0.f;
}

}  // namespace

namespace gqa {

void prof_begin(int kind, hipStream_t st) {
    if (!g_prof_on) return;
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return;
    if (hipEventRecord(e, st) != hipSuccess) {  // no timing for this launch
        (void)hipEventDestroy(e);
        return;
    }
    g_pending[kind] = e;
}

void prof_end(int kind, hipStream_t st) {
    if (!g_prof_on || !g_pending[kind]) return;
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess || hipEventRecord(e, st) != hipSuccess) {
        if (e) (void)hipEventDestroy(e);
        (void)hipEventDestroy(g_pending[kind]);
        g_pending[kind] = nullptr;
        return;
    }
    g_prof[kind].push_back(EvPair{g_pending[kind], e});
    g_pending[kind] = nullptr;
}

}  // namespace gqa

// Pair frequency over the r rotated dims, base^(-2i/r), then the context
// extension rule ([P7] module L7.4 names PI, NTK, YaRN and Llama-3 scaling;
// [KV] "Training details that matter" names the Llama-3 fields; the pages give
// no formulas, so each rule is its published definition):
//   the wavelength ramp shared by Llama-3 scaling and YaRN: short wavelengths
//     keep their frequency, long ones are divided by the factor, and the band
//     between blends the two linearly in original_max_pos / wavelength (the
//     turns the pair makes over the original context);
//   position interpolation: every frequency divided by the factor;
//   NTK-aware scaling only changes the base.
// Computed in fp64 on the host, once per call: the kernels multiply the
// position by these values and take sin / cos of the product.
static double pair_frequency(int i, int r, double base, int sc, const gqa_rope_params* rope) {
    double f = pow(base, -(2.0 * (double)i) / (double)r);
    if (sc == GQA_ROPE_SCALING_LLAMA3 || sc == GQA_ROPE_SCALING_YARN) {
        const double two_pi = 6.283185307179586476925286766559;
        const double wavelength = two_pi / f;
        const double long_cut = rope->original_max_pos / rope->low_freq_factor;
        const double short_cut = rope->original_max_pos / rope->high_freq_factor;
        if (wavelength < short_cut) {
            // unchanged
        } else if (wavelength > long_cut) {
            f = f / rope->factor;
        } else {
            const double s = (rope->original_max_pos / wavelength - rope->low_freq_factor) /
                             (rope->high_freq_factor - rope->low_freq_factor);
            f = (1.0 - s) * f / rope->factor + s * f;
        }
    } else if (sc == GQA_ROPE_SCALING_LINEAR) {
        f = f / rope->factor;
    }
    return f;
}

// Validate RoPE parameters for head size d and fill the device-side form.
static int make_rope(const gqa_rope_params* rope, int d, gqa::RopeDev& rd) {
    if (!(rope->theta > 0.0) || !isfinite(rope->theta)) return GQA_ERR_INVALID_ARG;
    if (rope->layout != GQA_ROPE_INTERLEAVED && rope->layout != GQA_ROPE_HALF) return GQA_ERR_INVALID_ARG;
    const int sc = rope->scaling;
    if (sc < GQA_ROPE_SCALING_NONE || sc > GQA_ROPE_SCALING_YARN) return GQA_ERR_INVALID_ARG;
    if (sc != GQA_ROPE_SCALING_NONE) {
        if (!(rope->factor > 0.0) || !isfinite(rope->factor)) return GQA_ERR_INVALID_ARG;
        if (sc != GQA_ROPE_SCALING_LLAMA3 && !(rope->factor >= 1.0)) return GQA_ERR_INVALID_ARG;
        if (sc == GQA_ROPE_SCALING_LLAMA3 || sc == GQA_ROPE_SCALING_YARN) {
            if (!(rope->low_freq_factor > 0.0) || !(rope->high_freq_factor > rope->low_freq_factor) ||
                !(rope->original_max_pos > 0.0) || !isfinite(rope->high_freq_factor) ||
                !isfinite(rope->original_max_pos))
                return GQA_ERR_INVALID_ARG;
        }
    }
    if (!(rope->attn_factor >= 0.0) || !isfinite(rope->attn_factor)) return GQA_ERR_INVALID_ARG;
    const int rdim = rope->rotary_dim == 0 ? d : rope->rotary_dim;
    if (rdim < 16 || rdim % 16 || rdim > d || rdim / 2 > (int)(sizeof(rd.freq) / sizeof(rd.freq[0])))
        return GQA_ERR_INVALID_ARG;
    rd.layout = rope->layout;
    rd.rotary_dim = rdim;
    rd.attn = 1.0;
    double base = rope->theta;
    if (sc == GQA_ROPE_SCALING_YARN) rd.attn = 0.1 * log(rope->factor) + 1.0;
    if (sc == GQA_ROPE_SCALING_NTK) base = rope->theta * pow(rope->factor, (double)rdim / (double)(rdim - 2));
    if (rope->attn_factor > 0.0) rd.attn = rope->attn_factor;
    for (int i = 0; i < (int)(sizeof(rd.freq) / sizeof(rd.freq[0])); ++i)
        rd.freq[i] = i < rdim / 2 ? pair_frequency(i, rdim, base, sc, rope) : 0.0;
    return GQA_OK;
}

extern "C" {


int gqa_rope_append(const void* q, void* q_rot, const void* k_new, const void* v_new, void* k_cache,
                    void* v_cache, const int32_t* past_len, int max_past_len, int B, int n_q, int n_kv, int T,
                    int d, int S, const gqa_rope_params* rope, void* stream) {
    if (!q || !q_rot || !k_new || !v_new || !k_cache || !v_cache || !past_len || !rope) return GQA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(q_rot) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
        !aligned16(v_cache) || (reinterpret_cast<uintptr_t>(past_len) & 3u))
        return GQA_ERR_INVALID_ARG;
    int st = check_shape(B, n_q, n_kv, T, d, S, max_past_len);
    if (st != GQA_OK) return st;
    gqa::RopeDev rd;
    st = make_rope(rope, d, rd);
    if (st != GQA_OK) return st;
    st = ensure_device();
    if (st != GQA_OK) return st;
    hipError_t e = gqa::launch_rope_append(
        static_cast<const uint16_t*>(q), static_cast<uint16_t*>(q_rot), static_cast<const uint16_t*>(k_new),
        static_cast<const uint16_t*>(v_new), static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
        past_len, max_past_len, B, n_q, n_kv, T, d, S, rd, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GQA_OK : hip_status(e);
}

size_t gqa_decode_workspace_bytes(int B, int n_q, int n_kv, int d, int S) {
    if (check_shape(B, n_q, n_kv, 1, d, S, 0) != GQA_OK) return 0;
    return gqa::decode_workspace_bytes(B, n_q, n_kv, d);
}

int gqa_decode_attn_ex(const void* q_rot, const void* k_cache, const void* v_cache, const int32_t* past_len,
                       int max_past_len, void* out, void* workspace, size_t workspace_bytes, int B, int n_q, int n_kv,
                       int d, int S, float scale, const gqa_attn_opts* opts, void* stream) {
    if (!q_rot || !k_cache || !v_cache || !past_len || !out || !workspace) return GQA_ERR_INVALID_ARG;
    const gqa_attn_opts o = opts ? *opts : gqa_attn_opts{0, 0, nullptr};
    if (o.window < 0 || o.n_sink < 0 || (o.sink_logits && (reinterpret_cast<uintptr_t>(o.sink_logits) & 3u)))
        return GQA_ERR_INVALID_ARG;
    if (!aligned16(q_rot) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        !aligned16(workspace) || (reinterpret_cast<uintptr_t>(past_len) & 3u))
        return GQA_ERR_INVALID_ARG;
    if (!(scale == scale) || isinf(scale)) return GQA_ERR_INVALID_ARG;
    int st = check_shape(B, n_q, n_kv, 1, d, S, max_past_len);
    if (st != GQA_OK) return st;
    if (workspace_bytes < gqa::decode_workspace_bytes(B, n_q, n_kv, d)) return GQA_ERR_WORKSPACE;
    st = ensure_device();
    if (st != GQA_OK) return st;
    hipError_t e = gqa::launch_decode(static_cast<const uint16_t*>(q_rot), static_cast<const uint16_t*>(k_cache),
                                      static_cast<const uint16_t*>(v_cache), past_len, max_past_len,
                                      static_cast<uint16_t*>(out), static_cast<float*>(workspace), B, n_q, n_kv, d,
                                      S, resolve_scale(scale, d), o.window, o.n_sink, o.sink_logits, g_decode_wg,
                                      static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GQA_OK : hip_status(e);
}

int gqa_decode_attn(const void* q_rot, const void* k_cache, const void* v_cache, const int32_t* past_len,
                    int max_past_len, void* out, void* workspace, size_t workspace_bytes, int B, int n_q, int n_kv,
                    int d, int S, float scale, void* stream) {
    return gqa_decode_attn_ex(q_rot, k_cache, v_cache, past_len, max_past_len, out, workspace, workspace_bytes, B,
                              n_q, n_kv, d, S, scale, nullptr, stream);
}

int gqa_decode_attn_noalloc(const void* q_rot, const void* k_cache, const void* v_cache, const int32_t* past_len,
                            int max_past_len, void* out, int B, int n_q, int n_kv, int d, int S, float scale,
                            const gqa_attn_opts* opts, void* stream) {
    if (!q_rot || !k_cache || !v_cache || !past_len || !out) return GQA_ERR_INVALID_ARG;
    const gqa_attn_opts o = opts ? *opts : gqa_attn_opts{0, 0, nullptr};
    if (o.window < 0 || o.n_sink < 0 || (o.sink_logits && (reinterpret_cast<uintptr_t>(o.sink_logits) & 3u)))
        return GQA_ERR_INVALID_ARG;
    if (!aligned16(q_rot) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(past_len) & 3u))
        return GQA_ERR_INVALID_ARG;
    if (!(scale == scale) || isinf(scale)) return GQA_ERR_INVALID_ARG;
    int st = check_shape(B, n_q, n_kv, 1, d, S, max_past_len);
    if (st != GQA_OK) return st;
    if (gqa::decode_launch_workspace_bytes(B, n_q, n_kv, d) > (size_t)GQA_DECODE_NOALLOC_MAX_BYTES)
        return GQA_ERR_SCRATCH;
    st = ensure_device();
    if (st != GQA_OK) return st;
    void* ws = nullptr;
    st = decode_scratch_ptr(&ws);
    if (st != GQA_OK) return st;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(clear_header_kernel, dim3(1), dim3(64), 0, hs, static_cast<float*>(ws));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e);
    e = gqa::launch_decode(static_cast<const uint16_t*>(q_rot), static_cast<const uint16_t*>(k_cache),
                           static_cast<const uint16_t*>(v_cache), past_len, max_past_len,
                           static_cast<uint16_t*>(out), static_cast<float*>(ws), B, n_q, n_kv, d, S,
                           resolve_scale(scale, d), o.window, o.n_sink, o.sink_logits, g_decode_wg, hs);
    return e == hipSuccess ? GQA_OK : hip_status(e);
}

size_t gqa_decode_step_workspace_bytes(int B, int n_q, int n_kv, int d, int S) {
    if (check_shape(B, n_q, n_kv, 1, d, S, 0) != GQA_OK) return 0;
    if (n_q / n_kv > GQA_DECODE_STEP_MAX_GROUP || B > 65535 || n_kv > 65535) return 0;
    return gqa::decode_step_workspace_bytes(B, n_q, n_kv, d);
}

int gqa_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                    const int32_t* past_len, int max_past_len, void* out, void* q_rot, void* workspace,
                    size_t workspace_bytes, int B, int n_q, int n_kv, int d, int S, const gqa_rope_params* rope,
                    float scale, const gqa_attn_opts* opts, void* stream) {
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !past_len || !out || !workspace || !rope)
        return GQA_ERR_INVALID_ARG;
    const gqa_attn_opts o = opts ? *opts : gqa_attn_opts{0, 0, nullptr};
    if (o.window < 0 || o.n_sink < 0 || (o.sink_logits && (reinterpret_cast<uintptr_t>(o.sink_logits) & 3u)))
        return GQA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned16(out) || (q_rot && !aligned16(q_rot)) || !aligned16(workspace) ||
        (reinterpret_cast<uintptr_t>(past_len) & 3u))
        return GQA_ERR_INVALID_ARG;
    if (!(scale == scale) || isinf(scale)) return GQA_ERR_INVALID_ARG;
    int st = check_shape(B, n_q, n_kv, 1, d, S, max_past_len);
    if (st != GQA_OK) return st;
    if (n_q / n_kv > GQA_DECODE_STEP_MAX_GROUP || B > 65535 || n_kv > 65535) return GQA_ERR_INVALID_ARG;
    gqa::RopeDev rd;
    st = make_rope(rope, d, rd);
    if (st != GQA_OK) return st;
    if (workspace_bytes < gqa::decode_step_workspace_bytes(B, n_q, n_kv, d)) return GQA_ERR_WORKSPACE;
    st = ensure_device();
    if (st != GQA_OK) return st;
    hipError_t e = gqa::launch_decode_step(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
        static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), past_len, max_past_len,
        static_cast<uint16_t*>(out), static_cast<uint16_t*>(q_rot), workspace, workspace_bytes, B, n_q, n_kv, d, S, rd,
        resolve_scale(scale, d), o.window, o.n_sink, o.sink_logits, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GQA_OK : hip_status(e);
}

int gqa_prefill_attn_ex(const void* q_rot, const void* k_cache, const void* v_cache, const int32_t* past_len,
                        int max_past_len, void* out, int B, int n_q, int n_kv, int T, int d, int S, float scale,
                        const gqa_attn_opts* opts, void* stream) {
    if (!q_rot || !k_cache || !v_cache || !past_len || !out) return GQA_ERR_INVALID_ARG;
    const gqa_attn_opts o = opts ? *opts : gqa_attn_opts{0, 0, nullptr};
    if (o.window < 0 || o.n_sink < 0 || (o.sink_logits && (reinterpret_cast<uintptr_t>(o.sink_logits) & 3u)))
        return GQA_ERR_INVALID_ARG;
    if (!aligned16(q_rot) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(past_len) & 3u))
        return GQA_ERR_INVALID_ARG;
    if (!(scale == scale) || isinf(scale)) return GQA_ERR_INVALID_ARG;
    int st = check_shape(B, n_q, n_kv, T, d, S, max_past_len);
    if (st != GQA_OK) return st;
    if (n_kv > 65535) return GQA_ERR_INVALID_ARG;
    st = ensure_device();
    if (st != GQA_OK) return st;
    hipError_t e = gqa::launch_prefill(static_cast<const uint16_t*>(q_rot), static_cast<const uint16_t*>(k_cache),
                                       static_cast<const uint16_t*>(v_cache), past_len, max_past_len,
                                       static_cast<uint16_t*>(out), B, n_q, n_kv, T, d, S, resolve_scale(scale, d),
                                       o.window, o.n_sink, o.sink_logits, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GQA_OK : hip_status(e);
}

int gqa_prefill_attn(const void* q_rot, const void* k_cache, const void* v_cache, const int32_t* past_len,
                     int max_past_len, void* out, int B, int n_q, int n_kv, int T, int d, int S, float scale,
                     void* stream) {
    return gqa_prefill_attn_ex(q_rot, k_cache, v_cache, past_len, max_past_len, out, B, n_q, n_kv, T, d, S, scale,
                               nullptr, stream);
}

const char* gqa_status_string(int status) {
    switch (status) {
        case GQA_OK: return "ok";
        case GQA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, non-positive size, odd d, bad RoPE parameters)";
        case GQA_ERR_GROUP: return "n_q is not a multiple of n_kv";
        case GQA_ERR_HEAD_DIM: return "head dimension must be 64 or 128";
        case GQA_ERR_RANGE: return "max_past_len must be >= 0 and max_past_len + T <= S";
        case GQA_ERR_WORKSPACE: return "workspace smaller than gqa_decode_workspace_bytes()";
        case GQA_ERR_SCRATCH:
            return "shape needs more decode scratch than the fixed no-allocation buffer holds "
                   "(its split-K records exceed GQA_DECODE_NOALLOC_MAX_BYTES)";
        case GQA_ERR_HIP: return g_hip_msg[0] ? g_hip_msg : "HIP error";
        default: return "unknown status";
    }
}

int gqa_measure_stream_read(const void* buf, size_t bytes, void* sink, int workgroups, void* stream) {
    if (!buf || !sink || !aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u) || (bytes & 15u) ||
        workgroups < 1 || workgroups > 65535)
        return GQA_ERR_INVALID_ARG;
    int st = ensure_device();
    if (st != GQA_OK) return st;
    hipError_t e = gqa::launch_stream_read(buf, bytes, static_cast<uint32_t*>(sink), workgroups,
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GQA_OK : hip_status(e);
}

int gqa_measure_mfma_rate(int workgroups, int iters, void* sink, void* stream) {
    if (!sink || (reinterpret_cast<uintptr_t>(sink) & 7u) || workgroups < 1 || workgroups > 65535 || iters < 1 ||
        iters > (1 << 24))
        return GQA_ERR_INVALID_ARG;
    int st = ensure_device();
    if (st != GQA_OK) return st;
    hipError_t e = gqa::launch_mfma_rate(static_cast<unsigned long long*>(sink), workgroups, iters,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GQA_OK : hip_status(e);
}

int gqa_profile_enable(int on) {
    g_prof_on = on != 0;
    return GQA_OK;
}

int gqa_profile_read(int kind, double* total_ms, long long* launches) {
    if (kind < 0 || kind >= gqa::K_KINDS || !total_ms || !launches) return GQA_ERR_INVALID_ARG;
    double sum = 0.0;
    for (const EvPair& p : g_prof[kind]) {
        hipError_t e = hipEventSynchronize(p.b);
        if (e != hipSuccess) return hip_status(e);
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, p.a, p.b);
        if (e != hipSuccess) return hip_status(e);
        sum += ms;
    }
    *total_ms = sum;
    *launches = (long long)g_prof[kind].size();
    return GQA_OK;
}

int gqa_profile_reset(void) {
    for (int k = 0; k < gqa::K_KINDS; ++k) {
        for (const EvPair& p : g_prof[k]) {
            (void)hipEventDestroy(p.a);
            (void)hipEventDestroy(p.b);
        }
        g_prof[k].clear();
        if (g_pending[k]) {
            (void)hipEventDestroy(g_pending[k]);
            g_pending[k] = nullptr;
        }
    }
    return GQA_OK;
}

int gqa_set_decode_workgroups(int n) {
    g_decode_wg = n < 0 ? 0 : (n > gqa::DECODE_MAX_WG ? gqa::DECODE_MAX_WG : n);
    return g_decode_wg;
}

int gqa_set_decode_wide_min_group(int g) {
    gqa::set_decode_wide_min_group(g);
    return gqa::decode_wide_min_group();
}

int gqa_set_decode_slot_ratio(int ratio_permille) {
    int r = ratio_permille;
    if (r > 0) r = r < 250 ? 250 : (r > 8000 ? 8000 : r);
    else r = 0;
    gqa::set_decode_slot_ratio(r);
    return gqa::decode_slot_ratio();
}

int gqa_set_decode_step_split_min_tiles(int tiles) {
    gqa::set_decode_step_split_min_tiles(tiles);
    return gqa::decode_step_split_min_tiles();
}

int gqa_set_decode_schedule(int static_permille, int chunk_tiles) {
    if (static_permille < 0 && chunk_tiles <= 0) {
        gqa::set_decode_schedule(-1, gqa::DECODE_DEFAULT_CHUNK);  // static fraction chosen per launch
        return GQA_OK;
    }
    if (static_permille < 0 || static_permille > 1000 || chunk_tiles < 1) return GQA_ERR_INVALID_ARG;
    gqa::set_decode_schedule(static_permille, chunk_tiles);
    return GQA_OK;
}

}  // extern "C"
