// Fused RoPE of q and the new k at offset past_len, plus the cache append of
// the rotated k rows and the v rows.
//
// [KV] "Llama 3.1 8B KV cache", section "RoPE has to know where it is": the
// rotary angle of a new token is its absolute position past_len + t times the
// pair frequency theta^(-2i/d).  [ATL] "Llama 3 8B - KV cache", cache formula:
// the rotated keys and the values are written at rows past_len .. past_len+T-1
// and nothing else in the cache changes.
//
// A token (t, b) is covered by one or more workgroups of 256 threads; each
// thread owns one item: 8 pairs of one head of q or of the new k (two 16-byte
// loads, two 16-byte stores), or 16 values of a v row or of the unrotated
// tail of a q/k head (partial rotary, [P7] module L7.3; copied).  Each
// workgroup computes the d/2 angles of the token's position in fp64 and keeps
// cos/sin in LDS; the item loads are issued before that, since the source rows
// do not depend on past_len.  All global accesses are 16-byte and contiguous
// along d.
#include "common.hpp"
#include "kernels.hpp"
#include "rope_math.hpp"

namespace gqa {

namespace {

// One workgroup covers up to 256 items of one token (t, b); an item is 8 pairs
// of one head (two 16-byte pieces), of q, of the new k, or of v (copied).  The
// source rows do not depend on past_len, so each thread issues its loads
// first; the angles are computed while they are in flight.
template <int D>
__global__ __launch_bounds__(256) void rope_append_kernel(const uint16_t* q, uint16_t* q_rot,
                                                          const uint16_t* __restrict__ k_new,
                                                          const uint16_t* __restrict__ v_new,
                                                          uint16_t* __restrict__ k_cache,
                                                          uint16_t* __restrict__ v_cache,
                                                          const int32_t* __restrict__ past_len, int max_past_len,
                                                          int n_q, int n_kv, int T, int S, RopeDev rp) {
    constexpr int HALF = D / 2;
    constexpr int ITEMS_PER_HEAD = D / 16;  // 8 pairs (16 values) per item
    __shared__ double s_cos[HALF];
    __shared__ double s_sin[HALF];

    const int t = blockIdx.x;
    const int b = blockIdx.y;
    const int P = past_len[b];
    const int heads = n_q + 2 * n_kv;
    const int it = blockIdx.z * blockDim.x + threadIdx.x;
    const bool active = it < heads * ITEMS_PER_HEAD;
    const int head = active ? it / ITEMS_PER_HEAD : 0;
    const int c = it % ITEMS_PER_HEAD;
    const bool is_v = head >= n_q + n_kv, is_k = !is_v && head >= n_q;
    const int R = rp.rotary_dim;          // multiple of 16, <= D (checked on the host)
    const bool turns = !is_v && 16 * c < R;  // else 16 values copied as they are
    // two 16-byte pieces: 8 (a, b) pairs, or 16 values copied
    const uint16_t* src;
    if (is_v)
        src = v_new + ((size_t)(b * n_kv + head - n_q - n_kv) * T + t) * D;
    else
        src = is_k ? k_new + ((size_t)(b * n_kv + head - n_q) * T + t) * D : q + ((size_t)(b * n_q + head) * T + t) * D;
    int off0 = 16 * c, off1 = 16 * c + 8;
    if (turns && rp.layout != 0) {  // half: pair i is dims (i, i + R/2)
        off0 = 8 * c;
        off1 = R / 2 + 8 * c;
    }
    uint4 x0 = make_uint4(0, 0, 0, 0), x1 = x0;
    if (active) {
        x0 = *reinterpret_cast<const uint4*>(src + off0);
        x1 = *reinterpret_cast<const uint4*>(src + off1);
    }

    if (P < 0 || P > max_past_len) return;  // caller error: write nothing for this sequence
    const int pos = P + t;                  // < max_past_len + T <= S (checked on the host)
    for (int i = threadIdx.x; i < R / 2; i += blockDim.x) {
        double ang = (double)pos * rp.freq[i];
        double sn, cs;
        sincos(ang, &sn, &cs);
        s_cos[i] = rp.attn * cs;  // attention factor (1 unless YaRN or given)
        s_sin[i] = rp.attn * sn;
    }
    __syncthreads();
    if (!active) return;

    uint16_t* dst;
    if (is_v)
        dst = v_cache + ((size_t)(b * n_kv + head - n_q - n_kv) * S + pos) * D;
    else
        dst = is_k ? k_cache + ((size_t)(b * n_kv + head - n_q) * S + pos) * D
                   : q_rot + ((size_t)(b * n_q + head) * T + t) * D;
    if (!turns) {
        *reinterpret_cast<uint4*>(dst + off0) = x0;
        *reinterpret_cast<uint4*>(dst + off1) = x1;
        return;
    }
    const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t o[8];
    rotate_item(w, c, rp.layout, s_cos, s_sin, o);
    *reinterpret_cast<uint4*>(dst + off0) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4*>(dst + off1) = make_uint4(o[4], o[5], o[6], o[7]);
}

}  // namespace

hipError_t launch_rope_append(const uint16_t* q, uint16_t* q_rot, const uint16_t* k_new, const uint16_t* v_new,
                              uint16_t* k_cache, uint16_t* v_cache, const int32_t* past_len, int max_past_len,
                              int B, int n_q, int n_kv, int T, int d, int S, const RopeDev& rope, hipStream_t st) {
    // grid.y is limited to 65535 sequences per launch: slice larger batches
    for (int b0 = 0; b0 < B; b0 += 65535) {
        const int nb = (B - b0) < 65535 ? (B - b0) : 65535;
        const int items = (n_q + 2 * n_kv) * (d / 16);
        dim3 grid(T, nb, (items + 255) / 256);
        const size_t qo = (size_t)b0 * n_q * T * d, ko = (size_t)b0 * n_kv * T * d, co = (size_t)b0 * n_kv * S * d;
        prof_begin(K_ROPE_APPEND, st);
        if (d == 128)
            hipLaunchKernelGGL(rope_append_kernel<128>, grid, dim3(256), 0, st, q + qo, q_rot + qo, k_new + ko,
                               v_new + ko, k_cache + co, v_cache + co, past_len + b0, max_past_len, n_q, n_kv, T, S,
                               rope);
        else
            hipLaunchKernelGGL(rope_append_kernel<64>, grid, dim3(256), 0, st, q + qo, q_rot + qo, k_new + ko,
                               v_new + ko, k_cache + co, v_cache + co, past_len + b0, max_past_len, n_q, n_kv, T, S,
                               rope);
        prof_end(K_ROPE_APPEND, st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gqa
