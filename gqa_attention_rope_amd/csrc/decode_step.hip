// One decode step in a single launch, for small batches: RoPE of q and of the
// new k at position past_len, the cache append of k_rot and v, attention of
// the new query over cache rows 0 .. past_len, and the merge of the splits.
//
// What is computed is the three-call path (rope_append, then the split-K
// attention and its combine): [KV] "Llama 3.1 8B KV cache", "RoPE has to know
// where it is" (angle = position * frequency) and "The cache itself is
// concatenation" (keys are cached after rotation, the new query attends to
// every cached row and to its own); [ATL] "Llama 3 8B - KV cache", cache
// formula (the call writes row past_len) and the Transformer.forward excerpt
// (write the new rows, then attend over 0 .. start_pos + seqlen); [REP]
// "Llama 3.1 8B - Repeat heads" formula (query head h reads KV head h / g).
//
// Why one launch: at one or a few sequences the step reads a few MB of K/V, a
// fraction of a microsecond of HBM time, and three dependent launches with
// their gaps cost more than the work.
//
// How:
//  * Grid (split, KV head j, sequence b); 4 waves per workgroup.  The tiles of
//    the (b, j) segment (64 cache rows each; only the sink and window tiles
//    under a window) are cut into nsplit contiguous ranges, one per split.
//  * Every workgroup issues its first K/V tile loads and its raw q rows, then
//    builds the fp64 angle table of position past_len and rotates the g query
//    rows of its group into LDS (rounded once to bf16, as the three-call path
//    stores q_rot).  Split 0 also writes q_rot out when asked.
//  * The last split holds the tile with row past_len.  It rotates k_new,
//    writes k_rot and v_new to cache row past_len, and puts the new row into
//    its staged tile in registers.  No workgroup reads row past_len from
//    memory (the load descriptors cover rows 0 .. past_len - 1 only), so the
//    result does not depend on when the append lands.
//  * q.k: wave w handles heads w, w+4, ..; lane r owns row r of the tile (K
//    stored in LDS with an XOR swizzle so the 64 lanes read distinct banks),
//    v_dot2_f32_bf16 over the head dimension.  Online softmax per head with
//    wave reductions; the weights go through LDS; for the weighted value sum
//    lane r owns value dims of all the wave's heads.
//  * Each split writes one (max, sum, unnormalised output) record per head,
//    written through to memory, and counts itself on the segment's counter.
//    The workgroup that brings the count to nsplit merges
//    the nsplit records in split order (a learned sink logit joins the
//    denominator) and writes the bf16 output, then clears the counter for the
//    next call.  The merge order is fixed, so the result is reproducible.
#include <float.h>

#include "attn_window.hpp"
#include "common.hpp"
#include "kernels.hpp"
#include "rope_math.hpp"

namespace gqa {

namespace {

constexpr int ST_THREADS = 256;
constexpr int ST_TILE = 64;
constexpr float ST_LOG2E = 1.4426950408889634f;
constexpr uint32_t ST_RSRC = 0x00020000u;  // raw buffer, 32-bit dwords

// Wave-wide max and sum with every lane receiving the result, in registers:
// DPP inside each row of 16 (quad_perm [1,0,3,2], [2,3,0,1], then row_ror:4
// and row_ror:8, which bring in the other three quads of the row), then the
// rows paired with v_permlane16_swap and v_permlane32_swap.  No LDS permutes.
// The sum is associated differently in different lanes; each lane's order is
// fixed, so every lane's result is reproducible.
template <bool MAX>
__device__ __forceinline__ float wave_reduce(float v) {
    auto op = [](float a, float b) { return MAX ? __builtin_elementwise_maximum(a, b) : a + b; };
    v = op(v, dpp_f32<0xB1>(v));
    v = op(v, dpp_f32<0x4E>(v));
    v = op(v, dpp_f32<0x124>(v));
    v = op(v, dpp_f32<0x128>(v));
    const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
    const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
}
__device__ __forceinline__ float wave_max(float v) { return wave_reduce<true>(v); }
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce<false>(v); }

// D head size, HPW most heads one wave handles (g <= 4 * HPW)
template <int D, int HPW>
__global__ __launch_bounds__(ST_THREADS) void decode_step_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache, const int32_t* __restrict__ past_len,
    int max_past_len, uint16_t* __restrict__ out, uint16_t* __restrict__ q_rot_out, float* __restrict__ recs,
    int* __restrict__ counters, int n_q, int n_kv, int S, int nsplit, float scale_log2, RopeDev rp, int window,
    int n_sink, const float* __restrict__ sink_logits) {
    constexpr int PPR = D / 8;                      // 16-byte pieces per row
    constexpr int ROWB = D * 2;                     // bytes per row
    constexpr int TILEB = ST_TILE * ROWB;           // bytes per tile of one tensor
    constexpr int LOADS = TILEB / (16 * ST_THREADS);  // 16-byte loads per thread per tile and tensor
    constexpr int DPL = D / 64;                     // value dims per lane
    constexpr int IPH = D / 16;                     // rotation items per head (8 pairs each)
    constexpr int MAXG = 4 * HPW;
    constexpr int MAXIT = (MAXG * IPH + 2 * IPH + ST_THREADS - 1) / ST_THREADS;
    constexpr int REC = D + 4;                      // m, l, 2 pad, o[D]

    __shared__ __align__(16) unsigned char s_k[TILEB];
    __shared__ __align__(16) unsigned char s_v[TILEB];
    __shared__ __align__(16) unsigned char s_q[MAXG * ROWB];  // rotated q rows of the group
    __shared__ __align__(16) unsigned char s_new[2][ROWB];    // rotated new k row, new v row
    __shared__ __align__(16) float s_p[MAXG][ST_TILE];        // softmax weights of a tile
    __shared__ double s_cos[D / 2], s_sin[D / 2];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sp = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int g = n_q / n_kv;
    const int Praw = past_len[b];
    const bool pvalid = Praw >= 0 && Praw <= max_past_len;  // else: write nothing, output unspecified
    const int P = Praw < 0 ? 0 : (Praw > max_past_len ? max_past_len : Praw);
    const int L = P + 1;
    const Geo geo = geo_of(L, window, n_sink);
    const int t0 = (int)((long long)sp * geo.nt / nsplit);
    const int t1 = (int)((long long)(sp + 1) * geo.nt / nsplit);
    const bool owner = sp == nsplit - 1;  // its range ends with the tile holding row P
    const int R = rp.rotary_dim;

    // ---- raw q rows of the group (and, for the owner, the new k and v rows)
    const int nq_items = g * IPH;
    const int n_items = nq_items + (owner ? 2 * IPH : 0);
    u32x4_t x0[MAXIT], x1[MAXIT];
#pragma unroll
    for (int u = 0; u < MAXIT; ++u) {
        const int it = tid + u * ST_THREADS;
        x0[u] = u32x4_t{0u, 0u, 0u, 0u};
        x1[u] = x0[u];
        if (it < n_items) {
            const int kind = it < nq_items ? 0 : 1 + (it - nq_items) / IPH;  // 0 q, 1 k, 2 v
            const int hl = it < nq_items ? it / IPH : 0;
            const int c = it < nq_items ? it % IPH : (it - nq_items) % IPH;
            const bool turns = kind != 2 && 16 * c < R;
            const int o0 = (turns && rp.layout != 0) ? 8 * c : 16 * c;
            const int o1 = (turns && rp.layout != 0) ? R / 2 + 8 * c : 16 * c + 8;
            const uint16_t* src = kind == 0 ? q + (size_t)(b * n_q + j * g + hl) * D
                                            : (kind == 1 ? k_new : v_new) + (size_t)(b * n_kv + j) * D;
            x0[u] = *reinterpret_cast<const u32x4_t*>(src + o0);
            x1[u] = *reinterpret_cast<const u32x4_t*>(src + o1);
        }
    }

    // ---- first tile: cache rows 0 .. P-1 of the segment (row P is the new one)
    const size_t seg = (size_t)(b * n_kv + j) * S * D;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(k_cache + seg), (short)0, P * ROWB, ST_RSRC);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(v_cache + seg), (short)0, P * ROWB, ST_RSRC);
    auto abs_tile = [&](int i) { return i < geo.nst ? i : geo.at0 + (i - geo.nst); };
    u32x4_t kb[LOADS], vb[LOADS];
    auto load_tile = [&](int i) {
        const int base = abs_tile(i) * TILEB + tid * 16;
#pragma unroll
        for (int x = 0; x < LOADS; ++x) {
            kb[x] = __builtin_amdgcn_raw_buffer_load_b128(rk, base + x * ST_THREADS * 16, 0, 0);
            vb[x] = __builtin_amdgcn_raw_buffer_load_b128(rv, base + x * ST_THREADS * 16, 0, 0);
        }
    };
    if (t0 < t1) load_tile(t0);

    // ---- angles of position P (fp64), scaled by the attention factor
    for (int i = tid; i < R / 2; i += ST_THREADS) {
        const double ang = (double)P * rp.freq[i];
        double sn, cs;
        sincos(ang, &sn, &cs);
        s_cos[i] = rp.attn * cs;
        s_sin[i] = rp.attn * sn;
    }
    __syncthreads();

    // ---- rotate: q rows into LDS (and q_rot out), the new k / v row into LDS and the cache
#pragma unroll
    for (int u = 0; u < MAXIT; ++u) {
        const int it = tid + u * ST_THREADS;
        if (it >= n_items) continue;
        const int kind = it < nq_items ? 0 : 1 + (it - nq_items) / IPH;
        const int hl = it < nq_items ? it / IPH : 0;
        const int c = it < nq_items ? it % IPH : (it - nq_items) % IPH;
        const bool turns = kind != 2 && 16 * c < R;
        const int o0 = (turns && rp.layout != 0) ? 8 * c : 16 * c;
        const int o1 = (turns && rp.layout != 0) ? R / 2 + 8 * c : 16 * c + 8;
        u32x4_t y0 = x0[u], y1 = x1[u];
        if (turns) {
            const uint32_t w[8] = {x0[u][0], x0[u][1], x0[u][2], x0[u][3], x1[u][0], x1[u][1], x1[u][2], x1[u][3]};
            uint32_t o[8];
            rotate_item(w, c, rp.layout, s_cos, s_sin, o);
            y0 = u32x4_t{o[0], o[1], o[2], o[3]};
            y1 = u32x4_t{o[4], o[5], o[6], o[7]};
        }
        unsigned char* lrow = kind == 0 ? s_q + hl * ROWB : s_new[kind - 1];
        *reinterpret_cast<u32x4_t*>(lrow + 2 * o0) = y0;
        *reinterpret_cast<u32x4_t*>(lrow + 2 * o1) = y1;
        uint16_t* dst = nullptr;
        if (kind == 0 && sp == 0 && q_rot_out) dst = q_rot_out + (size_t)(b * n_q + j * g + hl) * D;
        if (kind != 0 && pvalid) dst = (kind == 1 ? k_cache : v_cache) + seg + (size_t)P * D;
        if (dst) {
            *reinterpret_cast<u32x4_t*>(dst + o0) = y0;
            *reinterpret_cast<u32x4_t*>(dst + o1) = y1;
        }
    }

    // ---- per-wave online softmax state for heads wave + 4k
    float m_run[HPW], l_run[HPW], o[HPW][DPL];
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
        m_run[k] = -INFINITY;
        l_run[k] = 0.f;
#pragma unroll
        for (int x = 0; x < DPL; ++x) o[k][x] = 0.f;
    }
    const int prow = P % ST_TILE;  // row of the new token inside its tile

    for (int i = t0; i < t1; ++i) {
        const int at = abs_tile(i);
        const bool has_new = owner && i == geo.nt - 1;
        __syncthreads();  // the previous tile is consumed (and s_q / s_new are written, first time)
#pragma unroll
        for (int x = 0; x < LOADS; ++x) {
            const int byte = tid * 16 + x * ST_THREADS * 16;
            const int row = byte / ROWB, pc = (byte % ROWB) / 16;
            u32x4_t kx = kb[x], vx = vb[x];
            if (has_new && row == prow) {
                kx = *reinterpret_cast<const u32x4_t*>(s_new[0] + 16 * pc);
                vx = *reinterpret_cast<const u32x4_t*>(s_new[1] + 16 * pc);
            }
            *reinterpret_cast<u32x4_t*>(s_k + row * ROWB + 16 * (pc ^ (row & (PPR - 1)))) = kx;
            *reinterpret_cast<u32x4_t*>(s_v + byte) = vx;
        }
        if (i + 1 < t1) load_tile(i + 1);
        __syncthreads();

        // q.k for row `lane` and the wave's heads
        float sc[HPW];
#pragma unroll
        for (int k = 0; k < HPW; ++k) sc[k] = 0.f;
#pragma unroll
        for (int e = 0; e < PPR; ++e) {
            const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(s_k + lane * ROWB + 16 * (e ^ (lane & (PPR - 1))));
#pragma unroll
            for (int k = 0; k < HPW; ++k) {
                if (wave + 4 * k >= g) break;
                const u32x4_t qv = *reinterpret_cast<const u32x4_t*>(s_q + (wave + 4 * k) * ROWB + 16 * e);
                float a = sc[k];
                a = dot2_bf16(kv[0], qv[0], a);
                a = dot2_bf16(kv[1], qv[1], a);
                a = dot2_bf16(kv[2], qv[2], a);
                a = dot2_bf16(kv[3], qv[3], a);
                sc[k] = a;
            }
        }
        const int row = at * ST_TILE + lane;
        const bool vis = row < L && (row >= geo.w0 || row < n_sink);
#pragma unroll
        for (int k = 0; k < HPW; ++k) {
            if (wave + 4 * k >= g) break;
            const float s = vis ? sc[k] * scale_log2 : -INFINITY;
            const float mn = fmaxf(m_run[k], wave_max(s));
            const float mref = mn == -INFINITY ? 0.f : mn;
            const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m_run[k] - mn);
            const float p = fast_exp2(s - mref);
            m_run[k] = mn;
            l_run[k] = l_run[k] * alpha + wave_sum(p);
            s_p[wave + 4 * k][lane] = p;
#pragma unroll
            for (int x = 0; x < DPL; ++x) o[k][x] *= alpha;
        }
        __builtin_amdgcn_wave_barrier();
        // weighted value sum: lane owns value dims DPL*lane .. DPL*lane+DPL-1
#pragma unroll 4
        for (int rr = 0; rr < ST_TILE; rr += 4) {
            float v[4][DPL];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (DPL == 2) {
                    const uint32_t vw = *reinterpret_cast<const uint32_t*>(s_v + (rr + u) * ROWB + 4 * lane);
                    v[u][0] = bf_lo(vw);
                    v[u][DPL - 1] = bf_hi(vw);
                } else {
                    const uint32_t vh = *reinterpret_cast<const uint16_t*>(s_v + (rr + u) * ROWB + 2 * lane);
                    v[u][0] = __uint_as_float(vh << 16);
                }
            }
#pragma unroll
            for (int k = 0; k < HPW; ++k) {
                if (wave + 4 * k >= g) break;
                const float4 p4 = *reinterpret_cast<const float4*>(&s_p[wave + 4 * k][rr]);
                const float pw[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int x = 0; x < DPL; ++x) o[k][x] += pw[u] * v[u][x];
            }
        }
    }

    // ---- this split's records, then count it on the segment's counter.  The
    // count is an agent-scope release (thread 0, after the workgroup barrier
    // that orders every thread's record stores before it), and the workgroup
    // whose count completes the segment executes an agent-scope acquire fence
    // before it reads the other splits' records: under the HIP memory model
    // the records happen-before the merge whichever XCD each split ran on.
    // The records are agent-scope atomic stores, written through to the
    // device's point of coherence, so the L2 write-back that the release
    // performs finds little to write (plain stores measured 2.9 us slower on
    // one Llama-3.1-8B layer; these 0.9 us slower than relaxed ordering).
    const size_t segi = (size_t)b * n_kv + j;
    float* rec0 = recs + segi * nsplit * g * REC;
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
        const int h = wave + 4 * k;
        if (h >= g) break;
        float* r = rec0 + ((size_t)sp * g + h) * REC;
        if (lane == 0) {
            __hip_atomic_store(r, m_run[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(r + 1, l_run[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int x = 0; x < DPL; ++x)
            __hip_atomic_store(r + 4 + DPL * lane + x, o[k][x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (tid == 0)
        s_last = __hip_atomic_fetch_add(&counters[segi], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == nsplit - 1;
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    auto rd = [](const float* a) { return *a; };

    // ---- last split of the segment: merge in split order.  Lane s holds split
    // s's (m, l); the outputs are read eight splits at a time so the loads
    // overlap.
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
        const int h = wave + 4 * k;
        if (h >= g) break;
        float m_l = -INFINITY, l_l = 0.f;
        if (lane < nsplit) {  // nsplit <= 64
            const float* r = rec0 + ((size_t)lane * g + h) * REC;
            m_l = rd(r);
            l_l = rd(r + 1);
        }
        const float sk = sink_logits ? sink_logits[j * g + h] * ST_LOG2E : -INFINITY;
        const float M = fmaxf(wave_max(m_l), sk);
        const float w_l = m_l == -INFINITY ? 0.f : fast_exp2(m_l - M);  // 0 for lanes >= nsplit
        const float lsum = wave_sum(w_l * l_l) + (sk == -INFINITY ? 0.f : fast_exp2(sk - M));
        float acc[DPL];
#pragma unroll
        for (int x = 0; x < DPL; ++x) acc[x] = 0.f;
        for (int s0 = 0; s0 < nsplit; s0 += 8) {
            float ov[8][DPL];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int s2 = s0 + u < nsplit ? s0 + u : 0;
                const float* r = rec0 + ((size_t)s2 * g + h) * REC + 4 + DPL * lane;
#pragma unroll
                for (int x = 0; x < DPL; ++x) ov[u][x] = rd(r + x);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                // s0 + u <= 63 (s0 is a multiple of 8 below nsplit <= 64); lanes >= nsplit hold 0
                const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l), s0 + u));
#pragma unroll
                for (int x = 0; x < DPL; ++x) acc[x] += w * ov[u][x];
            }
        }
        const float inv = 1.f / lsum;
        uint16_t* dst = out + (size_t)(b * n_q + j * g + h) * D;
        if (DPL == 2)
            *reinterpret_cast<uint32_t*>(dst + 2 * lane) = cvt_pk_bf16(acc[0] * inv, acc[DPL - 1] * inv);
        else
            dst[lane] = (uint16_t)(cvt_pk_bf16(acc[0] * inv, 0.f) & 0xffffu);
    }
    if (tid == 0) counters[segi] = 0;  // ready for the next call
}

using step_fn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, uint16_t*, const int32_t*,
                         int, uint16_t*, uint16_t*, float*, int*, int, int, int, int, float, RopeDev, int, int,
                         const float*);

template <int D>
step_fn pick_step(int g) {
    if (g <= 4) return decode_step_kernel<D, 1>;
    if (g <= 8) return decode_step_kernel<D, 2>;
    if (g <= 16) return decode_step_kernel<D, 4>;
    if (g <= 32) return decode_step_kernel<D, 8>;
    return decode_step_kernel<D, 16>;
}

size_t step_counter_bytes(int B, int n_kv) {
    return ((size_t)B * n_kv * sizeof(int) + 255) / 256 * 256;
}

}  // namespace

int decode_step_splits(int B, int n_kv, int max_past_len, int window, int n_sink) {
    int cu_count = 256;  // (the launch itself reports a device error)
    if (device_cu_count(&cu_count) != hipSuccess) cu_count = 256;
    long long tiles = (max_past_len + 1 + 63) / 64;
    if (window > 0) {
        const long long wt = (n_sink + 63) / 64 + window / 64 + 2;
        if (wt < tiles) tiles = wt;
    }
    const long long segs = (long long)B * n_kv;
    long long n = (2LL * cu_count + segs - 1) / segs;
    if (n > tiles) n = tiles;
    if (n > DECODE_STEP_MAX_SPLITS) n = DECODE_STEP_MAX_SPLITS;
    return n < 1 ? 1 : (int)n;
}

// Groups of 16 and more heads run the step as rope_append followed by the
// wide-group decode kernel (both products on MFMA), which is several times
// faster there than this kernel's VALU products.  That route keeps the rotated
// q and the wide kernel's records after the counter region, which stays zero.
static bool step_takes_wide_route(int n_q, int n_kv) {
    const int g = n_q / n_kv;
    return g >= decode_wide_min_group() && g <= DECODE_WIDE_MAX_G && n_kv <= DECODE_WIDE_MAX_SEGS;
}
static size_t step_qrot_bytes(int B, int n_q, int d) { return ((size_t)B * n_q * d * 2 + 255) / 256 * 256; }

// Larger batches run the step as rope_append followed by the split-K decode
// (partials + combine), which is faster there.  Measured at 32/8 heads, d 128
// (graph replays, cold caches): at contexts U[512, 8191] the single launch
// takes 17.7 / 19.8 / 37.3 / 64.3 / 178 us at B = 1 / 2 / 4 / 8 / 32 against
// 18.8 / 20.1 / 25.3 / 38.0 / 105 us for the two calls; at past_len 1000,
// 11.9 / 14.7 / 19.6 us at B = 1 / 2 / 4 against 15.1 / 15.5 / 18.4 us.  The
// crossover sits between 256 and 700 tiles of 64 rows (bounded with every
// past_len at max_past_len); from DECODE_STEP_SPLIT_MIN_TILES on the step
// takes the two calls.
constexpr int DECODE_STEP_SPLIT_MIN_TILES = 512;
static int g_step_split_min_tiles = DECODE_STEP_SPLIT_MIN_TILES;

static bool step_takes_split_route(int B, int n_kv, int max_past_len, int window, int n_sink) {
    long long per_seg = (max_past_len + 1 + 63) / 64;
    if (window > 0) {
        const long long wt = (n_sink + 63) / 64 + (window + 63) / 64 + 1;
        if (wt < per_seg) per_seg = wt;
    }
    return (long long)B * n_kv * per_seg >= g_step_split_min_tiles;
}

// Workspace of the step.  The per-segment counters of the single-launch route
// (one per (sequence, KV head)) start the workspace and are zero at rest; the
// split route keeps its scheduling header (the ticket counter, also zero at
// rest) in the first 256 bytes, which every route leaves zero at rest.  All
// else a call writes (the single-launch records; the rotated q and the records
// of the wide or split route) sits at the end of the caller's workspace: a
// call with B sequences touches only the last step_tail_bytes(B) bytes beyond
// its counters, so a workspace sized for some batch size serves every smaller
// one, through every route, in any order (were the records placed right after
// the counters, a small batch's records would overwrite the counters of a
// larger batch's later call).
static size_t step_tail_bytes(int B, int n_q, int n_kv, int d) {
    size_t t = (size_t)B * n_q * DECODE_STEP_MAX_SPLITS * (d + 4) * sizeof(float);  // single launch
    const int g = n_q / n_kv;
    if (g <= DECODE_WIDE_MAX_G && n_kv <= DECODE_WIDE_MAX_SEGS) {  // any threshold may send the shape there
        const size_t wide = step_qrot_bytes(B, n_q, d) + DECODE_WS_HEADER_FLOATS * sizeof(float) +
                            decode_wide_record_bytes(B, n_q, n_kv, d);
        if (wide > t) t = wide;
    }
    const size_t split = step_qrot_bytes(B, n_q, d) + decode_workspace_bytes(B, n_q, n_kv, d);
    if (split > t) t = split;
    return (t + 255) / 256 * 256;
}

size_t decode_step_workspace_bytes(int B, int n_q, int n_kv, int d) {
    return step_counter_bytes(B, n_kv) + step_tail_bytes(B, n_q, n_kv, d);
}

void set_decode_step_split_min_tiles(int tiles) {
    g_step_split_min_tiles = tiles > 0 ? tiles : DECODE_STEP_SPLIT_MIN_TILES;
}
int decode_step_split_min_tiles() { return g_step_split_min_tiles; }

hipError_t launch_decode_step(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_cache,
                              uint16_t* v_cache, const int32_t* past_len, int max_past_len, uint16_t* out,
                              uint16_t* q_rot, void* ws, size_t ws_bytes, int B, int n_q, int n_kv, int d, int S,
                              const RopeDev& rope, float scale, int window, int n_sink, const float* sink_logits,
                              hipStream_t st) {
    const int g = n_q / n_kv;
    // the tail: the last step_tail_bytes of the workspace, 256-byte aligned
    // (ws_bytes >= decode_step_workspace_bytes, checked by the caller)
    const size_t tail_at = (ws_bytes - step_tail_bytes(B, n_q, n_kv, d)) / 256 * 256;
    char* const base = static_cast<char*>(ws) + tail_at;
    if (step_takes_wide_route(n_q, n_kv)) {
        uint16_t* qr = q_rot ? q_rot : reinterpret_cast<uint16_t*>(base);
        float* wws = reinterpret_cast<float*>(base + step_qrot_bytes(B, n_q, d));
        hipError_t e = launch_rope_append(q, qr, k_new, v_new, k_cache, v_cache, past_len, max_past_len, B, n_q, n_kv,
                                          1, d, S, rope, st);
        if (e != hipSuccess) return e;
        return launch_decode_wide(qr, k_cache, v_cache, past_len, max_past_len, out, wws, B, n_q, n_kv, d, S, scale,
                                  window, n_sink, sink_logits, 0, st);
    }
    if (step_takes_split_route(B, n_kv, max_past_len, window, n_sink)) {
        uint16_t* qr = q_rot ? q_rot : reinterpret_cast<uint16_t*>(base);
        float* sws = reinterpret_cast<float*>(base + step_qrot_bytes(B, n_q, d));
        hipError_t e = launch_rope_append(q, qr, k_new, v_new, k_cache, v_cache, past_len, max_past_len, B, n_q, n_kv,
                                          1, d, S, rope, st);
        if (e != hipSuccess) return e;
        return launch_decode(qr, k_cache, v_cache, past_len, max_past_len, out, sws, B, n_q, n_kv, d, S, scale, window,
                             n_sink, sink_logits, 0, st, static_cast<float*>(ws));
    }
    const int nsplit = decode_step_splits(B, n_kv, max_past_len, window, n_sink);
    int* counters = static_cast<int*>(ws);
    float* recs = reinterpret_cast<float*>(base);
    const step_fn fn = d == 128 ? pick_step<128>(g) : pick_step<64>(g);
    prof_begin(K_DECODE_STEP, st);
    hipLaunchKernelGGL(fn, dim3(nsplit, n_kv, B), dim3(ST_THREADS), 0, st, q, k_new, v_new, k_cache, v_cache, past_len,
                       max_past_len, out, q_rot, recs, counters, n_q, n_kv, S, nsplit, scale * ST_LOG2E, rope, window,
                       n_sink, sink_logits);
    prof_end(K_DECODE_STEP, st);
    return hipGetLastError();
}

}  // namespace gqa
