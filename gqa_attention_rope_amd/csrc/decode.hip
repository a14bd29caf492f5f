// Split-K flash-decoding for grouped-query attention over a bf16 KV cache.
//
// What is computed ([KV] "Llama 3.1 8B KV cache", "The cache itself is
// concatenation"; [ATL] "Llama 3 8B - KV cache", decode formula and prose):
// for sequence b the one new query of head h attends to cache rows
// 0 .. past_len[b] of KV head floor(h / g) ([REP] "Llama 3.1 8B - Repeat
// heads" formula): softmax(q . k_r * scale) weighted sum of v_r.
//
// How ("grouped queries without repeat_kv" in [KV]: the g query heads of a
// group share each K/V row they read):
//
//  * Work unit: a tile of 64 cache rows of one (sequence, KV head, head chunk)
//    segment.  All tiles of all segments are laid end to end and every
//    workgroup takes one contiguous, equal share of that list (stream-K
//    style), so ragged past lengths cost nothing in balance and no workgroup
//    is launched idle.  A share may start or end inside a segment; each
//    (segment, workgroup) piece leaves one partial record per wave and head.
//  * Inside a workgroup (4 waves) a tile's K and V rows are loaded once from
//    HBM with 16-byte coalesced loads, staged through registers into LDS, and
//    the next tile's loads are in flight while the current one is computed.
//  * Waves split the tile by (head group, row group).  Within a wave, lane
//    (r = lane/8, e = lane%8) owns 16-byte pieces e and e+8 of a row: q.k is a
//    v_dot2_f32_bf16 chain over those pieces followed by a DPP reduction over
//    the 8 lanes of the row.  Online softmax keeps a running max and sum per
//    head (wave reductions by DPP / lane shuffles), and the weighted value sum
//    is accumulated by the same lanes over pairs of rows.
//  * A second kernel merges the records of each (sequence, head) in a fixed
//    order: M = max m, l = sum l e^(m-M), o = sum o e^(m-M) / l.  No atomics,
//    so results are bitwise reproducible for a given workgroup count.
#include <float.h>

#include "common.hpp"
#include "kernels.hpp"

namespace gqa {

namespace {

constexpr int TILE = 64;
constexpr int THREADS = 256;
constexpr float LOG2E = 1.4426950408889634f;

template <int D, int HGW, int NHG>
struct Cfg {
    static constexpr int NP = D / 64;              // 16-byte pieces per lane per row
    static constexpr int PPR = D / 8;              // 16-byte pieces per row
    static constexpr int RG = 4 / NHG;             // row groups per tile
    static constexpr int ROWS_W = TILE / RG;       // rows of a tile one wave handles
    static constexpr int PASSES = ROWS_W / 8;      // q.k passes of 8 rows
    static constexpr int GC = HGW * NHG;           // heads per segment
    static constexpr int REC = D + 4;              // m, l, 2 pad, o[D]
    static constexpr int SLOT = RG * GC * REC;     // floats per (segment, workgroup) piece
    static constexpr int LOADS = 2 * TILE * PPR / THREADS;  // 16-byte loads per thread per tile
};

// LDS position of 16-byte piece c of tile row R.  Rows two apart land in
// opposite halves of the 64 banks, so the 16 lanes of one LDS access phase
// never collide.
template <int PPR>
__device__ __forceinline__ int lds_pos(int R, int c) {
    return PPR == 16 ? (R * PPR + (c ^ (((R >> 1) & 1) << 3))) : (R * PPR + c);
}

__device__ __forceinline__ int tiles_of(const int32_t* past_len, int b, int pmax) {
    int P = past_len[b];
    P = P < 0 ? 0 : (P > pmax ? pmax : P);
    return (P + 1 + TILE - 1) / TILE;  // rows 0..P
}

// Exclusive prefix of per-sequence tile counts into s_pre[0..B] (B <= DECODE_MAX_B).
__device__ void tile_prefix(const int32_t* past_len, int B, int pmax, int* s_pre, int* s_wsum) {
    constexpr int PER = DECODE_MAX_B / THREADS;
    const int tid = threadIdx.x;
    int loc[PER];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int b = tid * PER + i;
        loc[i] = sum;
        sum += (b < B) ? tiles_of(past_len, b, pmax) : 0;
    }
    const int lane = tid & 63, wv = tid >> 6;
    int x = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_wsum[wv] = x;
    __syncthreads();
    int base = 0;
    for (int k = 0; k < wv; ++k) base += s_wsum[k];
    const int excl = base + x - sum;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int b = tid * PER + i;
        if (b < B) s_pre[b] = excl + loc[i];
    }
    if (tid == THREADS - 1) s_pre[B] = excl + sum;
    __syncthreads();
}

// workgroup w of G covers tiles [w*T/G, (w+1)*T/G)
__device__ __forceinline__ long long share_begin(long long w, long long T, long long G) { return (w * T) / G; }
// the workgroup whose share holds tile tau: the largest w with share_begin(w) <= tau
__device__ __forceinline__ long long owner_of(long long tau, long long T, long long G) {
    return ((tau + 1) * G - 1) / T;
}

template <int D, int HGW, int NHG>
__global__ __launch_bounds__(THREADS, 2) void decode_partial_kernel(
    const uint16_t* __restrict__ q_rot, const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ past_len, int pmax, float* __restrict__ ws, int B, int n_q, int n_kv, int S, int nhc,
    float scale_log2) {
    using C = Cfg<D, HGW, NHG>;
    constexpr int NP = C::NP, PPR = C::PPR, PASSES = C::PASSES;
    __shared__ uint4 s_k[TILE * PPR];
    __shared__ uint4 s_v[TILE * PPR];
    __shared__ int s_pre[DECODE_MAX_B + 1];
    __shared__ int s_wsum[THREADS / 64];

    tile_prefix(past_len, B, pmax, s_pre, s_wsum);

    const long long segs_per_b = (long long)n_kv * nhc;
    const long long T_all = segs_per_b * s_pre[B];
    const long long G = gridDim.x, w = blockIdx.x;
    long long tau = share_begin(w, T_all, G);
    const long long tau_end = share_begin(w + 1, T_all, G);
    if (tau >= tau_end) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane >> 3, e = lane & 7;
    const int hg = wave / C::RG, rg = wave % C::RG;
    const int rbase = rg * C::ROWS_W;
    const int g = n_q / n_kv;

    // locate the segment holding the first tile: largest b with segs_per_b*s_pre[b] <= tau
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (segs_per_b * s_pre[mid] <= tau) lo = mid; else hi = mid - 1;
    }
    int b = lo;
    int nt = s_pre[b + 1] - s_pre[b];
    long long off = tau - segs_per_b * s_pre[b];
    int sj = (int)(off / nt);   // segment within the sequence: j * nhc + hc
    int tt = (int)(off % nt);   // tile within the segment

    auto seq_rows = [&](int bb) {
        int P = past_len[bb];
        P = P < 0 ? 0 : (P > pmax ? pmax : P);
        return P + 1;
    };
    int L = seq_rows(b);

    // ---- staged tile loads (registers), zero beyond the last valid row
    uint4 stage[C::LOADS];
    auto load_tile = [&](int bb, int sjj, int ttt, int LL) {
        const int j = sjj / nhc;
        const size_t base = ((size_t)(bb * n_kv + j) * S + (size_t)ttt * TILE) * D;
        const int valid = LL - ttt * TILE;
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            const int pi = tid + THREADS * i;
            const int which = pi / (TILE * PPR);  // 0 = K, 1 = V
            const int row = (pi / PPR) % TILE;
            const int c = pi % PPR;
            const uint16_t* src = (which ? v_cache : k_cache) + base + (size_t)row * D + 8 * c;
            stage[i] = row < valid ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            const int pi = tid + THREADS * i;
            const int which = pi / (TILE * PPR);
            const int row = (pi / PPR) % TILE;
            const int c = pi % PPR;
            (which ? s_v : s_k)[lds_pos<PPR>(row, c)] = stage[i];
        }
    };

    // ---- per-wave softmax state for its HGW heads
    uint4 qv[HGW][NP];
    float m_run[HGW], l_run[HGW];
    float o[HGW][8 * NP];
    auto reset_state = [&]() {
#pragma unroll
        for (int h = 0; h < HGW; ++h) {
            m_run[h] = -INFINITY;
            l_run[h] = 0.f;
#pragma unroll
            for (int x = 0; x < 8 * NP; ++x) o[h][x] = 0.f;
        }
    };
    auto load_q = [&](int bb, int sjj) {
        const int j = sjj / nhc, hc = sjj % nhc;
#pragma unroll
        for (int h = 0; h < HGW; ++h) {
            const int hq = j * g + hc * C::GC + hg * HGW + h;
            const uint4* src = reinterpret_cast<const uint4*>(q_rot + (size_t)(bb * n_q + hq) * D);
#pragma unroll
            for (int pp = 0; pp < NP; ++pp) qv[h][pp] = src[e + 8 * pp];
        }
    };
    auto flush = [&](int bb, int sjj) {
        const long long seg = (long long)bb * segs_per_b + sjj;
        float* slot = ws + (size_t)(seg + w) * C::SLOT;
#pragma unroll
        for (int h = 0; h < HGW; ++h) {
            const float l_tot = sum_hi3(l_run[h]);
            float ov[8 * NP];
#pragma unroll
            for (int x = 0; x < 8 * NP; ++x) ov[x] = sum_hi3(o[h][x]);
            if (r == 0) {
                float* rec = slot + (size_t)(rg * C::GC + hg * HGW + h) * C::REC;
                if (e == 0) {
                    rec[0] = m_run[h];
                    rec[1] = l_tot;
                }
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) {
                    float4* dst = reinterpret_cast<float4*>(rec + 4 + 8 * (e + 8 * pp));
                    dst[0] = make_float4(ov[8 * pp + 0], ov[8 * pp + 1], ov[8 * pp + 2], ov[8 * pp + 3]);
                    dst[1] = make_float4(ov[8 * pp + 4], ov[8 * pp + 5], ov[8 * pp + 6], ov[8 * pp + 7]);
                }
            }
        }
    };

    reset_state();
    load_tile(b, sj, tt, L);
    bool seg_start = true;

    for (; tau < tau_end; ++tau) {
        if (seg_start) load_q(b, sj);
        __syncthreads();  // every wave is done reading the previous tile
        store_tile();
        __syncthreads();

        // coordinates of the next tile; issue its loads before computing this one
        int nb = b, nsj = sj, ntt = tt + 1, nL = L, nnt = nt;
        if (ntt == nt) {
            ntt = 0;
            if (++nsj == (int)segs_per_b) {
                nsj = 0;
                ++nb;
                if (nb < B) {
                    nnt = s_pre[nb + 1] - s_pre[nb];
                    nL = seq_rows(nb);
                }
            }
        }
        const bool more = tau + 1 < tau_end;
        if (more) load_tile(nb, nsj, ntt, nL);

        // ---- q.k for this wave's rows, HGW heads
        const int row0 = tt * TILE;
        float sc[PASSES][HGW];
#pragma unroll
        for (int k = 0; k < PASSES; ++k) {
            const int R = rbase + 16 * (k >> 1) + 2 * r + (k & 1);
            uint4 kp[NP];
#pragma unroll
            for (int pp = 0; pp < NP; ++pp) kp[pp] = s_k[lds_pos<PPR>(R, e + 8 * pp)];
            const bool valid = row0 + R < L;
#pragma unroll
            for (int h = 0; h < HGW; ++h) {
                float acc = 0.f;
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) {
                    acc = dot2_bf16(kp[pp].x, qv[h][pp].x, acc);
                    acc = dot2_bf16(kp[pp].y, qv[h][pp].y, acc);
                    acc = dot2_bf16(kp[pp].z, qv[h][pp].z, acc);
                    acc = dot2_bf16(kp[pp].w, qv[h][pp].w, acc);
                }
                acc = sum8(acc);
                sc[k][h] = valid ? acc * scale_log2 : -INFINITY;
            }
        }

        // ---- online softmax (base-2 exponent, scores already scaled by log2 e)
        bool rescale = false;
        float alpha[HGW];
#pragma unroll
        for (int h = 0; h < HGW; ++h) {
            float tm = sc[0][h];
#pragma unroll
            for (int k = 1; k < PASSES; ++k) tm = fmaxf(tm, sc[k][h]);
            tm = max_hi3(tm);
            const float mn = fmaxf(m_run[h], tm);
            const float mref = (mn == -INFINITY) ? 0.f : mn;
            alpha[h] = (mn == -INFINITY) ? 1.f : fast_exp2(m_run[h] - mn);
            m_run[h] = mn;
            float ps = 0.f;
#pragma unroll
            for (int k = 0; k < PASSES; ++k) {
                sc[k][h] = fast_exp2(sc[k][h] - mref);
                ps += sc[k][h];
            }
            l_run[h] = l_run[h] * alpha[h] + ps;
            rescale |= alpha[h] != 1.f;
        }
        if (rescale) {
#pragma unroll
            for (int h = 0; h < HGW; ++h)
#pragma unroll
                for (int x = 0; x < 8 * NP; ++x) o[h][x] *= alpha[h];
        }

        // ---- weighted value sum over row pairs (rows of passes 2m and 2m+1)
#pragma unroll
        for (int mm = 0; mm < NHG; ++mm) {
            const int R0 = rbase + 16 * mm + 2 * r;
#pragma unroll
            for (int pp = 0; pp < NP; ++pp) {
                const uint4 v0 = s_v[lds_pos<PPR>(R0, e + 8 * pp)];
                const uint4 v1 = s_v[lds_pos<PPR>(R0 + 1, e + 8 * pp)];
                const uint32_t a[4] = {v0.x, v0.y, v0.z, v0.w};
                const uint32_t c[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float a0 = bf_lo(a[x]), a1 = bf_hi(a[x]);
                    const float c0 = bf_lo(c[x]), c1 = bf_hi(c[x]);
#pragma unroll
                    for (int h = 0; h < HGW; ++h) {
                        const float p0 = sc[2 * mm][h], p1 = sc[2 * mm + 1][h];
                        o[h][8 * pp + 2 * x] += p0 * a0 + p1 * c0;
                        o[h][8 * pp + 2 * x + 1] += p0 * a1 + p1 * c1;
                    }
                }
            }
        }

        const bool seg_end = !more || nb != b || nsj != sj;
        if (seg_end) {
            flush(b, sj);
            reset_state();
        }
        seg_start = seg_end;
        b = nb;
        sj = nsj;
        tt = ntt;
        L = nL;
        nt = nnt;
    }
}

// Merge of the partial records of one (sequence, query head).
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ ws,
                                                            const int32_t* __restrict__ past_len, int pmax,
                                                            uint16_t* __restrict__ out, int B, int n_q, int n_kv,
                                                            int nhc, int gc, int rg_count, int slot_floats, int G) {
    constexpr int DPL = D / 64;  // dims per lane
    const int h = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x;
    const int g = n_q / n_kv;

    // prefix of tile counts (same clamping as the partial kernel)
    long long pre_b = 0, total = 0;
    int nt_b = 0;
    for (int base = 0; base < B; base += 64) {
        const int bb = base + lane;
        const int n = bb < B ? tiles_of(past_len, bb, pmax) : 0;
        int before = (bb < b) ? n : 0;
        int all = n;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            before += __shfl_xor(before, off, 64);
            all += __shfl_xor(all, off, 64);
        }
        pre_b += before;
        total += all;
    }
    nt_b = tiles_of(past_len, b, pmax);

    const int j = h / g, hh = h % g, hc = hh / gc, hl = hh % gc;
    const long long segs_per_b = (long long)n_kv * nhc;
    const long long T_all = segs_per_b * total;
    const long long seg = (long long)b * segs_per_b + (long long)j * nhc + hc;
    const long long start = segs_per_b * pre_b + (long long)(j * nhc + hc) * nt_b;
    const long long end = start + nt_b;
    const long long w_lo = owner_of(start, T_all, G), w_hi = owner_of(end - 1, T_all, G);

    float M = -INFINITY;
    for (long long w = w_lo; w <= w_hi; ++w) {
        const long long s0 = share_begin(w, T_all, G), s1 = share_begin(w + 1, T_all, G);
        if (s0 >= s1) continue;
        const float* slot = ws + (size_t)(seg + w) * slot_floats;
        for (int rg = 0; rg < rg_count; ++rg) M = fmaxf(M, slot[(size_t)(rg * gc + hl) * (D + 4)]);
    }
    float acc[DPL];
#pragma unroll
    for (int x = 0; x < DPL; ++x) acc[x] = 0.f;
    float lsum = 0.f;
    for (long long w = w_lo; w <= w_hi; ++w) {
        const long long s0 = share_begin(w, T_all, G), s1 = share_begin(w + 1, T_all, G);
        if (s0 >= s1) continue;
        const float* slot = ws + (size_t)(seg + w) * slot_floats;
        for (int rg = 0; rg < rg_count; ++rg) {
            const float* rec = slot + (size_t)(rg * gc + hl) * (D + 4);
            const float m = rec[0];
            const float f = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
            lsum += f * rec[1];
#pragma unroll
            for (int x = 0; x < DPL; ++x) acc[x] += f * rec[4 + DPL * lane + x];
        }
    }
    const float inv = 1.f / lsum;
    uint16_t* dst = out + (size_t)(b * n_q + h) * D + DPL * lane;
    if (DPL == 2) {
        *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(acc[0] * inv, acc[DPL - 1] * inv);
    } else {
        dst[0] = (uint16_t)f32_to_bf16_rne(acc[0] * inv);
    }
}

template <int D, int HGW, int NHG>
hipError_t launch_partial_t(int G, const uint16_t* q_rot, const uint16_t* k_cache, const uint16_t* v_cache,
                            const int32_t* past_len, int pmax, float* ws, int B, int n_q, int n_kv, int S, int nhc,
                            float scale_log2, hipStream_t st) {
    hipLaunchKernelGGL((decode_partial_kernel<D, HGW, NHG>), dim3(G), dim3(THREADS), 0, st, q_rot, k_cache, v_cache,
                       past_len, pmax, ws, B, n_q, n_kv, S, nhc, scale_log2);
    return hipGetLastError();
}

template <int D, int HGW, int NHG>
int occupancy_t() {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_partial_kernel<D, HGW, NHG>, THREADS, 0) !=
        hipSuccess)
        return 1;
    return blocks > 0 ? blocks : 1;
}

using partial_fn = hipError_t (*)(int, const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*, int, float*,
                                  int, int, int, int, int, float, hipStream_t);
using occ_fn = int (*)();

struct Variant {
    int hgw, nhg;
    partial_fn fn128, fn64;
    occ_fn occ128, occ64;
};

#define GQA_VARIANT(H, N)                                                                                   \
    Variant {                                                                                               \
        H, N, launch_partial_t<128, H, N>, launch_partial_t<64, H, N>, occupancy_t<128, H, N>, occupancy_t<64, H, N> \
    }

// heads per segment, largest first: (heads per wave, head groups)
const Variant kVariants[] = {GQA_VARIANT(4, 4), GQA_VARIANT(3, 4), GQA_VARIANT(4, 2), GQA_VARIANT(3, 2),
                             GQA_VARIANT(4, 1), GQA_VARIANT(3, 1), GQA_VARIANT(2, 1), GQA_VARIANT(1, 1)};

const Variant& pick_variant(int g) {
    for (const Variant& v : kVariants)
        if (g % (v.hgw * v.nhg) == 0) return v;
    return kVariants[sizeof(kVariants) / sizeof(kVariants[0]) - 1];
}

}  // namespace

DecodePlan decode_plan(int n_q, int n_kv, int d) {
    const int g = n_q / n_kv;
    const Variant& v = pick_variant(g);
    DecodePlan p;
    p.hgw = v.hgw;
    p.nhg = v.nhg;
    p.gc = v.hgw * v.nhg;
    p.nhc = g / p.gc;
    p.rg = 4 / v.nhg;
    p.rec = d + 4;
    p.slot_floats = (size_t)p.rg * p.gc * p.rec;
    return p;
}

size_t decode_workspace_bytes(int B, int n_q, int n_kv, int d) {
    const DecodePlan p = decode_plan(n_q, n_kv, d);
    const int bs = B < DECODE_MAX_B ? B : DECODE_MAX_B;
    const size_t segs = (size_t)bs * n_kv * p.nhc;
    return (segs + DECODE_MAX_WG) * p.slot_floats * sizeof(float);
}

hipError_t launch_decode(const uint16_t* q_rot, const uint16_t* k_cache, const uint16_t* v_cache,
                         const int32_t* past_len, int max_past_len, uint16_t* out, float* ws, int B, int n_q,
                         int n_kv, int d, int S, float scale, int wg_override, hipStream_t st) {
    const DecodePlan p = decode_plan(n_q, n_kv, d);
    const Variant& v = pick_variant(n_q / n_kv);

    static int cu_count = 0;
    if (cu_count == 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        e = hipDeviceGetAttribute(&cu_count, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
    }
    int G = wg_override;
    if (G <= 0) G = cu_count * (d == 128 ? v.occ128() : v.occ64());
    if (G > DECODE_MAX_WG) G = DECODE_MAX_WG;
    if (G < 1) G = 1;
    const float scale_log2 = scale * LOG2E;

    for (int b0 = 0; b0 < B; b0 += DECODE_MAX_B) {
        const int nb = (B - b0) < DECODE_MAX_B ? (B - b0) : DECODE_MAX_B;
        const uint16_t* q = q_rot + (size_t)b0 * n_q * d;
        const uint16_t* kc = k_cache + (size_t)b0 * n_kv * S * d;
        const uint16_t* vc = v_cache + (size_t)b0 * n_kv * S * d;
        const int32_t* pl = past_len + b0;
        uint16_t* o = out + (size_t)b0 * n_q * d;

        prof_begin(K_DECODE_PARTIAL, st);
        hipError_t e = (d == 128 ? v.fn128 : v.fn64)(G, q, kc, vc, pl, max_past_len, ws, nb, n_q, n_kv, S, p.nhc,
                                                     scale_log2, st);
        prof_end(K_DECODE_PARTIAL, st);
        if (e != hipSuccess) return e;

        prof_begin(K_DECODE_COMBINE, st);
        if (d == 128)
            hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(n_q, nb), dim3(64), 0, st, ws, pl, max_past_len, o,
                               nb, n_q, n_kv, p.nhc, p.gc, p.rg, (int)p.slot_floats, G);
        else
            hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(n_q, nb), dim3(64), 0, st, ws, pl, max_past_len, o,
                               nb, n_q, n_kv, p.nhc, p.gc, p.rg, (int)p.slot_floats, G);
        prof_end(K_DECODE_COMBINE, st);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gqa
