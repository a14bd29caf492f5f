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
//    HBM with 16-byte coalesced raw buffer loads (the descriptor covers only
//    the segment's valid rows, so the hardware range check zero-fills the
//    rest), staged through two register stages into LDS, so the loads of the
//    next two tiles are in flight while one is computed.
//  * Waves split the tile by (head group, row group).  For q.k, lane
//    (r = lane/8, e = lane%8) owns 16-byte pieces e and e+8 of a row: a
//    v_dot2_f32_bf16 chain over those pieces, then a DPP reduction over the 8
//    lanes of the row.  Online softmax keeps a running max and sum per head
//    (wave reductions by DPP / lane shuffles).  The weights go through a small
//    per-wave LDS buffer, and for the weighted value sum every lane owns d/64
//    output dims of all the wave's heads, so the accumulator is a few
//    registers and the kernel fits four workgroups per CU.
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
constexpr int PARK = 2;  // finished pieces a workgroup keeps in LDS until its share is done
constexpr int WAVES = THREADS / 64;
constexpr float LOG2E = 1.4426950408889634f;

template <int D, int HGW, int NHG>
struct Cfg {
    static constexpr int NP = D / 64;              // 16-byte pieces per lane per row
    static constexpr int PPR = D / 8;              // 16-byte pieces per row
    static constexpr int RG = WAVES / NHG;         // row groups per tile
    static constexpr int ROWS_W = TILE / RG;       // rows of a tile one wave handles
    static constexpr int PASSES = ROWS_W / 8;      // q.k passes of 8 rows
    static constexpr int GC = HGW * NHG;           // heads per segment
    static constexpr int REC = D + 4;              // m, l, 2 pad, o[D]
    static constexpr int SLOT = RG * GC * REC;     // floats per (segment, workgroup) piece
    static constexpr int LOADS = 2 * TILE * PPR / THREADS;  // 16-byte loads per thread per tile
};

__device__ __forceinline__ int tiles_of(const int32_t* past_len, int b, int pmax) {
    int P = past_len[b];
    P = P < 0 ? 0 : (P > pmax ? pmax : P);
    return (P + 1 + TILE - 1) / TILE;  // rows 0..P
}

// Exclusive prefix of per-sequence tile counts into s_pre[0..B], 256 sequences
// per pass with one (clamped, unconditional) load per thread, so every pass
// costs a single memory round trip.
__device__ void tile_prefix(const int32_t* past_len, int B, int pmax, int* s_pre, int* s_wsum) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    int carry = 0;
    for (int base = 0; base < B; base += THREADS) {
        const int b = base + tid;
        const int n = tiles_of(past_len, b < B ? b : B - 1, pmax);
        const int mine = b < B ? n : 0;
        int x = mine;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) s_wsum[wv] = x;
        __syncthreads();
        int before = carry;
        for (int k = 0; k < wv; ++k) before += s_wsum[k];
        if (b < B) s_pre[b] = before + x - mine;
        int total = carry;
        for (int k = 0; k < THREADS / 64; ++k) total += s_wsum[k];
        carry = total;
        __syncthreads();
    }
    if (tid == 0) s_pre[B] = carry;
    __syncthreads();
}

// workgroup w of G covers tiles [w*T/G, (w+1)*T/G)
__device__ __forceinline__ long long share_begin(long long w, long long T, long long G) { return (w * T) / G; }
// the workgroup whose share holds tile tau: the largest w with share_begin(w) <= tau
__device__ __forceinline__ long long owner_of(long long tau, long long T, long long G) {
    return ((tau + 1) * G - 1) / T;
}

// Position of one tile in the concatenated tile list: sequence b, segment sj
// (= KV head * head chunks + chunk) inside it, tile tt inside the segment.
struct Cursor {
    int b, sj, tt, nt, L;
};

// Byte offset in the LDS tile of 16-byte piece c of row R (rows of D bf16).
// For d = 128, rows two apart use opposite halves of the 64 banks (piece
// index XOR 8), so the 16 lanes of one LDS access phase never collide.
template <int D>
__device__ __forceinline__ int lds_byte(int R, int c) {
    return D == 128 ? R * 256 + ((c ^ (((R >> 1) & 1) << 3)) << 4) : R * 128 + (c << 4);
}

template <int D, int HGW, int NHG>
__global__ __launch_bounds__(THREADS, 2) void decode_partial_kernel(
    const uint16_t* __restrict__ q_rot, const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ past_len, int pmax, float* __restrict__ ws, int B, int n_q, int n_kv, int S, int nhc,
    float scale_log2) {
    using C = Cfg<D, HGW, NHG>;
    constexpr int NP = C::NP, PASSES = C::PASSES;
    constexpr int DPL = D / 64;                  // value dims each lane accumulates
    constexpr int ROWB = D * 2;                  // bytes per cache row
    constexpr int TILEB = TILE * ROWB;           // bytes per K (or V) tile
    constexpr int HALF = C::LOADS / 2;           // 16-byte loads per thread per K (or V) tile
    __shared__ __align__(16) unsigned char s_kv[2 * TILEB];  // K tile, then V tile
    __shared__ float4 s_p[THREADS / 64][PASSES][8];          // softmax weights of each wave's rows
    __shared__ u32x4_t s_q[C::GC * (D / 8)];                  // the segment's GC query rows
    __shared__ int s_wsum[THREADS / 64];
    // Finished pieces are parked here (each wave in its own region) and
    // written to the workspace after the loop: global stores inside the loop
    // share the in-order load counter with the tile prefetches, and every
    // wait for a tile would also wait for their completion.
    __shared__ float s_park[PARK][THREADS / 64][HGW][D + 12];  // o[D], l per row lane [D, D+8), m at D+8
    __shared__ int s_park_seg[PARK];
    extern __shared__ int s_pre[];  // B + 1 entries

    tile_prefix(past_len, B, pmax, s_pre, s_wsum);

    // values read from LDS are the same in every lane: keep them in scalar registers
    auto uni = [] __attribute__((always_inline)) (int x) { return __builtin_amdgcn_readfirstlane(x); };
    const int segs_per_b = n_kv * nhc;
    const long long T_all = (long long)segs_per_b * uni(s_pre[B]);
    const long long G = gridDim.x, w = blockIdx.x;
    const long long tau0 = share_begin(w, T_all, G);
    const long long tau_end = share_begin(w + 1, T_all, G);
    if (tau0 >= tau_end) return;
    const int n_tiles = (int)(tau_end - tau0);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane >> 3, e = lane & 7;
    const int hg = wave / C::RG, rg = wave % C::RG;
    const int rbase = rg * C::ROWS_W;
    const int g = n_q / n_kv;

    auto rows_of = [&] __attribute__((always_inline)) (int bb) {
        int P = past_len[bb];
        P = P < 0 ? 0 : (P > pmax ? pmax : P);
        return P + 1;
    };
    Cursor cur;  // first tile: largest b with segs_per_b * s_pre[b] <= tau0
    {
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((long long)segs_per_b * uni(s_pre[mid]) <= tau0) lo = mid; else hi = mid - 1;
        }
        cur.b = uni(lo);
        cur.nt = uni(s_pre[cur.b + 1] - s_pre[cur.b]);
        const long long off = tau0 - (long long)segs_per_b * uni(s_pre[cur.b]);
        cur.sj = uni((int)(off / cur.nt));
        cur.tt = uni((int)(off % cur.nt));
        cur.L = uni(rows_of(cur.b));
    }
    auto advance = [&] __attribute__((always_inline)) (Cursor& c) {
        if (++c.tt < c.nt) return;
        c.tt = 0;
        if (++c.sj < segs_per_b) return;
        c.sj = 0;
        if (++c.b < B) {
            c.nt = uni(s_pre[c.b + 1] - s_pre[c.b]);
            c.L = uni(rows_of(c.b));
        }
    };

    // ---- tile loads: raw buffer loads over the segment's valid rows only.  The
    // descriptor's range check returns zeros for rows at or beyond L, so the
    // last partial tile needs no clamping and never touches rows beyond L.
    // Thread tid loads bytes tid*16 + i*4096 of the tile: 16 consecutive lanes
    // cover one 256-byte row, fully coalesced.
    u32x4_t st[C::LOADS];
    auto load_tile = [&] __attribute__((always_inline)) (const Cursor& c) {
        const size_t seg_off = (size_t)(c.b * n_kv + c.sj / nhc) * S * D;
        const int valid_bytes = c.L * ROWB;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void*)(k_cache + seg_off), (short)0, valid_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)(v_cache + seg_off), (short)0, valid_bytes, 0x00020000);
        const int soff = c.tt * TILEB;
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
            st[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, tid * 16, soff + i * THREADS * 16, 0);
            st[HALF + i] = __builtin_amdgcn_raw_buffer_load_b128(rv, tid * 16, soff + i * THREADS * 16, 0);
        }
    };
    // LDS position of the bytes this thread loaded: row tid*16/ROWB + i*(4096/ROWB), piece (tid*16 % ROWB)/16;
    // the swizzle bit depends only on tid, so every store is base + constant.
    const int st_base = lds_byte<D>((tid * 16) / ROWB, ((tid * 16) % ROWB) >> 4);
    auto store_tile = [&] __attribute__((always_inline)) () {
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
            *reinterpret_cast<u32x4_t*>(s_kv + st_base + i * THREADS * 16) = st[i];
            *reinterpret_cast<u32x4_t*>(s_kv + TILEB + st_base + i * THREADS * 16) = st[HALF + i];
        }
    };

    // ---- per-wave softmax state for its HGW heads; lane owns value dims DPL*lane ..
    float m_run[HGW], l_run[HGW];
    float o[HGW][DPL];
    auto reset_state = [&] __attribute__((always_inline)) () {
#pragma unroll
        for (int h = 0; h < HGW; ++h) {
            m_run[h] = -INFINITY;
            l_run[h] = 0.f;
#pragma unroll
            for (int x = 0; x < DPL; ++x) o[h][x] = 0.f;
        }
    };
    // The segment's GC query rows, one 16-byte piece per thread.  The piece is
    // loaded together with the segment's first tile (same register stage), so
    // waiting for that tile's loads also covers it and never drains the
    // younger prefetches.
    constexpr int QPIECES = C::GC * (D / 8);
    auto load_q = [&] __attribute__((always_inline)) (const Cursor& c) -> u32x4_t {
        const int j = c.sj / nhc, hc = c.sj % nhc;
        const int piece = tid < QPIECES ? tid : 0;
        const int hq = j * g + hc * C::GC + piece / (D / 8);
        return reinterpret_cast<const u32x4_t*>(q_rot + (size_t)(c.b * n_q + hq) * D)[piece % (D / 8)];
    };
    // write one finished piece's records straight to the workspace (used past
    // the parking capacity, and after the loop for the parked pieces)
    auto write_records = [&] __attribute__((always_inline)) (long long seg, const float* m4, const float* l4,
                                                             const float (*o4)[DPL]) {
        float* slot = ws + (size_t)(seg + w) * C::SLOT;
#pragma unroll
        for (int h = 0; h < HGW; ++h) {
            float* rec = slot + (size_t)(rg * C::GC + hg * HGW + h) * C::REC;
            if (lane == 0) {
                rec[0] = m4[h];
                rec[1] = l4[h];
            }
            if (DPL == 2)
                *reinterpret_cast<float2*>(rec + 4 + 2 * lane) = make_float2(o4[h][0], o4[h][DPL - 1]);
            else
                rec[4 + lane] = o4[h][0];
        }
    };
    int n_parked = 0;
    auto flush = [&] __attribute__((always_inline)) (const Cursor& c) {
        const long long seg = (long long)c.b * segs_per_b + c.sj;
        if (n_parked < PARK) {
            // wave-private LDS: o, m, and the 8 per-row-lane partial sums of l
#pragma unroll
            for (int h = 0; h < HGW; ++h) {
                float* pk = s_park[n_parked][wave][h];
                if (DPL == 2)
                    *reinterpret_cast<float2*>(pk + 2 * lane) = make_float2(o[h][0], o[h][DPL - 1]);
                else
                    pk[lane] = o[h][0];
                if (e == 0) pk[D + r] = l_run[h];
                if (lane == 0) pk[D + 8] = m_run[h];
            }
            if (tid == 0) s_park_seg[n_parked] = (int)seg;
            ++n_parked;
        } else {
            float l4[HGW];
#pragma unroll
            for (int h = 0; h < HGW; ++h) l4[h] = sum_hi3(l_run[h]);
            write_records(seg, m_run, l4, o);
        }
    };

    // LDS read bases.  q.k: lane (r, e) reads pieces e + 8pp of rows rbase + 2r + const.
    int qk_base[NP];
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) qk_base[pp] = lds_byte<D>(rbase + 2 * r, e + 8 * pp);
    // value sum: every lane reads its DPL dims of a row; the swizzle depends on the row's parity class.
    const int pv_base0 = D == 128 ? lds_byte<D>(rbase, lane >> 2) + (lane & 3) * 4 : rbase * ROWB + lane * 2;
    const int pv_base1 = D == 128 ? lds_byte<D>(rbase + 2, lane >> 2) + (lane & 3) * 4 - 2 * ROWB : pv_base0;

    // ---- one tile: q.k, online softmax, weighted value sum (this wave's rows and heads)
    auto compute_tile = [&] __attribute__((always_inline)) (const Cursor& c) {
        const int row0 = c.tt * TILE;
        float sc[PASSES][HGW];
#pragma unroll
        for (int k = 0; k < PASSES; ++k) {
            const int dR = 16 * (k >> 1) + (k & 1);  // row offset of this pass (rows rbase + 2r + dR)
            u32x4_t kp[NP];
#pragma unroll
            for (int pp = 0; pp < NP; ++pp)
                kp[pp] = *reinterpret_cast<const u32x4_t*>(s_kv + qk_base[pp] + dR * ROWB);
            u32x4_t qv[HGW][NP];
#pragma unroll
            for (int h = 0; h < HGW; ++h)
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) qv[h][pp] = s_q[(hg * HGW + h) * (D / 8) + e + 8 * pp];
            const bool valid = row0 + rbase + 2 * r + dR < c.L;
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
        // online softmax (base-2 exponent: scores already carry the log2 e factor)
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
#pragma unroll
            for (int x = 0; x < DPL; ++x) o[h][x] *= alpha[h];
        }
        // weights to LDS (one lane per row), then every lane sums its value dims over the rows
        if (e == 0) {
#pragma unroll
            for (int k = 0; k < PASSES; ++k) {
                float pv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int h = 0; h < HGW; ++h) pv[h] = sc[k][h];
                s_p[wave][k][r] = make_float4(pv[0], pv[1], pv[2], pv[3]);
            }
        }
        __builtin_amdgcn_wave_barrier();
        const unsigned char* vt = s_kv + TILEB;
#pragma unroll
        for (int k = 0; k < PASSES; ++k) {
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const int dR = 16 * (k >> 1) + 2 * rr + (k & 1);  // row rbase + dR; parity class of dR>>1 is rr&1
                const float4 p4 = s_p[wave][k][rr];
                const float pw[4] = {p4.x, p4.y, p4.z, p4.w};
                if (DPL == 2) {
                    const uint32_t vw =
                        *reinterpret_cast<const uint32_t*>(vt + ((rr & 1) ? pv_base1 : pv_base0) + dR * ROWB);
                    const float v0 = bf_lo(vw), v1 = bf_hi(vw);
#pragma unroll
                    for (int h = 0; h < HGW; ++h) {
                        o[h][0] += pw[h] * v0;
                        o[h][DPL - 1] += pw[h] * v1;
                    }
                } else {
                    const uint32_t vh = *reinterpret_cast<const uint16_t*>(vt + pv_base0 + dR * ROWB);
                    const float v0 = __uint_as_float(vh << 16);
#pragma unroll
                    for (int h = 0; h < HGW; ++h) o[h][0] += pw[h] * v0;
                }
                // keep at most two rows' LDS reads in flight: the empty asm pins the
                // accumulators here, so the sums above cannot sink below later reads
                if (rr & 1) {
#pragma unroll
                    for (int h = 0; h < HGW; ++h)
#pragma unroll
                        for (int x = 0; x < DPL; ++x) asm volatile("" : "+v"(o[h][x]));
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    };

    // ---- main loop: two register stages, so the next two tiles' loads are in
    // flight while one is computed from LDS.  Every step issues the same loads
    // on every path (past the end of the share it re-reads the current tile,
    // and it always fetches the q piece of the tile's segment), so the count
    // of outstanding loads is path-independent and each wait drains only the
    // stage it needs.
    u32x4_t st2[C::LOADS];
    Cursor ld = cur;  // next tile to load
    u32x4_t q2 = load_q(ld);
    load_tile(ld);
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) st2[i] = st[i];
    if (n_tiles > 1) advance(ld);
    u32x4_t q1 = load_q(ld);
    load_tile(ld);  // into st: st2 holds the first tile, st the second
    if (n_tiles > 2) advance(ld);
    reset_state();
    bool seg_start = true;
    auto step = [&] __attribute__((always_inline)) (u32x4_t (&buf)[C::LOADS], u32x4_t& qbuf, int i) {
        __syncthreads();  // every wave is done with the previous tile in LDS
#pragma unroll
        for (int x = 0; x < HALF; ++x) {
            *reinterpret_cast<u32x4_t*>(s_kv + st_base + x * THREADS * 16) = buf[x];
            *reinterpret_cast<u32x4_t*>(s_kv + TILEB + st_base + x * THREADS * 16) = buf[HALF + x];
        }
        if (seg_start && tid < QPIECES) s_q[tid] = qbuf;
        __syncthreads();
        {
            // loads of tile i+2 (or, past the end, the last tile again) into the stage just drained
            const size_t seg_off = (size_t)(ld.b * n_kv + ld.sj / nhc) * S * D;
            const int valid_bytes = ld.L * ROWB;
            const __amdgpu_buffer_rsrc_t rk =
                __builtin_amdgcn_make_buffer_rsrc((void*)(k_cache + seg_off), (short)0, valid_bytes, 0x00020000);
            const __amdgpu_buffer_rsrc_t rv =
                __builtin_amdgcn_make_buffer_rsrc((void*)(v_cache + seg_off), (short)0, valid_bytes, 0x00020000);
            const int soff = ld.tt * TILEB;
#pragma unroll
            for (int x = 0; x < HALF; ++x) {
                buf[x] = __builtin_amdgcn_raw_buffer_load_b128(rk, tid * 16, soff + x * THREADS * 16, 0);
                buf[HALF + x] = __builtin_amdgcn_raw_buffer_load_b128(rv, tid * 16, soff + x * THREADS * 16, 0);
            }
            qbuf = load_q(ld);
            if (i + 3 < n_tiles) advance(ld);
        }
        compute_tile(cur);
        Cursor nx = cur;
        advance(nx);
        const bool seg_end = i + 1 == n_tiles || nx.b != cur.b || nx.sj != cur.sj;
        if (seg_end) {
            flush(cur);
            reset_state();
        }
        seg_start = seg_end;
        cur = nx;
    };
    int i = 0;
    for (; i + 1 < n_tiles; i += 2) {  // straight-line pairs: no path-dependent load counts
        step(st2, q2, i);
        step(st, q1, i + 1);
    }
    if (i < n_tiles) step(st2, q2, i);

    // records of the parked pieces
    __syncthreads();
    for (int pk = 0; pk < n_parked; ++pk) {
        float m4[HGW], l4[HGW], o4[HGW][DPL];
#pragma unroll
        for (int h = 0; h < HGW; ++h) {
            const float* src = s_park[pk][wave][h];
#pragma unroll
            for (int x = 0; x < DPL; ++x) o4[h][x] = src[DPL * lane + x];
            float l = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) l += src[D + k];
            l4[h] = l;
            m4[h] = src[D + 8];
        }
        write_records(s_park_seg[pk], m4, l4, o4);
    }
}

// Merge of the partial records of one (sequence, query head), in a fixed
// order.  Lane i first reads the (max, sum) of record i; the output sum then
// walks the records in batches of 8 whose loads are all in flight together.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ ws,
                                                            const int32_t* __restrict__ past_len, int pmax,
                                                            uint16_t* __restrict__ out, int B, int n_q, int n_kv,
                                                            int nhc, int gc, int rg_count, int slot_floats, int G) {
    constexpr int DPL = D / 64;  // dims per lane
    constexpr int REC = D + 4;
    const int h = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x;
    const int g = n_q / n_kv;

    // prefix of tile counts (same clamping as the partial kernel)
    long long pre_b = 0, total = 0;
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
    const int nt_b = tiles_of(past_len, b, pmax);

    const int j = h / g, hh = h % g, hc = hh / gc, hl = hh % gc;
    const long long segs_per_b = (long long)n_kv * nhc;
    const long long T_all = segs_per_b * total;
    const long long seg = (long long)b * segs_per_b + (long long)j * nhc + hc;
    const long long start = segs_per_b * pre_b + (long long)(j * nhc + hc) * nt_b;
    const long long end = start + nt_b;
    const long long w_lo = owner_of(start, T_all, G), w_hi = owner_of(end - 1, T_all, G);
    const int nrec = (int)(w_hi - w_lo + 1) * rg_count;

    auto rec_ptr = [&](int idx) -> const float* {
        const long long w = w_lo + idx / rg_count;
        return ws + (size_t)(seg + w) * slot_floats + (size_t)((idx % rg_count) * gc + hl) * REC;
    };
    auto live = [&](int idx) {  // the workgroup of this record had a non-empty share
        const long long w = w_lo + idx / rg_count;
        return share_begin(w, T_all, G) < share_begin(w + 1, T_all, G);
    };

    float M = -INFINITY;
    for (int base = 0; base < nrec; base += 64) {
        const int idx = base + lane;
        if (idx < nrec && live(idx)) M = fmaxf(M, rec_ptr(idx)[0]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));

    float acc[DPL];
#pragma unroll
    for (int x = 0; x < DPL; ++x) acc[x] = 0.f;
    float lpart = 0.f;
    for (int base = 0; base < nrec; base += 64) {
        const int idx = base + lane;
        float f = 0.f;
        if (idx < nrec && live(idx)) {
            const float* rp = rec_ptr(idx);
            const float m = rp[0];
            f = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
            lpart += f * rp[1];
        }
        const int cnt = (nrec - base) < 64 ? (nrec - base) : 64;
        for (int i = 0; i < cnt; i += 8) {
            float fb[8];
            float ob[8][DPL];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                fb[k] = (i + k < cnt) ? __shfl(f, i + k, 64) : 0.f;
#pragma unroll
                for (int x = 0; x < DPL; ++x) ob[k][x] = 0.f;
                if (fb[k] != 0.f) {
                    const float* rp = rec_ptr(base + i + k) + 4 + DPL * lane;
#pragma unroll
                    for (int x = 0; x < DPL; ++x) ob[k][x] = rp[x];
                }
            }
#pragma unroll
            for (int k = 0; k < 8; ++k)
#pragma unroll
                for (int x = 0; x < DPL; ++x) acc[x] += fb[k] * ob[k][x];
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lpart += __shfl_xor(lpart, off, 64);

    const float inv = 1.f / lpart;
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
    const size_t dyn = (size_t)(B + 1) * sizeof(int);
    hipLaunchKernelGGL((decode_partial_kernel<D, HGW, NHG>), dim3(G), dim3(THREADS), dyn, st, q_rot, k_cache,
                       v_cache, past_len, pmax, ws, B, n_q, n_kv, S, nhc, scale_log2);
    return hipGetLastError();
}

template <int D, int HGW, int NHG>
int occupancy_t(int B) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_partial_kernel<D, HGW, NHG>, THREADS,
                                                     (size_t)(B + 1) * sizeof(int)) != hipSuccess)
        return 1;
    return blocks > 0 ? blocks : 1;
}

using occ_fn = int (*)(int);
using partial_fn = hipError_t (*)(int, const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*, int, float*,
                                  int, int, int, int, int, float, hipStream_t);

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
    p.rg = WAVES / v.nhg;
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
    // default: as many workgroups as fit on the chip at once (one wave of workgroups)
    if (G <= 0) {
        const int bs = B < DECODE_MAX_B ? B : DECODE_MAX_B;
        G = cu_count * (d == 128 ? v.occ128(bs) : v.occ64(bs));
    }
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
