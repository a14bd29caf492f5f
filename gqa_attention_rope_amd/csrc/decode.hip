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
//    segment.  All tiles of all segments are laid end to end.  The first part
//    of that list (a fixed fraction) is cut into one contiguous, equal share
//    per workgroup (stream-K style); the rest is cut into small fixed chunks
//    that workgroups take from a shared ticket counter as they run out of
//    work.  Workgroups resident on one CU do not progress at the same rate
//    (instruction issue favours the oldest waves, and the first loads of the
//    later ones queue behind the earlier ones), so equal static shares alone
//    leave the slowest workgroup finishing long after the mean; the dynamic
//    tail absorbs that spread.  Which chunk a ticket names is fixed, so the
//    records, and the result, do not depend on which workgroup ran it.
//  * A piece is the part of one segment inside one share or chunk; it leaves
//    one (max, sum, unnormalised output) record per query head, merged across
//    the waves of the workgroup through LDS.
//  * Inside a workgroup (4 waves) a tile's K and V rows are loaded once from
//    HBM with 16-byte coalesced raw buffer loads (the descriptor covers only
//    the segment's valid rows, so the hardware range check zero-fills the
//    rest), staged through two register stages into LDS, so the loads of the
//    next two tiles are in flight while one is computed.
//  * Every step issues the same sequence of vector memory instructions: the
//    record store of the previous piece, the ticket atomic and the loads.  When
//    one of them has nothing to do its buffer descriptor has a zero range, so
//    the hardware drops it.  With a path-independent count, every wait for a
//    stage drains exactly that stage and never the younger prefetches.
//  * Waves split the tile by (head group, row group).  q.k runs on MFMA
//    (v_mfma_f32_16x16x32_bf16): 16 K rows from an XOR-swizzled LDS tile are
//    the A operand, the segment's rotated q rows (held in registers) the B
//    operand, so each 16-row block gives every head's scores at once.  Online
//    softmax keeps a running max and sum per head (lane shuffles).  The
//    weights go through a small per-wave LDS buffer, and for the weighted
//    value sum every lane owns d/64 output dims of all the wave's heads, so
//    the accumulator is a few registers.
//  * Before its first loads, each workgroup also writes the record directory
//    entries of a few segments (where their records are and how many), so
//    the merge needs neither past_len nor the share arithmetic.
//  * A second kernel merges the records of each (sequence, head) in a fixed
//    order: M = max m, l = sum l e^(m-M), o = sum o e^(m-M) / l, and clears
//    the ticket counter for the next call.  Results are bitwise reproducible
//    for a given launch shape.
#include <float.h>

#include "attn_window.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace gqa {

namespace {

constexpr int TILE = 64;
constexpr int THREADS = 256;
constexpr int WAVES = THREADS / 64;
constexpr float LOG2E = 1.4426950408889634f;
// The workspace starts with a 256-byte scheduling header (the ticket counter
// at offset 0); the records follow.
constexpr int HDR_FLOATS = DECODE_WS_HEADER_FLOATS;
constexpr uint32_t RSRC_FLAGS = 0x00020000u;  // raw buffer, 32-bit dwords
constexpr int OOB = 0x7ffffff0;               // a buffer offset past any range: the access is dropped

template <int D, int HGW, int NHG>
struct Cfg {
    static constexpr int PPR = D / 8;              // 16-byte pieces per row
    static constexpr int RG = WAVES / NHG;         // row groups per tile
    static constexpr int ROWS_W = TILE / RG;       // rows of a tile one wave handles
    static constexpr int KB = ROWS_W / 16;         // 16-row blocks of a wave (one MFMA output block each)
    static constexpr int KS = D / 32;              // MFMA k-steps over the head dimension
    static constexpr int GC = HGW * NHG;           // heads per segment
    static constexpr int REC = D + 4;              // m, l, 2 pad, o[D]
    static constexpr int SLOT = GC * REC;          // floats per piece (one merged record per head)
    static constexpr int LOADS = 2 * TILE * PPR / THREADS;  // 16-byte loads per thread per tile
};

__device__ __forceinline__ int rows_clamped(const int32_t* past_len, int b, int pmax) {
    int P = past_len[b];
    P = P < 0 ? 0 : (P > pmax ? pmax : P);
    return P + 1;  // rows 0..P
}

// Exclusive prefix of per-sequence tile counts into s_pre[0..B], and each
// sequence's row count into s_len[0..B-1] (so that no later step reads
// past_len from memory again), 256 sequences per pass with one (clamped,
// unconditional) load per thread, so every pass costs a single memory round
// trip.
__device__ void tile_prefix(const int32_t* past_len, int B, int pmax, int window, int n_sink, int* s_pre,
                            int* s_len, int* s_wsum) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    int carry = 0;
    for (int base = 0; base < B; base += THREADS) {
        const int b = base + tid;
        const int L = rows_clamped(past_len, b < B ? b : B - 1, pmax);
        const int n = geo_of(L, window, n_sink).nt;
        if (b < B) s_len[b] = L;
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

// Static shares weighted by dispatch slot.  The hardware hands out a grid one
// workgroup per CU per round, so workgroup w is the (w / n_cu)-th resident of
// its CU.  Older residents win instruction issue and stream faster (measured
// at three per CU: about 1.5x per slot), so equal shares would leave the
// youngest finishing long after the rest; slot s gets a share proportional to
// its weight.  Shares are 32.32 fixed-point fractions of the static tiles:
// workgroup w starts at floor(Ts F(w) / 2^32), where F(w) is the fraction of
// all workgroups before it.  Both kernels evaluate this with multiplies only
// (no integer division on the combine's critical path).
struct Shares {
    int n_cu;                          // workgroups per dispatch round
    int ns;                            // rounds (slots) in the grid, 1 .. 4
    int G;                             // workgroups in the grid
    unsigned long long f1, f2, f3;     // fraction before slot 1, 2, 3 (before slot 0: 0)
    unsigned long long g0, g1, g2, g3; // fraction of one workgroup of slot 0 .. 3
};
// Fields selected without indexing: the struct stays in scalar registers
// (an indexed array member would be copied to scratch memory).
__device__ __forceinline__ unsigned long long frac_before_slot(const Shares& sh, int s) {
    return s <= 0 ? 0ull : (s == 1 ? sh.f1 : (s == 2 ? sh.f2 : sh.f3));
}
__device__ __forceinline__ unsigned long long frac_per_wg(const Shares& sh, int s) {
    return s == 0 ? sh.g0 : (s == 1 ? sh.g1 : (s == 2 ? sh.g2 : sh.g3));
}
// first tile of workgroup w's static share (w = G gives Ts); Ts < 2^31 and
// F <= 2^32, so the product fits in 64 bits
__device__ __forceinline__ long long share_begin(int w, long long Ts, const Shares& sh) {
    if (w >= sh.G) return Ts;
    // slot w / n_cu, capped at ns - 1 (compares instead of a division)
    int s = (w >= sh.n_cu) + (w >= 2 * sh.n_cu) + (w >= 3 * sh.n_cu);
    if (s > sh.ns - 1) s = sh.ns - 1;
    const unsigned long long f = frac_before_slot(sh, s) + (unsigned long long)(w - s * sh.n_cu) * frac_per_wg(sh, s);
    return (long long)(((unsigned long long)Ts * f) >> 32);
}
// a * b <= x, exactly (the product may exceed 64 bits)
__device__ __forceinline__ bool prod_le(unsigned long long a, unsigned long long b, unsigned long long x) {
    return __umul64hi(a, b) == 0 && a * b <= x;
}
// The workgroup whose share holds tile tau < Ts: the largest w < G with
// share_begin(w) <= tau, i.e. with Ts F(w) < R = (tau + 1) 2^32.  The slot is
// the last one whose first workgroup qualifies; inside it F grows by a fixed
// step E / Ts per workgroup, so the count is floor((R - Ts F(first) - 1) / E),
// estimated in fp64 and made exact with integer checks.
__device__ __forceinline__ long long owner_of(long long tau, long long Ts, const Shares& sh) {
    const unsigned long long R = (unsigned long long)(tau + 1) << 32;
    const unsigned long long T = (unsigned long long)Ts;
    int s = 0;
#pragma unroll
    for (int k = 1; k < 4; ++k)
        if (k < sh.ns && T * frac_before_slot(sh, k) < R) s = k;
    const int first = s * sh.n_cu;
    const int cnt = (sh.G - first) < sh.n_cu ? (sh.G - first) : sh.n_cu;
    const unsigned long long X = R - T * frac_before_slot(sh, s) - 1;
    const unsigned long long E = T * frac_per_wg(sh, s);
    double qd = floor((double)X / (double)E);
    unsigned long long q = qd > 0.0 ? (unsigned long long)qd : 0ull;
    // the estimate is off by at most one
#pragma unroll
    for (int i = 0; i < 2; ++i)
        if (q > 0 && !prod_le(q, E, X)) --q;
#pragma unroll
    for (int i = 0; i < 2; ++i)
        if (prod_le(q + 1, E, X)) ++q;
    const long long k = (long long)q < cnt - 1 ? (long long)q : cnt - 1;
    return first + k;
}

// Position of one tile in the concatenated tile list: sequence b, segment sj
// (= KV head * head chunks + chunk) inside it, tile tt inside the segment.
struct Cursor {
    int b, sj, tt, nt, L;  // tt: index among the segment's nt tiles
    int nst, at0, w0;      // the sequence's tile geometry (see geo_of)
    // kept up to date by the cursor so that issuing a tile needs no division:
    int hc;                // head chunk of the segment (sj % nhc)
    int seg;               // global segment index b * segs_per_b + sj
    int qoff;              // element offset of the segment's query rows in q_rot
    long long kvoff;       // element offset of the segment's K (and V) slab
};

// Byte offset in the LDS tile of 16-byte piece c of row R (rows of D bf16).
// For d = 128, rows two apart use opposite halves of the 64 banks (piece
// index XOR 8), so the 16 lanes of one LDS access phase never collide.
template <int D>
__device__ __forceinline__ int lds_byte(int R, int c) {
    return D == 128 ? R * 256 + ((c ^ (((R >> 1) & 1) << 3)) << 4) : R * 128 + (c << 4);
}
// Byte offset of piece c of row R in the LDS K tile, read as MFMA A operands:
// 16 lanes read one piece index of 16 consecutive rows, so the piece slot is
// XOR-ed with the row's low bits and those 16 reads hit distinct banks.
template <int D>
__device__ __forceinline__ int kpos_byte(int R, int c) {
    constexpr int PPR = D / 8;
    return R * (D * 2) + ((c ^ (R & (PPR - 1))) << 4);
}

// Tile schedule shared by the partial kernel and its record directory: tiles
// [0, Ts) are split into contiguous shares, tiles [Ts, T_all) into chunks of
// C.  Tile counts fit in 32 bits: at most 2048 sequences x n_q segments x
// S/64 tiles.
struct Sched {
    int T_all, Ts, n_dyn, C;
};
__device__ __forceinline__ Sched make_sched(int T_all, int static_pm, int chunk) {
    Sched s;
    s.T_all = T_all;
    // floor(T_all * static_pm / 1000) in 32-bit arithmetic (T_all < 2^31, static_pm <= 1000)
    s.Ts = (T_all / 1000) * static_pm + (T_all % 1000) * static_pm / 1000;
    s.C = chunk;
    s.n_dyn = (T_all - s.Ts + chunk - 1) / chunk;
    return s;
}

// What one register stage holds (the same in every lane).
struct Stage {
    int tt, L;   // absolute 64-row tile index of the tile, rows of the segment
    int w0;      // first visible window row of the segment (0: all rows visible)
    int slot;    // record slot of the piece the tile belongs to
    int flags;   // kind (TILE, BUBBLE = nothing loaded but work to come, END) | PIECE_END | GRABBED
};
constexpr int K_TILE = 0, K_BUBBLE = 1, K_END = 2, KIND_MASK = 3;
constexpr int F_PIECE_END = 4;  // last tile of its segment or of its range
constexpr int F_GRABBED = 8;    // this stage's atomic took a ticket

template <int D, int HGW, int NHG>
__global__ __launch_bounds__(THREADS, 2) void decode_partial_kernel(
    const uint16_t* __restrict__ q_rot, const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ past_len, int pmax, float* __restrict__ ws, int4* __restrict__ dir,
    float* __restrict__ recs, int B, int n_q, int n_kv, int S, int nhc, float scale_log2, int static_pm, int chunk,
    int window, int n_sink, Shares shares) {
    using C = Cfg<D, HGW, NHG>;
    constexpr int KB = C::KB, KS = C::KS;
    constexpr int DPL = D / 64;                  // value dims each lane accumulates
    constexpr int ROWB = D * 2;                  // bytes per cache row
    constexpr int TILEB = TILE * ROWB;           // bytes per K (or V) tile
    constexpr int HALF = C::LOADS / 2;           // 16-byte loads per thread per K (or V) tile
    __shared__ __align__(16) unsigned char s_kv[2 * TILEB];  // K tile, then V tile
    __shared__ float4 s_p[THREADS / 64][C::ROWS_W];         // softmax weights of each wave's rows (4 heads)
    __shared__ u32x4_t s_q[C::GC * (D / 8)];                  // the segment's GC query rows
    __shared__ int s_wsum[THREADS / 64];
    // state of each wave when a piece ends: o[D], m at D, l at D+1
    __shared__ float s_park[WAVES][HGW][D + 4];
    __shared__ int s_ticket;
    extern __shared__ int s_pre[];  // B + 1 entries, then s_len
    int* const s_len = s_pre + B + 1;  // B entries

    tile_prefix(past_len, B, pmax, window, n_sink, s_pre, s_len, s_wsum);

    // values read from LDS are the same in every lane: keep them in scalar registers
    auto uni = [] __attribute__((always_inline)) (int x) { return __builtin_amdgcn_readfirstlane(x); };
    const int segs_per_b = n_kv * nhc;
    const int n_segs = B * segs_per_b;
    const Sched sc = make_sched(segs_per_b * uni(s_pre[B]), static_pm, chunk);
    const int G = gridDim.x, w = blockIdx.x;
    const int dyn_slot0 = n_segs + G;  // slot of chunk t's piece in segment s: dyn_slot0 + t + s
    int* const ticket_ctr = reinterpret_cast<int*>(ws);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int hg = wave / C::RG, rg = wave % C::RG;
    const int rbase = rg * C::ROWS_W;
    const int g = n_q / n_kv;

    auto rows_of = [&] __attribute__((always_inline)) (int bb) { return s_len[bb]; };
    // cursor of global tile tau: the largest b with segs_per_b * s_pre[b] <= tau,
    // i.e. the number of b in 1 .. B-1 that qualify, counted 64 at a time by
    // ballot (independent LDS reads instead of a dependent binary search)
    auto cursor_at = [&] __attribute__((always_inline)) (int tau) {
        int cnt = 0;
        for (int b0 = 1; b0 < B; b0 += 64) {
            const int bb = b0 + lane;
            const bool qual = bb < B && segs_per_b * s_pre[bb < B ? bb : 0] <= tau;
            cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(qual));
        }
        Cursor c;
        c.b = uni(cnt);
        c.nt = uni(s_pre[c.b + 1] - s_pre[c.b]);
        const int off = tau - segs_per_b * uni(s_pre[c.b]);
        c.sj = uni(off / c.nt);
        c.tt = uni(off % c.nt);
        c.L = uni(rows_of(c.b));
        const Geo gg = geo_of(c.L, window, n_sink);
        c.nst = uni(gg.nst);
        c.at0 = uni(gg.at0);
        c.w0 = uni(gg.w0);
        const int j = c.sj / nhc;
        c.hc = c.sj - j * nhc;
        c.seg = c.b * segs_per_b + c.sj;
        c.qoff = (c.b * n_q + j * g + c.hc * C::GC) * D;
        c.kvoff = (long long)(c.b * n_kv + j) * S * D;
        return c;
    };
    // next tile; on a segment change the q rows move by one head chunk and the
    // K/V slab by one KV head whenever the head chunks of a KV head are done
    auto advance = [&] __attribute__((always_inline)) (Cursor& c) {
        if (++c.tt < c.nt) return;
        c.tt = 0;
        ++c.seg;
        c.qoff += C::GC * D;
        if (++c.hc == nhc) {
            c.hc = 0;
            c.kvoff += (long long)S * D;
        }
        if (++c.sj < segs_per_b) return;
        c.sj = 0;
        if (++c.b < B) {
            c.nt = uni(s_pre[c.b + 1] - s_pre[c.b]);
            c.L = uni(rows_of(c.b));
            const Geo gg = geo_of(c.L, window, n_sink);
            c.nst = uni(gg.nst);
            c.at0 = uni(gg.at0);
            c.w0 = uni(gg.w0);
        }
    };

    // ---- loader: the current range (static share first, then chunks) and at
    // most one ticket in flight or in hand
    Cursor ld;
    ld.b = 0; ld.sj = 0; ld.tt = 0; ld.nt = 1; ld.L = 1; ld.nst = 1; ld.at0 = 1; ld.w0 = 0;
    ld.hc = 0; ld.seg = 0; ld.qoff = 0; ld.kvoff = 0;
    const int tau_w = (int)share_begin(w, sc.Ts, shares);
    int ld_left = (int)share_begin(w + 1, sc.Ts, shares) - tau_w;
    int ld_rid = w;
    if (ld_left > 0) ld = cursor_at(tau_w);
    int nx_tau = 0, nx_len = 0, nx_rid = 0;
    bool have_next = false, no_more = sc.n_dyn == 0, pending = false;  // no chunks: no ticket is ever taken
    auto take_ticket = [&] __attribute__((always_inline)) (int t) {
        if (t >= 0 && t < sc.n_dyn) {  // (a counter left non-zero by a broken caller only loses work)
            have_next = true;
            nx_tau = sc.Ts + t * sc.C;
            nx_len = (sc.T_all - nx_tau) < sc.C ? (sc.T_all - nx_tau) : sc.C;
            nx_rid = dyn_slot0 + t;
        } else {
            no_more = true;
        }
    };
    // a short share needs the first chunk before the pipeline is primed
    if (ld_left <= 2 && !no_more) {
        if (tid == 0) s_ticket = atomicAdd(ticket_ctr, 1);
        __syncthreads();
        take_ticket(uni(s_ticket));
        __syncthreads();
    }

    // Record directory for the combine: for segment s, the slot of its first
    // static piece and their count, the slot of its first chunk piece and
    // their count, the first static workgroup and the static tile total.
    // The last workgroups of the grid fill it, one segment per thread (the
    // last one segments 0 .. 255, the one before it the next 256, ...): each
    // entry costs two owner searches, about 0.85 us of one wave, which would
    // otherwise delay the first loads of the first-slot workgroups, the ones
    // with the larger shares.  The stores go out before the first tile loads,
    // so the waits for those loads keep their fixed counts.
    for (int s = (G - 1 - w) * THREADS + tid; s < n_segs; s += G * THREADS) {
        const int b = s / segs_per_b, sj = s - b * segs_per_b;
        const int nt = s_pre[b + 1] - s_pre[b];
        const long long start = (long long)segs_per_b * s_pre[b] + (long long)sj * nt;
        const long long end = start + nt;
        const long long s_end = end < sc.Ts ? end : sc.Ts;
        int w_lo = 0, n_st = 0;
        if (start < s_end) {
            w_lo = (int)owner_of(start, sc.Ts, shares);
            n_st = (int)owner_of(s_end - 1, sc.Ts, shares) - w_lo + 1;
        }
        const long long d_start = start > sc.Ts ? start : sc.Ts;
        int t_lo = 0, n_dy = 0;
        if (d_start < end) {
            t_lo = (int)((d_start - sc.Ts) / sc.C);
            n_dy = (int)((end - 1 - sc.Ts) / sc.C) - t_lo + 1;
        }
        dir[2 * s] = make_int4(w_lo + s, n_st, dyn_slot0 + t_lo + s, n_dy);
        dir[2 * s + 1] = make_int4(w_lo, sc.Ts, 0, 0);
    }

    // The q piece of a tile's segment, one 16-byte piece per thread (the
    // segment's GC query rows); the descriptor is empty when nothing is loaded.
    constexpr int QPIECES = C::GC * (D / 8);
    // Issue one stage: the ticket atomic, the K/V tile loads and the q piece.
    auto issue = [&] __attribute__((always_inline)) (u32x4_t (&buf)[C::LOADS], u32x4_t& qbuf, int& tkbuf,
                                                      Stage& stg) {
        if (ld_left == 0 && have_next) {
            ld = cursor_at(nx_tau);
            ld_left = nx_len;
            ld_rid = nx_rid;
            have_next = false;
        }
        const bool tile = ld_left > 0;
        const int rem = tile ? ld_left - 1 : 0;
        // the next ticket is taken with the range's last tile but one: its value is
        // read when this stage is consumed two steps later, just in time for the
        // issue after the range's last tile, and no earlier commitment is made
        const bool grab = !no_more && !have_next && !pending && rem <= 1;
        const int at = ld.tt < ld.nst ? ld.tt : ld.at0 + (ld.tt - ld.nst);  // absolute tile of this one
        stg.tt = uni(at);
        stg.L = uni(ld.L);
        stg.w0 = uni(ld.w0);
        stg.slot = uni(ld_rid + ld.seg);
        stg.flags = uni((tile ? K_TILE : ((no_more && !pending) ? K_END : K_BUBBLE)) |
                        ((ld_left == 1 || ld.tt + 1 == ld.nt) ? F_PIECE_END : 0) | (grab ? F_GRABBED : 0));
        if (grab) pending = true;
        // Descriptor fields must be wave-uniform (scalar registers); readfirstlane
        // states that for values the compiler cannot prove uniform through the loop.
        // ticket: only lane 0 of wave 0 is inside the 4-byte range, and only when grabbing
        const __amdgpu_buffer_rsrc_t rt =
            __builtin_amdgcn_make_buffer_rsrc((void*)ticket_ctr, (short)0, uni(grab ? 4 : 0), RSRC_FLAGS);
        tkbuf = __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, rt, tid == 0 ? 0 : OOB, 0, 0);
        // K/V rows of the tile; thread tid loads bytes tid*16 + x*4096 of each
        const long long seg_off = ld.kvoff;
        const int valid_bytes = uni(tile ? ld.L * ROWB : 0);
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void*)(k_cache + seg_off), (short)0, valid_bytes, RSRC_FLAGS);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)(v_cache + seg_off), (short)0, valid_bytes, RSRC_FLAGS);
        const int soff = uni(at * TILEB);
        // K/V rows are read once per launch: non-temporal loads (nt) keep them from
        // displacing the split-K records and other reused lines in the caches
        // (measured: 108.7 -> 99.5 us for one Llama-3.1-8B layer at B = 32)
#pragma unroll
        for (int x = 0; x < HALF; ++x) {
            buf[x] = __builtin_amdgcn_raw_buffer_load_b128(rk, tid * 16, soff + x * THREADS * 16, CPOL_NT);
            buf[HALF + x] = __builtin_amdgcn_raw_buffer_load_b128(rv, tid * 16, soff + x * THREADS * 16, CPOL_NT);
        }
        {
            const uint16_t* qseg = q_rot + ld.qoff;
            const __amdgpu_buffer_rsrc_t rq =
                __builtin_amdgcn_make_buffer_rsrc((void*)qseg, (short)0, uni(tile ? QPIECES * 16 : 0), RSRC_FLAGS);
            qbuf = __builtin_amdgcn_raw_buffer_load_b128(rq, tid < QPIECES ? tid * 16 : OOB, 0, 0);
        }
        if (tile) {
            advance(ld);
            --ld_left;
        }
    };

    // LDS position of the bytes this thread loaded: row tid*16/ROWB + i*(4096/ROWB), piece (tid*16 % ROWB)/16;
    // both swizzles depend only on tid, so every store is base + constant.
    const int st_base = lds_byte<D>((tid * 16) / ROWB, ((tid * 16) % ROWB) >> 4);  // V tile
    const int stk_base = kpos_byte<D>((tid * 16) / ROWB, ((tid * 16) % ROWB) >> 4);  // K tile

    // ---- per-wave softmax state.  Scores live in the MFMA output layout: lane
    // (n = lane % 16, lq = lane / 16) holds head n (n < HGW) at 4 of the rows of
    // each 16-row block, so m_run (the head's running max, equal in its four
    // lanes) and l_run (this lane's share of the head's running sum) belong to
    // head n.  For the weighted value sum every lane owns DPL value dims of all
    // of the wave's heads.
    const int l16 = lane & 15, lq = lane >> 4;
    float m_run, l_run;
    float o[HGW][DPL];
    bf16x8_t qop[KS];  // B operand: 8 dims of head l16 per k-step (zero for l16 >= HGW)
    auto reset_state = [&] __attribute__((always_inline)) () {
        m_run = -INFINITY;
        l_run = 0.f;
#pragma unroll
        for (int h = 0; h < HGW; ++h)
#pragma unroll
            for (int x = 0; x < DPL; ++x) o[h][x] = 0.f;
    };
    auto load_qop = [&] __attribute__((always_inline)) () {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4_t v = s_q[(hg * HGW + (l16 < HGW ? l16 : 0)) * (D / 8) + 4 * ks + lq];
            qop[ks] = __builtin_bit_cast(bf16x8_t, l16 < HGW ? v : u32x4_t{0u, 0u, 0u, 0u});
        }
    };
    auto park = [&] __attribute__((always_inline)) () {
#pragma unroll
        for (int h = 0; h < HGW; ++h) {
            float* pk = s_park[wave][h];
            if (DPL == 2)
                *reinterpret_cast<float2*>(pk + 2 * lane) = make_float2(o[h][0], o[h][DPL - 1]);
            else
                pk[lane] = o[h][0];
        }
        float l = l_run;
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        if (lane < HGW) *reinterpret_cast<float2*>(&s_park[wave][lane][D]) = make_float2(m_run, l);
    };
    // Merge the parked wave states of the finished piece into one record per
    // head and store it.  The stores are issued on every call; with
    // valid == false the descriptor range is zero and they are dropped.
    constexpr int OPAIRS = C::GC * D / 2;
    constexpr int OITER = (OPAIRS + THREADS - 1) / THREADS;
    auto merge_weights = [&] __attribute__((always_inline)) (int hh, float (&f)[C::RG], float& M) {
        const int hgx = hh / HGW, hx = hh % HGW;
        M = -INFINITY;
#pragma unroll
        for (int k = 0; k < C::RG; ++k) M = fmaxf(M, s_park[hgx * C::RG + k][hx][D]);
#pragma unroll
        for (int k = 0; k < C::RG; ++k) {
            const float m = s_park[hgx * C::RG + k][hx][D];
            f[k] = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
        }
    };
    auto store_record = [&] __attribute__((always_inline)) (bool valid, int slot) {
        const __amdgpu_buffer_rsrc_t rr =
            __builtin_amdgcn_make_buffer_rsrc((void*)(recs + (size_t)uni(valid ? slot : 0) * C::SLOT), (short)0,
                                              uni(valid ? C::SLOT * 4 : 0), RSRC_FLAGS);
#pragma unroll
        for (int k = 0; k < OITER; ++k) {
            const int p = tid + THREADS * k;
            const bool in = p < OPAIRS;
            const int hh = in ? (2 * p) / D : 0, x = (2 * p) % D;
            float2 v = make_float2(0.f, 0.f);
            if (valid && in) {
                float f[C::RG], M;
                merge_weights(hh, f, M);
#pragma unroll
                for (int kk = 0; kk < C::RG; ++kk) {
                    const float2 ov =
                        *reinterpret_cast<const float2*>(&s_park[(hh / HGW) * C::RG + kk][hh % HGW][x]);
                    v.x += f[kk] * ov.x;
                    v.y += f[kk] * ov.y;
                }
            }
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), rr,
                                                  in ? (hh * C::REC + 4 + x) * 4 : OOB, 0, 0);
        }
        {
            const bool in = tid < C::GC;
            float2 v = make_float2(-INFINITY, 0.f);
            if (valid && in) {
                float f[C::RG], M;
                merge_weights(tid, f, M);
                float l = 0.f;
#pragma unroll
                for (int kk = 0; kk < C::RG; ++kk) l += f[kk] * s_park[(tid / HGW) * C::RG + kk][tid % HGW][D + 1];
                v = make_float2(M, l);
            }
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), rr, in ? tid * C::REC * 4 : OOB,
                                                  0, 0);
        }
    };

    // value sum: every lane reads its DPL dims of a row; the swizzle depends on the row's parity class.
    const int pv_base0 = D == 128 ? lds_byte<D>(rbase, lane >> 2) + (lane & 3) * 4 : rbase * ROWB + lane * 2;
    const int pv_base1 = D == 128 ? lds_byte<D>(rbase + 2, lane >> 2) + (lane & 3) * 4 - 2 * ROWB : pv_base0;

    // ---- one tile: q.k on MFMA, online softmax, weighted value sum (this wave's rows and heads)
    // vrows: rows of the tile below L (1..64); wrow: rows of the tile below the
    // window start w0 are hidden unless they are sinks (absolute row < n_sink)
    auto compute_tile = [&] __attribute__((always_inline)) (int vrows, int row0, int w0) {
        // S^T = K Q^T: A = 16 K rows x 32 dims (lane: row l16, dims 8 lq + 0..7), B = Q^T
        f32x4_t sacc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            sacc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4_t kv =
                    *reinterpret_cast<const u32x4_t*>(s_kv + kpos_byte<D>(rbase + 16 * kb + l16, 4 * ks + lq));
                sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv), qop[ks],
                                                                     sacc[kb], 0, 0, 0);
            }
        }
        // online softmax for head l16 over rows rbase + 16 kb + 4 lq + i (base-2 exponent)
        float sc[KB][4];
        float tm = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = rbase + 16 * kb + 4 * lq + i;
                const bool valid = rr < vrows && (row0 + rr >= w0 || row0 + rr < n_sink);
                sc[kb][i] = valid ? sacc[kb][i] * scale_log2 : -INFINITY;
                tm = fmaxf(tm, sc[kb][i]);
            }
        tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
        tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
        const float mn = fmaxf(m_run, tm);
        const float mref = (mn == -INFINITY) ? 0.f : mn;
        const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m_run - mn);
        m_run = mn;
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc[kb][i] = fast_exp2(sc[kb][i] - mref);
                ps += sc[kb][i];
            }
        l_run = l_run * alpha + ps;
        // weights to LDS: s_p[wave][row][head]
        if (l16 < HGW) {
            float* sp = reinterpret_cast<float*>(s_p[wave]);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) sp[(16 * kb + 4 * lq + i) * 4 + l16] = sc[kb][i];
        }
#pragma unroll
        for (int h = 0; h < HGW; ++h) {
            const float ah = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), h));
#pragma unroll
            for (int x = 0; x < DPL; ++x) o[h][x] *= ah;
        }
        __builtin_amdgcn_wave_barrier();
        const unsigned char* vt = s_kv + TILEB;
#pragma unroll
        for (int rr = 0; rr < C::ROWS_W; ++rr) {
            const float4 p4 = s_p[wave][rr];
            const float pw[4] = {p4.x, p4.y, p4.z, p4.w};
            if (DPL == 2) {
                // row rbase + rr (rbase is a multiple of 16): its swizzle class is (rr >> 1) & 1
                const uint32_t vw =
                    *reinterpret_cast<const uint32_t*>(vt + (((rr >> 1) & 1) ? pv_base1 : pv_base0) + rr * ROWB);
                const float v0 = bf_lo(vw), v1 = bf_hi(vw);
#pragma unroll
                for (int h = 0; h < HGW; ++h) {
                    o[h][0] += pw[h] * v0;
                    o[h][DPL - 1] += pw[h] * v1;
                }
            } else {
                const uint32_t vh = *reinterpret_cast<const uint16_t*>(vt + pv_base0 + rr * ROWB);
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
        __builtin_amdgcn_wave_barrier();
    };

    // ---- main loop: two register stages, so the next two tiles' loads are in
    // flight while one is computed from LDS.  The prologue issues each stage
    // exactly as a step does (record stores first), so the counts of
    // outstanding loads on loop entry equal those on the back edge.
    u32x4_t st[C::LOADS], st2[C::LOADS];
    u32x4_t q1, q2;
    int tk1, tk2;
    Stage sA, sB;
    store_record(false, 0);
    issue(st2, q2, tk2, sA);
    store_record(false, 0);
    issue(st, q1, tk1, sB);
    reset_state();
    bool seg_start = true;  // the next tile computed starts a piece: its q rows go to LDS
    bool pend = false;      // a finished piece waits in s_park for its record store
    int pend_slot = 0;
    auto step = [&] __attribute__((always_inline)) (u32x4_t (&buf)[C::LOADS], u32x4_t& qbuf, int& tkbuf,
                                                     Stage& stg) {
        const Stage cs = stg;
        __syncthreads();  // every wave is done with the previous tile in LDS and has parked its state
        store_record(pend, pend_slot);
        pend = false;
#pragma unroll
        for (int x = 0; x < HALF; ++x) {
            *reinterpret_cast<u32x4_t*>(s_kv + stk_base + x * THREADS * 16) = buf[x];
            *reinterpret_cast<u32x4_t*>(s_kv + TILEB + st_base + x * THREADS * 16) = buf[HALF + x];
        }
        if (seg_start && tid < QPIECES) s_q[tid] = qbuf;
        if ((cs.flags & F_GRABBED) && tid == 0) s_ticket = tkbuf;
        __syncthreads();
        if (cs.flags & F_GRABBED) {
            take_ticket(uni(s_ticket));
            pending = false;
        }
        if (seg_start) load_qop();
        issue(buf, qbuf, tkbuf, stg);
        if ((cs.flags & KIND_MASK) == K_TILE) {
            compute_tile(cs.L - cs.tt * TILE, cs.tt * TILE, cs.w0);
            seg_start = (cs.flags & F_PIECE_END) != 0;
            if (seg_start) {
                park();
                reset_state();
                pend = true;
                pend_slot = cs.slot;
            }
        }
    };
    // Stages end in order (once one is END all later ones are), so a single
    // exit at the bottom suffices: stage A is never END at the top, and a step
    // on an END stage (possible for B) only stores the pending record.  One
    // exit keeps every path into the loop head issuing the same loads.
    if ((sA.flags & KIND_MASK) != K_END) {
        do {
            step(st2, q2, tk2, sA);
            step(st, q1, tk1, sB);
        } while ((sA.flags & KIND_MASK) != K_END);
    }
    __syncthreads();
    store_record(pend, pend_slot);
}

// Merge of the partial records of one (sequence, query head), in a fixed
// order: the static shares that hold tiles of the head's segment, in
// workgroup order, then its chunks in chunk order.  Where they are comes from
// the directory the partial kernel wrote.  Four waves share the records
// (wave k takes records k, k+4, ...), each merging its own online (running
// max, rescaled sum and output) with all of its loads in flight together; the
// four states then merge in wave order through LDS.  Block (0, 0) also clears
// the ticket counter, so the next call starts from zero.
constexpr int CMB_WAVES = 4;
// The records of one segment, in merge order: the static shares of
// workgroups w_lo .. w_lo + n_st - 1 (slots st0 ..), then consecutive chunk
// records (slots dy0 ..).
struct RecordList {
    int nrec, n_st, w_lo, st0, dy0;
    long long Ts;
};
// Slot of record idx (record 0's for idx >= nrec) and whether it holds data:
// a static share can be empty when the weights make it shorter than a tile.
__device__ __forceinline__ int record_slot(const RecordList rl, int idx, const Shares sh, bool& use) {
    use = idx < rl.nrec;
    if (!use) idx = 0;
    if (idx < rl.n_st) {
        const int w = rl.w_lo + idx;
        use = use && share_begin(w, rl.Ts, sh) < share_begin(w + 1, rl.Ts, sh);
        return rl.st0 + idx;
    }
    return rl.dy0 + (idx - rl.n_st);
}
template <int D>
__global__ __launch_bounds__(64 * CMB_WAVES) void decode_combine_kernel(float* __restrict__ ws,
                                                                        const int4* __restrict__ dir,
                                                                        const float* __restrict__ recs,
                                                                        uint16_t* __restrict__ out, int n_q,
                                                                        int n_kv, int nhc, int gc,
                                                                        const float* sink_logits, Shares shares) {
    constexpr int DPL = D / 64;  // dims per lane
    constexpr int REC = D + 4;
    constexpr int RB = 8;        // records per wave and batch
    __shared__ float s_acc[CMB_WAVES][D];
    __shared__ float2 s_ml[CMB_WAVES];
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = n_q / n_kv;
    if (h == 0 && b == 0 && tid == 0) reinterpret_cast<int*>(ws)[0] = 0;
    const size_t slot_floats = (size_t)gc * REC;

    const int j = h / g, hh = h % g, hc = hh / gc, hl = hh % gc;
    const int seg = (b * n_kv + j) * nhc + hc;
    const int4 e0 = dir[2 * seg], e1 = dir[2 * seg + 1];
    // record idx is used if it exists and (static) its workgroup had a non-empty share;
    // record 0 always exists, so unused entries read it and are ignored
    const RecordList rl{e0.y + e0.w, e0.y, e1.x, e0.x, e0.z, e1.y};
    const int nrec = rl.nrec;

    float M = -INFINITY, L = 0.f, acc[DPL];
#pragma unroll
    for (int x = 0; x < DPL; ++x) acc[x] = 0.f;
    for (int base = wave; base < nrec; base += CMB_WAVES * RB) {
        float2 ml[RB];
        float ov[RB][DPL];
        bool use[RB];
        // lane u (< RB) locates record u of the batch once; the wave reads the results back
        bool use_l;
        const int slot_l = record_slot(rl, base + CMB_WAVES * (lane % RB), shares, use_l);
        const unsigned long long use_mask = __builtin_amdgcn_ballot_w64(use_l);
#pragma unroll
        for (int u = 0; u < RB; ++u) {
            use[u] = ((use_mask >> u) & 1ull) != 0;
            const int slot_u = __builtin_amdgcn_readlane(slot_l, u);
            const float* rp = recs + (size_t)slot_u * slot_floats + (size_t)hl * REC;
            ml[u] = *reinterpret_cast<const float2*>(rp);
#pragma unroll
            for (int x = 0; x < DPL; ++x) ov[u][x] = rp[4 + DPL * lane + x];
        }
#pragma unroll
        for (int u = 0; u < RB; ++u) {
            const float m = ml[u].x;
            if (!use[u] || m == -INFINITY) continue;
            const float mn = fmaxf(M, m);
            const float a = (M == -INFINITY) ? 0.f : fast_exp2(M - mn);
            const float f = fast_exp2(m - mn);
            L = L * a + f * ml[u].y;
#pragma unroll
            for (int x = 0; x < DPL; ++x) acc[x] = acc[x] * a + f * ov[u][x];
            M = mn;
        }
    }
#pragma unroll
    for (int x = 0; x < DPL; ++x) s_acc[wave][DPL * lane + x] = acc[x];
    if (lane == 0) s_ml[wave] = make_float2(M, L);
    __syncthreads();
    if (wave != 0) return;
    // a learned sink logit (natural units, like the scaled scores) joins the
    // normaliser as one more term with no value
    const float sk = sink_logits ? sink_logits[h] * LOG2E : -INFINITY;
    float Mt = sk;
#pragma unroll
    for (int k = 0; k < CMB_WAVES; ++k) Mt = fmaxf(Mt, s_ml[k].x);
    float Lt = sk == -INFINITY ? 0.f : fast_exp2(sk - Mt), o[DPL];
#pragma unroll
    for (int x = 0; x < DPL; ++x) o[x] = 0.f;
#pragma unroll
    for (int k = 0; k < CMB_WAVES; ++k) {
        const float2 mlk = s_ml[k];
        if (mlk.x == -INFINITY) continue;
        const float f = fast_exp2(mlk.x - Mt);
        Lt += f * mlk.y;
#pragma unroll
        for (int x = 0; x < DPL; ++x) o[x] += f * s_acc[k][DPL * lane + x];
    }
    const float inv = 1.f / Lt;
    uint16_t* dst = out + (size_t)(b * n_q + h) * D + DPL * lane;
    if (DPL == 2) {
        *reinterpret_cast<uint32_t*>(dst) = cvt_pk_bf16(o[0] * inv, o[DPL - 1] * inv);
    } else {
        dst[0] = (uint16_t)f32_to_bf16_rne(o[0] * inv);
    }
}

template <int D, int HGW, int NHG>
hipError_t launch_partial_t(int G, const uint16_t* q_rot, const uint16_t* k_cache, const uint16_t* v_cache,
                            const int32_t* past_len, int pmax, float* ws, int4* dir, float* recs, int B, int n_q,
                            int n_kv, int S, int nhc, float scale_log2, int static_pm, int chunk, int window,
                            int n_sink, const Shares& shares, hipStream_t st) {
    const size_t dyn = (size_t)(2 * B + 1) * sizeof(int);
    hipLaunchKernelGGL((decode_partial_kernel<D, HGW, NHG>), dim3(G), dim3(THREADS), dyn, st, q_rot, k_cache,
                       v_cache, past_len, pmax, ws, dir, recs, B, n_q, n_kv, S, nhc, scale_log2, static_pm, chunk,
                       window, n_sink, shares);
    return hipGetLastError();
}

template <int D, int HGW, int NHG>
int occupancy_t(int B) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_partial_kernel<D, HGW, NHG>, THREADS,
                                                     (size_t)(2 * B + 1) * sizeof(int)) != hipSuccess)
        return 1;
    return blocks > 0 ? blocks : 1;
}

using occ_fn = int (*)(int);
using partial_fn = hipError_t (*)(int, const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*, int, float*,
                                  int4*, float*, int, int, int, int, int, float, int, int, int, int, const Shares&,
                                  hipStream_t);

struct Variant {
    int hgw, nhg;
    partial_fn fn128, fn64;
    occ_fn occ128, occ64;
};
// Default share ratio between dispatch slots, by head groups per workgroup:
// measured best at 1.4 for one head group (g = 4, 32/8 heads, two workgroups
// per CU) and 1.2 for two (g = 8, 64/8 heads, three per CU); the others take
// 1.2.
int default_slot_ratio(const Variant& v) { return v.nhg == 1 ? 1400 : 1200; }

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

int g_static_pm = -1;  // -1: chosen per launch (see launch_decode)
int g_chunk = DECODE_DEFAULT_CHUNK;
int g_slot_ratio_pm = 0;  // 0: the kernel variant's default

// Share weights for a grid of G workgroups on n_cu CUs: slot s (of ns) weighs
// ratio^(ns - 1 - s), the youngest slot 1 (in units of 1/1000).
Shares make_shares(int G, int n_cu, int ratio_pm) {
    static_assert(DECODE_MAX_SLOTS == 4, "the share struct holds four slots");
    if (n_cu < 1) n_cu = 1;
    // more rounds than weights (a small GPU with a large grid): widen the rounds
    if ((G + n_cu - 1) / n_cu > DECODE_MAX_SLOTS) n_cu = (G + DECODE_MAX_SLOTS - 1) / DECODE_MAX_SLOTS;
    int ns = (G + n_cu - 1) / n_cu;
    if (ns < 1) ns = 1;
    unsigned long long wt[DECODE_MAX_SLOTS] = {0, 0, 0, 0}, cnt[DECODE_MAX_SLOTS] = {0, 0, 0, 0};
    double w = 1000.0;
    for (int s = ns - 1; s >= 0; --s) {
        wt[s] = (unsigned long long)(w + 0.5);
        w = w * ratio_pm / 1000.0;
        if (w > 1.0e6) w = 1.0e6;  // bounded: wt << 32 stays below 2^52
    }
    unsigned long long total = 0;
    for (int s = 0; s < ns; ++s) {
        cnt[s] = (s + 1) * n_cu <= G ? n_cu : G - s * n_cu;
        total += cnt[s] * wt[s];
    }
    // per-workgroup fractions rounded down, so the fractions sum to at most 2^32
    unsigned long long g[DECODE_MAX_SLOTS], f[DECODE_MAX_SLOTS + 1];
    f[0] = 0;
    for (int s = 0; s < DECODE_MAX_SLOTS; ++s) {
        g[s] = (wt[s] << 32) / total;
        f[s + 1] = f[s] + cnt[s] * g[s];
    }
    Shares sh;
    sh.n_cu = n_cu;
    sh.ns = ns;
    sh.G = G;
    sh.f1 = f[1]; sh.f2 = f[2]; sh.f3 = f[3];
    sh.g0 = g[0]; sh.g1 = g[1]; sh.g2 = g[2]; sh.g3 = g[3];
    return sh;
}

}  // namespace

void set_decode_schedule(int static_permille, int chunk_tiles) {
    g_static_pm = static_permille;
    g_chunk = chunk_tiles;
}


void set_decode_slot_ratio(int ratio_permille) { g_slot_ratio_pm = ratio_permille; }
int decode_slot_ratio() { return g_slot_ratio_pm; }

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
    p.slot_floats = (size_t)p.gc * p.rec;
    return p;
}

namespace {
int g_wide_min = DECODE_WIDE_MIN_G;

// workspace of the split-K path, and of the wide-group path where it can take the shape
// Split-K workspace layout: the 256-byte header, the record directory (two
// int4 per segment of one launch), then the records.
size_t split_segments(int B, int n_q, int n_kv, int d) {
    const DecodePlan p = decode_plan(n_q, n_kv, d);
    const int bs = B < DECODE_MAX_B ? B : DECODE_MAX_B;
    return (size_t)bs * n_kv * p.nhc;
}
size_t split_workspace_bytes(int B, int n_q, int n_kv, int d) {
    const DecodePlan p = decode_plan(n_q, n_kv, d);
    const size_t segs = split_segments(B, n_q, n_kv, d);
    // static pieces: segment + workgroup < segs + G; chunk pieces: segs + G + chunk + segment
    const size_t slots = 2 * segs + DECODE_MAX_WG + DECODE_MAX_CHUNKS;
    return (HDR_FLOATS + 8 * segs + slots * p.slot_floats) * sizeof(float);
}
bool wide_eligible(int n_q, int n_kv) { return n_q / n_kv <= DECODE_WIDE_MAX_G && n_kv <= DECODE_WIDE_MAX_SEGS; }
size_t wide_workspace_bytes(int B, int n_q, int n_kv, int d) {
    return HDR_FLOATS * sizeof(float) + decode_wide_record_bytes(B, n_q, n_kv, d);
}
bool takes_wide(int n_q, int n_kv) { return wide_eligible(n_q, n_kv) && n_q / n_kv >= g_wide_min; }
}  // namespace

size_t decode_workspace_bytes(int B, int n_q, int n_kv, int d) {
    size_t need = split_workspace_bytes(B, n_q, n_kv, d);
    // the same workspace serves the wide-group kernel whenever it may take the
    // shape (its threshold can be changed between calls)
    if (wide_eligible(n_q, n_kv)) {
        const size_t wide = wide_workspace_bytes(B, n_q, n_kv, d);
        if (wide > need) need = wide;
    }
    return need;
}

size_t decode_launch_workspace_bytes(int B, int n_q, int n_kv, int d) {
    return takes_wide(n_q, n_kv) ? wide_workspace_bytes(B, n_q, n_kv, d) : split_workspace_bytes(B, n_q, n_kv, d);
}

void set_decode_wide_min_group(int g) { g_wide_min = g > 0 ? g : DECODE_WIDE_MIN_G; }
int decode_wide_min_group() { return g_wide_min; }

// sched_hdr: where the split-K scheduling header (the ticket counter) lives,
// when not at the start of ws (the caller keeps it zero at rest); the record
// directory and the records follow ws's own header either way.
hipError_t launch_decode(const uint16_t* q_rot, const uint16_t* k_cache, const uint16_t* v_cache,
                         const int32_t* past_len, int max_past_len, uint16_t* out, float* ws, int B, int n_q,
                         int n_kv, int d, int S, float scale, int window, int n_sink, const float* sink_logits,
                         int wg_override, hipStream_t st, float* sched_hdr) {
    if (takes_wide(n_q, n_kv))
        return launch_decode_wide(q_rot, k_cache, v_cache, past_len, max_past_len, out, ws, B, n_q, n_kv, d, S, scale,
                                  window, n_sink, sink_logits, wg_override, st);
    const DecodePlan p = decode_plan(n_q, n_kv, d);
    const Variant& v = pick_variant(n_q / n_kv);

    int cu_count = 0;
    {
        const hipError_t e = device_cu_count(&cu_count);
        if (e != hipSuccess) return e;
    }
    int G = wg_override;
    // default: one wave of workgroups, as many as fit on the chip at once, but
    // at most two per CU for one head group per workgroup (up to 4 heads per
    // segment): there two already keep HBM busy, and with fewer, longer
    // workgroups the ones still running at the end finish sooner
    if (G <= 0) {
        const int bs = B < DECODE_MAX_B ? B : DECODE_MAX_B;
        int per_cu = d == 128 ? v.occ128(bs) : v.occ64(bs);
        if (v.nhg == 1 && per_cu > 2) per_cu = 2;
        G = cu_count * per_cu;
    }
    // never more workgroups than tiles: a small problem would otherwise have
    // most workgroups queue on the ticket counter with nothing to do
    long long tiles_bound;  // tiles of one launch with every past_len at max_past_len
    {
        long long per_seg = (max_past_len + 1 + TILE - 1) / TILE;
        if (window > 0) {
            const long long wt = (n_sink + TILE - 1) / TILE + (window + TILE - 1) / TILE + 1;
            if (wt < per_seg) per_seg = wt;
        }
        const long long bs = B < DECODE_MAX_B ? B : DECODE_MAX_B;
        tiles_bound = bs * n_kv * p.nhc * per_seg;
        if (G > tiles_bound) G = (int)tiles_bound;
    }
    if (G > DECODE_MAX_WG) G = DECODE_MAX_WG;
    if (G < 1) G = 1;
    const float scale_log2 = scale * LOG2E;
    // Default schedule: with at most DECODE_STATIC_ONLY_TILES tiles per
    // workgroup (small batches) every tile goes into a static share.  There the
    // slot-weighted shares already balance the workgroups, and a dynamic tail
    // only adds ticket round trips ahead of the first loads and more records
    // (measured: B4 30.1 -> 23.9 us, B16 59.7 -> 57.3 us at contexts up to
    // 8192); with many tiles per workgroup the tail absorbs the spread
    // between workgroups (the 70B shape is 1.2 % faster with it).
    const int spm = g_static_pm >= 0 ? g_static_pm
                  : (tiles_bound <= (long long)DECODE_STATIC_ONLY_TILES * G ? 1000 : DECODE_DEFAULT_STATIC_PM);
    const Shares shares = make_shares(G, cu_count, g_slot_ratio_pm > 0 ? g_slot_ratio_pm : default_slot_ratio(v));
    float* const hdr = sched_hdr ? sched_hdr : ws;
    int4* const dir = reinterpret_cast<int4*>(ws + HDR_FLOATS);
    float* const recs = ws + HDR_FLOATS + 8 * split_segments(B, n_q, n_kv, d);

    for (int b0 = 0; b0 < B; b0 += DECODE_MAX_B) {
        const int nb = (B - b0) < DECODE_MAX_B ? (B - b0) : DECODE_MAX_B;
        const uint16_t* q = q_rot + (size_t)b0 * n_q * d;
        const uint16_t* kc = k_cache + (size_t)b0 * n_kv * S * d;
        const uint16_t* vc = v_cache + (size_t)b0 * n_kv * S * d;
        const int32_t* pl = past_len + b0;
        uint16_t* o = out + (size_t)b0 * n_q * d;

        // chunk size: the requested one, grown if the dynamic part could need
        // more than DECODE_MAX_CHUNKS chunks (bounded with every past_len at max_past_len)
        const long long t_max = (long long)nb * n_kv * p.nhc * ((max_past_len + 1 + TILE - 1) / TILE);
        const long long t_dyn = t_max - t_max * spm / 1000;
        long long chunk = g_chunk;
        const long long need = (t_dyn + DECODE_MAX_CHUNKS - 1) / DECODE_MAX_CHUNKS;
        if (chunk < need) chunk = need;

        prof_begin(K_DECODE_PARTIAL, st);
        hipError_t e = (d == 128 ? v.fn128 : v.fn64)(G, q, kc, vc, pl, max_past_len, hdr, dir, recs, nb, n_q, n_kv, S,
                                                     p.nhc, scale_log2, spm, (int)chunk, window, n_sink, shares, st);
        prof_end(K_DECODE_PARTIAL, st);
        if (e != hipSuccess) return e;

        prof_begin(K_DECODE_COMBINE, st);
        if (d == 128)
            hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(n_q, nb), dim3(64 * CMB_WAVES), 0, st, hdr, dir, recs,
                               o, n_q, n_kv, p.nhc, p.gc, sink_logits, shares);
        else
            hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(n_q, nb), dim3(64 * CMB_WAVES), 0, st, hdr, dir, recs,
                               o, n_q, n_kv, p.nhc, p.gc, sink_logits, shares);
        prof_end(K_DECODE_COMBINE, st);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gqa
