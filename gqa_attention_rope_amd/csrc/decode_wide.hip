// Decode attention for wide query groups (16 or more query heads per KV head, up
// to multi-query attention with g = n_q): both products on MFMA, each K/V row
// read once for all g heads.
//
// What is computed is the same as the split-K decode path ([KV] "Llama 3.1 8B
// KV cache", "The cache itself is concatenation"; [REP] "Llama 3.1 8B - Repeat
// heads" formula: query head h reads KV head floor(h / g); [EP18]
// "Grouped-query attention: a smaller KV cache", where n_kv = 1 is MQA): the
// new query of each head attends to cache rows 0 .. past_len[b] (or its
// window and sinks).
//
// Why a separate kernel: with g query heads per K/V row the work per byte is
// g times that of one head.  The split-K kernel keeps at most 16 heads per
// segment (its weighted value sum runs on VALU) and streams the rows again
// for every further 16; here a workgroup keeps all g heads and both q.k and
// the weighted value sum are dense [g x 64] products on the matrix cores.
//
// How:
//  * Grid (split, KV head j, sequence b), 4 waves.  A segment's tiles (64 rows;
//    sink and window tiles only, under a window) are cut into nsplit
//    contiguous ranges.  Wave w owns head block hb = w % HB (16 heads; HB = 1,
//    2 or 4 blocks for g <= 16, 32, 64) and row group w / HB of each tile
//    (RG = 4 / HB groups of 64 / RG rows).
//  * A tile's K and V rows go from HBM straight into LDS (range-checked
//    buffer loads with the LDS destination), row-major with an XOR swizzle of
//    the 16-byte pieces: the MFMA A operand reads of K (16 rows of one piece)
//    and the transposed V reads (ds_read_b64_tr_b16, 16 rows of two pieces)
//    both spread over all banks.  Double-buffered: the next tile's loads are
//    in flight while the current one is computed, one barrier per tile.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (A: 16 K rows x 32 dims; B: the
//    wave's 16 rotated q rows, held in registers).  Lane l then holds rows
//    4(l/16)+i of each 16-row block for head l%16: exactly the A operand of
//    O += P V when the 32 rows of a K-step are taken in that order, so P never
//    leaves the registers.  P enters as a bf16 high part plus a bf16
//    remainder (two MFMAs, about 16 significant bits); V's B operand follows
//    the same row order (two transposed 8-byte reads per lane).  With 16 rows
//    per wave (g <= 16) the k-step is those 16 rows, on
//    v_mfma_f32_16x16x16_bf16 with one transposed read.
//  * Online softmax per head (two lane shuffles per reduction); the output
//    rescale fetches each head's factor from the lanes that own it.
//  * The row groups of a head block merge their (max, sum, unnormalised
//    output) states through LDS in row-group order, and each split writes one
//    record per head.  The split count keeps every segment's records (all
//    heads of all splits) within 2048, which bounds the record traffic for
//    large g against the parallelism that more splits buy.  A second kernel merges the
//    records of each (sequence, query head) in a fixed order with one wave per
//    head: reproducible for a given shape.
#include <float.h>

#include "attn_window.hpp"
#include "common.hpp"
#include "kernels.hpp"
#include "lds_direct.hpp"

namespace gqa {

namespace {

constexpr int WD_THREADS = 256;
constexpr int WD_TILE = 64;
constexpr float WD_LOG2E = 1.4426950408889634f;
constexpr uint32_t WD_RSRC = 0x00020000u;  // raw buffer, 32-bit dwords

// Wave-wide max and sum in registers: DPP inside each row of 16 (quad_perm
// [1,0,3,2], [2,3,0,1], row_ror:4, row_ror:8), then the rows paired with
// v_permlane16_swap and v_permlane32_swap; no LDS permutes.  The sum's
// association differs between lanes, so it is returned as lane 0's value:
// every lane then uses the same, reproducible total.
template <bool MAX>
__device__ __forceinline__ float wd_wave_reduce(float v) {
    auto op = [](float a, float b) { return MAX ? __builtin_elementwise_maximum(a, b) : a + b; };
    v = op(v, dpp_f32<0xB1>(v));
    v = op(v, dpp_f32<0x4E>(v));
    v = op(v, dpp_f32<0x124>(v));
    v = op(v, dpp_f32<0x128>(v));
    const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
    const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
__device__ __forceinline__ float wd_wave_max(float v) { return wd_wave_reduce<true>(v); }
__device__ __forceinline__ float wd_wave_sum(float v) { return wd_wave_reduce<false>(v); }

// D head size; HB blocks of 16 heads (g <= 16 HB), HB in {1, 2, 4}
template <int D, int HB>
__global__ __launch_bounds__(WD_THREADS, 2) void decode_wide_kernel(
    const uint16_t* __restrict__ q_rot, const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ past_len, int pmax, float* __restrict__ recs, int n_q, int n_kv, int S, int nsplit,
    float scale_log2, int window, int n_sink) {
    constexpr int PPR = D / 8;                       // 16-byte pieces per row
    constexpr int ROWB = D * 2;
    constexpr int TILEB = WD_TILE * ROWB;            // bytes of one tensor's tile
    constexpr int HALF = TILEB / (16 * WD_THREADS);  // 16-byte loads per thread per tensor
    constexpr int RG = 4 / HB;                       // row groups
    constexpr int ROWS_W = WD_TILE / RG;             // rows of a tile per wave (16, 32 or 64)
    constexpr int KB = ROWS_W / 16;                  // 16-row blocks per wave
    constexpr int KS = D / 32;                       // MFMA k-steps over the head dim
    constexpr int DB = D / 16;                       // 16-dim blocks of the output
    constexpr int REC = D + 4;

    // K buffers 0 and 1, then V buffers 0 and 1
    __shared__ __align__(16) unsigned char smem[4 * TILEB];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    const int hb = wave % HB, rg = wave / HB;
    const int sp = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int g = n_q / n_kv;
    int P = past_len[b];
    P = P < 0 ? 0 : (P > pmax ? pmax : P);
    const int L = P + 1;
    const Geo geo = geo_of(L, window, n_sink);
    const int t0 = (int)((long long)sp * geo.nt / nsplit);
    const int t1 = (int)((long long)(sp + 1) * geo.nt / nsplit);
    auto abs_tile = [&](int i) { return i < geo.nst ? i : geo.at0 + (i - geo.nst); };

    // K/V rows 0 .. L-1 of the segment (the hardware range check zero-fills the rest)
    const size_t seg = (size_t)(b * n_kv + j) * S * D;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(k_cache + seg), (short)0, L * ROWB, WD_RSRC);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(v_cache + seg), (short)0, L * ROWB, WD_RSRC);
    // Load x of wave w fills slots x * 256 + 64 w + lane of a tile (lane i's 16
    // bytes land at the wave's LDS base + 16 i), so each lane fetches the
    // global piece that the swizzle puts at its slot: piece c of row r sits
    // at slot r * PPR + (c ^ (r mod PPR)).
    int dma_off[HALF];
#pragma unroll
    for (int x = 0; x < HALF; ++x) {
        const int slot = x * WD_THREADS + wave * 64 + lane;
        const int r = slot / PPR, c = (slot % PPR) ^ (r & (PPR - 1));
        dma_off[x] = r * ROWB + c * 16;
    }
    const uint32_t lds_base = lds_addr(smem);
    auto load_tile = [&](int i, int buf) {
        const int soff = abs_tile(i) * TILEB;
#pragma unroll
        for (int x = 0; x < HALF; ++x) {
            const uint32_t dst = lds_base + (uint32_t)((x * WD_THREADS + wave * 64) * 16);
            if (HB <= 2) {  // non-temporal: each row is read once per launch
                load_lds16_nt(rk, dst + (uint32_t)(buf * TILEB), dma_off[x], soff);
                load_lds16_nt(rv, dst + (uint32_t)((2 + buf) * TILEB), dma_off[x], soff);
            } else {
                load_lds16(rk, dst + (uint32_t)(buf * TILEB), dma_off[x], soff);
                load_lds16(rv, dst + (uint32_t)((2 + buf) * TILEB), dma_off[x], soff);
            }
        }
    };
    if (t0 < t1) load_tile(t0, 0);
    // V operand reads: lane 16G + 4i + q names row 4G + i (+ the 16-row offset
    // of the read) and dims 16 db + 4q .. + 3, and receives rows 4G + 0..3 of
    // dim 16 db + (lane mod 16): the row order of the weights' registers.
    const int vr = lane >> 2, vq = lane & 3;
    int v_rd[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        v_rd[db] = vr * ROWB + (((2 * db + (vq >> 1)) ^ (vr & (PPR - 1))) << 4) + ((vq & 1) << 3);

    // B operand of the scores: 8 dims of head 16 hb + l16 per k-step (zero beyond g)
    const int hq = 16 * hb + l16;
    bf16x8_t qop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
        if (hq < g) v = *reinterpret_cast<const u32x4_t*>(q_rot + (size_t)(b * n_q + j * g + hq) * D + 32 * ks + 8 * lq);
        qop[ks] = __builtin_bit_cast(bf16x8_t, v);
    }

    float m_run = -INFINITY, l_run = 0.f;  // head l16 of the block (l_run: this lane's share)
    f32x4_t oacc[DB];                      // O[head 4 lq + i][dim 16 db + l16]
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int i = t0; i < t1; ++i) {
        const int at = abs_tile(i);
        const int buf = (i - t0) & 1;
        // this wave's loads of the tile are done; after the barrier every
        // wave's are, and every wave has finished the previous tile, whose
        // buffers the next loads overwrite
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (i + 1 < t1) load_tile(i + 1, buf ^ 1);
        const unsigned char* s_k = smem + buf * TILEB;
        const unsigned char* s_v = smem + (2 + buf) * TILEB;
        // Issue priority grows with the tiles left, so that of two workgroups
        // sharing a CU the one with more work is served first and the two
        // tend to finish together (ragged contexts make the splits unequal).
        {
            const int rem = t1 - i;
            if (rem > 12) __builtin_amdgcn_s_setprio(3);
            else if (rem > 8) __builtin_amdgcn_s_setprio(2);
            else if (rem > 4) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        }

        // scores of this wave's rows for its 16 heads
        f32x4_t sacc[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            sacc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            const int r = rg * ROWS_W + 16 * k + l16;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4_t kv =
                    *reinterpret_cast<const u32x4_t*>(s_k + r * ROWB + 16 * ((4 * ks + lq) ^ (r & (PPR - 1))));
                sacc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv), qop[ks], sacc[k],
                                                                   0, 0, 0);
            }
        }
        // online softmax for head l16 over rows rg*ROWS_W + 16k + 4lq + e
        float tm = -INFINITY;
#pragma unroll
        for (int k = 0; k < KB; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = at * WD_TILE + rg * ROWS_W + 16 * k + 4 * lq + e;
                const bool vis = row < L && (row >= geo.w0 || row < n_sink);
                sacc[k][e] = vis ? sacc[k][e] * scale_log2 : -INFINITY;
                tm = __builtin_elementwise_maximum(tm, sacc[k][e]);  // v_maximum3: no input canonicalising
            }
        {
            // lanes l, l ^ 16, l ^ 32, l ^ 48 hold the same head: in-register lane swaps, not LDS permutes
            const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tm), __float_as_uint(tm), false, false);
            tm = __builtin_elementwise_maximum(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
            const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tm), __float_as_uint(tm), false, false);
            tm = __builtin_elementwise_maximum(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
        }
        const float mn = fmaxf(m_run, tm);
        const float mref = mn == -INFINITY ? 0.f : mn;
        const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m_run - mn);
        m_run = mn;
        float ps = 0.f;
#pragma unroll
        for (int k = 0; k < KB; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sacc[k][e] = fast_exp2(sacc[k][e] - mref);
                ps += sacc[k][e];
            }
        l_run = l_run * alpha + ps;
        // rescale the output rows: lane holds heads 4 lq + e
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = __shfl(alpha, 4 * lq + e, 64);
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db][e] *= a;
        }
        if constexpr (KB == 1) {
            // O += P V over the wave's 16 rows in one k-step: k index 4 lq + e <-> row 4 lq + e
            const f32x4_t p0 = sacc[0];
            const uint32_t h0 = cvt_pk_bf16(p0[0], p0[1]), h1 = cvt_pk_bf16(p0[2], p0[3]);
            const i16x4_t hi = __builtin_bit_cast(i16x4_t, make_uint2(h0, h1));
            const i16x4_t lo = __builtin_bit_cast(
                i16x4_t, make_uint2(cvt_pk_bf16(p0[0] - bf_lo(h0), p0[1] - bf_hi(h0)),
                                    cvt_pk_bf16(p0[2] - bf_lo(h1), p0[3] - bf_hi(h1))));
            const int r0 = rg * ROWS_W;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const i16x4_t bop = read_tr16(s_v + v_rd[db] + r0 * ROWB);
                oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, bop, oacc[db], 0, 0, 0);
                oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, bop, oacc[db], 0, 0, 0);
            }
        } else {
            // O += P V, 32 rows per k-step: k index 8 lq + e <-> row 16 (2 kk) + 4 lq + e (e < 4),
            // row 16 (2 kk + 1) + 4 lq + e - 4 (e >= 4), the order the score registers already have
    #pragma unroll
            for (int kk = 0; kk < KB / 2; ++kk) {
                const f32x4_t p0 = sacc[2 * kk], p1 = sacc[2 * kk + 1];
                const uint32_t h0 = cvt_pk_bf16(p0[0], p0[1]), h1 = cvt_pk_bf16(p0[2], p0[3]);
                const uint32_t h2 = cvt_pk_bf16(p1[0], p1[1]), h3 = cvt_pk_bf16(p1[2], p1[3]);
                const u32x4_t hi = {h0, h1, h2, h3};
                const u32x4_t lo = {cvt_pk_bf16(p0[0] - bf_lo(h0), p0[1] - bf_hi(h0)),
                                    cvt_pk_bf16(p0[2] - bf_lo(h1), p0[3] - bf_hi(h1)),
                                    cvt_pk_bf16(p1[0] - bf_lo(h2), p1[1] - bf_hi(h2)),
                                    cvt_pk_bf16(p1[2] - bf_lo(h3), p1[3] - bf_hi(h3))};
                const int r0 = rg * ROWS_W + 32 * kk + 4 * lq;
    #pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const i16x4_t a = read_tr16(s_v + v_rd[db] + (r0 - 4 * lq) * ROWB);
                    const i16x4_t c = read_tr16(s_v + v_rd[db] + (r0 - 4 * lq + 16) * ROWB);
                    const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a, c, 0, 1, 2, 3, 4, 5, 6, 7));
                    oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, hi), bop, oacc[db], 0,
                                                                        0, 0);
                    oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, lo), bop, oacc[db], 0,
                                                                        0, 0);
                }
            }
        }
    }

    // ---- record of this split: (m, l, pad, pad, o[D]) per head
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    const size_t segi = (size_t)b * n_kv + j;
    float* rbase = recs + (segi * nsplit + sp) * g * REC;
    if constexpr (RG > 1) {
        // Row groups merge in order through LDS (the tile buffers, free once
        // every wave is past its last tile): M = max m, l = sum l e^(m - M),
        // o = sum o e^(m - M); row group 0 of each head block writes the record.
        constexpr int NH = 16 * HB;  // heads of the workgroup
        float* s_o = reinterpret_cast<float*>(smem);                           // [RG][NH][D]
        float2* s_ml = reinterpret_cast<float2*>(s_o + (size_t)RG * NH * D);  // [RG][NH]
        static_assert((size_t)RG * NH * (D * 4 + 8) <= sizeof(smem), "merge state fits the tile buffers");
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                s_o[((size_t)rg * NH + 16 * hb + 4 * lq + e) * D + 16 * db + l16] = oacc[db][e];
        if (lq == 0) s_ml[rg * NH + 16 * hb + l16] = make_float2(m_run, l_run);
        __syncthreads();
        if (rg != 0) return;
        {
            float M = -INFINITY;
#pragma unroll
            for (int r = 0; r < RG; ++r) M = fmaxf(M, s_ml[r * NH + hq].x);
            float L = 0.f;
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                const float2 ml = s_ml[r * NH + hq];
                L += ml.x == -INFINITY ? 0.f : fast_exp2(ml.x - M) * ml.y;
            }
            m_run = M;
            l_run = L;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int hw = 16 * hb + 4 * lq + e;  // this lane's output head
            float M = -INFINITY;
#pragma unroll
            for (int r = 0; r < RG; ++r) M = fmaxf(M, s_ml[r * NH + hw].x);
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db][e] = 0.f;
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                const float mr = s_ml[r * NH + hw].x;
                const float w = mr == -INFINITY ? 0.f : fast_exp2(mr - M);
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db][e] += w * s_o[((size_t)r * NH + hw) * D + 16 * db + l16];
            }
        }
    }
    if (lq == 0 && hq < g) *reinterpret_cast<float2*>(rbase + (size_t)hq * REC) = make_float2(m_run, l_run);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int h = 16 * hb + 4 * lq + e;
        if (h < g) {
#pragma unroll
            for (int db = 0; db < DB; ++db) rbase[(size_t)h * REC + 4 + 16 * db + l16] = oacc[db][e];
        }
    }
}

// Merge the records of one (sequence, query head) in order: M = max m,
// out = sum o e^(m - M) / (sum l e^(m - M) [+ e^(sink - M)]).  One wave; lane r
// holds record r's (m, l).  Every load is issued before the first use: the
// (m, l) pairs and the output slices of records 0 .. NR-1 (NR >= nrec; the
// records past nrec re-read the last one and get weight zero), so the merge
// waits on memory once.
template <int D, int NR>
__global__ __launch_bounds__(64) void decode_wide_combine_kernel(const float* __restrict__ recs,
                                                                 uint16_t* __restrict__ out, int n_q, int n_kv,
                                                                 int nrec, const float* __restrict__ sink_logits) {
    constexpr int REC = D + 4, DPL = D / 64;
    const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const int g = n_q / n_kv, j = h / g, hl = h % g;
    // record r of head hl: recs + ((segment * nrec + r) * g + hl) * REC, one record per split, in split order
    const float* r0p = recs + ((size_t)(b * n_kv + j) * nrec * g + hl) * REC;
    const size_t stride = (size_t)g * REC;
    float m_l = -INFINITY, l_l = 0.f;
    if (lane < nrec) {  // nrec <= NR <= 64
        const float2 ml = *reinterpret_cast<const float2*>(r0p + lane * stride);
        m_l = ml.x;
        l_l = ml.y;
    }
    float ov[NR][DPL];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const float* rr = r0p + (r < nrec ? r : nrec - 1) * stride + 4 + DPL * lane;
#pragma unroll
        for (int x = 0; x < DPL; ++x) ov[r][x] = rr[x];
    }
    const float sk = sink_logits ? sink_logits[h] * WD_LOG2E : -INFINITY;
    const float M = fmaxf(wd_wave_max(m_l), sk);
    const float w_l = m_l == -INFINITY ? 0.f : fast_exp2(m_l - M);  // 0 for lanes >= nrec
    const float lsum = wd_wave_sum(w_l * l_l) + (sk == -INFINITY ? 0.f : fast_exp2(sk - M));
    float acc[DPL];
#pragma unroll
    for (int x = 0; x < DPL; ++x) acc[x] = 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l), r));
#pragma unroll
        for (int x = 0; x < DPL; ++x) acc[x] += w * ov[r][x];
    }
    const float inv = 1.f / lsum;
    uint16_t* dst = out + (size_t)(b * n_q + h) * D;
    if (DPL == 2)
        *reinterpret_cast<uint32_t*>(dst + 2 * lane) = cvt_pk_bf16(acc[0] * inv, acc[DPL - 1] * inv);
    else
        dst[lane] = (uint16_t)(cvt_pk_bf16(acc[0] * inv, 0.f) & 0xffffu);
}

template <int D>
hipError_t launch_wide_combine(const float* recs, uint16_t* out, int n_q, int n_kv, int nb, int nrec,
                               const float* sink_logits, hipStream_t st) {
    const dim3 grid(n_q, nb);
    if (nrec <= 16)
        hipLaunchKernelGGL((decode_wide_combine_kernel<D, 16>), grid, dim3(64), 0, st, recs, out, n_q, n_kv, nrec,
                           sink_logits);
    else if (nrec <= 32)
        hipLaunchKernelGGL((decode_wide_combine_kernel<D, 32>), grid, dim3(64), 0, st, recs, out, n_q, n_kv, nrec,
                           sink_logits);
    else
        hipLaunchKernelGGL((decode_wide_combine_kernel<D, 64>), grid, dim3(64), 0, st, recs, out, n_q, n_kv, nrec,
                           sink_logits);
    return hipGetLastError();
}

using wide_fn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*, int, float*, int, int, int,
                         int, float, int, int);

}  // namespace

// records per segment (all heads of all splits) stay within this many.  More
// splits buy parallelism with record traffic: for g = 64 at this cap a
// segment's records are about 40 % of its K/V bytes at 5k rows, and 1024
// (half the splits) measured 6.5 % slower on 16 MQA sequences.
constexpr int WD_MAX_SEG_RECORDS = 2048;

int decode_wide_splits(int nb, int n_kv, int g, int max_past_len, int window, int n_sink, int wg_override) {
    int cu_count = 256;  // (the launch itself reports a device error)
    if (device_cu_count(&cu_count) != hipSuccess) cu_count = 256;
    long long tiles = (max_past_len + 1 + 63) / 64;
    if (window > 0) {
        const long long wt = (n_sink + 63) / 64 + window / 64 + 2;
        if (wt < tiles) tiles = wt;
    }
    const long long segs = (long long)nb * n_kv;
    const long long target = wg_override > 0 ? wg_override : 2LL * cu_count;
    long long n = (target + segs - 1) / segs;
    const long long cap = WD_MAX_SEG_RECORDS / g;  // one record per head and split
    if (n > cap) n = cap;
    if (n > tiles) n = tiles;
    if (n > DECODE_WIDE_MAX_SPLITS) n = DECODE_WIDE_MAX_SPLITS;
    return n < 1 ? 1 : (int)n;
}

size_t decode_wide_record_bytes(int B, int n_q, int n_kv, int d) {
    int nb = DECODE_WIDE_MAX_SEGS / n_kv;
    if (nb > B) nb = B;
    // records per segment: g heads per split, at most DECODE_WIDE_MAX_SPLITS
    // splits and at most WD_MAX_SEG_RECORDS in all
    const int g = n_q / n_kv;
    long long recs = (long long)g * DECODE_WIDE_MAX_SPLITS;
    if (recs > WD_MAX_SEG_RECORDS) recs = WD_MAX_SEG_RECORDS;
    return (size_t)nb * n_kv * (size_t)recs * (d + 4) * sizeof(float);
}

hipError_t launch_decode_wide(const uint16_t* q_rot, const uint16_t* k_cache, const uint16_t* v_cache,
                              const int32_t* past_len, int max_past_len, uint16_t* out, float* ws, int B, int n_q,
                              int n_kv, int d, int S, float scale, int window, int n_sink, const float* sink_logits,
                              int wg_override, hipStream_t st) {
    const int g = n_q / n_kv;
    float* recs = ws + DECODE_WS_HEADER_FLOATS;
    wide_fn fn;
    if (d == 128)
        fn = g <= 16 ? decode_wide_kernel<128, 1> : g <= 32 ? decode_wide_kernel<128, 2> : decode_wide_kernel<128, 4>;
    else
        fn = g <= 16 ? decode_wide_kernel<64, 1> : g <= 32 ? decode_wide_kernel<64, 2> : decode_wide_kernel<64, 4>;
    const int per = DECODE_WIDE_MAX_SEGS / n_kv;  // sequences per launch (bounds the record space)
    for (int b0 = 0; b0 < B; b0 += per) {
        const int nb = (B - b0) < per ? (B - b0) : per;
        const int nsplit = decode_wide_splits(nb, n_kv, g, max_past_len, window, n_sink, wg_override);
        prof_begin(K_DECODE_WIDE, st);
        hipLaunchKernelGGL(fn, dim3(nsplit, n_kv, nb), dim3(WD_THREADS), 0, st, q_rot + (size_t)b0 * n_q * d,
                           k_cache + (size_t)b0 * n_kv * S * d, v_cache + (size_t)b0 * n_kv * S * d, past_len + b0,
                           max_past_len, recs, n_q, n_kv, S, nsplit, scale * WD_LOG2E, window, n_sink);
        prof_end(K_DECODE_WIDE, st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        prof_begin(K_DECODE_COMBINE, st);
        e = d == 128 ? launch_wide_combine<128>(recs, out + (size_t)b0 * n_q * d, n_q, n_kv, nb, nsplit, sink_logits,
                                                st)
                     : launch_wide_combine<64>(recs, out + (size_t)b0 * n_q * d, n_q, n_kv, nb, nsplit, sink_logits, st);
        prof_end(K_DECODE_COMBINE, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gqa
