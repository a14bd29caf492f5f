// Chunked-prefill attention on gfx950 bf16 MFMA.
//
// What is computed ([ATL] "Llama 3 8B - KV cache", Transformer.forward excerpt
// and its comment on the mask under a cache; [KV] "Llama 3.1 8B KV cache",
// "The cache itself is concatenation"): new row t of sequence b sits at
// position past_len[b] + t and attends to cache rows 0 .. past_len[b] + t of
// KV head floor(h / g).  The score block is rectangular, T x (past_len + T).
//
// How: a workgroup (4 waves) owns 128 query rows of one (sequence, KV head):
// up to 128/g positions times the g heads of the group, so every K/V tile it
// loads serves all heads that share it.  Per 64-key tile:
//   S^T = K Q^T   (v_mfma_f32_16x16x32_bf16: A = K rows from LDS, B = the
//                  wave's 32 query rows held in registers)
//   online softmax per query row (each lane holds one query row per 16-row
//                  block, so only two cross-lane steps are needed)
//   O^T += V^T P^T (A = V^T read from the row-major V tile with the
//                  transposing LDS read ds_read_b64_tr_b16, B = the softmax
//                  weights already in the right lanes, split into a bf16 high
//                  part and a bf16 remainder so that the weights enter the
//                  product with ~16 significant bits)
// K and V tiles go from HBM straight into LDS (range-checked buffer loads with
// the LDS destination, no register staging), each in its own double buffer
// with V one tile behind K, and one workgroup barrier per tile both publishes
// the new tiles and frees the old buffers.  The loop is software-pipelined:
// the score MFMAs of tile j+1 run while the weights of tile j are formed, and
// the second half of those weights while the first half goes through P V, so
// that exponentials and conversions overlap matrix work.  Tiles entirely
// above every row's causal bound are never loaded; tiles that straddle a
// bound are masked element-wise.
#include "common.hpp"
#include "kernels.hpp"
#include "lds_direct.hpp"

namespace gqa {

namespace {

constexpr int KT = 64;        // keys per tile
constexpr int NTHR = 256;     // 4 waves
constexpr int ROWS = 128;     // query rows per workgroup (32 per wave)
constexpr float LOG2E_P = 1.4426950408889634f;

// LDS tiles ([64 keys][D] bf16, row-major) are kept in 16-byte pieces; piece c
// of key row r sits at slot c ^ (r mod PPR).  With this swizzle the K operand
// reads (16 B per lane: 16 rows x 4 pieces) and the transposed V reads (8 B per
// lane: 16 rows x 2 pieces) each spread over all banks.
template <int D>
__global__ __launch_bounds__(NTHR, 2) void prefill_kernel(const uint16_t* __restrict__ q_rot,
                                                          const uint16_t* __restrict__ k_cache,
                                                          const uint16_t* __restrict__ v_cache,
                                                          const int32_t* __restrict__ past_len, int pmax,
                                                          uint16_t* __restrict__ out, int n_q, int n_kv, int T,
                                                          int S, int hpw, int tq, int n_tq, float scale_log2,
                                                          int window, int n_sink, const float* sink_logits) {
    static_assert(D == 64 || D == 128, "head sizes 64 and 128");
    constexpr int PPR = D / 8;                 // 16-byte pieces per key row
    constexpr int KS = D / 32;                 // MFMA k-steps over d
    constexpr int DB = D / 16;                 // 16-dim blocks of the output
    constexpr int ROW_B = D * 2;               // bytes per key row
    constexpr int TILE_B = KT * ROW_B;         // bytes per K (or V) tile
    constexpr int DMA_N = KT * PPR / NTHR;     // 16-byte pieces per thread, per tensor and tile
    // K buffers 0 and 1, then V buffers 0 and 1
    __shared__ __align__(16) unsigned char smem[4 * TILE_B];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    const int g = n_q / n_kv;
    // Work item of this workgroup: query tile tq_idx of group (b, j, hc).
    // Workgroups are dealt to the 8 XCDs round-robin by linear id, and when
    // the grid is two workgroups per CU, the CU pairs ids L and L + N/2, the
    // first of which wins most issue cycles.  Where the sizes allow, the map
    // therefore (a) keeps every group's query tiles on one XCD, so its K/V
    // tiles are reused from that XCD's L2, and (b) gives the ids of the first
    // half the tiles longest first and those of the second half shortest
    // first, so the two workgroups sharing a CU hold complementary amounts of
    // work.  Otherwise it falls back to longest first within each group.
    const int n_hc = gridDim.x / n_tq;
    const int n_groups = n_hc * (int)gridDim.y * (int)gridDim.z;
    const int n_wg = n_tq * n_groups;
    const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    int tq_idx, grp;
    if (n_groups % 16 == 0) {
        const int half = n_wg / 2;                 // a multiple of 8 n_tq
        const int hi = lin >= half, lh = lin - hi * half;
        const int xcd = lh & 7, k = lh >> 3;       // k-th workgroup of this half on this XCD
        const int per_xcd = n_groups / 16;         // groups per XCD and half
        grp = hi * (n_groups / 2) + xcd * per_xcd + k / n_tq;
        tq_idx = hi ? k % n_tq : n_tq - 1 - k % n_tq;
    } else {
        tq_idx = n_tq - 1 - (int)(blockIdx.x % n_tq);  // longest rows first
        grp = blockIdx.x / n_tq + n_hc * (blockIdx.y + gridDim.y * blockIdx.z);
    }
    const int hc = grp % n_hc;
    const int j = (grp / n_hc) % (int)gridDim.y, b = grp / (n_hc * (int)gridDim.y);
    int P = past_len[b];
    if (P < 0 || P > pmax) return;  // caller error: nothing is written for this sequence
    const int t0 = tq_idx * tq;

    // ---- this lane's query row in each of its two 16-row blocks
    int row_t[2], row_h[2];
    bool row_ok[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int rho = wave * 32 + nb * 16 + l16;
        const int hl = rho / tq, tl = rho % tq;
        const int h = hc * hpw + hl;
        row_ok[nb] = rho < hpw * tq && hl < hpw && h < g && t0 + tl < T;
        row_h[nb] = j * g + (h < g ? h : g - 1);
        row_t[nb] = row_ok[nb] ? t0 + tl : (t0 < T ? t0 : T - 1);
    }
    const int t_hi = (t0 + tq < T ? t0 + tq : T) - 1;
    const int kv_end = P + t_hi + 1;            // keys visible to the last row of this workgroup
    const int n_tiles = (kv_end + KT - 1) / KT;
    const int first_masked_tile = (P + t0 + 1) / KT;  // tiles before this one are fully visible (no window)
    // Under a sliding window, tiles wholly after the sink rows and before the
    // first row's window start (the earliest of this workgroup) hold no visible
    // key: the loop runs over the nst sink tiles, then from tile wt0 on.
    int nst = n_tiles, wt0 = n_tiles;
    if (window > 0) {
        const int ws0 = P + t0 - window + 1;  // first visible window key of row t0
        if (ws0 > n_sink) {
            nst = (n_sink + KT - 1) / KT;
            const int a0 = ws0 / KT;
            wt0 = a0 > nst ? a0 : nst;
        }
    }
    const int n_iter = nst < n_tiles ? nst + (n_tiles - wt0) : n_tiles;

    // ---- Q^T operand: 8 dims of one query row per lane and k-step
    bf16x8_t qop[2][KS];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const uint4* src = reinterpret_cast<const uint4*>(q_rot + ((size_t)row_h[nb] * T + row_t[nb]) * D +
                                                         (size_t)b * n_q * T * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 x = src[4 * ks + lq];
            qop[nb][ks] = __builtin_bit_cast(bf16x8_t, x);
        }
    }

    const uint16_t* kbase = k_cache + (size_t)(b * n_kv + j) * S * D;
    const uint16_t* vbase = v_cache + (size_t)(b * n_kv + j) * S * D;

    // Raw buffer loads over the visible rows only: the descriptor range is
    // kv_end rows, so the hardware returns zeros for keys past the last row any
    // query of this workgroup can see (no per-row branch, no read beyond them).
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, kv_end * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, kv_end * D * 2, 0x00020000);
    // Load x of wave w fills slots x * NTHR + 64 w + lane of a tile (the
    // hardware places lane i's 16 bytes at the wave's LDS base + 16 i), so each
    // lane fetches the global piece that the swizzle puts at its slot.
    int dma_off[DMA_N];
#pragma unroll
    for (int x = 0; x < DMA_N; ++x) {
        const int slot = x * NTHR + wave * 64 + lane;
        const int r = slot / PPR, c = (slot % PPR) ^ (r & (PPR - 1));
        dma_off[x] = r * ROW_B + c * 16;
    }
    const uint32_t lds_base = lds_addr(smem);
    // S operand: lane reads key row 16 mb + l16, piece 4 ks + lq.
    int k_rd[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k_rd[ks] = l16 * ROW_B + (((4 * ks + lq) ^ (l16 & (PPR - 1))) << 4);
    // V^T operand, one transposed read per 4 keys: lanes 4i..4i+3 of each
    // 16-lane group name key row i of the group (4 dims each) and lane n of the
    // group receives dim n of all four rows.  Lane 16G + 4i + q names row
    // 4G + i (+ 16 h + 32 kb) and dims 16 db + 4q .. 16 db + 4q + 3, so it gets
    // keys 4G + 0..3 of dim 16 db + (lane mod 16): the key order of the
    // weights that the score layout leaves in its registers.
    const int vr = lane >> 2, vq = lane & 3;
    int v_rd[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        v_rd[db] = vr * ROW_B + (((2 * db + (vq >> 1)) ^ (vr & (PPR - 1))) << 4) + ((vq & 1) << 3);

    f32x4_t oacc[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) oacc[db][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

    auto tile_of = [&](int it) { return it < nst ? it : wt0 + (it - nst); };
    auto load_k = [&](int tile, int buf) {
        const int soff = tile * TILE_B;
#pragma unroll
        for (int x = 0; x < DMA_N; ++x)
            load_lds16(rk, lds_base + (uint32_t)((x * NTHR + wave * 64) * 16 + buf * TILE_B), dma_off[x], soff);
    };
    auto load_v = [&](int tile, int buf) {
        const int soff = tile * TILE_B;
#pragma unroll
        for (int x = 0; x < DMA_N; ++x)
            load_lds16(rv, lds_base + (uint32_t)((x * NTHR + wave * 64) * 16 + (2 + buf) * TILE_B), dma_off[x],
                       soff);
    };

    // S^T = K Q^T for 64 keys x 32 query rows, in one block (used where nothing
    // runs beside it)
    auto qk = [&](const unsigned char* ktile, f32x4_t (&s)[4][2]) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) s[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(ktile + k_rd[ks] + 16 * mb * ROW_B);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    s[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[nb][ks], s[mb][nb], 0, 0, 0);
            }
        }
    };
    // hide the keys of a tile that cross a row's causal bound (or left its window)
    auto mask = [&](int tile, f32x4_t (&s)[4][2]) {
        const int key0 = tile * KT;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int lim = P + row_t[nb];                   // last visible key of this row
            const int wlo = window > 0 ? lim - window : -1;  // keys at or below it left the window
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = key0 + 16 * mb + 4 * lq + i;
                    // bitwise, not short-circuit: a select per score instead of a branch
                    const bool hide = (key > lim) | ((key <= wlo) & (key >= n_sink));
                    s[mb][nb][i] = hide ? -INFINITY : s[mb][nb][i];
                }
        }
    };
    // raw score maximum of row block nb: v_maximum3 needs no canonicalising of its
    // inputs (fmaxf does); lanes l, l ^ 16, l ^ 32 and l ^ 48 hold the same query
    // row, so two in-register lane swaps finish it
    auto rowmax_part = [&](const f32x4_t (&s)[4][2], int nb) {
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
            mx = __builtin_elementwise_maximum(
                mx, __builtin_elementwise_maximum(__builtin_elementwise_maximum(s[mb][nb][0], s[mb][nb][1]),
                                                  __builtin_elementwise_maximum(s[mb][nb][2], s[mb][nb][3])));
        return mx;
    };
    auto rowmax_finish = [&](float mx) {
        const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = __builtin_elementwise_maximum(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        return __builtin_elementwise_maximum(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
    };
    // [hi/lo][kb][nb]: the weights as PV B operands, split p = hi + lo with both parts
    // in bf16 so the product with V keeps ~16 significant bits of p
    u32x4_t pk[2][2][2];
    // weights of scores 2 ip, 2 ip + 1 of block (mb, nb) against the exponent
    // reference mref; their sum goes to ps
    auto wpair = [&](const f32x4_t (&s)[4][2], int mb, int nb, int ip, const float (&mref)[2], float (&ps)[2]) {
        const float p0 = fast_exp2(__builtin_fmaf(s[mb][nb][2 * ip], scale_log2, -mref[nb]));
        const float p1 = fast_exp2(__builtin_fmaf(s[mb][nb][2 * ip + 1], scale_log2, -mref[nb]));
        ps[nb] += p0 + p1;
        const uint32_t h = cvt_pk_bf16(p0, p1);
        const uint32_t l = cvt_pk_bf16(p0 - bf_lo(h), p1 - bf_hi(h));
        pk[0][mb >> 1][nb][(mb & 1) * 2 + ip] = h;
        pk[1][mb >> 1][nb][(mb & 1) * 2 + ip] = l;
    };
    // the 8 score pairs of keys 32 kb .. 32 kb + 31, in the order they are formed
    auto wpair_k = [&](const f32x4_t (&s)[4][2], int kb, int c, const float (&mref)[2], float (&ps)[2]) {
        wpair(s, 2 * kb + (c >> 2), (c >> 1) & 1, c & 1, mref, ps);
    };
    // V^T operand of keys 32 kb .. 32 kb + 31 and dims 16 db .. 16 db + 15
    auto vread = [&](const unsigned char* vtile, int kb, int db) {
        const i16x4_t u0 = read_tr16(vtile + v_rd[db] + 32 * kb * ROW_B);
        const i16x4_t u1 = read_tr16(vtile + v_rd[db] + (32 * kb + 16) * ROW_B);
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(u0, u1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto pv_mfma = [&](const bf16x8_t& a, int kb, int db, int hl) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
            oacc[db][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, __builtin_bit_cast(bf16x8_t, pk[hl][kb][nb]), oacc[db][nb], 0, 0, 0);
    };
    // The order below is fixed by hand (sched_barrier): left to itself the
    // compiler issues all MFMAs of a phase back to back and the exponentials
    // after them, so the matrix pipe and the VALU take turns instead of
    // working together.  The LDS operands of each MFMA are read one slot
    // ahead.
#define PF_FENCE() __builtin_amdgcn_sched_barrier(0)

    // K and V tiles sit in separate double buffers with V one tile behind K.
    // Iteration it holds the scores of tile it in registers.  Phase A runs the
    // score MFMAs of tile it+1 with the weights of keys 0..31 of tile it formed
    // between them; phase B runs P V over keys 0..31 with the weights of keys
    // 32..63 formed between, then P V over keys 32..63 with the row maxima of
    // tile it+1 (its raw scores; a tile that needs a mask recomputes them).
    float mx_cur[2];
    auto iter = [&](int it, f32x4_t (&cur)[4][2], f32x4_t (&nxt)[4][2]) {
        // this wave's loads are done; after the barrier every wave's are (V(it),
        // K(it+1)), and every wave has finished iteration it-1, so the buffers of
        // K(it) and V(it-1) are free for the next loads
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (it + 2 < n_iter) load_k(tile_of(it + 2), it & 1);
        if (it + 1 < n_iter) load_v(tile_of(it + 1), (it + 1) & 1);
        // Issue priority grows with the tiles left: of two workgroups sharing
        // a CU the one with more work left is served first, so both tend to
        // finish together instead of the second running alone (one wave per
        // SIMD) at the end.
        {
            const int rem = n_iter - it;
            if (rem > 12) __builtin_amdgcn_s_setprio(3);
            else if (rem > 8) __builtin_amdgcn_s_setprio(2);
            else if (rem > 4) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        }
        const int tile = tile_of(it);
        if (tile >= first_masked_tile || window > 0) {
            mask(tile, cur);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) mx_cur[nb] = rowmax_finish(rowmax_part(cur, nb));
        }
        // The exponent reference m_ref (scaled, base 2) only moves when the row
        // maximum exceeds it by more than 8: weights then stay below 2^8, and
        // the accumulators are rescaled rarely instead of on every tile.
        float mref[2], alpha[2], ps[2] = {0.f, 0.f};
        bool move[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const float mxs = mx_cur[nb] * scale_log2;
            move[nb] = mxs > m_run[nb] + 8.f;
            const float mn = move[nb] ? mxs : m_run[nb];
            alpha[nb] = move[nb] ? fast_exp2(m_run[nb] - mn) : 1.f;
            m_run[nb] = mn;
            // a row that has seen no key yet (possible under a window) keeps weight 0
            mref[nb] = mn == -INFINITY ? 0.f : mn;
        }
        if (__builtin_amdgcn_ballot_w64(move[0] | move[1]) != 0) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) oacc[db][nb] *= alpha[nb];
        }

        // ---- phase A: 4 KS slots (k-step ks, key block mb), two MFMAs each,
        // with the 8 weight pairs of keys 0..31 spread over them
        {
            const unsigned char* ktile = smem + ((it + 1) & 1) * TILE_B;
            bf16x8_t ka[2];
            auto kread = [&](int slot) {
                return *reinterpret_cast<const bf16x8_t*>(ktile + k_rd[slot >> 2] + 16 * (slot & 3) * ROW_B);
            };
            ka[0] = kread(0);
            PF_FENCE();
            constexpr int NSLOT = 4 * KS;
#pragma unroll
            for (int slot = 0; slot < NSLOT; ++slot) {
                if (slot + 1 < NSLOT) ka[(slot + 1) & 1] = kread(slot + 1);
                const int ks = slot >> 2, mb = slot & 3;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    nxt[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        ka[slot & 1], qop[nb][ks], ks == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : nxt[mb][nb], 0, 0, 0);
#pragma unroll
                for (int c = slot * 8 / NSLOT; c < (slot + 1) * 8 / NSLOT; ++c) wpair_k(cur, 0, c, mref, ps);
                PF_FENCE();
            }
        }
        // ---- phase B: P V over keys 0..31 (a weight pair of keys 32..63 per
        // 16-dim block), then over keys 32..63 (the row maxima of tile it+1)
        const unsigned char* vtile = smem + (2 + (it & 1)) * TILE_B;
        {
            bf16x8_t va[2];
            va[0] = vread(vtile, 0, 0);
            PF_FENCE();
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                if (db + 1 < DB) va[(db + 1) & 1] = vread(vtile, 0, db + 1);
                pv_mfma(va[db & 1], 0, db, 0);
                pv_mfma(va[db & 1], 0, db, 1);
#pragma unroll
                for (int c = db * 8 / DB; c < (db + 1) * 8 / DB; ++c) wpair_k(cur, 1, c, mref, ps);
                PF_FENCE();
            }
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) l_run[nb] = l_run[nb] * alpha[nb] + ps[nb];
        {
            bf16x8_t va[2];
            float mxp[2];
            va[0] = vread(vtile, 1, 0);
            PF_FENCE();
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                if (db + 1 < DB) va[(db + 1) & 1] = vread(vtile, 1, db + 1);
                pv_mfma(va[db & 1], 1, db, 0);
                pv_mfma(va[db & 1], 1, db, 1);
                constexpr int Q4 = DB / 4;  // the four steps of the row maxima, one per quarter
                if (db == Q4 - 1) mxp[0] = rowmax_part(nxt, 0);
                if (db == 2 * Q4 - 1) mxp[1] = rowmax_part(nxt, 1);
                if (db == 3 * Q4 - 1) mx_cur[0] = rowmax_finish(mxp[0]);
                if (db == 4 * Q4 - 1) mx_cur[1] = rowmax_finish(mxp[1]);
                PF_FENCE();
            }
        }
    };
#undef PF_FENCE

    f32x4_t sA[4][2], sB[4][2];
    load_k(tile_of(0), 0);
    load_v(tile_of(0), 0);
    if (n_iter > 1) load_k(tile_of(1), 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    qk(smem, sA);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) mx_cur[nb] = rowmax_finish(rowmax_part(sA, nb));
    for (int it = 0; it < n_iter; it += 2) {
        iter(it, sA, sB);
        if (it + 1 < n_iter) iter(it + 1, sB, sA);
    }

    // ---- normalise and store: lane holds dims 16db + 4*lq + 0..3 of its row
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        float l = l_run[nb];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        if (!row_ok[nb]) continue;
        // a learned sink logit joins the normaliser (same exponent reference as the weights)
        if (sink_logits) l += fast_exp2(sink_logits[row_h[nb]] * LOG2E_P - m_run[nb]);
        const float inv = 1.f / l;
        uint16_t* dst = out + ((size_t)b * n_q * T + (size_t)row_h[nb] * T + row_t[nb]) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const f32x4_t o = oacc[db][nb];
            *reinterpret_cast<uint2*>(dst + 16 * db + 4 * lq) =
                make_uint2(cvt_pk_bf16(o[0] * inv, o[1] * inv), cvt_pk_bf16(o[2] * inv, o[3] * inv));
        }
    }
}

}  // namespace

hipError_t launch_prefill(const uint16_t* q_rot, const uint16_t* k_cache, const uint16_t* v_cache,
                          const int32_t* past_len, int max_past_len, uint16_t* out, int B, int n_q, int n_kv, int T,
                          int d, int S, float scale, int window, int n_sink, const float* sink_logits,
                          hipStream_t st) {
    const int g = n_q / n_kv;
    const int hpw = g < ROWS ? g : ROWS;  // heads per workgroup
    const int tq = ROWS / hpw;            // positions per workgroup
    const int n_tq = (T + tq - 1) / tq;
    const int n_hc = (g + hpw - 1) / hpw;
    const float scale_log2 = scale * LOG2E_P;
    for (int b0 = 0; b0 < B; b0 += 65535) {
        const int nb = (B - b0) < 65535 ? (B - b0) : 65535;
        dim3 grid((unsigned)(n_tq * n_hc), n_kv, nb);
        const size_t qo = (size_t)b0 * n_q * T * d, co = (size_t)b0 * n_kv * S * d;
        prof_begin(K_PREFILL, st);
        if (d == 128)
            hipLaunchKernelGGL(prefill_kernel<128>, grid, dim3(NTHR), 0, st, q_rot + qo, k_cache + co,
                               v_cache + co, past_len + b0, max_past_len, out + qo, n_q, n_kv, T, S, hpw, tq, n_tq,
                               scale_log2, window, n_sink, sink_logits);
        else
            hipLaunchKernelGGL(prefill_kernel<64>, grid, dim3(NTHR), 0, st, q_rot + qo, k_cache + co, v_cache + co,
                               past_len + b0, max_past_len, out + qo, n_q, n_kv, T, S, hpw, tq, n_tq, scale_log2,
                               window, n_sink, sink_logits);
        prof_end(K_PREFILL, st);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gqa
