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
// stages serves all heads that share it.  Per 64-key tile:
//   S^T = K Q^T   (v_mfma_f32_16x16x32_bf16: A = K rows from LDS, B = the
//                  wave's 32 query rows held in registers)
//   online softmax per query row (each lane holds one query row per 16-row
//                  block, so only two cross-lane steps are needed)
//   O^T += V^T P^T (A = V^T from a transposed LDS copy of the V tile,
//                  B = the softmax weights already in the right lanes, split
//                  into a bf16 high part and a bf16 remainder so that the
//                  weights enter the product with ~16 significant bits)
// Tiles entirely above every row's causal bound are never loaded; tiles that
// straddle a bound are masked element-wise.  The next tile's global loads are
// in flight while the current tile is computed.
#include "common.hpp"
#include "kernels.hpp"

namespace gqa {

namespace {

constexpr int KT = 64;        // keys per tile
constexpr int NTHR = 256;     // 4 waves
constexpr int ROWS = 128;     // query rows per workgroup (32 per wave)
constexpr float LOG2E_P = 1.4426950408889634f;

// K tile: [64 keys][D] bf16 in 16-byte pieces; piece c of key r sits at c ^ (r mod PPR)
template <int PPR>
__device__ __forceinline__ int kpos(int key, int c) {
    return key * PPR + (c ^ (key & (PPR - 1)));
}
// V^T tile: [D dims][64 keys] bf16 in 8-byte units of 4 keys; unit u of dim row d sits at u ^ (d mod 16)
__device__ __forceinline__ int vt_byte(int dim, int unit) { return dim * 128 + ((unit ^ (dim & 15)) << 3); }

template <int D>
__global__ __launch_bounds__(NTHR, 2) void prefill_kernel(const uint16_t* __restrict__ q_rot,
                                                          const uint16_t* __restrict__ k_cache,
                                                          const uint16_t* __restrict__ v_cache,
                                                          const int32_t* __restrict__ past_len, int pmax,
                                                          uint16_t* __restrict__ out, int n_q, int n_kv, int T,
                                                          int S, int hpw, int tq, int n_tq, float scale_log2,
                                                          int window, int n_sink, const float* sink_logits) {
    constexpr int PPR = D / 8;     // 16-byte pieces per key row
    constexpr int KS = D / 32;     // MFMA k-steps over d
    constexpr int DB = D / 16;     // 16-dim blocks of the output
    constexpr int K_LOADS = KT * PPR / NTHR;        // 16-byte K loads per thread
    constexpr int V_ITEMS = (KT / 2) * PPR / NTHR;  // (key pair, piece) items per thread
    __shared__ uint4 s_k[KT * PPR];
    __shared__ __align__(16) unsigned char s_vt[D * 128];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const int g = n_q / n_kv;
    const int tq_idx = n_tq - 1 - (int)(blockIdx.x % n_tq);  // longest rows first
    const int hc = blockIdx.x / n_tq;
    const int j = blockIdx.y, b = blockIdx.z;
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
    u32x4_t kst[K_LOADS];
    u32x4_t vst[V_ITEMS][2];
    auto load = [&](int tile) {
        const int soff = tile * KT * D * 2;
#pragma unroll
        for (int i = 0; i < K_LOADS; ++i) {
            const int pi = tid + NTHR * i;
            const int key = pi / PPR, c = pi % PPR;
            kst[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, (key * D + 8 * c) * 2, soff, 0);
        }
#pragma unroll
        for (int i = 0; i < V_ITEMS; ++i) {
            const int it = tid + NTHR * i;
            const int kp = it % (KT / 2), c = it / (KT / 2);
            vst[i][0] = __builtin_amdgcn_raw_buffer_load_b128(rv, (2 * kp * D + 8 * c) * 2, soff, 0);
            vst[i][1] = __builtin_amdgcn_raw_buffer_load_b128(rv, ((2 * kp + 1) * D + 8 * c) * 2, soff, 0);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < K_LOADS; ++i) {
            const int pi = tid + NTHR * i;
            s_k[kpos<PPR>(pi / PPR, pi % PPR)] = __builtin_bit_cast(uint4, kst[i]);
        }
#pragma unroll
        for (int i = 0; i < V_ITEMS; ++i) {
            const int it = tid + NTHR * i;
            const int kp = it % (KT / 2), c = it / (KT / 2);
            const uint32_t a[4] = {vst[i][0].x, vst[i][0].y, vst[i][0].z, vst[i][0].w};
            const uint32_t bq[4] = {vst[i][1].x, vst[i][1].y, vst[i][1].z, vst[i][1].w};
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                // dims 8c+2x and 8c+2x+1, keys 2kp and 2kp+1
                const uint32_t lo = (a[x] & 0xffffu) | (bq[x] << 16);
                const uint32_t hi = (a[x] >> 16) | (bq[x] & 0xffff0000u);
                const int d0 = 8 * c + 2 * x;
                const int unit = kp >> 1, sub = (kp & 1) * 4;
                *reinterpret_cast<uint32_t*>(s_vt + vt_byte(d0, unit) + sub) = lo;
                *reinterpret_cast<uint32_t*>(s_vt + vt_byte(d0 + 1, unit) + sub) = hi;
            }
        }
    };

    f32x4_t oacc[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) oacc[db][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

    auto tile_of = [&](int it) { return it < nst ? it : wt0 + (it - nst); };
    load(tile_of(0));
    for (int it = 0; it < n_iter; ++it) {
        const int tile = tile_of(it);
        __syncthreads();
        store();
        __syncthreads();
        if (it + 1 < n_iter) load(tile_of(it + 1));

        // ---- S^T = K Q^T for 64 keys x 32 query rows
        f32x4_t sacc[4][2];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) sacc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, s_k[kpos<PPR>(16 * mb + l16, 4 * ks + lq)]);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    sacc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[nb][ks], sacc[mb][nb], 0, 0, 0);
            }
        }

        // ---- mask (only tiles that cross a row's causal bound), online softmax per query row
        const int key0 = tile * KT;
        if (tile >= first_masked_tile || window > 0) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int lim = P + row_t[nb];  // last visible key of this row
                const int wlo = window > 0 ? lim - window : -1;  // keys at or below it left the window
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = key0 + 16 * mb + 4 * lq + i;
                        // bitwise, not short-circuit: a select per score instead of a branch
                        const bool hide = (key > lim) | ((key <= wlo) & (key >= n_sink));
                        sacc[mb][nb][i] = hide ? -INFINITY : sacc[mb][nb][i];
                    }
            }
        }
        // [hi/lo][kb][nb]: the weights as PV B operands, split p = hi + lo with both parts
        // in bf16 so the product with V keeps ~16 significant bits of p
        u32x4_t pk[2][2][2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            float mx = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) mx = fmaxf(mx, fmaxf(fmaxf(sacc[mb][nb][0], sacc[mb][nb][1]),
                                                              fmaxf(sacc[mb][nb][2], sacc[mb][nb][3])));
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            // The exponent reference m_ref (scaled, base 2) only moves when the row
            // maximum exceeds it by more than 8: weights then stay below 2^8, and
            // the accumulators are rescaled rarely instead of on every tile.
            const float mxs = mx * scale_log2;
            const bool move = mxs > m_run[nb] + 8.f;
            const float mn = move ? mxs : m_run[nb];
            const float alpha = move ? fast_exp2(m_run[nb] - mn) : 1.f;
            m_run[nb] = mn;
            // a row that has seen no key yet (possible under a window) keeps weight 0
            const float mref = mn == -INFINITY ? 0.f : mn;
            float ps = 0.f;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = fast_exp2(__builtin_fmaf(sacc[mb][nb][i], scale_log2, -mref));
                    ps += p[i];
                }
                const uint32_t h01 = cvt_pk_bf16(p[0], p[1]), h23 = cvt_pk_bf16(p[2], p[3]);
                const uint32_t l01 = cvt_pk_bf16(p[0] - bf_lo(h01), p[1] - bf_hi(h01));
                const uint32_t l23 = cvt_pk_bf16(p[2] - bf_lo(h23), p[3] - bf_hi(h23));
                const int w0 = (mb & 1) * 2;
                pk[0][mb >> 1][nb][w0] = h01;
                pk[0][mb >> 1][nb][w0 + 1] = h23;
                pk[1][mb >> 1][nb][w0] = l01;
                pk[1][mb >> 1][nb][w0 + 1] = l23;
            }
            l_run[nb] = l_run[nb] * alpha + ps;
            if (__builtin_amdgcn_ballot_w64(move) != 0) {
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db][nb] *= alpha;
            }
        }

        // ---- O^T += V^T P^T
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            bf16x8_t bop[2][2];
#pragma unroll
            for (int hl = 0; hl < 2; ++hl)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) bop[hl][nb] = __builtin_bit_cast(bf16x8_t, pk[hl][kb][nb]);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int dim = 16 * db + l16;
                const uint2 u0 = *reinterpret_cast<const uint2*>(s_vt + vt_byte(dim, 8 * kb + lq));
                const uint2 u1 = *reinterpret_cast<const uint2*>(s_vt + vt_byte(dim, 8 * kb + 4 + lq));
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(u0.x, u0.y, u1.x, u1.y));
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    oacc[db][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bop[0][nb], oacc[db][nb], 0, 0, 0);
                    oacc[db][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bop[1][nb], oacc[db][nb], 0, 0, 0);
                }
            }
        }
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
