/*
 * gqa.h -- C ABI of libgqa: one grouped-query attention step with RoPE over a
 * preallocated bf16 KV cache, on one AMD Instinct MI355X (gfx950).
 *
 * Pages this interface follows (title, then section / formula / excerpt):
 *   [KV]   "Llama 3.1 8B KV cache" (alijanati.com)
 *   [ATL]  "Llama 3 8B - KV cache" (OpenModelAtlas, decode at position 1000)
 *   [REP]  "Llama 3.1 8B - Repeat heads" (OpenModelAtlas)
 *   [EP18] "Grouped-query attention: a smaller KV cache" (mvgpt, episode 18)
 *   [P7]   "Part 7: The Modern Decoder Block" (openlearn)
 *
 * Conventions shared by every entry point
 *   - bf16 tensors are passed as device pointers to 16-bit patterns (no C bf16
 *     type is needed); int32 tensors as device pointers to int32_t.
 *   - Every tensor is dense, row-major, and its device pointer is 16-byte
 *     aligned.  Shapes:
 *        q, q_rot, out  [B, n_q,  T, d]
 *        k_new, v_new   [B, n_kv, T, d]
 *        k_cache,v_cache[B, n_kv, S, d]   (keys are stored already rotated)
 *        past_len       [B]  int32, rows already cached for each sequence
 *   - n_q = g * n_kv; query head h reads KV head floor(h / g) ([REP] formula;
 *     [EP18] "Our six heads, three ways").  No copy of a KV head is made.
 *   - d is 64 or 128 (the kernels are built for these two head sizes), and
 *     S * d * 2 < 2^31 (one KV head's cache slab is addressed with 32-bit
 *     byte offsets; INVALID_ARG otherwise).
 *   - past_len lives in device memory so that calls can be captured and
 *     replayed; max_past_len is the host-side upper bound the caller vouches
 *     for (past_len[b] <= max_past_len for every b).  Every launch is sized
 *     from it, and kernels never touch a cache row >= S.  A past_len[b] outside
 *     [0, max_past_len] is a caller error: rows it would address are skipped
 *     rather than written out of bounds, and the outputs of that sequence are
 *     unspecified.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued on it; no call synchronises, allocates or frees
 *     memory.  The caller owns every buffer, including workspaces.
 *   - Calls on one stream are ordered: gqa_rope_append must be enqueued before
 *     the attention call that reads the rows it writes.
 *   - Return value: GQA_OK or a negative status (below).  All argument checks
 *     run on the host before any HIP call; a failed check launches nothing.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define GQA_OK 0
#define GQA_ERR_INVALID_ARG (-1) /* null/misaligned pointer, size <= 0, odd d, bad RoPE params */
#define GQA_ERR_GROUP (-2)       /* n_q is not a multiple of n_kv ([EP18] "Grouped-query attention in code") */
#define GQA_ERR_HEAD_DIM (-3)    /* d is not 64 or 128 */
#define GQA_ERR_RANGE (-4)       /* max_past_len < 0, or max_past_len + T > S */
#define GQA_ERR_WORKSPACE (-5)   /* workspace smaller than gqa_decode_workspace_bytes() */
#define GQA_ERR_HIP (-6)         /* no device, launch or runtime failure; see gqa_status_string */
#define GQA_ERR_SCRATCH (-7)     /* gqa_decode_attn_noalloc: the shape needs more than GQA_DECODE_NOALLOC_MAX_BYTES */

/* ---- RoPE parameters ------------------------------------------------- */
#define GQA_ROPE_INTERLEAVED 0 /* pair i is dims (2i, 2i+1) */
#define GQA_ROPE_HALF 1        /* pair i is dims (i, i + d/2) */

/* Context-extension rules ([P7] module L7.4 names PI, NTK, YaRN and Llama-3
 * scaling; [KV] "Training details that matter" names the Llama-3 fields).  The
 * pages print no formulas; each rule follows its published definition:
 *   LLAMA3  wavelength lambda = 2 pi / freq: lambda < original_max_pos /
 *           high_freq_factor keeps freq, lambda > original_max_pos /
 *           low_freq_factor gives freq / factor, between the two the mix
 *           (1 - s) freq / factor + s freq, s = (original_max_pos / lambda -
 *           low_freq_factor) / (high_freq_factor - low_freq_factor).
 *   LINEAR  position interpolation: every frequency divided by factor.
 *   NTK     NTK-aware base change: theta becomes theta * factor^(r / (r - 2)).
 *   YARN    YaRN's ramp in rho = original_max_pos / lambda (the turns a pair
 *           makes over the original context): the LLAMA3 mix with
 *           low_freq_factor = alpha (beta_slow, rho below it: freq / factor)
 *           and high_freq_factor = beta (beta_fast, rho above it: freq), plus
 *           the attention factor 0.1 ln(factor) + 1 on the rotated dims. */
#define GQA_ROPE_SCALING_NONE 0
#define GQA_ROPE_SCALING_LLAMA3 1
#define GQA_ROPE_SCALING_LINEAR 2
#define GQA_ROPE_SCALING_NTK 3
#define GQA_ROPE_SCALING_YARN 4

typedef struct gqa_rope_params {
    double theta;            /* base: freq_i = theta^(-2i/r)  ([KV] "RoPE has to know where it is") */
    int layout;              /* GQA_ROPE_INTERLEAVED or GQA_ROPE_HALF ([P7] module L7.3) */
    int scaling;             /* GQA_ROPE_SCALING_*: NONE ignores the four fields below */
    double factor;           /* context-extension factor s: >= 1 for LINEAR, NTK, YARN; > 0 for LLAMA3 */
    double low_freq_factor;  /* LLAMA3 low cutoff / YARN alpha (> 0) */
    double high_freq_factor; /* LLAMA3 high cutoff / YARN beta (> low_freq_factor) */
    double original_max_pos; /* context length the base model was trained on (> 0; LLAMA3, YARN) */
    int rotary_dim;          /* r, rotated dims: 0 = all d; else a multiple of 16 in [16, d] ([P7] L7.3
                                "partial rotary"): dims r .. d-1 are copied, the half layout pairs
                                dim i with i + r/2, and the exponent uses r */
    double attn_factor;      /* multiplier of the rotated dims: 0 = default (YARN 0.1 ln(factor) + 1,
                                otherwise 1), else > 0 and used as given */
} gqa_rope_params;

/*
 * gqa_rope_append -- rotate q and the new k at their positions and write the
 * rotated k and the v rows into the cache.
 *
 * [KV] "RoPE has to know where it is": new token t of sequence b sits at
 * position p = past_len[b] + t.  Pair i of every head of q and k_new is turned
 * by the angle p * freq_i: (a, b) -> (a cos - b sin, a sin + b cos).
 * [ATL] cache formula: cache rows p = past_len[b] .. past_len[b]+T-1 receive
 * the rotated keys and the values; no other cache row is touched.
 *
 * With rotary_dim r < d only the first r dims of each head turn (pair i at
 * freq_i = theta^(-2i/r)); the other dims are copied.
 *
 * Precision: frequencies, angles, sin/cos and the rotation are computed in
 * fp64 on the device and each result is rounded once to bf16 (nearest, ties
 * to even).  v rows and unrotated dims are copied bit for bit.
 *
 *   q        in   [B, n_q, T, d] bf16
 *   q_rot    out  [B, n_q, T, d] bf16, may equal q (rotated in place)
 *   k_new    in   [B, n_kv, T, d] bf16 (unrotated)
 *   v_new    in   [B, n_kv, T, d] bf16
 *   k_cache  in/out [B, n_kv, S, d] bf16
 *   v_cache  in/out [B, n_kv, S, d] bf16
 *   past_len in   [B] int32 (device)
 *   rope     in   host pointer; theta > 0, layout and scaling valid, the
 *                 scaling fields as stated above, rotary_dim 0 or a multiple
 *                 of 16 in [16, d], attn_factor >= 0 and finite
 * Errors: INVALID_ARG, GROUP, HEAD_DIM, RANGE (max_past_len + T > S), HIP.
 */
int gqa_rope_append(const void* q, void* q_rot, const void* k_new, const void* v_new, void* k_cache,
                    void* v_cache, const int32_t* past_len, int max_past_len, int B, int n_q, int n_kv, int T,
                    int d, int S, const gqa_rope_params* rope, void* stream);

/*
 * gqa_decode_workspace_bytes -- bytes of device workspace gqa_decode_attn
 * needs for this shape (0 when the shape is invalid).  The size depends only
 * on the arguments and on library constants, not on past_len.
 *
 * The first 256 bytes of a workspace are a scheduling header (the counter
 * that hands out work chunks).  They must be zero before the first
 * gqa_decode_attn call that uses the workspace (allocate it zero-filled, or
 * clear it once); every call leaves them zero again when it completes.  Calls
 * that use one workspace must not overlap in time (order them on one stream).
 */
size_t gqa_decode_workspace_bytes(int B, int n_q, int n_kv, int d, int S);

/*
 * gqa_decode_attn -- one new query token per sequence attends to cache rows
 * 0 .. past_len[b] (the row written by the matching gqa_rope_append included).
 *
 * [ATL] prose: the decode call at position p reads rows 0..p; with one new
 * token there is nothing to mask inside that range ([ATL] Transformer.forward
 * excerpt builds no mask when seqlen is 1).  Scores are q.k * scale, softmax
 * over the rows, then the weighted sum of the value rows ([KV] "The cache
 * itself is concatenation").  Each KV head's rows are read from memory once
 * for all g query heads of its group.
 *
 * The work is split over the rows ("split-K"): most of it in equal
 * contiguous shares per workgroup, the rest in small fixed chunks taken from
 * a counter in the workspace header as workgroups become free.  Each part
 * writes (max, sum, partial output) records into the workspace, and a second
 * kernel merges them in a fixed order.  Which rows form a part does not
 * depend on timing, so results are bitwise reproducible for a given launch
 * shape.
 *
 *   q_rot     in  [B, n_q, 1, d] bf16 (already rotated)
 *   k_cache   in  [B, n_kv, S, d] bf16;  v_cache likewise
 *   past_len  in  [B] int32 (device); rows 0..past_len[b] are attended
 *   out       out [B, n_q, 1, d] bf16
 *   workspace device scratch of at least gqa_decode_workspace_bytes(...),
 *             header zeroed before its first use (see above)
 *   scale     score scale; <= 0 selects 1/sqrt(d)
 * Errors: INVALID_ARG, GROUP, HEAD_DIM, RANGE (max_past_len + 1 > S),
 *         WORKSPACE, HIP.
 */
int gqa_decode_attn(const void* q_rot, const void* k_cache, const void* v_cache, const int32_t* past_len,
                    int max_past_len, void* out, void* workspace, size_t workspace_bytes, int B, int n_q, int n_kv,
                    int d, int S, float scale, void* stream);

/*
 * gqa_prefill_attn -- T new query tokens per sequence attend to the cache
 * under the rectangular causal mask: row t (position past_len[b] + t) sees
 * cache rows 0 .. past_len[b] + t ([ATL] Transformer.forward excerpt and its
 * comment on the mask with a cache).  QK^T and PV run on bf16 MFMA with fp32
 * accumulation; the softmax weights enter the PV product as a bf16 high part
 * plus a bf16 remainder (about 16 significant bits).
 *
 *   q_rot   in  [B, n_q, T, d] bf16 (already rotated)
 *   k_cache in  [B, n_kv, S, d] bf16 (rows up to past_len[b]+T-1 written)
 *   out     out [B, n_q, T, d] bf16
 *   scale   <= 0 selects 1/sqrt(d)
 * Errors: INVALID_ARG, GROUP, HEAD_DIM, RANGE (max_past_len + T > S), HIP.
 */
int gqa_prefill_attn(const void* q_rot, const void* k_cache, const void* v_cache, const int32_t* past_len,
                     int max_past_len, void* out, int B, int n_q, int n_kv, int T, int d, int S, float scale,
                     void* stream);

/*
 * Attention options ([P7] "Part 7: The Modern Decoder Block", modules L7.5
 * and L7.7, name the sliding window, StreamingLLM sinks and learned sinks; the
 * pages give no formula, the rules below are the plainest reading):
 *   window       > 0: the query at position p sees cache rows p - window + 1
 *                .. p only (its own row and the window - 1 before it), plus
 *                the sinks; 0: no window (every row 0 .. p).
 *   n_sink       under a window, rows 0 .. n_sink - 1 stay visible to every
 *                query.  Ignored without a window.
 *   sink_logits  NULL, or a device fp32 array [n_q]: one learned logit per
 *                query head, in the units of the scaled scores q.k * scale;
 *                it joins the softmax normaliser as one more term and carries
 *                no value (4-byte aligned).
 * With the _ex entry points the decode kernel visits only the tiles holding
 * visible rows, so a window makes the KV read O(window); the prefill kernel
 * skips tiles that lie wholly between the sinks and the earliest window.
 * Rows are read in 64-row tiles.  A row of a read tile that a query does not
 * see enters that query's sums with weight zero, and zero times Inf or NaN
 * is NaN, so every row of a read tile must be finite.  Under a window, the
 * tiles that hold no row visible to any query of the call (those wholly
 * between the sink tiles and the window of the query at past_len) are never
 * read and may hold anything.
 */
typedef struct gqa_attn_opts {
    int window;
    int n_sink;
    const float* sink_logits;
} gqa_attn_opts;

/* gqa_decode_attn / gqa_prefill_attn with options (NULL = none, the plain
 * entry points); same arguments, layouts and errors otherwise, plus
 * INVALID_ARG for a negative window or n_sink or a misaligned sink_logits. */
int gqa_decode_attn_ex(const void* q_rot, const void* k_cache, const void* v_cache, const int32_t* past_len,
                       int max_past_len, void* out, void* workspace, size_t workspace_bytes, int B, int n_q, int n_kv,
                       int d, int S, float scale, const gqa_attn_opts* opts, void* stream);
int gqa_prefill_attn_ex(const void* q_rot, const void* k_cache, const void* v_cache, const int32_t* past_len,
                        int max_past_len, void* out, int B, int n_q, int n_kv, int T, int d, int S, float scale,
                        const gqa_attn_opts* opts, void* stream);

/*
 * gqa_decode_attn_noalloc -- gqa_decode_attn_ex without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * split-K records live in a fixed buffer inside the library, one copy per
 * GPU of GQA_DECODE_NOALLOC_MAX_BYTES (64 MiB), reserved when the library is
 * loaded and held until the process ends.  Same kernels, launch shape and
 * results as gqa_decode_attn_ex (bitwise), plus one small kernel that clears
 * the buffer's scheduling header first.  The call allocates nothing (no
 * hipMalloc, no allocating library routine).
 *
 * Every call on one GPU shares that GPU's buffer: calls that may overlap in
 * time on one GPU (different streams without ordering, several host threads)
 * race and give wrong results.  Order them on one stream.
 *
 * Arguments, layouts and ownership as gqa_decode_attn_ex.  Errors:
 * INVALID_ARG, GROUP, HEAD_DIM, RANGE, SCRATCH (the records of the decode
 * path the shape takes need more than GQA_DECODE_NOALLOC_MAX_BYTES: never
 * for sizes where gqa_decode_workspace_bytes() is within it, e.g. any batch at
 * 32/8 heads or B <= 300 at 64/8, d 128; checked on the host, nothing
 * launched), HIP.
 */
#define GQA_DECODE_NOALLOC_MAX_BYTES (64u << 20)
int gqa_decode_attn_noalloc(const void* q_rot, const void* k_cache, const void* v_cache, const int32_t* past_len,
                            int max_past_len, void* out, int B, int n_q, int n_kv, int d, int S, float scale,
                            const gqa_attn_opts* opts, void* stream);

/*
 * gqa_decode_step -- one decode step: gqa_rope_append (T = 1) followed by
 * gqa_decode_attn, same results, in a single launch for small batches.
 *
 * [KV] "RoPE has to know where it is" and "The cache itself is
 * concatenation"; [ATL] "Llama 3 8B - KV cache", cache formula and the
 * Transformer.forward excerpt (write row past_len, then attend over rows
 * 0 .. past_len); [REP] head map h -> floor(h / g).  The new token's q and k
 * are rotated at position past_len[b] (fp64, one rounding to bf16), k_rot
 * and v_new are written to cache row past_len[b], and the new query attends
 * to rows 0 .. past_len[b] (under opts: the window, sinks and learned sink
 * logits of gqa_attn_opts).  The new row enters the attention from the
 * kernel's registers, so the result never depends on when the append lands.
 * The splits of each (sequence, KV head) are merged by the last one to
 * finish, in split order: bitwise reproducible for a given shape.  Groups of
 * g >= 16 heads (the threshold of gqa_set_decode_wide_min_group) run instead
 * as gqa_rope_append followed by the wide-group decode kernel, three launches
 * whose matrix-core products beat one launch's vector arithmetic there; the
 * results and the cache writes are the same.  Likewise larger batches (from
 * 512 tiles of 64 rows, B * n_kv * ceil((max_past_len + 1) / 64), or fewer
 * under a window; see gqa_set_decode_step_split_min_tiles) run as
 * gqa_rope_append followed by the split-K decode, the faster path there.
 *
 *   q, k_new, v_new in [B, n_q | n_kv, 1, d] bf16 (q and k unrotated)
 *   k_cache, v_cache in/out [B, n_kv, S, d] bf16; row past_len[b] is written
 *   out      out [B, n_q, 1, d] bf16
 *   q_rot    out [B, n_q, 1, d] bf16, or NULL (not written)
 *   rope     host pointer, as for gqa_rope_append
 *   scale    <= 0 selects 1/sqrt(d)
 *   workspace  device memory of at least gqa_decode_step_workspace_bytes(),
 *            zero-filled before the first call: it starts with one counter per
 *            (sequence, KV head) and the split-K scheduling header, which every
 *            call leaves zero; everything else a call writes sits at the end of
 *            the workspace_bytes given.  So a workspace sized for B sequences
 *            serves calls of any batch size up to B, through any route, in any
 *            order.  Calls that share a workspace must be stream-ordered, and it
 *            must not be shared with gqa_decode_attn.
 * n_q / n_kv must be at most GQA_DECODE_STEP_MAX_GROUP; B and n_kv at most
 * 65535.  Errors: INVALID_ARG, GROUP, HEAD_DIM, RANGE (max_past_len + 1 > S),
 * WORKSPACE, HIP.
 */
#define GQA_DECODE_STEP_MAX_GROUP 64
size_t gqa_decode_step_workspace_bytes(int B, int n_q, int n_kv, int d, int S);
int gqa_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                    const int32_t* past_len, int max_past_len, void* out, void* q_rot, void* workspace,
                    size_t workspace_bytes, int B, int n_q, int n_kv, int d, int S, const gqa_rope_params* rope,
                    float scale, const gqa_attn_opts* opts, void* stream);

/* Human-readable text for a status code; for GQA_ERR_HIP it includes the
 * last HIP error message recorded by this thread.  Never NULL. */
const char* gqa_status_string(int status);

/*
 * Kernel timing -- measurement support for benchmarks.  While enabled, every
 * kernel launch of this library is bracketed by two HIP events recorded on
 * the launch stream; gqa_profile_read synchronises those events and returns
 * the summed device time and launch count of one kernel kind.
 *   kind: 0 rope_append, 1 decode split-K partials, 2 decode combine,
 *         3 prefill, 4 single-launch decode step, 5 wide-group decode,
 *         6 the streaming-read measurement kernel.
 * Not thread-safe; for single-threaded benchmark drivers.
 */
int gqa_profile_enable(int on);
int gqa_profile_read(int kind, double* total_ms, long long* launches);
int gqa_profile_reset(void);

/*
 * Measurement support: the HBM read ceiling that the decode kernels are
 * compared with.  Reads `bytes` (a multiple of 16) of device memory at `buf`
 * (16-byte aligned) once, with 16-byte non-temporal loads spread over
 * `workgroups` workgroups of 256 threads, and writes one 32-bit word per
 * workgroup to `sink` (device, at least 4 * workgroups bytes) so the loads
 * are not dropped.  It computes nothing of the attention step.  Errors:
 * INVALID_ARG (null or misaligned pointer, bytes not a multiple of 16,
 * workgroups outside 1..65535), HIP.
 */
int gqa_measure_stream_read(const void* buf, size_t bytes, void* sink, int workgroups, void* stream);

/*
 * Measurement support: the sustained rate of the prefill kernel's matrix
 * instruction (v_mfma_f32_16x16x32_bf16, 16 384 flops each), the ceiling a
 * matrix-bound kernel can reach on this GPU at the clock it holds under a
 * full matrix load.  Launches `workgroups` workgroups of 4 waves; every wave
 * issues 8 MFMAs per iteration for `iters` iterations on random operands, so
 * a launch performs workgroups * 4 * iters * 8 * 16384 flops (time it with
 * events on `stream`).  `sink` (device, 8-byte aligned, at least
 * 64 * workgroups bytes) receives, per workgroup, 8 64-bit words: 0..3 the
 * folded results of its waves, 4 the shader-clock cycles and 5 the 100 MHz
 * counter ticks of wave 0 over its loop (their ratio times 100 MHz is the
 * shader clock), 6..7 zero.  It computes nothing of the attention step.
 * Errors: INVALID_ARG (null or misaligned sink, workgroups outside 1..65535,
 * iters outside 1..2^24), HIP.
 */
int gqa_measure_mfma_rate(int workgroups, int iters, void* sink, void* stream);

/*
 * Launch-shape override for tests and tuning: the number of workgroups the
 * decode split-K kernel uses (0 = the occupancy-derived default).  Values
 * above the library maximum are clamped.  Results do not depend on it beyond
 * floating-point rounding.  Returns the value in effect.
 */
int gqa_set_decode_workgroups(int n);

/*
 * Work-schedule override for tests and tuning: static_permille (0..1000) of
 * the decode tiles are split into static shares, the rest into chunks of
 * chunk_tiles (>= 1) tiles handed out dynamically.  (-1, 0) restores the
 * defaults: chunks of 4 tiles, and 900 per mille static, or every tile static
 * when a launch has at most 32 tiles per workgroup with every past_len at
 * max_past_len (small batches).  Results do not depend on it beyond
 * floating-point rounding.
 * Returns GQA_OK or GQA_ERR_INVALID_ARG.
 */
int gqa_set_decode_schedule(int static_permille, int chunk_tiles);

/*
 * Work-split tuning of the decode split-K kernel: the static share of each
 * workgroup dispatch slot (the k-th workgroup resident on a CU) is
 * ratio_permille / 1000 times that of the next younger slot.  Older residents
 * win instruction issue on a CU and stream faster, so equal shares
 * (ratio_permille = 1000) leave the youngest finishing last.  A value <= 0
 * restores the defaults, which depend on the kernel variant (1400 when a
 * workgroup holds one head group, i.e. up to 4 query heads per segment, and
 * 1200 otherwise); others are
 * clamped to [250, 8000].  Results do not depend on it beyond floating-point
 * rounding.  Returns the override in effect, 0 for the defaults.
 */
int gqa_set_decode_slot_ratio(int ratio_permille);

/*
 * Path override for tests and tuning: the smallest group size g = n_q / n_kv
 * that gqa_decode_attn(_ex) hands to its wide-group kernel (both products on
 * the matrix cores, every K/V row read once for all g heads; taken only for
 * g <= 64 and n_kv <= 64).  Smaller groups use the split-K kernel, which reads
 * K/V once per 16 heads and is the faster one for g <= 8.  0 restores the
 * default (16); a value above 64 turns the wide kernel off.  Results agree between the paths within the attention
 * tolerance.  Returns the value in effect.
 */
int gqa_set_decode_wide_min_group(int g);

/*
 * Path override for tests and tuning of gqa_decode_step: the tile bound
 * (B * n_kv * ceil((max_past_len + 1) / 64), fewer under a window) from which
 * a step runs as gqa_rope_append followed by the split-K decode instead of
 * its single-launch kernel.  0 or less restores the default (512); a large
 * value keeps every step in one launch.  Results agree between the paths
 * within the attention tolerance (the rotated rows are identical).  Returns
 * the value in effect.
 */
int gqa_set_decode_step_split_min_tiles(int tiles);

#ifdef __cplusplus
}
#endif
#endif /* GQA_H */
