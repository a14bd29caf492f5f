// Internal launch interface between the C ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

// RoPE parameters as the kernels see them (validated on the host).
struct RopeDev {
    double attn;     // multiplier of the rotated dims
    int layout;      // 0 interleaved pairs (2i, 2i+1); 1 half pairs (i, i + r/2)
    int rotary_dim;  // rotated dims r (multiple of 16, <= d <= 128)
    // angle per position of pair i < r/2 (radians), with the context-extension
    // rule already applied; position-independent, so the host computes them
    // once per call and the kernels only multiply by the position
    double freq[64];
};

// Kernel kinds for the timing hooks.
enum KernelKind {
    K_ROPE_APPEND = 0,
    K_DECODE_PARTIAL = 1,
    K_DECODE_COMBINE = 2,
    K_PREFILL = 3,
    K_DECODE_STEP = 4,
    K_DECODE_WIDE = 5,
    K_STREAM_READ = 6,
    K_KINDS = 7
};

// Timing hooks (no-ops unless enabled through gqa_profile_enable).
void prof_begin(int kind, hipStream_t st);
void prof_end(int kind, hipStream_t st);

// ---- rope_append ---------------------------------------------------------------
hipError_t launch_rope_append(const uint16_t* q, uint16_t* q_rot, const uint16_t* k_new, const uint16_t* v_new,
                              uint16_t* k_cache, uint16_t* v_cache, const int32_t* past_len, int max_past_len,
                              int B, int n_q, int n_kv, int T, int d, int S, const RopeDev& rope, hipStream_t st);

// ---- decode (split-K partials + combine) ----------------------------------------
// Largest batch one decode launch handles; larger batches are processed in
// slices of this many sequences.
constexpr int DECODE_MAX_B = 1024;
// Upper bound on the number of split-K workgroups (sizes the workspace).
constexpr int DECODE_MAX_WG = 2048;
// Work schedule of the split-K kernel: this many per-mille of the tiles are
// split into static shares (weighted by dispatch slot), the rest into chunks of DECODE_DEFAULT_CHUNK
// tiles handed out by a ticket counter (at most DECODE_MAX_CHUNKS chunks; the
// chunk grows when a launch would need more).
constexpr int DECODE_DEFAULT_STATIC_PM = 900;
// Chunks of 4 tiles measured best (one Llama-3.1-8B layer at B = 32: 99.5 us
// against 100.0 us with 3, 100.5 with 5, 101.3 with 6; the 70B shape level
// or 1 % faster); 1-tile chunks at the end of the list were slower still
// (every piece adds a record and a ticket round trip).
constexpr int DECODE_DEFAULT_CHUNK = 4;
// ... unless a launch has at most this many tiles per workgroup (bounded with
// every past_len at max_past_len): then every tile is in a static share.
constexpr int DECODE_STATIC_ONLY_TILES = 32;
constexpr int DECODE_MAX_CHUNKS = 8192;
// The static shares are weighted by dispatch slot (the k-th workgroup resident
// on a CU): each slot's share is a fixed multiple of the next younger one's,
// by default chosen per kernel variant; at most this many distinct slots.
constexpr int DECODE_MAX_SLOTS = 4;

struct DecodePlan {
    int hgw;   // query heads per wave (1..4)
    int nhg;   // head groups per workgroup (1, 2 or 4)
    int gc;    // heads per segment = hgw * nhg
    int nhc;   // segments per (sequence, KV head) = g / gc
    int rg;    // row groups per workgroup = 4 / nhg
    int rec;   // floats per partial record = d + 4
    size_t slot_floats;  // gc * rec: one record per head of a piece
};
DecodePlan decode_plan(int n_q, int n_kv, int d);
size_t decode_workspace_bytes(int B, int n_q, int n_kv, int d);
// the part of it that a launch with the current settings uses (split-K or wide-group records)
size_t decode_launch_workspace_bytes(int B, int n_q, int n_kv, int d);
void set_decode_schedule(int static_permille, int chunk_tiles);
void set_decode_slot_ratio(int ratio_permille);  // 0: per-variant defaults
int decode_slot_ratio();
hipError_t launch_decode(const uint16_t* q_rot, const uint16_t* k_cache, const uint16_t* v_cache,
                         const int32_t* past_len, int max_past_len, uint16_t* out, float* ws, int B, int n_q,
                         int n_kv, int d, int S, float scale, int window, int n_sink, const float* sink_logits,
                         int wg_override, hipStream_t st, float* sched_hdr = nullptr);

// Compute units of the current device, looked up once per device (launch
// shapes are sized from it).
hipError_t device_cu_count(int* n);

// ---- prefill -----------------------------------------------------------------------
hipError_t launch_prefill(const uint16_t* q_rot, const uint16_t* k_cache, const uint16_t* v_cache,
                          const int32_t* past_len, int max_past_len, uint16_t* out, int B, int n_q, int n_kv, int T,
                          int d, int S, float scale, int window, int n_sink, const float* sink_logits,
                          hipStream_t st);

// ---- single-launch decode step (rope + append + attention + merge) ------------
// Most splits of one (sequence, KV head) segment; sizes the workspace.
constexpr int DECODE_STEP_MAX_SPLITS = 64;
// Splits a launch uses: about two workgroups per CU over all segments, at most
// one per tile of the longest context and at most DECODE_STEP_MAX_SPLITS.
int decode_step_splits(int B, int n_kv, int max_past_len, int window, int n_sink);
size_t decode_step_workspace_bytes(int B, int n_q, int n_kv, int d);
// tile bound from which gqa_decode_step runs as rope_append + split-K decode (<= 0: the default)
void set_decode_step_split_min_tiles(int tiles);
int decode_step_split_min_tiles();
hipError_t launch_decode_step(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_cache,
                              uint16_t* v_cache, const int32_t* past_len, int max_past_len, uint16_t* out,
                              uint16_t* q_rot, void* ws, size_t ws_bytes, int B, int n_q, int n_kv, int d, int S,
                              const RopeDev& rope, float scale, int window, int n_sink, const float* sink_logits,
                              hipStream_t st);

// ---- decode for wide query groups (g >= 16: both products on MFMA) ------------
// The decode workspace starts with a header of this many floats (256 bytes)
// that holds the split-K ticket counter; records follow it.
constexpr int DECODE_WS_HEADER_FLOATS = 64;
constexpr int DECODE_WIDE_MIN_G = 16;       // used from this group size on
constexpr int DECODE_WIDE_MAX_G = 64;
constexpr int DECODE_WIDE_MAX_SEGS = 64;    // segments per launch (bounds the record space)
constexpr int DECODE_WIDE_MAX_SPLITS = 64;  // splits per segment (the wide combine merges at most 64 records)
int decode_wide_splits(int nb, int n_kv, int g, int max_past_len, int window, int n_sink, int wg_override);
size_t decode_wide_record_bytes(int B, int n_q, int n_kv, int d);
// Smallest group size that takes the wide kernel (0 restores the default).
void set_decode_wide_min_group(int g);
int decode_wide_min_group();
hipError_t launch_decode_wide(const uint16_t* q_rot, const uint16_t* k_cache, const uint16_t* v_cache,
                              const int32_t* past_len, int max_past_len, uint16_t* out, float* ws, int B, int n_q,
                              int n_kv, int d, int S, float scale, int window, int n_sink, const float* sink_logits,
                              int wg_override, hipStream_t st);

// ---- measurement: a read-only streaming kernel (the HBM read ceiling) ------------
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups, hipStream_t st);

}  // namespace gqa
