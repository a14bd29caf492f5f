/* A plain C11 consumer of libgqa: includes only include/gqa.h, links against
 * the built library, and drives the host-side paths of the C ABI (size
 * queries, every argument check, status strings).  None of these calls
 * reaches the GPU: each check fails on the host before any HIP call, so the
 * program runs without a device.  Prints one line per check and exits with
 * the number of failures. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gqa.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
    if (got != want) {
        printf("FAIL %s: got %d (%s), want %d\n", what, got, gqa_status_string(got), want);
        ++failures;
    } else {
        printf("ok   %s -> %d\n", what, got);
    }
}

int main(void) {
    /* stand-in device pointers: 16-byte aligned, never dereferenced on the host */
    static _Alignas(16) unsigned char buf[1024];
    void* p = buf;
    const int32_t* pl = (const int32_t*)(const void*)buf;
    gqa_rope_params rope;
    memset(&rope, 0, sizeof(rope));
    rope.theta = 500000.0;
    rope.layout = GQA_ROPE_INTERLEAVED;
    rope.scaling = GQA_ROPE_SCALING_NONE;

    /* size queries: valid shapes give a non-zero size, invalid ones 0 */
    {
        size_t a = gqa_decode_workspace_bytes(32, 32, 8, 128, 8192);
        size_t b = gqa_decode_workspace_bytes(64, 32, 8, 128, 8192);
        printf("%s decode workspace B32 %zu bytes, B64 %zu bytes\n", (a > 256 && b >= a) ? "ok  " : "FAIL", a, b);
        if (!(a > 256 && b >= a)) ++failures;
        expect("workspace bytes of n_q % n_kv != 0 is 0", (int)gqa_decode_workspace_bytes(32, 30, 8, 128, 8192), 0);
        expect("workspace bytes of d = 96 is 0", (int)gqa_decode_workspace_bytes(32, 32, 8, 96, 8192), 0);
        expect("step workspace of a valid shape is non-zero",
               gqa_decode_step_workspace_bytes(4, 32, 8, 128, 2048) > 0, 1);
    }

    /* rope_append argument checks */
    expect("rope_append null q", gqa_rope_append(NULL, p, p, p, p, p, pl, 10, 1, 32, 8, 1, 128, 64, &rope, NULL),
           GQA_ERR_INVALID_ARG);
    expect("rope_append misaligned k_cache",
           gqa_rope_append(p, p, p, p, buf + 8, p, pl, 10, 1, 32, 8, 1, 128, 64, &rope, NULL), GQA_ERR_INVALID_ARG);
    expect("rope_append n_q % n_kv", gqa_rope_append(p, p, p, p, p, p, pl, 10, 1, 30, 8, 1, 128, 64, &rope, NULL),
           GQA_ERR_GROUP);
    expect("rope_append d = 96", gqa_rope_append(p, p, p, p, p, p, pl, 10, 1, 32, 8, 1, 96, 64, &rope, NULL),
           GQA_ERR_HEAD_DIM);
    expect("rope_append past + T > S", gqa_rope_append(p, p, p, p, p, p, pl, 64, 1, 32, 8, 1, 128, 64, &rope, NULL),
           GQA_ERR_RANGE);
    rope.theta = -1.0;
    expect("rope_append theta < 0", gqa_rope_append(p, p, p, p, p, p, pl, 10, 1, 32, 8, 1, 128, 64, &rope, NULL),
           GQA_ERR_INVALID_ARG);
    rope.theta = 500000.0;
    rope.rotary_dim = 24;
    expect("rope_append rotary_dim not a multiple of 16",
           gqa_rope_append(p, p, p, p, p, p, pl, 10, 1, 32, 8, 1, 128, 64, &rope, NULL), GQA_ERR_INVALID_ARG);
    rope.rotary_dim = 0;

    /* decode attention */
    expect("decode_attn workspace too small",
           gqa_decode_attn(p, p, p, pl, 10, p, p, 16, 1, 32, 8, 128, 64, 0.0f, NULL), GQA_ERR_WORKSPACE);
    expect("decode_attn max_past_len = S", gqa_decode_attn(p, p, p, pl, 64, p, p, 1u << 30, 1, 32, 8, 128, 64, 0.0f,
                                                           NULL),
           GQA_ERR_RANGE);
    expect("decode_attn B = 0", gqa_decode_attn(p, p, p, pl, 10, p, p, 1u << 30, 0, 32, 8, 128, 64, 0.0f, NULL),
           GQA_ERR_INVALID_ARG);
    {
        gqa_attn_opts o;
        o.window = -1;
        o.n_sink = 0;
        o.sink_logits = NULL;
        expect("decode_attn_ex negative window",
               gqa_decode_attn_ex(p, p, p, pl, 10, p, p, 1u << 30, 1, 32, 8, 128, 64, 0.0f, &o, NULL),
               GQA_ERR_INVALID_ARG);
    }
    expect("decode_attn_noalloc over its buffer",
           gqa_decode_attn_noalloc(p, p, p, pl, 10, p, 1024, 64, 8, 128, 8192, 0.0f, NULL, NULL), GQA_ERR_SCRATCH);

    /* prefill and the single-launch step */
    expect("prefill_attn n_q % n_kv", gqa_prefill_attn(p, p, p, pl, 10, p, 1, 12, 8, 4, 128, 64, 0.0f, NULL),
           GQA_ERR_GROUP);
    expect("decode_step group above the maximum",
           gqa_decode_step(p, p, p, p, p, pl, 10, p, NULL, p, 1u << 30, 1, 128, 1, 128, 64, &rope, 0.0f, NULL, NULL),
           GQA_ERR_INVALID_ARG);

    /* every status has a message */
    {
        int codes[] = {GQA_OK, GQA_ERR_INVALID_ARG, GQA_ERR_GROUP, GQA_ERR_HEAD_DIM, GQA_ERR_RANGE,
                       GQA_ERR_WORKSPACE, GQA_ERR_HIP, GQA_ERR_SCRATCH};
        for (unsigned i = 0; i < sizeof(codes) / sizeof(codes[0]); ++i) {
            const char* s = gqa_status_string(codes[i]);
            if (!s || !s[0]) {
                printf("FAIL status %d has no message\n", codes[i]);
                ++failures;
            }
        }
        printf("ok   status strings\n");
    }
    printf("%d failure(s)\n", failures);
    return failures;
}
