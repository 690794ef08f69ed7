/*
 * Host-side exercise of the C ABI (include/dflash.h) for the sanitizer build: every
 * entry point called with arguments its host checks must refuse, plus (with the
 * argument "no-gpu", on a machine without a GPU) fully valid calls that reach their
 * first HIP call and must return DFLASH_EHIP.  No pointer passed here is ever
 * dereferenced by the host code.  Exit status: the number of failed checks.
 */
#include <stdio.h>
#include <string.h>

#include "dflash.h"

static int failures = 0;

#define EXPECT(call, want)                                                          \
    do {                                                                            \
        long long got_ = (long long)(call);                                         \
        if (got_ != (long long)(want)) {                                            \
            printf("FAIL %s: got %lld want %lld\n", #call, got_, (long long)(want)); \
            failures++;                                                             \
        }                                                                           \
    } while (0)

#define P(x) ((void *)(unsigned long)(x))
#define FAKE 0x10000ul

static dflash_config tiny(void) {
    dflash_config c;
    memset(&c, 0, sizeof c);
    c.n_layers = 1; c.hidden = 256; c.ffn = 768; c.n_q_heads = 4; c.n_kv_heads = 2;
    c.head_dim = 64; c.window = 32; c.vocab = 4096; c.n_taps = 5; c.block = 8; c.top_k = 4;
    c.sel_rank = 32; c.weight_fmt = DFLASH_W_Q4K;
    c.rms_eps = 1e-6f; c.rope_theta = 1e6f; c.pair_scale = 0.1767767f;
    return c;
}

static dflash_weights fake_weights(int layers) {
    dflash_weights w;
    memset(&w, 0, sizeof w);
    w.fc = P(FAKE); w.hidden_norm = P(FAKE); w.final_norm = P(FAKE); w.embed = P(FAKE);
    w.lm_head = P(FAKE); w.mask_emb = P(FAKE); w.sel_proj = P(FAKE); w.code_a = P(FAKE);
    w.code_b = P(FAKE);
    for (int l = 0; l < layers; l++) {
        dflash_layer_weights *lw = &w.layer[l];
        lw->wq = lw->wk = lw->wv = lw->wo = lw->wg = lw->wu = lw->wd = P(FAKE);
        lw->in_norm = lw->post_norm = lw->q_norm = lw->k_norm = lw->w_conv = P(FAKE);
    }
    w.linear_layout = DFLASH_LAYOUT_TILED;
    return w;
}

static int step(const dflash_config *c, const dflash_weights *w, int batch, int t_new,
                void *ws, size_t ws_bytes) {
    return dflash_draft_step(c, w, batch, P(FAKE), t_new, P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                             64, P(FAKE), P(FAKE), P(FAKE), NULL, NULL, ws, ws_bytes, NULL, NULL);
}

int main(int argc, char **argv) {
    const int no_gpu = argc > 1 && strcmp(argv[1], "no-gpu") == 0;
    for (int s = -8; s <= 1; s++) EXPECT(dflash_status_str(s) != NULL, 1);

    dflash_config c = tiny();
    dflash_weights w = fake_weights(1);
    EXPECT(dflash_workspace_bytes(NULL, 1, 8), 0);
    EXPECT(dflash_workspace_bytes(&c, 0, 8) , 0);
    EXPECT(dflash_workspace_bytes(&c, 1, 9), 0);
    EXPECT(dflash_workspace_bytes(&c, 1, 8) > 0, 1);

    EXPECT(step(NULL, &w, 1, 8, P(FAKE << 8), 1ull << 40), DFLASH_EINVAL);
    EXPECT(step(&c, NULL, 1, 8, P(FAKE << 8), 1ull << 40), DFLASH_EINVAL);
    EXPECT(step(&c, &w, 0, 8, P(FAKE << 8), 1ull << 40), DFLASH_EINVAL);
    EXPECT(step(&c, &w, 1, 0, P(FAKE << 8), 1ull << 40), DFLASH_EINVAL);
    EXPECT(step(&c, &w, 1, 8, NULL, 1ull << 40), DFLASH_EWORKSPACE);
    EXPECT(step(&c, &w, 1, 8, P(FAKE << 8), 16), DFLASH_EWORKSPACE);
    EXPECT(step(&c, &w, 1, 8, P((FAKE << 8) + 16), 1ull << 40), DFLASH_EWORKSPACE);
    dflash_config bad = tiny();
    bad.head_dim = 96;
    EXPECT(step(&bad, &w, 1, 8, P(FAKE << 8), 1ull << 40), DFLASH_ESHAPE);
    bad = tiny();
    bad.n_layers = DFLASH_MAX_LAYERS + 1;
    EXPECT(step(&bad, &w, 1, 8, P(FAKE << 8), 1ull << 40), DFLASH_ESHAPE);
    bad = tiny();
    bad.weight_fmt = 9;
    EXPECT(step(&bad, &w, 1, 8, P(FAKE << 8), 1ull << 40), DFLASH_EINVAL);
    dflash_weights w2 = w;
    w2.layer[0].wq = P(FAKE + 4);
    EXPECT(step(&c, &w2, 1, 8, P(FAKE << 8), 1ull << 40), DFLASH_EALIGN);
    w2 = w;
    w2.linear_layout = DFLASH_LAYOUT_ROWMAJOR;
    EXPECT(step(&c, &w2, 1, 8, P(FAKE << 8), 1ull << 40), DFLASH_ELAYOUT);

    dflash_config full = tiny();
    full.n_layers = 5; full.hidden = 5120; full.ffn = 17408; full.n_q_heads = 32;
    full.n_kv_heads = 8; full.head_dim = 128; full.window = 2048; full.vocab = 248320;
    full.top_k = 16; full.sel_rank = 256;
    dflash_weights wf = fake_weights(5);
    EXPECT(dflash_draft_step_noalloc(&full, &wf, 16, P(FAKE), 8, P(FAKE), P(FAKE), P(FAKE),
                                     P(FAKE), 64, P(FAKE), P(FAKE), P(FAKE), NULL, NULL, NULL),
           DFLASH_ESCRATCH);
    EXPECT(dflash_draft_step_noalloc(&full, NULL, 1, P(FAKE), 8, P(FAKE), P(FAKE), P(FAKE),
                                     P(FAKE), 64, P(FAKE), P(FAKE), P(FAKE), NULL, NULL, NULL),
           DFLASH_EINVAL);

    EXPECT(dflash_verify_prefix(P(FAKE), P(FAKE), 1, 0, P(FAKE), P(FAKE), NULL), DFLASH_EINVAL);
    EXPECT(dflash_verify_prefix(NULL, P(FAKE), 1, 7, P(FAKE), P(FAKE), NULL), DFLASH_EINVAL);
    EXPECT(dflash_verify_sampled_workspace_bytes(0, 7, 4096), 0);
    EXPECT(dflash_verify_sampled(P(FAKE), P(FAKE), P(FAKE), 2, 7, 4096, 0.f, 20, 0.95f, P(FAKE),
                                 1ull << 40, P(FAKE), P(FAKE), NULL), DFLASH_EINVAL);
    EXPECT(dflash_verify_sampled(P(FAKE), P(FAKE + 2), P(FAKE), 2, 7, 4096, 1.f, 20, 0.95f,
                                 P(FAKE), 1ull << 40, P(FAKE), P(FAKE), NULL), DFLASH_EALIGN);

    EXPECT(q4k_gemm_workspace_bytes(8, 5120, 100), 0);
    EXPECT(q4k_gemm(P(FAKE), P(FAKE), P(FAKE), 8, 5121, 5120, P(FAKE), 1ull << 40, NULL), DFLASH_ESHAPE);
    EXPECT(q4k_gemm(P(FAKE), P(FAKE), P(FAKE), 8, 5120, 5120, P(FAKE), 1ull << 40, NULL), DFLASH_EINVAL);
    EXPECT(q4k_gemm_tiled(P(FAKE + 4), P(FAKE), P(FAKE), 8, 5120, 5120, P(FAKE), 1ull << 40, NULL),
           DFLASH_EALIGN);
    EXPECT(q8_0_gemm(P(FAKE), P(FAKE), P(FAKE), 0, 5120, 5120, P(FAKE), 1ull << 40, NULL), DFLASH_ESHAPE);
    EXPECT(q8_0_gemm_tiled(P(FAKE), P(FAKE), P(FAKE), 8, 5120, 5120, P(FAKE), 16, NULL),
           DFLASH_EWORKSPACE);
    EXPECT(q4k_to_tiled(P(FAKE), P(FAKE + 1024), 16, 256, NULL), DFLASH_EINVAL);
    EXPECT(q8_0_to_tiled(P(FAKE), P(FAKE + (1ul << 30)), 24, 256, NULL), DFLASH_ESHAPE);
    EXPECT(q4k_dequantize(P(FAKE), P(FAKE), 0, NULL), DFLASH_EINVAL);
    EXPECT(q8_0_dequantize(P(FAKE + 2), P(FAKE), 1, NULL), DFLASH_EALIGN);
    EXPECT(fp8_gemm_workspace_bytes(8, 5120, 100), 0);
    EXPECT(fp8_gemm(P(FAKE), P(FAKE), P(FAKE), 8, 5120, 5120, P(FAKE), 1ull << 40, NULL), DFLASH_EINVAL);
    EXPECT(fp8_gemm_tiled(P(FAKE), P(FAKE), P(FAKE), 8, 5121, 5120, P(FAKE), 1ull << 40, NULL),
           DFLASH_ESHAPE);
    EXPECT(fp8_to_tiled(P(FAKE), P(FAKE + 4096), 16, 256, NULL), DFLASH_EINVAL);
    EXPECT(fp8_dequantize(P(FAKE), P(FAKE), 4, 250, NULL), DFLASH_ESHAPE);

    if (no_gpu) {
        /* valid on the host: the first HIP call fails */
        EXPECT(step(&c, &w, 1, 8, P(FAKE << 8), 1ull << 40), DFLASH_EHIP);
        EXPECT(dflash_draft_step_noalloc(&c, &w, 1, P(FAKE), 8, P(FAKE), P(FAKE), P(FAKE),
                                         P(FAKE), 64, P(FAKE), P(FAKE), P(FAKE), NULL, NULL, NULL),
               DFLASH_EHIP);
        EXPECT(dflash_verify_prefix(P(FAKE), P(FAKE), 1, 7, P(FAKE), P(FAKE), NULL), DFLASH_EHIP);
        EXPECT(q4k_gemm_tiled(P(FAKE), P(FAKE), P(FAKE), 8, 5120, 5120, P(FAKE), 1ull << 40, NULL),
               DFLASH_EHIP);
        EXPECT(q4k_gemm(P(FAKE), P(FAKE), P(FAKE), 8, 5120, 5120, P(FAKE << 12), 1ull << 40, NULL),
               DFLASH_EHIP);
    }
    printf("%d failed checks\n", failures);
    return failures;
}
