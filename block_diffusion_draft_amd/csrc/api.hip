// C ABI of the draft-step library: argument checks, workspace plan and the
// launch sequence of one step on the caller's stream.  Nothing is allocated.
#include "../../include/dflash.h"
#include "kernels.h"
#include <cmath>

#include <mutex>
#include <string.h>

int topk_chunk_size();

namespace {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
    int B, T, P, t_new, H, F, n_q, n_kv, d, qd, kd, V, K, r, L;
    int M_blk, M_ctx, M_qkv, R, G, QR;
    int attn_chunk, attn_nch;
    int topk_nch;
    bool lm_skinny;
    int head_nrun, head_rc;      // column runs of the head's statistics (rc 0: none)
    int head_rt;                 // > 0: balanced runs over this many 16-column tiles
    // byte offsets into the workspace
    size_t o_valid, o_h, o_xc, o_u2, o_fcout, o_Q, o_Kb, o_Vb, o_attnO, o_attnML, o_o, o_zp,
        o_Y, o_mid2, o_f, o_logits, o_topk, o_rstat, o_ssq_x, o_ssq_c, o_ssq_u, o_part;
    size_t total;
};

// fp32 partial sums of one GEMM: [splits][M][N] (Q4_K split-K) or [M][N] (bf16)
// Which kernel runs a product: the 16-row streaming kernels (Q4_K, Q8_0, FP8) where
// their shape rules allow, else the many-row GEMM; bf16 up to 16 rows on the tiled kernel.
int big_fmt(int fmt) {
    return fmt == DFLASH_W_Q4K ? 2 : (fmt == DFLASH_W_Q8_0 ? 1 : (fmt == DFLASH_W_FP8 ? 3 : 0));
}
bool quant_fmt(int fmt) {
    return fmt == DFLASH_W_Q4K || fmt == DFLASH_W_Q8_0 || fmt == DFLASH_W_FP8;
}
bool use_stream(int fmt, int M, int N, int K) {
    switch (fmt) {
        case DFLASH_W_Q4K: return q4k_stream_ok(M, N, K);
        case DFLASH_W_Q8_0: return q8_stream_ok(M, N, K);
        case DFLASH_W_FP8: return f8_stream_ok(M, N, K);
        default: return false;
    }
}
Q4kStreamPlan stream_plan(int fmt, int M, int N, int K, int pair = 0) {
    return fmt == DFLASH_W_Q4K ? q4k_stream_plan(M, N, K, pair)
                               : (fmt == DFLASH_W_Q8_0 ? q8_stream_plan(M, N, K, pair)
                                                       : f8_stream_plan(M, N, K, pair));
}
bool use_big(int fmt, int M, int N, int K) {
    if (fmt != DFLASH_W_BF16 && use_stream(fmt, M, N, K)) return false;
    if (fmt == DFLASH_W_BF16 && M <= 16) return false;
    return big_gemm_ok(big_fmt(fmt), M, N, K);
}

size_t gemm_part_bytes(int fmt, int M, int N, int K) {
    if (use_big(fmt, M, N, K)) return big_gemm_plan(big_fmt(fmt), M, N, K).part_bytes;
    if (quant_fmt(fmt) && use_stream(fmt, M, N, K)) return stream_plan(fmt, M, N, K).part_bytes;
    return (size_t)M * N * 4;
}

bool make_plan(const dflash_config *c, int B, int t_new, Plan &p) {
    p.B = B;
    p.T = c->block;
    p.P = c->block - 1;
    p.t_new = t_new;
    p.H = c->hidden;
    p.F = c->ffn;
    p.n_q = c->n_q_heads;
    p.n_kv = c->n_kv_heads;
    p.d = c->head_dim;
    p.qd = p.n_q * p.d;
    p.kd = p.n_kv * p.d;
    p.V = c->vocab;
    p.K = c->top_k;
    p.r = c->sel_rank;
    p.L = c->n_layers;
    p.M_blk = B * p.T;
    p.M_ctx = B * t_new;
    p.M_qkv = p.M_blk + p.M_ctx;
    p.R = B * p.P;
    p.G = p.n_q / p.n_kv;
    p.QR = p.G * p.T;
    // keys per attention workgroup: 64 at batch 1 (more workgroups), larger when
    // the batch already fills the chip (fewer partials to merge)
    const int win = c->window;
    const long long wgs64 = (long long)B * p.n_kv * ((win + 63) / 64);
    p.attn_chunk = wgs64 >= 4096 ? 256 : 64;
    p.attn_nch = win > 0 ? (win + p.attn_chunk - 1) / p.attn_chunk : 0;
    p.topk_nch = (p.V + topk_chunk_size() - 1) / topk_chunk_size();
    // output-head rows held in LDS: K/32 fragments of 512 bytes (+1 zero entry)
    p.lm_skinny = p.R <= 8 && p.H % 256 == 0 &&
                  ((size_t)(p.H / 32) * 32 + 16 + 8 * 512) * 16 <= 160 * 1024;
    // the streaming head leaves per-run softmax statistics for the selector (one launch
    // after the head instead of two passes over the logits) where the runs fit it
    p.head_nrun = p.head_rc = p.head_rt = 0;
    if (p.lm_skinny) {
        head_runs(p.V, p.H, &p.head_nrun, &p.head_rc, &p.head_rt);
    } else if (big_gemm_ok(0, p.R, p.V, p.H)) {
        // the many-row head: runs of one or two waves' columns within its tiles
        const BigGemmPlan hp = big_gemm_plan_grid(0, p.R, p.V, p.H);
        p.head_rc = big_gemm_head_run_cols(hp.bn);
        p.head_nrun = (p.V + p.head_rc - 1) / p.head_rc;
    }
    if (p.head_rc > 512 || (p.head_rc & (p.head_rc - 1)) || p.head_nrun > 2048)
        p.head_nrun = p.head_rc = p.head_rt = 0;

    size_t part = 0;
    const int fmt = c->weight_fmt;
    auto upd = [&](size_t x) { if (x > part) part = x; };
    upd(gemm_part_bytes(fmt, p.M_ctx, p.H, c->n_taps * p.H));
    upd(gemm_part_bytes(fmt, p.M_qkv, p.qd + 2 * p.kd, p.H));
    upd(gemm_part_bytes(fmt, p.M_blk, p.H, p.qd));
    // the MLP runs over [hi rows; lo rows] of its bf16-pair activations
    upd(gemm_part_bytes(fmt, 2 * p.M_blk, 2 * p.F, p.H));
    upd(gemm_part_bytes(fmt, 2 * p.M_blk, p.H, p.F));

    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
    p.o_valid = take((size_t)B * 4);
    p.o_h = take((size_t)p.M_blk * p.H * 4);
    p.o_xc = take((size_t)p.M_qkv * p.H * 2);
    p.o_u2 = take((size_t)2 * p.M_blk * p.H * 2);
    p.o_fcout = take((size_t)p.M_ctx * p.H * 4);
    p.o_Q = take((size_t)p.M_blk * p.qd * 2);
    p.o_Kb = take((size_t)p.M_blk * p.kd * 2);
    p.o_Vb = take((size_t)p.M_blk * p.kd * 2);
    const size_t nslots = (size_t)B * p.n_kv * (p.attn_nch + 1) * p.QR;
    p.o_attnO = take(nslots * p.d * 4);
    p.o_attnML = take(nslots * 2 * 4);
    p.o_o = take((size_t)p.M_blk * p.qd * 4);
    p.o_zp = take((size_t)B * p.n_q * (p.d / 32) * p.T * 2 * p.n_q * 4);
    p.o_Y = take((size_t)p.M_blk * p.qd * 2);
    p.o_mid2 = take((size_t)2 * p.M_blk * p.F * 2);
    p.o_f = take((size_t)p.R * p.H * 2);
    p.o_logits = take((size_t)p.R * p.V * 4);
    p.o_topk = take(topk_workspace_floats(p.R, p.V) * 4);
    p.o_rstat = take((size_t)p.R * p.head_nrun * 2 * 4);
    p.o_ssq_x = take((size_t)p.M_blk * (p.H / 256) * 4);
    p.o_ssq_c = take((size_t)p.M_ctx * (p.H / 256) * 4);
    p.o_ssq_u = take((size_t)p.M_blk * (p.H / 256) * 4);
    p.o_part = take(part);
    p.total = o;
    return true;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

int check_config(const dflash_config *c) {
    if (!c) return DFLASH_EINVAL;
    if (c->n_layers < 1 || c->n_layers > DFLASH_MAX_LAYERS) return DFLASH_ESHAPE;
    if (c->hidden <= 0 || c->hidden % 256 || c->hidden > 8192 || c->ffn <= 0 || c->ffn % 256)
        return DFLASH_ESHAPE;
    if (c->head_dim != 64 && c->head_dim != 128) return DFLASH_ESHAPE;
    if (c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->n_q_heads % c->n_kv_heads) return DFLASH_ESHAPE;
    if (c->n_q_heads / c->n_kv_heads > 4 || c->n_q_heads % 2 || c->n_q_heads > 64)
        return DFLASH_ESHAPE;
    const int qd = c->n_q_heads * c->head_dim;
    if (qd % 256 || qd > 8192) return DFLASH_ESHAPE;
    if (c->block < 2 || c->block > DFLASH_BLOCK) return DFLASH_ESHAPE;
    if (c->n_taps < 1 || c->n_taps > 16) return DFLASH_ESHAPE;
    if (c->top_k < 1 || c->top_k > DFLASH_MAX_TOPK) return DFLASH_ESHAPE;
    if (c->vocab < c->top_k || c->vocab % 16) return DFLASH_ESHAPE;
    // the candidate merge handles up to 1024 chunk lists per row
    if ((c->vocab + topk_chunk_size() - 1) / topk_chunk_size() > 1024) return DFLASH_ESHAPE;
    if (c->sel_rank < 32 || c->sel_rank % 32 || c->sel_rank > 4096) return DFLASH_ESHAPE;
    if (c->window < 0) return DFLASH_EINVAL;
    if (c->window > 65536) return DFLASH_ESHAPE;     // attention-merge weights live in LDS
    if (!quant_fmt(c->weight_fmt) && c->weight_fmt != DFLASH_W_BF16) return DFLASH_EINVAL;
    if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.f)) return DFLASH_EINVAL;
    return DFLASH_OK;
}

#define HIPCHK(x)                                 \
    do {                                          \
        if ((x) != hipSuccess) return DFLASH_EHIP; \
    } while (0)

struct Ctx {
    const dflash_config *c;
    const Plan *p;
    unsigned char *ws;
    hipStream_t st;
    template <class T> T *at(size_t off) const { return reinterpret_cast<T *>(ws + off); }
};

// The many-row GEMM (more than 16 rows) into partials [splits][M][N]; returns the
// number of splits or a negative status.  With pair > 0, rows r and r + pair are the
// (hi, lo) halves of one activation row; *folded is set when the kernel adds them itself
// (each M tile then takes half a tile of hi rows and their lo rows), leaving partials of
// M / 2 rows.
int run_big(int wfmt, const void *const *w, const int *seg_end, int nseg, const uint16_t *A,
            int lda, int M, int N, int K, float *part, hipStream_t st, int pair = 0,
            bool *folded = nullptr) {
    BigGemmArgs g = {};
    g.lo_row = pair;
    for (int i = 0; i < 3; i++) {
        g.w[i] = w[i];
        g.seg_end[i] = seg_end[i];
    }
    g.nseg = nseg;
    g.wfmt = wfmt;
    g.A = A;
    g.lda = lda;
    g.M = M;
    g.N = N;
    g.K = K;
    g.C = part;
    g.ldc = N;
    const BigGemmPlan p = big_gemm_plan(wfmt, M, N, K);
    HIPCHK(launch_big_gemm(g, p, st));
    // (the kernels' own test: whole half tiles of hi rows, 256-column tiles)
    if (folded) *folded = pair > 0 && 2 * pair == M && pair % (p.bm / 2) == 0 && p.bn == 256;
    return p.splits;
}

// Q4_K / Q8_0 / FP8 product into partials: the streaming kernels for up to 16 rows, else
// the many-row GEMM.  Returns the number of splits or a negative status; *pair_left is
// the row pair the partial still holds (0 once the kernel has added the halves).
int run_quant(int fmt, const Q4kFusedArgs &a, hipStream_t st, int *pair_left) {
    const int K = a.KB * 256;
    *pair_left = a.pair;
    if (use_stream(fmt, a.M, a.N, K)) {
        const Q4kStreamPlan p = stream_plan(fmt, a.M, a.N, K, a.pair);
        HIPCHK(fmt == DFLASH_W_Q4K ? launch_q4k_stream(a, p, st)
                                   : (fmt == DFLASH_W_Q8_0 ? launch_q8_stream(a, p, st)
                                                           : launch_f8_stream(a, p, st)));
        if (p.pair_done) *pair_left = 0;
        return p.splits;
    }
    if (use_big(fmt, a.M, a.N, K)) {
        const void *w[3] = {a.w[0], a.w[1], a.w[2]};
        bool folded = false;
        const int splits = run_big(big_fmt(fmt), w, a.seg_end, a.nseg, a.src.A, a.src.lda, a.M,
                                   a.N, K, a.part, st, a.pair, &folded);
        if (folded) *pair_left = 0;
        return splits;
    }
    return DFLASH_ESHAPE;      // (every valid quantised shape takes one of the two above)
}

// y = A . W^T over up to 3 weight matrices stacked along N, as fp32 partial sums in
// the workspace's partial buffer [splits][M][N]: up to 16 rows the streaming Q4_K /
// Q8_0 / FP8 kernels (or the tiled MFMA kernel for bf16), more rows the many-row GEMM.  Rows r and
// r + pair (pair > 0) are the (hi, lo) halves of one activation row; *pair_left is
// the pair the partial still holds (the reduction adds those rows).  Returns the
// number of splits (> 0) or a negative status.
int run_gemm(const Ctx &x, const void *const *w, const int *seg_n, int nseg, const uint16_t *A,
             int lda, int M, int K, int pair, int *pair_left) {
    *pair_left = pair;
    int N = 0;
    int seg_end[3] = {0, 0, 0};
    for (int i = 0; i < 3; i++) {
        if (i < nseg) N += seg_n[i];
        seg_end[i] = N;
    }
    float *part = x.at<float>(x.p->o_part);
    if (quant_fmt(x.c->weight_fmt)) {
        Q4kFusedArgs a;
        for (int i = 0; i < 3; i++) {
            a.w[i] = (const unsigned char *)(i < nseg ? w[i] : w[0]);
            a.seg_end[i] = seg_end[i];
        }
        a.nseg = nseg;
        a.M = M;
        a.N = N;
        a.KB = K / 256;
        a.src.A = A;
        a.src.lda = lda;
        a.part = part;
        a.pair = pair;
        return run_quant(x.c->weight_fmt, a, x.st, pair_left);
    }
    if (use_big(DFLASH_W_BF16, M, N, K)) {
        const void *wv[3] = {w[0], nseg > 1 ? w[1] : w[0], nseg > 2 ? w[2] : w[0]};
        bool folded = false;
        const int splits = run_big(0, wv, seg_end, nseg, A, lda, M, N, K, part, x.st, pair, &folded);
        if (folded) *pair_left = 0;
        return splits;
    }
    Bf16GemmArgs a = {};
    for (int i = 0; i < 3; i++) {
        a.w[i] = (const uint16_t *)(i < nseg ? w[i] : w[0]);
        a.seg_end[i] = seg_end[i];
    }
    a.nseg = nseg;
    a.A = A;
    a.lda = lda;
    a.M = M;
    a.N = N;
    a.K = K;
    a.C = part;
    a.ldc = N;
    HIPCHK(launch_bf16_gemm_tiled(a, x.st));
    return 1;
}

}  // namespace

extern "C" {

const char *dflash_status_str(int s) {
    switch (s) {
        case DFLASH_OK: return "ok";
        case DFLASH_EINVAL: return "invalid argument (null pointer or value out of range)";
        case DFLASH_ESHAPE: return "shape not supported";
        case DFLASH_EALIGN: return "pointer not 16-byte aligned";
        case DFLASH_EWORKSPACE: return "workspace missing or too small";
        case DFLASH_EHIP: return "HIP runtime error";
        case DFLASH_ELAYOUT: return "quantised weights not declared in the tiled layout";
        case DFLASH_ESCRATCH: return "request exceeds the static scratch of the no-allocation entry point";
        default: return "unknown status";
    }
}

size_t dflash_workspace_bytes(const dflash_config *cfg, int batch, int t_new) {
    if (check_config(cfg) != DFLASH_OK || batch < 1 || t_new < 1 || t_new > DFLASH_BLOCK) return 0;
    Plan p;
    make_plan(cfg, batch, t_new, p);
    return p.total;
}

}  // extern "C"

namespace {

// Host-side validation of a draft step's arguments (everything but the workspace).
int check_step(const dflash_config *cfg, const dflash_weights *w, int batch, const uint16_t *taps,
               int t_new, const int32_t *last_token, const int32_t *ctx_len,
               const uint16_t *k_cache, const uint16_t *v_cache, int cache_cap,
               const int32_t *draft_tokens, const int32_t *cand_ids, const float *cand_logp,
               const float *dbg_hidden, const float *dbg_logits) {
    int rc = check_config(cfg);
    if (rc != DFLASH_OK) return rc;
    if (!w || !taps || !last_token || !ctx_len || !k_cache || !v_cache || !draft_tokens ||
        !cand_ids || !cand_logp)
        return DFLASH_EINVAL;
    if (batch < 1 || batch > 4096 || t_new < 1 || t_new > DFLASH_BLOCK || cache_cap < t_new)
        return DFLASH_EINVAL;
    if (!w->fc || !w->hidden_norm || !w->final_norm || !w->embed || !w->lm_head ||
        !w->mask_emb || !w->code_a || !w->code_b)
        return DFLASH_EINVAL;
    const void *ptrs[] = {w->fc, w->hidden_norm, w->final_norm, w->embed, w->lm_head,
                          w->mask_emb, w->code_a, w->code_b, taps, k_cache, v_cache,
                          dbg_hidden, dbg_logits};
    for (const void *q : ptrs)
        if (q && !aligned16(q)) return DFLASH_EALIGN;
    for (int l = 0; l < cfg->n_layers; l++) {
        const dflash_layer_weights &lw = w->layer[l];
        const void *lp[] = {lw.wq, lw.wk, lw.wv, lw.wo, lw.wg, lw.wu, lw.wd, lw.in_norm,
                            lw.post_norm, lw.q_norm, lw.k_norm, lw.w_conv};
        for (const void *q : lp) {
            if (!q) return DFLASH_EINVAL;
            if (!aligned16(q)) return DFLASH_EALIGN;
        }
    }
    // quantised matrices are read in the tiled layouts only: the caller must say so
    if (cfg->weight_fmt != DFLASH_W_BF16 && w->linear_layout != DFLASH_LAYOUT_TILED)
        return DFLASH_ELAYOUT;
    return DFLASH_OK;
}

// The launch sequence of one step on a validated call, workspace of p.total bytes.
int draft_step_impl(const dflash_config *cfg, const dflash_weights *w, int batch,
                    const uint16_t *taps, int t_new, const int32_t *last_token,
                    const int32_t *ctx_len, uint16_t *k_cache, uint16_t *v_cache,
                    int cache_cap, int32_t *draft_tokens, int32_t *cand_ids,
                    float *cand_logp, float *dbg_hidden, float *dbg_logits,
                    unsigned char *workspace, const Plan &p, const dflash_probe *probe,
                    hipStream_t stream) {
    Ctx x{cfg, &p, workspace, stream};
    const int H = p.H, L = p.L;
    float *h = x.at<float>(p.o_h);
    uint16_t *xc = x.at<uint16_t>(p.o_xc);
    int32_t *valid = x.at<int32_t>(p.o_valid);
    float *fcout = x.at<float>(p.o_fcout);
    float *part = x.at<float>(p.o_part);
    const float eps = cfg->rms_eps;
    float *ssq_x = x.at<float>(p.o_ssq_x);      // row sums of squares behind each deferred norm
    float *ssq_c = x.at<float>(p.o_ssq_c);
    float *ssq_u = x.at<float>(p.o_ssq_u);
    auto rowscale = [&](const float *ssq, int map) {
        RowScale r;
        r.ssq = ssq; r.nchunk = H / 256; r.map = map; r.n = (float)H; r.eps = eps;
        return r;
    };
    uint16_t *u2 = x.at<uint16_t>(p.o_u2);
    uint16_t *mid2 = x.at<uint16_t>(p.o_mid2);
    uint16_t *f = x.at<uint16_t>(p.o_f);
    const size_t cache_layer = (size_t)batch * p.n_kv * cache_cap * p.d;
    int splits, pair_left;
#define GEMM(...)                                          \
    do {                                                   \
        splits = run_gemm(x, __VA_ARGS__, &pair_left);     \
        if (splits < 0) return splits;                     \
    } while (0)

    // S1: fused taps c = RMSNorm(X . W_fc^T), the context rows of the K/V projection input;
    // its reduction shares one launch with S0 (independent of it): block assembly h,
    // per-sequence validity, first layer's input bf16(h * g_in).  RMSNorms are deferred:
    // the GEMM consumer scales each output row by 1 / rms.
    {
        const void *ws[1] = {w->fc};
        const int sn[1] = {H};
        GEMM(ws, sn, 1, taps, cfg->n_taps * H, p.M_ctx, cfg->n_taps * H, 0);
        const ReduceRowsArgs ra = {part, splits, p.M_ctx, H, 0, 0, fcout, ssq_c, w->hidden_norm,
                                   xc + (size_t)p.M_blk * H, nullptr, H, 0};
        const EmbedArgs ea = {w->embed, w->mask_emb, last_token, ctx_len, p.T, H, p.V, t_new,
                              cache_cap, h, w->layer[0].in_norm, xc, ssq_x, valid};
        HIPCHK(launch_reduce_norm_embed(ra, ea, batch, x.st));
    }
    if (dbg_hidden)
        HIPCHK(hipMemcpyAsync(dbg_hidden, h, (size_t)p.M_blk * H * 4, hipMemcpyDeviceToDevice, x.st));

    for (int l = 0; l < L; l++) {
        const dflash_layer_weights &lw = w->layer[l];
        const bool last = l == L - 1;
        uint16_t *kc = k_cache + (size_t)l * cache_layer;
        uint16_t *vc = v_cache + (size_t)l * cache_layer;
        // S2 + S3: [Q | K | V] of the block rows, K and V of the context rows
        {
            const void *ws[3] = {lw.wq, lw.wk, lw.wv};
            const int sn[3] = {p.qd, p.kd, p.kd};
            GEMM(ws, sn, 3, xc, H, p.M_qkv, H, 0);
        }
        // S4: split sum, per-head norms, rotary embedding, cache append
        {
            RopeArgs a;
            a.qkv = part; a.splits = splits;
            a.B = batch; a.T = p.T; a.t_new = t_new; a.n_q = p.n_q; a.n_kv = p.n_kv; a.d = p.d;
            a.blk = rowscale(ssq_x, 0); a.ctx = rowscale(ssq_c, 0);
            a.q_norm = lw.q_norm; a.k_norm = lw.k_norm; a.eps = eps;
            a.log2_theta = log2((double)cfg->rope_theta); a.ctx_len = ctx_len; a.valid = valid;
            a.Q = x.at<uint16_t>(p.o_Q); a.Kb = x.at<uint16_t>(p.o_Kb); a.Vb = x.at<uint16_t>(p.o_Vb);
            a.k_cache = kc; a.v_cache = vc; a.cap = cache_cap;
            HIPCHK(launch_qk_norm_rope(a, x.st));
        }
        // S5: split-window attention partials
        {
            AttnArgs a;
            a.Q = x.at<uint16_t>(p.o_Q); a.Kb = x.at<uint16_t>(p.o_Kb); a.Vb = x.at<uint16_t>(p.o_Vb);
            a.k_cache = kc; a.v_cache = vc; a.ctx_len = ctx_len; a.valid = valid;
            a.B = batch; a.T = p.T; a.t_new = t_new; a.n_q = p.n_q; a.n_kv = p.n_kv; a.d = p.d;
            a.window = cfg->window; a.cap = cache_cap; a.chunk = p.attn_chunk;
            a.n_chunks = p.attn_nch; a.O = x.at<float>(p.o_attnO); a.ml = x.at<float>(p.o_attnML);
            HIPCHK(launch_attention(a, x.st));
        }
        // S6: merge + two-tap dynamic convolution -> Y
        {
            MergeConvArgs a;
            a.O = x.at<float>(p.o_attnO); a.ml = x.at<float>(p.o_attnML);
            a.ctx_len = ctx_len; a.valid = valid;
            a.B = batch; a.T = p.T; a.t_new = t_new; a.n_q = p.n_q; a.n_kv = p.n_kv; a.d = p.d;
            a.window = cfg->window; a.chunk = p.attn_chunk; a.n_chunks = p.attn_nch;
            a.w_conv = lw.w_conv; a.o = x.at<float>(p.o_o); a.zp = x.at<float>(p.o_zp);
            a.Y = x.at<uint16_t>(p.o_Y);
            HIPCHK(launch_merge_conv(a, x.st));
        }
        // S7: h += Y . W_o^T; u = RMSNorm(h) as bf16 (hi, lo) pairs
        {
            const void *ws[1] = {lw.wo};
            const int sn[1] = {H};
            GEMM(ws, sn, 1, x.at<uint16_t>(p.o_Y), p.qd, p.M_blk, p.qd, 0);
            HIPCHK(launch_reduce_norm(part, splits, p.M_blk, H, 0, 1, h, ssq_u, lw.post_norm, u2,
                                      u2 + (size_t)p.M_blk * H, H, 0, x.st));
        }
        // S8: h += (silu(u Wg^T) * u Wu^T) Wd^T.  u and the SwiGLU output are carried as
        // bf16 (hi, lo) pairs (the MLP inputs dominate the rounding error), so both
        // products run over [hi rows; lo rows] and the reductions add row r and r + M.
        {
            const void *ws[2] = {lw.wg, lw.wu};
            const int sn[2] = {p.F, p.F};
            const bool probe_ffn = probe && probe->kernel == DFLASH_PROBE_FFN_GATE_UP && probe->layer == l;
            if (probe_ffn) HIPCHK(hipEventRecord((hipEvent_t)probe->ev_start, x.st));
            GEMM(ws, sn, 2, u2, H, 2 * p.M_blk, H, p.M_blk);
            if (probe_ffn) HIPCHK(hipEventRecord((hipEvent_t)probe->ev_stop, x.st));
            HIPCHK(launch_swiglu(part, splits, p.M_blk, 2 * p.F, pair_left, mid2,
                                 mid2 + (size_t)p.M_blk * p.F, p.F, rowscale(ssq_u, 0), x.st));
        }
        // down projection + residual; then the next layer's input norm, or after the last
        // layer the final norm of the proposal rows (block positions 1..7) for the head
        {
            const void *ws[1] = {lw.wd};
            const int sn[1] = {H};
            GEMM(ws, sn, 1, mid2, p.F, 2 * p.M_blk, p.F, p.M_blk);
            const uint16_t *gain = last ? w->final_norm : w->layer[l + 1].in_norm;
            HIPCHK(launch_reduce_norm(part, splits, p.M_blk, H, pair_left, 1, h, ssq_x, gain,
                                      last ? f : xc, nullptr, H, last ? p.T : 0, x.st));
        }
        if (dbg_hidden)
            HIPCHK(hipMemcpyAsync(dbg_hidden + (size_t)(l + 1) * p.M_blk * H, h,
                                  (size_t)p.M_blk * H * 4, hipMemcpyDeviceToDevice, x.st));
    }
#undef GEMM

    // S9 + S10: logits of the proposal rows with the shared output head
    float *logits = dbg_logits ? dbg_logits : x.at<float>(p.o_logits);
    {
        Bf16GemmArgs a = {};
        a.w[0] = a.w[1] = a.w[2] = w->lm_head;
        a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = p.V;
        a.nseg = 1;
        a.M = p.R; a.N = p.V; a.K = H; a.C = logits; a.ldc = p.V;
        a.A = f; a.lda = H;
        a.rs = rowscale(ssq_x, p.T);           // the final norm of the proposal rows
        if (p.head_rc) a.rstat = x.at<float>(p.o_rstat);
        const bool probe_lm = probe && probe->kernel == DFLASH_PROBE_LM_HEAD;
        if (probe_lm) HIPCHK(hipEventRecord((hipEvent_t)probe->ev_start, x.st));
        if (p.lm_skinny) {
            HIPCHK(launch_bf16_gemm_skinny(a, x.st));
        } else if (big_gemm_ok(0, p.R, p.V, H)) {
            BigGemmArgs g = {};
            g.w[0] = g.w[1] = g.w[2] = w->lm_head;
            g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = p.V;
            g.nseg = 1;
            g.wfmt = 0;
            g.A = f; g.lda = H; g.M = p.R; g.N = p.V; g.K = H; g.C = logits; g.ldc = p.V;
            g.rs = a.rs;
            g.rstat = a.rstat;
            // one split: the row scale is applied in the epilogue
            const BigGemmPlan bp = big_gemm_plan_grid(0, p.R, p.V, H);
            HIPCHK(launch_big_gemm(g, bp, x.st));
        } else {
            HIPCHK(launch_bf16_gemm_tiled(a, x.st));
        }
        if (probe_lm) HIPCHK(hipEventRecord((hipEvent_t)probe->ev_stop, x.st));
    }
    // S10 + S11: log-softmax statistics, top-K, and the selector path
    if (p.head_rc)
        HIPCHK(launch_topk_path_runs(logits, x.at<float>(p.o_rstat), p.head_nrun, p.head_rc,
                                     p.head_rt, batch, p.P, p.V, p.K, valid, x.at<float>(p.o_topk), w->code_a,
                                     w->code_b, p.r, cfg->pair_scale, cand_ids, cand_logp,
                                     draft_tokens, x.st));
    else
        HIPCHK(launch_topk_path(logits, batch, p.P, p.V, p.K, valid, x.at<float>(p.o_topk),
                                w->code_a, w->code_b, p.r, cfg->pair_scale, cand_ids, cand_logp,
                                draft_tokens, x.st));
    return DFLASH_OK;
}

// ---- the no-allocation step: its workspace is a file-scope device array.  Each GPU
// the library runs on holds its own copy (allocated when the code object is loaded on
// that device, kept until the process ends); host code reaches it only through the
// address hipGetSymbolAddress returns for that device (the array's name on the host is
// a stand-in, not a device address).
__device__ __align__(256) unsigned char scratch[DFLASH_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void *scratch_ptr[MAX_DEVICES];

// device address of `scratch` on the device of `stream`, looked up once per device with
// that device current; null (and *rc set) on failure
void *scratch_of(hipStream_t stream, int *rc) {
    int dev = -1;
    if (stream) {
        hipDevice_t d;
        if (hipStreamGetDevice(stream, &d) != hipSuccess) { *rc = DFLASH_EHIP; return nullptr; }
        dev = (int)d;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        *rc = DFLASH_EHIP;
        return nullptr;
    }
    if (dev < 0 || dev >= MAX_DEVICES) { *rc = DFLASH_EHIP; return nullptr; }
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) { *rc = DFLASH_EHIP; return nullptr; }
        if (cur != dev && hipSetDevice(dev) != hipSuccess) { *rc = DFLASH_EHIP; return nullptr; }
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !ptr) { *rc = DFLASH_EHIP; return nullptr; }
        scratch_ptr[dev] = ptr;
    }
    return scratch_ptr[dev];
}

}  // namespace

extern "C" {

int dflash_draft_step_noalloc(const dflash_config *cfg, const dflash_weights *w, int batch,
                              const uint16_t *taps, int t_new, const int32_t *last_token,
                              const int32_t *ctx_len, uint16_t *k_cache, uint16_t *v_cache,
                              int cache_cap, int32_t *draft_tokens, int32_t *cand_ids,
                              float *cand_logp, float *dbg_hidden, float *dbg_logits,
                              void *stream) {
    int rc = check_step(cfg, w, batch, taps, t_new, last_token, ctx_len, k_cache, v_cache,
                        cache_cap, draft_tokens, cand_ids, cand_logp, dbg_hidden, dbg_logits);
    if (rc != DFLASH_OK) return rc;
    Plan p;
    make_plan(cfg, batch, t_new, p);
    if (p.total > DFLASH_NOALLOC_SCRATCH_BYTES) return DFLASH_ESCRATCH;
    void *ws = scratch_of((hipStream_t)stream, &rc);
    if (!ws) return rc;
    return draft_step_impl(cfg, w, batch, taps, t_new, last_token, ctx_len, k_cache, v_cache,
                           cache_cap, draft_tokens, cand_ids, cand_logp, dbg_hidden, dbg_logits,
                           (unsigned char *)ws, p, nullptr, (hipStream_t)stream);
}

int dflash_draft_step(const dflash_config *cfg, const dflash_weights *w, int batch,
                      const uint16_t *taps, int t_new, const int32_t *last_token,
                      const int32_t *ctx_len, uint16_t *k_cache, uint16_t *v_cache,
                      int cache_cap, int32_t *draft_tokens, int32_t *cand_ids,
                      float *cand_logp, float *dbg_hidden, float *dbg_logits,
                      void *workspace, size_t ws_bytes, const dflash_probe *probe,
                      void *stream) {
    const int rc = check_step(cfg, w, batch, taps, t_new, last_token, ctx_len, k_cache, v_cache,
                              cache_cap, draft_tokens, cand_ids, cand_logp, dbg_hidden, dbg_logits);
    if (rc != DFLASH_OK) return rc;
    Plan p;
    make_plan(cfg, batch, t_new, p);
    if (!workspace || ws_bytes < p.total || ((uintptr_t)workspace & 255)) return DFLASH_EWORKSPACE;
    return draft_step_impl(cfg, w, batch, taps, t_new, last_token, ctx_len, k_cache, v_cache,
                           cache_cap, draft_tokens, cand_ids, cand_logp, dbg_hidden, dbg_logits,
                           (unsigned char *)workspace, p, probe, (hipStream_t)stream);
}

int dflash_verify_prefix(const int32_t *draft, const int32_t *target, int batch, int n,
                         int32_t *accept_len, int32_t *out_tokens, void *stream) {
    if (!draft || !target || !accept_len || !out_tokens) return DFLASH_EINVAL;
    if (batch < 1 || n < 1 || n > 64) return DFLASH_EINVAL;
    HIPCHK(launch_verify(draft, target, batch, n, accept_len, out_tokens, (hipStream_t)stream));
    return DFLASH_OK;
}

static bool sample_shape_ok(int batch, int n, int vocab) {
    return batch >= 1 && n >= 1 && n <= DFLASH_SAMPLE_MAX_N && vocab >= 1 &&
           vocab <= DFLASH_SAMPLE_MAX_VOCAB && (long long)batch * (n + 1) <= 65535;
}

size_t dflash_verify_sampled_workspace_bytes(int batch, int n, int vocab) {
    if (!sample_shape_ok(batch, n, vocab)) return 0;
    return topk_workspace_floats(batch * (n + 1), vocab) * sizeof(float);
}

int dflash_verify_sampled(const int32_t *draft, const float *target_logits, const float *uniforms,
                          int batch, int n, int vocab, float temperature, int top_k, float top_p,
                          void *workspace, size_t ws_bytes, int32_t *accept_len,
                          int32_t *out_tokens, void *stream) {
    if (!draft || !target_logits || !uniforms || !accept_len || !out_tokens) return DFLASH_EINVAL;
    if (batch < 1 || n < 1 || vocab < 1) return DFLASH_EINVAL;
    if (!(temperature > 0.f) || !std::isfinite(temperature)) return DFLASH_EINVAL;
    if (!(top_p > 0.f && top_p <= 1.f)) return DFLASH_EINVAL;
    if (top_k < 1 || top_k > vocab) return DFLASH_EINVAL;
    if (!sample_shape_ok(batch, n, vocab) || top_k > DFLASH_SAMPLE_MAX_TOPK) return DFLASH_ESHAPE;
    const void *ptrs[5] = {draft, target_logits, uniforms, accept_len, out_tokens};
    for (const void *q : ptrs)
        if ((uintptr_t)q % 4) return DFLASH_EALIGN;
    const size_t need = dflash_verify_sampled_workspace_bytes(batch, n, vocab);
    if (!workspace || ws_bytes < need || !aligned16(workspace)) return DFLASH_EWORKSPACE;
    HIPCHK(launch_topk_sample(target_logits, batch, n, vocab, top_k, (float *)workspace, draft,
                              uniforms, temperature, top_p, accept_len, out_tokens,
                              (hipStream_t)stream));
    return DFLASH_OK;
}

}  // extern "C"

namespace {

bool qgemm_shape_ok(int M, int N, int K) {
    return M >= 1 && M <= 4096 && N >= 16 && N % 16 == 0 && K >= 256 && K % 256 == 0;
}

size_t quant_matrix_bytes(int fmt, int N, int K) {
    if (fmt == DFLASH_W_Q4K) return (size_t)N * (K / 256) * 144;
    if (fmt == DFLASH_W_Q8_0) return (size_t)N * (K / 32) * Q8_BLOCK_BYTES;
    return (size_t)N * K + (size_t)N * 4;                  // FP8: codes, then row scales
}

// y = x . W^T for a tiled Q4_K / Q8_0 / FP8 matrix: product into partials, split sum to bf16
int quant_gemm_tiled(int fmt, const void *w, const uint16_t *x, uint16_t *y, int M, int N, int K,
                     float *part, hipStream_t st) {
    Q4kFusedArgs a;
    a.w[0] = a.w[1] = a.w[2] = (const unsigned char *)w;
    a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = N;
    a.nseg = 1;
    a.M = M; a.N = N; a.KB = K / 256;
    a.src.A = x;
    a.src.lda = K;
    a.part = part;
    a.pair = 0;
    int pair_left;
    const int splits = run_quant(fmt, a, st, &pair_left);
    if (splits < 0) return splits;
    HIPCHK(launch_reduce_epilogue(a.part, splits, M, N, 0, EPI_STORE_BF16, nullptr, y, nullptr, N,
                                  RowScale{}, st));
    return DFLASH_OK;
}

// argument checks shared by the four GEMM entry points
int quant_gemm_check(const void *w, const uint16_t *x, const uint16_t *y, int M, int N, int K,
                     const void *workspace, size_t ws_bytes, size_t need) {
    if (!w || !x || !y) return DFLASH_EINVAL;
    if (!qgemm_shape_ok(M, N, K)) return DFLASH_ESHAPE;
    if (!aligned16(w) || !aligned16(x) || !aligned16(y)) return DFLASH_EALIGN;
    if (!workspace || ws_bytes < need || !aligned16(workspace)) return DFLASH_EWORKSPACE;
    return DFLASH_OK;
}

size_t quant_gemm_tiled_ws(int fmt, int M, int N, int K) {
    if (!qgemm_shape_ok(M, N, K)) return 0;
    return gemm_part_bytes(fmt, M, N, K);
}

// row-major W: the tiled copy first in the workspace, then the partials
size_t quant_gemm_rowmajor_ws(int fmt, int M, int N, int K) {
    if (!qgemm_shape_ok(M, N, K)) return 0;
    return align256(quant_matrix_bytes(fmt, N, K)) + gemm_part_bytes(fmt, M, N, K);
}

int quant_gemm_rowmajor(int fmt, const void *w, const uint16_t *x, uint16_t *y, int M, int N,
                        int K, void *workspace, size_t ws_bytes, hipStream_t st) {
    const int rc = quant_gemm_check(w, x, y, M, N, K, workspace, ws_bytes,
                                    quant_gemm_rowmajor_ws(fmt, M, N, K));
    if (rc != DFLASH_OK) return rc;
    if ((uintptr_t)workspace & 255) return DFLASH_EWORKSPACE;
    unsigned char *tiled = (unsigned char *)workspace;
    const size_t wb = quant_matrix_bytes(fmt, N, K);
    const uintptr_t s0 = (uintptr_t)w, d0 = (uintptr_t)tiled;
    if (s0 < d0 + ws_bytes && d0 < s0 + wb) return DFLASH_EINVAL;      // W inside the workspace
    if (fmt == DFLASH_W_Q4K)
        HIPCHK(launch_q4k_to_tiled((const unsigned char *)w, tiled, N, K / 256, st));
    else if (fmt == DFLASH_W_Q8_0)
        HIPCHK(launch_q8_0_to_tiled((const unsigned char *)w, tiled, N, K / 256, st));
    else
        HIPCHK(launch_fp8_to_tiled((const unsigned char *)w, tiled, N, K / 256, st));
    return quant_gemm_tiled(fmt, tiled, x, y, M, N, K, (float *)(tiled + align256(wb)), st);
}

}  // namespace

extern "C" {

size_t q4k_gemm_workspace_bytes(int M, int N, int K) {
    return quant_gemm_rowmajor_ws(DFLASH_W_Q4K, M, N, K);
}

int q4k_gemm(const void *w, const uint16_t *x, uint16_t *y, int M, int N, int K,
             void *workspace, size_t ws_bytes, void *stream) {
    return quant_gemm_rowmajor(DFLASH_W_Q4K, w, x, y, M, N, K, workspace, ws_bytes,
                               (hipStream_t)stream);
}

size_t q4k_gemm_tiled_workspace_bytes(int M, int N, int K) {
    return quant_gemm_tiled_ws(DFLASH_W_Q4K, M, N, K);
}

int q4k_gemm_tiled(const void *w, const uint16_t *x, uint16_t *y, int M, int N, int K,
                   void *workspace, size_t ws_bytes, void *stream) {
    const int rc = quant_gemm_check(w, x, y, M, N, K, workspace, ws_bytes,
                                    quant_gemm_tiled_ws(DFLASH_W_Q4K, M, N, K));
    if (rc != DFLASH_OK) return rc;
    return quant_gemm_tiled(DFLASH_W_Q4K, w, x, y, M, N, K, (float *)workspace, (hipStream_t)stream);
}

size_t q8_0_gemm_workspace_bytes(int M, int N, int K) {
    return quant_gemm_rowmajor_ws(DFLASH_W_Q8_0, M, N, K);
}

int q8_0_gemm(const void *w, const uint16_t *x, uint16_t *y, int M, int N, int K,
              void *workspace, size_t ws_bytes, void *stream) {
    return quant_gemm_rowmajor(DFLASH_W_Q8_0, w, x, y, M, N, K, workspace, ws_bytes,
                               (hipStream_t)stream);
}

size_t q8_0_gemm_tiled_workspace_bytes(int M, int N, int K) {
    return quant_gemm_tiled_ws(DFLASH_W_Q8_0, M, N, K);
}

int q8_0_gemm_tiled(const void *w, const uint16_t *x, uint16_t *y, int M, int N, int K,
                    void *workspace, size_t ws_bytes, void *stream) {
    const int rc = quant_gemm_check(w, x, y, M, N, K, workspace, ws_bytes,
                                    quant_gemm_tiled_ws(DFLASH_W_Q8_0, M, N, K));
    if (rc != DFLASH_OK) return rc;
    return quant_gemm_tiled(DFLASH_W_Q8_0, w, x, y, M, N, K, (float *)workspace, (hipStream_t)stream);
}

int q8_0_to_tiled(const void *src, void *dst, int N, int K, void *stream) {
    if (!src || !dst) return DFLASH_EINVAL;
    if (N < 16 || N % 16 || K < 256 || K % 256) return DFLASH_ESHAPE;
    if (!aligned16(src) || !aligned16(dst)) return DFLASH_EALIGN;
    const size_t bytes = (size_t)N * (K / 32) * Q8_BLOCK_BYTES;
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
    if (s0 < d0 + bytes && d0 < s0 + bytes) return DFLASH_EINVAL;      // overlap
    HIPCHK(launch_q8_0_to_tiled((const unsigned char *)src, (unsigned char *)dst, N, K / 256,
                                (hipStream_t)stream));
    return DFLASH_OK;
}

int q8_0_dequantize(const void *w, float *out, long long n_blocks, void *stream) {
    if (!w || !out || n_blocks < 1) return DFLASH_EINVAL;
    if (!aligned16(w) || !aligned16(out)) return DFLASH_EALIGN;
    HIPCHK(launch_q8_0_dequant(w, out, n_blocks, (hipStream_t)stream));
    return DFLASH_OK;
}

size_t fp8_gemm_workspace_bytes(int M, int N, int K) {
    return quant_gemm_rowmajor_ws(DFLASH_W_FP8, M, N, K);
}

int fp8_gemm(const void *w, const uint16_t *x, uint16_t *y, int M, int N, int K,
             void *workspace, size_t ws_bytes, void *stream) {
    return quant_gemm_rowmajor(DFLASH_W_FP8, w, x, y, M, N, K, workspace, ws_bytes,
                               (hipStream_t)stream);
}

size_t fp8_gemm_tiled_workspace_bytes(int M, int N, int K) {
    return quant_gemm_tiled_ws(DFLASH_W_FP8, M, N, K);
}

int fp8_gemm_tiled(const void *w, const uint16_t *x, uint16_t *y, int M, int N, int K,
                   void *workspace, size_t ws_bytes, void *stream) {
    const int rc = quant_gemm_check(w, x, y, M, N, K, workspace, ws_bytes,
                                    quant_gemm_tiled_ws(DFLASH_W_FP8, M, N, K));
    if (rc != DFLASH_OK) return rc;
    return quant_gemm_tiled(DFLASH_W_FP8, w, x, y, M, N, K, (float *)workspace, (hipStream_t)stream);
}

int fp8_to_tiled(const void *src, void *dst, int N, int K, void *stream) {
    if (!src || !dst) return DFLASH_EINVAL;
    if (N < 16 || N % 16 || K < 256 || K % 256) return DFLASH_ESHAPE;
    if (!aligned16(src) || !aligned16(dst)) return DFLASH_EALIGN;
    const size_t bytes = quant_matrix_bytes(DFLASH_W_FP8, N, K);
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
    if (s0 < d0 + bytes && d0 < s0 + bytes) return DFLASH_EINVAL;      // overlap
    HIPCHK(launch_fp8_to_tiled((const unsigned char *)src, (unsigned char *)dst, N, K / 256,
                               (hipStream_t)stream));
    return DFLASH_OK;
}

int fp8_dequantize(const void *w, float *out, int N, int K, void *stream) {
    if (!w || !out) return DFLASH_EINVAL;
    if (N < 1 || K < 1 || K % 4 || (long long)N * K > (1LL << 40)) return DFLASH_ESHAPE;
    if (!aligned16(w) || !aligned16(out)) return DFLASH_EALIGN;
    HIPCHK(launch_fp8_dequant(w, out, N, K, (hipStream_t)stream));
    return DFLASH_OK;
}

int q4k_to_tiled(const void *src, void *dst, int N, int K, void *stream) {
    if (!src || !dst) return DFLASH_EINVAL;
    if (N < 16 || N % 16 || K < 256 || K % 256) return DFLASH_ESHAPE;
    if (!aligned16(src) || !aligned16(dst)) return DFLASH_EALIGN;
    const size_t bytes = (size_t)N * (K / 256) * 144;
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
    if (s0 < d0 + bytes && d0 < s0 + bytes) return DFLASH_EINVAL;      // overlap
    HIPCHK(launch_q4k_to_tiled((const unsigned char *)src, (unsigned char *)dst, N, K / 256,
                               (hipStream_t)stream));
    return DFLASH_OK;
}

int q4k_dequantize(const void *w, float *out, long long n_blocks, void *stream) {
    if (!w || !out || n_blocks < 1) return DFLASH_EINVAL;
    if (!aligned16(w) || !aligned16(out)) return DFLASH_EALIGN;
    HIPCHK(launch_q4k_dequant(w, out, n_blocks, (hipStream_t)stream));
    return DFLASH_OK;
}

}  // extern "C"
