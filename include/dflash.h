/*
 * dflash.h - C ABI of the MI355X (gfx950) DFlash 2 block-draft library.
 *
 * The library runs one step of DFlash 2 speculative drafting on one GPU:
 *
 *   dflash_draft_step    the drafter reads five tapped target features, proposes
 *                        a block of 8 tokens in one forward (position 0 = the last
 *                        accepted token, positions 1..7 = mask positions), keeps
 *                        the top-K candidates of the shared output head at each of
 *                        the 7 proposal positions and picks one path through them.
 *                        FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2": spec table
 *                        rows "Draft", "Weights", "Taps"; section "How it is used".
 *   dflash_verify_prefix greedy acceptance: keep the longest drafted prefix the
 *                        target agrees with, plus one target token.  Same card,
 *                        sections "How it is used" and "FastFlowLM measurements".
 *   dflash_verify_sampled
 *                        sampled acceptance: exact rejection sampling of the drafted
 *                        tokens against the target's temperature / top-k / top-p
 *                        distribution.  Mindket kit page "Qwen3.8-27B-DFlash2-GGUF by
 *                        z-lab", sections "For newcomers and experts" and "Good to
 *                        know".
 *   q4k_gemm             y = x . W^T with W in Q4_K super-blocks (the format of
 *                        the draft's fc, q/k/v/o and MLP matrices: same card,
 *                        "Weights" row), fp32 accumulation, bf16 output; W row-major
 *                        as in a GGUF file (q4k_gemm_tiled: W in the tiled layout).
 *   q8_0_gemm            the same product with W in Q8_0 blocks (the pages' second
 *                        quantised draft file: Mindket kit page "Qwen3.8-27B-DFlash2-
 *                        GGUF by z-lab", draft-file table); q8_0_to_tiled and
 *                        q8_0_dequantize as for Q4_K.
 *   fp8_gemm             the same product with W as FP8 (E4M3) codes and one scale
 *                        per row (aiqre model page "Qwen3.8-27B-DFlash2", "Memory":
 *                        an fp8 format at one byte per parameter); fp8_to_tiled and
 *                        fp8_dequantize as for Q4_K.
 *   q4k_to_tiled         regroups a row-major Q4_K matrix into the tiled device
 *                        layout every Q4_K entry point above reads (done once, when
 *                        the weights are loaded).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE memory owned by the caller.  The library
 *     allocates nothing, keeps no state between calls and writes only the
 *     buffers documented as outputs, the caller's workspace and the KV-cache rows
 *     named below.
 *   - bf16 tensors are passed as uint16_t bit patterns; all arrays are dense and
 *     row-major in the order their shapes are written.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *     work and return; results are valid once the stream has reached them.
 *   - Arguments are validated on the host before anything is enqueued: a
 *     negative dflash_status is returned and nothing is launched.  A HIP launch
 *     error after validation returns DFLASH_EHIP.  Nothing is thrown across the
 *     ABI.  Calls on distinct workspaces may run concurrently.
 *   - Values held in device memory (token ids, context lengths) cannot be seen
 *     by the host check; the kernels guard every access against them (see each
 *     entry point).
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_MAX_LAYERS 8
#define DFLASH_BLOCK 8          /* the drafter's block: 1 anchor + 7 proposals; also the
                                   largest block and t_new the kernels take */
#define DFLASH_MAX_TOPK 16
#define DFLASH_SAMPLE_MAX_N 63          /* dflash_verify_sampled: drafted tokens per row */
#define DFLASH_SAMPLE_MAX_TOPK 64       /* dflash_verify_sampled: target top_k */
#define DFLASH_SAMPLE_MAX_VOCAB (1 << 20)

typedef enum {
    DFLASH_OK = 0,
    DFLASH_EINVAL = -1,       /* null pointer or value out of range */
    DFLASH_ESHAPE = -2,       /* shape not supported by the kernels */
    DFLASH_EALIGN = -3,       /* pointer misaligned (16-byte alignment required) */
    DFLASH_EWORKSPACE = -4,   /* workspace missing or too small */
    DFLASH_EHIP = -5,         /* a HIP call failed */
    DFLASH_ELAYOUT = -6,      /* quantised weights not declared in the tiled layout */
    DFLASH_ESCRATCH = -7      /* the request needs more than the static scratch holds */
} dflash_status;

/* Layout tag of the quantised linear weights in dflash_weights.linear_layout.  The
 * draft step reads Q4_K, Q8_0 and FP8 matrices only in the tiled layouts written by
 * q4k_to_tiled / q8_0_to_tiled / fp8_to_tiled; the caller states that it converted them by setting
 * the tag to DFLASH_LAYOUT_TILED (a zero-initialised struct says row-major, and a
 * step with quantised weights then returns DFLASH_ELAYOUT instead of reading
 * row-major bytes as tiled ones).  bf16 weights are row-major and ignore the tag. */
#define DFLASH_LAYOUT_ROWMAJOR 0u
#define DFLASH_LAYOUT_TILED 0x444C4954u     /* "TILD" */

typedef enum { DFLASH_W_Q4K = 0, DFLASH_W_BF16 = 1, DFLASH_W_Q8_0 = 2, DFLASH_W_FP8 = 3 } dflash_weight_fmt;

/* Drafter shape.  The 27B draft: 5 layers, hidden 5120, FFN 17408, 32 query and
 * 8 KV heads of 128, window 2048, vocab 248320, 5 taps, block 8, top 16, rank
 * 256 (FastFlowLM card spec table "Draft" row; aiqre page "Specification").
 * Supported by the kernels: hidden, ffn and n_q*head_dim multiples of 256; hidden
 * and n_q*head_dim at most 8192; head_dim 64 or 128; n_q even, at most 64 and a
 * multiple of n_kv with n_q / n_kv <= 4; 2 <= block <= 8 (P = block - 1 proposals;
 * the JetBrains card "Qwen3.8-3.6-27B-blend DFlash2", "Quick start", runs a quantized
 * drafter with block size 5); 1 <= top_k <= 16; sel_rank a multiple of 32 up to 4096;
 * vocab >= top_k, a multiple of 16, at most 1,048,576; window at most 65536. */
typedef struct {
    int n_layers, hidden, ffn, n_q_heads, n_kv_heads, head_dim, window, vocab;
    int n_taps, block, top_k, sel_rank, weight_fmt;
    float rms_eps;     /* RMSNorm epsilon (1e-6) */
    float rope_theta;  /* rotary base */
    float pair_scale;  /* selector pair-score scale, 1/sqrt(sel_rank) */
} dflash_config;

/* Linear weights are [out][in] (y = x . W^T).  bf16: row-major, `in` values per
 * row.  Q4_K / Q8_0 / FP8: the tiled layouts written by q4k_to_tiled / q8_0_to_tiled /
 * fp8_to_tiled (the row-major matrix regrouped; same size), declared by linear_layout. */
typedef struct {
    const void *wq, *wk, *wv, *wo, *wg, *wu, *wd;
    const uint16_t *in_norm, *post_norm;   /* [hidden] */
    const uint16_t *q_norm, *k_norm;       /* [head_dim], per-head RMSNorm gains */
    const uint16_t *w_conv;                /* [2 n_q][n_q head_dim] dynamic-conv taps */
} dflash_layer_weights;

typedef struct {
    const void *fc;                        /* [hidden][n_taps hidden] */
    const uint16_t *hidden_norm;           /* [hidden] norm of the fused taps */
    dflash_layer_weights layer[DFLASH_MAX_LAYERS];
    const uint16_t *final_norm;            /* [hidden] */
    const uint16_t *embed;                 /* [vocab][hidden] target embedding table */
    const uint16_t *lm_head;               /* [vocab][hidden] target output head (may alias embed) */
    const uint16_t *mask_emb;              /* [hidden] embedding of the mask positions */
    const uint16_t *sel_proj;              /* [sel_rank][hidden] selector projection (not read) */
    const uint16_t *code_a, *code_b;       /* [vocab][sel_rank] selector codebooks */
    uint32_t linear_layout;                /* DFLASH_LAYOUT_TILED (required for Q4_K / Q8_0 / FP8) */
} dflash_weights;

/* Optional live timing of one kernel inside dflash_draft_step: HIP events
 * recorded on `stream` immediately before and after that kernel's launch. */
typedef enum { DFLASH_PROBE_NONE = 0, DFLASH_PROBE_LM_HEAD = 1, DFLASH_PROBE_FFN_GATE_UP = 2 } dflash_probe_kernel;
typedef struct {
    int kernel;            /* dflash_probe_kernel */
    int layer;             /* layer index for per-layer kernels */
    void *ev_start, *ev_stop;   /* hipEvent_t */
} dflash_probe;

/* Bytes of workspace dflash_draft_step needs for (cfg, batch, t_new); 0 on bad
 * arguments. */
size_t dflash_workspace_bytes(const dflash_config *cfg, int batch, int t_new);

/*
 * One draft step for `batch` independent sequences.
 *
 *  taps         bf16 [batch][t_new][n_taps*hidden]: the target's residual stream
 *               at its tapped layers for the t_new newest context positions,
 *               concatenated in the listed layer order (FastFlowLM card "Taps").
 *  t_new        1..8 context rows appended this step.
 *  last_token   int32 [batch] device: last accepted token (block position 0).
 *  ctx_len      int32 [batch] device: rows already cached before the step (n).
 *  k_cache,     bf16 [n_layers][batch][n_kv][cache_cap][head_dim] device.
 *  v_cache      Rows [n, n+t_new) are written (keys after per-head norm and
 *               rotary embedding at positions n..n+t_new-1; values as projected);
 *               rows [max(0, n+t_new-window), n) are read.  Block position t
 *               sits at rotary position n+t_new+t.
 *  draft_tokens int32 [batch][P]: the chosen path, P = block - 1 (7 for the 27B draft).
 *  cand_ids     int32 [batch][P][top_k], cand_logp fp32 [batch][P][top_k]:
 *               candidates ordered by (logit desc, id asc) and their log-softmax.
 *  dbg_hidden   nullable fp32 [n_layers+1][batch][block][hidden]: the residual stream
 *               after block assembly and after each layer.
 *  dbg_logits   nullable fp32 [batch][P][vocab].
 *  workspace    device, >= dflash_workspace_bytes(cfg, batch, t_new), 256-byte aligned.
 *  probe        nullable; see dflash_probe.
 *
 * A sequence whose ctx_len is negative or whose n+t_new exceeds cache_cap, or
 * whose last_token is outside [0, vocab), is not computed: its draft tokens are
 * set to -1, its candidates to -1 / -inf, and no cache row is written.
 */
int dflash_draft_step(const dflash_config *cfg, const dflash_weights *w, int batch,
                      const uint16_t *taps, int t_new, const int32_t *last_token,
                      const int32_t *ctx_len, uint16_t *k_cache, uint16_t *v_cache,
                      int cache_cap, int32_t *draft_tokens, int32_t *cand_ids,
                      float *cand_logp, float *dbg_hidden, float *dbg_logits,
                      void *workspace, size_t ws_bytes, const dflash_probe *probe,
                      void *stream);

/*
 * dflash_draft_step without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The step's workspace is a static device array of
 * DFLASH_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until
 * the process ends (the GPU is the device of `stream`, or the current device for the
 * NULL stream).  The call itself allocates nothing.  Arguments and results are those
 * of dflash_draft_step (no probe).  A configuration whose workspace
 * (dflash_workspace_bytes) exceeds the array returns DFLASH_ESCRATCH before anything
 * is launched; the 27B-draft shape at batch 1 fits (23.3 MiB).  Every call on one GPU
 * uses the same array, which keeps the last call's contents (nothing in it needs to
 * start at zero): calls that overlap on one GPU (other streams, other threads) race
 * and must be serialised by the caller.
 */
#define DFLASH_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int dflash_draft_step_noalloc(const dflash_config *cfg, const dflash_weights *w, int batch,
                              const uint16_t *taps, int t_new, const int32_t *last_token,
                              const int32_t *ctx_len, uint16_t *k_cache, uint16_t *v_cache,
                              int cache_cap, int32_t *draft_tokens, int32_t *cand_ids,
                              float *cand_logp, float *dbg_hidden, float *dbg_logits,
                              void *stream);

/*
 * Greedy prefix acceptance for `batch` rows.
 *  draft      int32 [batch][n] drafted tokens (n = 7 for a block of 8).
 *  target     int32 [batch][n+1]: target[j] is the target's greedy token after
 *             block position j.
 *  accept_len int32 [batch]: k = number of leading j with draft[j] == target[j].
 *  out_tokens int32 [batch][n+1]: draft[0..k-1], target[k], then -1.
 * 1 <= n <= 64.
 */
int dflash_verify_prefix(const int32_t *draft, const int32_t *target, int batch, int n,
                         int32_t *accept_len, int32_t *out_tokens, void *stream);

/* Workspace bytes dflash_verify_sampled needs (0 if the shape is not supported). */
size_t dflash_verify_sampled_workspace_bytes(int batch, int n, int vocab);

/*
 * Sampled acceptance for `batch` rows: exact rejection sampling of the drafted tokens
 * against the target's sampling distribution (Mindket kit page "Qwen3.8-27B-DFlash2-GGUF
 * by z-lab": "For newcomers and experts", sampling keeps the target's distribution;
 * "Good to know", temperature 1.0, top-p 0.95, top-k 20).
 *  draft         int32 [batch][n] drafted tokens (the selector's path).
 *  target_logits fp32 [batch][n+1][vocab]: row j holds the target's logits after block
 *                position j (position 0 = the last accepted token).
 *  uniforms      fp32 [batch][n+1][2] in [0, 1): [j][0] decides acceptance of draft[j],
 *                [j][1] draws the token emitted at j (after a rejection, or the bonus
 *                token at j = n).
 *  p_j           target distribution of row j: logits / temperature, the top_k largest
 *                (ties: lowest id first), softmax over those, then the smallest prefix
 *                in (probability desc, id asc) order whose mass reaches top_p,
 *                renormalised.
 *  procedure     for j = 0..n-1: accept draft[j] when uniforms[j][0] < p_j(draft[j]);
 *                otherwise emit a token drawn from p_j with draft[j] removed and stop.
 *                When all n are accepted, emit a token drawn from p_n.  A draw takes the
 *                first token (same order) whose cumulative weight exceeds u times the
 *                total weight.  The proposals are deterministic, so the proposal
 *                distribution is a point mass; each emitted token then follows p_j
 *                given the tokens before it.
 *  accept_len    int32 [batch]: k, the number of accepted drafted tokens.
 *  out_tokens    int32 [batch][n+1]: draft[0..k-1], the emitted token, then -1.
 *  workspace     device, >= dflash_verify_sampled_workspace_bytes(batch, n, vocab),
 *                16-byte aligned.
 * 1 <= n <= DFLASH_SAMPLE_MAX_N, 1 <= top_k <= min(vocab, DFLASH_SAMPLE_MAX_TOPK),
 * 0 < top_p <= 1, temperature > 0 and finite, vocab <= DFLASH_SAMPLE_MAX_VOCAB,
 * batch * (n+1) <= 65535; int32 / fp32 pointers 4-byte aligned.  Each row needs a
 * finite maximum.  A drafted token outside [0, vocab) has probability 0 (rejected).
 * The probabilities are computed in fp32: a decision whose threshold lies within
 * fp32 rounding of the uniform may differ from an exact-arithmetic evaluation.
 */
int dflash_verify_sampled(const int32_t *draft, const float *target_logits,
                          const float *uniforms, int batch, int n, int vocab,
                          float temperature, int top_k, float top_p, void *workspace,
                          size_t workspace_bytes, int32_t *accept_len, int32_t *out_tokens,
                          void *stream);

/* Workspace bytes q4k_gemm needs for an M x N x K product (the tiled copy of W plus
 * the split-K partial sums); 0 if the shape is not supported. */
size_t q4k_gemm_workspace_bytes(int M, int N, int K);

/*
 * y[M][N] (bf16) = x[M][K] (bf16) . W^T, W [N][K] in Q4_K as stored in a GGUF file:
 * row-major, each row K/256 consecutive 144-byte super-blocks (fp16 d, fp16 dmin, 12
 * bytes of 6-bit scales and mins, 128 quant bytes; w = d sc_j q - dmin m_j for
 * sub-block j), fp32 accumulation.  FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2",
 * "Weights" row.  The call regroups W into the tiled layout inside its workspace
 * (q4k_to_tiled) and runs q4k_gemm_tiled; a caller that multiplies by one matrix
 * many times converts it once and calls q4k_gemm_tiled.
 * K % 256 == 0, N % 16 == 0, 1 <= M <= 4096.  w, x, y and workspace 16-byte aligned.
 */
int q4k_gemm(const void *w, const uint16_t *x, uint16_t *y, int M, int N, int K,
             void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes q4k_gemm_tiled needs for an M x N x K product; 0 if unsupported. */
size_t q4k_gemm_tiled_workspace_bytes(int M, int N, int K);

/*
 * The product of q4k_gemm with W already in the tiled layout of q4k_to_tiled (the
 * layout the draft step reads).  Up to 16 rows with K % 1024 == 0 every product
 * d sc_j q and dmin m_j enters the sum exactly; otherwise each decoded weight enters
 * as two bf16 terms whose sum is within 2^-18 of it (below fp32 accumulation error).
 * Same shape and alignment rules as q4k_gemm.
 */
int q4k_gemm_tiled(const void *w_tiled, const uint16_t *x, uint16_t *y, int M, int N, int K,
                   void *workspace, size_t ws_bytes, void *stream);

/*
 * Tiled Q4_K layout (FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", "Weights" row, for
 * the Q4_K format itself).  src: a row-major Q4_K matrix [N][K] (each row K/256
 * super-blocks of 144 bytes: fp16 d, fp16 dmin, 12 scale bytes, 128 quant bytes read
 * as 4 chunks of 32).  dst (same size, N K / 256 * 144 bytes) receives, for every
 * 16-row tile t and super-block kb, one 2304-byte unit at (t K/256 + kb) 2304:
 *   bytes [0, 256): the 16 block headers, row 16 t + r at 16 r;
 *   bytes 256 + 1024 h + 16 (16 g + r) .. + 15 (h < 2, g < 4, r < 16): quant bytes
 *   8 g .. 8 g + 7 of chunk 2 h, then of chunk 2 h + 1, of row 16 t + r's block.
 * Every byte is copied, none changed.  N % 16 == 0, K % 256 == 0, both > 0; src and
 * dst device pointers, 16-byte aligned, not overlapping.  Enqueued on `stream`.
 */
int q4k_to_tiled(const void *src, void *dst, int N, int K, void *stream);

/*
 * Q8_0 (Mindket kit page "Qwen3.8-27B-DFlash2-GGUF by z-lab": the draft-file table lists
 * a Q8_0 file; the bytes are the GGUF Q8_0 block): 34 bytes per 32 consecutive weights
 * of a row, fp16 scale d (little endian) then 32 signed bytes q; w = d q.  A row-major
 * matrix [N][K] is N rows of K/32 blocks.  With weight_fmt DFLASH_W_Q8_0 the draft
 * step's fc, q/k/v/o and MLP matrices are Q8_0 in the tiled layout below.
 *
 * q8_0_to_tiled: src row-major Q8_0 [N][K] -> dst (same size, N K / 32 * 34 bytes): for
 * every 16-row tile t and 256-wide K-group g one 4352-byte unit at (t K/256 + g) 4352:
 *   bytes [0, 256): the 8 block scales of row 16 t + r (fp16, block order) at 16 r;
 *   bytes 256 + 1024 p + 16 (16 h + r) .. + 15 (p, h < 4, r < 16): quant bytes
 *   8 h .. 8 h + 7 of block 8 g + 2 p of row 16 t + r, then of block 8 g + 2 p + 1.
 * Every byte is copied, none changed.  N % 16 == 0, K % 256 == 0, both > 0; device
 * pointers, 16-byte aligned, not overlapping.
 */
int q8_0_to_tiled(const void *src, void *dst, int N, int K, void *stream);

/* Workspace bytes q8_0_gemm needs for an M x N x K product (the tiled copy of W
 * plus the split-K partial sums); 0 if the shape is not supported. */
size_t q8_0_gemm_workspace_bytes(int M, int N, int K);

/*
 * y[M][N] (bf16) = x[M][K] (bf16) . W^T, W [N][K] in row-major Q8_0 (GGUF blocks, see
 * above), fp32 accumulation.  The call regroups W into the tiled layout inside its
 * workspace and runs q8_0_gemm_tiled.
 * K % 256 == 0, N % 16 == 0, 1 <= M <= 4096.  w, x, y and workspace 16-byte aligned.
 */
int q8_0_gemm(const void *w, const uint16_t *x, uint16_t *y, int M, int N, int K,
              void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes q8_0_gemm_tiled needs for an M x N x K product; 0 if unsupported. */
size_t q8_0_gemm_tiled_workspace_bytes(int M, int N, int K);

/*
 * The product of q8_0_gemm with W in the tiled layout of q8_0_to_tiled.  Up to 16 rows
 * with K % 1024 == 0 the products d q enter the sum exactly; otherwise each decoded
 * weight d q enters as two bf16 terms whose sum is within 2^-18 of it.
 */
int q8_0_gemm_tiled(const void *w_tiled, const uint16_t *x, uint16_t *y, int M, int N, int K,
                    void *workspace, size_t ws_bytes, void *stream);

/* Decode n_blocks consecutive row-major Q8_0 blocks to fp32 (32 values each, exact). */
int q8_0_dequantize(const void *w, float *out, long long n_blocks, void *stream);

/*
 * FP8 (aiqre model page "Qwen3.8-27B-DFlash2", "Memory": besides bf16 and int4 the
 * drafter's weights come in an fp8 format at one byte per parameter, 1.8 GiB; the page
 * names no encoding).  Read as OCP FP8 E4M3: sign, 4 exponent bits of bias 7, 3 mantissa
 * bits, no infinities, codes 0x7F / 0xFF NaN, largest finite 448; one fp32 scale per
 * output row.  A row-major matrix [N][K] is its N K codes in row order (row n at byte
 * n K), then N little-endian fp32 scales at byte N K: w[n][k] = s[n] e4m3(code[n][k]).
 * With weight_fmt DFLASH_W_FP8 the draft step's fc, q/k/v/o and MLP matrices are FP8
 * in the tiled layout below.  Every E4M3 value is exact in bf16, so the GEMMs multiply
 * the codes' values exactly and apply the row scale to the fp32 sum.
 *
 * fp8_to_tiled: src row-major FP8 [N][K] -> dst (same size, N K + 4 N bytes): for every
 * 16-row tile t and 256-wide K-group g one 4096-byte unit at (t K/256 + g) 4096:
 *   bytes 1024 p + 16 (16 h + r) .. + 15 (p, h < 4, r < 16): codes 64 p + 8 h .. + 7 of
 *   row 16 t + r's K-group g, then its codes 64 p + 32 + 8 h .. + 7;
 * then the N scales at byte N K, unchanged.  Every byte is copied, none changed.
 * N % 16 == 0, K % 256 == 0, both > 0; device pointers, 16-byte aligned, not overlapping.
 */
int fp8_to_tiled(const void *src, void *dst, int N, int K, void *stream);

/* Workspace bytes fp8_gemm needs for an M x N x K product (the tiled copy of W plus
 * the split-K partial sums); 0 if the shape is not supported. */
size_t fp8_gemm_workspace_bytes(int M, int N, int K);

/*
 * y[M][N] (bf16) = x[M][K] (bf16) . W^T, W [N][K] in row-major FP8 (see above), fp32
 * accumulation.  The call regroups W into the tiled layout inside its workspace and
 * runs fp8_gemm_tiled.  K % 256 == 0, N % 16 == 0, 1 <= M <= 4096.  w, x, y and
 * workspace 16-byte aligned.  A NaN code gives NaN outputs in its row's column.
 */
int fp8_gemm(const void *w, const uint16_t *x, uint16_t *y, int M, int N, int K,
             void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes fp8_gemm_tiled needs for an M x N x K product; 0 if unsupported. */
size_t fp8_gemm_tiled_workspace_bytes(int M, int N, int K);

/* The product of fp8_gemm with W in the tiled layout of fp8_to_tiled. */
int fp8_gemm_tiled(const void *w_tiled, const uint16_t *x, uint16_t *y, int M, int N, int K,
                   void *workspace, size_t ws_bytes, void *stream);

/* Decode a row-major FP8 matrix [N][K] to fp32: out[n K + k] = s[n] e4m3(code), the exact
 * product rounded once to fp32.  N, K >= 1, K % 4 == 0; 16-byte aligned pointers. */
int fp8_dequantize(const void *w, float *out, int N, int K, void *stream);

/* Decode n_blocks consecutive row-major Q4_K super-blocks to fp32 (256 values each). */
int q4k_dequantize(const void *w, float *out, long long n_blocks, void *stream);

/* Text of a dflash_status code. */
const char *dflash_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
