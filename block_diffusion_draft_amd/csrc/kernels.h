// Launch interface of the draft-step kernels (host side of each .hip file).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

// ---------------------------------------------------------------- Q4_K decode
hipError_t launch_q4k_dequant(const void *w, float *out, long long n_blocks, hipStream_t st);
// Row-major Q4_K [N rows][K/256 blocks] -> the tiled layout the GEMM kernels stream:
// unit (t, kb) of 2304 bytes at (t * K/256 + kb) * 2304 holds the 16 block headers of
// rows 16 t .. 16 t + 15 (16 bytes each), then two halves h of 64 slots s = 16 g + r
// (16 bytes each): quant bytes 8 g .. 8 g + 7 of chunk 2 h, then of chunk 2 h + 1, of
// row r's block (chunk c = quant bytes 32 c .. 32 c + 31).
constexpr int Q4K_UNIT_BYTES = 2304;
hipError_t launch_q4k_to_tiled(const unsigned char *src, unsigned char *dst, int N, int KB,
                               hipStream_t st);

// ---------------------------------------------------------------- bf16 GEMMs
struct Bf16GemmArgs {
    const uint16_t *w[3];        // bf16 weights [N_seg][K], stacked along N
    int seg_end[3];
    int nseg;
    const uint16_t *A;           // bf16 [M][lda]
    int lda;
    int M, N, K;
    float *C;                    // fp32 [M][ldc]
    int ldc;
    RowScale rs;                 // output row r multiplied by row_inv(rs, r) (ssq null: none)
    float *rstat;                // nullable (skinny head only): per output row and column
                                 // run, the run's max and sum of exp(value - max)
};
// tiled 128x128 MFMA GEMM, any M
hipError_t launch_bf16_gemm_tiled(const Bf16GemmArgs &a, hipStream_t st);
// rows <= 8, one weight matrix (nseg == 1), K a multiple of 256 (else
// hipErrorInvalidValue): activations resident in LDS, every wave streams whole weight tiles
hipError_t launch_bf16_gemm_skinny(const Bf16GemmArgs &a, hipStream_t st);
// Column runs of the skinny head's softmax statistics for an N x K head: wave w of the
// streaming head kernel's nrun waves covers the 16-column tiles [w T / nrun, (w + 1) T /
// nrun) of the T = run_tiles tiles (at most run_cols columns, a power of two) and, given
// a.rstat, writes per row r the pair (max, sum exp(v - max)) of its run at
// rstat[2 (r nrun + w)].  run_cols 0: the streaming head does not take the shape.
void head_runs(int N, int K, int *nrun, int *run_cols, int *run_tiles);

// ---------------------------------------------------------------- layer ops
enum EpiMode { EPI_STORE_F32 = 0, EPI_ADD_F32 = 1, EPI_SWIGLU_BF16 = 2, EPI_STORE_BF16 = 3 };
// out row r = sum over splits of partial rows r (+ r + pair), times row_inv(rs, r);
// SWIGLU writes bf16 hi (and lo when out_bf16_lo) of silu(gate) * up, gate in columns
// [0, N/2)
hipError_t launch_reduce_epilogue(const float *part, int splits, int M, int N, int pair,
                                  int mode, float *out_f32, uint16_t *out_bf16,
                                  uint16_t *out_bf16_lo, int ldo, const RowScale &rs,
                                  hipStream_t st);

// SwiGLU of a [gate | up] product's split partials (N = 2F columns, rows r and r + pair
// summed): out = bf16 hi / lo of silu(g * inv) * (u * inv), inv = row_inv(rs, r)
hipError_t launch_swiglu(const float *part, int splits, int M, int N, int pair, uint16_t *out,
                         uint16_t *out_lo, int ldo, const RowScale &rs, hipStream_t st);

// per-sequence validity flags + block assembly h[b][0] = E[last], h[b][1..] = mask, and
// the first layer's input x = bf16(h * gain), [B*T][H], with its row sums of squares
// in ssq[row][0] (ssq[row][1 .. H/256) = 0)
struct EmbedArgs {
    const uint16_t *embed, *mask;
    const int32_t *last, *ctx_len;
    int T, H, V, t_new, cap;
    float *h;
    const uint16_t *gain;
    uint16_t *x;
    float *ssq;
    int32_t *valid;
};
hipError_t launch_embed(const EmbedArgs &a, int B, hipStream_t st);

struct RopeArgs {
    const float *qkv;            // fp32 partials [splits][B*(T + t_new)][qd + 2 kd]: block rows
                                 // then context rows, summed here in split order
    int splits;
    int B, T, t_new, n_q, n_kv, d;
    RowScale blk, ctx;           // deferred input norms of the block rows and context rows
    const uint16_t *q_norm, *k_norm;
    float eps;
    double log2_theta;           // log2 of the rotary base
    const int32_t *ctx_len, *valid;
    uint16_t *Q, *Kb, *Vb;       // bf16 [B][T][heads][d]
    uint16_t *k_cache, *v_cache; // layer base, [B][n_kv][cap][d]
    int cap;
};
hipError_t launch_qk_norm_rope(const RopeArgs &a, hipStream_t st);

struct AttnArgs {
    const uint16_t *Q, *Kb, *Vb;
    const uint16_t *k_cache, *v_cache;   // layer base, [B][n_kv][cap][d]
    const int32_t *ctx_len, *valid;
    int B, T, t_new, n_q, n_kv, d, window, cap;
    int chunk;                   // keys per workgroup (multiple of 64)
    int n_chunks;                // cache chunks per sequence (max); grid.x = n_chunks + 1
    float *O;                    // fp32 [B][n_kv][n_chunks+1][QR][d] unnormalised
    float *ml;                   // fp32 [B][n_kv][n_chunks+1][QR][2] (max, sum)
};
hipError_t launch_attention(const AttnArgs &a, hipStream_t st);

struct MergeConvArgs {
    const float *O, *ml;
    const int32_t *ctx_len, *valid;
    int B, T, t_new, n_q, n_kv, d, window, chunk, n_chunks;
    const uint16_t *w_conv;      // bf16 [2 n_q][n_q d]
    float *o;                    // fp32 [B*T][n_q d] merged attention output
    float *zp;                   // fp32 [B][n_q][d/32][T][2 n_q] conv-tap partials per 32-column slice
    uint16_t *Y;                 // bf16 [B*T][n_q d]
};
hipError_t launch_merge_conv(const MergeConvArgs &a, hipStream_t st);

// ---------------------------------------------------------------- LM head / top-K / path
// Log-softmax statistics and top-K per row of fp32 logits [B P][V] (ids by logit desc,
// id asc; logp = logit - logsumexp), then per sequence the Viterbi path through its P
// rows of candidates (pair score pair_scale <A[u], B[v]>); invalid sequences get -1 /
// -inf candidates and -1 tokens.  ws: topk_workspace_floats(B P, V) floats.  P, K <= 16.
size_t topk_workspace_floats(int R, int V);
hipError_t launch_topk_path(const float *logits, int B, int P, int V, int K, const int32_t *valid,
                            float *ws, const uint16_t *code_a, const uint16_t *code_b, int r,
                            float pair_scale, int32_t *cand_ids, float *cand_logp,
                            int32_t *draft_tokens, hipStream_t st);
// The same selection and path from the head's column-run statistics: one launch; per
// row the threshold and logsumexp come from the runs' (max, sum) pairs and only the runs
// whose max reaches the threshold are read back.  run_tiles 0: run w is columns
// [w run_cols, (w + 1) run_cols); run_tiles T > 0: the balanced runs of head_runs (run w
// is the 16-column tiles [w T / nrun, (w + 1) T / nrun), at most run_cols columns).
// ws: as above.
hipError_t launch_topk_path_runs(const float *logits, const float *rstat, int nrun, int run_cols,
                                 int run_tiles, int B, int P, int V, int K, const int32_t *valid,
                                 float *ws,
                                 const uint16_t *code_a, const uint16_t *code_b, int r,
                                 float pair_scale, int32_t *cand_ids, float *cand_logp,
                                 int32_t *draft_tokens, hipStream_t st);

// Sampled acceptance of B sequences of n drafted tokens against target logits
// [B][n + 1][V]: top-K of every row (the same threshold passes), then per sequence the
// rejection-sampling walk (uniform draws u [B][n + 1][2]).  ws: topk_workspace_floats(
// B (n + 1), V) floats.  n + 1 <= 64, K <= 64, K <= V.
hipError_t launch_topk_sample(const float *logits, int B, int n, int V, int K, float *ws,
                              const int32_t *draft, const float *u, float temperature, float top_p,
                              int32_t *accept_len, int32_t *out_tokens, hipStream_t st);

// ---------------------------------------------------------------- verify
hipError_t launch_verify(const int32_t *draft, const int32_t *target, int B, int n,
                         int32_t *accept_len, int32_t *out_tokens, hipStream_t st);

// ---------------------------------------------------------------- fused Q4_K GEMM
// Activation source of a fused Q4_K GEMM: bf16 rows A[r][lda] (r < M).
struct Q4kSrc {
    const uint16_t *A;
    int lda;
};
struct Q4kFusedArgs {
    const unsigned char *w[3];
    int seg_end[3];
    int nseg;
    int M, N, KB;                // GEMM rows, columns, K/256
    Q4kSrc src;
    float *part;                 // [splits][M][N], or [splits][pair][N] when combined
    int pair;                    // > 0: rows r and r + pair are the (hi, lo) halves of one row
};
// Streaming variant for M <= 16 rows and K/256 a multiple of 4: splits of 4 super-blocks,
// each wave streams tpw consecutive column tiles.  Partials [splits][M][N]; when
// pair is 4 or 8 and M = 2 pair, the kernel adds each (hi, lo) row pair itself and
// writes [splits][pair][N] (pair_done).
struct Q4kStreamPlan {
    int splits, tpw, grid_x;
    int wpg;                     // waves per workgroup
    int px;                      // lane distance of the row pair (16, 32) or 0
    bool pair_done;
    size_t lds_bytes, part_bytes;
};
bool q4k_stream_ok(int M, int N, int K);
// target_waves: about that many waves in all.  4096 (two 8-wave workgroups per CU) was
// measured 0.4% faster on the batch-1 step than 2048 with the loads two stages ahead;
// 3072 leaves the CUs unevenly loaded (3% slower).
Q4kStreamPlan q4k_stream_plan(int M, int N, int K, int pair = 0, int target_waves = 4096,
                              int wpg = 0);
hipError_t launch_q4k_stream(const Q4kFusedArgs &a, const Q4kStreamPlan &p, hipStream_t st);

// Output rows r < M_out: v = sum over splits of partial rows r (+ r + pair), N a multiple
// of 256; add ? f[r] += v : f[r] = v (fp32), with per-256-column sums of squares in
// ssq [M_out][N/256].  Then, if out: bf16(v * gain) (and its residual in out_lo) at
// output row map(r): map 0 -> r; map T > 1 -> the proposal rows of each block of T
// (row r % T == 0 skipped, others to (r / T) (T - 1) + r % T - 1).  The consumer
// applies the row's 1 / rms (RowScale).
struct ReduceRowsArgs {
    const float *part;
    int splits, M_out, N, pair, add;
    float *f, *ssq;
    const uint16_t *gain;
    uint16_t *out, *out_lo;
    int ldo, map;
};
hipError_t launch_reduce_norm(const ReduceRowsArgs &a, hipStream_t st);
hipError_t launch_reduce_norm(const float *part, int splits, int M_out, int N, int pair, int add,
                              float *f, float *ssq, const uint16_t *gain, uint16_t *out,
                              uint16_t *out_lo, int ldo, int map, hipStream_t st);
// the reduction and the block assembly (independent) as one launch
hipError_t launch_reduce_norm_embed(const ReduceRowsArgs &a, const EmbedArgs &e, int B,
                                    hipStream_t st);

// ---------------------------------------------------------------- Q8_0
// Row-major Q8_0 (34-byte blocks of 32 weights: fp16 d, 32 signed bytes) and the
// tiled layout the GEMM kernels read: unit (t, g) of 4352 bytes at (t K/256 + g) 4352
// holds the 8 block scales of rows 16 t .. 16 t + 15 (16 bytes each), then per block
// pair p < 4 the 16-byte slots 16 h + r: bytes 8 h .. 8 h + 7 of block 8 g + 2 p of
// row r, then of block 8 g + 2 p + 1.
constexpr int Q8_BLOCK_BYTES = 34;
constexpr int Q8_UNIT_BYTES = 4352;
hipError_t launch_q8_0_dequant(const void *w, float *out, long long n_blocks, hipStream_t st);
hipError_t launch_q8_0_to_tiled(const unsigned char *src, unsigned char *dst, int N, int G,
                                hipStream_t st);
// streaming GEMM for M <= 16 rows, K a multiple of 1024 (splits of 4 K-groups), the same
// plan fields and partial layout as the Q4_K streaming kernel (a.KB = K / 256)
bool q8_stream_ok(int M, int N, int K);
// (2048 waves: 4096 measured 0.3% slower on the batch-1 step)
Q4kStreamPlan q8_stream_plan(int M, int N, int K, int pair = 0, int target_waves = 2048,
                             int wpg = 0);
hipError_t launch_q8_stream(const Q4kFusedArgs &a, const Q4kStreamPlan &p, hipStream_t st);

// ---------------------------------------------------------------- FP8 (E4M3)
// Row-major FP8 matrix: N K E4M3 codes (row n at n K), then N fp32 row scales; tiled
// layout: unit (t, g) of 4096 bytes at (t K/256 + g) 4096 holds per pair p < 4 the
// 16-byte slots 16 h + r: codes 64 p + 8 h .. + 7 of row 16 t + r's K-group g, then
// codes 64 p + 32 + 8 h .. + 7; the scales follow the codes unchanged.
constexpr int FP8_UNIT_BYTES = 4096;
hipError_t launch_fp8_dequant(const void *w, float *out, int N, int K, hipStream_t st);
hipError_t launch_fp8_to_tiled(const unsigned char *src, unsigned char *dst, int N, int G,
                               hipStream_t st);
// streaming GEMM for M <= 16 rows, K a multiple of 1024, the plan fields and partial
// layout of the Q4_K streaming kernel (a.KB = K / 256); the row scales are applied
bool f8_stream_ok(int M, int N, int K);
// (2048 waves: 4096 measured 0.7% slower on the batch-1 step)
Q4kStreamPlan f8_stream_plan(int M, int N, int K, int pair = 0, int target_waves = 2048,
                             int wpg = 0);
hipError_t launch_f8_stream(const Q4kFusedArgs &a, const Q4kStreamPlan &p, hipStream_t st);

// ---------------------------------------------------------------- many-row GEMM
// C[split][M][N] fp32 = A[M][K] bf16 . W^T over the split's share of K; W stacked along
// N from up to 3 matrices in bf16 ([N][K]), Q8_0, Q4_K or FP8 (tiled layouts), decoded
// to bf16 MFMA operands per 256 x 256 tile ((hi, lo) pairs for Q8_0 and Q4_K; FP8 codes
// are exact in bf16 and their row scale multiplies the output column).  One split: rows
// scaled by row_inv(rs, r).
struct BigGemmArgs {
    const void *w[3];
    int seg_end[3];
    int nseg;
    int wfmt;                    // 0 bf16, 1 Q8_0, 2 Q4_K, 3 FP8
    const uint16_t *A;
    int lda;
    int M, N, K;
    float *C;
    int ldc;
    RowScale rs;
    int lo_row;                  // rows >= lo_row are the lo terms of (hi, lo) activation
                                 // pairs (0: none): their product with the weights' own
                                 // lo terms (2^-18 of the sum) is skipped
    float *rstat;                // nullable, one split with a row scale (the output head):
                                 // per row and N tile (run of bn columns) the tile's max
                                 // and sum of exp(v - max) at rstat[2 (row grid_x + tile)]
};
struct BigGemmPlan {
    int bm, bn, grid_x, grid_y;  // tile rows (128 / 256) and columns (256; 512 for bf16 at
                                 // up to 128 rows); N and M tiles
    int splits;                  // partial slots [splits][M][N] the consumer sums
    int wgs;                     // 0: grid (N tiles, M tiles, splits); else stream-K workgroups
    int gs;                      // > 0: grouped stream-K over groups of gs weight slabs
    size_t part_bytes;
};
// columns per run of the output head's softmax statistics on tiles bn columns wide
int big_gemm_head_run_cols(int bn);
bool big_gemm_ok(int wf, int M, int N, int K);
// the schedule (grid with K splits, or stream-K) of least estimated time; wf as in BigGemmArgs
BigGemmPlan big_gemm_plan(int wf, int M, int N, int K);
// grid, one split
BigGemmPlan big_gemm_plan_grid(int wf, int M, int N, int K);
hipError_t launch_big_gemm(const BigGemmArgs &a, const BigGemmPlan &p, hipStream_t st);
