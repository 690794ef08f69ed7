// Per-layer elementwise and row kernels of the draft step, gfx950:
//   block assembly (+ first RMSNorm), split-K reductions with fused epilogues
//   (residual add + RMSNorm, SwiGLU), per-head q/k RMSNorm + rotary embedding + KV-cache append, and the
//   attention-partial merge fused with the two-tap dynamic convolution.
// Sources: FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", spec table "Draft" row
// (Qwen3-style layers, 32 query / 8 KV heads of 128, two-tap dynamic
// convolutions, block of 8) and "How it is used"; Mindket kit page, "For
// newcomers and experts" (convolutions keep draft quality along the block).
#include "common.h"
#include "kernels.h"

namespace {

__device__ __forceinline__ float block_sum_256(float v, float *scratch) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    return scratch[0] + scratch[1] + scratch[2] + scratch[3];
}

// ---------------------------------------------------------------- block assembly
// h[b][0] = E[last token], h[b][1..] = mask embedding, and the first layer's input
// x = bf16(h * gain) with the row's sum of squares in ssq[row][0] (the other partials
// of the row are zero; the consumer applies 1 / rms).  Each thread owns up to EMB_V
// runs of 8 values, loaded together (H <= 256 * 8 * EMB_V).
constexpr int EMB_V = 4;

__device__ void embed_row(const EmbedArgs &a, int row) {
    const uint16_t *embed = a.embed, *mask = a.mask, *gain = a.gain;
    const int32_t *last = a.last, *ctx_len = a.ctx_len;
    const int T = a.T, H = a.H, V = a.V, t_new = a.t_new, cap = a.cap;
    float *h = a.h, *ssq = a.ssq;
    uint16_t *x = a.x;
    int32_t *valid = a.valid;
    __shared__ float scratch[4];
    const int b = row / T, t = row % T, tid = threadIdx.x;
    const int n = ctx_len[b], tok = last[b];
    const bool ok = n >= 0 && n <= cap - t_new && tok >= 0 && tok < V;
    if (t == 0 && tid == 0) valid[b] = ok ? 1 : 0;
    const uint16_t *src = t == 0 ? embed + (size_t)(ok ? tok : 0) * H : mask;
    const int nv = H / 8;
    u32x4_t raw[EMB_V], gw[EMB_V];
#pragma unroll
    for (int u = 0; u < EMB_V; u++) {
        const int v = tid + 256 * u;
        const int vc = v < nv ? v : nv - 1;
        raw[u] = *reinterpret_cast<const u32x4_t *>(src + 8 * vc);
        gw[u] = *reinterpret_cast<const u32x4_t *>(gain + 8 * vc);
    }
    float s = 0.f;
    float val[EMB_V][8];
#pragma unroll
    for (int u = 0; u < EMB_V; u++) {
        const bool in = tid + 256 * u < nv;
        const uint32_t wv[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const float f = bf16_to_f32((uint16_t)(wv[i / 2] >> (16 * (i & 1))));
            val[u][i] = (ok && in) ? f : 0.f;
            s += val[u][i] * val[u][i];
        }
    }
    s = block_sum_256(s, scratch);
    const int nchunk = H / 256;
    if (tid < nchunk) ssq[(size_t)row * nchunk + tid] = tid == 0 ? s : 0.f;
    float *hr = h + (size_t)row * H;
    uint16_t *xr = x + (size_t)row * H;
#pragma unroll
    for (int u = 0; u < EMB_V; u++) {
        const int v = tid + 256 * u;
        if (v < nv) {
            const uint32_t g4[4] = {gw[u].x, gw[u].y, gw[u].z, gw[u].w};
            float4 *hp = reinterpret_cast<float4 *>(hr + 8 * v);
            hp[0] = make_float4(val[u][0], val[u][1], val[u][2], val[u][3]);
            hp[1] = make_float4(val[u][4], val[u][5], val[u][6], val[u][7]);
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float g0 = bf16_to_f32((uint16_t)(g4[i] & 0xFFFF)), g1 = bf16_to_f32((uint16_t)(g4[i] >> 16));
                o[i] = pack_bf16x2(val[u][2 * i] * g0, val[u][2 * i + 1] * g1);
            }
            *reinterpret_cast<u32x4_t *>(xr + 8 * v) = (u32x4_t){o[0], o[1], o[2], o[3]};
        }
    }
}

// ---------------------------------------------------------------- reduction + residual (+ norm input)
// Workgroup per (256 columns, output row): the 4 waves sum interleaved subsets of the
// splits (each lane 4 adjacent columns), combined through LDS in a fixed order, so the
// result is deterministic.  v (+ f when adding) is stored to f, the workgroup's sum of
// v^2 goes to ssq[r][blockIdx.x], and with out the next GEMM's input bf16(v * gain)
// (+ its bf16 residual in out_lo) goes to output row map(r).  The RMSNorm's 1 / rms is
// applied by the consumer of that GEMM (RowScale).
template <int RB>
__device__ void reduce_rows_block(const ReduceRowsArgs &a, int cx, int r) {
    const float *part = a.part;
    const int splits = a.splits, M_out = a.M_out, N = a.N, pair = a.pair, add = a.add;
    const int ldo = a.ldo, map = a.map;
    float *f = a.f, *ssq = a.ssq;
    const uint16_t *gain = a.gain;
    uint16_t *out = a.out, *out_lo = a.out_lo;
    __shared__ float4 red[4][64];
    __shared__ float scratch[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c0 = cx * 256;
    const size_t stride = (size_t)(pair ? 2 * M_out : M_out) * N;
    const float *p = part + (size_t)r * N + c0 + 4 * lane;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    // this wave's splits k = wave, wave + 4, ...: RB of them in flight per batch (8 where
    // there are more than 16 splits: the down projection's 17 and the fc's 25 at batch 1
    // then take one memory round trip; else 4, fewer registers, more resident waves)
    for (int k0 = wave; k0 < splits; k0 += 4 * RB) {
        float4 va[RB], vb[RB];
#pragma unroll
        for (int u = 0; u < RB; u++) {
            const float *q = p + (size_t)min(k0 + 4 * u, splits - 1) * stride;
            va[u] = *reinterpret_cast<const float4 *>(q);
            vb[u] = pair ? *reinterpret_cast<const float4 *>(q + (size_t)pair * N)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < RB; u++)
            if (k0 + 4 * u < splits) {
                s.x += va[u].x + vb[u].x;
                s.y += va[u].y + vb[u].y;
                s.z += va[u].z + vb[u].z;
                s.w += va[u].w + vb[u].w;
            }
    }
    red[wave][lane] = s;
    __syncthreads();
    const float *rf = reinterpret_cast<const float *>(red);
    const int c = tid;                              // column c0 + c: lane c / 4, element c % 4
    float v = ((rf[c] + rf[256 + c]) + rf[512 + c]) + rf[768 + c];
    float *fp = f + (size_t)r * N + c0 + c;
    if (add) v += *fp;
    *fp = v;
    const float sq = block_sum_256(v * v, scratch);
    if (tid == 0) ssq[(size_t)r * (N / 256) + cx] = sq;
    if (!out || (map > 0 && r % map == 0)) return;
    const int orow = map > 0 ? (r / map) * (map - 1) + r % map - 1 : r;
    const float x = v * bf16_to_f32(gain[c0 + c]);
    const uint16_t hb = f32_to_bf16(x);
    out[(size_t)orow * ldo + c0 + c] = hb;
    if (out_lo) out_lo[(size_t)orow * ldo + c0 + c] = f32_to_bf16(x - bf16_to_f32(hb));
}

__global__ __launch_bounds__(256) void k_embed(EmbedArgs a) { embed_row(a, blockIdx.x); }

template <int RB>
__global__ __launch_bounds__(256) void k_reduce_rows(ReduceRowsArgs a) {
    reduce_rows_block<RB>(a, blockIdx.x, blockIdx.y);
}

// The same reduction with one wave per (row, 256 columns), four per workgroup, and no
// workgroup barrier, for many rows: each lane holds 4 adjacent columns and issues the
// loads of up to SB splits at once.  It keeps reduce_rows_block's order of additions (the
// sums of splits w, w + 4, ... for w = 0..3, added in w order; the sum of squares as four
// wave sums over 64-column groups, added in group order); the results still differ from
// it in the last bits (a 5-layer batch-1 step's hidden states by up to 3e-4), so which
// kernel runs is fixed by the row count.  Measured per step: 64 sequences 6.028 ->
// 5.960 ms; 16 sequences 2.686 -> 2.701 ms and batch 1 0.849 -> 0.859 ms, where
// reduce_rows_block stays.
template <int SB>
__global__ __launch_bounds__(256) void k_reduce_rows_w(ReduceRowsArgs a) {
    static_assert(SB % 4 == 0, "a batch holds whole rounds of the four split classes");
    __shared__ float sqs[4][256];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nc = a.N / 256, item = blockIdx.x * 4 + wave;
    if (item >= a.M_out * nc) return;
    const int r = item / nc, cx = item % nc, c0 = cx * 256 + 4 * lane;
    const int splits = a.splits, pair = a.pair, N = a.N;
    const size_t stride = (size_t)(pair ? 2 * a.M_out : a.M_out) * N;
    const float *p = a.part + (size_t)r * N + c0;
    float4 s[4];
#pragma unroll
    for (int w = 0; w < 4; w++) s[w] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = 0; k0 < splits; k0 += SB) {
        float4 va[SB], vb[SB];
#pragma unroll
        for (int u = 0; u < SB; u++) {
            const float *q = p + (size_t)min(k0 + u, splits - 1) * stride;
            va[u] = *reinterpret_cast<const float4 *>(q);
            vb[u] = pair ? *reinterpret_cast<const float4 *>(q + (size_t)pair * N)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < SB; u++)
            if (k0 + u < splits) {
                float4 &t = s[u & 3];               // split k0 + u is of class (k0 + u) % 4 = u % 4
                t.x += va[u].x + vb[u].x;
                t.y += va[u].y + vb[u].y;
                t.z += va[u].z + vb[u].z;
                t.w += va[u].w + vb[u].w;
            }
    }
    float v[4] = {((s[0].x + s[1].x) + s[2].x) + s[3].x, ((s[0].y + s[1].y) + s[2].y) + s[3].y,
                  ((s[0].z + s[1].z) + s[2].z) + s[3].z, ((s[0].w + s[1].w) + s[2].w) + s[3].w};
    float *fp = a.f + (size_t)r * N + c0;
    if (a.add) {
        const float4 f = *reinterpret_cast<const float4 *>(fp);
        v[0] += f.x; v[1] += f.y; v[2] += f.z; v[3] += f.w;
    }
    *reinterpret_cast<float4 *>(fp) = make_float4(v[0], v[1], v[2], v[3]);
    // squares regrouped so that lane l holds column 64 g + l of each 64-column group g
    *reinterpret_cast<float4 *>(&sqs[wave][4 * lane]) =
        make_float4(v[0] * v[0], v[1] * v[1], v[2] * v[2], v[3] * v[3]);
    __builtin_amdgcn_wave_barrier();
    float q[4];
#pragma unroll
    for (int g = 0; g < 4; g++) q[g] = wave_sum(sqs[wave][64 * g + lane]);
    if (lane == 0) a.ssq[(size_t)r * nc + cx] = q[0] + q[1] + q[2] + q[3];
    if (!a.out || (a.map > 0 && r % a.map == 0)) return;
    const int orow = a.map > 0 ? (r / a.map) * (a.map - 1) + r % a.map - 1 : r;
    uint16_t hb[4], lb[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float x = v[i] * bf16_to_f32(a.gain[c0 + i]);
        hb[i] = f32_to_bf16(x);
        lb[i] = f32_to_bf16(x - bf16_to_f32(hb[i]));
    }
    *reinterpret_cast<u32x2_t *>(a.out + (size_t)orow * a.ldo + c0) =
        (u32x2_t){(uint32_t)hb[0] | ((uint32_t)hb[1] << 16), (uint32_t)hb[2] | ((uint32_t)hb[3] << 16)};
    if (a.out_lo)
        *reinterpret_cast<u32x2_t *>(a.out_lo + (size_t)orow * a.ldo + c0) =
            (u32x2_t){(uint32_t)lb[0] | ((uint32_t)lb[1] << 16), (uint32_t)lb[2] | ((uint32_t)lb[3] << 16)};
}

// one launch for two independent jobs: the reduction's (N / 256) x M_out workgroups,
// then the block assembly's B T workgroups
template <int RB>
__global__ __launch_bounds__(256) void k_reduce_rows_embed(ReduceRowsArgs a, EmbedArgs e) {
    const int nc = a.N / 256, nred = nc * a.M_out;
    const int bid = blockIdx.x;
    if (bid < nred) reduce_rows_block<RB>(a, bid % nc, bid / nc);
    else embed_row(e, bid - nred);
}

// ---------------------------------------------------------------- split-K reduction
// Output row r sums the partial rows r (and r + pair when the GEMM ran over
// [hi rows; lo rows]) over all splits in a fixed order.
__global__ __launch_bounds__(256) void k_reduce(const float *part, int splits, int M, int N,
                                                int pair, int mode, float *of, uint16_t *ob,
                                                uint16_t *ob_lo, int ldo, RowScale rs) {
    const int Nout = mode == EPI_SWIGLU_BF16 ? N / 2 : N;
    const size_t total = (size_t)M * Nout;
    const int Min = pair ? 2 * M : M;
    const size_t stride = (size_t)Min * N;
    for (size_t e = blockIdx.x * 256ull + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
        const int r = (int)(e / Nout), c = (int)(e % Nout);
        const float *p = part + (size_t)r * N + c;
        const float *q = part + (size_t)(r + pair) * N + c;
        float s = 0.f;
        for (int k = 0; k < splits; k++) s += p[k * stride] + (pair ? q[k * stride] : 0.f);
        const float inv = row_inv(rs, r);
        s *= inv;
        if (mode == EPI_STORE_F32) {
            of[(size_t)r * ldo + c] = s;
        } else if (mode == EPI_ADD_F32) {
            of[(size_t)r * ldo + c] += s;
        } else if (mode == EPI_STORE_BF16) {
            ob[(size_t)r * ldo + c] = f32_to_bf16(s);
        } else {
            float u = 0.f;
            for (int k = 0; k < splits; k++)
                u += p[k * stride + Nout] + (pair ? q[k * stride + Nout] : 0.f);
            u *= inv;
            const float act = s / (1.f + expf(-s));          // silu(gate)
            const float v = act * u;
            const uint16_t hb = f32_to_bf16(v);
            ob[(size_t)r * ldo + c] = hb;
            if (ob_lo) ob_lo[(size_t)r * ldo + c] = f32_to_bf16(v - bf16_to_f32(hb));
        }
    }
}

// row_inv for a whole wave (every lane calls it, same r): lane i loads partial i (and
// i + 64, ...), the partials are added by a wave reduction
__device__ __forceinline__ float row_inv_wave(const RowScale &s, int r, int lane) {
    if (!s.ssq) return 1.f;
    const int br = s.map ? (r / (s.map - 1)) * s.map + r % (s.map - 1) + 1 : r;
    const float *p = s.ssq + (size_t)br * s.nchunk;
    float ss = 0.f;
    for (int i = lane; i < s.nchunk; i += 64) ss += p[i];
    return rsqrtf(wave_sum(ss) / s.n + s.eps);
}

// ---------------------------------------------------------------- SwiGLU from split partials
// Workgroup per (1024 columns, output row r), four consecutive columns per thread
// (16-byte loads, three splits in flight): gate and up (columns c and c + N/2 of the [gate | up] product) summed
// over the splits (in split order) and the [hi; lo] row pair, scaled by the row's
// deferred 1 / rms (formed once per workgroup), then silu(gate) * up as a bf16 (hi, lo)
// pair.  SB splits' loads in flight per batch: 6 where there are more than 3 splits (one
// round trip for batch 1's 5; the 1 / rms then comes from the first wave, one load per
// lane), else 3 (1 / rms from one thread: measured faster at 64 sequences).  Needs N / 2
// a multiple of 4.
template <int SB>
__global__ __launch_bounds__(256) void k_swiglu(const float *part, int splits, int M, int N, int pair,
                                                uint16_t *ob, uint16_t *ob_lo, int ldo, RowScale rs) {
    const int r = blockIdx.y, c = 4 * (blockIdx.x * 256 + threadIdx.x);
    const int F = N / 2;
    __shared__ float s_inv;
    if (SB > 3) {
        if (threadIdx.x < 64) {
            const float ri = row_inv_wave(rs, r, threadIdx.x);
            if (threadIdx.x == 0) s_inv = ri;
        }
    } else if (threadIdx.x == 0) {
        s_inv = row_inv(rs, r);
    }
    const size_t stride = (size_t)(pair ? 2 * M : M) * N;
    const float *p = part + (size_t)r * N + min(c, F - 4);
    float4 gs = {0.f, 0.f, 0.f, 0.f}, us = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < splits; k0 += SB) {
        float4 gv[SB], uv[SB], gq[SB], uq[SB];
#pragma unroll
        for (int u = 0; u < SB; u++) {
            const float *p0 = p + (size_t)min(k0 + u, splits - 1) * stride;
            gv[u] = *reinterpret_cast<const float4 *>(p0);
            uv[u] = *reinterpret_cast<const float4 *>(p0 + F);
            const float4 z = {0.f, 0.f, 0.f, 0.f};
            gq[u] = pair ? *reinterpret_cast<const float4 *>(p0 + (size_t)pair * N) : z;
            uq[u] = pair ? *reinterpret_cast<const float4 *>(p0 + (size_t)pair * N + F) : z;
        }
#pragma unroll
        for (int u = 0; u < SB; u++)
            if (k0 + u < splits) {
                gs.x += gv[u].x + gq[u].x; gs.y += gv[u].y + gq[u].y;
                gs.z += gv[u].z + gq[u].z; gs.w += gv[u].w + gq[u].w;
                us.x += uv[u].x + uq[u].x; us.y += uv[u].y + uq[u].y;
                us.z += uv[u].z + uq[u].z; us.w += uv[u].w + uq[u].w;
            }
    }
    __syncthreads();
    if (c >= F) return;
    const float inv = s_inv;
    const float g4[4] = {gs.x, gs.y, gs.z, gs.w}, u4[4] = {us.x, us.y, us.z, us.w};
    uint16_t hb[4], lb[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float gt = g4[i] * inv, up = u4[i] * inv;
        const float v = gt / (1.f + expf(-gt)) * up;
        hb[i] = f32_to_bf16(v);
        lb[i] = f32_to_bf16(v - bf16_to_f32(hb[i]));
    }
    *reinterpret_cast<u32x2_t *>(ob + (size_t)r * ldo + c) =
        (u32x2_t){(uint32_t)hb[0] | ((uint32_t)hb[1] << 16), (uint32_t)hb[2] | ((uint32_t)hb[3] << 16)};
    if (ob_lo)
        *reinterpret_cast<u32x2_t *>(ob_lo + (size_t)r * ldo + c) =
            (u32x2_t){(uint32_t)lb[0] | ((uint32_t)lb[1] << 16), (uint32_t)lb[2] | ((uint32_t)lb[3] << 16)};
}

// ---------------------------------------------------------------- q/k norm, rotary, append
// One wave per (row, head).  Lane j < d/2 owns the rotary pair (j, j + d/2).  QB splits'
// loads in flight per batch: 8 where the product has more than 4 splits (one round trip
// for the 5 of the q|k|v product at batch 1), else 4.
template <int QB>
__global__ __launch_bounds__(64) void k_qk_norm_rope(RopeArgs a) {
    const int r = blockIdx.x, hh = blockIdx.y, lane = threadIdx.x;
    const int d = a.d, half = d / 2;
    const int qd = a.n_q * d, kd = a.n_kv * d;
    const int nblk = a.B * a.T;
    int b, pos, t = 0, j = 0;
    const bool is_blk = r < nblk;
    if (is_blk) {
        b = r / a.T;
        t = r % a.T;
    } else {
        b = (r - nblk) / a.t_new;
        j = (r - nblk) % a.t_new;
    }
    if (!a.valid[b]) return;
    const int n = a.ctx_len[b];
    pos = is_blk ? n + a.t_new + t : n + j;
    const bool is_q = hh < a.n_q, is_k = !is_q && hh < a.n_q + a.n_kv;
    if (is_q && !is_blk) return;                      // context rows need K and V only
    const float *x = a.qkv + (size_t)r * (qd + 2 * kd) + (size_t)hh * d;
    const size_t pstride = (size_t)a.B * (a.T + a.t_new) * (qd + 2 * kd);
    float x1 = 0.f, x2 = 0.f;
    if (lane < half) {
        // only the splits present
        for (int s0 = 0; s0 < a.splits; s0 += QB) {
            float v1[QB], v2[QB];
#pragma unroll
            for (int u = 0; u < QB; u++) {
                v1[u] = v2[u] = 0.f;
                if (s0 + u < a.splits) {
                    v1[u] = x[(s0 + u) * pstride + lane];
                    v2[u] = x[(s0 + u) * pstride + lane + half];
                }
            }
#pragma unroll
            for (int u = 0; u < QB; u++) {
                x1 += v1[u];
                x2 += v2[u];
            }
        }
    }
    // the projection input's deferred RMSNorm (its partial sums of squares split over
    // the lanes)
    const float rinv = is_blk ? row_inv_wave(a.blk, r, lane) : row_inv_wave(a.ctx, r - nblk, lane);
    x1 *= rinv;
    x2 *= rinv;
    if (is_q || is_k) {
        const uint16_t *g = is_q ? a.q_norm : a.k_norm;
        const float ss = wave_sum(x1 * x1 + x2 * x2);
        const float inv = rsqrtf(ss / (float)d + a.eps);
        if (lane < half) {
            x1 *= inv * bf16_to_f32(g[lane]);
            x2 *= inv * bf16_to_f32(g[lane + half]);
            // rotation angle pos * theta^(-2 lane / d): the inverse frequency and the
            // product in fp64, the angle reduced modulo 2 pi in fp64 (a two-term 2 pi;
            // the fma rounds only the small remainder), then fp32 sine and cosine of the
            // reduced angle (|r| <= pi, where the fp32 routines need no long reduction)
            const double ang = (double)pos * exp2(-2.0 * lane / d * a.log2_theta);
            const double k = rint(ang * 0.15915494309189535);              // ang / (2 pi)
            const double rr = fma(-k, 2.4492935982947064e-16, fma(-k, 6.283185307179586, ang));
            float s, c;
            sincosf((float)rr, &s, &c);
            const float y1 = x1 * c - x2 * s, y2 = x2 * c + x1 * s;
            x1 = y1;
            x2 = y2;
        }
    }
    if (lane >= half) return;
    uint16_t *dst;
    if (is_blk) {
        if (is_q) dst = a.Q + ((size_t)r * a.n_q + hh) * d;
        else if (is_k) dst = a.Kb + ((size_t)r * a.n_kv + (hh - a.n_q)) * d;
        else dst = a.Vb + ((size_t)r * a.n_kv + (hh - a.n_q - a.n_kv)) * d;
    } else {
        const int kvh = is_k ? hh - a.n_q : hh - a.n_q - a.n_kv;
        uint16_t *cache = is_k ? a.k_cache : a.v_cache;
        dst = cache + (((size_t)b * a.n_kv + kvh) * a.cap + (n + j)) * d;
    }
    dst[lane] = f32_to_bf16(x1);
    dst[lane + half] = f32_to_bf16(x2);
}

// ---------------------------------------------------------------- merge + dynamic conv
// k_attn_merge: one workgroup per (query head h, 32-column slice cc of the head,
// sequence b); each wave sums a quarter of the chunks over the 8 x 32 block (16 bytes
// per lane), the waves' sums are added in LDS.  Combines the split-window partials of
// head h (log-sum-exp merge: weight exp(m_c - M) / sum_c exp(m_c - M) l_c
// on the unnormalised chunk outputs) into o[b][t][h d + 32 cc + col] (fp32), then
// contributes this slice's share of the convolution taps
//     zp[b][h][cc][t][q] = sum_{e in slice} W_c[q][h d + e] o[b][t][h d + e],  q < 2 n_q,
// so that z_t = W_c . vec(o_t) = the sum of zp over (h, cc).
constexpr int MC = 32;              // columns per merge workgroup

// MW: chunk partials per lane loaded up front (x 4 waves): 9 covers the 33 chunks of a
// 2048-key window in 64-key chunks; 3 the 9 of 256-key chunks (fewer registers, more
// resident workgroups).  Chunks past 4 MW are read in further batches, same order.
constexpr int MAXE = 4;             // conv-tap outputs per thread (T 2 n_q <= 1024)

template <int MW>
__global__ __launch_bounds__(256) void k_attn_merge(MergeConvArgs a) {
    const int h = blockIdx.x, cc = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int d = a.d, T = a.T, G = a.n_q / a.n_kv, QR = G * T, qd = a.n_q * d;
    const int kvh = h / G, hq = h % G;
    const int nch1 = a.n_chunks + 1;
    const int nq2 = 2 * a.n_q, CC = d / MC;
    const int c0 = h * d + cc * MC;
    extern __shared__ float sm[];
    float *w = sm;                      // [T][nch1] merge weights
    float *os = sm + T * nch1;          // [T][MC] merged output slice
    float *wp = os + T * MC;            // [4 waves][T][MC] per-wave partial sums
    // [2 n_q][MC / 8] W_c slice, at the next 16-byte boundary
    u32x4_t *wcs = reinterpret_cast<u32x4_t *>(sm + (T * (nch1 + 5 * MC) + 3) / 4 * 4);
    float *zp = a.zp + (((size_t)b * a.n_q + h) * CC + cc) * T * nq2;

    // ---- every load first, so the kernel waits on memory once.  Wave w sums chunks
    // w, w + 4, ...: lane (t, c4) = (lane / 8, lane % 8) holds row t, columns 4 c4 ..
    // 4 c4 + 3 of the slice (16-byte loads).  Also the (m, l) pairs of the wave's rows
    // (rows wave and wave + 4, the first 64 chunks) and the conv-tap weights of the
    // thread's (t, q) pairs.  Indices are clamped (in bounds); what is not used is
    // discarded by selects.
    const int lt = lane >> 3, c4 = lane & 7;            // rows lt >= T (blocks under 8) idle
    const float *O = a.O + ((size_t)(b * a.n_kv + kvh) * nch1 * QR + hq * T + min(lt, T - 1)) * d +
                     cc * MC + 4 * c4;
    const size_t cstride = (size_t)QR * d;
    float4 pv[MW];
#pragma unroll
    for (int u = 0; u < MW; u++)
        pv[u] = *reinterpret_cast<const float4 *>(O + (size_t)min(wave + 4 * u, nch1 - 1) * cstride);
    const float *ml = a.ml + ((size_t)(b * a.n_kv + kvh) * nch1) * QR * 2;
    float2 mlv[2];
#pragma unroll
    for (int ri = 0; ri < 2; ri++) {
        const int tr = min(wave + 4 * ri, T - 1), c = min(lane, nch1 - 1);
        mlv[ri] = *reinterpret_cast<const float2 *>(ml + ((size_t)c * QR + hq * T + tr) * 2);
    }
    const int ne = T * nq2;
    // the slice of W_c ([2 n_q][MC] bf16, 16-byte pieces: piece p = row p / 4, columns
    // 8 (p % 4) ..), staged in LDS for the conv-tap partials
    u32x4_t wl[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int pc = min(tid + 256 * j, nq2 * (MC / 8) - 1);
        wl[j] = *reinterpret_cast<const u32x4_t *>(a.w_conv + (size_t)(pc / (MC / 8)) * qd + c0 +
                                                   8 * (pc % (MC / 8)));
    }

    const int t = tid / MC, col = tid % MC;             // 8 * MC == 256; rows t >= T idle
    if (!a.valid[b]) {
        if (t < T) a.o[((size_t)b * T + t) * qd + c0 + col] = 0.f;
        for (int e = tid; e < ne; e += 256) zp[e] = 0.f;
        return;
    }
    const int n = a.ctx_len[b];
    const int hi = n + a.t_new;
    const int lo = hi - a.window > 0 ? hi - a.window : 0;
    const int nch_b = ceil_div(hi - lo, a.chunk);
    auto used = [&](int c) { return c < nch_b || c == a.n_chunks; };
    // merge weights exp(m_c - M) / sum_c exp(m_c - M) l_c: wave per row, lanes over chunks
#pragma unroll
    for (int ri = 0; ri < 2; ri++) {
        const int tr = wave + 4 * ri;
        if (tr >= T) break;
        auto mlc = [&](int c) -> float2 {            // chunks past the first 64 (long windows)
            return c < 64 ? mlv[ri] : *reinterpret_cast<const float2 *>(ml + ((size_t)c * QR + hq * T + tr) * 2);
        };
        float M = -INFINITY;
        for (int c = lane; c < nch1; c += 64)
            if (used(c)) M = fmaxf(M, mlc(c).x);
        M = wave_max(M);
        float L = 0.f;
        for (int c = lane; c < nch1; c += 64) {
            float e = 0.f;
            if (used(c)) {
                const float2 v = mlc(c);
                e = expf(v.x - M);
                L += e * v.y;
            }
            w[tr * nch1 + c] = e;
        }
        L = wave_sum(L);
        const float invL = 1.f / L;
        for (int c = lane; c < nch1; c += 64) w[tr * nch1 + c] *= invL;
    }
    __syncthreads();
    // this wave's chunks, weighted (unused chunks skipped)
    const float *wt = w + min(lt, T - 1) * nch1;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    auto add = [&](int c, float4 v) {
        if (c < nch1 && used(c)) {
            const float wc = wt[c];
            acc.x += wc * v.x; acc.y += wc * v.y; acc.z += wc * v.z; acc.w += wc * v.w;
        }
    };
#pragma unroll
    for (int u = 0; u < MW; u++) add(wave + 4 * u, pv[u]);
    for (int cb = wave + 4 * MW; cb < nch1; cb += 4 * 8) {     // long windows
        float4 pb[8];
#pragma unroll
        for (int u = 0; u < 8; u++) pb[u] = *reinterpret_cast<const float4 *>(O + (size_t)min(cb + 4 * u, nch1 - 1) * cstride);
#pragma unroll
        for (int u = 0; u < 8; u++) add(cb + 4 * u, pb[u]);
    }
    if (lt < T) *reinterpret_cast<float4 *>(&wp[(wave * T + lt) * MC + 4 * c4]) = acc;
#pragma unroll
    for (int j = 0; j < 2; j++)
        if (tid + 256 * j < nq2 * (MC / 8)) wcs[tid + 256 * j] = wl[j];
    __syncthreads();
    // merged output of (t, col): the 4 waves' sums in wave order
    if (t < T) {
        const float ov = wp[(0 * T + t) * MC + col] + wp[(1 * T + t) * MC + col] +
                         wp[(2 * T + t) * MC + col] + wp[(3 * T + t) * MC + col];
        os[t * MC + col] = ov;
        a.o[((size_t)b * T + t) * qd + c0 + col] = ov;
    }
    __syncthreads();
    // conv-tap partials of this slice: (t, q) pairs over the threads
#pragma unroll
    for (int i = 0; i < MAXE; i++) {
        const int e = tid + 256 * i;
        if (e >= ne) break;
        const int tt = e / nq2, q = e % nq2;
        const float *ot = os + tt * MC;
        float acc2 = 0.f;
#pragma unroll
        for (int k = 0; k < MC / 8; k++) {
            const u32x4_t v = wcs[q * (MC / 8) + k];
            const float *o8 = ot + 8 * k;
            acc2 += bf16_to_f32(v.x & 0xFFFF) * o8[0] + bf16_to_f32(v.x >> 16) * o8[1];
            acc2 += bf16_to_f32(v.y & 0xFFFF) * o8[2] + bf16_to_f32(v.y >> 16) * o8[3];
            acc2 += bf16_to_f32(v.z & 0xFFFF) * o8[4] + bf16_to_f32(v.z >> 16) * o8[5];
            acc2 += bf16_to_f32(v.w & 0xFFFF) * o8[6] + bf16_to_f32(v.w >> 16) * o8[7];
        }
        zp[e] = acc2;
    }
}

// k_conv_apply: one workgroup per (sequence b, block row t, pair of heads):
//   z_t[h], z_t[n_q + h] for the two heads = sums of the (h', cc) partials;
//   y_{t,h} = z_t[h] o_{t,h} + z_t[n_q + h] o_{t-1,h},  o_{-1} = 0.
constexpr int CONV_HEADS = 2;       // heads per conv workgroup
// block rows from which k_conv_rows takes the taps: measured at 64 sequences (512 rows)
// 6.287 -> 6.250 ms per step, at 16 (128 rows) 2.759 -> 2.775 ms, so from 512
constexpr int CONV_ROWS_MIN = 512;

__global__ __launch_bounds__(256) void k_conv_apply(MergeConvArgs a) {
    __shared__ float z[2 * CONV_HEADS];
    const int b = blockIdx.x / a.T, t = blockIdx.x % a.T, tid = threadIdx.x;
    const int qd = a.n_q * a.d, nq2 = 2 * a.n_q, CC = a.d / MC;
    const int np = a.n_q * CC;                          // partials per (b, t, q)
    const int h0 = blockIdx.y * CONV_HEADS;
    // the 2 CONV_HEADS tap values this workgroup needs: q = h0 + k (a) and n_q + h0 + k (b)
    constexpr int NQ = 2 * CONV_HEADS, PER_Q = 256 / NQ;
    const int qi = tid / PER_Q, part = tid % PER_Q;
    const int q = qi < CONV_HEADS ? h0 + qi : a.n_q + h0 + qi - CONV_HEADS;
    // the attention outputs this thread scales are loaded together with the partials
    const float *ot = a.o + ((size_t)b * a.T + t) * qd;
    const float *op = t > 0 ? ot - qd : ot;             // row t - 1 (t = 0: unused)
    const int i0 = h0 * a.d, i1 = min(i0 + CONV_HEADS * a.d, qd);
    constexpr int NI = CONV_HEADS * 128 / 256;           // outputs per thread (d <= 128)
    float ocur[NI], oprev[NI];
#pragma unroll
    for (int u = 0; u < NI; u++) {
        const int i = min(i0 + tid + 256 * u, i1 - 1);
        ocur[u] = ot[i];
        oprev[u] = op[i];
    }
    constexpr int NP = 4;                                // partials per thread per batch
    float s = 0.f;
    for (int p0 = part; p0 < np; p0 += NP * PER_Q) {
        float v[NP];
#pragma unroll
        for (int u = 0; u < NP; u++) {
            const int p = min(p0 + u * PER_Q, np - 1);
            v[u] = a.zp[(((size_t)b * np + p) * a.T + t) * nq2 + q];
        }
#pragma unroll
        for (int u = 0; u < NP; u++)
            if (p0 + u * PER_Q < np) s += v[u];
    }
    // PER_Q == 64: tap value qi is the sum over wave qi
    s = wave_sum(s);
    if ((tid & 63) == 0) z[qi] = s;
    __syncthreads();
    uint16_t *Y = a.Y + ((size_t)b * a.T + t) * qd;
#pragma unroll
    for (int u = 0; u < NI; u++) {
        const int i = i0 + tid + 256 * u;
        if (i < i1) {
            const int k = (i - i0) / a.d;
            Y[i] = f32_to_bf16(z[k] * ocur[u] + (t > 0 ? z[CONV_HEADS + k] * oprev[u] : 0.f));
        }
    }
}

// k_conv_rows: the same taps and outputs with one workgroup per (sequence b, block row
// t), for batches large enough to fill the chip with rows.  The row's partials
// ([B][n_q][d/32][T][2 n_q]: 2 n_q contiguous values per (head, slice)) are read as whole
// lines into LDS, where k_conv_apply's 16 workgroups per row each used 8 bytes of every
// 128-byte line they read; each tap is then summed exactly as k_conv_apply sums it (lane
// j adds the partials j, j + 64, ... in order, then the same wave sum), so the two
// kernels give identical bits.
constexpr int ROW_NI = 16;          // outputs per thread (n_q d <= 4096)

__global__ __launch_bounds__(256) void k_conv_rows(MergeConvArgs a) {
    extern __shared__ float zrow[];
    const int b = blockIdx.x / a.T, t = blockIdx.x % a.T, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int qd = a.n_q * a.d, nq2 = 2 * a.n_q, np = a.n_q * (a.d / MC), ZS = nq2 + 1;
    float *Z = zrow, *z = zrow + np * ZS;
    // the attention outputs of rows t and t - 1 this thread scales, loaded with the partials
    const float *ot = a.o + ((size_t)b * a.T + t) * qd;
    const float *op = t > 0 ? ot - qd : ot;              // row t - 1 (t = 0: unused)
    float ocur[ROW_NI], oprev[ROW_NI];
#pragma unroll
    for (int u = 0; u < ROW_NI; u++) {
        const int i = min(tid + 256 * u, qd - 1);
        ocur[u] = ot[i];
        oprev[u] = op[i];
    }
    const float *zp = a.zp + (size_t)b * np * a.T * nq2 + (size_t)t * nq2;
    for (int e = tid; e < np * nq2 / 4; e += 256) {
        const int p = e / (nq2 / 4), q = 4 * (e % (nq2 / 4));
        const float4 v = *reinterpret_cast<const float4 *>(zp + (size_t)p * a.T * nq2 + q);
        float *d = Z + p * ZS + q;
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
    __syncthreads();
    for (int q = wave; q < nq2; q += 4) {
        float s = 0.f;
        for (int p = lane; p < np; p += 64) s += Z[p * ZS + q];
        s = wave_sum(s);
        if (lane == 0) z[q] = s;
    }
    __syncthreads();
    uint16_t *Y = a.Y + ((size_t)b * a.T + t) * qd;
#pragma unroll
    for (int u = 0; u < ROW_NI; u++) {
        const int i = tid + 256 * u;
        if (i < qd) {
            const int h = i / a.d;
            Y[i] = f32_to_bf16(z[h] * ocur[u] + (t > 0 ? z[a.n_q + h] * oprev[u] : 0.f));
        }
    }
}

}  // namespace

hipError_t launch_embed(const EmbedArgs &a, int B, hipStream_t st) {
    hipLaunchKernelGGL(k_embed, dim3(B * a.T), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_reduce_epilogue(const float *part, int splits, int M, int N, int pair,
                                  int mode, float *out_f32, uint16_t *out_bf16,
                                  uint16_t *out_bf16_lo, int ldo, const RowScale &rs,
                                  hipStream_t st) {
    const size_t total = (size_t)M * (mode == EPI_SWIGLU_BF16 ? N / 2 : N);
    size_t grid = (total + 255) / 256;
    if (grid > 8192) grid = 8192;
    hipLaunchKernelGGL(k_reduce, dim3((unsigned)grid), dim3(256), 0, st, part, splits, M, N, pair,
                       mode, out_f32, out_bf16, out_bf16_lo, ldo, rs);
    return hipGetLastError();
}

hipError_t launch_swiglu(const float *part, int splits, int M, int N, int pair, uint16_t *out,
                         uint16_t *out_lo, int ldo, const RowScale &rs, hipStream_t st) {
    if ((N / 2) % 4 || ldo % 4) return hipErrorInvalidValue;
    if (splits > 3)
        hipLaunchKernelGGL(k_swiglu<6>, dim3(ceil_div(N / 2, 1024), M), dim3(256), 0, st, part, splits, M,
                           N, pair, out, out_lo, ldo, rs);
    else
        hipLaunchKernelGGL(k_swiglu<3>, dim3(ceil_div(N / 2, 1024), M), dim3(256), 0, st, part, splits, M,
                           N, pair, out, out_lo, ldo, rs);
    return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const RopeArgs &a, hipStream_t st) {
    dim3 grid(a.B * (a.T + a.t_new), a.n_q + 2 * a.n_kv);
    if (a.splits > 4) hipLaunchKernelGGL(k_qk_norm_rope<8>, grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL(k_qk_norm_rope<4>, grid, dim3(64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_merge_conv(const MergeConvArgs &a, hipStream_t st) {
    // (then the W_c slice, from the next 16-byte boundary)
    size_t lds = (size_t)(a.T * (a.n_chunks + 1) + a.T * MC + 4 * a.T * MC) * 4;
    lds = (lds + 15) / 16 * 16 + (size_t)2 * a.n_q * MC * 2;
    if (a.n_chunks + 1 <= 12)
        hipLaunchKernelGGL(k_attn_merge<3>, dim3(a.n_q, a.d / MC, a.B), dim3(256), lds, st, a);
    else
        hipLaunchKernelGGL(k_attn_merge<9>, dim3(a.n_q, a.d / MC, a.B), dim3(256), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // one workgroup per row where the rows fill the chip (and the row's partials fit LDS)
    const int np = a.n_q * (a.d / MC), nq2 = 2 * a.n_q;
    const size_t zl = ((size_t)np * (nq2 + 1) + nq2) * 4;
    if (a.B * a.T >= CONV_ROWS_MIN && a.n_q * a.d <= 256 * ROW_NI && nq2 % 4 == 0 && zl <= 64 * 1024)
        hipLaunchKernelGGL(k_conv_rows, dim3(a.B * a.T), dim3(256), zl, st, a);
    else
        hipLaunchKernelGGL(k_conv_apply, dim3(a.B * a.T, a.n_q / CONV_HEADS), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_reduce_norm(const ReduceRowsArgs &a, hipStream_t st) {
    // many rows: a wave per (row, 256 columns), its splits' loads in one batch up to 20
    const unsigned grid = (unsigned)ceil_div(a.M_out * (a.N / 256), 4);
    if (a.M_out >= 512 && a.ldo % 4 == 0) {
        if (a.splits > 8) hipLaunchKernelGGL(k_reduce_rows_w<20>, dim3(grid), dim3(256), 0, st, a);
        else if (a.splits > 4) hipLaunchKernelGGL(k_reduce_rows_w<8>, dim3(grid), dim3(256), 0, st, a);
        else hipLaunchKernelGGL(k_reduce_rows_w<4>, dim3(grid), dim3(256), 0, st, a);
        return hipGetLastError();
    }
    if (a.splits > 16) hipLaunchKernelGGL(k_reduce_rows<8>, dim3(a.N / 256, a.M_out), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(k_reduce_rows<4>, dim3(a.N / 256, a.M_out), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_reduce_norm(const float *part, int splits, int M_out, int N, int pair, int add,
                              float *f, float *ssq, const uint16_t *gain, uint16_t *out,
                              uint16_t *out_lo, int ldo, int map, hipStream_t st) {
    const ReduceRowsArgs a = {part, splits, M_out, N, pair, add, f, ssq, gain, out, out_lo, ldo, map};
    return launch_reduce_norm(a, st);
}

hipError_t launch_reduce_norm_embed(const ReduceRowsArgs &a, const EmbedArgs &e, int B,
                                    hipStream_t st) {
    const int grid = (a.N / 256) * a.M_out + B * e.T;
    if (a.splits > 16) hipLaunchKernelGGL(k_reduce_rows_embed<8>, dim3(grid), dim3(256), 0, st, a, e);
    else hipLaunchKernelGGL(k_reduce_rows_embed<4>, dim3(grid), dim3(256), 0, st, a, e);
    return hipGetLastError();
}
