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
// x = bf16(RMSNorm(h) * gain)
__global__ __launch_bounds__(256) void k_embed(const uint16_t *embed, const uint16_t *mask,
                                               const int32_t *last, const int32_t *ctx_len,
                                               int T, int H, int V, int t_new, int cap,
                                               float *h, const uint16_t *gain, float eps,
                                               uint16_t *x, int32_t *valid) {
    __shared__ float scratch[4];
    const int b = blockIdx.x / T, t = blockIdx.x % T;
    const int n = ctx_len[b], tok = last[b];
    const bool ok = n >= 0 && n <= cap - t_new && tok >= 0 && tok < V;
    if (t == 0 && threadIdx.x == 0) valid[b] = ok ? 1 : 0;
    float *row = h + (size_t)blockIdx.x * H;
    const uint16_t *src = t == 0 ? embed + (size_t)(ok ? tok : 0) * H : mask;
    float s = 0.f;
    for (int i = threadIdx.x; i < H; i += 256) {
        const float v = ok ? bf16_to_f32(src[i]) : 0.f;
        row[i] = v;
        s += v * v;
    }
    s = block_sum_256(s, scratch);
    const float inv = rsqrtf(s / (float)H + eps);
    uint16_t *xr = x + (size_t)blockIdx.x * H;
    for (int i = threadIdx.x; i < H; i += 256) xr[i] = f32_to_bf16(row[i] * inv * bf16_to_f32(gain[i]));
}

// ---------------------------------------------------------------- reduction + residual + RMSNorm
// Phase 1, workgroup per (256 columns, output row): the 4 waves sum interleaved subsets
// of the splits (each lane 4 adjacent columns), combined through LDS in a fixed order,
// so the result is deterministic.  v (+ f when adding) is stored to f, and the
// workgroup's sum of v^2 goes to ssq[r][blockIdx.x].
__global__ __launch_bounds__(256) void k_reduce_rows(const float *part, int splits, int M_out, int N,
                                                     int pair, int add, float *f, float *ssq) {
    __shared__ float4 red[4][64];
    __shared__ float scratch[4];
    const int r = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c0 = blockIdx.x * 256;
    const size_t stride = (size_t)(pair ? 2 * M_out : M_out) * N;
    const float *p = part + (size_t)r * N + c0 + 4 * lane;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int k = wave; k < splits; k += 4) {
        const float4 a = *reinterpret_cast<const float4 *>(p + k * stride);
        s.x += a.x; s.y += a.y; s.z += a.z; s.w += a.w;
        if (pair) {
            const float4 b = *reinterpret_cast<const float4 *>(p + k * stride + (size_t)pair * N);
            s.x += b.x; s.y += b.y; s.z += b.z; s.w += b.w;
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
    if (tid == 0) ssq[(size_t)r * gridDim.x + blockIdx.x] = sq;
}

// Phase 2, workgroup per (256 columns, output row): out = bf16(v * rsqrt(mean v^2 + eps)
// * gain) (+ its bf16 residual in out_lo) at output row map(r).
__global__ __launch_bounds__(256) void k_norm_rows(const float *f, const float *ssq, int nchunk, int N,
                                                   const uint16_t *gain, float eps, uint16_t *out,
                                                   uint16_t *out_lo, int ldo, int map) {
    const int r = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
    int orow = r;
    if (map == 1) {
        if (r % 8 == 0) return;
        orow = (r / 8) * 7 + r % 8 - 1;
    }
    float ss = 0.f;
    for (int i = 0; i < nchunk; i++) ss += ssq[(size_t)r * nchunk + i];
    const float inv = rsqrtf(ss / (float)N + eps);
    const float x = f[(size_t)r * N + c] * inv * bf16_to_f32(gain[c]);
    const uint16_t hb = f32_to_bf16(x);
    out[(size_t)orow * ldo + c] = hb;
    if (out_lo) out_lo[(size_t)orow * ldo + c] = f32_to_bf16(x - bf16_to_f32(hb));
}

// ---------------------------------------------------------------- split-K reduction
// Output row r sums the partial rows r (and r + pair when the GEMM ran over
// [hi rows; lo rows]) over all splits in a fixed order.
__global__ __launch_bounds__(256) void k_reduce(const float *part, int splits, int M, int N,
                                                int pair, int mode, float *of, uint16_t *ob,
                                                uint16_t *ob_lo, int ldo) {
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
            const float act = s / (1.f + expf(-s));          // silu(gate)
            const float v = act * u;
            const uint16_t hb = f32_to_bf16(v);
            ob[(size_t)r * ldo + c] = hb;
            if (ob_lo) ob_lo[(size_t)r * ldo + c] = f32_to_bf16(v - bf16_to_f32(hb));
        }
    }
}

// ---------------------------------------------------------------- q/k norm, rotary, append
// One wave per (row, head).  Lane j < d/2 owns the rotary pair (j, j + d/2).
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
    if (lane < half)
        for (int s = 0; s < a.splits; s++) {
            x1 += x[s * pstride + lane];
            x2 += x[s * pstride + lane + half];
        }
    if (is_q || is_k) {
        const uint16_t *g = is_q ? a.q_norm : a.k_norm;
        const float ss = wave_sum(x1 * x1 + x2 * x2);
        const float inv = rsqrtf(ss / (float)d + a.eps);
        if (lane < half) {
            x1 *= inv * bf16_to_f32(g[lane]);
            x2 *= inv * bf16_to_f32(g[lane + half]);
            // rotation angle pos * theta^(-2 lane / d), evaluated in fp64
            const double ang = (double)pos * pow((double)a.theta, -2.0 * lane / d);
            const float c = (float)cos(ang), s = (float)sin(ang);
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
// k_attn_merge: one workgroup per (query head h, sequence b).  Combines the
// split-window partials of the 8 block rows of head h (log-sum-exp merge) into
// o[b][t][h*d..] (fp32), and contributes head h's share of the convolution taps
//     zp[b][h][t][q] = sum_e W_c[q][h d + e] o[b][t][h][e],   q < 2 n_q,
// so that z_t = W_c . vec(o_t) = sum_h zp[b][h][t][:].
__global__ __launch_bounds__(256) void k_attn_merge(MergeConvArgs a) {
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int d = a.d, T = a.T, G = a.n_q / a.n_kv, QR = G * T, qd = a.n_q * d;
    const int kvh = h / G, hq = h % G;
    const int nch1 = a.n_chunks + 1;
    const int nq2 = 2 * a.n_q;
    extern __shared__ float sm[];
    float *o = sm;                      // [T][d]
    float *w = sm + T * d;              // [T][nch1] merge weights
    float *mx = w + T * nch1;           // [T]
    if (!a.valid[b]) {
        for (int e = tid; e < T * d; e += 256) a.o[((size_t)b * T + e / d) * qd + h * d + e % d] = 0.f;
        for (int e = tid; e < T * nq2; e += 256) a.zp[(((size_t)b * a.n_q + h) * T) * nq2 + e] = 0.f;
        return;
    }
    const int n = a.ctx_len[b];
    const int hi = n + a.t_new;
    const int lo = hi - a.window > 0 ? hi - a.window : 0;
    const int nch_b = ceil_div(hi - lo, a.chunk);
    const float *ml = a.ml + ((size_t)(b * a.n_kv + kvh) * nch1) * QR * 2;
    // all (row, chunk) statistics are loaded in parallel
    for (int e = tid; e < T * nch1; e += 256) {
        const int t = e / nch1, c = e % nch1;
        const bool used = c < nch_b || c == a.n_chunks;
        w[e] = used ? ml[((size_t)c * QR + hq * T + t) * 2] : -INFINITY;
    }
    __syncthreads();
    if (tid < T) {
        float M = -INFINITY;
        for (int c = 0; c < nch1; c++) M = fmaxf(M, w[tid * nch1 + c]);
        mx[tid] = M;
    }
    __syncthreads();
    for (int e = tid; e < T * nch1; e += 256) {
        const int t = e / nch1, c = e % nch1;
        const float m = w[e];
        w[e] = m == -INFINITY ? 0.f : expf(m - mx[t]) * ml[((size_t)c * QR + hq * T + t) * 2 + 1];
    }
    __syncthreads();
    if (tid < T) {
        float L = 0.f;
        for (int c = 0; c < nch1; c++) L += w[tid * nch1 + c];
        mx[tid] = 1.f / L;
    }
    __syncthreads();
    // weights exp(m_c - M) / L multiply the unnormalised partials (l_c already folded in
    // the sum above, so divide it back out per chunk)
    for (int e = tid; e < T * nch1; e += 256) {
        const int t = e / nch1, c = e % nch1;
        const float lc = ml[((size_t)c * QR + hq * T + t) * 2 + 1];
        w[e] = w[e] == 0.f ? 0.f : w[e] / lc * mx[t];
    }
    __syncthreads();
    const float *O = a.O + ((size_t)(b * a.n_kv + kvh) * nch1) * QR * d;
    for (int e = tid; e < T * d; e += 256) {
        const int t = e / d, col = e % d, row = hq * T + t;
        const float *wt = w + t * nch1;
        float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
        int c = 0;
        for (; c + 4 <= nch1; c += 4) {
            acc0 += wt[c] * O[((size_t)c * QR + row) * d + col];
            acc1 += wt[c + 1] * O[((size_t)(c + 1) * QR + row) * d + col];
            acc2 += wt[c + 2] * O[((size_t)(c + 2) * QR + row) * d + col];
            acc3 += wt[c + 3] * O[((size_t)(c + 3) * QR + row) * d + col];
        }
        for (; c < nch1; c++) acc0 += wt[c] * O[((size_t)c * QR + row) * d + col];
        const float acc = (acc0 + acc1) + (acc2 + acc3);
        o[e] = acc;
        a.o[((size_t)b * T + t) * qd + h * d + col] = acc;
    }
    __syncthreads();
    for (int e = tid; e < T * nq2; e += 256) {
        const int t = e / nq2, q = e % nq2;
        const uint16_t *wr = a.w_conv + (size_t)q * qd + h * d;
        const float *ot = o + t * d;
        float s = 0.f;
        for (int i = 0; i < d; i += 8) {
            const u32x4_t wv = *reinterpret_cast<const u32x4_t *>(wr + i);
            s += bf16_to_f32(wv.x & 0xFFFF) * ot[i] + bf16_to_f32(wv.x >> 16) * ot[i + 1];
            s += bf16_to_f32(wv.y & 0xFFFF) * ot[i + 2] + bf16_to_f32(wv.y >> 16) * ot[i + 3];
            s += bf16_to_f32(wv.z & 0xFFFF) * ot[i + 4] + bf16_to_f32(wv.z >> 16) * ot[i + 5];
            s += bf16_to_f32(wv.w & 0xFFFF) * ot[i + 6] + bf16_to_f32(wv.w >> 16) * ot[i + 7];
        }
        a.zp[(((size_t)b * a.n_q + h) * T + t) * nq2 + q] = s;
    }
}

// k_conv_apply: one workgroup per (sequence, block row t):
//   z_t = sum_h zp[b][h][t];  y_{t,h} = z_t[h] o_{t,h} + z_t[n_q + h] o_{t-1,h},  o_{-1} = 0.
__global__ __launch_bounds__(256) void k_conv_apply(MergeConvArgs a) {
    __shared__ float zpart[256];
    __shared__ float z[2 * 256];
    const int b = blockIdx.x / a.T, t = blockIdx.x % a.T, tid = threadIdx.x;
    const int qd = a.n_q * a.d, nq2 = 2 * a.n_q;
    // z_t[q] = sum over heads of zp[b][h][t][q]: (q, head-quarter) per thread
    for (int q0 = 0; q0 < nq2; q0 += 64) {
        const int q = q0 + (tid & 63), part = tid >> 6;
        float s = 0.f;
        if (q < nq2)
            for (int h = part; h < a.n_q; h += 4) s += a.zp[(((size_t)b * a.n_q + h) * a.T + t) * nq2 + q];
        zpart[tid] = s;
        __syncthreads();
        if (tid < 64 && q0 + tid < nq2) z[q0 + tid] = (zpart[tid] + zpart[tid + 64]) + (zpart[tid + 128] + zpart[tid + 192]);
        __syncthreads();
    }
    const float *ot = a.o + ((size_t)b * a.T + t) * qd;
    const float *op = ot - qd;
    uint16_t *Y = a.Y + ((size_t)b * a.T + t) * qd;
    for (int i = tid; i < qd; i += 256) {
        const int h = i / a.d;
        const float prev = t > 0 ? op[i] : 0.f;
        Y[i] = f32_to_bf16(z[h] * ot[i] + z[a.n_q + h] * prev);
    }
}

}  // namespace

hipError_t launch_embed(const uint16_t *embed, const uint16_t *mask_emb, const int32_t *last,
                        const int32_t *ctx_len, int B, int T, int H, int V, int t_new, int cap,
                        float *h, const uint16_t *gain, float eps, uint16_t *x, int32_t *valid,
                        hipStream_t st) {
    hipLaunchKernelGGL(k_embed, dim3(B * T), dim3(256), 0, st, embed, mask_emb, last, ctx_len, T, H,
                       V, t_new, cap, h, gain, eps, x, valid);
    return hipGetLastError();
}

hipError_t launch_reduce_epilogue(const float *part, int splits, int M, int N, int pair,
                                  int mode, float *out_f32, uint16_t *out_bf16,
                                  uint16_t *out_bf16_lo, int ldo, hipStream_t st) {
    const size_t total = (size_t)M * (mode == EPI_SWIGLU_BF16 ? N / 2 : N);
    size_t grid = (total + 255) / 256;
    if (grid > 8192) grid = 8192;
    hipLaunchKernelGGL(k_reduce, dim3((unsigned)grid), dim3(256), 0, st, part, splits, M, N, pair,
                       mode, out_f32, out_bf16, out_bf16_lo, ldo);
    return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const RopeArgs &a, hipStream_t st) {
    dim3 grid(a.B * (a.T + a.t_new), a.n_q + 2 * a.n_kv);
    hipLaunchKernelGGL(k_qk_norm_rope, grid, dim3(64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_merge_conv(const MergeConvArgs &a, hipStream_t st) {
    const size_t lds = (size_t)(a.T * a.d + a.T * (a.n_chunks + 1) + a.T) * 4;
    hipLaunchKernelGGL(k_attn_merge, dim3(a.n_q, a.B), dim3(256), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_conv_apply, dim3(a.B * a.T), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_reduce_norm(const float *part, int splits, int M_out, int N, int pair, int add,
                              float *f, float *ssq, const uint16_t *gain, float eps, uint16_t *out,
                              uint16_t *out_lo, int ldo, int map, hipStream_t st) {
    const dim3 grid(N / 256, M_out);
    hipLaunchKernelGGL(k_reduce_rows, grid, dim3(256), 0, st, part, splits, M_out, N, pair, add, f,
                       ssq);
    if (out)
        hipLaunchKernelGGL(k_norm_rows, grid, dim3(256), 0, st, f, ssq, N / 256, N, gain, eps, out,
                           out_lo, ldo, map);
    return hipGetLastError();
}
