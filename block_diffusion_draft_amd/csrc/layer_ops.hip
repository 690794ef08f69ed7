// Per-layer elementwise and row kernels of the draft step, gfx950:
//   block assembly, RMSNorm, split-K reduction with fused epilogues (residual add,
//   SwiGLU), per-head q/k RMSNorm + rotary embedding + KV-cache append, and the
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
__global__ __launch_bounds__(256) void k_embed(const uint16_t *embed, const uint16_t *mask,
                                               const int32_t *last, const int32_t *ctx_len,
                                               int T, int H, int V, int t_new, int cap,
                                               float *h, int32_t *valid) {
    const int b = blockIdx.x / T, t = blockIdx.x % T;
    const int n = ctx_len[b], tok = last[b];
    const bool ok = n >= 0 && n <= cap - t_new && tok >= 0 && tok < V;
    if (t == 0 && threadIdx.x == 0) valid[b] = ok ? 1 : 0;
    float *row = h + (size_t)blockIdx.x * H;
    const uint16_t *src = t == 0 ? embed + (size_t)(ok ? tok : 0) * H : mask;
    for (int i = threadIdx.x; i < H; i += 256) row[i] = ok ? bf16_to_f32(src[i]) : 0.f;
}

// ---------------------------------------------------------------- RMSNorm -> bf16
__global__ __launch_bounds__(256) void k_rmsnorm(const float *in, int H, int per, int in_group,
                                                 int in_off, const uint16_t *gain, float eps,
                                                 uint16_t *out, int ldo) {
    __shared__ float scratch[4];
    const int r = blockIdx.x;
    const float *x = in + ((size_t)(r / per) * in_group + in_off + r % per) * H;
    float ss = 0.f;
    for (int i = threadIdx.x; i < H; i += 256) ss += x[i] * x[i];
    ss = block_sum_256(ss, scratch);
    const float inv = rsqrtf(ss / (float)H + eps);
    uint16_t *o = out + (size_t)r * ldo;
    for (int i = threadIdx.x; i < H; i += 256) o[i] = f32_to_bf16(x[i] * inv * bf16_to_f32(gain[i]));
}

// ---------------------------------------------------------------- split-K reduction
__global__ __launch_bounds__(256) void k_reduce(const float *part, int splits, int M, int N,
                                                int mode, float *of, uint16_t *ob, int ldo) {
    const int Nout = mode == EPI_SWIGLU_BF16 ? N / 2 : N;
    const size_t total = (size_t)M * Nout;
    const size_t stride = (size_t)M * N;
    for (size_t e = blockIdx.x * 256ull + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
        const int r = (int)(e / Nout), c = (int)(e % Nout);
        const float *p = part + (size_t)r * N + c;
        float s = 0.f;
        for (int k = 0; k < splits; k++) s += p[k * stride];
        if (mode == EPI_STORE_F32) {
            of[(size_t)r * ldo + c] = s;
        } else if (mode == EPI_ADD_F32) {
            of[(size_t)r * ldo + c] += s;
        } else if (mode == EPI_STORE_BF16) {
            ob[(size_t)r * ldo + c] = f32_to_bf16(s);
        } else {
            float u = 0.f;
            for (int k = 0; k < splits; k++) u += p[k * stride + Nout];
            const float act = s / (1.f + expf(-s));          // silu(gate)
            ob[(size_t)r * ldo + c] = f32_to_bf16(act * u);
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
    float x1 = 0.f, x2 = 0.f;
    if (lane < half) { x1 = x[lane]; x2 = x[lane + half]; }
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
// One workgroup per (sequence, block row t): merges the split-window attention
// partials of rows t and t-1 for every query head, then
//   z_t = W_c . vec(o_t),  y_{t,h} = z_t[h] o_{t,h} + z_t[n_q + h] o_{t-1,h}.
__global__ __launch_bounds__(256) void k_merge_conv(MergeConvArgs a) {
    extern __shared__ float sm[];
    const int b = blockIdx.x / a.T, t = blockIdx.x % a.T;
    const int tid = threadIdx.x;
    const int qd = a.n_q * a.d, G = a.n_q / a.n_kv, QR = G * a.T;
    const int nch1 = a.n_chunks + 1;
    float *o_cur = sm;                 // [qd]
    float *o_prev = sm + qd;           // [qd]
    float *wts = sm + 2 * qd;          // [2][n_q][nch1] merge weights
    float *z = wts + 2 * a.n_q * nch1; // [2 n_q]
    uint16_t *Y = a.Y + (size_t)blockIdx.x * qd;
    if (!a.valid[b]) {
        for (int i = tid; i < qd; i += 256) Y[i] = 0;
        return;
    }
    const int n = a.ctx_len[b];
    const int hi = n + a.t_new;
    const int lo = hi - a.window > 0 ? hi - a.window : 0;
    const int nch_b = ceil_div(hi - lo, a.chunk);

    // merge weights exp(m_c - M) / L for (row t, row t-1) x heads
    for (int p = tid; p < 2 * a.n_q; p += 256) {
        const int which = p / a.n_q, h = p % a.n_q;
        const int tt = t - which;
        float *w = wts + (size_t)p * nch1;
        if (tt < 0) {
            for (int c = 0; c < nch1; c++) w[c] = 0.f;
            continue;
        }
        const int kvh = h / G, row = (h % G) * a.T + tt;
        const float *ml = a.ml + ((size_t)(b * a.n_kv + kvh) * nch1) * QR * 2;
        float M = -INFINITY;
        for (int c = 0; c < nch1; c++) {
            if (c >= nch_b && c != a.n_chunks) continue;
            M = fmaxf(M, ml[((size_t)c * QR + row) * 2]);
        }
        float L = 0.f;
        for (int c = 0; c < nch1; c++) {
            if (c >= nch_b && c != a.n_chunks) { w[c] = 0.f; continue; }
            const float e = expf(ml[((size_t)c * QR + row) * 2] - M);
            w[c] = e;
            L += e * ml[((size_t)c * QR + row) * 2 + 1];
        }
        const float invL = 1.f / L;
        for (int c = 0; c < nch1; c++) w[c] *= invL;
    }
    __syncthreads();
    for (int e = tid; e < 2 * qd; e += 256) {
        const int which = e / qd, i = e % qd;
        const int tt = t - which;
        float acc = 0.f;
        if (tt >= 0) {
            const int h = i / a.d, col = i % a.d;
            const int kvh = h / G, row = (h % G) * a.T + tt;
            const float *w = wts + (size_t)(which * a.n_q + h) * nch1;
            const float *O = a.O + ((size_t)(b * a.n_kv + kvh) * nch1) * QR * a.d;
            for (int c = 0; c < nch1; c++)
                if (w[c] != 0.f) acc += w[c] * O[((size_t)c * QR + row) * a.d + col];
        }
        (which == 0 ? o_cur : o_prev)[i] = acc;
    }
    __syncthreads();
    // z = W_c . o_t : wave w computes outputs w, w+4, ...
    const int lane = tid & 63, wave = tid >> 6;
    for (int q = wave; q < 2 * a.n_q; q += 4) {
        const uint16_t *wr = a.w_conv + (size_t)q * qd;
        float s = 0.f;
        for (int i = lane; i < qd; i += 64) s += bf16_to_f32(wr[i]) * o_cur[i];
        s = wave_sum(s);
        if (lane == 0) z[q] = s;
    }
    __syncthreads();
    for (int i = tid; i < qd; i += 256) {
        const int h = i / a.d;
        Y[i] = f32_to_bf16(z[h] * o_cur[i] + z[a.n_q + h] * o_prev[i]);
    }
}

}  // namespace

hipError_t launch_embed(const uint16_t *embed, const uint16_t *mask_emb, const int32_t *last,
                        const int32_t *ctx_len, int B, int T, int H, int V, int t_new, int cap,
                        float *h, int32_t *valid, hipStream_t st) {
    hipLaunchKernelGGL(k_embed, dim3(B * T), dim3(256), 0, st, embed, mask_emb, last, ctx_len,
                       T, H, V, t_new, cap, h, valid);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const float *in, int R, int H, int per, int in_group, int in_off,
                          const uint16_t *gain, float eps, uint16_t *out, int ldo,
                          hipStream_t st) {
    hipLaunchKernelGGL(k_rmsnorm, dim3(R), dim3(256), 0, st, in, H, per, in_group, in_off, gain,
                       eps, out, ldo);
    return hipGetLastError();
}

hipError_t launch_reduce_epilogue(const float *part, int splits, int M, int N, int mode,
                                  float *out_f32, uint16_t *out_bf16, int ldo, hipStream_t st) {
    const size_t total = (size_t)M * (mode == EPI_SWIGLU_BF16 ? N / 2 : N);
    size_t grid = (total + 255) / 256;
    if (grid > 8192) grid = 8192;
    hipLaunchKernelGGL(k_reduce, dim3((unsigned)grid), dim3(256), 0, st, part, splits, M, N, mode,
                       out_f32, out_bf16, ldo);
    return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const RopeArgs &a, hipStream_t st) {
    dim3 grid(a.B * (a.T + a.t_new), a.n_q + 2 * a.n_kv);
    hipLaunchKernelGGL(k_qk_norm_rope, grid, dim3(64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_merge_conv(const MergeConvArgs &a, hipStream_t st) {
    const size_t lds = (size_t)(2 * a.n_q * a.d + 2 * a.n_q * (a.n_chunks + 1) + 2 * a.n_q) * 4;
    hipLaunchKernelGGL(k_merge_conv, dim3(a.B * a.T), dim3(256), lds, st, a);
    return hipGetLastError();
}
