// Split-window grouped-query attention of the 8 block queries, gfx950.
//
// FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", spec table "Draft" row: 32 query /
// 8 KV heads of 128 and a sliding window of 2048; section "How it is used": the
// whole block is drafted in one pass.  Every block query attends to the last
// `window` cache rows (the rows appended this step included) and to all 8 block
// rows (bidirectional within the block), scale 1/sqrt(d), softmax over keys.
//
// Decomposition: workgroup = (key chunk, KV head, sequence).  The G query heads
// that share a KV head and the 8 block positions form QR = 8 G query rows, so
// S = Q K^T and O = P V are MFMA tiles (16x16x32 bf16, fp32 accumulate).  Keys are
// processed 64 at a time with an online softmax; the workgroup writes its
// unnormalised O with the running (max, sum), and the merge kernel combines the
// chunks (log-sum-exp merge).  The last chunk index holds the 8 block rows.
// P is rounded to bf16 for the MFMA and the row sum is taken over the same
// rounded values, so the normalisation matches the products.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int KT = 64;           // keys per inner step
constexpr int MAXQR = 32;        // query rows per workgroup (G <= 4)

__global__ __launch_bounds__(256) void k_attention(AttnArgs a) {
    const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int d = a.d, G = a.n_q / a.n_kv, QR = G * a.T;
    const int RTQ = ceil_div(QR, 16);
    if (!a.valid[b]) return;
    const int n = a.ctx_len[b];
    const int hi = n + a.t_new;
    const int lo = hi - a.window > 0 ? hi - a.window : 0;
    const int nch_b = ceil_div(hi - lo, a.chunk);
    const bool blk = c == a.n_chunks;
    if (!blk && c >= nch_b) return;
    int k0, nkeys;
    if (blk) {
        k0 = 0;
        nkeys = a.T;
    } else {
        k0 = lo + c * a.chunk;
        nkeys = min(a.chunk, hi - k0);
    }

    const int DS = d + 8;                   // padded LDS row stride (bf16)
    __shared__ __align__(16) uint16_t Qs[MAXQR * (128 + 8)];
    __shared__ __align__(16) uint16_t Ks[KT * (128 + 8)];
    __shared__ __align__(16) uint16_t Vt[128 * (KT + 8)];
    __shared__ __align__(16) uint16_t Ps[MAXQR * (KT + 8)];
    __shared__ float Ss[MAXQR * KT];
    __shared__ float m_run[MAXQR], l_run[MAXQR], alpha[MAXQR];

    // Q rows: row = hq * T + t  <-  Q[b][t][kvh*G + hq][:]
    for (int e = tid; e < RTQ * 16 * (d / 8); e += 256) {
        const int row = e / (d / 8), q8 = e % (d / 8);
        u32x4_t v = {0, 0, 0, 0};
        if (row < QR) {
            const int hq = row / a.T, t = row % a.T;
            const uint16_t *src = a.Q + (((size_t)b * a.T + t) * a.n_q + kvh * G + hq) * d + 8 * q8;
            v = *reinterpret_cast<const u32x4_t *>(src);
        }
        *reinterpret_cast<u32x4_t *>(&Qs[row * DS + 8 * q8]) = v;
    }
    if (tid < MAXQR) {
        m_run[tid] = -INFINITY;
        l_run[tid] = 0.f;
    }
    const float scale = rsqrtf((float)d);

    // O accumulators: tiles (rt, dt), rt < RTQ, dt < d/16, distributed over waves
    const int nto = RTQ * (d / 16);
    f32x4_t acc[4];
#pragma unroll
    for (int u = 0; u < 4; u++) acc[u] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    const int g = lane >> 4, cl = lane & 15;

    for (int kk = 0; kk < nkeys; kk += KT) {
        const int nk = min(KT, nkeys - kk);
        __syncthreads();
        // stage K rows and V^T for keys kk .. kk+nk-1
        for (int e = tid; e < KT * (d / 8); e += 256) {
            const int j = e / (d / 8), q8 = e % (d / 8);
            u32x4_t kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
            if (j < nk) {
                const uint16_t *ks, *vs;
                if (blk) {
                    const size_t off = (((size_t)b * a.T + j) * a.n_kv + kvh) * d + 8 * q8;
                    ks = a.Kb + off;
                    vs = a.Vb + off;
                } else {
                    const size_t off = (((size_t)b * a.n_kv + kvh) * a.cap + (k0 + kk + j)) * d + 8 * q8;
                    ks = a.k_cache + off;
                    vs = a.v_cache + off;
                }
                kv = *reinterpret_cast<const u32x4_t *>(ks);
                vv = *reinterpret_cast<const u32x4_t *>(vs);
            }
            *reinterpret_cast<u32x4_t *>(&Ks[j * DS + 8 * q8]) = kv;
            const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                Vt[(8 * q8 + 2 * i) * (KT + 8) + j] = (uint16_t)(w4[i] & 0xFFFF);
                Vt[(8 * q8 + 2 * i + 1) * (KT + 8) + j] = (uint16_t)(w4[i] >> 16);
            }
        }
        __syncthreads();
        // S = Q K^T (scaled, masked)
        for (int ti = wave; ti < RTQ * 4; ti += 4) {
            const int rt = ti >> 2, kt = ti & 3;
            f32x4_t s = {0.f, 0.f, 0.f, 0.f};
            for (int ks = 0; ks < d / 32; ks++) {
                const u32x4_t qa = *reinterpret_cast<const u32x4_t *>(&Qs[(rt * 16 + cl) * DS + ks * 32 + 8 * g]);
                const u32x4_t kb = *reinterpret_cast<const u32x4_t *>(&Ks[(kt * 16 + cl) * DS + ks * 32 + 8 * g]);
                s = mfma16x16x32(qa, kb, s);
            }
            const int key = kt * 16 + cl;
#pragma unroll
            for (int v = 0; v < 4; v++)
                Ss[(rt * 16 + 4 * g + v) * KT + key] = key < nk ? s[v] * scale : -INFINITY;
        }
        __syncthreads();
        // online softmax: 8 threads per query row, 8 keys each
        if ((tid >> 3) < RTQ * 16) {
            const int row = tid >> 3, part = tid & 7;
            float mx = -INFINITY;
            float sv[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                sv[i] = Ss[row * KT + part * 8 + i];
                mx = fmaxf(mx, sv[i]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 1, WAVE));
            mx = fmaxf(mx, __shfl_xor(mx, 2, WAVE));
            mx = fmaxf(mx, __shfl_xor(mx, 4, WAVE));
            const float m_old = m_run[row];
            const float m_new = fmaxf(m_old, mx);
            float ls = 0.f;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const float p = sv[i] == -INFINITY ? 0.f : expf(sv[i] - m_new);
                const uint16_t pb = f32_to_bf16(p);
                Ps[row * (KT + 8) + part * 8 + i] = pb;
                ls += bf16_to_f32(pb);
            }
            ls += __shfl_xor(ls, 1, WAVE);
            ls += __shfl_xor(ls, 2, WAVE);
            ls += __shfl_xor(ls, 4, WAVE);
            if (part == 0) {
                const float al = m_old == -INFINITY ? 0.f : expf(m_old - m_new);
                alpha[row] = al;
                l_run[row] = l_run[row] * al + ls;
                m_run[row] = m_new;
            }
        }
        __syncthreads();
        // O = alpha O + P V
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int ti = wave + 4 * u;
            if (ti < nto) {
                const int rt = ti / (d / 16), dt = ti % (d / 16);
#pragma unroll
                for (int v = 0; v < 4; v++) acc[u][v] *= alpha[rt * 16 + 4 * g + v];
                for (int ks = 0; ks < KT / 32; ks++) {
                    const u32x4_t pa = *reinterpret_cast<const u32x4_t *>(&Ps[(rt * 16 + cl) * (KT + 8) + ks * 32 + 8 * g]);
                    const u32x4_t vb = *reinterpret_cast<const u32x4_t *>(&Vt[(dt * 16 + cl) * (KT + 8) + ks * 32 + 8 * g]);
                    acc[u] = mfma16x16x32(pa, vb, acc[u]);
                }
            }
        }
    }
    __syncthreads();
    const int nch1 = a.n_chunks + 1;
    const size_t base = ((size_t)(b * a.n_kv + kvh) * nch1 + c) * QR;
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const int ti = wave + 4 * u;
        if (ti < nto) {
            const int rt = ti / (d / 16), dt = ti % (d / 16);
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int row = rt * 16 + 4 * g + v;
                if (row < QR) a.O[(base + row) * d + dt * 16 + cl] = acc[u][v];
            }
        }
    }
    if (tid < QR) {
        a.ml[(base + tid) * 2] = m_run[tid];
        a.ml[(base + tid) * 2 + 1] = l_run[tid];
    }
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, hipStream_t st) {
    dim3 grid(a.n_chunks + 1, a.n_kv, a.B);
    hipLaunchKernelGGL(k_attention, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}
