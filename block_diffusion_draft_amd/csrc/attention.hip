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
// K and V rows sit in LDS as loaded (key-major); the V operand of O = P V (keys
// along the MFMA's k) comes from gfx950's transposing LDS read, which hands each
// lane 4 consecutive keys of one column.  O leaves through LDS as whole rows.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int KT = 64;           // keys per inner step
typedef short v4i16_t __attribute__((ext_vector_type(4)));
constexpr int MAXQR = 32;        // query rows per workgroup (G <= 4)

template <int D>
__global__ __launch_bounds__(256) void k_attention(AttnArgs a) {
    const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int d = D;                    // head dim as a constant: fixed trip counts
    const int G = a.n_q / a.n_kv, QR = G * a.T;
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

    const int DS = d + 8;                   // padded LDS row stride of Q and K (bf16)
    constexpr int VS = D + 16;              // V row stride: 4 rows of a transposing read
                                            // land 8 banks apart (no conflicts)
    constexpr int OS = D + 4;               // fp32 row stride of the output staging
    // K and V rows; after the key loop the same bytes stage O (fp32 [QR][OS])
    __shared__ __align__(16) uint16_t KVs[KT * (128 + 8) + KT * (128 + 16)];
    uint16_t *Ks = KVs, *Vs = KVs + KT * (128 + 8);
    float *Os = reinterpret_cast<float *>(KVs);
    __shared__ __align__(16) uint16_t Qs[MAXQR * (128 + 8)];
    // scores (fp32) and, once every score of the step is in registers, the bf16 P rows
    // in the same bytes (keeps the workgroup at 53 KB of LDS: 3 per CU)
    __shared__ __align__(16) float Ss[MAXQR * KT];
    uint16_t *Ps = reinterpret_cast<uint16_t *>(Ss);
    static_assert(MAXQR * (KT + 8) * 2 <= MAXQR * KT * 4, "P fits in the score buffer");
    __shared__ float m_run[MAXQR], l_run[MAXQR], alpha[MAXQR];
    static_assert(MAXQR * (128 + 4) * 4 <= (KT * (128 + 8) + KT * (128 + 16)) * 2, "O staging fits");

    // Q rows: row = hq * T + t  <-  Q[b][t][kvh*G + hq][:] (rows >= QR: zeros)
    {
        constexpr int QPT = MAXQR * (d / 8) / 256;
        u32x4_t qv[QPT];
#pragma unroll
        for (int i = 0; i < QPT; i++) {
            const int e = tid + 256 * i;
            const int row = e / (d / 8), q8 = e % (d / 8);
            const int rc = min(row, QR - 1);
            const int hq = rc / a.T, t = rc % a.T;
            qv[i] = *reinterpret_cast<const u32x4_t *>(
                a.Q + (((size_t)b * a.T + t) * a.n_q + kvh * G + hq) * d + 8 * q8);
        }
#pragma unroll
        for (int i = 0; i < QPT; i++) {
            const int e = tid + 256 * i;
            const int row = e / (d / 8), q8 = e % (d / 8);
            if (row < RTQ * 16)
                *reinterpret_cast<u32x4_t *>(&Qs[row * DS + 8 * q8]) =
                    row < QR ? qv[i] : (u32x4_t){0, 0, 0, 0};
        }
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

    // K and V rows of keys kk .. kk + KT - 1 into registers (rows past the chunk clamped
    // to a real row; their values are replaced by zeros when staged)
    constexpr int SPT = KT * (d / 8) / 256;              // 16-byte vectors per thread
    u32x4_t kv[SPT], vv[SPT];
    auto load_kv = [&](int kk) {
        const int nk = min(KT, nkeys - kk);
#pragma unroll
        for (int i = 0; i < SPT; i++) {
            const int e = tid + 256 * i;
            const int j = e / (d / 8), q8 = e % (d / 8);
            const int jc = min(j, nk - 1);
            size_t off;
            const uint16_t *kbase, *vbase;
            if (blk) {
                off = (((size_t)b * a.T + jc) * a.n_kv + kvh) * d + 8 * q8;
                kbase = a.Kb;
                vbase = a.Vb;
            } else {
                off = (((size_t)b * a.n_kv + kvh) * a.cap + (k0 + kk + jc)) * d + 8 * q8;
                kbase = a.k_cache;
                vbase = a.v_cache;
            }
            kv[i] = *reinterpret_cast<const u32x4_t *>(kbase + off);
            vv[i] = *reinterpret_cast<const u32x4_t *>(vbase + off);
        }
    };
    load_kv(0);
    for (int kk = 0; kk < nkeys; kk += KT) {
        const int nk = min(KT, nkeys - kk);
        __syncthreads();
        // stage this step's K rows and V rows, then issue the next step's loads so that
        // they land while this step is multiplied
#pragma unroll
        for (int i = 0; i < SPT; i++) {
            const int e = tid + 256 * i;
            const int j = e / (d / 8), q8 = e % (d / 8);
            const bool in = j < nk;
            const u32x4_t z = {0, 0, 0, 0};
            *reinterpret_cast<u32x4_t *>(&Ks[j * DS + 8 * q8]) = in ? kv[i] : z;
            *reinterpret_cast<u32x4_t *>(&Vs[j * VS + 8 * q8]) = in ? vv[i] : z;
        }
        if (kk + KT < nkeys) load_kv(kk + KT);
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
        const bool srow = (tid >> 3) < RTQ * 16;
        float sv[8];
        if (srow) {
#pragma unroll
            for (int i = 0; i < 8; i++) sv[i] = Ss[(tid >> 3) * KT + (tid & 7) * 8 + i];
        }
        __syncthreads();                    // every score read before P overwrites them
        if (srow) {
            const int row = tid >> 3, part = tid & 7;
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 8; i++) mx = fmaxf(mx, sv[i]);
            mx = fmaxf(mx, xor_lane<1>(mx));
            mx = fmaxf(mx, xor_lane<2>(mx));
            mx = fmaxf(mx, xor_lane<4>(mx));
            const float m_old = m_run[row];
            const float m_new = fmaxf(m_old, mx);
            float ls = 0.f;
            uint32_t pw[4];
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const float p0 = sv[i] == -INFINITY ? 0.f : expf(sv[i] - m_new);
                const float p1 = sv[i + 1] == -INFINITY ? 0.f : expf(sv[i + 1] - m_new);
                const uint16_t b0 = f32_to_bf16(p0), b1 = f32_to_bf16(p1);
                pw[i / 2] = (uint32_t)b0 | ((uint32_t)b1 << 16);
                ls += bf16_to_f32(b0);
                ls += bf16_to_f32(b1);
            }
            *reinterpret_cast<u32x4_t *>(&Ps[row * (KT + 8) + part * 8]) = (u32x4_t){pw[0], pw[1], pw[2], pw[3]};
            ls += xor_lane<1>(ls);
            ls += xor_lane<2>(ls);
            ls += xor_lane<4>(ls);
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
                    // lane (g, cl) needs V[ks 32 + 8 g + 0..7][dt 16 + cl]: two transposing
                    // reads; source lane (k, q) = (cl >> 2, cl & 3) names row base + k,
                    // columns 4 q .. 4 q + 3, and lane cl receives column cl of the 4 rows
                    const uint16_t *vrow = &Vs[(ks * 32 + 8 * g + (cl >> 2)) * VS + dt * 16 + 4 * (cl & 3)];
                    const v4i16_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16_t *)(vrow));
                    const v4i16_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16_t *)(vrow + 4 * VS));
                    const u32x4_t vb = {(uint32_t)(uint16_t)v0.x | ((uint32_t)(uint16_t)v0.y << 16),
                                        (uint32_t)(uint16_t)v0.z | ((uint32_t)(uint16_t)v0.w << 16),
                                        (uint32_t)(uint16_t)v1.x | ((uint32_t)(uint16_t)v1.y << 16),
                                        (uint32_t)(uint16_t)v1.z | ((uint32_t)(uint16_t)v1.w << 16)};
                    acc[u] = mfma16x16x32(pa, vb, acc[u]);
                }
            }
        }
    }
    __syncthreads();
    // O tiles -> LDS rows, then whole rows to global (16 bytes per lane)
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const int ti = wave + 4 * u;
        if (ti < nto) {
            const int rt = ti / (d / 16), dt = ti % (d / 16);
#pragma unroll
            for (int v = 0; v < 4; v++) Os[(rt * 16 + 4 * g + v) * OS + dt * 16 + cl] = acc[u][v];
        }
    }
    __syncthreads();
    const int nch1 = a.n_chunks + 1;
    const size_t base = ((size_t)(b * a.n_kv + kvh) * nch1 + c) * QR;
    for (int e = tid; e < QR * (d / 4); e += 256) {
        const int row = e / (d / 4), c4 = e % (d / 4);
        *reinterpret_cast<float4 *>(&a.O[(base + row) * d + 4 * c4]) =
            *reinterpret_cast<const float4 *>(&Os[row * OS + 4 * c4]);
    }
    if (tid < QR) {
        a.ml[(base + tid) * 2] = m_run[tid];
        a.ml[(base + tid) * 2 + 1] = l_run[tid];
    }
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, hipStream_t st) {
    dim3 grid(a.n_chunks + 1, a.n_kv, a.B);
    if (a.d == 128) hipLaunchKernelGGL(k_attention<128>, grid, dim3(256), 0, st, a);
    else if (a.d == 64) hipLaunchKernelGGL(k_attention<64>, grid, dim3(256), 0, st, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}
