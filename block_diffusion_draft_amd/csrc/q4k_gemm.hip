// Q4_K dequantize-fused GEMM for few activation rows (the draft's fc, q/k/v/o and
// SwiGLU matrices at M = 8 or 16 rows per sequence), gfx950.
//
// Format (FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", "Weights" row: the draft's
// matrices in Q4_K): 144-byte super-blocks of 256 weights along K, with
// w = d * sc_j * q - dmin * m_j for sub-block j (32 weights), q in 0..15.
//
// Per super-block and output column n the contribution to row r is
//     sum_j [ d sc_j sum_k x_rk q_k  -  dmin m_j S_rj ],   S_rj = sum_{k in j} x_rk.
// The integer codes enter the MFMA exactly: a nibble q becomes the bf16 value
// 128 + q (bit pattern 0x4300 | q), so one 16x16x32 MFMA per sub-block gives
// D_j = sum_k x_k (128 + q_k) = 128 S_j + sum_k x_k q_k with fp32 accumulation.
// Hence the column's super-block term is
//     d * sum_j sc_j D_j  -  sum_j (128 d sc_j + dmin m_j) S_rj ,
// and the only roundings are those of the fp32 accumulation.
//
// Work split: a workgroup (4 waves) owns 4 column tiles of 16 and one range of
// super-blocks (split-K).  Its activation rows for that range are staged once in
// LDS, already in MFMA lane order, with the per-sub-block row sums next to them.
// Each wave streams its 16 columns' super-blocks straight from HBM: lane l reads
// column (l & 15), 8 quant bytes per 64-weight chunk at offset 8 (l >> 4), and
// the 16-byte header.  Partial sums go to a [split][M][N] fp32 buffer that the
// epilogue kernel reduces in a fixed order (deterministic, no atomics).
#include "common.h"
#include "kernels.h"

namespace {

constexpr int MAX_RT = 4;          // row tiles of 16 per workgroup

// Reorder 8 consecutive bf16 x0..x7 (as 4 dwords) into the slot order the
// nibble decode produces: (x0,x2) (x1,x3) (x4,x6) (x5,x7).
__device__ __forceinline__ u32x4_t permute_slots(u32x4_t v) {
    u32x4_t o;
    o.x = (v.x & 0xFFFFu) | (v.y << 16);
    o.y = (v.x >> 16) | (v.y & 0xFFFF0000u);
    o.z = (v.z & 0xFFFFu) | (v.w << 16);
    o.w = (v.z >> 16) | (v.w & 0xFFFF0000u);
    return o;
}

// 8 nibbles (2 dwords of bytes b0..b7, low or high nibble already shifted to
// bits 0..3 of each byte) -> 8 bf16 values 128 + q in slot order
// (b0,b2) (b1,b3) (b4,b6) (b5,b7).
__device__ __forceinline__ u32x4_t nibbles_to_bf16(uint32_t p0, uint32_t p1) {
    const uint32_t M = 0x000F000Fu, C = 0x43004300u;
    u32x4_t b;
    b.x = (p0 & M) | C;
    b.y = ((p0 >> 8) & M) | C;
    b.z = (p1 & M) | C;
    b.w = ((p1 >> 8) & M) | C;
    return b;
}

// Weight bytes of one super-block for one lane: the 16-byte header of its column
// and its 8 quant bytes in each of the 4 64-weight chunks.
struct WStage {
    u32x4_t hdr;
    u32x2_t q[4];
};

__device__ __forceinline__ WStage load_stage(const unsigned char *blk, int g) {
    WStage s;
    s.hdr = *reinterpret_cast<const u32x4_t *>(blk);
#pragma unroll
    for (int c = 0; c < 4; c++) s.q[c] = *reinterpret_cast<const u32x2_t *>(blk + 16 + 32 * c + 8 * g);
    return s;
}

constexpr int PD = 4;              // super-blocks in flight per wave
constexpr int KB_LDS = 4;          // super-blocks x row tiles staged per workgroup

template <int RT>
__global__ __launch_bounds__(256) void k_q4k_gemm(Q4kGemmArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = blockIdx.y;
    const int row0 = blockIdx.z * (RT * 16);
    const int rt_n = min(RT, ceil_div(a.M - row0, 16));
    const int sb0 = split * a.kb_per;
    const int nsb = min(a.kb_per, a.KB - sb0);        // >= 1 by construction of the grid

    // column tile of this wave; a tile past N (last workgroup only) computes on
    // the last valid tile and stores nothing
    const int ntile = a.N / 16;
    const int ct = blockIdx.x * 4 + wave;
    const bool active = ct < ntile;
    const int cte = active ? ct : ntile - 1;
    const int c16 = cte * 16;
    const int n = c16 + (lane & 15);
    const int g = lane >> 4;
    // weight segment (segments are multiples of 16 columns); no dynamic indexing
    const int si = (a.nseg > 1 && c16 >= a.seg_end[0]) + (a.nseg > 2 && c16 >= a.seg_end[1]);
    const unsigned char *wseg = si == 0 ? a.w[0] : (si == 1 ? a.w[1] : a.w[2]);
    const int nbase = si == 0 ? 0 : (si == 1 ? a.seg_end[0] : a.seg_end[1]);
    const unsigned char *wrow = wseg + ((size_t)(n - nbase) * a.KB + sb0) * 144;
    auto blk = [&](int i) { return wrow + (size_t)min(i, nsb - 1) * 144; };

    // 1) activation loads for the LDS stage (at most 8 per thread)
    constexpr int MAXA = 2 * KB_LDS;
    const int entries = nsb * 8 * rt_n * 64;
    // branch-free: indices are clamped into range and out-of-range values zeroed
    u32x4_t av[MAXA];
#pragma unroll
    for (int i = 0; i < MAXA; i++) {
        const int e = min(tid + 256 * i, entries - 1);
        const int ln = e & 63;
        int rest = e >> 6;
        const int rt = rest % rt_n; rest /= rt_n;
        const int j = rest & 7, sbi = rest >> 3;
        const int row = row0 + rt * 16 + (ln & 15);
        const size_t k = (size_t)(sb0 + sbi) * 256 + 32 * j + 8 * (ln >> 4);
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(a.A + (size_t)min(row, a.M - 1) * a.lda + k);
        const bool ok = row < a.M && tid + 256 * i < entries;
        av[i] = ok ? v : (u32x4_t){0u, 0u, 0u, 0u};
    }
    // 2) weight stream starts before the stage completes
    WStage st[PD];
#pragma unroll
    for (int u = 0; u < PD - 1; u++) st[u] = load_stage(blk(u), g);

    // 3) activations -> LDS in MFMA lane order, with per-sub-block row sums
    u32x4_t *A_lds = reinterpret_cast<u32x4_t *>(lds);      // [nsb][8][rt_n][64]
    float *S_lds = reinterpret_cast<float *>(lds + (size_t)nsb * 8 * rt_n * 64 * 16);  // [nsb][8][rt_n*16]
#pragma unroll
    for (int i = 0; i < MAXA; i++) {
        const int e = tid + 256 * i;
        if (e < entries) {                               // uniform per wave
            const u32x4_t v = av[i];
            const int ln = e & 63;
            int rest = e >> 6;
            const int rt = rest % rt_n; rest /= rt_n;
            const int j = rest & 7, sbi = rest >> 3;
            float s = 0.f;
            s += bf16_to_f32(v.x & 0xFFFF) + bf16_to_f32(v.x >> 16);
            s += bf16_to_f32(v.y & 0xFFFF) + bf16_to_f32(v.y >> 16);
            s += bf16_to_f32(v.z & 0xFFFF) + bf16_to_f32(v.z >> 16);
            s += bf16_to_f32(v.w & 0xFFFF) + bf16_to_f32(v.w >> 16);
            s += __shfl_xor(s, 16, WAVE);
            s += __shfl_xor(s, 32, WAVE);
            A_lds[e] = permute_slots(v);
            if ((ln >> 4) == 0) S_lds[((sbi * 8 + j) * rt_n + rt) * 16 + (ln & 15)] = s;
        }
    }
    __syncthreads();

    f32x4_t acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; rt++) acc[rt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    for (int s0 = 0; s0 < nsb; s0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; u++) {
            const int sbi = s0 + u;
            st[(u + PD - 1) % PD] = load_stage(blk(sbi + PD - 1), g);
            const bool live = sbi < nsb;
            const int sbl = live ? sbi : 0;              // stays inside the LDS stage
            const WStage &w = st[u];
            const float d = half_bits_to_f32(w.hdr.x & 0xFFFF);
            const float dmin = half_bits_to_f32(w.hdr.x >> 16);
            const uint32_t s0w = w.hdr.y, s1w = w.hdr.z, s2w = w.hdr.w;
            const uint32_t sc_lo = s0w & 0x3F3F3F3Fu;
            const uint32_t m_lo = s1w & 0x3F3F3F3Fu;
            const uint32_t sc_hi = (s2w & 0x0F0F0F0Fu) | ((s0w >> 2) & 0x30303030u);
            const uint32_t m_hi = ((s2w >> 4) & 0x0F0F0F0Fu) | ((s1w >> 2) & 0x30303030u);
            f32x4_t tacc[RT], bias[RT];
#pragma unroll
            for (int rt = 0; rt < RT; rt++) {
                tacc[rt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
                bias[rt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const uint32_t scw = j < 4 ? sc_lo : sc_hi;
                const uint32_t mw = j < 4 ? m_lo : m_hi;
                const float sc = (float)((scw >> (8 * (j & 3))) & 0xFF);
                const float mm = (float)((mw >> (8 * (j & 3))) & 0xFF);
                const float coef = 128.f * d * sc + dmin * mm;
                uint32_t p0 = w.q[j >> 1].x, p1 = w.q[j >> 1].y;
                if (j & 1) { p0 >>= 4; p1 >>= 4; }
                const u32x4_t b = nibbles_to_bf16(p0, p1);
#pragma unroll
                for (int rt = 0; rt < RT; rt++) {
                    const int rtl = rt < rt_n ? rt : 0;
                    const u32x4_t av2 = A_lds[((sbl * 8 + j) * rt_n + rtl) * 64 + lane];
                    const f32x4_t D = mfma16x16x32(av2, b, (f32x4_t){0.f, 0.f, 0.f, 0.f});
                    const f32x4_t S = *reinterpret_cast<const f32x4_t *>(
                        &S_lds[((sbl * 8 + j) * rt_n + rtl) * 16 + 4 * g]);
                    tacc[rt] += sc * D;
                    bias[rt] += coef * S;
                }
            }
            const float on = live ? 1.f : 0.f;
#pragma unroll
            for (int rt = 0; rt < RT; rt++) acc[rt] += on * (d * tacc[rt] - bias[rt]);
        }
    }

    if (!active) return;
    float *out = a.part + (size_t)split * a.M * a.N;
#pragma unroll
    for (int rt = 0; rt < RT; rt++) {
        if (rt < rt_n) {
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int row = row0 + rt * 16 + 4 * g + v;
                if (row < a.M) out[(size_t)row * a.N + n] = acc[rt][v];
            }
        }
    }
}

__global__ void k_q4k_dequant(const unsigned char *w, float *out, long long n_blocks) {
    const long long b = blockIdx.x * (long long)(blockDim.x / 64) + (threadIdx.x >> 6);
    if (b >= n_blocks) return;
    const int lane = threadIdx.x & 63;
    const unsigned char *blk = w + b * 144;
    const float d = half_bits_to_f32(blk[0] | (blk[1] << 8));
    const float dmin = half_bits_to_f32(blk[2] | (blk[3] << 8));
    const unsigned char *s = blk + 4;
#pragma unroll
    for (int h = 0; h < 4; h++) {
        const int i = lane + 64 * h;                 // weight index in the block
        const int c = i >> 6, r = i & 63;
        const int j = i >> 5;
        int sc, m;
        if (j < 4) {
            sc = s[j] & 63;
            m = s[j + 4] & 63;
        } else {
            sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
            m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
        }
        const int byte = blk[16 + 32 * c + (r & 31)];
        const int q = r < 32 ? (byte & 15) : (byte >> 4);
        // d*sc*q and dmin*m are exact in fp32; one rounding in the difference
        out[b * 256 + i] = d * (float)sc * (float)q - dmin * (float)m;
    }
}

}  // namespace

Q4kPlan q4k_plan(int M, int N, int K) {
    Q4kPlan p;
    p.KB = K / 256;
    const int rt_total = ceil_div(M, 16);
    p.rt = rt_total <= 1 ? 1 : (rt_total <= 2 ? 2 : MAX_RT);
    p.row_groups = ceil_div(rt_total, p.rt);
    const int tiles = N / 16;
    // aim for ~8192 waves; at most 4 super-blocks x row tiles per workgroup in LDS
    int s_target = ceil_div(8192, tiles * p.row_groups);
    if (s_target < 1) s_target = 1;
    int kb_max = KB_LDS / p.rt;
    if (kb_max < 1) kb_max = 1;
    int kb = ceil_div(p.KB, s_target);
    p.kb_per = kb < kb_max ? kb : kb_max;
    p.splits = ceil_div(p.KB, p.kb_per);
    p.lds_bytes = (size_t)p.kb_per * 8 * p.rt * (64 * 16 + 16 * 4);
    p.grid_x = ceil_div(tiles, 4);
    return p;
}

hipError_t launch_q4k_gemm(const Q4kGemmArgs &a, const Q4kPlan &p, hipStream_t st) {
    dim3 grid(p.grid_x, p.splits, p.row_groups);
    if (p.rt == 1)
        hipLaunchKernelGGL(k_q4k_gemm<1>, grid, dim3(256), p.lds_bytes, st, a);
    else if (p.rt == 2)
        hipLaunchKernelGGL(k_q4k_gemm<2>, grid, dim3(256), p.lds_bytes, st, a);
    else
        hipLaunchKernelGGL(k_q4k_gemm<MAX_RT>, grid, dim3(256), p.lds_bytes, st, a);
    return hipGetLastError();
}

hipError_t launch_q4k_dequant(const void *w, float *out, long long n_blocks, hipStream_t st) {
    const long long grid = (n_blocks + 3) / 4;
    hipLaunchKernelGGL(k_q4k_dequant, dim3((unsigned)grid), dim3(256), 0, st,
                       (const unsigned char *)w, out, n_blocks);
    return hipGetLastError();
}
