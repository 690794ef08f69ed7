// Q4_K dequantize-fused GEMM (split-K partials), gfx950.
//
// Format (FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", "Weights" row: the draft's fc,
// q/k/v/o and MLP matrices in Q4_K): 144-byte super-blocks of 256 weights along K,
// w = d * sc_j * q - dmin * m_j for sub-block j (32 weights), q in 0..15, held in the
// tiled layout of q4k_tiled.hip (16 rows x one super-block per 2304-byte unit).
//
// Arithmetic.  For output column n, activation row r and super-block b:
//     sum_k x_rk w_k = d sum_j sc_j (sum_k x_rk q_k)  -  dmin sum_j m_j S_rj,
//     S_rj = sum over sub-block j of x_rk.
//  * A nibble q enters the MFMA as the bf16 value 128 + q (bits 0x4300 | q); the
//    MFMA accumulator starts at -128 S_rj, so D_j = sum_k x_rk q_k exactly up to
//    fp32 accumulation.  Then sum_j sc_j D_j takes 4 FMAs per sub-block and lane.
//  * sum_j m_j S_rj is one more MFMA per super-block: A carries each fp32 S_rj as four
//    bf16 terms that add up to it exactly, B the small integers m_j (exact in bf16).
//
// Work split.  A workgroup (4 waves) owns a column group and a range of NSB
// super-blocks (split-K).  Its bf16 activation rows for that range are staged once
// in LDS in MFMA lane order with their per-sub-block sums.  Each wave streams STEPS
// (column tile, super-block) pairs
// from HBM with 4 super-blocks in flight, in a fully unrolled loop (no branch, so
// the loads stay in flight).  Partials go to [split][M][N]; a reduction kernel sums
// them in split order (deterministic) and applies the epilogue.  Workgroups never
// communicate, so no device-scope fence (an L2 write-back on this chip) is needed.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int PD_MAX = 4;          // super-blocks in flight per wave

struct WStage {
    u32x4_t hdr;
    u32x2_t q[4];
};

// one (tile, super-block) unit of the tiled layout (q4k_tiled.hip): this lane reads the
// header of row cl and its quant slot in each half (chunks 0, 1 and 2, 3)
__device__ __forceinline__ WStage load_stage(const unsigned char *unit, int cl, int lane) {
    WStage s;
    s.hdr = *reinterpret_cast<const u32x4_t *>(unit + 16 * cl);
    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(unit + 256 + 16 * lane);
    const u32x4_t b = *reinterpret_cast<const u32x4_t *>(unit + 1280 + 16 * lane);
    s.q[0] = (u32x2_t){a.x, a.y};
    s.q[1] = (u32x2_t){a.z, a.w};
    s.q[2] = (u32x2_t){b.x, b.y};
    s.q[3] = (u32x2_t){b.z, b.w};
    return s;
}

// x0..x7 -> slots (x0,x2) (x1,x3) (x4,x6) (x5,x7), the order the nibble decode uses
__device__ __forceinline__ u32x4_t permute_slots(u32x4_t v) {
    u32x4_t o;
    o.x = (v.x & 0xFFFFu) | (v.y << 16);
    o.y = (v.x >> 16) | (v.y & 0xFFFF0000u);
    o.z = (v.z & 0xFFFFu) | (v.w << 16);
    o.w = (v.z >> 16) | (v.w & 0xFFFF0000u);
    return o;
}

// 8 quant bytes b0..b7 -> bf16 (128 + q) operands of the low-nibble sub-block and
// of the high-nibble sub-block, slots (b0,b2) (b1,b3) (b4,b6) (b5,b7)
__device__ __forceinline__ void decode_pair(u32x2_t q, u32x4_t &lo, u32x4_t &hi) {
    const uint32_t N = 0x0F0F0F0Fu, E = 0x00FF00FFu, C = 0x43004300u;
    const uint32_t l0 = q.x & N, l1 = q.y & N;
    const uint32_t h0 = (q.x >> 4) & N, h1 = (q.y >> 4) & N;
    lo.x = (l0 & E) | C;
    lo.y = ((l0 >> 8) & E) | C;
    lo.z = (l1 & E) | C;
    lo.w = ((l1 >> 8) & E) | C;
    hi.x = (h0 & E) | C;
    hi.y = ((h0 >> 8) & E) | C;
    hi.z = (h1 & E) | C;
    hi.w = ((h1 >> 8) & E) | C;
}

// bf16 of a small non-negative integer held in byte k of w, duplicated in both halves
__device__ __forceinline__ uint32_t int_byte_bf16x2(uint32_t w, int k) {
    const uint32_t fb = __float_as_uint((float)((w >> (8 * k)) & 0xFF));
    return (fb >> 16) | (fb & 0xFFFF0000u);
}

template <int RT, int NSB, int STEPS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void k_q4k_fused(Q4kFusedArgs a) {
    constexpr int CT = STEPS / NSB;                  // column tiles per wave
    constexpr int PD = STEPS < PD_MAX ? STEPS : PD_MAX;
    constexpr int MAXA = 2 * NSB * RT;               // staged fragments per thread
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, cl = lane & 15;
    const int split = blockIdx.y;
    const int row0 = blockIdx.z * (RT * 16);
    const int rt_n = min(RT, ceil_div(a.M - row0, 16));
    const int sb0 = split * NSB;
    constexpr int nsb = NSB;                         // NSB divides KB (host plan)
    const int ntile = a.N / 16;

    // ---- column tiles of this wave and their weight rows
    const int tile0 = blockIdx.x * 4 * CT + wave * CT;
    const unsigned char *wrow[CT];
#pragma unroll
    for (int ti = 0; ti < CT; ti++) {
        const int c16 = min(tile0 + ti, ntile - 1) * 16;
        const int si = (a.nseg > 1 && c16 >= a.seg_end[0]) + (a.nseg > 2 && c16 >= a.seg_end[1]);
        const unsigned char *wseg = si == 0 ? a.w[0] : (si == 1 ? a.w[1] : a.w[2]);
        const int nbase = si == 0 ? 0 : (si == 1 ? a.seg_end[0] : a.seg_end[1]);
        wrow[ti] = wseg + ((size_t)((c16 - nbase) >> 4) * a.KB + sb0) * Q4K_UNIT_BYTES;
    }
    // step order: super-block major (step / CT), tile minor (step % CT), so the LDS
    // operands of a super-block are read once and reused for the wave's CT tiles
    auto stage_at = [&](int step) {
        return load_stage(wrow[step % CT] + (step / CT) * Q4K_UNIT_BYTES, cl, lane);
    };

    // ---- LDS layout
    u32x4_t *A_lds = reinterpret_cast<u32x4_t *>(lds);                                  // [nsb][8][rt_n][64]
    float *C_lds = reinterpret_cast<float *>(lds + (size_t)nsb * 8 * rt_n * 1024);       // [nsb][8][rt_n][16] = -128 S
    u32x4_t *B_lds = reinterpret_cast<u32x4_t *>(lds + (size_t)nsb * 8 * rt_n * 1088);  // [nsb][rt_n][64] bias A

    // ---- 2) activation loads (clamped, branch-free), then the first weight stages
    const int entries = nsb * 8 * rt_n * 64;
    u32x4_t av[MAXA];
#pragma unroll
    for (int i = 0; i < MAXA; i++) {
        const int e = min(tid + 256 * i, entries - 1);
        const int ln = e & 63;
        int rest = e >> 6;
        const int rt = rest % rt_n;
        rest /= rt_n;
        const int j = rest & 7, sbi = rest >> 3;
        const int R = row0 + rt * 16 + (ln & 15);
        const int Rc = min(R, a.M - 1);
        const size_t k = (size_t)(sb0 + sbi) * 256 + 32 * j + 8 * (ln >> 4);
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(a.src.A + (size_t)Rc * a.src.lda + k);
        const bool ok = R < a.M && tid + 256 * i < entries;
        av[i] = ok ? v : (u32x4_t){0u, 0u, 0u, 0u};
    }
    WStage st[PD];
#pragma unroll
    for (int u = 0; u < PD - 1; u++) st[u] = stage_at(u);

    // ---- 3) stage: lane-ordered fragments, -128 S per (sub-block, row)
#pragma unroll
    for (int i = 0; i < MAXA; i++) {
        const int e = tid + 256 * i;
        if (e < entries) {                                   // uniform per wave
            const u32x4_t v = av[i];
            const int ln = e & 63;
            int rest = e >> 6;
            const int rt = rest % rt_n;
            rest /= rt_n;
            const int j = rest & 7, sbi = rest >> 3;
            float s = 0.f;
            s += bf16_to_f32(v.x & 0xFFFF) + bf16_to_f32(v.x >> 16);
            s += bf16_to_f32(v.y & 0xFFFF) + bf16_to_f32(v.y >> 16);
            s += bf16_to_f32(v.z & 0xFFFF) + bf16_to_f32(v.z >> 16);
            s += bf16_to_f32(v.w & 0xFFFF) + bf16_to_f32(v.w >> 16);
            s += __shfl_xor(s, 16, WAVE);
            s += __shfl_xor(s, 32, WAVE);
            A_lds[e] = permute_slots(v);
            if ((ln >> 4) == 0) C_lds[((sbi * 8 + j) * rt_n + rt) * 16 + (ln & 15)] = -128.f * s;
        }
    }
    __syncthreads();
    // bias operand: lane (row r, group gg) holds S_j for j = 2 gg and 2 gg + 1, each as four
    // bf16 terms whose sum is the fp32 value exactly (8 + 8 + 8 + 8 >= 24 bits)
    if (tid < nsb * rt_n * 64) {
        const int ln = tid & 63, rest = tid >> 6;
        const int rt = rest % rt_n, sbi = rest / rt_n;
        const int r = ln & 15, gg = ln >> 4;
        uint32_t o[4];
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
            const int j = 2 * gg + jj;
            float rem = C_lds[((sbi * 8 + j) * rt_n + rt) * 16 + r] * (-1.f / 128.f);
            uint16_t t[4];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                t[q] = f32_to_bf16(rem);
                rem -= bf16_to_f32(t[q]);
            }
            o[2 * jj] = (uint32_t)t[0] | ((uint32_t)t[1] << 16);
            o[2 * jj + 1] = (uint32_t)t[2] | ((uint32_t)t[3] << 16);
        }
        B_lds[tid] = (u32x4_t){o[0], o[1], o[2], o[3]};
    }
    __syncthreads();

    // ---- 4) stream the weights
    f32x4_t acc[CT][RT];
#pragma unroll
    for (int ti = 0; ti < CT; ti++)
#pragma unroll
        for (int rt = 0; rt < RT; rt++) acc[ti][rt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int i = 0; i < STEPS; i++) {
        if (i + PD - 1 < STEPS) st[(i + PD - 1) % PD] = stage_at(i + PD - 1);
        const int ti = i % CT, sbl = i / CT;
        const WStage &w = st[i % PD];
        const float d = half_bits_to_f32(w.hdr.x & 0xFFFF);
        const float dmin = half_bits_to_f32(w.hdr.x >> 16);
        const uint32_t s0w = w.hdr.y, s1w = w.hdr.z, s2w = w.hdr.w;
        const uint32_t sc_lo = s0w & 0x3F3F3F3Fu;
        const uint32_t m_lo = s1w & 0x3F3F3F3Fu;
        const uint32_t sc_hi = (s2w & 0x0F0F0F0Fu) | ((s0w >> 2) & 0x30303030u);
        const uint32_t m_hi = ((s2w >> 4) & 0x0F0F0F0Fu) | ((s1w >> 2) & 0x30303030u);
        f32x4_t tacc[RT];
#pragma unroll
        for (int rt = 0; rt < RT; rt++) tacc[rt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jp = 0; jp < 4; jp++) {
            u32x4_t blo, bhi;
            decode_pair(w.q[jp], blo, bhi);
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int j = 2 * jp + h;
                const uint32_t scw = j < 4 ? sc_lo : sc_hi;
                const float sc = (float)((scw >> (8 * (j & 3))) & 0xFF);
#pragma unroll
                for (int rt = 0; rt < RT; rt++) {
                    const int rtl = rt < rt_n ? rt : 0;
                    const int at = (sbl * 8 + j) * rt_n + rtl;
                    const u32x4_t avv = A_lds[at * 64 + lane];
                    const f32x4_t cv = *reinterpret_cast<const f32x4_t *>(&C_lds[at * 16 + 4 * g]);
                    const f32x4_t D = mfma16x16x32(avv, h ? bhi : blo, cv);
                    tacc[rt] += sc * D;
                }
            }
        }
        // bias: sum_j m_j S_j via one MFMA; B slots of lane group g: m_{2g} x4, m_{2g+1} x4
        const uint32_t mw = g < 2 ? m_lo : m_hi;
        const uint32_t m0 = int_byte_bf16x2(mw, (2 * g) & 3), m1 = int_byte_bf16x2(mw, (2 * g + 1) & 3);
        const u32x4_t bb = {m0, m0, m1, m1};
#pragma unroll
        for (int rt = 0; rt < RT; rt++) {
            const int rtl = rt < rt_n ? rt : 0;
            const u32x4_t ab = B_lds[(sbl * rt_n + rtl) * 64 + lane];
            const f32x4_t Db = mfma16x16x32(ab, bb, (f32x4_t){0.f, 0.f, 0.f, 0.f});
            acc[ti][rt] += d * tacc[rt] - dmin * Db;
        }
    }

    // ---- 5) partials
    float *part = a.part + (size_t)split * a.M * a.N;
#pragma unroll
    for (int ti = 0; ti < CT; ti++) {
        const int tile = tile0 + ti;
        if (tile >= ntile) continue;
        const int n = tile * 16 + cl;
#pragma unroll
        for (int rt = 0; rt < RT; rt++) {
            if (rt >= rt_n) continue;
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int R = row0 + rt * 16 + 4 * g + v;
                if (R < a.M) part[(size_t)R * a.N + n] = acc[ti][rt][v];
            }
        }
    }

}

}  // namespace

Q4kFusedPlan q4k_fused_plan(int M, int N, int K) {
    Q4kFusedPlan p;
    const int KB = K / 256;
    const int rt_total = ceil_div(M, 16);
    p.rt = rt_total <= 1 ? 1 : (rt_total <= 2 ? 2 : 4);
    p.row_groups = ceil_div(rt_total, p.rt);
    // super-blocks per split: the largest of 4/rt, 2, 1 that divides KB (LDS holds nsb x rt)
    p.nsb = 1;
    for (int c = 4 / p.rt; c >= 1; c /= 2)
        if (KB % c == 0) { p.nsb = c; break; }
    const int tiles = N / 16;
    const long long work = (long long)tiles * KB * p.row_groups;
    // steps per wave: (column tile, super-block) pairs; accumulators are CT x RT tiles
    (void)work;
    p.steps = p.rt == 1 ? 4 : p.nsb;      // RT > 1: one column tile per wave
    if (p.steps < p.nsb) p.steps = p.nsb;
    p.ct = p.steps / p.nsb;
    p.splits = KB / p.nsb;
    p.grid_x = ceil_div(tiles, 4 * p.ct);
    p.lds_bytes = (size_t)p.nsb * p.rt * (8 * 1088 + 1024);
    p.part_bytes = (size_t)p.splits * M * N * 4;
    return p;
}

hipError_t launch_q4k_fused(const Q4kFusedArgs &a, const Q4kFusedPlan &p, hipStream_t st) {
    dim3 grid(p.grid_x, p.splits, p.row_groups);
    const size_t lds = p.lds_bytes;
#define Q4K_CASE(RT, NSB, STEPS)                                                         \
    if (p.rt == RT && p.nsb == NSB && p.steps == STEPS) {                                 \
        hipLaunchKernelGGL((k_q4k_fused<RT, NSB, STEPS>), grid, dim3(256), lds, st, a);   \
        return hipGetLastError();                                                         \
    }
    Q4K_CASE(1, 4, 4)
    Q4K_CASE(1, 2, 4)
    Q4K_CASE(1, 1, 4)
    Q4K_CASE(2, 2, 2)
    Q4K_CASE(2, 1, 1)
    Q4K_CASE(4, 1, 1)
#undef Q4K_CASE
    return hipErrorInvalidValue;
}

