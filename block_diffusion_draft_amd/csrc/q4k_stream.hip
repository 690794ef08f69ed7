// Q4_K dequantize-fused GEMM for at most 16 activation rows (one draft block of 8 rows,
// or its bf16 hi/lo pair), gfx950.  Split-K partials [split][rows][N].
//
// Format (FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", "Weights" row: the draft's fc,
// q/k/v/o and MLP matrices in Q4_K): 144-byte super-blocks of 256 weights along K,
// w = d * sc_j * q - dmin * m_j for sub-block j (32 weights), q in 0..15.  The
// matrices sit in HBM in the tiled layout of q4k_tiled.hip: the 16 rows of a column
// tile and one super-block form one contiguous 2304-byte unit, headers first, so
// every load below reads whole cache lines that no other wave touches.
//
// Arithmetic, per output column n, row r and super-block:
//     sum_k x_rk w_k = d (sum_j sc_j sum_k x_rk q_k) - dmin sum_j m_j S_rj,
//     S_rj = sum of x_rk over sub-block j.
//  * A nibble q enters a bf16 MFMA as the value 128 + q (bytes 0x43, q: one byte
//    permute per two weights), so D_j = sum_k x_rk (128 + q_k) with fp32 accumulation;
//  * T = sum_j sc_j D_j takes 4 FMAs per sub-block and lane;
//  * sum_j sc_j S_rj and sum_j m_j S_rj are two more MFMAs per super-block whose A
//    operand holds each fp32 S_rj as three bf16 terms summing to it exactly and whose
//    B operand holds the 6-bit sc_j or m_j (exact in bf16);
//  * the super-block adds d (T - 128 sum_j sc_j S_rj) - dmin sum_j m_j S_rj.
//
// Work split: a workgroup (8 waves) owns one split of 4 super-blocks (1024 values
// of K); the split's column tiles are dealt to its waves in balanced runs (wave w of
// the split's nw takes tiles [w T / nw, (w + 1) T / nw)), and the grid has about two
// workgroups per CU where the matrix has the tiles for it, so every CU streams nearly the
// same number of bytes.  The split's
// activation rows are staged once in LDS in MFMA lane order; their sub-block sums
// come from the staging lanes (a sum of 8 and two lane exchanges), and each lane keeps
// the bias operands it needs in registers.  Each wave then streams its tiles'
// super-blocks as one flat sequence of (tile, super-block) stages, loaded SAHEAD
// stages ahead of their use in a branch-free loop (loads past the end are clamped to
// the last stage, in bounds and unused), so the loads stay in flight across tiles.  The weights are
// read once, with non-temporal loads.  Each tile's partial is stored when its 4
// super-blocks are done; for a (hi, lo) row pair the two halves are added first.
// Workgroups never communicate; a reduction kernel sums the splits.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int SNSB = 4;        // super-blocks per split
// stages a wave's loads run ahead of their use (the ring holds SNSB stages).  Measured at
// batch 1: 2 ahead is fastest (gate|up 18.3 -> 17.6 us, down 21.5 -> 20.8 us against 3
// ahead, the whole step 0.860 -> 0.851 ms); 4 ahead was slower still than 3 (gate|up
// 23.6 -> 25.2 us): more bytes in flight per wave do not raise the stream's rate.
constexpr int SAHEAD = 2;
static_assert(SAHEAD >= 1 && SAHEAD < SNSB, "the ring holds the stage in use and those ahead");

struct SStage {
    u32x4_t hdr;               // d, dmin, 12 scale bytes of column cl's block
    u32x4_t q[2];              // chunks (2 h, 2 h + 1): 8 quant bytes each, lane group g
};

// one stage: the unit's base address; this lane reads the header of row cl and its
// two 16-byte quant slots
__device__ __forceinline__ SStage s_load(const unsigned char *unit, int cl, int lane) {
    SStage s;
    s.hdr = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(unit + 16 * cl));
    s.q[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(unit + 256 + 16 * lane));
    s.q[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(unit + 1280 + 16 * lane));
    return s;
}

// 8 quant bytes -> bf16 (128 + q) operands, natural k order: low nibbles (first
// sub-block of the chunk) and high nibbles (second sub-block)
__device__ __forceinline__ void s_decode(uint32_t qx, uint32_t qy, u32x4_t &lo, u32x4_t &hi) {
    const uint32_t C = 0x43434343u;
    const uint32_t lx = qx & 0x0F0F0F0Fu, ly = qy & 0x0F0F0F0Fu;
    const uint32_t hx = (qx >> 4) & 0x0F0F0F0Fu, hy = (qy >> 4) & 0x0F0F0F0Fu;
    // byte selectors: {q0, 0x43, q1, 0x43} and {q2, 0x43, q3, 0x43}
    lo.x = __builtin_amdgcn_perm(C, lx, 0x04010400u);
    lo.y = __builtin_amdgcn_perm(C, lx, 0x04030402u);
    lo.z = __builtin_amdgcn_perm(C, ly, 0x04010400u);
    lo.w = __builtin_amdgcn_perm(C, ly, 0x04030402u);
    hi.x = __builtin_amdgcn_perm(C, hx, 0x04010400u);
    hi.y = __builtin_amdgcn_perm(C, hx, 0x04030402u);
    hi.z = __builtin_amdgcn_perm(C, hy, 0x04010400u);
    hi.w = __builtin_amdgcn_perm(C, hy, 0x04030402u);
}

// bias B operand of lane group g: bf16(v_{2g}) | bf16(v_{2g+1}) << 16 for the 6-bit
// values v_0..3 in the bytes of lo and v_4..7 in the bytes of hi (sel picks bytes 2g,
// 2g+1 of {hi, lo})
__device__ __forceinline__ uint32_t bias_pair(uint32_t lo, uint32_t hi, uint32_t sel) {
    const uint32_t y = __builtin_amdgcn_perm(hi, lo, sel);
    const float fa = (float)(y & 0xFF), fb = (float)((y >> 8) & 0xFF);
    return __builtin_amdgcn_perm(__float_as_uint(fb), __float_as_uint(fa), 0x07060302u);
}

// PX > 0: rows r and r + PX / 4 are one (hi, lo) pair, held PX lanes apart
template <int WPG, int PX>
__global__ __launch_bounds__(64 * WPG) void k_q4k_stream(Q4kFusedArgs a) {
    constexpr int NT = 64 * WPG;                    // threads per workgroup
    extern __shared__ __align__(16) unsigned char lds[];
    u32x4_t *A_lds = reinterpret_cast<u32x4_t *>(lds);              // [SNSB][8][64]
    float *S_lds = reinterpret_cast<float *>(A_lds + SNSB * 8 * 64); // [SNSB][8][16]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    const int g = lane >> 4, cl = lane & 15;
    const int split = blockIdx.y, sb0 = split * SNSB;
    const int ntile = a.N / 16;
    const int nw = gridDim.x * WPG, w = blockIdx.x * WPG + wave;
    const int t0 = (int)((long long)w * ntile / nw);
    const int t1 = (int)((long long)(w + 1) * ntile / nw);
    const int tlast = (t1 > t0 ? t1 : ntile) - 1;       // clamp target, always a real tile

    // ---- weight stream.  Stage (tile t, super-block sb) is the unit at tile_base(t)
    // + sb * 2304; loads run SAHEAD stages ahead, so tile t's loop issues (t, SAHEAD ..
    // 3) and (t + 1, 0 .. SAHEAD - 1).  In the run's last tile the loads ahead re-read
    // unit (t, 3), just requested, so they hit in L2 (in bounds, unused; re-reading the
    // tile's first units instead, evicted by then, cost that many units of HBM traffic
    // per wave: 14 MB per gate|up launch at 3 ahead).
    auto tile_base = [&](int t) -> const unsigned char * {
        const int tt = t < t1 ? t : tlast;
        const int c16 = tt * 16;
        const int si = (a.nseg > 1 && c16 >= a.seg_end[0]) + (a.nseg > 2 && c16 >= a.seg_end[1]);
        const unsigned char *wseg = si == 0 ? a.w[0] : (si == 1 ? a.w[1] : a.w[2]);
        const int nbase = si == 0 ? 0 : (si == 1 ? a.seg_end[0] : a.seg_end[1]);
        return wseg + ((size_t)((c16 - nbase) >> 4) * a.KB + sb0) * Q4K_UNIT_BYTES;
    };
    auto stage = [&](const unsigned char *tb, int sb) -> SStage {
        return s_load(tb + sb * Q4K_UNIT_BYTES, cl, lane);
    };
    // ---- activations of this split -> LDS in lane order: entry (sbi, j, lane) holds
    // row cl's values k = (sb0 + sbi) 256 + 32 j + 8 g .. + 7 (rows >= M: zeros)
    // (loaded before the first weight stages: the wait for them then does not include
    // the weights' HBM latency, which overlaps the staging instead)
    constexpr int PER = SNSB * 8 / WPG;             // entries per thread
    SStage st[SNSB];
    {
        const int Rc = min(cl, a.M - 1);
        const uint16_t *arow = a.src.A + (size_t)Rc * a.src.lda + (size_t)sb0 * 256 + 8 * g;
        u32x4_t av[PER];
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int e = wave + WPG * i;           // (sbi, j) = (e >> 3, e & 7)
            av[i] = *reinterpret_cast<const u32x4_t *>(arow + (e >> 3) * 256 + 32 * (e & 7));
        }
        __builtin_amdgcn_sched_barrier(0);
        const unsigned char *b0 = tile_base(t0);
        // (written out: as a loop over the ring the loads lose their non-temporal hint)
        st[0] = stage(b0, 0);
        if (SAHEAD > 1) st[1] = stage(b0, 1);
        if (SAHEAD > 2) st[2] = stage(b0, 2);
        __builtin_amdgcn_sched_barrier(0);
        // sub-block sums S[sbi][j][r] of the staged rows: each lane adds its 8 values
        // (bf16 -> fp32 is exact), then the 4 lanes holding a row's sub-block add theirs
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int e = wave + WPG * i;
            const u32x4_t v = cl < a.M ? av[i] : (u32x4_t){0u, 0u, 0u, 0u};
            float sa = 0.f;
#pragma unroll
            for (int w = 0; w < 4; w++)
                sa += __uint_as_float(v[w] << 16) + __uint_as_float(v[w] & 0xFFFF0000u);
            sa += __shfl_xor(sa, 16, WAVE);
            sa += __shfl_xor(sa, 32, WAVE);
            if (g == 0) S_lds[e * 16 + cl] = sa;
            A_lds[e * 64 + lane] = v;
        }
    }
    __syncthreads();
    // bias A operands of this lane (row r = cl, group gg = g), one per super-block of the
    // split, kept in registers: S_a, S_b (a = 2 gg, b = 2 gg + 1) as three bf16 terms
    // each, taken by truncation (each term keeps the top 8 significant bits of what is
    // left, so three hold an fp32 significand exactly), interleaved: dword q = term q of
    // S_a | term q of S_b << 16; dword 3 = 0
    u32x4_t abias[SNSB];
#pragma unroll
    for (int sbi = 0; sbi < SNSB; sbi++) {
        uint32_t tb[2][3];
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
            float rem = S_lds[(sbi * 8 + 2 * g + jj) * 16 + cl];
#pragma unroll
            for (int q = 0; q < 3; q++) {
                const uint32_t tq = __float_as_uint(rem) & 0xFFFF0000u;
                tb[jj][q] = tq;
                rem -= __uint_as_float(tq);
            }
        }
        abias[sbi] = (u32x4_t){__builtin_amdgcn_perm(tb[1][0], tb[0][0], 0x07060302u),
                               __builtin_amdgcn_perm(tb[1][1], tb[0][1], 0x07060302u),
                               __builtin_amdgcn_perm(tb[1][2], tb[0][2], 0x07060302u), 0u};
    }

    // ---- stream
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    const int m_out = PX ? PX / 4 : a.M;            // rows of the partial written
    float *part = a.part + (size_t)split * m_out * a.N;
    const uint32_t bsel = 0x0C0C0000u | ((uint32_t)(2 * g + 1) << 8) | (uint32_t)(2 * g);
    int a_off = lane;
    for (int t = t0; t < t1; t++) {
        // opaque to the compiler: keeps the 32 activation fragments in LDS instead of
        // hoisting them into registers (which would cost waves per SIMD)
        asm volatile("" : "+v"(a_off));
        const unsigned char *bcur = tile_base(t), *bnext = tile_base(t + 1);
        const bool more = t + 1 < t1;               // (wave-uniform)
        f32x4_t acc = zero;
#pragma unroll
        for (int sb = 0; sb < SNSB; sb++) {
            const int ns = sb + SAHEAD;             // stage loaded now: (t, ns) or (t + 1, ns - 4)
            st[ns % SNSB] = ns < SNSB ? stage(bcur, ns)
                                      : stage(more ? bnext : bcur, more ? ns - SNSB : SNSB - 1);
            // keep the loads here, SAHEAD stages ahead of their use (left alone, the
            // scheduler sinks them to the end of the tile and the latency shows)
            __builtin_amdgcn_sched_barrier(0);
            const SStage &w = st[sb];
            const float d = half_bits_to_f32(w.hdr.x & 0xFFFF);
            const float dmin = half_bits_to_f32(w.hdr.x >> 16);
            const uint32_t s0w = w.hdr.y, s1w = w.hdr.z, s2w = w.hdr.w;
            const uint32_t sc_lo = s0w & 0x3F3F3F3Fu;
            const uint32_t m_lo = s1w & 0x3F3F3F3Fu;
            const uint32_t sc_hi = (s2w & 0x0F0F0F0Fu) | ((s0w >> 2) & 0x30303030u);
            const uint32_t m_hi = ((s2w >> 4) & 0x0F0F0F0Fu) | ((s1w >> 2) & 0x30303030u);
            f32x4_t tacc = zero;
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const u32x4_t &qv = w.q[c >> 1];
                u32x4_t blo, bhi;
                if (c & 1) s_decode(qv.z, qv.w, blo, bhi);
                else s_decode(qv.x, qv.y, blo, bhi);
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const int j = 2 * c + h;
                    const uint32_t scw = j < 4 ? sc_lo : sc_hi;
                    const float sc = (float)((scw >> (8 * (j & 3))) & 0xFF);
                    const f32x4_t D = mfma16x16x32(A_lds[(sb * 8 + j) * 64 + a_off], h ? bhi : blo, zero);
                    tacc += sc * D;
                }
            }
            const uint32_t mb = bias_pair(m_lo, m_hi, bsel), cb = bias_pair(sc_lo, sc_hi, bsel);
            const u32x4_t ab = abias[sb];
            const f32x4_t Dm = mfma16x16x32(ab, (u32x4_t){mb, mb, mb, mb}, zero);
            const f32x4_t Ds = mfma16x16x32(ab, (u32x4_t){cb, cb, cb, cb}, zero);
            acc += d * (tacc - 128.f * Ds) - dmin * Dm;
        }
        if (PX) {
#pragma unroll
            for (int v = 0; v < 4; v++) acc[v] += __shfl_xor(acc[v], PX, WAVE);
        }
        const int n = t * 16 + cl;
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int R = 4 * g + v;
            if (R < m_out) part[(size_t)R * a.N + n] = acc[v];
        }
    }
}

}  // namespace

bool q4k_stream_ok(int M, int N, int K) { return M >= 1 && M <= 16 && (K / 256) % SNSB == 0 && N % 16 == 0; }

Q4kStreamPlan q4k_stream_plan(int M, int N, int K, int pair, int target_waves, int wpg) {
    Q4kStreamPlan p;
    const int KB = K / 256, ntile = N / 16;
    p.splits = KB / SNSB;
    // wpg 0: 8-wave workgroups (one activation staging feeds 8 runs of tiles; measured
    // 3-7% faster than 4 waves at every drafter shape)
    p.wpg = wpg > 0 ? wpg : 8;
    wpg = p.wpg;
    // about target_waves waves in all (two 8-wave workgroups per CU at the default), and
    // no more workgroups per split than it has tiles for a wave each
    p.grid_x = max(1, min(target_waves / (wpg * p.splits), ceil_div(ntile, wpg)));
    p.tpw = ceil_div(ntile, p.grid_x * wpg);            // (the longest run)
    // the (hi, lo) halves of a pair sit pair / 4 lane groups = 4 pair lanes apart
    p.pair_done = (pair == 4 || pair == 8) && M == 2 * pair;
    p.px = p.pair_done ? 4 * pair : 0;
    p.lds_bytes = (size_t)SNSB * 8 * 64 * 16 + SNSB * 8 * 16 * 4;
    p.part_bytes = (size_t)p.splits * (p.pair_done ? pair : M) * N * 4;
    return p;
}

hipError_t launch_q4k_stream(const Q4kFusedArgs &a, const Q4kStreamPlan &p, hipStream_t st) {
    const dim3 grid(p.grid_x, p.splits);
#define QS_CASE(WPG, PX)                                                                              \
    if (p.wpg == WPG && p.px == PX) {                                                                 \
        hipLaunchKernelGGL((k_q4k_stream<WPG, PX>), grid, dim3(64 * WPG), p.lds_bytes, st, a);        \
        return hipGetLastError();                                                                     \
    }
    QS_CASE(4, 0)
    QS_CASE(4, 16)
    QS_CASE(4, 32)
    QS_CASE(8, 0)
    QS_CASE(8, 16)
    QS_CASE(8, 32)
#undef QS_CASE
    return hipErrorInvalidValue;
}
