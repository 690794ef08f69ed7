// bf16 MFMA GEMMs, gfx950: C[M][N] (fp32) = A[M][K] . W[N][K]^T.
//
//  * tiled: 128 x 128 output tile per workgroup (2 x 2 waves of 64 x 64), K in
//    steps of 32 staged through double-buffered LDS in MFMA lane order.  Used for
//    the unquantised drafter matrices at many rows and for the shared output head
//    when more than 16 rows need logits.  The same kernel reads Q8_0 weights in their
//    tiled layout (more than 16 rows, or K not a multiple of 1024): each k-step is
//    one Q8_0 block, decoded on load to bf16(d q) (round to nearest even, relative
//    error <= 2^-9 per weight; the 16-row streaming kernel keeps d q exact).
//  * skinny: at most 8 rows (the 7 proposal rows of one draft block).  The rows
//    sit in LDS for the whole launch; every wave streams its own contiguous run
//    of 16-row weight tiles over the full K with 8 fragment loads in flight, so
//    the output head (248320 x 5120 bf16, the bulk of the step's bytes) is read
//    exactly once with 16-byte loads and no cross-wave reduction.
#include "common.h"
#include "kernels.h"

namespace {

__device__ __forceinline__ const uint16_t *seg_row(const Bf16GemmArgs &a, int n) {
    int si = 0;
    while (si + 1 < a.nseg && n >= a.seg_end[si]) si++;
    const int base = si == 0 ? 0 : a.seg_end[si - 1];
    return a.w[si] + (size_t)(n - base) * a.K;
}

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// row n of a Q8_0 matrix set in the tiled layout: the base of its tile's units and
// its row within the tile
__device__ __forceinline__ const unsigned char *q8_tile_row(const Bf16GemmArgs &a, int n, int &r) {
    int si = 0;
    while (si + 1 < a.nseg && n >= a.seg_end[si]) si++;
    const int nn = n - (si == 0 ? 0 : a.seg_end[si - 1]);
    r = nn & 15;
    return reinterpret_cast<const unsigned char *>(a.w[si]) +
           (size_t)(nn >> 4) * (a.K / 256) * Q8_UNIT_BYTES;
}

// bf16(d q) of 8 signed bytes, k order
__device__ __forceinline__ u32x4_t q8_scaled(u32x2_t q, float d) {
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t w = q[i >> 1] >> (16 * (i & 1));
        const float lo = d * (float)(int8_t)(w & 0xFF), hi = d * (float)(int8_t)(w >> 8);
        o[i] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
    }
    return o;
}

// WF 0: bf16 weights [N][K]; WF 1: Q8_0 weights in the tiled layout
template <int WF>
__global__ __launch_bounds__(256) void k_gemm_tiled(Bf16GemmArgs a) {
    __shared__ u32x4_t As[2][8][64];
    __shared__ u32x4_t Bs[2][8][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * 128, n0 = blockIdx.x * 128;
    const int lr = tid >> 2, lg = tid & 3;          // load row (0..63) and k-group

    const uint16_t *arow[2];
    const uint16_t *brow[2];
    const unsigned char *bq[2];
    int rq[2] = {0, 0};
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int m = m0 + lr + 64 * h;
        arow[h] = m < a.M ? a.A + (size_t)m * a.lda : nullptr;
        const int n = n0 + lr + 64 * h;
        if (WF == 0) brow[h] = n < a.N ? seg_row(a, n) : nullptr;
        else bq[h] = n < a.N ? q8_tile_row(a, n, rq[h]) : nullptr;
    }
    const int nk = a.K / 32;
    u32x4_t ra[2], rb[2];
    auto gload = [&](int kt) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int k = kt * 32 + 8 * lg;
            ra[h] = arow[h] ? *reinterpret_cast<const u32x4_t *>(arow[h] + k) : (u32x4_t){0, 0, 0, 0};
            if (WF == 0) {
                rb[h] = brow[h] ? *reinterpret_cast<const u32x4_t *>(brow[h] + k)
                                : (u32x4_t){0, 0, 0, 0};
            } else if (bq[h]) {
                // k-step kt = block kt: unit kt / 8 of the row's tile, block j = kt % 8
                const unsigned char *unit = bq[h] + (size_t)(kt >> 3) * Q8_UNIT_BYTES;
                const int j = kt & 7;
                const u32x2_t q = *reinterpret_cast<const u32x2_t *>(
                    unit + 256 + 1024 * (j >> 1) + 16 * (16 * lg + rq[h]) + 8 * (j & 1));
                const float d = half_bits_to_f32(*reinterpret_cast<const uint16_t *>(
                    unit + 16 * rq[h] + 2 * j));
                rb[h] = q8_scaled(q, d);
            } else {
                rb[h] = (u32x4_t){0, 0, 0, 0};
            }
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int row = lr + 64 * h;
            const int ln = (row & 15) + 16 * lg;
            As[buf][row >> 4][ln] = ra[h];
            Bs[buf][row >> 4][ln] = rb[h];
        }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        u32x4_t af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; i++) af[i] = As[buf][4 * wm + i][lane];
#pragma unroll
        for (int j = 0; j < 4; j++) bfr[j] = Bs[buf][4 * wn + j][lane];
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 4; j++) acc[i][j] = mfma16x16x32(af[i], bfr[j], acc[i][j]);
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    const int g = lane >> 4, c = lane & 15;
    float rinv[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int m = m0 + 64 * wm + 16 * i + 4 * g + v;
            rinv[i][v] = m < a.M ? row_inv(a.rs, m) : 0.f;
        }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int n = n0 + 64 * wn + 16 * j + c;
            if (n >= a.N) continue;
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int m = m0 + 64 * wm + 16 * i + 4 * g + v;
                if (m < a.M) a.C[(size_t)m * a.ldc + n] = acc[i][j][v] * rinv[i][v];
            }
        }
}

// Skinny product for at most 8 activation rows (one block's 7 proposal rows).
// The rows live in LDS for the whole launch, already in MFMA lane order, so each
// wave can run the full K of its own weight tiles with no cross-wave reduction.
// Each wave owns a contiguous range of 16-row weight tiles and streams them as a
// flat sequence of (tile, k-step) fragments with LM_PD loads in flight.
constexpr int LM_PD = 8;

__global__ __launch_bounds__(256) void k_bf16_gemm_skinny(Bf16GemmArgs a, int tiles_per_wave) {
    extern __shared__ __align__(16) u32x4_t Alds[];   // [nks][32] lanes with row < 8, + 1 zero entry
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int nks = a.K / 32;                        // a multiple of LM_PD
    const int ntiles = a.N / 16;
    const int t0 = (blockIdx.x * 4 + wave) * tiles_per_wave;
    const int t1 = min(t0 + tiles_per_wave, ntiles);
    const int steps = t1 > t0 ? (t1 - t0) * nks : 0;

    // flat stream of fragments (tile, k-step); loads past the wave's range are
    // clamped to its last fragment (in bounds, value unused)
    const uint16_t *W = a.w[0] + (size_t)c * a.K + 8 * g;
    const size_t tile_stride = (size_t)16 * a.K;
    int lt = t0, lk = 0, nload = 0;
    auto load_next = [&]() -> u32x4_t {
        const bool ok = nload < steps;
        const int tt = ok ? lt : t1 - 1, kk = ok ? lk : nks - 1;
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(W + (size_t)tt * tile_stride + kk * 32);
        nload++;
        lk++;
        const bool wrap = lk == nks;
        lk = wrap ? 0 : lk;
        lt += wrap ? 1 : 0;
        return v;
    };
    u32x4_t eb[LM_PD];
    if (steps > 0) {
#pragma unroll
        for (int u = 0; u < LM_PD - 1; u++) eb[u] = load_next();
    }
    for (int e = tid; e < nks * 32 + 1; e += 256) {
        const int ks = e >> 5, slot = e & 31, gg = slot >> 3, r = slot & 7;
        u32x4_t v = {0, 0, 0, 0};
        if (e < nks * 32 && r < a.M)
            v = *reinterpret_cast<const u32x4_t *>(a.A + (size_t)r * a.lda + ks * 32 + 8 * gg);
        Alds[e] = v;
    }
    __syncthreads();

    // deferred RMSNorm of the rows this lane stores (rows 4g + v, g < 2): computed for
    // all 8 rows with wave-uniform (scalar) loads, which do not wait behind the weight
    // loads already in flight
    float inv8[8];
#pragma unroll
    for (int r = 0; r < 8; r++) inv8[r] = r < a.M ? row_inv(a.rs, r) : 0.f;
    float rinv[4];
#pragma unroll
    for (int v = 0; v < 4; v++) rinv[v] = g == 0 ? inv8[v] : (g == 1 ? inv8[4 + v] : 0.f);

    // lanes of rows >= 8 read the zero entry
    const int aoff = c < 8 ? g * 8 + c : 0;
    const int astep = c < 8 ? 32 : 0;
    const int abase = c < 8 ? 0 : nks * 32;
    for (int tile = t0; tile < t1; tile++) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        for (int ks0 = 0; ks0 < nks; ks0 += LM_PD) {
#pragma unroll
            for (int u = 0; u < LM_PD; u++) {
                eb[(u + LM_PD - 1) % LM_PD] = load_next();
                const u32x4_t af = Alds[abase + (ks0 + u) * astep + aoff];
                acc = mfma16x16x32(af, eb[u], acc);
            }
        }
        if (g < 2) {
            const int n = tile * 16 + c;
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int m = 4 * g + v;
                if (m < a.M) a.C[(size_t)m * a.ldc + n] = acc[v] * rinv[v];
            }
        }
    }
}

// Output head for at most 8 activation rows, weights read as whole cache lines.
// One workgroup of 8 waves per CU; the rows sit in LDS in MFMA lane order.  A wave
// streams its run of 16-row weight tiles in groups of 16 rows x 128 columns: each of a
// group's 4 loads reads 4 rows x 256 contiguous bytes (non-temporal: read once), so
// every load covers full lines.  The group passes through a 4 KB per-wave LDS buffer
// (16-byte chunks XOR-swizzled by row: conflict-free writes and fragment reads) into
// MFMA lane order.  Groups are loaded HS_D - 1 ahead in registers, across tiles.
// The outputs of up to 8 consecutive tiles stay in registers and are then written as
// 128 consecutive columns per row (lanes over columns, whole lines): written tile by
// tile in the MFMA layout, the rows' 64-byte pieces cost the stream about 8%.
constexpr int HS_WAVES = 8;
constexpr int HS_D = 4;
constexpr int HS_TB = 8;           // tiles per output batch

__global__ __launch_bounds__(512) void k_head_stream(Bf16GemmArgs a, int tiles_per_wave) {
    extern __shared__ __align__(16) u32x4_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int nks = a.K / 32;
    const int ngr = a.K / 128;                       // groups per tile, a multiple of HS_D
    const int ntiles = a.N / 16;
    const int t0 = (blockIdx.x * HS_WAVES + wave) * tiles_per_wave;
    const int t1 = min(t0 + tiles_per_wave, ntiles);
    const int nst = t1 > t0 ? (t1 - t0) * ngr : 0;
    const int tlast = (t1 > t0 ? t1 : ntiles) - 1;
    u32x4_t *Alds = lds;                                          // [nks][32] + zero entry
    u32x4_t *Tb = lds + nks * 32 + 16 + wave * 512;               // 2 x [16 rows][16 chunks]

    // load lane mapping: row 4 i + lr of the tile, 16-byte chunk ls of the group
    const int lr = lane >> 4, ls = lane & 15;
    const uint16_t *Wl = a.w[0] + (size_t)lr * a.K + 8 * ls;
    int lt = t0, lq = 0, nload = 0;
    auto load_group = [&](u32x4_t (&v)[4]) {
        const bool ok = nload < nst;
        const int tt = ok ? lt : tlast, qq = ok ? lq : ngr - 1;
        const uint16_t *p = Wl + (size_t)tt * 16 * a.K + qq * 128;
#pragma unroll
        for (int i = 0; i < 4; i++)
            v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p + (size_t)(4 * i) * a.K));
        nload++;
        lq++;
        const bool wrap = lq == ngr;
        lq = wrap ? 0 : lq;
        lt += wrap ? 1 : 0;
    };
    u32x4_t ring[HS_D][4];
#pragma unroll
    for (int u = 0; u < HS_D - 1; u++) load_group(ring[u]);

    // row scales (deferred RMSNorm): lane l < 8 sums row l's partial sums of squares,
    // loaded 8 at a time; issued before the activation loads so both are in flight
    const RowScale &rs = a.rs;
    float ssl = 0.f;
    if (rs.ssq && lane < 8 && lane < a.M) {
        const int br = rs.map ? (lane / (rs.map - 1)) * rs.map + lane % (rs.map - 1) + 1 : lane;
        const float *sp = rs.ssq + (size_t)br * rs.nchunk;
        for (int i0 = 0; i0 < rs.nchunk; i0 += 8) {
            float pv[8];
#pragma unroll
            for (int u = 0; u < 8; u++) pv[u] = sp[min(i0 + u, rs.nchunk - 1)];
#pragma unroll
            for (int u = 0; u < 8; u++)
                if (i0 + u < rs.nchunk) ssl += pv[u];
        }
    }
    // activations -> LDS in lane order (8 loads in flight per thread)
    const int nA = nks * 32 + 16;
    for (int e0 = tid; e0 < nA; e0 += 8 * 512) {
        u32x4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int e = min(e0 + 512 * u, nks * 32 - 1);
            const int ks = e >> 5, slot = e & 31, gg = slot >> 3, r = min(slot & 7, a.M - 1);
            v[u] = *reinterpret_cast<const u32x4_t *>(a.A + (size_t)r * a.lda + ks * 32 + 8 * gg);
        }
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int e = e0 + 512 * u;
            const int r = e & 7;
            if (e < nA) Alds[e] = (e < nks * 32 && r < a.M) ? v[u] : (u32x4_t){0, 0, 0, 0};
        }
    }
    __syncthreads();

    float inv8[8];
#pragma unroll
    for (int r = 0; r < 8; r++) {
        const float ss = __shfl(ssl, r, WAVE);
        inv8[r] = r < a.M ? (rs.ssq ? rsqrtf(ss / rs.n + rs.eps) : 1.f) : 0.f;
    }

    // lanes of rows >= 8 read the zero entry
    const int aoff = c < 8 ? g * 8 + c : 0;
    const int astep = c < 8 ? 32 : 0;
    const int abase = c < 8 ? 0 : nks * 32;
    for (int tb = t0; tb < t1; tb += HS_TB) {
        // tile tb + u -> res[u]: D rows 4 g + v, column c of the tile
        f32x4_t res[HS_TB];
#pragma unroll
        for (int u0 = 0; u0 < HS_TB; u0++) {
            res[u0] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
            if (tb + u0 >= t1) continue;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            for (int q0 = 0; q0 < ngr; q0 += HS_D) {
#pragma unroll
                for (int u = 0; u < HS_D; u++) {
                    load_group(ring[(u + HS_D - 1) % HS_D]);
                    u32x4_t *T = Tb + (u & 1) * 256;
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int r = 4 * i + lr;
                        T[r * 16 + (ls ^ r)] = ring[u][i];
                    }
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const u32x4_t bf = T[c * 16 + ((4 * j + g) ^ c)];
                        const u32x4_t af = Alds[abase + ((q0 + u) * 4 + j) * astep + aoff];
                        acc = mfma16x16x32(af, bf, acc);
                    }
                }
            }
            res[u0] = acc;
        }
        // row m, columns 16 tb + 64 h + lane: tile 4 h + lane / 16, column lane % 16,
        // held by lane 16 (m / 4) + lane % 16 as component m % 4
        const int ncols = min(HS_TB, t1 - tb) * 16;
#pragma unroll
        for (int m = 0; m < 8; m++) {
            if (m >= a.M) break;
            const int src = 16 * (m / 4) + (lane & 15);
#pragma unroll
            for (int h = 0; h < HS_TB / 4; h++) {
                float v = 0.f;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const float x = __shfl(res[4 * h + j][m % 4], src, WAVE);
                    v = (lane >> 4) == j ? x : v;
                }
                const int col = 64 * h + lane;
                if (col < ncols) a.C[(size_t)m * a.ldc + (size_t)tb * 16 + col] = v * inv8[m];
            }
        }
    }
}

}  // namespace

hipError_t launch_bf16_gemm_tiled(const Bf16GemmArgs &a, hipStream_t st) {
    dim3 grid(ceil_div(a.N, 128), ceil_div(a.M, 128));
    if (a.wfmt == 1) {
        if (a.K % 256) return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_gemm_tiled<1>, grid, dim3(256), 0, st, a);
    } else {
        hipLaunchKernelGGL(k_gemm_tiled<0>, grid, dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_bf16_gemm_skinny(const Bf16GemmArgs &a, hipStream_t st) {
    const int ntiles = a.N / 16;
    if (a.K % (128 * HS_D) == 0) {
        // one workgroup of HS_WAVES waves per CU
        const int tpw = ceil_div(ntiles, 256 * HS_WAVES);
        const int waves = ceil_div(ntiles, tpw);
        const size_t lds = ((size_t)(a.K / 32) * 32 + 16 + HS_WAVES * 512) * 16;
        static size_t hs_lds_set = 0;
        if (lds > hs_lds_set) {
            hipError_t e = hipFuncSetAttribute((const void *)k_head_stream,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            hs_lds_set = lds;
        }
        hipLaunchKernelGGL(k_head_stream, dim3(ceil_div(waves, HS_WAVES)), dim3(512), lds, st, a, tpw);
        return hipGetLastError();
    }
    const int tpw = ceil_div(ntiles, 2048);               // ~2048 waves, 2 workgroups per CU
    const int waves = ceil_div(ntiles, tpw);
    const size_t lds = ((size_t)(a.K / 32) * 32 + 1) * 16;
    static size_t lds_set = 0;
    if (lds > 65536 && lds > lds_set) {
        hipError_t e = hipFuncSetAttribute((const void *)k_bf16_gemm_skinny,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        lds_set = lds;
    }
    hipLaunchKernelGGL(k_bf16_gemm_skinny, dim3(ceil_div(waves, 4)), dim3(256), lds, st, a, tpw);
    return hipGetLastError();
}
