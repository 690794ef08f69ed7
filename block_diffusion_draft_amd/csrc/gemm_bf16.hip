// bf16 MFMA GEMMs, gfx950: C[M][N] (fp32) = A[M][K] . W[N][K]^T.
//
//  * tiled: 128 x 128 output tile per workgroup (2 x 2 waves of 64 x 64), K in
//    steps of 32 staged through double-buffered LDS in MFMA lane order.  Used for
//    the unquantised drafter matrices at many rows and for the shared output head
//    when more than 16 rows need logits.
//  * the streaming head (k_head_stream): at most 8 rows (the 7 proposal rows of one
//    draft block), K a multiple of 256.  The rows sit in LDS for the whole launch;
//    every wave streams its own run of 16-row weight tiles over the full K with
//    whole-line loads, so the output head (248320 x 5120 bf16, the bulk of the
//    step's bytes) is read exactly once with no cross-wave reduction.
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

// bf16 weights [N][K]
__global__ __launch_bounds__(256) void k_gemm_tiled(Bf16GemmArgs a) {
    __shared__ u32x4_t As[2][8][64];
    __shared__ u32x4_t Bs[2][8][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * 128, n0 = blockIdx.x * 128;
    const int lr = tid >> 2, lg = tid & 3;          // load row (0..63) and k-group

    const uint16_t *arow[2];
    const uint16_t *brow[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int m = m0 + lr + 64 * h;
        arow[h] = m < a.M ? a.A + (size_t)m * a.lda : nullptr;
        const int n = n0 + lr + 64 * h;
        brow[h] = n < a.N ? seg_row(a, n) : nullptr;
    }
    const int nk = a.K / 32;
    u32x4_t ra[2], rb[2];
    auto gload = [&](int kt) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int k = kt * 32 + 8 * lg;
            ra[h] = arow[h] ? *reinterpret_cast<const u32x4_t *>(arow[h] + k) : (u32x4_t){0, 0, 0, 0};
            rb[h] = brow[h] ? *reinterpret_cast<const u32x4_t *>(brow[h] + k) : (u32x4_t){0, 0, 0, 0};
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

// Output head for at most 8 activation rows, weights read as whole cache lines.
// One workgroup of 8 waves per CU; the rows sit in LDS in MFMA lane order.  The N / 16
// weight tiles are dealt to the grid's waves in balanced runs (wave w of nw takes tiles
// [w T / nw, (w + 1) T / nw)), so a grid of one workgroup per CU keeps every CU
// streaming the same number of bytes (at V = 248320: 7 or 8 tiles per wave on all 256
// CUs, where runs of 8 left 13 CUs idle).  A wave
// streams its run of 16-row weight tiles in groups of 16 rows x 128 columns: each of a
// group's 4 loads reads 4 rows x 256 contiguous bytes (non-temporal: read once), so
// every load covers full lines.  The group passes through a 4 KB per-wave LDS buffer
// (16-byte chunks XOR-swizzled by row: conflict-free writes and fragment reads) into
// MFMA lane order.  Groups are loaded HS_D - 1 ahead in registers, across tiles: one
// ahead streamed the 2.54 GB of the 27B drafter's head at 6.65 TB/s, three ahead at 6.52
// and four at 6.51 (batch-1 step, interleaved on one box).
// The outputs of up to 8 consecutive tiles stay in registers and are then written as
// 128 consecutive columns per row (lanes over columns, whole lines): written tile by
// tile in the MFMA layout, the rows' 64-byte pieces cost the stream about 8%.
// With a.rstat, each wave also leaves the softmax statistics of its run of columns per
// row: the run's max M and sum of exp(v - M) over the values it wrote (merged across
// its output batches), the pair at rstat[2 (row nrun + wave index)].
constexpr int HS_WAVES = 8;
constexpr int HS_D = 2;
constexpr int HS_TB = 8;           // tiles per output batch

__global__ __launch_bounds__(512) void k_head_stream(Bf16GemmArgs a) {
    extern __shared__ __align__(16) u32x4_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int nks = a.K / 32;
    const int ngr = a.K / 128;                       // groups per tile, a multiple of HS_D
    const int ntiles = a.N / 16;
    const int nw = gridDim.x * HS_WAVES, w = blockIdx.x * HS_WAVES + wave;
    const int t0 = (int)((long long)w * ntiles / nw);
    const int t1 = (int)((long long)(w + 1) * ntiles / nw);
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

    // running softmax statistics of this wave's columns, per row (lane-uniform)
    float rmax[8], rsum[8];
#pragma unroll
    for (int m = 0; m < 8; m++) {
        rmax[m] = -INFINITY;
        rsum[m] = 0.f;
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
        float vh[8][HS_TB / 4];                    // row m's values of this lane (rows >= M: -inf)
#pragma unroll
        for (int m = 0; m < 8; m++) {
            const bool mok = m < a.M;
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
                v *= inv8[m];
                vh[m][h] = mok && col < ncols ? v : -INFINITY;
                if (mok && col < ncols) a.C[(size_t)m * a.ldc + (size_t)tb * 16 + col] = v;
            }
        }
        if (a.rstat) {
            // the 8 rows' reductions interleaved (independent shuffle chains)
            float bm[8], bs[8];
#pragma unroll
            for (int m = 0; m < 8; m++) {
                bm[m] = vh[m][0];
#pragma unroll
                for (int h = 1; h < HS_TB / 4; h++) bm[m] = fmaxf(bm[m], vh[m][h]);
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1)
#pragma unroll
                for (int m = 0; m < 8; m++) bm[m] = fmaxf(bm[m], xor_lane_n(bm[m], o));
#pragma unroll
            for (int m = 0; m < 8; m++) {
                bs[m] = 0.f;
#pragma unroll
                for (int h = 0; h < HS_TB / 4; h++)
                    bs[m] += vh[m][h] == -INFINITY ? 0.f : __expf(vh[m][h] - bm[m]);
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1)
#pragma unroll
                for (int m = 0; m < 8; m++) bs[m] += xor_lane_n(bs[m], o);
            // merge with the earlier batches of the run (a row's batch max is finite when
            // the row exists: a batch has a column)
#pragma unroll
            for (int m = 0; m < 8; m++) {
                if (bm[m] == -INFINITY) continue;
                const float nm = fmaxf(rmax[m], bm[m]);
                rsum[m] = (rmax[m] == -INFINITY ? 0.f : rsum[m] * __expf(rmax[m] - nm)) +
                          bs[m] * __expf(bm[m] - nm);
                rmax[m] = nm;
            }
        }
    }
    if (a.rstat && lane < 8 && lane < a.M) {
        // lane m writes row m's pair (register arrays indexed by constants only)
        float mx = rmax[0], sm = rsum[0];
#pragma unroll
        for (int m = 1; m < 8; m++) {
            mx = lane == m ? rmax[m] : mx;
            sm = lane == m ? rsum[m] : sm;
        }
        *reinterpret_cast<float2 *>(a.rstat + 2 * ((size_t)lane * nw + w)) = make_float2(mx, sm);
    }
}

}  // namespace

hipError_t launch_bf16_gemm_tiled(const Bf16GemmArgs &a, hipStream_t st) {
    dim3 grid(ceil_div(a.N, 128), ceil_div(a.M, 128));
    hipLaunchKernelGGL(k_gemm_tiled, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

namespace {
// waves of the streaming head: one workgroup per CU (256 CUs), fewer for small N
int head_waves(int ntiles) { return ceil_div(min(ntiles, 256 * HS_WAVES), HS_WAVES) * HS_WAVES; }
}  // namespace

void head_runs(int N, int K, int *nrun, int *run_cols, int *run_tiles) {
    const int ntiles = N / 16;
    *nrun = *run_cols = *run_tiles = 0;
    if (K % (128 * HS_D) != 0 || ntiles < 1) return;
    const int nw = head_waves(ntiles);
    int rc = 16;                                            // widest run, rounded up to 2^k
    while (rc < 16 * ceil_div(ntiles, nw)) rc *= 2;
    *nrun = nw;
    *run_cols = rc;
    *run_tiles = ntiles;
}

// K must be a multiple of 128 HS_D (else hipErrorInvalidValue)
hipError_t launch_bf16_gemm_skinny(const Bf16GemmArgs &a, hipStream_t st) {
    const int ntiles = a.N / 16;
    if (a.K % (128 * HS_D) == 0) {
        // one workgroup of HS_WAVES waves per CU
        const int waves = head_waves(ntiles);
        const size_t lds = ((size_t)(a.K / 32) * 32 + 16 + HS_WAVES * 512) * 16;
        static size_t hs_lds_set = 0;
        if (lds > hs_lds_set) {
            hipError_t e = hipFuncSetAttribute((const void *)k_head_stream,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            hs_lds_set = lds;
        }
        hipLaunchKernelGGL(k_head_stream, dim3(waves / HS_WAVES), dim3(512), lds, st, a);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}
