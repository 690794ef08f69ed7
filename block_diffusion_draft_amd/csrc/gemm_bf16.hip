// bf16 MFMA GEMMs, gfx950: C[M][N] (fp32) = A[M][K] . W[N][K]^T.
//
//  * tiled: 128 x 128 output tile per workgroup (2 x 2 waves of 64 x 64), K in
//    steps of 32 staged through double-buffered LDS in MFMA lane order.  Used for
//    the unquantised drafter matrices at many rows and for the shared output head
//    when more than 16 rows need logits.
//  * skinny: at most 16 rows (one draft block of one sequence).  The workgroup's
//    4 waves split K; each wave holds its quarter of the activation rows in VGPRs
//    for the whole launch and streams 16 weight rows per tile from HBM, so the
//    output head (248320 x 5120 bf16, the bulk of the step's bytes) is read
//    exactly once with 16-byte loads.  Partial tiles are summed through LDS.
#include "common.h"
#include "kernels.h"

namespace {

__device__ __forceinline__ const uint16_t *seg_row(const Bf16GemmArgs &a, int n) {
    int si = 0;
    while (si + 1 < a.nseg && n >= a.seg_end[si]) si++;
    const int base = si == 0 ? 0 : a.seg_end[si - 1];
    return a.w[si] + (size_t)(n - base) * a.K;
}

__global__ __launch_bounds__(256) void k_bf16_gemm_tiled(Bf16GemmArgs a) {
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
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int n = n0 + 64 * wn + 16 * j + c;
            if (n >= a.N) continue;
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int m = m0 + 64 * wm + 16 * i + 4 * g + v;
                if (m < a.M) a.C[(size_t)m * a.ldc + n] = acc[i][j][v];
            }
        }
}

constexpr int SKINNY_MAXKS = 40;    // k-steps of 32 per wave: K <= 4 * 40 * 32 = 5120

__global__ __launch_bounds__(256) void k_bf16_gemm_skinny(Bf16GemmArgs a) {
    __shared__ f32x4_t red[4][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int kq = a.K / 4;
    const int nks = kq / 32;
    const int kbase = wave * kq;

    u32x4_t af[SKINNY_MAXKS];
    const bool row_ok = c < a.M;
#pragma unroll
    for (int ks = 0; ks < SKINNY_MAXKS; ks++) {
        if (ks < nks && row_ok)
            af[ks] = *reinterpret_cast<const u32x4_t *>(a.A + (size_t)c * a.lda + kbase + ks * 32 + 8 * g);
        else
            af[ks] = (u32x4_t){0, 0, 0, 0};
    }

    const int ntiles = a.N / 16;
    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int n = tile * 16 + c;
        const uint16_t *wr = seg_row(a, n) + kbase + 8 * g;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < SKINNY_MAXKS; k0 += 8) {
            u32x4_t b[8];
#pragma unroll
            for (int u = 0; u < 8; u++)
                if (k0 + u < nks) b[u] = *reinterpret_cast<const u32x4_t *>(wr + (k0 + u) * 32);
#pragma unroll
            for (int u = 0; u < 8; u++)
                if (k0 + u < nks) acc = mfma16x16x32(af[k0 + u], b[u], acc);
        }
        red[wave][lane] = acc;
        __syncthreads();
        if (wave == 0) {
            f32x4_t s = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int m = 4 * g + v;
                if (m < a.M) a.C[(size_t)m * a.ldc + n] = s[v];
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_bf16_gemm_tiled(const Bf16GemmArgs &a, hipStream_t st) {
    dim3 grid(ceil_div(a.N, 128), ceil_div(a.M, 128));
    hipLaunchKernelGGL(k_bf16_gemm_tiled, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_bf16_gemm_skinny(const Bf16GemmArgs &a, hipStream_t st) {
    const int ntiles = a.N / 16;
    const int grid = ntiles < 1024 ? ntiles : 1024;
    hipLaunchKernelGGL(k_bf16_gemm_skinny, dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}
