// FP8 weights on gfx950: decode, the tiled device layout, and the streaming GEMM for at
// most 16 activation rows.  Split-K partials [split][rows][N].
//
// Format (aiqre model page "Qwen3.8-27B-DFlash2", "Memory": an fp8 weight format at one
// byte per parameter): OCP E4M3 codes (sign, 4 exponent bits of bias 7, 3 mantissa
// bits) in row order, then one fp32 scale per row; w[n][k] = s[n] e4m3(code[n][k]).
//
// Tiled layout (what the GEMM kernels read): for column tile t (16 rows of W) and
// K-group g (256 weights) one 4096-byte unit at (t K/256 + g) 4096: bytes
// 1024 p + 16 (16 h + r) (p, h < 4, r < 16) hold codes 64 p + 8 h .. + 7 of row 16 t + r's
// group, then its codes 64 p + 32 + 8 h .. + 7.  The scales follow the N K code bytes,
// as in the row-major layout.  Lane (r = lane & 15, h = lane >> 4) of a wave reads pair
// p's slot with one 16-byte load, all 64 lanes one contiguous kilobyte: the MFMA B
// operands (column r, k = 8 h .. 8 h + 7 of a 32-wide k-step) of two k-steps.
//
// Every E4M3 value is exact in bf16 (3 mantissa bits, exponents 2^-9 .. 2^8), so the
// codes enter the bf16 MFMA as they are (v_cvt_scalef32_pk_bf16_fp8 with scale 1: two
// codes per instruction); the row scale multiplies the finished fp32 sum.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int F8_SG = 4;        // K-groups of 256 per split of the streaming kernel
// stages a wave's loads run ahead of their use (ring of F8_SG).  Measured on the batch-1
// step (interleaved, one box): 2 ahead 0.937 ms, 1 or 3 ahead 0.940
constexpr int F8_AHEAD = 2;
static_assert(F8_AHEAD >= 1 && F8_AHEAD < F8_SG, "the ring holds the stage in use and those ahead");

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// two E4M3 codes (bytes 0, 1 or 2, 3 of v) -> their bf16 values (exact), first in the low half
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_bf16(uint32_t v) {
    const bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}

// 8 codes (two dwords, k order) -> the bf16 MFMA operand of their values
__device__ __forceinline__ u32x4_t e4m3x8_bf16(uint32_t w0, uint32_t w1) {
    return (u32x4_t){e4m3x2_bf16<false>(w0), e4m3x2_bf16<true>(w0), e4m3x2_bf16<false>(w1),
                     e4m3x2_bf16<true>(w1)};
}

// one thread per weight: out = fp32(s[n] e4m3(code)) (one rounding of the exact product)
__global__ __launch_bounds__(256) void k_fp8_dequant(const unsigned char *w, float *out, int N, int K) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long n_w = (long long)N * K;
    if (i >= n_w) return;
    const int n = (int)(i / K);
    const float s = reinterpret_cast<const float *>(w + n_w)[n];
    const f32x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)w[i], 1.0f, false);
    out[i] = s * v.x;
}

// one thread per 16-byte piece: 256 pieces per unit, then the scales (N / 4 pieces)
__global__ __launch_bounds__(256) void k_fp8_to_tiled(const unsigned char *src, unsigned char *dst,
                                                      int N, int G) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long units = (long long)(N / 16) * G;
    const long long K = (long long)G * 256;
    if (idx >= units * 256) {
        const long long j = idx - units * 256;                 // scale piece
        if (j >= N / 4) return;
        const size_t at = (size_t)N * K + 16 * j;
        *reinterpret_cast<u32x4_t *>(dst + at) = *reinterpret_cast<const u32x4_t *>(src + at);
        return;
    }
    const long long u = idx >> 8;
    const int piece = (int)(idx & 255);
    const int t = (int)(u / G), g = (int)(u - (long long)t * G);
    const int p = piece >> 6, l = piece & 63, h = l >> 4, r = l & 15;
    const unsigned char *row = src + (size_t)(16 * t + r) * K + 256 * g + 64 * p + 8 * h;
    const uint2 a = *reinterpret_cast<const uint2 *>(row);
    const uint2 b = *reinterpret_cast<const uint2 *>(row + 32);
    *reinterpret_cast<u32x4_t *>(dst + u * FP8_UNIT_BYTES + 16 * piece) = (u32x4_t){a.x, a.y, b.x, b.y};
}

struct F8Stage {
    u32x4_t q[4];               // pair p: 8 codes of k-step 2 p, then of k-step 2 p + 1
};

__device__ __forceinline__ F8Stage f8_load(const unsigned char *unit, int lane) {
    F8Stage s;
#pragma unroll
    for (int p = 0; p < 4; p++)
        s.q[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(unit + 1024 * p + 16 * lane));
    return s;
}

// Work split and stream as in the Q8_0 streaming kernel: a workgroup of WPG waves per
// (column-tile range, K split of 4 groups); the split's activation rows staged once in
// LDS in lane order; each wave streams a balanced run of the split's column tiles as
// (tile, group) units, 3 ahead.  PX > 0: rows r and r + PX / 4 are one (hi, lo) pair, held PX lanes
// apart, added before the store.
template <int WPG, int PX>
__global__ __launch_bounds__(64 * WPG) void k_f8_stream(Q4kFusedArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    u32x4_t *A_lds = reinterpret_cast<u32x4_t *>(lds);                     // [SG][8][64]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, cl = lane & 15;
    const int split = blockIdx.y, g0 = split * F8_SG;
    const int ntile = a.N / 16;
    // balanced runs of the split's column tiles over its nw waves
    const int nw = gridDim.x * WPG, w = blockIdx.x * WPG + wave;
    const int t0 = (int)((long long)w * ntile / nw);
    const int t1 = (int)((long long)(w + 1) * ntile / nw);
    const int tlast = (t1 > t0 ? t1 : ntile) - 1;       // clamp target, always a real tile

    // the segment of tile t: its code base and its first column
    auto seg = [&](int t, int &nbase, int &nrows) -> const unsigned char * {
        const int c16 = t * 16;
        const int si = (a.nseg > 1 && c16 >= a.seg_end[0]) + (a.nseg > 2 && c16 >= a.seg_end[1]);
        nbase = si == 0 ? 0 : (si == 1 ? a.seg_end[0] : a.seg_end[1]);
        nrows = (si == 0 ? a.seg_end[0] : (si == 1 ? a.seg_end[1] : a.seg_end[2])) - nbase;
        return si == 0 ? a.w[0] : (si == 1 ? a.w[1] : a.w[2]);
    };
    // stage (tile t, group sg of the split) is the unit at tile_base(t) + sg * 4096;
    // tiles past t1 - 1 clamp to tlast (in bounds, unused)
    auto tile_base = [&](int t) -> const unsigned char * {
        const int tt = t < t1 ? t : tlast;
        int nb, nr;
        const unsigned char *ws = seg(tt, nb, nr);
        return ws + ((size_t)((tt * 16 - nb) >> 4) * a.KB + g0) * FP8_UNIT_BYTES;
    };
    // the row scale of this lane's column of tile t
    auto col_scale = [&](int t) -> float {
        const int tt = t < t1 ? t : tlast;
        int nb, nr;
        const unsigned char *ws = seg(tt, nb, nr);
        const float *sc = reinterpret_cast<const float *>(ws + (size_t)nr * a.KB * 256);
        return sc[tt * 16 + cl - nb];
    };
    // activations of this split -> LDS in lane order: entry (sg, j, lane) holds row cl's
    // values k = (g0 + sg) 256 + 32 j + 8 g .. + 7 (rows >= M: zeros); loaded before the
    // first weight stages so that their wait does not include the weights' latency
    constexpr int PER = F8_SG * 8 / WPG;
    F8Stage st[F8_SG];
    {
        const int Rc = min(cl, a.M - 1);
        const uint16_t *arow = a.src.A + (size_t)Rc * a.src.lda + (size_t)g0 * 256 + 8 * g;
        u32x4_t av[PER];
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int e = wave + WPG * i;
            av[i] = *reinterpret_cast<const u32x4_t *>(arow + (e >> 3) * 256 + 32 * (e & 7));
        }
        __builtin_amdgcn_sched_barrier(0);
        const unsigned char *b0 = tile_base(t0);
        // (written out: as a loop over the ring the loads lose their non-temporal hint)
        st[0] = f8_load(b0, lane);
        if (F8_AHEAD > 1) st[1] = f8_load(b0 + FP8_UNIT_BYTES, lane);
        if (F8_AHEAD > 2) st[2] = f8_load(b0 + 2 * FP8_UNIT_BYTES, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < PER; i++)
            A_lds[(wave + WPG * i) * 64 + lane] = cl < a.M ? av[i] : (u32x4_t){0u, 0u, 0u, 0u};
    }
    __syncthreads();

    const int m_out = PX ? PX / 4 : a.M;
    float *part = a.part + (size_t)split * m_out * a.N;
    int a_off = lane;
    float s_next = col_scale(t0);
    for (int t = t0; t < t1; t++) {
        // opaque to the compiler: keeps the activation fragments in LDS
        asm volatile("" : "+v"(a_off));
        const unsigned char *bcur = tile_base(t), *bnext = tile_base(t + 1);
        // in the run's last tile the loads ahead re-read unit (t, 3), just requested (an
        // L2 hit, unused)
        const bool more = t + 1 < t1;
        const float s = s_next;
        s_next = col_scale(t + 1);
        f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sg = 0; sg < F8_SG; sg++) {
            const int ns = sg + F8_AHEAD;           // stage loaded now: (t, ns) or (t + 1, ns - 4)
            st[ns % F8_SG] = ns < F8_SG ? f8_load(bcur + ns * FP8_UNIT_BYTES, lane)
                                        : f8_load(more ? bnext + (ns - F8_SG) * FP8_UNIT_BYTES
                                                       : bcur + (F8_SG - 1) * FP8_UNIT_BYTES, lane);
            __builtin_amdgcn_sched_barrier(0);
            const F8Stage &w = st[sg];
#pragma unroll
            for (int p = 0; p < 4; p++) {
                const int e = sg * 8 + 2 * p;
                // two independent accumulation chains (even and odd k-steps)
                acc0 = mfma16x16x32(A_lds[e * 64 + a_off], e4m3x8_bf16(w.q[p].x, w.q[p].y), acc0);
                acc1 = mfma16x16x32(A_lds[(e + 1) * 64 + a_off], e4m3x8_bf16(w.q[p].z, w.q[p].w), acc1);
            }
        }
        f32x4_t acc = acc0 + acc1;
        if (PX) {
#pragma unroll
            for (int v = 0; v < 4; v++) acc[v] += __shfl_xor(acc[v], PX, WAVE);
        }
        const int n = t * 16 + cl;
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int R = 4 * g + v;
            if (R < m_out) part[(size_t)R * a.N + n] = acc[v] * s;
        }
    }
}

}  // namespace

hipError_t launch_fp8_dequant(const void *w, float *out, int N, int K, hipStream_t st) {
    const long long n = (long long)N * K;
    const long long blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_fp8_dequant, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const unsigned char *)w, out, N, K);
    return hipGetLastError();
}

hipError_t launch_fp8_to_tiled(const unsigned char *src, unsigned char *dst, int N, int G,
                               hipStream_t st) {
    const long long pieces = (long long)(N / 16) * G * 256 + N / 4;
    const long long blocks = (pieces + 255) / 256;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_fp8_to_tiled, dim3((unsigned)blocks), dim3(256), 0, st, src, dst, N, G);
    return hipGetLastError();
}

bool f8_stream_ok(int M, int N, int K) {
    return M >= 1 && M <= 16 && K % 256 == 0 && (K / 256) % F8_SG == 0 && N % 16 == 0;
}

Q4kStreamPlan f8_stream_plan(int M, int N, int K, int pair, int target_waves, int wpg) {
    Q4kStreamPlan p;
    const int G = K / 256, ntile = N / 16;
    p.splits = G / F8_SG;
    p.wpg = wpg > 0 ? wpg : 8;
    // about target_waves waves in all, no more workgroups per split than it has tiles
    // for a wave each
    p.grid_x = max(1, min(target_waves / (p.wpg * p.splits), ceil_div(ntile, p.wpg)));
    p.tpw = ceil_div(ntile, p.grid_x * p.wpg);          // (the longest run)
    p.pair_done = (pair == 4 || pair == 8) && M == 2 * pair;
    p.px = p.pair_done ? 4 * pair : 0;
    p.lds_bytes = (size_t)F8_SG * 8 * 64 * 16;
    p.part_bytes = (size_t)p.splits * (p.pair_done ? pair : M) * N * 4;
    return p;
}

hipError_t launch_f8_stream(const Q4kFusedArgs &a, const Q4kStreamPlan &p, hipStream_t st) {
    const dim3 grid(p.grid_x, p.splits);
#define F8_CASE(WPG, PX)                                                                             \
    if (p.wpg == WPG && p.px == PX) {                                                                \
        hipLaunchKernelGGL((k_f8_stream<WPG, PX>), grid, dim3(64 * WPG), p.lds_bytes, st, a);        \
        return hipGetLastError();                                                                    \
    }
    F8_CASE(4, 0)
    F8_CASE(4, 16)
    F8_CASE(4, 32)
    F8_CASE(8, 0)
    F8_CASE(8, 16)
    F8_CASE(8, 32)
#undef F8_CASE
    return hipErrorInvalidValue;
}
