// Q8_0 weights on gfx950: decode, the tiled device layout, and the dequantize-fused
// GEMM for at most 16 activation rows.  Split-K partials [split][rows][N].
//
// Format (Mindket kit page "Qwen3.8-27B-DFlash2-GGUF by z-lab", draft-file table: the
// draft also ships as a Q8_0 file; the bytes are the GGUF Q8_0 block): 34 bytes per 32
// consecutive weights of a row, an fp16 scale d then 32 signed bytes q, w = d q.
//
// Tiled layout (what the GEMM kernels read): for column tile t (16 rows of W) and
// K-group g (256 weights = 8 blocks) one 4352-byte unit at (t K/256 + g) 4352:
//   bytes [0, 256): the 8 block scales of row 16 t + r (fp16, block order) at 16 r;
//   bytes 256 + 1024 p + 16 (16 h + r) (p, h < 4, r < 16): quant bytes 8 h .. 8 h + 7 of
//   block 2 p of row 16 t + r, then the same bytes of block 2 p + 1.
// Lane (r = lane & 15, h = lane >> 4) of a wave reads pair p's slot with one 16-byte
// load, all 64 lanes one contiguous kilobyte: the MFMA B operand (column r, k = 8 h ..
// 8 h + 7 of a 32-wide k-step = one block) of two consecutive blocks.
//
// Arithmetic of the streaming GEMM, per output column n, row m and block:
//     sum_k x_mk d q_k = d (sum_k x_mk (q_k + 128) - 128 S_m),   S_m = sum_k x_mk.
// The byte q + 128 (q xor 0x80, an integer 0..255) is exact in bf16; the block's MFMA
// takes -128 S_m as its accumulator input, so a block costs one MFMA and 4 FMAs
// (d times the result) per lane.  S comes from MFMAs against a ones operand when the
// split's activation rows are staged.  Work split, staging and the stream of
// (tile, group) units 3 ahead follow the Q4_K streaming kernel.
#include "common.h"
#include "kernels.h"

#include <string.h>

namespace {

constexpr int Q8_SG = 4;        // K-groups of 256 per split of the streaming kernel
// stages a wave's loads run ahead of their use (ring of Q8_SG).  Measured on the batch-1
// step (interleaved, one box): 1 ahead 0.976 ms, 2 ahead 0.982, 3 ahead 0.985
constexpr int Q8_AHEAD = 1;
static_assert(Q8_AHEAD >= 1 && Q8_AHEAD < Q8_SG, "the ring holds the stage in use and those ahead");

__global__ __launch_bounds__(256) void k_q8_0_dequant(const unsigned char *w, float *out,
                                                      long long n) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;    // weight index
    if (i >= n) return;
    const unsigned char *blk = w + (i >> 5) * Q8_BLOCK_BYTES;
    const uint32_t h = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8);
    out[i] = half_bits_to_f32(h) * (float)(int8_t)blk[2 + (i & 31)];   // exact in fp32
}

// one thread per 16-byte piece of the tiled layout (272 pieces per unit)
__global__ __launch_bounds__(256) void k_q8_0_to_tiled(const unsigned char *src, unsigned char *dst,
                                                       int N, int G) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long units = (long long)(N / 16) * G;
    if (idx >= units * 272) return;
    const long long u = idx / 272;
    const int piece = (int)(idx - u * 272);
    const int t = (int)(u / G), g = (int)(u - (long long)t * G);
    const int KB = G * 8;                                  // blocks per row
    unsigned char out[16];
    if (piece < 16) {
        const unsigned char *row = src + ((size_t)(16 * t + piece) * KB + 8 * g) * Q8_BLOCK_BYTES;
#pragma unroll
        for (int b = 0; b < 8; b++) {
            out[2 * b] = row[Q8_BLOCK_BYTES * b];
            out[2 * b + 1] = row[Q8_BLOCK_BYTES * b + 1];
        }
    } else {
        const int j = piece - 16, p = j >> 6, l = j & 63, h = l >> 4, r = l & 15;
        const unsigned char *blk =
            src + ((size_t)(16 * t + r) * KB + 8 * g + 2 * p) * Q8_BLOCK_BYTES + 2 + 8 * h;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            out[i] = blk[i];
            out[8 + i] = blk[Q8_BLOCK_BYTES + i];
        }
    }
    u32x4_t v;
    memcpy(&v, out, 16);
    *reinterpret_cast<u32x4_t *>(dst + u * Q8_UNIT_BYTES + 16 * piece) = v;
}

struct Q8Stage {
    u32x4_t sc;                 // the 8 block scales of column cl (fp16 pairs)
    u32x4_t q[4];               // pairs of blocks: 8 bytes of block 2 p, then of 2 p + 1
};

__device__ __forceinline__ Q8Stage q8_load(const unsigned char *unit, int cl, int lane) {
    Q8Stage s;
    s.sc = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(unit + 16 * cl));
#pragma unroll
    for (int p = 0; p < 4; p++)
        s.q[p] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t *>(unit + 256 + 1024 * p + 16 * lane));
    return s;
}

// bf16 pair (lo = a, hi = b) of two floats whose values are exact in bf16
__device__ __forceinline__ uint32_t pack_exact(float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// 8 signed bytes (two dwords, k order) -> bf16 MFMA operand of the bytes + 128
__device__ __forceinline__ u32x4_t q8_decode(uint32_t w0, uint32_t w1) {
    const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
    u32x4_t b;
    b.x = pack_exact((float)(x0 & 0xFF), (float)((x0 >> 8) & 0xFF));
    b.y = pack_exact((float)((x0 >> 16) & 0xFF), (float)(x0 >> 24));
    b.z = pack_exact((float)(x1 & 0xFF), (float)((x1 >> 8) & 0xFF));
    b.w = pack_exact((float)((x1 >> 16) & 0xFF), (float)(x1 >> 24));
    return b;
}

// PX > 0: rows r and r + PX / 4 are one (hi, lo) pair, held PX lanes apart
template <int WPG, int PX>
__global__ __launch_bounds__(64 * WPG) void k_q8_stream(Q4kFusedArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    u32x4_t *A_lds = reinterpret_cast<u32x4_t *>(lds);                     // [SG][8][64]
    f32x4_t *C_lds = reinterpret_cast<f32x4_t *>(A_lds + Q8_SG * 8 * 64);  // [SG][8][4]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, cl = lane & 15;
    const int split = blockIdx.y, g0 = split * Q8_SG;
    const int ntile = a.N / 16;
    // balanced runs of the split's column tiles over its nw waves
    const int nw = gridDim.x * WPG, w = blockIdx.x * WPG + wave;
    const int t0 = (int)((long long)w * ntile / nw);
    const int t1 = (int)((long long)(w + 1) * ntile / nw);
    const int tlast = (t1 > t0 ? t1 : ntile) - 1;       // clamp target, always a real tile

    // stage (tile t, group sg of the split) is the unit at tile_base(t) + sg * 4352;
    // tiles past t1 - 1 clamp to tlast (in bounds, unused)
    auto tile_base = [&](int t) -> const unsigned char * {
        const int tt = t < t1 ? t : tlast;
        const int c16 = tt * 16;
        const int si = (a.nseg > 1 && c16 >= a.seg_end[0]) + (a.nseg > 2 && c16 >= a.seg_end[1]);
        const unsigned char *wseg = si == 0 ? a.w[0] : (si == 1 ? a.w[1] : a.w[2]);
        const int nbase = si == 0 ? 0 : (si == 1 ? a.seg_end[0] : a.seg_end[1]);
        return wseg + ((size_t)((c16 - nbase) >> 4) * a.KB + g0) * Q8_UNIT_BYTES;
    };
    auto stage = [&](const unsigned char *tb, int sg) -> Q8Stage {
        return q8_load(tb + sg * Q8_UNIT_BYTES, cl, lane);
    };
    // activations of this split -> LDS in lane order: entry (sg, j, lane) holds row cl's
    // values k = (g0 + sg) 256 + 32 j + 8 g .. + 7 (rows >= M: zeros); loaded before the
    // first weight stages so that their wait does not include the weights' latency
    constexpr int PER = Q8_SG * 8 / WPG;
    Q8Stage st[Q8_SG];
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
        st[0] = stage(b0, 0);
        if (Q8_AHEAD > 1) st[1] = stage(b0, 1);
        if (Q8_AHEAD > 2) st[2] = stage(b0, 2);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < PER; i++)
            A_lds[(wave + WPG * i) * 64 + lane] = cl < a.M ? av[i] : (u32x4_t){0u, 0u, 0u, 0u};
    }
    __syncthreads();
    // block sums: MFMA of each entry with a ones operand (every column of the product
    // is the row sum); kept as -128 S, the accumulator input of that block's MFMA
    {
        const uint32_t one2 = 0x3F803F80u;
        const u32x4_t ones = {one2, one2, one2, one2};
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int e = wave + WPG * i;
            const f32x4_t D = mfma16x16x32(A_lds[e * 64 + lane], ones, (f32x4_t){0.f, 0.f, 0.f, 0.f});
            if (cl == 0) C_lds[e * 4 + g] = -128.f * D;
        }
    }
    __syncthreads();

    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    const int m_out = PX ? PX / 4 : a.M;
    float *part = a.part + (size_t)split * m_out * a.N;
    int a_off = lane, c_off = g;
    for (int t = t0; t < t1; t++) {
        // opaque to the compiler: keeps the activation fragments in LDS
        asm volatile("" : "+v"(a_off), "+v"(c_off));
        const unsigned char *bcur = tile_base(t), *bnext = tile_base(t + 1);
        // in the run's last tile the loads ahead re-read unit (t, 3), just requested (an
        // L2 hit, unused)
        const bool more = t + 1 < t1;
        f32x4_t acc = zero;
#pragma unroll
        for (int sg = 0; sg < Q8_SG; sg++) {
            const int ns = sg + Q8_AHEAD;           // stage loaded now: (t, ns) or (t + 1, ns - 4)
            st[ns % Q8_SG] = ns < Q8_SG ? stage(bcur, ns)
                                        : stage(more ? bnext : bcur, more ? ns - Q8_SG : Q8_SG - 1);
            __builtin_amdgcn_sched_barrier(0);
            const Q8Stage &w = st[sg];
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const u32x4_t &qv = w.q[j >> 1];
                const u32x4_t B = (j & 1) ? q8_decode(qv.z, qv.w) : q8_decode(qv.x, qv.y);
                const uint32_t sw = w.sc[j >> 1];
                const float d = half_bits_to_f32((j & 1) ? (sw >> 16) : (sw & 0xFFFFu));
                const int e = sg * 8 + j;
                const f32x4_t D = mfma16x16x32(A_lds[e * 64 + a_off], B, C_lds[e * 4 + c_off]);
                acc += d * D;
            }
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

hipError_t launch_q8_0_dequant(const void *w, float *out, long long n_blocks, hipStream_t st) {
    const long long n = n_blocks * 32;
    const long long blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_q8_0_dequant, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const unsigned char *)w, out, n);
    return hipGetLastError();
}

hipError_t launch_q8_0_to_tiled(const unsigned char *src, unsigned char *dst, int N, int G,
                                hipStream_t st) {
    const long long pieces = (long long)(N / 16) * G * 272;
    const long long blocks = (pieces + 255) / 256;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_q8_0_to_tiled, dim3((unsigned)blocks), dim3(256), 0, st, src, dst, N, G);
    return hipGetLastError();
}

bool q8_stream_ok(int M, int N, int K) {
    return M >= 1 && M <= 16 && K % 256 == 0 && (K / 256) % Q8_SG == 0 && N % 16 == 0;
}

Q4kStreamPlan q8_stream_plan(int M, int N, int K, int pair, int target_waves, int wpg) {
    Q4kStreamPlan p;
    const int G = K / 256, ntile = N / 16;
    p.splits = G / Q8_SG;
    p.wpg = wpg > 0 ? wpg : 8;
    // about target_waves waves in all, no more workgroups per split than it has tiles
    // for a wave each
    p.grid_x = max(1, min(target_waves / (p.wpg * p.splits), ceil_div(ntile, p.wpg)));
    p.tpw = ceil_div(ntile, p.grid_x * p.wpg);          // (the longest run)
    p.pair_done = (pair == 4 || pair == 8) && M == 2 * pair;
    p.px = p.pair_done ? 4 * pair : 0;
    p.lds_bytes = (size_t)Q8_SG * 8 * 64 * 16 + (size_t)Q8_SG * 8 * 4 * 16;
    p.part_bytes = (size_t)p.splits * (p.pair_done ? pair : M) * N * 4;
    return p;
}

hipError_t launch_q8_stream(const Q4kFusedArgs &a, const Q4kStreamPlan &p, hipStream_t st) {
    const dim3 grid(p.grid_x, p.splits);
#define Q8_CASE(WPG, PX)                                                                             \
    if (p.wpg == WPG && p.px == PX) {                                                                \
        hipLaunchKernelGGL((k_q8_stream<WPG, PX>), grid, dim3(64 * WPG), p.lds_bytes, st, a);        \
        return hipGetLastError();                                                                    \
    }
    Q8_CASE(4, 0)
    Q8_CASE(4, 16)
    Q8_CASE(4, 32)
    Q8_CASE(8, 0)
    Q8_CASE(8, 16)
    Q8_CASE(8, 32)
#undef Q8_CASE
    return hipErrorInvalidValue;
}
