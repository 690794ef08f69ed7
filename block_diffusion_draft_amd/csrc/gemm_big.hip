// Dense-contraction GEMM for many activation rows (the batched draft steps), gfx950:
// C[split][M][N] (fp32) = A[M][K] (bf16) . W[N][K]^T over the split's K range, with W in
// bf16, Q8_0 or Q4_K (tiled layouts of q8_0.hip / q4k_tiled.hip).
//
// At 100+ rows the drafter's products are MFMA-bound (2 M flops per weight against
// 0.56-2 bytes), so the weights are decoded once per 256 x 256 output tile into bf16
// MFMA operands (Q4_K: d sc q - dmin m, Q8_0: d q, rounded to nearest even: relative
// error <= 2^-9 per weight) and the tile runs on v_mfma_f32_32x32x16_bf16 (on this chip
// the 32x32 form runs at twice the rate of the 16x16x32 one: 2.4 against 1.3 PFLOP/s
// measured with independent chains).
//
// Workgroup: 8 waves (2 along M x 4 along N), each a 128 x 64 block of 4 x 2 MFMA tiles
// (128 accumulators per lane).  K advances 64 per stage (4 MFMA k-steps): the stage's A
// rows and decoded W rows sit in LDS in MFMA lane order (16-byte entries, conflict-free
// reads), double buffered; the next stage's global loads are issued before the current
// stage's MFMAs and written to the other buffer after them, so one barrier per stage.
// Split-K over grid.z keeps at least about one workgroup per CU when M x N is small;
// the splits' partials are summed by the consumers (reduce kernels), as for every other
// GEMM of the step.  With one split, an optional row scale (deferred RMSNorm) is applied.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int BN = 256, BK = 64, NTH = 512;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// weight segment of output column n: its base pointer and the first column of the segment
__device__ __forceinline__ const unsigned char *seg_of(const BigGemmArgs &a, int n, int &nbase) {
    const int si = (a.nseg > 1 && n >= a.seg_end[0]) + (a.nseg > 2 && n >= a.seg_end[1]);
    nbase = si == 0 ? 0 : (si == 1 ? a.seg_end[0] : a.seg_end[1]);
    return reinterpret_cast<const unsigned char *>(si == 0 ? a.w[0] : (si == 1 ? a.w[1] : a.w[2]));
}

// slot of fragment lane l (k group k8 = 2 ks + l / 32 of the stage) in its 1 KB block:
// the lane index xor 2 k8.  Reads (16 lanes of one half: a constant xor) and writes (a
// wave's 8 rows x 8 k groups, or 16 columns of one k group) then reach 16 distinct
// 16-byte bank groups per 16 lanes.
__device__ __forceinline__ int swz(int l, int k8) { return l ^ (2 * k8); }

// raw weight data of one stage held by a thread between its load and its LDS store
struct WRaw {
    u32x4_t v[4];
};

// bf16 of x0 * s - t for the 8 integers of a fragment entry
__device__ __forceinline__ u32x4_t scale8(const float (&q)[8], float s, float t) {
    return (u32x4_t){pack_bf16x2(q[0] * s - t, q[1] * s - t), pack_bf16x2(q[2] * s - t, q[3] * s - t),
                     pack_bf16x2(q[4] * s - t, q[5] * s - t), pack_bf16x2(q[6] * s - t, q[7] * s - t)};
}

template <int WF, int BM>
__global__ __launch_bounds__(NTH) void k_gemm_big(BigGemmArgs a) {
    constexpr int RG = BM / 32;                       // 32-row groups of A per stage
    constexpr int WM = BM / 2;                        // rows per wave
    constexpr int FM = WM / 32;                       // MFMA row tiles per wave
    constexpr int APT = BM * 8 / NTH;                 // A entries per thread per stage
    extern __shared__ __align__(16) u32x4_t lds[];
    // stage entries [4 ks][32-row / 32-column group][64 slots]: fragment lane (r % 32) +
    // 32 h (row r's 8 values k = 16 ks + 8 h .. + 7) at slot swz(lane, 2 ks + h)
    u32x4_t *As = lds;                                // [2][4][RG][64]
    u32x4_t *Bs = lds + 2 * 4 * RG * 64;              // [2][4][8][64]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int nst = a.K / BK;
    const int s0 = (int)((long long)nst * blockIdx.z / gridDim.z);
    const int s1 = (int)((long long)nst * (blockIdx.z + 1) / gridDim.z);

    // ---- A: entry e = tid + NTH i: row e / 8, 8-value group kg = e % 8 of the stage
    const uint16_t *arow[APT];
    bool aok[APT];
#pragma unroll
    for (int i = 0; i < APT; i++) {
        const int e = tid + NTH * i, r = m0 + e / 8;
        aok[i] = r < a.M;
        arow[i] = a.A + (size_t)(aok[i] ? r : a.M - 1) * a.lda + 8 * (e % 8);
    }
    // ---- W: bf16: entry e = tid + NTH i (i < 4): row e / 8, group e % 8.  Q8_0 / Q4_K:
    // task e = tid + NTH i (i < 2): 16-column group cg = e / 64, lane ln = e % 64 of the
    // MFMA fragment (column ln % 16, k group ln / 16)
    const unsigned char *wbase[4];
    bool wok[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        int n;
        if (WF == 0) n = n0 + (tid + NTH * i) / 8;
        else n = n0 + 16 * ((tid + NTH * (i & 1)) / 64) + ((tid + NTH * (i & 1)) & 15);
        wok[i] = n < a.N;
        int nb;
        const unsigned char *ws = seg_of(a, wok[i] ? n : a.N - 1, nb);
        const int nn = (wok[i] ? n : a.N - 1) - nb;
        if (WF == 0) wbase[i] = ws + ((size_t)nn * a.K + 8 * ((tid + NTH * i) % 8)) * 2;
        else if (WF == 1) wbase[i] = ws + (size_t)(nn >> 4) * (a.K / 256) * Q8_UNIT_BYTES;
        else wbase[i] = ws + (size_t)(nn >> 4) * (a.K / 256) * Q4K_UNIT_BYTES;
    }

    // registers of one stage between its global loads and its LDS store
    struct Regs {
        u32x4_t ra[APT];
        WRaw rw;
    };
    auto gload = [&](Regs &R, int s) {
        u32x4_t (&ra)[APT] = R.ra;
        WRaw &rw = R.rw;
        const int k0 = s * BK;
#pragma unroll
        for (int i = 0; i < APT; i++) ra[i] = *reinterpret_cast<const u32x4_t *>(arow[i] + k0);
        if (WF == 0) {
#pragma unroll
            for (int i = 0; i < 4; i++)
                rw.v[i] = *reinterpret_cast<const u32x4_t *>(wbase[i] + (size_t)k0 * 2);
        } else if (WF == 1) {
            // unit of K-group k0 / 256; this stage is the block pair p = (k0 % 256) / 64
            const int g = k0 >> 8, p = (k0 & 255) >> 6;
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int ln = (tid + NTH * i) & 63;
                const unsigned char *unit = wbase[i] + (size_t)g * Q8_UNIT_BYTES;
                rw.v[2 * i] = *reinterpret_cast<const u32x4_t *>(unit + 256 + 1024 * p + 16 * ln);
                // the fp16 scales of blocks 2 p and 2 p + 1 of column ln % 16
                rw.v[2 * i + 1].x = *reinterpret_cast<const uint32_t *>(unit + 16 * (ln & 15) + 4 * p);
            }
        } else {
            // super-block k0 / 256; this stage is chunk c = (k0 % 256) / 64, 8 bytes of the
            // lane's slot in half c / 2
            const int sb = k0 >> 8, c = (k0 & 255) >> 6;
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int ln = (tid + NTH * i) & 63;
                const unsigned char *unit = wbase[i] + (size_t)sb * Q4K_UNIT_BYTES;
                const u32x2_t q = *reinterpret_cast<const u32x2_t *>(
                    unit + 256 + 1024 * (c >> 1) + 16 * ln + 8 * (c & 1));
                rw.v[2 * i] = (u32x4_t){q.x, q.y, (uint32_t)c, 0u};
                rw.v[2 * i + 1] = *reinterpret_cast<const u32x4_t *>(unit + 16 * (ln & 15));
            }
        }
    };
    auto lstore = [&](const Regs &R, int buf) {
        const u32x4_t (&ra)[APT] = R.ra;
        const WRaw &rw = R.rw;
        u32x4_t *Ab = As + buf * 4 * RG * 64;
        u32x4_t *Bb = Bs + buf * 4 * 8 * 64;
#pragma unroll
        for (int i = 0; i < APT; i++) {
            const int e = tid + NTH * i, r = e / 8, kg = e % 8;
            Ab[((kg >> 1) * RG + (r >> 5)) * 64 + swz((r & 31) + 32 * (kg & 1), kg)] =
                aok[i] ? ra[i] : (u32x4_t){0u, 0u, 0u, 0u};
        }
        if (WF == 0) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int e = tid + NTH * i, r = e / 8, kg = e % 8;
                Bb[((kg >> 1) * 8 + (r >> 5)) * 64 + swz((r & 31) + 32 * (kg & 1), kg)] =
                    wok[i] ? rw.v[i] : (u32x4_t){0u, 0u, 0u, 0u};
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int e = tid + NTH * i, cg = e / 64, ln = e & 63;
                u32x4_t o0 = {0u, 0u, 0u, 0u}, o1 = {0u, 0u, 0u, 0u};
                if (wok[i]) {
                    const u32x4_t q = rw.v[2 * i], h = rw.v[2 * i + 1];
                    float lo[8], hi[8];
                    if (WF == 1) {
                        // blocks 2 p and 2 p + 1 of the pair: 8 signed bytes each
#pragma unroll
                        for (int b = 0; b < 8; b++) {
                            lo[b] = (float)(int8_t)((b < 4 ? q.x : q.y) >> (8 * (b & 3)));
                            hi[b] = (float)(int8_t)((b < 4 ? q.z : q.w) >> (8 * (b & 3)));
                        }
                    } else {
#pragma unroll
                        for (int b = 0; b < 8; b++) {
                            const uint32_t w = (b < 4 ? q.x : q.y) >> (8 * (b & 3));
                            lo[b] = (float)(w & 15u);
                            hi[b] = (float)((w >> 4) & 15u);
                        }
                    }
                    if (WF == 1) {
                        const uint32_t sw = h.x;
                        o0 = scale8(lo, half_bits_to_f32(sw & 0xFFFFu), 0.f);
                        o1 = scale8(hi, half_bits_to_f32(sw >> 16), 0.f);
                    } else {
                        // header: d, dmin, 6-bit scales and mins of sub-blocks 2 c, 2 c + 1
                        const int c = (int)q.z;
                        const float d = half_bits_to_f32(h.x & 0xFFFFu);
                        const float dmin = half_bits_to_f32(h.x >> 16);
                        const uint32_t sb[3] = {h.y, h.z, h.w};
                        auto byte = [&](int i2) { return (sb[i2 >> 2] >> (8 * (i2 & 3))) & 0xFFu; };
                        float sc[2], mn[2];
#pragma unroll
                        for (int u = 0; u < 2; u++) {
                            const int j = 2 * c + u;
                            uint32_t s6, m6;
                            if (j < 4) {
                                s6 = byte(j) & 63u;
                                m6 = byte(j + 4) & 63u;
                            } else {
                                s6 = (byte(j + 4) & 15u) | ((byte(j - 4) >> 6) << 4);
                                m6 = (byte(j + 4) >> 4) | ((byte(j) >> 6) << 4);
                            }
                            sc[u] = d * (float)s6;
                            mn[u] = dmin * (float)m6;
                        }
                        o0 = scale8(lo, sc[0], mn[0]);
                        o1 = scale8(hi, sc[1], mn[1]);
                    }
                }
                // the task's column c = 16 cg + ln % 16 and k group ln / 16 of each of the
                // stage's two 32-wide halves (o0: k 0..31, o1: k 32..63)
                const int kgr = ln >> 4, col = 16 * cg + (ln & 15);
                const int li = (col & 31) + 32 * (kgr & 1);
                Bb[((kgr >> 1) * 8 + (col >> 5)) * 64 + swz(li, kgr)] = o0;
                Bb[((2 + (kgr >> 1)) * 8 + (col >> 5)) * 64 + swz(li, 4 + kgr)] = o1;
            }
        }
    };

    f32x16_t acc[FM][2];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

    auto compute = [&](int buf) {
        const u32x4_t *Ab = As + buf * 4 * RG * 64;
        const u32x4_t *Bb = Bs + buf * 4 * 8 * 64;
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            u32x4_t bf[2];
#pragma unroll
            for (int j = 0; j < 2; j++) bf[j] = Bb[(ks * 8 + wn * 2 + j) * 64 + swz(lane, 2 * ks + (lane >> 5))];
#pragma unroll
            for (int i = 0; i < FM; i++) {
                const u32x4_t af = Ab[(ks * RG + wm * FM + i) * 64 + swz(lane, 2 * ks + (lane >> 5))];
#pragma unroll
                for (int j = 0; j < 2; j++) acc[i][j] = mfma32x32x16(af, bf[j], acc[i][j]);
            }
        }
    };
    Regs R;
    if (s0 < s1) {
        gload(R, s0);
        lstore(R, 0);
    }
    __syncthreads();
    // stage s sits in LDS buffer (s - s0) & 1; R carries the next stage's global loads
    for (int s = s0; s < s1; s++) {
        const int buf = (s - s0) & 1;
        if (s + 1 < s1) gload(R, s + 1);
        compute(buf);
        if (s + 1 < s1) lstore(R, buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane l of tile (i, j), register v: row 8 (v / 4) + 4 (l / 32) + v % 4,
    // column l % 32
    const int hl = lane >> 5, c = lane & 31;
    float *C = a.C + (size_t)blockIdx.z * a.M * a.ldc;
    const bool scale = gridDim.z == 1 && a.rs.ssq;
#pragma unroll
    for (int i = 0; i < FM; i++) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = m0 + wm * WM + 32 * i + 8 * (v >> 2) + 4 * hl + (v & 3);
            if (m >= a.M) continue;
            const float ri = scale ? row_inv(a.rs, m) : 1.f;
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int n = n0 + wn * 64 + 32 * j + c;
                if (n < a.N) C[(size_t)m * a.ldc + n] = acc[i][j][v] * ri;
            }
        }
    }
}

// bf16 weights: both operands travel global -> LDS by direct 16-byte loads
// (global_load_lds_dwordx4, no registers), K advancing 32 per stage through a ring of NS
// LDS buffers, so NS - 1 stages are in flight while one is multiplied.  A stage holds
// 32-row groups of 32 rows x 64 bytes (2 KB); lane L of a load instruction fills the
// 16-byte slot L of one 1 KB half, i.e. row 16 h + L / 4, chunk slot L % 4, and it loads
// the chunk (L % 4) ^ ((row / 4) % 4) of that row: four lanes cover a row's 64 bytes, and
// the 16 rows read together by an MFMA operand load (one chunk each) fall on 16
// distinct 16-byte bank groups.  Rows and columns past M / N load row M - 1 / column
// N - 1 (in bounds) and are never stored.
constexpr int BKD = 32;

__device__ __forceinline__ int dma_pos(int row, int chunk) { return 4 * row + (chunk ^ ((row >> 2) & 3)); }

template <int BM, int NS>
__global__ __launch_bounds__(NTH) void k_gemm_big_dma(BigGemmArgs a) {
    constexpr int RG = BM / 32, WM = BM / 2, FM = WM / 32;
    constexpr int NG = RG + 8;                        // 2 KB groups per stage (A, then W)
    constexpr int PW = 2 * NG / 8;                    // load instructions per wave and stage
    extern __shared__ __align__(16) u32x4_t lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int nst = a.K / BKD;
    const int s0 = (int)((long long)nst * blockIdx.z / gridDim.z);
    const int s1 = (int)((long long)nst * (blockIdx.z + 1) / gridDim.z);

    // this lane's source pointer for each of the wave's load instructions (k of stage added)
    const uint16_t *src[PW];
#pragma unroll
    for (int j = 0; j < PW; j++) {
        const int h = wave + 8 * j;                   // 1 KB half: group h / 2, rows 16 (h % 2) ..
        const int g = h >> 1, row = 16 * (h & 1) + (lane >> 2);
        const int chunk = (lane & 3) ^ ((row >> 2) & 3);
        if (g < RG) {
            const int r = min(m0 + 32 * g + row, a.M - 1);
            src[j] = a.A + (size_t)r * a.lda + 8 * chunk;
        } else {
            const int n = min(n0 + 32 * (g - RG) + row, a.N - 1);
            int nb;
            const unsigned char *ws = seg_of(a, n, nb);
            src[j] = reinterpret_cast<const uint16_t *>(ws) + (size_t)(n - nb) * a.K + 8 * chunk;
        }
    }
    auto issue = [&](int s, int buf) {
        const int k0 = s * BKD;
#pragma unroll
        for (int j = 0; j < PW; j++) {
            const int h = wave + 8 * j;
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1))) *)(src[j] + k0),
                (void __attribute__((address_space(3))) *)(lds + (buf * NG * 2 + h) * 64), 16, 0, 0);
        }
    };

    f32x16_t acc[FM][2];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

    // read positions of this lane's MFMA operands for the two k steps of a stage
    const int rl = lane & 31;
    const int rp0 = dma_pos(rl, lane >> 5), rp1 = dma_pos(rl, 2 + (lane >> 5));

    // prologue: stages s0 .. s0 + NS - 2 in flight (past the end: the last stage again,
    // into a buffer no stage reads, so every iteration waits on the same count)
#pragma unroll
    for (int p = 0; p < NS - 1; p++) issue(min(s0 + p, s1 - 1), p);
    for (int s = s0; s < s1; s++) {
        const int buf = (s - s0) % NS;
        // stage s has landed (the NS - 2 later ones may be in flight) in every wave; a
        // bare barrier, since a workgroup fence would wait for every load in flight
        __builtin_amdgcn_s_waitcnt(0xF70 | ((NS - 2) * PW));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // the buffer of stage s - 1 is free: stage s + NS - 1 goes there
        issue(min(s + NS - 1, s1 - 1), (s - s0 + NS - 1) % NS);
        const u32x4_t *Ab = lds + buf * NG * 128;
        const u32x4_t *Bb = Ab + RG * 128;
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
            const int rp = ks ? rp1 : rp0;
            u32x4_t bf[2];
#pragma unroll
            for (int j = 0; j < 2; j++) bf[j] = Bb[(wn * 2 + j) * 128 + rp];
#pragma unroll
            for (int i = 0; i < FM; i++) {
                const u32x4_t af = Ab[(wm * FM + i) * 128 + rp];
#pragma unroll
                for (int j = 0; j < 2; j++) acc[i][j] = mfma32x32x16(af, bf[j], acc[i][j]);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0xF70);      // no load may land after the workgroup ends

    const int hl = lane >> 5, c = lane & 31;
    float *C = a.C + (size_t)blockIdx.z * a.M * a.ldc;
    const bool scale = gridDim.z == 1 && a.rs.ssq;
#pragma unroll
    for (int i = 0; i < FM; i++) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = m0 + wm * WM + 32 * i + 8 * (v >> 2) + 4 * hl + (v & 3);
            if (m >= a.M) continue;
            const float ri = scale ? row_inv(a.rs, m) : 1.f;
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int n = n0 + wn * 64 + 32 * j + c;
                if (n < a.N) C[(size_t)m * a.ldc + n] = acc[i][j][v] * ri;
            }
        }
    }
}

}  // namespace

size_t big_gemm_lds_bytes(int BM) { return ((size_t)2 * 4 * (BM / 32) + 2 * 4 * 8) * 64 * 16; }
constexpr int DMA_NS = 4;
size_t big_gemm_dma_lds_bytes(int BM) { return (size_t)DMA_NS * (BM / 32 + 8) * 2048; }

BigGemmPlan big_gemm_plan(int M, int N, int K) {
    BigGemmPlan p;
    p.bm = M <= 128 ? 128 : 256;
    p.grid_x = ceil_div(N, BN);
    p.grid_y = ceil_div(M, p.bm);
    // split K while there are fewer than about two workgroups per CU, keeping at least
    // 8 stages (512 of K) per split
    const int nst = K / BK;
    p.splits = 1;
    while ((long long)p.grid_x * p.grid_y * p.splits * 2 <= 512 && nst / (p.splits * 2) >= 8 &&
           p.splits < 16)
        p.splits *= 2;
    p.lds_bytes = big_gemm_lds_bytes(p.bm);
    // (the bf16 kernel's ring is smaller; its launch sets its own size)
    p.part_bytes = (size_t)p.splits * M * N * 4;
    return p;
}

bool big_gemm_ok(int wf, int M, int N, int K) {
    if (M < 1 || N < 16 || N % 16) return false;
    return wf == 0 ? K % BK == 0 && K >= BK : K % 256 == 0 && K >= 256;
}

hipError_t launch_big_gemm(const BigGemmArgs &a, const BigGemmPlan &p, hipStream_t st) {
    if (!big_gemm_ok(a.wfmt, a.M, a.N, a.K)) return hipErrorInvalidValue;
    const dim3 grid(p.grid_x, p.grid_y, p.splits);
    static bool attr_set[3][2] = {};
#define BIG_CASE(WF, BMV)                                                                             \
    if (a.wfmt == WF && p.bm == BMV) {                                                               \
        if (!attr_set[WF][BMV == 256]) {                                                             \
            hipError_t e = hipFuncSetAttribute((const void *)k_gemm_big<WF, BMV>,                     \
                                               hipFuncAttributeMaxDynamicSharedMemorySize,            \
                                               (int)big_gemm_lds_bytes(BMV));                         \
            if (e != hipSuccess) return e;                                                           \
            attr_set[WF][BMV == 256] = true;                                                         \
        }                                                                                            \
        hipLaunchKernelGGL((k_gemm_big<WF, BMV>), grid, dim3(NTH), p.lds_bytes, st, a);             \
        return hipGetLastError();                                                                    \
    }
    if (a.wfmt == 0 && a.K % BKD == 0 && a.K / BKD >= p.splits) {
        static bool dma_set[2] = {false, false};
        const int bi = p.bm == 256;
        const size_t lb = big_gemm_dma_lds_bytes(p.bm);
        const void *fn = bi ? (const void *)k_gemm_big_dma<256, DMA_NS> : (const void *)k_gemm_big_dma<128, DMA_NS>;
        if (!dma_set[bi]) {
            hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lb);
            if (e != hipSuccess) return e;
            dma_set[bi] = true;
        }
        if (bi) hipLaunchKernelGGL((k_gemm_big_dma<256, DMA_NS>), grid, dim3(NTH), lb, st, a);
        else hipLaunchKernelGGL((k_gemm_big_dma<128, DMA_NS>), grid, dim3(NTH), lb, st, a);
        return hipGetLastError();
    }
    BIG_CASE(0, 128)
    BIG_CASE(0, 256)
    BIG_CASE(1, 128)
    BIG_CASE(1, 256)
    BIG_CASE(2, 128)
    BIG_CASE(2, 256)
#undef BIG_CASE
    return hipErrorInvalidValue;
}
