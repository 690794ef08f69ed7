// Dense-contraction GEMM for many activation rows (the batched draft steps), gfx950:
// C[slot][M][N] (fp32) = A[M][K] (bf16) . W[N][K]^T over the slot's share of K, with W
// in bf16, Q8_0 or Q4_K (tiled layouts of q8_0.hip / q4k_tiled.hip).  The consumers sum
// the slots (reduce kernels), as for every other GEMM of the step.
//
// At 100+ rows the drafter's products are MFMA-bound (2 M flops per weight against
// 0.56-2 bytes), so the weights are decoded once per 256 x 256 output tile into bf16
// MFMA operands (Q4_K: d sc q - dmin m, Q8_0: d q, rounded to nearest even: relative
// error <= 2^-9 per weight) and the tile runs on v_mfma_f32_32x32x16_bf16 (on this chip
// the 32x32 form runs at twice the rate of the 16x16x32 one: 2.4 against 1.3 PFLOP/s
// measured with independent chains).
//
// Workgroup: 8 waves (2 along M x 4 along N), each a 128 x 64 block (BM = 256; 64 x 64
// for BM = 128) of 32 x 32 MFMA tiles.  The operands sit in LDS in MFMA lane order,
// 16-byte entries placed so that operand reads are free of bank conflicts.  A (and bf16
// W) travel global -> LDS by direct loads (global_load_lds_dwordx4: no registers, no
// LDS store instructions) through a ring of K stages, several stages in flight while one
// is multiplied; Q8_0 / Q4_K weights are loaded into registers two stages ahead and
// decoded into a double-buffered LDS tile.
//
// Work split: a grid over (N tile, M tile, K split), or stream-K where the tiles would
// leave a partly empty last round of workgroups: the (tile, 64-deep K stage) units are
// cut into one equal range per CU; a range covers pieces of one to a few tiles, the
// piece with ordinal j of its tile goes to slot j, and a tile's last piece zeroes the
// tile's unused slots.  Either way the work is dealt so that each XCD (workgroup b
// runs on XCD b mod 8) takes a contiguous run of it: the M tiles of a weight slab
// then share that XCD's L2.  With a single slot, an optional row scale (deferred
// RMSNorm) is applied in the epilogue.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int BN = 256, BK = 64, NTH = 512;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// schedule of the workgroups: wgs == 0: one workgroup per (N tile, M tile, K split)
// item (a 1-D grid, items dealt to XCDs in contiguous runs); else stream-K
// over wgs workgroups (a multiple of 8), tx x ty tiles of nst stages, `slots` slots
struct BigSched {
    int wgs, tx, ty, nst, slots;
};

// weight segment of output column n: its base pointer and the first column of the segment
__device__ __forceinline__ const unsigned char *seg_of(const BigGemmArgs &a, int n, int &nbase) {
    const int si = (a.nseg > 1 && n >= a.seg_end[0]) + (a.nseg > 2 && n >= a.seg_end[1]);
    nbase = si == 0 ? 0 : (si == 1 ? a.seg_end[0] : a.seg_end[1]);
    return reinterpret_cast<const unsigned char *>(si == 0 ? a.w[0] : (si == 1 ? a.w[1] : a.w[2]));
}

// slot of fragment lane l (k group k8 = 2 ks + l / 32 of a 64-deep stage) in its 1 KB
// block of the decoded weight tile: the lane index xor 2 k8.  Reads (16 lanes of one
// half: a constant xor) and writes (16 columns of one k group) then reach 16 distinct
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

// Epilogue: lane l of tile (i, j), register v holds row 8 (v / 4) + 4 (l / 32) + v % 4,
// column l % 32.  With the row scale, it is computed once per row of the tile into LDS
// (rinv, free once every wave has left the K loop).
template <int BM, int FM, int FN = 2>
__device__ __forceinline__ void store_tile(const BigGemmArgs &a, const f32x16_t (&acc)[FM][FN],
                                           float *rinv, int m0, int n0, int wm, int wn, int tid,
                                           int slot, bool scale) {
    constexpr int WM = BM / 2, WN = 32 * FN;
    const int lane = tid & 63, hl = lane >> 5, c = lane & 31;
    float *C = a.C + (size_t)slot * a.M * a.ldc;
    if (scale) {
        __syncthreads();
        for (int r = tid; r < BM; r += NTH) rinv[r] = row_inv(a.rs, min(m0 + r, a.M - 1));
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < FM; i++) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int r = wm * WM + 32 * i + 8 * (v >> 2) + 4 * hl + (v & 3);
            if (m0 + r >= a.M) continue;
            const float ri = scale ? rinv[r] : 1.f;
#pragma unroll
            for (int j = 0; j < FN; j++) {
                const int n = n0 + wn * WN + 32 * j + c;
                if (n < a.N) C[(size_t)(m0 + r) * a.ldc + n] = acc[i][j][v] * ri;
            }
        }
    }
}

// zeroes slots [from, to) of a tile (N and ldc are multiples of 4)
template <int BM, int TBN = BN>
__device__ __forceinline__ void zero_slots(const BigGemmArgs &a, int m0, int n0, int from, int to, int tid) {
    for (int z = from; z < to; z++) {
        float *C = a.C + (size_t)z * a.M * a.ldc;
        for (int e = tid; e < BM * TBN / 4; e += NTH) {
            const int m = m0 + e / (TBN / 4), n = n0 + 4 * (e % (TBN / 4));
            if (m < a.M && n < a.N)
                *reinterpret_cast<float4 *>(C + (size_t)m * a.ldc + n) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
}

// The workgroup's work as tile pieces (64-deep K stages [s0, s1) of the tile at m0, n0,
// into slot `slot`).  Stream-K: the units (tile t, stage s), t in M-fastest order, are
// cut into wgs ranges [g U / wgs, (g + 1) U / wgs); range g belongs to workgroup id
// (g % (wgs / 8)) * 8 + g / (wgs / 8), so that neighbouring ranges (the M tiles of one
// weight slab) run on one XCD (workgroups are dealt round robin over the 8 XCDs) and
// share its L2.  A piece's slot is its distance from the range holding the tile's
// first unit; `last`: the tile's last piece (it zeroes the slots after its own).
struct Piece {
    int m0, n0, s0, s1, slot;
    bool scale, last;
};
struct Pieces {
    long long u, u1, U;
    int g;
    __device__ __forceinline__ Pieces(const BigGemmArgs &a, const BigSched &sc) {
        if (sc.wgs == 0) {
            u = 0;
            u1 = 1;
            U = 1;
            g = 0;
        } else {
            g = (blockIdx.x & 7) * (sc.wgs >> 3) + (blockIdx.x >> 3);
            U = (long long)sc.tx * sc.ty * sc.nst;
            u = (long long)g * U / sc.wgs;
            u1 = (long long)(g + 1) * U / sc.wgs;
        }
    }
    template <int BM, int TBN = BN>
    __device__ __forceinline__ bool next(const BigGemmArgs &a, const BigSched &sc, Piece &p) {
        if (u >= u1) return false;
        if (sc.wgs == 0) {
            // grid of tx * ty * slots workgroups, one piece each: workgroup b takes item
            // L, the items in (split, N tile, M tile) order with M fastest, dealt so that
            // each XCD runs a contiguous run of items (the M tiles of one weight slab,
            // and neighbouring slabs of one K split, share that XCD's L2)
            const int total = sc.tx * sc.ty * sc.slots, q = total >> 3, r = total & 7;
            const int x8 = blockIdx.x & 7;
            const int L = x8 * q + min(x8, r) + (int)(blockIdx.x >> 3);
            const int z = L / (sc.tx * sc.ty), rem = L - z * sc.tx * sc.ty;
            const int nst = a.K / BK;
            p.m0 = (rem % sc.ty) * BM;
            p.n0 = (rem / sc.ty) * TBN;
            p.s0 = (int)((long long)nst * z / sc.slots);
            p.s1 = (int)((long long)nst * (z + 1) / sc.slots);
            p.slot = z;
            p.scale = sc.slots == 1 && a.rs.ssq;
            p.last = false;
            u = u1;
            return true;
        }
        const int t = (int)(u / sc.nst);
        p.s0 = (int)(u - (long long)t * sc.nst);
        p.s1 = (int)min((long long)sc.nst, p.s0 + (u1 - u));
        const long long x = (long long)t * sc.nst;
        p.slot = g - ((int)(((x + 1) * sc.wgs + U - 1) / U) - 1);   // (range holding unit x)
        p.m0 = (t % sc.ty) * BM;
        p.n0 = (t / sc.ty) * TBN;
        p.scale = sc.slots == 1 && a.rs.ssq;
        p.last = p.s1 == sc.nst;
        u += p.s1 - p.s0;
        return true;
    }
};

// ---- Q8_0 / Q4_K weight tasks.  Task e = tid + NTH i (i < 2) of a thread: 16-column
// group cg = e / 64 of the tile, lane ln = e % 64 of the MFMA fragment (column ln % 16,
// k group ln / 16).  wbase: the column group's first tiled unit.
template <int WF>
__device__ __forceinline__ void wq_setup(const BigGemmArgs &a, int n0, int tid,
                                         const unsigned char *(&wbase)[2], bool (&wok)[2]) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int e = tid + NTH * i;
        const int n = n0 + 16 * (e / 64) + (e & 15);
        wok[i] = n < a.N;
        int nb;
        const unsigned char *ws = seg_of(a, wok[i] ? n : a.N - 1, nb);
        const int nn = (wok[i] ? n : a.N - 1) - nb;
        wbase[i] = ws + (size_t)(nn >> 4) * (a.K / 256) * (WF == 1 ? Q8_UNIT_BYTES : Q4K_UNIT_BYTES);
    }
}

// raw bytes of the stage at k0 (64 deep): Q8_0: the 16 bytes of blocks 2 p, 2 p + 1 of
// the lane's slot and their two fp16 scales; Q4_K: 8 bytes of the lane's slot (chunk c of
// the super-block) and the column's 16-byte header.  Four loads per thread.
template <int WF>
__device__ __forceinline__ void wq_load(WRaw &rw, const unsigned char *const (&wbase)[2], int tid, int k0) {
    if (WF == 1) {
        const int g = k0 >> 8, p = (k0 & 255) >> 6;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int ln = (tid + NTH * i) & 63;
            const unsigned char *unit = wbase[i] + (size_t)g * Q8_UNIT_BYTES;
            rw.v[2 * i] = *reinterpret_cast<const u32x4_t *>(unit + 256 + 1024 * p + 16 * ln);
            rw.v[2 * i + 1].x = *reinterpret_cast<const uint32_t *>(unit + 16 * (ln & 15) + 4 * p);
        }
    } else {
        const int sb = k0 >> 8, c = (k0 & 255) >> 6;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int ln = (tid + NTH * i) & 63;
            const unsigned char *unit = wbase[i] + (size_t)sb * Q4K_UNIT_BYTES;
            const u32x2_t q = *reinterpret_cast<const u32x2_t *>(unit + 256 + 1024 * (c >> 1) + 16 * ln + 8 * (c & 1));
            rw.v[2 * i] = (u32x4_t){q.x, q.y, (uint32_t)c, 0u};
            rw.v[2 * i + 1] = *reinterpret_cast<const u32x4_t *>(unit + 16 * (ln & 15));
        }
    }
}

// decode a stage's raw bytes into bf16 MFMA operands in the W tile Bb ([4 ks][8][64],
// slot swz): entry o0 holds k 0..31 of the stage, o1 k 32..63
template <int WF>
__device__ __forceinline__ void wq_store(u32x4_t *Bb, const WRaw &rw, const bool (&wok)[2], int tid) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int e = tid + NTH * i, cg = e / 64, ln = e & 63;
        u32x4_t o0 = {0u, 0u, 0u, 0u}, o1 = {0u, 0u, 0u, 0u};
        if (wok[i]) {
            const u32x4_t q = rw.v[2 * i], h = rw.v[2 * i + 1];
            float lo[8], hi[8];
            if (WF == 1) {
#pragma unroll
                for (int b = 0; b < 8; b++) {
                    lo[b] = (float)(int8_t)((b < 4 ? q.x : q.y) >> (8 * (b & 3)));
                    hi[b] = (float)(int8_t)((b < 4 ? q.z : q.w) >> (8 * (b & 3)));
                }
                o0 = scale8(lo, half_bits_to_f32(h.x & 0xFFFFu), 0.f);
                o1 = scale8(hi, half_bits_to_f32(h.x >> 16), 0.f);
            } else {
#pragma unroll
                for (int b = 0; b < 8; b++) {
                    const uint32_t w = (b < 4 ? q.x : q.y) >> (8 * (b & 3));
                    lo[b] = (float)(w & 15u);
                    hi[b] = (float)((w >> 4) & 15u);
                }
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
        const int kgr = ln >> 4, col = 16 * cg + (ln & 15);
        const int li = (col & 31) + 32 * (kgr & 1);
        Bb[((kgr >> 1) * 8 + (col >> 5)) * 64 + swz(li, kgr)] = o0;
        Bb[((2 + (kgr >> 1)) * 8 + (col >> 5)) * 64 + swz(li, 4 + kgr)] = o1;
    }
}

// bf16 weights: both operands through a ring of NS stages of 32 K.  A stage holds
// 32-row groups of 32 rows x 64 bytes (2 KB); lane L of a load instruction fills the
// 16-byte slot L of one 1 KB half, i.e. row 16 h + L / 4, chunk slot L % 4, and it loads
// the chunk (L % 4) ^ ((row / 4) % 4) of that row: four lanes cover a row's 64 bytes, and
// the 16 rows read together by an MFMA operand load (one chunk each) fall on 16
// distinct 16-byte bank groups.  Rows and columns past M / N load row M - 1 / column
// N - 1 (in bounds) and are never stored.
constexpr int BKD = 32, DMA_NS = 4;

__device__ __forceinline__ int dma_pos(int row, int chunk) { return 4 * row + (chunk ^ ((row >> 2) & 3)); }

// one tile piece (BM x TBN) over 32-deep stages [s0, s1)
template <int BM, int NS, int TBN>
__device__ __forceinline__ void dma_piece(const BigGemmArgs &a, u32x4_t *lds, int m0, int n0, int s0,
                                          int s1, int slot, bool scale) {
    constexpr int RG = BM / 32, WM = BM / 2, FM = WM / 32, FN = TBN / 128;
    constexpr int NG = RG + TBN / 32;                 // 2 KB groups per stage (A, then W)
    constexpr int PW = 2 * NG / 8;                    // load instructions per wave and stage
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;

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

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
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
            u32x4_t bf[FN];
#pragma unroll
            for (int j = 0; j < FN; j++) bf[j] = Bb[(wn * FN + j) * 128 + rp];
#pragma unroll
            for (int i = 0; i < FM; i++) {
                const u32x4_t af = Ab[(wm * FM + i) * 128 + rp];
#pragma unroll
                for (int j = 0; j < FN; j++) acc[i][j] = mfma32x32x16(af, bf[j], acc[i][j]);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0xF70);      // no load may land after the piece ends

    store_tile<BM, FM, FN>(a, acc, reinterpret_cast<float *>(lds), m0, n0, wm, wn, tid, slot, scale);
}

template <int BM, int TBN>
__global__ __launch_bounds__(NTH) void k_gemm_big_dma(BigGemmArgs a, BigSched sc) {
    extern __shared__ __align__(16) u32x4_t lds[];
    Pieces it(a, sc);
    Piece pc;
    for (bool first = true; it.next<BM, TBN>(a, sc, pc); first = false) {
        if (!first) __syncthreads();                  // the previous piece is done with LDS
        dma_piece<BM, DMA_NS, TBN>(a, lds, pc.m0, pc.n0, 2 * pc.s0, 2 * pc.s1, pc.slot, pc.scale);
        if (pc.last) zero_slots<BM, TBN>(a, pc.m0, pc.n0, pc.slot + 1, sc.slots, threadIdx.x);
    }
}

// Q8_0 / Q4_K weights: A through a ring of QNS stages of 64 K (two in flight while one
// is multiplied): stage rows of 128 bytes, eight lanes per row, lane L of a load
// instruction at slot L of its 1 KB piece (row 8 piece + L / 8) loading chunk
// (L % 8) ^ ((row / 2) % 8), so the 16 rows of an MFMA operand load fall on distinct bank
// groups.  The raw weight bytes of a stage are loaded into registers two stages ahead
// (two register sets, alternating) and decoded into the double-buffered W tile after
// the current stage's MFMAs.
constexpr int QNS = 3;

// one tile piece over 64-deep stages [s0, s1)
template <int WF, int BM>
__device__ __forceinline__ void q_piece(const BigGemmArgs &a, u32x4_t *lds, int m0, int n0, int s0,
                                        int s1, int slot, bool scale) {
    constexpr int WM = BM / 2, FM = WM / 32;
    constexpr int PA = BM / 64;                       // A load instructions per wave and stage
    constexpr int AST = BM * 8;                       // entries of one A stage
    constexpr int PWQ = 4;                            // weight loads per thread and stage
    u32x4_t *As = lds;                                // [QNS][BM][8]
    u32x4_t *Bs = lds + QNS * AST;                    // [2][4 ks][8][64]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;

    const uint16_t *asrc[PA];
#pragma unroll
    for (int j = 0; j < PA; j++) {
        const int row = 8 * (wave + 8 * j) + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        asrc[j] = a.A + (size_t)min(m0 + row, a.M - 1) * a.lda + 8 * chunk;
    }
    auto issue_a = [&](int s, int buf) {
#pragma unroll
        for (int j = 0; j < PA; j++)
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1))) *)(asrc[j] + s * BK),
                (void __attribute__((address_space(3))) *)(As + buf * AST + (wave + 8 * j) * 64), 16, 0, 0);
    };
    const unsigned char *wbase[2];
    bool wok[2];
    wq_setup<WF>(a, n0, tid, wbase, wok);

    f32x16_t acc[FM][2];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

    const int rl = lane & 31, rsw = (rl >> 1) & 7;
    auto compute = [&](const u32x4_t *Ab, const u32x4_t *Bb) {
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            const int c = 2 * ks + (lane >> 5);
            u32x4_t bf[2];
#pragma unroll
            for (int j = 0; j < 2; j++) bf[j] = Bb[(ks * 8 + wn * 2 + j) * 64 + swz(lane, c)];
#pragma unroll
            for (int i = 0; i < FM; i++) {
                const u32x4_t af = Ab[(32 * (wm * FM + i) + rl) * 8 + (c ^ rsw)];
#pragma unroll
                for (int j = 0; j < 2; j++) acc[i][j] = mfma32x32x16(af, bf[j], acc[i][j]);
            }
        }
    };
    // wait until at most one stage's loads are in flight (the one issued last)
    auto wait_one = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xF70 | (PA + PWQ));
        asm volatile("" ::: "memory");
    };
    // stage s: A(s) and the decoded W(s) are in LDS once every wave passes the barrier;
    // rn1 holds the raw weights of stage s + 1 (in flight), rn2 receives stage s + 2.
    // Stages past the end load the last stage again into buffers no stage reads, so the
    // wait counts stay fixed.
    auto body = [&](int s, WRaw &rn1, WRaw &rn2) {
        const int i = s - s0;
        __builtin_amdgcn_s_waitcnt(0xC07F);           // this wave's LDS stores done
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int s2 = min(s + 2, s1 - 1);
        issue_a(s2, (i + 2) % QNS);
        wq_load<WF>(rn2, wbase, tid, s2 * BK);
        asm volatile("" ::: "memory");                // (issued before the MFMAs)
        compute(As + (i % QNS) * AST, Bs + (i & 1) * 2048);
        wait_one();
        wq_store<WF>(Bs + ((i + 1) & 1) * 2048, rn1, wok, tid);
    };
    WRaw ra, rb;
    issue_a(s0, 0);
    wq_load<WF>(ra, wbase, tid, s0 * BK);
    issue_a(min(s0 + 1, s1 - 1), 1);
    wq_load<WF>(rb, wbase, tid, min(s0 + 1, s1 - 1) * BK);
    wait_one();
    wq_store<WF>(Bs, ra, wok, tid);
    int s = s0;
    for (; s + 1 < s1; s += 2) {
        body(s, rb, ra);
        body(s + 1, ra, rb);
    }
    if (s < s1) body(s, rb, ra);
    __builtin_amdgcn_s_waitcnt(0xF70);      // no load may land after the piece ends

    store_tile<BM, FM>(a, acc, reinterpret_cast<float *>(lds), m0, n0, wm, wn, tid, slot, scale);
}

template <int WF, int BM>
__global__ __launch_bounds__(NTH) void k_gemm_big_q(BigGemmArgs a, BigSched sc) {
    extern __shared__ __align__(16) u32x4_t lds[];
    Pieces it(a, sc);
    Piece pc;
    for (bool first = true; it.next<BM>(a, sc, pc); first = false) {
        if (!first) __syncthreads();                  // the previous piece is done with LDS
        q_piece<WF, BM>(a, lds, pc.m0, pc.n0, pc.s0, pc.s1, pc.slot, pc.scale);
        if (pc.last) zero_slots<BM>(a, pc.m0, pc.n0, pc.slot + 1, sc.slots, threadIdx.x);
    }
}

}  // namespace

size_t dma_lds_bytes(int BM, int TBN) { return (size_t)DMA_NS * (BM / 32 + TBN / 32) * 2048; }
size_t q_lds_bytes(int BM) { return ((size_t)QNS * BM * 8 + 2 * 2048) * 16; }

namespace {

// Stream-K range count and the CU count the schedule is planned for: 256, the CUs of
// this part.  Fixed rather than read from the device, so that a product's partial sums
// (hence its rounding) are the same on every device; on a part with another CU count
// the 256 ranges simply run in more or fewer rounds.
int cu_count() { return 256; }

// most pieces any tile is cut into by G stream-K ranges over T tiles of nst stages
int sk_slots(long long T, int nst, int G) {
    const long long U = T * nst;
    int mx = 0;
    for (long long t = 0; t < T; t++) {
        const long long x0 = t * nst, x1 = x0 + nst - 1;
        const long long g0 = ((x0 + 1) * G + U - 1) / U - 1, g1 = ((x1 + 1) * G + U - 1) / U - 1;
        mx = max(mx, (int)(g1 - g0 + 1));
    }
    return mx;
}

}  // namespace

BigGemmPlan big_gemm_plan_grid(int wf, int M, int N, int K) {
    BigGemmPlan p;
    p.bm = M <= 128 ? 128 : 256;
    // bf16 at up to 128 rows with enough columns for a tile per CU even at 512 wide (the
    // output head): 128 x 512 tiles, each wave 64 x 128, as few LDS operand bytes per
    // MFMA as the 256 x 256 tile (measured 565 against 603 µs at 112 x 248320 x 5120;
    // slower on the drafter's narrower products, which need their tiles for splits)
    p.bn = wf == 0 && M <= 128 && ceil_div(N, 512) >= cu_count() ? 512 : BN;
    p.grid_x = ceil_div(N, p.bn);
    p.grid_y = ceil_div(M, p.bm);
    p.wgs = 0;
    p.splits = 1;
    p.part_bytes = (size_t)M * N * 4;
    return p;
}

BigGemmPlan big_gemm_plan(int wf, int M, int N, int K) {
    // Estimated time, in stage times (one 64-deep K stage of one tile on one CU, measured
    // ≈ 2.0 µs for bf16 256-row tiles, ≈ 1.3 µs for 128-row ones, 1.3× that with weight
    // decoding), of each schedule; the least wins.  Grid with S splits: its rounds of
    // one workgroup per CU, each of nst / S stages and an epilogue of about two; stream-K:
    // one range per CU, 1.15× per stage (the CUs are at different K offsets, so fewer
    // operand reads hit L2), plus the epilogues of its pieces.  Each partial slot costs
    // its write and the consumer's read (M N 4 bytes each way at about 5 TB/s).
    BigGemmPlan p = big_gemm_plan_grid(wf, M, N, K);
    const int G = cu_count();
    const long long T = (long long)p.grid_x * p.grid_y;
    const int nst = K / BK;
    const double ts = (p.bm == 256 || p.bn == 512 ? 2.0 : 1.3) * (wf ? 1.3 : 1.0);
    const double slot = 2.0 * M * (double)N * 4 / 5e12 * 1e6 / ts;
    const double epi = 2.0;
    double best = 1e300;
    for (int S = 1; S <= 16 && (S == 1 || nst / S >= 4); S++) {
        const double rounds = (double)((T * S + G - 1) / G);
        const double c = rounds * ((double)nst / S + epi) + S * slot;
        if (c < best) {
            best = c;
            p.splits = S;
        }
    }
    const long long U = T * nst;
    if (U >= 4LL * G) {
        // (cached: the slot count walks every tile)
        static thread_local struct { int M, N, K, G, slots; } cache[8] = {};
        static thread_local int next = 0;
        int slots = 0;
        for (auto &c : cache)
            if (c.M == M && c.N == N && c.K == K && c.G == G) slots = c.slots;
        if (!slots) {
            slots = sk_slots(T, nst, G);
            cache[next] = {M, N, K, G, slots};
            next = (next + 1) % 8;
        }
        const long long per = (U + G - 1) / G;
        const double c = 1.15 * per + epi * (1 + (per + nst - 1) / nst) + slots * slot;
        if (slots <= 16 && c < best) {
            p.wgs = G;
            p.splits = slots;
        }
    }
    p.part_bytes = (size_t)p.splits * M * N * 4;
    return p;
}

bool big_gemm_ok(int wf, int M, int N, int K) {
    if (M < 1 || N < 16 || N % 16) return false;
    return wf == 0 ? K % BK == 0 && K >= BK : K % 256 == 0 && K >= 256;
}

hipError_t launch_big_gemm(const BigGemmArgs &a, const BigGemmPlan &p, hipStream_t st) {
    if (!big_gemm_ok(a.wfmt, a.M, a.N, a.K) || a.wfmt < 0 || a.wfmt > 2) return hipErrorInvalidValue;
    if (p.wgs && (p.wgs % 8 || a.ldc % 4)) return hipErrorInvalidValue;
    // operand rows are fetched as 16-byte pieces straight into LDS
    if (reinterpret_cast<uintptr_t>(a.A) % 16 || a.lda % 8) return hipErrorInvalidValue;
    BigSched sc = {p.wgs, p.grid_x, p.grid_y, a.K / BK, p.splits};
    const dim3 grid(p.wgs ? p.wgs : p.grid_x * p.grid_y * p.splits);
    const int bi = p.bm == 256;
    const void *fn;
    size_t lb;
    if ((a.wfmt != 0 || bi) && p.bn != BN) return hipErrorInvalidValue;
    if (a.wfmt == 0) {
        fn = bi ? (const void *)k_gemm_big_dma<256, 256>
                : (p.bn == 512 ? (const void *)k_gemm_big_dma<128, 512> : (const void *)k_gemm_big_dma<128, 256>);
        lb = dma_lds_bytes(p.bm, p.bn);
    } else if (a.wfmt == 1) {
        fn = bi ? (const void *)k_gemm_big_q<1, 256> : (const void *)k_gemm_big_q<1, 128>;
        lb = q_lds_bytes(p.bm);
    } else {
        fn = bi ? (const void *)k_gemm_big_q<2, 256> : (const void *)k_gemm_big_q<2, 128>;
        lb = q_lds_bytes(p.bm);
    }
    // (the LDS limit is raised once per device and kernel)
    static bool attr_set[64][3][2][2] = {};
    const int wide = p.bn == 512;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (!attr_set[dev][a.wfmt][bi][wide]) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lb);
        if (e != hipSuccess) return e;
        attr_set[dev][a.wfmt][bi][wide] = true;
    }
    void *args[] = {const_cast<BigGemmArgs *>(&a), &sc};
    const hipError_t e = hipLaunchKernel(fn, grid, dim3(NTH), args, lb, st);
    return e != hipSuccess ? e : hipGetLastError();
}
