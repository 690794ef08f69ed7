// Dense-contraction GEMM for many activation rows (the batched draft steps), gfx950:
// C[slot][M][N] (fp32) = A[M][K] (bf16) . W[N][K]^T over the slot's share of K, with W
// in bf16, Q8_0, Q4_K or FP8 (tiled layouts of q8_0.hip / q4k_tiled.hip / fp8.hip).  The consumers sum
// the slots (reduce kernels), as for every other GEMM of the step; (hi, lo) activation
// row pairs are added by the GEMM itself where they fill whole half tiles (fold_pairs).
//
// At 100+ rows the drafter's products are MFMA-bound (2 M flops per weight against
// 0.56-2 bytes), so the weights are decoded once per 256 x 256 output tile into bf16
// MFMA operands and the tile runs on v_mfma_f32_32x32x16_bf16 (on this chip the 32x32
// form runs at twice the rate of the 16x16x32 one: 2.4 against 1.3 PFLOP/s measured
// with independent chains).  A quantised weight w (Q4_K: d sc q - dmin m, Q8_0: d q,
// formed in fp32) enters as two bf16 terms, hi = bf16(w) and lo = bf16(w - hi), each
// multiplied by the same activation operand: hi + lo carries w to 2^-18 of itself,
// below the fp32 accumulation's own rounding over K of a few thousand.  Where the
// activations are themselves (hi, lo) pairs (rows >= lo_row, the MLP inputs), the lo
// rows skip the weights' lo term: that product is within 2^-18 of the pair's sum.  FP8
// (E4M3) codes are exact in bf16: they enter as a single term, and their row scale
// multiplies the output column in the epilogue.
//
// Workgroup: 8 waves (2 along M x 4 along N), each a 128 x 64 block (BM = 256; 64 x 64
// for BM = 128) of 32 x 32 MFMA tiles.  The operands sit in LDS in MFMA lane order,
// 16-byte entries placed so that operand reads are free of bank conflicts.  A (and bf16
// W) travel global -> LDS by direct loads (global_load_lds_dwordx4: no registers, no
// LDS store instructions) through a ring of K stages, the next ones in flight while one
// is multiplied (bf16: 64-deep stages, a ring of 2, for the 256 x 256 and 128 x 512
// tiles; 32-deep, a ring of 4, for 128 x 256); Q8_0 / FP8 weights are loaded into
// registers two stages ahead, Q4_K weights by direct loads into a ring of raw LDS slots
// four stages ahead, and either is decoded into a double-buffered LDS tile of (hi, lo)
// operands.
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

#include <type_traits>

namespace {

constexpr int BN = 256, BK = 64, NTH = 512;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// s_waitcnt immediate that waits until at most n (< 64) vector loads are outstanding and
// leaves the other counters alone: vmcnt is split over bits 3:0 and 15:14
constexpr int vm_wait(int n) { return 0xF70 | (n & 15) | ((n >> 4) << 14); }

// schedule of the workgroups: wgs == 0: one workgroup per (N tile, M tile, K split)
// item (a 1-D grid, items dealt to XCDs in contiguous runs); else stream-K
// over wgs workgroups (a multiple of 8), tx x ty tiles of nst stages, `slots` slots;
// gs > 0: grouped stream-K (below) over groups of gs weight slabs
struct BigSched {
    int wgs, tx, ty, nst, slots, gs;
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

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// bf16 (round to nearest even, v_cvt_pk_bf16_f32) of two floats, a in the low half
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// the 8 weights w_b = q_b s - t of a fragment entry as bf16 (hi, lo) operands
__device__ __forceinline__ void split8(const float (&q)[8], float s, float t, u32x4_t &hi,
                                       u32x4_t &lo) {
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const float w0 = q[2 * p] * s - t, w1 = q[2 * p + 1] * s - t;
        const uint32_t h = cvt_bf16x2(w0, w1);
        hi[p] = h;
        lo[p] = cvt_bf16x2(w0 - __uint_as_float(h << 16), w1 - __uint_as_float(h & 0xFFFF0000u));
    }
}

// FP8 row scale of output column n (clamped into range): the float after the codes of
// the column's weight segment
__device__ __forceinline__ float fp8_col_scale(const BigGemmArgs &a, int n) {
    n = min(n, a.N - 1);
    int nb;
    const unsigned char *ws = seg_of(a, n, nb);
    const int si = (a.nseg > 1 && n >= a.seg_end[0]) + (a.nseg > 2 && n >= a.seg_end[1]);
    const int rows = (si == 0 ? a.seg_end[0] : (si == 1 ? a.seg_end[1] : a.seg_end[2])) - nb;
    return reinterpret_cast<const float *>(ws + (size_t)rows * a.K)[n - nb];
}

// columns per run of the softmax statistics the many-row head leaves for the selector,
// for waves of wn columns: one wave's columns, or two waves' (at most 2048 runs per row
// of a 248320-row vocabulary)
constexpr int big_head_run_cols(int wn) { return wn > 128 ? wn : 128; }

// Epilogue: lane l of tile (i, j), register v holds row 8 (v / 4) + 4 (l / 32) + v % 4,
// column l % 32.  With the row scale, it is computed once per row of the tile into LDS
// (rinv, free once every wave has left the K loop).  CS: FP8 weights, whose row scale
// multiplies each output column.
// (hi, lo) pair fold.  When the activation rows are (hi, lo) pairs, row r and its lo row
// lo_row + r (the MLP products of the batched steps), and the hi rows come in whole
// half tiles, each M tile takes BM / 2 hi rows and their lo rows (act_row), and the
// waves of the second M half pass their accumulators through LDS, one 32-row block at a
// time (32 KB), to the wave of the first half that holds the same columns, which adds
// them: hi + lo, the sum the reduction would otherwise form from a partial twice the
// size (the same two fp32 terms, so the same result).  The lane layouts of the two
// waves match row for row; the tile's output rows are m0 / 2 .. m0 / 2 + BM / 2 - 1.
__device__ __forceinline__ bool fold_pairs_here(const BigGemmArgs &a, int BM) {
    return a.lo_row > 0 && 2 * a.lo_row == a.M && a.lo_row % (BM / 2) == 0;
}
// activation row of tile row L (L = m0 + local row): with folding, M tile t holds hi rows
// [t BM/2, (t + 1) BM/2) in its first half and their lo rows in its second half (the
// activations are stored [hi rows; lo rows]); else row L itself
__device__ __forceinline__ int act_row(const BigGemmArgs &a, int L, int BM, bool fold) {
    if (!fold) return L;
    const int t = L / BM, r = L - t * BM, h = BM / 2;
    return r < h ? t * h + r : a.lo_row + t * h + (r - h);
}
template <int FM>
__device__ __forceinline__ void fold_pairs(f32x16_t (&acc)[FM][2], float *xf, int wm, int wn, int lane) {
#pragma unroll
    for (int i = 0; i < FM; i++) {
        __syncthreads();                    // (first block: every wave is done with its operands)
        if (wm) {
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int v = 0; v < 16; v++) xf[((wn * 2 + j) * 16 + v) * 64 + lane] = acc[i][j][v];
        }
        __syncthreads();
        if (!wm) {
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int v = 0; v < 16; v++) acc[i][j][v] += xf[((wn * 2 + j) * 16 + v) * 64 + lane];
        }
    }
}

// Folded (fold_pairs): the tile's second M half held the lo rows of the first half's
// (hi, lo) activation pairs and has been added into it; only the first half's waves
// store, as rows m0 / 2 + r of a partial of M / 2 rows.
template <int BM, int FM, int FN = 2, bool CS = false>
__device__ __forceinline__ void store_tile(const BigGemmArgs &a, const f32x16_t (&acc)[FM][FN],
                                           float *rinv, int m0, int n0, int wm, int wn, int tid,
                                           int slot, bool scale, bool folded = false) {
    constexpr int WM = BM / 2, WN = 32 * FN;
    const int lane = tid & 63, hl = lane >> 5, c = lane & 31;
    if (folded && wm) return;
    const int m_rows = folded ? a.M / 2 : a.M;
    if (folded) m0 /= 2;
    float *C = a.C + (size_t)slot * m_rows * a.ldc;
    float cs[FN];
#pragma unroll
    for (int j = 0; j < FN; j++) cs[j] = CS ? fp8_col_scale(a, n0 + wn * WN + 32 * j + c) : 1.f;
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
            if (m0 + r >= m_rows) continue;
            const float ri = scale ? rinv[r] : 1.f;
#pragma unroll
            for (int j = 0; j < FN; j++) {
                const int n = n0 + wn * WN + 32 * j + c;
                if (n < a.N) C[(size_t)(m0 + r) * a.ldc + n] = CS ? acc[i][j][v] * cs[j] * ri
                                                                  : acc[i][j][v] * ri;
            }
        }
    }
    if (!CS && scale && a.rstat) {
        // softmax statistics per row of the tile's column runs of RC = max(WN, 128) columns
        // (one or two waves' columns; the selector reads back only the runs that can hold
        // a candidate, so finer runs cost it fewer logits).  Each wave stages a 32-row
        // block of its values in LDS, lane (row, half) = (l % 32, l / 32) reduces half a
        // row's WN columns serially (one shuffle joins the halves); the waves of a run
        // merge through LDS; one thread per (row, run) writes the pair.
        float *ws = rinv + BM;                     // [BM][4 waves][2]
        // (row stride WN + 1: the 32 lanes of a half-wave read 32 banks)
        constexpr int TS = WN + 1;
        float *tb = rinv + 9 * BM + (wm * 4 + wn) * 32 * TS;
        const int sr = lane & 31, sh = lane >> 5;
#pragma unroll
        for (int i = 0; i < FM; i++) {
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int rr = 8 * (v >> 2) + 4 * hl + (v & 3);
                const float ri = rinv[wm * WM + 32 * i + rr];
#pragma unroll
                for (int j = 0; j < FN; j++) {
                    const int n = n0 + wn * WN + 32 * j + c;
                    tb[rr * TS + 32 * j + c] = n < a.N ? acc[i][j][v] * ri : -INFINITY;
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);    // this wave's LDS stores done
            __builtin_amdgcn_wave_barrier();
            const float *src = tb + sr * TS + sh * (WN / 2);
            float mx = -INFINITY;
#pragma unroll
            for (int k = 0; k < WN / 2; k++) mx = fmaxf(mx, src[k]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
            float se = 0.f;
#pragma unroll
            for (int k = 0; k < WN / 2; k++) se += src[k] == -INFINITY ? 0.f : __expf(src[k] - mx);
            se += __shfl_xor(se, 32, WAVE);
            if (sh == 0) {
                const int r = wm * WM + 32 * i + sr;
                ws[(r * 4 + wn) * 2] = mx;
                ws[(r * 4 + wn) * 2 + 1] = se;
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();       // (the next block reuses the staging)
        }
        __syncthreads();
        constexpr int RC = big_head_run_cols(WN), RPW = RC / WN, NRT = 4 / RPW;
        const int nrun = ceil_div(a.N, RC);
        for (int e = tid; e < BM * NRT; e += NTH) {
            const int r = e / NRT, q = e % NRT, run = n0 / RC + q;
            if (m0 + r >= a.M || run >= nrun) continue;   // (runs wholly past N: none)
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < RPW; w++) M = fmaxf(M, ws[(r * 4 + q * RPW + w) * 2]);
            float S = 0.f;
#pragma unroll
            for (int w = 0; w < RPW; w++) {
                const float m = ws[(r * 4 + q * RPW + w) * 2];
                S += m == -INFINITY ? 0.f : ws[(r * 4 + q * RPW + w) * 2 + 1] * expf(m - M);
            }
            *reinterpret_cast<float2 *>(a.rstat + 2 * ((size_t)(m0 + r) * nrun + run)) = make_float2(M, S);
        }
    }
}

// zeroes slots [from, to) of a tile (N and ldc are multiples of 4)
template <int BM, int TBN = BN>
__device__ __forceinline__ void zero_slots(const BigGemmArgs &a, int m0, int n0, int from, int to, int tid,
                                           bool folded = false) {
    const int m_rows = folded ? a.M / 2 : a.M, rows = folded ? BM / 2 : BM;
    if (folded) m0 /= 2;
    for (int z = from; z < to; z++) {
        float *C = a.C + (size_t)z * m_rows * a.ldc;
        for (int e = tid; e < rows * TBN / 4; e += NTH) {
            const int m = m0 + e / (TBN / 4), n = n0 + 4 * (e % (TBN / 4));
            if (m < m_rows && n < a.N)
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
// Grouped stream-K: the units (group of gs weight slabs, stage s) are cut into
// wgs / (ty gs) ranges, and range q is worked by ty gs workgroups on one XCD, one per
// (M tile, slab of the group), which start together at the same K offset: each stage
// of a slab and of an M tile's rows comes from HBM once and serves the group's other
// tiles from L2 (the M-fastest ranges left the tiles sharing a slab or a row block at
// different K offsets: at 64 sequences gate|up fetched 2.56 GB per launch, 7.2x its
// weights).
struct Piece {
    int m0, n0, s0, s1, slot;
    bool scale, last;
};
struct Pieces {
    long long u, u1, U;
    int g, m, j;
    __device__ __forceinline__ Pieces(const BigGemmArgs &a, const BigSched &sc) {
        m = j = 0;
        if (sc.wgs == 0) {
            u = 0;
            u1 = 1;
            U = 1;
            g = 0;
        } else if (sc.gs) {
            // workgroup b on XCD b % 8, index i = b / 8 there: M tile i % ty, slab
            // (i / ty) % gs of its group, range x (wgs / 8 / (ty gs)) + i / (ty gs)
            const int i = blockIdx.x >> 3, tg = sc.ty * sc.gs, R = sc.wgs / tg;
            m = i % sc.ty;
            j = (i / sc.ty) % sc.gs;
            g = (blockIdx.x & 7) * ((sc.wgs >> 3) / tg) + i / tg;
            U = (long long)ceil_div(sc.tx, sc.gs) * sc.nst;
            u = (long long)g * U / R;
            u1 = (long long)(g + 1) * U / R;
        } else {
            g = (blockIdx.x & 7) * (sc.wgs >> 3) + (blockIdx.x >> 3);
            U = (long long)sc.tx * sc.ty * sc.nst;
            u = (long long)g * U / sc.wgs;
            u1 = (long long)(g + 1) * U / sc.wgs;
        }
    }
    template <int BM, int TBN = BN>
    __device__ __forceinline__ bool next(const BigGemmArgs &a, const BigSched &sc, Piece &p) {
        // grouped: a group's slab j may lie past the last slab; the pieces are skipped
        while (sc.gs && u < u1 && (int)(u / sc.nst) * sc.gs + j >= sc.tx)
            u = min(u1, (u / sc.nst + 1) * sc.nst);
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
        const int R = sc.gs ? sc.wgs / (sc.ty * sc.gs) : sc.wgs;      // ranges
        p.slot = g - ((int)(((x + 1) * R + U - 1) / U) - 1);         // (range holding unit x)
        p.m0 = (sc.gs ? m : t % sc.ty) * BM;
        p.n0 = (sc.gs ? t * sc.gs + j : t / sc.ty) * TBN;
        p.scale = sc.slots == 1 && a.rs.ssq;
        p.last = p.s1 == sc.nst;
        u += p.s1 - p.s0;
        return true;
    }
};

// ---- Q8_0 / Q4_K / FP8 weight tasks.  Task e = tid + NTH i (i < 2) of a thread: 16-column
// group cg = e / 64 of the tile, lane ln = e % 64 of the MFMA fragment (column ln % 16,
// k group ln / 16).  wbase: the column group's first tiled unit.
template <int WF>
__device__ __forceinline__ void wq_setup(const BigGemmArgs &a, int n0, int tid,
                                         const unsigned char *(&wbase)[2]) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int e = tid + NTH * i;
        const int n = min(n0 + 16 * (e / 64) + (e & 15), a.N - 1);   // (columns past N: the last)
        int nb;
        const unsigned char *ws = seg_of(a, n, nb);
        wbase[i] = ws + (size_t)((n - nb) >> 4) * (a.K / 256) *
                            (WF == 1 ? Q8_UNIT_BYTES : (WF == 2 ? Q4K_UNIT_BYTES : FP8_UNIT_BYTES));
    }
}

// raw bytes of the 32-deep stage st (K [32 st, 32 st + 32)): Q8_0: 8 bytes of block st
// of the lane's slot (k group ln / 16) and the block's fp16 scale; Q4_K: the 8 bytes of
// chunk c = (st % 8) / 2 of the lane's slot (sub-block st % 8 is their low or high
// nibbles) and the column's 16-byte header; FP8: the 8 codes of k-step st % 8 of the
// lane's slot.  Two loads per task, four per thread (FP8: one and two).
template <int WF>
constexpr int wq_loads() { return WF == 3 ? 2 : 4; }

template <int WF>
__device__ __forceinline__ void wq_load(WRaw &rw, const unsigned char *const (&wbase)[2], int tid, int st) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int ln = (tid + NTH * i) & 63;
        if (WF == 3) {
            const int g = st >> 3, ks = st & 7;
            const unsigned char *unit = wbase[i] + (size_t)g * FP8_UNIT_BYTES;
            const u32x2_t q = *reinterpret_cast<const u32x2_t *>(unit + 1024 * (ks >> 1) + 16 * ln + 8 * (ks & 1));
            rw.v[2 * i] = (u32x4_t){q.x, q.y, 0u, 0u};
        } else if (WF == 1) {
            const int g = st >> 3, blk = st & 7, pr = blk >> 1;
            const unsigned char *unit = wbase[i] + (size_t)g * Q8_UNIT_BYTES;
            const u32x2_t q = *reinterpret_cast<const u32x2_t *>(unit + 256 + 1024 * pr + 16 * ln + 8 * (blk & 1));
            const uint32_t sc = *reinterpret_cast<const uint32_t *>(unit + 16 * (ln & 15) + 4 * pr);
            rw.v[2 * i] = (u32x4_t){q.x, q.y, 0u, 0u};
            rw.v[2 * i + 1] = (u32x4_t){sc, 0u, 0u, 0u};
        } else {
            const int sb = st >> 3, j = st & 7, c = j >> 1;
            const unsigned char *unit = wbase[i] + (size_t)sb * Q4K_UNIT_BYTES;
            const u32x2_t q = *reinterpret_cast<const u32x2_t *>(unit + 256 + 1024 * (c >> 1) + 16 * ln + 8 * (c & 1));
            rw.v[2 * i] = (u32x4_t){q.x, q.y, 0u, 0u};
            rw.v[2 * i + 1] = *reinterpret_cast<const u32x4_t *>(unit + 16 * (ln & 15));
        }
    }
}

// two E4M3 codes (bytes 0, 1 or 2, 3 of v) -> their bf16 values (exact), first in the low half
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_bf16(uint32_t v) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, HI));
}

// decode a stage's raw bytes into the (hi, lo) MFMA operands of the W tile Bb
// ([2 (hi, lo)][2 ks][8][64], slot swz): task (column, k group kg) fills entry kg of its
// column's fragment: ks = kg / 2, lane (column % 32) + 32 (kg % 2).  sub = stage % 8 (the
// Q4_K sub-block, the Q8_0 block of the pair).  FP8: the codes' bf16 values only (no lo
// term).  Columns past N decode the last column's bytes (wq_setup clamps them): their
// products reach only output columns past N, which are never stored.
template <int WF>
__device__ __forceinline__ void wq_store(u32x4_t *Bb, const WRaw &rw, int tid, int sub) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int e = tid + NTH * i, cg = e / 64, ln = e & 63;
        const u32x4_t zero = {0u, 0u, 0u, 0u};
        u32x4_t oh = zero, ol = zero;
        const u32x4_t q = rw.v[2 * i], h = rw.v[2 * i + 1];
        float v[8];
        if constexpr (WF == 3) {
            oh = (u32x4_t){e4m3x2_bf16<false>(q.x), e4m3x2_bf16<true>(q.x),
                           e4m3x2_bf16<false>(q.y), e4m3x2_bf16<true>(q.y)};
        } else if constexpr (WF == 1) {
#pragma unroll
            for (int b = 0; b < 8; b++)
                v[b] = (float)(int8_t)((b < 4 ? q.x : q.y) >> (8 * (b & 3)));
            const uint32_t sc = (sub & 1) ? (h.x >> 16) : (h.x & 0xFFFFu);
            split8(v, half_bits_to_f32(sc), 0.f, oh, ol);
        } else {
            // sub-block j: the low (j even) or high (j odd) nibbles of the chunk
            const int j = sub, shift = 4 * (j & 1);
            const uint32_t mx = (q.x >> shift) & 0x0F0F0F0Fu, my = (q.y >> shift) & 0x0F0F0F0Fu;
#pragma unroll
            for (int b = 0; b < 8; b++) v[b] = (float)(((b < 4 ? mx : my) >> (8 * (b & 3))) & 0xFFu);
            // header: d, dmin, 6-bit scale and min of sub-block j (scale bytes j, j + 4
            // and j % 4 of h.y, h.z, h.w)
            const float d = half_bits_to_f32(h.x & 0xFFFFu);
            const float dmin = half_bits_to_f32(h.x >> 16);
            auto byte = [&](int i2) {
                const uint32_t w = i2 < 4 ? h.y : (i2 < 8 ? h.z : h.w);
                return (w >> (8 * (i2 & 3))) & 0xFFu;
            };
            const uint32_t bj = byte(j), bj4 = byte(j + 4), bjl = byte(j & 3);
            const uint32_t lo4 = (uint32_t)((j - 4) >> 31);       // all ones for j < 4
            const uint32_t s6 = ((bj & 63u) & lo4) | (((bj4 & 15u) | ((bjl >> 6) << 4)) & ~lo4);
            const uint32_t m6 = ((bj4 & 63u) & lo4) | (((bj4 >> 4) | ((bj >> 6) << 4)) & ~lo4);
            split8(v, d * (float)s6, dmin * (float)m6, oh, ol);
        }
        const int kg = ln >> 4, col = 16 * cg + (ln & 15);
        const int li = (col & 31) + 32 * (kg & 1);
        const int at = ((kg >> 1) * 8 + (col >> 5)) * 64 + swz(li, kg);
        Bb[at] = oh;
        if (WF != 3) Bb[1024 + at] = ol;
    }
}

// bf16 weights: both operands through a ring of NS stages of BKD = 32 or 64 K.  A stage
// holds 32-row groups of 32 rows x 2 BKD bytes; a row's bytes are CH = BKD / 8 16-byte
// chunks.  Lane L of a load instruction fills the 16-byte slot L of one 1 KB piece of a
// group, i.e. row RPK h + L / CH (RPK = 64 / CH rows per piece), chunk slot L % CH, and it
// loads the chunk (L % CH) ^ sw(row) of that row, sw(row) = (row / 4) % 4 for 32 K and
// (row / 2) % 8 for 64 K: CH lanes cover a row's bytes of the stage, and the 16 rows read
// together by an MFMA operand load (one chunk each) fall on 16 distinct 16-byte bank
// groups.  64-deep stages read 128 bytes of each row per load (whole lines): in a
// load-only probe over the output head's matrix, 64-byte row pieces streamed at 4.1-4.4
// TB/s and 128-byte ones at 6.9.  Rows and columns past M / N load row M - 1 / column
// N - 1 (in bounds) and are never stored.
template <int BKD>
__device__ __forceinline__ int dma_pos(int row, int chunk) {
    if constexpr (BKD == 32) return 4 * row + (chunk ^ ((row >> 2) & 3));
    else return 8 * row + (chunk ^ ((row >> 1) & 7));
}

// stage depth per tile, and the ring: as many stages as fit 160 KB of LDS, at most 4.
// 64-deep stages (rings of 2) measured faster for the 256 x 256 tiles (the 64-sequence
// step 6.49-6.54 -> 6.21-6.28 ms, gate|up 395 -> 363 us: half the barriers per K and
// whole-line row pieces) and the 128 x 512 output-head tiles (112 rows: 543 -> 510 us);
// 128 x 256 tiles with 64-deep stages (a ring of 3) ran that head in 529 us.
template <int BM, int TBN> constexpr int dma_bkd() { return BM == 256 || TBN == 512 ? 64 : 32; }
constexpr int dma_ring(int BM, int TBN, int bkd) {
    const int n = 163840 / ((BM + TBN) * 2 * bkd);
    return n < 4 ? n : 4;
}
template <int BM, int TBN> constexpr int dma_ns() { return dma_ring(BM, TBN, dma_bkd<BM, TBN>()); }

// one tile piece (BM x TBN) over BKD-deep stages [s0, s1)
template <int BM, int NS, int TBN, int BKD>
__device__ __forceinline__ void dma_piece(const BigGemmArgs &a, u32x4_t *lds, int m0, int n0, int s0,
                                          int s1, int slot, bool scale) {
    constexpr int RG = BM / 32, WM = BM / 2, FM = WM / 32, FN = TBN / 128;
    constexpr int NG = RG + TBN / 32;                 // 32-row groups per stage (A, then W)
    constexpr int CH = BKD / 8, RPK = 64 / CH, LPG = 32 / RPK, GE = 32 * CH;
    constexpr int PW = NG * LPG / 8;                  // load instructions per wave and stage
    static_assert(NG * LPG % 8 == 0, "whole load instructions per wave");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const bool fold = FN == 2 && fold_pairs_here(a, BM);

    // this lane's source pointer for each of the wave's load instructions (k of stage added)
    const uint16_t *src[PW];
#pragma unroll
    for (int j = 0; j < PW; j++) {
        const int h = wave + 8 * j;                   // 1 KB piece: group h / LPG, rows RPK (h % LPG) ..
        const int g = h / LPG, row = RPK * (h % LPG) + lane / CH;
        const int sw = BKD == 32 ? (row >> 2) & 3 : (row >> 1) & 7;
        const int chunk = (lane % CH) ^ sw;
        if (g < RG) {
            const int r = act_row(a, min(m0 + 32 * g + row, a.M - 1), BM, fold);
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
                (void __attribute__((address_space(3))) *)(lds + buf * NG * GE + h * 64), 16, 0, 0);
        }
    };

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

    // read positions of this lane's MFMA operands for the BKD / 16 k steps of a stage
    constexpr int KS = BKD / 16;
    const int rl = lane & 31;
    int rp[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ks++) rp[ks] = dma_pos<BKD>(rl, 2 * ks + (lane >> 5));

    // prologue: stages s0 .. s0 + NS - 2 in flight (past the end: the last stage again,
    // into a buffer no stage reads, so every iteration waits on the same count)
#pragma unroll
    for (int p = 0; p < NS - 1; p++) issue(min(s0 + p, s1 - 1), p);
    for (int s = s0; s < s1; s++) {
        const int buf = (s - s0) % NS;
        // stage s has landed (the NS - 2 later ones may be in flight) in every wave; a
        // bare barrier, since a workgroup fence would wait for every load in flight
        static_assert((NS - 2) * PW < 64, "vmcnt holds 6 bits");
        __builtin_amdgcn_s_waitcnt(vm_wait((NS - 2) * PW));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // the buffer of stage s - 1 is free: stage s + NS - 1 goes there
        issue(min(s + NS - 1, s1 - 1), (s - s0 + NS - 1) % NS);
        const u32x4_t *Ab = lds + buf * NG * GE;
        const u32x4_t *Bb = Ab + RG * GE;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            u32x4_t bf[FN];
#pragma unroll
            for (int j = 0; j < FN; j++) bf[j] = Bb[(wn * FN + j) * GE + rp[ks]];
#pragma unroll
            for (int i = 0; i < FM; i++) {
                const u32x4_t af = Ab[(wm * FM + i) * GE + rp[ks]];
#pragma unroll
                for (int j = 0; j < FN; j++) acc[i][j] = mfma32x32x16(af, bf[j], acc[i][j]);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0xF70);      // no load may land after the piece ends

    if constexpr (FN == 2) {
        if (fold) fold_pairs<FM>(acc, reinterpret_cast<float *>(lds), wm, wn, lane);
    }
    store_tile<BM, FM, FN>(a, acc, reinterpret_cast<float *>(lds), m0, n0, wm, wn, tid, slot,
                           scale && !fold, fold);
}

template <int BM, int TBN>
__global__ __launch_bounds__(NTH) void k_gemm_big_dma(BigGemmArgs a, BigSched sc) {
    extern __shared__ __align__(16) u32x4_t lds[];
    Pieces it(a, sc);
    Piece pc;
    for (bool first = true; it.next<BM, TBN>(a, sc, pc); first = false) {
        if (!first) __syncthreads();                  // the previous piece is done with LDS
        constexpr int BKD = dma_bkd<BM, TBN>(), SPB = BK / BKD;   // stages per 64-deep unit
        dma_piece<BM, dma_ns<BM, TBN>(), TBN, BKD>(a, lds, pc.m0, pc.n0, SPB * pc.s0, SPB * pc.s1,
                                                    pc.slot, pc.scale);
        if (pc.last) zero_slots<BM, TBN>(a, pc.m0, pc.n0, pc.slot + 1, sc.slots, threadIdx.x,
                                         TBN == 256 && fold_pairs_here(a, BM));
    }
}

// Q8_0 / Q4_K / FP8 weights, 32-deep K stages: A global -> LDS by direct loads through a ring
// of QNS stages (the bf16 path's 64-byte row pieces and chunk swizzle), the raw weight
// bytes of a stage loaded into registers two stages ahead (two register sets,
// alternating) and decoded into the double-buffered (hi, lo) W tile: after the current
// stage's MFMAs by the waves of the first M half, before them by those of the second.
// Each k step multiplies the A operand by both terms of the weights.
constexpr int QNS = 3, QBKD = 32;

// one tile piece over 32-deep stages [s0, s1)
template <int WF, int BM>
__device__ __forceinline__ void q_piece(const BigGemmArgs &a, u32x4_t *lds, int m0, int n0, int s0,
                                        int s1, int slot, bool scale) {
    constexpr int RG = BM / 32, WM = BM / 2, FM = WM / 32;
    constexpr int PA = 2 * RG / 8;                    // A load instructions per wave and stage
    constexpr int AST = RG * 128;                     // entries of one A stage
    constexpr int PWQ = wq_loads<WF>();               // weight loads per thread and stage
    u32x4_t *As = lds;                                // [QNS][RG][128]
    u32x4_t *Bs = lds + QNS * AST;                    // [2][2 (hi, lo)][2 ks][8][64]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const bool folded = fold_pairs_here(a, BM);

    const uint16_t *asrc[PA];
#pragma unroll
    for (int j = 0; j < PA; j++) {
        const int h = wave + 8 * j;                   // 1 KB half: group h / 2, rows 16 (h % 2) ..
        const int g = h >> 1, row = 16 * (h & 1) + (lane >> 2);
        const int chunk = (lane & 3) ^ ((row >> 2) & 3);
        asrc[j] = a.A + (size_t)act_row(a, min(m0 + 32 * g + row, a.M - 1), BM, folded) * a.lda + 8 * chunk;
    }
    auto issue_a = [&](int st, int buf) {
#pragma unroll
        for (int j = 0; j < PA; j++)
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1))) *)(asrc[j] + st * QBKD),
                (void __attribute__((address_space(3))) *)(As + buf * AST + (wave + 8 * j) * 64), 16, 0, 0);
    };
    const unsigned char *wbase[2];
    wq_setup<WF>(a, n0, tid, wbase);

    f32x16_t acc[FM][2];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

    const int rl = lane & 31;
    const int rp0 = dma_pos<QBKD>(rl, lane >> 5), rp1 = dma_pos<QBKD>(rl, 2 + (lane >> 5));
    // wait until at most one stage's loads are in flight (the one issued last)
    auto wait_one = [&]() {
        asm volatile("" ::: "memory");
        static_assert(PA + PWQ < 64, "vmcnt holds 6 bits");
        __builtin_amdgcn_s_waitcnt(vm_wait(PA + PWQ));
        asm volatile("" ::: "memory");
    };
    // LO: this wave's rows are all lo terms of activation pairs, and their products with
    // the weights' lo terms (<= 2^-18 of the sum) are skipped.  DF: the wave decodes the
    // next stage before its MFMAs (the waves of the second M half), so that the two waves
    // on a SIMD (w and w + 4) overlap one's MFMAs with the other's decode.
    auto run = [&](auto lo_tag, auto df_tag) {
        constexpr bool TWO = WF != 3 && !decltype(lo_tag)::value;   // both weight terms
        constexpr bool DF = decltype(df_tag)::value;                // decode first
        auto compute = [&](const u32x4_t *Ab, const u32x4_t *Bb) {
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const int c = 2 * ks + (lane >> 5), rp = ks ? rp1 : rp0;
                u32x4_t bh[2], bl[2];
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    bh[j] = Bb[(ks * 8 + wn * 2 + j) * 64 + swz(lane, c)];
                    if constexpr (TWO) bl[j] = Bb[1024 + (ks * 8 + wn * 2 + j) * 64 + swz(lane, c)];
                }
#pragma unroll
                for (int i = 0; i < FM; i++) {
                    const u32x4_t af = Ab[(wm * FM + i) * 128 + rp];
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        acc[i][j] = mfma32x32x16(af, bh[j], acc[i][j]);
                        if constexpr (TWO) acc[i][j] = mfma32x32x16(af, bl[j], acc[i][j]);
                    }
                }
            }
        };
        // stage st: A(st) and the decoded W(st) are in LDS once every wave passes the
        // barrier; rn1 holds the raw weights of stage st + 1 (loaded a stage ago), rn2
        // receives stage st + 2; the decode of stage st + 1 goes to the other W buffer.
        // Stages past the end load the last stage again into buffers no stage reads, so
        // the wait counts stay fixed.
        auto body = [&](int st, WRaw &rn1, WRaw &rn2) {
            const int i = st - s0;
            __builtin_amdgcn_s_waitcnt(0xC07F);           // this wave's LDS stores done
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            const int s2 = min(st + 2, s1 - 1);
            issue_a(s2, (i + 2) % QNS);
            wq_load<WF>(rn2, wbase, tid, s2);
            asm volatile("" ::: "memory");                // (issued before the MFMAs)
            const u32x4_t *Ab = As + (i % QNS) * AST, *Bb = Bs + (i & 1) * 2048;
            u32x4_t *Bn = Bs + ((i + 1) & 1) * 2048;
            const int sub = min(st + 1, s1 - 1) & 7;
            if constexpr (!DF) {
                compute(Ab, Bb);
                wait_one();                               // rn1 has landed
                wq_store<WF>(Bn, rn1, tid, sub);
            } else {
                wait_one();
                wq_store<WF>(Bn, rn1, tid, sub);
                compute(Ab, Bb);
            }
        };
        WRaw ra, rb;
        issue_a(s0, 0);
        wq_load<WF>(ra, wbase, tid, s0);
        issue_a(min(s0 + 1, s1 - 1), 1);
        wq_load<WF>(rb, wbase, tid, min(s0 + 1, s1 - 1));
        wait_one();
        wq_store<WF>(Bs, ra, tid, s0 & 7);
        int st = s0;
        for (; st + 1 < s1; st += 2) {
            body(st, rb, ra);
            body(st + 1, ra, rb);
        }
        if (st < s1) body(st, rb, ra);
    };
    // (each case is its own straight-line stage loop: a branch inside the loop body
    // made the register allocation spill)
    using T = std::integral_constant<bool, true>;
    using F = std::integral_constant<bool, false>;
    // (folded: every tile's second M half holds lo rows)
    const bool lo = a.lo_row > 0 && (folded ? wm == 1 : m0 + wm * WM >= a.lo_row);
    if (lo) {
        if (wm) run(T(), T());
        else run(T(), F());
    } else {
        if (wm) run(F(), T());
        else run(F(), F());
    }
    __builtin_amdgcn_s_waitcnt(0xF70);      // no load may land after the piece ends

    if (folded) fold_pairs<FM>(acc, reinterpret_cast<float *>(lds), wm, wn, lane);
    store_tile<BM, FM, 2, WF == 3>(a, acc, reinterpret_cast<float *>(lds), m0, n0, wm, wn, tid, slot,
                                   scale && !folded, folded);
}

// Q4_K weights with their raw bytes staged in LDS instead of registers, so that they can
// be requested further ahead.  A raw "half" H covers the 4 sub-blocks 4 (H % 2) .. + 3 of
// super-block H / 2 (128 values of K): per 16-column group, the 1 KB of quant slots of
// that half of the tiled unit and the unit's 256-byte header area.  Wave w requests the
// halves of column groups w and w + 8, which are exactly the groups its lanes decode,
// so a wave only ever reads raw bytes it requested itself.  Halves go into a ring of 2
// slots; half H + 2 is requested after the barrier of stage 4 H + 3, once the last
// decode from half H (stage 4 H + 3, decoded during stage 4 H + 2) is done, and is first
// decoded during stage 4 H + 7: four stages of lead, where the register sets of q_piece
// gave one (at 16 sequences the stage time sat at the HBM latency, ~4700 cycles for
// ~1500 of matrix-core work).  Every other step is q_piece's, and the decode is
// wq_store<2> on the same bytes, so the results are bit-identical to it.
constexpr int RAW_SLOT = 16 * 64 + 16 * 16;          // u32x4 entries of one raw half slot

template <int BM>
__device__ __forceinline__ void q4k_piece(const BigGemmArgs &a, u32x4_t *lds, int m0, int n0, int s0,
                                          int s1, int slot, bool scale) {
    constexpr int WF = 2;
    constexpr int RG = BM / 32, WM = BM / 2, FM = WM / 32;
    constexpr int PA = 2 * RG / 8;                    // A load instructions per wave and stage
    constexpr int AST = RG * 128;                     // entries of one A stage
    constexpr int PR = 4;                             // raw load instructions per wave and half
    u32x4_t *As = lds;                                // [QNS][RG][128]
    u32x4_t *Bs = lds + QNS * AST;                    // [2][2 (hi, lo)][2 ks][8][64]
    u32x4_t *Rs = Bs + 2 * 2048;                      // [2 slots][16 groups x 64 quant slots,
                                                      //           16 groups x 16 headers]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const bool folded = fold_pairs_here(a, BM);

    const uint16_t *asrc[PA];
#pragma unroll
    for (int j = 0; j < PA; j++) {
        const int h = wave + 8 * j;
        const int g = h >> 1, row = 16 * (h & 1) + (lane >> 2);
        const int chunk = (lane & 3) ^ ((row >> 2) & 3);
        asrc[j] = a.A + (size_t)act_row(a, min(m0 + 32 * g + row, a.M - 1), BM, folded) * a.lda + 8 * chunk;
    }
    auto issue_a = [&](int st, int buf) {
#pragma unroll
        for (int j = 0; j < PA; j++)
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1))) *)(asrc[j] + st * QBKD),
                (void __attribute__((address_space(3))) *)(As + buf * AST + (wave + 8 * j) * 64), 16, 0, 0);
    };
    // first tiled unit of column groups wave and wave + 8 (groups past N: the last one,
    // in bounds; their columns are never stored)
    const unsigned char *wcg[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int n = min(n0 + 16 * (wave + 8 * i), a.N - 1);
        int nb;
        const unsigned char *ws = seg_of(a, n, nb);
        wcg[i] = ws + (size_t)((n - nb) >> 4) * (a.K / 256) * Q4K_UNIT_BYTES;
    }
    const int h_last = (s1 - 1) >> 2;
    // half H (past the piece's last: that one again, into a slot no later decode reads
    // before it is rewritten) into slot H % 2: quant slots by 16-byte lanes, headers by
    // 4-byte lanes (64 dwords = the unit's 16 headers)
    auto issue_raw = [&](int H) {
        const int Hc = min(H, h_last);
        u32x4_t *R = Rs + (H & 1) * RAW_SLOT;
        const size_t off = (size_t)(Hc >> 1) * Q4K_UNIT_BYTES;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int cg = wave + 8 * i;
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1))) *)(wcg[i] + off + 256 + 1024 * (Hc & 1) + 16 * lane),
                (void __attribute__((address_space(3))) *)(R + cg * 64), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int cg = wave + 8 * i;
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1))) *)(wcg[i] + off + 4 * lane),
                (void __attribute__((address_space(3))) *)(R + 16 * 64 + cg * 16), 4, 0, 0);
        }
    };
    // the raw bytes of stage st for this thread's two tasks (column group wave + 8 i,
    // fragment lane `lane`), from half st / 4, as wq_load<2> would have loaded them
    auto raw_of = [&](int st) -> WRaw {
        const u32x4_t *R = Rs + ((st >> 2) & 1) * RAW_SLOT;
        const int c = (st & 7) >> 1;
        WRaw rw;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int cg = wave + 8 * i;
            const u32x2_t q = reinterpret_cast<const u32x2_t *>(R + cg * 64 + lane)[c & 1];
            rw.v[2 * i] = (u32x4_t){q.x, q.y, 0u, 0u};
            rw.v[2 * i + 1] = R[16 * 64 + cg * 16 + (lane & 15)];
        }
        return rw;
    };

    f32x16_t acc[FM][2];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

    const int rl = lane & 31;
    const int rp0 = dma_pos<QBKD>(rl, lane >> 5), rp1 = dma_pos<QBKD>(rl, 2 + (lane >> 5));
    auto wait_vm = [&](auto n_tag) {
        constexpr int n = decltype(n_tag)::value;
        static_assert(n < 64, "vmcnt holds 6 bits");
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(vm_wait(n));
        asm volatile("" ::: "memory");
    };
    using IA = std::integral_constant<int, PA>;
    using IAR = std::integral_constant<int, PA + PR>;

    // Loads in issue order: stage st issues A(st + 2), then, when st % 4 == 3, half
    // st / 4 + 2.  The wait at the end of stage st lets through what was issued after
    // A(st + 1) (issued during stage st - 1): A(st + 2), and the halves issued during
    // stages st - 1 and st; so A(st + 1) and every half issued before it, including the
    // one decoded during stage st + 1 (half (st + 2) / 4, issued by stage st - 3), have
    // landed before the barrier of stage st + 1.
    auto run = [&](auto lo_tag, auto df_tag) {
        constexpr bool TWO = !decltype(lo_tag)::value;
        constexpr bool DF = decltype(df_tag)::value;
        auto compute = [&](const u32x4_t *Ab, const u32x4_t *Bb) {
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const int c = 2 * ks + (lane >> 5), rp = ks ? rp1 : rp0;
                u32x4_t bh[2], bl[2];
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    bh[j] = Bb[(ks * 8 + wn * 2 + j) * 64 + swz(lane, c)];
                    if constexpr (TWO) bl[j] = Bb[1024 + (ks * 8 + wn * 2 + j) * 64 + swz(lane, c)];
                }
#pragma unroll
                for (int i = 0; i < FM; i++) {
                    const u32x4_t af = Ab[(wm * FM + i) * 128 + rp];
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        acc[i][j] = mfma32x32x16(af, bh[j], acc[i][j]);
                        if constexpr (TWO) acc[i][j] = mfma32x32x16(af, bl[j], acc[i][j]);
                    }
                }
            }
        };
        auto decode = [&](u32x4_t *Bn, int st) {
            const WRaw rw = raw_of(st);
            wq_store<WF>(Bn, rw, tid, st & 7);
        };
        // prologue: A(s0), A(s0 + 1) and the halves of stages s0 .. s0 + 4, ordered as
        // the stage loop would have issued them (s0 is even: s0 % 4 is 0 or 2)
        const int H0 = s0 >> 2;
        if ((s0 & 3) == 0) {
            issue_a(s0, 0);
            issue_raw(H0);
            issue_a(min(s0 + 1, s1 - 1), 1);
            issue_raw(H0 + 1);
            wait_vm(IAR());                           // A(s0), half H0
        } else {
            issue_raw(H0);
            issue_raw(H0 + 1);
            issue_a(s0, 0);
            issue_a(min(s0 + 1, s1 - 1), 1);
            wait_vm(IA());                            // halves H0, H0 + 1, A(s0)
        }
        decode(Bs, s0);
        for (int st = s0; st < s1; st++) {
            const int i = st - s0, ph = st & 3;
            __builtin_amdgcn_s_waitcnt(0xC07F);       // this wave's LDS reads and stores done
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            issue_a(min(st + 2, s1 - 1), (i + 2) % QNS);
            if (ph == 3) issue_raw((st >> 2) + 2);
            asm volatile("" ::: "memory");            // (issued before the MFMAs)
            const u32x4_t *Ab = As + (i % QNS) * AST, *Bb = Bs + (i & 1) * 2048;
            u32x4_t *Bn = Bs + ((i + 1) & 1) * 2048;
            const bool more = st + 1 < s1;
            if constexpr (!DF) {
                compute(Ab, Bb);
                if (more) decode(Bn, st + 1);
            } else {
                if (more) decode(Bn, st + 1);
                compute(Ab, Bb);
            }
            if (ph == 0 || ph == 3) wait_vm(IAR());
            else wait_vm(IA());
        }
    };
    using T = std::integral_constant<bool, true>;
    using F = std::integral_constant<bool, false>;
    // (folded: every tile's second M half holds lo rows)
    const bool lo = a.lo_row > 0 && (folded ? wm == 1 : m0 + wm * WM >= a.lo_row);
    if (lo) {
        if (wm) run(T(), T());
        else run(T(), F());
    } else {
        if (wm) run(F(), T());
        else run(F(), F());
    }
    __builtin_amdgcn_s_waitcnt(0xF70);      // no load may land after the piece ends

    if (folded) fold_pairs<FM>(acc, reinterpret_cast<float *>(lds), wm, wn, lane);
    store_tile<BM, FM, 2, false>(a, acc, reinterpret_cast<float *>(lds), m0, n0, wm, wn, tid, slot,
                                 scale && !folded, folded);
}

template <int WF, int BM>
__global__ __launch_bounds__(NTH) void k_gemm_big_q(BigGemmArgs a, BigSched sc) {
    extern __shared__ __align__(16) u32x4_t lds[];
    Pieces it(a, sc);
    Piece pc;
    for (bool first = true; it.next<BM>(a, sc, pc); first = false) {
        if (!first) __syncthreads();                  // the previous piece is done with LDS
        if constexpr (WF == 2)
            q4k_piece<BM>(a, lds, pc.m0, pc.n0, 2 * pc.s0, 2 * pc.s1, pc.slot, pc.scale);
        else
            q_piece<WF, BM>(a, lds, pc.m0, pc.n0, 2 * pc.s0, 2 * pc.s1, pc.slot, pc.scale);
        if (pc.last) zero_slots<BM>(a, pc.m0, pc.n0, pc.slot + 1, sc.slots, threadIdx.x, fold_pairs_here(a, BM));
    }
}

}  // namespace

size_t dma_lds_bytes(int BM, int TBN) {
    // ring: NS stages of (BM + TBN) rows x 2 BKD bytes
    const int bkd = BM == 256 ? dma_bkd<256, 256>() : TBN == 512 ? dma_bkd<128, 512>() : dma_bkd<128, 256>();
    return (size_t)dma_ring(BM, TBN, bkd) * (BM + TBN) * 2 * bkd;
}
size_t q_lds_bytes(int wf, int BM) {
    // A ring + decoded (hi, lo) W double buffer; Q4_K adds its two raw half slots
    return ((size_t)QNS * BM * 4 + 2 * 2048 + (wf == 2 ? 2 * RAW_SLOT : 0)) * 16;
}

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
    p.gs = 0;
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
        // grouped stream-K where the M tiles divide each XCD's workgroups: the largest
        // group of gs slabs (gs dividing G / 8 / ty) whose last group leaves at most 10%
        // of its workgroups idle; ranges over (group, stage) units, else over tiles
        int gs = 0;
        if (p.grid_y > 1 && (G / 8) % p.grid_y == 0)
            for (int c = (G / 8) / p.grid_y; c >= 1 && !gs; c /= 2) {
                const int ng = ceil_div(p.grid_x, c);
                if ((G / 8) % (p.grid_y * c) == 0 && 10 * (ng * c - p.grid_x) <= ng * c) gs = c;
            }
        const long long Ts = gs ? ceil_div(p.grid_x, gs) : T;
        const int Gs = gs ? G / (p.grid_y * gs) : G;
        // (cached on exactly the inputs of sk_slots: the slot count walks every tile)
        static thread_local struct { long long T; int nst, G, slots; } cache[8] = {};
        static thread_local int next = 0;
        int slots = 0;
        for (auto &c : cache)
            if (c.slots && c.T == Ts && c.nst == nst && c.G == Gs) slots = c.slots;
        if (!slots) {
            slots = sk_slots(Ts, nst, Gs);
            cache[next] = {Ts, nst, Gs, slots};
            next = (next + 1) % 8;
        }
        const long long per = (U + G - 1) / G;
        const double c = 1.15 * per + epi * (1 + (per + nst - 1) / nst) + slots * slot;
        if (slots <= 16 && c < best) {
            p.wgs = G;
            p.gs = gs;
            p.splits = slots;
        }
    }
    p.part_bytes = (size_t)p.splits * M * N * 4;
    return p;
}

int big_gemm_head_run_cols(int bn) { return big_head_run_cols(32 * (bn / 128)); }

bool big_gemm_ok(int wf, int M, int N, int K) {
    if (M < 1 || N < 16 || N % 16) return false;
    return wf == 0 ? K % BK == 0 && K >= BK : K % 256 == 0 && K >= 256;
}

hipError_t launch_big_gemm(const BigGemmArgs &a, const BigGemmPlan &p, hipStream_t st) {
    if (!big_gemm_ok(a.wfmt, a.M, a.N, a.K) || a.wfmt < 0 || a.wfmt > 3) return hipErrorInvalidValue;
    if (p.wgs && (p.wgs % 8 || a.ldc % 4)) return hipErrorInvalidValue;
    // operand rows are fetched as 16-byte pieces straight into LDS
    if (reinterpret_cast<uintptr_t>(a.A) % 16 || a.lda % 8) return hipErrorInvalidValue;
    if (p.gs && (p.gs < 1 || (p.wgs / 8) % (p.grid_y * p.gs))) return hipErrorInvalidValue;
    BigSched sc = {p.wgs, p.grid_x, p.grid_y, a.K / BK, p.splits, p.gs};
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
        lb = q_lds_bytes(a.wfmt, p.bm);
    } else if (a.wfmt == 3) {
        fn = bi ? (const void *)k_gemm_big_q<3, 256> : (const void *)k_gemm_big_q<3, 128>;
        lb = q_lds_bytes(a.wfmt, p.bm);
    } else {
        fn = bi ? (const void *)k_gemm_big_q<2, 256> : (const void *)k_gemm_big_q<2, 128>;
        lb = q_lds_bytes(a.wfmt, p.bm);
    }
    // (the LDS limit is raised once per device and kernel)
    static bool attr_set[64][4][2][2] = {};
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
