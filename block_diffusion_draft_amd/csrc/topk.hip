// Log-softmax statistics, top-K candidates of the shared output head and the
// candidate-path selector, gfx950.
//
// FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2": the draft shares the target's output
// head (spec table "Draft" row) and keeps the top 16 candidates per proposal
// position (section "How it is used").  Candidates are ordered by (logit desc,
// token id asc); cand_logp = logit - logsumexp(logits).
//
// Threshold selection, three short passes per row of V fp32 logits:
//  1. wave per 1024-logit chunk: the chunk's max and sum of exp(logit - max) (and the
//     row's candidate count reset);
//  2. wave per chunk: theta = the K-th largest of the 64 lane maxima of the row's chunk
//     maxima (a wave sort; each lane maximum is a distinct logit, so K logits are
//     >= theta and every top-K candidate is >= theta), then every logit >= theta of
//     the chunk is appended to the row's candidate list (an integer atomic hands out
//     slots; the order of the list does not matter);
//     (the row's first wave also forms its logsumexp from the chunk statistics);
//  3. wave per row: the K best candidates by
//     (value desc, id asc): a wave sort when at most 64 reached theta, else K rounds
//     of arg-max.  If more than CAP logits reach theta (many equal logits), the row is
//     selected by an exact scan of all its chunks instead.
// Every choice is an arg-max under a total order, so the result is exact and does
// not depend on thread scheduling.  K <= 64 (the threshold is a lane maximum).
//
// Pass 3 runs inside the selector's workgroup (one per sequence): its waves select the
// sequence's rows, then the candidate-path search runs on them.
//
// With the statistics of the output head's column runs (the streaming head writes, per
// row and per run of 16 tpw columns, the run's max and sum of exp(v - max)), passes 1 and
// 2 are not launched: the selector's wave for a row reads the run statistics (all loads
// in flight), forms the row's logsumexp and theta = the K-th largest of the 64 lane
// maxima of the run maxima (again K distinct logits reach it), and reads back only the
// runs whose maximum reaches theta: their logits >= theta form the candidate list.  Selector (same card,
// spec table "Draft" row: candidate selector, top 16, rank 256; "Weights" row: two
// 248320 x 256 codebooks; "How it is used": one coherent path through the top 16
// candidates per position): the path objective used here is the sum over positions of
// the candidates' log-probabilities plus s <A[u], B[v]> for every pair of adjacent
// chosen candidates u (earlier) and v (later), maximised by Viterbi; ties go to the
// lowest candidate index.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int PER_LANE = 16;
constexpr int CHUNK = 64 * PER_LANE;     // logits per wave in passes 1 and 2
constexpr int CAP = 1024;                // candidate slots per row
constexpr int CPL = CAP / 64;            // candidates per lane in pass 3

__device__ __forceinline__ bool take(float v, int i, float bv, int bi) {
    return i >= 0 && (bi < 0 || cand_better(v, i, bv, bi));
}

__device__ __forceinline__ void wave_best(float &v, int &i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = xor_lane_n(v, o);
        const int oi = (int)xor_lane_n((uint32_t)i, o);
        if (take(ov, oi, v, i)) { v = ov; i = oi; }
    }
}

__device__ __forceinline__ unsigned long long xor_lane_key(unsigned long long k, int j) {
    const uint32_t lo = xor_lane_n((uint32_t)k, j), hi = xor_lane_n((uint32_t)(k >> 32), j);
    return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ float xor_lane_key(float k, int j) { return xor_lane_n(k, j); }

// (value desc, id asc) as one unsigned 64-bit key: larger key = better candidate
__device__ __forceinline__ unsigned long long cand_key(float v, int id) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);    // order-preserving
    return ((unsigned long long)o << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ float key_value(unsigned long long k) {
    const uint32_t o = (uint32_t)(k >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ int key_id(unsigned long long k) {
    return (int)(0xFFFFFFFFu - (uint32_t)k);
}

// bitonic sort of one value per lane across the wave, descending (lane 0 = largest)
template <class Key>
__device__ __forceinline__ Key wave_sort_desc(Key x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const Key o = xor_lane_key(x, j);
            const bool keep_max = ((lane & j) == 0) == ((lane & k) == 0);
            x = keep_max ? (x > o ? x : o) : (x < o ? x : o);
        }
    }
    return x;
}

// 1. chunk max and sum of exp(logit - max)
__global__ __launch_bounds__(256) void k_chunk_stats(const float *logits, int V, int nch, float *pm,
                                                     float *ps, int *count) {
    const int lane = threadIdx.x & 63;
    const int c = blockIdx.x * 4 + (threadIdx.x >> 6), r = blockIdx.y;
    if (c >= nch) return;
    if (c == 0 && lane == 0) count[r] = 0;
    const float *row = logits + (size_t)r * V + (size_t)c * CHUNK;
    const int n = min(CHUNK, V - c * CHUNK);
    float val[PER_LANE];
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < PER_LANE; k++) {
        const int i = lane + 64 * k;
        val[k] = i < n ? row[i] : -INFINITY;
        mx = fmaxf(mx, val[k]);
    }
    mx = wave_max(mx);
    float se = 0.f;
#pragma unroll
    for (int k = 0; k < PER_LANE; k++) se += val[k] == -INFINITY ? 0.f : expf(val[k] - mx);
    se = wave_sum(se);
    if (lane == 0) {
        pm[(size_t)r * nch + c] = mx;
        ps[(size_t)r * nch + c] = se;
    }
}

// theta of row r: the K-th largest of the 64 lane maxima of its chunk maxima; with
// lse non-null (one wave per row) also the row's logsumexp from its chunk statistics
__device__ __forceinline__ float row_theta(const float *pm, const float *ps, int nch, int K, int r,
                                           float *lse) {
    const int lane = threadIdx.x & 63;
    float m[PER_LANE];
    float lm = -INFINITY;
#pragma unroll
    for (int k = 0; k < PER_LANE; k++) {
        const int c = lane + 64 * k;
        m[k] = c < nch ? pm[(size_t)r * nch + c] : -INFINITY;
        lm = fmaxf(lm, m[k]);
    }
    if (lse) {
        float sm[PER_LANE];
#pragma unroll
        for (int k = 0; k < PER_LANE; k++) {
            const int c = lane + 64 * k;
            sm[k] = c < nch ? ps[(size_t)r * nch + c] : 0.f;
        }
        const float mx = wave_max(lm);
        float se = 0.f;
#pragma unroll
        for (int k = 0; k < PER_LANE; k++) se += m[k] == -INFINITY ? 0.f : sm[k] * expf(m[k] - mx);
        se = wave_sum(se);
        if (lane == 0) lse[r] = mx + logf(se);
    }
    const float sorted = wave_sort_desc(lm);
    return __shfl(sorted, K - 1, WAVE);
}

// 2. wave per chunk: the row's theta (and, in the row's first wave, its logsumexp), then
// append the chunk's logits >= theta to the row's candidate list
__global__ __launch_bounds__(256) void k_collect(const float *logits, int V, int nch, int K,
                                                 const float *pm, const float *ps, float *lse,
                                                 int *count, float *cv, int32_t *ci) {
    const int lane = threadIdx.x & 63;
    const int c = blockIdx.x * 4 + (threadIdx.x >> 6), r = blockIdx.y;
    if (c >= nch) return;
    const float *row = logits + (size_t)r * V + (size_t)c * CHUNK;
    const int n = min(CHUNK, V - c * CHUNK);
    float val[PER_LANE];
#pragma unroll
    for (int k = 0; k < PER_LANE; k++) {
        const int i = lane + 64 * k;
        val[k] = i < n ? row[i] : -INFINITY;
    }
    const float th = row_theta(pm, ps, nch, K, r, c == 0 ? lse : nullptr);   // loads overlap
    unsigned long long mask[PER_LANE];
    int total = 0;
#pragma unroll
    for (int k = 0; k < PER_LANE; k++) {
        const int i = lane + 64 * k;
        mask[k] = __ballot(i < n && val[k] >= th);
        total += __popcll(mask[k]);
    }
    if (total == 0) return;
    int base = 0;
    if (lane == 0) base = atomicAdd(count + r, total);
    base = __shfl(base, 0, WAVE);
    const unsigned long long below = (1ull << lane) - 1ull;
    int off = base;
#pragma unroll
    for (int k = 0; k < PER_LANE; k++) {
        if ((mask[k] >> lane) & 1ull) {
            const int slot = off + __popcll(mask[k] & below);
            if (slot < CAP) {
                cv[(size_t)r * CAP + slot] = val[k];
                ci[(size_t)r * CAP + slot] = c * CHUNK + lane + 64 * k;
            }
        }
        off += __popcll(mask[k]);
    }
}

// 3. one wave, row r: exact top-K of the candidates (or of the whole row on overflow)
// into sid[k], slp[k] = logit - L (k < K; LDS of the calling workgroup)
__device__ void select_row(const float *logits, int V, int nch, int K, int r, const int *count,
                           const float *cv, const int32_t *ci, float L, int *sid, float *slp) {
    const int lane = threadIdx.x & 63;
    const int n = count[r];
    if (n <= 64) {
        // one candidate per lane: sort the wave, the first K lanes are the answer
        const unsigned long long key = lane < n ? cand_key(cv[(size_t)r * CAP + lane],
                                                           ci[(size_t)r * CAP + lane])
                                                : 0ull;
        const unsigned long long sk = wave_sort_desc(key);
        if (lane < K) {
            const bool have = lane < n;
            sid[lane] = have ? key_id(sk) : -1;
            slp[lane] = have ? key_value(sk) - L : -INFINITY;
        }
        return;
    }
    if (n <= CAP) {
        float v[CPL];
        int id[CPL];
#pragma unroll
        for (int k = 0; k < CPL; k++) {
            const int s = lane + 64 * k;
            v[k] = s < n ? cv[(size_t)r * CAP + s] : -INFINITY;
            id[k] = s < n ? ci[(size_t)r * CAP + s] : -1;
        }
        for (int round = 0; round < K; round++) {
            float bv = -INFINITY;
            int bi = -1;
#pragma unroll
            for (int k = 0; k < CPL; k++)
                if (take(v[k], id[k], bv, bi)) { bv = v[k]; bi = id[k]; }
            wave_best(bv, bi);
#pragma unroll
            for (int k = 0; k < CPL; k++)
                if (id[k] == bi) id[k] = -1;
            if (lane == 0) {
                sid[round] = bi;
                slp[round] = bi >= 0 ? bv - L : -INFINITY;
            }
        }
        return;
    }
    // overflow: running top-K over every chunk of the row (lanes < K hold the list)
    float lv = -INFINITY;
    int li = -1;
    const float *row = logits + (size_t)r * V;
    for (int c = 0; c < nch; c++) {
        float v[PER_LANE];
        int id[PER_LANE];
#pragma unroll
        for (int k = 0; k < PER_LANE; k++) {
            const int i = c * CHUNK + lane + 64 * k;
            v[k] = i < V ? row[i] : -INFINITY;
            id[k] = i < V ? i : -1;
        }
        float nv = -INFINITY;
        int ni = -1;
        for (int round = 0; round < K; round++) {
            float bv = lv;
            int bi = li;
#pragma unroll
            for (int k = 0; k < PER_LANE; k++)
                if (take(v[k], id[k], bv, bi)) { bv = v[k]; bi = id[k]; }
            wave_best(bv, bi);
            if (li == bi) li = -1;
#pragma unroll
            for (int k = 0; k < PER_LANE; k++)
                if (id[k] == bi) id[k] = -1;
            if (lane == round) { nv = bv; ni = bi; }
        }
        lv = nv;
        li = ni;
    }
    if (lane < K) {
        sid[lane] = li;
        slp[lane] = li >= 0 ? lv - L : -INFINITY;
    }
}


// top-K of n candidates (v, id) held in LDS (n <= RCAP), into sid / slp (logit - L)
constexpr int RCAP = 512;                // candidate logits per row (LDS, run selection)
constexpr int RUNCAP = 256;              // candidate runs per row
constexpr int RPL = 32;                  // run statistics per lane (runs per row <= 2048)

__device__ void select_lds_list(int n, const float *cvl, const int *cil, int K, float L,
                                int *sid, float *slp) {
    const int lane = threadIdx.x & 63;
    if (n <= 64) {
        const unsigned long long key = lane < n ? cand_key(cvl[lane], cil[lane]) : 0ull;
        const unsigned long long sk = wave_sort_desc(key);
        if (lane < K) {
            const bool have = lane < n;
            sid[lane] = have ? key_id(sk) : -1;
            slp[lane] = have ? key_value(sk) - L : -INFINITY;
        }
        return;
    }
    constexpr int PL = RCAP / 64;
    float v[PL];
    int id[PL];
#pragma unroll
    for (int k = 0; k < PL; k++) {
        const int s = lane + 64 * k;
        v[k] = s < n ? cvl[s] : -INFINITY;
        id[k] = s < n ? cil[s] : -1;
    }
    for (int round = 0; round < K; round++) {
        float bv = -INFINITY;
        int bi = -1;
#pragma unroll
        for (int k = 0; k < PL; k++)
            if (take(v[k], id[k], bv, bi)) { bv = v[k]; bi = id[k]; }
        wave_best(bv, bi);
#pragma unroll
        for (int k = 0; k < PL; k++)
            if (id[k] == bi) id[k] = -1;
        if (lane == 0) {
            sid[round] = bi;
            slp[round] = bi >= 0 ? bv - L : -INFINITY;
        }
    }
}

// exact running top-K over every logit of row r (lanes < K hold the list)
__device__ void select_full_scan(const float *logits, int V, int nch, int K, int r, float L,
                                 int *sid, float *slp) {
    const int lane = threadIdx.x & 63;
    float lv = -INFINITY;
    int li = -1;
    const float *row = logits + (size_t)r * V;
    for (int c = 0; c < nch; c++) {
        float v[PER_LANE];
        int id[PER_LANE];
#pragma unroll
        for (int k = 0; k < PER_LANE; k++) {
            const int i = c * CHUNK + lane + 64 * k;
            v[k] = i < V ? row[i] : -INFINITY;
            id[k] = i < V ? i : -1;
        }
        float nv = -INFINITY;
        int ni = -1;
        for (int round = 0; round < K; round++) {
            float bv = lv;
            int bi = li;
#pragma unroll
            for (int k = 0; k < PER_LANE; k++)
                if (take(v[k], id[k], bv, bi)) { bv = v[k]; bi = id[k]; }
            wave_best(bv, bi);
            if (li == bi) li = -1;
#pragma unroll
            for (int k = 0; k < PER_LANE; k++)
                if (id[k] == bi) id[k] = -1;
            if (lane == round) { nv = bv; ni = bi; }
        }
        lv = nv;
        li = ni;
    }
    if (lane < K) {
        sid[lane] = li;
        slp[lane] = li >= 0 ? lv - L : -INFINITY;
    }
}

// one wave, row r: top-K from the head's run statistics (nrun <= 64 RPL runs of at most
// rc = 2^lrc <= 512 columns: run w is columns [w rc, (w + 1) rc) when nt is 0, else the
// 16-column tiles [w nt / nrun, (w + 1) nt / nrun)); cvl, cil, crun, cwid, cmax: this
// wave's LDS scratch.  theta1 = the K-th
// largest of the 64 lane maxima of the run maxima; among the runs reaching it (at least
// K), theta2 = the K-th largest run maximum, which is the K-th largest of all run maxima:
// the K runs above it each hold a logit >= theta2, so every top-K logit is >= theta2 and
// lies in a run whose maximum reaches theta2.  Those runs' logits >= theta2 are the
// candidates (with more than 64 runs at theta1, theta1 is used instead).
__device__ void select_row_runs(const float *logits, int V, int nrun, int lrc, int nt, int K,
                                int r, const float *rstat, float *cvl, int *cil, int *crun,
                                int *cwid, float *cmax, int *sid, float *slp) {
    const int lane = threadIdx.x & 63;
    const int rc = 1 << lrc;
    const float2 *st = reinterpret_cast<const float2 *>(rstat) + (size_t)r * nrun;
    float rm[RPL], rsm[RPL];
#pragma unroll
    for (int u = 0; u < RPL; u++) {                 // every load in flight (clamped: in bounds)
        const float2 v = st[min(lane + 64 * u, nrun - 1)];
        const bool ok = lane + 64 * u < nrun;
        rm[u] = ok ? v.x : -INFINITY;
        rsm[u] = ok ? v.y : 0.f;
    }
    float lm = -INFINITY;
#pragma unroll
    for (int u = 0; u < RPL; u++) lm = fmaxf(lm, rm[u]);
    const float M = wave_max(lm);
    float se = 0.f;
#pragma unroll
    for (int u = 0; u < RPL; u++) se += rm[u] == -INFINITY ? 0.f : rsm[u] * expf(rm[u] - M);
    const float L = M + logf(wave_sum(se));
    const float th1 = __shfl(wave_sort_desc(lm), K - 1, WAVE);
    // runs reaching theta1, with their maxima
    const unsigned long long below = (1ull << lane) - 1ull;
    int nc = 0;
#pragma unroll
    for (int u = 0; u < RPL; u++) {
        const bool c = rm[u] >= th1;
        const unsigned long long mk = __ballot(c);
        const int slot = nc + __popcll(mk & below);
        if (c && slot < RUNCAP) {
            crun[slot] = lane + 64 * u;
            cmax[slot] = rm[u];
        }
        nc += __popcll(mk);
    }
    __builtin_amdgcn_wave_barrier();
    float th = th1;
    if (nc <= 64) {
        // theta2: the K-th largest maximum of those runs; keep the runs reaching it
        const float mv = lane < nc ? cmax[lane] : -INFINITY;
        const int rv = lane < nc ? crun[lane] : 0;
        th = __shfl(wave_sort_desc(mv), K - 1, WAVE);
        const bool c = lane < nc && mv >= th;
        const unsigned long long mk = __ballot(c);
        __builtin_amdgcn_wave_barrier();
        if (c) crun[__popcll(mk & below)] = rv;
        nc = __popcll(mk);
        __builtin_amdgcn_wave_barrier();
    }
    int n = 0;
    if (nc <= RUNCAP) {
        // the runs' first columns and widths (32-bit products: nrun nt < 2^27)
        for (int q = lane; q < nc; q += 64) {
            const int w = crun[q];
            int c0 = w << lrc, cw = rc;
            if (nt) {
                const int a0 = (int)((unsigned)(w * nt) / (unsigned)nrun);
                const int a1 = (int)((unsigned)((w + 1) * nt) / (unsigned)nrun);
                c0 = 16 * a0;
                cw = 16 * (a1 - a0);
            }
            crun[q] = c0;
            cwid[q] = cw;
        }
        __builtin_amdgcn_wave_barrier();
        // their logits >= theta (32 loads per lane in flight per batch)
        const int ncols = nc << lrc;
        for (int e0 = 0; e0 < ncols && n <= RCAP; e0 += 64 * 32) {
            float v[32];
            int id[32];
#pragma unroll
            for (int u = 0; u < 32; u++) {
                const int e = e0 + 64 * u + lane;
                const int q = e < ncols ? e >> lrc : 0, off = e & (rc - 1);
                const int col = crun[q] + off;
                id[u] = e < ncols && off < cwid[q] && col < V ? col : -1;
                v[u] = logits[(size_t)r * V + (id[u] >= 0 ? col : 0)];
            }
#pragma unroll
            for (int u = 0; u < 32; u++) {
                const bool t = id[u] >= 0 && v[u] >= th;
                const unsigned long long mk = __ballot(t);
                const int slot = n + __popcll(mk & below);
                if (t && slot < RCAP) {
                    cvl[slot] = v[u];
                    cil[slot] = id[u];
                }
                n += __popcll(mk);
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
    if (nc > RUNCAP || n > RCAP)                   // (many equal logits): exact scan
        select_full_scan(logits, V, ceil_div(V, CHUNK), K, r, L, sid, slp);
    else
        select_lds_list(n, cvl, cil, K, L, sid, slp);
}

constexpr int MAXK = 16;
constexpr int MAXP = 16;
constexpr int PATH_WAVES = 8;

// One workgroup (8 waves) per sequence.  Waves select the sequence's P rows (pass 3)
// into LDS and the outputs.  The pair scores of adjacent positions are K x K products of
// gathered codebook rows, T_t = s A[ids_t] B[ids_{t+1}]^T, computed as 16x16xr MFMA
// tiles (exact bf16 products, fp32 accumulation) straight from the gathered rows: lane
// (i, k-group) loads its 16-byte fragments of A[ids_t[i]] and B[ids_{t+1}[i]] for
// every k-step, all loads in flight at once.  Wave w handles positions t = w, w + 8,
// ...; the dynamic programme then runs on K lanes.
__global__ __launch_bounds__(64 * PATH_WAVES) void k_select_path(
    const float *logits, int V, int nch, int K, const int *count, const float *cv,
    const int32_t *ci, const float *lse, const float *rstat, int nrun, int lrc, int nt, int P,
    const int32_t *valid, const uint16_t *code_a, const uint16_t *code_b, int r, float s,
    int32_t *cand_ids, float *cand_logp, int32_t *draft) {
    __shared__ int ids[MAXP][MAXK];
    __shared__ float lp[MAXP][MAXK];
    __shared__ float Tm[MAXP][MAXK][MAXK];
    __shared__ float delta[2][MAXK];
    __shared__ int psi[MAXP][MAXK];
    // run selection: per wave the candidate logits and runs of its row
    __shared__ float cvl[PATH_WAVES][RCAP];
    __shared__ int cil[PATH_WAVES][RCAP];
    __shared__ int crun[PATH_WAVES][RUNCAP];
    __shared__ int cwid[PATH_WAVES][RUNCAP];
    __shared__ float cmax[PATH_WAVES][RUNCAP];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool ok = valid[b] != 0;
    for (int t = wave; t < P; t += PATH_WAVES) {
        const int row = b * P + t;
        if (ok) {
            if (rstat)
                select_row_runs(logits, V, nrun, lrc, nt, K, row, rstat, cvl[wave], cil[wave],
                                crun[wave], cwid[wave], cmax[wave], ids[t], lp[t]);
            else
                select_row(logits, V, nch, K, row, count, cv, ci, lse[row], ids[t], lp[t]);
        }
        if (lane < MAXK && (lane >= K || !ok)) {
            ids[t][lane] = -1;
            lp[t][lane] = -INFINITY;
        }
        __builtin_amdgcn_wave_barrier();
        if (lane < K) {
            cand_ids[(size_t)row * K + lane] = ids[t][lane];
            cand_logp[(size_t)row * K + lane] = lp[t][lane];
        }
    }
    __syncthreads();
    if (!ok) {
        if (tid < P) draft[(size_t)b * P + tid] = -1;
        return;
    }
    const int c = lane & 15, g = lane >> 4;
    const int nks = r / 32;
    for (int t = wave; t + 1 < P; t += PATH_WAVES) {
        const int ua = ids[t][c], vb = ids[t + 1][c];
        const uint16_t *ar = code_a + (size_t)(ua >= 0 ? ua : 0) * r + 8 * g;
        const uint16_t *br = code_b + (size_t)(vb >= 0 ? vb : 0) * r + 8 * g;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        // 8 k-steps of fragments in flight, then their MFMAs (indices past the rank are
        // clamped: in bounds, and their products skipped)
        for (int ks0 = 0; ks0 < nks; ks0 += 8) {
            u32x4_t av[8], bv[8];
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const int ks = min(ks0 + u, nks - 1);
                av[u] = *reinterpret_cast<const u32x4_t *>(ar + ks * 32);
                bv[u] = *reinterpret_cast<const u32x4_t *>(br + ks * 32);
            }
#pragma unroll
            for (int u = 0; u < 8; u++) {
                if (ks0 + u < nks) {
                    const u32x4_t a0 = ua < 0 ? (u32x4_t){0, 0, 0, 0} : av[u];
                    const u32x4_t b0 = vb < 0 ? (u32x4_t){0, 0, 0, 0} : bv[u];
                    acc = mfma16x16x32(a0, b0, acc);
                }
            }
        }
#pragma unroll
        for (int v = 0; v < 4; v++) Tm[t][4 * g + v][c] = s * acc[v];
    }
    __syncthreads();
    if (wave == 0) {
        // delta over candidates j < K on lanes 0..K-1; ties to the lowest index
        const int j = lane;
        float dcur = j < K ? lp[0][j] : -INFINITY;
        for (int t = 0; t + 1 < P; t++) {
            if (j < K) delta[t & 1][j] = dcur;
            __builtin_amdgcn_wave_barrier();
            if (j < K) {
                // every predecessor's score read first (-inf past K), then the running
                // best in index order: ties keep the lowest index
                float sc[MAXK];
#pragma unroll
                for (int i = 0; i < MAXK; i++)
                    sc[i] = i < K ? delta[t & 1][i] + Tm[t][i][j] : -INFINITY;
                float best = sc[0];
                int bi = 0;
#pragma unroll
                for (int i = 1; i < MAXK; i++)
                    if (sc[i] > best) { best = sc[i]; bi = i; }
                psi[t + 1][j] = bi;
                dcur = lp[t + 1][j] + best;
            }
            __builtin_amdgcn_wave_barrier();
        }
        if (j < K) delta[(P - 1) & 1][j] = dcur;
        __builtin_amdgcn_wave_barrier();
        if (lane == 0) {
            const int fin = (P - 1) & 1;
            float dv[MAXK];
#pragma unroll
            for (int i = 0; i < MAXK; i++) dv[i] = i < K ? delta[fin][i] : -INFINITY;
            int jj = 0;
#pragma unroll
            for (int i = 1; i < MAXK; i++)
                if (dv[i] > dv[jj]) jj = i;
            for (int t = P - 1; t >= 0; t--) {
                draft[(size_t)b * P + t] = ids[t][jj];
                if (t > 0) jj = psi[t][jj];
            }
        }
    }
}

// ---------------------------------------------------------------- sampled acceptance
// Mindket kit page "Qwen3.8-27B-DFlash2-GGUF by z-lab": sampling keeps the target's
// distribution ("For newcomers and experts"), sampler temperature 1.0, top-p 0.95,
// top-k 20 ("Good to know").  The draft's proposals are deterministic (the selector's
// path), so rejection sampling runs against a point-mass proposal: x_j is accepted when
// u < p_j(x_j); on rejection a token is drawn from p_j without x_j; when all n are
// accepted a bonus token is drawn from p_n.  p_j = softmax(logits / T) over the top_k
// logits, cut to the smallest (prob desc, id asc) prefix with mass >= top_p.

constexpr int SAMPLE_MAXK = 64;
constexpr int SAMPLE_MAXROWS = 64;
constexpr int SAMPLE_WAVES = 8;

__device__ __forceinline__ float wave_incl_scan(float v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float t = __shfl_up(v, o, WAVE);
        if (lane >= o) v += t;
    }
    return v;
}

// inverse CDF over the lanes' weights r (lane order): the first eligible lane whose
// cumulative weight exceeds u * total; the last eligible lane if rounding runs past the
// end (lane 0 if none is eligible)
__device__ __forceinline__ int draw_lane(float r, float u, bool elig) {
    const float total = wave_sum(r);
    const float c = wave_incl_scan(r);
    const unsigned long long hit = __ballot(elig && c > u * total);
    if (hit) return __builtin_ctzll(hit);
    const unsigned long long e = __ballot(elig);
    return e ? 63 - __builtin_clzll(e) : 0;
}

// One workgroup per sequence: waves select the sequence's n + 1 rows (top_k by logit
// desc, id asc) into LDS, then wave 0 walks the positions in order, one lane per
// candidate.
__global__ __launch_bounds__(64 * SAMPLE_WAVES) void k_sample_accept(
    const float *logits, int V, int nch, int K, const int *count, const float *cv,
    const int32_t *ci, const int32_t *draft, const float *u, int n, float temperature,
    float top_p, int32_t *accept_len, int32_t *out) {
    __shared__ int sid[SAMPLE_MAXROWS][SAMPLE_MAXK];
    __shared__ float sv[SAMPLE_MAXROWS][SAMPLE_MAXK];
    const int b = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rows = n + 1;
    for (int j = wave; j < rows; j += SAMPLE_WAVES)
        select_row(logits, V, nch, K, b * rows + j, count, cv, ci, 0.f, sid[j], sv[j]);
    __syncthreads();
    if (wave != 0) return;
    const float *ub = u + (size_t)b * rows * 2;
    int32_t *ob = out + (size_t)b * rows;
    int k = n;
    for (int j = 0; j < rows; j++) {
        const bool in = lane < K;
        const int id = in ? sid[j][lane] : -1;
        const float w = in ? expf((sv[j][lane] - sv[j][0]) / temperature) : 0.f;
        const float S = wave_sum(w);
        float before = __shfl_up(wave_incl_scan(w), 1, WAVE);   // mass of the lanes below
        if (lane == 0) before = 0.f;
        const bool keep = in && before < top_p * S;             // a prefix of the lanes
        const float wk = keep ? w : 0.f;
        if (j == n) {                                           // every proposal accepted
            const int c = draw_lane(wk, ub[2 * j + 1], keep);
            if (lane == 0) ob[j] = sid[j][c];
            break;
        }
        const int x = draft[(size_t)b * n + j];
        const float Sm = wave_sum(wk);
        const unsigned long long hm = __ballot(keep && id == x);
        const float px = hm ? __shfl(wk, __builtin_ctzll(hm), WAVE) / Sm : 0.f;
        if (ub[2 * j] < px) {
            if (lane == 0) ob[j] = x;
            continue;
        }
        const bool elig = keep && id != x;
        const int c = draw_lane(elig ? w : 0.f, ub[2 * j + 1], elig);
        if (lane == 0) ob[j] = sid[j][c];
        k = j;
        break;
    }
    if (lane > k && lane < rows) ob[lane] = -1;
    if (lane == 0) accept_len[b] = k;
}

}  // namespace

size_t topk_workspace_floats(int R, int V) {
    const int nch = ceil_div(V, CHUNK);
    return (size_t)R * (2 * nch + 2 + 2 * CAP);
}

hipError_t launch_topk_path(const float *logits, int B, int P, int V, int K, const int32_t *valid,
                            float *ws, const uint16_t *code_a, const uint16_t *code_b, int r,
                            float pair_scale, int32_t *cand_ids, float *cand_logp,
                            int32_t *draft_tokens, hipStream_t st) {
    if (P > MAXP || K > MAXK) return hipErrorInvalidValue;
    const int R = B * P;
    const int nch = ceil_div(V, CHUNK);
    float *pm = ws, *ps = pm + (size_t)R * nch, *lse = ps + (size_t)R * nch;
    int *count = reinterpret_cast<int *>(lse + R);
    float *cv = reinterpret_cast<float *>(count + R);
    int32_t *ci = reinterpret_cast<int32_t *>(cv + (size_t)R * CAP);
    const dim3 grid(ceil_div(nch, 4), R);
    hipLaunchKernelGGL(k_chunk_stats, grid, dim3(256), 0, st, logits, V, nch, pm, ps, count);
    hipLaunchKernelGGL(k_collect, grid, dim3(256), 0, st, logits, V, nch, K, pm, ps, lse, count, cv,
                       ci);
    hipLaunchKernelGGL(k_select_path, dim3(B), dim3(64 * PATH_WAVES), 0, st, logits, V, nch, K, count,
                       cv, ci, lse, (const float *)nullptr, 0, 0, 0, P, valid, code_a, code_b, r,
                       pair_scale, cand_ids, cand_logp, draft_tokens);
    return hipGetLastError();
}

hipError_t launch_topk_path_runs(const float *logits, const float *rstat, int nrun, int run_cols,
                                 int run_tiles, int B, int P, int V, int K, const int32_t *valid,
                                 float *ws, const uint16_t *code_a, const uint16_t *code_b, int r,
                                 float pair_scale, int32_t *cand_ids, float *cand_logp,
                                 int32_t *draft_tokens, hipStream_t st) {
    int lrc = 0;
    while ((1 << lrc) < run_cols) lrc++;
    if (P > MAXP || K > MAXK || nrun < 1 || nrun > 64 * RPL || run_cols < 1 || run_cols > 512 ||
        (1 << lrc) != run_cols || (long long)nrun * run_cols < V)
        return hipErrorInvalidValue;
    // balanced runs: they cover the tiles exactly, none wider than run_cols
    if (run_tiles < 0 || (run_tiles && ((long long)run_tiles * 16 < V || run_tiles > 65536 ||
                                        16 * ceil_div(run_tiles, nrun) > run_cols)))
        return hipErrorInvalidValue;
    (void)ws;
    hipLaunchKernelGGL(k_select_path, dim3(B), dim3(64 * PATH_WAVES), 0, st, logits, V,
                       ceil_div(V, CHUNK), K, (const int *)nullptr, (const float *)nullptr,
                       (const int32_t *)nullptr, (const float *)nullptr, rstat, nrun, lrc, run_tiles, P,
                       valid, code_a, code_b, r, pair_scale, cand_ids, cand_logp, draft_tokens);
    return hipGetLastError();
}

hipError_t launch_topk_sample(const float *logits, int B, int n, int V, int K, float *ws,
                              const int32_t *draft, const float *u, float temperature, float top_p,
                              int32_t *accept_len, int32_t *out_tokens, hipStream_t st) {
    if (n + 1 > SAMPLE_MAXROWS || K > SAMPLE_MAXK || K > V) return hipErrorInvalidValue;
    const int R = B * (n + 1);
    const int nch = ceil_div(V, CHUNK);
    float *pm = ws, *ps = pm + (size_t)R * nch, *lse = ps + (size_t)R * nch;
    int *count = reinterpret_cast<int *>(lse + R);
    float *cv = reinterpret_cast<float *>(count + R);
    int32_t *ci = reinterpret_cast<int32_t *>(cv + (size_t)R * CAP);
    const dim3 grid(ceil_div(nch, 4), R);
    hipLaunchKernelGGL(k_chunk_stats, grid, dim3(256), 0, st, logits, V, nch, pm, ps, count);
    hipLaunchKernelGGL(k_collect, grid, dim3(256), 0, st, logits, V, nch, K, pm, ps, nullptr, count,
                       cv, ci);
    hipLaunchKernelGGL(k_sample_accept, dim3(B), dim3(64 * SAMPLE_WAVES), 0, st, logits, V, nch, K,
                       count, cv, ci, draft, u, n, temperature, top_p, accept_len, out_tokens);
    return hipGetLastError();
}

int topk_chunk_size() { return CHUNK; }
