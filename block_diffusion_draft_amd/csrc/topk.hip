// Log-softmax statistics and top-K candidates of the shared output head, gfx950.
//
// FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2": the draft shares the target's output
// head (spec table "Draft" row) and keeps the top 16 candidates per proposal
// position (section "How it is used").  Candidates are ordered by (logit desc,
// token id asc); cand_logp = logit - logsumexp(logits).
//
// Two passes over the fp32 logits: per (row, 1024-logit chunk) a wave keeps its
// chunk's max, sum of exp(logit - max) and top-K; one workgroup per row then
// merges the chunk lists and statistics.  Every selection is an arg-max under the
// (value desc, id asc) order, so the result is exact and independent of thread
// scheduling.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int PER_LANE = 16;
constexpr int CHUNK = 64 * PER_LANE;     // logits per wave in the first pass
constexpr int LPT = 4;                   // chunk lists per thread in the merge

__device__ __forceinline__ bool take(float v, int i, float bv, int bi) {
    return i >= 0 && (bi < 0 || cand_better(v, i, bv, bi));
}

__device__ __forceinline__ void wave_best(float &v, int &i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(v, o, WAVE);
        const int oi = __shfl_xor(i, o, WAVE);
        if (take(ov, oi, v, i)) { v = ov; i = oi; }
    }
}

// One wave per 1024-logit chunk of one row: chunk max, sum of exp(logit - max)
// and the chunk's top-K in (value desc, id asc) order, with shuffles only.
__global__ __launch_bounds__(256) void k_topk_partial(const float *logits, int V, int K, int nch,
                                                      float *pv, int32_t *pi, float *pm,
                                                      float *ps) {
    const int lane = threadIdx.x & 63;
    const int c = blockIdx.x * 4 + (threadIdx.x >> 6), r = blockIdx.y;
    if (c >= nch) return;
    const int base = c * CHUNK;
    const float *row = logits + (size_t)r * V;
    float val[PER_LANE];
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < PER_LANE; k++) {
        const int id = base + lane + 64 * k;
        val[k] = id < V ? row[id] : -INFINITY;
        mx = fmaxf(mx, val[k]);
    }
    mx = wave_max(mx);
    float se = 0.f;
#pragma unroll
    for (int k = 0; k < PER_LANE; k++) se += val[k] == -INFINITY ? 0.f : expf(val[k] - mx);
    se = wave_sum(se);
    const size_t o = (size_t)r * nch + c;
    if (lane == 0) {
        pm[o] = mx;
        ps[o] = se;
    }
    for (int round = 0; round < K; round++) {
        float bv = -INFINITY;
        int bi = -1;
#pragma unroll
        for (int k = 0; k < PER_LANE; k++) {
            const int id = base + lane + 64 * k;
            if (val[k] != -INFINITY && take(val[k], id, bv, bi)) { bv = val[k]; bi = id; }
        }
        wave_best(bv, bi);
        if (lane == 0) {
            pv[o * K + round] = bv;
            pi[o * K + round] = bi;
        }
#pragma unroll
        for (int k = 0; k < PER_LANE; k++)
            if (base + lane + 64 * k == bi) val[k] = -INFINITY;
    }
}

// One workgroup per row: log-sum-exp from the chunk statistics, then a K-way
// selection over the chunks' sorted lists (each thread owns up to LPT lists and
// offers the best of their heads each round).
__global__ __launch_bounds__(256) void k_topk_merge(const float *pv, const int32_t *pi,
                                                    const float *pm, const float *ps, int nch,
                                                    int K, int rows_per_seq, const int32_t *valid,
                                                    int32_t *cand_ids, float *cand_logp) {
    __shared__ float sf[4];
    __shared__ float wv[4];
    __shared__ int wi[4];
    const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float mx = -INFINITY;
    for (int c = tid; c < nch; c += 256) mx = fmaxf(mx, pm[(size_t)r * nch + c]);
    mx = wave_max(mx);
    if (lane == 0) sf[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(sf[0], sf[1]), fmaxf(sf[2], sf[3]));
    __syncthreads();
    float se = 0.f;
    for (int c = tid; c < nch; c += 256) {
        const float m = pm[(size_t)r * nch + c];
        if (m != -INFINITY) se += ps[(size_t)r * nch + c] * expf(m - mx);
    }
    se = wave_sum(se);
    if (lane == 0) sf[wave] = se;
    __syncthreads();
    const float lse = mx + logf((sf[0] + sf[1]) + (sf[2] + sf[3]));
    const bool ok = valid[r / rows_per_seq] != 0;
    int ptr[LPT];
#pragma unroll
    for (int q = 0; q < LPT; q++) ptr[q] = 0;
    for (int round = 0; round < K; round++) {
        float bv = -INFINITY;
        int bi = -1, bq = -1;
#pragma unroll
        for (int q = 0; q < LPT; q++) {
            const int c = tid + 256 * q;
            if (c < nch && ptr[q] < K) {
                const size_t at = ((size_t)r * nch + c) * K + ptr[q];
                const int id = pi[at];
                const float v = pv[at];
                if (take(v, id, bv, bi)) { bv = v; bi = id; bq = q; }
            }
        }
        float wbv = bv;
        int wbi = bi;
        wave_best(wbv, wbi);
        __syncthreads();
        if (lane == 0) { wv[wave] = wbv; wi[wave] = wbi; }
        __syncthreads();
        float gv = wv[0];
        int gi = wi[0];
        for (int w = 1; w < 4; w++)
            if (take(wv[w], wi[w], gv, gi)) { gv = wv[w]; gi = wi[w]; }
        if (bi >= 0 && bi == gi) ptr[bq]++;          // ids are unique across lists
        if (tid == 0) {
            cand_ids[(size_t)r * K + round] = ok ? gi : -1;
            cand_logp[(size_t)r * K + round] = ok && gi >= 0 ? gv - lse : -INFINITY;
        }
    }
}

}  // namespace

hipError_t launch_topk_partial(const float *logits, int R, int V, int chunk, int K, float *pv,
                               int32_t *pi, float *pm, float *ps, hipStream_t st) {
    (void)chunk;
    const int nch = ceil_div(V, CHUNK);
    dim3 grid(ceil_div(nch, 4), R);
    hipLaunchKernelGGL(k_topk_partial, grid, dim3(256), 0, st, logits, V, K, nch, pv, pi, pm, ps);
    return hipGetLastError();
}

hipError_t launch_topk_merge(const float *pv, const int32_t *pi, const float *pm, const float *ps,
                             int R, int n_chunks, int K, int rows_per_seq, const int32_t *valid,
                             int32_t *cand_ids, float *cand_logp, hipStream_t st) {
    hipLaunchKernelGGL(k_topk_merge, dim3(R), dim3(256), 0, st, pv, pi, pm, ps, n_chunks, K,
                       rows_per_seq, valid, cand_ids, cand_logp);
    return hipGetLastError();
}

int topk_chunk_size() { return CHUNK; }
