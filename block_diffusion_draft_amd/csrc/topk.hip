// Log-softmax statistics and top-K candidates of the shared output head, gfx950.
//
// FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2": the draft shares the target's output
// head (spec table "Draft" row) and keeps the top 16 candidates per proposal
// position (section "How it is used").  Candidates are ordered by (logit desc,
// token id asc); cand_logp = logit - logsumexp(logits).
//
// Two passes over the fp32 logits: per (row, 4096-logit chunk) a workgroup keeps
// its chunk's max, sum of exp(logit - max) and top-K; one workgroup per row then
// merges the chunk lists and statistics.  Selection is K rounds of a
// workgroup-wide arg-max with the (value, id) order, so the result is exact and
// independent of thread scheduling.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int PER_THREAD = 16;
constexpr int CHUNK = 256 * PER_THREAD;

struct Best {
    float v;
    int i;
};

__device__ __forceinline__ Best better(Best a, Best b) {
    return cand_better(a.v, a.i, b.v, b.i) ? a : b;
}

// workgroup (256 threads) arg-max under (value desc, id asc); id -1 = none
__device__ Best block_argmax(Best x, Best *scratch) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        Best y;
        y.v = __shfl_xor(x.v, o, WAVE);
        y.i = __shfl_xor(x.i, o, WAVE);
        if (y.i >= 0 && (x.i < 0 || cand_better(y.v, y.i, x.v, x.i))) x = y;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) scratch[wave] = x;
    __syncthreads();
    Best r = scratch[0];
    for (int w = 1; w < 4; w++) {
        const Best y = scratch[w];
        if (y.i >= 0 && (r.i < 0 || cand_better(y.v, y.i, r.v, r.i))) r = y;
    }
    return r;
}

__device__ float block_reduce(float v, bool is_max, float *scratch) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float y = __shfl_xor(v, o, WAVE);
        v = is_max ? fmaxf(v, y) : v + y;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    float r = scratch[0];
    for (int w = 1; w < 4; w++) r = is_max ? fmaxf(r, scratch[w]) : r + scratch[w];
    return r;
}

__global__ __launch_bounds__(256) void k_topk_partial(const float *logits, int V, int K,
                                                      float *pv, int32_t *pi, float *pm,
                                                      float *ps) {
    __shared__ Best sb[4];
    __shared__ float sf[4];
    const int c = blockIdx.x, r = blockIdx.y, nch = gridDim.x;
    const int base = c * CHUNK;
    const float *row = logits + (size_t)r * V;
    float val[PER_THREAD];
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < PER_THREAD; k++) {
        const int id = base + threadIdx.x + 256 * k;
        val[k] = id < V ? row[id] : -INFINITY;
        mx = fmaxf(mx, val[k]);
    }
    mx = block_reduce(mx, true, sf);
    float se = 0.f;
#pragma unroll
    for (int k = 0; k < PER_THREAD; k++) se += val[k] == -INFINITY ? 0.f : expf(val[k] - mx);
    se = block_reduce(se, false, sf);
    const size_t o = (size_t)r * nch + c;
    if (threadIdx.x == 0) {
        pm[o] = mx;
        ps[o] = se;
    }
    for (int round = 0; round < K; round++) {
        Best x = {-INFINITY, -1};
#pragma unroll
        for (int k = 0; k < PER_THREAD; k++) {
            const int id = base + threadIdx.x + 256 * k;
            if (id < V && val[k] != -INFINITY && (x.i < 0 || cand_better(val[k], id, x.v, x.i)))
                x = {val[k], id};
        }
        const Best w = block_argmax(x, sb);
        if (threadIdx.x == 0) {
            pv[o * K + round] = w.v;
            pi[o * K + round] = w.i;
        }
#pragma unroll
        for (int k = 0; k < PER_THREAD; k++)
            if (base + threadIdx.x + 256 * k == w.i) val[k] = -INFINITY;
    }
}

constexpr int MERGE_PER_THREAD = 8;     // up to 2048 candidates per row

__global__ __launch_bounds__(256) void k_topk_merge(const float *pv, const int32_t *pi,
                                                    const float *pm, const float *ps, int nch,
                                                    int K, int rows_per_seq, const int32_t *valid,
                                                    int32_t *cand_ids, float *cand_logp) {
    __shared__ Best sb[4];
    __shared__ float sf[4];
    const int r = blockIdx.x;
    const int ncand = nch * K;
    float mx = -INFINITY;
    for (int c = threadIdx.x; c < nch; c += 256) mx = fmaxf(mx, pm[(size_t)r * nch + c]);
    mx = block_reduce(mx, true, sf);
    float se = 0.f;
    for (int c = threadIdx.x; c < nch; c += 256) {
        const float m = pm[(size_t)r * nch + c];
        if (m != -INFINITY) se += ps[(size_t)r * nch + c] * expf(m - mx);
    }
    se = block_reduce(se, false, sf);
    const float lse = mx + logf(se);
    float val[MERGE_PER_THREAD];
    int idv[MERGE_PER_THREAD];
#pragma unroll
    for (int k = 0; k < MERGE_PER_THREAD; k++) {
        const int e = threadIdx.x + 256 * k;
        idv[k] = e < ncand ? pi[(size_t)r * ncand + e] : -1;
        val[k] = idv[k] >= 0 ? pv[(size_t)r * ncand + e] : -INFINITY;
    }
    const bool ok = valid[r / rows_per_seq] != 0;
    for (int round = 0; round < K; round++) {
        Best x = {-INFINITY, -1};
#pragma unroll
        for (int k = 0; k < MERGE_PER_THREAD; k++)
            if (idv[k] >= 0 && (x.i < 0 || cand_better(val[k], idv[k], x.v, x.i))) x = {val[k], idv[k]};
        const Best w = block_argmax(x, sb);
        if (threadIdx.x == 0) {
            cand_ids[(size_t)r * K + round] = ok ? w.i : -1;
            cand_logp[(size_t)r * K + round] = ok && w.i >= 0 ? w.v - lse : -INFINITY;
        }
#pragma unroll
        for (int k = 0; k < MERGE_PER_THREAD; k++)
            if (idv[k] == w.i) idv[k] = -1;
    }
}

}  // namespace

hipError_t launch_topk_partial(const float *logits, int R, int V, int chunk, int K, float *pv,
                               int32_t *pi, float *pm, float *ps, hipStream_t st) {
    (void)chunk;
    dim3 grid(ceil_div(V, CHUNK), R);
    hipLaunchKernelGGL(k_topk_partial, grid, dim3(256), 0, st, logits, V, K, pv, pi, pm, ps);
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
