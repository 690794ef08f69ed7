// Candidate-path selector and greedy prefix acceptance, gfx950.
//
// Selector (FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", spec table "Draft" row:
// candidate selector, top 16, rank 256; "Weights" row: two 248320 x 256
// codebooks; "How it is used": one coherent path through the top 16 candidates
// per position).  The path objective used here: the sum over positions of the
// candidates' log-probabilities plus s <A[u], B[v]> for every pair of adjacent
// chosen candidates u (earlier) and v (later), maximised by Viterbi; ties go to
// the lowest candidate index.
//
// One workgroup per sequence: the codebook rows of each adjacent position pair
// are gathered into LDS, the K x K pair scores are dot products of r bf16 values
// in fp32, and the dynamic programme runs on K threads.
//
// Acceptance (same card, "How it is used" and "FastFlowLM measurements"): the
// longest drafted prefix equal to the target's greedy tokens, plus one target
// token.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int MAXK = 16;
constexpr int MAXP = 16;
constexpr int MAXR = 512;

__global__ __launch_bounds__(256) void k_viterbi(const int32_t *cand_ids, const float *cand_logp,
                                                 const uint16_t *code_a, const uint16_t *code_b,
                                                 int P, int K, int r, float s, const int32_t *valid,
                                                 int32_t *draft) {
    __shared__ int ids[MAXP][MAXK];
    __shared__ float lp[MAXP][MAXK];
    __shared__ __align__(16) uint16_t Ar[MAXK * MAXR];
    __shared__ __align__(16) uint16_t Br[MAXK * MAXR];
    __shared__ float Tm[MAXP][MAXK][MAXK];
    __shared__ float delta[2][MAXK];
    __shared__ int psi[MAXP][MAXK];
    const int b = blockIdx.x, tid = threadIdx.x;
    if (!valid[b]) {
        if (tid < P) draft[(size_t)b * P + tid] = -1;
        return;
    }
    for (int e = tid; e < P * K; e += 256) {
        ids[e / K][e % K] = cand_ids[(size_t)b * P * K + e];
        lp[e / K][e % K] = cand_logp[(size_t)b * P * K + e];
    }
    __syncthreads();
    for (int t = 0; t + 1 < P; t++) {
        // gather A rows of position t and B rows of position t+1 (16-byte pieces)
        const int pieces = r / 8;
        for (int e = tid; e < K * pieces; e += 256) {
            const int i = e / pieces, q = e % pieces;
            const int ua = ids[t][i], vb = ids[t + 1][i];
            const u32x4_t z = {0, 0, 0, 0};
            *reinterpret_cast<u32x4_t *>(&Ar[i * r + 8 * q]) =
                ua >= 0 ? *reinterpret_cast<const u32x4_t *>(code_a + (size_t)ua * r + 8 * q) : z;
            *reinterpret_cast<u32x4_t *>(&Br[i * r + 8 * q]) =
                vb >= 0 ? *reinterpret_cast<const u32x4_t *>(code_b + (size_t)vb * r + 8 * q) : z;
        }
        __syncthreads();
        if (tid < K * K) {
            const int i = tid / K, j = tid % K;
            float acc = 0.f;
            for (int k = 0; k < r; k++) acc += bf16_to_f32(Ar[i * r + k]) * bf16_to_f32(Br[j * r + k]);
            Tm[t][i][j] = s * acc;
        }
        __syncthreads();
    }
    if (tid < K) delta[0][tid] = lp[0][tid];
    __syncthreads();
    for (int t = 0; t + 1 < P; t++) {
        const int cur = t & 1;
        if (tid < K) {
            const int j = tid;
            float best = delta[cur][0] + Tm[t][0][j];
            int bi = 0;
            for (int i = 1; i < K; i++) {
                const float v = delta[cur][i] + Tm[t][i][j];
                if (v > best) { best = v; bi = i; }
            }
            delta[cur ^ 1][j] = lp[t + 1][j] + best;
            psi[t + 1][j] = bi;
        }
        __syncthreads();
    }
    if (tid == 0) {
        const int fin = (P - 1) & 1;
        int j = 0;
        for (int i = 1; i < K; i++)
            if (delta[fin][i] > delta[fin][j]) j = i;
        for (int t = P - 1; t >= 0; t--) {
            draft[(size_t)b * P + t] = ids[t][j];
            if (t > 0) j = psi[t][j];
        }
    }
}

__global__ void k_verify(const int32_t *draft, const int32_t *target, int B, int n,
                         int32_t *accept_len, int32_t *out) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int32_t *dr = draft + (size_t)b * n;
    const int32_t *tg = target + (size_t)b * (n + 1);
    int k = 0;
    while (k < n && dr[k] == tg[k]) k++;
    accept_len[b] = k;
    int32_t *o = out + (size_t)b * (n + 1);
    for (int j = 0; j <= n; j++) o[j] = j < k ? dr[j] : (j == k ? tg[k] : -1);
}

}  // namespace

hipError_t launch_viterbi(const int32_t *cand_ids, const float *cand_logp, const uint16_t *code_a,
                          const uint16_t *code_b, int B, int P, int K, int r, float pair_scale,
                          const int32_t *valid, int32_t *draft_tokens, hipStream_t st) {
    hipLaunchKernelGGL(k_viterbi, dim3(B), dim3(256), 0, st, cand_ids, cand_logp, code_a, code_b,
                       P, K, r, pair_scale, valid, draft_tokens);
    return hipGetLastError();
}

hipError_t launch_verify(const int32_t *draft, const int32_t *target, int B, int n,
                         int32_t *accept_len, int32_t *out_tokens, hipStream_t st) {
    hipLaunchKernelGGL(k_verify, dim3(ceil_div(B, 64)), dim3(64), 0, st, draft, target, B, n,
                       accept_len, out_tokens);
    return hipGetLastError();
}
