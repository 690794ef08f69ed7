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
// Acceptance (same card, "How it is used" and "FastFlowLM measurements"): the
// longest drafted prefix equal to the target's greedy tokens, plus one target
// token.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int MAXK = 16;
constexpr int MAXP = 16;

// One workgroup (8 waves) per sequence.  The pair scores of adjacent positions are
// K x K products of gathered codebook rows, T_t = s A[ids_t] B[ids_{t+1}]^T, computed
// as 16x16xr MFMA tiles (exact bf16 products, fp32 accumulation) straight from the
// gathered rows: lane (i, k-group) loads its 16-byte fragments of A[ids_t[i]] and
// B[ids_{t+1}[i]] for every k-step, all loads in flight at once.  Wave w handles
// positions t = w, w + 8, ... (one each for the 8-token block); the dynamic
// programme then runs on K lanes.
constexpr int VIT_WAVES = 8;

__global__ __launch_bounds__(64 * VIT_WAVES) void k_viterbi(const int32_t *cand_ids, const float *cand_logp,
                                                 const uint16_t *code_a, const uint16_t *code_b,
                                                 int P, int K, int r, float s, const int32_t *valid,
                                                 int32_t *draft) {
    __shared__ int ids[MAXP][MAXK];
    __shared__ float lp[MAXP][MAXK];
    __shared__ float Tm[MAXP][MAXK][MAXK];
    __shared__ float delta[2][MAXK];
    __shared__ int psi[MAXP][MAXK];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (!valid[b]) {
        if (tid < P) draft[(size_t)b * P + tid] = -1;
        return;
    }
    for (int e = tid; e < P * MAXK; e += 64 * VIT_WAVES) {
        const int t = e / MAXK, i = e % MAXK;
        ids[t][i] = i < K ? cand_ids[(size_t)b * P * K + t * K + i] : -1;
        lp[t][i] = i < K ? cand_logp[(size_t)b * P * K + t * K + i] : -INFINITY;
    }
    __syncthreads();
    const int c = lane & 15, g = lane >> 4;
    const int nks = r / 32;
    for (int t = wave; t + 1 < P; t += VIT_WAVES) {
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
            float best = -INFINITY;
            int bi = 0;
            if (j < K) {
                best = delta[t & 1][0] + Tm[t][0][j];
                for (int i = 1; i < K; i++) {
                    const float v = delta[t & 1][i] + Tm[t][i][j];
                    if (v > best) { best = v; bi = i; }
                }
                psi[t + 1][j] = bi;
                dcur = lp[t + 1][j] + best;
            }
            __builtin_amdgcn_wave_barrier();
        }
        if (j < K) delta[(P - 1) & 1][j] = dcur;
        __builtin_amdgcn_wave_barrier();
        if (lane == 0) {
            const int fin = (P - 1) & 1;
            int jj = 0;
            for (int i = 1; i < K; i++)
                if (delta[fin][i] > delta[fin][jj]) jj = i;
            for (int t = P - 1; t >= 0; t--) {
                draft[(size_t)b * P + t] = ids[t][jj];
                if (t > 0) jj = psi[t][jj];
            }
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
    hipLaunchKernelGGL(k_viterbi, dim3(B), dim3(64 * VIT_WAVES), 0, st, cand_ids, cand_logp, code_a, code_b,
                       P, K, r, pair_scale, valid, draft_tokens);
    return hipGetLastError();
}

hipError_t launch_verify(const int32_t *draft, const int32_t *target, int B, int n,
                         int32_t *accept_len, int32_t *out_tokens, hipStream_t st) {
    hipLaunchKernelGGL(k_verify, dim3(ceil_div(B, 64)), dim3(64), 0, st, draft, target, B, n,
                       accept_len, out_tokens);
    return hipGetLastError();
}
