// Greedy prefix acceptance, gfx950.
//
// FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", sections "How it is used" and
// "FastFlowLM measurements": the longest drafted prefix equal to the target's greedy
// tokens is accepted, plus one target token.
#include "common.h"
#include "kernels.h"

namespace {

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

hipError_t launch_verify(const int32_t *draft, const int32_t *target, int B, int n,
                         int32_t *accept_len, int32_t *out_tokens, hipStream_t st) {
    hipLaunchKernelGGL(k_verify, dim3(ceil_div(B, 64)), dim3(64), 0, st, draft, target, B, n,
                       accept_len, out_tokens);
    return hipGetLastError();
}
