// Q4_K super-block decode to fp32, gfx950 (one wave per 144-byte super-block).
//
// Format (FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", "Weights" row: the draft's
// matrices in Q4_K): 256 weights along K per super-block, fp16 d and dmin, twelve
// bytes of packed 6-bit sub-block scales sc_j and mins m_j, 128 bytes of nibbles;
// w = d * sc_j * q - dmin * m_j for sub-block j (32 weights), q in 0..15.
#include "common.h"
#include "kernels.h"

namespace {

__global__ void k_q4k_dequant(const unsigned char *w, float *out, long long n_blocks) {
    const long long b = blockIdx.x * (long long)(blockDim.x / 64) + (threadIdx.x >> 6);
    if (b >= n_blocks) return;
    const int lane = threadIdx.x & 63;
    const unsigned char *blk = w + b * 144;
    const float d = half_bits_to_f32(blk[0] | (blk[1] << 8));
    const float dmin = half_bits_to_f32(blk[2] | (blk[3] << 8));
    const unsigned char *s = blk + 4;
#pragma unroll
    for (int h = 0; h < 4; h++) {
        const int i = lane + 64 * h;                 // weight index in the block
        const int c = i >> 6, r = i & 63;
        const int j = i >> 5;
        int sc, m;
        if (j < 4) {
            sc = s[j] & 63;
            m = s[j + 4] & 63;
        } else {
            sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
            m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
        }
        const int byte = blk[16 + 32 * c + (r & 31)];
        const int q = r < 32 ? (byte & 15) : (byte >> 4);
        // d*sc*q and dmin*m are exact in fp32; one rounding in the difference
        out[b * 256 + i] = d * (float)sc * (float)q - dmin * (float)m;
    }
}

}  // namespace

hipError_t launch_q4k_dequant(const void *w, float *out, long long n_blocks, hipStream_t st) {
    const long long grid = (n_blocks + 3) / 4;
    hipLaunchKernelGGL(k_q4k_dequant, dim3((unsigned)grid), dim3(256), 0, st,
                       (const unsigned char *)w, out, n_blocks);
    return hipGetLastError();
}
