// Row-major Q4_K -> the tiled device layout of the Q4_K GEMM kernels, gfx950.
//
// Format (FastFlowLM card "Qwen3.8-27B-DFlash2-NPU2", "Weights" row: the draft's
// linear weights in Q4_K): each row of K weights is K/256 super-blocks of 144 bytes:
// a 16-byte header (fp16 d, fp16 dmin, 12 bytes of 6-bit scales and mins), then 128
// quant bytes, read as 4 chunks of 32 (chunk c holds weights 64 c .. 64 c + 31 in its
// low nibbles and 64 c + 32 .. 64 c + 63 in its high nibbles).
//
// Tiled layout: the same blocks, byte for byte, regrouped so that the 16 rows of a
// 16-column output tile and one super-block are one contiguous 2304-byte unit.  Unit
// (t, kb) sits at (t * K/256 + kb) * 2304:
//     [0, 256)       the 16 headers, row r at 16 r;
//     [256, 2304)    two halves h of 64 slots of 16 bytes, slot s = 16 g + r at
//                    256 + 1024 h + 16 s: quant bytes 8 g .. 8 g + 7 of chunk 2 h, then
//                    of chunk 2 h + 1, of row r's block.
// A wave of 64 lanes (lane = 16 g + r) then reads a unit with three 16-byte loads per
// lane (header of row r, slot lane of each half), every byte once, whole lines.
#include "common.h"
#include "kernels.h"

namespace {

// one thread per 16-byte piece of the output: 144 pieces per unit (16 headers, 128
// quant slots)
__global__ __launch_bounds__(256) void k_q4k_to_tiled(const unsigned char *src, unsigned char *dst,
                                                      int KB, long long n_pieces) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_pieces) return;
    const long long unit = i / 144;
    const int p = (int)(i - unit * 144);
    const long long t = unit / KB;
    const int kb = (int)(unit - t * KB);
    u32x4_t v;
    if (p < 16) {
        const unsigned char *blk = src + ((t * 16 + p) * KB + kb) * 144;
        v = *reinterpret_cast<const u32x4_t *>(blk);
    } else {
        const int q = p - 16, h = q >> 6, s = q & 63, g = s >> 4, r = s & 15;
        const unsigned char *blk = src + ((t * 16 + r) * KB + kb) * 144;
        const u32x2_t a = *reinterpret_cast<const u32x2_t *>(blk + 16 + 32 * (2 * h) + 8 * g);
        const u32x2_t b = *reinterpret_cast<const u32x2_t *>(blk + 16 + 32 * (2 * h + 1) + 8 * g);
        v = (u32x4_t){a.x, a.y, b.x, b.y};
    }
    *reinterpret_cast<u32x4_t *>(dst + unit * Q4K_UNIT_BYTES + 16 * p) = v;
}

}  // namespace

hipError_t launch_q4k_to_tiled(const unsigned char *src, unsigned char *dst, int N, int KB,
                               hipStream_t st) {
    const long long n_pieces = (long long)(N / 16) * KB * 144;
    if (n_pieces == 0) return hipSuccess;
    const long long grid = (n_pieces + 255) / 256;
    hipLaunchKernelGGL(k_q4k_to_tiled, dim3((unsigned)grid), dim3(256), 0, st, src, dst, KB, n_pieces);
    return hipGetLastError();
}
