// Device helpers shared by the gfx950 kernels of the draft step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

#define WAVE 64

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// float -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}

// D = A . B + C on a 16x16x32 bf16 MFMA tile.
// Lane l: A row (l & 15), B column (l & 15), k slots 8*(l >> 4) .. +7;
// D rows 4*(l >> 4) + v (v = 0..3), column (l & 15).
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D = A . B + C on a 32x32x16 bf16 MFMA tile (gfx950; twice the rate of 16x16x32).
// Lane l: A row (l & 31), B column (l & 31), k slots 8*(l >> 5) .. +7;
// D register j: row 8*(j >> 2) + 4*(l >> 5) + (j & 3), column (l & 31).
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// The value of lane (lane ^ J) of the wave, J a power of two below 64.  J < 16 stays in
// the VALU (DPP: quad permutes for 1 and 2; for 4 and 8 the row shifts by J up and down,
// chosen by the lane's bit J), 16 is a ds_swizzle (xor within 32 lanes), 32 a
// ds_bpermute: the short distances of a butterfly avoid the LDS crossbar's latency.
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
    const int x = (int)v;
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
    } else if constexpr (J == 4 || J == 8) {
        const int up = __builtin_amdgcn_update_dpp(x, x, 0x100 + J, 0xF, 0xF, false);  // row_shl: lane + J
        const int dn = __builtin_amdgcn_update_dpp(x, x, 0x110 + J, 0xF, 0xF, false);  // row_shr: lane - J
        return (uint32_t)((__lane_id() & J) ? dn : up);
    } else if constexpr (J == 16) {
        return (uint32_t)__builtin_amdgcn_ds_swizzle(x, 0x401F);   // and 31, xor 16
    } else {
        static_assert(J == 32, "lane distance");
        return (uint32_t)__shfl_xor(x, 32, WAVE);
    }
}

template <int J>
__device__ __forceinline__ float xor_lane(float v) {
    return __uint_as_float(xor_lane<J>(__float_as_uint(v)));
}

// xor_lane for a distance known after unrolling (the switch folds away)
template <class T>
__device__ __forceinline__ T xor_lane_n(T v, int j) {
    switch (j) {
        case 1: return xor_lane<1>(v);
        case 2: return xor_lane<2>(v);
        case 4: return xor_lane<4>(v);
        case 8: return xor_lane<8>(v);
        case 16: return xor_lane<16>(v);
        default: return xor_lane<32>(v);
    }
}

// butterfly reductions over the wave (distances 32, 16, .., 1: every lane ends with the
// same value, summed in the same order in every lane)
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += xor_lane_n(v, o);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, xor_lane_n(v, o));
    return v;
}

// (value desc, id asc) ordering of candidates
__device__ __forceinline__ bool cand_better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Deferred RMSNorm: a row's activations enter a GEMM as bf16(v * gain) and the GEMM's
// output row is multiplied by 1 / rms(v) = rsqrt(sum(v^2) / n + eps) afterwards (the
// norm is a per-row scale).  sum(v^2) is kept as nchunk partial sums per row.
struct RowScale {
    const float *ssq;          // [rows][nchunk]; null: scale 1
    int nchunk;
    int map;                   // 0: row r; T > 1: proposal row r of blocks of T (T - 1 proposals
                               // each) -> block row (r / (T - 1)) T + r % (T - 1) + 1
    float n, eps;
};

__device__ __forceinline__ float row_inv(const RowScale &s, int r) {
    if (!s.ssq) return 1.f;
    const int br = s.map ? (r / (s.map - 1)) * s.map + r % (s.map - 1) + 1 : r;
    const float *p = s.ssq + (size_t)br * s.nchunk;
    float ss = 0.f;
    for (int i0 = 0; i0 < s.nchunk; i0 += 8) {          // 8 loads in flight, summed in order
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) v[u] = p[min(i0 + u, s.nchunk - 1)];
#pragma unroll
        for (int u = 0; u < 8; u++)
            if (i0 + u < s.nchunk) ss += v[u];
    }
    return rsqrtf(ss / s.n + s.eps);
}
