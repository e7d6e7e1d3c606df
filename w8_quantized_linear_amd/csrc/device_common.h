// Small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitnest {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// fp16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// 16 bytes that are read exactly once per call: non-temporal, so the plane
// stream does not evict the activations and scales from the caches.
__device__ __forceinline__ u32x4 load_stream16(const uint8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// DPP lane moves (gfx9 encodings of the dpp_ctrl field).
enum : int {
    kDppQuadSwap1 = 0xB1,   // quad_perm [1,0,3,2]
    kDppQuadSwap2 = 0x4E,   // quad_perm [2,3,0,1]
    kDppRowRor4 = 0x124,    // rotate right by 4 within each row of 16 lanes
    kDppRowRor8 = 0x128,    // rotate right by 8 within each row of 16 lanes
    kDppRowBcast15 = 0x142, // lane 15 of each row to the whole next row
    kDppRowBcast31 = 0x143, // lane 31 to rows 2 and 3
};

template <int kCtrl>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                  kCtrl, 0xF, 0xF, false));
}

// DPP move with a row mask: rows outside the mask keep their old value and
// receive 0 to add (the old operand is 0 and bound_ctrl is off).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_f32_masked(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                                                  kRowMask, 0xF, false));
}

// Exact integer sum over the 4 lanes of a quad; every lane of the quad gets it.
__device__ __forceinline__ int quad_sum_i32(int v) {
    v += dpp_i32<kDppQuadSwap1>(v);
    v += dpp_i32<kDppQuadSwap2>(v);
    return v;
}

// Sum over the 16 quads of a wave of a value that is uniform within each quad.
// The association order is fixed, so the result is deterministic. Lane 0
// holds the sum (all lanes do, with lane-dependent association).
__device__ __forceinline__ float sum_over_quads_f32(float v) {
    v += dpp_f32<kDppRowRor4>(v);
    v += dpp_f32<kDppRowRor8>(v);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// The activation quantisation rule of the public header: q = 0 if s == 0,
// else clamp(round_half_even(x / s), -127, 127), x / s an IEEE fp32 division.
//
// Computed without a division per element: with r = fl(1/s) and
// t = fl(x * r), |t - x/s| <= |x/s| (2u + u^2) and the correctly rounded
// quotient q = fl(x/s) has |q - x/s| <= |x/s| u (u = 2^-24), so
// |t - q| <= 3.0001 u |x/s| <= 2.3e-5 for |x/s| <= 127.5 (|x| <= amax, hence
// |x/s| <= 127 (1 + u)). When t is farther than that from every half-integer
// tie, rint(t) == rint(q); only the rare elements within 3e-5 of a tie take
// the exact division (hipcc's default division is correctly rounded).
__device__ __forceinline__ int quant_code_r(float x, float s, float r) {
    if (s == 0.0f) return 0;
    const float t = x * r;
    float c = rintf(t);                     // v_rndne_f32: ties to even
    if (!(fabsf(t - c) <= 0.49997f)) c = rintf(x / s);   // near a tie, or r overflowed
    c = fminf(fmaxf(c, -127.0f), 127.0f);
    return static_cast<int>(c);
}

__device__ __forceinline__ float quant_recip(float s) { return s == 0.0f ? 0.0f : 1.0f / s; }

// Four codes packed into a dword (first element in the low byte); r is
// quant_recip(s).
__device__ __forceinline__ unsigned quant_pack4(const float4 &v, float s, float r) {
    return (static_cast<unsigned>(quant_code_r(v.x, s, r)) & 0xFFu) |
           ((static_cast<unsigned>(quant_code_r(v.y, s, r)) & 0xFFu) << 8) |
           ((static_cast<unsigned>(quant_code_r(v.z, s, r)) & 0xFFu) << 16) |
           ((static_cast<unsigned>(quant_code_r(v.w, s, r)) & 0xFFu) << 24);
}

__device__ __forceinline__ float absmax4(const float4 &v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ int sdot4(unsigned a, unsigned b, int acc) {
    return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), acc, false);
}

}  // namespace bitnest
