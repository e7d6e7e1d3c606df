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

// DPP lane moves (gfx9 encodings of the dpp_ctrl field).
enum : int {
    kDppQuadSwap1 = 0xB1,   // quad_perm [1,0,3,2]
    kDppQuadSwap2 = 0x4E,   // quad_perm [2,3,0,1]
    kDppRowRor4 = 0x124,    // rotate right by 4 within each row of 16 lanes
    kDppRowRor8 = 0x128,    // rotate right by 8 within each row of 16 lanes
    kDppRowHalfMirror = 0x141, // reverse each half-row of 8 lanes
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

// The activation quantisation rule of the public header: q = 0 if s == 0,
// else clamp(round_half_even(x / s), -127, 127), x / s an IEEE fp32 division.
//
// Computed without a division per element. With r = fl(1/s), the exact
// product x r is within u |x/s| of x/s, and so is the correctly rounded
// quotient fl(x/s) (u = 2^-24, |x/s| <= 127 (1 + u) because |x| <= amax), so
// the two are within 1.6e-5 of each other. One fma rounds x r to the nearest
// integer c (ties to even; see kRoundMagic) and a second one gives the
// distance |x r - c| to a rounding error of 2^-25. When that distance is at
// most 0.49997, x r is at least 3e-5 from every half-integer, fl(x/s) lies on
// the same side of all of them, and rint(fl(x/s)) == c. Otherwise (a value
// within 3e-5 of a tie, or 1/s overflowed) the whole unit of values is
// redone with the exact division. The clamp can never act: |x/s| <= 127 (1+u)
// rounds to at most 127.
//
// kRoundMagic = 1.5 * 2^23: for |v| < 2^22, v + kRoundMagic lies in [2^23,
// 2^24), where the fp32 spacing is 1, so the sum is v rounded to an integer
// (ties to even: kRoundMagic is even), and the low byte of its bit pattern is
// that integer modulo 256, i.e. the int8 code.
constexpr float kRoundMagic = 12582912.0f;

// Codes of n values with one scale: y[i] holds code i in its low byte.
template <int n>
__device__ __forceinline__ void quant_codes(const float (&x)[n], float s, float r, unsigned (&y)[n]) {
    float dist = 0.0f;
#pragma unroll
    for (int i = 0; i < n; ++i) {
        const float v = __builtin_fmaf(x[i], r, kRoundMagic);
        dist = fmaxf(dist, fabsf(__builtin_fmaf(x[i], r, -(v - kRoundMagic))));
        y[i] = __builtin_bit_cast(unsigned, v);
    }
    // The redo is rare: the test is made wave-wide first, so that the
    // divisions are branched over (not computed for every lane and
    // discarded) when no lane of the wave needs them. The empty asm passes
    // the scale through a register the compiler cannot see into, so that the
    // divisions stay inside the branch instead of being hoisted above it.
    const bool redo = !(dist <= 0.49997f) || !(r <= 3.0e38f);
    if (__builtin_amdgcn_ballot_w64(redo) != 0) {
        float sv = s;
        asm volatile("" : "+v"(sv));
        if (redo) {
#pragma unroll
            for (int i = 0; i < n; ++i) y[i] = __builtin_bit_cast(unsigned, rintf(x[i] / sv) + kRoundMagic);
        }
    }
}

__device__ __forceinline__ float quant_recip(float s) { return s == 0.0f ? 0.0f : 1.0f / s; }

// The low bytes of y0..y3 as one dword, y0's in the lowest byte.
__device__ __forceinline__ unsigned pack_low_bytes(unsigned y0, unsigned y1, unsigned y2, unsigned y3) {
    const unsigned p01 = __builtin_amdgcn_perm(y1, y0, 0x0c0c0400u);
    const unsigned p23 = __builtin_amdgcn_perm(y3, y2, 0x0c0c0400u);
    return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
}

// Four codes packed into a dword (first element in the low byte); r is
// quant_recip(s).
__device__ __forceinline__ unsigned quant_pack4(const float4 &v, float s, float r) {
    const float x[4] = {v.x, v.y, v.z, v.w};
    unsigned y[4];
    quant_codes<4>(x, s, r, y);
    return pack_low_bytes(y[0], y[1], y[2], y[3]);
}

// Maximum over each row of 16 lanes, in every lane of the row.
__device__ __forceinline__ float row16_max_f32(float v) {
    v = fmaxf(v, dpp_f32<kDppQuadSwap1>(v));
    v = fmaxf(v, dpp_f32<kDppQuadSwap2>(v));
    v = fmaxf(v, dpp_f32<kDppRowRor4>(v));
    v = fmaxf(v, dpp_f32<kDppRowRor8>(v));
    return v;
}

// Maximum over the wave, wave-uniform.
__device__ __forceinline__ float wave_max_dpp_f32(float v) {
    v = row16_max_f32(v);
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// One cross-lane stage of fwht_unit: lanes with bit m clear hold a = z[i],
// their partners (lane ^ m) hold c = z[i + 8 m]; the lower lane keeps
// a + c, the upper one a - c, computed as fma(own, +-1, partner): the product
// by +-1 is exact and the fma rounds once, so the bits are those of a + c and
// a - c. The partner's value comes without LDS traffic where the hardware
// allows: DPP quad permutes (m = 1, 2), DPP row rotate by 8 (m = 8), a
// swizzle (m = 4); for m = 16 and 32 the gfx950 row / half-wave swaps
// exchange the two halves of (v, v), after which the first result holds the
// lower lane's value and the second the upper lane's, in both lanes of a
// pair.
template <int m>
__device__ __forceinline__ void fwht_cross_stage(float (&v)[8], int lane) {
    static_assert(m == 1 || m == 2 || m == 4 || m == 8 || m == 16 || m == 32, "lane masks 1..32");
    const float sgn = (lane & m) ? -1.0f : 1.0f;          // upper lanes subtract their own value
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const unsigned u = __builtin_bit_cast(unsigned, v[i]);
        if constexpr (m == 16 || m == 32) {
            unsigned lo, hi;
            if constexpr (m == 16) {
                const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
                lo = r[0];
                hi = r[1];
            } else {
                const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
                lo = r[0];
                hi = r[1];
            }
            v[i] = __builtin_fmaf(__builtin_bit_cast(float, hi), sgn, __builtin_bit_cast(float, lo));
        } else {
            float p;
            if constexpr (m == 1) p = dpp_f32<kDppQuadSwap1>(v[i]);
            else if constexpr (m == 2) p = dpp_f32<kDppQuadSwap2>(v[i]);
            else if constexpr (m == 8) p = dpp_f32<kDppRowRor8>(v[i]);
            else p = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(static_cast<int>(u), 0x1F | (4 << 10)));
            v[i] = __builtin_fmaf(v[i], sgn, p);
        }
    }
}

// The stages of fwht_unit inside one lane, h = 1, 2, 4 while h < b.
__device__ __forceinline__ void fwht_lane_stage(float (&v)[8], int h) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (i & h) continue;
        const float a = v[i], c = v[i + h];
        v[i] = a + c;
        v[i + h] = a - c;
    }
}

// One 8-value unit of the R4 rotation of the down_proj input (model card,
// recipe table row "Rotation": an online Hadamard on the down_proj inputs;
// the matrices are not given, the reading here is the Sylvester-Hadamard
// transform per block of b columns). Lane `lane` holds elements
// 8 j .. 8 j + 7 of its block, j = lane mod b/8 (b a power of two,
// 2 <= b <= 512, so a block never leaves a wave). Stages h = 1, 2, ..., b/2
// in that order, each replacing the pair (a, c) = (z[i], z[i + h]), i with
// bit h clear, by (a + c, a - c): h < 8 inside the lane, h >= 8 with the
// partner lane lane ^ (h / 8). The caller then scales by r_b.
__device__ __forceinline__ void fwht_unit(float (&v)[8], int lane, int b) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
        if (h < b) fwht_lane_stage(v, h);               // uniform
    if (b > 8) fwht_cross_stage<1>(v, lane);            // uniform conditions
    if (b > 16) fwht_cross_stage<2>(v, lane);
    if (b > 32) fwht_cross_stage<4>(v, lane);
    if (b > 64) fwht_cross_stage<8>(v, lane);
    if (b > 128) fwht_cross_stage<16>(v, lane);
    if (b > 256) fwht_cross_stage<32>(v, lane);
}

// fwht_unit with the block size B fixed when compiling: the same stages as
// straight-line code (with a run-time size, the compiler places each stage
// behind a branch, away from the rest).
template <int B>
__device__ __forceinline__ void fwht_unit_fixed(float (&v)[8], int lane) {
    static_assert(B >= 2 && B <= 512 && (B & (B - 1)) == 0, "a power of two in [2, 512]");
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
        if (h < B) fwht_lane_stage(v, h);
    if constexpr (B > 8) fwht_cross_stage<1>(v, lane);
    if constexpr (B > 16) fwht_cross_stage<2>(v, lane);
    if constexpr (B > 32) fwht_cross_stage<4>(v, lane);
    if constexpr (B > 64) fwht_cross_stage<8>(v, lane);
    if constexpr (B > 128) fwht_cross_stage<16>(v, lane);
    if constexpr (B > 256) fwht_cross_stage<32>(v, lane);
}

__device__ __forceinline__ float absmax4(const float4 &v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ int sdot4(unsigned a, unsigned b, int acc) {
    return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), acc, false);
}

}  // namespace bitnest
