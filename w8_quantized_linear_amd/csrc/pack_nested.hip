// Offline nested packing of fp32 weights into the hi / lo planes (model card
// "BitNest-Llama-3-8B": introduction - the high nibble is a GPTQ-W4 model
// fitted first, the low nibble the closed-form residual back to W8; section
// "Files", entry planes.safetensors - the format). GPTQ itself needs
// calibration data; this is the symmetric round-to-nearest quantiser it
// builds on (15 steps, zero point 8), per (row, 128-column group), with the
// stored fp16 scale (the rule is written out in bitnest.h).
//
// One lane per 8 consecutive columns, so one 128-column group is one row of
// 16 lanes: the group maximum is a DPP reduction inside the row, the codes
// of the lane's 8 columns give 4 bytes of each plane (one 32-bit store per
// plane), and the row's first lane stores the scale. The kernel streams
// 4 bytes per weight in and 1 byte per weight out; flat group g covers
// floats [128 g, 128 g + 128) of the row-major [N, K] input.
#include "bitnest_internal.h"
#include "device_common.h"

namespace bitnest {
namespace {

constexpr int kPackThreads = 256;            // 16 groups per workgroup

// clamp(rne(x / s), -8, 7) for 8 values (quant_codes: exact rounding of the
// IEEE quotient), returned as signed ints
__device__ __forceinline__ void codes4bit(const float (&x)[8], float s, float r, int (&c)[8]) {
    unsigned y[8];
    quant_codes<8>(x, s, r, y);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int v = static_cast<int>(static_cast<int8_t>(y[i] & 0xFFu));
        c[i] = v < -8 ? -8 : (v > 7 ? 7 : v);
    }
}

// 8 signed codes in [-8, 7] -> 4 plane bytes (column 2j in the low nibble of
// byte j, column 2j + 1 in the high nibble), u = c + 8
__device__ __forceinline__ unsigned pack_nibbles(const int (&c)[8]) {
    unsigned w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= static_cast<unsigned>(c[i] + 8) << (4 * i);
    return w;
}

__global__ __launch_bounds__(kPackThreads) void pack_nested_kernel(const float *__restrict__ W, long long groups,
                                                                  uint8_t *__restrict__ hi, uint8_t *__restrict__ lo,
                                                                  uint16_t *__restrict__ scale) {
    const long long t = static_cast<long long>(blockIdx.x) * kPackThreads + threadIdx.x;
    const long long g = t >> 4;                      // flat (row, group) index
    const int lane16 = threadIdx.x & 15;
    const bool live = g < groups;                    // uniform within a row of 16 lanes
    float w[8];
    if (live) {
        const float4 *src = reinterpret_cast<const float4 *>(W + t * 8);
        const float4 a = src[0], b = src[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = 0.0f;
    }
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(w[i]));
    am = row16_max_f32(am);
    // s = fp16(amax / 7.5): IEEE fp32 division, then binary16 round to nearest even
    const _Float16 s16 = static_cast<_Float16>(am / 7.5f);
    const float s = static_cast<float>(s16);
    const float s16th = s * 0.0625f;                 // exact: a power-of-two scaling
    int ch[8], cl[8];
    codes4bit(w, s, quant_recip(s), ch);
    float res[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) res[i] = w[i] - static_cast<float>(ch[i]) * s;   // ch * s is exact
    codes4bit(res, s16th, quant_recip(s16th), cl);
    if (live) {
        reinterpret_cast<unsigned *>(hi)[t] = pack_nibbles(ch);
        reinterpret_cast<unsigned *>(lo)[t] = pack_nibbles(cl);
        if (lane16 == 0) scale[g] = __builtin_bit_cast(uint16_t, s16);
    }
}

}  // namespace

hipError_t launch_pack_nested(const float *W, int N, int K, uint8_t *hi, uint8_t *lo, uint16_t *scale,
                              hipStream_t stream) {
    const long long groups = static_cast<long long>(N) * (K / kGroup);
    const long long threads = groups * 16;
    const long long blocks = (threads + kPackThreads - 1) / kPackThreads;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_nested_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kPackThreads), 0, stream, W,
                       groups, hi, lo, scale);
    return hipGetLastError();
}

}  // namespace bitnest
