// Activation quantisation to symmetric int8 (BitNest-Llama-3-8B model card,
// recipe table row "Activations": per token, and per 128-column group for
// o_proj). The rule, which the pages leave open and the public header states:
//   s = amax / 127 (IEEE fp32 division), q = 0 if s == 0, otherwise
//   q = clamp(round_half_even(x / s), -127, 127) with x / s an IEEE fp32
//   division (computed by quant_codes in device_common.h, shared with the
//   fused GEMV).
//
// The work is a few KiB per token and latency-bound: one workgroup per token
// holds its whole row in registers (one HBM round trip), reduces |x| with
// DPP and LDS and writes packed codes with 4-byte stores. (Measured on
// MI355X: 512-thread workgroups finish sooner than 1024-thread ones, and
// splitting a row's quantisation over several workgroups does not pay.)
#include "bitnest_internal.h"
#include "device_common.h"

namespace bitnest {
namespace {

constexpr int kQuantThreads = 256;     // grouped kernel
constexpr int kTokenThreads = 512;     // per-token kernel

// One token per workgroup of 512 threads; each thread keeps up to NV float4
// of the row in registers. All loads are issued unconditionally (clamped
// index) before any use, so the row costs one memory round trip.
template <int NV>
__global__ __launch_bounds__(kTokenThreads) void quant_token_kernel(
    const float *__restrict__ x, int K, int8_t *__restrict__ q, float *__restrict__ s) {
    __shared__ float part[kTokenThreads / 64];
    const int m = blockIdx.x;
    const float4 *xr = reinterpret_cast<const float4 *>(x + static_cast<size_t>(m) * K);
    const int n4 = K >> 2;
    float4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = threadIdx.x + i * kTokenThreads;
        v[i] = xr[idx < n4 ? idx : 0];
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = threadIdx.x + i * kTokenThreads;
        if (idx < n4) amax = fmaxf(amax, absmax4(v[i]));
    }
    amax = wave_max_dpp_f32(amax);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = part[0];
#pragma unroll
    for (int w = 1; w < kTokenThreads / 64; ++w) amax = fmaxf(amax, part[w]);
    const float sc = amax / 127.0f;
    const float rc = quant_recip(sc);
    if (threadIdx.x == 0) s[m] = sc;
    unsigned *qr = reinterpret_cast<unsigned *>(q + static_cast<size_t>(m) * K);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = threadIdx.x + i * kTokenThreads;
        if (idx < n4) qr[idx] = quant_pack4(v[i], sc, rc);
    }
}

// One (token, 128-column group) per 32 lanes, eight per workgroup. Row-major
// x [M, K] makes (m, g) -> m*K + 128 g = 128 (m*G + g), so the flat group
// index addresses both x/q and the [M, K/128] scales.
__global__ __launch_bounds__(kQuantThreads) void quant_group_kernel(
    const float *__restrict__ x, int total_groups, int8_t *__restrict__ q, float *__restrict__ s) {
    const int gid = blockIdx.x * (kQuantThreads / 32) + (threadIdx.x >> 5);
    const int l = threadIdx.x & 31;
    const bool active = gid < total_groups;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (active) v = reinterpret_cast<const float4 *>(x + static_cast<size_t>(gid) * kGroup)[l];
    float amax = absmax4(v);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float sc = amax / 127.0f;
    const float rc = quant_recip(sc);
    if (active) {
        if (l == 0) s[gid] = sc;
        reinterpret_cast<unsigned *>(q + static_cast<size_t>(gid) * kGroup)[l] = quant_pack4(v, sc, rc);
    }
}

// The down_proj input path: the R4 rotation (fwht_unit per 8-column unit,
// then one multiply by rot_scale), then the per-token rule above on the
// rotated values. One token per workgroup of TH threads; unit u = tid + k *
// TH (k < NU) holds columns 8 u .. 8 u + 7, so the units of one wave at one
// k are 512 consecutive columns and every rotation block (<= 512 columns)
// lies inside one wave. Units past K read as zero through the buffer
// descriptor and are not written. (The transform makes this kernel
// ALU-bound on its one compute unit, so it runs 16 waves, where the plain
// quantisation is latency-bound and runs 8.)
constexpr int kRotThreads = 1024;
// the block size with a straight-line transform (RB below); others take the
// block from the arguments (RB = 0)
constexpr int kRotFixedBlock = 512;

template <int NU, int RB>
__global__ __launch_bounds__(kRotThreads) void hadamard_quant_kernel(
    const float *__restrict__ x, int K, int block, float rot_scale, int8_t *__restrict__ q, float *__restrict__ s,
    float *__restrict__ xr) {
    constexpr int TH = kRotThreads;
    __shared__ float part[TH / 64];
    const int m = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int nunit = K >> 3;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(x + static_cast<size_t>(m) * K), static_cast<short>(0), K * 4, 0x00020000);
    float v[NU][8];
#pragma unroll
    for (int k = 0; k < NU; ++k) {
        const int off = (threadIdx.x + k * TH) * 32;
        const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
        const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16, 0, 0));
        // (elements copied out before the bit cast: a bit cast of a
        // vector-element lvalue reads element 0 with this compiler)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[k][i] = __builtin_bit_cast(float, static_cast<unsigned>(a[i]));
            v[k][4 + i] = __builtin_bit_cast(float, static_cast<unsigned>(b[i]));
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < NU; ++k) {
        if (k * TH + (threadIdx.x & ~63) < nunit) {    // wave-uniform: units past K stay zero
            if constexpr (RB == 0) fwht_unit(v[k], lane, block);
            else fwht_unit_fixed<RB>(v[k], lane);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v[k][i] = v[k][i] * rot_scale;
                amax = fmaxf(amax, fabsf(v[k][i]));
            }
        }
    }
    amax = wave_max_dpp_f32(amax);
    if (lane == 0) part[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = part[0];
#pragma unroll
    for (int w = 1; w < TH / 64; ++w) amax = fmaxf(amax, part[w]);
    const float sc = amax / 127.0f;
    const float rc = quant_recip(sc);
    if (threadIdx.x == 0) s[m] = sc;
#pragma unroll
    for (int k = 0; k < NU; ++k) {
        const int u = threadIdx.x + k * TH;
        if (u < nunit) {
            unsigned y[8];
            quant_codes<8>(v[k], sc, rc, y);
            *reinterpret_cast<uint2 *>(q + static_cast<size_t>(m) * K + u * 8) =
                make_uint2(pack_low_bytes(y[0], y[1], y[2], y[3]), pack_low_bytes(y[4], y[5], y[6], y[7]));
            if (xr) {
                float4 *o = reinterpret_cast<float4 *>(xr + static_cast<size_t>(m) * K + u * 8);
                o[0] = make_float4(v[k][0], v[k][1], v[k][2], v[k][3]);
                o[1] = make_float4(v[k][4], v[k][5], v[k][6], v[k][7]);
            }
        }
    }
}

}  // namespace

hipError_t launch_hadamard_quant_act(const float *x, int M, int K, int block, float rot_scale, int8_t *xq,
                                     float *xs, float *xr, hipStream_t stream) {
    const int nu = (K / 8 + kRotThreads - 1) / kRotThreads;
    void (*k)(const float *, int, int, float, int8_t *, float *, float *);
    const bool fixed = block == kRotFixedBlock;
    switch (nu) {
        case 1: k = fixed ? hadamard_quant_kernel<1, kRotFixedBlock> : hadamard_quant_kernel<1, 0>; break;
        case 2: k = fixed ? hadamard_quant_kernel<2, kRotFixedBlock> : hadamard_quant_kernel<2, 0>; break;
        default: return hipErrorInvalidValue;   // K > kMaxK: rejected by the ABI before this point
    }
    hipLaunchKernelGGL(k, dim3(M), dim3(kRotThreads), 0, stream, x, K, block, rot_scale, xq, xs, xr);
    return hipGetLastError();
}

hipError_t launch_quant_act(const float *x, int M, int K, int act_group, int8_t *xq, float *xs,
                            hipStream_t stream) {
    if (act_group == kGroup) {
        const int total = M * (K / kGroup);
        const int per_block = kQuantThreads / 32;
        const int blocks = (total + per_block - 1) / per_block;
        hipLaunchKernelGGL(quant_group_kernel, dim3(blocks), dim3(kQuantThreads), 0, stream, x,
                           total, xq, xs);
    } else {
        const int nv = (K / 4 + kTokenThreads - 1) / kTokenThreads;   // float4 per thread
        void (*k)(const float *, int, int8_t *, float *);
        switch (nv) {
            case 1: k = quant_token_kernel<1>; break;
            case 2: k = quant_token_kernel<2>; break;
            case 3: k = quant_token_kernel<3>; break;
            case 4: k = quant_token_kernel<4>; break;
            case 5: k = quant_token_kernel<5>; break;
            case 6: k = quant_token_kernel<6>; break;
            case 7: k = quant_token_kernel<7>; break;
            case 8: k = quant_token_kernel<8>; break;
            default: return hipErrorInvalidValue;   // K > kMaxK: rejected by the ABI before this point
        }
        hipLaunchKernelGGL(k, dim3(M), dim3(kTokenThreads), 0, stream, x, K, xq, xs);
    }
    return hipGetLastError();
}

}  // namespace bitnest
