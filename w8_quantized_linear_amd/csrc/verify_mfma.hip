// Batched-verify kernel for the nested W4/W8 linear, 8 <= M <= 32 tokens,
// on the gfx950 int8 matrix cores (v_mfma_i32_16x16x64_i8).
//
// Operation: the same as the GEMV (BitNest-Llama-3-8B model card, "Files",
// planes.safetensors: draft W4 = (hi - 8) scale, target W8 =
// (16 (hi - 8) + (lo - 8)) scale / 16), with several verify sequences
// batched so that the product is a real dense contraction: M tokens x 16
// weight rows x 64 columns per instruction.
//
// Operand construction. One MFMA computes D[i][j] += sum_k A[i][k] B[k][j]
// with A = 16 tokens x 64 columns (lane l holds token l % 16) and B = 64
// columns x 16 weight rows (lane l holds weight row l % 16); both take 16
// columns per lane from the same column set, chosen by l / 16. The columns
// of a group can be visited in any order as long as A and B agree, so:
//  - lane l loads the 16 plane bytes (32 columns) of its weight row that sit
//    in quarter l / 16 of the group, one 128-bit load per plane;
//  - the nibbles are turned into signed int8 bytes equal to 16 * (u - 8)
//    (xor 0x88 turns each nibble into the 4-bit two's complement of u - 8;
//    placing it in the high half of a byte multiplies it by 16): the odd
//    columns with one mask, the even columns with a shift and a mask;
//  - the activation bytes of the same 32 columns are split into the even and
//    the odd columns with v_perm_b32, matching the weight operand byte for
//    byte.
// Two MFMAs (even, odd columns) per plane and token tile give 16 * P_hi and
// 16 * P_lo for one 128-column group exactly; P8 = 16 P_hi + P_lo =
// D_hi + (D_lo >> 4). The 8-bit code is never formed as an int8; each plane
// has its own contraction, combined in int32.
// Epilogue per group: fp32 accumulate of float(P) * scale (/16 for the
// target) (* the group's activation scale for o_proj).
//
// Work split: a workgroup owns 16 weight rows; its 8 waves split the groups
// of K into contiguous ranges (one read of every plane byte), and the
// partial sums meet in LDS in a fixed order.
#include "bitnest_internal.h"
#include "device_common.h"

namespace bitnest {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerBlock = 16;
constexpr unsigned kSelEven = 0x06040200u;
constexpr unsigned kSelOdd = 0x07050301u;

// 16 plane bytes -> even / odd column operands, each byte = 16 * (u - 8).
__device__ __forceinline__ void signed16(const u32x4 w, i32x4 &even, i32x4 &odd) {
    const u32x4 x = w ^ 0x88888888u;
    even = __builtin_bit_cast(i32x4, (x << 4u) & 0xF0F0F0F0u);
    odd = __builtin_bit_cast(i32x4, x & 0xF0F0F0F0u);
}

// 32 activation bytes (two 16-byte loads) -> even / odd column operands.
__device__ __forceinline__ void split_act(const u32x4 v0, const u32x4 v1, i32x4 &even, i32x4 &odd) {
    even = i32x4{static_cast<int>(__builtin_amdgcn_perm(v0.y, v0.x, kSelEven)),
                 static_cast<int>(__builtin_amdgcn_perm(v0.w, v0.z, kSelEven)),
                 static_cast<int>(__builtin_amdgcn_perm(v1.y, v1.x, kSelEven)),
                 static_cast<int>(__builtin_amdgcn_perm(v1.w, v1.z, kSelEven))};
    odd = i32x4{static_cast<int>(__builtin_amdgcn_perm(v0.y, v0.x, kSelOdd)),
                static_cast<int>(__builtin_amdgcn_perm(v0.w, v0.z, kSelOdd)),
                static_cast<int>(__builtin_amdgcn_perm(v1.y, v1.x, kSelOdd)),
                static_cast<int>(__builtin_amdgcn_perm(v1.w, v1.z, kSelOdd))};
}

// T: 16-token tiles (1 for M <= 16, 2 for M <= 32).
template <int PLANES, int T, bool GA, bool EXPORT>
__global__ __launch_bounds__(kThreads) void verify_mfma_kernel(const LinearArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    float *red = reinterpret_cast<float *>(smem);                       // [kWaves][T][4][64]
    float *sact = red + kWaves * T * 4 * 64;                             // [G][16 T] (GA)

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int K = a.K, N = a.N, M = a.M;
    const int G = K >> 7;
    const int row_bytes = K >> 1;
    const int col = lane & 15;          // weight row within the tile; token within an A tile
    const int kq = lane >> 4;           // quarter of the group; token quad of a D tile
    const int row = blockIdx.x * kRowsPerBlock + col;
    const bool row_ok = row < N;

    if (GA && !EXPORT) {
        for (int i = threadIdx.x; i < G * 16 * T; i += kThreads) {
            const int g = i / (16 * T);
            const int t = i - g * 16 * T;
            sact[i] = t < M ? a.xs[static_cast<size_t>(t) * G + g] : 0.0f;
        }
        __syncthreads();
    }

    const int g0 = (G * wave) / kWaves;
    const int g1 = (G * (wave + 1)) / kWaves;
    const float fscale = PLANES == 2 ? 0.0625f : 1.0f;
    const size_t roff = static_cast<size_t>(row_ok ? row : 0) * row_bytes + kq * 16;
    const uint8_t *hrow = a.hi + roff;
    const uint8_t *lrow = PLANES == 2 ? a.lo + roff : nullptr;
    const uint16_t *srow = a.scale + static_cast<size_t>(row_ok ? row : 0) * G;

    float yacc[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[t][r] = 0.0f;

#pragma unroll 2
    for (int g = g0; g < g1; ++g) {
        u32x4 wh = u32x4{0u, 0u, 0u, 0u}, wl = u32x4{0u, 0u, 0u, 0u};
        float sc = 0.0f;
        if (row_ok) {
            wh = load_stream16(hrow + g * 64);
            if (PLANES == 2) wl = load_stream16(lrow + g * 64);
            if (!EXPORT) sc = half_bits_to_float(srow[g]) * fscale;
        }
        u32x4 av[T][2];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int tok = 16 * t + col;
            av[t][0] = u32x4{0u, 0u, 0u, 0u};
            av[t][1] = u32x4{0u, 0u, 0u, 0u};
            if (tok < M) {
                const u32x4 *p = reinterpret_cast<const u32x4 *>(
                    a.xq + static_cast<size_t>(tok) * K + g * kGroup + kq * 32);
                av[t][0] = p[0];
                av[t][1] = p[1];
            }
        }
        i32x4 bhe, bho, ble, blo;
        signed16(wh, bhe, bho);
        if (PLANES == 2) signed16(wl, ble, blo);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            i32x4 ae, ao;
            split_act(av[t][0], av[t][1], ae, ao);
            const i32x4 zero = {0, 0, 0, 0};
            i32x4 dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(ae, bhe, zero, 0, 0, 0);
            dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(ao, bho, dh, 0, 0, 0);
            i32x4 dl = zero;
            if (PLANES == 2) {
                dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(ae, ble, zero, 0, 0, 0);
                dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(ao, blo, dl, 0, 0, 0);
            }
            if (EXPORT) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tok = 16 * t + 4 * kq + r;
                    if (tok < M && row_ok) {
                        const size_t o = (static_cast<size_t>(tok) * N + row) * G + g;
                        const int ph = dh[r] >> 4;
                        a.p_hi[o] = ph;
                        if (PLANES == 2) {
                            const int pl = dl[r] >> 4;
                            a.p_lo[o] = pl;
                            a.p8[o] = dh[r] + pl;
                        }
                    }
                }
            } else {
                float sa[4] = {1.0f, 1.0f, 1.0f, 1.0f};
                if (GA) {
                    const float4 v = *reinterpret_cast<const float4 *>(sact + g * 16 * T + 16 * t + 4 * kq);
                    sa[0] = v.x; sa[1] = v.y; sa[2] = v.z; sa[3] = v.w;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int p = PLANES == 2 ? dh[r] + (dl[r] >> 4) : (dh[r] >> 4);
                    const float w = GA ? sc * sa[r] : sc;
                    yacc[t][r] += static_cast<float>(p) * w;
                }
            }
        }
    }

    if (!EXPORT) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[((wave * T + t) * 4 + r) * 64 + lane] = yacc[t][r];
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int t = 0; t < T; ++t) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = red[((0 * T + t) * 4 + r) * 64 + lane];
#pragma unroll
                    for (int w = 1; w < kWaves; ++w) v += red[((w * T + t) * 4 + r) * 64 + lane];
                    const int tok = 16 * t + 4 * kq + r;
                    if (tok < M && row_ok)
                        a.y[static_cast<size_t>(tok) * N + row] = GA ? v : v * a.xs[tok];
                }
            }
        }
    }
}

typedef void (*VerifyKernel)(const LinearArgs);

template <int PLANES, int T>
VerifyKernel pick_mode(bool grouped, bool exporting) {
    if (exporting) return verify_mfma_kernel<PLANES, T, false, true>;
    return grouped ? verify_mfma_kernel<PLANES, T, true, false> : verify_mfma_kernel<PLANES, T, false, false>;
}

}  // namespace

hipError_t launch_verify_mfma(const LinearArgs &a, bool export_partials, hipStream_t stream) {
    if (a.M < 8 || a.M > kMaxM) return hipErrorInvalidValue;
    const int T = a.M <= 16 ? 1 : 2;
    const bool target = a.lo != nullptr;
    const bool grouped = a.act_group == kGroup && !export_partials;
    VerifyKernel k;
    if (target)
        k = T == 1 ? pick_mode<2, 1>(grouped, export_partials) : pick_mode<2, 2>(grouped, export_partials);
    else
        k = T == 1 ? pick_mode<1, 1>(grouped, export_partials) : pick_mode<1, 2>(grouped, export_partials);
    const size_t G = a.K / kGroup;
    const size_t lds = static_cast<size_t>(kWaves) * T * 4 * 64 * sizeof(float) +
                       (grouped ? G * 16 * T * sizeof(float) : 0);
    DeviceInfo dev;
    hipError_t e = device_info(&dev);
    if (e != hipSuccess) return e;
    if (lds > static_cast<size_t>(dev.max_lds)) return hipErrorInvalidValue;
    if (lds > 65536) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    const int blocks = (a.N + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(k, dim3(blocks), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace bitnest
