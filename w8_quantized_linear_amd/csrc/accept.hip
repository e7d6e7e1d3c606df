// Greedy verification of a speculative round (model card "BitNest-Llama-3-8B",
// introduction: every draft token is verified with the target, so the output
// is exactly the W8A8 target's greedy output). The rule is written out in
// bitnest.h: per verify row the target's argmax (ties to the smallest
// index), the longest prefix of draft tokens equal to it, and the target's
// token after that prefix.
//
// Two launches: one workgroup per row scans the row (16-byte loads when the
// rows are 16-byte aligned) and reduces (value, index) pairs, whose order
// (larger value, then smaller index) makes the result independent of the
// reduction order; then one thread walks the at most 31 draft tokens.
#include "bitnest_internal.h"
#include "device_common.h"

namespace bitnest {
namespace {

constexpr int kArgThreads = 1024;

// (v, i) replaces (bv, bi) when larger, or equal with a smaller index
__device__ __forceinline__ void take(float &bv, int &bi, float v, int i) {
    if (v > bv || (v == bv && i < bi)) {
        bv = v;
        bi = i;
    }
}

template <bool VEC>
__global__ __launch_bounds__(kArgThreads) void row_argmax_kernel(const float *__restrict__ logits, int V,
                                                                  int32_t *__restrict__ targ) {
    __shared__ float sv[kArgThreads / 64];
    __shared__ int si[kArgThreads / 64];
    const float *row = logits + static_cast<size_t>(blockIdx.x) * V;
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;
    if (VEC) {
        // columns 4 j .. 4 j + 3 per float4 j; a thread visits j = tid, tid + T, ...
        // in increasing order and its four columns in order, so the first
        // maximum it sees is its smallest index. A chunk of U float4 per
        // thread (half the row of a 128K vocabulary; as many as the register
        // budget of 1024 threads holds) is requested at once; a float4 whose
        // maximum is below the running best cannot change it, so the exact
        // pairwise update runs only when it can.
        const float4 *r4 = reinterpret_cast<const float4 *>(row);
        const int n4 = V >> 2;
        constexpr int U = 16;
        for (int base = 0; base < n4; base += U * kArgThreads) {
            float4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = base + u * kArgThreads + threadIdx.x;
                v[u] = r4[j < n4 ? j : 0];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = base + u * kArgThreads + threadIdx.x;
                const float m4 = fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w));
                if (j < n4 && m4 >= bv) {
                    take(bv, bi, v[u].x, 4 * j);
                    take(bv, bi, v[u].y, 4 * j + 1);
                    take(bv, bi, v[u].z, 4 * j + 2);
                    take(bv, bi, v[u].w, 4 * j + 3);
                }
            }
        }
    } else {
        for (int j = threadIdx.x; j < V; j += kArgThreads) take(bv, bi, row[j], j);
    }
    // wave, then workgroup: the pair order makes the result independent of
    // the reduction order
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        take(bv, bi, ov, oi);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sv[wave] = bv;
        si[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kArgThreads / 64; ++w) take(bv, bi, sv[w], si[w]);
        targ[blockIdx.x] = bi;
    }
}

__global__ void accept_kernel(int R, const int32_t *__restrict__ draft, const int32_t *__restrict__ targ,
                              int32_t *__restrict__ result) {
    if (threadIdx.x != 0) return;
    int n = 0;
    while (n < R - 1 && draft[n] == targ[n]) ++n;
    result[0] = n;
    result[1] = targ[n];
}

}  // namespace

hipError_t launch_greedy_accept(const float *logits, int R, int V, const int32_t *draft, int32_t *targ,
                                int32_t *result, hipStream_t stream) {
    const bool vec = (V % 4) == 0;   // rows then stay 16-byte aligned
    if (vec)
        hipLaunchKernelGGL(row_argmax_kernel<true>, dim3(R), dim3(kArgThreads), 0, stream, logits, V, targ);
    else
        hipLaunchKernelGGL(row_argmax_kernel<false>, dim3(R), dim3(kArgThreads), 0, stream, logits, V, targ);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(64), 0, stream, R, draft, targ, result);
    return hipGetLastError();
}

}  // namespace bitnest
