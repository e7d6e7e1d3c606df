// Greedy verification of a speculative round (model card "BitNest-Llama-3-8B",
// introduction: every draft token is verified with the target, so the output
// is exactly the W8A8 target's greedy output). The rule is written out in
// bitnest.h: per verify row the target's argmax (ties to the smallest
// index), the longest prefix of draft tokens equal to it, and the target's
// token after that prefix.
//
// Two launches: every row is cut into S slices of about 4K logits, one
// 256-thread workgroup per (slice, row) scans its slice (16-byte loads when
// the rows are 16-byte aligned, all in flight together) and writes its
// (value, index) pair to the caller's workspace; then one wave per row
// reduces the row's S pairs, and one thread walks the at most 31 draft
// tokens. The pair order
// (larger value, then smaller index) makes every result independent of the
// order of the reductions.
#include "bitnest.h"
#include "bitnest_internal.h"
#include "device_common.h"

#include <atomic>

namespace bitnest {
namespace {

constexpr int kSliceThreads = 256;
constexpr int kSliceLogits = 4096;     // about this many logits per slice
constexpr int kMaxSlices = 64;         // one per lane of the final wave

// (v, i) replaces (bv, bi) when larger, or equal with a smaller index
__device__ __forceinline__ void take(float &bv, int &bi, float v, int i) {
    if (v > bv || (v == bv && i < bi)) {
        bv = v;
        bi = i;
    }
}

// wave-wide (value, index) reduction; every lane ends with the result
__device__ __forceinline__ void wave_take(float &bv, int &bi) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        take(bv, bi, ov, oi);
    }
}

int accept_slices(int V) {
    const long long s = (static_cast<long long>(V) + kSliceLogits - 1) / kSliceLogits;   // any V >= 1
    return s < 1 ? 1 : (s > kMaxSlices ? kMaxSlices : static_cast<int>(s));
}

// slice length: ceil(V / S) rounded up to a multiple of 4 (whole float4s)
int accept_slice_len(int V, int S) {
    return static_cast<int>((((static_cast<long long>(V) + S - 1) / S) + 3) & ~3LL);
}

// part[r S + s] = {bits of the slice's largest logit, its smallest column}
template <bool VEC>
__global__ __launch_bounds__(kSliceThreads) void slice_argmax_kernel(const float *__restrict__ logits, int V, int L,
                                                                     uint2 *__restrict__ part) {
    __shared__ float sv[kSliceThreads / 64];
    __shared__ int si[kSliceThreads / 64];
    const int s = blockIdx.x, r = blockIdx.y;
    const float *row = logits + static_cast<size_t>(r) * V;
    const int c0 = s * L;
    const int c1 = c0 + L < V ? c0 + L : V;
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;
    if (VEC) {
        // float4 j holds columns 4 j .. 4 j + 3; U float4 per thread are
        // requested together (a 4096-logit slice is one round); a float4 whose
        // maximum is below the running best cannot change it
        const float4 *r4 = reinterpret_cast<const float4 *>(row);
        const int j1 = c1 >> 2;
        constexpr int U = 4;
        for (int base = c0 >> 2; base < j1; base += U * kSliceThreads) {
            float4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = base + u * kSliceThreads + threadIdx.x;
                v[u] = r4[j < j1 ? j : 0];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = base + u * kSliceThreads + threadIdx.x;
                const float m4 = fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w));
                if (j < j1 && m4 >= bv) {
                    take(bv, bi, v[u].x, 4 * j);
                    take(bv, bi, v[u].y, 4 * j + 1);
                    take(bv, bi, v[u].z, 4 * j + 2);
                    take(bv, bi, v[u].w, 4 * j + 3);
                }
            }
        }
    } else {
        for (int j = c0 + threadIdx.x; j < c1; j += kSliceThreads) take(bv, bi, row[j], j);
    }
    wave_take(bv, bi);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sv[wave] = bv;
        si[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kSliceThreads / 64; ++w) take(bv, bi, sv[w], si[w]);
        part[static_cast<size_t>(r) * gridDim.x + s] = make_uint2(__builtin_bit_cast(unsigned, bv), static_cast<unsigned>(bi));
    }
}

// One wave per row (up to 16 rows at a time): lane l holds slice l, the
// wave reduces them; then thread 0 walks the draft tokens.
constexpr int kAcceptWaves = 16;
__global__ __launch_bounds__(64 * kAcceptWaves) void accept_kernel(int R, int S, const uint2 *__restrict__ part,
                                                                   const int32_t *__restrict__ draft,
                                                                   int32_t *__restrict__ targ,
                                                                   int32_t *__restrict__ result) {
    __shared__ int st[kMaxM];                    // R <= kMaxM (checked by the ABI)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int r = wave; r < R; r += blockDim.x >> 6) {
        float bv = -__builtin_inff();
        int bi = 0x7FFFFFFF;
        if (lane < S) {
            const uint2 p = part[static_cast<size_t>(r) * S + lane];
            bv = __builtin_bit_cast(float, p.x);
            bi = static_cast<int>(p.y);
        }
        wave_take(bv, bi);
        if (lane == 0) {
            st[r] = bi;
            targ[r] = bi;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int n = 0;
        while (n < R - 1 && draft[n] == st[n]) ++n;
        result[0] = n;
        result[1] = st[n];
    }
}

// Scratch of the entry point that allocates nothing: the per-slice pairs of
// the largest call (kMaxM rows x kMaxSlices slices). Each GPU the library
// runs on holds its own copy until the process ends. Host code uses the
// device address from hipGetSymbolAddress, never this name.
constexpr size_t kNoAllocScratchBytes = static_cast<size_t>(kMaxM) * kMaxSlices * sizeof(uint2);   // 16 KiB
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
static_assert(kNoAllocScratchBytes == BITNEST_ACCEPT_NOALLOC_SCRATCH_BYTES, "the size the header states");

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];

// The scratch array's device address on the current device, looked up once
// per device (with that device current) and kept.
hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

size_t accept_workspace_bytes(int R, int V) {
    return static_cast<size_t>(R) * accept_slices(V) * sizeof(uint2);
}

hipError_t launch_greedy_accept(const float *logits, int R, int V, const int32_t *draft, int32_t *targ,
                                int32_t *result, void *work, hipStream_t stream) {
    const int S = accept_slices(V);
    const int L = accept_slice_len(V, S);
    uint2 *part = static_cast<uint2 *>(work);
    if ((V % 4) == 0)      // rows then stay 16-byte aligned
        hipLaunchKernelGGL(slice_argmax_kernel<true>, dim3(S, R), dim3(kSliceThreads), 0, stream, logits, V, L, part);
    else
        hipLaunchKernelGGL(slice_argmax_kernel<false>, dim3(S, R), dim3(kSliceThreads), 0, stream, logits, V, L, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int waves = R < kAcceptWaves ? R : kAcceptWaves;
    hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(64 * waves), 0, stream, R, S, part, draft, targ, result);
    return hipGetLastError();
}

size_t accept_noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t launch_greedy_accept_noalloc(const float *logits, int R, int V, const int32_t *draft, int32_t *targ,
                                        int32_t *result, hipStream_t stream) {
    if (accept_workspace_bytes(R, V) > kNoAllocScratchBytes) return hipErrorInvalidValue;
    void *work = nullptr;
    const hipError_t e = scratch_address(&work);
    if (e != hipSuccess) return e;
    // every pair the second launch reads is written by the first: nothing
    // of the scratch needs clearing
    return launch_greedy_accept(logits, R, V, draft, targ, result, work, stream);
}

}  // namespace bitnest
