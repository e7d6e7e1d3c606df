// Plane-streaming GEMV for the nested W4/W8 linear, M <= 7 tokens.
//
// Operation (BitNest-Llama-3-8B model card, "Files", planes.safetensors, and
// the recipe table rows "Weights" and "Activations"):
//   draft : y[m,n] = sum_g float(P_hi) * scale[n,g] * s_a            (reads hi only)
//   target: y[m,n] = sum_g float(16 P_hi + P_lo) * scale[n,g]/16 * s_a
//   P_plane[m,n,g] = sum_{k in g} q[m,k] * (u_plane[n,k] - 8), exact in int32.
//
// Layout in HBM: planes uint8 [N, K/2] row-major (byte j = columns 2j (low
// nibble) and 2j+1 (high nibble)); scales fp16 [N, K/128]; codes int8 [M, K].
//
// Work split. The kernel is bound by HBM: every plane byte is read once.
//  - A wave owns whole weight rows (grid-stride over rows). Lane l reads the
//    16-byte slot l of each 1 KiB chunk of the row with one 128-bit
//    non-temporal load, so one wave instruction moves 1 KiB, fully coalesced.
//    All chunks of a row (and both planes for the target) are issued before
//    any arithmetic, to keep enough bytes in flight.
//  - A 16-byte slot holds 32 columns, a quarter of a 128-column group, so the
//    four lanes of a quad hold one group.
//  - The workgroup first copies the int8 codes of all M tokens into LDS,
//    permuted so that each activation dword lines up with the even or the odd
//    nibbles of a weight dword; the tile is shared by the M tokens' rows and
//    by both planes.
//  - Per slot: even nibbles = w & 0x0F0F0F0F, odd nibbles = (w >> 4) &
//    0x0F0F0F0F (unsigned 0..15), two v_dot4_i32_i8 per weight dword per
//    token. The sign shift (u - 8) is applied per group as - 8 * sum(q) for
//    the draft and - 136 * sum(q) for the target's 16 hi + lo, with the
//    per-(group, token) code sums precomputed in LDS. The 8-bit code
//    16 (hi - 8) + (lo - 8) in [-136, 119] is never formed as an int8.
//  - A 2-step DPP quad sum gives the exact int32 group partial, converted
//    once to fp32 and scaled by the group's weight scale (and, for o_proj,
//    the group's activation scale). A 4-step reduction over the 16 quads
//    ends the row.
// The draft and the target run the same code with the same fp32 operation
// order, and scale/16 is an exact power-of-two scaling, so lo == 8 makes
// the target bit-identical to the draft; rows of an M-token call are
// bit-identical to single-token calls.
#include "bitnest_internal.h"
#include "device_common.h"

#include <atomic>

namespace bitnest {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr unsigned kLowNibbles = 0x0F0F0F0Fu;

// v_perm_b32 selectors: bytes {0,2} of lo and {0,2} of hi (even columns),
// and bytes {1,3}, {1,3} (odd columns).
constexpr unsigned kSelEven = 0x06040200u;
constexpr unsigned kSelOdd = 0x07050301u;

// Unpacked nibbles of one 16-byte slot: e[d] / o[d] are the even / odd
// columns of weight dword d, one unsigned nibble per byte.
struct Nibbles {
    unsigned e[4], o[4];
};

__device__ __forceinline__ Nibbles unpack(const u32x4 w) {
    Nibbles n;
    n.e[0] = w.x & kLowNibbles; n.o[0] = (w.x >> 4) & kLowNibbles;
    n.e[1] = w.y & kLowNibbles; n.o[1] = (w.y >> 4) & kLowNibbles;
    n.e[2] = w.z & kLowNibbles; n.o[2] = (w.z >> 4) & kLowNibbles;
    n.e[3] = w.w & kLowNibbles; n.o[3] = (w.w >> 4) & kLowNibbles;
    return n;
}

// Sum over the slot's 32 columns of q * u (u unsigned), with the activation
// halves a0 = [e0 o0 e1 o1], a1 = [e2 o2 e3 o3] as staged in LDS.
__device__ __forceinline__ int dot_slot(const Nibbles &n, const u32x4 a0, const u32x4 a1) {
    int acc = 0;
    acc = sdot4(a0.x, n.e[0], acc);
    acc = sdot4(a0.y, n.o[0], acc);
    acc = sdot4(a0.z, n.e[1], acc);
    acc = sdot4(a0.w, n.o[1], acc);
    acc = sdot4(a1.x, n.e[2], acc);
    acc = sdot4(a1.y, n.o[2], acc);
    acc = sdot4(a1.z, n.e[3], acc);
    acc = sdot4(a1.w, n.o[3], acc);
    return acc;
}

template <int M>
struct GemvLds {
    static constexpr int kMP = (M + 3) & ~3;   // tokens padded to 4 in the per-group tables
    static size_t bytes(int K, bool grouped_act) {
        const size_t G = K / kGroup;
        return static_cast<size_t>(M) * K + G * kMP * sizeof(int) +
               (grouped_act ? G * kMP * sizeof(float) : 0);
    }
};

// PLANES: 1 draft (hi), 2 target (hi + lo). GA: per-128-group activation
// scales. EXPORT: write the integer partials instead of y. CB: chunk slots
// unrolled per row (a row has C = ceil(K / 2048) chunks, C <= CB).
template <int PLANES, int M, bool GA, bool EXPORT, int CB>
__global__ __launch_bounds__(kThreads) void gemv_planes_kernel(const LinearArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int kMP = GemvLds<M>::kMP;
    const int K = a.K;
    const int N = a.N;
    const int G = K >> 7;
    const int slots = K >> 5;       // 16-byte slots per plane row
    const int row_bytes = K >> 1;   // bytes per plane row

    unsigned char *act = smem;                                       // [M][2][slots][16]
    int *sumq = reinterpret_cast<int *>(smem + static_cast<size_t>(M) * K);   // [G][kMP]
    float *sact = reinterpret_cast<float *>(sumq + G * kMP);        // [G][kMP] (GA)

    // ---- stage the codes, permuted: 16-column block j of token m is half
    // (j & 1) of slot (j >> 1).
    const int nb16 = K >> 4;
    for (int i = threadIdx.x; i < M * nb16; i += kThreads) {
        const int m = i / nb16;
        const int j = i - m * nb16;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(a.xq + static_cast<size_t>(m) * K + 16 * j);
        u32x4 o;
        o.x = __builtin_amdgcn_perm(v.y, v.x, kSelEven);
        o.y = __builtin_amdgcn_perm(v.y, v.x, kSelOdd);
        o.z = __builtin_amdgcn_perm(v.w, v.z, kSelEven);
        o.w = __builtin_amdgcn_perm(v.w, v.z, kSelOdd);
        *reinterpret_cast<u32x4 *>(act + static_cast<size_t>(m) * K + (j & 1) * row_bytes +
                                   (j >> 1) * 16) = o;
    }
    // ---- per (group, token) code sums and grouped activation scales
    for (int i = threadIdx.x; i < G * kMP; i += kThreads) {
        const int g = i / kMP;
        const int m = i - g * kMP;
        int acc = 0;
        float sv = 0.0f;
        if (m < M) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(a.xq + static_cast<size_t>(m) * K + g * kGroup);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const u32x4 v = p[t];
                acc = sdot4(v.x, 0x01010101u, acc);
                acc = sdot4(v.y, 0x01010101u, acc);
                acc = sdot4(v.z, 0x01010101u, acc);
                acc = sdot4(v.w, 0x01010101u, acc);
            }
            if (GA) sv = a.xs[static_cast<size_t>(m) * G + g];
        }
        sumq[i] = acc;
        if (GA) sact[i] = sv;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int C = (slots + 63) >> 6;
    const float fscale = PLANES == 2 ? 0.0625f : 1.0f;    // scale / 16 for the target
    constexpr int kOff = PLANES == 2 ? 136 : 8;             // 16*8 + 8, or 8
    const u32x4 *act4 = reinterpret_cast<const u32x4 *>(act);
    const int tok4 = K >> 4;     // u32x4 per token
    const int half4 = K >> 5;    // u32x4 per half (= slots)

    for (int row = blockIdx.x * kWaves + wave; row < N; row += gridDim.x * kWaves) {
        const uint8_t *hrow = a.hi + static_cast<size_t>(row) * row_bytes;
        const uint8_t *lrow = PLANES == 2 ? a.lo + static_cast<size_t>(row) * row_bytes : nullptr;
        const uint16_t *srow = a.scale + static_cast<size_t>(row) * G;

        u32x4 wh[CB], wl[CB];
        float sc[CB];
#pragma unroll
        for (int b = 0; b < CB; ++b) {
            const int s = b * 64 + lane;
            wh[b] = u32x4{0u, 0u, 0u, 0u};
            wl[b] = u32x4{0u, 0u, 0u, 0u};
            sc[b] = 0.0f;
            if (b < C && s < slots) {
                wh[b] = load_stream16(hrow + s * 16);
                if (PLANES == 2) wl[b] = load_stream16(lrow + s * 16);
                if (!EXPORT) sc[b] = half_bits_to_float(srow[s >> 2]) * fscale;
            }
        }

        float acc[M];
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = 0.0f;

#pragma unroll
        for (int b = 0; b < CB; ++b) {
            if (b >= C) break;                       // uniform across the wave
            const int s = b * 64 + lane;
            const bool valid = s < slots;            // uniform within each quad
            const int ss = valid ? s : 0;
            const int g = ss >> 2;
            const Nibbles nh = unpack(wh[b]);
            Nibbles nl;
            if (PLANES == 2) nl = unpack(wl[b]);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const u32x4 a0 = act4[m * tok4 + ss];
                const u32x4 a1 = act4[m * tok4 + half4 + ss];
                const int sq = sumq[g * kMP + m];
                if (EXPORT) {
                    const int ph = quad_sum_i32(dot_slot(nh, a0, a1)) - 8 * sq;
                    int pl = 0;
                    if (PLANES == 2) pl = quad_sum_i32(dot_slot(nl, a0, a1)) - 8 * sq;
                    if (valid && (lane & 3) == 0) {
                        const size_t o = (static_cast<size_t>(m) * N + row) * G + g;
                        a.p_hi[o] = ph;
                        if (PLANES == 2) {
                            a.p_lo[o] = pl;
                            a.p8[o] = 16 * ph + pl;
                        }
                    }
                } else {
                    int p = dot_slot(nh, a0, a1);
                    if (PLANES == 2) p = 16 * p + dot_slot(nl, a0, a1);
                    p = quad_sum_i32(p) - kOff * sq;
                    const float w = GA ? sc[b] * sact[g * kMP + m] : sc[b];
                    const float f = static_cast<float>(p) * w;
                    acc[m] += valid ? f : 0.0f;
                }
            }
        }
        if (!EXPORT) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float v = sum_over_quads_f32(acc[m]);
                if (lane == 0) a.y[static_cast<size_t>(m) * N + row] = GA ? v : v * a.xs[m];
            }
        }
    }
}

typedef void (*GemvKernel)(const LinearArgs);

template <int PLANES, int M, int CB>
GemvKernel pick_mode(bool grouped, bool exporting) {
    if (exporting) return gemv_planes_kernel<PLANES, M, false, true, CB>;
    return grouped ? gemv_planes_kernel<PLANES, M, true, false, CB>
                   : gemv_planes_kernel<PLANES, M, false, false, CB>;
}

template <int PLANES, int M>
GemvKernel pick_cb(int C, bool grouped, bool exporting) {
    return C <= 2 ? pick_mode<PLANES, M, 2>(grouped, exporting)
                  : pick_mode<PLANES, M, 8>(grouped, exporting);
}

template <int PLANES>
GemvKernel pick_m(int M, int C, bool grouped, bool exporting) {
    switch (M) {
        case 1: return pick_cb<PLANES, 1>(C, grouped, exporting);
        case 2: return pick_cb<PLANES, 2>(C, grouped, exporting);
        case 3: return pick_cb<PLANES, 3>(C, grouped, exporting);
        case 4: return pick_cb<PLANES, 4>(C, grouped, exporting);
        case 5: return pick_cb<PLANES, 5>(C, grouped, exporting);
        case 6: return pick_cb<PLANES, 6>(C, grouped, exporting);
        case 7: return pick_cb<PLANES, 7>(C, grouped, exporting);
        default: return nullptr;
    }
}

size_t gemv_lds_bytes(int M, int K, bool grouped) {
    switch (M) {
        case 1: return GemvLds<1>::bytes(K, grouped);
        case 2: return GemvLds<2>::bytes(K, grouped);
        case 3: return GemvLds<3>::bytes(K, grouped);
        case 4: return GemvLds<4>::bytes(K, grouped);
        case 5: return GemvLds<5>::bytes(K, grouped);
        case 6: return GemvLds<6>::bytes(K, grouped);
        case 7: return GemvLds<7>::bytes(K, grouped);
        default: return 0;
    }
}

}  // namespace

hipError_t launch_gemv(const LinearArgs &a, bool export_partials, hipStream_t stream) {
    const int slots = a.K / 32;
    const int C = (slots + 63) / 64;
    const bool target = a.lo != nullptr;
    const bool grouped = a.act_group == kGroup && !export_partials;
    GemvKernel k = target ? pick_m<2>(a.M, C, grouped, export_partials)
                          : pick_m<1>(a.M, C, grouped, export_partials);
    if (!k || C > 8) return hipErrorInvalidValue;
    DeviceInfo dev;
    hipError_t e = device_info(&dev);
    if (e != hipSuccess) return e;
    const size_t lds = gemv_lds_bytes(a.M, a.K, grouped);
    if (lds > static_cast<size_t>(dev.max_lds)) return hipErrorInvalidValue;
    if (lds > 65536) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    const int rows_blocks = (a.N + kWaves - 1) / kWaves;
    const int blocks = rows_blocks < dev.cus * 2 ? rows_blocks : dev.cus * 2;
    hipLaunchKernelGGL(k, dim3(blocks), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace bitnest
