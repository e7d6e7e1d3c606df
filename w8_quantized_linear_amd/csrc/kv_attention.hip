// Decode attention over the nested KV cache (model card "BitNest-Llama-3-8B",
// recipe table row "KV cache": nested at runtime, the draft reads KV4 and
// the target KV8; abstract: the progressive-precision design extends to the
// KV cache for long contexts). The reading, written out in bitnest.h: every
// (token, KV head) vector of 128 values is packed like one 128-column weight
// group (planes [T, Hkv, 64], fp16 scales [T, Hkv]); KV4 = (hi - 8) s,
// KV8 = (16 (hi - 8) + (lo - 8)) s / 16; grouped-query heads; the M query
// tokens are the last M positions (token i sees t <= T - M + i).
//
// Split over the sequence (the draft reads only the hi planes, the target
// both; both are HBM streams of a few bytes per position and head):
//  - kv_attn_split_kernel: one workgroup per (split, KV head), for all M x G
//    query rows of that head; a split is a contiguous run of 64-position
//    chunks, and the number of splits is sized to about two workgroups per
//    compute unit. Per chunk: its K and V rows are staged in LDS (one
//    16-byte load per thread and plane, all in flight together, the next
//    chunk's loads issued while the current one is scored); scores with one
//    lane per position (unsigned nibble codes, the offset applied once per
//    score through the row's sum of q); the running softmax per row
//    (maximum, sum and the rescale of what is accumulated, DPP reductions);
//    P.V with one lane per two dimensions and each wave on 16 positions.
//    At the end the waves' outputs are summed in a fixed order and the
//    split's (output, maximum, sum) per row go to the caller's workspace.
//  - kv_attn_combine_kernel: one workgroup per query row merges the splits:
//    out = sum_s o_s e^(m_s - m) / sum_s l_s e^(m_s - m), the splits' weights
//    staged in LDS and the partial loads spread over four thread groups.
#include "bitnest_internal.h"
#include "device_common.h"

namespace bitnest {
namespace {

constexpr int kD = kKvHeadDim;       // 128
constexpr int kC = kKvChunk;         // 64 positions per workgroup
constexpr int kKvThreads = 256;

__device__ __forceinline__ float wave_sum_f32(float v) {
    v += dpp_f32<kDppQuadSwap1>(v);
    v += dpp_f32<kDppQuadSwap2>(v);
    v += dpp_f32<kDppRowRor4>(v);
    v += dpp_f32<kDppRowRor8>(v);
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

// byte n of x as a float (v_cvt_f32_ubyteN)
template <int n>
__device__ __forceinline__ float ubyte_f(unsigned x) {
    return static_cast<float>((x >> (8 * n)) & 0xFFu);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0), static_cast<int>(bytes),
                                             0x00020000);
}

// RW: query rows per wave (the M x G rows padded to 4 RW). KV8: read the lo
// planes. cps: chunks per split.
template <int RW, bool KV8>
__global__ __launch_bounds__(kKvThreads) void kv_attn_split_kernel(const KvArgs a, int cps) {
    constexpr int RP = 4 * RW;
    constexpr int NPL = KV8 ? 4 : 2;
    __shared__ float sq[RP][kD];
    __shared__ float sqs[RP];
    __shared__ float sp[kC][RP];
    __shared__ float sm[RP], sl[RP], sa[RP];           // running maximum and sum, this chunk's rescale
    __shared__ float so[4][RP][kD];
    // the chunk's planes: [plane][position][16-byte piece] (a fifth piece of
    // padding spreads the per-position reads over the banks), planes K hi,
    // V hi, then K lo, V lo
    __shared__ u32x4 sk[NPL][kC][5];
    __shared__ float sks[kC], svs[kC];

    const int s = blockIdx.x, h = blockIdx.y;
    const int splits = gridDim.x;
    const int nchunks = (a.T + kC - 1) / kC;
    const int c_begin = s * cps;
    const int c_end = min(nchunks, c_begin + cps);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = a.Hq / a.Hkv;
    const int R = a.M * G;

    // staging: thread = (position, 16-byte piece); positions past T read as
    // zero (an offset past the end of the buffer)
    const unsigned cache_bytes = static_cast<unsigned>(a.T) * a.Hkv * (kD / 2);
    const int spos = threadIdx.x >> 2, piece = threadIdx.x & 3;
    const uint8_t *src[4] = {a.k_hi, a.v_hi, a.k_lo, a.v_lo};
    u32x4 v[NPL];
    unsigned short ks = 0, vs = 0;                     // fp16 bits: converted when stored, so that
    auto fetch = [&](int c) {                          // nothing waits on the loads before then
        const int t = c * kC + spos;
        const unsigned off = t < a.T ? (static_cast<unsigned>(t) * a.Hkv + h) * (kD / 2) + 16 * piece : cache_bytes;
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl)
            v[pl] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc(src[pl], cache_bytes), off, 0, 0));
        const int ts = c * kC + threadIdx.x;
        unsigned short k1 = 0, v1 = 0;
        if (threadIdx.x < kC && ts < a.T) {
            k1 = a.k_scale[static_cast<size_t>(ts) * a.Hkv + h];
            v1 = a.v_scale[static_cast<size_t>(ts) * a.Hkv + h];
        }
        ks = k1;
        vs = v1;
    };
    if (c_begin < c_end) fetch(c_begin);

    // query rows r = i G + g (token i, query head h G + g), and their sums
    for (int idx = threadIdx.x; idx < RP * kD; idx += kKvThreads) {
        const int r = idx / kD, j = idx - (idx / kD) * kD;
        float x = 0.0f;
        if (r < R) {
            const int i = r / G, g = r - (r / G) * G;
            x = a.q[(static_cast<size_t>(i) * a.Hq + h * G + g) * kD + j];
        }
        sq[r][j] = x;
    }
    if (threadIdx.x < RP) {
        sm[threadIdx.x] = -__builtin_inff();
        sl[threadIdx.x] = 0.0f;
    }
    __syncthreads();
    if (threadIdx.x < RP) {
        float sum = 0.0f;
        for (int j = 0; j < kD; ++j) sum += sq[threadIdx.x][j];
        sqs[threadIdx.x] = sum;
    }

    float o0[RP], o1[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) o0[r] = o1[r] = 0.0f;

#pragma unroll 1
    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * kC;
        __syncthreads();                               // sqs ready; the previous chunk's P.V is done
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) sk[pl][spos][piece] = v[pl];
        if (threadIdx.x < kC) {
            sks[threadIdx.x] = half_bits_to_float(ks);
            svs[threadIdx.x] = half_bits_to_float(vs);
        }
        __syncthreads();
        if (c + 1 < c_end) fetch(c + 1);               // in flight while this chunk is consumed

        // ---- scores: lane = position t0 + lane, wave = rows [RW wave, RW wave + RW)
        const int t = t0 + lane;
        const bool tv = t < a.T;
        const float kscale = sks[lane];
        // acc: sum u_hi q; accl (KV8): sum u_lo q, accumulated like the row
        // sum of q (j ascending), so that lo = 8 makes it exactly 8 sum(q)
        float acc[RW], accl[RW];
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) acc[rr] = accl[rr] = 0.0f;
        // 16 bytes of each plane (32 columns) per step; a rolled loop keeps
        // the broadcast query reads of one step live at a time
#pragma unroll 1
        for (int cc = 0; cc < 4; ++cc) {
            const u32x4 kh = sk[0][lane][cc];
            const u32x4 kl = KV8 ? sk[2][lane][cc] : kh;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // dword w: columns 32 cc + 8 w + 0 .. 7 (low nibble = even column)
                const unsigned hw = kh[w];
                const unsigned he = hw & 0x0F0F0F0Fu, ho = (hw >> 4) & 0x0F0F0F0Fu;
                float u[8];
                u[0] = ubyte_f<0>(he); u[1] = ubyte_f<0>(ho);
                u[2] = ubyte_f<1>(he); u[3] = ubyte_f<1>(ho);
                u[4] = ubyte_f<2>(he); u[5] = ubyte_f<2>(ho);
                u[6] = ubyte_f<3>(he); u[7] = ubyte_f<3>(ho);
                float ul[8];
                if (KV8) {
                    const unsigned lw = kl[w];
                    const unsigned le = lw & 0x0F0F0F0Fu, lo = (lw >> 4) & 0x0F0F0F0Fu;
                    ul[0] = ubyte_f<0>(le); ul[1] = ubyte_f<0>(lo);
                    ul[2] = ubyte_f<1>(le); ul[3] = ubyte_f<1>(lo);
                    ul[4] = ubyte_f<2>(le); ul[5] = ubyte_f<2>(lo);
                    ul[6] = ubyte_f<3>(le); ul[7] = ubyte_f<3>(lo);
                }
                const int j0 = 32 * cc + 8 * w;
#pragma unroll
                for (int rr = 0; rr < RW; ++rr) {
                    const float4 qa = *reinterpret_cast<const float4 *>(&sq[wave * RW + rr][j0]);
                    const float4 qb = *reinterpret_cast<const float4 *>(&sq[wave * RW + rr][j0 + 4]);
                    float d = acc[rr];
                    d = fmaf(u[0], qa.x, d); d = fmaf(u[1], qa.y, d); d = fmaf(u[2], qa.z, d); d = fmaf(u[3], qa.w, d);
                    d = fmaf(u[4], qb.x, d); d = fmaf(u[5], qb.y, d); d = fmaf(u[6], qb.z, d); d = fmaf(u[7], qb.w, d);
                    acc[rr] = d;
                    if (KV8) {
                        float e = accl[rr];
                        e = fmaf(ul[0], qa.x, e); e = fmaf(ul[1], qa.y, e); e = fmaf(ul[2], qa.z, e); e = fmaf(ul[3], qa.w, e);
                        e = fmaf(ul[4], qb.x, e); e = fmaf(ul[5], qb.y, e); e = fmaf(ul[6], qb.z, e); e = fmaf(ul[7], qb.w, e);
                        accl[rr] = e;
                    }
                }
            }
        }
        // KV4 score = (sum u_hi q - 8 sum q) * s / sqrt(128); KV8 score =
        // (16 (sum u_hi q - 8 sum q) + (sum u_lo q - 8 sum q)) * (s / 16) / sqrt(128):
        // with lo = 8 the second term is exactly 0 and the power-of-two
        // factors cancel exactly, so KV8 then equals KV4 bit for bit.
        // Running softmax: m' = max(m, chunk max), what is accumulated is
        // rescaled by e^(m - m') (0 while nothing is seen yet).
        const float sfac = kscale * a.inv_sqrt_d;
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            const int r = wave * RW + rr;
            const int i = r / G;
            const bool vis = tv && r < R && t <= a.T - a.M + i;
            float dot = acc[rr] - 8.0f * sqs[r];
            if (KV8) dot = 16.0f * dot + (accl[rr] - 8.0f * sqs[r]);
            const float sc = vis ? dot * (KV8 ? sfac * 0.0625f : sfac) : -__builtin_inff();
            const float mo = sm[r];
            const float mn = fmaxf(mo, wave_max_dpp_f32(sc));
            float p = 0.0f;
            if (mn != -__builtin_inff()) p = vis ? expf(sc - mn) : 0.0f;
            const float alpha = mo == -__builtin_inff() ? 0.0f : expf(mo - mn);
            const float l = fmaf(sl[r], alpha, wave_sum_f32(p));
            sp[lane][r] = p;
            if (lane == 0) {
                sm[r] = mn;
                sl[r] = l;
                sa[r] = alpha;
            }
        }
        __syncthreads();

        // ---- P.V: wave = positions t0 + 16 wave + k, lane = dimensions 2 lane, 2 lane + 1
#pragma unroll
        for (int r4 = 0; r4 < RP; r4 += 4) {
            const float4 al = *reinterpret_cast<const float4 *>(&sa[r4]);
            o0[r4] *= al.x; o1[r4] *= al.x;
            o0[r4 + 1] *= al.y; o1[r4 + 1] *= al.y;
            o0[r4 + 2] *= al.z; o1[r4 + 2] *= al.z;
            o0[r4 + 3] *= al.w; o1[r4 + 3] *= al.w;
        }
        // (a rolled loop: unrolled, the compiler hoists every position's
        // loads and runs out of registers)
#pragma unroll 1
        for (int k = 0; k < kC / 4; ++k) {
            const int pl = (kC / 4) * wave + k;
            if (t0 + pl >= a.T) break;                 // uniform
            const float vsc = svs[pl];
            const unsigned vb = reinterpret_cast<const uint8_t *>(&sk[1][pl][0])[lane];
            float v0, v1;
            if (KV8) {
                const unsigned lb = reinterpret_cast<const uint8_t *>(&sk[3][pl][0])[lane];
                v0 = static_cast<float>(16 * (static_cast<int>(vb & 15u) - 8) + (static_cast<int>(lb & 15u) - 8)) *
                     (vsc * 0.0625f);
                v1 = static_cast<float>(16 * (static_cast<int>(vb >> 4) - 8) + (static_cast<int>(lb >> 4) - 8)) *
                     (vsc * 0.0625f);
            } else {
                v0 = static_cast<float>(static_cast<int>(vb & 15u) - 8) * vsc;
                v1 = static_cast<float>(static_cast<int>(vb >> 4) - 8) * vsc;
            }
#pragma unroll
            for (int r4 = 0; r4 < RP; r4 += 4) {
                const float4 p = *reinterpret_cast<const float4 *>(&sp[pl][r4]);
                o0[r4] = fmaf(p.x, v0, o0[r4]); o1[r4] = fmaf(p.x, v1, o1[r4]);
                o0[r4 + 1] = fmaf(p.y, v0, o0[r4 + 1]); o1[r4 + 1] = fmaf(p.y, v1, o1[r4 + 1]);
                o0[r4 + 2] = fmaf(p.z, v0, o0[r4 + 2]); o1[r4 + 2] = fmaf(p.z, v1, o1[r4 + 2]);
                o0[r4 + 3] = fmaf(p.w, v0, o0[r4 + 3]); o1[r4 + 3] = fmaf(p.w, v1, o1[r4 + 3]);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < RP; ++r) {
        so[wave][r][2 * lane] = o0[r];
        so[wave][r][2 * lane + 1] = o1[r];
    }
    __syncthreads();
    float *part = a.work + (static_cast<size_t>(h) * splits + s) * R * (kD + 2);
    for (int idx = threadIdx.x; idx < R * kD; idx += kKvThreads) {
        const int r = idx / kD, j = idx - (idx / kD) * kD;
        part[r * (kD + 2) + j] = ((so[0][r][j] + so[1][r][j]) + so[2][r][j]) + so[3][r][j];
    }
    if (threadIdx.x < R) {
        part[threadIdx.x * (kD + 2) + kD] = sm[threadIdx.x];
        part[threadIdx.x * (kD + 2) + kD + 1] = sl[threadIdx.x];
    }
}

constexpr int kCombineGroups = 4;
constexpr int kKvMaxSplits = 512;

// One workgroup (4 groups of 128 threads, one thread per dimension) per
// output row (token i, query head hq), merging the splits of its KV head.
__global__ __launch_bounds__(kD * kCombineGroups) void kv_attn_combine_kernel(const KvArgs a, int splits) {
    __shared__ float cm[kKvMaxSplits], cl[kKvMaxSplits], cw[kKvMaxSplits];
    __shared__ float cmax[kCombineGroups * kD / 64];
    __shared__ float cnum[kCombineGroups][kD], cden[kCombineGroups];
    const int row = blockIdx.x;                       // i Hq + hq
    const int i = row / a.Hq, hq = row - (row / a.Hq) * a.Hq;
    const int G = a.Hq / a.Hkv;
    const int h = hq / G, g = hq - (hq / G) * G;
    const int R = a.M * G;
    const int r = i * G + g;
    const float *base = a.work + static_cast<size_t>(h) * splits * R * (kD + 2) + static_cast<size_t>(r) * (kD + 2);
    const size_t stride = static_cast<size_t>(R) * (kD + 2);
    constexpr int nthreads = kD * kCombineGroups;

    float mx = -__builtin_inff();
    for (int s = threadIdx.x; s < splits; s += nthreads) {
        const float m = base[s * stride + kD];
        cm[s] = m;
        cl[s] = base[s * stride + kD + 1];
        mx = fmaxf(mx, m);
    }
    mx = wave_max_dpp_f32(mx);
    if ((threadIdx.x & 63) == 0) cmax[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = cmax[0];
#pragma unroll
    for (int w = 1; w < nthreads / 64; ++w) mx = fmaxf(mx, cmax[w]);
    for (int s = threadIdx.x; s < splits; s += nthreads) cw[s] = cl[s] > 0.0f ? expf(cm[s] - mx) : 0.0f;
    __syncthreads();

    const int grp = threadIdx.x / kD, j = threadIdx.x - grp * kD;
    float num = 0.0f, den = 0.0f;
#pragma unroll 8
    for (int s = grp; s < splits; s += kCombineGroups) {
        const float w = cw[s];
        num = fmaf(base[s * stride + j], w, num);
        den = fmaf(cl[s], w, den);
    }
    cnum[grp][j] = num;
    if (j == 0) cden[grp] = den;
    __syncthreads();
    if (grp == 0) {
        const float n = ((cnum[0][j] + cnum[1][j]) + cnum[2][j]) + cnum[3][j];
        const float d = ((cden[0] + cden[1]) + cden[2]) + cden[3];
        a.out[static_cast<size_t>(row) * kD + j] = n / d;
    }
}

typedef void (*KvSplit)(const KvArgs, int);

template <int RW>
KvSplit pick_kv(bool kv8) {
    return kv8 ? kv_attn_split_kernel<RW, true> : kv_attn_split_kernel<RW, false>;
}

int kv_max_splits(int T) {
    const int nchunks = (T + kC - 1) / kC;
    return nchunks < kKvMaxSplits ? nchunks : kKvMaxSplits;
}

}  // namespace

size_t kv_attention_workspace_bytes(int M, int Hq, int T) {
    return static_cast<size_t>(kv_max_splits(T)) * static_cast<size_t>(M) * Hq * (kD + 2) * sizeof(float);
}

hipError_t launch_kv_attention(const KvArgs &a, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    const int R = a.M * G;
    const int RW = (R + 3) / 4;
    const bool kv8 = a.k_lo != nullptr;
    KvSplit k;
    switch (RW) {
        case 1: k = pick_kv<1>(kv8); break;
        case 2: k = pick_kv<2>(kv8); break;
        case 3: k = pick_kv<3>(kv8); break;
        case 4: k = pick_kv<4>(kv8); break;
        default: return hipErrorInvalidValue;       // rejected by the ABI before this point
    }
    DeviceInfo dev;
    hipError_t e = device_info(&dev);
    if (e != hipSuccess) return e;
    // about two workgroups per compute unit over the KV heads, each split a
    // run of cps chunks (no split empty)
    const int nchunks = (a.T + kC - 1) / kC;
    int want = (2 * dev.cus + a.Hkv - 1) / a.Hkv;
    if (want > kv_max_splits(a.T)) want = kv_max_splits(a.T);
    if (want < 1) want = 1;
    const int cps = (nchunks + want - 1) / want;
    const int splits = (nchunks + cps - 1) / cps;
    hipLaunchKernelGGL(k, dim3(splits, a.Hkv), dim3(kKvThreads), 0, stream, a, cps);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kv_attn_combine_kernel, dim3(a.M * a.Hq), dim3(kD * kCombineGroups), 0, stream, a, splits);
    return hipGetLastError();
}

}  // namespace bitnest
