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
//  - kv_attn_split_kernel: one workgroup per (64-position chunk, KV head),
//    for all M x G query rows of that head. The chunk's K and V rows are
//    staged in LDS first (one 16-byte load per thread and plane, all in
//    flight together). Scores with one lane per
//    position (the row's K planes in registers, the query rows broadcast from
//    LDS, unsigned nibble codes with the offset applied once per score
//    through the row's sum of q); a softmax inside the chunk (DPP maximum
//    and sum per row); P.V with one lane per two dimensions and each wave on
//    16 positions, summed over the waves in a fixed order. The chunk's
//    (output, maximum, sum) per row go to the caller's workspace.
//  - kv_attn_combine_kernel: one workgroup per query row merges the chunks
//    in order: out = sum_s o_s e^(m_s - m) / sum_s l_s e^(m_s - m).
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

// RW: query rows per wave (the M x G rows padded to 4 RW). KV8: read the lo planes.
template <int RW, bool KV8>
__global__ __launch_bounds__(kKvThreads) void kv_attn_split_kernel(const KvArgs a) {
    constexpr int RP = 4 * RW;
    __shared__ float sq[RP][kD];
    __shared__ float sqs[RP];
    __shared__ float sp[kC][RP];
    __shared__ float sm[RP], sl[RP];
    __shared__ float so[4][RP][kD];
    // the chunk's planes: [plane][position][16-byte piece], planes K hi, K lo, V hi, V lo
    __shared__ u32x4 sk[KV8 ? 4 : 2][kC][4];
    __shared__ float sks[kC], svs[kC];

    const int s = blockIdx.x, h = blockIdx.y;
    const int S = gridDim.x;
    const int t0 = s * kC;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = a.Hq / a.Hkv;
    const int R = a.M * G;

    // stage the chunk's cache rows (one 16-byte piece per thread and plane,
    // all in flight together; positions past T read as zero) and scales
    {
        const unsigned cache_bytes = static_cast<unsigned>(a.T) * a.Hkv * (kD / 2);
        const int pos = threadIdx.x >> 2, piece = threadIdx.x & 3;
        const int off = ((t0 + pos) * a.Hkv + h) * (kD / 2) + 16 * piece;
        const uint8_t *src[4] = {a.k_hi, a.v_hi, a.k_lo, a.v_lo};
        u32x4 v[KV8 ? 4 : 2];
#pragma unroll
        for (int pl = 0; pl < (KV8 ? 4 : 2); ++pl)
            v[pl] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc(src[pl], cache_bytes), off, 0, 0));
        float ks = 0.0f, vs = 0.0f;
        if (threadIdx.x < kC && t0 + threadIdx.x < a.T) {
            ks = half_bits_to_float(a.k_scale[(t0 + threadIdx.x) * a.Hkv + h]);
            vs = half_bits_to_float(a.v_scale[(t0 + threadIdx.x) * a.Hkv + h]);
        }
        sk[0][pos][piece] = v[0];                      // K hi
        sk[1][pos][piece] = v[1];                      // V hi
        if (KV8) {
            sk[2][pos][piece] = v[2];                  // K lo
            sk[3][pos][piece] = v[3];                  // V lo
        }
        if (threadIdx.x < kC) {
            sks[threadIdx.x] = ks;
            svs[threadIdx.x] = vs;
        }
    }
    // query rows r = i G + g (token i, query head h G + g), and their sums
    for (int idx = threadIdx.x; idx < RP * kD; idx += kKvThreads) {
        const int r = idx / kD, j = idx - (idx / kD) * kD;
        float v = 0.0f;
        if (r < R) {
            const int i = r / G, g = r - (r / G) * G;
            v = a.q[(static_cast<size_t>(i) * a.Hq + h * G + g) * kD + j];
        }
        sq[r][j] = v;
    }
    __syncthreads();
    if (threadIdx.x < RP) {
        float sum = 0.0f;
        for (int j = 0; j < kD; ++j) sum += sq[threadIdx.x][j];
        sqs[threadIdx.x] = sum;
    }

    // ---- scores: lane = position t0 + lane, wave = rows [RW wave, RW wave + RW)
    const int t = t0 + lane;
    const bool tv = t < a.T;
    __syncthreads();                                   // sqs ready
    const float kscale = sks[lane];

    // acc: sum u_hi q; accl (KV8): sum u_lo q, accumulated like the row sum
    // of q (j ascending), so that lo = 8 makes it exactly 8 sum(q)
    float acc[RW], accl[RW];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) acc[rr] = accl[rr] = 0.0f;
    // 16 bytes of each plane (32 columns) per step; a rolled loop keeps the
    // broadcast query reads of one step live at a time
#pragma unroll 1
    for (int c = 0; c < 4; ++c) {
        const u32x4 kh = sk[0][lane][c];
        const u32x4 kl = KV8 ? sk[2][lane][c] : kh;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // dword w: columns 32 c + 8 w + 0 .. 7 (low nibble = even column)
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
            const int j0 = 32 * c + 8 * w;
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
    // with lo = 8 the second term is exactly 0 and the power-of-two factors
    // cancel exactly, so KV8 then equals KV4 bit for bit
    const float sfac = kscale * a.inv_sqrt_d;
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
        const int r = wave * RW + rr;
        const int i = r / G;
        const bool vis = tv && r < R && t <= a.T - a.M + i;
        float dot = acc[rr] - 8.0f * sqs[r];
        if (KV8) dot = 16.0f * dot + (accl[rr] - 8.0f * sqs[r]);
        const float sc = vis ? dot * (KV8 ? sfac * 0.0625f : sfac) : -__builtin_inff();
        float m = wave_max_dpp_f32(sc);
        float p = 0.0f;
        if (m != -__builtin_inff()) p = vis ? expf(sc - m) : 0.0f;
        const float l = wave_sum_f32(p);
        sp[lane][r] = p;
        if (lane == 0) {
            sm[r] = m;
            sl[r] = l;
        }
    }
    __syncthreads();

    // ---- P.V: wave = positions t0 + 16 wave + k, lane = dimensions 2 lane, 2 lane + 1
    float o0[RP], o1[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) o0[r] = o1[r] = 0.0f;
    // (a rolled loop: unrolled, the compiler hoists every position's loads
    // and runs out of registers)
#pragma unroll 1
    for (int k = 0; k < kC / 4; ++k) {
        const int pl = (kC / 4) * wave + k;
        const int tt = t0 + pl;
        if (tt >= a.T) break;                          // uniform
        const float vs = svs[pl];
        const unsigned vb = reinterpret_cast<const uint8_t *>(&sk[1][pl][0])[lane];
        float v0, v1;
        if (KV8) {
            const unsigned lb = reinterpret_cast<const uint8_t *>(&sk[3][pl][0])[lane];
            v0 = static_cast<float>(16 * (static_cast<int>(vb & 15u) - 8) + (static_cast<int>(lb & 15u) - 8)) *
                 (vs * 0.0625f);
            v1 = static_cast<float>(16 * (static_cast<int>(vb >> 4) - 8) + (static_cast<int>(lb >> 4) - 8)) *
                 (vs * 0.0625f);
        } else {
            v0 = static_cast<float>(static_cast<int>(vb & 15u) - 8) * vs;
            v1 = static_cast<float>(static_cast<int>(vb >> 4) - 8) * vs;
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
#pragma unroll
    for (int r = 0; r < RP; ++r) {
        so[wave][r][2 * lane] = o0[r];
        so[wave][r][2 * lane + 1] = o1[r];
    }
    __syncthreads();
    float *part = a.work + (static_cast<size_t>(h) * S + s) * R * (kD + 2);
    for (int idx = threadIdx.x; idx < R * kD; idx += kKvThreads) {
        const int r = idx / kD, j = idx - (idx / kD) * kD;
        part[r * (kD + 2) + j] = ((so[0][r][j] + so[1][r][j]) + so[2][r][j]) + so[3][r][j];
    }
    if (threadIdx.x < R) {
        part[threadIdx.x * (kD + 2) + kD] = sm[threadIdx.x];
        part[threadIdx.x * (kD + 2) + kD + 1] = sl[threadIdx.x];
    }
}

// One workgroup (128 threads, one per dimension) per output row (token i,
// query head hq), merging the S chunk partials of its KV head in order.
__global__ __launch_bounds__(kD) void kv_attn_combine_kernel(const KvArgs a, int S) {
    const int row = blockIdx.x;                       // i Hq + hq
    const int i = row / a.Hq, hq = row - (row / a.Hq) * a.Hq;
    const int G = a.Hq / a.Hkv;
    const int h = hq / G, g = hq - (hq / G) * G;
    const int R = a.M * G;
    const int r = i * G + g;
    const int j = threadIdx.x;
    const float *base = a.work + static_cast<size_t>(h) * S * R * (kD + 2) + static_cast<size_t>(r) * (kD + 2);
    const size_t stride = static_cast<size_t>(R) * (kD + 2);
    float mx = -__builtin_inff();
    for (int s = 0; s < S; ++s) mx = fmaxf(mx, base[s * stride + kD]);
    float num = 0.0f, den = 0.0f;
    for (int s = 0; s < S; ++s) {
        const float *p = base + s * stride;
        const float l = p[kD + 1];
        if (l > 0.0f) {
            const float w = expf(p[kD] - mx);
            num = fmaf(p[j], w, num);
            den = fmaf(l, w, den);
        }
    }
    a.out[static_cast<size_t>(row) * kD + j] = num / den;
}

typedef void (*KvSplit)(const KvArgs);

template <int RW>
KvSplit pick_kv(bool kv8) {
    return kv8 ? kv_attn_split_kernel<RW, true> : kv_attn_split_kernel<RW, false>;
}

}  // namespace

size_t kv_attention_workspace_bytes(int M, int Hq, int T) {
    const size_t S = (static_cast<size_t>(T) + kC - 1) / kC;
    return S * static_cast<size_t>(M) * Hq * (kD + 2) * sizeof(float);
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
    const int S = (a.T + kC - 1) / kC;
    hipLaunchKernelGGL(k, dim3(S, a.Hkv), dim3(kKvThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kv_attn_combine_kernel, dim3(a.M * a.Hq), dim3(kD), 0, stream, a, S);
    return hipGetLastError();
}

}  // namespace bitnest
