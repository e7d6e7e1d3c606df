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
//    (<= 16) query rows of that head; a split is a contiguous run of
//    64-position chunks, their number sized to about two workgroups per
//    compute unit. Each wave walks every fourth 16-position tile of the
//    split on its own (the next tile's loads in flight while the current one
//    is consumed): scores and P.V on the fp16 matrix cores, a running
//    softmax per query row. The four waves then merge in LDS in a fixed
//    order and the split's (output, maximum, sum) per row go to the caller's
//    workspace.
//  - kv_attn_combine_kernel: one workgroup per query row merges the splits:
//    out = sum_s o_s e^(m_s - m) / sum_s l_s e^(m_s - m), the splits' weights
//    staged in LDS and the partial loads spread over four thread groups.
#include "bitnest_internal.h"
#include "device_common.h"

namespace bitnest {
namespace {

constexpr int kD = kKvHeadDim;       // 128
constexpr int kC = kKvChunk;         // 64 positions: one step of the four waves
constexpr int kTile = 16;            // positions per wave step
constexpr int kRows = kKvMaxRows;    // 16 query rows: one matrix-core tile
constexpr int kKvThreads = 256;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr unsigned kF16Base = 0x64006400u;      // fp16 1024.0 in both halves

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0), static_cast<int>(bytes),
                                             0x00020000);
}

// Two fp16 halves 1024 + b (b a small integer) -> b - off, exact.
__device__ __forceinline__ unsigned f16_unbias(unsigned bits, float off) {
    const f16x2 o = {static_cast<_Float16>(-off), static_cast<_Float16>(-off)};
    return __builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2, bits) + o);
}

// (x0, x1) -> three fp16 pairs p1 + p2 + p3: each piece rounds toward zero
// and the remainders are exact in fp32, so the pieces carry 33 bits of
// |x| < 2^15 (below 2^-24 the last piece floors at the fp16 subnormals).
__device__ __forceinline__ void split3(float x0, float x1, unsigned &p1, unsigned &p2, unsigned &p3) {
    const auto a = __builtin_amdgcn_cvt_pkrtz(x0, x1);
    const float r0 = x0 - static_cast<float>(a[0]), r1 = x1 - static_cast<float>(a[1]);
    const auto b = __builtin_amdgcn_cvt_pkrtz(r0, r1);
    const float s0 = r0 - static_cast<float>(b[0]), s1 = r1 - static_cast<float>(b[1]);
    const auto c = __builtin_amdgcn_cvt_pkrtz(s0, s1);
    p1 = __builtin_bit_cast(unsigned, a);
    p2 = __builtin_bit_cast(unsigned, b);
    p3 = __builtin_bit_cast(unsigned, c);
}

// Maximum / sum over the four lanes c, c + 16, c + 32, c + 48 (the same in
// all four, the sum in one fixed order).
__device__ __forceinline__ float quad_group_max(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    v = fmaxf(__builtin_bit_cast(float, static_cast<unsigned>(r[0])), __builtin_bit_cast(float, static_cast<unsigned>(r[1])));
    const unsigned w = __builtin_bit_cast(unsigned, v);
    const auto t = __builtin_amdgcn_permlane16_swap(w, w, false, false);
    return fmaxf(__builtin_bit_cast(float, static_cast<unsigned>(t[0])), __builtin_bit_cast(float, static_cast<unsigned>(t[1])));
}
__device__ __forceinline__ float quad_group_sum(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    v = __builtin_bit_cast(float, static_cast<unsigned>(r[0])) + __builtin_bit_cast(float, static_cast<unsigned>(r[1]));
    const unsigned w = __builtin_bit_cast(unsigned, v);
    const auto t = __builtin_amdgcn_permlane16_swap(w, w, false, false);
    return __builtin_bit_cast(float, static_cast<unsigned>(t[0])) + __builtin_bit_cast(float, static_cast<unsigned>(t[1]));
}

// Both products on the fp16 matrix cores, every code exact in fp16 and the
// fp32 operands (q, p v_scale) split into three fp16 pieces after a power-of-
// two scaling, so the products are those of fp32 values to about 2^-32.
//
// Lanes: c = lane % 16, g = lane / 16. Per 16-position tile of a wave:
//  - scores S^T = K Q^T (v_mfma_f32_16x16x32_f16, 4 steps of 32 dimensions):
//    A = K codes, lane = position c, dimensions 32 g + 8 s + {j, j + 4} in
//    pair j of step s (one 16-byte load per plane); B = q pieces, lane =
//    query row c, the same dimensions. The accumulator gives lane (c, g) the
//    scores of query row c at positions 4 g + i.
//  - softmax per query row over the tile (the four lanes of a row combine
//    with lane swaps), running maximum and sum per row.
//  - P.V as O^T = V^T P^T (v_mfma_f32_16x16x16f16 per 16-dimension tile t):
//    B = the score accumulator's own layout (lane = query row c, k =
//    positions 4 g + i), A = V codes, lane = dimension 8 c + t at positions
//    4 g + i (dword c of four position rows). The accumulator gives lane
//    (c, g) the outputs of query row c at dimensions 32 g + 8 i + t.
// Codes: KV4 u - 8, KV8 16 (u_hi - 8) + (u_lo - 8), both from fp16 1024 + code
// bits and one packed subtraction. The KV8 codes with lo = 8 are 16 times the
// KV4 codes and every scale factor differs by a power of two, so the two
// paths then agree bit for bit.
template <bool KV8>
__global__ __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(2))) void kv_attn_split_kernel(const KvArgs a, int cps) {
    __shared__ float sO[4][kRows][kD];
    __shared__ float sM[4][kRows], sL[4][kRows], sW[4][kRows];
    __shared__ float4 ssc[4][2][kTile / 4];          // per wave: K and V scales of its tile

    const int s = blockIdx.x, h = blockIdx.y;
    const int splits = gridDim.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int G = a.Hq / a.Hkv;
    const int R = a.M * G;
    const int span0 = s * cps * kC;
    const int span1 = min(a.T, span0 + cps * kC);

    // query row c: token c / G, head h G + c % G; last visible position
    const bool rv = c < R;
    const int tok = rv ? c / G : 0;
    const int limit = rv ? a.T - a.M + tok : -1;

    // tile loads: this lane's K row (position c, bytes 16 g ..), its V dwords
    // (dword c of positions 4 g + i) and the K / V scales of position c
    const unsigned cache_bytes = static_cast<unsigned>(a.T) * a.Hkv * (kD / 2);
    const unsigned scale_bytes = static_cast<unsigned>(a.T) * a.Hkv * 2;
    const __amdgpu_buffer_rsrc_t rkh = rsrc(a.k_hi, cache_bytes), rvh = rsrc(a.v_hi, cache_bytes);
    const __amdgpu_buffer_rsrc_t rkl = rsrc(KV8 ? a.k_lo : a.k_hi, cache_bytes);
    const __amdgpu_buffer_rsrc_t rvl = rsrc(KV8 ? a.v_lo : a.v_hi, cache_bytes);
    const __amdgpu_buffer_rsrc_t rks = rsrc(a.k_scale, scale_bytes), rvs = rsrc(a.v_scale, scale_bytes);
    struct Stage {
        u32x4 kh, kl;
        unsigned vh[4], vl[4];
        unsigned short ks, vs;
    };
    // every load is issued (past the split: an offset past the end, which
    // reads zero and touches no memory), so the waits count exactly
    auto fetch = [&](Stage &st, int p0) {
        const int tk = p0 + c;
        const unsigned ok = tk < span1 ? (static_cast<unsigned>(tk) * a.Hkv + h) * (kD / 2) + 16 * g : cache_bytes;
        st.kh = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rkh, ok, 0, 0));
        if (KV8) st.kl = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rkl, ok, 0, 0));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tv = p0 + 4 * g + i;
            const unsigned ov = tv < span1 ? (static_cast<unsigned>(tv) * a.Hkv + h) * (kD / 2) + 4 * c : cache_bytes;
            st.vh[i] = __builtin_amdgcn_raw_buffer_load_b32(rvh, ov, 0, 0);
            if (KV8) st.vl[i] = __builtin_amdgcn_raw_buffer_load_b32(rvl, ov, 0, 0);
        }
        const unsigned os = tk < span1 ? (static_cast<unsigned>(tk) * a.Hkv + h) * 2 : scale_bytes;
        st.ks = __builtin_amdgcn_raw_buffer_load_b16(rks, os, 0, 0);
        st.vs = __builtin_amdgcn_raw_buffer_load_b16(rvs, os, 0, 0);
    };
    // q row c (rows past R read row 0 and are zeroed), loaded before the
    // tiles so that waiting for it leaves the tile loads in flight
    float x[32];
    {
        const int qr = rv ? c : 0;
        const float4 *src = reinterpret_cast<const float4 *>(
            a.q + (static_cast<size_t>(qr / G) * a.Hq + h * G + qr % G) * kD + 32 * g);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float4 v = src[k];
            x[4 * k] = rv ? v.x : 0.0f; x[4 * k + 1] = rv ? v.y : 0.0f;
            x[4 * k + 2] = rv ? v.z : 0.0f; x[4 * k + 3] = rv ? v.w : 0.0f;
        }
    }
    // a ring of two tiles in flight while one is consumed
    Stage s0, s1;
    if (!KV8) s0.kl = s1.kl = u32x4{0, 0, 0, 0};
    int p0 = span0 + kTile * wave;
    fetch(s0, p0);
    fetch(s1, p0 + kC);

    // q row c scaled by 2^kq (its largest |q| in [2^14, 2^15)), three fp16
    // pieces per step s and pair j (dimensions 32 g + 8 s + j, + j + 4)
    unsigned qb[3][4][4];
    float gscale;                                    // 2^-kq / sqrt(128) (/ 16: KV8 codes)
    {
        float mx = 0.0f;
#pragma unroll
        for (int k = 0; k < 32; ++k) mx = fmaxf(mx, fabsf(x[k]));
        mx = quad_group_max(mx);
        const int kq = mx > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                split3(__builtin_amdgcn_ldexpf(x[8 * st + j], kq), __builtin_amdgcn_ldexpf(x[8 * st + j + 4], kq),
                       qb[0][st][j], qb[1][st][j], qb[2][st][j]);
        gscale = __builtin_amdgcn_ldexpf(a.inv_sqrt_d, -kq) * (KV8 ? 0.0625f : 1.0f);
    }

    float m_run = -__builtin_inff(), l_run = 0.0f;
    int kt_run = 0;                                  // the accumulators hold O 2^kt_run
    f32x4 o[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto consume = [&](const Stage &cur, int p0) {
        const u32x4 ckh = cur.kh, ckl = cur.kl;
        const unsigned *cvh = cur.vh, *cvl = cur.vl;
        const unsigned short cks = cur.ks, cvs = cur.vs;

        // scales of positions 4 g + i through the wave's LDS slot
        reinterpret_cast<float *>(ssc[wave][0])[c] = half_bits_to_float(cks);
        reinterpret_cast<float *>(ssc[wave][1])[c] = half_bits_to_float(cvs);
        const float4 ksv = ssc[wave][0][g];
        const float4 vsv = ssc[wave][1][g];

        // ---- scores
        f16x8 ka[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            unsigned pr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (KV8) {
                    // byte of each half: 16 u_hi + u_lo of dimensions j, j + 4
                    const unsigned lo = ((ckl[st] >> (4 * j)) & 0x000F000Fu) | kF16Base;
                    const unsigned hi = j == 0 ? (ckh[st] << 4) : (ckh[st] >> (4 * j - 4));
                    pr[j] = f16_unbias((hi & 0x00F000F0u) | lo, 1024.0f + 136.0f);
                } else {
                    pr[j] = f16_unbias(((ckh[st] >> (4 * j)) & 0x000F000Fu) | kF16Base, 1024.0f + 8.0f);
                }
            }
            ka[st] = __builtin_bit_cast(f16x8, u32x4{pr[0], pr[1], pr[2], pr[3]});
        }
        f32x4 d[3];
#pragma unroll
        for (int pc = 0; pc < 3; ++pc) {
            d[pc] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < 4; ++st)
                d[pc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    ka[st], __builtin_bit_cast(f16x8, u32x4{qb[pc][st][0], qb[pc][st][1], qb[pc][st][2], qb[pc][st][3]}),
                    d[pc], 0, 0, 0);
        }

        // ---- running softmax of query row c over the tile
        const float ks4[4] = {ksv.x, ksv.y, ksv.z, ksv.w};
        const float vs4[4] = {vsv.x, vsv.y, vsv.z, vsv.w};
        float sc[4];
        float tmax = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool vis = p0 + 4 * g + i <= limit;
            const float dot = (d[2][i] + d[1][i]) + d[0][i];
            sc[i] = vis ? dot * (ks4[i] * gscale) : -__builtin_inff();
            tmax = fmaxf(tmax, sc[i]);
        }
        const float m_new = fmaxf(m_run, quad_group_max(tmax));
        const float alpha = m_run == -__builtin_inff() ? 0.0f : expf(m_run - m_new);
        float pv[4], psum = 0.0f, pmax = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = sc[i] == -__builtin_inff() ? 0.0f : expf(sc[i] - m_new);
            psum += p;
            pv[i] = p * vs4[i];
            pmax = fmaxf(pmax, fabsf(pv[i]));
        }
        l_run = fmaf(l_run, alpha, quad_group_sum(psum));
        m_run = m_new;
        // p v_scale of the row scaled into [2^14, 2^15) and split into pieces;
        // the accumulators follow the row's scale
        pmax = quad_group_max(pmax);
        const int kt = pmax > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(pmax) : kt_run;
        const float f = __builtin_amdgcn_ldexpf(alpha, kt - kt_run);
        kt_run = kt;
#pragma unroll
        for (int t = 0; t < 8; ++t) o[t] *= f;
        unsigned pb[3][2];
        split3(__builtin_amdgcn_ldexpf(pv[0], kt), __builtin_amdgcn_ldexpf(pv[1], kt), pb[0][0], pb[1][0], pb[2][0]);
        split3(__builtin_amdgcn_ldexpf(pv[2], kt), __builtin_amdgcn_ldexpf(pv[3], kt), pb[0][1], pb[1][1], pb[2][1]);

        // ---- P.V: V codes of dimension 8 c + t at positions 4 g + i
        unsigned ve[4], vo[4];                          // codes of even / odd nibbles as bytes (KV8: full codes)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (KV8) {
                ve[i] = ((cvh[i] & 0x0F0F0F0Fu) << 4) | (cvl[i] & 0x0F0F0F0Fu);
                vo[i] = (cvh[i] & 0xF0F0F0F0u) | ((cvl[i] >> 4) & 0x0F0F0F0Fu);
            } else {
                ve[i] = cvh[i] & 0x0F0F0F0Fu;
                vo[i] = (cvh[i] >> 4) & 0x0F0F0F0Fu;
            }
        }
        f16x4 va[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            // byte t / 2 of positions (0, 1) and (2, 3) into the low bytes of the halves
            const unsigned sel = 0x0C000C00u | ((4u + t / 2) << 16) | static_cast<unsigned>(t / 2);
            const unsigned *src = (t & 1) ? vo : ve;
            const unsigned b01 = __builtin_amdgcn_perm(src[1], src[0], sel) | kF16Base;
            const unsigned b23 = __builtin_amdgcn_perm(src[3], src[2], sel) | kF16Base;
            const float off = 1024.0f + (KV8 ? 136.0f : 8.0f);
            va[t] = __builtin_bit_cast(f16x4, u32x2{f16_unbias(b01, off), f16_unbias(b23, off)});
        }
#pragma unroll
        for (int pc = 2; pc >= 0; --pc) {
            const f16x4 bp = __builtin_bit_cast(f16x4, u32x2{pb[pc][0], pb[pc][1]});
#pragma unroll
            for (int t = 0; t < 8; ++t) o[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(va[t], bp, o[t], 0, 0, 0);
        }
    };
#pragma unroll 1
    for (; p0 < span1; p0 += 2 * kC) {
        {
            const Stage cur = s0;
            fetch(s0, p0 + 2 * kC);
            consume(cur, p0);
        }
        if (p0 + kC >= span1) break;                 // uniform
        {
            const Stage cur = s1;
            fetch(s1, p0 + 3 * kC);
            consume(cur, p0 + kC);
        }
    }

    // ---- the four waves' (maximum, sum, output) merged in a fixed order
    const float unscale = __builtin_amdgcn_ldexpf(KV8 ? 0.0625f : 1.0f, -kt_run);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float4 *dst = reinterpret_cast<float4 *>(&sO[wave][c][32 * g + 8 * i]);
        dst[0] = float4{o[0][i] * unscale, o[1][i] * unscale, o[2][i] * unscale, o[3][i] * unscale};
        dst[1] = float4{o[4][i] * unscale, o[5][i] * unscale, o[6][i] * unscale, o[7][i] * unscale};
    }
    if (g == 0) {
        sM[wave][c] = m_run;
        sL[wave][c] = l_run;
    }
    __syncthreads();
    if (threadIdx.x < kRows) {
        const int r = threadIdx.x;
        float mx = sM[0][r];
#pragma unroll
        for (int w = 1; w < 4; ++w) mx = fmaxf(mx, sM[w][r]);
#pragma unroll
        for (int w = 0; w < 4; ++w) sW[w][r] = sM[w][r] == -__builtin_inff() ? 0.0f : expf(sM[w][r] - mx);
        sM[0][r] = mx;
        sL[0][r] = ((sL[0][r] * sW[0][r] + sL[1][r] * sW[1][r]) + sL[2][r] * sW[2][r]) + sL[3][r] * sW[3][r];
    }
    __syncthreads();
    float *part = a.work + (static_cast<size_t>(h) * splits + s) * R * (kD + 2);
    for (int idx = threadIdx.x; idx < R * kD; idx += kKvThreads) {
        const int r = idx / kD, j = idx - (idx / kD) * kD;
        part[r * (kD + 2) + j] = ((sO[0][r][j] * sW[0][r] + sO[1][r][j] * sW[1][r]) + sO[2][r][j] * sW[2][r]) +
                                 sO[3][r][j] * sW[3][r];
    }
    if (threadIdx.x < R) {
        part[threadIdx.x * (kD + 2) + kD] = sM[0][threadIdx.x];
        part[threadIdx.x * (kD + 2) + kD + 1] = sL[0][threadIdx.x];
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

int kv_max_splits(int T) {
    const int nchunks = (T + kC - 1) / kC;
    return nchunks < kKvMaxSplits ? nchunks : kKvMaxSplits;
}

}  // namespace

size_t kv_attention_workspace_bytes(int M, int Hq, int T) {
    return static_cast<size_t>(kv_max_splits(T)) * static_cast<size_t>(M) * Hq * (kD + 2) * sizeof(float);
}

hipError_t launch_kv_attention(const KvArgs &a, hipStream_t stream) {
    if (a.M * (a.Hq / a.Hkv) > kRows) return hipErrorInvalidValue;   // rejected by the ABI before this point
    const KvSplit k = a.k_lo != nullptr ? kv_attn_split_kernel<true> : kv_attn_split_kernel<false>;
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
