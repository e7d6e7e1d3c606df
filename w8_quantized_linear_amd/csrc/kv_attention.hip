// Decode attention over the nested KV cache (model card "BitNest-Llama-3-8B",
// recipe table row "KV cache": nested at runtime, the draft reads KV4 and
// the target KV8; abstract: the progressive-precision design extends to the
// KV cache for long contexts). The reading, written out in bitnest.h: every
// (token, KV head) vector of 128 values is packed like one 128-column weight
// group, head-major (planes [Hkv, t_cap, 64], fp16 scales [Hkv, t_cap], the
// first T positions of each head valid); KV4 = (hi - 8) s,
// KV8 = (16 (hi - 8) + (lo - 8)) s / 16; grouped-query heads; the M query
// tokens are the last M positions (token i sees t <= T - M + i).
//
// Split over the sequence (the draft reads only the hi planes, the target
// both; both are HBM streams of a few bytes per position and head):
//  - kv_attn_split_kernel: one workgroup per (split, KV head), for all M x G
//    (<= 16) query rows of that head; a split is a contiguous run of
//    64-position chunks, their number sized to about two workgroups per
//    compute unit. Each wave walks every fourth step of the split on its own
//    (a step is 16 positions, or 32 when a split holds several chunks; the
//    loads of the next one or two steps are in flight while one is
//    consumed): scores and P.V on the fp16 matrix cores, a running softmax
//    per query row. The four waves then merge in LDS in a fixed order and
//    the split's (output, maximum, sum) per row go to the caller's
//    workspace. Scores are kept in base-2 units (log2(e) folded into the
//    scale), so every exponential is one v_exp_f32.
//  - kv_attn_combine_kernel: one workgroup per query row merges the splits:
//    out = sum_s o_s 2^(m_s - m) / sum_s l_s 2^(m_s - m), as four thread
//    groups with running maxima over interleaved splits, then merged.
#include "bitnest_internal.h"
#include "device_common.h"

namespace bitnest {
namespace {

constexpr int kD = kKvHeadDim;       // 128
constexpr int kC = kKvChunk;         // 64 positions: the unit a split is made of
constexpr int kTile = 16;            // positions per score tile (a wave step is NT tiles)
constexpr int kRows = kKvMaxRows;    // 16 query rows: one matrix-core tile
constexpr int kKvThreads = 256;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr unsigned kF16Base = 0x64006400u;      // fp16 1024.0 in both halves
constexpr float kLog2e = 1.44269504088896340736f;

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

// (x0, x1) -> two fp16 pairs p1 + p2: 22 bits of each value (the second
// piece floors at the fp16 subnormals, 2^-24).
__device__ __forceinline__ void split2(float x0, float x1, unsigned &p1, unsigned &p2) {
    const auto a = __builtin_amdgcn_cvt_pkrtz(x0, x1);
    const float r0 = x0 - static_cast<float>(a[0]), r1 = x1 - static_cast<float>(a[1]);
    const auto b = __builtin_amdgcn_cvt_pkrtz(r0, r1);
    p1 = __builtin_bit_cast(unsigned, a);
    p2 = __builtin_bit_cast(unsigned, b);
}

// Both products on the fp16 matrix cores with every code exact in fp16; the
// fp32 operands are scaled by a power of two and split into fp16 pieces:
// q into three (33 bits, the scores to about 2^-32 of the row's largest
// term), p v_scale into two (22 bits of each term).
//
// Lanes: c = lane % 16, g = lane / 16. A wave step covers NT tiles of 16
// positions (u = 0 .. NT - 1):
//  - scores S^T = K Q^T per tile (v_mfma_f32_16x16x32_f16, 4 steps of 32
//    dimensions): A = K codes, lane = position c, dimensions 32 g + 8 s +
//    {j, j + 4} in pair j of step s (one 16-byte load per plane); B = q
//    pieces, lane = query row c, the same dimensions. The accumulator gives
//    lane (c, g) the scores of query row c at positions 16 u + 4 g + i.
//  - softmax per query row over the step (the four lanes of a row combine
//    with lane swaps), running maximum and sum per row.
//  - P.V as O^T = V^T P^T per 16-dimension tile t (k = the step's 16 NT
//    positions: v_mfma_f32_16x16x16f16 for NT = 1, 16x16x32 for NT = 2):
//    B = the score accumulators' own layout (lane = query row c, k-slot
//    4 u + i = position 16 u + 4 g + i), A = V codes, lane = dimension
//    8 c + t at the same positions (dword c of 4 NT position rows). The
//    accumulator gives lane (c, g) the outputs of query row c at dimensions
//    32 g + 8 i + t.
// Codes: KV4 u - 8, KV8 16 (u_hi - 8) + (u_lo - 8), both from fp16 1024 + code
// bits and one packed subtraction. The KV8 codes with lo = 8 are 16 times the
// KV4 codes and every scale factor differs by a power of two, so the two
// paths then agree bit for bit.
template <bool KV8, int NT>
__global__ __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(2)))
void kv_attn_split_kernel(const KvArgs a, int cps) {
    constexpr int STEP = kTile * NT;                 // positions per wave step
    constexpr int WSTEP = 4 * STEP;                  // positions per workgroup step
    constexpr int NP = 4 * NT;                       // positions per lane per step
    typedef _Float16 f16xk __attribute__((ext_vector_type(NP)));
    typedef unsigned u32xk __attribute__((ext_vector_type(NP / 2)));
    __shared__ float sO[4][kRows][kD];
    __shared__ float sM[4][kRows], sL[4][kRows], sW[4][kRows];
    __shared__ float4 ssc[4][2][STEP / 4];           // per wave: K and V scales of its step

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

    // step loads: this lane's K rows (position 16 u + c, bytes 16 g ..), its
    // V dwords (dword c of positions 16 u + 4 g + i) and the K / V scales of
    // positions 16 u + c, all within KV head h's run of positions (the cache
    // is head-major, so a 16-position K load is 1 KiB of contiguous bytes).
    // The descriptors end at the split's last position: rows past it read
    // zero and touch no memory (T 64 < 2^31 keeps every offset below 2^32).
    const size_t head_planes = static_cast<size_t>(h) * a.t_cap * (kD / 2);
    const size_t head_scales = static_cast<size_t>(h) * a.t_cap;
    const unsigned cache_bytes = static_cast<unsigned>(span1) * (kD / 2);
    const unsigned scale_bytes = static_cast<unsigned>(span1) * 2;
    const __amdgpu_buffer_rsrc_t rkh = rsrc(a.k_hi + head_planes, cache_bytes);
    const __amdgpu_buffer_rsrc_t rvh = rsrc(a.v_hi + head_planes, cache_bytes);
    const __amdgpu_buffer_rsrc_t rkl = rsrc((KV8 ? a.k_lo : a.k_hi) + head_planes, cache_bytes);
    const __amdgpu_buffer_rsrc_t rvl = rsrc((KV8 ? a.v_lo : a.v_hi) + head_planes, cache_bytes);
    const __amdgpu_buffer_rsrc_t rks = rsrc(a.k_scale + head_scales, scale_bytes);
    const __amdgpu_buffer_rsrc_t rvs = rsrc(a.v_scale + head_scales, scale_bytes);
    struct Stage {
        u32x4 kh[NT], kl[NT];
        unsigned vh[NP], vl[NP];
        unsigned short ks[NT], vs[NT];
    };
    // every load is issued (past the split they read zero), so the waits
    // count exactly; the offsets advance by one workgroup step per fetch
    const int pf = span0 + STEP * wave;              // the wave's first step
    unsigned ok[NT], ov[NP], os[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        ok[u] = static_cast<unsigned>(pf + 16 * u + c) * (kD / 2) + 16 * g;
        os[u] = static_cast<unsigned>(pf + 16 * u + c) * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ov[4 * u + i] = static_cast<unsigned>(pf + 16 * u + 4 * g + i) * (kD / 2) + 4 * c;
    }
    constexpr unsigned step_planes = static_cast<unsigned>(WSTEP) * (kD / 2);
    constexpr unsigned step_scales = static_cast<unsigned>(WSTEP) * 2;
    auto fetch = [&](Stage &st) {
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            st.kh[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rkh, ok[u], 0, 0));
            if (KV8) st.kl[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rkl, ok[u], 0, 0));
        }
#pragma unroll
        for (int e = 0; e < NP; ++e) {
            st.vh[e] = __builtin_amdgcn_raw_buffer_load_b32(rvh, ov[e], 0, 0);
            if (KV8) st.vl[e] = __builtin_amdgcn_raw_buffer_load_b32(rvl, ov[e], 0, 0);
        }
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            st.ks[u] = __builtin_amdgcn_raw_buffer_load_b16(rks, os[u], 0, 0);
            st.vs[u] = __builtin_amdgcn_raw_buffer_load_b16(rvs, os[u], 0, 0);
            ok[u] += step_planes;
            os[u] += step_scales;
        }
#pragma unroll
        for (int e = 0; e < NP; ++e) ov[e] += step_planes;
    };

    // q row c (rows past R read row 0 and are zeroed), loaded before the
    // steps so that waiting for it leaves the step loads in flight
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
    // a ring of RING steps in flight while one is consumed (one for the
    // 32-position KV8 steps, which fill the registers with two)
    constexpr int RING = (KV8 && NT == 2) ? 1 : 2;
    Stage s0, s1;
#pragma unroll
    for (int u = 0; u < NT; ++u) s0.kl[u] = s1.kl[u] = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < NP; ++e) s0.vl[e] = s1.vl[e] = 0;
    int p0 = pf;
    fetch(s0);
    if (RING == 2) fetch(s1);

    // q row c scaled by 2^kq (its largest |q| in [2^14, 2^15)), three fp16
    // pieces per step s and pair j (dimensions 32 g + 8 s + j, + j + 4)
    unsigned qb[3][4][4];
    float gscale;                                    // 2^-kq log2(e) / sqrt(128) (/ 16: KV8 codes)
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
        gscale = __builtin_amdgcn_ldexpf(a.inv_sqrt_d * kLog2e, -kq) * (KV8 ? 0.0625f : 1.0f);
    }

    float m_run = -__builtin_inff(), l_run = 0.0f;
    int kt_run = 0;                                  // the accumulators hold O 2^kt_run
    f32x4 o[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // consume one step from its stage: the codes and scales are converted
    // first, so the stage can take the loads of the step RING ahead
    auto consume = [&](Stage &cur, int p0) {
        // scales of positions 16 u + 4 g + i through the wave's LDS slot
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            reinterpret_cast<float *>(ssc[wave][0])[16 * u + c] = half_bits_to_float(cur.ks[u]);
            reinterpret_cast<float *>(ssc[wave][1])[16 * u + c] = half_bits_to_float(cur.vs[u]);
        }
        float ks[NP], vs[NP];
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            const float4 kv = ssc[wave][0][4 * u + g], vv = ssc[wave][1][4 * u + g];
            ks[4 * u] = kv.x; ks[4 * u + 1] = kv.y; ks[4 * u + 2] = kv.z; ks[4 * u + 3] = kv.w;
            vs[4 * u] = vv.x; vs[4 * u + 1] = vv.y; vs[4 * u + 2] = vv.z; vs[4 * u + 3] = vv.w;
        }

        // K codes (the A operands of the scores)
        f16x8 ka[NT][4];
#pragma unroll
        for (int u = 0; u < NT; ++u)
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const unsigned wh = cur.kh[u][st], wl = cur.kl[u][st];
                unsigned pr[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (KV8) {
                        // byte of each half: 16 u_hi + u_lo of dimensions j, j + 4
                        const unsigned lo = ((wl >> (4 * j)) & 0x000F000Fu) | kF16Base;
                        const unsigned hi = j == 0 ? (wh << 4) : (wh >> (4 * j - 4));
                        pr[j] = f16_unbias((hi & 0x00F000F0u) | lo, 1024.0f + 136.0f);
                    } else {
                        pr[j] = f16_unbias(((wh >> (4 * j)) & 0x000F000Fu) | kF16Base, 1024.0f + 8.0f);
                    }
                }
                ka[u][st] = __builtin_bit_cast(f16x8, u32x4{pr[0], pr[1], pr[2], pr[3]});
            }
        // V codes of dimension 8 c + t at positions 16 u + 4 g + i (the A
        // operands of P.V, k-slot 4 u + i)
        unsigned ve[NP], vo[NP];                     // codes of even / odd nibbles as bytes (KV8: full codes)
#pragma unroll
        for (int e = 0; e < NP; ++e) {
            if (KV8) {
                ve[e] = ((cur.vh[e] & 0x0F0F0F0Fu) << 4) | (cur.vl[e] & 0x0F0F0F0Fu);
                vo[e] = (cur.vh[e] & 0xF0F0F0F0u) | ((cur.vl[e] >> 4) & 0x0F0F0F0Fu);
            } else {
                ve[e] = cur.vh[e] & 0x0F0F0F0Fu;
                vo[e] = (cur.vh[e] >> 4) & 0x0F0F0F0Fu;
            }
        }
        f16xk va[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            // byte t / 2 of two positions into the low bytes of the halves
            const unsigned sel = 0x0C000C00u | ((4u + t / 2) << 16) | static_cast<unsigned>(t / 2);
            const unsigned *src = (t & 1) ? vo : ve;
            const float off = 1024.0f + (KV8 ? 136.0f : 8.0f);
            u32xk pk;
#pragma unroll
            for (int e = 0; e < NP; e += 2)
                pk[e / 2] = f16_unbias(__builtin_amdgcn_perm(src[e + 1], src[e], sel) | kF16Base, off);
            va[t] = __builtin_bit_cast(f16xk, pk);
        }
        fetch(cur);                                  // the step RING ahead

        // ---- scores, the small pieces first
        float sc[NP];
        float tmax = -__builtin_inff();
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int pc = 2; pc >= 0; --pc)
#pragma unroll
                for (int st = 0; st < 4; ++st)
                    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        ka[u][st],
                        __builtin_bit_cast(f16x8, u32x4{qb[pc][st][0], qb[pc][st][1], qb[pc][st][2], qb[pc][st][3]}),
                        d, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool vis = p0 + 16 * u + 4 * g + i <= limit;
                sc[4 * u + i] = vis ? d[i] * (ks[4 * u + i] * gscale) : -__builtin_inff();
                tmax = fmaxf(tmax, sc[4 * u + i]);
            }
        }

        // ---- running softmax of query row c over the step (base 2)
        const float m_new = fmaxf(m_run, quad_group_max(tmax));
        const bool fresh = m_run == -__builtin_inff();   // nothing accumulated yet
        const float alpha = fresh ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        float pv[NP], psum = 0.0f, pmax = 0.0f;
#pragma unroll
        for (int e = 0; e < NP; ++e) {
            const float p = sc[e] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(sc[e] - m_new);
            psum += p;
            pv[e] = p * vs[e];
            pmax = fmaxf(pmax, fabsf(pv[e]));
        }
        l_run = fmaf(l_run, alpha, quad_group_sum(psum));
        m_run = m_new;
        // p v_scale of the row times 2^kt, split into pieces: kt is kept while
        // the step's largest value stays in [2^7, 2^15), else reset to put it
        // in [2^14, 2^15); the accumulators hold O 2^kt and follow the row's
        // scale and maximum
        pmax = quad_group_max(pmax);
        int kt = kt_run;
        if (pmax > 0.0f) {
            const int ex = __builtin_amdgcn_frexp_expf(pmax);      // pmax < 2^ex
            if (fresh || ex + kt_run > 15 || ex + kt_run < 8) kt = 15 - ex;
        }
        const float f = __builtin_amdgcn_ldexpf(alpha, kt - kt_run);
        kt_run = kt;
        // (f = 1 leaves the accumulators as they are, and so does any f while
        // nothing is accumulated)
        if (__builtin_amdgcn_ballot_w64(!fresh && f != 1.0f) != 0) {
#pragma unroll
            for (int t = 0; t < 8; ++t) o[t] *= f;
        }
        u32xk pb[2];
#pragma unroll
        for (int e = 0; e < NP; e += 2) {
            unsigned p1, p2;
            split2(__builtin_amdgcn_ldexpf(pv[e], kt), __builtin_amdgcn_ldexpf(pv[e + 1], kt), p1, p2);
            pb[0][e / 2] = p1;
            pb[1][e / 2] = p2;
        }

        // ---- P.V, the small piece first
#pragma unroll
        for (int pc = 1; pc >= 0; --pc) {
            const f16xk bp = __builtin_bit_cast(f16xk, pb[pc]);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if constexpr (NT == 1)
                    o[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(va[t], bp, o[t], 0, 0, 0);
                else
                    o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[t], bp, o[t], 0, 0, 0);
            }
        }
    };
    if constexpr (RING == 2) {
#pragma unroll 1
        for (; p0 < span1; p0 += 2 * WSTEP) {
            consume(s0, p0);
            if (p0 + WSTEP >= span1) break;          // uniform
            consume(s1, p0 + WSTEP);
        }
    } else {
#pragma unroll 1
        for (; p0 < span1; p0 += WSTEP) consume(s0, p0);
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
        for (int w = 0; w < 4; ++w)
            sW[w][r] = sM[w][r] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(sM[w][r] - mx);
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
// output row (token i, query head hq), merging the splits of its KV head:
// group q takes the splits s = q, q + 4, .. in ascending order with a
// running maximum (the loads of a split do not wait on the previous one),
// then the four groups merge in LDS in a fixed order.
__global__ __launch_bounds__(kD * kCombineGroups) void kv_attn_combine_kernel(const KvArgs a, int splits) {
    __shared__ float cnum[kCombineGroups][kD], cden[kCombineGroups], cmx[kCombineGroups];
    const int row = blockIdx.x;                       // i Hq + hq
    const int i = row / a.Hq, hq = row - (row / a.Hq) * a.Hq;
    const int G = a.Hq / a.Hkv;
    const int h = hq / G, g = hq - (hq / G) * G;
    const int R = a.M * G;
    const int r = i * G + g;
    const float *base = a.work + static_cast<size_t>(h) * splits * R * (kD + 2) + static_cast<size_t>(r) * (kD + 2);
    const size_t stride = static_cast<size_t>(R) * (kD + 2);
    const int grp = threadIdx.x / kD, j = threadIdx.x - grp * kD;

    float mx = -__builtin_inff(), num = 0.0f, den = 0.0f;
#pragma unroll 4
    for (int s = grp; s < splits; s += kCombineGroups) {
        const float *p = base + s * stride;
        const float m = p[kD], l = p[kD + 1], o = p[j];
        const bool seen = l > 0.0f;                   // a split that saw a visible position
        const float mn = seen ? fmaxf(mx, m) : mx;
        const float wa = seen ? __builtin_amdgcn_exp2f(mx - mn) : 1.0f;
        const float wb = seen ? __builtin_amdgcn_exp2f(m - mn) : 0.0f;
        num = fmaf(num, wa, o * wb);
        den = fmaf(den, wa, l * wb);
        mx = mn;
    }
    cnum[grp][j] = num;
    if (j == 0) {
        cden[grp] = den;
        cmx[grp] = mx;
    }
    __syncthreads();
    if (grp == 0) {
        float m = cmx[0];
#pragma unroll
        for (int q = 1; q < kCombineGroups; ++q) m = fmaxf(m, cmx[q]);
        float n = 0.0f, d = 0.0f;
#pragma unroll
        for (int q = 0; q < kCombineGroups; ++q) {
            const float w = cden[q] > 0.0f ? __builtin_amdgcn_exp2f(cmx[q] - m) : 0.0f;
            n = fmaf(cnum[q][j], w, n);
            d = fmaf(cden[q], w, d);
        }
        a.out[static_cast<size_t>(row) * kD + j] = n / d;
    }
}

typedef void (*KvSplit)(const KvArgs, int);

int kv_max_splits(int T) {
    const long long nchunks = (static_cast<long long>(T) + kC - 1) / kC;   // any T >= 1
    return nchunks < kKvMaxSplits ? static_cast<int>(nchunks) : kKvMaxSplits;
}

}  // namespace

size_t kv_attention_workspace_bytes(int M, int Hq, int T) {
    return static_cast<size_t>(kv_max_splits(T)) * static_cast<size_t>(M) * Hq * (kD + 2) * sizeof(float);
}

hipError_t launch_kv_attention(const KvArgs &a, hipStream_t stream) {
    if (static_cast<long long>(a.M) * (a.Hq / a.Hkv) > kRows) return hipErrorInvalidValue;   // rejected by the ABI before this point
    DeviceInfo dev;
    hipError_t e = device_info(&dev);
    if (e != hipSuccess) return e;
    // about two workgroups per compute unit over the KV heads, each split a
    // run of cps chunks (no split empty); runs of several chunks take
    // 32-position wave steps (cps made even: whole workgroup steps)
    const int nchunks = (a.T + kC - 1) / kC;
    int want = (2 * dev.cus + a.Hkv - 1) / a.Hkv;
    if (want > kv_max_splits(a.T)) want = kv_max_splits(a.T);
    if (want < 1) want = 1;
    int cps = (nchunks + want - 1) / want;
    if (cps > 1) cps += cps & 1;
    const int splits = (nchunks + cps - 1) / cps;
    const bool kv8 = a.k_lo != nullptr;
    const KvSplit k = cps > 1 ? (kv8 ? kv_attn_split_kernel<true, 2> : kv_attn_split_kernel<false, 2>)
                              : (kv8 ? kv_attn_split_kernel<true, 1> : kv_attn_split_kernel<false, 1>);
    hipLaunchKernelGGL(k, dim3(splits, a.Hkv), dim3(kKvThreads), 0, stream, a, cps);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kv_attn_combine_kernel, dim3(a.M * a.Hq), dim3(kD * kCombineGroups), 0, stream, a, splits);
    return hipGetLastError();
}

}  // namespace bitnest
