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
//  - A wave owns a contiguous run of whole weight rows. Lane l reads the
//    16-byte slot l of each 1 KiB chunk of a row with one 128-bit
//    non-temporal buffer load, so one wave instruction moves 1 KiB, fully
//    coalesced. The wave streams its (row, chunk) items through a ring of D
//    items in flight (both planes of an item for the target).
//  - A 16-byte slot holds 32 columns, a quarter of a 128-column group, so the
//    four lanes of a quad hold one group.
//  - The workgroup first copies the int8 codes of all M tokens into LDS,
//    permuted so that each activation dword lines up with the even or the odd
//    nibbles of a weight dword; the tile is shared by the M tokens' rows and
//    by both planes.
//  - Draft, per 16-byte slot: each nibble u becomes the signed byte
//    16 (u - 8) (xor 0x8, then placed in the high half of a byte), the even
//    and the odd columns of a weight dword in separate dwords, and two
//    v_dot4_i32_i8 per weight dword per token give 16 P_hi exactly.
//  - Target: both planes are combined inside the dot product. The byte
//    16 (hi - 8) + lo (hi xor 8 in the high half, the unsigned lo nibble in
//    the low half; no carry between the two fields) is w8 + 8 in [-128, 127],
//    so by linearity one dot4 per dword gives 16 P_hi + P_lo + 8 sum(q) =
//    P8 + 8 sum(q), and the per-(group, token) code sums staged in LDS remove
//    the 8 sum(q). The 8-bit code w8 = 16 (hi - 8) + (lo - 8) in [-136, 119]
//    itself is never formed as an int8. The partials export runs this same
//    loop: it writes P8 as computed here, P_hi from the draft's loop and
//    P_lo = P8 - 16 P_hi.
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
#include "gemv_common.h"

#include <atomic>

namespace bitnest {
namespace {

template <int M>
struct GemvLds {
    static constexpr int kMP = (M + 3) & ~3;   // tokens padded to 4 in the per-group tables
    // codes [M][K] bytes; then either the grouped activation scales
    // [G][kMP] or (fused per-token quantisation) a [waves][M] scratch for
    // the maxima, padded to 16 bytes; then (target) the code sums [G][kMP]
    __host__ __device__ static size_t scales_bytes(int K, bool grouped_act, bool fused, int waves) {
        const size_t G = K / kGroup;
        size_t tail = grouped_act ? G * kMP * sizeof(float) : 0;
        if (fused && !grouped_act) tail = static_cast<size_t>(waves) * M * sizeof(float);
        return (tail + 15) & ~static_cast<size_t>(15);
    }
    static size_t bytes(int K, bool grouped_act, bool fused, int waves, bool code_sums) {
        const size_t G = K / kGroup;
        return static_cast<size_t>(M) * K + scales_bytes(K, grouped_act, fused, waves) +
               (code_sums ? G * kMP * sizeof(int) : 0);
    }
};

// PLANES: 1 draft (hi), 2 target (hi + lo). GA: per-128-group activation
// scales. EXPORT: write the integer partials instead of y. D: items in flight
// per wave. WAVES: waves per workgroup. XU: 0, or quantise the fp32 input in
// the prologue, XU 8-column units per thread and token (several tokens only
// with XU = 1 and no rotation). ROT (with XU):
// 0, or apply the R4 rotation (blocks of a.rot_block columns, times
// a.rot_scale) to the fp32 input before quantising it: ROT = 1 takes the
// block size from a.rot_block, any other value is that block size fixed when
// compiling (which the launcher picks only when a.rot_block equals it).
//
// A row of K columns is C = ceil(K / 2048) chunks; the (row, chunk) items of
// the whole call are split into contiguous runs, one per wave, and each wave
// streams its run with D items in flight: the loads of item i + D are issued
// as soon as item i has been consumed. Item addresses are wave-uniform
// (scalar registers) plus a fixed lane offset, so address arithmetic stays
// off the vector ALU; loads past the end of a plane return 0. The workgroup
// stages the codes once into LDS while its first D items are in flight.
template <int PLANES, int M, bool GA, bool EXPORT, int D, int WAVES, int XU, int ROT>
__global__ __launch_bounds__(64 * WAVES) void gemv_planes_kernel(const LinearArgs a) {
    constexpr bool FUSED = XU > 0;
    constexpr int kThreads = 64 * WAVES;
    constexpr int kPB = (kMaxK / 16 + kThreads - 1) / kThreads;   // code blocks per thread and token
    constexpr int kMP = GemvLds<M>::kMP;
    extern __shared__ __align__(16) unsigned char smem[];
    const int K = a.K;
    const int N = a.N;
    const int G = K >> 7;
    const int slots = K >> 5;       // 16-byte slots per plane row
    const int row_bytes = K >> 1;   // bytes per plane row
    const int C = (slots + 63) >> 6;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // draft: (16 P_hi) * scale / 16; target: P8 * scale / 16
    const float fscale = 0.0625f;
    constexpr bool kSums = PLANES == 2;   // the target's code sums (also when exporting)

    const unsigned plane_bytes = static_cast<unsigned>(N) * static_cast<unsigned>(row_bytes);
    const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.hi, plane_bytes);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(PLANES == 2 ? a.lo : a.hi, plane_bytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scale, static_cast<unsigned>(N) * G * 2u);
    const int voff_plane = lane * 16;          // lane's 16 bytes within a chunk
    const int voff_scale = (lane >> 2) * 2;    // its group's scale within the chunk's 16 groups

    // this wave's rows [row_begin, row_begin + rows): whole rows, so that
    // exactly one wave owns each output; its items are the C chunks of each
    // row, in order. Of the grid's waves, the first rows_r take rows_q + 1
    // rows and the rest rows_q (the launcher's quotient and remainder of N by
    // the wave count, so no division is made here).
    const int gw = static_cast<int>(blockIdx.x) * WAVES + wave;
    const int row_begin = gw * a.rows_q + min(gw, a.rows_r);
    const int n_items = (a.rows_q + (gw < a.rows_r ? 1 : 0)) * C;

    // Issue the loads of the next item in order. Items past this wave's run
    // are given an offset beyond the plane, which the buffer unit answers
    // with zeros and no memory traffic; so every issue is unconditional and
    // the number of loads in flight is the same on every path.
    const int oob = static_cast<int>(plane_bytes);
    int irow = row_begin, ichunk = 0, iseq = 0;    // next item to issue (wave-uniform)
    auto issue = [&](Item<PLANES> &x) {
        const bool live = iseq < n_items;
        const int soff = live ? irow * row_bytes + ichunk * 1024 : oob;
        const int soff_s = live ? (irow * G + ichunk * 16) * 2 : static_cast<int>(N * G * 2);
        x.h = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rh, voff_plane, soff, kAuxStream));
        if (PLANES == 2)
            x.l = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rl, voff_plane, soff, kAuxStream));
        if (!EXPORT) x.sbits = __builtin_amdgcn_raw_buffer_load_b16(rs, voff_scale, soff_s, 0);
        ++iseq;
        if (++ichunk == C) {
            ichunk = 0;
            ++irow;
        }
    };

    unsigned char *act = smem;                                                    // [M][2][slots][16]
    float *sact = reinterpret_cast<float *>(smem + static_cast<size_t>(M) * K);   // [G][kMP] (GA)
    int *qsum = reinterpret_cast<int *>(smem + static_cast<size_t>(M) * K +
                                        GemvLds<M>::scales_bytes(K, GA, FUSED, WAVES));   // [G][kMP]
    const int nb16 = K >> 4;
    float tok_scale[M];
    Item<PLANES> ring[D];

    if constexpr (!FUSED) {
        // 1) codes (kPB 16-column blocks per thread and token cover K), the
        //    activation scales, then the first D items
        u32x4 pre[M][kPB];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int t = 0; t < kPB; ++t) {
                const int j = threadIdx.x + t * kThreads;
                if (j < nb16) pre[m][t] = *reinterpret_cast<const u32x4 *>(a.xq + static_cast<size_t>(m) * K + j * 16);
            }
        if (!GA && !EXPORT) {
#pragma unroll
            for (int m = 0; m < M; ++m) tok_scale[m] = a.xs[m];
        }
        constexpr int kGAPer = (kGroup * 8 + kThreads - 1) / kThreads;
        float gscale[kGAPer];
        if (GA) {
#pragma unroll
            for (int t = 0; t < kGAPer; ++t) {
                const int i = threadIdx.x + t * kThreads;     // flat [G][kMP]
                gscale[t] = 0.0f;
                if (i < G * kMP) {
                    const int g = i / kMP, m = i - (i / kMP) * kMP;
                    if (m < M) gscale[t] = a.xs[static_cast<size_t>(m) * G + g];
                }
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d) issue(ring[d]);

        // 2) stage the codes into LDS while the ring is in flight; for the
        //    target, also the per-(group, token) code sums (the eight blocks of
        //    a group are eight consecutive lanes)
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int t = 0; t < kPB; ++t) {
                const int j = threadIdx.x + t * kThreads;
                if (j < nb16) stage_block(act + static_cast<size_t>(m) * K, j, row_bytes, pre[m][t]);
                if (kSums) {
                    int cs = 0;
                    if (j < nb16) {
                        cs = sdot4(pre[m][t].x, 0x01010101u, cs);
                        cs = sdot4(pre[m][t].y, 0x01010101u, cs);
                        cs = sdot4(pre[m][t].z, 0x01010101u, cs);
                        cs = sdot4(pre[m][t].w, 0x01010101u, cs);
                    }
                    cs = quad_sum_i32(cs);
                    cs += dpp_i32<kDppRowHalfMirror>(cs);
                    if (j < nb16 && (j & 7) == 0) qsum[(j >> 3) * kMP + m] = cs;
                }
            }
        if (GA) {
#pragma unroll
            for (int t = 0; t < kGAPer; ++t) {
                const int i = threadIdx.x + t * kThreads;
                if (i < G * kMP) sact[i] = gscale[t];
            }
        }
        __syncthreads();
    } else {
        static_assert(M == 1 || (XU == 1 && ROT == 0), "several tokens: one unit per thread, no rotation");
        // 1) the fp32 rows in 8-column units u = tid + k * threads (k < XU),
        //    two 16-byte loads each; units past a row read zeros (an offset
        //    past the descriptor's end makes no memory traffic). The loads
        //    are unconditional (under a branch, the compiler adds register
        //    copies at its join). Every code needs its row's maximum, so the
        //    row loads are the critical path: a workgroup barrier (which
        //    waits for no data) puts every wave's row loads ahead of any item
        //    load in the compute unit's load queue, and the ring is then
        //    issued at once, its latency overlapping the rows' arrival and
        //    the quantisation. (Measured: issued per wave right behind its
        //    own row loads, the later waves' row loads queued behind the
        //    earlier waves' items; waiting for the rows before issuing the
        //    ring cost 0.1-0.2 us more per launch than this order.)
        const unsigned x_bytes = static_cast<unsigned>(M) * static_cast<unsigned>(K) * 4u;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, x_bytes);
        const int nunit = K >> 3;
        u32x4 xr[M][XU][2];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int k = 0; k < XU; ++k) {
                const int u = threadIdx.x + k * kThreads;
                const int off = u < nunit ? (m * K + u * 8) * 4 : static_cast<int>(x_bytes);
                xr[m][k][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
                xr[m][k][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16, 0, 0));
            }
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int d = 0; d < D; ++d) issue(ring[d]);

        // (each element is copied out before the bit cast: a bit cast applied
        // directly to a vector-element lvalue reads element 0 with this
        // compiler)
        float xf[M][XU][8];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int k = 0; k < XU; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xf[m][k][i] = __builtin_bit_cast(float, static_cast<unsigned>(xr[m][k][0][i]));
                    xf[m][k][4 + i] = __builtin_bit_cast(float, static_cast<unsigned>(xr[m][k][1][i]));
                }
        if constexpr (ROT != 0) {
            // unit u = tid + k * threads: one wave's units at one k are 512
            // consecutive columns, so every rotation block is inside a wave
#pragma unroll
            for (int k = 0; k < XU; ++k) {
                // wave-uniform: units past the row stay zero (marked as the
                // rare case, so that the transform is laid out in line)
                if (__builtin_expect(k * kThreads + wave * 64 < nunit, 1)) {
                    if constexpr (ROT == 1) fwht_unit(xf[0][k], lane, a.rot_block);
                    else fwht_unit_fixed<ROT>(xf[0][k], lane);
#pragma unroll
                    for (int i = 0; i < 8; ++i) xf[0][k][i] = xf[0][k][i] * a.rot_scale;
                }
            }
        }
        auto absmax8 = [](const float (&v)[8]) {
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
            return m;
        };

        // 2) scales: per 128-column group (16 consecutive units = one row of
        //    16 lanes) or per token (a workgroup-wide maximum)
        float us[M][XU], ur[M][XU];
        if (GA) {
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int k = 0; k < XU; ++k) {
                    const int u = threadIdx.x + k * kThreads;
                    us[m][k] = row16_max_f32(absmax8(xf[m][k])) / 127.0f;
                    ur[m][k] = quant_recip(us[m][k]);
                    if (u < nunit && (u & 15) == 0) {
                        sact[(u >> 4) * kMP + m] = us[m][k];
                        if (blockIdx.x == 0) a.xs_out[static_cast<size_t>(m) * G + (u >> 4)] = us[m][k];
                    }
                }
        } else {
            float *part = sact;                 // [M][WAVES] scratch (no grouped table)
#pragma unroll
            for (int m = 0; m < M; ++m) {
                float am = 0.0f;
#pragma unroll
                for (int k = 0; k < XU; ++k) am = fmaxf(am, absmax8(xf[m][k]));
                am = wave_max_dpp_f32(am);
                if (lane == 0) part[m * WAVES + wave] = am;
            }
            __syncthreads();
            // each token's per-wave maxima as 16-byte reads, all in flight
            // together
            static_assert(WAVES % 4 == 0, "per-wave maxima are read four at a time");
#pragma unroll
            for (int m = 0; m < M; ++m) {
                float4 pm[WAVES / 4];
#pragma unroll
                for (int w = 0; w < WAVES / 4; ++w) pm[w] = reinterpret_cast<const float4 *>(part + m * WAVES)[w];
                float am = fmaxf(fmaxf(pm[0].x, pm[0].y), fmaxf(pm[0].z, pm[0].w));
#pragma unroll
                for (int w = 1; w < WAVES / 4; ++w)
                    am = fmaxf(am, fmaxf(fmaxf(pm[w].x, pm[w].y), fmaxf(pm[w].z, pm[w].w)));
                tok_scale[m] = am / 127.0f;
                const float r = quant_recip(tok_scale[m]);
                if (blockIdx.x == 0 && threadIdx.x == 0) a.xs_out[m] = tok_scale[m];
#pragma unroll
                for (int k = 0; k < XU; ++k) {
                    us[m][k] = tok_scale[m];
                    ur[m][k] = r;
                }
            }
        }
        // 3) codes -> LDS, unit u as the 8-byte [even | odd] pair (u & 1) of
        //    half (u >> 1) & 1 of slot u >> 2 of its token's row; and to
        //    xq_out from workgroup 0
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int k = 0; k < XU; ++k) {
                const int u = threadIdx.x + k * kThreads;
                int cs = 0;
                if (u < nunit) {
                    unsigned y[8];
                    quant_codes<8>(xf[m][k], us[m][k], ur[m][k], y);
                    unsigned char *dst = act + static_cast<size_t>(m) * K + ((u >> 1) & 1) * row_bytes + (u >> 2) * 16 +
                                         (u & 1) * 8;
                    *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_low_bytes(y[0], y[2], y[4], y[6]),
                                                                 pack_low_bytes(y[1], y[3], y[5], y[7]));
                    const unsigned c0 = pack_low_bytes(y[0], y[1], y[2], y[3]);
                    const unsigned c1 = pack_low_bytes(y[4], y[5], y[6], y[7]);
                    if (blockIdx.x == 0)
                        *reinterpret_cast<uint2 *>(a.xq_out + static_cast<size_t>(m) * K + static_cast<size_t>(u) * 8) =
                            make_uint2(c0, c1);
                    if (kSums) cs = sdot4(c1, 0x01010101u, sdot4(c0, 0x01010101u, 0));
                }
                if (kSums) {
                    // a group is 16 units = one row of 16 lanes
                    cs = quad_sum_i32(cs);
                    cs += dpp_i32<kDppRowRor4>(cs);
                    cs += dpp_i32<kDppRowRor8>(cs);
                    if (u < nunit && (u & 15) == 0) qsum[(u >> 4) * kMP + m] = cs;
                }
            }
        __syncthreads();
    }

    const u32x4 *act4 = reinterpret_cast<const u32x4 *>(act);
    const int tok4 = K >> 4;     // u32x4 per token
    const int half4 = K >> 5;    // u32x4 per half (= slots)

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.0f;

    // consume one item: its group partials, accumulated into the row sums;
    // the last chunk of a row ends the row.
    int crow = row_begin, cchunk = 0;          // next item to consume (wave-uniform)
    auto consume = [&](const Item<PLANES> &x) {
        const int row = crow;
        const int s = cchunk * 64 + lane;
        const bool valid = s < slots;            // uniform within each quad
        const int ss = valid ? s : 0;
        const int g = ss >> 2;
        const float sc = half_bits_to_float(static_cast<uint16_t>(x.sbits)) * fscale;
        if constexpr (PLANES == 2) {
            // target: P8 = sum q (16 (hi - 8) + lo) - 8 sum q, one dot product
            // per dword for both planes (the merged byte of to_combined16)
            const Signed16 n = to_combined16(x.h, x.l);
            int cs[kMP];
#pragma unroll
            for (int i = 0; i < kMP; i += 4) {
                const i32x4 v = *reinterpret_cast<const i32x4 *>(qsum + g * kMP + i);
                cs[i] = v.x; cs[i + 1] = v.y; cs[i + 2] = v.z; cs[i + 3] = v.w;
            }
            Signed16 nh;
            if (EXPORT) nh = to_signed16(x.h);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const u32x4 a0 = act4[m * tok4 + ss];
                const u32x4 a1 = act4[m * tok4 + half4 + ss];
                const int p8 = quad_sum_i32(dot_slot16(n, a0, a1)) - 8 * cs[m];
                if (EXPORT) {
                    // the production P8 as computed above; P_hi from the
                    // draft's loop; P_lo the rest of P8
                    const int ph = quad_sum_i32(dot_slot16(nh, a0, a1)) >> 4;
                    if (valid && (lane & 3) == 0) {
                        const size_t o = (static_cast<size_t>(m) * N + row) * G + g;
                        a.p_hi[o] = ph;
                        a.p8[o] = p8;
                        a.p_lo[o] = p8 - 16 * ph;
                    }
                } else {
                    const float w = GA ? sc * sact[g * kMP + m] : sc;
                    acc[m] += valid ? static_cast<float>(p8) * w : 0.0f;
                }
            }
        } else {
            // draft: 16 P_hi
            const Signed16 n = to_signed16(x.h);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const u32x4 a0 = act4[m * tok4 + ss];
                const u32x4 a1 = act4[m * tok4 + half4 + ss];
                const int p = quad_sum_i32(dot_slot16(n, a0, a1));
                if (EXPORT) {
                    if (valid && (lane & 3) == 0) a.p_hi[(static_cast<size_t>(m) * N + row) * G + g] = p >> 4;
                } else {
                    const float w = GA ? sc * sact[g * kMP + m] : sc;
                    acc[m] += valid ? static_cast<float>(p) * w : 0.0f;
                }
            }
        }
        if (++cchunk == C) {                     // row complete (uniform)
            cchunk = 0;
            ++crow;
            if (!EXPORT) {
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const float v = sum_quads_to_lane63(acc[m]);
                    if (lane == 63) a.y[static_cast<size_t>(m) * N + row] = GA ? v : v * tok_scale[m];
                    acc[m] = 0.0f;
                }
            }
        }
    };

    // steady state: consume item i, then issue item i + D into its slot
    for (int base = 0; base < n_items; base += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (base + d < n_items) consume(ring[d]);    // uniform
            issue(ring[d]);
        }
    }
}

typedef void (*GemvKernel)(const LinearArgs);

// Launch shape: waves per workgroup and items (1 KiB chunks per plane) in
// flight per wave. (Measured on MI355X over the Llama-3-8B shapes: 2-4 items
// per wave with 8-wave workgroups beat deeper rings, whose code has no spills
// and the same waits: the bigger first burst of requests is itself slower.)
constexpr int kGemvWaves = 8;
// The fused single-token kernel quantises the whole row in every workgroup,
// so it runs one workgroup per compute unit. (Measured on MI355X: 8 waves
// and one workgroup per CU beat 16-wave and two-per-CU shapes on all four
// Llama-3-8B shapes.)
constexpr int kFusedWaves = 8;
template <int PLANES>
constexpr int items_in_flight() {
    return PLANES == 1 ? 4 : 2;
}

template <int PLANES, int M>
GemvKernel pick_mode(bool grouped, bool exporting) {
    constexpr int D = items_in_flight<PLANES>();
    constexpr int W = kGemvWaves;
    if (exporting) return gemv_planes_kernel<PLANES, M, false, true, D, W, 0, 0>;
    return grouped ? gemv_planes_kernel<PLANES, M, true, false, D, W, 0, 0>
                   : gemv_planes_kernel<PLANES, M, false, false, D, W, 0, 0>;
}

template <int PLANES>
GemvKernel pick_m(int M, bool grouped, bool exporting) {
    switch (M) {
        case 1: return pick_mode<PLANES, 1>(grouped, exporting);
        case 2: return pick_mode<PLANES, 2>(grouped, exporting);
        case 3: return pick_mode<PLANES, 3>(grouped, exporting);
        case 4: return pick_mode<PLANES, 4>(grouped, exporting);
        case 5: return pick_mode<PLANES, 5>(grouped, exporting);
        case 6: return pick_mode<PLANES, 6>(grouped, exporting);
        case 7: return pick_mode<PLANES, 7>(grouped, exporting);
        default: return nullptr;
    }
}

// fp32 8-column units per thread that cover a row of K <= kFusedMaxMK.
constexpr int fused_units(int K) { return (K / 8 + 64 * kFusedWaves - 1) / (64 * kFusedWaves); }
static_assert(fused_units(kFusedMaxMK) <= 4, "pick_fused covers up to four units per thread");

// The rotation block the fused kernel has a straight-line instantiation for
// (the R4 recipe's block here); other block sizes take it from the arguments.
constexpr int kRotFixedBlock = 512;
static_assert(kRotFixedBlock <= kMaxRotBlock, "a rotation block stays inside one wave");

template <int PLANES, int XU>
GemvKernel pick_fused_xu(bool grouped, int rot_block) {
    constexpr int D = items_in_flight<PLANES>();
    if (rot_block == kRotFixedBlock) return gemv_planes_kernel<PLANES, 1, false, false, D, kFusedWaves, XU, kRotFixedBlock>;
    if (rot_block > 0) return gemv_planes_kernel<PLANES, 1, false, false, D, kFusedWaves, XU, 1>;
    return grouped ? gemv_planes_kernel<PLANES, 1, true, false, D, kFusedWaves, XU, 0>
                   : gemv_planes_kernel<PLANES, 1, false, false, D, kFusedWaves, XU, 0>;
}

// several tokens (M <= kFusedMaxTokens, one unit per thread, no rotation)
template <int PLANES, int M>
GemvKernel pick_fused_tokens(bool grouped) {
    constexpr int D = items_in_flight<PLANES>();
    return grouped ? gemv_planes_kernel<PLANES, M, true, false, D, kFusedWaves, 1, 0>
                   : gemv_planes_kernel<PLANES, M, false, false, D, kFusedWaves, 1, 0>;
}

template <int PLANES>
GemvKernel pick_fused(int M, int K, bool grouped, int rot_block) {
    static_assert(kFusedMaxTokens == 4, "pick_fused covers up to four tokens");
    if (M > 1) {
        if (fused_units(K) > 1 || rot_block > 0) return nullptr;
        return M == 2 ? pick_fused_tokens<PLANES, 2>(grouped)
                      : M == 3 ? pick_fused_tokens<PLANES, 3>(grouped) : pick_fused_tokens<PLANES, 4>(grouped);
    }
    const int xu = fused_units(K);
    return xu <= 1 ? pick_fused_xu<PLANES, 1>(grouped, rot_block)
                   : xu <= 2 ? pick_fused_xu<PLANES, 2>(grouped, rot_block)
                             : pick_fused_xu<PLANES, 4>(grouped, rot_block);
}

size_t gemv_lds_bytes(int M, int K, bool grouped, bool fused, int waves, bool sums) {
    switch (M) {
        case 1: return GemvLds<1>::bytes(K, grouped, fused, waves, sums);
        case 2: return GemvLds<2>::bytes(K, grouped, fused, waves, sums);
        case 3: return GemvLds<3>::bytes(K, grouped, fused, waves, sums);
        case 4: return GemvLds<4>::bytes(K, grouped, fused, waves, sums);
        case 5: return GemvLds<5>::bytes(K, grouped, fused, waves, sums);
        case 6: return GemvLds<6>::bytes(K, grouped, fused, waves, sums);
        case 7: return GemvLds<7>::bytes(K, grouped, fused, waves, sums);
        default: return 0;
    }
}

hipError_t launch(const LinearArgs &a, bool exporting, bool fused, hipStream_t stream) {
    const bool target = a.lo != nullptr;
    const bool grouped = a.act_group == kGroup && !exporting;
    GemvKernel k;
    if (fused)
        k = target ? pick_fused<2>(a.M, a.K, grouped, a.rot_block) : pick_fused<1>(a.M, a.K, grouped, a.rot_block);
    else
        k = target ? pick_m<2>(a.M, grouped, exporting) : pick_m<1>(a.M, grouped, exporting);
    if (!k) return hipErrorInvalidValue;
    DeviceInfo dev;
    hipError_t e = device_info(&dev);
    if (e != hipSuccess) return e;
    const int waves = fused ? kFusedWaves : kGemvWaves;
    const size_t lds = gemv_lds_bytes(a.M, a.K, grouped, fused, waves, target);
    if (lds > static_cast<size_t>(dev.max_lds)) return hipErrorInvalidValue;
    e = set_max_dynamic_lds(reinterpret_cast<const void *>(k), lds);
    if (e != hipSuccess) return e;
    // One resident wave of workgroups (as many as the occupancy of this
    // instantiation allows; one per compute unit for the fused kernel),
    // never more workgroups than rows / waves.
    int occ = 1;
    const int threads = 64 * waves;
    if (!fused) {
        e = occupancy(reinterpret_cast<const void *>(k), threads, lds, &occ);
        if (e != hipSuccess) return e;
        if (occ < 1) occ = 1;
    }
    const int rows_blocks = (a.N + waves - 1) / waves;
    const int full = dev.cus * occ;
    const int blocks = rows_blocks < full ? rows_blocks : full;
    LinearArgs b = a;
    b.rows_q = a.N / (blocks * waves);
    b.rows_r = a.N % (blocks * waves);
    hipLaunchKernelGGL(k, dim3(blocks), dim3(threads), lds, stream, b);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const LinearArgs &a, bool export_partials, hipStream_t stream) {
    return launch(a, export_partials, false, stream);
}

hipError_t launch_gemv_fused(const LinearArgs &a, hipStream_t stream) {
    if (!fused_in_one_launch(a.M, a.N, a.K, a.rot_block)) return hipErrorNotSupported;
    if (a.rot_block > 0 && (a.act_group != 0 || a.rot_block > kMaxRotBlock)) return hipErrorInvalidValue;
    return launch(a, false, true, stream);
}

}  // namespace bitnest
