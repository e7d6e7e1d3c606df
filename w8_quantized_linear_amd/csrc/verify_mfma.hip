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
// Two MFMAs (even, odd columns) per plane and token tile give D_hi = 16 P_hi
// and D_lo = 16 P_lo for one 128-column group exactly; the target combines
// them in int32 as 16 D_hi + D_lo = 16 P8 (|16 P8| < 2^26). The 8-bit code is
// never formed as an int8; each plane has its own contraction.
// Epilogue per group: fp32 accumulate of float(16 P) * scale / 16 (draft) or
// float(16 P8) * scale / 256 (target), times the group's activation scale
// for o_proj; both factors are powers of two, so the draft and the target
// round alike.
//
// Work split: a workgroup owns R consecutive weight rows, held in 16-row
// tiles (verify_rows picks R); its 8 waves split the groups of K (one read
// of every plane byte), and the partial sums meet in LDS in a fixed order.
// With one tile per workgroup the plane bytes are read a row at a time and
// staged through LDS (verify_rowload_kernel); with several, straight into
// the operand registers (verify_mfma_kernel).
#include "bitnest_internal.h"
#include "device_common.h"

namespace bitnest {
namespace {

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

// Buffer descriptor over [p, p + bytes): loads beyond it return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

constexpr int kAuxStream = 2;   // non-temporal: plane bytes are read once
constexpr int kTmGroups = 4;    // largest K range (groups) per wave of the tile-major order
constexpr int kOOB = 0x7FFFFFF0;


// One item = one 128-column group of the workgroup's RT 16-row tiles: 16
// plane bytes per lane per plane and tile, the group's scale bits for the
// lane's row in each tile, and the 32 activation bytes of the lane's token
// (per 16-token tile) in the same columns, shared by the RT row tiles.
template <int PLANES, int T, int RT>
struct VItem {
    u32x4 h[RT], l[RT];
    unsigned sbits[RT];
    u32x4 x[T][2];
};

// T: 16-token tiles (1 for M <= 16, 2 for M <= 32). SPLIT: waves per
// workgroup (each streams a contiguous range of the K groups). D: items in
// flight. RT: 16-row tiles per workgroup.
//
// A workgroup owns R consecutive rows (R <= 16 RT, a multiple of 8), held in
// RT 16-row tiles. Lane l works on weight row l % 16 of each tile and token
// l % 16 (+16 t) in quarter l / 16 of each group, so every load has a
// lane-constant vector offset and a wave-uniform scalar offset; rows past the
// workgroup's R (or past N) and tokens past M fall outside the buffer
// descriptors and read as zero, with no memory traffic. Each activation load feeds the MFMAs of all
// RT row tiles, so the activation bytes a workgroup reads from L2 per plane
// byte fall by RT.
template <int PLANES, int T, bool GA, bool EXPORT, int SPLIT, int D, int RT, bool TM>
__global__ __launch_bounds__(64 * SPLIT) void verify_mfma_kernel(const LinearArgs a, int R) {
    static_assert(RT <= SPLIT, "one wave per row tile writes the outputs");
    static_assert(!TM || !EXPORT, "the tile-major order is for the outputs");
    extern __shared__ __align__(16) unsigned char smem[];
    float *red = reinterpret_cast<float *>(smem);                       // [SPLIT][RT][T][4][64]
    float *sact = red + SPLIT * RT * T * 4 * 64;                         // [G][16 T] (GA)

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K = a.K, N = a.N, M = a.M;
    const int G = K >> 7;
    const int row_bytes = K >> 1;
    const int col = lane & 15;          // weight row within the tile; token within an A tile
    const int kq = lane >> 4;           // quarter of the group; token quad of a D tile
    const int row0 = blockIdx.x * R;
    const int rows = N - row0 < R ? N - row0 : R;   // of the RT tiles (R <= 16 RT)
    // draft: (16 P_hi) * scale / 16; target: 16 (16 P_hi + P_lo) * scale / 256
    const float fscale = PLANES == 2 ? 0.00390625f : 0.0625f;

    const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.hi + static_cast<size_t>(row0) * row_bytes,
                                                static_cast<unsigned>(rows) * row_bytes);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc((PLANES == 2 ? a.lo : a.hi) + static_cast<size_t>(row0) * row_bytes,
                                                static_cast<unsigned>(rows) * row_bytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scale + static_cast<size_t>(row0) * G,
                                                static_cast<unsigned>(rows) * G * 2u);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.xq, static_cast<unsigned>(M) * K);
    int voff_w[RT], voff_s[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        voff_w[rt] = (16 * rt + col) * row_bytes + kq * 16;
        voff_s[rt] = (16 * rt + col) * G * 2;
    }
    int voff_x[T];
#pragma unroll
    for (int t = 0; t < T; ++t) voff_x[t] = (16 * t + col) * K + kq * 32;

    if (GA && !EXPORT) {
        for (int i = threadIdx.x; i < G * 16 * T; i += 64 * SPLIT) {
            const int g = i / (16 * T);
            const int t = i - g * 16 * T;
            sact[i] = t < M ? a.xs[static_cast<size_t>(t) * G + g] : 0.0f;
        }
        __syncthreads();
    }

    // this wave's groups [g_begin, g_end)
    const int g_begin = G * wave / SPLIT;
    const int g_end = G * (wave + 1) / SPLIT;
    const int n_items = g_end - g_begin;

    float yacc[RT][T][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) yacc[rt][t][r] = 0.0f;
    if constexpr (!TM) {
        int iseq = 0;
        auto issue = [&](VItem<PLANES, T, RT> &x) {
            const int g = g_begin + iseq;
            const bool live = iseq < n_items;
            const int sw = live ? g * 64 : kOOB;
    #pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                x.h[rt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rh, voff_w[rt], sw, kAuxStream));
                if (PLANES == 2)
                    x.l[rt] =
                        __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rl, voff_w[rt], sw, kAuxStream));
                if (!EXPORT) x.sbits[rt] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff_s[rt], live ? g * 2 : kOOB, 0);
            }
            const int sx = live ? g * kGroup : kOOB;
    #pragma unroll
            for (int t = 0; t < T; ++t) {
                x.x[t][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff_x[t], sx, 0));
                x.x[t][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff_x[t] + 16, sx, 0));
            }
            ++iseq;
        };


        int cseq = 0;
        auto consume = [&](const VItem<PLANES, T, RT> &x) {
            const int g = g_begin + cseq;
            ++cseq;
            i32x4 ae[T], ao[T];
    #pragma unroll
            for (int t = 0; t < T; ++t) split_act(x.x[t][0], x.x[t][1], ae[t], ao[t]);
            float sa[T][4];
    #pragma unroll
            for (int t = 0; t < T; ++t) {
                sa[t][0] = sa[t][1] = sa[t][2] = sa[t][3] = 1.0f;
                if (GA && !EXPORT) {
                    const float4 v = *reinterpret_cast<const float4 *>(sact + g * 16 * T + 16 * t + 4 * kq);
                    sa[t][0] = v.x; sa[t][1] = v.y; sa[t][2] = v.z; sa[t][3] = v.w;
                }
            }
    #pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                i32x4 bhe, bho, ble, blo;
                signed16(x.h[rt], bhe, bho);
                if (PLANES == 2) signed16(x.l[rt], ble, blo);
                const float sc = half_bits_to_float(static_cast<uint16_t>(x.sbits[rt])) * fscale;
    #pragma unroll
                for (int t = 0; t < T; ++t) {
                    const i32x4 zero = {0, 0, 0, 0};
                    i32x4 dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(ae[t], bhe, zero, 0, 0, 0);
                    dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(ao[t], bho, dh, 0, 0, 0);
                    i32x4 dl = zero;
                    if (PLANES == 2) {
                        dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(ae[t], ble, zero, 0, 0, 0);
                        dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(ao[t], blo, dl, 0, 0, 0);
                    }
                    if (EXPORT) {
    #pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int tok = 16 * t + 4 * kq + r;
                            const int row = 16 * rt + col;
                            if (tok < M && row < rows) {
                                const size_t o = (static_cast<size_t>(tok) * N + row0 + row) * G + g;
                                const int ph = dh[r] >> 4;
                                a.p_hi[o] = ph;
                                if (PLANES == 2) {
                                    const int pl = dl[r] >> 4;
                                    a.p_lo[o] = pl;
                                    a.p8[o] = 16 * ph + pl;
                                }
                            }
                        }
                    } else {
    #pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            // draft: 16 P_hi; target: 16 (16 P_hi) + 16 P_lo = 16 P8
                            const int p = PLANES == 2 ? 16 * dh[r] + dl[r] : dh[r];
                            const float w = GA ? sc * sa[t][r] : sc;
                            yacc[rt][t][r] += static_cast<float>(p) * w;
                        }
                    }
                }
            }
        };

        VItem<PLANES, T, RT> ring[D];
    #pragma unroll
        for (int d = 0; d < D; ++d) issue(ring[d]);
        for (int base = 0; base < n_items; base += D) {
    #pragma unroll
            for (int d = 0; d < D; ++d) {
                if (base + d < n_items) consume(ring[d]);     // uniform
                issue(ring[d]);
            }
        }
    } else {
        // Tile-major order: the wave's K range is at most kTmGroups groups,
        // its activations stay in registers, and the ring's items are whole
        // row tiles (16 rows x the range's bytes, per plane). The bytes a CU
        // has in flight are then a few whole rows rather than a slice of
        // every row of the workgroup, which the memory serves far faster
        // (the same plane bytes read in this order: 5.3 against 3.0-3.5 TB/s).
        constexpr int NG = kTmGroups;
        u32x4 xa[NG][T][2];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const int sx = gi < n_items ? (g_begin + gi) * kGroup : kOOB;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                xa[gi][t][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff_x[t], sx, 0));
                xa[gi][t][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff_x[t] + 16, sx, 0));
            }
        }
        struct TItem {
            u32x4 h[NG], l[NG];
            unsigned sbits[NG];
        };
        auto issue_tile = [&](TItem &x, int rt) {
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const bool live = gi < n_items;
                const int sw = live ? (g_begin + gi) * 64 : kOOB;
                x.h[gi] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rh, voff_w[rt], sw, kAuxStream));
                if (PLANES == 2)
                    x.l[gi] = __builtin_bit_cast(u32x4,
                                                 __builtin_amdgcn_raw_buffer_load_b128(rl, voff_w[rt], sw, kAuxStream));
                x.sbits[gi] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff_s[rt], live ? (g_begin + gi) * 2 : kOOB, 0);
            }
        };
        auto consume_tile = [&](const TItem &x, int rt) {
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                if (gi >= n_items) continue;                 // uniform
                const int g = g_begin + gi;
                i32x4 bhe, bho, ble, blo;
                signed16(x.h[gi], bhe, bho);
                if (PLANES == 2) signed16(x.l[gi], ble, blo);
                const float sc = half_bits_to_float(static_cast<uint16_t>(x.sbits[gi])) * fscale;
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    i32x4 ae, ao;
                    split_act(xa[gi][t][0], xa[gi][t][1], ae, ao);
                    float sa[4] = {1.0f, 1.0f, 1.0f, 1.0f};
                    if (GA) {
                        const float4 v = *reinterpret_cast<const float4 *>(sact + g * 16 * T + 16 * t + 4 * kq);
                        sa[0] = v.x; sa[1] = v.y; sa[2] = v.z; sa[3] = v.w;
                    }
                    const i32x4 zero = {0, 0, 0, 0};
                    i32x4 dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(ae, bhe, zero, 0, 0, 0);
                    dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(ao, bho, dh, 0, 0, 0);
                    i32x4 dl = zero;
                    if (PLANES == 2) {
                        dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(ae, ble, zero, 0, 0, 0);
                        dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(ao, blo, dl, 0, 0, 0);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        // draft: 16 P_hi; target: 16 (16 P_hi) + 16 P_lo = 16 P8
                        const int pv = PLANES == 2 ? 16 * dh[r] + dl[r] : dh[r];
                        const float w = GA ? sc * sa[r] : sc;
                        yacc[rt][t][r] += static_cast<float>(pv) * w;
                    }
                }
            }
        };
        TItem tr[2];
        issue_tile(tr[0], 0);
        if (RT > 1) issue_tile(tr[1], 1);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            consume_tile(tr[rt & 1], rt);
            if (rt + 2 < RT) issue_tile(tr[rt & 1], rt + 2);
        }
    }

    if (!EXPORT) {
        // the waves' partial sums meet in LDS; wave rt sums them in wave
        // order for row tile rt and writes its outputs
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) red[(((wave * RT + rt) * T + t) * 4 + r) * 64 + lane] = yacc[rt][t][r];
        __syncthreads();
        if (wave < RT) {
            const int rt = wave;
            const int row = 16 * rt + col;
            float tok_scale[T][4];
            if (!GA) {
#pragma unroll
                for (int t = 0; t < T; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int tok = 16 * t + 4 * kq + r;
                        tok_scale[t][r] = tok < M ? a.xs[tok] : 0.0f;
                    }
            }
#pragma unroll
            for (int t = 0; t < T; ++t) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = red[(((0 * RT + rt) * T + t) * 4 + r) * 64 + lane];
#pragma unroll
                    for (int w = 1; w < SPLIT; ++w) v += red[(((w * RT + rt) * T + t) * 4 + r) * 64 + lane];
                    const int tok = 16 * t + 4 * kq + r;
                    if (tok < M && row < rows)
                        a.y[static_cast<size_t>(tok) * N + row0 + row] = GA ? v : v * tok_scale[t][r];
                }
            }
        }
    }
}

// Row-contiguous order for one 16-row tile per workgroup (N spread at most
// 16 rows per CU, e.g. N = 4096). A B operand needs 16 rows per load, so the
// kernel above reads a 64-byte slice of 16 rows per instruction; here every
// plane load is 1 KiB of one row (a probe reading down_proj's planes: 5.9
// TB/s in this order against 4.0 TB/s in slices), and the chunk of the tile
// is turned into the matrix-core layout through LDS.
//
// Chunk c = plane bytes [c kChunk, (c + 1) kChunk) of the 16 rows (16
// groups). Wave w loads rows 2w and 2w + 1 of each plane into registers,
// kChunkLead chunks ahead, writes them to LDS buffer c % 2 and, after a
// barrier, takes groups w and w + 8 of the chunk: B from LDS (the row pitch
// puts the 16 rows of an operand in distinct banks), A from its own
// activation loads, issued together with the chunk's plane loads so that
// the in-order load counter never waits for a later chunk. The epilogue is
// the kernel above's with one tile.
constexpr int kChunk = 1024;                    // plane bytes per row per chunk
constexpr int kChunkGroups = kChunk / 64;       // 16
constexpr int kRowPitch = kChunk + 16;          // LDS bytes per row of a chunk
constexpr int kChunkLead = 2;                   // chunks in flight (and LDS buffers)

template <int PLANES>
constexpr size_t chunk_lds_bytes() { return static_cast<size_t>(PLANES) * kRowsPerBlock * kRowPitch; }

template <int PLANES, int T, bool GA>
__global__ __launch_bounds__(64 * 8) void verify_rowload_kernel(const LinearArgs a, int R) {
    constexpr int SPLIT = 8;
    constexpr int NL = 2 * PLANES;                // plane loads per wave per chunk
    static_assert(kChunkGroups == 2 * SPLIT, "two groups of a chunk per wave");
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *lbuf = smem;                                             // [kChunkLead][PLANES][16][kRowPitch]
    float *sact = reinterpret_cast<float *>(smem + kChunkLead * chunk_lds_bytes<PLANES>());   // [G][16 T] (GA)
    float *red = reinterpret_cast<float *>(smem);                          // [SPLIT][T][4][64], after the stream

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K = a.K, N = a.N, M = a.M;
    const int G = K >> 7;
    const int row_bytes = K >> 1;
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int row0 = blockIdx.x * R;
    const int rows = N - row0 < R ? N - row0 : R;
    const float fscale = PLANES == 2 ? 0.00390625f : 0.0625f;
    const int nchunks = (row_bytes + kChunk - 1) / kChunk;

    const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.hi + static_cast<size_t>(row0) * row_bytes,
                                                static_cast<unsigned>(rows) * row_bytes);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc((PLANES == 2 ? a.lo : a.hi) + static_cast<size_t>(row0) * row_bytes,
                                                static_cast<unsigned>(rows) * row_bytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scale + static_cast<size_t>(row0) * G,
                                                static_cast<unsigned>(rows) * G * 2u);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.xq, static_cast<unsigned>(M) * K);
    const int voff_s = col * G * 2;
    int voff_x[T];
#pragma unroll
    for (int t = 0; t < T; ++t) voff_x[t] = (16 * t + col) * K + kq * 32;

    if (GA) {
        for (int i = threadIdx.x; i < G * 16 * T; i += 64 * SPLIT) {
            const int g = i / (16 * T);
            const int t = i - g * 16 * T;
            sact[i] = t < M ? a.xs[static_cast<size_t>(t) * G + g] : 0.0f;
        }
        // made visible by the first chunk's barrier
    }

    struct Chunk {
        u32x4 p[NL];                 // load j: plane j / 2, row 2 wave + j % 2
        u32x4 x[2][T][2];            // activation bytes of groups wave, wave + 8
        uint16_t sbits[2];
    };
    auto issue = [&](Chunk &ck, int c) {
        const bool live = c < nchunks;
        // lanes past the row's end (a last, partial chunk) read nothing: an
        // offset of at least kOOB is outside the descriptor (whose size is
        // below 2^31), and the sums stay below 2^32
        const int left = row_bytes - c * kChunk;
        const unsigned lane_off = lane * 16 < left ? static_cast<unsigned>(lane * 16) : static_cast<unsigned>(kOOB);
        const int sc = live ? c * kChunk : kOOB;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const unsigned vo = static_cast<unsigned>((2 * wave + (j & 1)) * row_bytes) + lane_off;
            ck.p[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    (j >> 1) ? rl : rh, static_cast<int>(vo), sc, kAuxStream));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int g = c * kChunkGroups + wave + SPLIT * i;
            const bool gl = live && g < G;
            const int sx = gl ? g * kGroup : kOOB;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                ck.x[i][t][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff_x[t], sx, 0));
                ck.x[i][t][1] = __builtin_bit_cast(u32x4,
                                                   __builtin_amdgcn_raw_buffer_load_b128(rx, voff_x[t] + 16, sx, 0));
            }
            ck.sbits[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff_s, gl ? g * 2 : kOOB, 0);
        }
    };

    float yacc[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[t][r] = 0.0f;

    auto consume = [&](const Chunk &ck, int c, unsigned char *buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int gl = wave + SPLIT * i;
            const int g = c * kChunkGroups + gl;
            if (g >= G) continue;                          // uniform
            const unsigned char *src = buf + col * kRowPitch + gl * 64 + kq * 16;
            i32x4 bhe, bho, ble, blo;
            signed16(*reinterpret_cast<const u32x4 *>(src), bhe, bho);
            if (PLANES == 2) signed16(*reinterpret_cast<const u32x4 *>(src + kRowsPerBlock * kRowPitch), ble, blo);
            const float sc = half_bits_to_float(ck.sbits[i]) * fscale;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                i32x4 ae, ao;
                split_act(ck.x[i][t][0], ck.x[i][t][1], ae, ao);
                float sa[4] = {1.0f, 1.0f, 1.0f, 1.0f};
                if (GA) {
                    const float4 v = *reinterpret_cast<const float4 *>(sact + g * 16 * T + 16 * t + 4 * kq);
                    sa[0] = v.x; sa[1] = v.y; sa[2] = v.z; sa[3] = v.w;
                }
                const i32x4 zero = {0, 0, 0, 0};
                i32x4 dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(ae, bhe, zero, 0, 0, 0);
                dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(ao, bho, dh, 0, 0, 0);
                i32x4 dl = zero;
                if (PLANES == 2) {
                    dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(ae, ble, zero, 0, 0, 0);
                    dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(ao, blo, dl, 0, 0, 0);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // draft: 16 P_hi; target: 16 (16 P_hi) + 16 P_lo = 16 P8
                    const int pv = PLANES == 2 ? 16 * dh[r] + dl[r] : dh[r];
                    const float w = GA ? sc * sa[r] : sc;
                    yacc[t][r] += static_cast<float>(pv) * w;
                }
            }
        }
    };

    // the chunks' loads are issued in chunk order (no scheduling across an
    // issue), so waiting for one chunk never waits for a later one
    Chunk ring[kChunkLead];
#pragma unroll
    for (int d = 0; d < kChunkLead; ++d) {
        issue(ring[d], d);
        __builtin_amdgcn_sched_barrier(0);
    }
    // every pass of the loop takes kChunkLead chunks with no early exit (a
    // chunk past the end writes zeros, has no groups and loads nothing), so
    // the load counter waits are the same on every path
    for (int base = 0; base < nchunks; base += kChunkLead) {
#pragma unroll
        for (int d = 0; d < kChunkLead; ++d) {
            const int c = base + d;
            unsigned char *buf = lbuf + d * chunk_lds_bytes<PLANES>();
            // buffer d was last read for chunk c - kChunkLead, before the
            // previous chunk's barrier
#pragma unroll
            for (int j = 0; j < NL; ++j)
                *reinterpret_cast<u32x4 *>(buf + ((j >> 1) * kRowsPerBlock + 2 * wave + (j & 1)) * kRowPitch +
                                           lane * 16) = ring[d].p[j];
            __syncthreads();
            consume(ring[d], c, buf);
            __builtin_amdgcn_sched_barrier(0);
            issue(ring[d], c + kChunkLead);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    __syncthreads();                                       // the chunk buffers become the exchange
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((wave * T + t) * 4 + r) * 64 + lane] = yacc[t][r];
    __syncthreads();
    if (wave == 0) {
        float tok_scale[T][4];
        if (!GA) {
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tok = 16 * t + 4 * kq + r;
                    tok_scale[t][r] = tok < M ? a.xs[tok] : 0.0f;
                }
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = red[((0 * T + t) * 4 + r) * 64 + lane];
#pragma unroll
                for (int w = 1; w < SPLIT; ++w) v += red[((w * T + t) * 4 + r) * 64 + lane];
                const int tok = 16 * t + 4 * kq + r;
                if (tok < M && col < rows)
                    a.y[static_cast<size_t>(tok) * N + row0 + col] = GA ? v : v * tok_scale[t][r];
            }
        }
    }
}

typedef void (*VerifyKernel)(const LinearArgs, int);

constexpr int kSplit = 8;     // waves per workgroup
constexpr int kVerifyItems = 2;

// Most 16-row tiles per workgroup without register spills (checked in the
// ISA): 8 for one token tile; for two, 7 with per-token activation scales
// and 6 with grouped ones (the 8-tile two-token-tile instantiations and the
// grouped 7-tile one spill, so they are not instantiated).
constexpr int max_row_tiles(int T, bool grouped) { return T == 1 ? 8 : (grouped ? 6 : 7); }

// the largest instantiation with at most rt tiles, down from RT (rt >= 2:
// one tile per workgroup takes verify_rowload_kernel)
template <int PLANES, int T, bool GA, bool TM, int RT>
VerifyKernel pick_rt_from(int rt) {
    if constexpr (RT > 2) {
        if (rt >= RT) return verify_mfma_kernel<PLANES, T, GA, false, kSplit, kVerifyItems, RT, TM>;
        return pick_rt_from<PLANES, T, GA, TM, RT - 1>(rt);
    } else {
        return verify_mfma_kernel<PLANES, T, GA, false, kSplit, kVerifyItems, 2, TM>;
    }
}

template <int PLANES, int T, bool TM>
VerifyKernel pick_rt_order(int rt, bool grouped) {
    if (grouped) return pick_rt_from<PLANES, T, true, TM, max_row_tiles(T, true)>(rt);
    return pick_rt_from<PLANES, T, false, TM, max_row_tiles(T, false)>(rt);
}

template <int PLANES, int T>
VerifyKernel pick_rt(int rt, bool grouped, bool exporting, bool tile_major) {
    if (exporting) return verify_mfma_kernel<PLANES, T, false, true, kSplit, kVerifyItems, 1, false>;
    return tile_major ? pick_rt_order<PLANES, T, true>(rt, grouped) : pick_rt_order<PLANES, T, false>(rt, grouped);
}

VerifyKernel pick_rowload(int planes, int T, bool grouped) {
    if (planes == 2) {
        if (T == 1) return grouped ? verify_rowload_kernel<2, 1, true> : verify_rowload_kernel<2, 1, false>;
        return grouped ? verify_rowload_kernel<2, 2, true> : verify_rowload_kernel<2, 2, false>;
    }
    if (T == 1) return grouped ? verify_rowload_kernel<1, 1, true> : verify_rowload_kernel<1, 1, false>;
    return grouped ? verify_rowload_kernel<1, 2, true> : verify_rowload_kernel<1, 2, false>;
}

constexpr int kMaxTileRule = 4;   // the whole-tile rule's largest tile count (a power of two)

// Rows per workgroup (R) and its 16-row tiles (RT). Where N spread over one
// workgroup per compute unit needs at most max_row_tiles tiles, every CU
// gets one workgroup of R = ceil(N / CUs) rows rounded up to 8 (N = 6144: 24
// rows on each of 256 CUs, where whole 16-row tiles would leave half of the
// CUs with two tiles and half with one; N = 28672: 112 rows, where whole
// tiles would take two rounds of residency). Otherwise whole tiles, as many
// (up to kMaxTileRule) as keep at least two workgroups per CU.
void verify_rows(int N, int T, bool grouped, int cus, int *R, int *RT) {
    const int even = ((N + cus - 1) / cus + 7) & ~7;
    if (even <= max_row_tiles(T, grouped) * kRowsPerBlock) {
        *R = even;
        *RT = (even + kRowsPerBlock - 1) / kRowsPerBlock;
        return;
    }
    const int tiles = (N + kRowsPerBlock - 1) / kRowsPerBlock;
    int rt = kMaxTileRule;
    while (rt > 1 && (tiles + rt - 1) / rt < 2 * cus) rt >>= 1;
    *R = rt * kRowsPerBlock;
    *RT = rt;
}

}  // namespace

hipError_t launch_verify_mfma(const LinearArgs &a, bool export_partials, hipStream_t stream) {
    if (a.M < 8 || a.M > kMaxM) return hipErrorInvalidValue;
    const int T = a.M <= 16 ? 1 : 2;
    const bool target = a.lo != nullptr;
    const bool grouped = a.act_group == kGroup && !export_partials;
    DeviceInfo dev;
    hipError_t e = device_info(&dev);
    if (e != hipSuccess) return e;
    int R = kRowsPerBlock, RT = 1;                     // the export is for checking: one tile
    if (!export_partials) verify_rows(a.N, T, grouped, dev.cus, &R, &RT);
    // tile-major order where a workgroup has several tiles and every wave's
    // K range fits the registers it keeps the activations in
    const int G_ = a.K / kGroup;
    const bool tm = !export_partials && RT >= 2 && (G_ + kSplit - 1) / kSplit <= kTmGroups;
    // one tile per workgroup: the row-contiguous order
    const bool rowload = !export_partials && RT == 1;
    VerifyKernel k;
    if (rowload)
        k = pick_rowload(target ? 2 : 1, T, grouped);
    else if (target)
        k = T == 1 ? pick_rt<2, 1>(RT, grouped, export_partials, tm) : pick_rt<2, 2>(RT, grouped, export_partials, tm);
    else
        k = T == 1 ? pick_rt<1, 1>(RT, grouped, export_partials, tm) : pick_rt<1, 2>(RT, grouped, export_partials, tm);
    // the partial-sum exchange [kSplit][RT][T][4][64] (for the row-contiguous
    // kernel: the chunk buffers, which it reuses for the exchange) and the
    // grouped activation-scale table [G][16 T]
    const size_t G = a.K / kGroup;
    const size_t exchange = static_cast<size_t>(kSplit) * RT * T * 4 * 64 * 4;
    const size_t stream_lds = rowload ? kChunkLead * (target ? chunk_lds_bytes<2>() : chunk_lds_bytes<1>()) : 0;
    const size_t lds = (stream_lds > exchange ? stream_lds : exchange) + (grouped ? G * 16 * T * 4 : 0);
    if (lds > static_cast<size_t>(dev.max_lds)) return hipErrorInvalidValue;
    if (lds > 65536) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    const int blocks = (a.N + R - 1) / R;
    hipLaunchKernelGGL(k, dim3(blocks), dim3(64 * kSplit), lds, stream, a, R);
    return hipGetLastError();
}

}  // namespace bitnest
