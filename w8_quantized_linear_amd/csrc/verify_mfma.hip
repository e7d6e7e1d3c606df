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
// Work split: a workgroup owns R consecutive weight rows, held in RT 16-row
// tiles (verify_rows picks R). A B operand needs 16 rows per load, so
// loading it straight from memory reads a 64-byte slice of 16 rows per
// instruction; instead every plane load here is 1 KiB of one row (a probe
// reading down_proj's planes: 5.9 TB/s in this order against 4.0 TB/s in
// slices), and the bytes reach the matrix-core layout through LDS:
//  - chunk c = plane bytes [c kChunk, (c + 1) kChunk) of each row (16
//    groups); slot (c, rt) = chunk c of row tile rt. Slots are taken chunk
//    by chunk, the RT tiles of a chunk in turn, so a chunk's activations are
//    loaded once for all its tiles;
//  - for each slot, wave w loads rows 2w and 2w + 1 of each plane into
//    registers kChunkLead slots ahead, writes them to LDS buffer (slot % 2)
//    and, after a barrier, takes groups w and w + 8 of the chunk: B from LDS
//    (the row pitch puts the 16 rows of an operand in distinct banks), A
//    from the chunk's activation registers;
//  - a chunk's activation loads are issued with its first slot's plane
//    loads, and no load of one slot is scheduled across another's, so the
//    in-order load counter never waits for a later slot;
//  - each wave keeps fp32 sums per tile over its groups; they meet in LDS
//    in wave order (deterministic), and wave rt writes tile rt's outputs.
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
constexpr int kOOB = 0x7FFFFFF0;

constexpr int kChunk = 1024;                    // plane bytes per row per chunk
constexpr int kChunkGroups = kChunk / 64;       // 16
constexpr int kRowPitch = kChunk + 16;          // LDS bytes per row of a chunk
constexpr int kChunkLead = 2;                   // slots in flight (and LDS buffers)

template <int PLANES>
constexpr size_t chunk_lds_bytes() { return static_cast<size_t>(PLANES) * kRowsPerBlock * kRowPitch; }

// T: 16-token tiles (1 for M <= 16, 2 for M <= 32). GA: per-group activation
// scales. EXPORT: write the exact per-group partials instead of y (one tile).
// RT: 16-row tiles per workgroup; R <= 16 RT rows, a multiple of 8. Lane l
// works on weight row l % 16 of a tile and token l % 16 (+16 t) in quarter
// l / 16 of each group; rows past R (or past N) and tokens past M fall
// outside the buffer descriptors and read as zero, with no memory traffic.
template <int PLANES, int T, bool GA, bool EXPORT, int RT>
__global__ __launch_bounds__(64 * 8) void verify_mfma_kernel(const LinearArgs a, int R) {
    constexpr int SPLIT = 8;
    constexpr int NL = 2 * PLANES;                // plane loads per wave per slot
    static_assert(kChunkGroups == 2 * SPLIT, "two groups of a chunk per wave");
    static_assert(kChunkLead == 2, "the slot parity picks the buffer");
    static_assert(RT <= SPLIT, "one wave per row tile writes the outputs");
    static_assert(!EXPORT || (RT == 1 && !GA), "the partials export takes one tile, per-token scales");
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *lbuf = smem;                                             // [2][PLANES][16][kRowPitch]
    float *red = reinterpret_cast<float *>(smem);                          // [SPLIT][RT][T][4][64], after the stream
    constexpr size_t kStream = kChunkLead * chunk_lds_bytes<PLANES>();
    constexpr size_t kExchange = static_cast<size_t>(SPLIT) * RT * T * 4 * 64 * 4;
    float *sact = reinterpret_cast<float *>(smem + (kStream > kExchange ? kStream : kExchange));   // [G][16 T] (GA)

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K = a.K, N = a.N, M = a.M;
    const int G = K >> 7;
    const int row_bytes = K >> 1;
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int row0 = blockIdx.x * R;
    const int rows = N - row0 < R ? N - row0 : R;   // of the RT tiles (R <= 16 RT)
    const float fscale = PLANES == 2 ? 0.00390625f : 0.0625f;
    const int nchunks = (row_bytes + kChunk - 1) / kChunk;

    const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.hi + static_cast<size_t>(row0) * row_bytes,
                                                static_cast<unsigned>(rows) * row_bytes);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc((PLANES == 2 ? a.lo : a.hi) + static_cast<size_t>(row0) * row_bytes,
                                                static_cast<unsigned>(rows) * row_bytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scale + static_cast<size_t>(row0) * G,
                                                static_cast<unsigned>(rows) * G * 2u);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.xq, static_cast<unsigned>(M) * K);
    int voff_x[T];
#pragma unroll
    for (int t = 0; t < T; ++t) voff_x[t] = (16 * t + col) * K + kq * 32;

    if (GA) {
        for (int i = threadIdx.x; i < G * 16 * T; i += 64 * SPLIT) {
            const int g = i / (16 * T);
            const int t = i - g * 16 * T;
            sact[i] = t < M ? a.xs[static_cast<size_t>(t) * G + g] : 0.0f;
        }
        // made visible by the first slot's barrier
    }

    struct Slot {
        u32x4 p[NL];                 // load j: plane j / 2, row 16 rt + 2 wave + j % 2
        uint16_t sbits[2];           // scales of the lane's row in groups wave, wave + 8
    };
    struct Act {
        u32x4 x[2][T][2];            // activation bytes of groups wave, wave + 8
    };
    auto issue_act = [&](Act &ac, int c) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int g = c * kChunkGroups + wave + SPLIT * i;
            const int sx = c < nchunks && g < G ? g * kGroup : kOOB;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                ac.x[i][t][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff_x[t], sx, 0));
                ac.x[i][t][1] = __builtin_bit_cast(u32x4,
                                                   __builtin_amdgcn_raw_buffer_load_b128(rx, voff_x[t] + 16, sx, 0));
            }
        }
    };
    auto issue_slot = [&](Slot &sl, int c, int rt) {
        const bool live = c < nchunks;
        // lanes past the row's end (a last, partial chunk) read nothing: an
        // offset of at least kOOB is outside the descriptor (whose size is
        // below 2^31), and the sums stay below 2^32; so are rows past R
        const int left = row_bytes - c * kChunk;
        const unsigned lane_off = lane * 16 < left ? static_cast<unsigned>(lane * 16) : static_cast<unsigned>(kOOB);
        const int sc = live ? c * kChunk : kOOB;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const unsigned vo = static_cast<unsigned>((16 * rt + 2 * wave + (j & 1)) * row_bytes) + lane_off;
            sl.p[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    (j >> 1) ? rl : rh, static_cast<int>(vo), sc, kAuxStream));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int g = c * kChunkGroups + wave + SPLIT * i;
            sl.sbits[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, (16 * rt + col) * G * 2,
                                                               live && g < G ? g * 2 : kOOB, 0);
        }
    };

    float yacc[RT][T][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) yacc[rt][t][r] = 0.0f;

    auto consume = [&](const Slot &sl, const Act &ac, int c, int rt, const unsigned char *buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int gl = wave + SPLIT * i;
            const int g = c * kChunkGroups + gl;
            if (g >= G) continue;                          // uniform
            const unsigned char *src = buf + col * kRowPitch + gl * 64 + kq * 16;
            i32x4 bhe, bho, ble, blo;
            signed16(*reinterpret_cast<const u32x4 *>(src), bhe, bho);
            if (PLANES == 2) signed16(*reinterpret_cast<const u32x4 *>(src + kRowsPerBlock * kRowPitch), ble, blo);
            const float sc = half_bits_to_float(sl.sbits[i]) * fscale;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                i32x4 ae, ao;
                split_act(ac.x[i][t][0], ac.x[i][t][1], ae, ao);
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
                if (EXPORT) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int tok = 16 * t + 4 * kq + r;
                        if (tok < M && col < rows) {
                            const size_t o = (static_cast<size_t>(tok) * N + row0 + col) * G + g;
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
                        const int pv = PLANES == 2 ? 16 * dh[r] + dl[r] : dh[r];
                        const float w = GA ? sc * sa[r] : sc;
                        yacc[rt][t][r] += static_cast<float>(pv) * w;
                    }
                }
            }
        }
    };

    // slot s = c RT + rt; the first kChunkLead slots, in slot order (no
    // scheduling across an issue)
    Slot ring[kChunkLead];
    Act act[2];
    issue_act(act[0], 0);
#pragma unroll
    for (int s = 0; s < kChunkLead; ++s) {
        if (s % RT == 0 && s > 0) issue_act(act[(s / RT) & 1], s / RT);
        issue_slot(ring[s], s / RT, s % RT);
        __builtin_amdgcn_sched_barrier(0);
    }
    // chunks are taken in pairs with no early exit (a chunk past the end
    // writes zeros, has no groups and loads nothing), so every slot's buffer
    // and registers are fixed at compile time and the load counter waits are
    // the same on every path
    for (int cb = 0; cb < nchunks; cb += 2) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = cb + e;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int d = (e * RT + rt) & 1;              // slot parity (cb RT is even)
                unsigned char *buf = lbuf + d * chunk_lds_bytes<PLANES>();
                // buffer d was last read two slots ago, before the previous
                // slot's barrier
#pragma unroll
                for (int j = 0; j < NL; ++j)
                    *reinterpret_cast<u32x4 *>(buf + ((j >> 1) * kRowsPerBlock + 2 * wave + (j & 1)) * kRowPitch +
                                               lane * 16) = ring[d].p[j];
                __syncthreads();
                consume(ring[d], act[e], c, rt, buf);
                __builtin_amdgcn_sched_barrier(0);
                // slot s + 2: tile (rt + 2) % RT of chunk c + (rt + 2) / RT;
                // a new chunk's activations go first (its register set held
                // chunk c - 1, or chunk c itself when RT = 1, both consumed)
                const int rt2 = (rt + kChunkLead) % RT;
                const int dc = (rt + kChunkLead) / RT;
                if (rt2 == 0) issue_act(act[(e + dc) & 1], c + dc);
                issue_slot(ring[d], c + dc, rt2);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    if (EXPORT) return;
    __syncthreads();                                       // the chunk buffers become the exchange
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

typedef void (*VerifyKernel)(const LinearArgs, int);

constexpr int kSplit = 8;     // waves per workgroup

// Most 16-row tiles per workgroup: every instantiation up to 8 fits the
// registers without spills (checked in the ISA), and the largest LDS need
// (8 tiles, two token tiles, grouped scales at the largest K) fits in 160 KiB.
constexpr int kMaxRowTiles = 8;
static_assert(static_cast<size_t>(kSplit) * kMaxRowTiles * 2 * 4 * 64 * 4 + (kMaxK / kGroup) * 16 * 2 * 4 <=
                  160 * 1024,
              "exchange and activation-scale table of the largest workgroup");

template <int PLANES, int T, bool GA, int RT>
VerifyKernel pick_rt_from(int rt) {
    if constexpr (RT > 1) {
        if (rt >= RT) return verify_mfma_kernel<PLANES, T, GA, false, RT>;
        return pick_rt_from<PLANES, T, GA, RT - 1>(rt);
    } else {
        return verify_mfma_kernel<PLANES, T, GA, false, 1>;
    }
}

template <int PLANES, int T>
VerifyKernel pick_rt(int rt, bool grouped, bool exporting) {
    if (exporting) return verify_mfma_kernel<PLANES, T, false, true, 1>;
    if (grouped) return pick_rt_from<PLANES, T, true, kMaxRowTiles>(rt);
    return pick_rt_from<PLANES, T, false, kMaxRowTiles>(rt);
}

constexpr int kMaxTileRule = 4;   // the whole-tile rule's largest tile count (a power of two)

// Rows per workgroup (R) and its 16-row tiles (RT). Where N spread over one
// workgroup per compute unit needs at most kMaxRowTiles tiles, every CU
// gets one workgroup of R = ceil(N / CUs) rows rounded up to 8 (N = 6144: 24
// rows on each of 256 CUs, where whole 16-row tiles would leave half of the
// CUs with two tiles and half with one; N = 28672: 112 rows, where whole
// tiles would take two rounds of residency). Otherwise whole tiles, as many
// (up to kMaxTileRule) as keep at least two workgroups per CU.
void verify_rows(int N, int cus, int *R, int *RT) {
    const int even = ((N + cus - 1) / cus + 7) & ~7;
    if (even <= kMaxRowTiles * kRowsPerBlock) {
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
    if (!export_partials) verify_rows(a.N, dev.cus, &R, &RT);
    VerifyKernel k;
    if (target)
        k = T == 1 ? pick_rt<2, 1>(RT, grouped, export_partials) : pick_rt<2, 2>(RT, grouped, export_partials);
    else
        k = T == 1 ? pick_rt<1, 1>(RT, grouped, export_partials) : pick_rt<1, 2>(RT, grouped, export_partials);
    // the two chunk buffers, reused afterwards for the partial-sum exchange
    // [kSplit][RT][T][4][64], and the grouped activation-scale table [G][16 T]
    const size_t G = a.K / kGroup;
    const size_t exchange = static_cast<size_t>(kSplit) * RT * T * 4 * 64 * 4;
    const size_t stream_lds = kChunkLead * (target ? chunk_lds_bytes<2>() : chunk_lds_bytes<1>());
    const size_t lds = (stream_lds > exchange ? stream_lds : exchange) + (grouped ? G * 16 * T * 4 : 0);
    if (lds > static_cast<size_t>(dev.max_lds)) return hipErrorInvalidValue;
    e = set_max_dynamic_lds(reinterpret_cast<const void *>(k), lds);
    if (e != hipSuccess) return e;
    const int blocks = (a.N + R - 1) / R;
    hipLaunchKernelGGL(k, dim3(blocks), dim3(64 * kSplit), lds, stream, a, R);
    return hipGetLastError();
}

}  // namespace bitnest
