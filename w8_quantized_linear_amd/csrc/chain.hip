// A chain of nested linears in one launch: link j+1 reads its input only
// after every output of link j is written, exactly as if each (quantise,
// linear) pair were its own launch in stream order, but the plane stream
// does not stop at the boundaries.
//
// Operation per link (BitNest-Llama-3-8B model card, "Files",
// planes.safetensors; recipe table rows "Weights" and "Activations"): the
// activation quantisation of bitnest_quant_act (per token, or per token and
// 128-column group), then the draft (hi plane, W4 = (hi - 8) scale) or the
// target (both planes, W8 = (16 (hi - 8) + (lo - 8)) scale / 16) linear,
// with the per-group integer partials and fp32 epilogue of the
// plane-streaming GEMV in the same operation order, so every output is bit
// for bit the GEMV's.
//
// Why one launch: a decode pass is a chain of linears whose weights do not
// depend on the activations. Between two launches the device drains and
// dispatches the next grid, and HBM idles for the gap and for the next
// kernel's prologue. Here a persistent grid (one workgroup per compute unit,
// all resident) streams every wave's (row, chunk) items of all links as one
// sequence through a ring of D items in flight that runs on across link
// boundaries: while the grid waits for the last outputs of link j and
// quantises the input of link j+1, the ring already holds the first items of
// the links that follow.
//
// Waves: 8 streaming waves (rows of each link, split as in the GEMV) and one
// control wave. The streaming waves only issue plane loads and compute, so
// their in-order load counter never waits on a store or a remote read; they
// leave each finished row's outputs in LDS. At a boundary the control wave
// writes the workgroup's outputs (device-coherent stores), waits for them,
// arrives at a two-level counter (its group of workgroups, blockIdx % 8, then
// the whole grid) and polls the grid counter, with a bounded number of polls:
// on running out it sets a sticky flag in the workspace and goes on, so the
// kernel always ends. All waves then read the next input (device-coherent
// loads) and quantise it. The last arrival of the chain resets the counters.
#include "bitnest.h"
#include "bitnest_internal.h"
#include "device_common.h"
#include "gemv_common.h"

namespace bitnest {
namespace {

constexpr int kStreamWaves = 8;
constexpr int kChainWaves = kStreamWaves + 1;           // + the control wave
constexpr int kChainThreads = 64 * kChainWaves;
constexpr int kQuantThreads = 64 * kStreamWaves;        // lanes that quantise (the streaming waves')
constexpr int kTokPad = 4;                              // tokens per row of the per-group tables (M <= 4)
constexpr int kGroups = 8;                              // barrier groups of workgroups (blockIdx % 8)
constexpr int kStageRows = 256;                         // outputs staged per workgroup and token
constexpr int kCounterStride = 32;                      // one 128-byte line per counter (uint32 words)

// Cache policy of a buffer access that is coherent across the whole device
// (the sc1 bit on gfx950): a link's x may have been written by another
// compute unit earlier in the same launch.
constexpr int kAuxDevice = 16;

// s_waitcnt immediate of "vmcnt(0)" on gfx9 (expcnt and lgkmcnt left at
// their no-wait maxima)
constexpr int kWaitVmcnt0 = 0x0F70;

struct ChainArgs {
    const bitnest_chain_linear *links;   // device copy of the chain
    int count;
    int kmax;                            // largest K of the chain (LDS layout)
    unsigned *sync;                      // workspace: counters and the time-out flag
    unsigned max_polls;
};

// A link as the kernel keeps it in LDS, with the row split of the streaming
// waves: N = rows_q * (streaming waves) + rows_r.
struct LinkRec {
    const float *x;
    const uint8_t *hi;
    const uint8_t *lo;
    const uint16_t *scale;
    float *y;
    int8_t *xq;
    float *xs;
    int N, K, act_group, rows_q, rows_r, pad;
};
static_assert(sizeof(LinkRec) == 80, "LinkRec layout");

// LDS: links | codes [M][kmax] | grouped scales [kmax/128][kTokPad] |
// code sums [kmax/128][kTokPad] | per-wave maxima [8][kTokPad] | staged
// outputs [M][kStageRows]
struct ChainLds {
    __host__ __device__ static size_t links(int count) { return static_cast<size_t>(count) * sizeof(LinkRec); }
    __host__ __device__ static size_t codes(int M, int kmax) { return static_cast<size_t>(M) * kmax; }
    __host__ __device__ static size_t table(int kmax) { return static_cast<size_t>(kmax / kGroup) * kTokPad * 4; }
    __host__ __device__ static size_t part() { return static_cast<size_t>(kStreamWaves) * kTokPad * 4; }
    __host__ __device__ static size_t stage(int M) { return static_cast<size_t>(M) * kStageRows * 4; }
    static size_t bytes(int count, int M, int kmax) {
        return links(count) + codes(M, kmax) + 2 * table(kmax) + part() + stage(M);
    }
};

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <typename T>
__device__ __forceinline__ T *uni_ptr(T *p) {
    const unsigned long long v = reinterpret_cast<unsigned long long>(p);
    const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v));
    const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v >> 32));
    return reinterpret_cast<T *>((static_cast<unsigned long long>(hi) << 32) | lo);
}

// First row and row count of streaming wave sw in a link.
__device__ __forceinline__ void wave_rows(const LinkRec &r, int sw, int &rb, int &nr) {
    rb = sw * r.rows_q + min(sw, r.rows_r);
    nr = r.rows_q + (sw < r.rows_r ? 1 : 0);
}

__device__ __forceinline__ unsigned agent_load(const unsigned *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned agent_add(unsigned *p, unsigned v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void agent_store(unsigned *p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// PLANES: 1 draft chain, 2 target chain. M tokens (<= 4). D items in flight
// per streaming wave. XU: 8-column units of the fp32 input per quantising
// thread and token (covers K <= 4096 XU).
template <int PLANES, int M, int D, int XU>
__global__ __launch_bounds__(kChainThreads) void chain_kernel(const ChainArgs a) {
    static_assert(M >= 1 && M <= kTokPad, "up to four tokens");
    static_assert(D >= 1, "ring depth");
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uni(tid >> 6);
    const bool control = wave == kStreamWaves;                 // uniform
    const int G = static_cast<int>(gridDim.x);
    const int swaves = G * kStreamWaves;
    const int sw0 = static_cast<int>(blockIdx.x) * kStreamWaves;
    const int sw = sw0 + (control ? 0 : wave);
    const int count = a.count;
    const int Gmax = a.kmax >> 7;

    LinkRec *recs = reinterpret_cast<LinkRec *>(smem);
    unsigned char *act = smem + ChainLds::links(count);
    float *sact = reinterpret_cast<float *>(act + ChainLds::codes(M, a.kmax));             // [G][kTokPad]
    int *qsum = reinterpret_cast<int *>(sact + static_cast<size_t>(Gmax) * kTokPad);       // [G][kTokPad]
    float *part = reinterpret_cast<float *>(qsum + static_cast<size_t>(Gmax) * kTokPad);   // [8][kTokPad]
    float *ystage = part + kStreamWaves * kTokPad;                                         // [M][kStageRows]

    // ---- 0) the links into LDS, with each link's row split
    for (int j = tid; j < count; j += kChainThreads) {
        const bitnest_chain_linear &L = a.links[j];
        LinkRec r;
        r.x = L.x;
        r.hi = L.hi;
        r.lo = L.lo;
        r.scale = L.scale;
        r.y = L.y;
        r.xq = L.xq;
        r.xs = L.xs;
        r.N = L.N;
        r.K = L.K;
        r.act_group = L.act_group;
        r.rows_q = static_cast<int>(static_cast<unsigned>(L.N) / static_cast<unsigned>(swaves));
        r.rows_r = L.N - r.rows_q * swaves;
        r.pad = 0;
        recs[j] = r;
    }
    __syncthreads();
    // a link's fields, the same in every lane
    auto link = [&](int j, LinkRec &r) {
        const LinkRec &s = recs[uni(j)];
        r.x = uni_ptr(s.x);
        r.hi = uni_ptr(s.hi);
        r.lo = uni_ptr(s.lo);
        r.scale = uni_ptr(s.scale);
        r.y = uni_ptr(s.y);
        r.xq = uni_ptr(s.xq);
        r.xs = uni_ptr(s.xs);
        r.N = uni(s.N);
        r.K = uni(s.K);
        r.act_group = uni(s.act_group);
        r.rows_q = uni(s.rows_q);
        r.rows_r = uni(s.rows_r);
        r.pad = 0;
    };

    // ---- issue side of a streaming wave. In link j the wave owns rows
    //      [rb, rb + nr), C chunks of 1 KiB per row and plane: n = nr C
    //      items, padded to a multiple of D with empty items (loads past the
    //      end of the buffer: zeros, no memory traffic, never consumed), so
    //      every link starts at ring slot 0 and the ring index stays a
    //      compile-time constant; the issue side moves to the next link only
    //      at the start of a block of D items.
    const int voff_plane = lane * 16;
    const int voff_scale = (lane >> 2) * 2;
    int ij = -1;                     // link of the block being issued
    int i_row = 0, i_chunk = 0, i_pos = 0, i_n = 0, i_np = 0;
    int i_rowb = 0, i_G = 0, i_C = 1, i_oob = 0, i_oobs = 0;
    __amdgpu_buffer_rsrc_t rh = make_rsrc(nullptr, 0), rl = rh, rs = rh;
    // on to the next link in which this wave has items (or past the end)
    auto advance_issue = [&]() {
        i_pos = 0;
        i_n = 0;
        i_np = 0;
        while (i_np == 0 && ij + 1 < count) {
            ++ij;
            LinkRec r;
            link(ij, r);
            int rb, nr;
            wave_rows(r, sw, rb, nr);
            i_rowb = r.K >> 1;
            i_G = r.K >> 7;
            i_C = ((r.K >> 5) + 63) >> 6;
            i_n = nr * i_C;
            i_np = (i_n + D - 1) / D * D;
            i_row = rb;
            i_chunk = 0;
            const unsigned pb = static_cast<unsigned>(r.N) * static_cast<unsigned>(i_rowb);
            rh = make_rsrc(r.hi, pb);
            rl = make_rsrc(PLANES == 2 ? r.lo : r.hi, pb);
            rs = make_rsrc(r.scale, static_cast<unsigned>(r.N) * i_G * 2u);
            i_oob = static_cast<int>(pb);
            i_oobs = static_cast<int>(static_cast<unsigned>(r.N) * i_G * 2u);
        }
        if (i_np == 0) ij = count;            // past the end: every further item is empty
    };
    auto issue = [&](Item<PLANES> &x) {
        const bool live = i_pos < i_n;
        const int soff = live ? i_row * i_rowb + i_chunk * 1024 : i_oob;
        const int soff_s = live ? (i_row * i_G + i_chunk * 16) * 2 : i_oobs;
        x.h = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rh, voff_plane, soff, kAuxStream));
        if (PLANES == 2)
            x.l = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rl, voff_plane, soff, kAuxStream));
        x.sbits = __builtin_amdgcn_raw_buffer_load_b16(rs, voff_scale, soff_s, 0);
        ++i_pos;
        if (live && ++i_chunk == i_C) {
            i_chunk = 0;
            ++i_row;
        }
    };

    // ---- quantisation of a link's input into LDS (the rule of
    //      bitnest_quant_act; workgroup 0 also writes xq / xs), TB tokens at
    //      a time: the loads of a batch (load_x), then the rest (quant_x), so
    //      that the first link's loads go out ahead of the first ring
    constexpr int TBX = XU >= 4 ? 1 : (XU == 2 ? 2 : 4);
    constexpr int TB = M < TBX ? M : TBX;
    u32x4 xr[TB][XU][2];
    auto load_x = [&](const LinkRec &r, int m0) {
        const int K = r.K;
        const int nunit = K >> 3;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(r.x, static_cast<unsigned>(M) * K * 4u);
        const int oobx = M * K * 4;
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int k = 0; k < XU; ++k) {
                const int m = m0 + t;
                const int u = tid + k * kQuantThreads;
                const int off = (!control && m < M && u < nunit) ? (m * K + u * 8) * 4 : oobx;
                xr[t][k][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, kAuxDevice));
                xr[t][k][1] =
                    __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16, 0, kAuxDevice));
            }
    };
    float tok_scale[M];
    // everything after the loads of the batch at m0; ends with every code
    // and table of the batch in LDS, behind a barrier
    auto quant_x = [&](const LinkRec &r, int m0) {
        const int K = r.K;
        const int G_j = K >> 7;
        const int nunit = K >> 3;
        const int row_bytes = K >> 1;
        const bool grouped = r.act_group == kGroup;
        const bool write_out = blockIdx.x == 0 && r.xq != nullptr;   // xq and xs are given together
        float xf[TB][XU][8];
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int k = 0; k < XU; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xf[t][k][i] = __builtin_bit_cast(float, static_cast<unsigned>(xr[t][k][0][i]));
                    xf[t][k][4 + i] = __builtin_bit_cast(float, static_cast<unsigned>(xr[t][k][1][i]));
                }
        auto absmax8 = [](const float (&v)[8]) {
            float mx = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(v[i]));
            return mx;
        };
        float us[TB][XU], ur[TB][XU];
        if (grouped) {
            // a group is 16 consecutive units = one row of 16 lanes
#pragma unroll
            for (int t = 0; t < TB; ++t)
#pragma unroll
                for (int k = 0; k < XU; ++k) {
                    const int m = m0 + t;
                    const int u = tid + k * kQuantThreads;
                    us[t][k] = row16_max_f32(absmax8(xf[t][k])) / 127.0f;
                    ur[t][k] = quant_recip(us[t][k]);
                    if (!control && m < M && u < nunit && (u & 15) == 0) {
                        sact[(u >> 4) * kTokPad + m] = us[t][k];
                        if (write_out) r.xs[m * G_j + (u >> 4)] = us[t][k];
                    }
                }
#pragma unroll
            for (int t = 0; t < TB; ++t)
                if (m0 + t < M) tok_scale[m0 + t] = 1.0f;
        } else {
            // the token's maximum: DPP in each wave, then the 8 streaming
            // waves' maxima through LDS
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                float am = 0.0f;
#pragma unroll
                for (int k = 0; k < XU; ++k) am = fmaxf(am, absmax8(xf[t][k]));
                am = wave_max_dpp_f32(am);
                if (!control && lane == 0) part[wave * kTokPad + t] = am;
            }
            __syncthreads();
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                const int m = m0 + t;
                float am = part[t];
#pragma unroll
                for (int w = 1; w < kStreamWaves; ++w) am = fmaxf(am, part[w * kTokPad + t]);
                const float sc = am / 127.0f;
                const float rc = quant_recip(sc);
                if (m < M) {
                    tok_scale[m] = sc;
                    if (write_out && tid == 0) r.xs[m] = sc;
                }
#pragma unroll
                for (int k = 0; k < XU; ++k) {
                    us[t][k] = sc;
                    ur[t][k] = rc;
                }
            }
        }
        // codes -> LDS: unit u is the 8-byte [even | odd] pair (u & 1) of
        // half (u >> 1) & 1 of slot u >> 2 of the token's [2][slots][16]
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int k = 0; k < XU; ++k) {
                const int m = m0 + t;
                const int u = tid + k * kQuantThreads;
                const bool mine = !control && m < M && u < nunit;
                int cs = 0;
                if (mine) {
                    unsigned y[8];
                    quant_codes<8>(xf[t][k], us[t][k], ur[t][k], y);
                    unsigned char *dst = act + static_cast<size_t>(m) * K + ((u >> 1) & 1) * row_bytes +
                                         (u >> 2) * 16 + (u & 1) * 8;
                    *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_low_bytes(y[0], y[2], y[4], y[6]),
                                                                 pack_low_bytes(y[1], y[3], y[5], y[7]));
                    const unsigned c0 = pack_low_bytes(y[0], y[1], y[2], y[3]);
                    const unsigned c1 = pack_low_bytes(y[4], y[5], y[6], y[7]);
                    if (write_out)
                        *reinterpret_cast<uint2 *>(r.xq + static_cast<size_t>(m) * K + u * 8) = make_uint2(c0, c1);
                    if (PLANES == 2) cs = sdot4(c1, 0x01010101u, sdot4(c0, 0x01010101u, 0));
                }
                if (PLANES == 2) {
                    // a group is 16 units = one row of 16 lanes
                    cs = quad_sum_i32(cs);
                    cs += dpp_i32<kDppRowRor4>(cs);
                    cs += dpp_i32<kDppRowRor8>(cs);
                    if (mine && (u & 15) == 0) qsum[(u >> 4) * kTokPad + m] = cs;
                }
            }
        __syncthreads();   // the batch's codes and tables are in LDS; part is free again
    };

    Item<PLANES> ring[D];

    // the first link's input goes out ahead of the first ring
    LinkRec cur;
    link(0, cur);
    load_x(cur, 0);
    if (!control) {
        advance_issue();
#pragma unroll
        for (int d = 0; d < D; ++d) issue(ring[d]);
    }

    unsigned *arrivals = a.sync;                                  // the grid's counter
    unsigned *timed_out = a.sync + 1;                             // sticky time-out flag
    const int grp = static_cast<int>(blockIdx.x) & (kGroups - 1);
    unsigned *grp_count = a.sync + kCounterStride * (1 + grp);    // this group's counter
    const unsigned ngroups = static_cast<unsigned>(G < kGroups ? G : kGroups);
    const unsigned in_group = static_cast<unsigned>((G - grp + kGroups - 1) / kGroups);

    for (int j = 0; j < count; ++j) {
        if (j > 0) {
            link(j, cur);
            load_x(cur, 0);
        }
        // ---- input of link j -> codes in LDS
#pragma unroll
        for (int m0 = 0; m0 < M; m0 += TB) {
            if (m0 > 0) load_x(cur, m0);
            quant_x(cur, m0);
        }

        // ---- the streaming waves' rows of link j
        const int N = cur.N;
        const int K = cur.K;
        int r0, nr0, rb, nr;
        wave_rows(cur, sw0, r0, nr0);     // the workgroup's first row
        wave_rows(cur, sw, rb, nr);
        if (!control) {
            const int slots = K >> 5;
            const int C = (slots + 63) >> 6;
            const int tok4 = K >> 4;      // u32x4 per token
            const int half4 = K >> 5;     // u32x4 per half (= slots)
            const bool grouped = cur.act_group == kGroup;
            const u32x4 *act4 = reinterpret_cast<const u32x4 *>(act);
            float acc[M];
#pragma unroll
            for (int m = 0; m < M; ++m) acc[m] = 0.0f;
            int crow = rb, cchunk = 0;
            bool direct = false;          // rows past the staging area went straight to memory
            const __amdgpu_buffer_rsrc_t ry = make_rsrc(cur.y, static_cast<unsigned>(M) * N * 4u);
            auto consume = [&](const Item<PLANES> &x) {
                const int s = cchunk * 64 + lane;
                const bool valid = s < slots;           // uniform within each quad
                const int ss = valid ? s : 0;
                const int g = ss >> 2;
                const float sc = half_bits_to_float(static_cast<uint16_t>(x.sbits)) * 0.0625f;
                if constexpr (PLANES == 2) {
                    const Signed16 n = to_combined16(x.h, x.l);
                    const i32x4 cs = *reinterpret_cast<const i32x4 *>(qsum + g * kTokPad);
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const u32x4 a0 = act4[m * tok4 + ss];
                        const u32x4 a1 = act4[m * tok4 + half4 + ss];
                        const int p8 = quad_sum_i32(dot_slot16(n, a0, a1)) - 8 * cs[m];
                        const float w = grouped ? sc * sact[g * kTokPad + m] : sc;
                        acc[m] += valid ? static_cast<float>(p8) * w : 0.0f;
                    }
                } else {
                    const Signed16 n = to_signed16(x.h);
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const u32x4 a0 = act4[m * tok4 + ss];
                        const u32x4 a1 = act4[m * tok4 + half4 + ss];
                        const int p = quad_sum_i32(dot_slot16(n, a0, a1));
                        const float w = grouped ? sc * sact[g * kTokPad + m] : sc;
                        acc[m] += valid ? static_cast<float>(p) * w : 0.0f;
                    }
                }
                if (++cchunk == C) {                    // row complete (uniform)
                    cchunk = 0;
                    const int lr = crow - r0;           // row within the workgroup's rows
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const float v = sum_quads_to_lane63(acc[m]);
                        const float out = grouped ? v : v * tok_scale[m];
                        if (lane == 63) {
                            if (lr < kStageRows)
                                ystage[m * kStageRows + lr] = out;
                            else
                                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, out), ry,
                                                                      (m * N + crow) * 4, 0, kAuxDevice);
                        }
                        acc[m] = 0.0f;
                    }
                    if (lr >= kStageRows) direct = true;
                    ++crow;
                }
            };
            // this wave's items, D per round: the block issued in a round is
            // the next one of the link being issued, or the first block of
            // the next link with items for this wave
            // Every ring item was issued before the wait for this link, so
            // waiting for all of them here costs nothing; it also starts the
            // loop from a state the compiler's load-wait placement tracks
            // exactly (without it, the prologue's branches made it wait for
            // every load before each item).
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            const int items = nr * C;
            const int padded = (items + D - 1) / D * D;
            for (int base = 0; base < padded; base += D) {
                if (i_pos == i_np) advance_issue();
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    if (base + d < items) consume(ring[d]);    // uniform
                    issue(ring[d]);
                }
            }
            if (direct) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();                          // the workgroup's rows of link j are in LDS

        // ---- the control wave: the workgroup's outputs to memory, then the
        //      arrival, then the wait for every workgroup
        if (control) {
            int rl, nl;
            wave_rows(cur, sw0 + kStreamWaves - 1, rl, nl);
            const int rows = rl + nl - r0;        // the workgroup's rows of link j
            const int staged = rows < kStageRows ? rows : kStageRows;
            const __amdgpu_buffer_rsrc_t ry = make_rsrc(cur.y, static_cast<unsigned>(M) * N * 4u);
#pragma unroll
            for (int m = 0; m < M; ++m)
                for (int r = lane; r < staged; r += 64)
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, ystage[m * kStageRows + r]), ry,
                                                          (m * N + r0 + r) * 4, 0, kAuxDevice);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            if (lane == 0) {
                const unsigned step = static_cast<unsigned>(j + 1);
                const unsigned old = agent_add(grp_count, 1u);
                // every in_group-th arrival of a group (the last of its
                // workgroups to finish a link) carries the group to the grid
                // counter; counted this way the totals stay exact even when a
                // wait has run out and workgroups are on different links
                if ((old + 1) % in_group == 0) {
                    const unsigned g_old = agent_add(arrivals, 1u);
                    if (g_old + 1 == static_cast<unsigned>(count) * ngroups) {
                        // the chain's very last arrival: every workgroup is past
                        // its last wait, nobody reads a counter any more
                        agent_store(arrivals, 0u);
                        for (int g = 0; g < kGroups; ++g) agent_store(a.sync + kCounterStride * (1 + g), 0u);
                    }
                }
                if (j + 1 < count) {
                    const unsigned target = step * ngroups;
                    unsigned polls = 0;
                    while (agent_load(arrivals) < target) {
                        if (++polls > a.max_polls) {
                            __hip_atomic_fetch_or(timed_out, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
            }
        }
        __syncthreads();                          // link j is complete on the whole grid
    }
}

typedef void (*ChainKernel)(const ChainArgs);

// Items in flight per streaming wave (1 KiB per plane each): enough that the
// items already on their way when a link ends cover the wait and the next
// input's quantisation.
template <int PLANES>
constexpr int chain_depth() {
    return PLANES == 1 ? 8 : 4;
}

template <int PLANES, int M>
ChainKernel pick_xu(int kmax) {
    constexpr int D = chain_depth<PLANES>();
    const int xu = (kmax / 8 + kQuantThreads - 1) / kQuantThreads;
    if (xu <= 1) return chain_kernel<PLANES, M, D, 1>;
    if (xu <= 2) return chain_kernel<PLANES, M, D, 2>;
    return chain_kernel<PLANES, M, D, 4>;
}

template <int PLANES>
ChainKernel pick_m(int M, int kmax) {
    switch (M) {
        case 1: return pick_xu<PLANES, 1>(kmax);
        case 2: return pick_xu<PLANES, 2>(kmax);
        case 3: return pick_xu<PLANES, 3>(kmax);
        case 4: return pick_xu<PLANES, 4>(kmax);
        default: return nullptr;
    }
}

}  // namespace

size_t chain_lds_bytes(int count, int M, int kmax) { return ChainLds::bytes(count, M, kmax); }

hipError_t launch_chain(const bitnest_chain_linear *links_dev, int count, int M, bool target, int kmax,
                        unsigned *sync, unsigned max_polls, hipStream_t stream) {
    static_assert(kMaxK / 8 <= 4 * kQuantThreads, "four units per thread cover the widest input");
    static_assert(kCounterStride * (1 + kGroups) * 4 <= BITNEST_CHAIN_WORKSPACE_BYTES, "workspace holds the counters");
    const ChainKernel k = target ? pick_m<2>(M, kmax) : pick_m<1>(M, kmax);
    if (!k) return hipErrorInvalidValue;
    DeviceInfo dev;
    hipError_t e = device_info(&dev);
    if (e != hipSuccess) return e;
    const size_t lds = ChainLds::bytes(count, M, kmax);
    if (lds > static_cast<size_t>(dev.max_lds)) return hipErrorInvalidValue;
    e = set_max_dynamic_lds(reinterpret_cast<const void *>(k), lds);
    if (e != hipSuccess) return e;
    const ChainArgs args{links_dev, count, kmax, sync, max_polls};
    // one workgroup per compute unit: all of them resident together, which
    // the waits between links rely on (and bound)
    hipLaunchKernelGGL(k, dim3(dev.cus), dim3(kChainThreads), lds, stream, args);
    return hipGetLastError();
}

}  // namespace bitnest
