// Device pieces shared by the plane-streaming kernels (the per-linear GEMV
// and the chain kernel that runs a sequence of linears in one launch): the
// operands of one 16-byte plane slot, their exact dot products with the
// even/odd-split activation codes, and the buffer descriptors of the item
// stream. Layout and formulas: BitNest-Llama-3-8B model card, "Files",
// planes.safetensors (byte j of a plane row holds column 2j in its low
// nibble and 2j+1 in its high nibble; W4 = (hi - 8) scale, W8 =
// (16 (hi - 8) + (lo - 8)) scale / 16).
#pragma once

#include "device_common.h"

namespace bitnest {

constexpr unsigned kHighNibbles = 0xF0F0F0F0u;

// v_perm_b32 selectors: bytes {0,2} of lo and {0,2} of hi (even columns),
// and bytes {1,3}, {1,3} (odd columns).
constexpr unsigned kSelEven = 0x06040200u;
constexpr unsigned kSelOdd = 0x07050301u;

// Signed operands of one 16-byte plane slot (32 columns). A nibble u holds
// the code u - 8; xor 0x8 turns it into the 4-bit two's complement of u - 8,
// and placing that in the high half of a byte gives the int8 value
// 16 * (u - 8). e[d] / o[d] hold the even / odd columns of weight dword d.
struct Signed16 {
    unsigned e[4], o[4];
};

__device__ __forceinline__ Signed16 to_signed16(const u32x4 w) {
    Signed16 n;
    const unsigned x0 = w.x ^ 0x88888888u, x1 = w.y ^ 0x88888888u;
    const unsigned x2 = w.z ^ 0x88888888u, x3 = w.w ^ 0x88888888u;
    n.e[0] = (x0 << 4) & kHighNibbles; n.o[0] = x0 & kHighNibbles;
    n.e[1] = (x1 << 4) & kHighNibbles; n.o[1] = x1 & kHighNibbles;
    n.e[2] = (x2 << 4) & kHighNibbles; n.o[2] = x2 & kHighNibbles;
    n.e[3] = (x3 << 4) & kHighNibbles; n.o[3] = x3 & kHighNibbles;
    return n;
}

// 16 * sum over the slot's 32 columns of q * (u - 8), exact, with the
// activation halves a0 = [e0 o0 e1 o1], a1 = [e2 o2 e3 o3] as staged in LDS.
__device__ __forceinline__ int dot_slot16(const Signed16 &n, const u32x4 a0, const u32x4 a1) {
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

// Target operands of one 16-byte slot of each plane: one signed byte per
// column, 16 (hi - 8) + lo in [-128, 127] (the hi nibble xor 8 in the high
// half, the unsigned lo nibble in the low half), so that one dot product per
// dword covers both planes: sum q * (16 (hi - 8) + lo) = P8 + 8 sum(q).
__device__ __forceinline__ Signed16 to_combined16(const u32x4 h, const u32x4 l) {
    Signed16 n;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const unsigned hx = h[d] ^ 0x88888888u, lw = l[d];
        n.e[d] = ((hx << 4) & kHighNibbles) | (lw & ~kHighNibbles);
        n.o[d] = (hx & kHighNibbles) | ((lw >> 4) & ~kHighNibbles);
    }
    return n;
}

// Buffer descriptor over [p, p + bytes): loads beyond it return 0 (gfx9 raw
// buffer, dword 3 = 0x00020000).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

constexpr int kAuxStream = 2;   // non-temporal: plane bytes are read once

// Sum over the 16 quads of a wave of a value that is uniform within each
// quad; the total lands in lane 63. Fixed association order.
__device__ __forceinline__ float sum_quads_to_lane63(float v) {
    v += dpp_f32<kDppRowRor4>(v);
    v += dpp_f32<kDppRowRor8>(v);
    v += dpp_f32_masked<kDppRowBcast15, 0xA>(v);
    v += dpp_f32_masked<kDppRowBcast31, 0xC>(v);
    return v;
}

// Permute one 16-column code block into its LDS place: columns 16 j .. 16 j + 15
// of a token are half (j & 1) of slot (j >> 1), split into even and odd columns.
__device__ __forceinline__ void stage_block(unsigned char *act_tok, int j, int row_bytes, const u32x4 v) {
    u32x4 o;
    o.x = __builtin_amdgcn_perm(v.y, v.x, kSelEven);
    o.y = __builtin_amdgcn_perm(v.y, v.x, kSelOdd);
    o.z = __builtin_amdgcn_perm(v.w, v.z, kSelEven);
    o.w = __builtin_amdgcn_perm(v.w, v.z, kSelOdd);
    *reinterpret_cast<u32x4 *>(act_tok + (j & 1) * row_bytes + (j >> 1) * 16) = o;
}

// One item = one 1 KiB chunk of one row, per plane: lane l holds 16 bytes,
// plus the fp16 bits of its group's scale (converted when consumed, so that
// no load result is needed before the next loads are issued).
template <int PLANES>
struct Item {
    u32x4 h, l;
    unsigned sbits;
};

}  // namespace bitnest
