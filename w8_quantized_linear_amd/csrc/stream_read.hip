// Read-only streaming kernel: the achievable HBM read rate of the access
// pattern the plane-streaming GEMV uses, with none of its arithmetic. It
// gives the per-size ceiling that the linear's plane GB/s is compared with
// (the model card's introduction counts a draft step's cost in plane bytes
// read, so the read rate of a buffer of one linear's plane size bounds it).
//
// The loads are the GEMV's: lane l reads the 16-byte slot l of a 1 KiB item
// with one non-temporal 128-bit buffer load, so one wave instruction moves
// 1 KiB. The buffer is cut into rounds of D items; each wave takes a
// contiguous run of whole rounds and keeps one round in flight while it
// folds the previous one, and issues nothing after its last round (only the
// buffer's last round can reach past the end, and those loads return zeros
// with no memory traffic). The grid is as many waves as there are rounds,
// at most the resident waves of the device. The data are folded with xor
// into one word per lane so that no load can be dropped; the word reaches
// memory only if it equals a value the caller passes (it never does for
// real data, but the compiler cannot know).
#include "bitnest_internal.h"
#include "gemv_common.h"

namespace bitnest {
namespace {

constexpr int kReadWaves = 8;

template <int D>
__global__ __launch_bounds__(64 * kReadWaves) void stream_read_kernel(const unsigned char *p, unsigned bytes,
                                                                      unsigned waves, unsigned rounds_q,
                                                                      unsigned rounds_r, unsigned never,
                                                                      unsigned *sink) {
    const unsigned gw = static_cast<unsigned>(blockIdx.x) * kReadWaves +
                        static_cast<unsigned>(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
    if (gw >= waves) return;
    const int lane = threadIdx.x & 63;
    // rounds [r0, r0 + nr): the first rounds_r waves take one more
    const unsigned r0 = gw * rounds_q + (gw < rounds_r ? gw : rounds_r);
    const unsigned nr = rounds_q + (gw < rounds_r ? 1u : 0u);
    const size_t begin = static_cast<size_t>(r0) * D * 1024;
    const unsigned run = nr * D * 1024u;
    const unsigned left = static_cast<unsigned>(bytes - begin);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(p + begin, run < left ? run : left);
    const int voff = lane * 16;
    u32x4 ring[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
        ring[d] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, d * 1024, kAuxStream));
    unsigned acc = 0;
    for (unsigned k = 1; k < nr; ++k) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            acc ^= ring[d].x ^ ring[d].y ^ ring[d].z ^ ring[d].w;
            ring[d] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, static_cast<int>((k * D + d) * 1024u),
                                                             kAuxStream));
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) acc ^= ring[d].x ^ ring[d].y ^ ring[d].z ^ ring[d].w;
    if (acc == never) sink[0] = acc;
}

typedef void (*ReadKernel)(const unsigned char *, unsigned, unsigned, unsigned, unsigned, unsigned, unsigned *);

template <int D>
hipError_t launch_depth(const void *p, size_t bytes, int waves_per_cu, unsigned never, unsigned *sink,
                        hipStream_t stream) {
    const ReadKernel k = stream_read_kernel<D>;
    DeviceInfo dev;
    hipError_t e = device_info(&dev);
    if (e != hipSuccess) return e;
    int occ = 0;
    e = occupancy(reinterpret_cast<const void *>(k), 64 * kReadWaves, 0, &occ);
    if (e != hipSuccess) return e;
    int per_cu = (occ < 1 ? 1 : occ) * kReadWaves;
    if (waves_per_cu > 0 && waves_per_cu < per_cu) per_cu = waves_per_cu;
    const size_t items = (bytes + 1023) / 1024;
    const size_t rounds = (items + D - 1) / D;
    const size_t resident = static_cast<size_t>(dev.cus) * static_cast<size_t>(per_cu);
    const unsigned waves = static_cast<unsigned>(rounds < resident ? rounds : resident);
    const unsigned blocks = (waves + kReadWaves - 1) / kReadWaves;
    hipLaunchKernelGGL(k, dim3(blocks), dim3(64 * kReadWaves), 0, stream, static_cast<const unsigned char *>(p),
                       static_cast<unsigned>(bytes), waves, static_cast<unsigned>(rounds / waves),
                       static_cast<unsigned>(rounds % waves), never, sink);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_read(const void *p, size_t bytes, int depth, int waves_per_cu, unsigned never,
                              unsigned *sink, hipStream_t stream) {
    switch (depth) {
        case 2: return launch_depth<2>(p, bytes, waves_per_cu, never, sink, stream);
        case 4: return launch_depth<4>(p, bytes, waves_per_cu, never, sink, stream);
        case 8: return launch_depth<8>(p, bytes, waves_per_cu, never, sink, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bitnest
