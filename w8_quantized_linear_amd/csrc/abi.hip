// C ABI of the nested W4/W8 linear (declared and documented in bitnest.h).
// Arguments are validated on the host before any HIP call; then the call is
// dispatched by M: the plane-streaming GEMV for M <= 7, the int8 matrix-core
// kernel for 8 <= M <= 32.
#include "bitnest.h"
#include "bitnest_internal.h"

#include <atomic>
#include <cmath>
#include <map>
#include <mutex>
#include <tuple>

namespace bitnest {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];
std::atomic<int> g_lds[kMaxDevices];

// Host-side facts about a kernel on a device, looked up once: whether its
// dynamic-LDS limit has been raised, and its occupancy per LDS size.
std::mutex g_kernel_mutex;
std::map<std::pair<const void *, int>, bool> g_lds_raised;
std::map<std::tuple<const void *, int, int, size_t>, int> g_occupancy;
}  // namespace

// The two lookups below are the library's only code that can throw (a map
// insertion, a mutex); they answer with an error code instead, so nothing
// throws across the C boundary.
hipError_t set_max_dynamic_lds(const void *kernel, size_t bytes) try {
    if (bytes <= 65536) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    DeviceInfo info;
    e = device_info(&info);
    if (e != hipSuccess) return e;
    if (bytes > static_cast<size_t>(info.max_lds)) return hipErrorInvalidValue;
    std::lock_guard<std::mutex> lock(g_kernel_mutex);
    const auto key = std::make_pair(kernel, dev);
    if (g_lds_raised.count(key)) return hipSuccess;
    // raised once to the device's limit, so every later size fits
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, info.max_lds);
    if (e != hipSuccess) return e;
    g_lds_raised[key] = true;
    return hipSuccess;
} catch (...) {
    return hipErrorUnknown;
}

hipError_t occupancy(const void *kernel, int threads, size_t lds, int *out) try {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const auto key = std::make_tuple(kernel, dev, threads, lds);
    {
        std::lock_guard<std::mutex> lock(g_kernel_mutex);
        const auto it = g_occupancy.find(key);
        if (it != g_occupancy.end()) {
            *out = it->second;
            return hipSuccess;
        }
    }
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, lds);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_kernel_mutex);
    g_occupancy[key] = occ;
    *out = occ;
    return hipSuccess;
} catch (...) {
    return hipErrorUnknown;
}

hipError_t device_info(DeviceInfo *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int cus = g_cus[dev].load(std::memory_order_acquire);
    int lds = g_lds[dev].load(std::memory_order_acquire);
    if (cus <= 0 || lds <= 0) {
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (e != hipSuccess) return e;
        g_cus[dev].store(cus, std::memory_order_release);
        g_lds[dev].store(lds, std::memory_order_release);
    }
    out->cus = cus;
    out->max_lds = lds;
    return hipSuccess;
}

}  // namespace bitnest

namespace {

using bitnest::kGroup;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared size checks for the linear calls. Returns BITNEST_OK or an error.
bitnest_status check_sizes(int M, int N, int K) {
    if (M < 0 || N < 0 || K <= 0 || K % kGroup != 0) return BITNEST_EINVAL;
    if (M > BITNEST_MAX_M || K > BITNEST_MAX_K) return BITNEST_EUNSUPPORTED;
    // plane offsets are 32-bit in the kernels
    if (static_cast<long long>(N) * (K / 2) > static_cast<long long>(BITNEST_MAX_PLANE_BYTES))
        return BITNEST_EUNSUPPORTED;
    return BITNEST_OK;
}

bitnest_status to_status(hipError_t e) { return e == hipSuccess ? BITNEST_OK : BITNEST_EHIP; }

// Rotation block of the R4 calls: a power of two, 2 <= block <= the largest
// supported, dividing K.
bool valid_rot_block(int block, int K) {
    return block >= 2 && block <= BITNEST_MAX_ROT_BLOCK && (block & (block - 1)) == 0 && K % block == 0;
}

// The fp32 value nearest 1 / sqrt(block) (block a power of two).
float rot_scale_of(int block) { return static_cast<float>(1.0 / std::sqrt(static_cast<double>(block))); }

bitnest_status run_linear(const bitnest::LinearArgs &a, bool exporting, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.M <= bitnest::kGemvMaxM) return to_status(bitnest::launch_gemv(a, exporting, s));
    return to_status(bitnest::launch_verify_mfma(a, exporting, s));
}

}  // namespace

extern "C" {

int bitnest_abi_version(void) { return BITNEST_ABI_VERSION; }

const char *bitnest_status_string(int status) {
    switch (status) {
        case BITNEST_OK: return "ok";
        case BITNEST_EINVAL: return "invalid argument (null pointer, negative size, K not a positive multiple of 128, act_group not 0/128, or an invalid rotation block)";
        case BITNEST_EALIGN: return "tensor pointer not 16-byte aligned";
        case BITNEST_EUNSUPPORTED: return "size beyond the library limits (M > BITNEST_MAX_M or K > BITNEST_MAX_K)";
        case BITNEST_EHIP: return "HIP runtime error while launching";
        default: return "unknown status";
    }
}

bitnest_status bitnest_quant_act(const float *x, int M, int K, int act_group, int8_t *xq, float *xs,
                                 void *stream) {
    if (act_group != 0 && act_group != kGroup) return BITNEST_EINVAL;
    // quantisation takes any number of tokens; only K is bounded
    if (M < 0 || K <= 0 || K % kGroup != 0) return BITNEST_EINVAL;
    if (K > BITNEST_MAX_K) return BITNEST_EUNSUPPORTED;
    if (M == 0) return BITNEST_OK;                  // empty: pointers may be NULL
    if (!x || !xq || !xs) return BITNEST_EINVAL;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(xs)) return BITNEST_EALIGN;
    return to_status(bitnest::launch_quant_act(x, M, K, act_group, xq, xs, static_cast<hipStream_t>(stream)));
}

bitnest_status bitnest_linear_draft(const int8_t *xq, const float *xs, int act_group, const uint8_t *hi,
                                    const uint16_t *scale, float *y, int M, int N, int K, void *stream) {
    if (act_group != 0 && act_group != kGroup) return BITNEST_EINVAL;
    bitnest_status st = check_sizes(M, N, K);
    if (st != BITNEST_OK) return st;
    if (M == 0 || N == 0) return BITNEST_OK;        // empty: pointers may be NULL
    if (!xq || !xs || !hi || !scale || !y) return BITNEST_EINVAL;
    if (!aligned16(xq) || !aligned16(xs) || !aligned16(hi) || !aligned16(scale) || !aligned16(y))
        return BITNEST_EALIGN;
    bitnest::LinearArgs a{xq, xs, hi, nullptr, scale, y, nullptr, nullptr, nullptr, M, N, K, act_group};
    return run_linear(a, false, stream);
}

bitnest_status bitnest_linear_target(const int8_t *xq, const float *xs, int act_group, const uint8_t *hi,
                                     const uint8_t *lo, const uint16_t *scale, float *y, int M, int N, int K,
                                     void *stream) {
    if (act_group != 0 && act_group != kGroup) return BITNEST_EINVAL;
    bitnest_status st = check_sizes(M, N, K);
    if (st != BITNEST_OK) return st;
    if (M == 0 || N == 0) return BITNEST_OK;        // empty: pointers may be NULL
    if (!xq || !xs || !hi || !lo || !scale || !y) return BITNEST_EINVAL;
    if (!aligned16(xq) || !aligned16(xs) || !aligned16(hi) || !aligned16(lo) || !aligned16(scale) ||
        !aligned16(y))
        return BITNEST_EALIGN;
    bitnest::LinearArgs a{xq, xs, hi, lo, scale, y, nullptr, nullptr, nullptr, M, N, K, act_group};
    return run_linear(a, false, stream);
}

}  // extern "C"

namespace {

// Shared body of the fused calls: (rotate and) quantise, then the linear;
// one launch when the fused GEMV takes the shape. rot_block 0: no rotation.
bitnest_status quant_linear(const float *x, int act_group, int rot_block, const uint8_t *hi, const uint8_t *lo,
                            const uint16_t *scale, float *y, int8_t *xq, float *xs, int M, int N, int K,
                            void *stream) {
    if (act_group != 0 && act_group != kGroup) return BITNEST_EINVAL;
    if (rot_block != 0 && (act_group != 0 || !valid_rot_block(rot_block, K))) return BITNEST_EINVAL;
    bitnest_status st = check_sizes(M, N, K);
    if (st != BITNEST_OK) return st;
    if (M == 0) return BITNEST_OK;                  // empty: pointers may be NULL
    if (!x || !xq || !xs) return BITNEST_EINVAL;
    if (N > 0 && (!hi || !scale || !y)) return BITNEST_EINVAL;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(xs)) return BITNEST_EALIGN;
    if (N > 0 && (!aligned16(hi) || !aligned16(scale) || !aligned16(y) || (lo && !aligned16(lo))))
        return BITNEST_EALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const float rs = rot_block ? rot_scale_of(rot_block) : 0.0f;
    bitnest::LinearArgs a{xq, xs, hi, lo, scale, y, nullptr, nullptr, nullptr, M, N, K, act_group, x, xq, xs,
                          rot_block, rs};
    if (N > 0 && bitnest::fused_in_one_launch(M, N, K, rot_block))
        return to_status(bitnest::launch_gemv_fused(a, s));
    if (rot_block)
        st = to_status(bitnest::launch_hadamard_quant_act(x, M, K, rot_block, rs, xq, xs, nullptr, s));
    else
        st = to_status(bitnest::launch_quant_act(x, M, K, act_group, xq, xs, s));
    if (st != BITNEST_OK || N == 0) return st;
    return run_linear(a, false, stream);
}

}  // namespace

extern "C" {

bitnest_status bitnest_quant_linear_draft(const float *x, int act_group, const uint8_t *hi, const uint16_t *scale,
                                          float *y, int8_t *xq, float *xs, int M, int N, int K, void *stream) {
    return quant_linear(x, act_group, 0, hi, nullptr, scale, y, xq, xs, M, N, K, stream);
}

bitnest_status bitnest_quant_linear_target(const float *x, int act_group, const uint8_t *hi, const uint8_t *lo,
                                           const uint16_t *scale, float *y, int8_t *xq, float *xs, int M, int N,
                                           int K, void *stream) {
    if (M > 0 && N > 0 && !lo) return BITNEST_EINVAL;
    return quant_linear(x, act_group, 0, hi, lo, scale, y, xq, xs, M, N, K, stream);
}

bitnest_status bitnest_hadamard_quant_act(const float *x, int M, int K, int block, int8_t *xq, float *xs,
                                          float *xr, void *stream) {
    // like bitnest_quant_act: any number of tokens, K bounded
    if (M < 0 || K <= 0 || K % kGroup != 0) return BITNEST_EINVAL;
    if (!valid_rot_block(block, K)) return BITNEST_EINVAL;
    if (K > BITNEST_MAX_K) return BITNEST_EUNSUPPORTED;
    if (M == 0) return BITNEST_OK;                  // empty: pointers may be NULL
    if (!x || !xq || !xs) return BITNEST_EINVAL;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(xs) || (xr && !aligned16(xr))) return BITNEST_EALIGN;
    return to_status(bitnest::launch_hadamard_quant_act(x, M, K, block, rot_scale_of(block), xq, xs, xr,
                                                        static_cast<hipStream_t>(stream)));
}

bitnest_status bitnest_hadamard_quant_linear_draft(const float *x, int block, const uint8_t *hi,
                                                   const uint16_t *scale, float *y, int8_t *xq, float *xs, int M,
                                                   int N, int K, void *stream) {
    if (block == 0) return BITNEST_EINVAL;
    return quant_linear(x, 0, block, hi, nullptr, scale, y, xq, xs, M, N, K, stream);
}

bitnest_status bitnest_hadamard_quant_linear_target(const float *x, int block, const uint8_t *hi,
                                                    const uint8_t *lo, const uint16_t *scale, float *y, int8_t *xq,
                                                    float *xs, int M, int N, int K, void *stream) {
    if (block == 0) return BITNEST_EINVAL;
    if (M > 0 && N > 0 && !lo) return BITNEST_EINVAL;
    return quant_linear(x, 0, block, hi, lo, scale, y, xq, xs, M, N, K, stream);
}

bitnest_status bitnest_pack_nested(const float *W, int N, int K, uint8_t *hi, uint8_t *lo, uint16_t *scale,
                                   void *stream) {
    if (N < 0 || K <= 0 || K % kGroup != 0) return BITNEST_EINVAL;
    if (static_cast<long long>(N) * (K / 2) > static_cast<long long>(BITNEST_MAX_PLANE_BYTES))
        return BITNEST_EUNSUPPORTED;
    if (N == 0) return BITNEST_OK;                  // empty: pointers may be NULL
    if (!W || !hi || !lo || !scale) return BITNEST_EINVAL;
    if (!aligned16(W) || !aligned16(hi) || !aligned16(lo) || !aligned16(scale)) return BITNEST_EALIGN;
    return to_status(bitnest::launch_pack_nested(W, N, K, hi, lo, scale, static_cast<hipStream_t>(stream)));
}

size_t bitnest_greedy_accept_workspace_bytes(int R, int V) {
    if (R < 1 || V < 1 || R > BITNEST_MAX_M || V > BITNEST_ACCEPT_MAX_V) return 0;
    return bitnest::accept_workspace_bytes(R, V);
}

bitnest_status bitnest_greedy_accept(const float *logits, int R, int V, const int32_t *draft, int32_t *targ,
                                     int32_t *result, void *work, size_t work_bytes, void *stream) {
    if (R < 1 || V < 1) return BITNEST_EINVAL;
    if (R > BITNEST_MAX_M || V > BITNEST_ACCEPT_MAX_V) return BITNEST_EUNSUPPORTED;
    if (!logits || !targ || !result || !work || (R > 1 && !draft)) return BITNEST_EINVAL;
    if (work_bytes < bitnest::accept_workspace_bytes(R, V)) return BITNEST_EINVAL;
    if (!aligned16(logits) || !aligned16(targ) || !aligned16(result) || !aligned16(work) ||
        (draft && !aligned16(draft)))
        return BITNEST_EALIGN;
    return to_status(bitnest::launch_greedy_accept(logits, R, V, draft, targ, result, work,
                                                   static_cast<hipStream_t>(stream)));
}

bitnest_status bitnest_greedy_accept_noalloc(const float *logits, int R, int V, const int32_t *draft,
                                             int32_t *targ, int32_t *result, void *stream) {
    if (R < 1 || V < 1) return BITNEST_EINVAL;
    if (R > BITNEST_MAX_M || V > BITNEST_ACCEPT_MAX_V) return BITNEST_EUNSUPPORTED;
    if (bitnest::accept_workspace_bytes(R, V) > BITNEST_ACCEPT_NOALLOC_SCRATCH_BYTES) return BITNEST_EUNSUPPORTED;
    if (!logits || !targ || !result || (R > 1 && !draft)) return BITNEST_EINVAL;
    if (!aligned16(logits) || !aligned16(targ) || !aligned16(result) || (draft && !aligned16(draft)))
        return BITNEST_EALIGN;
    return to_status(bitnest::launch_greedy_accept_noalloc(logits, R, V, draft, targ, result,
                                                           static_cast<hipStream_t>(stream)));
}

bitnest_status bitnest_stream_read(const void *p, size_t bytes, int depth, int waves_per_cu, uint32_t never,
                                   uint32_t *sink, void *stream) {
    if (!p || !sink || bytes < 1024 || bytes % 1024 != 0 || bytes > 0xFFFFFC00ull) return BITNEST_EINVAL;
    if ((depth != 2 && depth != 4 && depth != 8) || waves_per_cu < 0) return BITNEST_EINVAL;
    if (!aligned16(p)) return BITNEST_EALIGN;
    return to_status(bitnest::launch_stream_read(p, bytes, depth, waves_per_cu, never, sink,
                                                 static_cast<hipStream_t>(stream)));
}

size_t bitnest_kv_attention_workspace_bytes(int M, int Hq, int T) {
    if (M < 1 || Hq < 1 || T < 1) return 0;
    return bitnest::kv_attention_workspace_bytes(M, Hq, T);
}

bitnest_status bitnest_kv_attention(const float *q, int M, int Hq, int Hkv, int T, int t_cap, const uint8_t *k_hi,
                                    const uint8_t *k_lo, const uint16_t *k_scale, const uint8_t *v_hi,
                                    const uint8_t *v_lo, const uint16_t *v_scale, float *out, void *work,
                                    size_t work_bytes, void *stream) {
    if (M < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || T < M || t_cap < T) return BITNEST_EINVAL;
    if (static_cast<long long>(M) * (Hq / Hkv) > BITNEST_KV_MAX_ROWS || Hkv > 65535) return BITNEST_EUNSUPPORTED;
    if (static_cast<long long>(T) * (BITNEST_KV_HEAD_DIM / 2) > 0x7FFFFFFFLL) return BITNEST_EUNSUPPORTED;
    if (!q || !k_hi || !k_scale || !v_hi || !v_scale || !out || !work) return BITNEST_EINVAL;
    if ((k_lo == nullptr) != (v_lo == nullptr)) return BITNEST_EINVAL;
    if (work_bytes < bitnest::kv_attention_workspace_bytes(M, Hq, T)) return BITNEST_EINVAL;
    if (!aligned16(q) || !aligned16(k_hi) || !aligned16(k_scale) || !aligned16(v_hi) || !aligned16(v_scale) ||
        !aligned16(out) || !aligned16(work) || (k_lo && (!aligned16(k_lo) || !aligned16(v_lo))))
        return BITNEST_EALIGN;
    bitnest::KvArgs a{q, k_hi, k_lo, k_scale, v_hi, v_lo, v_scale, out, static_cast<float *>(work),
                      M, Hq, Hkv, T, t_cap,
                      static_cast<float>(1.0 / std::sqrt(static_cast<double>(BITNEST_KV_HEAD_DIM)))};
    return to_status(bitnest::launch_kv_attention(a, static_cast<hipStream_t>(stream)));
}

bitnest_status bitnest_linear_chain(const bitnest_chain_linear *links, const bitnest_chain_linear *links_dev,
                                    int count, int M, uint32_t max_polls, void *work, size_t work_bytes,
                                    void *stream) {
    if (count < 0) return BITNEST_EINVAL;
    if (count > BITNEST_CHAIN_MAX_LINEARS) return BITNEST_EUNSUPPORTED;
    if (count == 0) return BITNEST_OK;
    if (M < 1) return BITNEST_EINVAL;
    if (M > BITNEST_CHAIN_MAX_M) return BITNEST_EUNSUPPORTED;
    if (!links || !links_dev || !work || work_bytes < BITNEST_CHAIN_WORKSPACE_BYTES) return BITNEST_EINVAL;
    if (!aligned16(links_dev) || !aligned16(work)) return BITNEST_EALIGN;
    // the kind of the chain: that of its links with rows (a link with N == 0
    // only quantises, and its weight pointers are not read)
    int first = 0;
    while (first < count && links[first].N == 0) ++first;
    const bool target = first < count && links[first].lo != nullptr;
    int kmax = 0;
    for (int j = 0; j < count; ++j) {
        const bitnest_chain_linear &L = links[j];
        if (L.N > 0 && (L.lo != nullptr) != target) return BITNEST_EINVAL;      // one kind per chain
        if (L.act_group != 0 && L.act_group != kGroup) return BITNEST_EINVAL;
        if (L.rot_block != 0) return BITNEST_EUNSUPPORTED;
        const bitnest_status st = check_sizes(M, L.N, L.K);
        if (st != BITNEST_OK) return st;
        if (!L.x || (L.xq == nullptr) != (L.xs == nullptr)) return BITNEST_EINVAL;
        if (L.N > 0 && (!L.hi || !L.scale || !L.y)) return BITNEST_EINVAL;
        if (!aligned16(L.x) || (L.xq && (!aligned16(L.xq) || !aligned16(L.xs)))) return BITNEST_EALIGN;
        if (L.N > 0 && (!aligned16(L.hi) || !aligned16(L.scale) || !aligned16(L.y) || (target && !aligned16(L.lo))))
            return BITNEST_EALIGN;
        if (L.K > kmax) kmax = L.K;
    }
    const unsigned polls = max_polls ? max_polls : BITNEST_CHAIN_DEFAULT_POLLS;
    return to_status(bitnest::launch_chain(links_dev, count, M, target, kmax, static_cast<unsigned *>(work), polls,
                                           static_cast<hipStream_t>(stream)));
}

size_t bitnest_chain_workspace_bytes(void) { return BITNEST_CHAIN_WORKSPACE_BYTES; }

bitnest_status bitnest_linear_partials(const int8_t *xq, const uint8_t *hi, const uint8_t *lo, int32_t *p_hi,
                                       int32_t *p_lo, int32_t *p8, int M, int N, int K, void *stream) {
    bitnest_status st = check_sizes(M, N, K);
    if (st != BITNEST_OK) return st;
    if (M == 0 || N == 0) return BITNEST_OK;        // empty: pointers may be NULL
    if (!xq || !hi || !p_hi) return BITNEST_EINVAL;
    if (lo && (!p_lo || !p8)) return BITNEST_EINVAL;
    if (!aligned16(xq) || !aligned16(hi) || !aligned16(p_hi)) return BITNEST_EALIGN;
    if (lo && (!aligned16(lo) || !aligned16(p_lo) || !aligned16(p8))) return BITNEST_EALIGN;
    bitnest::LinearArgs a{xq, nullptr, hi, lo, nullptr, nullptr, p_hi, lo ? p_lo : nullptr, lo ? p8 : nullptr,
                          M, N, K, 0};
    return run_linear(a, true, stream);
}

}  // extern "C"
