// Internal interface between the C ABI (abi.hip) and the gfx950 kernels.
// Not installed; the public interface is include/bitnest.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitnest {

constexpr int kGroup = 128;     // columns per weight scale and per grouped act scale
constexpr int kGemvMaxM = 7;    // tokens handled by the plane-streaming GEMV
constexpr int kMaxM = 32;       // tokens handled by the batched-verify matrix-core kernel
constexpr int kMaxK = 16384;

// Per-device facts the launchers need, read once per device.
struct DeviceInfo {
    int cus = 0;                // compute units
    int max_lds = 0;            // bytes of LDS one workgroup may use
};
hipError_t device_info(DeviceInfo *out);

// Raise a kernel's dynamic-LDS limit on the current device when a launch
// needs more than 64 KiB (once per kernel and device).
hipError_t set_max_dynamic_lds(const void *kernel, size_t bytes);

// Workgroups of `threads` threads with `lds` bytes of dynamic LDS that fit on
// one compute unit of the current device (looked up once and kept).
hipError_t occupancy(const void *kernel, int threads, size_t lds, int *out);

// Everything a linear launch needs. Pointers are device pointers.
struct LinearArgs {
    const int8_t *xq;
    const float *xs;
    const uint8_t *hi;
    const uint8_t *lo;          // nullptr: draft
    const uint16_t *scale;
    float *y;
    int32_t *p_hi;              // partials export (nullptr unless exporting)
    int32_t *p_lo;
    int32_t *p8;
    int M, N, K;
    int act_group;              // 0 or 128
    // fused activation quantisation (launch_gemv_fused): fp32 input; the
    // codes and scales are also written to xq_out / xs_out
    const float *x;
    int8_t *xq_out;
    float *xs_out;
    // R4 rotation of the fp32 input before its quantisation (fused launch
    // only): block size (0 = none) and the fp32 value nearest 1/sqrt(block)
    int rot_block;
    float rot_scale;
    // set by the plane-streaming GEMV's launcher: N = rows_q * waves + rows_r
    // over the launch's waves
    int rows_q;
    int rows_r;
};

constexpr int kMaxRotBlock = 512;   // a rotation block stays inside one wave (64 lanes x 8)

hipError_t launch_quant_act(const float *x, int M, int K, int act_group, int8_t *xq, float *xs,
                            hipStream_t stream);

// R4 rotation (blocks of `block` columns, scaled by rot_scale) then per-token
// quantisation; xr (may be null) receives the rotated fp32 values.
hipError_t launch_hadamard_quant_act(const float *x, int M, int K, int block, float rot_scale, int8_t *xq,
                                     float *xs, float *xr, hipStream_t stream);

// fp32 weights [N, K] -> nested planes hi, lo [N, K/2] and fp16 scales [N, K/128].
hipError_t launch_pack_nested(const float *W, int N, int K, uint8_t *hi, uint8_t *lo, uint16_t *scale,
                              hipStream_t stream);

// Greedy verification: target argmax per row of logits [R, V] -> targ [R];
// result = {accepted count, next token}.
// work: accept_workspace_bytes(R, V) bytes of per-slice partials.
size_t accept_workspace_bytes(int R, int V);
hipError_t launch_greedy_accept(const float *logits, int R, int V, const int32_t *draft, int32_t *targ,
                                int32_t *result, void *work, hipStream_t stream);
// The same with the library's own per-device scratch (a static device array
// of accept_noalloc_scratch_bytes(), enough for R <= kMaxM and any V): no
// allocation; calls that overlap on one device race on it.
size_t accept_noalloc_scratch_bytes();
hipError_t launch_stream_read(const void *p, size_t bytes, int depth, int waves_per_cu, unsigned never,
                              unsigned *sink, hipStream_t stream);
hipError_t launch_greedy_accept_noalloc(const float *logits, int R, int V, const int32_t *draft, int32_t *targ,
                                        int32_t *result, hipStream_t stream);

// Decode attention over the nested KV cache.
constexpr int kKvHeadDim = 128;
constexpr int kKvChunk = 64;        // positions per chunk; a split (one partial) is a run of chunks
constexpr int kKvMaxRows = 16;      // M x (Hq / Hkv) query rows per KV head
struct KvArgs {
    const float *q;                 // [M, Hq, 128]
    const uint8_t *k_hi, *k_lo;     // [Hkv, t_cap, 64] (k_lo, v_lo null: KV4)
    const uint16_t *k_scale;        // [Hkv, t_cap]
    const uint8_t *v_hi, *v_lo;
    const uint16_t *v_scale;
    float *out;                     // [M, Hq, 128]
    float *work;                    // kv_attention_workspace_bytes(M, Hq, T)
    int M, Hq, Hkv, T;
    int t_cap;                      // positions per head in the cache, >= T
    float inv_sqrt_d;
};
size_t kv_attention_workspace_bytes(int M, int Hq, int T);
hipError_t launch_kv_attention(const KvArgs &a, hipStream_t stream);

// M <= kGemvMaxM. export_partials selects the integer export instead of y.
hipError_t launch_gemv(const LinearArgs &a, bool export_partials, hipStream_t stream);

// Activation quantisation fused into the GEMV prologue: every workgroup
// quantises the fp32 input itself and workgroup 0 writes the codes and
// scales to a.xq_out / a.xs_out. Worth it only while the per-workgroup
// quantisation is small next to the launch it saves: on MI355X that holds
// for one token (M == 1) and not for the 4-token verify batch. Other shapes
// return hipErrorNotSupported; the caller then runs launch_quant_act and a
// linear launch.
constexpr int kFusedMaxMK = 16384;
// Several tokens fit one launch when each thread holds one 8-column unit of
// every token (K <= 8 units x 512 threads), without the rotation, and when a
// wave has few rows: the one-launch grid is one 8-wave workgroup per CU, and
// with many rows per wave (gate_up's 28672 over 2048 waves) the two-launch
// linear, sized by occupancy, streams faster than the saved launch is worth.
constexpr int kFusedMaxTokens = 4;
constexpr int kFusedMaxTokensK = 4096;
constexpr int kFusedMaxTokensN = 8192;
inline bool fused_in_one_launch(int M, int N, int K, int rot_block) {
    return (M == 1 && K <= kFusedMaxMK) || (rot_block == 0 && M >= 1 && M <= kFusedMaxTokens &&
                                            K <= kFusedMaxTokensK && N <= kFusedMaxTokensN);
}
hipError_t launch_gemv_fused(const LinearArgs &a, hipStream_t stream);

// 8 <= M <= kMaxM.
hipError_t launch_verify_mfma(const LinearArgs &a, bool export_partials, hipStream_t stream);

}  // namespace bitnest

struct bitnest_chain_linear;

namespace bitnest {

// A chain of quantise + linear steps in one launch (chain.hip). links_dev:
// device copy of the validated chain; M <= 4 tokens; kmax the largest K;
// sync: the caller's workspace words (arrival counter, time-out flag).
constexpr int kChainMaxM = 4;
size_t chain_lds_bytes(int count, int M, int kmax);
hipError_t launch_chain(const bitnest_chain_linear *links_dev, int count, int M, bool target, int kmax,
                        unsigned *sync, unsigned max_polls, hipStream_t stream);

}  // namespace bitnest
