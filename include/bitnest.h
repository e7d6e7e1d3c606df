/*
 * bitnest.h - C ABI of the bit-nested W4/W8 quantized linear on AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (BitNest-Llama-3-8B model card, section "Files", entry
 * planes.safetensors; recipe table rows "Weights" and "Activations"):
 *
 *   One 8-bit weight is kept as two planes of unsigned nibbles, `hi` and `lo`,
 *   each uint8 [N, K/2], nibble u = q + 8. Byte j of a row holds column 2j in
 *   its low nibble and column 2j+1 in its high nibble. `scale` is fp16
 *   [N, K/128], one scale per row and per 128 input columns.
 *     draft  weight W4 = (hi - 8) * scale                        (reads hi only)
 *     target weight W8 = (16 * (hi - 8) + (lo - 8)) * scale / 16 (reads hi and lo)
 *   Activations are symmetric int8, one scale per token, or one per token and
 *   128-column group (the o_proj recipe).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. The library
 *     allocates nothing, frees nothing, keeps no pointer after returning, holds
 *     no per-call state (the one exception: the scratch array of
 *     bitnest_greedy_accept_noalloc, below) and never synchronises. Work is
 *     enqueued on `stream` (a hipStream_t passed as void*; NULL is the default
 *     stream); results are ready when that stream reaches the point of the
 *     call.
 *   - Every call works on the calling thread's current HIP device (the one
 *     hipGetDevice returns): the tensors and the stream must belong to it.
 *   - Tensors are row-major and contiguous. Every tensor pointer must be
 *     16-byte aligned.
 *   - Sizes: 0 <= M <= BITNEST_MAX_M, 0 <= N, 128 <= K <= BITNEST_MAX_K, K a
 *     multiple of 128. M == 0 or N == 0 is a valid call that does nothing;
 *     its tensor pointers are not checked and may be NULL.
 *   - Arguments are checked on the host before anything is launched:
 *       BITNEST_EINVAL       a required pointer is NULL, a size is negative,
 *                            K is not a positive multiple of 128, or
 *                            act_group is neither 0 nor 128;
 *       BITNEST_EALIGN       a tensor pointer is not 16-byte aligned;
 *       BITNEST_EUNSUPPORTED M > BITNEST_MAX_M, K > BITNEST_MAX_K, or one
 *                            plane larger than BITNEST_MAX_PLANE_BYTES;
 *       BITNEST_EHIP         the HIP runtime reported an error while
 *                            launching (an error left pending on the calling
 *                            thread by an earlier HIP call is reported too).
 *     A fault inside a kernel surfaces at the caller's next synchronisation
 *     of the stream, as for any HIP kernel.
 *   - Outputs must not overlap inputs.
 *   - Inputs are finite. Results are the definitions below computed in fp32
 *     (the integer parts exactly) as long as they stay within fp32's range;
 *     a result that overflows it is undefined (+-inf or NaN). Subnormal
 *     inputs and scales are handled as IEEE values, not flushed.
 *   - Calls are reentrant; calls on different streams may run concurrently,
 *     except two bitnest_greedy_accept_noalloc calls on one device, which
 *     share that device's scratch, and two calls that share a workspace.
 *   - Nothing throws across this boundary.
 */
#ifndef BITNEST_H
#define BITNEST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITNEST_ABI_VERSION 8
#define BITNEST_GROUP 128      /* columns per weight scale (and per o_proj act scale) */
#define BITNEST_MAX_M 32       /* most tokens per call */
#define BITNEST_MAX_K 16384    /* largest input width */
#define BITNEST_MAX_PLANE_BYTES 2147483647LL  /* largest N * K / 2 (bytes of one plane) */
#define BITNEST_MAX_ROT_BLOCK 512 /* largest rotation block of the R4 calls */
#define BITNEST_KV_HEAD_DIM 128   /* head dimension of the nested KV cache */
#define BITNEST_KV_MAX_ROWS 16    /* most query rows (M x Hq / Hkv) per KV head */

typedef enum bitnest_status {
    BITNEST_OK = 0,
    BITNEST_EINVAL = 1,
    BITNEST_EALIGN = 2,
    BITNEST_EUNSUPPORTED = 3,
    BITNEST_EHIP = 4
} bitnest_status;

/* Version of this interface; equals BITNEST_ABI_VERSION of the built library. */
int bitnest_abi_version(void);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char *bitnest_status_string(int status);

/*
 * Activation quantisation (model card, recipe table, row "Activations":
 * symmetric int8, per token; o_proj per 128-column group).
 *
 * The pages do not fix the scale formula or the rounding. This library uses,
 * for each token m and each column set R (the whole row when act_group == 0,
 * each run of 128 columns when act_group == 128):
 *     amax = max_{k in R} |x[m,k]|
 *     s    = amax / 127                  IEEE fp32 division, round to nearest even
 *     q    = 0                           if s == 0
 *            clamp(rne(x / s), -127, 127) otherwise, x / s an IEEE fp32 division
 *   (rne = round half to even; -128 is never produced.)
 *
 *   x   fp32 [M, K], finite values (NaN/Inf are outside the contract).
 *   xq  int8 [M, K] codes, written.
 *   xs  fp32 [M] (act_group 0) or [M, K/128] (act_group 128), written.
 */
bitnest_status bitnest_quant_act(const float *x, int M, int K, int act_group,
                                 int8_t *xq, float *xs, void *stream);

/*
 * Draft linear, W4A8 (model card: the draft reads only the high nibble plane).
 *   y[m, n] = sum_g float(P_hi[m,n,g]) * scale[n,g] * s_a
 *   P_hi[m,n,g] = sum_{k in group g} xq[m,k] * (hi_nibble[n,k] - 8)   (exact int32)
 *   s_a = xs[m] (act_group 0) or xs[m, g] (act_group 128).
 * This equals sum_k (xq[m,k] * s_a) * W4[n,k] up to fp32 rounding.
 *
 *   xq     int8 [M, K] codes;  xs  fp32 [M] or [M, K/128]
 *   hi     uint8 [N, K/2]      scale  fp16 bit patterns [N, K/128], any finite
 *                              value (negative, zero and subnormal included)
 *   y      fp32 [M, N], every element overwritten.
 * Only `hi` and `scale` are read from the weights.
 */
bitnest_status bitnest_linear_draft(const int8_t *xq, const float *xs, int act_group,
                                    const uint8_t *hi, const uint16_t *scale,
                                    float *y, int M, int N, int K, void *stream);

/*
 * Target linear, W8A8 (model card: the target reads all 8 bits).
 *   P8[m,n,g] = 16 * P_hi[m,n,g] + P_lo[m,n,g]         (exact int32; the 8-bit
 *               code 16*(hi-8) + (lo-8) spans [-136, 119] and is never formed
 *               as an int8)
 *   y[m, n]   = sum_g float(P8[m,n,g]) * (scale[n,g] / 16) * s_a
 * Arguments as for the draft, plus `lo` uint8 [N, K/2]. M <= 7 runs the
 * plane-streaming GEMV, M >= 8 the batched-verify int8 matrix-core kernel; the
 * results obey the same definition. How each kernel forms P8 (both exact):
 *   M <= 7  one dot product per column for both planes, on the byte
 *           16*(hi-8) + lo = w8 + 8 in [-128, 127] (the two nibble fields
 *           carry into each other nowhere, so by linearity the dot product
 *           is 16 P_hi + P_lo + 8 sum_k xq), then minus 8 * sum_k xq over the
 *           group;
 *   M >= 8  separate int8 matrix-core contractions of the hi and the lo
 *           plane, combined as 16 P_hi + P_lo in int32.
 * Rows and batches (draft and target alike): for M <= 7 every row of y is bit
 * for bit the y of a one-token call on that row's codes, so a verify batch
 * computes exactly what one-token steps would (the model card's introduction:
 * speculative decoding returns the target's own greedy output). For M >= 8 a
 * row does not depend on the other rows either (bit for bit across M = 8 to
 * 32), but the fp32 sums run in another order than for M <= 7, so those rows
 * agree with one-token calls to fp32 rounding, not bit for bit.
 */
bitnest_status bitnest_linear_target(const int8_t *xq, const float *xs, int act_group,
                                     const uint8_t *hi, const uint8_t *lo,
                                     const uint16_t *scale,
                                     float *y, int M, int N, int K, void *stream);

/*
 * Activation quantisation fused with the draft linear: the same codes, scales
 * and y, bit for bit, as bitnest_quant_act(x, M, K, act_group, xq, xs, stream)
 * followed by bitnest_linear_draft(xq, xs, act_group, hi, scale, y, M, N, K,
 * stream). For one token up to K = 16384, and for up to four tokens up to
 * K = 4096 and N = 8192, each workgroup quantises x itself and the whole
 * linear is one launch; otherwise the call makes the two launches.
 *   x    fp32 [M, K] input;  xq int8 [M, K], xs fp32 [M] or [M, K/128]:
 *        outputs, as written by bitnest_quant_act (always required)
 *   hi, scale, y as for bitnest_linear_draft (may be NULL when N == 0).
 */
bitnest_status bitnest_quant_linear_draft(const float *x, int act_group,
                                          const uint8_t *hi, const uint16_t *scale,
                                          float *y, int8_t *xq, float *xs,
                                          int M, int N, int K, void *stream);

/* The same for the target linear (bitnest_quant_act + bitnest_linear_target). */
bitnest_status bitnest_quant_linear_target(const float *x, int act_group,
                                           const uint8_t *hi, const uint8_t *lo,
                                           const uint16_t *scale,
                                           float *y, int8_t *xq, float *xs,
                                           int M, int N, int K, void *stream);

/*
 * The down_proj input path with its online rotation (model card, recipe table
 * row "Rotation": an online Hadamard, R4, on the down_proj inputs; the R4
 * matrices ship in aux.safetensors, which the pages do not reproduce, and
 * their construction is not stated). This library's reading: R4 is block-
 * diagonal, every block of `block` columns the normalised Sylvester-Hadamard
 * matrix H_b / sqrt(b), H_b[i][j] = (-1)^popcount(i & j). Per token m and
 * block, in fp32:
 *     z = H_b x[m, blk]  by the fast transform, stages h = 1, 2, 4, ..., b/2
 *                        in that order, each replacing the pair
 *                        (a, c) = (z[i], z[i + h]) (bit h of i clear) by
 *                        (a + c, a - c)
 *     r[m, blk] = z * r_b  one fp32 multiply, r_b = the fp32 value nearest
 *                        1/sqrt(b)
 * then the quantisation rule of bitnest_quant_act with act_group 0 (one
 * scale per token) on r. The stage order and the single multiply make the
 * rotated values, and so the codes, exact functions of x.
 *
 *   x      fp32 [M, K], finite values
 *   block  power of two, 2 <= block <= BITNEST_MAX_ROT_BLOCK, K % block == 0
 *          (512 for the Llama-3-8B down_proj: K = 14336 = 28 x 512);
 *          otherwise BITNEST_EINVAL
 *   xq     int8 [M, K] codes, xs fp32 [M] scales: written
 *   xr     fp32 [M, K]: the rotated values r, written if not NULL
 * The weights of the linear that consumes these codes must carry the same
 * rotation (applied offline), as the package's down_proj weights do.
 */
bitnest_status bitnest_hadamard_quant_act(const float *x, int M, int K, int block,
                                          int8_t *xq, float *xs, float *xr, void *stream);

/*
 * Rotation and quantisation fused with the draft / target linear: the same
 * codes, scales and y, bit for bit, as bitnest_hadamard_quant_act (xr NULL)
 * followed by bitnest_linear_draft / bitnest_linear_target with act_group 0.
 * For one token (M == 1) each workgroup rotates and quantises x itself and
 * the whole linear is one launch; otherwise the call makes two launches.
 * Arguments as for bitnest_quant_linear_draft / _target, with `block` in
 * place of act_group.
 */
bitnest_status bitnest_hadamard_quant_linear_draft(const float *x, int block,
                                                   const uint8_t *hi, const uint16_t *scale,
                                                   float *y, int8_t *xq, float *xs,
                                                   int M, int N, int K, void *stream);

bitnest_status bitnest_hadamard_quant_linear_target(const float *x, int block,
                                                    const uint8_t *hi, const uint8_t *lo,
                                                    const uint16_t *scale,
                                                    float *y, int8_t *xq, float *xs,
                                                    int M, int N, int K, void *stream);

/*
 * A chain of linears in one launch (model card introduction: the draft runs
 * the model's linears on the high-nibble plane for each of the gamma = 3
 * draft tokens, then the target runs them on both planes over the gamma + 1
 * verify tokens; each of these passes is a sequence of linears in which
 * every input is produced after the previous linear's output).
 *
 * bitnest_linear_chain runs links[0], links[1], ..., links[count - 1] in
 * that order, each the call bitnest_quant_linear_draft (a draft chain: `lo`
 * NULL in every link with N > 0) or bitnest_quant_linear_target (a target
 * chain: no such `lo` NULL) on its own tensors, M tokens each, with the same
 * results bit for bit (codes, activation scales, y).
 * Ordering: everything link j reads from `x` is read after every output of
 * links 0 .. j-1 is written, so a link's input may be an earlier link's
 * output (or be written by nothing in the chain); outputs of one link must
 * not overlap its own inputs, and no output may overlap any link's planes or
 * scales (weights are read ahead of the ordering: they are constant for the
 * whole call).
 *
 * One launch instead of count: a persistent grid (one workgroup per compute
 * unit, every workgroup resident at once) streams the planes of all links
 * and waits on a device-scope counter in `work` between links. Each wait is
 * bounded: after `max_polls` polls (0 selects BITNEST_CHAIN_DEFAULT_POLLS,
 * about a second) the workgroup stops waiting, sets the time-out word, and
 * the kernel runs to its end; the results of that call are then not
 * defined. A wait runs out only when the grid cannot be resident at once
 * (e.g. other kernels holding compute units for that long).
 * Speed: on MI355X a chain is not faster than the same links as single
 * calls replayed from a HIP graph (measured: 4.5-6.6 us per link against
 * 4.0-4.8 us per single draft call at the Llama-3-8B shapes); a device-wide
 * wait across the chip costs about as much as a dependent kernel launch. It
 * serves callers that want one launch per sequence of linears.
 *
 *   links      HOST array of `count` links, validated before anything is
 *              launched (the fields below; BITNEST_EINVAL /
 *              BITNEST_EALIGN / BITNEST_EUNSUPPORTED as for the single calls)
 *   links_dev  DEVICE copy of the same array (same bytes), 16-byte aligned;
 *              the kernel reads the links from it
 *   count      0 <= count <= BITNEST_CHAIN_MAX_LINEARS (0: nothing is done)
 *   M          1 <= M <= BITNEST_CHAIN_MAX_M tokens, the same for every link
 *   work       caller-owned device workspace of at least
 *              BITNEST_CHAIN_WORKSPACE_BYTES, 16-byte aligned, ZERO-FILLED
 *              before its first use; a call leaves word 0 (uint32 arrival
 *              counter) at zero again; word 1 (uint32) becomes nonzero,
 *              and stays so, when a wait of some call ran out. Calls that may
 *              overlap in time must not share a workspace.
 * Per link: x fp32 [M, K]; hi, lo uint8 [N, K/2]; scale fp16 bits
 * [N, K/128]; y fp32 [M, N]; xq int8 [M, K] and xs fp32 [M] (act_group 0)
 * or [M, K/128] (act_group 128): both written, or both NULL and not
 * written; 128 <= K <= BITNEST_MAX_K, K % 128 == 0; N >= 0 (N == 0: only
 * the quantisation); act_group 0 or 128; rot_block must be 0 (reserved).
 */
typedef struct bitnest_chain_linear {
    const float *x;
    const uint8_t *hi;
    const uint8_t *lo;
    const uint16_t *scale;
    float *y;
    int8_t *xq;
    float *xs;
    int32_t N;
    int32_t K;
    int32_t act_group;
    int32_t rot_block;
} bitnest_chain_linear;

#define BITNEST_CHAIN_MAX_LINEARS 512
#define BITNEST_CHAIN_MAX_M 4
#define BITNEST_CHAIN_WORKSPACE_BYTES 2048
#define BITNEST_CHAIN_DEFAULT_POLLS (1u << 20)

/* BITNEST_CHAIN_WORKSPACE_BYTES, for callers that load the library at run time. */
size_t bitnest_chain_workspace_bytes(void);

bitnest_status bitnest_linear_chain(const bitnest_chain_linear *links,
                                    const bitnest_chain_linear *links_dev, int count, int M,
                                    uint32_t max_polls, void *work, size_t work_bytes,
                                    void *stream);

/*
 * Offline nested packing of fp32 weights into the two planes (model card
 * introduction: the high nibble is a GPTQ-W4 model fitted first, the low
 * nibble the closed-form residual back to W8; section "Files", entry
 * planes.safetensors: the format). GPTQ needs calibration data; this is the
 * symmetric round-to-nearest quantiser it builds on (15 steps, zero point 8)
 * per row and 128-column group, with the stored fp16 scale:
 *     amax = max |W| over the group
 *     s    = fp16(amax / 7.5)        IEEE fp32 division, then round to
 *                                    nearest even in binary16
 *     c_hi = clamp(rne(W / s), -8, 7)                 hi nibble = c_hi + 8
 *     c_lo = clamp(rne((W - c_hi * s) / (s / 16)), -8, 7)  lo nibble = c_lo + 8
 *   (fp32 arithmetic, IEEE divisions; s == 0 gives both codes 0). The draft
 *   and target weights of the calls above are then W4 = c_hi * s and
 *   W8 = (16 c_hi + c_lo) * s / 16, and |W8 - W| <= s / 32 wherever neither
 *   code clamps.
 *
 *   W      fp32 [N, K], finite, |W| < 7.5 * 65504 (the fp16 scale must be finite)
 *   hi, lo uint8 [N, K/2] planes (byte j: column 2j low nibble, 2j+1 high), written
 *   scale  fp16 bit patterns [N, K/128], written
 * Sizes as for the linear calls (K a positive multiple of 128, one plane at
 * most BITNEST_MAX_PLANE_BYTES; M does not apply, K is not bounded by
 * BITNEST_MAX_K); N == 0 is a no-op.
 */
bitnest_status bitnest_pack_nested(const float *W, int N, int K,
                                   uint8_t *hi, uint8_t *lo, uint16_t *scale, void *stream);

/*
 * Greedy verification of a speculative round (model card introduction:
 * every draft token is verified with the target, so the output is exactly
 * the W8A8 target's greedy output). With the target's logits for the
 * gamma + 1 verify positions (row r: the position after the prefix extended
 * by the first r draft tokens):
 *     targ[r] = argmax_v logits[r, v]   (ties: the smallest index)
 *     n       = length of the longest prefix with draft[r] == targ[r]
 *     result  = {n, targ[n]}            the round emits draft[0 .. n-1], then targ[n]
 *
 *   logits  fp32 [R, V], R = gamma + 1 (1 <= R <= BITNEST_MAX_M),
 *           1 <= V <= BITNEST_ACCEPT_MAX_V (column indices and slice bounds
 *           are 32-bit; a larger V gives BITNEST_EUNSUPPORTED), finite
 *   draft   int32 [R - 1] (may be NULL when R == 1)
 *   targ    int32 [R], written;  result int32 [2], written
 *   work    caller-owned scratch of at least
 *           bitnest_greedy_accept_workspace_bytes(R, V) bytes (per-slice partials:
 *           8 bytes per row and slice of about 4096 logits, at most 64 slices),
 *           overwritten; 16-byte aligned
 */
#define BITNEST_ACCEPT_MAX_V (1 << 30)   /* most logits per row */
size_t bitnest_greedy_accept_workspace_bytes(int R, int V);   /* 0 if R or V is out of range */

bitnest_status bitnest_greedy_accept(const float *logits, int R, int V, const int32_t *draft,
                                     int32_t *targ, int32_t *result, void *work, size_t work_bytes,
                                     void *stream);

/*
 * bitnest_greedy_accept without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The per-slice partials go to a scratch
 * array the library holds in each device's memory for the life of the
 * process (BITNEST_ACCEPT_NOALLOC_SCRATCH_BYTES, enough for every R <=
 * BITNEST_MAX_M and every V <= BITNEST_ACCEPT_MAX_V). The call allocates and
 * frees nothing. Results are those of bitnest_greedy_accept, bit for bit.
 * All calls on one device share that device's scratch: calls that may
 * overlap on one device (different streams without ordering between them)
 * race and must not be made; calls
 * in one stream's order are safe. Arguments and errors as for
 * bitnest_greedy_accept, without `work` / `work_bytes`; a size beyond the
 * scratch (R > BITNEST_MAX_M) gives BITNEST_EUNSUPPORTED.
 */
#define BITNEST_ACCEPT_NOALLOC_SCRATCH_BYTES 16384
bitnest_status bitnest_greedy_accept_noalloc(const float *logits, int R, int V, const int32_t *draft,
                                             int32_t *targ, int32_t *result, void *stream);

/*
 * Decode attention over the nested KV cache (model card, recipe table row
 * "KV cache": nested at runtime, the draft reads KV4 and the target KV8;
 * abstract: the progressive-precision design extends to the KV cache for
 * long contexts). The layout and the scale granularity are in meta.json,
 * which the pages do not reproduce; this library's reading:
 *   - every (token t, KV head h) vector of K or V, 128 values, is packed like
 *     one 128-column group of a weight row (byte j: dimension 2j low nibble,
 *     2j+1 high nibble) with one fp16 scale. The cache is head-major: planes
 *     uint8 [Hkv, t_cap, 64] and scales [Hkv, t_cap], where t_cap >= T is
 *     the number of positions allocated per head and positions t < T are
 *     read, so a head's positions are contiguous bytes (the layout this
 *     library's loads stream fastest). Writing positions [t0, t1) of head h
 *     is bitnest_pack_nested with N = t1 - t0 rows of K = 128 columns at row
 *     h t_cap + t0;
 *   - KV4 = (hi - 8) s, KV8 = (16 (hi - 8) + (lo - 8)) s / 16, the weight
 *     formulas;
 *   - the M query tokens are the last M positions of the sequence (the
 *     verify batch; M = 1 for a draft step): token i sees positions
 *     t <= T - M + i;
 *   - query head hq reads KV head hq / (Hq / Hkv) (grouped-query attention);
 *   - out[i, hq] = sum_t softmax_t(q[i, hq] . k[t] / sqrt(128)) v[t].
 * Computed in fp32: the sequence is cut into splits (runs of 64-position
 * chunks, their number sized to the device), each split keeps a running
 * softmax, and the splits are merged exactly as the softmax requires.
 * Scores and P.V run on the fp16 matrix cores with each fp32 operand split
 * into three fp16 pieces, so each (token, head) output is within 1e-5 of
 * its own largest magnitude (measured: below 1e-6) of the exact result.
 *
 *   q        fp32 [M, Hq, 128]
 *   T        positions in the sequence; t_cap  positions per head in the cache
 *   k_hi, v_hi  uint8 [Hkv, t_cap, 64];  k_lo, v_lo  the same or both NULL (KV4)
 *   k_scale, v_scale  fp16 bit patterns [Hkv, t_cap]
 *   out      fp32 [M, Hq, 128], written
 *   work     caller-owned scratch of at least
 *            bitnest_kv_attention_workspace_bytes(M, Hq, T) bytes, overwritten
 *            (= min(ceil(T / 64), 512) M Hq 130 floats: per split and query
 *            row, 128 output values, the maximum and the sum; 0 for
 *            M, Hq or T below 1)
 * Limits: M >= 1, Hq a multiple of Hkv, M Hq / Hkv <= BITNEST_KV_MAX_ROWS,
 * M <= T <= t_cap, Hkv <= 65535, T 64 < 2^31; otherwise BITNEST_EINVAL /
 * BITNEST_EUNSUPPORTED. q and the scales are finite.
 */
size_t bitnest_kv_attention_workspace_bytes(int M, int Hq, int T);

bitnest_status bitnest_kv_attention(const float *q, int M, int Hq, int Hkv, int T, int t_cap,
                                    const uint8_t *k_hi, const uint8_t *k_lo, const uint16_t *k_scale,
                                    const uint8_t *v_hi, const uint8_t *v_lo, const uint16_t *v_scale,
                                    float *out, void *work, size_t work_bytes, void *stream);

/*
 * Measurement, not part of the linear: reads `bytes` bytes at p with the
 * plane stream's loads (1 KiB per wave load instruction, non-temporal
 * 128-bit loads, 8-wave workgroups, each wave a contiguous run of rounds of
 * `depth` items with one round in flight) and none of its arithmetic, so
 * that the time of one call bounds what a linear streaming that many plane
 * bytes can reach (the model card's introduction prices a draft step by the
 * plane bytes it reads). The data are folded into one word, which is
 * written to sink[0] only if it equals `never` (pick a value the data
 * cannot fold to; the store keeps the loads from being dropped).
 *   p      device memory, 16-byte aligned; bytes a multiple of 1024,
 *          1024 <= bytes <= 2^32 - 1024
 *   depth  items in flight per wave: 2, 4 or 8
 *   waves_per_cu  resident waves per compute unit to use at most (0: as
 *          many as fit); the grid is min(rounds, that many per CU) waves
 *   sink   device memory for one uint32, written at most once
 */
bitnest_status bitnest_stream_read(const void *p, size_t bytes, int depth, int waves_per_cu, uint32_t never,
                                   uint32_t *sink, void *stream);

/*
 * The integer partials of the draft and target calls above, for checking (not a
 * fast path), from the same kernels and integer loops as those calls:
 *   M <= 7  the GEMV's loop: P8 exactly as the target forms it (the merged
 *           byte and the code-sum correction), P_hi from the draft's loop,
 *           P_lo = P8 - 16 P_hi;
 *   M >= 8  the matrix-core kernel's two contractions: P_hi and P_lo as
 *           computed, P8 = 16 P_hi + P_lo as the target combines them.
 *   p_hi  int32 [M, N, K/128] <- P_hi (always written)
 *   p_lo  int32 [M, N, K/128] <- P_lo              (only if lo != NULL)
 *   p8    int32 [M, N, K/128] <- 16 * P_hi + P_lo  (only if lo != NULL)
 * lo == NULL selects the draft kernels (p_lo and p8 are then ignored and may
 * be NULL); otherwise p_lo and p8 are required.
 */
bitnest_status bitnest_linear_partials(const int8_t *xq, const uint8_t *hi, const uint8_t *lo,
                                       int32_t *p_hi, int32_t *p_lo, int32_t *p8,
                                       int M, int N, int K, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BITNEST_H */
