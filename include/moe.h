/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE layer forward library, libmoe.so.
 *
 * The layer: router linear layer over the hidden state, softmax over experts,
 * top-k with renormalised gate weights, dispatch (per-expert histogram, prefix
 * sum, stable permutation), per-expert SwiGLU FFN, weighted combine back into
 * token order.
 *
 * Passages cited (page title, section):
 *   [P1] "Colibri：专为MoE模型优化的纯C高性能推理引擎" (trdm.cn/news/527833)
 *   [P2] "Colibri不是一只蜂鸟，而是一套为前沿MoE模型量身定制的C语言推理引擎" (discosf.com/news/4731160)
 *   [P3] Colibri C engine walkthrough (wzjinhao.cn/news/17934)
 *   [P4] "Colibri：轻量级MoE推理引擎的C语言实践" (mhpn.cn/news/2221639)
 *   [P5] "一只蜂鸟如何喂饱九头大象" (wth2jhl.online/blog/colibri-justvugg-deep-dive)
 *
 * Conventions (all entry points):
 *   - Every tensor pointer is a DEVICE pointer, row-major, 16-byte aligned
 *     (256-byte alignment recommended, as [P1] §2.2 aligns expert tensors).
 *     The caller owns every buffer; the library keeps no state between calls
 *     and never allocates device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued asynchronously; no entry point synchronises the device,
 *     except that MOE_DEBUG_SYNC=1 in the environment makes each entry point
 *     synchronise its stream and report kernel faults as MOE_EHIP.
 *   - Return value: MOE_OK (0) or a negative moe_status.  On error a
 *     NUL-terminated message is written to err[0..err_len) when err != NULL
 *     and err_len > 0 (truncated to fit), and nothing has been enqueued.  The
 *     int-status + caller-buffer convention follows [P4] §3.3.
 *   - Inputs must be finite; there is no check on the hot path.
 *   - Calls on one stream are ordered; calls that share output or workspace
 *     buffers on different streams race.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* bad shape, null pointer, misaligned pointer */
    MOE_ENOMEM = -2,        /* workspace smaller than moe_workspace_bytes() */
    MOE_EHIP = -3,          /* HIP launch or runtime error */
    MOE_EUNSUPPORTED = -4   /* valid shape that this build does not implement */
} moe_status;

typedef enum {
    MOE_F32 = 0,            /* IEEE binary32 */
    MOE_BF16 = 1,           /* bfloat16 (upper half of binary32), RNE when produced */
    MOE_INT4_G128 = 2,      /* weights only: symmetric int4 codes (two's complement,
                               two per byte, even K index in the low nibble) with one
                               fp16 scale per 128 consecutive K elements; w = q * s
                               ([P5] §7.3: int4 experts, per-group scales) */
    MOE_INT4_G128_TILED = 3,/* weights only: the same codes and scales, the code bytes
                               of every [N][K/2] matrix in the tiled order that
                               moe_pack_int4_tiled writes (scales stay [N][K/128]);
                               needs d and F multiples of 1024, at most 8192 */
    MOE_INT4_G64 = 4,       /* weights only: int4 codes as MOE_INT4_G128 with one fp16
                               scale per 64 consecutive K elements ([P5] §7.3 weighs
                               group size 64 against 128 and per-row) */
    MOE_MXFP4 = 5,          /* weights only: OCP MX fp4, E2M1 codes two per byte (even K
                               index in the low nibble), one E8M0 scale byte per 32
                               consecutive K elements: w = e2m1 * 2^(s - 127) */
    MOE_MXFP8 = 6,          /* weights only: OCP MX fp8, E4M3 codes one per byte, one
                               E8M0 scale byte per 32 K elements ([P5] §6: models
                               shipped as native MXFP4 / FP8 checkpoints) */
    MOE_MXFP4_TILED = 7,    /* weights only: MXFP4 codes and scales, the code bytes of
                               every [N][K/2] matrix in the tiled order that
                               moe_pack_int4_tiled writes (scales stay [N][K/32]);
                               every group runs the skinny matrix-core kernel; needs d
                               and F multiples of 1024 */
    MOE_MXFP8_TILED = 8     /* weights only: MXFP8 codes and scales, the code bytes of
                               every [N][K] matrix in the tiled order that
                               moe_pack_mxfp8_tiled writes (scales stay [N][K/32]);
                               every group runs the skinny matrix-core kernel; needs d
                               and F multiples of 1024 */
} moe_dtype;

/* Shape of one MoE layer call.
 *   T tokens, hidden size d, E routed experts, top-k, expert FFN width F.
 *   n_shared: 0 or 1 always-on shared expert of width F (weight 1).
 *   act: dtype of x, residual and y (MOE_F32 or MOE_BF16).
 *   wt:  dtype of expert weights (MOE_F32 with act F32; MOE_BF16 or any of the
 *        quantised formats with act BF16).  Quantised weights are widened to
 *        bf16 in registers before the matrix cores: exactly for MXFP4/MXFP8
 *        and for int4-g128 groups of at most tau rows; larger int4 groups and
 *        every int4-g64 group round q*s to the nearest bf16 (<= 2^-9 relative
 *        per weight).
 *   tau: bf16 expert groups with at most tau rows run the HBM-streaming
 *        kernels (the GEMV, or, when some group is larger than one GEMV pass,
 *        the skinny MFMA kernel, which covers up to 64 rows and needs d and F
 *        multiples of 64), larger groups the MFMA grouped GEMM.  0 selects
 *        the default: 64 where the skinny kernel serves both projections and
 *        d and F are at least 4096, else 16.  Negative forces the GEMV for every group.
 *        int4-g128 (row-major codes): groups of at most tau rows (0: 32) run
 *        the skinny int4 kernels (matrix cores for K a multiple of 1024, else
 *        the GEMV), larger ones the dequantising grouped GEMM (when every group
 *        runs it, a group's last partial 128-row tile of at most 16 rows goes
 *        to the skinny matrix-core kernel); negative keeps every group on the
 *        skinny kernels.  MXFP4 and MXFP8 with d and F multiples of 1024: the
 *        same rule on the skinny matrix-core kernel (without the short-tile
 *        path); other MX shapes, fp32, the tiled formats and int4-g64 ignore tau.
 * Limits (MOE_EINVAL otherwise): T >= 0, 1 <= k <= E <= 256, k <= 16,
 *   d, F >= 8 and multiples of 8; int4-g128: d and F multiples of 128;
 *   int4-g64, MXFP4, MXFP8: multiples of 64.
 * Limits of this build (MOE_EUNSUPPORTED otherwise): d, F <= 16384 (bf16 and
 *   the quantised formats), <= 8192 (fp32); bf16 and quantised weights:
 *   T*k*F*2 and T*d*2 bytes < 2 GiB. */
typedef struct {
    int32_t T, d, E, k, F;
    int32_t n_shared;
    int32_t act;
    int32_t wt;
    int32_t tau;
} moe_shape;

/* Expert weights, [E][N][K] with K contiguous (the merged per-layer expert
 * tensor, experts contiguous, of [P3] §3.1; gate/up/down = w1/w3/w2 of [P1] §3.1):
 *   w_gate, w_up: [E][F][d]   (int4, MXFP4: uint8 [E][F][d/2]; MXFP8: uint8 [E][F][d])
 *   w_down:       [E][d][F]   (int4, MXFP4: uint8 [E][d][F/2]; MXFP8: uint8 [E][d][F])
 *   s_*: scales of the quantised formats, NULL otherwise: fp16 [E][N][K/128]
 *        (MOE_INT4_G128, _TILED) or [E][N][K/64] (MOE_INT4_G64); uint8 E8M0
 *        [E][N][K/32] (MOE_MXFP4, MOE_MXFP8, _TILED).
 *   sh_*: the shared expert, same layouts with E = 1; NULL when n_shared == 0. */
typedef struct {
    const void *w_gate, *w_up, *w_down;
    const void *s_gate, *s_up, *s_down;
    const void *sh_gate, *sh_up, *sh_down;
    const void *sh_s_gate, *sh_s_up, *sh_s_down;
} moe_weights;

/* Router + softmax + top-k with renormalised gate weights (steps A1-A3).
 * [P1] §2.1 (linear gating + softmax, top-2 indices, normalised gate weights),
 * [P1] §3.2 (one fused gating kernel, maximum first then runner-up),
 * [P3] §3.2 (softmax(x W + b), max-subtracted), [P2] §2.1 (router output is
 * only k ids and k scores).
 *   x        [T][d] act dtype
 *   w_router [E][d] fp32;  b_router [E] fp32 or NULL
 *   logits   [T][E] fp32 output: logits[t][e] = sum_j x[t][j] w_router[e][j] + b[e],
 *            fp32 accumulation (required: it is also the kernel's scratch)
 *   topk_idx [T][k] int32 output: the k largest logits, descending, ties to
 *            the lower expert index
 *   topk_w   [T][k] fp32 output: softmax over experts restricted to the k
 *            selected ones, i.e. P[idx_j] / sum_m P[idx_m] */
int moe_route(const moe_shape *shape, const void *x, const float *w_router,
              const float *b_router, float *logits, int32_t *topk_idx, float *topk_w,
              void *stream, char *err, size_t err_len);

/* Dispatch (step A4): group the T*k assignments a = t*k + j by expert.
 * Histogram + prefix sum + stable placement: the counting-sort dispatcher of
 * [P2] §4.2 and the token_to_expert_map + expert_offset pair of [P1] §3.3.
 *   topk_idx [T*k] int32 input, values in [0, E) (entries outside are ignored:
 *            they are not counted and their slots of perm/inv are not written)
 *   counts   [E] int32: number of assignments to each expert
 *   offsets  [E+1] int32: exclusive prefix sum of counts (offsets[E] = T*k)
 *   perm     [T*k] int32: perm[p] = a, expert segments in ascending e, and
 *            within a segment ascending a (stable)
 *   inv      [T*k] int32: inv[perm[p]] = p
 * Bit-exact and deterministic (integer work only). */
int moe_dispatch(const moe_shape *shape, const int32_t *topk_idx, int32_t *counts,
                 int32_t *offsets, int32_t *perm, int32_t *inv,
                 void *stream, char *err, size_t err_len);

/* Per-expert SwiGLU FFN over dispatched rows (steps A5-A7).
 * [P1] §2.1 (per-expert FFN over active experts, then weighted merge),
 * [P1] §3.1 (w1/w2/w3 per expert, no bias), [P1] §3.3 (per-expert kernels
 * read the token map and expert offsets), [P3] §2.3 (only active experts run).
 * For row p of expert e's segment [offsets[e], offsets[e+1]), t = perm[p] / k:
 *   h = silu(x[t] . W_gate[e]^T) * (x[t] . W_up[e]^T)     (h stored bf16 for bf16
 *                                                        activations, fp32 for fp32)
 *   y_perm[p] = h . W_down[e]^T                           fp32 [T*k][d]
 * Shared expert (n_shared == 1): y_shared[t] = SwiGLU_sh(x[t]), fp32 [T][d],
 * else y_shared may be NULL.
 *   counts/offsets/perm: as written by moe_dispatch
 *   ws / ws_bytes: device workspace of at least moe_workspace_bytes(shape)
 *   bytes (MOE_ENOMEM otherwise); contents on entry are ignored. */
int moe_expert_ffn(const moe_shape *shape, const void *x, const moe_weights *w,
                   const int32_t *counts, const int32_t *offsets, const int32_t *perm,
                   float *y_perm, float *y_shared, void *ws, size_t ws_bytes,
                   void *stream, char *err, size_t err_len);

/* Weighted combine back into token order (step A8): the weighted merge of
 * [P1] §2.1 and the K-slot merge in token order of [P4] §2.3, as a
 * deterministic gather-reduce (one writer per output element, slots summed
 * in order j = 0..k-1, fp32 accumulation):
 *   y[t] = sum_j topk_w[t][j] * y_perm[inv[t*k+j]] (+ y_shared[t]) (+ residual[t])
 *   y_perm [T*k][d] fp32; inv [T*k]; topk_w [T][k] fp32;
 *   y_shared [T][d] fp32 or NULL; residual [T][d] act dtype or NULL;
 *   y [T][d] act dtype output (bf16 rounded to nearest even). */
int moe_combine(const moe_shape *shape, const float *y_perm, const int32_t *inv,
                const float *topk_w, const float *y_shared, const void *residual, void *y,
                void *stream, char *err, size_t err_len);

/* The whole layer: moe_route -> moe_dispatch -> moe_expert_ffn -> moe_combine
 * on one stream with no host synchronisation and no allocation.
 *   x [T][d] act; w_router [E][d] fp32; b_router [E] fp32 or NULL;
 *   residual [T][d] act or NULL; y [T][d] act output.
 *   counts_out [E] int32 or NULL: per-expert assignment counts (the usage
 *   histogram); topk_idx_out [T][k] int32 or NULL: the chosen experts.
 *   ws / ws_bytes: at least moe_workspace_bytes(shape). */
int moe_layer_forward(const moe_shape *shape, const void *x, const float *w_router,
                      const float *b_router, const moe_weights *w, const void *residual,
                      void *y, int32_t *counts_out, int32_t *topk_idx_out,
                      void *ws, size_t ws_bytes, void *stream, char *err, size_t err_len);

/* moe_layer_forward without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * moe_layer_forward minus ws / ws_bytes: the workspace is a fixed device
 * array of the library, 128 MiB on each GPU the library runs on (held until
 * the process ends; its address is looked up once per device on the first
 * call there, with that device current).  The call allocates nothing.
 *   MOE_ENOMEM when moe_workspace_bytes(shape) exceeds 128 MiB (decode and
 *   stack-layer shapes fit; a Mixtral-sized prefill batch does not: use
 *   moe_layer_forward with a caller workspace).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs to start at zero): calls that overlap on one
 * GPU (different streams or host threads without ordering) race. */
int moe_layer_forward_noalloc(const moe_shape *shape, const void *x, const float *w_router,
                              const float *b_router, const moe_weights *w, const void *residual,
                              void *y, int32_t *counts_out, int32_t *topk_idx_out,
                              void *stream, char *err, size_t err_len);

/* Bytes of device workspace needed by moe_layer_forward (and sufficient for
 * moe_expert_ffn) for this shape; 0 when the shape is invalid.  The fixed
 * scratch budget computed up front follows [P3] §2.3.  Host-only. */
size_t moe_workspace_bytes(const moe_shape *shape);

/* RMSNorm of the pre-norm stack: out[t] = h[t] / sqrt(mean_i h[t][i]^2 + eps) * gamma,
 * fp32 math, h and out in shape->act dtype, gamma [d] fp32 (NULL = ones).
 * (The pages name the residual around each MoE layer, [P3] §2.3; the norm is
 * the stacked workload's own definition.)  Uses shape->T and shape->d only. */
int moe_rmsnorm(const moe_shape *shape, const void *h, const float *gamma, float eps,
                void *out, void *stream, char *err, size_t err_len);

/* One-layer-ahead expert prediction, scored ([P5] §4.2: the router of the next
 * layer run one layer early chooses the experts to fetch ahead; [P5] §二
 * quotes the share it gets right).  A prediction is moe_route with layer
 * l+1's router on layer l's input; this call compares it with the experts
 * layer l+1 then chose.
 *   pred_idx, actual_idx [T][k] int32 (uses shape->T and shape->k only;
 *   entries compared as sets per token, values not range-checked)
 *   hist [k+1] int32 output: hist[j] = tokens whose two selections share
 *   exactly j experts; the hit rate is sum_j j*hist[j] / (T*k).
 * Integer work, bit-exact. */
int moe_topk_overlap(const moe_shape *shape, const int32_t *pred_idx, const int32_t *actual_idx,
                     int32_t *hist, void *stream, char *err, size_t err_len);

/* Weight preparation, once per weight set: rewrite 4-bit code bytes from the
 * row-major layout of MOE_INT4_G128 or MOE_MXFP4 ([N][K/2] per matrix, [P5]
 * §7.3, §6) into the tiled layout of MOE_INT4_G128_TILED / MOE_MXFP4_TILED.  The tiled matrix cuts the rows into
 * sets of 16; set s, 128-element group g (K = 128 g .. 128 g + 127) is 1 KB at
 * byte ((s * K/128) + g) * 1024, made of 64 pieces of 16 bytes: piece
 * 16 q + r (q = 0..3, r = 0..15) is bytes [64 g + 16 q, 64 g + 16 q + 16) of
 * row 16 s + r (its K elements 128 g + 32 q .. + 31).  Nibble order inside a
 * byte is unchanged; the matrix size (N * K/2 bytes) too.
 *   src, dst: device, n_mats * N * K/2 bytes each, 16-byte aligned, not
 *             overlapping (caller-owned; dst is written, src only read)
 *   n_mats >= 0 matrices of N rows (N a positive multiple of 16) and K columns
 *   (K a positive multiple of 128); e.g. w_gate: n_mats = E, N = F, K = d.
 * MOE_EINVAL for a bad size, a NULL, misaligned or overlapping pointer.
 * Asynchronous on stream. */
int moe_pack_int4_tiled(const void *src, void *dst, int64_t n_mats, int32_t N, int32_t K,
                        void *stream, char *err, size_t err_len);

/* Weight preparation, once per weight set: rewrite MXFP8 code bytes (E4M3, one
 * per byte) from the row-major layout of MOE_MXFP8 ([N][K] per matrix, [P5] §6)
 * into the tiled layout of MOE_MXFP8_TILED.  The tiled matrix cuts the rows into
 * sets of 16; set s, 128-element group g (K = 128 g .. 128 g + 127) is 2 KB at
 * byte ((s * K/128) + g) * 2048, made of 128 pieces of 16 bytes: piece
 * 64 w + 16 q + r (w = 0..1, q = 0..3, r = 0..15) is bytes
 * [128 g + 32 q + 16 w, + 16) of row 16 s + r (its K elements
 * 128 g + 32 q + 16 w .. + 15).  The matrix size (N * K bytes) is unchanged.
 *   src, dst: device, n_mats * N * K bytes each, 16-byte aligned, not
 *             overlapping (caller-owned; dst is written, src only read)
 *   n_mats >= 0 matrices of N rows (N a positive multiple of 16) and K columns
 *   (K a positive multiple of 128); e.g. w_gate: n_mats = E, N = F, K = d.
 * MOE_EINVAL for a bad size, a NULL, misaligned or overlapping pointer.
 * Asynchronous on stream. */
int moe_pack_mxfp8_tiled(const void *src, void *dst, int64_t n_mats, int32_t N, int32_t K,
                         void *stream, char *err, size_t err_len);

/* Static text of a moe_status. */
const char *moe_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
