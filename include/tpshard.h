/*
 * tpshard.h - C ABI for one rank's share of a tensor-parallel transformer block
 * on AMD MI355X (gfx950).
 *
 * The operations follow these pages:
 *   [KL]  "Tensor Parallelism" (inference-engineering notes), first paragraph:
 *         Y = XW; column parallelism splits W = [W_1 .. W_p] along its output
 *         dimension, so device i computes Y_i = X W_i; row parallelism splits W
 *         along its input dimension and X = [X_1 .. X_p] to match, so device i
 *         computes the full-shape partial Z_i = X_i W_i and Y = sum_i Z_i.
 *         Second paragraph: GQA bookkeeping (h=8192, 64 Q heads, 8 KV heads,
 *         head dim 128, p=8: 8 Q heads and 1 KV head per rank).
 *   [FFN] "How does tensor parallelism split a transformer feed-forward
 *         block's two matmuls across devices?", sections "The shape of the
 *         block", "Column split, then row split" (First matmul,
 *         column-parallel / The nonlinearity is free / Second matmul,
 *         row-parallel / One collective) and "The backward pass".
 *   [MLX] "Tensor-parallel all-reduce count per transformer layer in MLX
 *         shard_linear", Facts: the sharded-to-all linear multiplies by its
 *         slice, sums across ranks, then adds the bias once.
 *
 * Conventions for every entry point
 *   - Pointers marked (device) are device memory owned by the caller; the
 *     library allocates nothing and keeps no state except a thread-local
 *     error string.  Host pointers are marked (host).
 *   - All matrices are dense, contiguous and row-major.  Weights are stored
 *     (in, out): W1 is (d, n), W2 is (n, d), as the feed-forward page writes
 *     W1 with shape (d, 4d).  This is NOT torch nn.Linear's (out, in).
 *   - dtype TP_BF16: inputs bf16, fp32 accumulation, outputs rounded to bf16
 *     with round-to-nearest-even unless an out_dtype says otherwise.
 *     dtype TP_F32: fp32 everywhere.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and is asynchronous: no call synchronises the host.
 *   - All argument checks run on the host before anything is launched, so a
 *     rejected call has no side effect.  A launch failure returns TP_ERR_HIP
 *     with the runtime's message in tp_last_error().
 *   - T == 0 (no tokens) is a valid no-op returning TP_OK.
 *   - Outputs may not alias inputs (except `h` in tp_act_inplace).
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TPSHARD_ABI_VERSION 1

typedef struct ihipStream_t* tp_stream; /* same type as hipStream_t */

typedef enum {
  TP_OK = 0,
  TP_ERR_NULL = 1,        /* a required pointer is NULL                       */
  TP_ERR_SHAPE = 2,       /* negative / overflowing size, uneven split, ...   */
  TP_ERR_DTYPE = 3,       /* unknown or unsupported dtype combination         */
  TP_ERR_ACT = 4,         /* unknown act, or up/w_up/bias inconsistent with it */
  TP_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required       */
  TP_ERR_UNSUPPORTED = 6, /* valid request the library does not implement    */
  TP_ERR_HIP = 7          /* the HIP runtime reported an error                */
} tp_status;

typedef enum { TP_BF16 = 0, TP_F32 = 1 } tp_dtype;

/* Activations on the owned columns ([FFN] "The nonlinearity is free"):
 *   RELU   max(a, 0)                      (derivative at 0 taken as 0)
 *   GELU   exact erf form 0.5 a (1 + erf(a / sqrt 2))
 *   SWIGLU silu(g) * u with silu(g) = g / (1 + exp(-g)), g = x W_gate_i and
 *          u = x W_up_i over the same owned column range. */
typedef enum { TP_ACT_NONE = 0, TP_ACT_RELU = 1, TP_ACT_GELU = 2, TP_ACT_SWIGLU = 3 } tp_act;

/* ---------------------------------------------------------------------------
 * Column-parallel linear ([KL] Y_i = X W_i; [FFN] "First matmul,
 * column-parallel" and "The nonlinearity is free").
 *   y = act(x . w + bias)                     for NONE / RELU / GELU
 *   y = silu(x . w) * (x . w_up)              for SWIGLU
 * x (T, K) (device), w and w_up (K, N_i) (device), bias (N_i) or NULL
 * (device; this shard's slice of the column bias; must be NULL for SWIGLU),
 * y (T, N_i) (device).  K == 0 gives act(bias) in every row (x and w may
 * then be NULL).  Errors: TP_ERR_NULL, TP_ERR_SHAPE (negative sizes),
 * TP_ERR_ACT (w_up given iff SWIGLU violated, or bias with SWIGLU),
 * TP_ERR_DTYPE, TP_ERR_HIP. */
tp_status tp_col_linear(const void* x, const void* w, const void* w_up, const void* bias, void* y,
                        void* ws, size_t ws_bytes, int64_t T, int64_t K, int64_t N_i, tp_dtype dtype,
                        tp_act act, tp_stream stream);

/* Optional workspace (bytes) for tp_col_linear: with it, decode-sized calls
 * (T <= 64) split K over more workgroups; ws may be NULL (then ws_bytes is
 * ignored and the call runs unsplit: on a streaming kernel that keeps the
 * activation slice in LDS when it fits, else on the register-staged tiled
 * kernel; correct, but slower at decode sizes, since fewer workgroups share
 * the weight stream).  A non-NULL ws smaller than this is TP_ERR_WORKSPACE.
 * Same zero-fill rule as tp_mlp_shard_fwd_workspace.  Returns 0 when no
 * workspace would be used. */
size_t tp_col_linear_workspace(int64_t T, int64_t K, int64_t N_i, tp_dtype dtype, tp_act act);

/* Activation applied in place to owned columns ([FFN] "The nonlinearity is
 * free").  h (T, N_i) (device) is overwritten with act(h); for SWIGLU h holds
 * the gate pre-activation and up (T, N_i) (device) the up pre-activation,
 * and h <- silu(h) * up.  NONE is a no-op.  `up` must be non-NULL iff SWIGLU
 * (TP_ERR_ACT otherwise). */
tp_status tp_act_inplace(void* h, const void* up, int64_t T, int64_t N_i, tp_dtype dtype,
                         tp_act act, tp_stream stream);

/* Row-parallel linear producing the full-shape partial ([KL] Z_i = X_i W_i;
 * [FFN] "Second matmul, row-parallel").  x_i (T, K_i), w_i (K_i, N), z_i
 * (T, N), all device.  Never adds a bias ([MLX]: the bias goes after the sum,
 * see tp_partial_sum).  in_dtype bf16 allows out_dtype bf16 or f32; in_dtype
 * f32 requires out_dtype f32.  ws/ws_bytes optional (see
 * tp_row_linear_partial_workspace). */
tp_status tp_row_linear_partial(const void* x_i, const void* w_i, void* z_i, void* ws,
                                size_t ws_bytes, int64_t T, int64_t K_i, int64_t N,
                                tp_dtype in_dtype, tp_dtype out_dtype, tp_stream stream);

/* Optional workspace (bytes) for tp_row_linear_partial; same rules as
 * tp_col_linear_workspace. */
size_t tp_row_linear_partial_workspace(int64_t T, int64_t K_i, int64_t N, tp_dtype in_dtype);

/* Workspace (bytes) tp_mlp_shard_fwd needs for these sizes.  Always > 0 for
 * T > 0.  The workspace must be zero-filled before its FIRST use (e.g. with
 * tp_workspace_init); every call leaves its counter region zeroed again, so a
 * workspace can be reused by later calls on the same stream, of any entry
 * point and shape: the split-K arrival counters always sit in a region at the
 * start of the workspace (at least 64 KiB) that no call writes anything else
 * to, which holds for every call needing at most 16384 counters (all shapes
 * up to 2^18 output columns).  Calls that run concurrently must not share a
 * workspace. */
size_t tp_mlp_shard_fwd_workspace(int64_t T, int64_t d, int64_t ff_i, tp_dtype dtype, tp_act act);

/* One rank's feed-forward shard ([FFN] "Column split, then row split"):
 *   y_i = act(x . w1_i [, x . w_up_i]) . w2_i
 * x (T, d), w1_i and w_up_i (d, ff_i), w2_i (ff_i, d), y_i (T, d): the
 * full-shape partial that the group's all-reduce would sum.  w_up_i must be
 * non-NULL iff SWIGLU.  The intermediate h_i (T, ff_i) is kept in the
 * workspace in `dtype` (bf16 for TP_BF16).  saved (device, nullable)
 * receives the pre-activations the backward needs: (T, 2*ff_i) as
 * [G_i | U_i] per row for SWIGLU, (T, ff_i) A_i otherwise, in `dtype`.
 * out_dtype: TP_BF16 or TP_F32 for dtype bf16, TP_F32 for dtype f32.
 * ws (device) of ws_bytes >= tp_mlp_shard_fwd_workspace(...). */
tp_status tp_mlp_shard_fwd(const void* x, const void* w1_i, const void* w_up_i, const void* w2_i,
                           void* y_i, void* saved, void* ws, size_t ws_bytes, int64_t T, int64_t d,
                           int64_t ff_i, tp_dtype dtype, tp_dtype out_dtype, tp_act act,
                           tp_stream stream);

/* Bytes of the static device scratch behind tp_mlp_shard_fwd_noalloc (per GPU). */
#define TP_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* tp_mlp_shard_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc.  Same arguments (minus ws/ws_bytes),
 * checks and results as tp_mlp_shard_fwd, computed by the same kernels; the
 * scratch those kernels use (split-K arrival counters and partials, h, the
 * packed activations) lives in a static device array of
 * TP_NOALLOC_SCRATCH_BYTES (32 MiB) that every GPU the library runs on holds
 * until the process ends.  Sizes whose tp_mlp_shard_fwd_workspace exceeds it
 * return TP_ERR_WORKSPACE before any launch.  The first call on a device
 * looks up the array's device address (with that device current) and clears
 * its counter region with a fill kernel on `stream`; no call allocates (no
 * hipMalloc, hipFree or allocating library routine).  Every call on a GPU
 * shares that GPU's array and leaves its counters zero: calls that overlap on
 * one GPU (other streams or threads) race, so the caller orders them. */
tp_status tp_mlp_shard_fwd_noalloc(const void* x, const void* w1_i, const void* w_up_i,
                                   const void* w2_i, void* y_i, void* saved, int64_t T, int64_t d,
                                   int64_t ff_i, tp_dtype dtype, tp_dtype out_dtype, tp_act act,
                                   tp_stream stream);

/* Workspace (bytes) tp_mlp_shard_bwd needs (same zero-fill rule as forward). */
size_t tp_mlp_shard_bwd_workspace(int64_t T, int64_t d, int64_t ff_i, tp_dtype dtype, tp_act act);

/* One rank's backward ([FFN] "The backward pass"): dy (T, d) is the same on
 * every rank; the shard produces its own weight gradients (no exchange) and a
 * partial input gradient dx_i (T, d) that the group sums.
 *   dW2_i = h_i^T dy,  dh_i = dy W2_i^T,
 *   SWIGLU: dG = dh_i * U * silu'(G), dU = dh_i * silu(G),
 *           dW1_i = x^T dG, dW_up_i = x^T dU, dx_i = dG W1_i^T + dU W_up_i^T
 *   RELU/GELU/NONE: dA = dh_i * act'(A), dW1_i = x^T dA, dx_i = dA W1_i^T
 * saved (device) must be what tp_mlp_shard_fwd wrote for the same x and
 * weights; h_i is recomputed from it.  dw1_i, dw_up_i (d, ff_i), dw2_i
 * (ff_i, d), dx_i (T, d), all device, in `dtype`.  dw_up_i and w_up_i
 * non-NULL iff SWIGLU.  ws as for the forward. */
tp_status tp_mlp_shard_bwd(const void* x, const void* w1_i, const void* w_up_i, const void* w2_i,
                           const void* saved, const void* dy, void* dw1_i, void* dw_up_i,
                           void* dw2_i, void* dx_i, void* ws, size_t ws_bytes, int64_t T,
                           int64_t d, int64_t ff_i, tp_dtype dtype, tp_act act, tp_stream stream);

/* Backward of one rank's shard of a linear layer y = x w ([FFN] "The backward
 * pass"; [KL] second paragraph: Q, K, V column-parallel by heads, o_proj
 * row-parallel).  With dy the gradient at y:
 *   dw = x^T dy   (K, N),   dx = dy w^T   (T, K).
 * Column-parallel shard (the fused QKV projection): x is the replicated
 * input, w = [Wq_i | Wk_i | Wv_i] and dy the rank's own output gradient; dw
 * is final (no exchange) and dx a partial for tp_partial_sum.  Row-parallel
 * shard (o_proj): x = the rank's attention output X_i, w = its row slice and
 * dy the gradient every rank holds; dw and dx are both final.
 * x (T, K), w (K, N), dy (T, N), dw (K, N), dx (T, K): device, row-major, in
 * `dtype`; bf16 operands accumulate in fp32 and are stored with RNE.  dw or
 * dx may be NULL to skip it (not both); x is read only for dw, w only for
 * dx; a pointer to an empty array may be NULL.  No bias gradient.  ws (device) of ws_bytes >=
 * tp_linear_shard_bwd_workspace(...) (0: none needed, ws may be NULL),
 * under the same zero-fill and reuse rules as tp_mlp_shard_fwd's workspace.
 * T == 0 zero-fills dw.  Errors: TP_ERR_NULL, TP_ERR_SHAPE, TP_ERR_DTYPE,
 * TP_ERR_WORKSPACE, TP_ERR_HIP. */
size_t tp_linear_shard_bwd_workspace(int64_t T, int64_t K, int64_t N, tp_dtype dtype);
tp_status tp_linear_shard_bwd(const void* x, const void* w, const void* dy, void* dw, void* dx,
                              void* ws, size_t ws_bytes, int64_t T, int64_t K, int64_t N,
                              tp_dtype dtype, tp_stream stream);

/* Attention over one rank's local heads, between the fused QKV projection and
 * o_proj ([KL] second paragraph: each rank owns whole query and KV heads and
 * computes attention locally; [FFN] attention paragraph: heads are
 * independent; [KL] FlashAttention paragraph: Q K^T, softmax and V tiled so
 * the scores stay on chip).  For query head j, with KV head
 * g = j / (n_q / n_kv):
 *   O_j = softmax_rows(scale * Q_j K_g^T  [keys > query dropped if causal]) V_g
 * qkv (T, (n_q + 2 n_kv) * head_dim) bf16, row t = [Q heads | K heads |
 * V heads] (the output of tp_col_linear with w = [Wq_i | Wk_i | Wv_i]);
 * out (T, n_q * head_dim) bf16, heads side by side (the input of o_proj).
 * Both device, 16-byte aligned.  One sequence of T tokens.  fp32 scores and
 * softmax, bf16 probabilities into the P V product, fp32 accumulation, bf16
 * output (RNE).  Errors: TP_ERR_SHAPE (sizes, n_q not a multiple of n_kv,
 * causal not 0/1, scale not finite and > 0), TP_ERR_UNSUPPORTED (head_dim
 * other than 128, unaligned pointers), TP_ERR_NULL, TP_ERR_HIP.  T == 0 is a
 * no-op. */
tp_status tp_gqa_attention_fwd(const void* qkv, void* out, int64_t T, int n_q, int n_kv, int head_dim,
                               int causal, float scale, tp_stream stream);

/* Sharded linears with fp8 weights, for decode-sized token counts (the
 * quantized form of the column- and row-parallel linear that [MLX] mentions
 * as the "quantized equivalent" of the sharded linear).  Weights are OCP
 * e4m3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; 0x7F /
 * 0xFF are NaN), one byte each, with one fp32 scale per output column:
 * W[k, n] = e4m3(code(k, n)) * scale[n].  The codes are stored 64-column
 * strip-major (as tp_fp8_pack_strips writes them): code (k, n) at byte
 * (n / 64) * 64 K + 64 k + n % 64, so each strip streams as one contiguous
 * run.  Activations stay
 * bf16; products accumulate in fp32 and the scale multiplies each column's
 * sum (exactly the product with the dequantized weights, up to rounding).
 *   tp_col_linear_fp8:          y = act(x W + bias), or
 *                               silu(x W) * (x W_up) for SWIGLU (wq_up and
 *                               scale_up given iff SWIGLU; no bias then)
 *   tp_row_linear_partial_fp8:  z_i = x_i W_i (no bias), out_dtype bf16/f32
 * x (T, K) bf16, 16-byte aligned with K % 8 == 0; wq (K x N codes,
 * strip-major), 16-byte aligned with N % 64 == 0; scale (N) fp32; y / z_i
 * (T, N).  All device.
 * 1 <= T <= 64 (TP_ERR_UNSUPPORTED above; T == 0 is a no-op).  ws (device)
 * of ws_bytes >= tp_linear_fp8_workspace(T, K, N, act), required, under the
 * zero-fill and reuse rules of tp_mlp_shard_fwd's workspace.  Errors:
 * TP_ERR_NULL, TP_ERR_SHAPE, TP_ERR_ACT, TP_ERR_DTYPE, TP_ERR_WORKSPACE,
 * TP_ERR_UNSUPPORTED, TP_ERR_HIP. */
size_t tp_linear_fp8_workspace(int64_t T, int64_t K, int64_t N, tp_act act);
/* One rank's feed-forward shard at decode size with fp8 weights (the same
 * block as tp_mlp_shard_fwd, [FFN] "Column split, then row split", with the
 * weights of the fp8 linears above, strip-major): y_i = act(x W1_i [, x
 * W_up_i]) W2_i with W = e4m3(codes) * per-column scale.  h_i stays in the
 * workspace (bf16, written by the column GEMM straight in the row GEMM's
 * packed activation order).  x (T, d) bf16; wq1_i, wq_up_i (d x ff_i codes),
 * wq2_i (ff_i x d codes); s1_i, s_up_i (ff_i), s2_i (d) fp32; y_i (T, d) in
 * out_dtype.  1 <= T <= 64, d and ff_i multiples of 64, 16-byte aligned
 * pointers (TP_ERR_UNSUPPORTED otherwise).  ws of ws_bytes >=
 * tp_mlp_shard_fwd_fp8_workspace(...), same rules as tp_mlp_shard_fwd's. */
size_t tp_mlp_shard_fwd_fp8_workspace(int64_t T, int64_t d, int64_t ff_i, tp_act act);
tp_status tp_mlp_shard_fwd_fp8(const void* x, const void* wq1_i, const float* s1_i, const void* wq_up_i,
                               const float* s_up_i, const void* wq2_i, const float* s2_i, void* y_i,
                               void* ws, size_t ws_bytes, int64_t T, int64_t d, int64_t ff_i,
                               tp_dtype out_dtype, tp_act act, tp_stream stream);
/* Mixture-of-experts block with the routed experts sharded in place
 * ([MLX] Facts: DeepSeek V3 and Qwen3-MoE shard their experts in place, keep
 * the router replicated and sum the block output once).
 * tp_moe_route: from router logits (T, E) fp32 (x times the replicated router
 * weight, e.g. tp_row_linear_partial with an f32 output) to idx (T, k) int32
 * and gate (T, k) fp32: the k largest logits per token in descending order
 * (equal logits: lower expert index first), gates = softmax over the chosen
 * k.  1 <= k <= min(E, 16), E <= 1024.
 * tp_moe_shard_fwd: y_i[t] = sum_j gate[t, j] * silu(x[t] W1[e]) * (x[t] Wup[e])
 * . W2[e] with e = idx[t, j]: this rank's partial (the group sums it).  x (T,
 * d) bf16; w1, w_up (E, d, ff_i) and w2 (E, ff_i, d) bf16, the rank's slice
 * of every expert, contiguous per expert; y_i (T, d) in out_dtype.  d and
 * ff_i multiples of 8, 16-byte aligned pointers (TP_ERR_UNSUPPORTED
 * otherwise).  Routed rows are grouped per expert on the device (no host
 * round trip); ws (device) of ws_bytes >= tp_moe_shard_fwd_workspace(...),
 * same rules as tp_mlp_shard_fwd's.  Results do not depend on the order in
 * which the rows are grouped.  A slot whose idx lies outside [0, E) (a
 * dropped slot) contributes nothing.  Each routed row's down projection is
 * kept in out_dtype (bf16 like h, or fp32) before the gate-weighted sum,
 * which accumulates in fp32. */
tp_status tp_moe_route(const float* logits, int64_t T, int E, int k, int32_t* idx, float* gate,
                       tp_stream stream);
size_t tp_moe_shard_fwd_workspace(int64_t T, int64_t d, int64_t ff_i, int E, int k);
tp_status tp_moe_shard_fwd(const void* x, const int32_t* idx, const float* gate, const void* w1,
                           const void* w_up, const void* w2, void* y_i, void* ws, size_t ws_bytes,
                           int64_t T, int64_t d, int64_t ff_i, int E, int k, tp_dtype out_dtype,
                           tp_stream stream);

/* Rearranges fp8 codes from (K, N) row-major (src) into the 64-column
 * strip-major order the fp8 linears read (dst), once per weight matrix.  Both
 * device, 16-byte aligned, not aliasing; N % 64 == 0 (TP_ERR_SHAPE).
 * A pure byte permutation. */
tp_status tp_fp8_pack_strips(const void* src, void* dst, int64_t K, int64_t N, tp_stream stream);
tp_status tp_col_linear_fp8(const void* x, const void* wq, const float* scale, const void* wq_up,
                            const float* scale_up, const void* bias, void* y, void* ws, size_t ws_bytes,
                            int64_t T, int64_t K, int64_t N_i, tp_act act, tp_stream stream);
tp_status tp_row_linear_partial_fp8(const void* x_i, const void* wq_i, const float* scale_i, void* z_i,
                                    void* ws, size_t ws_bytes, int64_t T, int64_t K_i, int64_t N,
                                    tp_dtype out_dtype, tp_stream stream);

/* ---- packed weights for decode-sized calls ---------------------------------
 * At decode size a rank's GEMMs are bound by streaming the weight shard from
 * HBM ([KL] fourth paragraph: one token costs the weight bytes over the HBM
 * bandwidth).  These entry points read weights rearranged ONCE (e.g. when the
 * shard is loaded) into the order the matrix cores consume them, so every
 * workgroup owns 16 output columns over the whole K range and reads its
 * operands straight into registers.  Layout of a packed (K, N) weight:
 * 1024-byte chunks, one per (block b of 32 rows, strip s of 16 columns), in
 * block-major order: byte 16*l + 2*j of chunk (s, b), at byte offset
 * (b * ceil(N/16) + s) * 1024, holds W[32b + 8*(l/16) + j][16s + l%16] for
 * l = 0..63, j = 0..7, zero outside K x N.  All activations and weights are
 * bf16; T <= 64 (TP_ERR_SHAPE beyond: prefill-sized calls take the (in, out)
 * row-major entry points above). */

/* Bytes of a packed (K, N) weight. */
size_t tp_packed_weight_bytes(int64_t K, int64_t N);

/* w (K, N) bf16 row-major (device) -> w_packed (tp_packed_weight_bytes(K, N)
 * bytes, device, 16-byte aligned), asynchronously on `stream`.  A pure
 * rearrangement (bitwise).  Errors: TP_ERR_NULL, TP_ERR_SHAPE (negative
 * sizes, unaligned w_packed), TP_ERR_HIP. */
tp_status tp_pack_weight(const void* w, void* w_packed, int64_t K, int64_t N, tp_stream stream);

/* Workspace (bytes, 16-byte aligned, zero-filled before first use like
 * tp_mlp_shard_fwd_workspace's) of tp_col_linear_packed and
 * tp_row_linear_partial_packed (act TP_ACT_NONE for the latter); 0 for T == 0
 * or T > 64.  The workspace is required: it holds x rearranged into the
 * matrix cores' operand order (a launch of its own) and the split-K
 * partials.  Calls whose GEMM reads few activation bytes in all (K a
 * multiple of 32, x 16-byte aligned, at most 48 MiB of operand fragments:
 * ceil(N/16 / strips per workgroup) * K * 32 * ceil(T/16 rounded to 1, 2,
 * 4) bytes) read x in place instead and skip that launch; the results are
 * bitwise the same either way.  Larger calls on these bf16 weights with K a
 * multiple of 64, x 16-byte aligned and at least two weight fragments per
 * k-block (SWIGLU, or more than 1008 columns, which such a call then
 * streams two 16-column strips per workgroup) skip it too: they load x in
 * whole 128-byte lines and rearrange it on chip; their fp32 sums run over
 * whole 64-row k-pairs and their own K splits, so where the packed launch
 * would cut K elsewhere the results can differ from it by one bf16
 * rounding. */
size_t tp_linear_packed_workspace(int64_t T, int64_t K, int64_t N, tp_act act);

/* tp_col_linear with packed weights ([KL] Y_i = X W_i; [FFN] "First matmul,
 * column-parallel", "The nonlinearity is free"): y (T, N_i) = act(x w + bias)
 * or silu(x w) * (x w_up).  x (T, K) bf16 row-major, w_packed / w_up_packed
 * packed (K, N_i) (w_up_packed iff SWIGLU), bias (N_i) bf16 or NULL (not with
 * SWIGLU), y (T, N_i) bf16; all device.  Errors as tp_col_linear, plus
 * TP_ERR_SHAPE for T > 64 and TP_ERR_WORKSPACE. */
tp_status tp_col_linear_packed(const void* x, const void* w_packed, const void* w_up_packed,
                               const void* bias, void* y, void* ws, size_t ws_bytes, int64_t T,
                               int64_t K, int64_t N_i, tp_act act, tp_stream stream);

/* tp_row_linear_partial with a packed weight ([KL] Z_i = X_i W_i; [FFN]
 * "Second matmul, row-parallel"): z_i (T, N) = x_i w, never a bias.  x_i
 * (T, K_i) bf16, w_packed packed (K_i, N), z_i (T, N) in out_dtype (bf16 or
 * f32); all device. */
tp_status tp_row_linear_partial_packed(const void* x_i, const void* w_packed, void* z_i, void* ws,
                                       size_t ws_bytes, int64_t T, int64_t K_i, int64_t N,
                                       tp_dtype out_dtype, tp_stream stream);

/* Bytes of x (T, K) in the packed-activation order the packed GEMMs read:
 * ceil(K/32) blocks of m chunks of 1024 bytes (m = 1, 2 or 4 for T <= 16,
 * <= 32, <= 64); byte 16*l + 2*j of chunk (block b, tile i), at byte offset
 * (b*m + i) * 1024, holds x[16i + l%16][32b + 8*(l/16) + j], zero outside
 * T x K.  0 for T == 0 or T > 64. */
size_t tp_packed_act_bytes(int64_t T, int64_t K);

/* x (T, K) bf16 row-major -> x_packed (tp_packed_act_bytes(T, K) bytes,
 * 16-byte aligned), all device; a pure rearrangement.  T <= 64. */
tp_status tp_pack_act(const void* x, void* x_packed, int64_t T, int64_t K, tp_stream stream);

/* The packed GEMM alone, on activations already in the packed order (from
 * tp_pack_act, or written that way by a previous kernel): y (T, N) =
 * act(x w + bias), silu(x w) * (x w_up) for SWIGLU, or x w for NONE without a
 * bias (out_dtype bf16 or f32; f32 only for NONE).  One kernel launch.  ws as
 * for tp_linear_packed_workspace(T, K, N, act). */
tp_status tp_linear_packed_gemm(const void* x_packed, const void* w_packed, const void* w_up_packed,
                                const void* bias, void* y, void* ws, size_t ws_bytes, int64_t T,
                                int64_t K, int64_t N, tp_act act, tp_dtype out_dtype,
                                tp_stream stream);

/* Workspace (bytes) of tp_mlp_shard_fwd_packed (same rules as
 * tp_linear_packed_workspace). */
size_t tp_mlp_shard_fwd_packed_workspace(int64_t T, int64_t d, int64_t ff_i, tp_act act);

/* tp_mlp_shard_fwd with packed weights ([FFN] "Column split, then row
 * split"): y_i = act(x w1_i [, x w_up_i]) w2_i.  x (T, d) bf16, w1_packed and
 * w_up_packed packed (d, ff_i), w2_packed packed (ff_i, d), y_i (T, d) in
 * out_dtype; all device.  h_i stays in the workspace (bf16), written by the
 * column GEMM's epilogue straight in the operand order the row GEMM reads.
 * Inference only: no saved pre-activations. */
tp_status tp_mlp_shard_fwd_packed(const void* x, const void* w1_packed, const void* w_up_packed,
                                  const void* w2_packed, void* y_i, void* ws, size_t ws_bytes, int64_t T,
                                  int64_t d, int64_t ff_i, tp_dtype out_dtype, tp_act act,
                                  tp_stream stream);

/* ---- packed fp8 weights for decode-sized calls ----------------------------
 * The fp8 linears above ([MLX] the quantized equivalent of the sharded
 * linear: W[k, n] = e4m3(code(k, n)) * scale[n], OCP e4m3 codes, one fp32
 * scale per output column, bf16 activations, fp32 sums, the scale applied to
 * each column's sum) on codes packed once like the bf16 packed weights, at
 * one byte per weight.  Layout of packed (K, N) codes: 1024-byte chunks, one
 * per (pair p of 64 rows, strip s of 16 columns), pair-major: byte
 * 16*l + 8*h + j of chunk (s, p), at byte offset (p * ceil(N/16) + s) * 1024,
 * holds code[64p + 32h + 8*(l/16) + j][16s + l%16] for l = 0..63, h = 0..1,
 * j = 0..7, zero outside K x N.  T <= 64 (TP_ERR_SHAPE beyond). */

/* Bytes of packed (K, N) fp8 codes. */
size_t tp_packed_fp8_weight_bytes(int64_t K, int64_t N);

/* codes (K, N) row-major bytes (device) -> w_packed (tp_packed_fp8_weight_bytes
 * (K, N) bytes, device, 16-byte aligned), asynchronously on `stream`.  A pure
 * rearrangement.  Errors: TP_ERR_NULL, TP_ERR_SHAPE, TP_ERR_HIP. */
tp_status tp_pack_weight_fp8(const void* codes, void* w_packed, int64_t K, int64_t N, tp_stream stream);

/* Workspace (bytes; rules of tp_linear_packed_workspace) of
 * tp_col_linear_packed_fp8 and tp_row_linear_partial_packed_fp8 (act
 * TP_ACT_NONE for the latter); 0 for T == 0 or T > 64. */
size_t tp_linear_packed_fp8_workspace(int64_t T, int64_t K, int64_t N, tp_act act);

/* tp_col_linear_fp8 on packed codes: y (T, N_i) = act(x W + bias) or
 * silu(x W) * (x W_up), W = e4m3(wq) * scale (wq_up_packed and scale_up iff
 * SWIGLU; no bias then).  x (T, K) bf16 row-major, scale / scale_up (N_i)
 * fp32, bias (N_i) bf16 or NULL, y (T, N_i) bf16; all device; any K and N_i.
 * Errors as tp_col_linear_packed. */
tp_status tp_col_linear_packed_fp8(const void* x, const void* wq_packed, const float* scale,
                                   const void* wq_up_packed, const float* scale_up, const void* bias,
                                   void* y, void* ws, size_t ws_bytes, int64_t T, int64_t K, int64_t N_i,
                                   tp_act act, tp_stream stream);

/* tp_row_linear_partial_fp8 on packed codes: z_i (T, N) = x_i W_i, W_i =
 * e4m3(wq) * scale_i, out_dtype bf16 or f32.  Errors as
 * tp_row_linear_partial_packed. */
tp_status tp_row_linear_partial_packed_fp8(const void* x_i, const void* wq_packed, const float* scale_i,
                                           void* z_i, void* ws, size_t ws_bytes, int64_t T, int64_t K_i,
                                           int64_t N, tp_dtype out_dtype, tp_stream stream);

/* Workspace (bytes) of tp_mlp_shard_fwd_packed_fp8; 0 for T == 0, T > 64 or
 * ff_i not a multiple of 64. */
size_t tp_mlp_shard_fwd_packed_fp8_workspace(int64_t T, int64_t d, int64_t ff_i, tp_act act);

/* tp_mlp_shard_fwd_fp8 on packed codes ([FFN] "Column split, then row split"
 * with fp8 weights): y_i = act(x W1_i [, x W_up_i]) W2_i.  wq1_packed and
 * wq_up_packed packed (d, ff_i) codes with scales s1_i, s_up_i (ff_i),
 * wq2_packed packed (ff_i, d) codes with s2_i (d); ff_i a multiple of 64
 * (TP_ERR_UNSUPPORTED otherwise).  h_i stays in the workspace (bf16), in the
 * row GEMM's operand order.  Other rules as tp_mlp_shard_fwd_packed. */
tp_status tp_mlp_shard_fwd_packed_fp8(const void* x, const void* wq1_packed, const float* s1_i,
                                      const void* wq_up_packed, const float* s_up_i, const void* wq2_packed,
                                      const float* s2_i, void* y_i, void* ws, size_t ws_bytes, int64_t T,
                                      int64_t d, int64_t ff_i, tp_dtype out_dtype, tp_act act,
                                      tp_stream stream);

/* Sum of the p full-shape partials, then the bias once ([KL] Y = sum_i Z_i;
 * [FFN] "One collective"; [MLX] bias after the sum).  This is the one-GPU
 * stand-in for the group's all-reduce.  z (host array of p device pointers),
 * each (T, N) in in_dtype; bias (N) in in_dtype or NULL (device); y (T, N)
 * in out_dtype (device).  Accumulation is fp32 (fp32 also for f32 inputs),
 * in ascending i, so the result is deterministic.  1 <= p <= 64. */
tp_status tp_partial_sum(const void* const* z, int p, const void* bias, void* y, int64_t T,
                         int64_t N, tp_dtype in_dtype, tp_dtype out_dtype, tp_stream stream);

/* Sequence-parallel boundary, one rank's share: with sequence parallelism the
 * block's all-reduce is replaced by a reduce-scatter followed by an
 * all-gather of the same bytes ([KS] "Where the 320 comes from", the
 * sequence-parallel paragraph), and the summed output feeds the residual add
 * and the following normalization ([FFN] "One collective").  Rank `rank` owns rows
 * [rank*T/p, (rank+1)*T/p) of the T x N partials; for each owned row r (row
 * R = rank*T/p + r of the partials):
 *   s[r]            = residual_in[r] + sum_i z[i][R] (ascending i) + bias     (fp32)
 *   residual_out[r] = s[r]
 *   y[r]            = s[r] / sqrt(mean_j s[r][j]^2 + eps) * norm_w           (RMSNorm)
 * The norm is taken over the fp32 sum (before residual_out is rounded).
 * z: host array of p device pointers, each (T, N) in in_dtype; bias (N) in
 * in_dtype or NULL; residual_in, residual_out, y: (T/p, N) in out_dtype;
 * norm_w (N) in out_dtype (all device).  1 <= p <= 64, 0 <= rank < p,
 * T % p == 0 (equal shares), N <= 32768, eps >= 0.  residual_out may alias
 * residual_in; y may not alias anything. */
tp_status tp_rs_residual_rmsnorm(const void* const* z, int p, int rank, const void* bias, const void* residual_in,
                                 const void* norm_w, float eps, void* residual_out, void* y, int64_t T, int64_t N,
                                 tp_dtype in_dtype, tp_dtype out_dtype, tp_stream stream);

/* Zero-fills `bytes` of device memory ws on `stream` with a kernel (no
 * memset node, so it is safe to capture in a graph). */
tp_status tp_workspace_init(void* ws, size_t bytes, tp_stream stream);

/* ---- host helpers (no GPU needed) ------------------------------------- */

/* Shard i of n_total cut into p equal contiguous chunks ([FFN] "Column split,
 * then row split": device i owns columns i*n/p .. (i+1)*n/p of W1 and the
 * matching rows of W2).  TP_ERR_SHAPE if n_total % p != 0, p <= 0, i out of
 * range or n_total < 0; TP_ERR_NULL if an output pointer is NULL (host). */
tp_status tp_shard_range(int64_t n_total, int p, int i, int64_t* begin, int64_t* len);

/* Rank i's GQA column ranges ([KL] second paragraph; [FFN] attention
 * paragraph: a head is never split, so both head counts must divide by p).
 * Heads are assigned contiguously, so Q head j shares KV head
 * j / (n_q_heads / n_kv_heads) and both live on the same rank.  Outputs
 * (host) are column offsets/lengths into the unsharded Q and K/V
 * projections.  TP_ERR_SHAPE if a head count is not divisible by p. */
tp_status tp_gqa_shard(int n_q_heads, int n_kv_heads, int head_dim, int p, int i,
                       int64_t* q_begin, int64_t* q_len, int64_t* kv_begin, int64_t* kv_len);

const char* tp_status_string(tp_status s);
const char* tp_last_error(void);
int tp_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TPSHARD_H */
