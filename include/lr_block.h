/*
 * lr_block.h -- C ABI of the gfx950 (MI355X) low-rank decoder-block library.
 *
 * The library computes the forward and backward pass of the linear stack of
 * one LLaMA-2-style decoder block whose every weight is factorised into a
 * down-projection A [r, in] followed by an up-projection B [out, r]
 * (BOOST project page, alvin-zyl.github.io/boost, section "Move the chunk
 * boundary to the bottleneck"), with the three supporting changes of the
 * section "Three supporting changes": Online RMSNorm fused into the
 * down-projection, linear layer grouping, and a backward that keeps only the
 * r-wide activations and recomputes the d-wide ones. The attention
 * score/softmax core is not part of it: the forward outputs Q, K, V and takes
 * the attention output O; the backward takes dQ, dK, dV and outputs dO.
 *
 * Conventions for every entry point
 *   - Matrices are row-major. Weights are [out, in], so a layer computes
 *     y = x W^T. Leading dimensions are in elements.
 *   - Every pointer is a device pointer (hipMalloc'd or from a device
 *     allocator) unless stated otherwise, 16-byte aligned, and every leading
 *     dimension is a multiple of 8 elements (bf16) or 4 elements (fp32);
 *     column offsets used to address sub-blocks keep that alignment.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work on it and return; read outputs after
 *     synchronising the stream.
 *   - The library allocates no memory, keeps no state between calls and is
 *     re-entrant across streams. Caller-provided workspace must not be used
 *     by two calls that may run concurrently.
 *   - Outputs are overwritten, never accumulated into.
 *   - A call enqueues kernel launches only (no memset, copy, allocation or
 *     synchronisation), so a sequence of calls may be captured into a HIP
 *     graph (hipStreamBeginCapture) and replayed. The first call of an entry
 *     point on a device may set kernel attributes; make it outside capture.
 *     The kernels are deterministic: the same inputs give the same bits.
 *   - Arguments are validated before anything is enqueued; on failure the
 *     call returns a negative status, enqueues nothing and records a
 *     message for lr_last_error(). A failed kernel launch returns
 *     LR_ERR_HIP. No C++ exception crosses this interface.
 */
#ifndef LR_BLOCK_H_
#define LR_BLOCK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LR_OK 0
#define LR_ERR_INVALID_ARG (-1) /* null pointer, bad size, misalignment   */
#define LR_ERR_UNSUPPORTED (-2) /* valid request this build cannot serve  */
#define LR_ERR_WORKSPACE (-3)   /* workspace missing or too small         */
#define LR_ERR_HIP (-4)         /* the HIP runtime reported an error      */

typedef enum { LR_F32 = 0, LR_BF16 = 1 } lr_dtype;

/* Which part of the block a call runs. PRE_ATTN is everything before the
 * attention core (forward: norm + grouped QKV down- and up-projections;
 * backward: from dQ, dK, dV to dX). POST_ATTN is everything after it
 * (forward: O's projections, the MLP and both residuals; backward: from dY to
 * dO). The backward's POST_ATTN part must run first and leaves dh in the
 * workspace for the PRE_ATTN part, so both calls must get the same
 * workspace. */
typedef enum {
  LR_STAGE_ALL = 0,
  LR_STAGE_PRE_ATTN = 1,
  LR_STAGE_POST_ATTN = 2
} lr_stage;

/* Operand layouts of lr_grouped_lowrank_gemm (see there). */
typedef enum { LR_LAYOUT_NT = 0, LR_LAYOUT_NN = 1, LR_LAYOUT_TN = 2 } lr_layout;

/* Epilogues of lr_grouped_lowrank_gemm (see there). */
typedef enum {
  LR_EPI_NONE = 0,
  LR_EPI_ADD_RESIDUAL = 1,
  LR_EPI_SWIGLU_PAIR = 2,
  LR_EPI_ROW_SCALE = 3
} lr_epilogue;

/* Shape of one block on this GPU.
 *   T         tokens (micro-batch x sequence), rows of every activation
 *   d         hidden width held by this GPU
 *   r         bottleneck rank of every factorised layer
 *   d_ff      MLP width held by this GPU
 *   d_norm    RMS divisor D: the global hidden width (= d unless this GPU
 *             holds one tensor-parallel rank's slice of the hidden vector)
 *   n_panels  Online RMSNorm K-panels P: d splits into P contiguous panels
 *             of equal width; 1 <= P <= 8, and with P > 1 the panel width
 *             d / P must be a multiple of 64
 *   n_heads   layout information only; the linear stack ignores it
 *   eps       RMSNorm epsilon, added to the mean square inside the root
 *   dtype     LR_BF16: bf16 storage, fp32 accumulation and statistics;
 *             LR_F32: fp32 everywhere (no reduced-precision MFMA)
 *   emit_partials  1: rank-share mode. The two norm chunks also emit their
 *             unreduced tensor-parallel payloads (lr_block_partials); the
 *             all-reduce that would sum them over ranks is the identity here.
 */
typedef struct {
  int64_t T, d, r, d_ff, d_norm;
  int32_t n_panels;
  int32_t n_heads;
  float eps;
  int32_t dtype;
  int32_t emit_partials;
} lr_block_shape;

/* Weights (device, in `dtype`). Grouped storage: A_qkv = [A_q; A_k; A_v]
 * is [3r, d] and A_gu = [A_gate; A_up] is [2r, d] (rows stacked in that
 * order). B_q, B_k, B_v, B_o, B_dn are [d, r]; B_g, B_u are [d_ff, r];
 * A_o is [r, d]; A_dn is [r, d_ff]; gamma1, gamma2 are [d]. */
typedef struct {
  const void *gamma1, *gamma2;
  const void *A_qkv, *B_q, *B_k, *B_v;
  const void *A_o, *B_o;
  const void *A_gu, *B_g, *B_u;
  const void *A_dn, *B_dn;
} lr_block_weights;

/* Activations the forward saves for the backward (device): the r-wide
 * chunk-boundary activations qkv_r [T, 3r] = [q_r | k_r | v_r],
 * o_r [T, r], gu_r [T, 2r] = [g_r | u_r], d_r [T, r] in `dtype`, and the
 * per-row RMS of the two norms, rms1, rms2 [T] in fp32. */
typedef struct {
  void *qkv_r, *o_r, *gu_r, *d_r;
  float *rms1, *rms2;
} lr_block_saved;

/* Weight and gamma gradients (device, fp32, same shapes as the weights). */
typedef struct {
  float *gamma1, *gamma2;
  float *A_qkv, *B_q, *B_k, *B_v;
  float *A_o, *B_o;
  float *A_gu, *B_g, *B_u;
  float *A_dn, *B_dn;
} lr_block_grads;

/* Rank-share outputs (emit_partials = 1). P_qkv [T, 3r] and P_gu [T, 2r]
 * (in `dtype`) are the unreduced payloads (gamma * x) A^T of the two norm
 * chunks and ss1, ss2 [T] (fp32) the sums of squares of this GPU's slice of
 * X and h that travel with them. The payloads of the other two chunks are
 * o_r and d_r themselves (lr_block_saved). In normal mode (emit_partials =
 * 0) with n_panels > 1 the struct is optional: non-NULL ss1, ss2 then
 * receive the per-panel sums of squares [P, T] of X and h, and P_qkv, P_gu
 * are ignored. */
typedef struct {
  void *P_qkv, *P_gu;
  float *ss1, *ss2;
} lr_block_partials;

/* Bytes of workspace lr_block_fwd (is_bwd = 0) or lr_block_bwd (is_bwd = 1)
 * needs for this shape; 0 if the shape is invalid. For bf16 shapes whose d,
 * r and d_ff are multiples of 64 the backward workspace also holds
 * transposed copies of the weights its data-gradient products multiply by
 * (r (11 d + 3 d_ff) elements), made at the start of each stage. */
size_t lr_block_workspace_bytes(const lr_block_shape* shape, int is_bwd);

/* Where a d-wide intermediate of the checkpointed stack sits in a block
 * workspace, for callers that check the low-rank activation checkpointing
 * (project page, "Three supporting changes": the backward recomputes the
 * d-wide activations from the saved r-wide ones instead of storing them).
 * which = LR_WS_H: h = X + o_r B_o^T [T, d]; LR_WS_M: m = SiLU(g) * u
 * [T, d_ff]; both row-major in `dtype`. After lr_block_fwd with ALL or
 * POST_ATTN the forward workspace (is_bwd = 0) holds the values the forward
 * computed; after lr_block_bwd with ALL or POST_ATTN the backward workspace
 * (is_bwd = 1) holds the values the backward recomputed. Writes the byte
 * offset from the workspace start and the byte size; returns
 * LR_ERR_INVALID_ARG for an invalid shape, `which` or a NULL output. */
typedef enum { LR_WS_H = 0, LR_WS_M = 1 } lr_ws_tensor;
int lr_block_workspace_tensor(const lr_block_shape* shape, int32_t is_bwd, int32_t which,
                              size_t* offset, size_t* bytes);

/* Forward pass (BOOST project page, "Three supporting changes"; the chunk
 * layout of "Move the chunk boundary to the bottleneck").
 *   X [T, d]        block input (residual stream), must stay unchanged
 *                   until the matching lr_block_bwd has run
 *   O_attn [T, d]   attention-core output (read by POST_ATTN and ALL)
 *   Q, K, V [T, d]  outputs for the attention core (PRE_ATTN and ALL)
 *   Y [T, d]        block output (POST_ATTN and ALL)
 *   saved           outputs kept for the backward
 *   partials        required when shape->emit_partials; otherwise NULL or
 *                   the per-panel statistics outputs (see lr_block_partials)
 *   ws, ws_bytes    workspace of lr_block_workspace_bytes(shape, 0) bytes
 * Steps: Online RMSNorm of X fused into the grouped QKV down-projection
 * (per-row sums of squares accumulated per K-panel from the staged X tiles,
 * 1/RMS applied as a per-row epilogue scale); the three QKV up-projections
 * as one grouped launch; O's down-projection; O's up-projection with the
 * residual added in its epilogue (h = X + o_r B_o^T); Online RMSNorm of h
 * fused into the grouped gate/up down-projection; both MLP up-projections
 * in one tile with SiLU(gate) * up in the epilogue; the MLP down-projection;
 * and its up-projection with the residual (Y = h + d_r B_dn^T). */
int lr_block_fwd(const lr_block_shape* shape, const lr_block_weights* w, const void* X,
                 const void* O_attn, void* Q, void* K, void* V, void* Y,
                 const lr_block_saved* saved, const lr_block_partials* partials,
                 int32_t stage, void* ws, size_t ws_bytes, void* stream);

/* Backward pass from the r-wide activations (BOOST project page, "Three
 * supporting changes": checkpointing without communication). It recomputes
 * h, g, u and m from X, o_r and gu_r and writes
 *   dX [T, d], dO_attn [T, d]  (in `dtype`)
 *   grads                       (fp32), every weight and gamma
 * from dY, dQ, dK, dV [T, d]. X, O_attn and `saved` are those of the
 * forward. The RMSNorm backward takes its per-row statistic from the r-wide
 * tensors (sum_j dz_r z_r, equal to sum_k dxn xn), so no d-wide reduction is
 * needed. With stages, call POST_ATTN (needs dY; writes dO_attn, the
 * post-attention weight grads and gamma2's grad) before PRE_ATTN (needs dQ,
 * dK, dV; writes dX, the QKV weight grads and gamma1's grad), with the same
 * workspace. */
int lr_block_bwd(const lr_block_shape* shape, const lr_block_weights* w, const void* X,
                 const void* O_attn, const lr_block_saved* saved, const void* dY,
                 const void* dQ, const void* dK, const void* dV, void* dX, void* dO_attn,
                 const lr_block_grads* grads, int32_t stage, void* ws, size_t ws_bytes,
                 void* stream);

/* One operand pair of lr_grouped_lowrank_gemm. Y is M x N; with
 *   NT: Y = X W^T,  X [M, K] (ldx >= K), W [N, K] (ldw >= K)
 *   NN: Y = X W,    X [M, K] (ldx >= K), W [K, N] (ldw >= N)
 *   TN: Y = X^T W,  X [K, M] (ldx >= M), W [K, N] (ldw >= N)
 * `aux` is the epilogue's extra input for this pair: the residual R [M, N]
 * (ldaux >= N, in `dtype`) for LR_EPI_ADD_RESIDUAL, the row divisors
 * [M] (fp32) for LR_EPI_ROW_SCALE; NULL otherwise. */
typedef struct {
  int64_t M, N, K;
  const void* X;
  int64_t ldx;
  const void* W;
  int64_t ldw;
  void* Y;
  int64_t ldy;
  const void* aux;
  int64_t ldaux;
} lr_gemm_pair;

/* Grouped low-rank GEMM: G operand pairs in one launch (BOOST project page,
 * "Three supporting changes", linear layer grouping; the awesome-system-
 * papers summary, a batched GEMM over (input, weight) pairs). All pairs of
 * one call must have equal M, N, K. 1 <= G <= 3.
 * Output type: `dtype` for NT and NN, fp32 for TN (weight-gradient form).
 * Epilogues:
 *   LR_EPI_NONE          Y = acc
 *   LR_EPI_ADD_RESIDUAL  Y = acc + aux            (NT, NN)
 *   LR_EPI_ROW_SCALE     Y[i, :] = acc[i, :] / aux[i]   (NT, NN)
 *   LR_EPI_SWIGLU_PAIR   G = 2, NT only: both pairs share one tile and
 *                        Y_0 = SiLU(acc_0) * acc_1 (SiLU(z) = z / (1 +
 *                        e^-z)); Y_1 is not written
 */
int lr_grouped_lowrank_gemm(int32_t G, const lr_gemm_pair* pairs, int32_t dtype,
                            int32_t layout, int32_t epilogue, void* stream);

/* lr_grouped_lowrank_gemm with a caller-owned workspace. For the TN layout
 * on the bf16 pipelined path, an output grid too small to fill the GPU
 * (weight gradients of small factors, K = tokens) is computed as K-slices
 * whose fp32 partial products go to ws and are then summed slice by slice
 * in a fixed order, so results are deterministic; the slice count depends
 * only on the shape. Every other layout, dtype or shape runs exactly as
 * lr_grouped_lowrank_gemm and does not touch ws.
 * lr_grouped_lowrank_gemm_workspace_bytes returns the bytes ws must hold
 * for these pairs (0: none needed); ws must then be 256-byte aligned and
 * must not be used by other work until the call's kernels have finished on
 * `stream`. Errors as lr_grouped_lowrank_gemm, plus LR_ERR_WORKSPACE for a
 * missing, short or misaligned workspace. */
size_t lr_grouped_lowrank_gemm_workspace_bytes(int32_t G, const lr_gemm_pair* pairs,
                                               int32_t dtype, int32_t layout);
int lr_grouped_lowrank_gemm_ws(int32_t G, const lr_gemm_pair* pairs, int32_t dtype,
                               int32_t layout, int32_t epilogue, void* ws, size_t ws_bytes,
                               void* stream);

/* Online RMSNorm fused into a down-projection (BOOST project page, "Three
 * supporting changes", Online RMSNorm; the correction alpha = RMS_local /
 * RMS_global of the awesome-system-papers summary):
 *   out = RMSNorm(X; gamma, D = d_norm, eps) A^T
 * with X [T, d] (ldx), gamma [d], A [N, d] (lda), out [T, N] (ldo). The
 * per-row sum of squares is accumulated per K-panel (n_panels contiguous
 * panels of d / n_panels columns) from the same X tiles the GEMM stages, and
 * the global 1/RMS is applied as a per-row epilogue scale; the panel
 * rescalings rms_p / rms_g of the method cancel exactly against the local
 * normalisations, so they are not performed.
 *   rms_out [T]          fp32, nullable: the global RMS per row
 *   ss_out  [P, T]       fp32, nullable: per-panel sums of squares
 * With emit_partial = 1, out = (gamma * X) A^T unscaled (the rank's
 * all-reduce payload), ss_out [T] receives the total sum of squares and
 * rms_out is not written.
 * gamma may be NULL (all ones). Otherwise gamma is folded into A in the
 * workspace ws, which must hold N * d elements of `dtype`
 * (lr_online_rmsnorm_gemm_workspace_bytes). */
size_t lr_online_rmsnorm_gemm_workspace_bytes(int64_t N, int64_t d, int32_t dtype);
int lr_online_rmsnorm_gemm(int64_t T, int64_t d, int64_t N, int32_t n_panels, int64_t d_norm,
                           float eps, const void* X, int64_t ldx, const void* gamma,
                           const void* A, int64_t lda, void* out, int64_t ldo, float* rms_out,
                           float* ss_out, int32_t emit_partial, int32_t dtype, void* ws,
                           size_t ws_bytes, void* stream);

/* The same Online RMSNorm GEMM without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). It allocates nothing and
 * calls no allocating routine: the gamma-folded copy of A goes to a scratch
 * array built into the library, lr_online_rmsnorm_gemm_noalloc_max_bytes()
 * bytes (64 MiB) per GPU, held by each GPU the library runs on until the
 * process ends. Arguments, outputs and errors are those of
 * lr_online_rmsnorm_gemm; in addition, with gamma given, N * d elements of
 * `dtype` beyond the scratch size return LR_ERR_WORKSPACE before anything
 * is enqueued. The calling thread's current device must be the one `stream`
 * belongs to. Every call on one GPU shares that GPU's scratch: calls that
 * may overlap in time on one GPU (several streams or host threads) race,
 * and the caller must order them. */
size_t lr_online_rmsnorm_gemm_noalloc_max_bytes(void);
int lr_online_rmsnorm_gemm_noalloc(int64_t T, int64_t d, int64_t N, int32_t n_panels,
                                   int64_t d_norm, float eps, const void* X, int64_t ldx,
                                   const void* gamma, const void* A, int64_t lda, void* out,
                                   int64_t ldo, float* rms_out, float* ss_out,
                                   int32_t emit_partial, int32_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * Causal self-attention with rotary position embedding (the attention core
 * the block's forward leaves between Q, K, V and O). The BOOST pages do not
 * define this operation: their block diagram runs the factorised layers
 * around it, their related work cites FlashAttention and grouped-query
 * attention, and the project page's scope section names grouped-query
 * attention as a case the design is argued for. The library computes the
 * LLaMA-2 family's textbook form:
 *   - RoPE, half-split: for head dimension 128 and i < 64, the pair
 *     (x_i, x_{i+64}) of a token at position p (0 .. seq_len - 1 within its
 *     sequence) is rotated by the angle p * rope_base^(-2i/128), applied to
 *     every head of Q and K;
 *   - per sequence and query head h: O = softmax(q k^T / sqrt(128)) v with
 *     keys after the query masked (causal), k and v from key/value head
 *     h / (n_heads / n_kv_heads) (grouped-query attention; n_kv_heads =
 *     n_heads is multi-head attention);
 *   - LSE[h][t] = log(sum_j exp(q_t . k_j / sqrt(128))) over the unmasked
 *     keys (natural log), saved for the backward;
 *   - the backward of the above with respect to Q, K and V (the transposed
 *     rotation applied to the gradients of the rotated q and k; the query
 *     heads of a group add their key/value gradients).
 * Layout: token-major, contiguous. Q, O, dO, dQ are [T][n_heads * 128];
 * K, V, dK, dV are [T][n_kv_heads * 128]; head h occupies columns
 * [128 h, 128 h + 128). The T tokens are T / seq_len sequences of seq_len
 * consecutive tokens. LSE is [n_heads][T] fp32.
 * Supported: dtype LR_BF16 (fp32 accumulation), head_dim 128; other values
 * return LR_ERR_UNSUPPORTED. Requirements: T % seq_len == 0,
 * n_heads % n_kv_heads == 0, seq_len * n_heads * 256 < 2^31, rope_base > 1
 * and finite; bf16 pointers 16-byte aligned, LSE 4-byte aligned.
 * ------------------------------------------------------------------------ */
typedef struct {
  int64_t T;          /* tokens (all sequences)                      */
  int64_t seq_len;    /* tokens per sequence                         */
  int32_t n_heads;    /* query heads                                 */
  int32_t n_kv_heads; /* key/value heads, dividing n_heads           */
  int32_t head_dim;   /* 128                                         */
  int32_t dtype;      /* LR_BF16                                     */
  double rope_base;   /* 10000 for LLaMA-2                           */
} lr_attn_shape;

/* Bytes of workspace lr_attention_fwd (is_bwd = 0) or lr_attention_bwd
 * (is_bwd = 1) needs: the rotated Q and K, and for the backward the row sums
 * rowsum(dO * O); 0 if the shape is invalid. The workspace carries nothing
 * from the forward to the backward. */
size_t lr_attention_workspace_bytes(const lr_attn_shape* shape, int32_t is_bwd);

/* Forward: O and LSE from Q, K, V (all device memory; O and LSE are
 * overwritten). ws: device workspace of lr_attention_workspace_bytes(shape,
 * 0) bytes, 16-byte aligned. */
int lr_attention_fwd(const lr_attn_shape* shape, const void* Q, const void* K, const void* V,
                     void* O, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Backward: dQ, dK, dV (overwritten) from Q, K, V, the forward's O and LSE,
 * and dO. ws: device workspace of lr_attention_workspace_bytes(shape, 1)
 * bytes, 16-byte aligned. */
int lr_attention_bwd(const lr_attn_shape* shape, const void* Q, const void* K, const void* V,
                     const void* O, const void* dO, const float* lse, void* dQ, void* dK,
                     void* dV, void* ws, size_t ws_bytes, void* stream);

/* Measurement hook. While enabled, every kernel the library enqueues is
 * bracketed by a pair of HIP events recorded on the stream it is launched on
 * (events are created on first use and reused; no device memory is
 * allocated). lr_profile_enable(1) starts a new recording, (0) stops it.
 * lr_profile_collect waits for the recorded events, writes up to `max`
 * per-kernel aggregates in order of first launch, clears the recording and
 * returns the number of distinct kernels (which may exceed `max`). Each
 * aggregate holds the kernel's name, its launch count, the summed
 * milliseconds between its events and, for the memory-bound kernels (gamma
 * fold, rank-share finalize, row dots, split-K sums, column sums), the
 * algorithmic HBM bytes of those launches (every input read once, every
 * output written once; 0 for the GEMMs). Not thread-safe against concurrent
 * recording from several host threads. */
typedef struct {
  char name[64];
  int32_t count;
  float total_ms;
  double bytes;
} lr_kernel_time;

int lr_profile_enable(int32_t on);
int lr_profile_collect(lr_kernel_time* out, int32_t max);

/* While recording, enqueue each memory-bound launch n times back to back
 * between its pair of events (1 <= n <= 1000; 1 at load). Those kernels
 * only read buffers they do not write, so repeating them changes no result;
 * total_ms / count then measures one launch on the GPU without most of the
 * host-to-GPU launch latency a single launch between two events includes.
 * count includes the repetitions. Returns LR_ERR_INVALID_ARG outside the
 * range. */
int lr_profile_repeat(int32_t n);

/* Message of the last failed call on this thread ("" if none). */
const char* lr_last_error(void);

/* Library version string. */
const char* lr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LR_BLOCK_H_ */
