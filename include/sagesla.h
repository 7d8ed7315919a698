/*
 * sagesla.h — C ABI of the SageSLA forward on MI355X (gfx950).
 *
 * SageSLA is sparse-linear attention (SLA) whose exact branch uses
 * SageAttention-style INT8 QK^T.  Pages: "揭秘TurboDiffusion：如何让视频生成实现百倍加速？"
 * (sections "支柱一：低比特注意力加速 – SageAttention", "支柱二：稀疏线性注意力 – SLA":
 * INT8 attention with outlier smoothing; exact attention on the important
 * block interactions, ~90% sparse, plus a light linear-attention component;
 * the two stack) and "TurboDiffusion跨模态：图文音视频多模态融合探索"
 * (zizhi168.cn; sections 2.1, 2.2: top-k sparse selection with sla_topk; linear
 * complexity through a kernel-function approximation).
 *
 * Operator, per head (b,h) of Q, K, V in [B,H,N,d] bf16, blocks of 64 rows:
 *   1. block means of Q and K (float32, rows summed in order);
 *   2. mu = mean of K over the N tokens;
 *   3. block scores s_ij = qbar_i . (kbar_j - mu) (float32 FMA chain);
 *   4. per query block i keep the kb = clamp(floor(topk*T + 1e-6), 1, T)
 *      highest-scoring key blocks (kb = 0 when topk = 0), ties to the lower j;
 *   5. Q -> INT8, one scale amax/127 per 64-row block, round-half-even;
 *   6. K' = K - mu -> INT8 likewise;
 *   7. exact branch: softmax over the kept key blocks of the logits
 *      (q8 . k8) * dq_i * dk_j * sm_scale, times V (bf16);
 *   8. linear branch over the other ("marginal") key blocks:
 *      phi(Q) H_i / (phi(Q) . z_i), H_i = sum of phi(K_s)^T V_s, z_i = sum of
 *      phi(K_s), phi = softmax over the d channels;
 *   9. out = O_sparse + O_linear W^T (W [d_out][d_in] bf16, no bias) when
 *      use_linear, else O_sparse; out is bf16 [B,H,N,d].
 * Steps 1-6 and the int32 products of 7 are reproduced bit for bit by the CPU
 * oracle; the rest matches it within max-abs 2e-2 and relative-L2 1e-2.
 *
 * Plain SLA (qk_int8 = 0; the same pages' SLA without the low-bit step):
 * steps 5-6 are skipped and step 7's logits are (Q_r . K_s) * sm_scale from
 * the bf16 inputs (bf16 products, float32 sums); everything else is the
 * same.  The oracle's float64 exact-logit mode is its reference.
 *
 * Conventions
 *  - All device pointers are device memory of the current HIP device; all
 *    tensors are contiguous, 16-byte aligned.  The workspace is owned by the
 *    caller, at least sla_plan_info()'s workspace_bytes and 256-byte aligned;
 *    one workspace may not serve two calls at once (sla_attention_fwd_noalloc
 *    takes none: it uses a static one the library holds).
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    work: no device allocation, no host synchronisation.
 *  - sla_quantize must run before sla_attention_fwd on the same workspace
 *    and stream with the same q and k.
 *  - Arguments are checked on the host before anything is launched; a launch
 *    failure is reported as SLA_EHIP; device faults surface at the caller's
 *    next synchronisation.
 *  - Inputs must be finite.
 */
#ifndef SAGESLA_H
#define SAGESLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SLA_OK = 0,
  SLA_EINVAL = 1,        /* bad argument: null pointer, size, misalignment, topk */
  SLA_EUNSUPPORTED = 2,  /* valid but not built: d not in {64,128}, block != 64, N too large */
  SLA_EWORKSPACE = 3,    /* workspace smaller than sla_plan_info() says */
  SLA_EHIP = 4,          /* a HIP launch failed */
  SLA_ENOMEM = 5,        /* host allocation of the plan failed */
  SLA_ETOOLARGE = 6      /* the plan's workspace exceeds SLA_NOALLOC_WS_BYTES */
} sla_status;

typedef struct {
  int32_t B, H, N, d;  /* batch, heads, tokens (>= 1), head dim (64 or 128) */
  int32_t block;       /* block size; must be 64 */
  float topk;          /* kept fraction of key blocks, in [0, 1] (sla_topk) */
  int32_t use_linear;  /* 1: add the projected linear branch; 0: sparse branch only */
  float sm_scale;      /* softmax scale; 0 selects float32(1/sqrt(d)) */
  int32_t qk_int8;     /* 1: INT8 QK^T (SageSLA); 0: bf16 QK^T (plain SLA); else EINVAL */
  int32_t qk_fine;     /* INT8 scale granularity: 0 one scale per 64-row block; 1 the
                          SageAttention2++-style thread-level scales, one per 16 query
                          rows and one per 4 keys (needs qk_int8 = 1); else EINVAL */
  int32_t backward;    /* 1: the workspace also holds what sla_attention_bwd needs
                          (needs qk_int8 = 0, else EUNSUPPORTED); 0: forward only */
} sla_config;

typedef struct sla_plan_s *sla_plan_t;

/* Validate cfg and build a plan (host only, no HIP call).  *out is set on
 * SLA_OK.  The plan is immutable and may be shared by threads. */
sla_status sla_plan(const sla_config *cfg, sla_plan_t *out);

/* Free a plan (NULL is accepted). */
sla_status sla_plan_destroy(sla_plan_t plan);

/* T = number of 64-row blocks, kb = kept key blocks per query block,
 * workspace_bytes = workspace size needed.  Any output pointer may be NULL. */
sla_status sla_plan_info(sla_plan_t plan, int32_t *T, int32_t *kb, size_t *workspace_bytes);

/* Selection and Q quantisation (steps 1-5): block pooling, K mean, block
 * scores, top-k mask and kept lists, INT8 Q with its scales, all into the
 * workspace (plain SLA: no INT8 step).  Step 6, K' to INT8, runs in
 * sla_prepare_kv, which reads K once for it and for the linear states.
 * q, k: bf16 [B,H,N,d]. */
sla_status sla_quantize(sla_plan_t plan, const void *q, const void *k, void *ws,
                        size_t ws_bytes, void *stream);

/* Attention (steps 6-9): K' INT8 codes and scales (plain SLA: a bf16 copy of
 * K), V re-layout and per-key-block linear states, marginal-block states per
 * query block, block-sparse INT8/bf16 flash attention with the linear branch
 * and projection fused in its epilogue.
 * w_proj: bf16 [d][d] ([d_out][d_in]); may be NULL when use_linear is 0.
 * out: bf16 [B,H,N,d]; padding rows are never written. */
sla_status sla_attention_fwd(sla_plan_t plan, const void *q, const void *k, const void *v,
                             const void *w_proj, void *out, void *ws, size_t ws_bytes,
                             void *stream);

/* Size of the workspace the library holds for sla_attention_fwd_noalloc, per
 * GPU: 64 MiB (B*H = 2, N = 16384, d = 128 takes about 49 MiB). */
#define SLA_NOALLOC_WS_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc): sla_quantize
 * followed by sla_attention_fwd, same arguments and results, on a workspace
 * the library holds instead of a caller's.  That workspace is a static device
 * array of SLA_NOALLOC_WS_BYTES on each GPU the call runs on (the current
 * device; stream must belong to it); its address is looked up on the first
 * call on the device, so make that call outside graph capture, and the array
 * is held until the process ends.  No call allocates device or host memory.
 * A plan whose workspace_bytes exceed SLA_NOALLOC_WS_BYTES gets
 * SLA_ETOOLARGE; other argument errors as for the two calls; nothing is
 * launched on an error.  Every call on one GPU uses the same array, which
 * keeps the last call's contents (a call reads only what it wrote itself), so
 * calls that overlap on one GPU (other streams, other threads) race: the
 * caller serialises them. */
sla_status sla_attention_fwd_noalloc(sla_plan_t plan, const void *q, const void *k, const void *v,
                                     const void *w_proj, void *out, void *stream);

/* The two stages of sla_attention_fwd, for callers that schedule or time
 * them separately (same arguments, same order on one stream):
 * sla_prepare_kv: K' INT8 codes and scales (plain SLA: the bf16 K copy), V
 *   re-layout, per key block linear states and the marginal states per query
 *   block (the last two only when the linear branch is on);
 * sla_attend: the block-sparse attention kernel with the linear branch and
 *   projection in its epilogue, writing out.
 * Needs sla_quantize first; sla_attend needs sla_prepare_kv first. */
sla_status sla_prepare_kv(sla_plan_t plan, const void *k, const void *v, const void *w_proj,
                          void *ws, size_t ws_bytes, void *stream);
sla_status sla_attend(sla_plan_t plan, const void *q, void *out, void *ws, size_t ws_bytes,
                      void *stream);

/* Backward pass of plain SLA (the trainable operator: pages "揭秘TurboDiffusion…"
 * section "支柱二：稀疏线性注意力 – SLA" and the aiho.net news report (量子位, 2025-12-26)
 * section "2. SLA稀疏线性注意力": the sparse pattern and the linear component are
 * learned, so the operator is differentiated).  Gradients of sum(dout * out)
 * with the block mask held fixed (the top-k selection passes no gradient):
 *   sparse branch: dS = P (dP - rowsum(dout * O_sparse)), dQ = sm_scale dS K,
 *     dK = sm_scale dS^T Q, dV = P^T dout over the kept blocks;
 *   linear branch: through the quotient phi(Q) H_i / (phi(Q) . z_i), the
 *     channel softmax phi, the sums H_i of the marginal key-block states and
 *     the projection (dW = sum over all rows of dout^T O_linear).
 * Needs a plan with backward = 1 (qk_int8 = 0) and, on the same workspace and
 * stream, sla_quantize and sla_attention_fwd with the same q, k, v, w_proj
 * (with backward = 1 that forward also keeps each row's softmax normaliser
 * and the sparse-branch output in the workspace).  q, k, v, dout: bf16 [B,H,N,d];
 * dq, dk, dv: bf16 [B,H,N,d] outputs (float32 sums, rounded once);
 * dw: float32 [d][d] output ([d_out][d_in], summed over all heads), written
 * (zeros when the linear branch has no marginal block); w_proj and dw may be
 * NULL when use_linear = 0.  SLA_EUNSUPPORTED for a plan without backward. */
sla_status sla_attention_bwd(sla_plan_t plan, const void *q, const void *k, const void *v,
                             const void *w_proj, const void *dout, void *dq, void *dk, void *dv,
                             float *dw, void *ws, size_t ws_bytes, void *stream);

/* Static text for a status code. */
const char *sla_status_string(sla_status s);

/* Workspace regions, for tests and debugging (layouts in the comments). */
enum {
  SLA_WS_QBAR = 0, /* float [B*H][T][d]  block means of Q                         */
  SLA_WS_KSUM = 1, /* float [B*H][T][d]  block sums of K                          */
  SLA_WS_KBAR = 2, /* float [B*H][T][d]  block means of K                         */
  SLA_WS_MU = 3,   /* float [B*H][d]     K channel mean                           */
  SLA_WS_MASK = 4, /* uint64 [B*H][T][ceil(T/64)]  bit j%64 of word j/64 = kept   */
  SLA_WS_KEPT = 5, /* int32 [B*H][T][kb] kept key blocks, ascending               */
  SLA_WS_Q8 = 6,   /* int8 [B*H][T][64*d] per block, MFMA-fragment order:
                      byte (((r/16)*(d/64) + c/64)*64 + r%16 + 16*((c%64)/16))*16 + c%16
                      holds row r, channel c                                      */
  SLA_WS_K8 = 7,   /* int8, same layout as Q8, of K - mu (Q8, K8: 0 bytes when
                      qk_int8 = 0)                                                */
  SLA_WS_DQ = 8,   /* float [B*H][T] Q block scales ([B*H][T][4] with qk_fine:
                      one per 16 rows)                                            */
  SLA_WS_DK = 9,   /* float [B*H][T] K' block scales (1 when qk_int8 = 0;
                      [B*H][T][16] with qk_fine: one per 4 keys)                  */
  SLA_WS_LSE = 10, /* float [B*H][T][64] log2 of each row's softmax normaliser in
                      log2-scaled logit units (written by the qk_int8 = 0 forward;
                      p = exp2(logit * sm_scale * log2(e) - lse))                 */
  SLA_WS_COUNT = 11
};

/* Device pointer and size of one workspace region. */
sla_status sla_ws_view(sla_plan_t plan, void *ws, int32_t which, void **dev_ptr, size_t *bytes);

/* The int32 QK^T block products the attention kernel computes, for n pairs
 * given as int32 (bh, i, j) triples in device memory; dev_out receives n
 * tiles of int32 [64 query rows][64 key rows] (zeros for a triple out of
 * range).  Runs the attention kernel's own bound-path loop, with kept list
 * {j} for query block (bh, i), and stores each score accumulator (minus the
 * loop's bias) where the softmax reads it; nothing else is written.  Needs
 * sla_quantize and sla_prepare_kv first (Q8 and K8) and qk_int8 = 1; n >= 0
 * (else SLA_EINVAL). */
sla_status sla_debug_qk_int32(sla_plan_t plan, const void *ws, const int32_t *dev_pairs, int32_t n,
                              int32_t *dev_out, void *stream);

/* ---- W8A8 linear layers ------------------------------------------------------
 * Pages: "揭秘TurboDiffusion…" section "支柱三：W8A8线性层量化" and
 * the aiho.net news report (量子位, 2025-12-26) section "4. W8A8量化+底层算子重写": the linear layers
 * around attention (QKV and output projections) run with weights and
 * activations both INT8, quantised over 128 x 128 blocks.  Readings: the step-5
 * recipe per block (symmetric, scale = amax / 127, codes = round half to even
 * of x * float32(127 / amax), clamped to [-127, 127]; an all-zero block has
 * scale 0); ragged edge blocks; no bias.  Reproduced bit for bit by the CPU
 * oracle (codes, scales and the bf16 outputs). */

/* Block-128 INT8 quantisation of a bf16 matrix.
 * x: bf16 [rows][cols] row-major; codes: int8 [rows][cols] row-major (same
 * shape); scales: float32 [ceil(rows/128)][ceil(cols/128)].  All device
 * memory owned by the caller; x and codes 16-byte aligned.  cols must be a
 * multiple of 16 and ceil(rows/128) <= 65535 (else SLA_EUNSUPPORTED);
 * rows, cols >= 1 (else SLA_EINVAL).  Asynchronous on stream. */
sla_status sla_quant_b128(const void *x, int32_t rows, int32_t cols, void *codes, float *scales,
                          void *stream);

/* Block-scaled INT8 GEMM, y = X W^T: xq int8 [M][K] with scales sx
 * [ceil(M/128)][K/128] (activations), wq int8 [N][K] with scales sw
 * [ceil(N/128)][K/128] (the [out][in] weight), as sla_quant_b128 writes them;
 * y bf16 [M][N] row-major.  y[m][n] is the float32 sum, over the K blocks kb
 * in ascending order and from +0, of one fused multiply-add each:
 * float32(sx[m/128][kb] * sw[n/128][kb]) times the exact int32 block dot
 * product; then rounded to bf16 (nearest even).  K must be a multiple of 128
 * (else SLA_EUNSUPPORTED); M, N, K >= 1 (else SLA_EINVAL); xq, wq 16-byte
 * aligned.  Asynchronous on stream. */
sla_status sla_w8a8_gemm(const void *xq, const float *sx, const void *wq, const float *sw,
                         int32_t M, int32_t N, int32_t K, void *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGESLA_H */
