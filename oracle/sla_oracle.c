/*
 * CPU oracle for the SageSLA forward (sparse-linear attention with INT8
 * SageAttention-style QK^T).  TEST INFRASTRUCTURE ONLY: the tests, the
 * benchmark's CPU baseline and the smoke check may call it; the product path
 * never does.  It shares no code, header or table with the HIP library.
 *
 * Plain, single threaded, written for a reader checking it by eye against the
 * pages.  Sources (TurboDiffusion pages; no line numbers):
 *  - "揭秘TurboDiffusion：如何让视频生成实现百倍加速？" (xugj520.cn), sections
 *    "支柱一：低比特注意力加速 – SageAttention" (INT8 attention with outlier
 *    smoothing) and "支柱二：稀疏线性注意力 – SLA" (exact attention on the most
 *    important block interactions, ~90% sparsity, plus a light linear-attention
 *    component; the two stack into SageSLA);
 *  - "TurboDiffusion跨模态：图文音视频多模态融合探索" (zizhi168.cn),
 *    sections 2.1 (Top-K sparse
 *    selection, sla_topk) and 2.2 (SLA via kernel-function approximation;
 *    sla_topk 0.05 / 0.1 / 0.15);
 *  - the aiho.net news report (量子位, 2025-12-26), sections
 *    "1. SageAttention2++" (outlier smoothing, INT8) and "2. SLA稀疏线性注意力"
 *    (SLA stacks on low-bit attention).
 * The pages fix the operator only in outline; every step below that they leave
 * open follows the reading stated next to it.
 *
 * Notation: block size b = 64 for queries and keys; T = ceil(N/64) blocks;
 * block t holds rows t*64 .. t*64+n_t-1 with n_t = min(64, N - t*64); rows past
 * N are padding.  Tensors of one head are row-major [N][d] bfloat16 bits.
 *
 * Precision: steps 1-7 (pooling, K mean, block scores, top-k, Q/K INT8
 * quantisation, int32 scores) are done in float32 / integer exactly as written
 * (this file is compiled with -ffp-contract=off and without fast-math), since
 * they decide integers (the mask, the codes) and the HIP path must reproduce
 * them bit for bit.  Steps 8-10 (softmax branch, linear branch, combine) are
 * float64.
 *
 * The W8A8 linear-layer functions at the end (block-128 INT8 quantisation and
 * the block-scaled GEMM) are integer / float32 exactly as written too.
 *
 * Parity pins: see tests/test_oracle_pins.py.  Every function here is pinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SLA_REF_BLOCK 64

static float bf16f(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static int nblocks(int N) { return (N + SLA_REF_BLOCK - 1) / SLA_REF_BLOCK; }

static int rows_in(int t, int N) {
  int n = N - t * SLA_REF_BLOCK;
  return n < SLA_REF_BLOCK ? n : SLA_REF_BLOCK;
}

/* Number of kept key blocks per query block.  sla_topk is the kept fraction of
 * key blocks (zizhi168.cn section 2.2; xugj520.cn tutorial "--sla_topk 0.1",
 * i.e. 90% sparsity).  Reading: kb = 0 when topk = 0 (pure linear attention),
 * else clamp(floor(topk*T + 1e-6), 1, T) in float64.  Returns -1 when topk is
 * outside [0, 1] or NaN. */
int sla_ref_kb(int T, double topk) {
  if (!(topk >= 0.0 && topk <= 1.0)) return -1;
  if (topk == 0.0) return 0;
  long kb = (long)floor(topk * (double)T + 1e-6);
  if (kb < 1) kb = 1;
  if (kb > T) kb = T;
  return (int)kb;
}

/* Step 1, block pooling (SLA's block scores come from mean-pooled blocks).
 * sums[t][c] = float32 sum of X[t*64 + r][c] over valid rows r = 0, 1, ...
 * taken left to right; means[t][c] = float32(sums / n_t) with the division in
 * float64. */
void sla_ref_pool(const uint16_t *X, int N, int d, float *sums, float *means) {
  int T = nblocks(N);
  for (int t = 0; t < T; ++t) {
    int n = rows_in(t, N);
    for (int c = 0; c < d; ++c) {
      float s = 0.0f;
      for (int r = 0; r < n; ++r) s = s + bf16f(X[(size_t)(t * SLA_REF_BLOCK + r) * d + c]);
      sums[(size_t)t * d + c] = s;
      means[(size_t)t * d + c] = (float)((double)s / (double)n);
    }
  }
}

/* Step 2, the K channel mean used for smoothing (SageAttention removes the
 * common K offset before quantising).  mu[c] = float32(S / N) where S is the
 * float32 left-to-right sum over blocks t of ksums[t][c]; division in float64. */
void sla_ref_kmean(const float *ksums, int N, int d, float *mu) {
  int T = nblocks(N);
  for (int c = 0; c < d; ++c) {
    float s = 0.0f;
    for (int t = 0; t < T; ++t) s = s + ksums[(size_t)t * d + c];
    mu[c] = (float)((double)s / (double)N);
  }
}

/* Step 3, block scores s[i][j] = qbar_i . (kbar_j - mu).  Reading: the plain
 * score is qbar_i . kbar_j; subtracting mu changes every score of row i by the
 * same amount qbar_i . mu, so the per-row ranking is the same in exact
 * arithmetic, and it keeps the float32 values away from a large common offset.
 * kt = float32(kbar - mu); the dot product is a float32 fused multiply-add
 * chain over c = 0 .. d-1 starting from +0. */
void sla_ref_scores(const float *qbar, const float *kbar, const float *mu, int T, int d,
                    float *scores) {
  float *kt = (float *)malloc(sizeof(float) * (size_t)T * d);
  for (int j = 0; j < T; ++j)
    for (int c = 0; c < d; ++c) kt[(size_t)j * d + c] = kbar[(size_t)j * d + c] - mu[c];
  for (int i = 0; i < T; ++i)
    for (int j = 0; j < T; ++j) {
      float acc = 0.0f;
      for (int c = 0; c < d; ++c) acc = fmaf(qbar[(size_t)i * d + c], kt[(size_t)j * d + c], acc);
      scores[(size_t)i * T + j] = acc;
    }
  free(kt);
}

/* Step 4, top-k block selection per query block (zizhi168.cn section 2.1 "Top-K
 * 稀疏选择"): row i keeps the kb key blocks with the largest scores; equal
 * scores go to the lower block index.  mask[i][j] in {0,1}; kept[i][0..kb-1]
 * lists the kept j in ascending order.  Selection by repeated arg-max, the
 * plainest correct form. */
void sla_ref_topk(const float *scores, int T, int kb, uint8_t *mask, int32_t *kept) {
  for (int i = 0; i < T; ++i) {
    const float *s = scores + (size_t)i * T;
    uint8_t *m = mask + (size_t)i * T;
    memset(m, 0, (size_t)T);
    for (int n = 0; n < kb; ++n) {
      int best = -1;
      for (int j = 0; j < T; ++j) {
        if (m[j]) continue;
        if (best < 0 || s[j] > s[best]) best = j; /* strict '>' keeps the lower index on ties */
      }
      m[best] = 1;
    }
    int n = 0;
    for (int j = 0; j < T; ++j)
      if (m[j]) kept[(size_t)i * kb + n++] = j;
  }
}

/* Symmetric INT8 quantisation of one 64-row block with one scale (steps 5 and
 * 6).  Reading: range [-127, 127], no zero point, scale delta = amax / 127;
 * codes = round-half-even(x * float32(127 / amax)), clamped.  Padding rows are
 * zero. */
static void quant_block(const float *x /* [n][d] */, int n, int d, int8_t *codes /* [64][d] */,
                        float *delta) {
  float a = 0.0f;
  for (int r = 0; r < n; ++r)
    for (int c = 0; c < d; ++c) {
      float v = fabsf(x[(size_t)r * d + c]);
      if (v > a) a = v;
    }
  *delta = (float)((double)a / 127.0);
  float inv = a > 0.0f ? (float)(127.0 / (double)a) : 0.0f;
  memset(codes, 0, (size_t)SLA_REF_BLOCK * d);
  for (int r = 0; r < n; ++r)
    for (int c = 0; c < d; ++c) {
      float y = rintf(x[(size_t)r * d + c] * inv);
      if (y > 127.0f) y = 127.0f;
      if (y < -127.0f) y = -127.0f;
      codes[(size_t)r * d + c] = (int8_t)y;
    }
}

/* One 64-row block quantised in groups of g consecutive rows (g divides 64),
 * each group with its own scale (quant_block on the group); rows past n are
 * padding (zero codes; a group of padding only has scale 0).  codes is
 * [64][d], delta [64/g]. */
static void quant_groups(const float *x /* [n][d] */, int n, int d, int g, int8_t *codes,
                         float *delta) {
  int8_t *tmp = (int8_t *)malloc((size_t)SLA_REF_BLOCK * d);
  for (int q = 0; q < SLA_REF_BLOCK / g; ++q) {
    int r0 = q * g;
    int ng = n - r0 < 0 ? 0 : (n - r0 < g ? n - r0 : g);
    quant_block(x + (size_t)r0 * d, ng, d, tmp, delta + q);
    memcpy(codes + (size_t)r0 * d, tmp, (size_t)g * d);
  }
  free(tmp);
}

/* Step 5: Q -> INT8, one scale per group of g rows of each 64-row block (g =
 * 64: one scale per block; g = 16: SageAttention2++-style finer scales, one
 * per 16 queries, the rows of one matrix-core output tile).  q8 is [T*64][d],
 * dq [T][64/g]. */
void sla_ref_quant_q_g(const uint16_t *Q, int N, int d, int g, int8_t *q8, float *dq) {
  int T = nblocks(N);
  float *x = (float *)malloc(sizeof(float) * SLA_REF_BLOCK * d);
  for (int t = 0; t < T; ++t) {
    int n = rows_in(t, N);
    for (int r = 0; r < n; ++r)
      for (int c = 0; c < d; ++c)
        x[(size_t)r * d + c] = bf16f(Q[(size_t)(t * SLA_REF_BLOCK + r) * d + c]);
    quant_groups(x, n, d, g, q8 + (size_t)t * SLA_REF_BLOCK * d, dq + (size_t)t * (SLA_REF_BLOCK / g));
  }
  free(x);
}

void sla_ref_quant_q(const uint16_t *Q, int N, int d, int8_t *q8, float *dq) {
  sla_ref_quant_q_g(Q, N, d, SLA_REF_BLOCK, q8, dq);
}

/* Step 6: K smoothing then INT8.  k' = float32(K - mu[c]) (mu = 0 turns the
 * smoothing off), then one scale per group of g rows as for Q (g = 64: per
 * block; g = 4: the finer, "thread-level" scales of SageAttention2++, one per
 * 4 keys).  dk is [T][64/g]. */
void sla_ref_quant_k_g(const uint16_t *K, const float *mu, int N, int d, int g, int8_t *k8,
                       float *dk) {
  int T = nblocks(N);
  float *x = (float *)malloc(sizeof(float) * SLA_REF_BLOCK * d);
  for (int t = 0; t < T; ++t) {
    int n = rows_in(t, N);
    for (int r = 0; r < n; ++r)
      for (int c = 0; c < d; ++c)
        x[(size_t)r * d + c] = bf16f(K[(size_t)(t * SLA_REF_BLOCK + r) * d + c]) - mu[c];
    quant_groups(x, n, d, g, k8 + (size_t)t * SLA_REF_BLOCK * d, dk + (size_t)t * (SLA_REF_BLOCK / g));
  }
  free(x);
}

void sla_ref_quant_k(const uint16_t *K, const float *mu, int N, int d, int8_t *k8, float *dk) {
  sla_ref_quant_k_g(K, mu, N, d, SLA_REF_BLOCK, k8, dk);
}

/* Step 7: int32 scores of query block i against key block j,
 * A[r][s] = sum_c q8[i*64+r][c] * k8[j*64+s][c] (exact). */
void sla_ref_qk_int32(const int8_t *q8, const int8_t *k8, int d, int i, int j, int32_t *A) {
  for (int r = 0; r < SLA_REF_BLOCK; ++r)
    for (int s = 0; s < SLA_REF_BLOCK; ++s) {
      int32_t acc = 0;
      for (int c = 0; c < d; ++c)
        acc += (int32_t)q8[(size_t)(i * SLA_REF_BLOCK + r) * d + c] *
               (int32_t)k8[(size_t)(j * SLA_REF_BLOCK + s) * d + c];
      A[r * SLA_REF_BLOCK + s] = acc;
    }
}

/* Step 8, the exact (softmax) branch for the valid rows of query block i,
 * restricted to its kept key blocks.  Quantised mode (quantized != 0): logit
 * = A[r][s] * dq(i, r) * dk(j, s) * sm_scale from the INT8 codes, the scales
 * of the row groups (gq query rows, gk keys; 64 = one per block) holding r
 * and s.  Exact mode: logit = (Q_r . K_s) * sm_scale from the bf16 inputs in
 * float64.  Padding keys are excluded.  Softmax in float64 with the row
 * maximum subtracted; out is [n_i][d]; all zeros when kb = 0. */
void sla_ref_sparse_block_g(int quantized, const int8_t *q8, const float *dq, const int8_t *k8,
                            const float *dk, int gq, int gk, const uint16_t *Q, const uint16_t *K,
                            const uint16_t *V, int N, int d, float sm_scale, const int32_t *kept_i,
                            int kb, int i, double *out) {
  int ni = rows_in(i, N);
  size_t nl = (size_t)kb * SLA_REF_BLOCK; /* logits per row */
  double *lg = (double *)malloc(sizeof(double) * (size_t)SLA_REF_BLOCK * (nl ? nl : 1));
  int32_t *A = (int32_t *)malloc(sizeof(int32_t) * SLA_REF_BLOCK * SLA_REF_BLOCK);
  double *acc = (double *)malloc(sizeof(double) * d);
  /* logits lg[r][n*64 + s] of every row against every kept key; padding keys -inf */
  for (int n = 0; n < kb; ++n) {
    int j = kept_i[n];
    int nj = rows_in(j, N);
    if (quantized) sla_ref_qk_int32(q8, k8, d, i, j, A);
    for (int r = 0; r < ni; ++r)
      for (int s = 0; s < SLA_REF_BLOCK; ++s) {
        double l = -INFINITY;
        if (s < nj) {
          if (quantized) {
            l = (double)A[r * SLA_REF_BLOCK + s] * (double)dq[i * (SLA_REF_BLOCK / gq) + r / gq] *
                (double)dk[j * (SLA_REF_BLOCK / gk) + s / gk] * (double)sm_scale;
          } else {
            double dot = 0.0;
            for (int c = 0; c < d; ++c)
              dot += (double)bf16f(Q[(size_t)(i * SLA_REF_BLOCK + r) * d + c]) *
                     (double)bf16f(K[(size_t)(j * SLA_REF_BLOCK + s) * d + c]);
            l = dot * (double)sm_scale;
          }
        }
        lg[(size_t)r * nl + (size_t)n * SLA_REF_BLOCK + s] = l;
      }
  }
  for (int r = 0; r < ni; ++r) {
    const double *row = lg + (size_t)r * nl;
    double m = -INFINITY;
    for (size_t e = 0; e < nl; ++e)
      if (row[e] > m) m = row[e];
    double den = 0.0;
    for (int c = 0; c < d; ++c) acc[c] = 0.0;
    for (int n = 0; n < kb; ++n) {
      int j = kept_i[n];
      int nj = rows_in(j, N);
      for (int s = 0; s < nj; ++s) {
        double p = exp(row[(size_t)n * SLA_REF_BLOCK + s] - m);
        den += p;
        for (int c = 0; c < d; ++c)
          acc[c] += p * (double)bf16f(V[(size_t)(j * SLA_REF_BLOCK + s) * d + c]);
      }
    }
    for (int c = 0; c < d; ++c) out[(size_t)r * d + c] = kb > 0 ? acc[c] / den : 0.0;
  }
  free(lg);
  free(A);
  free(acc);
}

void sla_ref_sparse_block(int quantized, const int8_t *q8, const float *dq, const int8_t *k8,
                          const float *dk, const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                          int N, int d, float sm_scale, const int32_t *kept_i, int kb, int i,
                          double *out) {
  sla_ref_sparse_block_g(quantized, q8, dq, k8, dk, SLA_REF_BLOCK, SLA_REF_BLOCK, Q, K, V, N, d,
                         sm_scale, kept_i, kb, i, out);
}

/* The linear-attention feature map phi.  The pages only say "kernel-function
 * approximation" (zizhi168.cn section 2.2).  Reading: phi(x) = softmax of x
 * over its d channels (positive, bounded, so the normaliser stays > 0 and the
 * states stay finite), in float64, applied to the raw bf16 Q and K rows. */
static void phi(const uint16_t *x, int d, double *f) {
  double mx = -INFINITY, s = 0.0;
  for (int c = 0; c < d; ++c)
    if ((double)bf16f(x[c]) > mx) mx = (double)bf16f(x[c]);
  for (int c = 0; c < d; ++c) {
    f[c] = exp((double)bf16f(x[c]) - mx);
    s += f[c];
  }
  for (int c = 0; c < d; ++c) f[c] /= s;
}

/* Step 9a, per key block linear-attention states:
 * Hb[j][c][c'] = sum over valid keys s of block j of phi(K_s)[c] * V_s[c'],
 * zb[j][c] = sum over the same keys of phi(K_s)[c].  Padding keys add
 * nothing. */
void sla_ref_linear_states(const uint16_t *K, const uint16_t *V, int N, int d, double *Hb,
                           double *zb) {
  int T = nblocks(N);
  double *f = (double *)malloc(sizeof(double) * d);
  memset(Hb, 0, sizeof(double) * (size_t)T * d * d);
  memset(zb, 0, sizeof(double) * (size_t)T * d);
  for (int j = 0; j < T; ++j) {
    int nj = rows_in(j, N);
    for (int s = 0; s < nj; ++s) {
      size_t row = (size_t)(j * SLA_REF_BLOCK + s) * d;
      phi(K + row, d, f);
      for (int c = 0; c < d; ++c) {
        zb[(size_t)j * d + c] += f[c];
        for (int c2 = 0; c2 < d; ++c2)
          Hb[((size_t)j * d + c) * d + c2] += f[c] * (double)bf16f(V[row + c2]);
      }
    }
  }
  free(f);
}

/* Step 9b, the linear branch for the valid rows of query block i over its
 * marginal key blocks (every valid block the top-k did not keep; reading: two
 * classes only, "the linear branch covers the remaining blocks").
 * H = sum_{j: mask[i][j] = 0} Hb[j], z likewise;
 * out[r] = phi(Q_r) H / (phi(Q_r) . z), and 0 when there is no marginal block
 * or the normaliser is not positive. */
void sla_ref_linear_block(const uint16_t *Q, const double *Hb, const double *zb,
                          const uint8_t *mask_i, int N, int d, int i, double *out) {
  int T = nblocks(N);
  int ni = rows_in(i, N);
  double *H = (double *)calloc((size_t)d * d, sizeof(double));
  double *z = (double *)calloc((size_t)d, sizeof(double));
  double *f = (double *)malloc(sizeof(double) * d);
  int nmarg = 0;
  for (int j = 0; j < T; ++j) {
    if (mask_i[j]) continue;
    ++nmarg;
    for (size_t e = 0; e < (size_t)d * d; ++e) H[e] += Hb[(size_t)j * d * d + e];
    for (int c = 0; c < d; ++c) z[c] += zb[(size_t)j * d + c];
  }
  for (int r = 0; r < ni; ++r) {
    phi(Q + (size_t)(i * SLA_REF_BLOCK + r) * d, d, f);
    double den = 0.0;
    for (int c = 0; c < d; ++c) den += f[c] * z[c];
    for (int c2 = 0; c2 < d; ++c2) {
      double num = 0.0;
      for (int c = 0; c < d; ++c) num += f[c] * H[(size_t)c * d + c2];
      out[(size_t)r * d + c2] = (nmarg > 0 && den > 0.0) ? num / den : 0.0;
    }
  }
  free(H);
  free(z);
  free(f);
}

/* Step 10, combine: O = O_s + O_l W^T when the linear branch is on, with W the
 * d x d projection stored [d_out][d_in] (bf16), no bias; otherwise O = O_s.
 * Applies to n rows. */
void sla_ref_combine(const double *Os, const double *Ol, const uint16_t *W, int use_linear, int n,
                     int d, double *out) {
  for (int r = 0; r < n; ++r)
    for (int c2 = 0; c2 < d; ++c2) {
      double v = Os[(size_t)r * d + c2];
      if (use_linear) {
        double p = 0.0;
        for (int c = 0; c < d; ++c) p += Ol[(size_t)r * d + c] * (double)bf16f(W[(size_t)c2 * d + c]);
        v += p;
      }
      out[(size_t)r * d + c2] = v;
    }
}

/* ---------------------------------------------------------------------------
 * W8A8 linear layers ("揭秘TurboDiffusion…" section "支柱三：W8A8线性层量化";
 * aiho.net news report (量子位, 2025-12-26) section "4. W8A8量化+底层算子重写"): weights and
 * activations both INT8, quantised over 128 x 128 blocks.  Readings: the
 * scale recipe of step 5 per block (symmetric, amax / 127, round half to
 * even, clamp to [-127, 127]; a block of zeros has scale 0 and zero codes);
 * edge blocks of a matrix whose sides are not multiples of 128 are ragged.
 * ------------------------------------------------------------------------- */
#define SLA_REF_WB 128

/* X bf16 [R][C] -> codes int8 [R][C], scales float [ceil(R/128)][ceil(C/128)]. */
void sla_ref_quant_b128(const uint16_t *X, int R, int C, int8_t *codes, float *scales) {
  int RB = (R + SLA_REF_WB - 1) / SLA_REF_WB, CB = (C + SLA_REF_WB - 1) / SLA_REF_WB;
  for (int rb = 0; rb < RB; ++rb)
    for (int cb = 0; cb < CB; ++cb) {
      int r0 = rb * SLA_REF_WB, c0 = cb * SLA_REF_WB;
      int r1 = r0 + SLA_REF_WB < R ? r0 + SLA_REF_WB : R;
      int c1 = c0 + SLA_REF_WB < C ? c0 + SLA_REF_WB : C;
      float a = 0.0f;
      for (int r = r0; r < r1; ++r)
        for (int c = c0; c < c1; ++c) {
          float v = fabsf(bf16f(X[(size_t)r * C + c]));
          if (v > a) a = v;
        }
      scales[(size_t)rb * CB + cb] = (float)((double)a / 127.0);
      float inv = a > 0.0f ? (float)(127.0 / (double)a) : 0.0f;
      for (int r = r0; r < r1; ++r)
        for (int c = c0; c < c1; ++c) {
          float y = rintf(bf16f(X[(size_t)r * C + c]) * inv);
          if (y > 127.0f) y = 127.0f;
          if (y < -127.0f) y = -127.0f;
          codes[(size_t)r * C + c] = (int8_t)y;
        }
    }
}

/* Y = X W^T for X [M][K], W [N][K] (the [out][in] weight of a linear layer):
 * y[m][n] = sum over the K blocks kb in ascending order of
 * float32(sx[m/128][kb] * sw[n/128][kb]) * A_kb, A_kb the exact int32 dot
 * product of the block's codes.  Reading: the block terms are accumulated in
 * float32 from +0, one fused multiply-add per block (the plain blocked
 * accumulation); no bias.  y32 (may be NULL) receives the float32 sums, y
 * (may be NULL) the bf16 results rounded to nearest even.  K is a multiple of
 * 128. */
void sla_ref_w8a8_gemm(const int8_t *xq, const float *sx, const int8_t *wq, const float *sw, int M,
                       int N, int K, float *y32, uint16_t *y) {
  int KB = K / SLA_REF_WB;
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n) {
      float acc = 0.0f;
      for (int kb = 0; kb < KB; ++kb) {
        int32_t A = 0;
        for (int k = kb * SLA_REF_WB; k < (kb + 1) * SLA_REF_WB; ++k)
          A += (int32_t)xq[(size_t)m * K + k] * (int32_t)wq[(size_t)n * K + k];
        float s = sx[(size_t)(m / SLA_REF_WB) * KB + kb] * sw[(size_t)(n / SLA_REF_WB) * KB + kb];
        acc = fmaf((float)A, s, acc);
      }
      if (y32) y32[(size_t)m * N + n] = acc;
      if (y) {
        /* bf16 nearest even: keep the upper half, round up past the midpoint
         * or at it when the kept half is odd (finite values) */
        uint32_t u;
        memcpy(&u, &acc, sizeof u);
        uint32_t hi = u >> 16, lo = u & 0xFFFFu;
        if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;
        y[(size_t)m * N + n] = (uint16_t)hi;
      }
    }
}
