// Block pooling, K channel mean and INT8 quantisation of Q and K - mu.
//
// Pages: "揭秘TurboDiffusion…" section "支柱一：低比特注意力加速 – SageAttention"
// (attention in INT8 with outlier smoothing) and section "支柱二：稀疏线性注意力 – SLA"
// (block selection from pooled blocks); the aiho.net news report (量子位, 2025-12-26)
// section "1. SageAttention2++" (outlier smoothing).  The float32 operation order below is
// part of the operator's definition (block means feed an integer decision, the
// top-k mask): sums run over the rows of a block in order, the K mean over the
// blocks in order, divisions are done in float64 and rounded once.
//
// Memory bound: each kernel streams its input once (Q, K: 2 x 2 bytes per
// element read by the pooling kernel, K once more by the K quantiser) and
// writes one byte per element.  Codes are staged in LDS so the global stores
// are whole 16-byte lanes of a 1 KiB fragment.
#include "sla_internal.h"

namespace sla {

// One wave per (head, block).  Lanes 0..D/4-1 own four channels of Q for all
// 64 rows, lanes 32..32+D/4-1 the same channels of K; each lane adds its rows
// in order (float32).  Q's values stay in registers for the quantisation
// (QUANT; the bf16 QK^T mode has no INT8 step).  FINE: one scale per 16 rows
// (dq [blk][4]) instead of one per block.
template <int D, bool QUANT, bool FINE>
__global__ __launch_bounds__(256) void k_pool_quant_q(const uint16_t *__restrict__ Q,
                                                      const uint16_t *__restrict__ K, int N, int T,
                                                      int nblk, float *__restrict__ qbar,
                                                      float *__restrict__ ksum,
                                                      float *__restrict__ kbar,
                                                      int8_t *__restrict__ q8,
                                                      float *__restrict__ dq) {
  constexpr int LPT = D / 4;  // lanes per tensor
  constexpr int KC = D / 64;
  __shared__ __attribute__((aligned(16))) int8_t stage[4][64 * D];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int blk = blockIdx.x * 4 + w;
  const bool live = blk < nblk;
  const int bh = live ? blk / T : 0, t = live ? blk - (blk / T) * T : 0;
  const int n = min(BLK, N - t * BLK);
  const int half = l >> 5, cl = l & 31;
  const bool act = live && cl < LPT;
  const uint16_t *X = half ? K : Q;
  const size_t base = ((size_t)bh * N + (size_t)t * BLK) * D + 4 * cl;

  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  float ag[4] = {0.f, 0.f, 0.f, 0.f};  // amax of rows 16 g .. 16 g + 15 (all rows: ag[0])
  uint2 vals[BLK];
  auto accum = [&](uint2 v, int r) {
    const float a = bf2f(v.x & 0xFFFF), b = bf2f(v.x >> 16), c = bf2f(v.y & 0xFFFF), d = bf2f(v.y >> 16);
    s0 = s0 + a;
    s1 = s1 + b;
    s2 = s2 + c;
    s3 = s3 + d;
    const int gi = FINE ? (r >> 4) : 0;
    ag[gi] = fmaxf(ag[gi], fmaxf(fmaxf(fabsf(a), fabsf(b)), fmaxf(fabsf(c), fabsf(d))));
  };
  if (n == BLK) {
    // full block (all but a head's last): every load is unconditional, so
    // they are all in flight at once; lanes without channels read channels
    // 0..3 of the same row (values already present: the block max is
    // unchanged, and their sums are not stored)
    const size_t base_c = base - 4 * cl + 4 * (cl < LPT ? cl : 0);
#pragma unroll
    for (int r = 0; r < BLK; ++r) vals[r] = *(const uint2 *)(X + base_c + (size_t)r * D);
#pragma unroll
    for (int r = 0; r < BLK; ++r) accum(vals[r], r);
  } else {
#pragma unroll
    for (int r = 0; r < BLK; ++r) {
      uint2 v = make_uint2(0u, 0u);
      if (act && r < n) v = *(const uint2 *)(X + base + (size_t)r * D);
      vals[r] = v;
      if (act && r < n) accum(v, r);
    }
  }
  if (act) {
    const size_t o = ((size_t)blk) * D + 4 * cl;
    const double dn = (double)n;
    float4 mean = make_float4((float)((double)s0 / dn), (float)((double)s1 / dn),
                              (float)((double)s2 / dn), (float)((double)s3 / dn));
    if (half == 0) {
      *(float4 *)(qbar + o) = mean;
    } else {
      *(float4 *)(ksum + o) = make_float4(s0, s1, s2, s3);
      *(float4 *)(kbar + o) = mean;
    }
  }
  if constexpr (!QUANT) return;
  // amax of Q over lanes 0..31, per block or per 16-row group (max is exact
  // in any order)
  constexpr int NG = FINE ? 4 : 1;
  float inv[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    float amax = ag[gi];
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    amax = __shfl(amax, 0, 64);
    inv[gi] = amax > 0.f ? (float)(127.0 / (double)amax) : 0.f;
    if (live && l == 0) dq[(size_t)blk * NG + gi] = (float)((double)amax / 127.0);
  }

  if (half == 0 && cl < LPT) {
#pragma unroll
    for (int r = 0; r < BLK; ++r) {
      uint2 v = vals[r];
      float x[4] = {bf2f(v.x & 0xFFFF), bf2f(v.x >> 16), bf2f(v.y & 0xFFFF), bf2f(v.y >> 16)};
      uint32_t packed = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float y = __builtin_rintf(x[e] * inv[FINE ? (r >> 4) : 0]);
        y = fminf(fmaxf(y, -127.f), 127.f);
        packed |= ((uint32_t)(uint8_t)(int8_t)(int)y) << (8 * e);
      }
      if (r >= n) packed = 0;
      *(uint32_t *)(&stage[w][i8_off(r, 4 * cl, KC)]) = packed;
    }
  }
  __syncthreads();
  if (live) {
    const uint4 *src = (const uint4 *)stage[w];
    uint4 *dst = (uint4 *)(q8 + (size_t)blk * BLK * D);
#pragma unroll
    for (int it = 0; it < (BLK * D) / (16 * 64); ++it) dst[it * 64 + l] = src[it * 64 + l];
  }
}

// mu[bh][c] = float32((sum over blocks t in order of ksum[bh][t][c]) / N).
// Loads are issued 32 at a time ahead of the (ordered) additions.
__global__ void k_kmean(const float *__restrict__ ksum, int N, int T, int D, float *__restrict__ mu) {
  constexpr int BATCH = 32;
  const int bh = blockIdx.x, c = threadIdx.x;
  const float *p = ksum + (size_t)bh * T * D + c;
  float s = 0.f;
  int t = 0;
  for (; t + BATCH <= T; t += BATCH) {
    float v[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) v[q] = p[(size_t)(t + q) * D];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) s = s + v[q];
  }
  for (; t < T; ++t) s = s + p[(size_t)t * D];
  mu[(size_t)bh * D + c] = (float)((double)s / (double)N);
}

// bf16 QK^T mode: one wave per (head, block): the raw K rows in bfk_off order
// (an exact copy, padding rows zero); dkn = the largest L2 norm of a row
// minus the K mean, ||k_s - mu||, over the block's 64 rows (padding rows
// count as zero rows, norm ||mu||): with ||q_r|| it bounds q_r . k_s - q_r . mu
// for every key of the block, the offset the attention kernel subtracts (the
// softmax is unchanged by a per-row constant); dk = 1 (the logit scale is
// sm_scale alone).
template <int D>
__global__ __launch_bounds__(256) void k_prep_kbf(const uint16_t *__restrict__ K,
                                                  const float *__restrict__ mu, int N, int T,
                                                  int nblk, uint16_t *__restrict__ kbf,
                                                  float *__restrict__ dk, float *__restrict__ dkn,
                                                  float *__restrict__ dkx) {
  constexpr int LPR = D / 4;       // lanes per row
  constexpr int RPI = 64 / LPR;    // rows per step
  constexpr int STEPS = BLK / RPI;
  constexpr int KC32 = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t stage[4][64 * D];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int blk = blockIdx.x * 4 + w;
  const bool live = blk < nblk;
  const int bh = live ? blk / T : 0, t = live ? blk - (blk / T) * T : 0;
  const int n = min(BLK, N - t * BLK);
  const int c0 = 4 * (l % LPR), r0 = l / LPR;
  const size_t base = ((size_t)bh * N + (size_t)t * BLK) * D + c0;
  const float4 m4 = *(const float4 *)(mu + (size_t)bh * D + c0);

  uint2 raw[STEPS];
  if (n == BLK) {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) raw[s] = *(const uint2 *)(K + base + (size_t)(s * RPI + r0) * D);
  } else {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const int r = s * RPI + r0;
      raw[s] = make_uint2(0u, 0u);
      if (live && r < n) raw[s] = *(const uint2 *)(K + base + (size_t)r * D);
    }
  }
  float nmax = 0.f;  // max over rows of the squared L2 norm
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int r = s * RPI + r0;
    const uint32_t p0 = raw[s].x, p1 = raw[s].y;  // zero for padding rows
    const float e0 = bf2f(p0 & 0xFFFF) - m4.x, e1 = bf2f(p0 >> 16) - m4.y,
                e2 = bf2f(p1 & 0xFFFF) - m4.z, e3 = bf2f(p1 >> 16) - m4.w;
    float sq = e0 * e0 + e1 * e1 + e2 * e2 + e3 * e3;
    *(uint2 *)(&stage[w][bfk_off(r, c0, KC32)]) = make_uint2(p0, p1);
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) sq += __shfl_xor(sq, off, 64);
    nmax = fmaxf(nmax, sq);
  }
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) nmax = fmaxf(nmax, __shfl_xor(nmax, off, 64));
  if (live && l == 0) {
    dk[blk] = 1.0f;
    dkx[blk] = 1.0f;
    dkn[blk] = sqrtf(nmax);
  }
  __syncthreads();
  if (live) {
    const uint4 *src = (const uint4 *)stage[w];
    uint4 *dst = (uint4 *)(kbf + (size_t)blk * BLK * D);
#pragma unroll
    for (int it = 0; it < (BLK * D * 2) / (16 * 64); ++it) dst[it * 64 + l] = src[it * 64 + l];
  }
}

void launch_pool_quant_q(const Plan &p, const uint16_t *q, const uint16_t *k, const WsPtrs &ws,
                         hipStream_t st) {
  const int nblk = p.BH * p.T;
  dim3 grid((nblk + 3) / 4), block(256);
  auto kern = p.d == 128
                  ? (p.qk_int8 ? (p.qk_fine ? k_pool_quant_q<128, true, true> : k_pool_quant_q<128, true, false>)
                               : k_pool_quant_q<128, false, false>)
                  : (p.qk_int8 ? (p.qk_fine ? k_pool_quant_q<64, true, true> : k_pool_quant_q<64, true, false>)
                               : k_pool_quant_q<64, false, false>);
  hipLaunchKernelGGL(kern, grid, block, 0, st, q, k, p.N, p.T, nblk, ws.qbar, ws.ksum, ws.kbar, ws.q8,
                     ws.dq);
}

void launch_kmean(const Plan &p, const WsPtrs &ws, hipStream_t st) {
  hipLaunchKernelGGL(k_kmean, dim3(p.BH), dim3(p.d), 0, st, ws.ksum, p.N, p.T, p.d, ws.mu);
}

void launch_prep_kbf(const Plan &p, const uint16_t *k, const WsPtrs &ws, hipStream_t st) {
  const int nblk = p.BH * p.T;
  dim3 grid((nblk + 3) / 4), block(256);
  if (p.d == 128)
    hipLaunchKernelGGL(k_prep_kbf<128>, grid, block, 0, st, k, ws.mu, p.N, p.T, nblk, ws.kbf, ws.dk,
                       ws.dkn, ws.dkx);
  else
    hipLaunchKernelGGL(k_prep_kbf<64>, grid, block, 0, st, k, ws.mu, p.N, p.T, nblk, ws.kbf, ws.dk,
                       ws.dkn, ws.dkx);
}

}  // namespace sla
