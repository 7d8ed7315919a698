// Linear-attention branch of SLA: per key block states and, per query block,
// their sum over the marginal (non-kept) key blocks.
//
// Pages: "揭秘TurboDiffusion…" section "支柱二：稀疏线性注意力 – SLA" (a light
// linear-attention component complements the sparse exact part);
// "TurboDiffusion深度解析…" section 2.2 (linear complexity through a
// kernel-function approximation).  The feature map phi is read as a softmax
// over the d channels of each raw K (and Q) row.
//
// k_kv_prep, one workgroup per key block j (memory bound: reads K_j and V_j,
//   writes V_j re-laid for the attention kernel and the state
//   Hb_j = phi(K_j)^T V_j (d x d) with zb_j = phi(K_j)^T 1, bf16, through
//   bf16 MFMA).
// k_marginal, per head a GEMM H = (1 - M) Hb of [T x T] by [T x F]
//   (F = d*d + d padded), bf16 MFMA with float32 accumulation; A is built on
//   the fly from the mask bits.
#include "sla_internal.h"

namespace sla {

// One workgroup (4 waves) per key block.  LDS: V and phi(K) as bf16 rows with
// an odd dword pitch (bank-conflict free column reads).
template <int D, bool LIN>
__global__ __launch_bounds__(256) void k_kv_prep(const uint16_t *__restrict__ K,
                                                 const uint16_t *__restrict__ V, int N, int T,
                                                 int F, uint16_t *__restrict__ vt,
                                                 uint16_t *__restrict__ hb) {
  constexpr int P = D + 2;  // row pitch in bf16 (odd number of dwords)
  constexpr int CG = D / 16;
  constexpr int KC32 = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 64 * P];
  uint16_t *sv = smem, *sk = smem + 64 * P;
  const int blk = blockIdx.x;
  const int bh = blk / T, j = blk - bh * T;
  const int n = min(BLK, N - j * BLK);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const size_t base = ((size_t)bh * N + (size_t)j * BLK) * D;

  // stage V and K rows (zeros past the valid rows)
  for (int x = tid; x < 64 * (D / 4); x += 256) {
    const int r = x / (D / 4), c = (x - r * (D / 4)) * 4;
    uint2 v = make_uint2(0u, 0u), k = make_uint2(0u, 0u);
    if (r < n) {
      v = *(const uint2 *)(V + base + (size_t)r * D + c);
      if (LIN) k = *(const uint2 *)(K + base + (size_t)r * D + c);
    }
    uint32_t *dv = (uint32_t *)(sv + r * P + c);  // 4-byte aligned: P even, c even
    dv[0] = v.x;
    dv[1] = v.y;
    if (LIN) {
      uint32_t *dk = (uint32_t *)(sk + r * P + c);
      dk[0] = k.x;
      dk[1] = k.y;
    }
  }
  __syncthreads();

  // phi(K) rows in float32, one lane per row, rounded to bf16 in place;
  // padding rows become 0.
  if (LIN && w == 0) {
    const int r = lane;
    uint16_t *row = sk + r * P;
    if (r < n) {
      float mx = -INFINITY;
      for (int c = 0; c < D; ++c) mx = fmaxf(mx, bf2f(row[c]));
      float s = 0.f;
      for (int c = 0; c < D; ++c) s += __expf(bf2f(row[c]) - mx);
      const float inv = 1.0f / s;
      for (int c = 0; c < D; ++c) row[c] = f2bf(__expf(bf2f(row[c]) - mx) * inv);
    } else {
      for (int c = 0; c < D; ++c) row[c] = 0;
    }
  }
  __syncthreads();

  // V in kmaj order: fragment (kc2, cg), lane holds channel 16cg + lane%16 and
  // the 8 keys 32kc2 + 16(e/4) + 4(lane/16) + e%4.
  const int g = lane >> 4, l16 = lane & 15;
  uint16_t *vdst = vt + (size_t)blk * BLK * D;
  for (int f = w; f < 2 * CG; f += 4) {
    const int kc2 = f / CG, cg = f - kc2 * CG;
    const int c = 16 * cg + l16;
    uint32_t pk[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int e0 = 2 * h, e1 = 2 * h + 1;
      const int s0 = 32 * kc2 + 16 * (e0 >> 2) + 4 * g + (e0 & 3);
      const int s1 = 32 * kc2 + 16 * (e1 >> 2) + 4 * g + (e1 & 3);
      pk[h] = (uint32_t)sv[s0 * P + c] | ((uint32_t)sv[s1 * P + c] << 16);
    }
    *(uint4 *)(vdst + ((size_t)f * 64 + lane) * 8) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
  if (!LIN) return;

  // Hb^T[c2][c] = sum_s V[s][c2] phi(K)[s][c]: A = V^T fragments (as above),
  // B = phi(K) fragments with the same key order.  Wave w owns rows
  // c2 in [D/4 * w, D/4 * (w+1)).
  constexpr int MT = CG / 4;  // row tiles per wave
  v4f acc[MT][CG];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < CG; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc2 = 0; kc2 < 2; ++kc2) {
    v4u af[MT], bf[CG];
#pragma unroll
    for (int a = 0; a < MT; ++a) {
      const int c = 16 * (w * MT + a) + l16;
      uint32_t pk[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int e0 = 2 * h, e1 = 2 * h + 1;
        const int s0 = 32 * kc2 + 16 * (e0 >> 2) + 4 * g + (e0 & 3);
        const int s1 = 32 * kc2 + 16 * (e1 >> 2) + 4 * g + (e1 & 3);
        pk[h] = (uint32_t)sv[s0 * P + c] | ((uint32_t)sv[s1 * P + c] << 16);
      }
      af[a] = v4u{pk[0], pk[1], pk[2], pk[3]};
    }
#pragma unroll
    for (int b = 0; b < CG; ++b) {
      const int c = 16 * b + l16;
      uint32_t pk[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int e0 = 2 * h, e1 = 2 * h + 1;
        const int s0 = 32 * kc2 + 16 * (e0 >> 2) + 4 * g + (e0 & 3);
        const int s1 = 32 * kc2 + 16 * (e1 >> 2) + 4 * g + (e1 & 3);
        pk[h] = (uint32_t)sk[s0 * P + c] | ((uint32_t)sk[s1 * P + c] << 16);
      }
      bf[b] = v4u{pk[0], pk[1], pk[2], pk[3]};
    }
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
      for (int b = 0; b < CG; ++b) acc[a][b] = mfma_bf16(af[a], bf[b], acc[a][b]);
  }
  // z[c] = sum over rows of the bf16 phi values (same values the product used)
  float zc = 0.f;
  if (tid < D)
    for (int r = 0; r < BLK; ++r) zc += bf2f(sk[r * P + tid]);
  __syncthreads();  // done reading sv/sk: reuse as the output stage
  uint16_t *so = smem;  // F bf16 values (F <= 2*64*P)
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < CG; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c2 = 16 * (w * MT + a) + 4 * g + r;  // accumulator row
        const int c = 16 * b + l16;                    // accumulator column
        so[hstate_off(c, c2, KC32)] = f2bf(acc[a][b][r]);
      }
  if (tid < D) so[D * D + tid] = f2bf(zc);
  for (int x = D * D + D + tid; x < F; x += 256) so[x] = 0;
  __syncthreads();
  uint4 *dst = (uint4 *)(hb + (size_t)blk * F);
  const uint4 *src = (const uint4 *)so;
  for (int x = tid; x < F / 8; x += 256) dst[x] = src[x];
}

// Projection W [d_out][d_in] into wfrag_off order (A operand, k = d_in).
__global__ void k_w_swizzle(const uint16_t *__restrict__ W, int D, uint16_t *__restrict__ wsw) {
  const int KC32 = D / 32;
  for (int x = threadIdx.x; x < D * D; x += blockDim.x) {
    const int row = x / D, k = x - row * D;
    wsw[wfrag_off(row, k, KC32)] = W[x];
  }
}

// Byte b -> 8 bf16 (bit e of b -> 1.0 or 0.0 at element e), as 4 dwords.
__device__ __forceinline__ v4u expand_bits(uint32_t b) {
  v4u r;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    uint32_t lo = ((b >> (2 * h)) & 1u) ? 0x3F80u : 0u;
    uint32_t hi = ((b >> (2 * h + 1)) & 1u) ? 0x3F800000u : 0u;
    r[h] = lo | hi;
  }
  return r;
}

// H[i][f] = sum_j (1 - M[i][j]) Hb[j][f] for one head; 128 x 128 output tile
// per workgroup, 4 waves in 2 x 2, 32 key blocks per step.  B rows are staged
// through LDS transposed ([f][j]) so each lane reads its 8 consecutive j with
// one 16-byte load.
template <int D>
__global__ __launch_bounds__(256) void k_marginal(const uint64_t *__restrict__ mask,
                                                  const uint16_t *__restrict__ hb, int T, int W64,
                                                  int F, uint16_t *__restrict__ hi) {
  constexpr int TM = 128, TN = 128, TK = 32;
  constexpr int PB = TK + 8;  // bf16 pitch of the transposed B tile (16-byte aligned rows)
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][TN * PB];
  const int mtiles = (T + TM - 1) / TM, ntiles = F / TN;
  int b = blockIdx.x;
  const int nt0 = b % ntiles;
  b /= ntiles;
  const int mt0 = b % mtiles;
  const int bh = b / mtiles;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  const int i_base = mt0 * TM + wm, f_base = nt0 * TN;
  const uint16_t *hbh = hb + (size_t)bh * T * F;

  v4f acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = v4f{0.f, 0.f, 0.f, 0.f};

  // global -> register loads of one B step: 32 rows x 128 columns, two
  // 16-byte pieces per thread
  auto load_b = [&](int j0, uint4 (&r)[2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int x = tid + 256 * q;
      const int jr = x >> 4, c8 = (x & 15) * 8;
      const int j = j0 + jr;
      r[q] = make_uint4(0u, 0u, 0u, 0u);
      if (j < T) r[q] = *(const uint4 *)(hbh + (size_t)j * F + f_base + c8);
    }
  };
  auto store_b = [&](int buf, const uint4 (&r)[2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int x = tid + 256 * q;
      const int jr = x >> 4, c8 = (x & 15) * 8;
      const uint32_t v[4] = {r[q].x, r[q].y, r[q].z, r[q].w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sB[buf][(c8 + e) * PB + jr] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
  };

  const int steps = (T + TK - 1) / TK;
  uint4 rb[2];
  load_b(0, rb);
  store_b(0, rb);
  __syncthreads();
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    const int j0 = s * TK;
    if (s + 1 < steps) load_b(j0 + TK, rb);
    // A fragments from the mask: rows i, the 8 key blocks j0 + 8g .. +7
    v4u af[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int i = i_base + 16 * a + l16;
      uint32_t byte = 0u;
      if (i < T) {
        const int jj = j0 + 8 * g;
        const uint64_t word = mask[((size_t)bh * T + i) * W64 + (jj >> 6)];
        uint32_t kept8 = (uint32_t)(word >> (jj & 63)) & 0xFFu;
        const int valid = min(8, max(0, T - jj));
        const uint32_t vmask = valid >= 8 ? 0xFFu : ((1u << valid) - 1u);
        byte = (~kept8) & vmask;
      }
      af[a] = expand_bits(byte);
    }
    v4u bfr[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      bfr[c] = *(const v4u *)(&sB[buf][(wn + 16 * c + l16) * PB + 8 * g]);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[a][c] = mfma_bf16(af[a], bfr[c], acc[a][c]);
    if (s + 1 < steps) store_b(buf ^ 1, rb);
    __syncthreads();
  }
  // store bf16 H rows i < T
  uint16_t *hih = hi + (size_t)bh * T * F;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i_base + 16 * a + 4 * g + r;
      if (i < T) {
#pragma unroll
        for (int c = 0; c < 4; ++c) hih[(size_t)i * F + f_base + wn + 16 * c + l16] = f2bf(acc[a][c][r]);
      }
    }
}

void launch_kv_prep(const Plan &p, const uint16_t *k, const uint16_t *v, const WsPtrs &ws,
                    hipStream_t st) {
  dim3 grid(p.BH * p.T), block(256);
  if (p.d == 128) {
    if (p.lin_on)
      hipLaunchKernelGGL((k_kv_prep<128, true>), grid, block, 0, st, k, v, p.N, p.T, p.F, ws.vt, ws.hb);
    else
      hipLaunchKernelGGL((k_kv_prep<128, false>), grid, block, 0, st, k, v, p.N, p.T, p.F, ws.vt, ws.hb);
  } else {
    if (p.lin_on)
      hipLaunchKernelGGL((k_kv_prep<64, true>), grid, block, 0, st, k, v, p.N, p.T, p.F, ws.vt, ws.hb);
    else
      hipLaunchKernelGGL((k_kv_prep<64, false>), grid, block, 0, st, k, v, p.N, p.T, p.F, ws.vt, ws.hb);
  }
}

void launch_w_swizzle(const Plan &p, const uint16_t *w, const WsPtrs &ws, hipStream_t st) {
  hipLaunchKernelGGL(k_w_swizzle, dim3(1), dim3(256), 0, st, w, p.d, ws.wsw);
}

void launch_marginal(const Plan &p, const WsPtrs &ws, hipStream_t st) {
  const int mtiles = (p.T + 127) / 128, ntiles = p.F / 128;
  dim3 grid(p.BH * mtiles * ntiles), block(256);
  if (p.d == 128)
    hipLaunchKernelGGL(k_marginal<128>, grid, block, 0, st, ws.mask, ws.hb, p.T, p.W64, p.F, ws.hi);
  else
    hipLaunchKernelGGL(k_marginal<64>, grid, block, 0, st, ws.mask, ws.hb, p.T, p.W64, p.F, ws.hi);
}

}  // namespace sla
