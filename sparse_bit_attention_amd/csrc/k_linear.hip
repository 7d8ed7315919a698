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

// H[i][f] = sum_j (1 - M[i][j]) Hb[j][f] for one head and a 32-column slice
// of f, all query-block rows i at once (so each Hb element is read once per
// head).  8 waves; wave w owns row tiles [MW*w, MW*w + MW) (16 rows each).
// Per step of 64 key blocks j: the B slice (64 x 32 bf16) is staged in LDS
// transposed to [f][j] so a lane's 8 consecutive j are one 16-byte read; the A
// fragments come from the row's mask word through a 16-entry LDS table that
// expands 4 complemented mask bits to 4 bf16 ones/zeros (8 bytes per entry:
// the 16 entries sit in distinct banks, so lookups never conflict).
constexpr int MARG_TN = 32;   // columns per workgroup
constexpr int MARG_TK = 64;   // key blocks per step (one mask word)
constexpr int MARG_MW = 10;   // row tiles per wave: 8 * 10 * 16 = 1280 rows per pass

template <int D>
__global__ __launch_bounds__(512) void k_marginal(const uint64_t *__restrict__ maskt,
                                                  const uint16_t *__restrict__ hb, int T, int W64,
                                                  int F, uint16_t *__restrict__ hi) {
  constexpr int PB = MARG_TK + 8;  // bf16 pitch of the transposed B slice (16-byte rows)
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][MARG_TN * PB];
  __shared__ __attribute__((aligned(16))) uint2 lut[16];
  const int nslices = F / MARG_TN;
  const int mpasses = (T + 8 * MARG_MW * 16 - 1) / (8 * MARG_MW * 16);
  // consecutive column slices of a head share 128-byte Hb lines: keep them
  // on one XCD
  int b = xcd_remap(blockIdx.x, gridDim.x);
  const int ns = b % nslices;
  b /= nslices;
  const int mp = b % mpasses;
  const int bh = b / mpasses;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int f_base = ns * MARG_TN;
  const int row0 = mp * (8 * MARG_MW * 16) + w * (MARG_MW * 16);
  const uint16_t *hbh = hb + (size_t)bh * T * F + f_base;
  const uint64_t *mh = maskt + (size_t)bh * W64 * T;  // word-major: [W64][T]

  if (tid < 16) {
    uint32_t v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      v[h] = (((tid >> (2 * h)) & 1) ? 0x3F80u : 0u) | (((tid >> (2 * h + 1)) & 1) ? 0x3F800000u : 0u);
    lut[tid] = make_uint2(v[0], v[1]);
  }

  v4f acc[MARG_MW][2];
#pragma unroll
  for (int a = 0; a < MARG_MW; ++a) {
    acc[a][0] = v4f{0.f, 0.f, 0.f, 0.f};
    acc[a][1] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  // one B step: 64 rows j x 32 columns; thread t loads 4 columns of row t/8
  const int bj = tid >> 3, bf4 = (tid & 7) * 4;
  auto load_b = [&](int j0) -> uint2 {
    const int j = j0 + bj;
    uint2 v = make_uint2(0u, 0u);
    if (j < T) v = *(const uint2 *)(hbh + (size_t)j * F + bf4);
    return v;
  };
  auto store_b = [&](int buf, uint2 v) {
    uint16_t *d = &sB[buf][bf4 * PB + bj];
    d[0] = (uint16_t)(v.x & 0xFFFF);
    d[PB] = (uint16_t)(v.x >> 16);
    d[2 * PB] = (uint16_t)(v.y & 0xFFFF);
    d[3 * PB] = (uint16_t)(v.y >> 16);
  };

  // mask words of this lane's rows, fetched one step ahead
  auto load_words = [&](int st, uint64_t (&wd)[MARG_MW]) {
#pragma unroll
    for (int a = 0; a < MARG_MW; ++a) {
      const int i = row0 + 16 * a + l16;
      wd[a] = mh[(size_t)st * T + min(i, T - 1)];
    }
  };
  // rows past T read a valid row and are then forced to "all kept" (A = 0)
  uint64_t rowpad[MARG_MW];
#pragma unroll
  for (int a = 0; a < MARG_MW; ++a) rowpad[a] = (row0 + 16 * a + l16) < T ? 0ull : ~0ull;
  const int steps = (T + MARG_TK - 1) / MARG_TK;
  uint64_t wnext[MARG_MW];
  load_words(0, wnext);
  uint2 rb = load_b(0);
  store_b(0, rb);
  __syncthreads();
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    const int j0 = s * MARG_TK;
    uint64_t wcur[MARG_MW];
#pragma unroll
    for (int a = 0; a < MARG_MW; ++a) wcur[a] = wnext[a];
    if (s + 1 < steps) {
      rb = load_b(j0 + MARG_TK);
      load_words(s + 1, wnext);
    }
    // key blocks j0 + 32kc + 8g + e past T must give A = 0: set their mask
    // bits (kept) before complementing; only the last step is short
    uint32_t pad[2] = {0u, 0u};
    if (j0 + MARG_TK > T) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int n = T - (j0 + 32 * kc);
        pad[kc] = n >= 32 ? 0u : (n <= 0 ? ~0u : (~0u << n));
      }
    }
    v4u bfr[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
        bfr[nt][kc] = *(const v4u *)(&sB[buf][(16 * nt + l16) * PB + 32 * kc + 8 * g]);
    // all A fragments of the step first (one LDS wait), then the products
    v4u af[MARG_MW][2];
#pragma unroll
    for (int a = 0; a < MARG_MW; ++a)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const uint32_t half = (uint32_t)((wcur[a] | rowpad[a]) >> (32 * kc)) | pad[kc];
        const uint32_t nb = ~half;
        const uint2 lo = lut[__builtin_amdgcn_ubfe(nb, 8 * g, 4)];
        const uint2 hi4 = lut[__builtin_amdgcn_ubfe(nb, 8 * g + 4, 4)];
        af[a][kc] = v4u{lo.x, lo.y, hi4.x, hi4.y};
      }
#pragma unroll
    for (int a = 0; a < MARG_MW; ++a)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        acc[a][0] = mfma_bf16(af[a][kc], bfr[0][kc], acc[a][0]);
        acc[a][1] = mfma_bf16(af[a][kc], bfr[1][kc], acc[a][1]);
      }
    // issue order: index math, every LDS read, then the products
    __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * MARG_MW + 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * MARG_MW, 0);
    if (s + 1 < steps) store_b(buf ^ 1, rb);
    __syncthreads();
  }
  // store bf16 rows i < T: lane holds column 16nt + l16, rows 4g + r of each tile
  uint16_t *hih = hi + (size_t)bh * T * F + f_base;
#pragma unroll
  for (int a = 0; a < MARG_MW; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = row0 + 16 * a + 4 * g + r;
      if (i < T) {
        hih[(size_t)i * F + l16] = f2bf(acc[a][0][r]);
        hih[(size_t)i * F + 16 + l16] = f2bf(acc[a][1][r]);
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
  const int nslices = p.F / MARG_TN;
  const int mpasses = (p.T + 8 * MARG_MW * 16 - 1) / (8 * MARG_MW * 16);
  dim3 grid(p.BH * mpasses * nslices), block(512);
  if (p.d == 128)
    hipLaunchKernelGGL(k_marginal<128>, grid, block, 0, st, ws.maskt, ws.hb, p.T, p.W64, p.F, ws.hi);
  else
    hipLaunchKernelGGL(k_marginal<64>, grid, block, 0, st, ws.maskt, ws.hb, p.T, p.W64, p.F, ws.hi);
}

}  // namespace sla
