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

// H[i][f] = sum_j (1 - M[i][j]) Hb[j][f]: per head a [T x T] by [T x F] GEMM,
// 32x32x16 bf16 MFMA with float32 accumulation, written back as bf16.
// A workgroup (4 waves, 2 x 2) owns a 256 x 256 output tile; each wave a
// 128 x 128 sub-tile held in 16 accumulator tiles.  Per step of 32 key blocks
// both operand tiles are built in LDS in MFMA fragment order (1 KiB per
// fragment, 16 bytes per lane): A from the rows' mask words (the complement
// bits become bf16 ones and zeros by integer arithmetic), B from Hb rows
// transposed to key pairs per column.  Two LDS buffers: step s+1 is built
// while step s is multiplied.  The row tiles of one column tile run one after
// another on one XCD, so each Hb column slice comes from HBM once.
constexpr int MG_BM = 256;  // rows per workgroup
constexpr int MG_BN = 256;  // columns per workgroup
constexpr int MG_BK = 32;   // key blocks per step

template <int D>
__global__ __launch_bounds__(256, 1) void k_marginal(const uint64_t *__restrict__ maskt,
                                                     const uint16_t *__restrict__ hb, int T,
                                                     int W64, int F, uint16_t *__restrict__ hi) {
  // two operand buffers of 32 KiB (A fragments, then B fragments); the
  // epilogue reuses all 128 KiB to stage each wave's bf16 tile
  __shared__ __attribute__((aligned(16))) uint4 smem[8192];
  const int RT = (T + MG_BM - 1) / MG_BM, CT = (F + MG_BN - 1) / MG_BN;
  int b = xcd_remap(blockIdx.x, gridDim.x);
  const int rt = b % RT;
  b /= RT;
  const int ct = b % CT;
  const int bh = b / CT;
  const int row0 = rt * MG_BM, col0 = ct * MG_BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = w >> 1, wc = w & 1;
  const uint16_t *hbh = hb + (size_t)bh * T * F;
  const uint64_t *mh = maskt + (size_t)bh * W64 * T;  // word-major: [W64][T]

  // A: thread tid builds row row0 + tid (32 keys = 4 chunks of 8) from its
  // mask word, which is loaded two steps ahead
  const int arow = row0 + tid;
  // rows past T read row T-1 (their outputs are never stored)
  const int arow_c = min(arow, T - 1);
  auto load_word = [&](int s) -> uint64_t {
    const int word = min((s * MG_BK) >> 6, W64 - 1);
    return mh[(size_t)word * T + arow_c];
  };
  auto gen_a = [&](int s, uint64_t wd, uint4 *buf) {
    const int j0 = s * MG_BK;
    uint32_t nb = ~(uint32_t)(wd >> (j0 & 32));
    const int nvalid = T - j0;  // key blocks past T contribute nothing
    if (nvalid < 32) nb &= nvalid > 0 ? (1u << nvalid) - 1u : 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // the 8 bits of keys 8c .. 8c+7: even keys to bits 0,2,4,6, odd keys to
      // bits 16,18,20,22; then bit pair h times (1.0bf16 >> 2h) is the dword
      // holding keys 2h (low half) and 2h+1 (high half)
      const uint32_t by = (nb >> (8 * c)) & 0xFFu;
      const uint32_t y = (by & 0x55u) | (((by >> 1) & 0x55u) << 16);
      uint4 v;
      v.x = __umul24(y & 0x00010001u, 0x3F80u);
      v.y = __umul24(y & 0x00040004u, 0x3F80u >> 2);
      v.z = __umul24(y & 0x00100010u, 0x3F80u >> 4);
      v.w = __umul24(y & 0x00400040u, 0x3F80u >> 6);
      // fragment (row tile tid/32, k-substep c/2), lane (row%32) + 32 (c%2)
      buf[((tid >> 5) * 2 + (c >> 1)) * 64 + (tid & 31) + 32 * (c & 1)] = v;
    }
  };
  // B: thread tid stages keys 2p, 2p+1 (p = tid/16) x columns 16q .. 16q+15
  // (q = tid%16) of the tile
  const int bp = tid >> 4, bq = tid & 15;
  // key blocks past T read row T-1 (their A entries are 0) and columns past F
  // read the last 8 columns (their outputs are never stored): no branches
  const int bcol0 = min(col0 + 16 * bq, F - 16);
  auto load_b = [&](int s, uint4 (&v)[2][2]) {
    const int j0 = s * MG_BK;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = min(j0 + 2 * bp + e, T - 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) v[e][h] = *(const uint4 *)(hbh + (size_t)j * F + bcol0 + 8 * h);
    }
  };
  // B fragment layout in LDS: column cl (tile-relative) and key pair p go to
  // fragment (cl/32, p/8), 16-byte slot ((cl%32) + 32 ((p/4)%2)) ^ ((cl/16)%8),
  // dword p%4.  The XOR spreads one transposing store over all banks (lanes
  // differ in cl/16 and p%4) and keeps each 8-lane group of a fragment read on
  // distinct slots.  Thread (p, q) writes columns 16q + j, j < 16.
  const int xw = bq & 7;
  const int bbase = (((bq >> 1) * 2 + (bp >> 3)) * 64 + 16 * (bq & 1) + 32 * ((bp >> 2) & 1)) * 4 + (bp & 3);
  int boff[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) boff[jj] = bbase + 4 * (jj ^ xw);
  auto store_b = [&](const uint4 (&v)[2][2], uint4 *buf) {
    uint32_t *bw = (uint32_t *)(buf + 1024);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t d0[4] = {v[0][h].x, v[0][h].y, v[0][h].z, v[0][h].w};
      const uint32_t d1[4] = {v[1][h].x, v[1][h].y, v[1][h].z, v[1][h].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        // column 2m: both keys' low halves; column 2m+1: both high halves
        bw[boff[2 * m] + 32 * h] = __builtin_amdgcn_perm(d1[m], d0[m], 0x05040100u);
        bw[boff[2 * m + 1] + 32 * h] = __builtin_amdgcn_perm(d1[m], d0[m], 0x07060302u);
      }
    }
  };

  v16f acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;

  // Step s multiplies buffer s&1 and builds step s+1 into the other buffer
  // from registers loaded during step s-1; its own loads are for step s+2.
  // The loop runs two steps per iteration so the two register sets keep
  // fixed names (a copy would wait for the loads in flight).
  // an even number of steps (a step past T has an all-zero A)
  const int steps = (((T + MG_BK - 1) / MG_BK) + 1) & ~1;
  uint4 bvA[2][2], bvB[2][2];
  uint64_t wdA, wdB;
  {
    uint4 b0[2][2];
    load_b(0, b0);
    const uint64_t w0 = load_word(0);
    load_b(1, bvA);
    wdA = load_word(1);
    gen_a(0, w0, smem);
    store_b(b0, smem);
  }
  __syncthreads();
  auto mma_step = [&](const uint4 *cur) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4u af[4], bf[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) af[x] = __builtin_bit_cast(v4u, cur[((4 * wr + x) * 2 + ks) * 64 + lane]);
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int ctile = 4 * wc + y;
        const int slot = lane ^ ((2 * ctile + ((lane & 31) >> 4)) & 7);
        bf[y] = __builtin_bit_cast(v4u, cur[1024 + (ctile * 2 + ks) * 64 + slot]);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = mfma32_bf16(af[x], bf[y], acc[x][y]);
    }
  };
  for (int s = 0; s < steps; s += 2) {
    // even step s: buffer 0; builds s+1 (bvA, wdA) into buffer 1; loads s+2
    load_b(s + 2, bvB);
    wdB = load_word(s + 2);
    mma_step(smem);
    gen_a(s + 1, wdA, smem + 2048);
    store_b(bvA, smem + 2048);
    __syncthreads();
    // odd step s+1: buffer 1; builds s+2 (bvB, wdB) into buffer 0; loads s+3
    load_b(s + 3, bvA);
    wdA = load_word(s + 3);
    mma_step(smem + 2048);
    gen_a(s + 2, wdB, smem);
    store_b(bvB, smem);
    __syncthreads();
  }

  // epilogue: each wave stages its 128 x 128 tile as bf16 rows (256 B pitch),
  // then writes 16-byte pieces of rows < T, columns < F
  uint16_t *st = (uint16_t *)(smem + w * 2048);
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = 32 * x + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int cc = 32 * y + (lane & 31);
        st[rr * 128 + cc] = f2bf(acc[x][y][r]);
      }
      // one accumulator tile at a time (keeps the register demand small)
      __builtin_amdgcn_sched_barrier(0);
    }
  __syncthreads();
  const int orow0 = row0 + 128 * wr, ocol0 = col0 + 128 * wc;
  uint16_t *hih = hi + (size_t)bh * T * F;
#pragma unroll 4
  for (int it = 0; it < 32; ++it) {
    const int piece = it * 64 + lane;  // 16 pieces of 8 columns per row
    const int rr = piece >> 4, c8 = (piece & 15) * 8;
    const int row = orow0 + rr, col = ocol0 + c8;
    if (row < T && col < F)
      *(uint4 *)(hih + (size_t)row * F + col) = *(const uint4 *)(st + rr * 128 + c8);
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
  const int RT = (p.T + MG_BM - 1) / MG_BM, CT = (p.F + MG_BN - 1) / MG_BN;
  dim3 grid(p.BH * CT * RT), block(256);
  if (p.d == 128)
    hipLaunchKernelGGL(k_marginal<128>, grid, block, 0, st, ws.maskt, ws.hb, p.T, p.W64, p.F, ws.hi);
  else
    hipLaunchKernelGGL(k_marginal<64>, grid, block, 0, st, ws.maskt, ws.hb, p.T, p.W64, p.F, ws.hi);
}

}  // namespace sla
