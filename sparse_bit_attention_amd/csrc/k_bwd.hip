// Backward pass of plain SLA (bf16 QK^T), the block mask held fixed.
//
// Pages: "揭秘TurboDiffusion…" section "支柱二：稀疏线性注意力 – SLA" and
// the aiho.net news report (量子位, 2025-12-26) section
// "2. SLA稀疏线性注意力": SLA's sparse pattern and
// linear component are trained, so the operator is differentiated.  The top-k
// selection is a discrete choice and passes no gradient.
//
// Launch order (one stream):
//  k_mask_t    transposed block mask (row j = the query blocks that keep key
//              block j), row-major and word-major, 64 x 64 bit tiles by wave
//              ballots.
//  k_bwd_qlin  one workgroup per query block, linear branch (bf16 MFMA on LDS
//              tiles): phi(Q), O_l = phi(Q) H_i / den, G = dO W, d phi(Q) and
//              its channel-softmax gradient (float32 rows), dH_i = phi(Q)^T G /
//              den and dz_i (bf16), O_l rows (bf16, for dW).
//  k_bwd_q     one workgroup per query block: D = rowsum(dO O_sparse) from
//              the sparse output the forward kept, then the sparse dQ over the
//              kept key blocks with one query per lane column (S^T = K Q^T,
//              P^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T); dQ (plus the
//              linear part) is rounded once.
//  k_marginal  (the forward's kernel) dHb = (1 - M)^T dH with the transposed mask.
//  k_bwd_kvlin one workgroup per key block: the key side of the linear branch
//              from dHb_j (float32 rows).
//  k_bwd_kv    one workgroup per key block: dV^T += dO^T P and dK^T += Q^T dS
//              over the query blocks that keep it (one key per lane column),
//              plus the linear parts; rounded once.
// The two sparse kernels fit two workgroups per CU (registers and LDS), so
// one workgroup's tile loads overlap the other's products.
//  k_bwd_dw    dW partials dO^T O_l per chunk of query blocks; k_dw_sum adds them.
//
// Precision: bf16 operands, float32 accumulation; P and dS are rounded to
// bf16 for their products (as the forward rounds P); the linear states and
// their gradients are bf16 in HBM.
#include "sla_internal.h"

namespace sla {

constexpr float BWD_LOG2E = 1.4426950408889634f;

template <int D>
struct BTile {
  static constexpr int P = D + 16;   // LDS row pitch (bf16 elements)
  static constexpr int CG = D / 16;  // 16-column tiles
  static constexpr int KC32 = D / 32;
  static constexpr int TILE = 64 * P;            // elements of a 64-row LDS tile
  static constexpr int NPT = 64 * D / 8 / 256;   // 16-byte pieces per thread and 64-row tile
};

// Gradient of a block's linear state, (c, c2) of dH and its z part at D*D + c:
// the accumulator order of the kernel that writes it (four consecutive c per
// lane, a wave's 16 x 16 tile in 512 contiguous bytes).
__device__ __forceinline__ int dh_off(int c, int c2, int CG) {
  return (((c >> 4) * CG + (c2 >> 4)) * 64 + (c2 & 15) + 16 * ((c & 15) >> 2)) * 4 + (c & 3);
}

// 64 rows x D bf16 (row stride D) into registers; rows >= nvalid read as 0.
template <int D>
__device__ __forceinline__ void tile_load(const uint16_t *src, int nvalid,
                                          uint4 (&r)[BTile<D>::NPT], int tid) {
#pragma unroll
  for (int e = 0; e < BTile<D>::NPT; ++e) {
    const int x = tid + 256 * e;
    const int row = x / (D / 8), c8 = (x - row * (D / 8)) * 8;
    r[e] = row < nvalid ? *(const uint4 *)(src + (size_t)row * D + c8) : make_uint4(0u, 0u, 0u, 0u);
  }
}

// The same rows for the two sparse loops, whose padding rows never reach a
// product with a nonzero weight (padding queries: normaliser +inf, so P = 0;
// padding keys: dS = 0): rows >= nvalid read row nvalid - 1 instead of 0, so
// every load is unconditional.
template <int D>
__device__ __forceinline__ void tile_load_clamped(const uint16_t *src, int nvalid,
                                                  uint4 (&r)[BTile<D>::NPT], int tid) {
#pragma unroll
  for (int e = 0; e < BTile<D>::NPT; ++e) {
    const int x = tid + 256 * e;
    const int row = x / (D / 8), c8 = (x - row * (D / 8)) * 8;
    r[e] = *(const uint4 *)(src + (size_t)min(row, nvalid - 1) * D + c8);
  }
}

template <int D>
__device__ __forceinline__ void tile_store(const uint4 (&r)[BTile<D>::NPT], uint16_t *lds, int tid) {
#pragma unroll
  for (int e = 0; e < BTile<D>::NPT; ++e) {
    const int x = tid + 256 * e;
    const int row = x / (D / 8), c8 = (x - row * (D / 8)) * 8;
    *(uint4 *)(lds + row * BTile<D>::P + c8) = r[e];
  }
}

// Tiles of the two sparse loops: 64 rows of D bf16 without padding, the
// 4-element (8-byte) units of row r XOR-swizzled by sw_unit<D>(r).  The LDS
// has 64 four-byte banks and serves an 8-byte read 32 lanes at a time, so
// each half-wave must touch 32 distinct 8-byte slots modulo 256 bytes:
//  * row reads of an MFMA operand: lanes l%16 read 16 consecutive rows at
//    unit u + l/16; with D = 128 the XOR is even and takes 16 distinct
//    values over any 16 consecutive rows, so the two unit parities of a
//    half-wave fill all 32 slots;
//  * transposing reads: a half-wave reads rows 8m .. 8m+7 at units
//    4x .. 4x+3; bits 2-4 of the XOR are row % 8, distinct over those rows.
// Even XOR values keep a row's unit pairs (2m, 2m+1) adjacent, so a thread
// stores its 16 bytes with one instruction.  With D = 64 (16 units, a row
// of 128 bytes) the XOR has four bits and separates 16 consecutive rows.
template <int D>
__device__ __forceinline__ int sw_unit(int r) {
  if constexpr (D == 128) return ((r & 7) << 2) | ((r >> 2) & 2);
  return ((r & 3) << 2) | ((r >> 2) & 3);
}

// element offset of (r, c) for c % 4 == 0
template <int D>
__device__ __forceinline__ int sw_off(int r, int c) {
  return r * D + ((((c >> 2) ^ sw_unit<D>(r))) << 2);
}

template <int D>
__device__ __forceinline__ void tile_store_sw(const uint4 (&r)[BTile<D>::NPT], uint16_t *lds,
                                              int tid) {
#pragma unroll
  for (int e = 0; e < BTile<D>::NPT; ++e) {
    const int x = tid + 256 * e;
    const int row = x / (D / 8), c8 = (x - row * (D / 8)) * 8;
    if constexpr (D == 128) {
      *(uint4 *)(lds + sw_off<D>(row, c8)) = make_uint4(r[e].x, r[e].y, r[e].z, r[e].w);
    } else {
      *(uint2 *)(lds + sw_off<D>(row, c8)) = make_uint2(r[e].x, r[e].y);
      *(uint2 *)(lds + sw_off<D>(row, c8 + 4)) = make_uint2(r[e].z, r[e].w);
    }
  }
}

// Swizzled 64-row tile (D = 128) straight from global memory into LDS by the
// load-to-LDS path: an instruction writes lane l's 16 bytes at byte 16 l of
// a 1 KiB piece (four rows).  sw_unit is even at D = 128, so a 16-byte
// source piece stays whole under the swizzle, and lane l fetches the piece
// that tile_store_sw would put at its place.  Rows past nvalid read row
// nvalid - 1.  Wave w fills rows 16 w .. 16 w + 15 (four instructions).
__device__ __forceinline__ void bwd_dma16(const void *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory");
}
__device__ __forceinline__ void bwd_dma4(const void *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds)
               : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}
__device__ __forceinline__ void tile_dma_sw128(const uint16_t *src, int nvalid, uint16_t *lds,
                                               int tid) {
  const int w = tid >> 6, lane = tid & 63;
  const uint32_t base = lds_addr(lds);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 16 * w + 4 * e + (lane >> 4), p = lane & 15;
    const int k = p ^ (sw_unit<128>(r) >> 1);
    bwd_dma16(src + (size_t)min(r, nvalid - 1) * 128 + 8 * k,
              __builtin_amdgcn_readfirstlane(base + (uint32_t)((16 * w + 4 * e) * 256)));
  }
}

// lds_rows on a swizzled tile.  The two 8-byte reads are volatile so that
// each lands in its own half of the operand: left to itself the compiler
// pairs halves of neighbouring fragments into one ds_read2st64_b64 and then
// spends a register move per dword putting them back together.
template <int D>
__device__ __forceinline__ v4u sw_rows(const uint16_t *tile, int r0, int kc, int lane) {
  typedef uint32_t u2v __attribute__((ext_vector_type(2)));
  typedef const volatile __attribute__((address_space(3))) u2v lds_u2v;
  const int r = r0 + (lane & 15), k0 = 32 * kc + 4 * (lane >> 4);
  const u2v lo = *(lds_u2v *)(tile + sw_off<D>(r, k0));
  const u2v hi = *(lds_u2v *)(tile + sw_off<D>(r, k0 + 16));
  return v4u{lo.x, lo.y, hi.x, hi.y};
}

// lds_frag on a swizzled tile: rows 32 kc2 + 4g + 0..3 and 32 kc2 + 16 + 4g
// + 0..3 of column n0 + l%16, through the transposing read
template <int D>
__device__ __forceinline__ v4u sw_frag(const uint16_t *tile, int kc2, int n0, int lane) {
  const int j = lane & 15, g = lane >> 4;
  const int rlo = 32 * kc2 + 4 * g + (j >> 2), c = n0 + 4 * (j & 3);
  typedef __attribute__((address_space(3))) v4s16 lds_v4s16;
  const v4s16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16 *)(tile + sw_off<D>(rlo, c)));
  const v4s16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16 *)(tile + sw_off<D>(rlo + 16, c)));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return v4u{a.x, a.y, b.x, b.y};
}

// phi of 64 rows (softmax over the D channels, rounded to bf16) into an LDS
// tile, four threads per row; rows >= nvalid become 0.  Returns this
// thread's partial dot of its phi values with zg (global bf16 [D]) when
// zg is given.
template <int D>
__device__ __forceinline__ float phi_rows(const uint16_t *src, int nvalid, uint16_t *lds,
                                          const uint16_t *zg, int tid) {
  constexpr int CPT = D / 4;
  const int r = tid >> 2, part = tid & 3;
  const bool ok = r < nvalid;
  float x[CPT];
#pragma unroll
  for (int c = 0; c < CPT; c += 8) {
    const uint4 v = ok ? *(const uint4 *)(src + (size_t)r * D + part * CPT + c) : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[c + e] = bf2f((uint16_t)(vv[e >> 1] >> (16 * (e & 1))));
  }
  float mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < CPT; ++c) mx = fmaxf(mx, x[c]);
  mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
  float sm = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    x[c] = __builtin_amdgcn_exp2f((x[c] - mx) * BWD_LOG2E);
    sm += x[c];
  }
  sm += __shfl_xor(sm, 1, 64);
  sm += __shfl_xor(sm, 2, 64);
  const float inv = ok ? 1.0f / sm : 0.0f;
  float dd = 0.f;
  uint16_t *row = lds + r * BTile<D>::P + part * CPT;
#pragma unroll
  for (int c = 0; c < CPT; c += 2) {
    const uint32_t pk = pack2bf(x[c] * inv, x[c + 1] * inv);
    *(uint32_t *)(row + c) = pk;
    if (zg) {
      dd = __builtin_fmaf(bf2f((uint16_t)(pk & 0xFFFF)), bf2f(zg[part * CPT + c]), dd);
      dd = __builtin_fmaf(bf2f((uint16_t)(pk >> 16)), bf2f(zg[part * CPT + c + 1]), dd);
    }
  }
  return dd;
}

// ---------------------------------------------------------------------------
// Transposed mask: wave (bh, c, w) turns the 64 x 64 bit tile of query blocks
// 64c .. and key blocks 64w .. around with 64 ballots.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_mask_t(const uint64_t *__restrict__ mask, int BH, int T,
                                                int W64, uint64_t *__restrict__ mt,
                                                uint64_t *__restrict__ mtt) {
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int per = W64 * W64;
  if (wv >= BH * per) return;  // whole waves; no barriers in this kernel
  const int bh = wv / per, rem = wv - bh * per, c = rem / W64, w = rem - c * W64;
  const int i = 64 * c + lane;
  const uint64_t word = i < T ? mask[((size_t)bh * T + i) * W64 + w] : 0ull;
  uint64_t mine = 0;
  for (int b = 0; b < 64; ++b) {
    const uint64_t bal = __ballot((int)((word >> b) & 1ull));
    if (lane == b) mine = bal;
  }
  const int j = 64 * w + lane;
  if (j < T) {
    mt[((size_t)bh * T + j) * W64 + c] = mine;
    if (mtt) mtt[((size_t)bh * W64 + c) * T + j] = mine;
  }
}

// ---------------------------------------------------------------------------
// dQ (and the linear branch's per-query-block gradients)
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Linear branch, query side: one workgroup per query block
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_bwd_qlin(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ W, const uint16_t *__restrict__ dO,
    const uint16_t *__restrict__ hi, int N, int T, int F, uint16_t *__restrict__ ol,
    uint16_t *__restrict__ dhi, float *__restrict__ dql_out) {
  using G = BTile<D>;
  constexpr int P = G::P, CG = G::CG, KC32 = G::KC32, TILE = G::TILE, NPT = G::NPT;
  // phi(Q), dO, O_l, dnum tiles; W and H^T tiles
  __shared__ __attribute__((aligned(16))) uint16_t ra[4 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t rb[2 * D * P];
  __shared__ float sden[64], sdden[64], sz[D];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int qb = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = qb / T, i = qb - bh * T;
  const int ni = min(BLK, N - i * BLK);
  const size_t rowbase = (size_t)bh * N + (size_t)i * BLK;
  const uint16_t *Qb = Q + rowbase * D, *dOb = dO + rowbase * D;
  {
    uint16_t *sa = ra, *sdo = ra + TILE, *sol = ra + 2 * TILE, *sdn = ra + 3 * TILE;
    uint16_t *sw = rb, *sht = rb + D * P;
    const uint16_t *hp = hi + (size_t)qb * F;
    {
      uint4 r[NPT];
      tile_load<D>(dOb, ni, r, tid);
      tile_store<D>(r, sdo, tid);
    }
    for (int x = tid; x < D * D / 8; x += 256) {  // W [o][i]
      const int row = x / (D / 8), c8 = (x - row * (D / 8)) * 8;
      *(uint4 *)(sw + row * P + c8) = *(const uint4 *)(W + (size_t)row * D + c8);
    }
    // H_i in hstate_off order: piece x holds channels c .. c+7 of value
    // column c2; stored as the transposed tile H^T [c2][c]
    for (int x = tid; x < D * D / 8; x += 256) {
      const int fr = x >> 6, ln = x & 63;
      const int xt = fr / KC32, kc = fr - xt * KC32;
      const int c2 = 16 * xt + (ln & 15), c = 32 * kc + 8 * (ln >> 4);
      *(uint4 *)(sht + c2 * P + c) = *(const uint4 *)(hp + (size_t)x * 8);
    }
    if (tid < D) sz[tid] = bf2f(hp[D * D + tid]);
    float dd = phi_rows<D>(Qb, ni, sa, hp + D * D, tid);
    dd += __shfl_xor(dd, 1, 64);
    dd += __shfl_xor(dd, 2, 64);
    if ((tid & 3) == 0) sden[tid >> 2] = dd;
    __syncthreads();

    // num = phi(Q) H, G = dO W: wave w owns rows 16w .. +15; accumulator
    // (x, r) is row 16w + 4g + r, column 16x + l16
    v4f an[CG], ag[CG];
#pragma unroll
    for (int x = 0; x < CG; ++x) an[x] = ag[x] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KC32; ++kc) {
      const v4u af = lds_rows(sa, P, 16 * w, kc, lane);
      const v4u df = lds_rows(sdo, P, 16 * w, kc, lane);
#pragma unroll
      for (int x = 0; x < CG; ++x) {
        an[x] = mfma_bf16(af, lds_rows(sht, P, 16 * x, kc, lane), an[x]);
        ag[x] = mfma_bf16(df, lds_frag(sw, P, kc, 16 * x, lane), ag[x]);
      }
    }
    float inv[4], gdot[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float den = sden[16 * w + 4 * g + r];
      inv[r] = den > 0.f ? 1.0f / den : 0.0f;  // padding rows: phi = 0, den = 0
      gdot[r] = 0.f;
    }
#pragma unroll
    for (int x = 0; x < CG; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        an[x][r] *= inv[r];  // O_l
        gdot[r] += ag[x][r] * an[x][r];
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) gdot[r] += __shfl_xor(gdot[r], m, 64);
      if (l16 == 0) sdden[16 * w + 4 * g + r] = -gdot[r] * inv[r];
    }
#pragma unroll
    for (int x = 0; x < CG; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * w + 4 * g + r, col = 16 * x + l16;
        sol[row * P + col] = f2bf(an[x][r]);
        sdn[row * P + col] = f2bf(ag[x][r] * inv[r]);
      }
    __syncthreads();

    // d phi(Q) = dnum H^T + dden z
    v4f ad[CG];
#pragma unroll
    for (int x = 0; x < CG; ++x) ad[x] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KC32; ++kc) {
      const v4u nf = lds_rows(sdn, P, 16 * w, kc, lane);
#pragma unroll
      for (int x = 0; x < CG; ++x) ad[x] = mfma_bf16(nf, lds_frag(sht, P, kc, 16 * x, lane), ad[x]);
    }
    float adot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < CG; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * w + 4 * g + r, col = 16 * x + l16;
        const float da = ad[x][r] + sdden[row] * sz[col];
        ad[x][r] = da;
        adot[r] += bf2f(sa[row * P + col]) * da;
      }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) adot[r] += __shfl_xor(adot[r], m, 64);
    float dql[CG][4];  // channel-softmax gradient of phi(Q)
#pragma unroll
    for (int x = 0; x < CG; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * w + 4 * g + r, col = 16 * x + l16;
        dql[x][r] = bf2f(sa[row * P + col]) * (ad[x][r] - adot[r]);
      }

    // dH_i = phi(Q)^T dnum (k = the 64 rows): wave w owns channel rows
    // 16 (CT w + ct) .. +15, all value columns
    constexpr int CT = D / 64;
    v4f ah[CT][CG];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int x = 0; x < CG; ++x) ah[ct][x] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2) {
      v4u bf[CG];
#pragma unroll
      for (int x = 0; x < CG; ++x) bf[x] = lds_frag(sdn, P, kc2, 16 * x, lane);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const v4u af = lds_frag(sa, P, kc2, 16 * (CT * w + ct), lane);
#pragma unroll
        for (int x = 0; x < CG; ++x) ah[ct][x] = mfma_bf16(af, bf[x], ah[ct][x]);
      }
    }
    uint16_t *dh = dhi + (size_t)qb * F;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int x = 0; x < CG; ++x)
        *(uint2 *)(dh + dh_off(16 * (CT * w + ct) + 4 * g, 16 * x + l16, CG)) =
            make_uint2(pack2bf(ah[ct][x][0], ah[ct][x][1]), pack2bf(ah[ct][x][2], ah[ct][x][3]));
    if (tid < D) {  // dz_i[c] = sum_r phi(Q)[r][c] dden[r]
      float s = 0.f;
      for (int r = 0; r < BLK; ++r) s = __builtin_fmaf(bf2f(sa[r * P + tid]), sdden[r], s);
      dh[D * D + tid] = f2bf(s);
    }
    for (int x = D * D + D + tid; x < F; x += 256) dh[x] = 0;
    // O_l rows for the projection gradient
    uint16_t *olb = ol + (size_t)qb * BLK * D;
    for (int x = tid; x < BLK * D / 8; x += 256) {
      const int row = x / (D / 8), c8 = (x - row * (D / 8)) * 8;
      *(uint4 *)(olb + (size_t)row * D + c8) = *(const uint4 *)(sol + row * P + c8);
    }
    float *dqb = dql_out + (size_t)qb * BLK * D;
#pragma unroll
    for (int x = 0; x < CG; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) dqb[(size_t)(16 * w + 4 * g + r) * D + 16 * x + l16] = dql[x][r];
    }
}

template <int D, bool LIN>
__global__ __launch_bounds__(256, 2) void k_bwd_q(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const uint16_t *__restrict__ Os, const uint16_t *__restrict__ dO,
    const float *__restrict__ lse, const int32_t *__restrict__ kept, const float *__restrict__ mu,
    const float *__restrict__ dql, int N, int T, int kb, float qk_scale, float sm_scale,
    float *__restrict__ delta, uint16_t *__restrict__ dq) {
  using G = BTile<D>;
  constexpr int P = G::P, CG = G::CG, KC32 = G::KC32, TILE = G::TILE, NPT = G::NPT;
  // K and V double buffers (swizzled tiles of 64 D elements)
  constexpr int ST = 64 * D;
  __shared__ __attribute__((aligned(16))) uint16_t ra[4 * ST];
  __shared__ float sdelta[64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int qb = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = qb / T, i = qb - bh * T;
  const int ni = min(BLK, N - i * BLK);
  const size_t rowbase = (size_t)bh * N + (size_t)i * BLK;
  const uint16_t *Qb = Q + rowbase * D, *dOb = dO + rowbase * D;
  const uint16_t *Osb = Os + (size_t)qb * BLK * D;  // O_sparse rows of this block

  {  // D = rowsum(dO O_sparse), four threads per row
    constexpr int CPT = D / 4;
    const int r = tid >> 2, part = tid & 3;
    float s = 0.f;
    if (r < ni) {
#pragma unroll
      for (int c = 0; c < CPT; c += 8) {
        const uint4 a = *(const uint4 *)(dOb + (size_t)r * D + part * CPT + c);
        const uint4 b = *(const uint4 *)(Osb + (size_t)r * D + part * CPT + c);
        const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          s = __builtin_fmaf(bf2f((uint16_t)(av[e >> 1] >> (16 * (e & 1)))),
                             bf2f((uint16_t)(bv[e >> 1] >> (16 * (e & 1)))), s);
      }
    }
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    if (part == 0) {
      sdelta[r] = s;
      delta[(size_t)qb * BLK + r] = s;
    }
  }

  __syncthreads();

  // sparse dQ: wave w, lane column = query 16w + l16.  Since sum_s dS_rs = 0,
  // dQ_r = sm_scale sum_s dS_rs (K_s - mu) for any mu; with mu the channel
  // mean of K, an error in D (which shifts every dS_rs by -P_rs dD) no
  // longer meets the large common part of the keys.  dQ is computed as
  // dS K - rowsum(dS) mu from the same bf16 dS values.
  const int q = 16 * w + l16;
  v4f adq[CG];
#pragma unroll
  for (int x = 0; x < CG; ++x) adq[x] = v4f{0.f, 0.f, 0.f, 0.f};
  float dsrow = 0.f;  // this lane's share of rowsum(dS) for query q
  if (kb > 0) {
    // buffer b: K at ra + 2 b ST, V at ra + (2 b + 1) ST
    v4u qf[KC32], of[KC32];
#pragma unroll
    for (int kc = 0; kc < KC32; ++kc) {
      uint2 a = make_uint2(0u, 0u), b = a, c = a, d = a;
      if (q < ni) {
        const uint16_t *qa = Qb + (size_t)q * D + 32 * kc + 4 * g;
        const uint16_t *oa = dOb + (size_t)q * D + 32 * kc + 4 * g;
        a = *(const uint2 *)qa;
        b = *(const uint2 *)(qa + 16);
        c = *(const uint2 *)oa;
        d = *(const uint2 *)(oa + 16);
      }
      qf[kc] = v4u{a.x, a.y, b.x, b.y};
      of[kc] = v4u{c.x, c.y, d.x, d.y};
    }
    float l2 = q < ni ? lse[(size_t)qb * BLK + q] : INFINITY;  // padding rows: P = 0
    const float dlt = sdelta[q];
    // Complete these loads here: left pending, the compiler's wait before
    // their first use inside the loop also waits for the tile copies the loop
    // issues for the next kept block.
#pragma unroll
    for (int kc = 0; kc < KC32; ++kc) asm volatile("" : "+v"(qf[kc]), "+v"(of[kc]));
    asm volatile("" : "+v"(l2));
    const int32_t *kl = kept + (size_t)qb * kb;
    const uint16_t *Kh = K + (size_t)bh * N * D, *Vh = V + (size_t)bh * N * D;
    // D = 128: the K and V tiles go straight into LDS buffer b by the
    // load-to-LDS path (no staging registers); D = 64 stages them in registers.
    constexpr bool DMA = D == 128;
    uint4 rk[DMA ? 1 : NPT], rv[DMA ? 1 : NPT];
    auto load_kv = [&](int j, int b) {
      const int nj = min(BLK, N - j * BLK);
      if constexpr (DMA) {
        tile_dma_sw128(Kh + (size_t)j * BLK * D, nj, ra + 2 * b * ST, tid);
        tile_dma_sw128(Vh + (size_t)j * BLK * D, nj, ra + (2 * b + 1) * ST, tid);
      } else {
        tile_load_clamped<D>(Kh + (size_t)j * BLK * D, nj, rk, tid);
        tile_load_clamped<D>(Vh + (size_t)j * BLK * D, nj, rv, tid);
      }
    };
    auto store_kv = [&](int b) {
      if constexpr (DMA) {
        // the wave's copies have landed; the barrier after this makes all
        // four waves' copies visible
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else {
        tile_store_sw<D>(rk, ra + 2 * b * ST, tid);
        tile_store_sw<D>(rv, ra + (2 * b + 1) * ST, tid);
      }
    };
    load_kv(kl[0], 0);
    store_kv(0);
    __syncthreads();
    for (int n = 0; n < kb; ++n) {
      const int cur = n & 1;
      if (n + 1 < kb) load_kv(kl[n + 1], cur ^ 1);
      const uint16_t *sk = ra + 2 * cur * ST, *sv = sk + ST;
      const int nj = min(BLK, N - kl[n] * BLK);  // padding keys get dS = 0
      v4f s[4], dp[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) s[t] = dp[t] = v4f{0.f, 0.f, 0.f, 0.f};
      // The fragments of channel chunk kc + 1 (K rows for S, V rows for dP,
      // four key tiles each) are read before chunk kc's products, so each
      // read has a whole chunk of products to land.  Raised wave priority
      // around each block of products, so the other workgroup's wave on this
      // SIMD does its vector and LDS work meanwhile.
      v4u fk[2][4], fv[2][4];
      auto frags = [&](int kc, v4u (&a)[4], v4u (&b)[4]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          a[t] = sw_rows<D>(sk, 16 * t, kc, lane);
          b[t] = sw_rows<D>(sv, 16 * t, kc, lane);
        }
      };
      frags(0, fk[0], fv[0]);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kc = 0; kc < KC32; ++kc) {
        if (kc + 1 < KC32) frags(kc + 1, fk[(kc + 1) & 1], fv[(kc + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          s[t] = mfma_bf16(fk[kc & 1][t], qf[kc], s[t]);
          dp[t] = mfma_bf16(fv[kc & 1][t], of[kc], dp[t]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      // the dQ products' first K fragments, read while dS is formed
      v4u fq[2][CG];
#pragma unroll
      for (int x = 0; x < CG; ++x) fq[0][x] = sw_frag<D>(sk, 0, 16 * x, lane);
      __builtin_amdgcn_sched_barrier(0);
      // dS^T = P^T (dP^T - D) in the key order of lds_frag (kmaj)
      v4u dsb[2];
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2) {
        uint32_t pk[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int t = 2 * kc2 + h;
          float ds[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], qk_scale, -l2));
            ds[r] = 16 * t + 4 * g + r < nj ? p * (dp[t][r] - dlt) : 0.f;
          }
          pk[2 * h] = pack2bf(ds[0], ds[1]);
          pk[2 * h + 1] = pack2bf(ds[2], ds[3]);
          dsrow += bf2f((uint16_t)(pk[2 * h] & 0xFFFF)) + bf2f((uint16_t)(pk[2 * h] >> 16)) +
                   bf2f((uint16_t)(pk[2 * h + 1] & 0xFFFF)) + bf2f((uint16_t)(pk[2 * h + 1] >> 16));
        }
        dsb[kc2] = v4u{pk[0], pk[1], pk[2], pk[3]};
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int x = 0; x < CG; ++x) fq[1][x] = sw_frag<D>(sk, 1, 16 * x, lane);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2)
#pragma unroll
        for (int x = 0; x < CG; ++x) adq[x] = mfma_bf16(fq[kc2][x], dsb[kc2], adq[x]);
      __builtin_amdgcn_s_setprio(0);
      if (n + 1 < kb) store_kv(cur ^ 1);
      __syncthreads();
    }
  }
  dsrow += __shfl_xor(dsrow, 16, 64);
  dsrow += __shfl_xor(dsrow, 32, 64);
  // dQ = sm_scale (dS K - rowsum(dS) mu) + dQ_linear: lane holds query q,
  // channels 16x + 4g .. +3
  if (q < ni) {
    uint16_t *dqr = dq + (rowbase + q) * D;
    const float *muh = mu + (size_t)bh * D;
#pragma unroll
    for (int x = 0; x < CG; ++x) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = sm_scale * __builtin_fmaf(-dsrow, muh[16 * x + 4 * g + r], adq[x][r]);
        if (LIN) v[r] += dql[((size_t)qb * BLK + q) * D + 16 * x + 4 * g + r];
      }
      *(uint2 *)(dqr + 16 * x + 4 * g) = make_uint2(pack2bf(v[0], v[1]), pack2bf(v[2], v[3]));
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV (and the key side of the linear branch)
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Linear branch, key side: one workgroup per key block.  Hb_j = phi(K_j)^T V_j,
// zb_j = phi(K_j)^T 1, so dV_lin = phi(K) dHb, d phi(K) = V dHb^T + dzb and
// dK_lin = phi(K) (d phi - rowsum(phi d phi)); float32 rows for k_bwd_kv.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_bwd_kvlin(const uint16_t *__restrict__ K,
                                                   const uint16_t *__restrict__ V,
                                                   const uint16_t *__restrict__ dhb, int N, int T,
                                                   int F, float *__restrict__ dkl,
                                                   float *__restrict__ dvl) {
  using G = BTile<D>;
  constexpr int P = G::P, CG = G::CG, KC32 = G::KC32, TILE = G::TILE, NPT = G::NPT;
  __shared__ __attribute__((aligned(16))) uint16_t ra[4 * TILE];
  __shared__ float szb[D];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int kblk = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = kblk / T, j = kblk - bh * T;
  const int nj = min(BLK, N - j * BLK);
  const size_t rowbase = (size_t)bh * N + (size_t)j * BLK;
  const int s = 16 * w + l16;  // this lane column's key
  v4f adv[CG];
#pragma unroll
  for (int x = 0; x < CG; ++x) adv[x] = v4f{0.f, 0.f, 0.f, 0.f};
  {
    // Hb_j = phi(K_j)^T V_j, zb_j = phi(K_j)^T 1: dV += phi(K) dHb,
    // d phi(K) = V dHb^T + dzb, dK += phi(K) (d phi - rowsum(phi d phi))
    uint16_t *sb = ra, *sv = ra + TILE, *sdh = ra + 2 * TILE;  // sdh: dHb^T [c2][c]
    {
      uint4 r[NPT];
      tile_load<D>(V + rowbase * D, nj, r, tid);
      tile_store<D>(r, sv, tid);
    }
    phi_rows<D>(K + rowbase * D, nj, sb, nullptr, tid);
    const uint16_t *dh = dhb + (size_t)kblk * F;
    for (int x = tid; x < D * D / 4; x += 256) {  // pieces of four consecutive c
      const int fr = x >> 6, ln = x & 63;
      const int ct = fr / CG, xt = fr - ct * CG;
      const int c2 = 16 * xt + (ln & 15), c = 16 * ct + 4 * (ln >> 4);
      *(uint2 *)(sdh + c2 * P + c) = *(const uint2 *)(dh + (size_t)x * 4);
    }
    if (tid < D) szb[tid] = bf2f(dh[D * D + tid]);
    __syncthreads();
    v4f aph[CG];
#pragma unroll
    for (int x = 0; x < CG; ++x) aph[x] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KC32; ++kc) {
      const v4u bfr = lds_rows(sb, P, 16 * w, kc, lane);  // phi(K): key column, k = c
      const v4u vfr = lds_rows(sv, P, 16 * w, kc, lane);  // V: key column, k = c2
#pragma unroll
      for (int x = 0; x < CG; ++x) {
        adv[x] = mfma_bf16(lds_rows(sdh, P, 16 * x, kc, lane), bfr, adv[x]);
        aph[x] = mfma_bf16(lds_frag(sdh, P, kc, 16 * x, lane), vfr, aph[x]);
      }
    }
    float bv[CG][4], dot = 0.f;
#pragma unroll
    for (int x = 0; x < CG; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 16 * x + 4 * g + r;
        bv[x][r] = bf2f(sb[s * P + c]);
        aph[x][r] += szb[c];
        dot += bv[x][r] * aph[x][r];
      }
    dot += __shfl_xor(dot, 16, 64);
    dot += __shfl_xor(dot, 32, 64);
    if (s < nj) {
      float *kl = dkl + ((size_t)kblk * BLK + s) * D, *vl = dvl + ((size_t)kblk * BLK + s) * D;
#pragma unroll
      for (int x = 0; x < CG; ++x) {
        *(float4 *)(kl + 16 * x + 4 * g) =
            make_float4(bv[x][0] * (aph[x][0] - dot), bv[x][1] * (aph[x][1] - dot),
                        bv[x][2] * (aph[x][2] - dot), bv[x][3] * (aph[x][3] - dot));
        *(float4 *)(vl + 16 * x + 4 * g) = make_float4(adv[x][0], adv[x][1], adv[x][2], adv[x][3]);
      }
    }
    }
}

template <int D, bool LIN>
__global__ __launch_bounds__(256, 2) void k_bwd_kv(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const uint16_t *__restrict__ dO, const float *__restrict__ lse, const float *__restrict__ delta,
    const uint64_t *__restrict__ mt, const float *__restrict__ dkl, const float *__restrict__ dvl,
    int N, int T, int W64, float qk_scale, float sm_scale, uint16_t *__restrict__ dk,
    uint16_t *__restrict__ dv) {
  using G = BTile<D>;
  constexpr int P = G::P, CG = G::CG, KC32 = G::KC32, TILE = G::TILE, NPT = G::NPT;
  // Q and dO double buffers (swizzled tiles of 64 D elements)
  constexpr int ST = 64 * D;
  __shared__ __attribute__((aligned(16))) uint16_t ra[4 * ST];
  __shared__ __attribute__((aligned(16))) float sl[2][64];
  __shared__ __attribute__((aligned(16))) float sd[2][64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int kblk = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = kblk / T, j = kblk - bh * T;
  const int nj = min(BLK, N - j * BLK);
  const size_t rowbase = (size_t)bh * N + (size_t)j * BLK;
  const int s = 16 * w + l16;  // this lane column's key
  // padding keys: P = 0 through a factor (a per-element condition on the
  // exp2 becomes divergent branches that split the loop's schedule); the
  // exp2 argument is always finite (padding keys' K rows are zero, padding
  // queries' normaliser is +inf)
  const float pkeep = s < nj ? 1.f : 0.f;

  // K and V fragments of the wave's 16 keys (B operands, k = channel)
  v4u kf[KC32], vf[KC32];
#pragma unroll
  for (int kc = 0; kc < KC32; ++kc) {
    uint2 a = make_uint2(0u, 0u), b = a, c = a, d = a;
    if (s < nj) {
      const uint16_t *ka = K + (rowbase + s) * D + 32 * kc + 4 * g;
      const uint16_t *va = V + (rowbase + s) * D + 32 * kc + 4 * g;
      a = *(const uint2 *)ka;
      b = *(const uint2 *)(ka + 16);
      c = *(const uint2 *)va;
      d = *(const uint2 *)(va + 16);
    }
    kf[kc] = v4u{a.x, a.y, b.x, b.y};
    vf[kc] = v4u{c.x, c.y, d.x, d.y};
  }
  // Complete these loads here: left pending, the compiler's wait before
  // their first use inside the loop counts against the loads the loop issues
  // for the next query block, so every iteration would wait for those too.
#pragma unroll
  for (int kc = 0; kc < KC32; ++kc) asm volatile("" : "+v"(kf[kc]), "+v"(vf[kc]));
  v4f adk[CG], adv[CG];
#pragma unroll
  for (int x = 0; x < CG; ++x) adk[x] = adv[x] = v4f{0.f, 0.f, 0.f, 0.f};

  // the query blocks that keep key block j, ascending (uniform control flow)
  const uint64_t *mrow = mt + ((size_t)bh * T + j) * W64;
  int wc = 0;
  uint64_t wd = mrow[0];
  auto next_i = [&]() -> int {
    while (wd == 0ull) {
      if (++wc >= W64) return -1;
      wd = mrow[wc];
    }
    const int b = __builtin_ctzll(wd);
    wd &= wd - 1ull;
    return 64 * wc + b;
  };
  const size_t headrow = (size_t)bh * N;
  // buffer b: Q at ra + 2 b ST, dO at ra + (2 b + 1) ST
  // D = 128: the Q and dO tiles go straight into LDS buffer b by the
  // load-to-LDS path (no staging registers); D = 64 stages them in registers.
  constexpr bool DMA = D == 128;
  uint4 rq[DMA ? 1 : NPT], ro[DMA ? 1 : NPT];
  float lsn = INFINITY, dn = 0.f;
  int nin = BLK;  // valid rows of the block being loaded
  auto load_block = [&](int i, int b) {
    const int ni = min(BLK, N - i * BLK);
    nin = ni;
    const size_t qb = (size_t)bh * T + i;
    if constexpr (DMA) {
      // wave 0 also copies the row statistics (rows past ni read row ni - 1
      // and are patched in store_block)
      if (w == 0) {
        const int r = min(lane, ni - 1);
        bwd_dma4(lse + qb * BLK + r, __builtin_amdgcn_readfirstlane(lds_addr(&sl[b][0])));
        bwd_dma4(delta + qb * BLK + r, __builtin_amdgcn_readfirstlane(lds_addr(&sd[b][0])));
      }
      tile_dma_sw128(Q + (headrow + (size_t)i * BLK) * D, ni, ra + 2 * b * ST, tid);
      tile_dma_sw128(dO + (headrow + (size_t)i * BLK) * D, ni, ra + (2 * b + 1) * ST, tid);
    } else {
      if (tid < BLK) {
        lsn = tid < ni ? lse[qb * BLK + tid] : INFINITY;  // padding rows: P = 0
        dn = tid < ni ? delta[qb * BLK + tid] : 0.f;
      }
      tile_load_clamped<D>(Q + (headrow + (size_t)i * BLK) * D, ni, rq, tid);
      tile_load_clamped<D>(dO + (headrow + (size_t)i * BLK) * D, ni, ro, tid);
    }
  };
  auto store_block = [&](int b) {
    if constexpr (DMA) {
      // the wave's copies have landed (the barrier after this makes all four
      // waves' copies visible); padding rows: P = 0
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (w == 0 && lane >= nin) {
        sl[b][lane] = INFINITY;
        sd[b][lane] = 0.f;
      }
    } else {
      tile_store_sw<D>(rq, ra + 2 * b * ST, tid);
      tile_store_sw<D>(ro, ra + (2 * b + 1) * ST, tid);
      if (tid < BLK) {
        sl[b][tid] = lsn;
        sd[b][tid] = dn;
      }
    }
  };
  int inext = next_i();
  if (inext >= 0) {
    load_block(inext, 0);
    store_block(0);
  }
  __syncthreads();
  int buf = 0;
  while (inext >= 0) {
    inext = next_i();
    if (inext >= 0) load_block(inext, buf ^ 1);
    const uint16_t *sq = ra + 2 * buf * ST, *so = sq + ST;
    // S and dP: query rows 16t + 4g + r, key column s
    v4f sa[4], dp[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) sa[t] = dp[t] = v4f{0.f, 0.f, 0.f, 0.f};
    // the Q and dO fragments of channel chunk kc + 1 are read before chunk
    // kc's products, so each read has a whole chunk of products to land
    v4u fq[2][4], fo[2][4];
    auto frags = [&](int kc, v4u (&a)[4], v4u (&b)[4]) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a[t] = sw_rows<D>(sq, 16 * t, kc, lane);
        b[t] = sw_rows<D>(so, 16 * t, kc, lane);
      }
    };
    frags(0, fq[0], fo[0]);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kc = 0; kc < KC32; ++kc) {
      if (kc + 1 < KC32) frags(kc + 1, fq[(kc + 1) & 1], fo[(kc + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        sa[t] = mfma_bf16(fq[kc & 1][t], kf[kc], sa[t]);
        dp[t] = mfma_bf16(fo[kc & 1][t], vf[kc], dp[t]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    // P and dS as B fragments in the query order of lds_frag
    v4u pb[2], dsb[2];
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2) {
      uint32_t pp[4], pd[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = 2 * kc2 + h;
        float pv[4], dv4[4];
        // query rows 16t + 4g .. +3: one 16-byte read each
        const float4 l4 = *(const float4 *)&sl[buf][16 * t + 4 * g];
        const float4 d4 = *(const float4 *)&sd[buf][16 * t + 4 * g];
        const float lr[4] = {l4.x, l4.y, l4.z, l4.w}, dr[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[t][r], qk_scale, -lr[r])) * pkeep;
          dv4[r] = pv[r] * (dp[t][r] - dr[r]);
        }
        pp[2 * h] = pack2bf(pv[0], pv[1]);
        pp[2 * h + 1] = pack2bf(pv[2], pv[3]);
        pd[2 * h] = pack2bf(dv4[0], dv4[1]);
        pd[2 * h + 1] = pack2bf(dv4[2], dv4[3]);
      }
      pb[kc2] = v4u{pp[0], pp[1], pp[2], pp[3]};
      dsb[kc2] = v4u{pd[0], pd[1], pd[2], pd[3]};
    }
    // dV^T += dO^T P, dK^T += Q^T dS: channel rows 16x + 4g + r, key column s
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2)
#pragma unroll
      for (int x = 0; x < CG; ++x) {
        adv[x] = mfma_bf16(sw_frag<D>(so, kc2, 16 * x, lane), pb[kc2], adv[x]);
        adk[x] = mfma_bf16(sw_frag<D>(sq, kc2, 16 * x, lane), dsb[kc2], adk[x]);
      }
    __builtin_amdgcn_s_setprio(0);
    if (inext >= 0) store_block(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // dK = sm_scale dK_sparse + dK_linear, dV = dV_sparse + dV_linear
  float ok4[CG][4];
#pragma unroll
  for (int x = 0; x < CG; ++x)
#pragma unroll
    for (int r = 0; r < 4; ++r) ok4[x][r] = sm_scale * adk[x][r];
  if (LIN && s < nj) {
    const float *kl = dkl + ((size_t)kblk * BLK + s) * D, *vl = dvl + ((size_t)kblk * BLK + s) * D;
#pragma unroll
    for (int x = 0; x < CG; ++x) {
      const float4 a = *(const float4 *)(kl + 16 * x + 4 * g);
      const float4 c = *(const float4 *)(vl + 16 * x + 4 * g);
      ok4[x][0] += a.x; ok4[x][1] += a.y; ok4[x][2] += a.z; ok4[x][3] += a.w;
      adv[x][0] += c.x; adv[x][1] += c.y; adv[x][2] += c.z; adv[x][3] += c.w;
    }
  }
  if (s < nj) {
    uint16_t *dkr = dk + (rowbase + s) * D, *dvr = dv + (rowbase + s) * D;
#pragma unroll
    for (int x = 0; x < CG; ++x) {
      *(uint2 *)(dkr + 16 * x + 4 * g) =
          make_uint2(pack2bf(ok4[x][0], ok4[x][1]), pack2bf(ok4[x][2], ok4[x][3]));
      *(uint2 *)(dvr + 16 * x + 4 * g) =
          make_uint2(pack2bf(adv[x][0], adv[x][1]), pack2bf(adv[x][2], adv[x][3]));
    }
  }
}

// ---------------------------------------------------------------------------
// dW = sum over all rows of dO^T O_l: partials per chunk of query blocks
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_bwd_dw(const uint16_t *__restrict__ dO,
                                                const uint16_t *__restrict__ ol, int N, int T,
                                                int nqb, float *__restrict__ dwp) {
  using G = BTile<D>;
  constexpr int P = G::P, CG = G::CG, TILE = G::TILE, NPT = G::NPT;
  constexpr int CT = D / 64;  // 16-row tiles of dW per wave
  __shared__ __attribute__((aligned(16))) uint16_t ra[2 * TILE];
  uint16_t *sdo = ra, *sol = ra + TILE;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int q0 = blockIdx.x * DW_CHUNK, q1 = min(nqb, q0 + DW_CHUNK);
  v4f acc[CT][CG];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int x = 0; x < CG; ++x) acc[ct][x] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int qb = q0; qb < q1; ++qb) {
    const int bh = qb / T, i = qb - bh * T;
    const int ni = min(BLK, N - i * BLK);
    uint4 r[NPT];
    tile_load<D>(dO + ((size_t)bh * N + (size_t)i * BLK) * D, ni, r, tid);
    tile_store<D>(r, sdo, tid);
    tile_load<D>(ol + (size_t)qb * BLK * D, BLK, r, tid);
    tile_store<D>(r, sol, tid);
    __syncthreads();
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2) {
      v4u bf[CG];
#pragma unroll
      for (int x = 0; x < CG; ++x) bf[x] = lds_frag(sol, P, kc2, 16 * x, lane);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const v4u af = lds_frag(sdo, P, kc2, 16 * (CT * w + ct), lane);
#pragma unroll
        for (int x = 0; x < CG; ++x) acc[ct][x] = mfma_bf16(af, bf[x], acc[ct][x]);
      }
    }
    __syncthreads();
  }
  float *out = dwp + (size_t)blockIdx.x * D * D;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int x = 0; x < CG; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        out[(size_t)(16 * (CT * w + ct) + 4 * g + r) * D + 16 * x + l16] = acc[ct][x][r];
}

__global__ void k_dw_sum(const float *__restrict__ dwp, int nchunk, int DD, float *__restrict__ dw) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= DD) return;
  float s = 0.f;
  for (int c = 0; c < nchunk; ++c) s += dwp[(size_t)c * DD + e];
  dw[e] = s;
}

__global__ void k_fill_zero_f32(float *__restrict__ x, int n) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n) x[e] = 0.f;
}

template <int D, bool LIN>
static void launch_bwd_t(const Plan &p, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const uint16_t *w, const uint16_t *dout, uint16_t *dq, uint16_t *dk,
                         uint16_t *dv, const WsPtrs &ws, hipStream_t st) {
  const float qk_scale = p.sm_scale * BWD_LOG2E;
  const int nqb = p.BH * p.T;
  if (LIN)
    hipLaunchKernelGGL(k_bwd_qlin<D>, dim3(nqb), dim3(256), 0, st, q, w, dout, ws.hi, p.N, p.T,
                       p.F, ws.ol, ws.dhi, ws.dql);
  hipLaunchKernelGGL((k_bwd_q<D, LIN>), dim3(nqb), dim3(256), 0, st, q, k, v, ws.os, dout, ws.lse,
                     ws.kept, ws.mu, ws.dql, p.N, p.T, p.kb, qk_scale, p.sm_scale, ws.delta, dq);
  if (LIN) {
    launch_marginal_ptrs(p, ws.mtt, ws.dhi, ws.dhb, st);
    hipLaunchKernelGGL(k_bwd_kvlin<D>, dim3(nqb), dim3(256), 0, st, k, v, ws.dhb, p.N, p.T, p.F,
                       ws.dkl, ws.dvl);
  }
  hipLaunchKernelGGL((k_bwd_kv<D, LIN>), dim3(nqb), dim3(256), 0, st, q, k, v, dout, ws.lse,
                     ws.delta, ws.mt, ws.dkl, ws.dvl, p.N, p.T, p.W64, qk_scale, p.sm_scale, dk, dv);
}

void launch_bwd(const Plan &p, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                const uint16_t *w, const uint16_t *dout, uint16_t *dq,
                uint16_t *dk, uint16_t *dv, float *dw, const WsPtrs &ws, hipStream_t st) {
  const int nwaves = p.BH * p.W64 * p.W64;
  hipLaunchKernelGGL(k_mask_t, dim3((nwaves + 3) / 4), dim3(256), 0, st, ws.mask, p.BH, p.T, p.W64,
                     ws.mt, p.lin_on ? ws.mtt : nullptr);
  if (p.d == 128) {
    if (p.lin_on) launch_bwd_t<128, true>(p, q, k, v, w, dout, dq, dk, dv, ws, st);
    else launch_bwd_t<128, false>(p, q, k, v, w, dout, dq, dk, dv, ws, st);
  } else {
    if (p.lin_on) launch_bwd_t<64, true>(p, q, k, v, w, dout, dq, dk, dv, ws, st);
    else launch_bwd_t<64, false>(p, q, k, v, w, dout, dq, dk, dv, ws, st);
  }
  if (!dw) return;
  const int DD = p.d * p.d;
  if (p.lin_on) {
    const int nqb = p.BH * p.T;
    if (p.d == 128)
      hipLaunchKernelGGL(k_bwd_dw<128>, dim3(p.dw_chunks), dim3(256), 0, st, dout, ws.ol, p.N, p.T, nqb, ws.dwp);
    else
      hipLaunchKernelGGL(k_bwd_dw<64>, dim3(p.dw_chunks), dim3(256), 0, st, dout, ws.ol, p.N, p.T, nqb, ws.dwp);
    hipLaunchKernelGGL(k_dw_sum, dim3((DD + 255) / 256), dim3(256), 0, st, ws.dwp, p.dw_chunks, DD, dw);
  } else {
    hipLaunchKernelGGL(k_fill_zero_f32, dim3((DD + 255) / 256), dim3(256), 0, st, dw, DD);
  }
}

}  // namespace sla
