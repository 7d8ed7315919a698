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

typedef short v4s16 __attribute__((ext_vector_type(4)));

// Four consecutive rows k0 .. k0+3 of column n0 + l%16 of a row-major bf16
// LDS tile (pitch in elements), by the transposing LDS read: lane j of each
// 16-lane group supplies row k0 + j/4, columns n0 + 4(j%4) .. +3.
__device__ __forceinline__ uint2 lds_col4(const uint16_t *tile, int pitch, int k0, int n0,
                                          int lane) {
  const int j = lane & 15;
  const uint16_t *a = tile + (k0 + (j >> 2)) * pitch + n0 + 4 * (j & 3);
  const v4s16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s16 *)a);
  return __builtin_bit_cast(uint2, r);
}

// MFMA operand (16x16x32 bf16, k order of kmaj_off) of the 16 columns n0 ..
// n0+15 and the 32 keys 32 kc2 .. of a row-major [key][column] LDS tile: lane
// (column n0 + l%16, group g = l/16) holds keys 32 kc2 + 4g + 0..3 and
// 32 kc2 + 16 + 4g + 0..3.
__device__ __forceinline__ v4u lds_frag(const uint16_t *tile, int pitch, int kc2, int n0, int lane) {
  const int g = lane >> 4;
  const uint2 lo = lds_col4(tile, pitch, 32 * kc2 + 4 * g, n0, lane);
  const uint2 hi = lds_col4(tile, pitch, 32 * kc2 + 16 + 4 * g, n0, lane);
  return v4u{lo.x, lo.y, hi.x, hi.y};
}

// One workgroup (4 waves) per key block.  LDS: V and phi(K) as row-major bf16
// [key][channel] tiles; the pitch (D + 16 elements) keeps the rows 8-byte
// aligned and puts four consecutive rows on distinct banks, so operand
// fragments come straight from the transposing read.  The state is computed
// as H = phi(K)^T V (rows: phi channel c, columns: value channel c2), whose
// accumulators hold four consecutive c per lane: one 8-byte store each into
// the hstate_off order.
template <int D, bool LIN>
__global__ __launch_bounds__(256) void k_kv_prep(const uint16_t *__restrict__ K,
                                                 const uint16_t *__restrict__ V, int N, int T,
                                                 int F, uint16_t *__restrict__ vt,
                                                 uint16_t *__restrict__ hb) {
  constexpr int P = D + 16;  // row pitch in bf16
  constexpr int CG = D / 16;
  constexpr int KC32 = D / 32;
  constexpr int MT = CG / 4;  // row tiles (16 phi channels) per wave
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 64 * P];
  uint16_t *sv = smem, *sk = smem + 64 * P;
  const int blk = blockIdx.x;
  const int bh = blk / T, j = blk - bh * T;
  const int n = min(BLK, N - j * BLK);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const size_t base = ((size_t)bh * N + (size_t)j * BLK) * D;

  // stage V and K rows (zeros past the valid rows); all loads are issued
  // before any is used
  constexpr int NX = 64 * (D / 4) / 256;  // 8-byte pieces per thread
  uint2 vv[NX], kk[NX];
#pragma unroll
  for (int e = 0; e < NX; ++e) {
    const int x = tid + 256 * e;
    const int r = x / (D / 4), c = (x - r * (D / 4)) * 4;
    const int rc = r < n ? r : n - 1;  // a valid row; zeroed below
    vv[e] = *(const uint2 *)(V + base + (size_t)rc * D + c);
    if (LIN) kk[e] = *(const uint2 *)(K + base + (size_t)rc * D + c);
  }
#pragma unroll
  for (int e = 0; e < NX; ++e) {
    const int x = tid + 256 * e;
    const int r = x / (D / 4), c = (x - r * (D / 4)) * 4;
    const bool ok = r < n;
    *(uint2 *)(sv + r * P + c) = ok ? vv[e] : make_uint2(0u, 0u);
    if (LIN) *(uint2 *)(sk + r * P + c) = ok ? kk[e] : make_uint2(0u, 0u);
  }
  __syncthreads();

  // phi(K) rows in float32, rounded to bf16 in place; four threads per row
  // (D/4 channels each, max and sum combined by shuffles); padding rows
  // become 0.
  if (LIN) {
    constexpr int CPT = D / 4;
    const int r = tid >> 2, part = tid & 3;
    uint16_t *row = sk + r * P + part * CPT;
    float x[CPT];
#pragma unroll
    for (int c = 0; c < CPT; c += 2) {
      const uint32_t two = *(const uint32_t *)(row + c);
      x[c] = bf2f((uint16_t)(two & 0xFFFF));
      x[c + 1] = bf2f((uint16_t)(two >> 16));
    }
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < CPT; ++c) mx = fmaxf(mx, x[c]);
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
    float sm = 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      x[c] = __expf(x[c] - mx);
      sm += x[c];
    }
    sm += __shfl_xor(sm, 1, 64);
    sm += __shfl_xor(sm, 2, 64);
    const float inv = r < n ? 1.0f / sm : 0.0f;
#pragma unroll
    for (int c = 0; c < CPT; c += 2)
      *(uint32_t *)(row + c) = pack2bf(x[c] * inv, x[c + 1] * inv);
  }
  __syncthreads();

  // V fragments (value channels 16 bt .., keys 32 kc2 ..) in the kmaj order
  // the attention kernel reads: B operands here, written out as they are;
  // wave w writes fragments f = kc2 * CG + bt with f % 4 == w
  v4u vf[2][CG];
#pragma unroll
  for (int kc2 = 0; kc2 < 2; ++kc2)
#pragma unroll
    for (int bt = 0; bt < CG; ++bt) vf[kc2][bt] = lds_frag(sv, P, kc2, 16 * bt, lane);
  uint16_t *vdst = vt + (size_t)blk * BLK * D;
#pragma unroll
  for (int kc2 = 0; kc2 < 2; ++kc2)
#pragma unroll
    for (int bt = 0; bt < CG; ++bt)
      if (((kc2 * CG + bt) & 3) == w)
        *(v4u *)(vdst + ((size_t)(kc2 * CG + bt) * 64 + lane) * 8) = vf[kc2][bt];
  if (!LIN) return;

  // H[c][c2] = sum_s phi(K)[s][c] V[s][c2], z[c] = sum_s phi(K)[s][c]: wave w
  // owns the phi rows 16 (MT w + a) .. +15, all value columns and a ones column
  v4f acc[MT][CG], accz[MT];
#pragma unroll
  for (int a = 0; a < MT; ++a) {
    accz[a] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int bt = 0; bt < CG; ++bt) acc[a][bt] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  const v4u ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
  for (int kc2 = 0; kc2 < 2; ++kc2)
#pragma unroll
    for (int a = 0; a < MT; ++a) {
      const v4u af = lds_frag(sk, P, kc2, 16 * (MT * w + a), lane);
#pragma unroll
      for (int bt = 0; bt < CG; ++bt) acc[a][bt] = mfma_bf16(af, vf[kc2][bt], acc[a][bt]);
      accz[a] = mfma_bf16(af, ones, accz[a]);
    }
  // accumulator (a, bt) register r: c = 16 (MT w + a) + 4g + r, c2 = 16 bt + l16;
  // the four c of a lane are consecutive elements of hstate_off, and a wave's
  // stores of one tile fill 512 contiguous bytes
  uint16_t *ho = hb + (size_t)blk * F;
#pragma unroll
  for (int a = 0; a < MT; ++a) {
    const int c0 = 16 * (MT * w + a) + 4 * g;
#pragma unroll
    for (int bt = 0; bt < CG; ++bt) {
      const int c2 = 16 * bt + l16;
      *(uint2 *)(ho + hstate_off(c0, c2, KC32)) =
          make_uint2(pack2bf(acc[a][bt][0], acc[a][bt][1]), pack2bf(acc[a][bt][2], acc[a][bt][3]));
    }
    if (l16 == 0)
      *(uint2 *)(ho + D * D + c0) =
          make_uint2(pack2bf(accz[a][0], accz[a][1]), pack2bf(accz[a][2], accz[a][3]));
  }
  for (int x = D * D + D + tid; x < F; x += 256) ho[x] = 0;
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
// A workgroup (8 waves, two per SIMD, so one wave's products cover the
// other's waits) owns a 256 x 256 output tile; wave w owns rows 64 (w/2) ..
// +63 and columns 128 (w%2) .. +127 in 8 accumulator tiles.  Per step of 32
// key blocks:
//  * A (the complement mask as bf16 ones and zeros) is built by each wave in
//    registers, straight from its rows' mask words;
//  * B (32 Hb rows x 256 columns) is staged in LDS in MFMA fragment order:
//    thread (w, l) loads keys 4w .. 4w+3 of columns 4l .. 4l+3 and writes
//    half of each of those columns' 16-byte fragment slots.  Slots are
//    XOR-swizzled by their 8-slot group, so both the writes and the fragment
//    reads spread over all banks.
// Global loads run two steps ahead; B is double-buffered in LDS.  The row
// tiles of one column tile run one after another on one XCD, so each Hb
// column slice comes from HBM once.
constexpr int MG_BM = 256;  // rows per workgroup
constexpr int MG_BN = 256;  // columns per workgroup
constexpr int MG_BK = 32;   // key blocks per step

// 8 mask bits (keys k .. k+7, bit i = key k+i, 1 = use the block) as the four
// dwords of an MFMA operand: dword h holds key 2h (low half) and 2h+1 (high
// half) as bf16 1.0 or 0.  Even keys go to bits 0,2,4,6, odd keys to bits
// 16,18,20,22; bit pair h times (0x3F80 >> 2h) is then dword h.
__device__ __forceinline__ v4u bits_to_bf16x8(uint32_t by) {
  const uint32_t y = (by & 0x55u) | (((by >> 1) & 0x55u) << 16);
  return v4u{(uint32_t)__umul24(y & 0x00010001u, 0x3F80u), (uint32_t)__umul24(y & 0x00040004u, 0x3F80u >> 2),
             (uint32_t)__umul24(y & 0x00100010u, 0x3F80u >> 4), (uint32_t)__umul24(y & 0x00400040u, 0x3F80u >> 6)};
}

template <int D>
__global__ __launch_bounds__(512, 1) void k_marginal(const uint64_t *__restrict__ maskt,
                                                     const uint16_t *__restrict__ hb, int T,
                                                     int W64, int F, uint16_t *__restrict__ hi) {
  // two B buffers of 16 KiB; the epilogue reuses all 128 KiB to stage each
  // wave's bf16 tile
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

  // ---- A: lane l owns rows 64 wr + 32 x + l%32 (x < 2) and keys 8 (l/32) ..
  // +7 of each 16-key half-step.  Rows past T read row T-1 (their outputs are
  // never stored).
  int arow[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) arow[x] = min(row0 + 64 * wr + 32 * x + (lane & 31), T - 1);
  auto load_words = [&](int word, uint64_t (&wd)[2]) {
    word = min(word, W64 - 1);
#pragma unroll
    for (int x = 0; x < 2; ++x) wd[x] = mh[(size_t)word * T + arow[x]];
  };
  const int kshift = 8 * (lane >> 5);

  // ---- B: thread (w, l) holds keys 4w .. 4w+3 of columns 4l .. 4l+3.  Keys
  // past T read row T-1 (their A entries are 0); columns past F read the last
  // four columns (never stored).
  const int bcol = min(col0 + 4 * lane, F - 4);
  auto load_b = [&](int s, uint2 (&v)[4]) {
    const int j0 = s * MG_BK + 4 * w;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = *(const uint2 *)(hbh + (size_t)min(j0 + k, T - 1) * F + bcol);
  };
  // column 4l + i, key group g = w/2 (8 keys): fragment (l/8, g/2), slot s =
  // 4 (l%8) + i + 32 (g%2), stored at s ^ ((s/8)%8) = 32 (g%2) + 4 ((l%8) ^
  // (g%2)) + (i ^ (l%8)/2); this thread fills 8 bytes at offset 8 (w%2)
  const int g8 = w >> 1;
  int bslot[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    bslot[i] = (((lane >> 3) * 2 + (g8 >> 1)) * 64) + 32 * (g8 & 1) + 4 * ((lane & 7) ^ (g8 & 1)) +
               (i ^ ((lane & 7) >> 1));
  auto store_b = [&](const uint2 (&v)[4], uint4 *buf) {
    uint2 *half = (uint2 *)buf + (w & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t d[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t lo = (i < 2) ? v[2 * h].x : v[2 * h].y;
        const uint32_t hi2 = (i < 2) ? v[2 * h + 1].x : v[2 * h + 1].y;
        d[h] = __builtin_amdgcn_perm(hi2, lo, (i & 1) ? 0x07060302u : 0x05040100u);
      }
      half[2 * bslot[i]] = make_uint2(d[0], d[1]);
    }
  };
  // fragment reads: lane l reads slot l ^ ((l/8)%8)
  const int rslot = lane ^ ((lane >> 3) & 7);

  v16f acc[2][4];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;

  // one step: A from the mask words, B from LDS buffer cur
  auto mma_step = [&](int s, const uint64_t (&wd)[2], const uint4 *cur) {
    const int j0 = s * MG_BK;
    const int nvalid = T - j0;  // key blocks past T contribute nothing
    const uint32_t valid = nvalid >= 32 ? ~0u : (nvalid > 0 ? (1u << nvalid) - 1u : 0u);
    uint32_t t[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) t[x] = ((~(uint32_t)(wd[x] >> (j0 & 32))) & valid) >> kshift;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4u af[2], bf[4];
#pragma unroll
      for (int x = 0; x < 2; ++x) af[x] = bits_to_bf16x8((t[x] >> (16 * ks)) & 0xFFu);
#pragma unroll
      for (int y = 0; y < 4; ++y) bf[y] = __builtin_bit_cast(v4u, cur[((4 * wc + y) * 2 + ks) * 64 + rslot]);
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = mfma32_bf16(af[x], bf[y], acc[x][y]);
    }
  };

  // Steps in pairs (an even count; a step past T has an all-zero A): the two
  // B register sets and the mask words keep fixed names, loaded two steps
  // (the words: one pair) ahead.
  const int steps = (((T + MG_BK - 1) / MG_BK) + 1) & ~1;
  uint2 bvA[4], bvB[4];
  uint64_t wdc[2], wdn[2];
  uint4 *buf0 = smem, *buf1 = smem + 1024;
  {
    uint2 b0[4];
    load_b(0, b0);
    load_b(1, bvA);
    load_words(0, wdc);
    store_b(b0, buf0);
  }
  __syncthreads();
  for (int s = 0; s < steps; s += 2) {
    // even step s: B buffer 0, words wdc (steps s, s+1).  The fences keep the
    // transposing stores (which wait for their loads) after the products.
    load_b(s + 2, bvB);
    load_words((s + 2) >> 1, wdn);
    __builtin_amdgcn_sched_barrier(0);
    mma_step(s, wdc, buf0);
    __builtin_amdgcn_sched_barrier(0);
    store_b(bvA, buf1);
    __syncthreads();
    // odd step s+1: B buffer 1
    load_b(s + 3, bvA);
    __builtin_amdgcn_sched_barrier(0);
    mma_step(s + 1, wdc, buf1);
    __builtin_amdgcn_sched_barrier(0);
    store_b(bvB, buf0);
    __syncthreads();
#pragma unroll
    for (int x = 0; x < 2; ++x) wdc[x] = wdn[x];
  }

  // epilogue: each wave stages its 64 x 128 tile as bf16 rows (256 B pitch),
  // then writes 16-byte pieces of rows < T, columns < F
  uint16_t *st = (uint16_t *)(smem + w * 1024);
#pragma unroll
  for (int x = 0; x < 2; ++x)
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
  const int orow0 = row0 + 64 * wr, ocol0 = col0 + 128 * wc;
  uint16_t *hih = hi + (size_t)bh * T * F;
#pragma unroll 4
  for (int it = 0; it < 16; ++it) {
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
  dim3 grid(p.BH * CT * RT), block(512);
  if (p.d == 128)
    hipLaunchKernelGGL(k_marginal<128>, grid, block, 0, st, ws.maskt, ws.hb, p.T, p.W64, p.F, ws.hi);
  else
    hipLaunchKernelGGL(k_marginal<64>, grid, block, 0, st, ws.maskt, ws.hb, p.T, p.W64, p.F, ws.hi);
}

}  // namespace sla
