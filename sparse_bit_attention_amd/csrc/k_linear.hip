// Linear-attention branch of SLA: per key block states and, per query block,
// their sum over the marginal (non-kept) key blocks.
//
// Pages: "揭秘TurboDiffusion…" section "支柱二：稀疏线性注意力 – SLA" (a light
// linear-attention component complements the sparse exact part);
// "TurboDiffusion跨模态：图文音视频多模态融合探索" (zizhi168.cn) section 2.2
// (linear complexity through a kernel-function approximation).  The feature map phi is read as a softmax
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

// One workgroup (4 waves) per key block.  KQ = 1 or 2: the block's K' = K - mu
// is also quantised to INT8 here (K is read once for both): one scale per
// block (KQ = 1) or per 4 keys (KQ = 2, the finer SageAttention2++-style
// granularity); k' = float32(K - mu[c]), scale = amax / 127 over the group's
// valid rows, codes = rint(k' * float32(127 / amax)) clamped to [-127, 127]
// (0 for padding rows) in the i8_off fragment order; dkn = the largest
// scale * ||k8 row|| (times 1 + 2^-20) over the block's groups, dkx = the
// largest scale.  LDS: V and phi(K) as row-major bf16
// [key][channel] tiles; the pitch (D + 16 elements) keeps the rows 8-byte
// aligned and puts four consecutive rows on distinct banks, so operand
// fragments come straight from the transposing read.  The state is computed
// as H = phi(K)^T V (rows: phi channel c, columns: value channel c2), whose
// accumulators hold four consecutive c per lane: one 8-byte store each into
// the hstate_off order.
template <int D, bool LIN, int KQ>
__global__ __launch_bounds__(256) void k_kv_prep(const uint16_t *__restrict__ K,
                                                 const uint16_t *__restrict__ V,
                                                 const float *__restrict__ mu, int N, int T,
                                                 int F, uint16_t *__restrict__ vt,
                                                 uint16_t *__restrict__ hb,
                                                 int8_t *__restrict__ k8, float *__restrict__ dk,
                                                 float *__restrict__ dkn,
                                                 float *__restrict__ dkx) {
  constexpr int P = D + 16;  // row pitch in bf16
  constexpr int CG = D / 16;
  constexpr int KC32 = D / 32;
  constexpr int MT = CG / 4;  // row tiles (16 phi channels) per wave
  constexpr int NG = KQ == 2 ? 16 : 1;  // K' scale groups per block
  constexpr bool LOADK = LIN || KQ > 0;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 64 * P];
  __shared__ __attribute__((aligned(16))) int8_t s8[KQ > 0 ? 64 * D : 16];
  __shared__ uint32_t s_amax[NG], s_gsq[NG];  // float bits (all values >= 0)
  uint16_t *sv = smem, *sk = smem + 64 * P;
  const int blk = blockIdx.x;
  const int bh = blk / T, j = blk - bh * T;
  const int n = min(BLK, N - j * BLK);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const size_t base = ((size_t)bh * N + (size_t)j * BLK) * D;
  if (KQ > 0 && tid < NG) s_amax[tid] = s_gsq[tid] = 0u;  // visible after the staging barrier

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
    if (LOADK) kk[e] = *(const uint2 *)(K + base + (size_t)rc * D + c);
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

  // K' quantisation, first half: each thread holds channels c .. c+3 of rows
  // tid / (D/4) + (256 / (D/4)) e; for every e the wave's 64 lanes lie in one
  // scale group, so a wave max then one LDS max per (wave, e) gives each
  // group's amax (exact in any order)
  constexpr int RPE = 256 / (D / 4);  // rows per piece index e
  const int kc0 = (tid % (D / 4)) * 4;
  float4 m4 = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (KQ > 0) {
    m4 = *(const float4 *)(mu + (size_t)bh * D + kc0);
#pragma unroll
    for (int e = 0; e < NX; ++e) {
      const int r = tid / (D / 4) + RPE * e;
      const uint2 v = kk[e];
      float a = fmaxf(fmaxf(fabsf(bf2f(v.x & 0xFFFF) - m4.x), fabsf(bf2f(v.x >> 16) - m4.y)),
                      fmaxf(fabsf(bf2f(v.y & 0xFFFF) - m4.z), fabsf(bf2f(v.y >> 16) - m4.w)));
      if (r >= n) a = 0.f;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
      const int q = NG == 1 ? 0 : (RPE * e + 64 * w / (D / 4)) / 4;
      if (lane == 0) atomicMax(&s_amax[q], __float_as_uint(a));
    }
  }

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

  // K' quantisation, second half: codes into LDS in fragment order, each
  // row's squared code norm (a sum over the row's D/4 lanes), its group max
  if constexpr (KQ > 0) {
    constexpr int KC = D / 64;
#pragma unroll
    for (int e = 0; e < NX; ++e) {
      const int r = tid / (D / 4) + RPE * e;
      const int q = NG == 1 ? 0 : (RPE * e + 64 * w / (D / 4)) / 4;
      const float amax = __uint_as_float(s_amax[q]);
      const float inv = amax > 0.f ? (float)(127.0 / (double)amax) : 0.f;
      const uint2 v = kk[e];
      const float xs[4] = {bf2f(v.x & 0xFFFF) - m4.x, bf2f(v.x >> 16) - m4.y,
                           bf2f(v.y & 0xFFFF) - m4.z, bf2f(v.y >> 16) - m4.w};
      uint32_t packed = 0;
      int sq = 0;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        float y = __builtin_rintf(xs[x] * inv);
        y = fminf(fmaxf(y, -127.f), 127.f);
        const int code = (int)y;
        sq += code * code;
        packed |= ((uint32_t)(uint8_t)(int8_t)code) << (8 * x);
      }
      if (r >= n) packed = 0, sq = 0;
      *(uint32_t *)(&s8[i8_off(r, kc0, KC)]) = packed;
#pragma unroll
      for (int off = D / 8; off >= 1; off >>= 1) sq += __shfl_xor(sq, off, 64);
      float gm = (float)sq;
#pragma unroll
      for (int off = D / 4; off < 64; off <<= 1) gm = fmaxf(gm, __shfl_xor(gm, off, 64));
      if (lane == 0) atomicMax(&s_gsq[q], __float_as_uint(gm));
    }
    __syncthreads();
    {
      const uint4 *src = (const uint4 *)s8;
      uint4 *dst = (uint4 *)(k8 + (size_t)blk * BLK * D);
#pragma unroll
      for (int it = 0; it < (BLK * D) / (16 * 256); ++it) dst[it * 256 + tid] = src[it * 256 + tid];
    }
    if (tid < NG) dk[(size_t)blk * NG + tid] = (float)((double)__uint_as_float(s_amax[tid]) / 127.0);
    if (tid == 0) {
      float bmax = 0.f, dmax = 0.f;
#pragma unroll
      for (int q = 0; q < NG; ++q) {
        const float delta = (float)((double)__uint_as_float(s_amax[q]) / 127.0);
        bmax = fmaxf(bmax, delta * (sqrtf(__uint_as_float(s_gsq[q])) * (1.0f + 0x1p-20f)));
        dmax = fmaxf(dmax, delta);
      }
      dkn[blk] = bmax;
      dkx[blk] = dmax;
    }
  }

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
// one element per thread, D*D/256 workgroups
__global__ __launch_bounds__(256) void k_w_swizzle(const uint16_t *__restrict__ W, int D,
                                                   uint16_t *__restrict__ wsw) {
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x >= D * D) return;
  const int row = x / D, k = x - row * D;
  wsw[wfrag_off(row, k, D / 32)] = W[x];
}

// H[i][f] = sum_j (1 - M[i][j]) Hb[j][f]: per head a [T x T] by [T x F] GEMM,
// 32x32x16 bf16 MFMA with float32 accumulation, written back as bf16.
// A workgroup (8 waves, two per SIMD, so one wave's products cover the
// other's waits) owns a 256 x 256 output tile; wave w owns rows 64 (w/2) ..
// +63 and columns 128 (w%2) .. +127 in 8 accumulator tiles.  Per step of 32
// key blocks:
//  * A (the complement mask as bf16 ones and zeros) is built by each wave
//    from its rows' mask words, four keys at a time through a 16-entry table
//    of bf16 patterns in LDS;
//  * B (32 Hb rows x 256 columns) is staged in LDS in MFMA fragment order:
//    thread (w, l) loads keys 4w .. 4w+3 of columns 4l .. 4l+3 and writes
//    half of each of those columns' 16-byte fragment slots.  Slots are
//    XOR-swizzled by their 8-slot group, so both the writes and the fragment
//    reads spread over all banks.
// Pipeline (step s): issue the global loads of step s+3, read step s+1's B
// fragments into registers, run step s's products from registers, then
// store step s+2's B (loaded one step earlier) into LDS.  B is triple-buffered
// in LDS, so one barrier per step suffices, and the products never wait for
// LDS.  The row tiles of one column tile run one after another on one XCD,
// so each Hb column slice comes from HBM once.
constexpr int MG_BM = 256;  // rows per workgroup
constexpr int MG_BN = 256;  // columns per workgroup
constexpr int MG_BK = 32;   // key blocks per step

template <int D>
__global__ __launch_bounds__(512, 1) void k_marginal(const uint64_t *__restrict__ maskt,
                                                     const uint16_t *__restrict__ hb, int T,
                                                     int W64, int F, int ntiles,
                                                     uint16_t *__restrict__ hi) {
  // three B buffers of 16 KiB; the epilogue reuses all 128 KiB to stage each
  // wave's bf16 tile
  // lds[0..8): the table, nibble n (keys k .. k+3, bit i = key k+i) as four
  // bf16 ones and zeros (at LDS address 0, so a table offset is an address)
  __shared__ __attribute__((aligned(16))) uint4 lds[8 + 8192];
  uint2 *lut = (uint2 *)lds;
  uint4 *smem = lds + 8;
  const int RT = (T + MG_BM - 1) / MG_BM, CT = (F + MG_BN - 1) / MG_BN;
  // Tiles in the order (head, column tile, row tile), row tile fastest; XCD x
  // (= blockIdx.x % 8) owns one contiguous eighth of that order and its
  // workgroups take every L-th tile of it, so the row tiles of a column tile
  // run close together in time on one XCD and share its L2.
  const int xcd = blockIdx.x & 7, L = gridDim.x >> 3;
  const int tq = ntiles >> 3, tr = ntiles & 7;
  const int tbeg = xcd * tq + min(xcd, tr), tcnt = tq + (xcd < tr ? 1 : 0);
  int li = blockIdx.x >> 3;
  if (li >= tcnt) return;  // no barriers before this point
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = w >> 1, wc = w & 1;
  const int kshift = 8 * (lane >> 5);
  if (tid < 16)  // visible after the first tile's first barrier
    lut[tid] = make_uint2(((tid & 1) ? 0x3F80u : 0u) | ((tid & 2) ? 0x3F800000u : 0u),
                          ((tid & 4) ? 0x3F80u : 0u) | ((tid & 8) ? 0x3F800000u : 0u));

  // ---- the current tile: A lane l owns rows 64 wr + 32 x + l%32 (x < 2) and
  // keys 8 (l/32) .. +7 of each 16-key half-step; rows past T read row T-1
  // (their outputs are never stored).  B: thread (w, l) holds keys 4w .. 4w+3
  // of columns 4l .. 4l+3; keys past T read row T-1 (their A entries are 0),
  // columns past F read the last four columns (never stored).
  int bh = 0, row0 = 0, col0 = 0, arow[2], bcol = 0;
  const uint16_t *hbh = hb;
  const uint64_t *mh = maskt;  // word-major: [W64][T]
  auto set_tile = [&](int t) {
    const int rt = t % RT, r2 = t / RT;
    col0 = (r2 % CT) * MG_BN;
    bh = r2 / CT;
    row0 = rt * MG_BM;
    hbh = hb + (size_t)bh * T * F;
    mh = maskt + (size_t)bh * W64 * T;
#pragma unroll
    for (int x = 0; x < 2; ++x) arow[x] = min(row0 + 64 * wr + 32 * x + (lane & 31), T - 1);
    bcol = min(col0 + 4 * lane, F - 4);
  };
  auto load_words = [&](int word, uint64_t (&wd)[2]) {
    word = min(word, W64 - 1);
#pragma unroll
    for (int x = 0; x < 2; ++x) wd[x] = mh[(size_t)word * T + arow[x]];
  };
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

  // B fragments of one step: [ks][y], column tile 4 wc + y
  auto read_b = [&](const uint4 *buf, v4u (&bf)[2][4]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int y = 0; y < 4; ++y) bf[ks][y] = __builtin_bit_cast(v4u, buf[((4 * wc + y) * 2 + ks) * 64 + rslot]);
  };
  // one step: A from the mask words, B from registers
  auto mma_step = [&](int s, const uint64_t (&wd)[2], const v4u (&bf)[2][4]) {
    const int j0 = s * MG_BK;
    const int nvalid = T - j0;  // key blocks past T contribute nothing
    const uint32_t valid = nvalid >= 32 ? ~0u : (nvalid > 0 ? (1u << nvalid) - 1u : 0u);
    // the four nibbles of a lane's keys (half-step ks, keys 8 (l/32) .. +7)
    // as byte offsets into the table: byte 2 ks + h = nibble h of byte ks, x 8
    uint32_t u[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const uint32_t t = ((~(uint32_t)(wd[x] >> (j0 & 32))) & valid) >> kshift;
      u[x] = ((t & 0x000F000Fu) << 3) | ((t & 0x00F000F0u) << 7);
    }
    const char *lb = (const char *)lut;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4u af[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const uint2 lo = *(const uint2 *)(lb + __builtin_amdgcn_ubfe(u[x], 16 * ks, 8));
        const uint2 hi2 = *(const uint2 *)(lb + __builtin_amdgcn_ubfe(u[x], 16 * ks + 8, 8));
        af[x] = v4u{lo.x, lo.y, hi2.x, hi2.y};
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = mfma32_bf16(af[x], bf[ks][y], acc[x][y]);
    }
  };
  auto nxt = [](int i) { return i == 2 ? 0 : i + 1; };

  // Steps in pairs (an even count; a step past T has an all-zero A, and
  // loads past the last step read clamped rows): the staging registers, the
  // B fragment sets and the mask words keep fixed names.
  const int steps = (((T + MG_BK - 1) / MG_BK) + 1) & ~1;
  uint2 gA[4], gB[4];        // global staging: steps of even / odd index
  v4u bf0[2][4], bf1[2][4];  // B fragments: steps of even / odd index
  uint64_t wdc[2], wdn[2];
  // the first tile's first loads; a later tile's are issued before the
  // previous tile's output stores, so those stores drain behind the next
  // tile's products
  set_tile(tbeg + li);
  load_b(0, gA);
  load_b(1, gB);
  load_words(0, wdc);
  for (; li < tcnt; li += L) {
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;
    store_b(gA, smem);
    store_b(gB, smem + 1024);
    load_b(2, gA);
    __syncthreads();
    read_b(smem, bf0);
    int bi = 0;  // LDS buffer of step s
    for (int s = 0; s < steps; s += 2) {
      int b1 = nxt(bi), b2 = nxt(b1);
      // even step s
      load_b(s + 3, gB);
      load_words((s + 2) >> 1, wdn);
      read_b(smem + 1024 * b1, bf1);
      __builtin_amdgcn_sched_barrier(0);
      // a wave issuing its products outranks the other wave of its SIMD, so
      // the two drift apart and one's LDS and vector work runs under the
      // other's MFMAs (s_setprio: wave priority only; ~2% here)
      __builtin_amdgcn_s_setprio(1);
      mma_step(s, wdc, bf0);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      store_b(gA, smem + 1024 * b2);
      __syncthreads();
      bi = b1;
      b1 = b2;
      b2 = nxt(b2);
      // odd step s+1
      load_b(s + 4, gA);
      read_b(smem + 1024 * b1, bf0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      mma_step(s + 1, wdc, bf1);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      store_b(gB, smem + 1024 * b2);
      __syncthreads();
      bi = b1;
#pragma unroll
      for (int x = 0; x < 2; ++x) wdc[x] = wdn[x];
    }

    // epilogue: each wave stages its 64 x 128 tile as bf16 rows (256 B
    // pitch), then writes 16-byte pieces of rows < T, columns < F
    const int orow0 = row0 + 64 * wr, ocol0 = col0 + 128 * wc;
    uint16_t *hih = hi + (size_t)bh * T * F;
    if (li + L < tcnt) {
      set_tile(tbeg + li + L);
      load_b(0, gA);
      load_b(1, gB);
      load_words(0, wdc);
    }
    uint16_t *st = (uint16_t *)(smem + w * 1024);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          // registers r, r+1: rows rr, rr+1 of column cc
          const int rr = 32 * x + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int cc = 32 * y + (lane & 31);
          const uint32_t pr = pack2bf(acc[x][y][r], acc[x][y][r + 1]);
          st[rr * 128 + cc] = (uint16_t)pr;
          st[(rr + 1) * 128 + cc] = (uint16_t)(pr >> 16);
        }
        // one accumulator tile at a time (keeps the register demand small)
        __builtin_amdgcn_sched_barrier(0);
      }
    // the staging area is private to the wave: its own LDS ordering suffices
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int piece = it * 64 + lane;  // 16 pieces of 8 columns per row
      const int rr = piece >> 4, c8 = (piece & 15) * 8;
      const int row = orow0 + rr, col = ocol0 + c8;
      if (row < T && col < F)
        *(uint4 *)(hih + (size_t)row * F + col) = *(const uint4 *)(st + rr * 128 + c8);
    }
    __syncthreads();  // staging reads done before the next tile's B stores
  }
}

void launch_kv_prep(const Plan &p, const uint16_t *k, const uint16_t *v, const WsPtrs &ws,
                    hipStream_t st) {
  dim3 grid(p.BH * p.T), block(256);
#define SLA_KVP(D, LIN, KQ)                                                                   \
  hipLaunchKernelGGL((k_kv_prep<D, LIN, KQ>), grid, block, 0, st, k, v, ws.mu, p.N, p.T, p.F, \
                     ws.vt, ws.hb, ws.k8, ws.dk, ws.dkn, ws.dkx)
#define SLA_KVP_D(D)                                          \
  do {                                                        \
    const int kq = p.qk_int8 ? (p.qk_fine ? 2 : 1) : 0;       \
    if (p.lin_on) {                                           \
      if (kq == 2) SLA_KVP(D, true, 2);                       \
      else if (kq == 1) SLA_KVP(D, true, 1);                  \
      else SLA_KVP(D, true, 0);                               \
    } else {                                                  \
      if (kq == 2) SLA_KVP(D, false, 2);                      \
      else if (kq == 1) SLA_KVP(D, false, 1);                 \
      else SLA_KVP(D, false, 0);                              \
    }                                                         \
  } while (0)
  if (p.d == 128)
    SLA_KVP_D(128);
  else
    SLA_KVP_D(64);
#undef SLA_KVP_D
#undef SLA_KVP
}

void launch_w_swizzle(const Plan &p, const uint16_t *w, const WsPtrs &ws, hipStream_t st) {
  hipLaunchKernelGGL(k_w_swizzle, dim3((p.d * p.d + 255) / 256), dim3(256), 0, st, w, p.d, ws.wsw);
}

void launch_marginal(const Plan &p, const WsPtrs &ws, hipStream_t st) {
  launch_marginal_ptrs(p, ws.maskt, ws.hb, ws.hi, st);
}

void launch_marginal_ptrs(const Plan &p, const uint64_t *maskt, const uint16_t *hb, uint16_t *hi,
                          hipStream_t st) {
  const int RT = (p.T + MG_BM - 1) / MG_BM, CT = (p.F + MG_BN - 1) / MG_BN;
  const int ntiles = p.BH * CT * RT;
  // persistent: one workgroup per CU (256 CUs, 8 XCDs), fewer for small
  // problems
  const int nwg = std::min(256, 8 * ((ntiles + 7) / 8));
  dim3 grid(nwg), block(512);
  if (p.d == 128)
    hipLaunchKernelGGL(k_marginal<128>, grid, block, 0, st, maskt, hb, p.T, p.W64, p.F, ntiles, hi);
  else
    hipLaunchKernelGGL(k_marginal<64>, grid, block, 0, st, maskt, hb, p.T, p.W64, p.F, ntiles, hi);
}

}  // namespace sla
