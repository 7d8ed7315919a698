// W8A8 linear layers: block-128 INT8 quantisation and the block-scaled INT8
// GEMM Y = X W^T.
//
// Pages: "揭秘TurboDiffusion…" section "支柱三：W8A8线性层量化" (weights and
// activations of the linear layers both INT8, quantised over 128 x 128
// blocks) and the aiho.net news report (量子位, 2025-12-26)
// section "4. W8A8量化+底层算子重写" (the same, run on the INT8 matrix units).
//
// k_quant_b128: one workgroup per 128 x 128 block of a bf16 [R][C] matrix:
//   scale = amax / 127 (float64 division), codes = rint(x * float32(127 /
//   amax)) clamped to [-127, 127] (round half to even); row-major int8 codes.
// k_w8a8_gemm: a workgroup computes a 128 x 256 tile of Y with 8 waves (two
//   per SIMD) of 64 x 64; per K block of 128 the exact int32 products come
//   from v_mfma_i32_16x16x64_i8 and are folded into float32 accumulators with
//   one fma by the block's scale product sx * sw (float32), blocks in
//   ascending order.  X and W tiles go from global memory straight into a
//   3-stage LDS ring by the load-to-LDS instruction, two K blocks ahead of
//   their use (16-byte pieces XOR-swizzled by row so the fragment reads
//   spread over all banks).
//
// On gfx950 the fold costs two vector ALU instructions per output element per
// K block (convert, fma): as much issue time as the block's MFMAs, so the
// kernel relies on its two waves per SIMD to overlap the two.
#include "sla_internal.h"

namespace sla {

constexpr int WB = 128;  // quantisation block

__global__ __launch_bounds__(256) void k_quant_b128(const uint16_t *__restrict__ X, int R, int C,
                                                    int8_t *__restrict__ codes,
                                                    float *__restrict__ scales) {
  __shared__ float wmax[4];
  const int cb = blockIdx.x, rb = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = rb * WB + (tid >> 1);
  const int c0 = cb * WB + 64 * (tid & 1);
  const bool rok = r < R;
  // 64 columns per thread as eight 16-byte pieces (C is a multiple of 16, so
  // a piece is entirely inside or outside the matrix)
  uint4 raw[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int c = c0 + 8 * p;
    raw[p] = (rok && c < C) ? *(const uint4 *)(X + (size_t)r * C + c) : make_uint4(0u, 0u, 0u, 0u);
  }
  float a = 0.f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint32_t v[4] = {raw[p].x, raw[p].y, raw[p].z, raw[p].w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      a = fmaxf(a, fmaxf(fabsf(bf2f((uint16_t)(v[e] & 0xFFFF))), fabsf(bf2f((uint16_t)(v[e] >> 16)))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  if (lane == 0) wmax[w] = a;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float inv = amax > 0.f ? (float)(127.0 / (double)amax) : 0.f;
  if (tid == 0) scales[(size_t)rb * gridDim.x + cb] = (float)((double)amax / 127.0);
  if (!rok) return;
#pragma unroll
  for (int p = 0; p < 4; ++p) {  // 16 codes per store
    const int c = c0 + 16 * p;
    if (c >= C) break;
    uint32_t out[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v4 = raw[2 * p + (q >> 1)];
      const uint32_t pair0 = (q & 1) ? v4.z : v4.x, pair1 = (q & 1) ? v4.w : v4.y;
      const float x[4] = {bf2f((uint16_t)(pair0 & 0xFFFF)), bf2f((uint16_t)(pair0 >> 16)),
                          bf2f((uint16_t)(pair1 & 0xFFFF)), bf2f((uint16_t)(pair1 >> 16))};
      uint32_t packed = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float y = __builtin_rintf(x[e] * inv);
        y = fminf(fmaxf(y, -127.f), 127.f);
        packed |= ((uint32_t)(uint8_t)(int8_t)(int)y) << (8 * e);
      }
      out[q] = packed;
    }
    *(uint4 *)(codes + (size_t)r * C + c) = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

constexpr int GM_BM = 128, GM_BN = 256, GM_BK = 128;
constexpr int GM_STAGES = 3;          // LDS ring of K blocks

// load-to-LDS copy: lane l's 16 bytes land at LDS address lds + 16 l (lds
// wave-uniform)
__device__ __forceinline__ void w8_copy16(const void *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory");
}
template <int N>
__device__ __forceinline__ void w8_wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// workgroup barrier without __syncthreads' memory fence (its vmcnt(0) would
// drain the copies in flight); the wave's LDS reads are complete on arrival
__device__ __forceinline__ void w8_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
constexpr int GM_G = 4;               // row tiles per ordering group
constexpr int GM_PITCH = GM_BK;       // bytes per LDS row
// LDS byte offset of the 16 bytes lane l reads for an MFMA operand: row
// row0 + l%16, k chunk kc, bytes 64 kc + 16 (l/16) of the row; the 16-byte
// pieces of a row are XOR-swizzled by its index, so the 16 rows of a
// fragment, and the 8 pieces of a row, fall on distinct banks.
__device__ __forceinline__ int lds_off(int row0, int kc, int lane) {
  const int row = row0 + (lane & 15);
  return row * GM_PITCH + 16 * ((4 * kc + (lane >> 4)) ^ (row & 7));
}

__global__ __launch_bounds__(512, 1) void k_w8a8_gemm(const int8_t *__restrict__ xq,
                                                      const float *__restrict__ sx,
                                                      const int8_t *__restrict__ wq,
                                                      const float *__restrict__ sw, int M, int N,
                                                      int K, uint16_t *__restrict__ y) {
  // a ring of stages of [A 128 rows | B 256 rows] x 128 bytes
  constexpr int STG = (GM_BM + GM_BN) * GM_PITCH;  // bytes per stage
  __shared__ __attribute__((aligned(16))) uint8_t lds[GM_STAGES * STG];
  // Tile order: groups of GM_G row tiles; inside a group the row tile runs
  // fastest, so consecutive workgroups (one XCD, xcd_remap) share a W tile
  // and a group's X tiles are reused across all column tiles.
  const int MT = (M + GM_BM - 1) / GM_BM, NT = (N + GM_BN - 1) / GM_BN;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = bid / (GM_G * NT), rem = bid - grp * (GM_G * NT);
  const int gs = min(GM_G, MT - grp * GM_G);
  const int tn = rem / gs, tm = grp * GM_G + (rem - tn * gs);
  const int m0 = tm * GM_BM, n0 = tn * GM_BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = w >> 2, wc = w & 3;  // wave tile rows 64 wr.., columns 64 wc..
  const int KB = K / GM_BK;
  const int mb = m0 / WB;             // one X scale row per workgroup
  // one W scale row per wave (clamped: a wave wholly past N stores nothing)
  const int nb = min((n0 + 64 * wc) / WB, (N - 1) / WB);

  // global -> LDS copies: 384 rows x 8 pieces of 16 bytes per K block; copy
  // it (0..5) of wave w covers rows 64 it + 8 w .. +7 (A rows first), lane l
  // row 64 it + 8 w + l/8 at LDS piece l%8, which holds global piece
  // (l%8) ^ (row%8).  Rows past M / N read the last row (their products are
  // never stored).
  const int pc = tid & 7;
  const int8_t *src_[6];
  uint32_t dst_[6];
#pragma unroll
  for (int it = 0; it < 6; ++it) {
    const int row = 64 * it + 8 * w + (lane >> 3);
    src_[it] = (row < GM_BM ? xq + (size_t)min(m0 + row, M - 1) * K
                            : wq + (size_t)min(n0 + row - GM_BM, N - 1) * K) +
               16 * (pc ^ (row & 7));
    dst_[it] = (64 * it + 8 * w) * GM_PITCH;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)lds;
  auto copy_kb = [&](int kb_) {
    const size_t ko = (size_t)kb_ * GM_BK;
    const uint32_t sb = lds0 + (uint32_t)((kb_ % GM_STAGES) * STG);
#pragma unroll
    for (int it = 0; it < 6; ++it)
      w8_copy16(src_[it] + ko, __builtin_amdgcn_readfirstlane(sb + dst_[it]));
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // K block kb is copied two blocks ahead; before a block's barrier each
  // wave waits for its copy of the next block, so the stage read next is
  // complete, and the barrier also frees the stage the next copy overwrites
  copy_kb(0);
  if (KB > 1) {
    copy_kb(1);
    w8_wait_vm<6>();
  } else {
    w8_wait_vm<0>();
  }
  w8_barrier();
  for (int kb = 0; kb < KB; ++kb) {
    const int s = kb % GM_STAGES;
    if (kb + 2 < KB) copy_kb(kb + 2);
    // exact int32 block products: lane (row 16 i + l%16, group g) reads
    // bytes 64 kc + 16 g .. +15 of its row
    v4i af[4][2], bf[4][2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i][kc] = *(const v4i *)(lds + s * STG + lds_off(64 * wr + 16 * i, kc, lane));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j][kc] = *(const v4i *)(lds + s * STG + lds_off(GM_BM + 64 * wc + 16 * j, kc, lane));
    }
    // Tile t = (i, j): its two MFMAs (the exact int32 block product), then
    // the fold of tile t-1 into the float32 sums, one fma by sx * sw per
    // element; the fences keep this order, so the fold's vector ALU work runs
    // while the matrix core computes the next tile.
    const float sc = sx[(size_t)mb * KB + kb] * sw[(size_t)nb * KB + kb];
    v4i ia[2];
    // raised wave priority while this wave issues its products and folds:
    // the other wave of the SIMD does its LDS reads meanwhile instead of in
    // lockstep
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t = 0; t <= 16; ++t) {
      if (t < 16) {
        const int i = t >> 2, j = t & 3;
        ia[t & 1] = mfma_i8(af[i][0], bf[j][0], v4i{0, 0, 0, 0});
        ia[t & 1] = mfma_i8(af[i][1], bf[j][1], ia[t & 1]);
      }
      if (t > 0) {
        const int i = (t - 1) >> 2, j = (t - 1) & 3;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[i][j][r] = __builtin_fmaf((float)ia[(t - 1) & 1][r], sc, acc[i][j][r]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    if (kb + 2 < KB) w8_wait_vm<6>(); else w8_wait_vm<0>();
    w8_barrier();
  }
  // store bf16: lane holds rows 4 (l/16) + r of column l%16 of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 64 * wc + 16 * j + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const int m = m0 + 64 * wr + 16 * i + 4 * (lane >> 4) + r;
        const uint32_t pr = pack2bf(acc[i][j][r], acc[i][j][r + 1]);
        if (n < N) {
          if (m < M) y[(size_t)m * N + n] = (uint16_t)pr;
          if (m + 1 < M) y[(size_t)(m + 1) * N + n] = (uint16_t)(pr >> 16);
        }
      }
    }
}

void launch_quant_b128(const uint16_t *x, int R, int C, int8_t *codes, float *scales,
                       hipStream_t st) {
  dim3 grid((C + WB - 1) / WB, (R + WB - 1) / WB), block(256);
  hipLaunchKernelGGL(k_quant_b128, grid, block, 0, st, x, R, C, codes, scales);
}

void launch_w8a8_gemm(const int8_t *xq, const float *sx, const int8_t *wq, const float *sw, int M,
                      int N, int K, uint16_t *y, hipStream_t st) {
  const int tiles = ((M + GM_BM - 1) / GM_BM) * ((N + GM_BN - 1) / GM_BN);
  hipLaunchKernelGGL(k_w8a8_gemm, dim3(tiles), dim3(512), 0, st, xq, sx, wq, sw, M, N, K, y);
}

}  // namespace sla
