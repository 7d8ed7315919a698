// Block scores and per-row top-k selection.
//
// Pages: "TurboDiffusion跨模态：图文音视频多模态融合探索" (zizhi168.cn)
// section 2.1 (Top-K sparse selection, sla_topk) and section 2.2 (sla_topk
// 0.05 / 0.1 / 0.15); "揭秘TurboDiffusion…" section
// "支柱二：稀疏线性注意力 – SLA" (only the most important block interactions get
// exact attention, ~90% sparsity).
//
// s_ij = qbar_i . (kbar_j - mu) is one float32 FMA chain over the channels in
// order from +0, so the scores, and hence the mask, are reproducible bit for
// bit.  Each row keeps the kb largest scores, ties to the lower block index.
//
// Work: T*T*d FMAs per head (plain fp32 ALU) into a float32 score matrix in
// the workspace, then a 32-step bitwise threshold search per row (one wave
// per row, its keys in registers).
#include "sla_internal.h"

namespace sla {

// Monotone map of a finite float32 to uint32 (larger float -> larger key);
// +0 and -0 map to the same key.  Never 0 for a finite float.
__device__ __forceinline__ uint32_t score_key(float v) {
  uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave selects one row: mask words (W64 of them) and the ascending kept
// list (kb entries).  Lane l holds the keys of j = 64e + l, e < E = ceil(T/64).
// EM > 0: the keys sit in EM registers per lane (E <= EM; entries past T hold
// 0, which is below every real key, so the counting loops run unguarded over
// all EM); EM = 0: every pass re-reads them from the score row.
constexpr int SEL_MAXE = 32;
constexpr int SEL_HI = 12;  // key bits decided over all keys before the candidates are packed

__device__ __forceinline__ uint32_t row_key(const float *srow, int T, int e, int lane) {
  const int j = e * 64 + lane;
  return j < T ? score_key(srow[j]) : 0u;  // 0 never equals a real key
}

template <int EM>
__device__ void select_row_t(const float *srow, int T, int kb, uint64_t *mrow, uint64_t *mcol,
                             int32_t *krow, uint32_t *scratch, int lane) {
  const int E = (T + 63) >> 6;
  uint32_t k[EM > 0 ? EM : 1];
  if constexpr (EM > 0) {
#pragma unroll
    for (int e = 0; e < EM; ++e) k[e] = row_key(srow, T, e, lane);
  }
  // th = the kb-th largest key: the largest th with #{key >= th} >= kb,
  // built one bit at a time from the top.
  auto count_ge = [&](uint32_t cand) {
    int cnt = 0;
    if constexpr (EM > 0) {
#pragma unroll
      for (int e = 0; e < EM; ++e) cnt += __popcll(__ballot(k[e] >= cand));
    } else {
      for (int e = 0; e < E; ++e) cnt += __popcll(__ballot(row_key(srow, T, e, lane) >= cand));
    }
    return cnt;
  };
  uint32_t th = 0u;
  int bit = 31;
  if constexpr (EM > 0) {
    // The top SEL_HI bits over all keys; then usually few keys share that
    // prefix P: count(key >= cand) = #(prefix > P) + #(prefix == P, key >=
    // cand), and the candidates fit one register per lane (packed through
    // the wave's LDS scratch), so the low bits cost one ballot per step.
    // (P is never 0: a finite float's key has a nonzero top-12-bit prefix,
    // so the zero entries past T are never candidates.)
    for (; bit >= 32 - SEL_HI; --bit) {
      const uint32_t cand = th | (1u << bit);
      if (count_ge(cand) >= kb) th = cand;
    }
    const uint32_t P = th >> (32 - SEL_HI);
    const int above = (P == (1u << SEL_HI) - 1u) ? 0 : count_ge((P + 1u) << (32 - SEL_HI));
    int ncand = 0;
#pragma unroll
    for (int e = 0; e < EM; ++e) ncand += __popcll(__ballot((k[e] >> (32 - SEL_HI)) == P));
    if (ncand <= 64) {
      int pos = 0;
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        const bool c = (k[e] >> (32 - SEL_HI)) == P;
        const uint64_t m = __ballot(c);
        if (c) scratch[pos + __popcll(m & ((1ull << lane) - 1ull))] = k[e];
        pos += __popcll(m);
      }
      __builtin_amdgcn_wave_barrier();
      const uint32_t cv = lane < ncand ? scratch[lane] : 0u;  // 0 never reaches a candidate
      __builtin_amdgcn_wave_barrier();
      for (; bit >= 0; --bit) {
        const uint32_t cand = th | (1u << bit);
        if (above + __popcll(__ballot(cv >= cand)) >= kb) th = cand;
      }
    }
  }
  for (; bit >= 0; --bit) {
    const uint32_t cand = th | (1u << bit);
    if (count_ge(cand) >= kb) th = cand;
  }
  int need = kb;  // ties at th still to take, lowest index first
  int pos = 0;
  auto emit = [&](int e, uint32_t key) {
    const int j = e * 64 + lane;
    const uint64_t bgt = __ballot(key > th);
    uint64_t beq = __ballot(key == th);
    uint64_t take = 0ull;
    if (need > 0) {
      if (__popcll(beq) <= need) {
        take = beq;
      } else {
        for (int q = 0; q < need; ++q) {
          take |= beq & (~beq + 1ull);
          beq &= beq - 1ull;
        }
      }
      need -= __popcll(take);
    }
    const uint64_t sel = bgt | take;
    if (lane == 0) {
      mrow[e] = sel;
      if (mcol) mcol[(size_t)e * T] = sel;
    }
    if ((sel >> lane) & 1ull) krow[pos + __popcll(sel & ((1ull << lane) - 1ull))] = j;
    pos += __popcll(sel);
  };
  if constexpr (EM > 0) {
#pragma unroll
    for (int e = 0; e < EM; ++e) need -= __popcll(__ballot(k[e] > th));
#pragma unroll
    for (int e = 0; e < EM; ++e)
      if (e < E) emit(e, k[e]);
  } else {
    for (int e = 0; e < E; ++e) need -= __popcll(__ballot(row_key(srow, T, e, lane) > th));
    for (int e = 0; e < E; ++e) emit(e, row_key(srow, T, e, lane));
  }
}

// mrow: the row's W64 words; mcol (may be null): word e goes to mcol[e * T];
// scratch: 64 words of LDS owned by the wave
template <int EM>
__device__ __forceinline__ void select_row(const float *srow, int T, int kb, uint64_t *mrow,
                                           uint64_t *mcol, int32_t *krow, uint32_t *scratch,
                                           int lane) {
  if (kb <= 0) {
    const int E = (T + 63) >> 6;
    for (int e = lane; e < E; e += 64) {
      mrow[e] = 0ull;
      if (mcol) mcol[(size_t)e * T] = 0ull;
    }
    return;
  }
  select_row_t<EM>(srow, T, kb, mrow, mcol, krow, scratch, lane);
}

// Scores S[bh][i][j] = qbar_i . (kbar_j - mu): one workgroup per (head, 64
// query blocks, 256 key blocks); thread (tr, tk) of an 8 x 32 grid owns rows
// 8 tr .. +7 and keys 4 tk .. +3 and 128 + 4 tk .. +3 (64 accumulators; a
// wave's key reads and score stores are contiguous).  Channels are staged
// through LDS 32 at a time, channel-major (qT[c][row], kT[c][key], with
// kbar - mu formed in float32 as it is staged), so each step of 4 channels
// takes 16 conflict-free 16-byte LDS reads for 256 FMAs.  Every score is one
// FMA chain over the channels in order from +0.
constexpr int SC_ROWS = 64;   // query blocks per workgroup
constexpr int SC_KEYS = 256;  // key blocks per workgroup
constexpr int SC_CH = 32;     // channels per LDS stage

template <int D>
__global__ __launch_bounds__(256) void k_scores(const float *__restrict__ qbar,
                                                const float *__restrict__ kbar,
                                                const float *__restrict__ mu, int T,
                                                float *__restrict__ S) {
  __shared__ __attribute__((aligned(16))) float qT[SC_CH][SC_ROWS];
  __shared__ __attribute__((aligned(16))) float kT[SC_CH][SC_KEYS];
  const int kc = (T + SC_KEYS - 1) / SC_KEYS, rg = (T + SC_ROWS - 1) / SC_ROWS;
  int b = blockIdx.x;
  const int jc = b % kc;
  b /= kc;
  const int ig = b % rg, bh = b / rg;
  const int i0 = ig * SC_ROWS, j0 = jc * SC_KEYS;
  const int tid = threadIdx.x, tr = tid >> 5, tk = tid & 31;
  const float *qh = qbar + (size_t)bh * T * D;
  const float *kh = kbar + (size_t)bh * T * D;
  const float *mh = mu + (size_t)bh * D;
  // staging: thread t loads channels c4 .. c4+3 of key j0 + t (8 float4
  // pieces per stage: 4 channel groups x 2) and of row i0 + t % 64 (2 pieces)
  const int kj = min(j0 + tid, T - 1);
  const int qi = min(i0 + (tid & 63), T - 1);
  float acc[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[r][k] = 0.0f;
  for (int c0 = 0; c0 < D; c0 += SC_CH) {
    float4 kv[SC_CH / 4], qv[SC_CH / 16];
#pragma unroll
    for (int x = 0; x < SC_CH / 4; ++x) kv[x] = *(const float4 *)(kh + (size_t)kj * D + c0 + 4 * x);
#pragma unroll
    for (int x = 0; x < SC_CH / 16; ++x)
      qv[x] = *(const float4 *)(qh + (size_t)qi * D + c0 + 4 * ((tid >> 6) + 4 * x));
    __syncthreads();  // the previous stage's reads are done
#pragma unroll
    for (int x = 0; x < SC_CH / 4; ++x) {
      const int c = 4 * x;
      kT[c + 0][tid] = kv[x].x - mh[c0 + c + 0];
      kT[c + 1][tid] = kv[x].y - mh[c0 + c + 1];
      kT[c + 2][tid] = kv[x].z - mh[c0 + c + 2];
      kT[c + 3][tid] = kv[x].w - mh[c0 + c + 3];
    }
#pragma unroll
    for (int x = 0; x < SC_CH / 16; ++x) {
      const int c = 4 * ((tid >> 6) + 4 * x);
      qT[c + 0][tid & 63] = qv[x].x;
      qT[c + 1][tid & 63] = qv[x].y;
      qT[c + 2][tid & 63] = qv[x].z;
      qT[c + 3][tid & 63] = qv[x].w;
    }
    __syncthreads();
#pragma unroll 4
    for (int c = 0; c < SC_CH; ++c) {
      const float4 q0 = *(const float4 *)&qT[c][8 * tr], q1 = *(const float4 *)&qT[c][8 * tr + 4];
      const float4 k0 = *(const float4 *)&kT[c][4 * tk], k1 = *(const float4 *)&kT[c][128 + 4 * tk];
      const float qa[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      const float ka[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[r][k] = __builtin_fmaf(qa[r], ka[k], acc[r][k]);
    }
  }
  // rows 8 tr + r, keys (two groups of four): a 16-byte store per group when
  // its keys are all inside (T a multiple of 4 keeps it aligned), else one by one
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int i = i0 + 8 * tr + r;
    if (i >= T) break;
    float *srow = S + ((size_t)bh * T + i) * T;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int jj = j0 + 128 * h + 4 * tk;
      if ((T & 3) == 0 && jj + 4 <= T) {
        *(float4 *)(srow + jj) =
            make_float4(acc[r][4 * h], acc[r][4 * h + 1], acc[r][4 * h + 2], acc[r][4 * h + 3]);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (jj + k < T) srow[jj + k] = acc[r][4 * h + k];
      }
    }
  }
}

// Selection: one wave per score row (query block), four rows per workgroup;
// EM = keys per lane held in registers (a multiple of 4 with EM >= ceil(T/64),
// or 0 past 32).
template <int EM>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ S, int T, int nrows,
                                              int kb, int W64, uint64_t *__restrict__ mask,
                                              uint64_t *__restrict__ maskt,
                                              int32_t *__restrict__ kept) {
  __shared__ uint32_t scr[4][64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + w;
  if (row >= nrows) return;  // wave-level sync only below
  const int bh = row / T, i = row - bh * T;
  uint64_t *mcol = maskt ? maskt + (size_t)bh * W64 * T + i : nullptr;
  select_row<EM>(S + (size_t)row * T, T, kb, mask + (size_t)row * W64, mcol,
                 kept + (size_t)row * (kb > 0 ? kb : 1), scr[w], lane);
}

void launch_select(const Plan &p, const WsPtrs &ws, hipStream_t st) {
  const int kc = (p.T + SC_KEYS - 1) / SC_KEYS, rg = (p.T + SC_ROWS - 1) / SC_ROWS;
  dim3 grid((unsigned)((size_t)p.BH * rg * kc)), block(SC_KEYS);
  if (p.d == 128)
    hipLaunchKernelGGL(k_scores<128>, grid, block, 0, st, ws.qbar, ws.kbar, ws.mu, p.T, ws.sc);
  else
    hipLaunchKernelGGL(k_scores<64>, grid, block, 0, st, ws.qbar, ws.kbar, ws.mu, p.T, ws.sc);
  const int nrows = p.BH * p.T;
  dim3 g2((nrows + 3) / 4), b2(256);
  uint64_t *mt = p.lin_on ? ws.maskt : nullptr;
#define SLA_TOPK(EM) \
  hipLaunchKernelGGL(k_topk<EM>, g2, b2, 0, st, ws.sc, p.T, nrows, p.kb, p.W64, ws.mask, mt, ws.kept)
  switch ((p.W64 + 3) >> 2) {  // W64 = ceil(T/64) keys per lane
    case 1: SLA_TOPK(4); break;
    case 2: SLA_TOPK(8); break;
    case 3: SLA_TOPK(12); break;
    case 4: SLA_TOPK(16); break;
    case 5: SLA_TOPK(20); break;
    case 6: SLA_TOPK(24); break;
    case 7: SLA_TOPK(28); break;
    case 8: SLA_TOPK(32); break;
    default: SLA_TOPK(0); break;
  }
#undef SLA_TOPK
}

}  // namespace sla
