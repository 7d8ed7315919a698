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
// Work: T*T*d FMAs per head (plain fp32 ALU) and a 32-step bitwise threshold
// search per row.  One workgroup holds R query-block means and R score rows in
// LDS; each thread keeps one key block's (kbar - mu) in registers and walks the
// R rows, reading qbar as LDS broadcasts.
#include "sla_internal.h"

namespace sla {

// Monotone map of a finite float32 to uint32 (larger float -> larger key);
// +0 and -0 map to the same key.  Never 0 for a finite float.
__device__ __forceinline__ uint32_t score_key(float v) {
  uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave selects one row: mask words (W64 of them) and the ascending kept
// list (kb entries).  Lane l holds the keys of j = 64e + l, e < E.  CACHED:
// the keys are in registers (E <= SEL_MAXE); otherwise every pass re-reads them
// from LDS.
constexpr int SEL_MAXE = 32;
constexpr int SEL_HI = 12;  // key bits decided over all keys before the candidates are packed

template <bool CACHED>
struct RowKeys {
  uint32_t k[CACHED ? SEL_MAXE : 1];
  const float *srow;
  int T, lane;
  __device__ __forceinline__ uint32_t load(int e) const {
    const int j = e * 64 + lane;
    return j < T ? score_key(srow[j]) : 0u;  // 0 never equals a real key
  }
  __device__ __forceinline__ uint32_t get(int e) const {
    if constexpr (CACHED) return k[e];
    else return load(e);
  }
};

template <bool CACHED>
__device__ void select_row_t(const float *srow, int T, int kb, uint64_t *mrow, uint64_t *mcol,
                             int32_t *krow, uint32_t *scratch, int lane) {
  constexpr int EMAX = CACHED ? SEL_MAXE : (1 << 30);
  const int E = (T + 63) >> 6;
  RowKeys<CACHED> rk;
  rk.srow = srow;
  rk.T = T;
  rk.lane = lane;
  if constexpr (CACHED) {
#pragma unroll
    for (int e = 0; e < SEL_MAXE; ++e) rk.k[e] = e < E ? rk.load(e) : 0u;
  }
  // th = the kb-th largest key: the largest th with #{key >= th} >= kb,
  // built one bit at a time from the top.
  auto count_ge = [&](uint32_t cand) {
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < (CACHED ? SEL_MAXE : 1); ++e) {
      if constexpr (CACHED) {
        if (e < E) cnt += __popcll(__ballot(rk.get(e) >= cand));
      } else {
        for (int x = 0; x < E; ++x) cnt += __popcll(__ballot(rk.get(x) >= cand));
      }
    }
    return cnt;
  };
  uint32_t th = 0u;
  int bit = 31;
  if constexpr (CACHED) {
    // The top SEL_HI bits over all keys; then usually few keys share that
    // prefix P: count(key >= cand) = #(prefix > P) + #(prefix == P, key >=
    // cand), and the candidates fit one register per lane (packed through
    // the wave's LDS scratch), so the low bits cost one ballot per step.
    for (; bit >= 32 - SEL_HI; --bit) {
      const uint32_t cand = th | (1u << bit);
      if (count_ge(cand) >= kb) th = cand;
    }
    const uint32_t P = th >> (32 - SEL_HI);
    const int above = (P == (1u << SEL_HI) - 1u) ? 0 : count_ge((P + 1u) << (32 - SEL_HI));
    int ncand = 0;
#pragma unroll
    for (int e = 0; e < SEL_MAXE; ++e)
      if (e < E) ncand += __popcll(__ballot((rk.get(e) >> (32 - SEL_HI)) == P));
    if (ncand <= 64) {
      int pos = 0;
#pragma unroll
      for (int e = 0; e < SEL_MAXE; ++e) {
        if (e < E) {
          const bool c = (rk.get(e) >> (32 - SEL_HI)) == P;
          const uint64_t m = __ballot(c);
          if (c) scratch[pos + __popcll(m & ((1ull << lane) - 1ull))] = rk.get(e);
          pos += __popcll(m);
        }
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
  if constexpr (CACHED) {
#pragma unroll
    for (int e = 0; e < SEL_MAXE; ++e)
      if (e < E) need -= __popcll(__ballot(rk.get(e) > th));
#pragma unroll
    for (int e = 0; e < SEL_MAXE; ++e)
      if (e < E) emit(e, rk.get(e));
  } else {
    for (int e = 0; e < E; ++e) need -= __popcll(__ballot(rk.get(e) > th));
    for (int e = 0; e < E; ++e) emit(e, rk.get(e));
  }
  (void)EMAX;
}

// mrow: the row's W64 words; mcol (may be null): word e goes to mcol[e * T];
// scratch: 64 words of LDS owned by the wave
__device__ void select_row(const float *srow, int T, int kb, uint64_t *mrow, uint64_t *mcol,
                           int32_t *krow, uint32_t *scratch, int lane) {
  const int E = (T + 63) >> 6;
  if (kb <= 0) {
    for (int e = lane; e < E; e += 64) {
      mrow[e] = 0ull;
      if (mcol) mcol[(size_t)e * T] = 0ull;
    }
    return;
  }
  if (E <= SEL_MAXE)
    select_row_t<true>(srow, T, kb, mrow, mcol, krow, scratch, lane);
  else
    select_row_t<false>(srow, T, kb, mrow, mcol, krow, scratch, lane);
}

template <int D>
__global__ __launch_bounds__(256) void k_scores_topk(const float *__restrict__ qbar,
                                                     const float *__restrict__ kbar,
                                                     const float *__restrict__ mu, int T, int R,
                                                     int kb, int W64,
                                                     uint64_t *__restrict__ mask,
                                                     uint64_t *__restrict__ maskt,
                                                     int32_t *__restrict__ kept) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  float *sq = smem;          // [R][D]
  float *ss = smem + R * D;  // [R][T]
  uint32_t *scr = (uint32_t *)(ss + R * T);  // [4 waves][64]
  const int groups = (T + R - 1) / R;
  const int bh = blockIdx.x / groups;
  const int i0 = (blockIdx.x - bh * groups) * R;
  const int nr = min(R, T - i0);
  const int tid = threadIdx.x;
  for (int x = tid; x < nr * D; x += 256) sq[x] = qbar[((size_t)bh * T + i0) * D + x];
  __syncthreads();
  for (int jb = 0; jb < T; jb += 256) {
    const int j = jb + tid;
    if (j < T) {
      float kt[D];
      const float4 *kp = (const float4 *)(kbar + ((size_t)bh * T + j) * D);
      const float4 *mp = (const float4 *)(mu + (size_t)bh * D);
#pragma unroll
      for (int c = 0; c < D / 4; ++c) {
        float4 a = kp[c], m = mp[c];
        kt[4 * c + 0] = a.x - m.x;
        kt[4 * c + 1] = a.y - m.y;
        kt[4 * c + 2] = a.z - m.z;
        kt[4 * c + 3] = a.w - m.w;
      }
      // four rows at a time: four independent FMA chains, each in channel order
      int r = 0;
      for (; r + 4 <= nr; r += 4) {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < D / 4; ++c) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float4 q = ((const float4 *)(sq + (r + u) * D))[c];
            acc[u] = __builtin_fmaf(q.x, kt[4 * c + 0], acc[u]);
            acc[u] = __builtin_fmaf(q.y, kt[4 * c + 1], acc[u]);
            acc[u] = __builtin_fmaf(q.z, kt[4 * c + 2], acc[u]);
            acc[u] = __builtin_fmaf(q.w, kt[4 * c + 3], acc[u]);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) ss[(r + u) * T + j] = acc[u];
      }
      for (; r < nr; ++r) {
        const float4 *qr = (const float4 *)(sq + r * D);
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < D / 4; ++c) {
          const float4 q = qr[c];
          acc = __builtin_fmaf(q.x, kt[4 * c + 0], acc);
          acc = __builtin_fmaf(q.y, kt[4 * c + 1], acc);
          acc = __builtin_fmaf(q.z, kt[4 * c + 2], acc);
          acc = __builtin_fmaf(q.w, kt[4 * c + 3], acc);
        }
        ss[r * T + j] = acc;
      }
    }
  }
  __syncthreads();
  const int w = tid >> 6, lane = tid & 63;
  for (int r = w; r < nr; r += 4) {
    const size_t row = (size_t)bh * T + i0 + r;
    uint64_t *mcol = maskt ? maskt + (size_t)bh * W64 * T + i0 + r : nullptr;
    select_row(ss + r * T, T, kb, mask + row * W64, mcol, kept + row * (size_t)(kb > 0 ? kb : 1),
               scr + 64 * w, lane);
  }
}

void launch_select(const Plan &p, const WsPtrs &ws, hipStream_t st) {
  const int R = p.rows_sel;
  const int groups = (p.T + R - 1) / R;
  const size_t lds = sizeof(float) * (size_t)R * (p.d + p.T) + 4 * 64 * sizeof(uint32_t);
  dim3 grid(p.BH * groups), block(256);
  if (p.d == 128)
    hipLaunchKernelGGL(k_scores_topk<128>, grid, block, lds, st, ws.qbar, ws.kbar, ws.mu, p.T, R,
                       p.kb, p.W64, ws.mask, p.lin_on ? ws.maskt : nullptr, ws.kept);
  else
    hipLaunchKernelGGL(k_scores_topk<64>, grid, block, lds, st, ws.qbar, ws.kbar, ws.mu, p.T, R,
                       p.kb, p.W64, ws.mask, p.lin_on ? ws.maskt : nullptr, ws.kept);
}

}  // namespace sla
