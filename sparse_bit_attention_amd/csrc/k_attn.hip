// Block-sparse SageAttention with the SLA linear branch in the epilogue.
//
// Pages: "揭秘TurboDiffusion…" sections "支柱一：低比特注意力加速 – SageAttention"
// (INT8 QK^T on the matrix units, outlier smoothing) and "支柱二：稀疏线性注意力 –
// SLA" (exact attention only on the kept block interactions, a linear
// component for the rest; sparse and low-bit computation stack as SageSLA);
// "TurboDiffusion跨模态…" sections "SageAttention2++" and "SLA稀疏线性注意力".
//
// One wave owns one 64-row query block and walks its kept key blocks in
// ascending order:
//   S^T = K8_j Q8_i^T          v_mfma_i32_16x16x64_i8 (exact int32)
//   p   = exp2(S * dq_i dk_j sm_scale log2(e) - m)   online softmax, bf16 P
//   O^T += V_j^T P^T           v_mfma_f32_16x16x32_bf16
// The S^T accumulator puts one query and 16 keys in each lane, so the row max
// is a register reduction plus two cross-lane steps, and a lane's
// probabilities are already the B operand of the PV product (the V fragments
// are stored in the matching key order).  The running max is only moved when
// a tile's max exceeds it by more than 2^8, so rescaling O is rare; the final
// O / l is unchanged by this.
// Epilogue: O_l^T = H_i^T phi(Q_i)^T / (phi(Q_i) . z_i), then
// O^T += W O_l^T, all bf16 MFMA into the same accumulators, bf16 store.
//
// MFMA work per kept pair (d = 128): 2*64*64*128 int8 ops + as many bf16
// flops; K8 (8 KiB) and V (16 KiB) fragments are loaded straight into
// registers with 16-byte lane loads (fragment order in memory), prefetched one
// key block ahead.
#include "sla_internal.h"

namespace sla {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_SLACK = 8.0f;  // log2 units

template <int D>
__device__ __forceinline__ void load_q8(const int8_t *q8blk, v4i (&qf)[4][D / 64], int lane) {
  const v4i *p = (const v4i *)q8blk;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int kc = 0; kc < D / 64; ++kc) qf[u][kc] = p[(u * (D / 64) + kc) * 64 + lane];
}

// S^T tile (key tile t, query tile u) = sum over channel chunks of K8 x Q8.
// Accumulator lane l, register r: key 16t + 4(l/16) + r, query 16u + l%16.
template <int D>
__device__ __forceinline__ void qk_int8(const v4i (&kf)[4][D / 64], const v4i (&qf)[4][D / 64],
                                        v4i (&s)[4][4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v4i a = {0, 0, 0, 0};
#pragma unroll
      for (int kc = 0; kc < D / 64; ++kc) a = mfma_i8(kf[t][kc], qf[u][kc], a);
      s[t][u] = a;
    }
}

template <int D, bool LIN>
__global__ __launch_bounds__(256, 1) void k_attn(
    const int8_t *__restrict__ q8, const int8_t *__restrict__ k8, const float *__restrict__ dq,
    const float *__restrict__ dk, const uint16_t *__restrict__ vt,
    const int32_t *__restrict__ kept, const uint16_t *__restrict__ Q,
    const uint16_t *__restrict__ hi, const uint16_t *__restrict__ wsw, uint16_t *__restrict__ out,
    int N, int T, int kb, int nqb, int F, float qk_scale) {
  constexpr int KC = D / 64, CG = D / 16, KC32 = D / 32;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int qb = xcd_remap(blockIdx.x, gridDim.x) * 4 + w;
  if (qb >= nqb) return;
  const int bh = qb / T, i = qb - bh * T;
  const int g = lane >> 4, l16 = lane & 15;
  const int nlast = N - (T - 1) * BLK;

  v4i qf[4][KC];
  load_q8<D>(q8 + (size_t)qb * BLK * D, qf, lane);
  const float dqi = dq[qb] * qk_scale;

  v4f o[CG][4];
#pragma unroll
  for (int a = 0; a < CG; ++a)
#pragma unroll
    for (int u = 0; u < 4; ++u) o[a][u] = v4f{0.f, 0.f, 0.f, 0.f};
  float m[4], lsum[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    m[u] = -INFINITY;
    lsum[u] = 0.f;
  }

  const int32_t *kl = kept + (size_t)qb * kb;
  const size_t headblk = (size_t)bh * T;

  // K8 of the next key block is fetched right after this block's QK^T, V of
  // the next block right after this block's PV product.
  v4i kf[4][KC];
  v4u vf[2][CG];
  auto load_k = [&](int j) {
    const v4i *kp = (const v4i *)(k8 + (headblk + j) * BLK * D);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) kf[t][kc] = kp[(t * KC + kc) * 64 + lane];
  };
  auto load_v = [&](int j) {
    const v4u *vp = (const v4u *)(vt + (headblk + j) * BLK * D);
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2)
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) vf[kc2][cg] = vp[(kc2 * CG + cg) * 64 + lane];
  };

  int jn = kb > 0 ? kl[0] : 0;
  if (kb > 0) {
    load_k(jn);
    load_v(jn);
  }
  for (int n = 0; n < kb; ++n) {
    const int j = jn;
    const float c = dqi * dk[headblk + j];
    v4i s[4][4];
    qk_int8<D>(kf, qf, s);
    if (n + 1 < kb) {
      jn = kl[n + 1];
      load_k(jn);
    }
    // keys past N in the last block are excluded
    const bool tail = (j == T - 1) && (nlast < BLK);
    int imax[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int mx = INT_MIN;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 16 * t + 4 * g + r;
          const int v = (!tail || key < nlast) ? s[t][u][r] : INT_MIN;
          mx = max(mx, v);
        }
      imax[u] = mx;
    }
    // lazy running max: move it only when a tile exceeds it by the slack
    bool need = false;
#pragma unroll
    for (int u = 0; u < 4; ++u) need |= ((float)imax[u] * c > m[u] + RESCALE_SLACK);
    if (__ballot(need) != 0ull) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float tm = (float)imax[u] * c;
        tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
        tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
        if (tm > m[u] + RESCALE_SLACK) {
          const float alpha = __builtin_amdgcn_exp2f(m[u] - tm);
          m[u] = tm;
          lsum[u] *= alpha;
#pragma unroll
          for (int a = 0; a < CG; ++a) o[a][u] *= alpha;
        }
      }
    }
    // probabilities -> bf16 B fragments (k order of kmaj_off), row sums
    v4u pf[2][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float nm = -m[u];
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = 2 * kc2 + (e >> 2), r = e & 3;
          float x = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[t][u][r], c, nm));
          if (tail && (16 * t + 4 * g + r) >= nlast) x = 0.f;
          p[e] = x;
        }
        // The pairs stay in scalars: bit-casting an element of an ext-vector
        // is miscompiled by this clang (every element reads element 0).
        uint32_t pk[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) pk[h] = pack2bf(p[2 * h], p[2 * h + 1]);
        pf[kc2][u] = v4u{pk[0], pk[1], pk[2], pk[3]};
        const v2bf one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int h = 0; h < 4; ++h)
          lsum[u] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, pk[h]), one, lsum[u], false);
      }
    }
#pragma unroll
    for (int a = 0; a < CG; ++a)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int kc2 = 0; kc2 < 2; ++kc2) o[a][u] = mfma_bf16(vf[kc2][a], pf[kc2][u], o[a][u]);
    if (n + 1 < kb) load_v(jn);
  }
  // normalise the sparse branch
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float l = lsum[u];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int a = 0; a < CG; ++a) o[a][u] *= inv;
  }

  if (LIN) {
    // phi(Q) fragments: lane (query 16u + l16, group g) holds channels
    // 32kc + 8g .. +7 of its row; softmax over the row's d channels.
    v4u pq[4][KC32];
    float den[4];
    const uint16_t *hp = hi + (size_t)qb * F;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = i * BLK + 16 * u + l16;
      const bool ok = row < N;
      float x[KC32][8];
      const uint16_t *qr = Q + ((size_t)bh * N + (ok ? row : 0)) * D;
#pragma unroll
      for (int kc = 0; kc < KC32; ++kc) {
        uint4 v = *(const uint4 *)(qr + 32 * kc + 8 * g);
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[kc][e] = bf2f((uint16_t)(vv[e >> 1] >> (16 * (e & 1))));
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kc = 0; kc < KC32; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, x[kc][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float sum = 0.f;
#pragma unroll
      for (int kc = 0; kc < KC32; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[kc][e] = __builtin_amdgcn_exp2f((x[kc][e] - mx) * LOG2E);
          sum += x[kc][e];
        }
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
      const float rs = 1.0f / sum;
      float dd = 0.f;
#pragma unroll
      for (int kc = 0; kc < KC32; ++kc) {
        uint4 zv = *(const uint4 *)(hp + D * D + 32 * kc + 8 * g);
        const uint32_t zz[4] = {zv.x, zv.y, zv.z, zv.w};
        v4u f;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          f[h] = pack2bf(x[kc][2 * h] * rs, x[kc][2 * h + 1] * rs);
          dd = __builtin_fmaf(bf2f((uint16_t)(f[h] & 0xFFFF)), bf2f((uint16_t)(zz[h] & 0xFFFF)), dd);
          dd = __builtin_fmaf(bf2f((uint16_t)(f[h] >> 16)), bf2f((uint16_t)(zz[h] >> 16)), dd);
        }
        pq[u][kc] = f;
      }
      dd += __shfl_xor(dd, 16, 64);
      dd += __shfl_xor(dd, 32, 64);
      den[u] = dd;
    }
    // O_l^T = H^T phi(Q)^T
    v4f ol[CG][4];
#pragma unroll
    for (int x = 0; x < CG; ++x) {
      v4u hf[KC32];
#pragma unroll
      for (int kc = 0; kc < KC32; ++kc)
        hf[kc] = *(const v4u *)(hp + ((size_t)(x * KC32 + kc) * 64 + lane) * 8);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v4f a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC32; ++kc) a = mfma_bf16(hf[kc], pq[u][kc], a);
        ol[x][u] = a;
      }
    }
    // normalise, pack as B fragments (k = value channel, kmaj order) and
    // project: O^T += W O_l^T
    v4u ob[KC32][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float r = den[u] > 0.f ? 1.0f / den[u] : 0.f;
#pragma unroll
      for (int kc = 0; kc < KC32; ++kc) {
        v4u f;
        f[0] = pack2bf(ol[2 * kc][u][0] * r, ol[2 * kc][u][1] * r);
        f[1] = pack2bf(ol[2 * kc][u][2] * r, ol[2 * kc][u][3] * r);
        f[2] = pack2bf(ol[2 * kc + 1][u][0] * r, ol[2 * kc + 1][u][1] * r);
        f[3] = pack2bf(ol[2 * kc + 1][u][2] * r, ol[2 * kc + 1][u][3] * r);
        ob[kc][u] = f;
      }
    }
#pragma unroll
    for (int y = 0; y < CG; ++y) {
      v4u wf[KC32];
#pragma unroll
      for (int kc = 0; kc < KC32; ++kc)
        wf[kc] = *(const v4u *)(wsw + ((size_t)(y * KC32 + kc) * 64 + lane) * 8);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int kc = 0; kc < KC32; ++kc) o[y][u] = mfma_bf16(wf[kc], ob[kc][u], o[y][u]);
    }
  }

  // store: lane holds query 16u + l16, channels 16a + 4g .. +3
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = i * BLK + 16 * u + l16;
    if (row < N) {
      uint16_t *orow = out + ((size_t)bh * N + row) * D;
#pragma unroll
      for (int a = 0; a < CG; ++a) {
        uint2 v = make_uint2(pack2bf(o[a][u][0], o[a][u][1]), pack2bf(o[a][u][2], o[a][u][3]));
        *(uint2 *)(orow + 16 * a + 4 * g) = v;
      }
    }
  }
}

// int32 QK^T of (bh, i, j) triples, one wave per triple; same fragment loads
// and MFMA sequence as k_attn.  Out-of-range triples give zeros.
template <int D>
__global__ __launch_bounds__(64) void k_debug_qk(const int8_t *__restrict__ q8,
                                                 const int8_t *__restrict__ k8, int BH, int T,
                                                 const int32_t *__restrict__ pairs, int n,
                                                 int32_t *__restrict__ out) {
  constexpr int KC = D / 64;
  const int p = blockIdx.x, lane = threadIdx.x;
  const int g = lane >> 4, l16 = lane & 15;
  const int bh = pairs[3 * p], i = pairs[3 * p + 1], j = pairs[3 * p + 2];
  int32_t *o = out + (size_t)p * BLK * BLK;
  if (bh < 0 || bh >= BH || i < 0 || i >= T || j < 0 || j >= T) {
    for (int x = lane; x < BLK * BLK; x += 64) o[x] = 0;
    return;
  }
  v4i qf[4][KC], kf[4][KC], s[4][4];
  load_q8<D>(q8 + ((size_t)bh * T + i) * BLK * D, qf, lane);
  load_q8<D>(k8 + ((size_t)bh * T + j) * BLK * D, kf, lane);
  qk_int8<D>(kf, qf, s);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[(16 * u + l16) * BLK + 16 * t + 4 * g + r] = s[t][u][r];
}

void launch_attn(const Plan &p, const uint16_t *q, const WsPtrs &ws, uint16_t *out, hipStream_t st) {
  const int nqb = p.BH * p.T;
  dim3 grid((nqb + 3) / 4), block(256);
  const float qk_scale = p.sm_scale * LOG2E;
  if (p.d == 128) {
    if (p.lin_on)
      hipLaunchKernelGGL((k_attn<128, true>), grid, block, 0, st, ws.q8, ws.k8, ws.dq, ws.dk, ws.vt,
                         ws.kept, q, ws.hi, ws.wsw, out, p.N, p.T, p.kb, nqb, p.F, qk_scale);
    else
      hipLaunchKernelGGL((k_attn<128, false>), grid, block, 0, st, ws.q8, ws.k8, ws.dq, ws.dk, ws.vt,
                         ws.kept, q, ws.hi, ws.wsw, out, p.N, p.T, p.kb, nqb, p.F, qk_scale);
  } else {
    if (p.lin_on)
      hipLaunchKernelGGL((k_attn<64, true>), grid, block, 0, st, ws.q8, ws.k8, ws.dq, ws.dk, ws.vt,
                         ws.kept, q, ws.hi, ws.wsw, out, p.N, p.T, p.kb, nqb, p.F, qk_scale);
    else
      hipLaunchKernelGGL((k_attn<64, false>), grid, block, 0, st, ws.q8, ws.k8, ws.dq, ws.dk, ws.vt,
                         ws.kept, q, ws.hi, ws.wsw, out, p.N, p.T, p.kb, nqb, p.F, qk_scale);
  }
}

void launch_debug_qk(const Plan &p, const WsPtrs &ws, const int32_t *pairs, int n, int32_t *out,
                     hipStream_t st) {
  if (n <= 0) return;
  if (p.d == 128)
    hipLaunchKernelGGL(k_debug_qk<128>, dim3(n), dim3(64), 0, st, ws.q8, ws.k8, p.BH, p.T, pairs, n, out);
  else
    hipLaunchKernelGGL(k_debug_qk<64>, dim3(n), dim3(64), 0, st, ws.q8, ws.k8, p.BH, p.T, pairs, n, out);
}

}  // namespace sla
