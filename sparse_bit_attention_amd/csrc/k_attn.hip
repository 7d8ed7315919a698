// Block-sparse SageAttention with the SLA linear branch in the epilogue.
//
// Pages: "揭秘TurboDiffusion…" sections "支柱一：低比特注意力加速 – SageAttention"
// (INT8 QK^T on the matrix units, outlier smoothing) and "支柱二：稀疏线性注意力 –
// SLA" (exact attention only on the kept block interactions, a linear
// component for the rest; sparse and low-bit computation stack as SageSLA);
// the aiho.net news report (量子位, 2025-12-26) sections
// "1. SageAttention2++" and "2. SLA稀疏线性注意力".
//
// One wave owns one 64-row query block and walks its kept key blocks in
// ascending order:
//   S^T = K_j Q_i^T       v_mfma_i32_16x16x64_i8 on the INT8 codes (exact
//                         int32), or v_mfma_f32_16x16x32_bf16 on bf16 Q and K
//                         (plain SLA, QK8 = false)
//   p   = exp2(S * c_ij - m)   c_ij = dq_i dk_j sm_scale log2(e) (INT8) or
//                              sm_scale log2(e) (bf16); P cut to bf16
//   O^T += V_j^T P^T      v_mfma_f32_16x16x32_bf16
// The S^T accumulator puts one query and 16 keys in each lane, so a lane's
// probabilities are already the B operand of the PV product (the V fragments
// are stored in the matching key order).  m is a per-row upper bound of the
// logits (Cauchy-Schwarz on the operands; bf16: of the logits minus
// c (q . mu), that constant added to the row's offset, with the key norms
// taken around the K mean), so no running max is kept; query
// blocks whose bound is too loose go to a second launch (INT8: online max;
// bf16: the rows' exact maxima first).  Row sums come from the matrix core
// (a ones operand, zero at the padding keys of a head's ragged last block).
// Epilogue: O_l^T = H_i^T phi(Q_i)^T / (phi(Q_i) . z_i), then
// O^T += W O_l^T, all bf16 MFMA into the same accumulators, bf16 store.
//
// Operands stream from HBM/L2 straight into registers in MFMA fragment order
// (no LDS), through register rings several 16-key tiles ahead.
//
// MFMA work per kept pair (d = 128): 2*64*64*128 int8 ops (or bf16 flops for
// QK^T in bf16) + 2*64*64*128 bf16 flops for PV.
#include "sla_internal.h"

namespace sla {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_SLACK = 8.0f;  // log2 units
// Largest per-row logit bound m (log2 units) the bound path accepts.  The
// Cauchy-Schwarz bound holds on both sides, -m <= logit <= m, so every
// probability exp2(logit - m) is at least 2^(-2m): with m <= 48 that is 2^-96,
// which keeps each probability, the row sum and every P*V product far inside
// the float32 normal range (2^-126) even when all of a row's kept logits sit
// near -m.  Rows with a larger bound go to the second launch.
constexpr float BOUND_LIMIT = 48.0f;

template <int D>
__device__ __forceinline__ void load_q8(const int8_t *q8blk, v4i (&qf)[4][D / 64], int lane) {
  const v4i *p = (const v4i *)q8blk;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int kc = 0; kc < D / 64; ++kc) qf[u][kc] = p[(u * (D / 64) + kc) * 64 + lane];
}

// One key block's operands, straight from HBM in register layout: the K8
// fragments (A operands of S^T) and the V^T fragments of both 32-key halves
// (A operands of O^T).
template <int D>
struct KVBlock {
  v4i k[4][D / 64];
  v4u v[2][D / 16];
};

template <int D>
__device__ __forceinline__ void load_kv(KVBlock<D> &x, const uint4 *k8u, const uint4 *vtu,
                                        size_t blk, int lane) {
  constexpr int KC = D / 64, CG = D / 16;
  const uint4 *kp = k8u + blk * (4 * KC * 64) + lane;
  const uint4 *vp = vtu + blk * (2 * CG * 64) + lane;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) x.k[t][kc] = __builtin_bit_cast(v4i, kp[(t * KC + kc) * 64]);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int a = 0; a < CG; ++a) x.v[hf][a] = __builtin_bit_cast(v4u, vp[(hf * CG + a) * 64]);
}

// The QK^T accumulators of the bound path start at the bit pattern of
// 1.5 * 2^23: with |score| < 2^22 the int32 sum then reads as the float
// 12582912 + score, so no int -> float conversion is needed; the constant is
// folded into the FMA.  Rounding that folded constant shifts a key block's
// logits by at most 0.75 c (log2 units), so this path is only taken when
// c <= 2^-10 for every kept block of the row.
constexpr int SCORE_BIAS_BITS = 0x4B400000;
constexpr float SCORE_BIAS = 12582912.0f;
constexpr float BIAS_C_LIMIT = 0x1p-10f;

// Probabilities of one 32-key half for query tile U as a bf16 B fragment (k
// order of kmaj_off) and their sum: p = exp2(score * c - m), c = c0 for the
// half's first key tile, c1 for its second.
template <int U, bool BIASED>
__device__ __forceinline__ v4u probs_half(const v4i (&s)[2][4], float c0, float c1, float m,
                                          float &lsum) {
  const v2bf one = {(__bf16)1.0f, (__bf16)1.0f};
  // The pairs stay in scalars: bit-casting an element of an ext-vector is
  // miscompiled by this clang (every element reads element 0).
  uint32_t pk[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int e0 = 2 * h, e1 = 2 * h + 1;
    const int a0 = s[e0 >> 2][U][e0 & 3], a1 = s[e1 >> 2][U][e1 & 3];
    const float f0 = BIASED ? __int_as_float(a0) : (float)a0;
    const float f1 = BIASED ? __int_as_float(a1) : (float)a1;
    const float c = h < 2 ? c0 : c1;  // elements 0..3: first tile, 4..7: second
    const float nm = BIASED ? -__builtin_fmaf(SCORE_BIAS, c, m) : -m;
    const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(f0, c, nm));
    const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(f1, c, nm));
    pk[h] = pack2bf(x0, x1);
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, pk[h]), one, lsum, false);
  }
  return v4u{pk[0], pk[1], pk[2], pk[3]};
}

// One kept key block, in two 32-key halves (QK^T half -> probabilities -> PV
// half).  BOUND: m is an upper bound of every logit of the row (set before the
// loop): no running max, no rescaling.  Otherwise m is a running max, moved
// lazily per half.  The logit scale of query tile u and key tile t (this
// lane's keys of it) is cq[u] * ck[t].
template <int D, bool BOUND>
__device__ __forceinline__ void attend_block(const KVBlock<D> &x, const v4i (&qf)[4][D / 64],
                                             v4f (&o)[D / 16][4], float (&m)[4],
                                             float (&lsum)[4], const float (&cq)[4],
                                             const float (&ck)[4], bool last, int npad_lane) {
  constexpr int KC = D / 64, CG = D / 16;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    // S^T for key tiles 2hf, 2hf+1
    v4i s[2][4];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int init = BOUND ? SCORE_BIAS_BITS : 0;
        v4i acc = {init, init, init, init};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) acc = mfma_i8(x.k[2 * hf + t2][kc], qf[u][kc], acc);
        s[t2][u] = acc;
      }
    if (!BOUND) {
      // half-tile max logit per query (padding keys score 0 and may only raise
      // it); the scales are positive, so each tile's max logit is at its max
      // score
      float lmax[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int a0 = max(max(s[0][u][0], s[0][u][1]), max(s[0][u][2], s[0][u][3]));
        const int a1 = max(max(s[1][u][0], s[1][u][1]), max(s[1][u][2], s[1][u][3]));
        lmax[u] = fmaxf((float)a0 * (cq[u] * ck[2 * hf]), (float)a1 * (cq[u] * ck[2 * hf + 1]));
      }
      bool need = false;
#pragma unroll
      for (int u = 0; u < 4; ++u) need |= (lmax[u] > m[u] + RESCALE_SLACK);
      if (__ballot(need) != 0ull) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float tm = lmax[u];
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
    }
    v4u pf[4];
    pf[0] = probs_half<0, BOUND>(s, cq[0] * ck[2 * hf], cq[0] * ck[2 * hf + 1], m[0], lsum[0]);
    pf[1] = probs_half<1, BOUND>(s, cq[1] * ck[2 * hf], cq[1] * ck[2 * hf + 1], m[1], lsum[1]);
    pf[2] = probs_half<2, BOUND>(s, cq[2] * ck[2 * hf], cq[2] * ck[2 * hf + 1], m[2], lsum[2]);
    pf[3] = probs_half<3, BOUND>(s, cq[3] * ck[2 * hf], cq[3] * ck[2 * hf + 1], m[3], lsum[3]);
#pragma unroll
    for (int a = 0; a < CG; ++a)
#pragma unroll
      for (int u = 0; u < 4; ++u) o[a][u] = mfma_bf16(x.v[hf][a], pf[u], o[a][u]);
  }
  if (last && npad_lane > 0) {
    // padding keys have score 0: remove exactly what the row sums received
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // the same arithmetic the probabilities of a zero score went through
      const float c = cq[u] * ck[3];  // the last tile holds every padding key
      const float xz = BOUND ? __builtin_fmaf(SCORE_BIAS, c, -__builtin_fmaf(SCORE_BIAS, c, m[u]))
                             : -m[u];
      const uint32_t pp = pack2bf(__builtin_amdgcn_exp2f(xz), 0.f);
      lsum[u] -= (float)npad_lane * bf2f((uint16_t)(pp & 0xFFFF));
    }
  }
}

// The kept-block loop.  Two register sets alternate: the loads of block n+1
// are issued before block n is computed, so each load has a whole block of
// work to land, and no operand passes through LDS.
// dqi[u]: dq of query tile u times sm_scale log2(e); FINE: dk holds 16 scales
// per key block (one per 4 keys), this lane's keys of tile t use scale 4t + g.
template <int D, bool BOUND, bool FINE>
__device__ __forceinline__ void kept_loop(const v4i (&qf)[4][D / 64], v4f (&o)[D / 16][4],
                                          float (&m)[4], float (&lsum)[4], const int32_t *kl,
                                          int kb, const float *dk, const uint4 *k8u,
                                          const uint4 *vtu, size_t headblk, const float (&dqi)[4],
                                          int T, int npad_lane, int lane) {
  if (kb <= 0) return;
  auto kscales = [&](int j, float (&ck)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      ck[t] = FINE ? dk[(headblk + j) * 16 + 4 * t + (lane >> 4)] : dk[headblk + j];
  };
  float cka[4], ckb[4];
  KVBlock<D> xa, xb;
  load_kv<D>(xa, k8u, vtu, headblk + kl[0], lane);
  int n = 0;
  for (; n + 1 < kb; n += 2) {
    const int ja = kl[n], jb = kl[n + 1];
    // the scheduling fences keep each block's loads ahead of the other
    // block's arithmetic
    __builtin_amdgcn_sched_barrier(0);
    load_kv<D>(xb, k8u, vtu, headblk + jb, lane);
    __builtin_amdgcn_sched_barrier(0);
    kscales(ja, cka);
    attend_block<D, BOUND>(xa, qf, o, m, lsum, dqi, cka, ja == T - 1, npad_lane);
    __builtin_amdgcn_sched_barrier(0);
    if (n + 2 < kb) load_kv<D>(xa, k8u, vtu, headblk + kl[n + 2], lane);
    __builtin_amdgcn_sched_barrier(0);
    kscales(jb, ckb);
    attend_block<D, BOUND>(xb, qf, o, m, lsum, dqi, ckb, jb == T - 1, npad_lane);
  }
  if (n < kb) {
    const int ja = kl[n];
    kscales(ja, cka);
    attend_block<D, BOUND>(xa, qf, o, m, lsum, dqi, cka, ja == T - 1, npad_lane);
  }
}

// ---------------------------------------------------------------------------
// Software-pipelined loop of the bound path.  The kept blocks are walked as a
// stream of 16-key tiles (sub-stage sigma = 4 n + t: block n, key tile t).
// Sub-stage sigma issues three independent pieces of work, interleaved in a
// fixed order so that vector ALU work runs while the matrix core is busy:
//   QK(sigma+1): S^T of tile sigma+1           (int8 or bf16 MFMA, by QK8)
//   SM(sigma):   probabilities of tile sigma, half a B fragment
//   PV:          O^T += V^T P^T for the 32-key chunk finished two
//                sub-stages earlier, half of the channel tiles (bf16 MFMA)
// Operands come straight from HBM in register layout, through two register
// rings: K tiles KLEAD sub-stages ahead, V quarters (32 keys x D/2 channels)
// VLEAD sub-stages ahead.  Nothing passes through LDS, and since every
// in-flight load is an ordinary register load the compiler's wait counts stay
// exact.  The loop body covers two blocks, which makes every ring index a
// constant.
// ---------------------------------------------------------------------------

// The QK^T operand types: QK8 = INT8 codes (v_mfma_i32_16x16x64_i8, exact
// int32, biased accumulators), otherwise bf16 (v_mfma_f32_16x16x32_bf16,
// float32 accumulators from zero).  NK = MFMAs (k chunks) per score tile.
template <int D, bool QK8>
struct QKOps {
  static constexpr int NK = QK8 ? D / 64 : D / 32;
  using frag = std::conditional_t<QK8, v4i, v4u>;  // K and Q fragments
  using acc = std::conditional_t<QK8, v4i, v4f>;   // S^T accumulator tile
  static __device__ __forceinline__ acc init() {
    if constexpr (QK8) return v4i{SCORE_BIAS_BITS, SCORE_BIAS_BITS, SCORE_BIAS_BITS, SCORE_BIAS_BITS};
    else return v4f{0.f, 0.f, 0.f, 0.f};
  }
  static __device__ __forceinline__ acc mma(const frag &k, const frag &q, const acc &c) {
    if constexpr (QK8) return mfma_i8(k, q, c);
    else return mfma_bf16(k, q, c);
  }
  // Whether the pipelined loop writes its scores with mma_first / mma_next
  // below in their ASM form: d = 128.  At d = 64 the compiler re-materialises
  // the initial-value registers within a few instructions of an asm MFMA
  // reading them, a distance the asm's hidden latency does not allow for.
  static constexpr bool VG = D == 128;
  // ASM: the same products written as inline asm with VGPR operands, so the
  // scores land in VGPRs whatever register class the compiler gives the
  // function's other MFMA results.  With the builtins the whole kernel's
  // MFMAs take the AGPR form (it needs more than 256 registers) and every
  // score the vector ALU reads costs a v_accvgpr_read first: 128 extra
  // instructions per two kept blocks, ~5% of the loop's time.  Every score
  // tile of a loop must be written this way (mixing forms makes the compiler
  // copy results between register classes right after the MFMA).
  // The compiler cannot see the latency of an asm MFMA, so nothing may read
  // its destination within the MFMA's result latency; the fixed slot order
  // of the pipelined loop puts every such read a sub-stage later (dozens of
  // instructions), and a test compiles this file and checks the distances
  // on the generated code.  Accumulating into the same registers (exact
  // srcC overlap) needs no wait.
  // c0: the tile's initial value (init()); in the ASM form a value the
  // compiler cannot re-materialise (see opaque_init), so it stays in one set
  // of registers for the whole loop instead of being rewritten next to the
  // MFMAs that read it.
  template <bool ASM>
  static __device__ __forceinline__ acc mma_first(const frag &k, const frag &q, const acc &c0) {
    if constexpr (ASM) {
      acc r;
      if constexpr (QK8)
        asm("v_mfma_i32_16x16x64_i8 %0, %1, %2, %3" : "=&v"(r) : "v"(k), "v"(q), "v"(c0));
      else
        asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %3" : "=&v"(r) : "v"(k), "v"(q), "v"(c0));
      return r;
    } else {
      return mma(k, q, c0);
    }
  }
  static __device__ __forceinline__ acc opaque_init() {
    acc c = init();
    asm volatile("" : "+v"(c));
    return c;
  }
  template <bool ASM>
  static __device__ __forceinline__ acc mma_next(const frag &k, const frag &q, const acc &c) {
    if constexpr (ASM) {
      acc r = c;
      if constexpr (QK8)
        asm("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+v"(r) : "v"(k), "v"(q));
      else
        asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(r) : "v"(k), "v"(q));
      return r;
    } else {
      return mma(k, q, c);
    }
  }
  // the score as the float the exp2 argument is formed from
  static __device__ __forceinline__ float score(const acc &s, int r) {
    if constexpr (QK8) return __int_as_float(s[r]);
    else return s[r];
  }
  // that float for a zero score, and the exp2 offset for row bound m
  static constexpr float ZERO = QK8 ? SCORE_BIAS : 0.0f;
  static __device__ __forceinline__ float nm(float c, float m) { return -__builtin_fmaf(ZERO, c, m); }
};

template <int D, bool QK8, bool FINE = false>
struct Pipe {
  static constexpr int KC = QKOps<D, QK8>::NK, CG = D / 16;
  static constexpr int KT = KC;          // 1 KiB fragments per K tile (16 keys)
  static constexpr int VQ = CG / 2;      // 1 KiB fragments per V quarter
  // K tile sigma + KLEAD and V quarter sigma + VLEAD are loaded at sub-stage
  // sigma; bf16 Q and K fragments take twice the registers of INT8 ones, so
  // that path keeps shorter rings.  INT8 block scales: K 3 ahead saves a few
  // accumulator copies (1.6% faster than 4).  Fine scales: the per-lane key
  // scales and the VGPR score tiles fit the register file with K 2 and V 3
  // ahead (K 3 / V 3 spills; K 2 / V 2 is 0.8% slower).
  static constexpr int KLEAD = QK8 ? (FINE ? 2 : 3) : 2;
  static constexpr int VLEAD = QK8 ? (FINE ? 3 : 4) : 2;
};

// Probabilities: p = exp2(score * c + nm) cut to bf16 by keeping the upper
// half of each float32, two per register in the k order of kmaj_off.  The row
// sums are taken by the matrix core from the same bf16 values, so the
// rounding of p enters numerator and denominator alike.
// A fragment of 16 rows of bf16 ones: the rows of ones^T P^T are row sums of P.
constexpr uint32_t BF16_ONE_PAIR = 0x3F803F80u;

template <int D, bool QK8>
struct PipeState {
  using Q = QKOps<D, QK8>;
  static constexpr int KC = Q::NK, CG = D / 16, VQ = CG / 2;
  v4f o[CG][4];
  v4f lacc[4];                   // row sums (every element of lacc[u] holds the same sum)
  typename Q::acc s[2][4];       // S^T of the two most recent tiles (by tile parity)
  typename Q::acc s0;            // a score tile's initial value
  v4u pf[2][4];                  // B fragments of the two most recent 32-key chunks
  typename Q::frag kr[8][KC];    // K tiles (by tile index mod 8)
  v4u vr[8][VQ];                 // V quarters (by quarter index mod 8)
};

// Block-level values of one loop iteration (two blocks)
struct PipeBlocks {
  float c[2];         // logit scale of block 2i, 2i+1
  float nm[2][4];     // QKOps::nm(c, m_u); -inf for a block past the kept list
  int last[3];        // block 2i-1, 2i, 2i+1 is the head's last (ragged) block
  // finer INT8 scales: this lane's key scale of each tile of block 2i, 2i+1,
  // the query-tile factors, the row bounds, and which blocks are real
  float ck[2][4], dq[4], m[4];
  int valid[2];
};

// Sub-stage R (0..7) of the loop body; sigma = 8 i + R.
// lm[h]: the ones fragment for half h of the head's last block, zero at its
// padding keys, so the row sums leave those keys out.
// DUMP (INT8 only): also store each score of block 2i (R < 4) as the exact
// int32 q.k sum, accumulator minus SCORE_BIAS_BITS, to dump[64 query][64 key]
// at the slot where the softmax reads it.
template <int D, bool QK8, bool FINE, int R, bool DUMP>
__device__ __forceinline__ void sub_stage(PipeState<D, QK8> &st,
                                          const typename QKOps<D, QK8>::frag (&qf)[4][QKOps<D, QK8>::NK],
                                          const PipeBlocks &pb, const v4u (&lm)[2],
                                          const uint4 *kload_src, const uint4 *vload_src,
                                          int lane, int32_t *dump) {
  static_assert(!DUMP || QK8, "the int32 read-back exists for INT8 scores only");
  using P = Pipe<D, QK8, FINE>;
  using Q = QKOps<D, QK8>;
  constexpr int KC = P::KC, VQ = P::VQ;
  // loads: K tile sigma+KLEAD, V quarter sigma+VLEAD, kept together at the
  // head of the sub-stage
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    st.kr[(R + P::KLEAD) % 8][kc] = __builtin_bit_cast(typename Q::frag, kload_src[kc * 64 + lane]);
#pragma unroll
  for (int a = 0; a < VQ; ++a)
    st.vr[(R + P::VLEAD) % 8][a] = __builtin_bit_cast(v4u, vload_src[a * 64 + lane]);
  __builtin_amdgcn_sched_barrier(0);
  // The sub-stage's MFMAs in a fixed order: QK(sigma+1) (kc outer, so the
  // two products into one score tile are four issues apart), the PV half,
  // then the row sums on even R.  One score of SM(sigma) (fma + exp2) follows
  // each of the first 16 MFMAs, and the byte permutes of a query tile follow
  // its fourth score; a scheduling fence after each slot keeps this order, so
  // the transcendental work is spread one per MFMA instead of clustered.
  // SM(sigma): tile parity R & 1 fills half of chunk sigma/2's B fragment;
  // PV: chunk sigma/2 - 1, channel tiles [VQ (R&1), VQ (R&1) + VQ), V quarter
  // sigma-2.
  constexpr int blk = R / 4;
  constexpr int par = (R / 2) & 1;         // chunk being filled by SM
  constexpr int par2 = ((R / 2) + 1) & 1;  // chunk consumed by PV
  constexpr int vs = (R + 6) % 8;
  constexpr int a0 = (R & 1) * VQ;
  constexpr int NM = 4 * KC + 4 * VQ + ((R & 1) == 0 ? 4 : 0);
  // row sums of chunk sigma/2 - 1 (even R): its block is 2i-1, 2i, 2i or
  // 2i+1 for R = 0, 2, 4, 6, and its half within the block is R/2 + 1 mod 2
  constexpr int cblk = R == 0 ? 0 : (R == 6 ? 2 : 1);
  constexpr int chf = ((R / 2) + 1) & 1;
  const v4u ones = {BF16_ONE_PAIR, BF16_ONE_PAIR, BF16_ONE_PAIR, BF16_ONE_PAIR};
  const v4u rs = pb.last[cblk] ? lm[chf] : ones;
  // logit scale and exp2 offset per query tile: one per block, or (FINE) the
  // query tile's factor times this lane's key-group scale of tile R % 4
  float cu[4], nmu[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if constexpr (FINE) {
      cu[u] = pb.dq[u] * pb.ck[blk][R & 3];
      nmu[u] = pb.valid[blk] ? Q::nm(cu[u], pb.m[u]) : -INFINITY;
    } else {
      cu[u] = pb.c[blk];
      nmu[u] = pb.nm[blk][u];
    }
  }
  // SP (INT8 block scales): the exp2 argument of the next score is formed one
  // slot ahead and a tile's byte permutes run one slot after its last exp2,
  // so no slot's vector work waits on its own previous instruction (1.5%
  // faster there; the fine-scale path measured 1.2% slower and the bf16 path
  // spills, so they keep the plain order).  d = 64 has fewer MFMAs than
  // scores on odd R; SP needs one slot past the 16 scores.
  constexpr bool SP = QK8 && !FINE;
  constexpr int NSLOT = NM > (SP ? 17 : 16) ? NM : (SP ? 17 : 16);
  uint32_t xs[4][4];
  float xn = SP ? __builtin_fmaf(Q::score(st.s[R & 1][0], 0), cu[0], nmu[0]) : 0.f;
#pragma unroll
  for (int i = 0; i < NSLOT; ++i) {
    if (i >= NM) {
      // no MFMA left in this slot
    } else if (i < 4 * KC) {
      const int kc = i / 4, u = i % 4;
      if (kc == 0)
        st.s[(R + 1) & 1][u] =
            Q::template mma_first<Q::VG>(st.kr[(R + 1) % 8][kc], qf[u][kc], st.s0);
      else
        st.s[(R + 1) & 1][u] =
            Q::template mma_next<Q::VG>(st.kr[(R + 1) % 8][kc], qf[u][kc], st.s[(R + 1) & 1][u]);
    } else if (i < 4 * KC + 4 * VQ) {
      const int j = i - 4 * KC, a = j / 4, u = j % 4;
      st.o[a0 + a][u] = mfma_bf16(st.vr[vs][a], st.pf[par2][u], st.o[a0 + a][u]);
    } else {
      const int u = i - 4 * KC - 4 * VQ;
      st.lacc[u] = mfma_bf16(rs, st.pf[par2][u], st.lacc[u]);
    }
    if (i < 16) {
      // p = exp2(score * c + nm), cut to bf16 by keeping the upper half of
      // the float32 (one byte permute per pair)
      const int u = i / 4, r = i % 4;
      float x;
      if constexpr (SP) {
        x = xn;
        if (i + 1 < 16) {
          const int u1 = (i + 1) / 4, r1 = (i + 1) % 4;
          xn = __builtin_fmaf(Q::score(st.s[R & 1][u1], r1), cu[u1], nmu[u1]);
        }
      } else {
        x = __builtin_fmaf(Q::score(st.s[R & 1][u], r), cu[u], nmu[u]);
      }
      xs[u][r] = __float_as_uint(__builtin_amdgcn_exp2f(x));
      if constexpr (DUMP && R < 4)
        dump[(16 * u + (lane & 15)) * BLK + 16 * R + 4 * (lane >> 4) + r] =
            st.s[R & 1][u][r] - SCORE_BIAS_BITS;
    }
    // tile pu's four probabilities are complete: pack them
    const int pu = SP ? (i >= 4 && i <= 16 && i % 4 == 0 ? i / 4 - 1 : -1)
                      : (i < 16 && i % 4 == 3 ? i / 4 : -1);
    if (pu >= 0) {
      const int u = pu;
      {
        // bytes 2,3 of the first value, then bytes 2,3 of the second
        const uint32_t p0 = __builtin_amdgcn_perm(xs[u][1], xs[u][0], 0x07060302u);
        const uint32_t p1 = __builtin_amdgcn_perm(xs[u][3], xs[u][2], 0x07060302u);
        if (R & 1) {
          st.pf[par][u][2] = p0;
          st.pf[par][u][3] = p1;
        } else {
          st.pf[par][u][0] = p0;
          st.pf[par][u][1] = p1;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// K fragments come from k8u (QK8: INT8 codes) or the bf16 copy (bfk_off).
// dqi[u]: the query tile's scale factor (all equal unless FINE); FINE: dk
// holds 16 scales per key block, this lane's keys of tile t use 4t + g.
template <int D, bool QK8, bool FINE, bool DUMP = false>
__device__ __forceinline__ void kept_loop_piped(
    const typename QKOps<D, QK8>::frag (&qf)[4][QKOps<D, QK8>::NK], v4f (&o)[D / 16][4],
    const float (&m)[4], float (&lsum)[4], const int32_t *kl, int kb, const float *dk,
    const uint4 *k8u, const uint4 *vtu, size_t headblk, const float (&dqi)[4], int T, int nlast,
    int lane, int32_t *dump = nullptr) {
  using P = Pipe<D, QK8, FINE>;
  using Q = QKOps<D, QK8>;
  constexpr int KC = P::KC, CG = P::CG, VQ = P::VQ, KT = P::KT;
  constexpr int KFR = 4 * KT, VFR = 4 * VQ;  // fragments per block
  if (kb <= 0) return;
  // global source of K tile x and V quarter x (blocks past the list: the last one)
  auto kblk = [&](int x) { const int n = x >> 2; return kl[n < kb ? n : kb - 1]; };
  auto ksrc = [&](int x) { return k8u + ((headblk + kblk(x)) * KFR + (x & 3) * KT) * 64; };
  auto vsrc = [&](int x) { return vtu + ((headblk + kblk(x)) * VFR + (x & 3) * VQ) * 64; };

  // ones fragments for the two halves of the last block, zero at its padding
  // keys: lane group g, element e holds key 32 h + 16 (e/4) + 4 g + e%4
  v4u lm[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t wv[4];
#pragma unroll
    for (int d2 = 0; d2 < 4; ++d2) {
      uint32_t x = 0u;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int e = 2 * d2 + b;
        const int key = 32 * h + 16 * (e >> 2) + 4 * (lane >> 4) + (e & 3);
        if (key < nlast) x |= 0x3F80u << (16 * b);
      }
      wv[d2] = x;
    }
    lm[h] = v4u{wv[0], wv[1], wv[2], wv[3]};
  }

  PipeState<D, QK8> st;
  st.s0 = Q::VG ? Q::opaque_init() : Q::init();
#pragma unroll
  for (int a = 0; a < CG; ++a)
#pragma unroll
    for (int u = 0; u < 4; ++u) st.o[a][u] = o[a][u];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    st.lacc[u] = v4f{0.f, 0.f, 0.f, 0.f};
    st.pf[1][u] = v4u{0u, 0u, 0u, 0u};  // chunk -1: zero probabilities
  }
  // prologue: K tiles 0 .. KLEAD-1, then V quarters 0 .. VLEAD-1, in this
  // order (fenced): the loop's first sub-stages count on the K tiles being
  // the oldest loads in flight, so their waits leave the later loads pending
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int x = 0; x < P::KLEAD; ++x)
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      st.kr[x][kc] = __builtin_bit_cast(typename Q::frag, ksrc(x)[kc * 64 + lane]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int x = 0; x < P::VLEAD; ++x)
#pragma unroll
    for (int a = 0; a < VQ; ++a) st.vr[x][a] = __builtin_bit_cast(v4u, vsrc(x)[a * 64 + lane]);
  __builtin_amdgcn_sched_barrier(0);
  // quarters -2, -1 meet zero probabilities: make them finite
#pragma unroll
  for (int a = 0; a < VQ; ++a) {
    st.vr[6][a] = v4u{0u, 0u, 0u, 0u};
    st.vr[7][a] = v4u{0u, 0u, 0u, 0u};
  }
  // QK(0)
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    typename Q::acc acc = Q::template mma_first<Q::VG>(st.kr[0][0], qf[u][0], st.s0);
#pragma unroll
    for (int kc = 1; kc < KC; ++kc)
      acc = Q::template mma_next<Q::VG>(st.kr[0][kc], qf[u][kc], acc);
    st.s[0][u] = acc;
  }

  // Per-block scalars run ahead of their use so that no scalar load is waited
  // for inside an iteration: kept entries two iterations ahead, logit scales
  // one iteration ahead.  jb[e] = kept entry of block 2 it + e (e < 4, the
  // last one for blocks past the list), cb[e] = its logit scale (e < 2).
  static_assert(P::KLEAD <= 8 && P::VLEAD <= 8, "load sources reach at most four blocks ahead");
  auto kle = [&](int n) { return kl[n < kb ? n : kb - 1]; };
  int jb[4] = {kle(0), kle(1), kle(2), kle(3)};
  int jprev = -1;  // kept entry of block 2 it - 1
  const int g = lane >> 4;
  // FINE: this lane's key scale of each tile of a block (one per 4 keys)
  auto kscales = [&](int j, float (&ck)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) ck[t] = dk[(headblk + j) * 16 + 4 * t + g];
  };
  float cb[2] = {0.f, 0.f};
  float ckc[2][4];
  if constexpr (FINE) {
    kscales(jb[0], ckc[0]);
    kscales(jb[1], ckc[1]);
  } else {
    cb[0] = dqi[0] * dk[headblk + jb[0]];
    cb[1] = dqi[0] * dk[headblk + jb[1]];
  }
  const int iters = (kb + 1) >> 1;
  for (int it = 0; it < iters; ++it) {
    // issued here, first read at the end of the iteration
    const int jn4 = kle(2 * it + 4), jn5 = kle(2 * it + 5);
    float dk2 = 0.f, dk3 = 0.f, ckn[2][4];
    if constexpr (FINE) {
      kscales(jb[2], ckn[0]);
      kscales(jb[3], ckn[1]);
    } else {
      dk2 = dk[headblk + jb[2]];
      dk3 = dk[headblk + jb[3]];
    }
    PipeBlocks pb;
    if constexpr (FINE) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        pb.dq[u] = dqi[u];
        pb.m[u] = m[u];
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        pb.valid[e] = 2 * it + e < kb;
#pragma unroll
        for (int t = 0; t < 4; ++t) pb.ck[e][t] = ckc[e][t];
      }
    }
    pb.last[0] = jprev == T - 1;
    pb.last[1] = jb[0] == T - 1;
    pb.last[2] = jb[1] == T - 1;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const bool valid = 2 * it + e < kb;
      pb.c[e] = cb[e];
#pragma unroll
      for (int u = 0; u < 4; ++u) pb.nm[e][u] = valid ? Q::nm(cb[e], m[u]) : -INFINITY;
    }
    // K tile / V quarter x = 8 it + R + LEAD lies in block 2 it + (R + LEAD) / 4
#define SLA_SRC(base, FR, PER, R, LEAD) \
    ((base) + ((headblk + jb[((R) + (LEAD)) >> 2]) * (FR) + (((R) + (LEAD)) & 3) * (PER)) * 64)
#define SLA_SUB(R) \
    sub_stage<D, QK8, FINE, R, DUMP>(st, qf, pb, lm, SLA_SRC(k8u, KFR, KT, R, P::KLEAD), SLA_SRC(vtu, VFR, VQ, R, P::VLEAD), lane, dump)
    SLA_SUB(0);
    SLA_SUB(1);
    SLA_SUB(2);
    SLA_SUB(3);
    SLA_SUB(4);
    SLA_SUB(5);
    SLA_SUB(6);
    SLA_SUB(7);
#undef SLA_SUB
#undef SLA_SRC
    jprev = jb[1];
    jb[0] = jb[2];
    jb[1] = jb[3];
    jb[2] = jn4;
    jb[3] = jn5;
    if constexpr (FINE) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        ckc[0][t] = ckn[0][t];
        ckc[1][t] = ckn[1][t];
      }
    } else {
      cb[0] = dqi[0] * dk2;
      cb[1] = dqi[0] * dk3;
    }
  }
  // drain: PV of the last chunk (parity 1, half 1 of block 2 iters - 1) with
  // V quarters in slots 6 and 7
  {
    const v4u ones = {BF16_ONE_PAIR, BF16_ONE_PAIR, BF16_ONE_PAIR, BF16_ONE_PAIR};
    const v4u rs = jprev == T - 1 ? lm[1] : ones;
#pragma unroll
    for (int u = 0; u < 4; ++u) st.lacc[u] = mfma_bf16(rs, st.pf[1][u], st.lacc[u]);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int a = 0; a < VQ; ++a)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        st.o[h * VQ + a][u] = mfma_bf16(st.vr[6 + h][a], st.pf[1][u], st.o[h * VQ + a][u]);
  // complete row sums (every valid key of every kept block; padding keys of
  // the last block met zeros in the row-sum operand, and their V rows are
  // zero, so they add nothing anywhere)
#pragma unroll
  for (int u = 0; u < 4; ++u) lsum[u] = st.lacc[u][0];
#pragma unroll
  for (int a = 0; a < CG; ++a)
#pragma unroll
    for (int u = 0; u < 4; ++u) o[a][u] = st.o[a][u];
}

// bf16 QK^T: Q fragments (B operands of S^T = K Q^T) straight from Q: lane
// (query 16u + l%16, group g) holds channels 32kc + 8g .. +7 of its row.
// Rows past N read row N-1 (their outputs are never stored).
template <int D>
__device__ __forceinline__ void load_qbf(const uint16_t *Qh, int i, int N, v4u (&qf)[4][D / 32],
                                         int lane) {
  const int g = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = min(i * BLK + 16 * u + l16, N - 1);
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc)
      qf[u][kc] = *(const v4u *)(Qh + (size_t)row * D + 32 * kc + 8 * g);
  }
}

// bf16 QK^T, a query block whose bound is too loose: the exact largest logit
// of each row (log2 units, at least 0) over the valid keys of its kept
// blocks, for the bound loop to use in place of the bound.
template <int D>
__device__ void exact_row_max(const v4u (&qf)[4][D / 32], const int32_t *kl, int kb,
                              const uint4 *kbu, size_t headblk, int T, int nlast, float c,
                              float (&m)[4], int lane) {
  constexpr int NK = D / 32;
  const int g = lane >> 4;
  float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int n = 0; n < kb; ++n) {
    const int j = kl[n];
    const int nj = j == T - 1 ? nlast : BLK;
    const uint4 *kp = kbu + (headblk + j) * (4 * NK * 64) + lane;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v4u kf[NK];
#pragma unroll
      for (int kc = 0; kc < NK; ++kc) kf[kc] = __builtin_bit_cast(v4u, kp[(t * NK + kc) * 64]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v4f a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < NK; ++kc) a = mfma_bf16(kf[kc], qf[u][kc], a);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * t + 4 * g + r < nj) mx[u] = fmaxf(mx[u], a[r]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    mx[u] = fmaxf(mx[u], __shfl_xor(mx[u], 16, 64));
    mx[u] = fmaxf(mx[u], __shfl_xor(mx[u], 32, 64));
    // at least 0: a padding key (score 0) then gets p <= 1, never an
    // overflow (its V row is zero and it is left out of the row sums)
    m[u] = fmaxf(mx[u] * c, 0.0f);
  }
}

// BOUND = true: the main launch.  A query block whose logit bound exceeds
// BOUND_LIMIT, or (INT8) whose logit scale c exceeds BIAS_C_LIMIT, is only
// flagged (flags[qb] = 1) and left to the second launch, BOUND = false, which
// handles flagged blocks only: INT8 with the online-max loop (plain int ->
// float scores), bf16 with the bound loop run on the rows' exact maxima.
// QK8 = false: QK^T in bf16 from Q itself and the bf16 copy of K in kfr (no
// INT8 step, no scales; the logit scale is sm_scale alone).  FINE (INT8
// only): one Q scale per 16 rows (dq [qb][4]) and one K' scale per 4 keys
// (dk [block][16]).
// DUMP (INT8, BOUND): the int32 read-back form.  Wave t takes the triple
// (bh, i, j) = dpairs[3t .. 3t+2] (t < ndump; nqb stays the number of query
// blocks) and runs query block bh*T + i through the same bound-path loop with
// the one-entry kept list {j}, storing the loop's own score accumulators,
// minus the bias, to dump[t][64 query][64 key] (zeros for a triple out of
// range); nothing else is written.
template <int D, bool LIN, bool BOUND, bool QK8, bool FINE, bool DUMP>
__global__ __launch_bounds__(256, 1) void k_attn(
    const int8_t *__restrict__ q8, const void *__restrict__ kfr, const float *__restrict__ dq,
    const float *__restrict__ dk, const float *__restrict__ dkn, const float *__restrict__ dkx,
    const float *__restrict__ mu, const uint16_t *__restrict__ vt,
    const int32_t *__restrict__ kept, const uint16_t *__restrict__ Q,
    const uint16_t *__restrict__ hi, const uint16_t *__restrict__ wsw, uint16_t *__restrict__ out,
    int32_t *__restrict__ flags, float *__restrict__ lse, uint16_t *__restrict__ os, int N, int T,
    int kb, int nqb, int F, float qk_scale, const int32_t *__restrict__ dpairs,
    int32_t *__restrict__ dump, int ndump) {
  static_assert(!DUMP || (QK8 && BOUND && !LIN), "read-back form: INT8 bound loop only");
  constexpr int CG = D / 16, KC32 = D / 32;
  constexpr int KC = QKOps<D, QK8>::NK;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int qb;
  const int32_t *kl;
  int32_t *dmp = nullptr;
  if constexpr (DUMP) {
    const int t = blockIdx.x * 4 + w;
    if (t >= ndump) return;  // no barriers below: waves are independent
    const int bh0 = dpairs[3 * t], i0 = dpairs[3 * t + 1], j0 = dpairs[3 * t + 2];
    dmp = dump + (size_t)t * BLK * BLK;
    if (bh0 < 0 || bh0 >= nqb / T || i0 < 0 || i0 >= T || j0 < 0 || j0 >= T) {
      for (int x = lane; x < BLK * BLK; x += 64) dmp[x] = 0;
      return;
    }
    qb = bh0 * T + i0;
    kl = dpairs + 3 * t + 2;
    // a list length the compiler cannot see, so the loop keeps the
    // production form (with a constant 1 it folds the loop and moves the
    // first score reads next to the asm MFMAs that write them)
    kb = 1;
    asm volatile("" : "+s"(kb));
  } else {
    qb = xcd_remap(blockIdx.x, gridDim.x) * 4 + w;
    if (qb >= nqb) return;  // no barriers below: waves are independent
    if (!BOUND && flags[qb] == 0) return;
    kl = kept + (size_t)qb * kb;
  }
  const int bh = qb / T, i = qb - bh * T;
  const int g = lane >> 4, l16 = lane & 15;
  const int nlast = N - (T - 1) * BLK;

  // bf16: the largest centred key norm over the kept list (one entry per lane and a
  // wave max) before the Q fragments are loaded, so they are not live across
  // it; the INT8 paths take it after the scales below
  float kmax_bf = 0.f;
  if constexpr (!QK8) {
    for (int n0 = 0; n0 < kb; n0 += 64) {
      const int n = n0 + lane;
      if (n < kb) kmax_bf = fmaxf(kmax_bf, dkn[(size_t)bh * T + kl[n]]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) kmax_bf = fmaxf(kmax_bf, __shfl_xor(kmax_bf, off, 64));
  }
  typename QKOps<D, QK8>::frag qf[4][KC];
  if constexpr (QK8) load_q8<D>(q8 + (size_t)qb * BLK * D, qf, lane);
  else load_qbf<D>(Q + (size_t)bh * N * D, i, N, qf, lane);
  // the query tile's logit-scale factor: dq * sm_scale log2(e)
  float dqi[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    dqi[u] = QK8 ? (FINE ? dq[(size_t)qb * 4 + u] : dq[qb]) * qk_scale : qk_scale;

  v4f o[CG][4];
#pragma unroll
  for (int a = 0; a < CG; ++a)
#pragma unroll
    for (int u = 0; u < 4; ++u) o[a][u] = v4f{0.f, 0.f, 0.f, 0.f};
  float m[4], lsum[4];

  const size_t headblk = (size_t)bh * T;
  // padding keys of the last block held by this lane (keys 16t + 4g + r >= nlast)
  int npad_lane = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) npad_lane += (16 * t + 4 * g + r) >= nlast;

  // Upper bound of the row's logits (log2 units): |q_r . k_s| <= ||q_r||
  // ||k_s||, so logit <= dq sm_scale log2(e) ||q_r|| max_j max_s (dk_s ||k_s||)
  // (INT8: codes and scales, dk per block or per key group, K centred on
  // its mean before quantisation; bf16: dq = dk = 1 and ||k_s - mu|| in
  // place of ||k_s||, which bounds the logit minus c (q_r . mu), with a
  // margin for the float32 sums of the products and norms).
  // INT8: one kept entry per lane and a wave max (a serial walk of the list
  // waits for two dependent scalar loads per kept block); the bf16 path keeps
  // the walk (with the wave form its register allocation puts an operand
  // copy right before an inline-asm MFMA)
  float kmax = 0.f, dkmax = 0.f;
  if constexpr (QK8) {
    for (int n0 = 0; n0 < kb; n0 += 64) {
      const int n = n0 + lane;
      if (n < kb) {
        const int jj = kl[n];
        kmax = fmaxf(kmax, dkn[headblk + jj]);
        dkmax = fmaxf(dkmax, dkx[headblk + jj]);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      kmax = fmaxf(kmax, __shfl_xor(kmax, off, 64));
      dkmax = fmaxf(dkmax, __shfl_xor(dkmax, off, 64));
    }
  } else {
    kmax = kmax_bf;
  }
  const float dqmax = fmaxf(fmaxf(dqi[0], dqi[1]), fmaxf(dqi[2], dqi[3]));
  bool bounded = !QK8 || dqmax * dkmax <= BIAS_C_LIMIT;
  float qmu[4] = {0.f, 0.f, 0.f, 0.f};  // bf16: q_r . mu per row
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float qn;
    if constexpr (QK8) {
      int sq = 0;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t wv = (uint32_t)qf[u][kc][e];
#pragma unroll
          for (int b8 = 0; b8 < 4; ++b8) {
            const int v8 = (int)(int8_t)(wv >> (8 * b8));
            sq += v8 * v8;
          }
        }
      sq += __shfl_xor(sq, 16, 64);
      sq += __shfl_xor(sq, 32, 64);
      qn = sqrtf((float)sq) * (1.0f + 0x1p-20f);
    } else {
      // also q_r . mu: kmax bounds ||k_s - mu|| (mu = the K mean), so m
      // bounds the row's logits minus c (q_r . mu) on both sides; that
      // per-row constant joins the exp2 offset below, which leaves the
      // softmax unchanged and keeps every probability >= 2^(-2m) (K is not
      // centred in this mode, and its raw norms would put most rows past
      // the limit)
      float sq = 0.f, qm = 0.f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const float *mk = mu + (size_t)bh * D + 32 * kc + 8 * g;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t wv = qf[u][kc][e];
          const float lo = bf2f((uint16_t)(wv & 0xFFFF)), hi2 = bf2f((uint16_t)(wv >> 16));
          sq = __builtin_fmaf(lo, lo, sq);
          sq = __builtin_fmaf(hi2, hi2, sq);
          if constexpr (BOUND) {
            qm = __builtin_fmaf(lo, mk[2 * e], qm);
            qm = __builtin_fmaf(hi2, mk[2 * e + 1], qm);
          }
        }
      }
      sq += __shfl_xor(sq, 16, 64);
      sq += __shfl_xor(sq, 32, 64);
      qn = sqrtf(sq) * (1.0f + 0x1p-12f);
      qm += __shfl_xor(qm, 16, 64);
      qm += __shfl_xor(qm, 32, 64);
      qmu[u] = qm;
    }
    m[u] = dqi[u] * qn * kmax;
    lsum[u] = 0.f;
    bounded = bounded && (m[u] <= BOUND_LIMIT);
  }
  if constexpr (DUMP) {
    // every score is read back, whatever the bound decides
    kept_loop_piped<D, QK8, FINE, true>(qf, o, m, lsum, kl, kb, dk, (const uint4 *)kfr,
                                        (const uint4 *)vt, headblk, dqi, T, nlast, lane, dmp);
    return;
  } else if (BOUND) {
    const bool fail = __ballot(!bounded) != 0ull;
    if (lane == 0) flags[qb] = fail ? 1 : 0;
    if (fail) return;
    if constexpr (!QK8) {
#pragma unroll
      for (int u = 0; u < 4; ++u) m[u] = __builtin_fmaf(dqi[u], qmu[u], m[u]);
    }
    kept_loop_piped<D, QK8, FINE>(qf, o, m, lsum, kl, kb, dk, (const uint4 *)kfr,
                                  (const uint4 *)vt, headblk, dqi, T, nlast, lane);
  } else if constexpr (QK8) {
#pragma unroll
    for (int u = 0; u < 4; ++u) m[u] = -INFINITY;
    kept_loop<D, false, FINE>(qf, o, m, lsum, kl, kb, dk, (const uint4 *)kfr, (const uint4 *)vt,
                              headblk, dqi, T, npad_lane, lane);
  } else {
    exact_row_max<D>(qf, kl, kb, (const uint4 *)kfr, headblk, T, nlast, dqi[0], m, lane);
    kept_loop_piped<D, false, false>(qf, o, m, lsum, kl, kb, dk, (const uint4 *)kfr,
                                     (const uint4 *)vt, headblk, dqi, T, nlast, lane);
  }
  // Row sums; O is normalised only while it is stored, so the accumulators
  // are not touched by vector ALU code in between (they stay in AGPRs).
  float linv[4], lrow[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float l = lsum[u];
    if (!BOUND && QK8) {  // the online loop keeps per-lane partial sums
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
    }
    // no kept key (kb = 0): O is zero, and l = 1 leaves the linear branch as is
    lrow[u] = l > 0.f ? l : 1.0f;
    linv[u] = 1.0f / lrow[u];
  }

  // bf16 QK^T with a backward pass planned: the normalised sparse output
  // O_sparse too (rows < N), so the backward's rowsum(dO O_sparse) does not
  // depend on the linear branch or on the rounding of the combined output
  if constexpr (!QK8) {
    if (os) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int row = i * BLK + 16 * u + l16;
        if (row < N) {
          uint16_t *orow = os + ((size_t)qb * BLK + 16 * u + l16) * D;
#pragma unroll
          for (int a = 0; a < CG; ++a)
            *(uint2 *)(orow + 16 * a + 4 * g) =
                make_uint2(pack2bf(o[a][u][0] * linv[u], o[a][u][1] * linv[u]),
                           pack2bf(o[a][u][2] * linv[u], o[a][u][3] * linv[u]));
        }
      }
    }
  }

  if (LIN) {
    // phi(Q) fragments: lane (query 16u + l16, group g) holds channels
    // 32kc + 8g .. +7 of its row; softmax over the row's d channels.
    v4u pq[4][KC32];
    float den[4];
    const uint16_t *hp = hi + (size_t)qb * F;
    // Every global load of the branch except the projection's (Q rows, z_i,
    // H_i fragments) is issued here, before any of them is used, so their
    // latencies overlap: issued round by round, each waited for before the
    // next, they left the SIMD idle for most of the epilogue (its only wave).
    uint4 qv[4][KC32], zv[KC32];
    v4u hfa[CG][KC32];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = i * BLK + 16 * u + l16;
      const uint16_t *qr = Q + ((size_t)bh * N + (row < N ? row : 0)) * D;
#pragma unroll
      for (int kc = 0; kc < KC32; ++kc) qv[u][kc] = *(const uint4 *)(qr + 32 * kc + 8 * g);
    }
#pragma unroll
    for (int kc = 0; kc < KC32; ++kc) zv[kc] = *(const uint4 *)(hp + D * D + 32 * kc + 8 * g);
#pragma unroll
    for (int x = 0; x < CG; ++x)
#pragma unroll
      for (int kc = 0; kc < KC32; ++kc)
        hfa[x][kc] = *(const v4u *)(hp + ((size_t)(x * KC32 + kc) * 64 + lane) * 8);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float x[KC32][8];
#pragma unroll
      for (int kc = 0; kc < KC32; ++kc) {
        const uint4 v = qv[u][kc];
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
        const uint32_t zz[4] = {zv[kc].x, zv[kc].y, zv[kc].z, zv[kc].w};
        uint32_t pk[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          pk[h] = pack2bf(x[kc][2 * h] * rs, x[kc][2 * h + 1] * rs);
          dd = __builtin_fmaf(bf2f((uint16_t)(pk[h] & 0xFFFF)), bf2f((uint16_t)(zz[h] & 0xFFFF)), dd);
          dd = __builtin_fmaf(bf2f((uint16_t)(pk[h] >> 16)), bf2f((uint16_t)(zz[h] >> 16)), dd);
        }
        pq[u][kc] = v4u{pk[0], pk[1], pk[2], pk[3]};
      }
      dd += __shfl_xor(dd, 16, 64);
      dd += __shfl_xor(dd, 32, 64);
      den[u] = dd;
    }
    // O_l^T = H^T phi(Q)^T, taken two channel groups at a time and packed at
    // once into B fragments of O_l^T * (l / den) (k = value channel, kmaj
    // order), so that O += W (O_l^T l) keeps the sparse sum unnormalised: the
    // final 1/l then yields O_s + O_l W^T.
    float rr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) rr[u] = den[u] > 0.f ? lrow[u] / den[u] : 0.f;
    v4u ob[KC32][4];
#pragma unroll
    for (int kc = 0; kc < KC32; ++kc) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KC32; ++k) {
          a0 = mfma_bf16(hfa[2 * kc][k], pq[u][k], a0);
          a1 = mfma_bf16(hfa[2 * kc + 1][k], pq[u][k], a1);
        }
        const float r = rr[u];
        ob[kc][u] = v4u{pack2bf(a0[0] * r, a0[1] * r), pack2bf(a0[2] * r, a0[3] * r),
                        pack2bf(a1[0] * r, a1[1] * r), pack2bf(a1[2] * r, a1[3] * r)};
      }
    }
    // The projection's fragments are all requested before the first is used.
    v4u wf[CG][KC32];
#pragma unroll
    for (int y = 0; y < CG; ++y)
#pragma unroll
      for (int kc = 0; kc < KC32; ++kc)
        wf[y][kc] = *(const v4u *)(wsw + ((size_t)(y * KC32 + kc) * 64 + lane) * 8);
#pragma unroll
    for (int y = 0; y < CG; ++y)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int kc = 0; kc < KC32; ++kc) o[y][u] = mfma_bf16(wf[y][kc], ob[kc][u], o[y][u]);
  }

  // store O / l: lane holds query 16u + l16, channels 16a + 4g .. +3.  The
  // bf16 QK^T path also stores each row's log2 normaliser m + log2(l), so a
  // backward pass can rebuild p = exp2(logit - lse) without the forward's max.
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = i * BLK + 16 * u + l16;
    if (!QK8 && g == 0 && row < N) lse[(size_t)qb * BLK + 16 * u + l16] = m[u] + log2f(lrow[u]);
    if (row < N) {
      uint16_t *orow = out + ((size_t)bh * N + row) * D;
      const float r = linv[u];
#pragma unroll
      for (int a = 0; a < CG; ++a) {
        uint2 v = make_uint2(pack2bf(o[a][u][0] * r, o[a][u][1] * r),
                             pack2bf(o[a][u][2] * r, o[a][u][3] * r));
        *(uint2 *)(orow + 16 * a + 4 * g) = v;
      }
    }
  }
}

template <int D, bool LIN, bool QK8, bool FINE>
static void launch_attn_t(const Plan &p, const uint16_t *q, const WsPtrs &ws, uint16_t *out,
                          hipStream_t st) {
  const int nqb = p.BH * p.T;
  dim3 grid((nqb + 3) / 4), block(256);
  const float qk_scale = p.sm_scale * LOG2E;
  const void *kfr = QK8 ? (const void *)ws.k8 : (const void *)ws.kbf;
  hipLaunchKernelGGL((k_attn<D, LIN, true, QK8, FINE, false>), grid, block, 0, st, ws.q8, kfr,
                     ws.dq, ws.dk, ws.dkn, ws.dkx, ws.mu, ws.vt, ws.kept, q, ws.hi, ws.wsw, out, ws.flags,
                     ws.lse, ws.os, p.N, p.T, p.kb, nqb, p.F, qk_scale, nullptr, nullptr, 0);
  hipLaunchKernelGGL((k_attn<D, LIN, false, QK8, FINE, false>), grid, block, 0, st, ws.q8, kfr,
                     ws.dq, ws.dk, ws.dkn, ws.dkx, ws.mu, ws.vt, ws.kept, q, ws.hi, ws.wsw, out, ws.flags,
                     ws.lse, ws.os, p.N, p.T, p.kb, nqb, p.F, qk_scale, nullptr, nullptr, 0);
}

template <int D, bool QK8, bool FINE>
static void launch_attn_d(const Plan &p, const uint16_t *q, const WsPtrs &ws, uint16_t *out,
                          hipStream_t st) {
  if (p.lin_on)
    launch_attn_t<D, true, QK8, FINE>(p, q, ws, out, st);
  else
    launch_attn_t<D, false, QK8, FINE>(p, q, ws, out, st);
}

template <int D>
static void launch_attn_m(const Plan &p, const uint16_t *q, const WsPtrs &ws, uint16_t *out,
                          hipStream_t st) {
  if (!p.qk_int8)
    launch_attn_d<D, false, false>(p, q, ws, out, st);
  else if (p.qk_fine)
    launch_attn_d<D, true, true>(p, q, ws, out, st);
  else
    launch_attn_d<D, true, false>(p, q, ws, out, st);
}

void launch_attn(const Plan &p, const uint16_t *q, const WsPtrs &ws, uint16_t *out, hipStream_t st) {
  if (p.d == 128)
    launch_attn_m<128>(p, q, ws, out, st);
  else
    launch_attn_m<64>(p, q, ws, out, st);
}

template <int D, bool FINE>
static void launch_debug_qk_t(const Plan &p, const WsPtrs &ws, const int32_t *pairs, int n,
                              int32_t *out, hipStream_t st) {
  const int nqb = p.BH * p.T;
  hipLaunchKernelGGL((k_attn<D, false, true, true, FINE, true>), dim3((n + 3) / 4), dim3(256), 0, st,
                     ws.q8, (const void *)ws.k8, ws.dq, ws.dk, ws.dkn, ws.dkx, ws.mu, ws.vt, ws.kept,
                     nullptr, ws.hi, ws.wsw, nullptr, ws.flags, ws.lse, ws.os, p.N, p.T, p.kb, nqb,
                     p.F, p.sm_scale * LOG2E, pairs, out, n);
}

void launch_debug_qk(const Plan &p, const WsPtrs &ws, const int32_t *pairs, int n, int32_t *out,
                     hipStream_t st) {
  if (n <= 0) return;
  if (p.d == 128)
    p.qk_fine ? launch_debug_qk_t<128, true>(p, ws, pairs, n, out, st)
              : launch_debug_qk_t<128, false>(p, ws, pairs, n, out, st);
  else
    p.qk_fine ? launch_debug_qk_t<64, true>(p, ws, pairs, n, out, st)
              : launch_debug_qk_t<64, false>(p, ws, pairs, n, out, st);
}

}  // namespace sla
