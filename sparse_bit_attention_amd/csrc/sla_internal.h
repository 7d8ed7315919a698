// Internal plan, workspace map and kernel launchers of libsagesla.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sagesla.h"
#include "sla_device.h"

namespace sla {

// Workspace regions in order; the first SLA_WS_COUNT match the public enum.
enum Region {
  R_QBAR = SLA_WS_QBAR,
  R_KSUM = SLA_WS_KSUM,
  R_KBAR = SLA_WS_KBAR,
  R_MU = SLA_WS_MU,
  R_MASK = SLA_WS_MASK,
  R_KEPT = SLA_WS_KEPT,
  R_Q8 = SLA_WS_Q8,
  R_K8 = SLA_WS_K8,
  R_DQ = SLA_WS_DQ,
  R_DK = SLA_WS_DK,
  R_LSE = SLA_WS_LSE,
  R_DKN,  // f32 dk_j * max row L2 norm of the block's K8 codes   [BH][T]
          //     (bf16 QK^T: max row L2 norm of the block's K rows)
  R_DKX,  // f32 largest K' scale of the block (bias check)       [BH][T]
  R_FLAG, // i32 query blocks left to the online-max attention    [BH][T]
  R_MASKT,// u64 mask words, word-major                          [BH][W64][T]
  R_VT,   // bf16 V per key block in kmaj_off order              [BH][T][64*d]
  R_KB,   // bf16 K per key block in bfk_off order (bf16 QK^T)    [BH][T][64*d]
  R_WSW,  // bf16 projection in wfrag_off order                  [d*d]
  R_HB,   // bf16 per key block linear state (hstate_off order)  [BH][T][F]
  R_HI,   // bf16 per query block marginal state (same order)    [BH][T][F]
  R_SC,   // f32 block scores, row i over key blocks j           [BH][T][T]
  // backward pass (plans with backward = 1)
  R_MT,   // u64 transposed mask, row j = key block, bits = query blocks [BH][T][W64]
  R_MTT,  // u64 the same, word-major (marginal GEMM operand)    [BH][W64][T]
  R_DELTA,// f32 rowsum(dO * O_sparse)                           [BH][T][64]
  R_OS,   // bf16 sparse-branch output O_sparse (forward)         [BH][T][64][d]
  R_OL,   // bf16 linear-branch rows O_l before the projection   [BH][T][64][d]
  R_DHI,  // bf16 gradient of the marginal state (dh_off order)  [BH][T][F]
  R_DHB,  // bf16 gradient of the key-block state (same order)   [BH][T][F]
  R_DWP,  // f32 partial projection gradients                    [nchunk][d][d]
  R_DQL,  // f32 linear-branch dQ rows                           [BH][T][64][d]
  R_DKL,  // f32 linear-branch dK rows                           [BH][T][64][d]
  R_DVL,  // f32 linear-branch dV rows                           [BH][T][64][d]
  R_COUNT
};

struct Plan {
  sla_config cfg;
  int B, H, N, d, BH, T, kb, W64;
  int F;          // per-block linear-state length, d*d + d padded to 128
  int lin_on;     // linear branch present (use_linear and kb < T)
  int qk_int8;
  int qk_fine;    // finer INT8 scales: 16 query rows, 4 keys per scale
  int bwd;        // workspace holds the backward regions
  int dw_chunks;  // query blocks are summed into dW partials in chunks of DW_CHUNK
  float sm_scale;
  size_t off[R_COUNT], size[R_COUNT], total;
};

struct WsPtrs {
  float *qbar, *ksum, *kbar, *mu, *dq, *dk, *dkn, *dkx, *lse, *delta, *dwp, *dql, *dkl, *dvl;
  uint64_t *mt, *mtt;
  uint16_t *ol, *dhi, *dhb, *os;
  uint64_t *mask, *maskt;
  int32_t *kept, *flags;
  int8_t *q8, *k8;
  uint16_t *vt, *kbf, *wsw, *hb, *hi;
  float *sc;
};

WsPtrs ws_ptrs(const Plan &p, void *ws);

void launch_pool_quant_q(const Plan &p, const uint16_t *q, const uint16_t *k, const WsPtrs &ws,
                         hipStream_t st);
void launch_kmean(const Plan &p, const WsPtrs &ws, hipStream_t st);
void launch_select(const Plan &p, const WsPtrs &ws, hipStream_t st);
// bf16 QK^T mode: K copied in bfk_off order with its block norms
void launch_prep_kbf(const Plan &p, const uint16_t *k, const WsPtrs &ws, hipStream_t st);
// V re-layout, per key block linear states and (INT8 QK^T) the K' codes and scales
void launch_kv_prep(const Plan &p, const uint16_t *k, const uint16_t *v, const WsPtrs &ws,
                    hipStream_t st);
void launch_w_swizzle(const Plan &p, const uint16_t *w, const WsPtrs &ws, hipStream_t st);
void launch_marginal(const Plan &p, const WsPtrs &ws, hipStream_t st);
// H = (1 - M) Hb per head for a word-major mask (the forward's M, or its
// transpose for the backward's dHb = (1 - M)^T dH)
void launch_marginal_ptrs(const Plan &p, const uint64_t *maskt, const uint16_t *hb, uint16_t *hi,
                          hipStream_t st);
void launch_attn(const Plan &p, const uint16_t *q, const WsPtrs &ws, uint16_t *out, hipStream_t st);
void launch_debug_qk(const Plan &p, const WsPtrs &ws, const int32_t *pairs, int n, int32_t *out,
                     hipStream_t st);
// backward pass of plain SLA
constexpr int DW_CHUNK = 64;  // query blocks per dW partial
void launch_bwd(const Plan &p, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                const uint16_t *w, const uint16_t *dout, uint16_t *dq,
                uint16_t *dk, uint16_t *dv, float *dw, const WsPtrs &ws, hipStream_t st);
void launch_quant_b128(const uint16_t *x, int R, int C, int8_t *codes, float *scales,
                       hipStream_t st);
void launch_w8a8_gemm(const int8_t *xq, const float *sx, const int8_t *wq, const float *sw, int M,
                      int N, int K, uint16_t *y, hipStream_t st);

}  // namespace sla
