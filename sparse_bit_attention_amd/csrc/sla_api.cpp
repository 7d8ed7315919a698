// C ABI of libsagesla: plan validation, workspace map and launch sequencing.
// All checks run on the host before anything is enqueued.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

#include "sla_internal.h"

struct sla_plan_s {
  sla::Plan p;
};

namespace sla {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsPtrs ws_ptrs(const Plan &p, void *ws) {
  char *b = (char *)ws;
  WsPtrs w;
  w.qbar = (float *)(b + p.off[R_QBAR]);
  w.ksum = (float *)(b + p.off[R_KSUM]);
  w.kbar = (float *)(b + p.off[R_KBAR]);
  w.mu = (float *)(b + p.off[R_MU]);
  w.mask = (uint64_t *)(b + p.off[R_MASK]);
  w.kept = (int32_t *)(b + p.off[R_KEPT]);
  w.q8 = (int8_t *)(b + p.off[R_Q8]);
  w.k8 = (int8_t *)(b + p.off[R_K8]);
  w.dq = (float *)(b + p.off[R_DQ]);
  w.dk = (float *)(b + p.off[R_DK]);
  w.dkn = (float *)(b + p.off[R_DKN]);
  w.dkx = (float *)(b + p.off[R_DKX]);
  w.flags = (int32_t *)(b + p.off[R_FLAG]);
  w.maskt = (uint64_t *)(b + p.off[R_MASKT]);
  w.vt = (uint16_t *)(b + p.off[R_VT]);
  w.kbf = (uint16_t *)(b + p.off[R_KB]);
  w.wsw = (uint16_t *)(b + p.off[R_WSW]);
  w.hb = (uint16_t *)(b + p.off[R_HB]);
  w.hi = (uint16_t *)(b + p.off[R_HI]);
  w.sc = (float *)(b + p.off[R_SC]);
  w.lse = (float *)(b + p.off[R_LSE]);
  w.mt = (uint64_t *)(b + p.off[R_MT]);
  w.mtt = (uint64_t *)(b + p.off[R_MTT]);
  w.delta = (float *)(b + p.off[R_DELTA]);
  w.ol = (uint16_t *)(b + p.off[R_OL]);
  w.dhi = (uint16_t *)(b + p.off[R_DHI]);
  w.dhb = (uint16_t *)(b + p.off[R_DHB]);
  w.dwp = (float *)(b + p.off[R_DWP]);
  w.os = p.size[R_OS] ? (uint16_t *)(b + p.off[R_OS]) : nullptr;
  w.dql = (float *)(b + p.off[R_DQL]);
  w.dkl = (float *)(b + p.off[R_DKL]);
  w.dvl = (float *)(b + p.off[R_DVL]);
  return w;
}

// The workspace of sla_attention_fwd_noalloc: one copy per GPU, at that GPU's
// own address.  In host code `scratch` names a host-side stand-in, never the
// device memory: only the per-device address from hipGetSymbolAddress is
// passed on.
static __device__ __align__(256) unsigned char scratch[SLA_NOALLOC_WS_BYTES];

constexpr int MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void *g_scratch[MAX_DEVICES];  // device address of `scratch`, per device

// The current device's copy of `scratch`, looked up on the first call on that
// device (with the device current).
static sla_status scratch_ptr(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return SLA_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SLA_EHIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return SLA_OK;
}

}  // namespace sla

using namespace sla;

extern "C" {

const char *sla_status_string(sla_status s) {
  switch (s) {
    case SLA_OK: return "ok";
    case SLA_EINVAL: return "invalid argument";
    case SLA_EUNSUPPORTED: return "unsupported configuration";
    case SLA_EWORKSPACE: return "workspace too small";
    case SLA_EHIP: return "HIP launch failed";
    case SLA_ENOMEM: return "host allocation failed";
    case SLA_ETOOLARGE: return "workspace exceeds the library's static workspace";
  }
  return "unknown status";
}

sla_status sla_plan(const sla_config *cfg, sla_plan_t *out) {
  if (!cfg || !out) return SLA_EINVAL;
  const sla_config c = *cfg;
  if (c.B < 1 || c.H < 1 || c.N < 1) return SLA_EINVAL;
  if (!(c.topk >= 0.0f && c.topk <= 1.0f)) return SLA_EINVAL;
  if (c.use_linear != 0 && c.use_linear != 1) return SLA_EINVAL;
  if (c.qk_int8 != 0 && c.qk_int8 != 1) return SLA_EINVAL;
  if (c.qk_fine != 0 && c.qk_fine != 1) return SLA_EINVAL;
  if (c.qk_fine && !c.qk_int8) return SLA_EINVAL;
  if (c.backward != 0 && c.backward != 1) return SLA_EINVAL;
  if (c.backward && c.qk_int8) return SLA_EUNSUPPORTED;  // the backward is plain SLA's
  if (!(c.sm_scale >= 0.0f) || isinf(c.sm_scale)) return SLA_EINVAL;
  if (c.block != BLK) return SLA_EUNSUPPORTED;
  if (c.d != 64 && c.d != 128) return SLA_EUNSUPPORTED;
  const long long T = ((long long)c.N + BLK - 1) / BLK;
  const long long BH = (long long)c.B * c.H;
  if (BH * T >= (1LL << 31) / BLK) return SLA_EUNSUPPORTED;
  // the score kernel's grid: one workgroup per (head, 32 query blocks, 256 key blocks)
  if (BH * ((T + 31) / 32) * ((T + 255) / 256) >= (1LL << 31)) return SLA_EUNSUPPORTED;

  sla_plan_s *h = new (std::nothrow) sla_plan_s;
  if (!h) return SLA_ENOMEM;
  Plan &p = h->p;
  memset(&p, 0, sizeof p);
  p.cfg = c;
  p.B = c.B;
  p.H = c.H;
  p.N = c.N;
  p.d = c.d;
  p.BH = (int)BH;
  p.T = (int)T;
  {
    // kb = 0 for topk = 0, else clamp(floor(topk*T + 1e-6), 1, T), in float64
    long kb = 0;
    if ((double)c.topk > 0.0) {
      kb = (long)floor((double)c.topk * (double)p.T + 1e-6);
      if (kb < 1) kb = 1;
      if (kb > p.T) kb = p.T;
    }
    p.kb = (int)kb;
  }
  p.W64 = (p.T + 63) / 64;
  p.F = ((c.d * c.d + c.d) + 127) / 128 * 128;
  p.lin_on = (c.use_linear == 1 && p.kb < p.T) ? 1 : 0;
  p.qk_int8 = c.qk_int8;
  p.qk_fine = c.qk_fine;
  p.bwd = c.backward;
  p.dw_chunks = (p.BH * p.T + DW_CHUNK - 1) / DW_CHUNK;
  p.sm_scale = c.sm_scale > 0.0f ? c.sm_scale : (float)(1.0 / sqrt((double)c.d));

  const size_t bt = (size_t)p.BH * p.T;
  const size_t blk_elems = bt * BLK * p.d;
  p.size[R_QBAR] = bt * p.d * 4;
  p.size[R_KSUM] = bt * p.d * 4;
  p.size[R_KBAR] = bt * p.d * 4;
  p.size[R_MU] = (size_t)p.BH * p.d * 4;
  p.size[R_MASK] = bt * p.W64 * 8;
  p.size[R_KEPT] = bt * (size_t)(p.kb > 0 ? p.kb : 1) * 4;
  p.size[R_Q8] = p.qk_int8 ? blk_elems : 0;
  p.size[R_K8] = p.qk_int8 ? blk_elems : 0;
  p.size[R_DQ] = bt * 4 * (p.qk_fine ? 4 : 1);
  p.size[R_DK] = bt * 4 * (p.qk_fine ? 16 : 1);
  p.size[R_DKN] = bt * 4;
  p.size[R_DKX] = bt * 4;
  p.size[R_FLAG] = bt * 4;
  p.size[R_MASKT] = p.lin_on ? bt * p.W64 * 8 : 0;
  p.size[R_VT] = blk_elems * 2;
  p.size[R_KB] = p.qk_int8 ? 0 : blk_elems * 2;
  p.size[R_WSW] = p.lin_on ? (size_t)p.d * p.d * 2 : 0;
  p.size[R_HB] = p.lin_on ? bt * p.F * 2 : 0;
  p.size[R_HI] = p.lin_on ? bt * p.F * 2 : 0;
  p.size[R_SC] = bt * p.T * 4;
  p.size[R_LSE] = bt * BLK * 4;
  p.size[R_MT] = p.bwd ? bt * p.W64 * 8 : 0;
  p.size[R_MTT] = p.bwd && p.lin_on ? bt * p.W64 * 8 : 0;
  p.size[R_DELTA] = p.bwd ? bt * BLK * 4 : 0;
  p.size[R_OS] = p.bwd ? blk_elems * 2 : 0;
  p.size[R_OL] = p.bwd && p.lin_on ? blk_elems * 2 : 0;
  p.size[R_DHI] = p.bwd && p.lin_on ? bt * p.F * 2 : 0;
  p.size[R_DHB] = p.bwd && p.lin_on ? bt * p.F * 2 : 0;
  p.size[R_DWP] = p.bwd && p.lin_on ? (size_t)p.dw_chunks * p.d * p.d * 4 : 0;
  p.size[R_DQL] = p.bwd && p.lin_on ? blk_elems * 4 : 0;
  p.size[R_DKL] = p.bwd && p.lin_on ? blk_elems * 4 : 0;
  p.size[R_DVL] = p.bwd && p.lin_on ? blk_elems * 4 : 0;
  size_t o = 0;
  for (int r = 0; r < R_COUNT; ++r) {
    p.off[r] = o;
    o += align256(p.size[r]);
  }
  p.total = o;
  *out = h;
  return SLA_OK;
}

sla_status sla_plan_destroy(sla_plan_t plan) {
  delete plan;
  return SLA_OK;
}

sla_status sla_plan_info(sla_plan_t plan, int32_t *T, int32_t *kb, size_t *workspace_bytes) {
  if (!plan) return SLA_EINVAL;
  if (T) *T = plan->p.T;
  if (kb) *kb = plan->p.kb;
  if (workspace_bytes) *workspace_bytes = plan->p.total;
  return SLA_OK;
}

static bool aligned(const void *x, size_t a) { return ((uintptr_t)x % a) == 0; }

static sla_status check_ws(const Plan &p, const void *ws, size_t ws_bytes) {
  if (!ws) return SLA_EINVAL;
  if (!aligned(ws, 256)) return SLA_EINVAL;
  if (ws_bytes < p.total) return SLA_EWORKSPACE;
  return SLA_OK;
}

static sla_status launched() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? SLA_OK : SLA_EHIP;
}

sla_status sla_quantize(sla_plan_t plan, const void *q, const void *k, void *ws, size_t ws_bytes,
                        void *stream) {
  if (!plan || !q || !k) return SLA_EINVAL;
  const Plan &p = plan->p;
  if (!aligned(q, 16) || !aligned(k, 16)) return SLA_EINVAL;
  sla_status s = check_ws(p, ws, ws_bytes);
  if (s != SLA_OK) return s;
  (void)hipGetLastError();
  hipStream_t st = (hipStream_t)stream;
  WsPtrs w = ws_ptrs(p, ws);
  launch_pool_quant_q(p, (const uint16_t *)q, (const uint16_t *)k, w, st);
  launch_kmean(p, w, st);
  launch_select(p, w, st);
  return launched();
}

sla_status sla_prepare_kv(sla_plan_t plan, const void *k, const void *v, const void *w_proj,
                          void *ws, size_t ws_bytes, void *stream) {
  if (!plan || !k || !v) return SLA_EINVAL;
  const Plan &p = plan->p;
  if (p.cfg.use_linear && !w_proj) return SLA_EINVAL;
  if (!aligned(k, 16) || !aligned(v, 16)) return SLA_EINVAL;
  if (w_proj && !aligned(w_proj, 16)) return SLA_EINVAL;
  sla_status s = check_ws(p, ws, ws_bytes);
  if (s != SLA_OK) return s;
  (void)hipGetLastError();
  hipStream_t st = (hipStream_t)stream;
  WsPtrs w = ws_ptrs(p, ws);
  if (!p.qk_int8) launch_prep_kbf(p, (const uint16_t *)k, w, st);
  launch_kv_prep(p, (const uint16_t *)k, (const uint16_t *)v, w, st);
  if (p.lin_on) {
    launch_w_swizzle(p, (const uint16_t *)w_proj, w, st);
    launch_marginal(p, w, st);
  }
  return launched();
}

sla_status sla_attend(sla_plan_t plan, const void *q, void *out, void *ws, size_t ws_bytes,
                      void *stream) {
  if (!plan || !q || !out) return SLA_EINVAL;
  const Plan &p = plan->p;
  if (!aligned(q, 16) || !aligned(out, 16)) return SLA_EINVAL;
  sla_status s = check_ws(p, ws, ws_bytes);
  if (s != SLA_OK) return s;
  (void)hipGetLastError();
  launch_attn(p, (const uint16_t *)q, ws_ptrs(p, ws), (uint16_t *)out, (hipStream_t)stream);
  return launched();
}

sla_status sla_attention_fwd(sla_plan_t plan, const void *q, const void *k, const void *v,
                             const void *w_proj, void *out, void *ws, size_t ws_bytes,
                             void *stream) {
  if (!plan || !q || !k || !v || !out) return SLA_EINVAL;
  const Plan &p = plan->p;
  if (p.cfg.use_linear && !w_proj) return SLA_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return SLA_EINVAL;
  if (w_proj && !aligned(w_proj, 16)) return SLA_EINVAL;
  sla_status s = check_ws(p, ws, ws_bytes);
  if (s != SLA_OK) return s;
  s = sla_prepare_kv(plan, k, v, w_proj, ws, ws_bytes, stream);
  if (s != SLA_OK) return s;
  return sla_attend(plan, q, out, ws, ws_bytes, stream);
}

sla_status sla_attention_fwd_noalloc(sla_plan_t plan, const void *q, const void *k, const void *v,
                                     const void *w_proj, void *out, void *stream) {
  // the checks of sla_quantize and sla_attention_fwd, all before any launch
  if (!plan || !q || !k || !v || !out) return SLA_EINVAL;
  const Plan &p = plan->p;
  if (p.cfg.use_linear && !w_proj) return SLA_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return SLA_EINVAL;
  if (w_proj && !aligned(w_proj, 16)) return SLA_EINVAL;
  if (p.total > SLA_NOALLOC_WS_BYTES) return SLA_ETOOLARGE;
  void *ws = nullptr;
  sla_status s = scratch_ptr(&ws);
  if (s != SLA_OK) return s;
  s = sla_quantize(plan, q, k, ws, SLA_NOALLOC_WS_BYTES, stream);
  if (s != SLA_OK) return s;
  return sla_attention_fwd(plan, q, k, v, w_proj, out, ws, SLA_NOALLOC_WS_BYTES, stream);
}

sla_status sla_ws_view(sla_plan_t plan, void *ws, int32_t which, void **dev_ptr, size_t *bytes) {
  if (!plan || !dev_ptr || !bytes) return SLA_EINVAL;
  if (which < 0 || which >= SLA_WS_COUNT) return SLA_EINVAL;
  *dev_ptr = (char *)ws + plan->p.off[which];
  *bytes = plan->p.size[which];
  return SLA_OK;
}

sla_status sla_debug_qk_int32(sla_plan_t plan, const void *ws, const int32_t *dev_pairs, int32_t n,
                              int32_t *dev_out, void *stream) {
  if (!plan || !ws || n < 0 || (n > 0 && (!dev_pairs || !dev_out))) return SLA_EINVAL;
  const Plan &p = plan->p;
  if (!p.qk_int8) return SLA_EUNSUPPORTED;
  if (!aligned(ws, 256)) return SLA_EINVAL;
  (void)hipGetLastError();
  WsPtrs w = ws_ptrs(p, (void *)ws);
  launch_debug_qk(p, w, dev_pairs, n, dev_out, (hipStream_t)stream);
  return launched();
}

sla_status sla_attention_bwd(sla_plan_t plan, const void *q, const void *k, const void *v,
                             const void *w_proj, const void *dout, void *dq, void *dk, void *dv,
                             float *dw, void *ws, size_t ws_bytes, void *stream) {
  if (!plan || !q || !k || !v || !dout || !dq || !dk || !dv) return SLA_EINVAL;
  const Plan &p = plan->p;
  if (!p.bwd) return SLA_EUNSUPPORTED;
  if (p.cfg.use_linear && (!w_proj || !dw)) return SLA_EINVAL;
  const void *a16[] = {q, k, v, dout, dq, dk, dv};
  for (const void *x : a16)
    if (!aligned(x, 16)) return SLA_EINVAL;
  if (w_proj && !aligned(w_proj, 16)) return SLA_EINVAL;
  if (dw && !aligned(dw, 4)) return SLA_EINVAL;
  sla_status s = check_ws(p, ws, ws_bytes);
  if (s != SLA_OK) return s;
  (void)hipGetLastError();
  launch_bwd(p, (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v,
             (const uint16_t *)w_proj, (const uint16_t *)dout,
             (uint16_t *)dq, (uint16_t *)dk, (uint16_t *)dv, p.cfg.use_linear ? dw : nullptr,
             ws_ptrs(p, ws), (hipStream_t)stream);
  return launched();
}

// ---- W8A8 linear layers ------------------------------------------------------

sla_status sla_quant_b128(const void *x, int32_t rows, int32_t cols, void *codes, float *scales,
                          void *stream) {
  if (!x || !codes || !scales) return SLA_EINVAL;
  if (rows < 1 || cols < 1) return SLA_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return SLA_EINVAL;
  if (cols % 16 != 0 || (rows + 127) / 128 > 65535) return SLA_EUNSUPPORTED;
  (void)hipGetLastError();
  launch_quant_b128((const uint16_t *)x, rows, cols, (int8_t *)codes, scales, (hipStream_t)stream);
  return launched();
}

sla_status sla_w8a8_gemm(const void *xq, const float *sx, const void *wq, const float *sw,
                         int32_t M, int32_t N, int32_t K, void *y, void *stream) {
  if (!xq || !sx || !wq || !sw || !y) return SLA_EINVAL;
  if (M < 1 || N < 1 || K < 1) return SLA_EINVAL;
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(y, 2) || !aligned(sx, 4) || !aligned(sw, 4))
    return SLA_EINVAL;
  if (K % 128 != 0) return SLA_EUNSUPPORTED;
  const long long tiles = (long long)((M + 127) / 128) * ((N + 255) / 256);
  if (tiles >= (1LL << 31)) return SLA_EUNSUPPORTED;
  (void)hipGetLastError();
  launch_w8a8_gemm((const int8_t *)xq, sx, (const int8_t *)wq, sw, M, N, K, (uint16_t *)y,
                   (hipStream_t)stream);
  return launched();
}

}  // extern "C"
