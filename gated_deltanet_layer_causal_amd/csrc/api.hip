// Exported C entry points of libgdn: host-side argument validation, then the
// launchers.  Nothing is launched unless every check passes.
#include <hip/hip_runtime.h>

#include "launch.h"

using namespace gdn;

namespace {

constexpr int64_t kMaxTokens = 0x7fffffffLL;  // cu_seqlens is int32

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t esize(gdn_dtype d) { return d == GDN_FP32 ? 4 : 2; }
bool dtype_ok(gdn_dtype d) { return d == GDN_BF16 || d == GDN_FP32 || d == GDN_FP16; }

gdn_status check_shape(const gdn_shape* s) {
  if (!s) return GDN_ERR_INVALID_ARG;
  if (s->n_seq < 1 || s->total_tokens < 0 || s->total_tokens > kMaxTokens || s->hk < 1 ||
      s->hv < 1 || s->dk < 1 || s->dv < 1 || !dtype_ok(s->dtype))
    return GDN_ERR_INVALID_ARG;
  if (s->hv % s->hk != 0) return GDN_ERR_INVALID_ARG;
  if (s->dk != s->dv || (s->dk != 32 && s->dk != 128)) return GDN_ERR_UNSUPPORTED;
  if (s->conv_k != 4 || s->chunk != CHUNK) return GDN_ERR_UNSUPPORTED;
  if (s->hv > 256 || s->n_seq > 65535) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

int64_t channels(const gdn_shape* s) { return 2LL * s->hk * s->dk + (int64_t)s->hv * s->dv; }

gdn_status check_ld(int64_t ld, int64_t min_cols) {
  if (ld < min_cols) return GDN_ERR_INVALID_ARG;
  if (ld % 8) return GDN_ERR_ALIGNMENT;
  return GDN_OK;
}

gdn_status check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    if (!p) return GDN_ERR_INVALID_ARG;
    if (!aligned16(p)) return GDN_ERR_ALIGNMENT;
  }
  return GDN_OK;
}

gdn_status chunk_supported(const gdn_shape* s) {
  // fp32 storage is supported at head dim 32 (the fp32 workload); bf16 and fp16 at 32 and 128
  if (s->dtype == GDN_FP32 && s->dk != 32) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

gdn_status launched(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH; }

#define GDN_TRY(x)                   \
  do {                               \
    gdn_status _st = (x);            \
    if (_st != GDN_OK) return _st;   \
  } while (0)

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported configuration";
    case GDN_ERR_ALIGNMENT: return "pointer or row stride not 16-byte aligned";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

gdn_status gdn_conv_fwd(const gdn_shape* s, const void* x, int64_t ldx, const float* w,
                        const int32_t* cu, int l2norm_qk, float l2_eps, void* y, int64_t ldy,
                        void* stream) {
  GDN_TRY(check_shape(s));
  GDN_TRY(check_ptrs({x, w, cu, y}));
  GDN_TRY(check_ld(ldx, channels(s)));
  GDN_TRY(check_ld(ldy, channels(s)));
  if (!(l2_eps >= 0.f)) return GDN_ERR_INVALID_ARG;
  return launched(launch_conv_fwd(*s, x, ldx, w, cu, l2norm_qk != 0, l2_eps, y, ldy, nullptr,
                                  nullptr, (hipStream_t)stream));
}

size_t gdn_conv_bwd_workspace(const gdn_shape* s) {
  if (check_shape(s) != GDN_OK) return 0;
  return sizeof(float) * (size_t)conv_partials(s->total_tokens, conv_tt(s->total_tokens, channels(s))) *
         (size_t)channels(s) * 4;
}

gdn_status gdn_conv_bwd(const gdn_shape* s, const void* x, int64_t ldx, const float* w,
                        const int32_t* cu, int l2norm_qk, float l2_eps, const void* dy,
                        int64_t lddy, void* dx, int64_t lddx, float* dw, void* ws,
                        size_t ws_bytes, void* stream) {
  GDN_TRY(check_shape(s));
  GDN_TRY(check_ptrs({x, w, cu, dy, dx, dw}));
  GDN_TRY(check_ld(ldx, channels(s)));
  GDN_TRY(check_ld(lddy, channels(s)));
  GDN_TRY(check_ld(lddx, channels(s)));
  if (!(l2_eps >= 0.f)) return GDN_ERR_INVALID_ARG;
  const size_t need = gdn_conv_bwd_workspace(s);
  if (need && (!ws || ws_bytes < need || !aligned16(ws))) return GDN_ERR_WORKSPACE;
  return launched(launch_conv_bwd(*s, x, ldx, w, cu, l2norm_qk != 0, l2_eps, dy, lddy, dx, lddx,
                                  dw, (float*)ws, nullptr, nullptr, nullptr, (hipStream_t)stream));
}

gdn_status gdn_conv_fwd_state(const gdn_shape* s, const void* x, int64_t ldx, const float* w,
                              const int32_t* cu, int l2norm_qk, float l2_eps,
                              const void* conv_state_in, void* y, int64_t ldy,
                              void* conv_state_out, void* stream) {
  GDN_TRY(check_shape(s));
  GDN_TRY(check_ptrs({x, w, cu, y}));
  GDN_TRY(check_ld(ldx, channels(s)));
  GDN_TRY(check_ld(ldy, channels(s)));
  if ((conv_state_in && !aligned16(conv_state_in)) || (conv_state_out && !aligned16(conv_state_out)))
    return GDN_ERR_ALIGNMENT;
  if (!(l2_eps >= 0.f)) return GDN_ERR_INVALID_ARG;
  return launched(launch_conv_fwd(*s, x, ldx, w, cu, l2norm_qk != 0, l2_eps, y, ldy, conv_state_in,
                                  conv_state_out, (hipStream_t)stream));
}

gdn_status gdn_conv_bwd_state(const gdn_shape* s, const void* x, int64_t ldx, const float* w,
                              const int32_t* cu, int l2norm_qk, float l2_eps,
                              const void* conv_state_in, const void* dy, int64_t lddy,
                              const void* d_conv_state_out, void* dx, int64_t lddx, float* dw,
                              void* d_conv_state_in, void* ws, size_t ws_bytes, void* stream) {
  GDN_TRY(check_shape(s));
  GDN_TRY(check_ptrs({x, w, cu, dy, dx, dw}));
  GDN_TRY(check_ld(ldx, channels(s)));
  GDN_TRY(check_ld(lddy, channels(s)));
  GDN_TRY(check_ld(lddx, channels(s)));
  for (const void* p : {conv_state_in, d_conv_state_out, (const void*)d_conv_state_in})
    if (p && !aligned16(p)) return GDN_ERR_ALIGNMENT;
  if (!(l2_eps >= 0.f)) return GDN_ERR_INVALID_ARG;
  const size_t need = gdn_conv_bwd_workspace(s);
  if (need && (!ws || ws_bytes < need || !aligned16(ws))) return GDN_ERR_WORKSPACE;
  return launched(launch_conv_bwd(*s, x, ldx, w, cu, l2norm_qk != 0, l2_eps, dy, lddy, dx, lddx,
                                  dw, (float*)ws, conv_state_in, d_conv_state_out, d_conv_state_in,
                                  (hipStream_t)stream));
}

gdn_status gdn_conv_bwd_noalloc(const gdn_shape* s, const void* x, int64_t ldx, const float* w,
                                const int32_t* cu, int l2norm_qk, float l2_eps, const void* dy,
                                int64_t lddy, void* dx, int64_t lddx, float* dw, void* stream) {
  GDN_TRY(check_shape(s));
  GDN_TRY(check_ptrs({x, w, cu, dy, dx, dw}));
  GDN_TRY(check_ld(ldx, channels(s)));
  GDN_TRY(check_ld(lddy, channels(s)));
  GDN_TRY(check_ld(lddx, channels(s)));
  if (!(l2_eps >= 0.f)) return GDN_ERR_INVALID_ARG;
  if (gdn_conv_bwd_workspace(s) > CONV_BWD_NOALLOC_MAX_BYTES) return GDN_ERR_WORKSPACE;
  return launched(launch_conv_bwd_noalloc(*s, x, ldx, w, cu, l2norm_qk != 0, l2_eps, dy, lddy,
                                          dx, lddx, dw, (hipStream_t)stream));
}

gdn_status gdn_gate_fwd(const gdn_shape* s, const void* a, const void* b, const float* A_log,
                        const float* dt_bias, float* g, float* beta, void* stream) {
  GDN_TRY(check_shape(s));
  if (!a || !b || !A_log || !dt_bias || !g || !beta) return GDN_ERR_INVALID_ARG;
  return launched(launch_gate_fwd(*s, a, b, A_log, dt_bias, g, beta, (hipStream_t)stream));
}

size_t gdn_gate_bwd_workspace(const gdn_shape* s) {
  if (check_shape(s) != GDN_OK) return 0;
  return sizeof(float) * (size_t)gate_partials(s->total_tokens) * 2 * (size_t)s->hv;
}

gdn_status gdn_gate_bwd(const gdn_shape* s, const void* a, const void* b, const float* A_log,
                        const float* dt_bias, const float* dg, const float* dbeta, void* da,
                        void* db, float* dA_log, float* ddt_bias, void* ws, size_t ws_bytes,
                        void* stream) {
  GDN_TRY(check_shape(s));
  if (!a || !b || !A_log || !dt_bias || !dg || !dbeta || !da || !db || !dA_log || !ddt_bias)
    return GDN_ERR_INVALID_ARG;
  const size_t need = gdn_gate_bwd_workspace(s);
  if (need && (!ws || ws_bytes < need || !aligned16(ws))) return GDN_ERR_WORKSPACE;
  return launched(launch_gate_bwd(*s, a, b, A_log, dt_bias, dg, dbeta, da, db, dA_log, ddt_bias,
                                  (float*)ws, (hipStream_t)stream));
}

size_t gdn_chunk_fwd_workspace(const gdn_shape* s) {
  if (check_shape(s) != GDN_OK) return 0;
  return chunk_fwd_ws_bytes(*s);
}

size_t gdn_chunk_bwd_workspace(const gdn_shape* s) {
  if (check_shape(s) != GDN_OK) return 0;
  return chunk_bwd_ws_bytes(*s);
}

gdn_status gdn_chunk_fwd(const gdn_shape* s, const void* q, const void* k, const void* v,
                         int64_t ldq, int64_t ldk, int64_t ldv, const float* g,
                         const float* beta, float scale, const float* S0, float* S_final,
                         const int32_t* cu, void* o, void* ws, size_t ws_bytes, void* stream) {
  GDN_TRY(check_shape(s));
  GDN_TRY(chunk_supported(s));
  GDN_TRY(check_ptrs({q, k, v, o, ws}));
  if (!g || !beta || !cu) return GDN_ERR_INVALID_ARG;
  if ((S0 && !aligned16(S0)) || (S_final && !aligned16(S_final))) return GDN_ERR_ALIGNMENT;
  GDN_TRY(check_ld(ldq, (int64_t)s->hk * s->dk));
  GDN_TRY(check_ld(ldk, (int64_t)s->hk * s->dk));
  GDN_TRY(check_ld(ldv, (int64_t)s->hv * s->dv));
  if (ws_bytes < chunk_fwd_ws_bytes(*s)) return GDN_ERR_WORKSPACE;
  return launched(launch_chunk_fwd(*s, q, k, v, ldq, ldk, ldv, g, beta, scale, S0, S_final, cu, o,
                                   ws, (hipStream_t)stream));
}

gdn_status gdn_chunk_bwd(const gdn_shape* s, const void* q, const void* k, const void* v,
                         int64_t ldq, int64_t ldk, int64_t ldv, const float* g,
                         const float* beta, float scale, const float* S0, const int32_t* cu,
                         const void* dout, const float* dS_final, void* dq, void* dk, void* dv,
                         int64_t lddq, int64_t lddk, int64_t lddv, float* dg, float* dbeta,
                         float* dS0, void* ws, size_t ws_bytes, void* stream) {
  GDN_TRY(check_shape(s));
  GDN_TRY(chunk_supported(s));
  GDN_TRY(check_ptrs({q, k, v, dout, dq, dk, dv, ws}));
  if (!g || !beta || !cu || !dg || !dbeta) return GDN_ERR_INVALID_ARG;
  if ((S0 && !aligned16(S0)) || (dS_final && !aligned16(dS_final)) || (dS0 && !aligned16(dS0)))
    return GDN_ERR_ALIGNMENT;
  GDN_TRY(check_ld(ldq, (int64_t)s->hk * s->dk));
  GDN_TRY(check_ld(ldk, (int64_t)s->hk * s->dk));
  GDN_TRY(check_ld(ldv, (int64_t)s->hv * s->dv));
  GDN_TRY(check_ld(lddq, (int64_t)s->hk * s->dk));
  GDN_TRY(check_ld(lddk, (int64_t)s->hk * s->dk));
  GDN_TRY(check_ld(lddv, (int64_t)s->hv * s->dv));
  if (ws_bytes < chunk_bwd_ws_bytes(*s)) return GDN_ERR_WORKSPACE;
  return launched(launch_chunk_bwd(*s, q, k, v, ldq, ldk, ldv, g, beta, scale, S0, cu, dout,
                                   dS_final, dq, dk, dv, lddq, lddk, lddv, dg, dbeta, dS0, ws,
                                   (hipStream_t)stream));
}

// ---- chunk phases -----------------------------------------------------------
namespace {
gdn_status check_chunk_common(const gdn_shape* s, const void* q, const void* k, int64_t ldq,
                              int64_t ldk, const void* cu, const void* ws, size_t ws_bytes,
                              size_t need) {
  GDN_TRY(check_shape(s));
  GDN_TRY(chunk_supported(s));
  GDN_TRY(check_ptrs({q, k, ws}));
  if (!cu) return GDN_ERR_INVALID_ARG;
  GDN_TRY(check_ld(ldq, (int64_t)s->hk * s->dk));
  GDN_TRY(check_ld(ldk, (int64_t)s->hk * s->dk));
  if (ws_bytes < need) return GDN_ERR_WORKSPACE;
  return GDN_OK;
}
}  // namespace

gdn_status gdn_chunk_prepare(const gdn_shape* s, const void* q, const void* k, int64_t ldq,
                             int64_t ldk, const float* g, const float* beta, float scale,
                             const int32_t* cu, void* ws, size_t ws_bytes, void* stream) {
  GDN_TRY(check_chunk_common(s, q, k, ldq, ldk, cu, ws, ws_bytes,
                             s ? chunk_fwd_ws_bytes(*s) : 0));
  if (!g || !beta) return GDN_ERR_INVALID_ARG;
  return launched(launch_chunk_prepare(*s, q, k, ldq, ldk, g, beta, scale, cu, ws, false,
                                       (hipStream_t)stream));
}

gdn_status gdn_chunk_prepare_bwd(const gdn_shape* s, const void* q, const void* k, int64_t ldq,
                                 int64_t ldk, const float* g, const float* beta, float scale,
                                 const int32_t* cu, void* ws, size_t ws_bytes, void* stream) {
  GDN_TRY(check_chunk_common(s, q, k, ldq, ldk, cu, ws, ws_bytes,
                             s ? chunk_bwd_ws_bytes(*s) : 0));
  if (!g || !beta) return GDN_ERR_INVALID_ARG;
  return launched(launch_chunk_prepare(*s, q, k, ldq, ldk, g, beta, scale, cu, ws, true,
                                       (hipStream_t)stream));
}

gdn_status gdn_chunk_fwd_states(const gdn_shape* s, const void* q, const void* k, const void* v,
                                int64_t ldq, int64_t ldk, int64_t ldv, float scale,
                                const float* S0, float* S_final, const int32_t* cu, void* o,
                                void* ws, size_t ws_bytes, void* stream) {
  GDN_TRY(check_chunk_common(s, q, k, ldq, ldk, cu, ws, ws_bytes,
                             s ? chunk_fwd_ws_bytes(*s) : 0));
  GDN_TRY(check_ptrs({v, o}));
  GDN_TRY(check_ld(ldv, (int64_t)s->hv * s->dv));
  if ((S0 && !aligned16(S0)) || (S_final && !aligned16(S_final))) return GDN_ERR_ALIGNMENT;
  return launched(launch_chunk_fwd_states(*s, q, k, v, ldq, ldk, ldv, scale, S0, S_final, cu, o,
                                          ws, (hipStream_t)stream));
}

gdn_status gdn_chunk_fwd_states_save(const gdn_shape* s, const void* q, const void* k,
                                     const void* v, int64_t ldq, int64_t ldk, int64_t ldv,
                                     float scale, const float* S0, float* S_final,
                                     const int32_t* cu, void* o, void* ws, size_t ws_bytes,
                                     void* stream) {
  GDN_TRY(check_chunk_common(s, q, k, ldq, ldk, cu, ws, ws_bytes,
                             s ? chunk_bwd_ws_bytes(*s) : 0));
  GDN_TRY(check_ptrs({v, o}));
  GDN_TRY(check_ld(ldv, (int64_t)s->hv * s->dv));
  if ((S0 && !aligned16(S0)) || (S_final && !aligned16(S_final))) return GDN_ERR_ALIGNMENT;
  return launched(launch_chunk_fwd_states_save(*s, q, k, v, ldq, ldk, ldv, scale, S0, S_final, cu,
                                               o, ws, (hipStream_t)stream));
}

gdn_status gdn_chunk_bwd_states(const gdn_shape* s, const void* q, const void* k, const void* v,
                                int64_t ldq, int64_t ldk, int64_t ldv, float scale,
                                const float* S0, const int32_t* cu, void* ws, size_t ws_bytes,
                                void* stream) {
  GDN_TRY(check_chunk_common(s, q, k, ldq, ldk, cu, ws, ws_bytes,
                             s ? chunk_bwd_ws_bytes(*s) : 0));
  GDN_TRY(check_ptrs({v}));
  GDN_TRY(check_ld(ldv, (int64_t)s->hv * s->dv));
  if (S0 && !aligned16(S0)) return GDN_ERR_ALIGNMENT;
  return launched(launch_chunk_bwd_states(*s, q, k, v, ldq, ldk, ldv, scale, S0, cu, ws,
                                          (hipStream_t)stream));
}

gdn_status gdn_chunk_bwd_reverse(const gdn_shape* s, const void* q, const void* k, int64_t ldq,
                                 int64_t ldk, float scale, const int32_t* cu, const void* dout,
                                 const float* dS_final, void* dv, int64_t lddv, float* dS0,
                                 void* ws, size_t ws_bytes, void* stream) {
  GDN_TRY(check_chunk_common(s, q, k, ldq, ldk, cu, ws, ws_bytes,
                             s ? chunk_bwd_ws_bytes(*s) : 0));
  GDN_TRY(check_ptrs({dout, dv}));
  GDN_TRY(check_ld(lddv, (int64_t)s->hv * s->dv));
  if ((dS_final && !aligned16(dS_final)) || (dS0 && !aligned16(dS0))) return GDN_ERR_ALIGNMENT;
  return launched(launch_chunk_bwd_reverse(*s, q, k, ldq, ldk, scale, cu, dout, dS_final, dv, lddv,
                                           dS0, ws, (hipStream_t)stream));
}

gdn_status gdn_chunk_bwd_grads(const gdn_shape* s, const void* q, const void* k, int64_t ldq,
                               int64_t ldk, const float* beta, float scale, const int32_t* cu,
                               const void* dout, const void* dv, int64_t lddv, void* dq, void* dk,
                               int64_t lddq, int64_t lddk, float* dg, float* dbeta, void* ws,
                               size_t ws_bytes, void* stream) {
  GDN_TRY(check_chunk_common(s, q, k, ldq, ldk, cu, ws, ws_bytes,
                             s ? chunk_bwd_ws_bytes(*s) : 0));
  GDN_TRY(check_ptrs({dout, dv, dq, dk}));
  if (!beta || !dg || !dbeta) return GDN_ERR_INVALID_ARG;
  GDN_TRY(check_ld(lddv, (int64_t)s->hv * s->dv));
  GDN_TRY(check_ld(lddq, (int64_t)s->hk * s->dk));
  GDN_TRY(check_ld(lddk, (int64_t)s->hk * s->dk));
  return launched(launch_chunk_bwd_grads(*s, q, k, ldq, ldk, beta, scale, cu, dout, dv, lddv, dq,
                                         dk, lddq, lddk, dg, dbeta, ws, (hipStream_t)stream));
}

gdn_status gdn_gated_norm_fwd(int64_t rows, int32_t dv, gdn_dtype dt, const void* o, const void* z,
                              const float* w, float eps, gdn_act act, void* y, void* stream) {
  if (rows < 0 || !dtype_ok(dt) || (act != GDN_ACT_SILU && act != GDN_ACT_SIGMOID))
    return GDN_ERR_INVALID_ARG;
  if (dv != 32 && dv != 128) return GDN_ERR_UNSUPPORTED;
  GDN_TRY(check_ptrs({o, z, w, y}));
  if (!(eps >= 0.f)) return GDN_ERR_INVALID_ARG;
  return launched(launch_norm_fwd(rows, dv, dt, o, z, w, eps, (int)act, y, (hipStream_t)stream));
}

size_t gdn_gated_norm_bwd_workspace(int64_t rows, int32_t dv) {
  if (rows < 0 || (dv != 32 && dv != 128)) return 0;
  return sizeof(float) * (size_t)norm_blocks(rows, dv) * (size_t)dv;
}

gdn_status gdn_gated_norm_bwd(int64_t rows, int32_t dv, gdn_dtype dt, const void* o, const void* z,
                              const float* w, float eps, gdn_act act, const void* dy, void* dout,
                              void* dz, float* dw, void* ws, size_t ws_bytes, void* stream) {
  if (rows < 0 || !dtype_ok(dt) || (act != GDN_ACT_SILU && act != GDN_ACT_SIGMOID))
    return GDN_ERR_INVALID_ARG;
  if (dv != 32 && dv != 128) return GDN_ERR_UNSUPPORTED;
  GDN_TRY(check_ptrs({o, z, w, dy, dout, dz, dw}));
  if (!(eps >= 0.f)) return GDN_ERR_INVALID_ARG;
  const size_t need = gdn_gated_norm_bwd_workspace(rows, dv);
  if (!ws || ws_bytes < need || !aligned16(ws)) return GDN_ERR_WORKSPACE;
  return launched(launch_norm_bwd(rows, dv, dt, o, z, w, eps, (int)act, dy, dout, dz, dw,
                                  (float*)ws, (hipStream_t)stream));
}

gdn_status gdn_check_cu_seqlens(const gdn_shape* s, const int32_t* cu, int32_t* violations,
                                void* stream) {
  GDN_TRY(check_shape(s));
  if (!cu || !violations) return GDN_ERR_INVALID_ARG;
  if (((uintptr_t)violations & 3u) != 0) return GDN_ERR_ALIGNMENT;
  return launched(gdn::launch_check_cu(*s, cu, violations, (hipStream_t)stream));
}

}  // extern "C"
