// Internal launchers (host side).  The exported C entry points in api.hip
// validate arguments and then call these; launchers assume valid input.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/libgdn.h"

namespace gdn {

// out[i] = sum over p of partials[p * width + i], added in a fixed order
hipError_t launch_reduce_partials(const float* partials, int64_t n_part, int64_t width, float* out,
                                  hipStream_t st);
// as above, with columns i >= split written to out1[i - split]
hipError_t launch_reduce_partials(const float* partials, int64_t n_part, int64_t width,
                                  float* out0, int64_t split, float* out1, hipStream_t st);

constexpr int CONV_RUNS_PER_BLOCK = 4;
constexpr int CHUNK = 64;

// Tokens per conv run (one wave): the longest of 256, 128, 64 that still
// gives 4096 runs x channel groups (16 waves per CU); longer runs stream
// better (at 65536 tokens x 10240 channels: 256 tokens, conv_bwd 0.88 -> 0.83
// ms), shorter ones keep small inputs spread over the chip.
inline int conv_tt(int64_t T, int C) {
  const int64_t groups = (C / 8 + 63) / 64;
  for (int tt = 256; tt > 64; tt /= 2)
    if ((T + tt - 1) / tt * groups >= 4096) return tt;
  return 64;
}
inline int64_t conv_runs(int64_t T, int tt) { return (T + tt - 1) / tt; }
inline int64_t conv_partials(int64_t T, int tt) {
  return (conv_runs(T, tt) + CONV_RUNS_PER_BLOCK - 1) / CONV_RUNS_PER_BLOCK;
}

// cs_in, cs_out, dcs_out, dcs_in: carried conv states [n_seq][3][C] (nullable)
hipError_t launch_conv_fwd(const gdn_shape& s, const void* x, int64_t ldx, const float* w,
                           const int32_t* cu, int l2, float eps, void* y, int64_t ldy,
                           const void* cs_in, void* cs_out, hipStream_t st);
hipError_t launch_conv_bwd(const gdn_shape& s, const void* x, int64_t ldx, const float* w,
                           const int32_t* cu, int l2, float eps, const void* dy, int64_t lddy,
                           void* dx, int64_t lddx, float* dw, float* partials, const void* cs_in,
                           const void* dcs_out, void* dcs_in, hipStream_t st);

constexpr size_t CONV_BWD_NOALLOC_MAX_BYTES = GDN_CONV_BWD_NOALLOC_MAX_BYTES;
// the conv backward into the library's own scratch (no workspace argument);
// partials of at most CONV_BWD_NOALLOC_MAX_BYTES
hipError_t launch_conv_bwd_noalloc(const gdn_shape& s, const void* x, int64_t ldx, const float* w,
                                   const int32_t* cu, int l2, float eps, const void* dy,
                                   int64_t lddy, void* dx, int64_t lddx, float* dw,
                                   hipStream_t st);

constexpr int GATE_TB = 64;      // tokens per gate-backward block
inline int64_t gate_partials(int64_t T) { return (T + GATE_TB - 1) / GATE_TB; }
hipError_t launch_gate_fwd(const gdn_shape& s, const void* a, const void* b, const float* A_log,
                           const float* dt_bias, float* g, float* beta, hipStream_t st);
hipError_t launch_gate_bwd(const gdn_shape& s, const void* a, const void* b, const float* A_log,
                           const float* dt_bias, const float* dg, const float* dbeta, void* da,
                           void* db, float* dA_log, float* ddt_bias, float* partials,
                           hipStream_t st);

constexpr int NORM_BLOCKS_MAX = 512;   // best of 256..4096 measured at 65536 tokens x 48 heads
int64_t norm_blocks(int64_t rows, int32_t dv);
hipError_t launch_norm_fwd(int64_t rows, int32_t dv, gdn_dtype dt, const void* o, const void* z,
                           const float* w, float eps, int act, void* y, hipStream_t st);
hipError_t launch_norm_bwd(int64_t rows, int32_t dv, gdn_dtype dt, const void* o, const void* z,
                           const float* w, float eps, int act, const void* dy, void* dout,
                           void* dz, float* dw, float* partials, hipStream_t st);

// Chunked gated delta rule.
struct ChunkWs;  // layout of the chunk workspace (chunk.hip)
size_t chunk_fwd_ws_bytes(const gdn_shape& s);
size_t chunk_bwd_ws_bytes(const gdn_shape& s);
hipError_t launch_chunk_fwd(const gdn_shape& s, const void* q, const void* k, const void* v,
                            int64_t ldq, int64_t ldk, int64_t ldv, const float* g,
                            const float* beta, float scale, const float* S0, float* S_final,
                            const int32_t* cu, void* o, void* ws, hipStream_t st);
// bwd: also write the operands of the reverse pass (backward workspace)
hipError_t launch_chunk_prepare(const gdn_shape& s, const void* q, const void* k, int64_t ldq,
                                int64_t ldk, const float* g, const float* beta, float scale,
                                const int32_t* cu, void* ws, bool bwd, hipStream_t st);
hipError_t launch_chunk_fwd_states(const gdn_shape& s, const void* q, const void* k, const void* v,
                                   int64_t ldq, int64_t ldk, int64_t ldv, float scale,
                                   const float* S0, float* S_final, const int32_t* cu, void* o,
                                   void* ws, hipStream_t st);
hipError_t launch_chunk_fwd_states_save(const gdn_shape& s, const void* q, const void* k,
                                        const void* v, int64_t ldq, int64_t ldk, int64_t ldv,
                                        float scale, const float* S0, float* S_final,
                                        const int32_t* cu, void* o, void* ws, hipStream_t st);
// R, Delta (and O when o is given) from the saved chunk-start states
hipError_t launch_chunk_outputs(const gdn_shape& s, const void* q, const void* k, const void* v,
                                int64_t ldq, int64_t ldk, int64_t ldv, float scale,
                                const int32_t* cu, void* o, void* ws, hipStream_t st);
hipError_t launch_chunk_bwd_states(const gdn_shape& s, const void* q, const void* k, const void* v,
                                   int64_t ldq, int64_t ldk, int64_t ldv, float scale,
                                   const float* S0, const int32_t* cu, void* ws, hipStream_t st);
hipError_t launch_chunk_bwd_reverse(const gdn_shape& s, const void* q, const void* k, int64_t ldq,
                                    int64_t ldk, float scale, const int32_t* cu, const void* dout,
                                    const float* dS_final, void* dv, int64_t lddv, float* dS0,
                                    void* ws, hipStream_t st);
hipError_t launch_chunk_bwd_grads(const gdn_shape& s, const void* q, const void* k, int64_t ldq,
                                  int64_t ldk, const float* beta, float scale, const int32_t* cu,
                                  const void* dout, const void* dv, int64_t lddv, void* dq,
                                  void* dk, int64_t lddq, int64_t lddk, float* dg, float* dbeta,
                                  void* ws, hipStream_t st);
hipError_t launch_chunk_bwd(const gdn_shape& s, const void* q, const void* k, const void* v,
                            int64_t ldq, int64_t ldk, int64_t ldv, const float* g,
                            const float* beta, float scale, const float* S0, const int32_t* cu,
                            const void* dout, const float* dS_final, void* dq, void* dk, void* dv,
                            int64_t lddq, int64_t lddk, int64_t lddv, float* dg, float* dbeta,
                            float* dS0, void* ws, hipStream_t st);

hipError_t launch_check_cu(const gdn_shape& s, const int32_t* cu, int32_t* out, hipStream_t st);

}  // namespace gdn
