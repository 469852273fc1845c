// Chunked gated delta rule: chunk table, WY/UT preparation and the
// sequential state pass (forward outputs, or the states the backward needs).
#include "chunk_common.h"

namespace gdn {

// seq_off[n] = number of 64-token chunks of sequences 0..n-1 (one block scan).
__global__ void __launch_bounds__(256) chunk_table_kernel(const int32_t* __restrict__ cu, int n_seq,
                                                          int32_t* __restrict__ seq_off) {
  __shared__ int32_t buf[256];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < n_seq; base += 256) {
    const int n = base + tid;
    int32_t v = 0;
    if (n < n_seq) {
      const int32_t len = cu[n + 1] - cu[n];
      v = (len + CHUNK - 1) / CHUNK;
    }
    buf[tid] = v;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {  // Hillis-Steele inclusive scan
      int32_t y = tid >= off ? buf[tid - off] : 0;
      __syncthreads();
      buf[tid] += y;
      __syncthreads();
    }
    if (n < n_seq) seq_off[n] = carry + buf[tid] - v;
    __syncthreads();
    if (tid == 255) carry += buf[255];
    __syncthreads();
  }
  if (tid == 0) seq_off[n_seq] = carry;
}

// ---------------------------------------------------------------------------
// Preparation, one workgroup per (chunk, key head): K K^T and Q K^T once
// (MFMA), then per value head of the group: gam, A, Tinv (fp32), and the
// MFMA operands M = Tinv diag(beta) and P written to the workspace.
template <typename T, int D>
struct PrepSmem {
  typedef typename Compute<T>::type CT;
  CT K[CHUNK][D + Pad<CT>::v];
  CT Q[CHUNK][D + Pad<CT>::v];
  float A[CHUNK][68];
  float Ti[CHUNK][68];
  float X[16][17];
  double gam[CHUNK];
  float bet[CHUNK];
};

template <typename T, int D>
__global__ void __launch_bounds__(256) chunk_prep_kernel(
    const T* __restrict__ q, const T* __restrict__ k, int64_t ldq, int64_t ldk,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ seq_off, int n_seq, int Hv, int G, float scale,
    double* __restrict__ gcum, typename Compute<T>::type* __restrict__ Mw,
    typename Compute<T>::type* __restrict__ Pw) {
  typedef typename Compute<T>::type CT;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  PrepSmem<T, D>& sm = *reinterpret_cast<PrepSmem<T, D>*>(smem_raw);
  constexpr int LD = D + Pad<CT>::v;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c = blockIdx.x;
  const int kh = blockIdx.y;
  if (c >= seq_off[n_seq]) return;
  int64_t t0;
  int L;
  chunk_span(seq_off, cu, n_seq, c, t0, L);

  stage_rows<CT, D>(&sm.K[0][0], LD, k + t0 * ldk + (int64_t)kh * D, ldk, L, tid);
  stage_rows<CT, D>(&sm.Q[0][0], LD, q + t0 * ldq + (int64_t)kh * D, ldq, L, tid);
  __syncthreads();

  // wave w owns rows [16w, 16w+16) of the 64 x 64 products
  floatx4 kk[4], qk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kk[j] = tile_mma<CT, true, true>(zero4(), &sm.K[0][0], LD, &sm.K[0][0], LD, 16 * wave, 16 * j, D, lane);
    qk[j] = tile_mma<CT, true, true>(zero4(), &sm.Q[0][0], LD, &sm.K[0][0], LD, 16 * wave, 16 * j, D, lane);
  }
  const int rbase = 16 * wave + 4 * (lane >> 4);
  const int ccol = lane & 15;

  for (int hh = 0; hh < G; ++hh) {
    const int h = kh * G + hh;
    if (wave == 0) {
      const double gl = lane < L ? (double)g[(t0 + lane) * Hv + h] : 0.0;
      const float bl = lane < L ? beta[(t0 + lane) * Hv + h] : 0.f;
      const double gm = wave_incl_scan(gl, lane);
      sm.gam[lane] = gm;
      sm.bet[lane] = bl;
      if (lane < L) gcum[(t0 + lane) * Hv + h] = gm;
    }
    __syncthreads();
    CT* Pout = Pw + ((int64_t)c * Hv + h) * CHUNK * CHUNK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = 16 * j + ccol;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = rbase + e;
        const float dec = dexp<T>(sm.gam[t] - sm.gam[s <= t ? s : t]);  // masked before exp
        sm.A[t][s] = (s < t) ? sm.bet[t] * dec * kk[j][e] : 0.f;
        Pout[t * CHUNK + s] = from_f<CT>((s <= t) ? dec * scale * qk[j][e] : 0.f);
      }
    }
    __syncthreads();
    invert_unit_lower(sm.A, sm.Ti, sm.X, tid);
    CT* Mout = Mw + ((int64_t)c * Hv + h) * CHUNK * CHUNK;
    for (int i = tid; i < CHUNK * 8; i += 256) {
      const int t = i >> 3, s8 = (i & 7) * 8;
      f8 v;
#pragma unroll
      for (int u = 0; u < 8; ++u) v.v[u] = sm.Ti[t][s8 + u] * sm.bet[s8 + u];
      store8(Mout + t * CHUNK + s8, v);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Sequential state pass, one workgroup per (value-row block, value head,
// sequence).  The state block S[vb*BV : vb*BV+BV, :] lives in MFMA
// accumulators as S^T tiles (d_k rows x BV columns) for the whole sequence;
// each chunk stages K (and Q) in LDS and reads M, P rows straight from the
// workspace.
//   MODE 0 (forward): writes o and S_final.
//   MODE 1 (backward recompute): writes the chunk-start states h ([dk][dv]
//   per chunk and head), R and Delta.
template <typename T, int D, int BV>
struct StateSmem {
  typedef typename Compute<T>::type CT;
  CT K[CHUNK][D + Pad<CT>::v];
  CT Q[CHUNK][D + Pad<CT>::v];
  CT V[CHUNK][BV + Pad<CT>::v];
  CT Sb[BV][D + Pad<CT>::v];       // S block (v-major), MFMA B operand of K S^T
  CT Rt[BV][CHUNK + Pad<CT>::v];   // R^T
  CT Dt[BV][CHUNK + Pad<CT>::v];   // Delta^T
  CT Dst[BV][CHUNK + Pad<CT>::v];  // (diag(dec) Delta)^T
  double gam[CHUNK];
};

template <typename T, int D, int BV, int MODE>
__global__ void __launch_bounds__(256) chunk_state_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t ldq,
    int64_t ldk, int64_t ldv, const int32_t* __restrict__ cu, const int32_t* __restrict__ seq_off,
    int Hv, int G, float scale, const double* __restrict__ gcum,
    const typename Compute<T>::type* __restrict__ Mw, const typename Compute<T>::type* __restrict__ Pw,
    const float* __restrict__ S0, float* __restrict__ S_final, T* __restrict__ o,
    T* __restrict__ hst, T* __restrict__ Rw, T* __restrict__ Dlw) {
  typedef typename Compute<T>::type CT;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  StateSmem<T, D, BV>& sm = *reinterpret_cast<StateSmem<T, D, BV>*>(smem_raw);
  constexpr int LD = D + Pad<CT>::v, LDV = BV + Pad<CT>::v, LDC = CHUNK + Pad<CT>::v;
  constexpr int NVT = BV / 16;                      // value tiles
  constexpr int NS = (D / 16) * NVT / 4;            // state tiles per wave
  constexpr int NA = (CHUNK / 16) * NVT / 4;        // token x value tiles per wave
  static_assert(NS >= 1 && NA >= 1, "tile split");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int vb = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
  const int kh = h / G;
  const int v0 = vb * BV;
  const int rsub = 4 * (lane >> 4), ccol = lane & 15;
  const int64_t HvD = (int64_t)Hv * D;

  floatx4 S[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int id = wave * NS + i, kt = id / NVT, vt = id % NVT;
    const int vv = v0 + 16 * vt + ccol;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kk = 16 * kt + rsub + e;
      S[i][e] = S0 ? S0[(((int64_t)n * Hv + h) * D + vv) * D + kk] : 0.f;
    }
  }

  const int64_t c_begin = seq_off[n], c_end = seq_off[n + 1];
  for (int64_t c = c_begin; c < c_end; ++c) {
    const int64_t t0 = (int64_t)cu[n] + CHUNK * (c - c_begin);
    const int L = (int64_t)cu[n + 1] - t0 < CHUNK ? (int)((int64_t)cu[n + 1] - t0) : CHUNK;
    __syncthreads();
    stage_rows<CT, D>(&sm.K[0][0], LD, k + t0 * ldk + (int64_t)kh * D, ldk, L, tid);
    if (MODE == 0) stage_rows<CT, D>(&sm.Q[0][0], LD, q + t0 * ldq + (int64_t)kh * D, ldq, L, tid);
    stage_rows<CT, BV>(&sm.V[0][0], LDV, v + t0 * ldv + (int64_t)h * D + v0, ldv, L, tid);
    if (tid < CHUNK) sm.gam[tid] = gcum[(t0 + (tid < L ? tid : L - 1)) * Hv + h];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int id = wave * NS + i, kt = id / NVT, vt = id % NVT;
      const int vv = 16 * vt + ccol, kk = 16 * kt + rsub;
      store4(&sm.Sb[vv][kk], S[i][0], S[i][1], S[i][2], S[i][3]);
      if (MODE == 1) {
        T* hp = hst + (((int64_t)c * Hv + h) * D + kk) * D + v0 + vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) hp[(int64_t)e * D] = from_f<T>(S[i][e]);
      }
    }
    __syncthreads();

    // Phase A: R = V - diag(Gam) K S^T   (and the Q S^T part of O)
    floatx4 oq[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int id = wave * NA + i, tt = id / NVT, vt = id % NVT;
      floatx4 ks = tile_mma<CT, true, true>(zero4(), &sm.K[0][0], LD, &sm.Sb[0][0], LD, 16 * tt,
                                           16 * vt, D, lane);
      if (MODE == 0)
        oq[i] = tile_mma<CT, true, true>(zero4(), &sm.Q[0][0], LD, &sm.Sb[0][0], LD, 16 * tt,
                                        16 * vt, D, lane);
      const int vv = 16 * vt + ccol, tb = 16 * tt + rsub;
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float Gm = dexp<T>(sm.gam[tb + e]);
        r[e] = to_f(sm.V[tb + e][vv]) - Gm * ks[e];
        if (MODE == 0) oq[i][e] *= Gm * scale;
      }
      store4(&sm.Rt[vv][tb], r[0], r[1], r[2], r[3]);
      if (MODE == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (tb + e < L) Rw[(t0 + tb + e) * HvD + (int64_t)h * D + v0 + vv] = from_f<T>(r[e]);
      }
    }
    __syncthreads();

    // Phase B: Delta = M R
    const CT* Mc = Mw + ((int64_t)c * Hv + h) * CHUNK * CHUNK;
    const double gl = sm.gam[CHUNK - 1];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int id = wave * NA + i, tt = id / NVT, vt = id % NVT;
      floatx4 dl = tile_mma<CT, true, true>(zero4(), Mc, CHUNK, &sm.Rt[0][0], LDC, 16 * tt, 16 * vt,
                                           CHUNK, lane);
      const int vv = 16 * vt + ccol, tb = 16 * tt + rsub;
      float ds[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ds[e] = dexp<T>(gl - sm.gam[tb + e]) * dl[e];
      store4(&sm.Dt[vv][tb], dl[0], dl[1], dl[2], dl[3]);
      store4(&sm.Dst[vv][tb], ds[0], ds[1], ds[2], ds[3]);
      if (MODE == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (tb + e < L) Dlw[(t0 + tb + e) * HvD + (int64_t)h * D + v0 + vv] = from_f<T>(dl[e]);
      }
    }
    __syncthreads();

    // Phase C: O = oq + P Delta;  S^T <- Gam_L S^T + K^T (diag(dec) Delta)
    if (MODE == 0) {
      const CT* Pc = Pw + ((int64_t)c * Hv + h) * CHUNK * CHUNK;
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int id = wave * NA + i, tt = id / NVT, vt = id % NVT;
        floatx4 ov = tile_mma<CT, true, true>(oq[i], Pc, CHUNK, &sm.Dt[0][0], LDC, 16 * tt, 16 * vt,
                                             CHUNK, lane);
        const int vv = 16 * vt + ccol, tb = 16 * tt + rsub;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (tb + e < L) o[(t0 + tb + e) * HvD + (int64_t)h * D + v0 + vv] = from_f<T>(ov[e]);
      }
    }
    const float GL = dexp<T>(gl);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int id = wave * NS + i, kt = id / NVT, vt = id % NVT;
#pragma unroll
      for (int e = 0; e < 4; ++e) S[i][e] *= GL;
      S[i] = tile_mma<CT, false, true>(S[i], &sm.K[0][0], LD, &sm.Dst[0][0], LDC, 16 * kt, 16 * vt,
                                      CHUNK, lane);
    }
  }
  if (MODE == 0 && S_final) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int id = wave * NS + i, kt = id / NVT, vt = id % NVT;
      const int vv = v0 + 16 * vt + ccol, kk = 16 * kt + rsub;
      store4(S_final + (((int64_t)n * Hv + h) * D + vv) * D + kk, S[i][0], S[i][1], S[i][2], S[i][3]);
    }
  }
}

// ---------------------------------------------------------------------------
constexpr int STATE_BV = 32;  // value rows of the state owned by one workgroup

template <typename T, int D>
static hipError_t chunk_prepare(const gdn_shape& s, const void* q, const void* k, int64_t ldq,
                                int64_t ldk, const float* g, const float* beta, float scale,
                                const int32_t* cu, const ChunkLayout& Ly, char* ws,
                                hipStream_t st) {
  int32_t* seq_off = (int32_t*)(ws + Ly.seq_off);
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, st, cu, s.n_seq, seq_off);
  if (Ly.nt_max > 0 && s.total_tokens > 0) {
    const size_t shm = sizeof(PrepSmem<T, D>);
    hipFuncSetAttribute((const void*)chunk_prep_kernel<T, D>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    hipLaunchKernelGGL((chunk_prep_kernel<T, D>), dim3((unsigned)Ly.nt_max, s.hk), dim3(256), shm,
                       st, (const T*)q, (const T*)k, ldq, ldk, g, beta, cu, seq_off, s.n_seq, s.hv,
                       s.hv / s.hk, scale, (double*)(ws + Ly.gcum),
                       (typename Compute<T>::type*)(ws + Ly.mw),
                       (typename Compute<T>::type*)(ws + Ly.pw));
  }
  return hipGetLastError();
}

template <typename T, int D, int MODE>
static hipError_t chunk_state(const gdn_shape& s, const void* q, const void* k, const void* v,
                              int64_t ldq, int64_t ldk, int64_t ldv, float scale, const float* S0,
                              float* S_final, const int32_t* cu, void* o, const ChunkLayout& Ly,
                              char* ws, hipStream_t st) {
  constexpr int BV = STATE_BV;
  const size_t shm = sizeof(StateSmem<T, D, BV>);
  auto kern = chunk_state_kernel<T, D, BV, MODE>;
  hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  hipLaunchKernelGGL(kern, dim3(D / BV, s.hv, s.n_seq), dim3(256), shm, st, (const T*)q,
                     (const T*)k, (const T*)v, ldq, ldk, ldv, cu, (const int32_t*)(ws + Ly.seq_off),
                     s.hv, s.hv / s.hk, scale, (const double*)(ws + Ly.gcum),
                     (const typename Compute<T>::type*)(ws + Ly.mw),
                     (const typename Compute<T>::type*)(ws + Ly.pw), S0, S_final, (T*)o,
                     (T*)(ws + Ly.h), (T*)(ws + Ly.rw), (T*)(ws + Ly.dlw));
  return hipGetLastError();
}

size_t chunk_fwd_ws_bytes(const gdn_shape& s) { return chunk_layout(s).total_fwd; }
size_t chunk_bwd_ws_bytes(const gdn_shape& s) { return chunk_layout(s).total_bwd; }

hipError_t launch_chunk_prepare(const gdn_shape& s, const void* q, const void* k, int64_t ldq,
                                int64_t ldk, const float* g, const float* beta, float scale,
                                const int32_t* cu, void* ws, hipStream_t st) {
  const ChunkLayout Ly = chunk_layout(s);
  return dispatch_chunk(s, [&](auto c) {
    using T = typename decltype(c)::type;
    return chunk_prepare<T, decltype(c)::d>(s, q, k, ldq, ldk, g, beta, scale, cu, Ly, (char*)ws, st);
  });
}

hipError_t launch_chunk_fwd_states(const gdn_shape& s, const void* q, const void* k, const void* v,
                                   int64_t ldq, int64_t ldk, int64_t ldv, float scale,
                                   const float* S0, float* S_final, const int32_t* cu, void* o,
                                   void* ws, hipStream_t st) {
  const ChunkLayout Ly = chunk_layout(s);
  return dispatch_chunk(s, [&](auto c) {
    using T = typename decltype(c)::type;
    return chunk_state<T, decltype(c)::d, 0>(s, q, k, v, ldq, ldk, ldv, scale, S0, S_final, cu, o,
                                             Ly, (char*)ws, st);
  });
}

hipError_t launch_chunk_bwd_states(const gdn_shape& s, const void* q, const void* k, const void* v,
                                   int64_t ldq, int64_t ldk, int64_t ldv, float scale,
                                   const float* S0, const int32_t* cu, void* ws, hipStream_t st) {
  const ChunkLayout Ly = chunk_layout(s);
  return dispatch_chunk(s, [&](auto c) {
    using T = typename decltype(c)::type;
    return chunk_state<T, decltype(c)::d, 1>(s, q, k, v, ldq, ldk, ldv, scale, S0, nullptr, cu,
                                             nullptr, Ly, (char*)ws, st);
  });
}

hipError_t launch_chunk_fwd(const gdn_shape& s, const void* q, const void* k, const void* v,
                            int64_t ldq, int64_t ldk, int64_t ldv, const float* g,
                            const float* beta, float scale, const float* S0, float* S_final,
                            const int32_t* cu, void* o, void* ws, hipStream_t st) {
  hipError_t e = launch_chunk_prepare(s, q, k, ldq, ldk, g, beta, scale, cu, ws, st);
  if (e != hipSuccess) return e;
  return launch_chunk_fwd_states(s, q, k, v, ldq, ldk, ldv, scale, S0, S_final, cu, o, ws, st);
}

}  // namespace gdn
