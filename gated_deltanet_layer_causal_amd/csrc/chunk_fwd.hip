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
// accumulators as S^T tiles (d_k rows x BV columns) for the whole sequence.
// Wave w owns token rows [16w, 16w+16) of every (token x value) product, so
// its A operands (Q, M, P rows) come straight from memory into registers;
// K is staged in LDS because the state update reads it transposed.
// Chunk c+1's inputs are loaded into registers while chunk c computes.
//   MODE 0 (forward): writes o and S_final.
//   MODE 1 (backward recompute): writes the chunk-start states h ([dk][dv]
//   per chunk and head), R and Delta.
template <typename T, int D, int BV>
struct StateSmem {
  typedef typename Compute<T>::type CT;
  CT K[CHUNK][D + Pad<CT>::v];
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
    T* __restrict__ hst, T* __restrict__ Rw, T* __restrict__ Dlw, void* __restrict__ sink,
    int n_items) {
  typedef typename Compute<T>::type CT;
  typedef Mma<CT> MM;
  typedef FragKC<CT, T> FQ;     // Q rows (storage type)
  typedef FragKC<CT, CT> FM;    // M, P rows (compute type)
  extern __shared__ __align__(16) unsigned char smem_raw[];
  StateSmem<T, D, BV>& sm = *reinterpret_cast<StateSmem<T, D, BV>*>(smem_raw);
  constexpr int LD = D + Pad<CT>::v, LDC = CHUNK + Pad<CT>::v;
  constexpr int KS = MM::KS;
  constexpr int NVT = BV / 16;                      // value tiles per wave (rows fixed)
  constexpr int NS = (D / 16) * NVT / 4;            // state tiles per wave
  constexpr int NKD = D / KS, NKC = CHUNK / KS;     // MFMA steps over d_k and over the chunk
  static_assert(NS >= 1, "tile split");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int item = xcd_item(blockIdx.x, n_items);
  const int vb = item % (D / BV), h = (item / (D / BV)) % Hv, n = item / ((D / BV) * Hv);
  const int kh = h / G;
  const int v0 = vb * BV;
  const int rsub = 4 * (lane >> 4), ccol = lane & 15, r16 = lane & 15;
  const int trow = 16 * wave;                       // this wave's token rows
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

  // ---- prefetch registers for one chunk
  struct Pref {
    RowPrefetch<T, D> k;                   // K rows -> LDS
    typename FQ::raw q[NKD];               // Q fragments (MODE 0)
    typename FM::raw m[NKC], p[NKC];       // M, P fragments
    T v[NVT][4];                           // V at this lane's output positions (raw)
    double g;                              // gam[tid & 63]
    int L;
    int64_t t0;
  };
  const int64_t c_begin = seq_off[n], c_end = seq_off[n + 1];
  const int64_t seq_t0 = cu[n], seq_t1 = cu[n + 1];
  auto prefetch = [&](Pref& P, int64_t c) {
    P.t0 = seq_t0 + CHUNK * (c - c_begin);
    const int64_t rem = seq_t1 - P.t0;
    const int L = rem < CHUNK ? (int)rem : CHUNK;
    const int64_t t0 = P.t0;
    P.L = L;
    P.k.load(k + t0 * ldk + (int64_t)kh * D, ldk, L, tid);
    const int tq = trow + r16 < L ? trow + r16 : L - 1;   // clamp: rows >= L never reach outputs
    if (MODE == 0) {
#pragma unroll
      for (int s = 0; s < NKD; ++s) P.q[s] = FQ::load(q + (t0 + tq) * ldq + (int64_t)kh * D, s * KS, lane);
    }
    const CT* Mc = Mw + ((int64_t)c * Hv + h) * CHUNK * CHUNK + (trow + r16) * CHUNK;
    const CT* Pc = Pw + ((int64_t)c * Hv + h) * CHUNK * CHUNK + (trow + r16) * CHUNK;
#pragma unroll
    for (int s = 0; s < NKC; ++s) {
      P.m[s] = FM::load(Mc, s * KS, lane);
      if (MODE == 0) P.p[s] = FM::load(Pc, s * KS, lane);
    }
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = trow + rsub + e;
        P.v[vt][e] = v[(t0 + (t < L ? t : L - 1)) * ldv + (int64_t)h * D + v0 + 16 * vt + ccol];
      }
    const int tg = tid & (CHUNK - 1);
    P.g = gcum[(t0 + (tg < L ? tg : L - 1)) * Hv + h];
  };

  // One chunk from prefetched registers `cur`; issues the prefetch of chunk
  // c + 1 into `nxt` before computing.
  auto step = [&](int64_t c, Pref& cur, Pref& nxt) {
    const int L = cur.L;
    const int64_t t0 = cur.t0;
    __syncthreads();  // previous chunk's LDS reads are done
    cur.k.store(&sm.K[0][0], LD, tid);
    sm.gam[tid & (CHUNK - 1)] = cur.g;  // the four waves write identical values
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
    prefetch(nxt, c + 1 < c_end ? c + 1 : c);  // unconditional (re-reads the last chunk at the end)
    issue_fence();
    __syncthreads();

    // Phase A: R = V - diag(Gam) K S^T   (and the Q S^T part of O)
    floatx4 oq[NVT];
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      floatx4 ks = zero4();
      oq[vt] = zero4();
#pragma unroll
      for (int s = 0; s < NKD; ++s) {
        const typename MM::frag b = MM::kc(&sm.Sb[16 * vt + r16][0], s * KS, lane);
        ks = MM::mma(MM::kc(&sm.K[trow + r16][0], s * KS, lane), b, ks);
        if (MODE == 0) oq[vt] = MM::mma(FQ::cvt(cur.q[s]), b, oq[vt]);
      }
      const int vv = 16 * vt + ccol, tb = trow + rsub;
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float Gm = dexp<T>(sm.gam[tb + e]);
        const float vin = tb + e < L ? to_f(cur.v[vt][e]) : 0.f;
        r[e] = vin - Gm * ks[e];
        if (MODE == 0) oq[vt][e] *= Gm * scale;
      }
      store4(&sm.Rt[vv][tb], r[0], r[1], r[2], r[3]);
      if (MODE == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *row_or_sink(Rw + (t0 + tb + e) * HvD + (int64_t)h * D + v0 + vv, tb + e < L, sink, tid) =
              from_f<T>(r[e]);
      }
    }
    __syncthreads();

    // Phase B: Delta = M R
    const double gl = sm.gam[CHUNK - 1];
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      floatx4 dl = zero4();
#pragma unroll
      for (int s = 0; s < NKC; ++s)
        dl = MM::mma(FM::cvt(cur.m[s]), MM::kc(&sm.Rt[16 * vt + r16][0], s * KS, lane), dl);
      const int vv = 16 * vt + ccol, tb = trow + rsub;
      float ds[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ds[e] = dexp<T>(gl - sm.gam[tb + e]) * dl[e];
      store4(&sm.Dt[vv][tb], dl[0], dl[1], dl[2], dl[3]);
      store4(&sm.Dst[vv][tb], ds[0], ds[1], ds[2], ds[3]);
      if (MODE == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *row_or_sink(Dlw + (t0 + tb + e) * HvD + (int64_t)h * D + v0 + vv, tb + e < L, sink, tid) =
              from_f<T>(dl[e]);
      }
    }
    __syncthreads();

    // Phase C: O = oq + P Delta;  S^T <- Gam_L S^T + K^T (diag(dec) Delta)
    if (MODE == 0) {
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        floatx4 ov = oq[vt];
#pragma unroll
        for (int s = 0; s < NKC; ++s)
          ov = MM::mma(FM::cvt(cur.p[s]), MM::kc(&sm.Dt[16 * vt + r16][0], s * KS, lane), ov);
        const int vv = 16 * vt + ccol, tb = trow + rsub;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *row_or_sink(o + (t0 + tb + e) * HvD + (int64_t)h * D + v0 + vv, tb + e < L, sink, tid) =
              from_f<T>(ov[e]);
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
  };

  Pref A, B;
  if (c_begin < c_end) prefetch(A, c_begin);
  for (int64_t c = c_begin; c < c_end; c += 2) {
    step(c, A, B);
    if (c + 1 < c_end) step(c + 1, B, A);
  }
  // Never taken (chunk offsets are non-negative): gives both prefetch buffers
  // a use on the loop-exit path, so their loads are not sunk into the branch
  // that runs the second step of a pair (which would serialise them).
  if (c_end < 0) {
    T* sk = reinterpret_cast<T*>(sink);
    *reinterpret_cast<Raw8<T>*>(sk) = A.k.r[0];
    *reinterpret_cast<Raw8<T>*>(sk + 64) = B.k.r[0];
    sk[128] = A.v[0][0];
    sk[129] = B.v[0][0];
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
  const int n_items = (D / BV) * s.hv * s.n_seq;
  hipLaunchKernelGGL(kern, dim3(n_items), dim3(256), shm, st, (const T*)q, (const T*)k,
                     (const T*)v, ldq, ldk, ldv, cu, (const int32_t*)(ws + Ly.seq_off), s.hv,
                     s.hv / s.hk, scale, (const double*)(ws + Ly.gcum),
                     (const typename Compute<T>::type*)(ws + Ly.mw),
                     (const typename Compute<T>::type*)(ws + Ly.pw), S0, S_final, (T*)o,
                     (T*)(ws + Ly.h), (T*)(ws + Ly.rw), (T*)(ws + Ly.dlw), (void*)(ws + Ly.sink),
                     n_items);
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
