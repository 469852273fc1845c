// Chunked gated delta rule, backward.
//
// Per chunk (notation of chunk_common.h), given dO and the gradient dS' of
// the state leaving the chunk:
//   dDelta = P^T dO + diag(dec) K dS'^T
//   dR     = M^T dDelta                        (= dv)
//   dS     = Gam_L dS' + (scale Q)^T diag(Gam) dO - K^T diag(Gam) dR
// is the sequential part (reverse over chunks, chunk_rev_kernel).  The rest
// is chunk-parallel (chunk_grad_kernel):
//   dM = dDelta R^T,  dTinv = strictly-lower(dM diag(beta)),
//   dA = strictly-lower(-Tinv^T dTinv Tinv^T),  dP = lower(dO Delta^T)
//   dq = scale [diag(Gam) dO S + (dP o D) K]
//   dk = scale (dP o D)^T Q - diag(Gam) dR S + diag(dec) Delta dS'
//        + (dA o beta D) K + (dA o beta D)^T K
//   dbeta_s = sum_t dM[t,s] Tinv[t,s] + sum_u dA[s,u] D[s,u] k_s.k_u
//   dgam from every place gam enters; dg = reverse cumsum of dgam in the chunk.
// dq and dk are summed over the value heads of a key head inside one
// workgroup, in ascending head order.
#include "chunk_common.h"

namespace gdn {

// ---------------------------------------------------------------------------
template <typename T, int D, int BV>
struct RevSmem {
  T K[CHUNK][D + Pad<T>::v];
  T Q[CHUNK][D + Pad<T>::v];
  T dO[CHUNK][BV + Pad<T>::v];
  T dOg[CHUNK][BV + Pad<T>::v];   // scale * Gam_t * dO
  T dSb[BV][D + Pad<T>::v];       // dS' block (v-major)
  T dDt[BV][CHUNK + Pad<T>::v];   // dDelta^T
  T dRg[BV][CHUNK + Pad<T>::v];   // (diag(Gam) dR)^T
  double gam[CHUNK];
};

template <typename T, int D, int BV>
__global__ void __launch_bounds__(256) chunk_rev_kernel(
    const T* __restrict__ q, const T* __restrict__ k, int64_t ldq, int64_t ldk,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ seq_off, int Hv, int G, float scale,
    const double* __restrict__ gcum, const typename Compute<T>::type* __restrict__ Mw,
    const typename Compute<T>::type* __restrict__ Pw, const T* __restrict__ dout, const float* __restrict__ dS_final, float* __restrict__ dS0,
    T* __restrict__ dhst, T* __restrict__ ddw, T* __restrict__ dvo, int64_t lddv) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  RevSmem<T, D, BV>& sm = *reinterpret_cast<RevSmem<T, D, BV>*>(smem_raw);
  constexpr int LD = D + Pad<T>::v, LDV = BV + Pad<T>::v, LDC = CHUNK + Pad<T>::v;
  constexpr int NVT = BV / 16;
  constexpr int NS = (D / 16) * NVT / 4;
  constexpr int NA = (CHUNK / 16) * NVT / 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int vb = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
  const int kh = h / G;
  const int v0 = vb * BV;
  const int rsub = 4 * (lane >> 4), ccol = lane & 15;
  const int64_t HvD = (int64_t)Hv * D;

  floatx4 dS[NS];  // dS^T tiles (d_k x BV)
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int id = wave * NS + i, kt = id / NVT, vt = id % NVT;
    const int vv = v0 + 16 * vt + ccol;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kk = 16 * kt + rsub + e;
      dS[i][e] = dS_final ? dS_final[(((int64_t)n * Hv + h) * D + vv) * D + kk] : 0.f;
    }
  }
  const int64_t c_begin = seq_off[n], c_end = seq_off[n + 1];
  for (int64_t c = c_end - 1; c >= c_begin; --c) {
    const int64_t t0 = (int64_t)cu[n] + CHUNK * (c - c_begin);
    const int L = (int64_t)cu[n + 1] - t0 < CHUNK ? (int)((int64_t)cu[n + 1] - t0) : CHUNK;
    __syncthreads();
    stage_rows<T, D>(&sm.K[0][0], LD, k + t0 * ldk + (int64_t)kh * D, ldk, L, tid);
    stage_rows<T, D>(&sm.Q[0][0], LD, q + t0 * ldq + (int64_t)kh * D, ldq, L, tid);
    stage_rows<T, BV>(&sm.dO[0][0], LDV, dout + t0 * HvD + (int64_t)h * D + v0, HvD, L, tid);
    if (tid < CHUNK) sm.gam[tid] = gcum[(t0 + (tid < L ? tid : L - 1)) * Hv + h];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int id = wave * NS + i, kt = id / NVT, vt = id % NVT;
      const int vv = 16 * vt + ccol, kk = 16 * kt + rsub;
      store4(&sm.dSb[vv][kk], dS[i][0], dS[i][1], dS[i][2], dS[i][3]);
      T* hp = dhst + (((int64_t)c * Hv + h) * D + kk) * D + v0 + vv;
#pragma unroll
      for (int e = 0; e < 4; ++e) hp[(int64_t)e * D] = from_f<T>(dS[i][e]);
    }
    __syncthreads();

    // scaled copy of dO for the state gradient
    for (int i = tid; i < CHUNK * BV; i += 256) {
      const int t = i / BV, vv = i % BV;
      sm.dOg[t][vv] = from_f<T>(scale * dexp<T>(sm.gam[t]) * to_f(sm.dO[t][vv]));
    }
    // Phase A: dDelta = P^T dO + diag(dec) K dS'^T
    const auto* Pc = Pw + ((int64_t)c * Hv + h) * CHUNK * CHUNK;
    const auto* Mc = Mw + ((int64_t)c * Hv + h) * CHUNK * CHUNK;
    const double gl = sm.gam[CHUNK - 1];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int id = wave * NA + i, tt = id / NVT, vt = id % NVT;
      floatx4 pt = tile_mma<T, false, false>(zero4(), Pc, CHUNK, &sm.dO[0][0], LDV, 16 * tt,
                                             16 * vt, CHUNK, lane);
      floatx4 kd = tile_mma<T, true, true>(zero4(), &sm.K[0][0], LD, &sm.dSb[0][0], LD, 16 * tt,
                                           16 * vt, D, lane);
      const int vv = 16 * vt + ccol, tb = 16 * tt + rsub;
      float dd[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) dd[e] = pt[e] + dexp<T>(gl - sm.gam[tb + e]) * kd[e];
      store4(&sm.dDt[vv][tb], dd[0], dd[1], dd[2], dd[3]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (tb + e < L) ddw[(t0 + tb + e) * HvD + (int64_t)h * D + v0 + vv] = from_f<T>(dd[e]);
    }
    __syncthreads();

    // Phase B: dR = M^T dDelta  (this is dv)
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int id = wave * NA + i, tt = id / NVT, vt = id % NVT;
      floatx4 dr = tile_mma<T, false, true>(zero4(), Mc, CHUNK, &sm.dDt[0][0], LDC, 16 * tt,
                                            16 * vt, CHUNK, lane);
      const int vv = 16 * vt + ccol, tb = 16 * tt + rsub;
      float rg[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rg[e] = dexp<T>(sm.gam[tb + e]) * dr[e];
        if (tb + e < L) dvo[(t0 + tb + e) * lddv + (int64_t)h * D + v0 + vv] = from_f<T>(dr[e]);
      }
      store4(&sm.dRg[vv][tb], rg[0], rg[1], rg[2], rg[3]);
    }
    __syncthreads();

    // Phase C: dS^T = Gam_L dS'^T + Q^T (scale diag(Gam) dO) - K^T (diag(Gam) dR)
    const float GL = dexp<T>(gl);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int id = wave * NS + i, kt = id / NVT, vt = id % NVT;
#pragma unroll
      for (int e = 0; e < 4; ++e) dS[i][e] *= GL;
      dS[i] = tile_mma<T, false, false>(dS[i], &sm.Q[0][0], LD, &sm.dOg[0][0], LDV, 16 * kt,
                                        16 * vt, CHUNK, lane);
      floatx4 kr = tile_mma<T, false, true>(zero4(), &sm.K[0][0], LD, &sm.dRg[0][0], LDC, 16 * kt,
                                            16 * vt, CHUNK, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) dS[i][e] -= kr[e];
    }
  }
  if (dS0) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int id = wave * NS + i, kt = id / NVT, vt = id % NVT;
      const int vv = v0 + 16 * vt + ccol, kk = 16 * kt + rsub;
      store4(dS0 + (((int64_t)n * Hv + h) * D + vv) * D + kk, dS[i][0], dS[i][1], dS[i][2], dS[i][3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Chunk-parallel gradients: one workgroup per (chunk, key head).
template <typename T, int D>
struct GradSmem {
  T Kt[D][CHUNK + Pad<T>::v];      // K^T (k-major)
  T Qt[D][CHUNK + Pad<T>::v];      // Q^T
  float Tm[CHUNK][68];             // Tinv
  float Sc1[CHUNK][68];            // A, then dTinv
  union {
    struct {
      T B1[CHUNK][D + Pad<T>::v];
      T B2[CHUNK][D + Pad<T>::v];
      T B3[CHUNK][D + Pad<T>::v];
    } t;
    struct {
      T Krm[CHUNK][D + Pad<T>::v];  // only while forming K K^T and Q K^T
      T Qrm[CHUNK][D + Pad<T>::v];
    } s;
    float Y[CHUNK][68];            // dTinv Tinv^T (B1/B2 are free while it lives)
  } u;
  T WA[CHUNK][CHUNK + Pad<T>::v];
  T dPD[CHUNK][CHUNK + Pad<T>::v];
  float X[16][17];
  double gam[CHUNK];
  float bet[CHUNK];
  float rowA[CHUNK], rowB[CHUNK];
  float colA[4][CHUNK], colB[4][CHUNK], rowX[4][CHUNK];
  float zp[4][64];
  float ip[256];
};

template <typename T, int D>
__global__ void __launch_bounds__(256) chunk_grad_kernel(
    const T* __restrict__ q, const T* __restrict__ k, int64_t ldq, int64_t ldk,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ seq_off, int n_seq, int Hv, int G,
    float scale, const double* __restrict__ gcum, const float* __restrict__ beta,
    const T* __restrict__ hst, const T* __restrict__ dhst, const T* __restrict__ Rw,
    const T* __restrict__ Dlw, const T* __restrict__ ddw, const T* __restrict__ dout,
    const T* __restrict__ dvo, int64_t lddv, T* __restrict__ dq, T* __restrict__ dk, int64_t lddq,
    int64_t lddk, float* __restrict__ dg, float* __restrict__ dbeta) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  GradSmem<T, D>& sm = *reinterpret_cast<GradSmem<T, D>*>(smem_raw);
  constexpr int LD = D + Pad<T>::v, LDC = CHUNK + Pad<T>::v;
  constexpr int NQ = (CHUNK / 16) * (D / 16) / 4;  // (t x k) tiles per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c = blockIdx.x;
  const int kh = blockIdx.y;
  if (c >= seq_off[n_seq]) return;
  int64_t t0;
  int L;
  chunk_span(seq_off, cu, n_seq, c, t0, L);
  const int rbase = 16 * wave + 4 * (lane >> 4), ccol = lane & 15, rsub = 4 * (lane >> 4);
  const int64_t HvD = (int64_t)Hv * D;

  // Stage K, Q (row-major for the Gram products) and their transposes.
  for (int i = tid; i < CHUNK * (D / 8); i += 256) {
    const int r = i / (D / 8), c8 = (i % (D / 8)) * 8;
    f8 kv, qv;
    if (r < L) {
      kv = load8(k + (t0 + r) * ldk + (int64_t)kh * D + c8);
      qv = load8(q + (t0 + r) * ldq + (int64_t)kh * D + c8);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) kv.v[j] = qv.v[j] = 0.f;
    }
    store8(&sm.u.s.Krm[r][c8], kv);
    store8(&sm.u.s.Qrm[r][c8], qv);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sm.Kt[c8 + j][r] = from_f<T>(kv.v[j]);
      sm.Qt[c8 + j][r] = from_f<T>(qv.v[j]);
    }
  }
  __syncthreads();
  floatx4 kk[4], qk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kk[j] = tile_mma<T, true, true>(zero4(), &sm.u.s.Krm[0][0], LD, &sm.u.s.Krm[0][0], LD,
                                    16 * wave, 16 * j, D, lane);
    qk[j] = tile_mma<T, true, true>(zero4(), &sm.u.s.Qrm[0][0], LD, &sm.u.s.Krm[0][0], LD,
                                    16 * wave, 16 * j, D, lane);
  }
  floatx4 dQa[NQ], dKa[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) dQa[i] = dKa[i] = zero4();
  __syncthreads();

  for (int hh = 0; hh < G; ++hh) {
    const int h = kh * G + hh;
    // ---- P0: gate values for the chunk
    if (wave == 0) {
      sm.gam[lane] = gcum[(t0 + (lane < L ? lane : L - 1)) * Hv + h];
      sm.bet[lane] = lane < L ? beta[(t0 + lane) * Hv + h] : 0.f;
    }
    if (tid < CHUNK) { sm.rowA[tid] = 0.f; sm.rowB[tid] = 0.f; }
    __syncthreads();
    // ---- P1: A, then Tinv
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = 16 * j + ccol;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = rbase + e;
        sm.Sc1[t][s] = (s < t) ? sm.bet[t] * dexp<T>(sm.gam[t] - sm.gam[s]) * kk[j][e] : 0.f;
      }
    }
    __syncthreads();
    invert_unit_lower(sm.Sc1, sm.Tm, sm.X, tid);
    // ---- P2: dM = dDelta R^T
    {
      const int64_t base = t0 * HvD + (int64_t)h * D;
      stage_rows<T, D>(&sm.u.t.B1[0][0], LD, ddw + base, HvD, L, tid);
      stage_rows<T, D>(&sm.u.t.B2[0][0], LD, Rw + base, HvD, L, tid);
    }
    __syncthreads();
    {
      float cb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        floatx4 dm = tile_mma<T, true, true>(zero4(), &sm.u.t.B1[0][0], LD, &sm.u.t.B2[0][0], LD,
                                             16 * wave, 16 * j, D, lane);
        const int s = 16 * j + ccol;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = rbase + e;
          cb[j] += dm[e] * sm.Tm[t][s];
          sm.Sc1[t][s] = (s < t) ? dm[e] * sm.bet[s] : 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = cb[j];
        x += __shfl_xor(x, 16, 64);
        x += __shfl_xor(x, 32, 64);
        if (lane < 16) sm.colB[wave][16 * j + lane] = x;
      }
    }
    __syncthreads();
    // ---- P3: Y = dTinv Tinv^T;  dA = -Tinv^T Y
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      floatx4 y = tile_mma<T, true, true>(zero4(), &sm.Sc1[0][0], 68, &sm.Tm[0][0], 68, 16 * wave,
                                          16 * j, CHUNK, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.u.Y[rbase + e][16 * j + ccol] = y[e];
    }
    __syncthreads();
    {
      float ca[4] = {0.f, 0.f, 0.f, 0.f};
      float ra[4] = {0.f, 0.f, 0.f, 0.f}, rb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        floatx4 da = tile_mma<T, false, false>(zero4(), &sm.Tm[0][0], 68, &sm.u.Y[0][0], 68,
                                               16 * wave, 16 * j, CHUNK, lane);
        const int s = 16 * j + ccol;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = rbase + e;
          float wa = 0.f;
          if (s < t) {
            const float dAv = -da[e];
            const float Dts = dexp<T>(sm.gam[t] - sm.gam[s]);
            const float Ats = sm.bet[t] * Dts * kk[j][e];
            const float EA = dAv * Ats;
            ra[e] += EA;
            ca[j] -= EA;
            rb[e] += dAv * Dts * kk[j][e];
            wa = dAv * sm.bet[t] * Dts;
          }
          sm.WA[t][s] = from_f<T>(wa);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = sum16(ra[e]), y = sum16(rb[e]);
        if (ccol == 0) { sm.rowA[rbase + e] += x; sm.rowB[rbase + e] += y; }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = ca[j];
        x += __shfl_xor(x, 16, 64);
        x += __shfl_xor(x, 32, 64);
        if (lane < 16) sm.colA[wave][16 * j + lane] = x;
      }
    }
    __syncthreads();
    // ---- P4: dP = dO Delta^T
    {
      const int64_t base = t0 * HvD + (int64_t)h * D;
      stage_rows<T, D>(&sm.u.t.B1[0][0], LD, dout + base, HvD, L, tid);
      stage_rows<T, D>(&sm.u.t.B2[0][0], LD, Dlw + base, HvD, L, tid);
      stage_rows<T, D>(&sm.u.t.B3[0][0], LD, dvo + t0 * lddv + (int64_t)h * D, lddv, L, tid);
    }
    __syncthreads();
    {
      float ca[4] = {0.f, 0.f, 0.f, 0.f}, ra[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        floatx4 dp = tile_mma<T, true, true>(zero4(), &sm.u.t.B1[0][0], LD, &sm.u.t.B2[0][0], LD,
                                             16 * wave, 16 * j, D, lane);
        const int s = 16 * j + ccol;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = rbase + e;
          float v = 0.f;
          if (s <= t) {
            const float Dts = dexp<T>(sm.gam[t] - sm.gam[s]);
            const float E = dp[e] * Dts * scale * qk[j][e];
            ra[e] += E;
            ca[j] -= E;
            v = dp[e] * Dts;
          }
          sm.dPD[t][s] = from_f<T>(v);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = sum16(ra[e]);
        if (ccol == 0) sm.rowA[rbase + e] += x;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = ca[j];
        x += __shfl_xor(x, 16, 64);
        x += __shfl_xor(x, 32, 64);
        if (lane < 16) sm.colA[wave][16 * j + lane] += x;
      }
    }
    __syncthreads();
    // ---- P5: (t x k) products
    {
      const T* Sg = hst + ((int64_t)c * Hv + h) * D * D;   // [k][v]
      const T* dSg = dhst + ((int64_t)c * Hv + h) * D * D;
      const double gl = sm.gam[CHUNK - 1];
      float rx[4][4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) rx[a][e] = 0.f;
      float zs = 0.f;
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int id = wave * NQ + i, tt = id % 4, kt = id / 4;
        floatx4 x1 = tile_mma<T, true, true>(zero4(), &sm.u.t.B1[0][0], LD, Sg, D, 16 * tt, 16 * kt, D, lane);
        floatx4 x2 = tile_mma<T, true, true>(zero4(), &sm.u.t.B3[0][0], LD, Sg, D, 16 * tt, 16 * kt, D, lane);
        floatx4 x3 = tile_mma<T, true, true>(zero4(), &sm.u.t.B2[0][0], LD, dSg, D, 16 * tt, 16 * kt, D, lane);
        floatx4 pq = tile_mma<T, false, true>(zero4(), &sm.dPD[0][0], LDC, &sm.Qt[0][0], LDC, 16 * tt,
                                              16 * kt, CHUNK, lane);
        dQa[i] = tile_mma<T, true, true>(dQa[i], &sm.dPD[0][0], LDC, &sm.Kt[0][0], LDC, 16 * tt, 16 * kt,
                                         CHUNK, lane);
        dKa[i] = tile_mma<T, true, true>(dKa[i], &sm.WA[0][0], LDC, &sm.Kt[0][0], LDC, 16 * tt, 16 * kt,
                                         CHUNK, lane);
        dKa[i] = tile_mma<T, false, true>(dKa[i], &sm.WA[0][0], LDC, &sm.Kt[0][0], LDC, 16 * tt, 16 * kt,
                                          CHUNK, lane);
        const int kc = 16 * kt + ccol;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * tt + rsub + e;
          const float Gm = dexp<T>(sm.gam[t]);
          const float dec = dexp<T>(gl - sm.gam[t]);
          const float qv = to_f(sm.Qt[kc][t]), kv = to_f(sm.Kt[kc][t]);
          dQa[i][e] += Gm * x1[e];
          dKa[i][e] += scale * pq[e] - Gm * x2[e] + dec * x3[e];
          const float z = dec * x3[e] * kv;
          rx[tt][e] += Gm * scale * x1[e] * qv - Gm * x2[e] * kv - z;
          zs += z;
        }
      }
      // per-wave row partials over this wave's k columns
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = sum16(rx[a][e]);
          if (ccol == 0) sm.rowX[wave][16 * a + rsub + e] = x;
        }
      sm.zp[wave][lane] = zs;
      // <dS', S> for the Gam_L term
      float ipv = 0.f;
      for (int i = tid; i < D * D / 8; i += 256) {
        f8 a = load8(Sg + i * 8), b = load8(dSg + i * 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) ipv += a.v[j] * b.v[j];
      }
      sm.ip[tid] = ipv;
    }
    __syncthreads();
    // ---- P6: assemble dgam -> dg (reverse cumsum), dbeta
    if (wave == 0) {
      const int t = lane;
      float dgm = sm.rowA[t];
      float db = sm.rowB[t];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        dgm += sm.colA[w][t] + sm.rowX[w][t];
        db += sm.colB[w][t];
      }
      float zsum = 0.f, ips = 0.f;
      for (int i = 0; i < 4 * 64; ++i) zsum += (&sm.zp[0][0])[i];
      for (int i = 0; i < 256; ++i) ips += sm.ip[i];
      if (t == L - 1) dgm += zsum + dexp<T>(sm.gam[CHUNK - 1]) * ips;
      if (t >= L) dgm = 0.f;
      const float dgs = wave_suffix_scan(dgm, lane);
      if (t < L) {
        dg[(t0 + t) * Hv + h] = dgs;
        dbeta[(t0 + t) * Hv + h] = db;
      }
    }
    __syncthreads();
  }
  // write dq = scale * dQa, dk = dKa
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int id = wave * NQ + i, tt = id % 4, kt = id / 4;
    const int kc = 16 * kt + ccol;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * tt + rsub + e;
      if (t < L) {
        dq[(t0 + t) * lddq + (int64_t)kh * D + kc] = from_f<T>(scale * dQa[i][e]);
        dk[(t0 + t) * lddk + (int64_t)kh * D + kc] = from_f<T>(dKa[i][e]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
constexpr int REV_BV = 32;

hipError_t launch_chunk_bwd_reverse(const gdn_shape& s, const void* q, const void* k, int64_t ldq,
                                    int64_t ldk, float scale, const int32_t* cu, const void* dout,
                                    const float* dS_final, void* dv, int64_t lddv, float* dS0,
                                    void* wsv, hipStream_t st) {
  char* ws = (char*)wsv;
  const ChunkLayout Ly = chunk_layout(s);
  return dispatch_chunk(s, [&](auto c) {
    using T = typename decltype(c)::type;
    constexpr int D = decltype(c)::d;
    constexpr int BV = REV_BV;
    static_assert(sizeof(RevSmem<T, D, BV>) <= 160 * 1024, "reverse kernel LDS budget");
    const size_t shm = sizeof(RevSmem<T, D, BV>);
    auto kern = chunk_rev_kernel<T, D, BV>;
    hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    hipLaunchKernelGGL(kern, dim3(D / BV, s.hv, s.n_seq), dim3(256), shm, st, (const T*)q,
                       (const T*)k, ldq, ldk, cu, (const int32_t*)(ws + Ly.seq_off), s.hv,
                       s.hv / s.hk, scale, (const double*)(ws + Ly.gcum),
                       (const typename Compute<T>::type*)(ws + Ly.mw),
                       (const typename Compute<T>::type*)(ws + Ly.pw), (const T*)dout, dS_final,
                       dS0, (T*)(ws + Ly.dh), (T*)(ws + Ly.ddw), (T*)dv, lddv);
    return hipGetLastError();
  });
}

hipError_t launch_chunk_bwd_grads(const gdn_shape& s, const void* q, const void* k, int64_t ldq,
                                  int64_t ldk, const float* beta, float scale, const int32_t* cu,
                                  const void* dout, const void* dv, int64_t lddv, void* dq,
                                  void* dk, int64_t lddq, int64_t lddk, float* dg, float* dbeta,
                                  void* wsv, hipStream_t st) {
  char* ws = (char*)wsv;
  const ChunkLayout Ly = chunk_layout(s);
  if (Ly.nt_max == 0 || s.total_tokens == 0) return hipSuccess;
  return dispatch_chunk(s, [&](auto c) {
    using T = typename decltype(c)::type;
    constexpr int D = decltype(c)::d;
    static_assert(sizeof(GradSmem<T, D>) <= 160 * 1024, "gradient kernel LDS budget");
    const size_t shm = sizeof(GradSmem<T, D>);
    auto kern = chunk_grad_kernel<T, D>;
    hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    hipLaunchKernelGGL(kern, dim3((unsigned)Ly.nt_max, s.hk), dim3(256), shm, st, (const T*)q,
                       (const T*)k, ldq, ldk, cu, (const int32_t*)(ws + Ly.seq_off), s.n_seq,
                       s.hv, s.hv / s.hk, scale, (const double*)(ws + Ly.gcum), beta,
                       (const T*)(ws + Ly.h), (const T*)(ws + Ly.dh), (const T*)(ws + Ly.rw),
                       (const T*)(ws + Ly.dlw), (const T*)(ws + Ly.ddw), (const T*)dout,
                       (const T*)dv, lddv, (T*)dq, (T*)dk, lddq, lddk, dg, dbeta);
    return hipGetLastError();
  });
}

hipError_t launch_chunk_bwd(const gdn_shape& s, const void* q, const void* k, const void* v,
                            int64_t ldq, int64_t ldk, int64_t ldv, const float* g,
                            const float* beta, float scale, const float* S0, const int32_t* cu,
                            const void* dout, const float* dS_final, void* dq, void* dk, void* dv,
                            int64_t lddq, int64_t lddk, int64_t lddv, float* dg, float* dbeta,
                            float* dS0, void* ws, hipStream_t st) {
  hipError_t e = launch_chunk_prepare(s, q, k, ldq, ldk, g, beta, scale, cu, ws, st);
  if (e == hipSuccess) e = launch_chunk_bwd_states(s, q, k, v, ldq, ldk, ldv, scale, S0, cu, ws, st);
  if (e == hipSuccess)
    e = launch_chunk_bwd_reverse(s, q, k, ldq, ldk, scale, cu, dout, dS_final, dv, lddv, dS0, ws, st);
  if (e == hipSuccess)
    e = launch_chunk_bwd_grads(s, q, k, ldq, ldk, beta, scale, cu, dout, dv, lddv, dq, dk, lddq,
                               lddk, dg, dbeta, ws, st);
  return e;
}

}  // namespace gdn
