// Chunked gated delta rule, backward.
//
// Per chunk (notation of chunk_common.h), given dO and the gradient dS' of
// the state leaving the chunk:
//   dDelta = P^T dO + diag(dec) K dS'^T
//   dR     = M^T dDelta                        (= dv)
//   dS     = Gam_L dS' + (scale Q)^T diag(Gam) dO - K^T diag(Gam) dR
// is the sequential part (reverse over chunks, chunk_rev.hip).  The rest
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
template <typename T, int D>
struct GradSmem {
  T Kt[D][CHUNK + Pad<T>::v];      // K^T (k-major)
  T Qt[D][CHUNK + Pad<T>::v];      // Q^T
  float Tm[CHUNK][68];             // Tinv
  float Sc1[CHUNK][68];            // dTinv, then the pair terms E
  union {
    struct {
      T B1[CHUNK][D + Pad<T>::v];
      T B2[CHUNK][D + Pad<T>::v];
      T B3[CHUNK][D + Pad<T>::v];
    } t;
    T Krm[CHUNK][D + Pad<T>::v];   // K rows, only while forming K K^T
    float Y[CHUNK][68];            // dTinv Tinv^T (B1/B2 are dead while it lives)
  } u;
  T WA[CHUNK][CHUNK + Pad<T>::v];
  T dPD[CHUNK][CHUNK + Pad<T>::v];
  double gam[CHUNK];
  float bet[CHUNK];
  float rowB[CHUNK];
  float colB[4][CHUNK], rowX[4][CHUNK], rowZ[4][CHUNK];
  float segE[4][CHUNK];            // per-(row block, column) totals of E
  float boxE[4][CHUNK];            // per-(column block, token) parts of the box sums
  float red[4];                    // per-wave partial sums of <dS', S>
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <typename T, int D>
__global__ void __launch_bounds__(256, 1) chunk_grad_kernel(
    const T* __restrict__ q, const T* __restrict__ k, int64_t ldq, int64_t ldk,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ seq_off, int n_seq, int Hv, int G,
    float scale, const double* __restrict__ gcum, const float* __restrict__ beta,
    const typename Compute<T>::type* __restrict__ Pw, const float* __restrict__ Tiw,
    const T* __restrict__ hst,
    const T* __restrict__ dhst, const T* __restrict__ Rw, const T* __restrict__ Dlw,
    const T* __restrict__ ddw, const T* __restrict__ dout, const T* __restrict__ dvo, int64_t lddv,
    T* __restrict__ dq, T* __restrict__ dk, int64_t lddq, int64_t lddk, float* __restrict__ dg,
    float* __restrict__ dbeta, void* __restrict__ sink) {
  typedef typename Compute<T>::type CT;
  typedef Mma<T> MM;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  GradSmem<T, D>& sm = *reinterpret_cast<GradSmem<T, D>*>(smem_raw);
  constexpr int LD = D + Pad<T>::v, LDC = CHUNK + Pad<T>::v;
  constexpr int KS = MM::KS;
  constexpr int NKD = D / KS;
  constexpr int NQ = (CHUNK / 16) * (D / 16) / 4;  // (t x k) tiles per wave
  int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t c = blockIdx.x;
  const int kh = blockIdx.y;
  if (c >= seq_off[n_seq]) return;
  int64_t t0;
  int L;
  chunk_span(seq_off, cu, n_seq, c, t0, L);
  const int rbase = 16 * wave + 4 * (lane >> 4), ccol = lane & 15, rsub = 4 * (lane >> 4);
  const int r16 = lane & 15;
  const int64_t HvD = (int64_t)Hv * D;

  // Stage K rows (for K K^T) and the transposes of K and Q.
  {
    RowPrefetch<T, D, true> pk, pq;
    pk.load(k + t0 * ldk + (int64_t)kh * D, ldk, L, tid);
    pq.load(q + t0 * ldq + (int64_t)kh * D, ldq, L, tid);
    pk.store(&sm.u.Krm[0][0], LD, tid);
    store_rows_transposed(pk, &sm.Kt[0][0], LDC, tid);
    store_rows_transposed(pq, &sm.Qt[0][0], LDC, tid);
  }
  __syncthreads();
  floatx4 kk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    kk[j] = tile_mma<T, true, true>(zero4(), &sm.u.Krm[0][0], LD, &sm.u.Krm[0][0], LD, 16 * wave,
                                    16 * j, D, lane);
  floatx4 dQa[NQ], dKa[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) dQa[i] = dKa[i] = zero4();
  __syncthreads();

  // prefetch registers: P2 tiles (dDelta, R) and P4 tiles (dO, Delta, dR)
  RowPrefetch<T, D> f_dd, f_r, f_do, f_dl, f_dr;
  auto prefetch_p2 = [&](int h) {
    const int64_t base = t0 * HvD + (int64_t)h * D;
    f_dd.load(ddw + base, HvD, L, tid);
    f_r.load(Rw + base, HvD, L, tid);
  };
  prefetch_p2(kh * G);

  for (int hh = 0; hh < G; ++hh) {
    const int h = kh * G + hh;
    // Address arithmetic derived from a laundered thread index stays inside
    // the loop instead of being hoisted (and spilled) as loop invariants.
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int rbase = 16 * wave + 4 * (lane >> 4), ccol = lane & 15, rsub = 4 * (lane >> 4);
    const int r16 = lane & 15;
    // ---- P0: gate values for the chunk; P values at this lane's positions;
    //      Tinv of this (chunk, head) as the preparation formed it
    {
      const float4* src = reinterpret_cast<const float4*>(Tiw + ((int64_t)c * Hv + h) * CHUNK * CHUNK);
#pragma unroll
      for (int j = 0; j < CHUNK * (CHUNK / 4) / 256; ++j) {
        const int i = tid + 256 * j;
        *reinterpret_cast<float4*>(&sm.Tm[i / (CHUNK / 4)][(i % (CHUNK / 4)) * 4]) = src[i];
      }
    }
    if (wave == 0) {
      sm.gam[lane] = gcum[(t0 + (lane < L ? lane : L - 1)) * Hv + h];
      sm.bet[lane] = lane < L ? beta[(t0 + lane) * Hv + h] : 0.f;
    }
    if (tid < CHUNK) sm.rowB[tid] = 0.f;
    CT pval[4][4];
    {
      const CT* Pc = Pw + ((int64_t)c * Hv + h) * CHUNK * CHUNK;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) pval[j][e] = Pc[(rbase + e) * CHUNK + acc_col<CT>(16 * j + ccol)];
    }
    __syncthreads();
    // ---- P2: dM = dDelta R^T
    f_dd.store(&sm.u.t.B1[0][0], LD, tid);
    f_r.store(&sm.u.t.B2[0][0], LD, tid);
    {
      const int64_t base = t0 * HvD + (int64_t)h * D;
      f_do.load(dout + base, HvD, L, tid);
      f_dl.load(Dlw + base, HvD, L, tid);
      f_dr.load(dvo + t0 * lddv + (int64_t)h * D, lddv, L, tid);
    }
    issue_fence();
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
        __builtin_amdgcn_sched_barrier(0);
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
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    // E[t][s] = dA[t][s] A[t][s] + dP[t][s] P[t][s] (s < t) collects in
    // Esm (the dead Sc1 storage, stride 65) for the box sums of P6.
    float(*Esm)[CHUNK + 1] = reinterpret_cast<float(*)[CHUNK + 1]>(&sm.Sc1[0][0]);
    {
      float rb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        floatx4 da = tile_mma<T, false, false>(zero4(), &sm.Tm[0][0], 68, &sm.u.Y[0][0], 68,
                                               16 * wave, 16 * j, CHUNK, lane);
        const int s = 16 * j + ccol;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = rbase + e;
          float wa = 0.f, EA = 0.f;
          if (s < t) {
            const float dAv = -da[e];
            const float Dts = dexp<T>(sm.gam[t] - sm.gam[s]);
            EA = dAv * (sm.bet[t] * Dts * kk[j][e]);
            rb[e] += dAv * Dts * kk[j][e];
            wa = dAv * sm.bet[t] * Dts;
          }
          sm.WA[t][s] = from_f<T>(wa);
          Esm[t][s] = EA;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y = sum16(rb[e]);
        if (ccol == 0) sm.rowB[rbase + e] += y;
      }
    }
    __syncthreads();
    // ---- P4: dP = dO Delta^T
    f_do.store(&sm.u.t.B1[0][0], LD, tid);
    f_dl.store(&sm.u.t.B2[0][0], LD, tid);
    f_dr.store(&sm.u.t.B3[0][0], LD, tid);
    prefetch_p2(hh + 1 < G ? h + 1 : h);   // unconditional: re-reads on the last head
    issue_fence();
    __syncthreads();
    {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        floatx4 dp = tile_mma<T, true, true>(zero4(), &sm.u.t.B1[0][0], LD, &sm.u.t.B2[0][0], LD,
                                             16 * wave, 16 * j, D, lane);
        const int s = 16 * j + ccol;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = rbase + e;
          float v = 0.f;
          if (s <= t) v = dp[e] * dexp<T>(sm.gam[t] - sm.gam[s]);
          if (s < t) Esm[t][s] += dp[e] * to_f(pval[j][e]);  // same lane wrote it in P3
          sm.dPD[t][s] = from_f<T>(v);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    // ---- P5: (token x key) products; tile (tt, kt), wave w owns tiles
    //      w*NQ .. w*NQ+NQ-1 (tt fastest), so the S / dS' columns it reads
    //      from memory change only when kt does.
    {
      const T* Sg = hst + ((int64_t)c * Hv + h) * D * D;   // [k][v]
      const T* dSg = dhst + ((int64_t)c * Hv + h) * D * D;
      const double gl = sm.gam[CHUNK - 1];
      float rx[4][4], rz[4][4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) rx[a][e] = rz[a][e] = 0.f;
      float ipv = 0.f;
      typename MM::frag sf[NKD], dsf[NKD];
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int id = wave * NQ + i, tt = id % 4, kt = id / 4;
        if (i == 0 || tt == 0) {
#pragma unroll
          for (int s = 0; s < NKD; ++s) {
            sf[s] = MM::kc(Sg + (int64_t)(16 * kt + r16) * D, s * KS, lane);
            dsf[s] = MM::kc(dSg + (int64_t)(16 * kt + r16) * D, s * KS, lane);
          }
          if (tt == 0) {   // each (v, k) element once over the workgroup
#pragma unroll
            for (int s = 0; s < NKD; ++s) {
              if constexpr (KS == 4) {
                ipv += to_f(sf[s]) * to_f(dsf[s]);
              } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) ipv += (float)sf[s][j] * (float)dsf[s][j];
              }
            }
          }
        }
        floatx4 x1 = zero4(), x2 = zero4(), x3 = zero4();
#pragma unroll
        for (int s = 0; s < NKD; ++s) {
          x1 = MM::mma(MM::kc(&sm.u.t.B1[16 * tt + r16][0], s * KS, lane), sf[s], x1);
          x2 = MM::mma(MM::kc(&sm.u.t.B3[16 * tt + r16][0], s * KS, lane), sf[s], x2);
          x3 = MM::mma(MM::kc(&sm.u.t.B2[16 * tt + r16][0], s * KS, lane), dsf[s], x3);
        }
        floatx4 pq = tile_mma<T, false, true>(zero4(), &sm.dPD[0][0], LDC, &sm.Qt[0][0], LDC, 16 * tt,
                                              16 * kt, CHUNK, lane);
        dQa[i] = tile_mma<T, true, true>(dQa[i], &sm.dPD[0][0], LDC, &sm.Kt[0][0], LDC, 16 * tt,
                                         16 * kt, CHUNK, lane);
        dKa[i] = tile_mma<T, true, true>(dKa[i], &sm.WA[0][0], LDC, &sm.Kt[0][0], LDC, 16 * tt,
                                         16 * kt, CHUNK, lane);
        dKa[i] = tile_mma<T, false, true>(dKa[i], &sm.WA[0][0], LDC, &sm.Kt[0][0], LDC, 16 * tt,
                                          16 * kt, CHUNK, lane);
        const int kc = 16 * kt + ccol;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * tt + rsub + e;
          const float Gm = dexp<T>(sm.gam[t]);
          const float dec = dexp<T>(gl - sm.gam[t]);
          const float qv = to_f(sm.Qt[kc][t]), kv = to_f(sm.Kt[kc][t]);
          dQa[i][e] += Gm * x1[e];
          dKa[i][e] += scale * pq[e] - Gm * x2[e] + dec * x3[e];
          rx[tt][e] += Gm * scale * x1[e] * qv - Gm * x2[e] * kv;
          rz[tt][e] += dec * x3[e] * kv;
        }
        __builtin_amdgcn_sched_barrier(0);  // bound live ranges: one tile at a time
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = sum16(rx[a][e]), z = sum16(rz[a][e]);
          if (ccol == 0) {
            sm.rowX[wave][16 * a + rsub + e] = x;
            sm.rowZ[wave][16 * a + rsub + e] = z;
          }
        }
      ipv = wave_sum(ipv);
      if (lane == 0) sm.red[wave] = ipv;
    }
    __syncthreads();
    // ---- P6: assemble dg, dbeta.  With gamma the in-chunk cumulative gate,
    //      dg_i = sum_{t >= i} dgam_t.  Three parts, each a sum of terms that
    //      all carry the decay across token i, so no large terms cancel when
    //      that decay is strong:
    //      - pair terms E[t][s] (s < t) add to dgam_t and subtract from
    //        dgam_s; their part of dg_i is the box sum over t >= i > s,
    //        taken as column suffix sums over rows, then row prefix sums;
    //      - the chunk-start terms y_t (rowX, and the state term at the last
    //        token) enter as the suffix sum over t >= i;
    //      - the decay-to-chunk-end terms z_t enter dgam as -z_t and as
    //        +sum z at the last token: their part is the prefix sum over t < i.
    {
      // column suffix sums within each 16-row block (wave = row block)
      const int cidx = lane, rb0 = 16 * wave;
      float acc = 0.f;
#pragma unroll
      for (int r = 15; r >= 0; --r) {
        acc += Esm[rb0 + r][cidx];
        Esm[rb0 + r][cidx] = acc;
      }
      sm.segE[wave][cidx] = acc;
    }
    __syncthreads();
    {
      // add the later row blocks, then the row-prefix part of each box sum
      const int cidx = lane, rb0 = 16 * wave;
      float off = 0.f;
      for (int w = 3; w > wave; --w) off += sm.segE[w][cidx];
#pragma unroll
      for (int r = 0; r < 16; ++r) Esm[rb0 + r][cidx] += off;
    }
    __syncthreads();
    {
      // token i = lane sums columns s < i of the column block owned by this wave
      const int i = lane, cb0 = 16 * wave;
      float part = 0.f;
#pragma unroll
      for (int s = 0; s < 16; ++s)
        if (cb0 + s < i) part += Esm[i][cb0 + s];
      sm.boxE[wave][i] = part;
    }
    __syncthreads();
    if (wave == 0) {
      const int t = lane;
      float y = 0.f, db = sm.rowB[t], zt = 0.f;
      const float box = ((sm.boxE[0][t] + sm.boxE[1][t]) + sm.boxE[2][t]) + sm.boxE[3][t];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        y += sm.rowX[w][t];
        db += sm.colB[w][t];
        zt += sm.rowZ[w][t];
      }
      const float ips = sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3];
      if (t == L - 1) y += dexp<T>(sm.gam[CHUNK - 1]) * ips;
      if (t >= L) { y = 0.f; zt = 0.f; }
      const float dgs = box + wave_suffix_scan(y, lane) + (wave_incl_scan_f(zt, lane) - zt);
      if (t < L) {
        dg[(t0 + t) * Hv + h] = dgs;
        dbeta[(t0 + t) * Hv + h] = db;
      }
    }
    __syncthreads();
  }
  // Never taken: keeps the last prefetch live on the exit path (see the
  // state kernel).
  if (G < 0) *reinterpret_cast<Raw8<T>*>(sink) = f_dd.r[0];
  // write dq = scale * dQa, dk = dKa
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int id = wave * NQ + i, tt = id % 4, kt = id / 4;
    const int kc = 16 * kt + ccol;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * tt + rsub + e;
      *row_or_sink(dq + (t0 + t) * lddq + (int64_t)kh * D + kc, t < L, sink, tid) =
          from_f<T>(scale * dQa[i][e]);
      *row_or_sink(dk + (t0 + t) * lddk + (int64_t)kh * D + kc, t < L, sink, tid) =
          from_f<T>(dKa[i][e]);
    }
  }
}

// ---------------------------------------------------------------------------
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
                       (const typename Compute<T>::type*)(ws + Ly.pw), (const float*)(ws + Ly.tiw),
                       (const T*)(ws + Ly.h),
                       (const T*)(ws + Ly.dh), (const T*)(ws + Ly.rw), (const T*)(ws + Ly.dlw),
                       (const T*)(ws + Ly.ddw), (const T*)dout, (const T*)dv, lddv, (T*)dq,
                       (T*)dk, lddq, lddk, dg, dbeta, (void*)(ws + Ly.sink));
    return hipGetLastError();
  });
}

hipError_t launch_chunk_bwd(const gdn_shape& s, const void* q, const void* k, const void* v,
                            int64_t ldq, int64_t ldk, int64_t ldv, const float* g,
                            const float* beta, float scale, const float* S0, const int32_t* cu,
                            const void* dout, const float* dS_final, void* dq, void* dk, void* dv,
                            int64_t lddq, int64_t lddk, int64_t lddv, float* dg, float* dbeta,
                            float* dS0, void* ws, hipStream_t st) {
  hipError_t e = launch_chunk_prepare(s, q, k, ldq, ldk, g, beta, scale, cu, ws, true, st);
  if (e == hipSuccess) e = launch_chunk_bwd_states(s, q, k, v, ldq, ldk, ldv, scale, S0, cu, ws, st);
  if (e == hipSuccess)
    e = launch_chunk_bwd_reverse(s, q, k, ldq, ldk, scale, cu, dout, dS_final, dv, lddv, dS0, ws, st);
  if (e == hipSuccess)
    e = launch_chunk_bwd_grads(s, q, k, ldq, ldk, beta, scale, cu, dout, dv, lddv, dq, dk, lddq,
                               lddk, dg, dbeta, ws, st);
  return e;
}

}  // namespace gdn
