// Chunked gated delta rule: chunk table and WY/UT preparation (the
// sequential state pass is in chunk_state.hip).
#include "chunk_common.h"

namespace gdn {

// The chunk and span tables (one block scan over the sequences):
//   seq_off[n] = number of 64-token chunks of sequences 0..n-1;
//   segb[n]    = number of spans of sequences 0..n-1, where a sequence is one
//                span (seg == 0) or ceil(chunks / seg) segments of seg chunks
//                (seg > 0; a sequence without tokens then has none);
//   spans[i]   = (first chunk, end chunk, first token, end token of the
//                sequence) of span i, the unit a sequential pass walks.
__global__ void __launch_bounds__(256) chunk_table_kernel(const int32_t* __restrict__ cu, int n_seq,
                                                          int seg, int32_t* __restrict__ seq_off,
                                                          int32_t* __restrict__ spans,
                                                          int32_t* __restrict__ segb) {
  __shared__ int32_t buf[2][256];
  __shared__ int32_t carry[2];
  const int tid = threadIdx.x;
  if (tid < 2) carry[tid] = 0;
  __syncthreads();
  for (int base = 0; base < n_seq; base += 256) {
    const int n = base + tid;
    int32_t v = 0, w = 0, t0 = 0, t1 = 0;
    if (n < n_seq) {
      t0 = cu[n];
      t1 = cu[n + 1];
      v = (t1 - t0 + CHUNK - 1) / CHUNK;
      w = seg > 0 ? (v + seg - 1) / seg : 1;
    }
    buf[0][tid] = v;
    buf[1][tid] = w;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {  // Hillis-Steele inclusive scans
      const int32_t y0 = tid >= off ? buf[0][tid - off] : 0;
      const int32_t y1 = tid >= off ? buf[1][tid - off] : 0;
      __syncthreads();
      buf[0][tid] += y0;
      buf[1][tid] += y1;
      __syncthreads();
    }
    if (n < n_seq) {
      const int32_t c0 = carry[0] + buf[0][tid] - v, s0 = carry[1] + buf[1][tid] - w;
      seq_off[n] = c0;
      segb[n] = s0;
      for (int32_t j = 0; j < w; ++j) {
        const int32_t cb = seg > 0 ? c0 + j * seg : c0;
        const int32_t ce = seg > 0 ? (cb + seg < c0 + v ? cb + seg : c0 + v) : c0 + v;
        reinterpret_cast<int4*>(spans)[s0 + j] = make_int4(cb, ce, t0 + CHUNK * (cb - c0), t1);
      }
    }
    __syncthreads();
    if (tid < 2) carry[tid] += buf[tid][255];
    __syncthreads();
  }
  if (tid == 0) {
    seq_off[n_seq] = carry[0];
    segb[n_seq] = carry[1];
  }
}

// ---------------------------------------------------------------------------
// The cu_seqlens contract, checked: one block ORs the violations it sees
// into an LDS word (bits: 1 cu[0] != 0, 2 cu[n_seq] != T, 4 a decrease).
__global__ void __launch_bounds__(256) check_cu_kernel(const int32_t* __restrict__ cu, int n_seq,
                                                       int64_t T, int32_t* __restrict__ out) {
  __shared__ int32_t acc;
  if (threadIdx.x == 0) acc = 0;
  __syncthreads();
  int32_t bad = 0;
  for (int n = threadIdx.x; n < n_seq; n += 256)
    if (cu[n + 1] < cu[n]) bad |= 4;
  if (threadIdx.x == 0) {
    if (cu[0] != 0) bad |= 1;
    if ((int64_t)cu[n_seq] != T) bad |= 2;
  }
  if (bad) atomicOr(&acc, bad);
  __syncthreads();
  if (threadIdx.x == 0) out[0] = acc;
}

hipError_t launch_check_cu(const gdn_shape& s, const int32_t* cu, int32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(check_cu_kernel, dim3(1), dim3(256), 0, st, cu, s.n_seq, s.total_tokens, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Preparation, one workgroup per (chunk, key head): K K^T and Q K^T once
// (MFMA) and K^T (and in backward mode K K^T) to the workspace, then per
// value head of the group: gam, A,
// Tinv (fp32), and the MFMA operands M = Tinv diag(beta), P and
// W = M diag(Gam) K, with the per-token factors Gam_t and dec_t.
template <typename T, int D>
struct PrepStage {                 // the chunk's K and Q rows
  typedef typename Compute<T>::type CT;
  static constexpr int KT_LD = CHUNK + Pad<CT>::v;
  CT K[CHUNK][D + Pad<CT>::v];
  union {
    CT Q[CHUNK][D + Pad<CT>::v];   // until Q K^T is formed
    CT Kt[D][KT_LD];               // then K^T
  } u;
};
struct PrepHead {                  // per value head: A, then Tinv
  float A[CHUNK][68];
  float Ti[CHUNK][68];
};
// With OVERLAY (backward mode, 16-bit types: no W, so the head loop reads no
// K row or K^T from LDS) A and Ti take the staging's storage once the key
// head's outputs are out, which halves the block's LDS.
template <typename T, int D, bool OVERLAY>
struct PrepSmem {
  typedef typename Compute<T>::type CT;
  static constexpr int KT_LD = PrepStage<T, D>::KT_LD;
  // 16-bit types stage P (and in backward mode P^T) in the Ti storage,
  // rows padded to PLD elements; in backward mode the two tiles reach past
  // Ti, into the overlay's spare bytes
  static constexpr bool STAGE_P = sizeof(T) == 2;
  static constexpr int PLD = CHUNK + 8;
  static constexpr size_t SB = sizeof(PrepStage<T, D>), HB = sizeof(PrepHead);
  static constexpr size_t HBS = sizeof(float) * CHUNK * 68 + (STAGE_P ? 2 * 2 * CHUNK * PLD : 0);
  static constexpr size_t HB2 = HB > HBS ? HB : HBS;
  static constexpr size_t RAW = OVERLAY ? (SB > HB2 ? SB : HB2) : SB + HB;
  static_assert(OVERLAY || !STAGE_P || 2 * CHUNK * PLD <= sizeof(float) * CHUNK * 68,
                "forward-mode P staging fits in Ti");
  __align__(16) unsigned char raw[RAW];
  float X[16][17];
  double gam[CHUNK];
  float bet[CHUNK];
  float sbg[CHUNK];                // beta_s Gam_s
  __device__ PrepStage<T, D>& st() { return *reinterpret_cast<PrepStage<T, D>*>(raw); }
  __device__ PrepHead& hd() { return *reinterpret_cast<PrepHead*>(raw + (OVERLAY ? 0 : SB)); }
  static_assert(sizeof(CT) * CHUNK * (D + Pad<CT>::v) <= sizeof(float) * CHUNK * 68,
                "W tile fits in the A storage");
};

// Three blocks per CU for 16-bit types (168 VGPRs; the backward mode's overlaid
// LDS is 37 KB): the head loop is a chain of short phases between barriers.
template <typename T, int D, bool BWD>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 3 : 1))) chunk_prep_kernel(
    const T* __restrict__ q, const T* __restrict__ k, int64_t ldq, int64_t ldk,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ seq_off, int n_seq, int Hv, int G, float scale,
    double* __restrict__ gcum, typename Compute<T>::type* __restrict__ Mw,
    typename Compute<T>::type* __restrict__ Pw, typename Compute<T>::type* __restrict__ Ww,
    typename Compute<T>::type* __restrict__ Ktw, typename Compute<T>::type* __restrict__ Q16w,
    typename Compute<T>::type* __restrict__ K16w, float* __restrict__ Gw, float* __restrict__ Dw,
    T* __restrict__ Kb, T* __restrict__ Ktb, T* __restrict__ Qtb, T* __restrict__ Ptb,
    float* __restrict__ Bw, T* __restrict__ Tib, typename Compute<T>::type* __restrict__ KKw) {
  typedef typename Compute<T>::type CT;
  typedef Mma<CT> MM;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  // backward, 16-bit types: the saved-state pass works from the K rows (in
  // the compute type) and needs neither W nor the compute-type K^T
  constexpr bool KROWS = BWD && sizeof(T) == 2;
  typedef PrepSmem<T, D, KROWS> SM;
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  static_assert(offsetof(SM, gam) % 16 == 0 && offsetof(SM, bet) % 16 == 0, "16-byte reads of gam, bet");
  auto& sK = sm.st().K;
  auto& su = sm.st().u;
  auto& sA = sm.hd().A;
  auto& sTi = sm.hd().Ti;
  constexpr int LD = D + Pad<CT>::v;
  constexpr int KT_LD = SM::KT_LD;
  constexpr int KS = MM::KS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c = blockIdx.x;
  const int kh = blockIdx.y;
  if (c >= seq_off[n_seq]) return;
  int64_t t0;
  int L;
  chunk_span(seq_off, cu, n_seq, c, t0, L);

  stage_rows2<CT, D>(&sK[0][0], k + t0 * ldk + (int64_t)kh * D, ldk, &su.Q[0][0],
                     q + t0 * ldq + (int64_t)kh * D, ldq, LD, L, tid);
  __syncthreads();

  // wave w owns rows [16w, 16w+16) of the 64 x 64 products
  // (and K Q^T for the P rows: P values of four consecutive s per lane)
  floatx4 kk[4], qk[4], kq[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kk[j] = tile_mma<CT, true, true>(zero4(), &sK[0][0], LD, &sK[0][0], LD, 16 * wave, 16 * j, D, lane);
    qk[j] = tile_mma<CT, true, true>(zero4(), &su.Q[0][0], LD, &sK[0][0], LD, 16 * wave, 16 * j, D, lane);
    kq[j] = tile_mma<CT, true, true>(zero4(), &sK[0][0], LD, &su.Q[0][0], LD, 16 * wave, 16 * j, D, lane);
  }
  const int rbase = 16 * wave + 4 * (lane >> 4);
  const int ccol = lane & 15;
  const int r16 = lane & 15;
  if constexpr (BWD) {
    // K K^T (compute type) for the chunk gradients, in 16 x 16 blocks of 256
    // contiguous elements: block (R, C) at 256 (4 R + C), element (r, c) of
    // a block at 4 (16 (c / 4) + r) + c % 4.  K K^T is symmetric, so this
    // lane's tile values k_{rbase+e} . k_s (s = 16 j + ccol) are row s,
    // columns rbase .. rbase + 3: block (j, wave), offset 4 lane + e -- each
    // wave writes whole 512-byte blocks (so the non-temporal hint is safe:
    // it is slow only on stores of part of a line).
    typename Compute<T>::type* ko = KKw + ((int64_t)c * (Hv / G) + kh) * CHUNK * CHUNK;
#pragma unroll
    for (int j = 0; j < 4; ++j) store4_nt(ko + (4 * j + wave) * 256 + 4 * lane, kk[j][0], kk[j][1], kk[j][2], kk[j][3]);
  }
  {
    // Q rows (compute type, zero past the chunk end, columns in accumulator
    // order; read only by the forward pass without saved states) to the
    // workspace; K rows in the storage type (backward) and, for 16-bit
    // types, in the compute type.  Every store is a whole 16-byte piece
    // (eight stored columns; acc_piece_col names their sources), so each
    // wave instruction writes whole 128-byte lines.
    constexpr int PR = D / 8;
    const int64_t base = ((int64_t)c * (Hv / G) + kh) * CHUNK * D;
    for (int i = tid; i < CHUNK * PR; i += 256) {
      const int r = i / PR, p = i % PR;
      const int dst = r * D + 8 * p;
      if constexpr (!BWD) {
        f8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v.v[j] = to_f(su.Q[r][acc_piece_col<CT>(p, j)]);
        store8_nt(Q16w + base + dst, v);
      }
      if constexpr (BWD) {
        f8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v.v[j] = to_f(sK[r][acc_piece_col<CT>(p, j)]);
        store8_nt(Kb + base + dst, v);
        if constexpr (KROWS) store8_nt(K16w + base + dst, v);
      }
    }
    if constexpr (BWD) {
      // Q^T in the storage type, columns (tokens) in accumulator order
      T* qo = Qtb + base;
      for (int i = tid; i < D * (CHUNK / 8); i += 256) {
        const int kr = i / (CHUNK / 8), p = i % (CHUNK / 8);
        f8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v.v[j] = to_f(su.Q[acc_piece_col<T>(p, j)][kr]);
        store8_nt(qo + kr * CHUNK + 8 * p, v);
        // K^T likewise, gathered from the K rows (no LDS transpose: A and
        // Ti take this storage in the head loop, after its first barrier)
        if constexpr (KROWS) {
#pragma unroll
          for (int j = 0; j < 8; ++j) v.v[j] = to_f(sK[acc_piece_col<T>(p, j)][kr]);
          store8_nt(Ktb + base + kr * CHUNK + 8 * p, v);
        }
      }
    }
  }
  if constexpr (!KROWS) {
    __syncthreads();  // Q is dead: its storage takes K^T
    for (int i = tid; i < CHUNK * D; i += 256) {
      const int kc = i % D, sr = i / D;
      su.Kt[kc][sr] = sK[sr][kc];
    }
    __syncthreads();
    // K^T rows of 64 (columns in accumulator order) to the workspace, in
    // 4-element pieces
    constexpr int PR = CHUNK / 4;
    CT* ko = Ktw + ((int64_t)c * (Hv / G) + kh) * D * CHUNK;
    for (int i = tid; i < D * PR; i += 256) {
      const int kr = i / PR, c4 = (i % PR) * 4;
      typedef CT v4 __attribute__((ext_vector_type(4)));
      *reinterpret_cast<v4*>(ko + kr * CHUNK + acc_col<CT>(c4)) =
          *reinterpret_cast<const v4*>(&su.Kt[kr][c4]);
      if constexpr (BWD) {
        store4(Ktb + ((int64_t)c * (Hv / G) + kh) * D * CHUNK + kr * CHUNK + acc_col<T>(c4),
               to_f(su.Kt[kr][c4]), to_f(su.Kt[kr][c4 + 1]), to_f(su.Kt[kr][c4 + 2]),
               to_f(su.Kt[kr][c4 + 3]));
      }
    }
  }

  // the gates of the next head load a head ahead (wave 0), out of the way
  // of the barrier that follows their scan
  float gnx = 0.f, bnx = 0.f;
  auto load_gates = [&](int h) __attribute__((always_inline)) {
    if (wave == 0 && lane < L) {
      gnx = g[(t0 + lane) * Hv + h];
      bnx = beta[(t0 + lane) * Hv + h];
    }
  };
  load_gates(kh * G);
  for (int hh = 0; hh < G; ++hh) {
    const int h = kh * G + hh;
    if (wave == 0) {
      // (taken before the next head's loads go out, so the wait for them
      // leaves those in flight)
      float gcur = gnx, bcur = bnx;
      asm volatile("" : "+v"(gcur), "+v"(bcur));
      const double gl = lane < L ? (double)gcur : 0.0;
      const float bl = lane < L ? bcur : 0.f;
      if (hh + 1 < G) load_gates(h + 1);
      const double gm = wave_incl_scan(gl, lane);
      sm.gam[lane] = gm;
      sm.bet[lane] = bl;
      gcum[((int64_t)c * Hv + h) * CHUNK + lane] = gm;
      // gam is flat past the chunk length (g = 0 there), so these are the
      // factors of token min(t, L - 1)
      const double glast = __shfl(gm, CHUNK - 1, 64);
      const float Gm = dexp<T>(gm);
      sm.sbg[lane] = bl * Gm;
      Gw[((int64_t)c * Hv + h) * CHUNK + lane] = Gm;
      Dw[((int64_t)c * Hv + h) * CHUNK + lane] = dexp<T>(glast - gm);
      if constexpr (BWD) Bw[((int64_t)c * Hv + h) * CHUNK + lane] = bl;
    }
    __syncthreads();
    // A (rows t of this wave), P^T rows s (four consecutive t per lane) and
    // P rows t (four consecutive s per lane, from K Q^T).  For 16-bit types
    // P and P^T are staged in the (not yet written) Ti storage in their
    // stored column order and leave in whole 16-byte pieces.
    CT* Pout = Pw + ((int64_t)c * Hv + h) * CHUNK * CHUNK;
    T* PTout = Ptb + ((int64_t)c * Hv + h) * CHUNK * CHUNK;
    CT (*Ps)[SM::PLD] = reinterpret_cast<CT (*)[SM::PLD]>(&sTi[0][0]);
    T (*Pts)[SM::PLD] = reinterpret_cast<T (*)[SM::PLD]>(&sTi[0][0] + CHUNK * SM::PLD / 2);
    // (the gam values of this lane's rows are read once, and masked
    // exponents are clamped rather than branched around: a branch per
    // element would serialise the gam loads)
    typedef double d2 __attribute__((ext_vector_type(2)));
    const d2 gra = *reinterpret_cast<const d2*>(&sm.gam[rbase]), grb = *reinterpret_cast<const d2*>(&sm.gam[rbase + 2]);
    const double gr[4] = {gra[0], gra[1], grb[0], grb[1]};
    const float4 br = *reinterpret_cast<const float4*>(&sm.bet[rbase]);
    const float brv[4] = {br.x, br.y, br.z, br.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = 16 * j + ccol;
      const double gsj = sm.gam[s];
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = rbase + e;
        const float dec = dexp<T>(s <= t ? gr[e] - gsj : 0.0);  // masked before exp
        sA[t][s] = (s < t) ? brv[e] * dec * kk[j][e] : 0.f;
        pv[e] = (s <= t) ? dec * scale * qk[j][e] : 0.f;
      }
      if constexpr (BWD) {
        if constexpr (SM::STAGE_P)
          store4(&Pts[s][acc_col<T>(rbase)], pv[0], pv[1], pv[2], pv[3]);
        else
          store4(PTout + s * CHUNK + acc_col<T>(rbase), pv[0], pv[1], pv[2], pv[3]);
      }
      const int t = 16 * j + ccol;   // (= s: gam[t] is gsj)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s2 = rbase + e;
        pv[e] = dexp<T>(s2 <= t ? gsj - gr[e] : -1e30) * scale * kq[j][e];
      }
      if constexpr (SM::STAGE_P)
        store4(&Ps[t][acc_col<CT>(rbase)], pv[0], pv[1], pv[2], pv[3]);
      else
        store4(Pout + t * CHUNK + acc_col<CT>(rbase), pv[0], pv[1], pv[2], pv[3]);
    }
    __syncthreads();
    if constexpr (SM::STAGE_P) {
      for (int i = tid; i < CHUNK * (CHUNK / 8); i += 256) {
        const int r = i >> 3, p = i & 7;
        store16_nt(Pout + r * CHUNK + 8 * p, *reinterpret_cast<const uint4*>(&Ps[r][8 * p]));
        if constexpr (BWD)
          store16_nt(PTout + r * CHUNK + 8 * p, *reinterpret_cast<const uint4*>(&Pts[r][8 * p]));
      }
      __syncthreads();  // the inverse overwrites the staging
    }
    invert_unit_lower(sA, sTi, sm.X, tid);
    // M = Tinv diag(beta), columns in accumulator order, in 16-byte pieces
    CT* Mout = Mw + ((int64_t)c * Hv + h) * CHUNK * CHUNK;
    for (int i = tid; i < CHUNK * (CHUNK / 8); i += 256) {
      const int t = i >> 3, p = i & 7;
      f8 v;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int s = acc_piece_col<CT>(p, j);
        v.v[j] = sTi[t][s] * sm.bet[s];
      }
      store8_nt(Mout + t * CHUNK + 8 * p, v);
    }
    if constexpr (BWD) {
      // Tinv in the storage type for the chunk gradients and the reverse pass
      // (which reads M^T = diag(beta) Tinv^T): rows t with the columns in
      // accumulator order, then, for fp32, Tinv^T (rows u, natural order)
      T* to = Tib + ((int64_t)c * Hv + h) * 2 * CHUNK * CHUNK;
      for (int i = tid; i < CHUNK * (CHUNK / 8); i += 256) {
        const int r = i >> 3, p = i & 7;
        f8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v.v[j] = sTi[r][acc_piece_col<T>(p, j)];
        store8_nt(to + r * CHUNK + 8 * p, v);
        if constexpr (sizeof(T) == 4) {   // (16-bit readers transpose Tinv in LDS)
#pragma unroll
          for (int j = 0; j < 8; ++j) v.v[j] = sTi[8 * p + j][r];
          store8_nt(to + CHUNK * CHUNK + r * CHUNK + 8 * p, v);
        }
      }
    }
    // W = Tinv diag(beta Gam) K: wave w forms rows [16w, 16w+16) in the dead
    // A storage (columns in accumulator order), then all rows go out in
    // 16-byte pieces.  beta Gam scales the A operand (Tinv columns).
    if constexpr (!KROWS) {
      typedef typename MM::frag frag;
      frag ta[CHUNK / KS];
#pragma unroll
      for (int s0 = 0; s0 < CHUNK / KS; ++s0) {
        if constexpr (KS == 4) {
          const int sc = s0 * KS + (lane >> 4);
          ta[s0] = sTi[16 * wave + r16][sc] * sm.sbg[sc];
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int sc = s0 * KS + 8 * (lane >> 4) + j;
            ta[s0][j] = (CT)(sTi[16 * wave + r16][sc] * sm.sbg[sc]);
          }
        }
      }
      CT (*Wl)[LD] = reinterpret_cast<CT (*)[LD]>(&sA[0][0]);
#pragma unroll
      for (int kt = 0; kt < D / 16; ++kt) {
        floatx4 acc = zero4();
#pragma unroll
        for (int s0 = 0; s0 < CHUNK / KS; ++s0)
          acc = MM::mma(ta[s0], MM::kc(&su.Kt[16 * kt + r16][0], s0 * KS, lane), acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) Wl[rbase + e][acc_col<CT>(16 * kt + ccol)] = from_f<CT>(acc[e]);
      }
      __syncthreads();
      constexpr int PR = D * (int)sizeof(CT) / 16;
      uint4* wo = reinterpret_cast<uint4*>(Ww + ((int64_t)c * Hv + h) * CHUNK * D);
      for (int i = tid; i < CHUNK * PR; i += 256)
        wo[i] = reinterpret_cast<const uint4*>(&Wl[i / PR][0])[i % PR];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D, bool BWD>
static hipError_t chunk_prepare(const gdn_shape& s, const void* q, const void* k, int64_t ldq,
                                int64_t ldk, const float* g, const float* beta, float scale,
                                const int32_t* cu, const ChunkLayout& Ly, char* ws,
                                hipStream_t st) {
  int32_t* seq_off = (int32_t*)(ws + Ly.seq_off);
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, st, cu, s.n_seq, (int)Ly.seg, seq_off,
                     (int32_t*)(ws + Ly.spans), (int32_t*)(ws + Ly.segb));
  if (Ly.nt_max > 0 && s.total_tokens > 0) {
    const size_t shm = sizeof(PrepSmem<T, D, BWD && sizeof(T) == 2>);
    hipFuncSetAttribute((const void*)chunk_prep_kernel<T, D, BWD>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    hipLaunchKernelGGL((chunk_prep_kernel<T, D, BWD>), dim3((unsigned)Ly.nt_max, s.hk), dim3(256), shm,
                       st, (const T*)q, (const T*)k, ldq, ldk, g, beta, cu, seq_off, s.n_seq, s.hv,
                       s.hv / s.hk, scale, (double*)(ws + Ly.gcum),
                       (typename Compute<T>::type*)(ws + Ly.mw),
                       (typename Compute<T>::type*)(ws + Ly.pw),
                       (typename Compute<T>::type*)(ws + Ly.ww),
                       (typename Compute<T>::type*)(ws + Ly.ktw),
                       (typename Compute<T>::type*)(ws + Ly.q16w),
                       BWD ? (typename Compute<T>::type*)(ws + Ly.k16w) : nullptr, (float*)(ws + Ly.gw),
                       (float*)(ws + Ly.dw), BWD ? (T*)(ws + Ly.kb) : nullptr,
                       BWD ? (T*)(ws + Ly.ktb) : nullptr, BWD ? (T*)(ws + Ly.qtb) : nullptr,
                       BWD ? (T*)(ws + Ly.ptb) : nullptr, BWD ? (float*)(ws + Ly.bw) : nullptr,
                       BWD ? (T*)(ws + Ly.tib) : nullptr,
                       BWD ? (typename Compute<T>::type*)(ws + Ly.kkw) : nullptr);
  }
  return hipGetLastError();
}

size_t chunk_fwd_ws_bytes(const gdn_shape& s) { return chunk_layout(s, ChunkFlow::Fwd).total_fwd; }
size_t chunk_bwd_ws_bytes(const gdn_shape& s) { return chunk_layout(s, ChunkFlow::Bwd).total_bwd; }

hipError_t launch_chunk_prepare(const gdn_shape& s, const void* q, const void* k, int64_t ldq,
                                int64_t ldk, const float* g, const float* beta, float scale,
                                const int32_t* cu, void* ws, bool bwd, hipStream_t st) {
  const ChunkLayout Ly = chunk_layout(s, bwd ? ChunkFlow::Bwd : ChunkFlow::Fwd);
  return dispatch_chunk(s, [&](auto c) {
    using T = typename decltype(c)::type;
    constexpr int D = decltype(c)::d;
    return bwd ? chunk_prepare<T, D, true>(s, q, k, ldq, ldk, g, beta, scale, cu, Ly, (char*)ws, st)
               : chunk_prepare<T, D, false>(s, q, k, ldq, ldk, g, beta, scale, cu, Ly, (char*)ws, st);
  });
}

hipError_t launch_chunk_fwd(const gdn_shape& s, const void* q, const void* k, const void* v,
                            int64_t ldq, int64_t ldk, int64_t ldv, const float* g,
                            const float* beta, float scale, const float* S0, float* S_final,
                            const int32_t* cu, void* o, void* ws, hipStream_t st) {
  hipError_t e = launch_chunk_prepare(s, q, k, ldq, ldk, g, beta, scale, cu, ws, false, st);
  if (e != hipSuccess) return e;
  return launch_chunk_fwd_states(s, q, k, v, ldq, ldk, ldv, scale, S0, S_final, cu, o, ws, st);
}

}  // namespace gdn
