// Chunked gated delta rule, backward: the chunk-parallel gradients.
//
// Per chunk (notation of chunk_common.h), given dO, the reverse pass's dR
// (= dv) and dDelta, the saved states S (entering the chunk) and dS' (the
// gradient of the state leaving it), and R, Delta of the forward:
//   dM = dDelta R^T,  dTinv = strictly-lower(dM diag(beta)),
//   Y  = dTinv Tinv^T,  dA = strictly-lower(-Tinv^T Y),  dP = lower(dO Delta^T)
//   WA = dA o (beta_t D),  WS = WA + WA^T  (symmetric; WA is strictly lower,
//   so WS takes WA in its lower and WA^T in its upper triangle)
//   dq = scale [diag(Gam) dO S + (dP o D) K]
//   dk = scale (dP o D)^T Q - diag(Gam) dR S + diag(dec) Delta dS' + WS K
//   dbeta_s = sum_t dM[t,s] Tinv[t,s] + sum_u dA[s,u] D[s,u] k_s.k_u
// and dg from every place gam enters, assembled without cancellation (the
// last phase below).
//
// One workgroup of eight waves per (up to four consecutive chunks, key head)
// walks, for each chunk, the G value heads of the group and sums dq, dk over
// them in registers (ascending head order, no atomics).  The operands of the
// next head are requested while a head finishes, across chunk boundaries
// too (K K^T, the K^T and Q^T rows and q, k of the next chunk with its first
// head), so only a workgroup's first head waits for memory.  Per head:
//  - the token-major tiles dO, Delta, dR, R come into LDS by direct copies
//    (issued while the previous head finishes); for bf16 data the fp16 Delta
//    of the saved-state pass is rounded to bf16 in place, once;
//  - phase A, pair products, as 64 x 64 tiles whose columns are a token t
//    and rows the other token s (every lane holds four consecutive s of one
//    t; waves w and w + 4 own the same 16 tokens t).  Waves 0-3 take the
//    Tinv chain: dM^T, dTinv^T (kept in the accumulators and used from
//    there as an A operand, accumulator order), Y (crossing waves once,
//    through LDS), dA^T, and with them WA, the dA part of the pair terms of
//    dg and dbeta.  Waves 4-7 take dP (both orientations), dP o D and the
//    dP part of the pair terms.  The element-wise work needs no exchange;
//  - phase B, token x key products: wave w owns 16 key columns of dq^T and
//    dk^T (k x t tiles: four consecutive k of one token per lane, stored in
//    8-byte pieces at the end).  The products with S and dS' take the
//    wave's rows of the saved states as A operands; those with dP o D, its
//    transpose and WS read LDS tiles written in phase A with their columns
//    in accumulator order, matching K^T and Q^T from the preparation.
// All MFMAs run on the storage type (bf16 operands for bf16 data, fp32 for
// fp32 data).
#include <type_traits>

#include "chunk_stream.h"

namespace gdn {

// Consecutive chunks per workgroup of the gradient kernel: up to four, as
// long as the launch keeps at least eight workgroups per CU (a few chunks
// per workgroup amortise its first head's wait for memory; fewer
// workgroups than that leave CUs idle on short inputs).
constexpr int GRAD_MAX_ITEMS = 4;
inline int grad_items(int64_t nt_max, int hk) {
  const int64_t per = nt_max * hk / (8 * 256);
  return per < 1 ? 1 : per > GRAD_MAX_ITEMS ? GRAD_MAX_ITEMS : (int)per;
}

template <typename T, int D> struct GradLds {
  typedef Tile<T, CHUNK, D, -1> TT;                           // token-major tile
  static constexpr int LDP = CHUNK + 16 / (int)sizeof(T);     // padded 64-wide rows
  static constexpr int NKT = D / 16;                          // key tiles (phase-B waves per token group)
  T tO[TT::PIECES * TT::EPP];     // dO
  T tDl[TT::PIECES * TT::EPP];    // Delta (bf16 data: the fp16 values, rounded to bf16 in place)
  T tdR[TT::PIECES * TT::EPP];    // dR
  T tR[TT::PIECES * TT::EPP];     // R
  T YT[CHUNK][LDP];               // Y^T: row s, column u
  T dPD[CHUNK][LDP];              // dP o D: row t, columns s in accumulator order
  T dPDt[CHUNK][LDP];             // scale (dP o D)^T: row s, columns t in accumulator order
  T WS[CHUNK][LDP];               // WA + WA^T: row x, columns u in accumulator order
  // (after phase B of an item's last head, YT .. WS hold its dq and dk rows,
  // QKR elements apart: 16 bytes of padding keep the rows 16-byte aligned
  // and spread a wave's puts of 16 rows x 4 consecutive pieces over the
  // banks)
  static constexpr int QKR = D + 16 / (int)sizeof(T);
  static_assert(2 * QKR <= 4 * LDP, "dq and dk rows fit in the pair tiles");
  float E[CHUNK][CHUNK + 1];      // pair terms of dg
  // Tinv (columns in accumulator order), copied for 16-bit types, whose
  // Tinv^T operands are transposing reads of it (fp32 reads Tinv and Tinv^T
  // from memory where used: the LDS holds no more)
  static constexpr bool TIN_LDS = sizeof(T) == 2;
  typedef Tile<T, CHUNK, CHUNK> TI;
  T Tin[TIN_LDS ? CHUNK * CHUNK : 8];
  double gam[CHUNK];
  float bet[CHUNK], Gm[CHUNK], dc[CHUNK];
  // the per-head partials of dg and dbeta, two sets by head parity (a head's
  // are summed and scanned while the next head runs)
  float colB[2][4][CHUNK], rowB[2][2][CHUNK], rowX[2][NKT][CHUNK], rowZ[2][NKT][CHUNK];
  float boxE[2][4][CHUNK], red[2][8];
  // k_t . k_s, the preparation's K K^T in the compute type (fp16 for 16-bit
  // data: |k_t . k_s| <= 1 for the L2-normalised keys) and in its layout of
  // 16 x 16 blocks (element (t, s) at 256 (4 (t / 16) + s / 16) +
  // 4 (16 ((s % 16) / 4) + t % 16) + s % 4), by plain direct copy
  typedef typename Compute<T>::type KKT;
  KKT KK[CHUNK * CHUNK];
};

// Four consecutive elements as floats (8 bytes for 16-bit types).
template <typename E> __device__ __forceinline__ floatx4 ld4(const E* p) {
  if constexpr (sizeof(E) == 4) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    return floatx4{v.x, v.y, v.z, v.w};
  } else {
    typedef E e4 __attribute__((ext_vector_type(4)));
    const e4 v = *reinterpret_cast<const e4*>(p);
    return floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(512, 1) chunk_grad_kernel(
    const T* __restrict__ q, const T* __restrict__ k, int64_t ldq, int64_t ldk,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ seq_off, int n_seq, int Hv, int G,
    float scale, const double* __restrict__ gcum, const float* __restrict__ bw,
    const typename Compute<T>::type* __restrict__ Pw, const T* __restrict__ Tib,
    const T* __restrict__ Ktb, const T* __restrict__ Qtb, const T* __restrict__ hst,
    const T* __restrict__ dhst, const T* __restrict__ Rw, const void* __restrict__ Dlw,
    const T* __restrict__ ddw, const typename Compute<T>::type* __restrict__ KKw,
    const T* __restrict__ dout, const T* __restrict__ dvo,
    int64_t lddv, T* __restrict__ dq, T* __restrict__ dk, int64_t lddq, int64_t lddk,
    float* __restrict__ dg, float* __restrict__ dbeta, int items) {
  typedef typename Compute<T>::type CT;
  typedef Mma<T> MM;
  typedef AccOrder<T> AO;
  typedef typename MM::frag frag;
  typedef GradLds<T, D> GL;
  typedef typename GL::TT TT;
  constexpr int KS = MM::KS;
  constexpr int NSD = D / KS, NSC = CHUNK / KS;
  constexpr int NKT = GL::NKT;            // phase B: key tiles; 8 / NKT token groups
  constexpr int TTW = 4 * NKT / 8;        // phase B: token tiles per wave
  static_assert(D == 32 || D == 128, "head dim 32 or 128");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  GL& sm = *reinterpret_cast<GL*>(smem_raw);
  static_assert(offsetof(GL, gam) % 16 == 0, "16-byte reads of gam");

  // Indices derived from the thread and wave numbers are recomputed at the
  // top of every head (from laundered copies, below), so that the compiler
  // does not hoist the addresses and masks built on them out of the loop
  // as loop invariants, where they would be spilled.
  int tid = threadIdx.x, lane = tid & 63;
  int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int g = lane >> 4, g4 = 4 * g, c16 = lane & 15;
  const int kh = blockIdx.y;
  const int64_t n_chunks = seq_off[n_seq];
  const int64_t c_first = (int64_t)blockIdx.x * items;
  if (c_first >= n_chunks) return;
  const int n_items = (int)(n_chunks - c_first < items ? n_chunks - c_first : items);
  // a work item: chunk c, its first token, its length
  struct Item { int64_t c, t0; int L; };
  auto item_of = [&](int64_t cc) __attribute__((always_inline)) -> Item {
    Item it;
    it.c = cc;
    chunk_span(seq_off, cu, n_seq, cc, it.t0, it.L);
    return it;
  };
  Item cur = item_of(c_first);   // the item being computed
  const int64_t HvD = (int64_t)Hv * D;
  const int Hk = Hv / G;
  int role = wave >> 2;                     // phase A: 0 Tinv chain, 1 dP side
  int tw = wave & 3, tl = 16 * tw + c16;    // phase A: this lane's token
  int kt = wave % NKT, tg = wave / NKT;     // phase B: key tile, token group
  auto derive = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+v"(tid));
    asm volatile("" : "+s"(wave));
    lane = tid & 63;
    g = lane >> 4;
    g4 = 4 * g;
    c16 = lane & 15;
    role = wave >> 2;
    tw = wave & 3;
    tl = 16 * tw + c16;
    kt = wave % NKT;
    tg = wave / NKT;
  };

  // element offset, in an operand row, of this lane's values for step p:
  // natural order (both operands stored alike) ...
  auto pcol = [&](int p) { return KS == 4 ? 4 * p + g : 32 * p + 8 * g; };
  // ... or the accumulator order of AO::from_acc (the other operand stored
  // with its columns in accumulator order)
  auto acol = [&](int p) { return KS == 4 ? 16 * (p >> 2) + g4 + (p & 3) : 32 * p + 8 * g; };
  auto rdf = [&](const T* rowp, int col) __attribute__((always_inline)) -> frag {
    if constexpr (KS == 4) return rowp[col];
    else return *reinterpret_cast<const frag*>(rowp + col);
  };
  // token-tile operand: row r, step p
  auto tfr = [&](const T* tile, int r, int p) __attribute__((always_inline)) -> frag {
    return rdf(tile, TT::at(r, pcol(p)));
  };
  // the same from the Delta tile (in the storage type once converted)
  auto dlfr = [&](int r, int p) __attribute__((always_inline)) -> frag {
    return tfr(sm.tDl, r, p);
  };
  // gam of tokens s0 .. s0 + 3 (s0 % 4 == 0), and the decay factor
  // e^(a - b) where keep holds, else 0.  Branch free: the masked exponent is
  // a large negative number, so every lane evaluates the exponential
  // (otherwise the compiler puts each masked gam load and exponential
  // behind a branch of its own, serialising the loads).
  typedef double d2 __attribute__((ext_vector_type(2)));
  auto gam4 = [&](int s0, double (&o)[4]) __attribute__((always_inline)) {
    const d2 a = *reinterpret_cast<const d2*>(&sm.gam[s0]), b = *reinterpret_cast<const d2*>(&sm.gam[s0 + 2]);
    o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
  };
  auto decay = [&](double a, double b, bool keep) __attribute__((always_inline)) -> float {
    return dexp<T>(keep ? a - b : -1e30);
  };

  // ---- per item: K K^T into LDS (direct copies, read at the phase-A
  // positions by the Tinv-chain waves) ...
  constexpr int KKE = 16 / (int)sizeof(typename GL::KKT);   // elements per 16-byte piece
  auto copy_kk = [&](const Item& it, bool live) __attribute__((always_inline)) {
    const char* src = reinterpret_cast<const char*>(KKw + (it.c * Hk + kh) * CHUNK * CHUNK);
    const uint32_t bytes = live ? CHUNK * CHUNK * sizeof(typename GL::KKT) : 0u;
#pragma unroll
    for (int j = 0; j < CHUNK * CHUNK / KKE / 512; ++j) {
      const int s = (j * 8 + wave) * 64 + lane;
      copy_to_lds<CACHE_NT>(buffer_of(src, bytes), sm.KK + (j * 8 + wave) * 64 * KKE, (uint32_t)s * 16u, 0);
    }
  };
  // k_tl . k_s for s = 16 st + g4 .. + 3: block (tw, st), offset 4 lane
  auto kkv = [&](int st) __attribute__((always_inline)) -> floatx4 {
    return ld4(sm.KK + 256 * (4 * tw + st) + 4 * lane);
  };
  // ... the wave's rows of the K^T and Q^T tiles (phase-B A operands) and
  // q, k at the phase-B positions (raw storage-type values, converted where
  // used: laundered there, so the converted values are not hoisted out of
  // the head loop, where they would take twice the registers)
  frag kta[NSC], qta[NSC];
  typedef typename std::conditional<sizeof(T) == 2, u32x2, u32x4>::type raw4;
  raw4 q4[TTW], k4[TTW];
  auto raw_f4 = [&](const raw4& r) __attribute__((always_inline)) -> floatx4 {
    if constexpr (sizeof(T) == 2)
      return floatx4{lo16<T>(r.x), hi16<T>(r.x), lo16<T>(r.y), hi16<T>(r.y)};
    else
      return __builtin_bit_cast(floatx4, r);
  };
  auto load_item = [&](const Item& it) __attribute__((always_inline)) {
    const int64_t r = ((int64_t)it.c * Hk + kh) * D * CHUNK + (int64_t)(16 * kt + c16) * CHUNK;
#pragma unroll
    for (int p = 0; p < NSC; ++p) {
      kta[p] = rdf(Ktb + r, pcol(p));
      qta[p] = rdf(Qtb + r, pcol(p));
    }
    const uint32_t ldkb = (uint32_t)(ldk * sizeof(T)), ldqb = (uint32_t)(ldq * sizeof(T));
    const auto rk = buffer_of(k + it.t0 * ldk + (int64_t)kh * D, (uint32_t)it.L * ldkb);
    const auto rq = buffer_of(q + it.t0 * ldq + (int64_t)kh * D, (uint32_t)it.L * ldqb);
#pragma unroll
    for (int tt = 0; tt < TTW; ++tt) {
      const int t = 16 * (tg * TTW + tt) + c16, kc = 16 * kt + g4;
      if constexpr (sizeof(T) == 2) {
        q4[tt] = __builtin_bit_cast(raw4, __builtin_amdgcn_raw_buffer_load_b64(rq, (uint32_t)t * ldqb + (uint32_t)kc * 2, 0, 0));
        k4[tt] = __builtin_bit_cast(raw4, __builtin_amdgcn_raw_buffer_load_b64(rk, (uint32_t)t * ldkb + (uint32_t)kc * 2, 0, 0));
      } else {
        q4[tt] = __builtin_bit_cast(raw4, __builtin_amdgcn_raw_buffer_load_b128(rq, (uint32_t)t * ldqb + (uint32_t)kc * 4, 0, 0));
        k4[tt] = __builtin_bit_cast(raw4, __builtin_amdgcn_raw_buffer_load_b128(rk, (uint32_t)t * ldkb + (uint32_t)kc * 4, 0, 0));
      }
    }
  };
  // ---- per head: the token tiles (direct copies by the first NCW waves,
  // rows past the chunk end re-read its last row) ...
  constexpr int NCW = TT::PIECES / 64 < 8 ? TT::PIECES / 64 : 8;
  // (live false: an empty source range, every copy reads zero and touches no
  // memory; the requests are issued all the same, so the wait counts after
  // them do not depend on whether a next head exists)
  auto copy_rows = [&](T* dst, const T* src, uint32_t ldb, int L, bool live) __attribute__((always_inline)) {
    if (NCW == 8 || wave < NCW) {   // (a test the compiler can drop when all waves copy)
      const auto rs = buffer_of(src, live ? (uint32_t)L * ldb : 0u);
#pragma unroll
      for (int j = 0; j < TT::PIECES / (64 * NCW); ++j) {
        const int s = (j * NCW + wave) * 64 + lane, r = s / TT::RP;
        const uint32_t off = (uint32_t)(r < L ? r : L - 1) * ldb + (uint32_t)((s % TT::RP) ^ TT::swz(r)) * 16u;
        copy_to_lds<CACHE_NT>(rs, dst + (j * NCW + wave) * 64 * TT::EPP, off, 0);
      }
    }
  };
  // ... the same from a chunk's blocks of SBV-column rows (R, Delta): piece
  // q of a row lies in block q / PPB
  auto copy_blk = [&](T* dst, const T* blk0, int L, bool live) __attribute__((always_inline)) {
    constexpr int PPB = SBV * (int)sizeof(T) / 16;   // pieces per block row
    if (NCW == 8 || wave < NCW) {
      const auto rs = buffer_of(blk0, live ? (uint32_t)(CHUNK * D * sizeof(T)) : 0u);
#pragma unroll
      for (int j = 0; j < TT::PIECES / (64 * NCW); ++j) {
        const int s = (j * NCW + wave) * 64 + lane, r = s / TT::RP, q = (s % TT::RP) ^ TT::swz(r);
        const uint32_t off = (uint32_t)(q / PPB) * (uint32_t)(CHUNK * SBV * sizeof(T)) +
                             (uint32_t)(r < L ? r : L - 1) * (uint32_t)(SBV * sizeof(T)) + (uint32_t)(q % PPB) * 16u;
        copy_to_lds<CACHE_NT>(rs, dst + (j * NCW + wave) * 64 * TT::EPP, off, 0);
      }
    }
  };
  // (R is read in phase A only, so it comes with Tinv, a phase earlier)
  auto copy_head = [&](const Item& it, int h, bool live) __attribute__((always_inline)) {
    const uint32_t rowb = (uint32_t)(HvD * sizeof(T));
    copy_rows(sm.tO, dout + it.t0 * HvD + (int64_t)h * D, rowb, it.L, live);
    copy_blk(sm.tDl, reinterpret_cast<const T*>(Dlw) + (it.c * Hv + h) * CHUNK * D, it.L, live);
    copy_rows(sm.tdR, dvo + it.t0 * lddv + (int64_t)h * D, (uint32_t)(lddv * sizeof(T)), it.L, live);
  };
  auto copy_r = [&](const Item& it, int h, bool live) __attribute__((always_inline)) {
    copy_blk(sm.tR, Rw + (it.c * Hv + h) * CHUNK * D, it.L, live);
  };
  // ... the gate values (wave 0: loaded into registers a phase before they
  // go to LDS) ...
  double gnext = 0.0;
  float bnext = 0.f;
  auto fetch_gates = [&](const Item& it, int h) __attribute__((always_inline)) {
    if (wave == 0) {
      gnext = gcum[(it.c * Hv + h) * CHUNK + lane];
      bnext = bw[(it.c * Hv + h) * CHUNK + lane];   // (zero past the chunk end)
    }
  };
  auto put_gates = [&]() __attribute__((always_inline)) {
    if (wave == 0) {
      sm.gam[lane] = gnext;
      sm.bet[lane] = bnext;
      // gam is flat past the chunk length, so these are the factors of
      // token min(t, L - 1)
      const double glast = __shfl(gnext, CHUNK - 1, 64);
      sm.Gm[lane] = dexp<T>(gnext);
      sm.dc[lane] = dexp<T>(glast - gnext);
    }
  };
  // ... Tinv (16-bit types: into LDS, by direct copies) ...
  typedef typename GL::TI TI;
  auto copy_tinv = [&](const Item& it, int h, bool live) __attribute__((always_inline)) {
    if constexpr (GL::TIN_LDS) {
      const char* src = reinterpret_cast<const char*>(Tib + (it.c * Hv + h) * 2 * CHUNK * CHUNK);
      const uint32_t bytes = live ? CHUNK * CHUNK * sizeof(T) : 0u;
#pragma unroll
      for (int j = 0; j < TI::PIECES / 512; ++j) {
        const int s = (j * 8 + wave) * 64 + lane, r = s / TI::RP;
        const uint32_t off = (uint32_t)(r * TI::RP + ((s % TI::RP) ^ TI::swz(r))) * 16u;
        copy_to_lds<CACHE_NT>(buffer_of(src, bytes), sm.Tin + (j * 8 + wave) * 64 * TI::EPP, off, 0);
      }
    }
  };
  // element (r, col) of Tinv (m = 0, columns in accumulator order) or, for
  // fp32, Tinv^T (m = 1)
  auto tin = [&](int h, int m, int r, int col) __attribute__((always_inline)) -> const T* {
    if constexpr (GL::TIN_LDS) return sm.Tin + TI::at(r, col);
    else return Tib + (cur.c * Hv + h) * 2 * CHUNK * CHUNK + m * CHUNK * CHUNK + r * CHUNK + col;
  };
  // B operand of step p from row tl of Tinv^T (reduction indices pcol(p)
  // .. + 7, natural order).  16-bit: two transposing reads down column tl of
  // Tinv, whose columns are in accumulator order: lanes 4a .. 4a + 3 of a
  // group point at stored columns 32 (tw / 2) + 8 a + 4 (tw % 2) .. + 3, and
  // lane j of group g at row 32 p + 8 g + j / 4 (then 4 rows further)
  auto tinvt_frag = [&](int h, int p) __attribute__((always_inline)) -> frag {
    if constexpr (GL::TIN_LDS) {
      const int col = 32 * (tw >> 1) + 8 * (c16 & 3) + 4 * (tw & 1), r = 32 * p + 8 * g + (c16 >> 2);
      const u32x2 lo = lds_read_tr4(sm.Tin + TI::at(r, col)), hi = lds_read_tr4(sm.Tin + TI::at(r + 4, col));
      return __builtin_bit_cast(frag, u32x4{lo[0], lo[1], hi[0], hi[1]});
    } else {
      return rdf(tin(h, 1, tl, pcol(p)), 0);
    }
  };
  // ... the phase-A operands: the Tinv-chain waves' rows of dDelta or the
  // dP-side waves' P values, as loaded, in one register array for both roles
  // (two arrays would each stay live across the head loop in the waves of
  // the other role); converted where used, so that nothing waits for the
  // loads where they are issued
  constexpr int FR = (int)(sizeof(frag) / 4);     // dwords per operand fragment
  constexpr int NAD = NSD * FR, NPD = 4 * (int)sizeof(CT);
  constexpr int NA = NAD > NPD ? NAD : NPD;
  uint32_t aop[NA];
  // (dDelta: row tl of the chunk's blocks of SBV columns, one buffer per
  // block, so that rows past the chunk end read zero)
  auto load_tinv = [&](const Item& it, int h, bool live) __attribute__((always_inline)) {
    constexpr uint32_t rowb = (uint32_t)(SBV * sizeof(T));
    const T* blk0 = ddw + (it.c * Hv + h) * CHUNK * D;
#pragma unroll
    for (int p = 0; p < NSD; ++p) {
      const int b = p * KS / SBV;   // the block of columns pcol(p) .. (the same for every lane)
      const auto rs = buffer_of(blk0 + (int64_t)b * CHUNK * SBV, live ? (uint32_t)it.L * rowb : 0u);
      const frag f = buffer_frag<T>(rs, (uint32_t)tl * rowb + (uint32_t)(pcol(p) - b * SBV) * sizeof(T));
      if constexpr (FR == 4) {
        const u32x4 w = __builtin_bit_cast(u32x4, f);
#pragma unroll
        for (int j = 0; j < 4; ++j) aop[4 * p + j] = w[j];
      } else {
        aop[p] = __builtin_bit_cast(uint32_t, f);
      }
    }
  };
  auto ddB = [&](int p) __attribute__((always_inline)) -> frag {
    if constexpr (FR == 4) return __builtin_bit_cast(frag, u32x4{aop[4 * p], aop[4 * p + 1], aop[4 * p + 2], aop[4 * p + 3]});
    else return __builtin_bit_cast(frag, aop[p]);
  };
  auto load_p = [&](const Item& it, int h, bool live) __attribute__((always_inline)) {
    const auto rs = buffer_of(Pw + (it.c * Hv + h) * CHUNK * CHUNK, live ? CHUNK * CHUNK * sizeof(CT) : 0u);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint32_t off = (uint32_t)(tl * CHUNK + acc_col<CT>(16 * st + g4)) * sizeof(CT);
      if constexpr (sizeof(CT) == 2) {
        const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, CACHE_NT));
        aop[2 * st] = w[0];
        aop[2 * st + 1] = w[1];
      } else {
        const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, CACHE_NT));
#pragma unroll
        for (int j = 0; j < 4; ++j) aop[4 * st + j] = w[j];
      }
    }
  };
  auto pE = [&](int st) __attribute__((always_inline)) -> floatx4 {
    if constexpr (sizeof(CT) == 2) {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      const h2 a = __builtin_bit_cast(h2, aop[2 * st]), b = __builtin_bit_cast(h2, aop[2 * st + 1]);
      return floatx4{(float)a[0], (float)a[1], (float)b[0], (float)b[1]};
    } else {
      return floatx4{__uint_as_float(aop[4 * st]), __uint_as_float(aop[4 * st + 1]),
                     __uint_as_float(aop[4 * st + 2]), __uint_as_float(aop[4 * st + 3])};
    }
  };
  // ... and every wave's rows of the saved states (phase B)
  frag hA[NSD], dhA[NSD];
  auto load_states = [&](int h) __attribute__((always_inline)) {
    const int64_t r = (cur.c * Hv + h) * D * D;
#pragma unroll
    for (int p = 0; p < NSD; ++p) {
      const int64_t e = r + blk_at(16 * kt + c16, pcol(p), D);
      if constexpr (KS == 4) {
        hA[p] = rdf(hst + e, 0);
        dhA[p] = rdf(dhst + e, 0);
      } else {   // read once, a kilobyte of whole lines per wave: non-temporal
        hA[p] = __builtin_nontemporal_load(reinterpret_cast<const frag*>(hst + e));
        dhA[p] = __builtin_nontemporal_load(reinterpret_cast<const frag*>(dhst + e));
      }
    }
  };
  auto load_a = [&](const Item& it, int h, bool live) __attribute__((always_inline)) {
    if (role == 0) load_tinv(it, h, live);
    else load_p(it, h, live);
  };

  load_item(cur);
  copy_kk(cur, true);
  copy_head(cur, kh * G, true);
  copy_r(cur, kh * G, true);
  copy_tinv(cur, kh * G, true);
  fetch_gates(cur, kh * G);
  load_a(cur, kh * G, true);
  put_gates();
  floatx4 dQa[TTW], dKa[TTW];
#pragma unroll
  for (int tt = 0; tt < TTW; ++tt) dQa[tt] = dKa[tt] = zero4();

  // Every operand of the next head (head h + 1, or the first head of the
  // next item) is requested while head h finishes: R, Tinv (and K K^T)
  // before phase B, the other tiles, the phase-A operands, the gates (and
  // the item's registers) after it.  The barriers they have to pass are
  // LDS-only (a full barrier would wait for the copies); the one at the top
  // of a head waits for all.  After the last head the same requests go out
  // with empty ranges (gates: the last head's again).
  // dg and dbeta of a head from its partials (set p): the box sums, the
  // suffix sum of the chunk-start terms and the exclusive prefix sum of the
  // chunk-end terms, one token per lane
  struct Prev { int64_t t0; int L, h; double glast; };
  Prev prev{0, 0, 0, 0.0};
  constexpr int TAIL_WAVE = 4;
  auto dg_tail = [&](int p, const Prev& pv) __attribute__((always_inline)) {
    const int t = lane;
    float y = 0.f, db = sm.rowB[p][0][t] + sm.rowB[p][1][t], zt = 0.f, ips = 0.f;
    const float box = ((sm.boxE[p][0][t] + sm.boxE[p][1][t]) + sm.boxE[p][2][t]) + sm.boxE[p][3][t];
#pragma unroll
    for (int w = 0; w < 4; ++w) db += sm.colB[p][w][t];
#pragma unroll
    for (int w = 0; w < NKT; ++w) {
      y += sm.rowX[p][w][t];
      zt += sm.rowZ[p][w][t];
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) ips += sm.red[p][w];
    if (t == pv.L - 1) y += dexp<T>(pv.glast) * ips;
    if (t >= pv.L) { y = 0.f; zt = 0.f; }
    const float dgs = box + wave_suffix_dpp(y, lane) + (wave_prefix_dpp(zt, lane) - zt);
    if (t < pv.L) {
      dg[(pv.t0 + t) * Hv + pv.h] = dgs;
      dbeta[(pv.t0 + t) * Hv + pv.h] = db;
    }
  };

  const int n_steps = n_items * G;
  for (int step = 0, hh = 0; step < n_steps; ++step) {
    const int h = kh * G + hh;
    const bool last = hh + 1 == G;           // the item's last head
    const bool live = step + 1 < n_steps;    // a next head exists
    const Item nx = last && live ? item_of(cur.c + 1) : cur;
    const int hn = !live ? h : last ? kh * G : h + 1;
    derive();
    issue_fence();
    __syncthreads();   // this head's tiles, gates and phase-A operands are in
    if constexpr (__is_same(T, bf16)) {
      // the saved-state pass's fp16 Delta, rounded to bf16 in place (one
      // 16-byte piece per thread and step), before any wave reads it
#pragma unroll
      for (int j = 0; j < (TT::PIECES + 511) / 512; ++j) {
        if (TT::PIECES % 512 != 0 && tid + 512 * j >= TT::PIECES) break;
        u32x4* pp = reinterpret_cast<u32x4*>(sm.tDl) + tid + 512 * j;
        const u32x4 w = *pp;
        u32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = pack2<bf16>(lo16<fp16>(w[e]), hi16<fp16>(w[e]));
        *pp = y;
      }
      lds_barrier();
    }
    // =============== phase A: pair products (s x t tiles, t = tl)
    const int par = step & 1;                 // this head's set of dg partials
    const double gt = sm.gam[tl];
    const double gl_head = sm.gam[CHUNK - 1];
    const float bt = sm.bet[tl];
    // the previous head's dg and dbeta, on a dP-side wave (that side has
    // slack in phase A; the Tinv chain does not)
    if (wave == TAIL_WAVE && step > 0) dg_tail(par ^ 1, prev);
    floatx4 ep[4];
    if (role == 0) {
      // dM^T = R dDelta^T
      floatx4 dMt[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        dMt[st] = zero4();
#pragma unroll
        for (int p = 0; p < NSD; ++p) dMt[st] = MM::mma(tfr(sm.tR, 16 * st + c16, p), ddB(p), dMt[st]);
      }
      // the first dbeta term summed over t (the 16 lanes of a group: lane
      // c16 of group g keeps the sum for s = 16 (c16 / 4) + 4 g + c16 % 4);
      // then dTinv^T in place of dM^T
      float cbm = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const float4 bs = *reinterpret_cast<const float4*>(&sm.bet[16 * st + g4]);
        const float bsv[4] = {bs.x, bs.y, bs.z, bs.w};
        const floatx4 te = ld4(tin(h, 0, tl, acc_col<T>(16 * st + g4)));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 16 * st + g4 + i;
          const float cb = lane_group_sum<16>(dMt[st][i] * te[i]);
          cbm = c16 == 4 * st + i ? cb : cbm;
          dMt[st][i] = s < tl ? dMt[st][i] * bsv[i] : 0.f;
        }
      }
      sm.colB[par][tw][16 * (c16 >> 2) + g4 + (c16 & 3)] = cbm;
      // Y = dTinv Tinv^T for tokens t of this wave (A from the accumulators),
      // into Y^T rows
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        floatx4 y = zero4();
#pragma unroll
        for (int p = 0; p < NSC; ++p) y = MM::mma(AO::from_acc(dMt, p), rdf(tin(h, 0, 16 * st + c16, acol(p)), 0), y);
        store4(&sm.YT[16 * st + c16][16 * tw + g4], y[0], y[1], y[2], y[3]);
      }
    } else {
      // dP^T = Delta dO^T and dP = dO Delta^T
      floatx4 dPt[4], dPn[4];
      {
        frag ob[NSD];
#pragma unroll
        for (int p = 0; p < NSD; ++p) ob[p] = tfr(sm.tO, tl, p);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          dPt[st] = dPn[st] = zero4();
#pragma unroll
          for (int p = 0; p < NSD; ++p) {
            const frag da = dlfr(16 * st + c16, p);
            dPt[st] = MM::mma(da, ob[p], dPt[st]);
            dPn[st] = MM::mma(ob[p], da, dPn[st]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // dP o D (rows t), the dP part of the pair terms (added to E once the
      // Tinv-chain waves have written theirs)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const floatx4 pv = pE(st);
        double gs[4];
        gam4(16 * st + g4, gs);
        float pd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 16 * st + g4 + i;
          const float Dts = decay(gt, gs[i], s <= tl);
          ep[st][i] = (s < tl && tl < cur.L) ? dPt[st][i] * pv[i] : 0.f;
          pd[i] = dPt[st][i] * Dts;
        }
        store4(&sm.dPD[tl][acc_col<T>(16 * st + g4)], pd[0], pd[1], pd[2], pd[3]);
      }
      // scale (dP o D)^T from the dP tiles: rows t = 16 tw + 4 g + i, column s
      double gtt[4];
      gam4(16 * tw + g4, gtt);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int s = 16 * st + c16;
        const double gs = sm.gam[s];
        float pd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * tw + g4 + i;
          pd[i] = scale * dPn[st][i] * decay(gtt[i], gs, s <= t);
        }
        store4(&sm.dPDt[s][acc_col<T>(16 * tw + g4)], pd[0], pd[1], pd[2], pd[3]);
      }
    }
    load_states(h);
    issue_fence();
    __syncthreads();   // Y^T is complete
    {
      // dA^T = -Y^T Tinv (rows s, column t = tl), then WA, the dA part of the
      // pair terms and the second dbeta term; the Tinv-chain waves take row
      // blocks s of 0 .. 31, the dP waves (the same columns t) 32 .. 63
      float rb = 0.f;
#pragma unroll
      for (int sj = 0; sj < 2; ++sj) {
        const int st = 2 * role + sj;
        const floatx4 kks = kkv(st);
        double gs[4];
        gam4(16 * st + g4, gs);
        floatx4 da = zero4();
#pragma unroll
        for (int p = 0; p < NSC; ++p)
          da = MM::mma(rdf(&sm.YT[16 * st + c16][0], pcol(p)), tinvt_frag(h, p), da);
        float wa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 16 * st + g4 + i;
          const bool lower = s < tl;
          const float Dts = decay(gt, gs[i], lower);
          const float dA = lower ? -da[i] : 0.f;
          const float dAD = dA * Dts;
          sm.E[tl][s] = tl < cur.L ? dAD * bt * kks[i] : 0.f;
          rb += dAD * kks[i];
          wa[i] = dAD * bt;
        }
        // WS: row tl takes wa for s <= tl (zero on the diagonal), row s
        // takes it at column tl for s < tl; every element has one writer.
        // A store that is not this lane's goes to a padding column of the
        // same row instead (branch free).
        const int s0 = 16 * st + g4, padc = CHUNK + (c16 & (GL::LDP - CHUNK - 1));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sm.WS[tl][s0 + i <= tl ? acc_col<T>(s0) + i : padc] = (T)wa[i];
          sm.WS[s0 + i][s0 + i < tl ? acc_col<T>(tl) : padc] = (T)wa[i];
        }
      }
      rb += __shfl_xor(rb, 16, 64);
      rb += __shfl_xor(rb, 32, 64);
      if (g == 0) sm.rowB[par][role][tl] = rb;
    }
    __syncthreads();   // WS and the dA part of the pair terms are in
    if (role == 1) {   // (E is read after phase B's barrier)
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.E[tl][16 * st + g4 + i] += ep[st][i];
    }
    // R and Tinv (and on the item's last head K K^T) are no longer read
    copy_r(nx, hn, live);
    copy_tinv(nx, hn, live);
    if (last) copy_kk(nx, live);

    // =============== phase B: token x key products (k x t tiles)
    {
      float ipv = 0.f;
      if (tg == 0) {
#pragma unroll
        for (int p = 0; p < NSD; ++p) {
          if constexpr (KS == 4) {
            ipv += to_f(hA[p]) * to_f(dhA[p]);
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) ipv += (float)hA[p][j] * (float)dhA[p][j];
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < TTW; ++tt) {
        const int t = 16 * (tg * TTW + tt) + c16;
        floatx4 x1 = zero4(), x2 = zero4(), x3 = zero4();
#pragma unroll
        for (int p = 0; p < NSD; ++p) {
          x1 = MM::mma(hA[p], tfr(sm.tO, t, p), x1);
          x2 = MM::mma(hA[p], tfr(sm.tdR, t, p), x2);
          x3 = MM::mma(dhA[p], dlfr(t, p), x3);
        }
#pragma unroll
        for (int p = 0; p < NSC; ++p) {
          dQa[tt] = MM::mma(kta[p], rdf(&sm.dPD[t][0], pcol(p)), dQa[tt]);
          dKa[tt] = MM::mma(qta[p], rdf(&sm.dPDt[t][0], pcol(p)), dKa[tt]);
          dKa[tt] = MM::mma(kta[p], rdf(&sm.WS[t][0], pcol(p)), dKa[tt]);
        }
        const float Gt = sm.Gm[t], dct = sm.dc[t];
        raw4 qr = q4[tt], kr = k4[tt];
        asm volatile("" : "+v"(qr), "+v"(kr));
        const floatx4 qv = raw_f4(qr), kv = raw_f4(kr);
        float rx = 0.f, rz = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dQa[tt][i] += Gt * x1[i];
          dKa[tt][i] += dct * x3[i] - Gt * x2[i];
          rx += Gt * (scale * x1[i] * qv[i] - x2[i] * kv[i]);
          rz += dct * x3[i] * kv[i];
        }
        rx += __shfl_xor(rx, 16, 64);
        rx += __shfl_xor(rx, 32, 64);
        rz += __shfl_xor(rz, 16, 64);
        rz += __shfl_xor(rz, 32, 64);
        if (g == 0) {
          sm.rowX[par][kt][t] = rx;
          sm.rowZ[par][kt][t] = rz;
        }
      }
      ipv = wave_sum_dpp(ipv);
      if (lane == 0) sm.red[par][wave] = ipv;
    }
    lds_barrier();   // the token tiles are free; every partial is in
    if (last) {
      // dq = scale dQ, dk of the item: each wave puts its four consecutive
      // key columns of a token per lane into rows of the pair tiles (free
      // until the next head's phase A), and after a barrier the rows leave
      // whole, 16 bytes per lane; then the next item's registers.  (Stores
      // straight from the accumulators wrote 32 bytes of each row per wave.)
      T* const stq = &sm.YT[0][0];
      T* const stk = stq + CHUNK * GL::QKR;
#pragma unroll
      for (int tt = 0; tt < TTW; ++tt) {
        const int t = 16 * (tg * TTW + tt) + c16, kc = 16 * kt + g4;
        const floatx4 xq = dQa[tt], xk = dKa[tt];
        store4(stq + t * GL::QKR + kc, scale * xq[0], scale * xq[1], scale * xq[2], scale * xq[3]);
        store4(stk + t * GL::QKR + kc, xk[0], xk[1], xk[2], xk[3]);
        dQa[tt] = dKa[tt] = zero4();
      }
      lds_barrier();
      const uint32_t rq = (uint32_t)(lddq * sizeof(T)), rk = (uint32_t)(lddk * sizeof(T));
      const auto bq = buffer_of(dq + cur.t0 * lddq + (int64_t)kh * D, (uint32_t)cur.L * rq);
      const auto bk = buffer_of(dk + cur.t0 * lddk + (int64_t)kh * D, (uint32_t)cur.L * rk);
      constexpr int PPRW = D * (int)sizeof(T) / 16;   // 16-byte pieces per row
      constexpr int NP = CHUNK * PPRW;                 // pieces per tile
#pragma unroll
      for (int j = 0; j < (NP + 511) / 512; ++j) {
        const int i = tid + 512 * j, r = i / PPRW, pc = i % PPRW;
        if (NP % 512 != 0 && i >= NP) break;
        // (inline asm reads, each waiting for itself: a plain LDS read here
        // would wait for the direct copies still in flight)
        u32x4 vq, vk;
        asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(vq), "=&v"(vk)
                     : "v"(lds_offset(stq + r * GL::QKR) + 16u * pc), "v"(lds_offset(stk + r * GL::QKR) + 16u * pc)
                     : "memory");
        __builtin_amdgcn_raw_buffer_store_b128(vq, bq, (uint32_t)r * rq + 16u * pc, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(vk, bk, (uint32_t)r * rk + 16u * pc, 0, 0);
      }
      if (live) load_item(nx);
    }
    copy_head(nx, hn, live);
    fetch_gates(nx, hn);
    load_a(nx, hn, live);

    // =============== dg, dbeta (waves 0-3).  With gamma the in-chunk
    // cumulative gate, dg_i = sum_{t >= i} dgam_t.  Three parts, each a sum
    // of terms that all carry the decay across token i, so no large terms
    // cancel when that decay is strong:
    //  - pair terms E[t][s] (s < t) add to dgam_t and subtract from dgam_s;
    //    their part of dg_i is the box sum over t >= i > s, taken as column
    //    suffix sums over rows, then sums along rows;
    //  - the chunk-start terms y_t (rowX, and the state term at the last
    //    token) enter as the suffix sum over t >= i;
    //  - the decay-to-chunk-end terms z_t enter dgam as -z_t and as +sum z
    //    at the last token: their part is the prefix sum over t < i.
    if (wave < 4) {
      // Wave w takes columns s = 16 w + j of E (j = lane % 16) over rows
      // 16 q .. 16 q + 15 (q = lane / 16).  Suffix sums down the quarter plus
      // the later quarters' column totals give C[i][s] = sum_{t >= i} E[t][s];
      // the block's part of the box sum of row i is the sum of C[i][s] over
      // its columns s < i, for the quarter's 16 rows at once: a
      // reduce-scatter over the 16 lanes, four DPP swaps that each pair lanes
      // differing in one bit (a lane keeps the half of its rows whose bit
      // matches its own and adds the partner's copy), leaving row 16 q + j in
      // lane j.
      const int j = lane & 15, q = lane >> 4, s = 16 * wave + j;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = sm.E[16 * q + r][s];
#pragma unroll
      for (int r = 14; r >= 0; --r) x[r] += x[r + 1];
      const float c1 = __shfl(x[0], j + 16, 64), c2 = __shfl(x[0], j + 32, 64),
                  c3 = __shfl(x[0], j + 48, 64);
      const float off = q == 0 ? (c3 + c2) + c1 : q == 1 ? c3 + c2 : q == 2 ? c3 : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = s < 16 * q + r ? x[r] + off : 0.f;
      auto split = [&](auto ctrl, int half, bool hi) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < half; ++r) {
          const float send = hi ? x[r] : x[r + half], keep = hi ? x[r + half] : x[r];
          x[r] = keep + dpp_f<decltype(ctrl)::value>(send);
        }
      };
      split(std::integral_constant<int, 0x140>{}, 8, (j & 8) != 0);   // row_mirror: bit 3
      split(std::integral_constant<int, 0x141>{}, 4, (j & 4) != 0);   // row_half_mirror: bit 2
      split(std::integral_constant<int, 0x4E>{}, 2, (j & 2) != 0);    // lane ^ 2
      split(std::integral_constant<int, 0xB1>{}, 1, (j & 1) != 0);    // lane ^ 1
      sm.boxE[par][wave][16 * q + j] = x[0];
    }
    lds_barrier();
    // (since phase B's barrier only wave 0 reads the gates, and it alone
    // writes the next head's)
    put_gates();
    prev = Prev{cur.t0, cur.L, h, gl_head};
    if (last) cur = nx;
    hh = last ? 0 : hh + 1;
  }
  // the last head's dg and dbeta (its partials are in since the loop's last
  // barrier)
  if (wave == TAIL_WAVE && n_steps > 0) dg_tail((n_steps - 1) & 1, prev);
}

// ---------------------------------------------------------------------------
hipError_t launch_chunk_bwd_grads(const gdn_shape& s, const void* q, const void* k, int64_t ldq,
                                  int64_t ldk, const float* beta, float scale, const int32_t* cu,
                                  const void* dout, const void* dv, int64_t lddv, void* dq,
                                  void* dk, int64_t lddq, int64_t lddk, float* dg, float* dbeta,
                                  void* wsv, hipStream_t st) {
  char* ws = (char*)wsv;
  const ChunkLayout Ly = chunk_layout(s, ChunkFlow::Bwd);
  if (Ly.nt_max == 0 || s.total_tokens == 0) return hipSuccess;
  return dispatch_chunk(s, [&](auto cf) {
    using T = typename decltype(cf)::type;
    constexpr int D = decltype(cf)::d;
    static_assert(sizeof(GradLds<T, D>) <= 160 * 1024, "gradient kernel LDS budget");
    const size_t shm = sizeof(GradLds<T, D>);
    auto kern = chunk_grad_kernel<T, D>;
    hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    const int items = grad_items(Ly.nt_max, s.hk);
    hipLaunchKernelGGL(kern, dim3((unsigned)((Ly.nt_max + items - 1) / items), s.hk), dim3(512), shm, st, (const T*)q,
                       (const T*)k, ldq, ldk, cu, (const int32_t*)(ws + Ly.seq_off), s.n_seq,
                       s.hv, s.hv / s.hk, scale, (const double*)(ws + Ly.gcum), (const float*)(ws + Ly.bw),
                       (const typename Compute<T>::type*)(ws + Ly.pw), (const T*)(ws + Ly.tib),
                       (const T*)(ws + Ly.ktb), (const T*)(ws + Ly.qtb), (const T*)(ws + Ly.h),
                       (const T*)(ws + Ly.dh), (const T*)(ws + Ly.rw),
                       sizeof(T) == 2 ? (const void*)(ws + Ly.dl16w) : (const void*)(ws + Ly.dlw),
                       (const T*)(ws + Ly.ddw), (const typename Compute<T>::type*)(ws + Ly.kkw),
                       (const T*)dout, (const T*)dv, lddv, (T*)dq,
                       (T*)dk, lddq, lddk, dg, dbeta, items);
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
