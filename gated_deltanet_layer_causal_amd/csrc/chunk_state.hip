// Chunked gated delta rule: the sequential state pass over the chunks of each
// sequence (forward outputs, or the states the backward needs).
//
// With the preparation's W = M diag(Gam) K, the chunk recurrence is
//   U     = M V                       (needs no state)
//   Delta = U - W S^T
//   S     <- Gam_L S + (diag(dec) Delta)^T K
// and the outputs O = diag(Gam) scale Q S^T + P Delta (MODE 0), or the
// chunk-start states S themselves (MODE 1), from which chunk_out.hip forms
// R, Delta and O chunk by chunk in parallel.  Only the two products through
// S are sequential; everything else hangs off them.  MODE 1 with 16-bit
// types takes the K rows alone: Delta = M R with R = V - diag(Gam) K S^T
// (W S^T = M diag(Gam) K S^T), and K^T for the update comes from the same
// rows by transposing LDS reads, so a chunk copies K, M and V only.
//
// One workgroup per (sequence, value head, block of 16 * NW value rows of the
// state); wave w owns 16 value rows and keeps its d_k x 16 slice of S^T in
// MFMA accumulators for the whole sequence.  Its products with S take S
// straight from those accumulators as the B operand: an accumulator tile
// holds rows 4 (l / 16) + i of column l % 16 in lane l, so two stacked tiles
// give every lane eight reduction indices, and the A operand is read from
// LDS in the same (permuted) reduction order (AccOrder; the preparation
// stores those operands with their columns in that order, acc_col).
//
// The chunk's shared operands (W, K^T, M, V, Gam, dec; Q and P in MODE 0) are copied
// from memory straight into LDS (global_load_lds, no registers), into one of
// two buffers: chunk c + 1 streams into one while chunk c computes from the
// other, so a chunk step has a single barrier.  A direct copy writes 64
// consecutive 16-byte pieces per wave, so the LDS tiles are unpadded and
// bank conflicts are avoided by permuting the 16-byte pieces of each row
// (Tile).  Every address that varies by lane is computed once: copies go
// through buffer resources (uniform base, per-lane offset) and LDS reads use
// per-lane offsets plus constants.
//
// Row blocks past D / BV (nblk = 2 D / BV, the first pass of the segmented
// scan) start from identity rows and read no values, so their rows end as the
// span's transition Phi.  The DRY instantiation (that first pass, which only
// needs S_final) stages and stores nothing: in the K-rows form its movers'
// counted waits leave out the stores (NFL = 0); elsewhere its stores go out
// with empty ranges (dropped).
#include "chunk_stream.h"

namespace gdn {

template <typename T, int D, int NW, int MODE> struct StateBuf {
  typedef typename Compute<T>::type CT;
  static constexpr int BV = 16 * NW;
  typedef Tile<CT, CHUNK, D> TW;        // W, and Q / K rows
  typedef Tile<CT, D, CHUNK> TKt;       // K^T
  typedef Tile<CT, CHUNK, CHUNK> TM;    // M, P
  typedef Tile<T, CHUNK, BV, 3> TV;     // value rows (storage type)
  static constexpr bool KR = MODE == 1 && sizeof(T) == 2;   // the K-rows form
  CT W[TW::PIECES * TW::EPP];           // W, or the K rows (KR)
  CT Kt[KR ? 8 : TKt::PIECES * TKt::EPP];
  CT X[MODE == 0 ? TW::PIECES * TW::EPP : 8];   // Q rows
  CT M[TM::PIECES * TM::EPP];
  CT P[MODE == 0 ? TM::PIECES * TM::EPP : 8];
  T V[TV::PIECES * TV::EPP];
  float G[CHUNK], Dc[CHUNK];            // Gam_t, dec_t
} __attribute__((aligned(16)));

template <typename T, int D, int NW, int MODE, bool DRY>
__global__ void __launch_bounds__((StateBuf<T, D, NW, MODE>::KR ? 128 * NW : 64 * NW)) chunk_state_kernel(
    const T* __restrict__ v, int64_t ldv, const int32_t* __restrict__ spans,
    const int32_t* __restrict__ n_spans, int nblk, int Hv, int G, float scale,
    const typename Compute<T>::type* __restrict__ Mw, const typename Compute<T>::type* __restrict__ Pw,
    const typename Compute<T>::type* __restrict__ Ww, const typename Compute<T>::type* __restrict__ Ktw,
    const typename Compute<T>::type* __restrict__ Xw, const float* __restrict__ Gw,
    const float* __restrict__ Dw, const float* __restrict__ S0, float* __restrict__ S_final,
    T* __restrict__ o, T* __restrict__ hst, T* __restrict__ Rw,
    typename Compute<T>::type* __restrict__ Dl16w, int n_items) {
  typedef typename Compute<T>::type CT;
  typedef Mma<CT> MM;
  typedef AccOrder<CT> AO;
  typedef typename MM::frag frag;
  typedef StateBuf<T, D, NW, MODE> SB;
  typedef typename SB::TW TW;
  typedef typename SB::TKt TKt;
  typedef typename SB::TM TM;
  typedef typename SB::TV TV;
  constexpr int THREADS = 64 * NW;
  constexpr int BV = SB::BV;
  constexpr int KS = MM::KS;
  constexpr int NSD = D / KS;       // MFMA steps over d_k
  constexpr int NSC = CHUNK / KS;   // MFMA steps over the chunk
  constexpr int NKT = D / 16;       // state tiles per wave
  constexpr int NV = KS == 4 ? 1 : 8;   // operand values per lane per step
  static_assert(TW::PIECES % THREADS == 0 && TKt::PIECES % THREADS == 0 &&
                TM::PIECES % THREADS == 0 && TV::PIECES % THREADS == 0,
                "direct copies cover whole waves");
  __shared__ SB bufA, bufB;

  const int tid = threadIdx.x, lane = tid & 63;
  // (K-rows form: waves [0, NW) compute, waves [NW, 2 NW) move the operands)
  const int wave_ = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool mover = SB::KR && wave_ >= NW;
  const int wave = mover ? wave_ - NW : wave_;
  // item -> (span n, value head h, row block vb); blocks vb >= D / BV (the
  // first pass of the segmented scan) carry identity rows with no values:
  // their state rows become the span's transition Phi
  const int item = xcd_item(blockIdx.x, n_items);
  const int vb = item % nblk, h = (item / nblk) % Hv, n = item / (nblk * Hv);
  if (n >= *n_spans) return;
  const bool phi = DRY && vb >= D / BV;   // (only the first pass has identity rows)
  const int kh = h / G, Hk = Hv / G;
  const int v0 = vb * BV;
  const int g = lane >> 4, g4 = 4 * g, c16 = lane & 15;
  const int vcol = 16 * wave + c16;                 // value row of S this lane's columns hold
  const int64_t HvD = (int64_t)Hv * D;

  floatx4 S[NKT];   // S^T tiles: rows k = 16 kt + g4 + i, column v0 + vcol
  // (one uniform branch around all the loads, so that they are issued
  // together rather than each behind a branch and a wait of its own)
  if (S0 && !phi) {
    const float* s0r = S0 + (((int64_t)n * Hv + h) * D + v0 + vcol) * D + g4;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[kt][i] = s0r[16 * kt + i];
  } else {
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[kt][i] = phi && v0 - D + vcol == 16 * kt + g4 + i ? 1.f : 0.f;
  }

  const int4 sp = reinterpret_cast<const int4*>(spans)[n];
  const int64_t c_begin = sp.x, c_end = sp.y;
  const int64_t seq_t0 = sp.z, seq_t1 = sp.w;

  // ---- per-lane offsets, the same for every chunk
  CopyLanes cl;
  cl.init(lane, wave, NW);
  // stores: byte offset of this lane's first row (g4) and column
  const uint32_t so = (uint32_t)(((int64_t)g4 * HvD + vcol) * sizeof(T));
  const uint32_t rowb = (uint32_t)(HvD * sizeof(T));
  // reads: element offsets of this lane's operand values for MFMA step p
  // (row c16 of a 16-row tile; tile index and buffer enter as constants)
  // (16-bit: the eight values are the 16-byte piece 4 p + g of the row, the
  // columns being stored in accumulator order)
  int rw[NSD], rk[NSC];
#pragma unroll
  for (int p = 0; p < NSD; ++p)
    rw[p] = KS == 4 ? TW::at(c16, 16 * (p >> 2) + g4 + (p & 3)) : TW::at(c16, 32 * p + 8 * g);
#pragma unroll
  for (int p = 0; p < NSC; ++p)
    rk[p] = KS == 4 ? TKt::at(c16, 16 * (p >> 2) + g4 + (p & 3)) : TKt::at(c16, 32 * p + 8 * g);
  // K^T, M and P rows all hold CHUNK elements, so rk addresses M and P too

  // ---- chunk c's operands into buffer B (value rows past a sequence end
  // re-read its last row)
  auto fetch = [&](SB& B, int64_t c) __attribute__((always_inline)) {
    // LDS destinations derived from a laundered wave index are formed here
    // (one scalar add each) instead of being hoisted into scalar registers.
    int wave = SB::KR ? wave_ - NW : wave_;   // (K-rows form: movers only)
    asm volatile("" : "+s"(wave));
    const int64_t t0 = seq_t0 + CHUNK * (c - c_begin);
    const int64_t rem = seq_t1 - t0;
    const int Lc = rem < CHUNK ? (int)rem : CHUNK;
    const int64_t ch = (int64_t)c * Hv + h, ck_ = (int64_t)c * Hk + kh;
    copy_tile<TW, NW>(B.W, Ww + (SB::KR ? ck_ : ch) * CHUNK * D, cl, wave);
    if constexpr (MODE == 0) copy_tile<TW, NW>(B.X, Xw + ck_ * CHUNK * D, cl, wave);
    if constexpr (!SB::KR) copy_tile<TKt, NW>(B.Kt, Ktw + ck_ * D * CHUNK, cl, wave);
    copy_tile<TM, NW>(B.M, Mw + ch * CHUNK * CHUNK, cl, wave);
    if constexpr (MODE == 0) copy_tile<TM, NW>(B.P, Pw + ch * CHUNK * CHUNK, cl, wave);
    {
      const uint32_t ldb = (uint32_t)(ldv * sizeof(T));
      // (identity-row blocks copy the value rows of block vb - D / BV, which
      // stay unused: their compute takes zero values); the block's value rows
      // are read by this workgroup alone, so with the non-temporal hint
      const auto rs = buffer_of(v + t0 * ldv + (int64_t)h * D + (phi ? v0 - D : v0), (uint32_t)Lc * ldb);
#pragma unroll
      for (int j = 0; j < TV::PIECES / THREADS; ++j) {
        const int s = (j * NW + wave) * 64 + lane, r = s / TV::RP;
        const uint32_t off = (uint32_t)(r < Lc ? r : Lc - 1) * ldb +
                             (uint32_t)((s % TV::RP) ^ TV::swz(r)) * 16u;
        copy_to_lds<CACHE_NT>(rs, B.V + (j * NW + wave) * 64 * TV::EPP, off, 0);
      }
    }
    // Gam and dec, 64 floats each: one copy per wave with two waves, so that
    // every wave issues the same number of copies
    if (lane < 16) {
      if (wave == 0) copy_to_lds(buffer_of(Gw + ch * CHUNK, CHUNK * 4), B.G, 16u * lane, 0);
      if (wave == NW - 1) copy_to_lds(buffer_of(Dw + ch * CHUNK, CHUNK * 4), B.Dc, 16u * lane, 0);
    }
  };
  // copies a wave issues per fetch, and stores per chunk (MODE 1)
  constexpr int NCOPY = TW::PIECES / THREADS * (MODE == 0 ? 2 : 1) + (SB::KR ? 0 : TKt::PIECES / THREADS) +
                        TM::PIECES / THREADS * (MODE == 0 ? 2 : 1) + TV::PIECES / THREADS +
                        (NW == 1 ? 2 : 1);
  constexpr int NSTORE = NKT * 2;
  static_assert(NW <= 2, "gate-factor copies are split over at most two waves");

  // chunk-start state, [d_k][d_v] per (chunk, head) (MODE 1)
  // (two adjacent value columns per store)
  PairStore ps;
  ps.init(lane);
  // the state and the token rows of this block of value columns (SBV = BV
  // of them) are stored as SBV-column rows
  static_assert(BV == SBV, "a workgroup owns one block of stored value columns");
  const uint32_t rowh = (uint32_t)(SBV * sizeof(T));
  const uint32_t hb = (uint32_t)(16 * wave * sizeof(T)) + ps.lane_off<T>(lane, rowh);
  auto store_state = [&](int64_t c) __attribute__((always_inline)) {
    const auto rs = buffer_of(hst + ((int64_t)c * Hv + h) * D * D + (int64_t)v0 * D,
                              DRY ? 0u : D * SBV * sizeof(T));
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) ps.store<T>(rs, hb + (uint32_t)(16 * kt) * rowh, rowh, S[kt]);
  };
  // (K-rows form) The compute waves put the chunk-start state, R and Delta
  // (Delta in the compute type, which the outputs and the gradients read)
  // into LDS rows of their own (paired words, ds_write2); a step later the
  // mover wave of the same index stores them in 16-byte pieces, so no store
  // sits on the recurrence.  Two sets of rows, by chunk parity.
  constexpr int SRR = D + 2 * CHUNK;   // staged rows per compute wave
  typedef StageCols<SRR> SR;
  constexpr int SROW_R = D, SROW_D16 = D + CHUNK;
  __shared__ __align__(16) char stg[SB::KR && !DRY ? 2 * NW * SR::BYTES : 16];
  auto stage_of = [&](int64_t c, int w) __attribute__((always_inline)) -> char* {
    return stg + (int)((((c - c_begin) & 1) * NW + w) * SR::BYTES);
  };
  // a tile of 16 rows (rows 16 tt + 4 g + i, column vcol) as element type E
  auto put_rows = [&](auto tag, char* st, int row0, const floatx4 (&x)[4]) __attribute__((always_inline)) {
    typedef decltype(tag) E;
    static_assert(sizeof(E) == sizeof(T), "same row layout");
    if constexpr (!DRY) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) SR::template put<E>(st, row0 + 16 * tt, lane, x[tt]);
    }
  };
  // (movers) chunk cp's staged rows to the state, R and Delta (compute
  // type) buffers, half of them per mover; token rows past the sequence
  // end fall outside the buffers and are dropped.  With valid false every
  // store is still issued but dropped (an empty range), so each step issues
  // the same count.  The dry pass stages and stores nothing (NFL = 0).
  constexpr int NFL = DRY ? 0 : SR::stores(D) + 2 * SR::stores(CHUNK);
  auto flush_chunk = [&](int64_t cp, bool valid) __attribute__((always_inline)) {
    if constexpr (DRY) return;
    const char* st = stage_of(cp, 0);   // both compute waves' rows: mover `wave` takes half of them
    const int64_t ca = valid ? cp : c_begin;
    const int64_t t0p = seq_t0 + CHUNK * (ca - c_begin);
    const int64_t rem = seq_t1 - t0p;
    const int Lp = valid ? (rem < CHUNK ? (int)rem : CHUNK) : 0;
    const int64_t blk = (ca * Hv + h) * CHUNK * D + (int64_t)v0 * CHUNK;
    SR::template flush_pair_async<CACHE_NT | CACHE_SC1>(st, 0, D,
        buffer_of(hst + (ca * Hv + h) * D * D + (int64_t)v0 * D, valid ? D * SBV * sizeof(T) : 0u), rowh, lane,
        wave);
    SR::template flush_pair_async<CACHE_NT | CACHE_SC1>(st, SROW_R, CHUNK, buffer_of(Rw + blk, (uint32_t)Lp * rowh), rowh, lane,
                                            wave);
    SR::template flush_pair_async<CACHE_NT | CACHE_SC1>(st, SROW_D16, CHUNK, buffer_of(Dl16w + blk, (uint32_t)Lp * rowh), rowh,
                                            lane, wave);
  };

  // A operand of MFMA step p from row 16 * tile + c16 of a tile (offset o).
  auto arow = [&](const CT* base, int o, int tile_elems) __attribute__((always_inline)) -> frag {
    if constexpr (KS == 4) return base[tile_elems + o];
    else return *reinterpret_cast<const frag*>(base + tile_elems + o);
  };

  // A operand of step p from rows 16 kt + c16 of K^T (columns t in
  // accumulator order): the K^T tile, or in the K-rows form two transposing
  // reads of the K rows (columns k in accumulator order): lanes 4a .. 4a + 3
  // of a group take stored columns 32 (kt / 2) + 8 a + 4 (kt % 2) .. + 3, and
  // lane j of group g points at token row 32 p + 4 g + j / 4 (then 16 rows
  // further)
  auto kt_frag = [&](const SB& B, int kt, int p) __attribute__((always_inline)) -> frag {
    if constexpr (SB::KR) {
      const int col = 32 * (kt >> 1) + 8 * (c16 & 3) + 4 * (kt & 1), r = 32 * p + g4 + (c16 >> 2);
      const u32x2 lo = lds_read_tr4(B.W + TW::at(r, col)), hi = lds_read_tr4(B.W + TW::at(r + 16, col));
      return __builtin_bit_cast(frag, u32x4{lo[0], lo[1], hi[0], hi[1]});
    } else {
      return arow(B.Kt, rk[p], 16 * kt * CHUNK);
    }
  };

  // ---- one chunk from buffer B
  auto compute = [&](const SB& B, int64_t c, char* stc) __attribute__((always_inline)) {
    const int64_t t0 = seq_t0 + CHUNK * (c - c_begin);
    const int64_t rem = seq_t1 - t0;
    const int L = rem < CHUNK ? (int)rem : CHUNK;

    floatx4 Dl[4];
    if constexpr (SB::KR) {
      // R = V - diag(Gam) K S^T (rows t = 16 tt + g4 + i, column vcol), then
      // Delta = M R with R straight from the accumulators
      frag sb[NSD];
#pragma unroll
      for (int p = 0; p < NSD; ++p) sb[p] = AO::from_acc(S, p);
      floatx4 kx[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        kx[tt] = zero4();
#pragma unroll
        for (int p = 0; p < NSD; ++p) kx[tt] = MM::mma(arow(B.W, rw[p], 16 * tt * D), sb[p], kx[tt]);
      }
      // the chunk-start state goes to its staging rows while the products
      // run (the puts are ordered after the K-row reads above)
      if constexpr (!DRY) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) SR::template put<T>(stc, 16 * kt, lane, S[kt]);
      }
      floatx4 R[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const float4 gm = *reinterpret_cast<const float4*>(&B.G[16 * tt + g4]);
        const float gv[4] = {gm.x, gm.y, gm.z, gm.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          R[tt][i] = (phi ? 0.f : to_f(B.V[TV::at(16 * tt + g4 + i, vcol)])) - gv[i] * kx[tt][i];
      }
      frag rf[NSC];
#pragma unroll
      for (int p = 0; p < NSC; ++p) rf[p] = AO::from_acc(R, p);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        Dl[tt] = zero4();
#pragma unroll
        for (int p = 0; p < NSC; ++p)
          Dl[tt] = MM::mma(*reinterpret_cast<const frag*>(B.M + 16 * tt * CHUNK + rk[p]), rf[p], Dl[tt]);
      }
      put_rows((T)0, stc, SROW_R, R);
    } else {
    // -S^T as B operands, straight from the accumulators
    frag sbn[NSD];
#pragma unroll
    for (int p = 0; p < NSD; ++p) sbn[p] = -AO::from_acc(S, p);

    // Delta = W (-S^T) + M V; V is gathered in accumulator order, as M's
    // columns are stored
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      Dl[tt] = zero4();
#pragma unroll
      for (int p = 0; p < NSD; ++p) Dl[tt] = MM::mma(arow(B.W, rw[p], 16 * tt * D), sbn[p], Dl[tt]);
    }
    {
      frag bv[NSC];
#pragma unroll
      for (int p = 0; p < NSC; ++p) {
        if constexpr (KS == 4) {
          bv[p] = phi ? 0.f : to_f(B.V[TV::at(16 * (p >> 2) + g4 + (p & 3), vcol)]);
        } else {
#pragma unroll
          for (int j = 0; j < NV; ++j)
            bv[p][j] = phi ? (CT)0.f : (CT)to_f(B.V[TV::at(32 * p + 16 * (j >> 2) + g4 + (j & 3), vcol)]);
        }
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int p = 0; p < NSC; ++p) {
          frag ma;
          if constexpr (KS == 4) ma = B.M[16 * tt * CHUNK + rk[p]];
          else ma = *reinterpret_cast<const frag*>(B.M + 16 * tt * CHUNK + rk[p]);
          Dl[tt] = MM::mma(ma, bv[p], Dl[tt]);
        }
    }
    }

    // Q (-S^T) (MODE 0)
    floatx4 xs[4];
    if constexpr (MODE == 0) {
      frag sbn[NSD];
#pragma unroll
      for (int p = 0; p < NSD; ++p) sbn[p] = -AO::from_acc(S, p);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        xs[tt] = zero4();
#pragma unroll
        for (int p = 0; p < NSD; ++p) xs[tt] = MM::mma(arow(B.X, rw[p], 16 * tt * D), sbn[p], xs[tt]);
      }
    }

    // state update: S^T <- Gam_L S^T + K^T diag(dec) Delta
    {
      floatx4 ds[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const float4 dc = *reinterpret_cast<const float4*>(&B.Dc[16 * tt + g4]);
        ds[tt][0] = dc.x * Dl[tt][0];
        ds[tt][1] = dc.y * Dl[tt][1];
        ds[tt][2] = dc.z * Dl[tt][2];
        ds[tt][3] = dc.w * Dl[tt][3];
      }
      frag dsf[NSC];
#pragma unroll
      for (int p = 0; p < NSC; ++p) dsf[p] = AO::from_acc(ds, p);
      const float GL = B.G[CHUNK - 1];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[kt][i] *= GL;
#pragma unroll
        for (int p = 0; p < NSC; ++p) S[kt] = MM::mma(kt_frag(B, kt, p), dsf[p], S[kt]);
      }
    }
    if constexpr (SB::KR) {
      put_rows((CT)0, stc, SROW_D16, Dl);
    }

    if constexpr (MODE == 0) {
      // O = diag(Gam) scale Q S^T + P Delta
      frag duf[NSC];
#pragma unroll
      for (int p = 0; p < NSC; ++p) duf[p] = AO::from_acc(Dl, p);
      // rows past the sequence end fall outside the buffer: dropped
      const auto rs = buffer_of(o + t0 * HvD + (int64_t)h * D + v0, DRY ? 0u : (uint32_t)L * rowb);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        floatx4 ov = zero4();
#pragma unroll
        for (int p = 0; p < NSC; ++p) ov = MM::mma(arow(B.P, rk[p], 16 * tt * CHUNK), duf[p], ov);
        const float4 gm = *reinterpret_cast<const float4*>(&B.G[16 * tt + g4]);
        const float gv[4] = {gm.x, gm.y, gm.z, gm.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          store_elem<T>(rs, so + (uint32_t)(16 * tt + i) * rowb, ov[i] - scale * gv[i] * xs[tt][i]);
      }
    }
  };

  if constexpr (MODE == 0) {
    // two buffers: the next chunk's copies are in flight while a chunk
    // computes
    if (c_begin < c_end) fetch(bufA, c_begin);
    __syncthreads();
    for (int64_t c = c_begin; c < c_end; c += 2) {
      fetch(bufB, c + 1 < c_end ? c + 1 : c);   // a repeat of chunk c at the end
      compute(bufA, c, nullptr);
      __syncthreads();   // waits for this wave's copies; then every wave's are visible
      if (c + 1 < c_end) {
        fetch(bufA, c + 2 < c_end ? c + 2 : c + 1);
        compute(bufB, c + 1, nullptr);
        __syncthreads();
      }
    }
  } else if constexpr (SB::KR) {
    // three buffers, the copies two chunks ahead, issued by the movers: a
    // step ends once the movers' copies for the next chunk (issued a step
    // earlier) and their stores of the chunk before are done, this step's
    // still in flight; the compute waves only compute and put the chunk's
    // state, R and Delta into their staging rows.  Past the end the last
    // chunk is copied again.
    __shared__ SB bufC;
    auto last = [&](int64_t x) { return x < c_end ? x : c_end - 1; };
    if (mover) {
      // A step issues the copies for chunk c + 2, then the stores of chunk
      // c - 1 (staged during the previous step), then waits for chunk c + 1's
      // copies: those were followed by the previous step's stores and this
      // step's copies and stores, which stay in flight, so a store has two
      // steps to complete.  The prologue issues (dropped) stores too, so that
      // the count is the same from the first step on.
      static_assert(NCOPY + 2 * NFL < 64, "vmcnt holds 6 bits");
      if (c_begin < c_end) {
        fetch(bufA, c_begin);
        fetch(bufB, last(c_begin + 1));
      }
      flush_chunk(c_begin - 2, false);
      wait_vm_barrier<NCOPY + NFL>();
      for (int64_t c = c_begin; c < c_end; c += 3) {
        fetch(bufC, last(c + 2));
        flush_chunk(c - 1, c > c_begin);
        wait_vm_barrier<NCOPY + 2 * NFL>();
        if (c + 1 >= c_end) break;
        fetch(bufA, last(c + 3));
        flush_chunk(c, true);
        wait_vm_barrier<NCOPY + 2 * NFL>();
        if (c + 2 >= c_end) break;
        fetch(bufB, last(c + 4));
        flush_chunk(c + 1, true);
        wait_vm_barrier<NCOPY + 2 * NFL>();
      }
      // the last chunk's rows, staged before the last barrier
      if (c_begin < c_end) flush_chunk(c_end - 1, true);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      return;
    }
    lds_barrier();
    for (int64_t c = c_begin; c < c_end; c += 3) {
      {
        char* st = stage_of(c, wave);
        compute(bufA, c, st);
      }
      lds_barrier();
      if (c + 1 >= c_end) break;
      {
        char* st = stage_of(c + 1, wave);
        compute(bufB, c + 1, st);
      }
      lds_barrier();
      if (c + 2 >= c_end) break;
      {
        char* st = stage_of(c + 2, wave);
        compute(bufC, c + 2, st);
      }
      lds_barrier();
    }
  } else {
    // three buffers: the copies run two chunks ahead.  A step issues the
    // chunk's state stores, then the copies for chunk c + 2, then computes
    // chunk c; it ends once this wave's copies for chunk c + 1 (issued a step
    // earlier, followed by exactly NSTORE stores and NCOPY copies) are done,
    // and a barrier makes every wave's visible.  Past the end the last chunk
    // is copied again, so every step issues the same operations.
    __shared__ SB bufC;
    auto last = [&](int64_t x) { return x < c_end ? x : c_end - 1; };
    auto step = [&](const SB& cur, SB& ahead, int64_t c) __attribute__((always_inline)) {
      store_state(c);
      fetch(ahead, last(c + 2));
      compute(cur, c, nullptr);
      wait_vm_barrier<NSTORE + NCOPY>();
    };
    if (c_begin < c_end) {
      fetch(bufA, c_begin);
      fetch(bufB, last(c_begin + 1));
    }
    wait_vm_barrier<NCOPY>();
    for (int64_t c = c_begin; c < c_end; c += 3) {
      step(bufA, bufC, c);
      if (c + 1 >= c_end) break;
      step(bufB, bufA, c + 1);
      if (c + 2 >= c_end) break;
      step(bufC, bufB, c + 2);
    }
  }

  if (S_final) {   // [span][head][nblk * BV rows][D]
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S_final[(((int64_t)n * Hv + h) * (nblk * BV) + v0 + vcol) * D + 16 * kt + g4 + i] = S[kt][i];
  }
}

// ---------------------------------------------------------------------------
constexpr int STATE_NW = 2;   // waves (16 value rows of the state each) per workgroup

// One launch over all spans: nblk row blocks per (span, head) (D / BV, or
// 2 D / BV for the first pass of the segmented scan, which carries the
// identity rows), stores dropped when dry.  With 16-bit MODE 1 (the K-rows
// form) the pass also stores R and Delta, which it forms on the way.
template <typename T, int D, int MODE>
static hipError_t chunk_state_launch(const gdn_shape& s, const void* v, int64_t ldv, float scale,
                                     const float* S0, float* S_final, void* o,
                                     const ChunkLayout& Ly, char* ws, int nblk, int dry,
                                     hipStream_t st) {
  constexpr bool KR = StateBuf<T, D, STATE_NW, MODE>::KR;
  constexpr int NW = STATE_NW;
  typedef typename Compute<T>::type CT;
  auto kern = dry ? chunk_state_kernel<T, D, NW, MODE, true> : chunk_state_kernel<T, D, NW, MODE, false>;
  const int n_items = nblk * s.hv * (int)Ly.nspan_max;
  hipLaunchKernelGGL(kern, dim3(n_items), dim3((KR ? 128 : 64) * NW), 0, st,
                     (const T*)v, ldv, (const int32_t*)(ws + Ly.spans),
                     (const int32_t*)(ws + Ly.segb) + s.n_seq, nblk, s.hv, s.hv / s.hk, scale,
                     (const CT*)(ws + Ly.mw), (const CT*)(ws + Ly.pw),
                     (const CT*)(ws + (KR ? Ly.k16w : Ly.ww)),
                     (const CT*)(ws + Ly.ktw), (const CT*)(ws + Ly.q16w),
                     (const float*)(ws + Ly.gw), (const float*)(ws + Ly.dw), S0, S_final, (T*)o,
                     (T*)(ws + Ly.h), KR ? (T*)(ws + Ly.rw) : nullptr,
                     KR ? (CT*)(ws + Ly.dl16w) : nullptr, n_items);
  return hipGetLastError();
}

// The state pass over every sequence: one chain per (sequence, head, row
// block), or the segmented scan (first pass from zero with the identity rows,
// the combine, then the pass per segment from its start state).
template <typename T, int D, int MODE>
static hipError_t chunk_state(const gdn_shape& s, const void* v, int64_t ldv, float scale,
                              const float* S0, float* S_final, const int32_t* cu, void* o,
                              const ChunkLayout& Ly, char* ws, hipStream_t st) {
  constexpr int NB = D / (16 * STATE_NW);
  if (Ly.seg == 0)
    return chunk_state_launch<T, D, MODE>(s, v, ldv, scale, S0, S_final, o, Ly, ws, NB, 0, st);
  hipError_t e = chunk_state_launch<T, D, MODE>(s, v, ldv, scale, nullptr, (float*)(ws + Ly.sumf),
                                                o, Ly, ws, 2 * NB, 1, st);
  if (e != hipSuccess) return e;
  e = launch_span_combine(s, Ly, ws, false, S0, S_final, st);
  if (e != hipSuccess) return e;
  return chunk_state_launch<T, D, MODE>(s, v, ldv, scale, (const float*)(ws + Ly.sst), nullptr, o,
                                        Ly, ws, NB, 0, st);
}

hipError_t launch_chunk_fwd_states(const gdn_shape& s, const void* q, const void* k, const void* v,
                                   int64_t ldq, int64_t ldk, int64_t ldv, float scale,
                                   const float* S0, float* S_final, const int32_t* cu, void* o,
                                   void* ws, hipStream_t st) {
  const ChunkLayout Ly = chunk_layout(s, ChunkFlow::Fwd);
  return dispatch_chunk(s, [&](auto c) {
    using T = typename decltype(c)::type;
    return chunk_state<T, decltype(c)::d, 0>(s, v, ldv, scale, S0, S_final, cu, o, Ly, (char*)ws,
                                             st);
  });
}

hipError_t launch_chunk_fwd_states_save(const gdn_shape& s, const void* q, const void* k,
                                        const void* v, int64_t ldq, int64_t ldk, int64_t ldv,
                                        float scale, const float* S0, float* S_final,
                                        const int32_t* cu, void* o, void* ws, hipStream_t st) {
  // the sequential pass stores the chunk-start states (and, with 16-bit
  // types, R and Delta); O (and for fp32 R and Delta) then follow chunk by
  // chunk in parallel
  const ChunkLayout Ly = chunk_layout(s, ChunkFlow::Bwd);
  hipError_t e = dispatch_chunk(s, [&](auto c) {
    using T = typename decltype(c)::type;
    return chunk_state<T, decltype(c)::d, 1>(s, v, ldv, scale, S0, S_final, cu, nullptr, Ly,
                                             (char*)ws, st);
  });
  if (e != hipSuccess) return e;
  return launch_chunk_outputs(s, q, k, v, ldq, ldk, ldv, scale, cu, o, ws, st);
}

hipError_t launch_chunk_bwd_states(const gdn_shape& s, const void* q, const void* k, const void* v,
                                   int64_t ldq, int64_t ldk, int64_t ldv, float scale,
                                   const float* S0, const int32_t* cu, void* ws, hipStream_t st) {
  const ChunkLayout Ly = chunk_layout(s, ChunkFlow::Bwd);
  hipError_t e = dispatch_chunk(s, [&](auto c) {
    using T = typename decltype(c)::type;
    return chunk_state<T, decltype(c)::d, 1>(s, v, ldv, scale, S0, nullptr, cu, nullptr, Ly,
                                             (char*)ws, st);
  });
  if (e != hipSuccess) return e;
  return launch_chunk_outputs(s, q, k, v, ldq, ldk, ldv, scale, cu, nullptr, ws, st);
}

}  // namespace gdn
