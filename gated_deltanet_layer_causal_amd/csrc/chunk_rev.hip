// Chunked gated delta rule, backward: the reverse pass over the chunks of
// each sequence.  Per chunk, given dO and the gradient dS' of the state
// leaving it:
//   dDelta = P^T dO + diag(dec) K dS'^T
//   dR     = M^T dDelta = diag(beta) Tinv^T dDelta        (= dv)
//   dS     = Gam_L dS' + (scale Q)^T diag(Gam) dO - K^T diag(Gam) dR
// It stores dS' per chunk (for the chunk-parallel gradients), dDelta and dv,
// and dS0 at the sequence start.  The DRY instantiation (the first pass of
// the segmented scan, which only needs each segment's dS0) stages and stores
// nothing.
//
// Same structure as the state pass (chunk_state.hip): one workgroup per
// (sequence, value head, block of 16 * NW value rows); compute wave w keeps
// its d_k x 16 slice of dS'^T in MFMA accumulators and feeds it straight
// back as B operand; NW mover waves (on the SIMDs the compute waves leave
// free) stream the chunk operands (K rows, K^T, Q^T, P^T and Tinv from the
// backward preparation, columns in accumulator order (fp32: Tinv^T); the dO
// rows of the block; Gam, dec, beta) into one of two LDS buffers by direct
// copies while the compute waves work on the other.  Operands are in the storage type (bf16
// keeps the range of dS).
#include "chunk_stream.h"

namespace gdn {

template <typename T, int D, int NW> struct RevBuf {
  static constexpr int BV = 16 * NW;
  typedef Tile<T, CHUNK, D> TK;        // K rows
  typedef Tile<T, D, CHUNK> TKt;       // K^T, Q^T
  typedef Tile<T, CHUNK, CHUNK> TM;    // P^T, Tinv (fp32: Tinv^T)
  typedef Tile<T, CHUNK, BV, 3> TO;    // dO rows of this block
  // 16-bit types read K^T from the K rows by transposing reads; fp32 copies it
  static constexpr bool KT_TR = sizeof(T) == 2;
  T K[TK::PIECES * TK::EPP];
  T Kt[KT_TR ? 8 : TKt::PIECES * TKt::EPP];
  T Qt[TKt::PIECES * TKt::EPP];
  T Pt[TM::PIECES * TM::EPP];
  T Mt[TM::PIECES * TM::EPP];          // Tinv (16-bit) or Tinv^T (fp32)
  T dO[TO::PIECES * TO::EPP];
  float G[CHUNK], Dc[CHUNK], Bt[CHUNK];   // Gam_t, dec_t, beta_t
} __attribute__((aligned(16)));

template <typename T, int D, int NW, bool DRY>
__global__ void __launch_bounds__(128 * NW) chunk_rev_kernel(
    const int32_t* __restrict__ spans, const int32_t* __restrict__ n_spans, int Hv, int G,
    float scale,
    const T* __restrict__ Kb, const T* __restrict__ Ktb, const T* __restrict__ Qtb,
    const T* __restrict__ Ptb, const T* __restrict__ Tib, const float* __restrict__ Gw,
    const float* __restrict__ Dw, const float* __restrict__ Bw, const T* __restrict__ dout, const float* __restrict__ dS_final,
    float* __restrict__ dS0, T* __restrict__ dhst, T* __restrict__ ddw, T* __restrict__ dvo,
    int64_t lddv, int n_items) {
  typedef Mma<T> MM;
  typedef AccOrder<T> AO;
  typedef typename MM::frag frag;
  typedef RevBuf<T, D, NW> RB;
  typedef typename RB::TK TK;
  typedef typename RB::TKt TKt;
  typedef typename RB::TM TM;
  typedef typename RB::TO TO;
  constexpr int BV = RB::BV;
  constexpr int KS = MM::KS;
  constexpr int NSD = D / KS;       // MFMA steps over d_k
  constexpr int NSC = CHUNK / KS;   // MFMA steps over the chunk
  constexpr int NKT = D / 16;       // gradient tiles per wave
  static_assert(TK::PIECES % (64 * NW) == 0 && TKt::PIECES % (64 * NW) == 0 &&
                TM::PIECES % (64 * NW) == 0 && TO::PIECES % (64 * NW) == 0,
                "direct copies cover whole waves");
  __shared__ RB bufA, bufB;
  // per wave: staged output rows (dS' rows k, then dDelta and dv rows t).
  // 16-bit data: two sets by step parity; the compute waves put a chunk's
  // rows and a step later the mover wave of the same index stores them, so
  // no store (nor the read-back before it) sits on the recurrence.  fp32
  // (one set, no room for two) stores from the compute waves.
  typedef StageRows<T> SR;        // (fp32: one set of row-major staging, stored by the compute waves)
  constexpr bool MSTORE = sizeof(T) == 2;
  constexpr int SRR = D + 2 * CHUNK;   // staged rows per compute wave
  typedef StageCols<SRR> SC;       // (16-bit: two sets of column-major staging, stored by the movers)
  constexpr int SWB = MSTORE ? SC::BYTES : SRR * SR::SB;   // staging bytes per wave and set
  __shared__ __align__(16) char stg[DRY ? 16 : (MSTORE ? 2 : 1) * NW * SWB];

  const int tid = threadIdx.x, lane = tid & 63;
  // waves [0, NW) compute, waves [NW, 2 NW) move the operands
  const int wave_ = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool mover = wave_ >= NW;
  const int wave = mover ? wave_ - NW : wave_;
  const int item = xcd_item(blockIdx.x, n_items);
  const int vb = item % (D / BV), h = (item / (D / BV)) % Hv, n = item / ((D / BV) * Hv);
  if (n >= *n_spans) return;
  const int kh = h / G, Hk = Hv / G;
  const int v0 = vb * BV;
  const int g = lane >> 4, g4 = 4 * g, c16 = lane & 15;
  const int vcol = 16 * wave + c16;
  const int64_t HvD = (int64_t)Hv * D;

  floatx4 dS[NKT];   // dS'^T tiles: rows k = 16 kt + g4 + i, column v0 + vcol
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dS[kt][i] = dS_final ? dS_final[(((int64_t)n * Hv + h) * D + v0 + vcol) * D + 16 * kt + g4 + i] : 0.f;

  const int4 sp = reinterpret_cast<const int4*>(spans)[n];
  const int64_t c_begin = sp.x, c_end = sp.y;
  const int64_t seq_t0 = sp.z, seq_t1 = sp.w;

  CopyLanes cl;
  cl.init(lane, wave, NW);
  const uint32_t rowb = (uint32_t)(HvD * sizeof(T));
  const uint32_t rowv = (uint32_t)(lddv * sizeof(T));
  // dS' and dDelta of this block of value columns (SBV = BV of them) are
  // stored as SBV-column rows
  static_assert(BV == SBV, "a workgroup owns one block of stored value columns");
  const uint32_t rowh = (uint32_t)(SBV * sizeof(T));
  // outputs leave through the wave's LDS rows in 16-byte pieces
  PairStore ps;
  ps.init(lane);
  const uint32_t wcol = (uint32_t)(16 * wave * sizeof(T));
  // one accumulator tile into rows row0.. of a wave's staging
  auto put = [&](char* st, int row0, const floatx4& x) __attribute__((always_inline)) {
    if constexpr (MSTORE) SC::template put<T>(st, row0, lane, x);
    else SR::put(st, row0, ps, lane, x);
  };
  // a chunk's staging rows of wave w
  auto stage_of = [&](int64_t c, int w) __attribute__((always_inline)) -> char* {
    return stg + (int)((((MSTORE ? (c_end - 1 - c) & 1 : 0) * NW) + w) * SWB);
  };
  // LDS read offsets (as in the state pass)
  int rw[NSD], rk[NSC];
#pragma unroll
  for (int p = 0; p < NSD; ++p)
    rw[p] = KS == 4 ? TK::at(c16, 16 * (p >> 2) + g4 + (p & 3)) : TK::at(c16, 32 * p + 8 * g);
#pragma unroll
  for (int p = 0; p < NSC; ++p)
    rk[p] = KS == 4 ? TKt::at(c16, 16 * (p >> 2) + g4 + (p & 3)) : TKt::at(c16, 32 * p + 8 * g);

  auto fetch = [&](RB& B, int64_t c) __attribute__((always_inline)) {
    int wave = wave_ - NW;   // (movers only)
    asm volatile("" : "+s"(wave));
    const int64_t t0 = seq_t0 + CHUNK * (c - c_begin);
    const int64_t rem = seq_t1 - t0;
    const int Lc = rem < CHUNK ? (int)rem : CHUNK;
    const int64_t ch = (int64_t)c * Hv + h, ck = (int64_t)c * Hk + kh;
    copy_tile<TK, NW>(B.K, Kb + ck * CHUNK * D, cl, wave);
    if constexpr (!RB::KT_TR) copy_tile<TKt, NW>(B.Kt, Ktb + ck * D * CHUNK, cl, wave);
    copy_tile<TKt, NW>(B.Qt, Qtb + ck * D * CHUNK, cl, wave);
    copy_tile<TM, NW>(B.Pt, Ptb + ch * CHUNK * CHUNK, cl, wave);
    copy_tile<TM, NW>(B.Mt, Tib + ch * 2 * CHUNK * CHUNK + (RB::KT_TR ? 0 : CHUNK * CHUNK), cl, wave);
    {
      // dO rows past the sequence end re-read its last row (their products
      // meet zero rows and columns of P^T, Q^T)
      const auto rs = buffer_of(dout + t0 * HvD + (int64_t)h * D + v0, (uint32_t)Lc * rowb);
#pragma unroll
      for (int j = 0; j < TO::PIECES / (64 * NW); ++j) {
        const int s = (j * NW + wave) * 64 + lane, r = s / TO::RP;
        const uint32_t off = (uint32_t)(r < Lc ? r : Lc - 1) * rowb +
                             (uint32_t)((s % TO::RP) ^ TO::swz(r)) * 16u;
        copy_to_lds(rs, B.dO + (j * NW + wave) * 64 * TO::EPP, off, 0);
      }
    }
    if (wave == 0 && lane < 16) {
      copy_to_lds(buffer_of(Gw + ch * CHUNK, CHUNK * 4), B.G, 16u * lane, 0);
      copy_to_lds(buffer_of(Dw + ch * CHUNK, CHUNK * 4), B.Dc, 16u * lane, 0);
    }
    if (wave == NW - 1 && lane < 16) copy_to_lds(buffer_of(Bw + ch * CHUNK, CHUNK * 4), B.Bt, 16u * lane, 0);
  };

  // (16-bit data) The movers also bring the lines of the chunk after the
  // one they copy into L2, a step ahead, so that its copies find them
  // there: one 4-byte direct copy per 128-byte line into a sink.  The four
  // workgroups of a head share the tiles of the chunk (they run on one XCD),
  // so each touches every fourth line of them: mover 0 of K and Q^T, mover
  // 1 of P^T and Tinv; and each mover every other row of its block's dO.
  // Lanes past a tile read out of range, which touches no memory.
  __shared__ float sink[64];
  constexpr int NTOUCH = MSTORE ? 3 : 0;   // touches a mover issues per step
  auto touch_tile = [&](const void* base, int bytes) __attribute__((always_inline)) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(buffer_of(base, (uint32_t)bytes),
                                             (__attribute__((address_space(3))) void*)sink, 4,
                                             (uint32_t)(4 * lane + vb) * 128u, 0, 0, 0);
  };
  auto touch = [&](int64_t c) __attribute__((always_inline)) {
    if constexpr (NTOUCH == 0) return;
    int wave = wave_ - NW;   // (movers only)
    asm volatile("" : "+s"(wave));
    const int64_t t0 = seq_t0 + CHUNK * (c - c_begin);
    const int64_t rem = seq_t1 - t0;
    const int Lc = rem < CHUNK ? (int)rem : CHUNK;
    const int64_t ch = (int64_t)c * Hv + h, ck = (int64_t)c * Hk + kh;
    constexpr int TKB = CHUNK * D * (int)sizeof(T), TMB = CHUNK * CHUNK * (int)sizeof(T);
    static_assert(TKB <= 4 * 64 * 128 && NW == 2, "one touch per tile and mover");
    if (wave == 0) {
      touch_tile(Kb + ck * CHUNK * D, TKB);
      touch_tile(Qtb + ck * D * CHUNK, TKB);
    } else {
      touch_tile(Ptb + ch * CHUNK * CHUNK, TMB);
      touch_tile(Tib + ch * 2 * CHUNK * CHUNK, TMB);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        buffer_of(dout + t0 * HvD + (int64_t)h * D + v0, (uint32_t)Lc * rowb),
        (__attribute__((address_space(3))) void*)sink, 4, (uint32_t)(2 * lane + wave) * rowb, 0, 0, 0);
  };
  // (movers, 16-bit data) chunk cp's rows staged by the compute waves to
  // dS', dDelta and dv, half of them per mover; token rows past the
  // sequence end fall outside the buffers and are dropped; with valid false
  // every store is issued into an empty range.  The reads are asm that waits for its own results (a plain
  // LDS read would wait for every direct copy in flight).
  constexpr int NFL = DRY || !MSTORE ? 0 : SC::stores(D) + 2 * SC::stores(CHUNK);
  static_assert(NTOUCH + NFL < 64, "vmcnt holds 6 bits");
  auto flush_chunk = [&](int64_t cp, bool valid) __attribute__((always_inline)) {
    if constexpr (NFL == 0) return;
    const char* st = stage_of(cp, 0);   // both compute waves' rows: mover `wave` takes half of them
    const int64_t ca = valid ? cp : c_begin;
    const int64_t t0p = seq_t0 + CHUNK * (ca - c_begin);
    const int64_t rem = seq_t1 - t0p;
    const int Lp = valid ? (rem < CHUNK ? (int)rem : CHUNK) : 0;
    SC::template flush_pair_async<CACHE_NT>(st, 0, D,
        buffer_of(dhst + (ca * Hv + h) * D * D + (int64_t)v0 * D, valid ? D * SBV * sizeof(T) : 0u), rowh, lane,
        wave);
    SC::template flush_pair_async<CACHE_NT>(st, D, CHUNK,
        buffer_of(ddw + (ca * Hv + h) * CHUNK * D + (int64_t)v0 * CHUNK, (uint32_t)Lp * rowh), rowh, lane, wave);
    // dv rows are the user's layout: this workgroup writes half of each line,
    // which measured faster as plain stores than non-temporal ones
    SC::template flush_pair_async<0>(st, D + CHUNK, CHUNK,
        buffer_of(dvo + t0p * lddv + (int64_t)h * D + v0, (uint32_t)Lp * rowv), rowv, lane, wave);
  };

  auto arow = [&](const T* base, int o, int tile_elems) __attribute__((always_inline)) -> frag {
    if constexpr (KS == 4) return base[tile_elems + o];
    else return *reinterpret_cast<const frag*>(base + tile_elems + o);
  };
  // A operand of step p from rows 16 kt + c16 of K^T (columns t in
  // accumulator order).  16-bit: two transposing reads of the K rows, whose
  // columns k are in accumulator order too: lanes 4a .. 4a + 3 of a group
  // take stored columns 32 (kt / 2) + 8 a + 4 (kt % 2) .. + 3, and lane j of
  // group g points at token row 32 p + 4 g + j / 4 (then 16 rows further).
  auto kt_frag = [&](const RB& B, int kt, int p) __attribute__((always_inline)) -> frag {
    if constexpr (RB::KT_TR) {
      const int col = 32 * (kt >> 1) + 8 * (c16 & 3) + 4 * (kt & 1), r = 32 * p + g4 + (c16 >> 2);
      const u32x2 lo = lds_read_tr4(B.K + TK::at(r, col)), hi = lds_read_tr4(B.K + TK::at(r + 16, col));
      return __builtin_bit_cast(frag, u32x4{lo[0], lo[1], hi[0], hi[1]});
    } else {
      return arow(B.Kt, rk[p], 16 * kt * CHUNK);
    }
  };

  // A operand of step p from row 16 tt + c16 of Tinv^T.  16-bit: the tile
  // holds Tinv (columns in accumulator order), read down column 16 tt + c16
  // by two transposing reads, as kt_frag reads the K rows: lanes 4a .. 4a + 3
  // of a group point at stored columns 32 (tt / 2) + 8 a + 4 (tt % 2) .. + 3,
  // lane j of group g at row 32 p + 4 g + j / 4 (then 16 rows further).
  // fp32: the tile holds Tinv^T (natural order), one index per step.
  auto tt_frag = [&](const RB& B, int tt, int p) __attribute__((always_inline)) -> frag {
    if constexpr (KS == 4) {
      return arow(B.Mt, rk[p], 16 * tt * CHUNK);
    } else {
      const int col = 32 * (tt >> 1) + 8 * (c16 & 3) + 4 * (tt & 1), r = 32 * p + g4 + (c16 >> 2);
      const u32x2 lo = lds_read_tr4(B.Mt + TM::at(r, col)), hi = lds_read_tr4(B.Mt + TM::at(r + 16, col));
      return __builtin_bit_cast(frag, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
  };

  auto compute = [&](const RB& B, int64_t c) __attribute__((always_inline)) {
    const int64_t t0 = seq_t0 + CHUNK * (c - c_begin);
    const int64_t rem = seq_t1 - t0;
    const int L = rem < CHUNK ? (int)rem : CHUNK;
    char* const myst = stage_of(c, wave);

    // dS'^T as B operands; dS' to the workspace ([d_k][d_v] per chunk, head)
    frag sb[NSD];
#pragma unroll
    for (int p = 0; p < NSD; ++p) sb[p] = AO::from_acc(dS, p);
    // diag(dec) K dS'^T first: it is on the recurrence; dS' is staged and
    // stored while these products run
    floatx4 kd[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      kd[tt] = zero4();
#pragma unroll
      for (int p = 0; p < NSD; ++p) kd[tt] = MM::mma(arow(B.K, rw[p], 16 * tt * D), sb[p], kd[tt]);
    }
    {
      const auto rs = buffer_of(dhst + ((int64_t)c * Hv + h) * D * D + (int64_t)v0 * D,
                                DRY ? 0u : D * SBV * sizeof(T));
      if constexpr (!DRY) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) put(myst, 16 * kt, dS[kt]);
        if constexpr (!MSTORE) SR::flush(myst, 0, D, rs, wcol, rowh, lane);
      }
    }

    // dO as B operands over the chunk index, plain and scaled by scale Gam_t
    frag ob[NSC], gob[NSC];
#pragma unroll
    for (int p = 0; p < NSC; ++p) {
      if constexpr (KS == 4) {
        const int t = 16 * (p >> 2) + g4 + (p & 3);
        const float x = to_f(B.dO[TO::at(t, vcol)]);
        ob[p] = x;
        gob[p] = scale * B.G[t] * x;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = 16 * (2 * p + j / 4) + g4 + (j & 3);
          const float x = to_f(B.dO[TO::at(t, vcol)]);
          ob[p][j] = from_f<T>(x);
          gob[p][j] = from_f<T>(scale * B.G[t] * x);
        }
      }
    }

    // dDelta = P^T dO + diag(dec) K dS'^T
    floatx4 dd[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      floatx4 pt = zero4();
#pragma unroll
      for (int p = 0; p < NSC; ++p) pt = MM::mma(arow(B.Pt, rk[p], 16 * tt * CHUNK), ob[p], pt);
      const float4 dc = *reinterpret_cast<const float4*>(&B.Dc[16 * tt + g4]);
      dd[tt][0] = pt[0] + dc.x * kd[tt][0];
      dd[tt][1] = pt[1] + dc.y * kd[tt][1];
      dd[tt][2] = pt[2] + dc.z * kd[tt][2];
      dd[tt][3] = pt[3] + dc.w * kd[tt][3];
    }
    {
      // rows past the sequence end fall outside the buffer: dropped
      const auto rs = buffer_of(ddw + ((int64_t)c * Hv + h) * CHUNK * D + (int64_t)v0 * CHUNK,
                                DRY ? 0u : (uint32_t)L * rowh);
      if constexpr (!DRY) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) put(myst, D + 16 * tt, dd[tt]);
        if constexpr (!MSTORE) SR::flush(myst, D, CHUNK, rs, wcol, rowh, lane);
      }
    }

    // dR = M^T dDelta (= dv); then -diag(Gam) dR as B operands
    floatx4 gr[4];
    {
      frag df[NSC];
#pragma unroll
      for (int p = 0; p < NSC; ++p) df[p] = AO::from_acc(dd, p);
      const auto rs = buffer_of(dvo + t0 * lddv + (int64_t)h * D + v0, DRY ? 0u : (uint32_t)L * rowv);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        floatx4 dr = zero4();
#pragma unroll
        for (int p = 0; p < NSC; ++p) dr = MM::mma(tt_frag(B, tt, p), df[p], dr);
        const float4 bt = *reinterpret_cast<const float4*>(&B.Bt[16 * tt + g4]);
        dr[0] *= bt.x;
        dr[1] *= bt.y;
        dr[2] *= bt.z;
        dr[3] *= bt.w;
        const float4 gm = *reinterpret_cast<const float4*>(&B.G[16 * tt + g4]);
        gr[tt][0] = -gm.x * dr[0];
        gr[tt][1] = -gm.y * dr[1];
        gr[tt][2] = -gm.z * dr[2];
        gr[tt][3] = -gm.w * dr[3];
        if constexpr (!DRY) put(myst, D + CHUNK + 16 * tt, dr);
      }
      if constexpr (!DRY && !MSTORE) SR::flush(myst, D + CHUNK, CHUNK, rs, wcol, rowv, lane);
    }

    // dS^T = Gam_L dS'^T + Q^T (scale diag(Gam) dO) - K^T (diag(Gam) dR)
    {
      frag gf[NSC];
#pragma unroll
      for (int p = 0; p < NSC; ++p) gf[p] = AO::from_acc(gr, p);
      const float GL = B.G[CHUNK - 1];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dS[kt][i] *= GL;
#pragma unroll
        for (int p = 0; p < NSC; ++p) {
          dS[kt] = MM::mma(arow(B.Qt, rk[p], 16 * kt * CHUNK), gob[p], dS[kt]);
          dS[kt] = MM::mma(kt_frag(B, kt, p), gf[p], dS[kt]);
        }
      }
    }
  };

  // The movers copy the next chunk's operands into the buffer that the
  // compute waves are not reading and end each step once their copies are
  // in; the compute waves only compute and store, so the copies' issue and
  // the waits for them stay off the recurrence.  One barrier per step: after
  // it the buffer just computed is free and the next one is filled.
  if (mover) {
    // each step ends once the copies are in, the touches (issued after
    // them) still in flight; at the end nothing is.  (16-bit data) a step also stores the rows that the compute waves
    // staged in the step before, after its copies; the stores stay in
    // flight until the next step's wait.  The first step's stores go to an
    // empty range, so that every step issues the same count.
    auto first = [&](int64_t x) { return x >= c_begin ? x : c_begin; };
    if (c_begin < c_end) {
      fetch(bufA, c_end - 1);
      touch(first(c_end - 2));
    }
    wait_vm_barrier<NTOUCH>();
    for (int64_t c = c_end - 1; c >= c_begin; c -= 2) {
      fetch(bufB, c - 1 >= c_begin ? c - 1 : c);   // a repeat of chunk c at the start
      touch(first(c - 2));
      flush_chunk(c + 1, c + 1 < c_end);
      wait_vm_barrier<NTOUCH + NFL>();
      if (c - 1 >= c_begin) {
        fetch(bufA, c - 2 >= c_begin ? c - 2 : c - 1);
        touch(first(c - 3));
        flush_chunk(c, true);
        wait_vm_barrier<NTOUCH + NFL>();
      }
    }
    // the first chunk's rows, staged before the last barrier
    if (c_begin < c_end) flush_chunk(c_begin, true);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    lds_barrier();
    for (int64_t c = c_end - 1; c >= c_begin; c -= 2) {
      compute(bufA, c);
      lds_barrier();
      if (c - 1 >= c_begin) {
        compute(bufB, c - 1);
        lds_barrier();
      }
    }
    if (dS0) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dS0[(((int64_t)n * Hv + h) * D + v0 + vcol) * D + 16 * kt + g4 + i] = dS[kt][i];
    }
  }
}

// ---------------------------------------------------------------------------
constexpr int REV_NW = 2;

// One launch over all spans (stores dropped when dry).
template <typename T, int D>
static hipError_t chunk_rev_launch(const gdn_shape& s, float scale, const void* dout,
                                   const float* dS_final, void* dv, int64_t lddv, float* dS0,
                                   const ChunkLayout& Ly, char* ws, int dry, hipStream_t st) {
  constexpr int NW = REV_NW, BV = 16 * NW;
  const int n_items = (D / BV) * s.hv * (int)Ly.nspan_max;
  auto kern = dry ? chunk_rev_kernel<T, D, NW, true> : chunk_rev_kernel<T, D, NW, false>;
  hipLaunchKernelGGL(kern, dim3(n_items), dim3(128 * NW), 0, st,
                     (const int32_t*)(ws + Ly.spans), (const int32_t*)(ws + Ly.segb) + s.n_seq,
                     s.hv, s.hv / s.hk, scale,
                     (const T*)(ws + Ly.kb), (const T*)(ws + Ly.ktb), (const T*)(ws + Ly.qtb),
                     (const T*)(ws + Ly.ptb), (const T*)(ws + Ly.tib), (const float*)(ws + Ly.gw),
                     (const float*)(ws + Ly.dw), (const float*)(ws + Ly.bw), (const T*)dout, dS_final, dS0, (T*)(ws + Ly.dh),
                     (T*)(ws + Ly.ddw), (T*)dv, lddv, n_items);
  return hipGetLastError();
}

// The reverse pass over every sequence, or the segmented scan: the pass over
// each segment from a zero gradient (its dB), the combine with the segments'
// transitions that the state pass left in the workspace, then the pass over
// each segment from the gradient at its end.
template <typename T, int D>
static hipError_t chunk_rev(const gdn_shape& s, float scale, const int32_t* cu, const void* dout,
                            const float* dS_final, void* dv, int64_t lddv, float* dS0,
                            const ChunkLayout& Ly, char* ws, hipStream_t st) {
  if (Ly.seg == 0)
    return chunk_rev_launch<T, D>(s, scale, dout, dS_final, dv, lddv, dS0, Ly, ws, 0, st);
  hipError_t e = chunk_rev_launch<T, D>(s, scale, dout, nullptr, dv, lddv, (float*)(ws + Ly.sumr),
                                        Ly, ws, 1, st);
  if (e != hipSuccess) return e;
  e = launch_span_combine(s, Ly, ws, true, dS_final, dS0, st);
  if (e != hipSuccess) return e;
  return chunk_rev_launch<T, D>(s, scale, dout, (const float*)(ws + Ly.dse), dv, lddv, nullptr, Ly,
                                ws, 0, st);
}

hipError_t launch_chunk_bwd_reverse(const gdn_shape& s, const void* q, const void* k, int64_t ldq,
                                    int64_t ldk, float scale, const int32_t* cu, const void* dout,
                                    const float* dS_final, void* dv, int64_t lddv, float* dS0,
                                    void* ws, hipStream_t st) {
  const ChunkLayout Ly = chunk_layout(s, ChunkFlow::Bwd);
  return dispatch_chunk(s, [&](auto c) {
    using T = typename decltype(c)::type;
    return chunk_rev<T, decltype(c)::d>(s, scale, cu, dout, dS_final, dv, lddv, dS0, Ly, (char*)ws,
                                        st);
  });
}

}  // namespace gdn
