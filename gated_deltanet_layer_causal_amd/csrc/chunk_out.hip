// Chunked gated delta rule: the chunk-parallel outputs of the saved
// chunk-start states.
//
// The state pass stores S, the state entering each chunk ([d_k][d_v] per
// (chunk, head)).  Given S every chunk is independent of the others:
//   R     = V - diag(Gam) K S^T
//   Delta = M R
//   O     = diag(Gam) scale Q S^T + P Delta
// so these products leave the chunk-to-chunk chain and run with one
// workgroup per (chunk, value head).
//
// Wave (vq, th) owns value columns [32 vq, 32 vq + 32) for tokens
// [32 th, 32 th + 32) and forms the transposed products
//   R^T = V^T - S K^T diag(Gam),  Delta^T = R^T M^T,
//   O^T = S (scale Q)^T diag(Gam) + Delta^T P^T,
// whose MFMA output tiles give each lane four consecutive value columns of
// one token: every output leaves in 8-byte pieces, and V comes in the same
// way.  S is the A operand of the first products: the two waves of a value
// quarter copy its d_k x 32 slice of S (stored [k][v]) into LDS rows and
// each reads its lanes' k values from it.  R^T and Delta^T, A operands of
// the products over all tokens, pass between the two token halves through a
// padded LDS tile per value quarter; their reads follow the accumulator
// order in which M and P store their columns (acc_col), so the B operands
// (rows of K, Q, M, P) are plain 16-byte reads.  With 16-bit operands both
// tiles are read by transposing reads (four rows of a column per lane),
// their rows 24 words apart so the four rows of a 16-lane group fall in
// different banks.  Every input a phase needs is
// requested before the phase that precedes it, so load latencies overlap.
// Rows of K, Q and V come straight from the conv output through
// range-checked buffer loads, which return zero past the chunk's end.
#include "chunk_stream.h"

namespace gdn {

template <typename T, int D> struct alignas(16) OutQuarter {
  typedef typename Compute<T>::type CT;
  static constexpr int LDH = sizeof(T) == 2 ? 48 : 33;    // S rows
  static constexpr int LDX = sizeof(CT) == 2 ? 48 : 34;   // R, Delta rows
  T hs[D][LDH];        // S^T slice: row k, value column
  CT xs[CHUNK][LDX];   // R, then Delta (compute type): row t, value column
};

// 32-bit words of the LDS slices: written as words, read as elements, so the
// word type must alias the element type.
typedef uint32_t __attribute__((may_alias)) word_alias;

template <typename T, int D, bool WITH_O>
__global__ void __launch_bounds__(4 * D) __attribute__((amdgpu_waves_per_eu(4))) chunk_out_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t ldq,
    int64_t ldk, int64_t ldv, const int32_t* __restrict__ cu, const int32_t* __restrict__ seq_off,
    int n_seq, int Hv, int G, float scale, const typename Compute<T>::type* __restrict__ Mw,
    const typename Compute<T>::type* __restrict__ Pw, const float* __restrict__ Gw,
    const T* __restrict__ hst, T* __restrict__ Rw, T* __restrict__ Dlw, T* __restrict__ o,
    int n_items) {
  typedef typename Compute<T>::type CT;
  typedef Mma<T> MS;     // products with S (storage-type operands)
  typedef Mma<CT> MC;    // products over tokens (compute type)
  typedef OutQuarter<T, D> OQ;
  typedef typename MS::frag sfrag;
  typedef typename MC::frag cfrag;
  constexpr int KS = MS::KS;
  static_assert(Mma<CT>::KS == KS, "both operand types step alike");
  constexpr int NQ = D / 32;                  // value quarters (of 32 columns)
  constexpr int NSD = D / KS, NSC = CHUNK / KS;
  constexpr int EPP = 16 / (int)sizeof(T), PPR = 32 / EPP;   // 16-byte pieces per 32-column row
  constexpr int NH = D * PPR / 128;           // S pieces per lane (two waves per slice)
  __shared__ OQ qs[NQ];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int vq = wave % NQ, th = wave / NQ;
  const int item = xcd_item(blockIdx.x, n_items);
  const int64_t c = item / Hv;
  const int h = item % Hv, kh = h / G;
  if (c >= seq_off[n_seq]) return;
  int64_t t0;
  int L;
  chunk_span(seq_off, cu, n_seq, c, t0, L);
  const int g = lane >> 4, g4 = 4 * g, c16 = lane & 15;
  const int v0 = 32 * vq;
  const int64_t ch = c * Hv + h, HvD = (int64_t)Hv * D;
  OQ& Q4 = qs[vq];
  const uint32_t rowb = (uint32_t)(HvD * sizeof(T));
  const float* gam = Gw + ch * CHUNK;
  const CT* Mc = Mw + ch * CHUNK * CHUNK;
  const CT* Pc = Pw + ch * CHUNK * CHUNK;

  // token tile j of this wave (j = 0, 1)
  auto tok = [&](int j) { return 16 * (2 * th + j); };
  // B operand of step p from token row r of X (K or Q rows): rows past the
  // chunk end read zero
  auto x_frag = [&](__amdgpu_buffer_rsrc_t rs, uint32_t ldb, int r, int p) __attribute__((always_inline)) {
    return buffer_frag<T>(rs, (uint32_t)r * ldb + (uint32_t)(p * KS + (KS == 4 ? g : 8 * g)) * sizeof(T));
  };
  // B operand of accumulator-order step p from token row r of a 64 x 64
  // operand stored with its columns in accumulator order (M, P)
  auto acc_row = [&](const CT* base, int r, int p) __attribute__((always_inline)) {
    const CT* rp = base + r * CHUNK;
    if constexpr (KS == 4) return rp[16 * (p >> 2) + g4 + (p & 3)];
    else return *reinterpret_cast<const cfrag*>(rp + 32 * p + 8 * g);
  };

  // ---- inputs of R and Delta, all requested up front
  uint4 hraw[NH];
  {
    const T* Sg = hst + ch * D * D + (int64_t)v0 * D;   // the quarter's block of the state
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const int i = lane + 64 * (2 * j + th), r = i / PPR, pc = i % PPR;
      hraw[j] = *reinterpret_cast<const uint4*>(Sg + (int64_t)r * SBV + pc * EPP);
    }
  }
  const uint32_t ldkb = (uint32_t)(ldk * sizeof(T)), ldqb = (uint32_t)(ldq * sizeof(T));
  const auto rk = buffer_of(k + t0 * ldk + (int64_t)kh * D, (uint32_t)L * ldkb);
  const auto rq = buffer_of(q + t0 * ldq + (int64_t)kh * D, (uint32_t)L * ldqb);
  sfrag kb[2][NSD];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int p = 0; p < NSD; ++p) kb[j][p] = x_frag(rk, ldkb, tok(j) + c16, p);
  floatx4 vv[2][2];
  {
    const uint32_t ldb = (uint32_t)(ldv * sizeof(T));
    const auto rs = buffer_of(v + t0 * ldv + (int64_t)h * D + v0, (uint32_t)L * ldb);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int vt = 0; vt < 2; ++vt)
        vv[vt][j] = buffer_load4<T>(rs, (uint32_t)(tok(j) + c16) * ldb +
                                            (uint32_t)((16 * vt + g4) * sizeof(T)));
  }
  float gm[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) gm[j] = gam[tok(j) + c16];
  cfrag mb[2][NSC];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int p = 0; p < NSC; ++p) mb[j][p] = acc_row(Mc, tok(j) + c16, p);
  issue_fence();

  // ---- the quarter's slice of S^T into LDS; S (rows v = 16 vt + c16 of the
  // slice) as A operands, reduction index p KS + (8 g + j | g)
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    const int i = lane + 64 * (2 * j + th), r = i / PPR, pc = i % PPR;
    word_alias* d = reinterpret_cast<word_alias*>(&Q4.hs[r][pc * EPP]);
    d[0] = hraw[j].x; d[1] = hraw[j].y; d[2] = hraw[j].z; d[3] = hraw[j].w;
  }
  __syncthreads();
  sfrag sa[2][NSD];
#pragma unroll
  for (int vt = 0; vt < 2; ++vt)
#pragma unroll
    for (int p = 0; p < NSD; ++p) {
      if constexpr (KS == 4) {
        sa[vt][p] = Q4.hs[p * KS + g][16 * vt + c16];
      } else {
        // rows p KS + 8 g + (0..3 | 4..7) of column 16 vt + c16
        const int r = p * KS + 8 * g + (c16 >> 2), col = 16 * vt + 4 * (c16 & 3);
        const u32x2 lo = lds_read_tr4(&Q4.hs[r][col]), hi = lds_read_tr4(&Q4.hs[r + 4][col]);
        sa[vt][p] = __builtin_bit_cast(sfrag, u32x4{lo[0], lo[1], hi[0], hi[1]});
      }
    }

  // A operand (rows v = 16 vt + c16) of accumulator-order step p from the
  // quarter's transposed tile
  auto xs_frag = [&](int vt, int p) __attribute__((always_inline)) {
    const int col = 16 * vt + c16;
    if constexpr (KS == 4) {
      return (cfrag)Q4.xs[16 * (p >> 2) + g4 + (p & 3)][col];
    } else {
      // rows 32 p + 4 g + 0..3 and 32 p + 16 + 4 g + 0..3 of column col
      const int r = 32 * p + g4 + (c16 >> 2), cc = 16 * vt + 4 * (c16 & 3);
      const u32x2 lo = lds_read_tr4(&Q4.xs[r][cc]), hi = lds_read_tr4(&Q4.xs[r + 16][cc]);
      return __builtin_bit_cast(cfrag, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
  };
  // this wave's transposed tiles into the quarter's tile (four consecutive
  // value columns per lane)
  auto put_xs = [&](const floatx4 (&x)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int j = 0; j < 2; ++j) store4(&Q4.xs[tok(j) + c16][16 * vt + g4], x[vt][j][0],
                                         x[vt][j][1], x[vt][j][2], x[vt][j][3]);
  };
  // byte offset of this lane's four value columns in token row c16
  const uint32_t so = (uint32_t)(((int64_t)c16 * HvD + v0 + g4) * sizeof(T));
  // ... and in the quarter's block of SBV-column rows of a stored
  // intermediate (R, Delta)
  static_assert(SBV == 32, "a quarter is one block of stored value columns");
  auto put_blk = [&](T* base, const floatx4 (&x)[2][2]) __attribute__((always_inline)) {
    const uint32_t rb = (uint32_t)(SBV * sizeof(T));
    const auto rs = buffer_of(base + ch * CHUNK * D + (int64_t)v0 * CHUNK, (uint32_t)L * rb);
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        buffer_store4<T>(rs, (uint32_t)(tok(j) + c16) * rb + (uint32_t)((16 * vt + g4) * sizeof(T)), x[vt][j]);
  };
  auto put_out = [&](T* base, const floatx4 (&x)[2][2]) __attribute__((always_inline)) {
    // rows past the chunk end fall outside the buffer: dropped
    const auto rs = buffer_of(base + t0 * HvD + (int64_t)h * D, (uint32_t)L * rowb);
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        buffer_store4<T>(rs, so + (uint32_t)tok(j) * rowb + (uint32_t)(16 * vt * sizeof(T)), x[vt][j]);
  };

  // ---- R^T = V^T - S K^T diag(Gam): x[vt][j] holds value rows
  // 16 vt + 4 g + i of token column tok(j) + c16
  floatx4 R[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int vt = 0; vt < 2; ++vt) {
      floatx4 acc = zero4();
#pragma unroll
      for (int p = 0; p < NSD; ++p) acc = MS::mma(sa[vt][p], kb[j][p], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) R[vt][j][i] = vv[vt][j][i] - gm[j] * acc[i];
    }
  put_blk(Rw, R);
  put_xs(R);
  __syncthreads();

  // ---- Delta^T = R^T M^T
  floatx4 Dl[2][2];
  {
    cfrag ra[2][NSC];
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int p = 0; p < NSC; ++p) ra[vt][p] = xs_frag(vt, p);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int vt = 0; vt < 2; ++vt) {
        Dl[vt][j] = zero4();
#pragma unroll
        for (int p = 0; p < NSC; ++p) Dl[vt][j] = MC::mma(ra[vt][p], mb[j][p], Dl[vt][j]);
      }
  }
  // Q and P for O, once K's and M's registers are free
  sfrag qb[2][NSD];
  cfrag pb[2][NSC];
  if constexpr (WITH_O) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int p = 0; p < NSD; ++p) qb[j][p] = x_frag(rq, ldqb, tok(j) + c16, p);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int p = 0; p < NSC; ++p) pb[j][p] = acc_row(Pc, tok(j) + c16, p);
    issue_fence();
  }
  put_blk(Dlw, Dl);

  if constexpr (WITH_O) {
    __syncthreads();   // both token halves have read R
    put_xs(Dl);
    __syncthreads();
    // ---- O^T = S (scale Q)^T diag(Gam) + Delta^T P^T
    cfrag da[2][NSC];
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int p = 0; p < NSC; ++p) da[vt][p] = xs_frag(vt, p);
    floatx4 O[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float sg = scale * gm[j];
#pragma unroll
      for (int vt = 0; vt < 2; ++vt) {
        floatx4 sq = zero4(), pd = zero4();
#pragma unroll
        for (int p = 0; p < NSD; ++p) sq = MS::mma(sa[vt][p], qb[j][p], sq);
#pragma unroll
        for (int p = 0; p < NSC; ++p) pd = MC::mma(da[vt][p], pb[j][p], pd);
#pragma unroll
        for (int i = 0; i < 4; ++i) O[vt][j][i] = pd[i] + sg * sq[i];
      }
    }
    put_out(o, O);
  }
}

// ---------------------------------------------------------------------------
// O alone, for 16-bit types, whose saved-state pass stores R and Delta on its
// way (it forms both on the chain), and Delta once more in the compute type
// for this product: per (chunk, value head)
//   O^T = S (scale Q)^T diag(Gam) + Delta^T P^T
// with the wave layout of chunk_out_kernel.  One workgroup per (chunk, key
// head) walks the G value heads of the group, so the Q rows (a B operand of
// every head) are loaded once for the group: loading them per value head
// was a fifth of the kernel's time.  Delta (compute type) enters the
// quarter's LDS tile as chunk_out_kernel puts its own.  Rows past the chunk
// end read zero (their P entries are zero anyway).
template <typename T, int D>
__global__ void __launch_bounds__(4 * D) __attribute__((amdgpu_waves_per_eu(4))) chunk_o_kernel(
    const T* __restrict__ q, int64_t ldq, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ seq_off, int n_seq, int Hv, int G, float scale,
    const typename Compute<T>::type* __restrict__ Pw, const float* __restrict__ Gw,
    const T* __restrict__ hst, const typename Compute<T>::type* __restrict__ Dlw,
    T* __restrict__ o, int n_items) {
  typedef typename Compute<T>::type CT;
  typedef Mma<T> MS;
  typedef Mma<CT> MC;
  typedef OutQuarter<T, D> OQ;
  typedef typename MS::frag sfrag;
  typedef typename MC::frag cfrag;
  constexpr int KS = MS::KS;
  static_assert(sizeof(T) == 2 && KS == 32, "16-bit operands");
  constexpr int NQ = D / 32;
  constexpr int NSD = D / KS, NSC = CHUNK / KS;
  constexpr int EPP = 8, PPR = 4;             // 16-byte pieces per 32-column row
  constexpr int NH = D * PPR / 128;           // S pieces per lane (two waves per slice)
  __shared__ OQ qs[NQ];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int vq = wave % NQ, th = wave / NQ;
  const int Hk = Hv / G;
  const int item = xcd_item(blockIdx.x, n_items);
  const int64_t c = item / Hk;
  const int kh = item % Hk;
  if (c >= seq_off[n_seq]) return;
  int64_t t0;
  int L;
  chunk_span(seq_off, cu, n_seq, c, t0, L);
  const int g = lane >> 4, g4 = 4 * g, c16 = lane & 15;
  const int v0 = 32 * vq;
  const int64_t HvD = (int64_t)Hv * D;
  OQ& Q4 = qs[vq];
  const uint32_t rowb = (uint32_t)(HvD * sizeof(T));
  auto tok = [&](int j) { return 16 * (2 * th + j); };

  // ---- the Q rows of this wave's tokens, once for the group
  const uint32_t ldqb = (uint32_t)(ldq * sizeof(T));
  const auto rq = buffer_of(q + t0 * ldq + (int64_t)kh * D, (uint32_t)L * ldqb);
  sfrag qb[2][NSD];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int p = 0; p < NSD; ++p)
      qb[j][p] = buffer_frag<T>(rq, (uint32_t)(tok(j) + c16) * ldqb + (uint32_t)(p * KS + 8 * g) * sizeof(T));
  const uint32_t so = (uint32_t)(((int64_t)c16 * HvD + v0 + g4) * sizeof(T));

  for (int hh = 0; hh < G; ++hh) {
    const int h = kh * G + hh;
    const int64_t ch = c * Hv + h;
    const float* gam = Gw + ch * CHUNK;
    const CT* Pc = Pw + ch * CHUNK * CHUNK;
    // ---- this head's inputs, requested up front: S slice, P rows, Delta rows
    // (the S slice and Delta rows, read once, with the non-temporal hint; P is
    // read by every quarter)
    uint4 hraw[NH];
    {
      const T* Sg = hst + ch * D * D + (int64_t)v0 * D;   // the quarter's block of the state
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const int i = lane + 64 * (2 * j + th), r = i / PPR, pc = i % PPR;
        hraw[j] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(Sg + (int64_t)r * SBV + pc * EPP)));
      }
    }
    cfrag pb[2][NSC];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int p = 0; p < NSC; ++p)
        pb[j][p] = *reinterpret_cast<const cfrag*>(Pc + (tok(j) + c16) * CHUNK + 32 * p + 8 * g);
    // this wave's 32 tokens of the quarter's Delta columns: 4 pieces per row
    cfrag draw[2];
    const uint32_t rdb = (uint32_t)(SBV * sizeof(CT));
    const auto rd = buffer_of(Dlw + ch * CHUNK * D + (int64_t)v0 * CHUNK, (uint32_t)L * rdb);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = lane + 64 * j, r = 32 * th + i / PPR, pc = i % PPR;
      draw[j] = buffer_frag<CT, CACHE_NT>(rd, (uint32_t)r * rdb + (uint32_t)(pc * 16));
    }
    float gm[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) gm[j] = gam[tok(j) + c16];
    issue_fence();
    if (hh > 0) __syncthreads();   // the previous head's LDS tiles are read

    // ---- S^T slice and Delta (compute type) into the quarter's LDS tiles
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const int i = lane + 64 * (2 * j + th), r = i / PPR, pc = i % PPR;
      word_alias* d = reinterpret_cast<word_alias*>(&Q4.hs[r][pc * EPP]);
      d[0] = hraw[j].x; d[1] = hraw[j].y; d[2] = hraw[j].z; d[3] = hraw[j].w;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = lane + 64 * j, r = 32 * th + i / PPR, pc = i % PPR;
      *reinterpret_cast<cfrag*>(&Q4.xs[r][pc * EPP]) = draw[j];
    }
    __syncthreads();

    // ---- O^T = S (scale Q)^T diag(Gam) + Delta^T P^T: value rows 16 vt + 4 g
    // + i of token column tok(j) + c16, out in 8-byte pieces; the A operands
    // (transposing reads) one value tile at a time, which keeps the group's Q
    // operands in registers without spills
    const auto rs = buffer_of(o + t0 * HvD + (int64_t)h * D, (uint32_t)L * rowb);
#pragma unroll
    for (int vt = 0; vt < 2; ++vt) {
      sfrag sa[NSD];
#pragma unroll
      for (int p = 0; p < NSD; ++p) {
        const int r = p * KS + 8 * g + (c16 >> 2), col = 16 * vt + 4 * (c16 & 3);
        const u32x2 lo = lds_read_tr4(&Q4.hs[r][col]), hi = lds_read_tr4(&Q4.hs[r + 4][col]);
        sa[p] = __builtin_bit_cast(sfrag, u32x4{lo[0], lo[1], hi[0], hi[1]});
      }
      cfrag da[NSC];
#pragma unroll
      for (int p = 0; p < NSC; ++p) {
        const int r = 32 * p + g4 + (c16 >> 2), cc = 16 * vt + 4 * (c16 & 3);
        const u32x2 lo = lds_read_tr4(&Q4.xs[r][cc]), hi = lds_read_tr4(&Q4.xs[r + 16][cc]);
        da[p] = __builtin_bit_cast(cfrag, u32x4{lo[0], lo[1], hi[0], hi[1]});
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        floatx4 sq = zero4(), pd = zero4();
#pragma unroll
        for (int p = 0; p < NSD; ++p) sq = MS::mma(sa[p], qb[j][p], sq);
#pragma unroll
        for (int p = 0; p < NSC; ++p) pd = MC::mma(da[p], pb[j][p], pd);
        const float sg = scale * gm[j];
        floatx4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = pd[i] + sg * sq[i];
        buffer_store4<T>(rs, so + (uint32_t)tok(j) * rowb + (uint32_t)(16 * vt * sizeof(T)), ov);
      }
    }
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_chunk_outputs(const gdn_shape& s, const void* q, const void* k, const void* v,
                                int64_t ldq, int64_t ldk, int64_t ldv, float scale,
                                const int32_t* cu, void* o, void* wsv, hipStream_t st) {
  char* ws = (char*)wsv;
  const ChunkLayout Ly = chunk_layout(s, ChunkFlow::Bwd);   // (saved-state and backward flows only)
  if (Ly.nt_max == 0 || s.total_tokens == 0) return hipSuccess;
  return dispatch_chunk(s, [&](auto cf) {
    using T = typename decltype(cf)::type;
    constexpr int D = decltype(cf)::d;
    typedef typename Compute<T>::type CT;
    const int n_items = (int)(Ly.nt_max * s.hv);
    if constexpr (sizeof(T) == 2) {
      // the saved-state pass has stored R and Delta: O alone, if wanted
      if (!o) return hipSuccess;
      const int n_group_items = (int)(Ly.nt_max * s.hk);   // (chunk, key head)
      hipLaunchKernelGGL((chunk_o_kernel<T, D>), dim3(n_group_items), dim3(4 * D), 0, st, (const T*)q,
                         ldq, cu, (const int32_t*)(ws + Ly.seq_off), s.n_seq, s.hv, s.hv / s.hk,
                         scale, (const CT*)(ws + Ly.pw), (const float*)(ws + Ly.gw),
                         (const T*)(ws + Ly.h), (const CT*)(ws + Ly.dl16w), (T*)o, n_group_items);
      return hipGetLastError();
    }
    auto kern = o ? chunk_out_kernel<T, D, true> : chunk_out_kernel<T, D, false>;
    hipLaunchKernelGGL(kern, dim3(n_items), dim3(4 * D), 0, st, (const T*)q, (const T*)k,
                       (const T*)v, ldq, ldk, ldv, cu, (const int32_t*)(ws + Ly.seq_off), s.n_seq,
                       s.hv, s.hv / s.hk, scale, (const CT*)(ws + Ly.mw), (const CT*)(ws + Ly.pw),
                       (const float*)(ws + Ly.gw), (const T*)(ws + Ly.h), (T*)(ws + Ly.rw),
                       (T*)(ws + Ly.dlw), (T*)o, n_items);
    return hipGetLastError();
  });
}

}  // namespace gdn
