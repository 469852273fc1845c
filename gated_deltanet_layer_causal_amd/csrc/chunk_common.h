// Shared pieces of the chunked gated delta rule kernels (forward and backward).
//
// Chunked (WY/UT) form used by every kernel.  For a chunk of L <= 64 tokens of
// one sequence and one value head, with S the d_v x d_k state entering it:
//   gam_t = g_1 + ... + g_t (inside the chunk),  Gam_t = exp(gam_t)
//   D[t,s] = exp(gam_t - gam_s) for s <= t
//   A[t,s] = beta_t D[t,s] (k_t . k_s) for s < t,   Tinv = (I + A)^-1
//   M = Tinv diag(beta)
//   R = V - diag(Gam) K S^T,   Delta = M R               (the delta-rule writes)
//   P = D o (scale Q K^T)  (s <= t)
//   O = diag(Gam) scale Q S^T + P Delta
//   S_next = Gam_L S + (diag(dec) Delta)^T K,  dec_t = exp(gam_L - gam_t)
// which reproduces the token-by-token recurrence exactly in exact arithmetic.
// Only differences gam_t - gam_s with s <= t are exponentiated, so with
// g <= 0 every exponential is <= 1 and never overflows.
#pragma once
#include "common.h"
#include "launch.h"

namespace gdn {

template <typename T> struct Pad { static constexpr int v = 16 / sizeof(T); };

// MFMA operand type of the forward-state kernels for a storage type: fp16 for
// 16-bit storage (11-bit significands for the operands and intermediates;
// the fp16 range, |x| <= 65504, bounds the values: see the range contract in
// libgdn.h), fp32 for fp32 storage.
template <typename T> struct Compute { typedef fp16 type; };
template <> struct Compute<float> { typedef float type; };

// Column order of the operands that the sequential kernels read as MFMA A
// operands in accumulator order (W, Q rows, K^T, M, P).  With 16-bit
// operands a step covers columns 32 p + 16 h + 4 g + i (h, i < 2, 4) for lane
// group g, so each block of 32 columns is stored as [g][h][i]: column
// 16 h + 4 g + i at position 8 g + 4 h + i, and a lane's eight values are one
// 16-byte piece.  fp32 operands keep the natural order.
template <typename CT> __device__ __forceinline__ int acc_col(int c) {
  if constexpr (sizeof(CT) == 4) {
    return c;
  } else {
    const int w = c & 31;
    return (c & ~31) + 8 * ((w >> 2) & 3) + 4 * (w >> 4) + (w & 3);
  }
}
// The inverse per 16-byte piece: the source column of element j of stored
// piece p (stored columns 8p..8p+7), so that acc_col(acc_piece_col(p, j))
// == 8p + j.  Row stores in accumulator order then go out whole.
template <typename CT> __device__ __forceinline__ int acc_piece_col(int p, int j) {
  if constexpr (sizeof(CT) == 4) {
    return 8 * p + j;
  } else {
    return 32 * (p >> 2) + 16 * (j >> 2) + 4 * (p & 3) + (j & 3);
  }
}

// exp of an in-chunk gate-sum difference.  The sums are kept in fp64: with
// strong decay they reach several hundred inside one chunk, where an fp32
// difference would lose ~3e-5 relative accuracy.  fp32 storage evaluates the
// exponential in fp64 too.
template <typename T> __device__ __forceinline__ float dexp(double x) { return __expf((float)x); }
template <> __device__ __forceinline__ float dexp<float>(double x) { return (float)exp(x); }

// Segment length (in chunks) of the segment-parallel state scan, or 0 for
// one sequential pass per sequence.  The sequential passes run one chain
// per (sequence, value head, block of 32 value rows), one workgroup per CU;
// when there are too few chains to fill the chip, each sequence is split
// into segments that run in parallel: a pass from a zero state per segment
// that also carries identity rows (giving the segment's end state B_s and its
// transition Phi_s), a short sequential combine S_{s+1} = S_s Phi_s + B_s,
// then the ordinary pass per segment from its true start state.  With ns
// segments and at most SEG_TARGET_CHAINS chains per pass (measured: 224
// one-per-CU workgroups run in one round on the 256 CUs, 256 take two),
// the first pass (twice the chains) takes two rounds and the last one, so
// the chain costs 3 / ns of the unsplit pass: the scan is used when ns >= 4.
// shape.seg_chunks > 0 forces a segment length, < 0 forbids splitting.
constexpr int SEG_TARGET_CHAINS = 224;
constexpr int SEG_MIN_SEGMENTS = 4;
constexpr int SEG_MIN_LEN = 8;
inline int64_t seg_len(const gdn_shape& s) {
  if (s.seg_chunks > 0) return s.seg_chunks;
  if (s.seg_chunks < 0 || s.total_tokens == 0) return 0;
  const int64_t chains = (int64_t)s.n_seq * s.hv * (s.dk / 32);
  const int64_t nseg = SEG_TARGET_CHAINS / chains;
  if (nseg < SEG_MIN_SEGMENTS) return 0;
  const int64_t nt = s.total_tokens / CHUNK + s.n_seq;
  const int64_t per_seq = (nt + s.n_seq - 1) / s.n_seq;
  int64_t L = (per_seq + nseg - 1) / nseg;
  if (L < SEG_MIN_LEN) L = SEG_MIN_LEN;
  return L >= per_seq ? 0 : L;
}

// Workspace layout (byte offsets; every region 256-byte aligned).
// The per-chunk intermediates that the sequential passes store (chunk-start
// states and their gradients, R, Delta, dDelta) keep each block of SBV value
// columns together: a sequential-pass workgroup owns SBV value columns, so
// it writes whole lines rather than a quarter of each row of the head.
//   states:     [chunk][head][dv / SBV][dk][SBV]
//   token rows: [chunk][head][dv / SBV][64][SBV] (row t: token t of the chunk)
constexpr int SBV = 32;
// element offset, in a (chunk, head) block of n rows, of row r and value
// column v (a run of up to 8 columns from v stays in one block when v % 8 == 0)
__host__ __device__ constexpr int64_t blk_at(int r, int v, int n) {
  return (int64_t)(v / SBV) * n * SBV + (int64_t)r * SBV + v % SBV;
}

struct ChunkLayout {
  int64_t nt_max;     // upper bound on the number of chunks: T/64 + n_seq
  int64_t seg;        // segment length in chunks (0: one span per sequence)
  int64_t nspan_max;  // upper bound on the number of spans (segments)
  size_t seq_off;     // int32 [n_seq + 1]: first chunk of each sequence; [n_seq] = #chunks
  size_t spans;       // int32 [nspan_max][4]: span = (first chunk, end chunk, token of its
                      // first chunk, end token of its sequence) -- the unit of a sequential pass
  size_t segb;        // int32 [n_seq + 1]: first span of each sequence; [n_seq] = #spans
  size_t sumf;        // fp32 [nspan_max][hv][2 dv][dk]: a span's end state from zero (rows
                      // < dv) and its transition Phi (rows >= dv) (segmented scan)
  size_t sst;         // fp32 [nspan_max][hv][dv][dk]: start state of each span (segmented)
  size_t sumr;        // fp32 [nspan_max][hv][dv][dk]: reverse pass from zero: dS at a span's start
  size_t dse;         // fp32 [nspan_max][hv][dv][dk]: dS at each span's end (segmented)
  size_t gcum;        // fp64 [nt_max][hv][64]: in-chunk cumulative gate (flat past the chunk end)
  size_t mw, pw;      // CT [nt_max][hv][64][64]: M = Tinv diag(beta), P (accumulator column order)
  size_t ww;          // CT [nt_max][hv][64][dk]: W = M diag(Gam) K
  size_t ktw;         // CT [nt_max][hk][dk][64]: K^T of each chunk
  size_t q16w;        // CT [nt_max][hk][64][dk]: Q rows of each chunk (zero past its end)
  size_t gw, dw;      // fp32 [nt_max][hv][64]: Gam_t and dec_t (clamped to the chunk length)
  size_t kb, ktb, qtb; // T [nt_max][hk]: K rows [64][dk], K^T and Q^T [dk][64] (backward)
  size_t k16w;        // CT [nt_max][hk][64][dk]: K rows, columns in accumulator order
                      // (backward, 16-bit types: the saved-state pass reads these in place of W, K^T)
  size_t ptb;         // T [nt_max][hv][64][64]: P^T (backward)
  size_t kkw;         // CT [nt_max][hk][64][64]: K K^T of each chunk (backward)
  size_t bw;          // fp32 [nt_max][hv][64]: beta_t, zero past the chunk end (backward)
  size_t tib;         // T [nt_max][hv][2][64][64]: Tinv (columns in accumulator order), Tinv^T (backward)
  size_t h, dh;       // T [nt_max][hv][dv / SBV][dk][SBV]: chunk-start state, chunk-end state gradient
  size_t rw, dlw, ddw;  // T [nt_max][hv][dv / SBV][64][SBV]: R, Delta (fp32 data only), dDelta
  size_t dl16w;       // CT [nt_max][hv][dv / SBV][64][SBV]: Delta in the compute type (16-bit data:
                      // for the outputs and the gradients)
  size_t sink;        // SINK_ELEMS scratch floats: target of stores for padding rows
  size_t total_fwd, total_bwd;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Stores for rows past the end of a sequence (padding rows of the last
// chunk) go to a scratch "sink" instead of being skipped: every store is then
// unconditional, which keeps the compiler's memory-counter waits exact so
// that prefetched loads stay in flight across the chunk.  Nothing reads it.
constexpr int SINK_ELEMS = 4096;
template <typename T>
__device__ __forceinline__ T* row_or_sink(T* p, bool valid, void* sink, int tid) {
  return valid ? p : reinterpret_cast<T*>(sink) + (tid & (SINK_ELEMS - 1));
}

// The workspace of the forward-only flow (preparation in forward mode, then
// the MODE 0 pass) or of the backward / saved-state flow.  The backward flow
// has no use for the Q rows in the compute type, nor, with 16-bit data
// (whose saved-state pass works from the K rows), for W and the compute-type
// K^T: those regions are empty there.  Every launcher of one flow uses the
// same layout.
enum class ChunkFlow { Fwd, Bwd };

inline ChunkLayout chunk_layout(const gdn_shape& s, ChunkFlow flow) {
  ChunkLayout L;
  const size_t es = s.dtype == GDN_FP32 ? 4 : 2;
  const bool bwd = flow == ChunkFlow::Bwd;
  const size_t es_w = bwd && es == 2 ? 0 : es;   // W and the compute-type K^T
  const size_t es_q = bwd ? 0 : es;               // Q rows in the compute type
  const int64_t T = s.total_tokens;
  L.nt_max = T / CHUNK + s.n_seq;
  L.seg = seg_len(s);
  L.nspan_max = L.seg > 0 ? L.nt_max / L.seg + s.n_seq + 1 : s.n_seq;
  const size_t st_bytes = L.seg > 0 ? sizeof(float) * (size_t)L.nspan_max * s.hv * s.dk * s.dv : 0;
  size_t off = 0;
  L.seq_off = off; off = align256(off + sizeof(int32_t) * (size_t)(s.n_seq + 1));
  L.spans = off; off = align256(off + sizeof(int32_t) * 4 * (size_t)L.nspan_max);
  L.segb = off; off = align256(off + sizeof(int32_t) * (size_t)(s.n_seq + 1));
  L.sumf = off; off = align256(off + 2 * st_bytes);
  L.sst = off; off = align256(off + st_bytes);
  L.sumr = off; off = align256(off + st_bytes);
  L.dse = off; off = align256(off + st_bytes);
  L.sink = off; off = align256(off + sizeof(float) * SINK_ELEMS);
  L.gcum = off; off = align256(off + sizeof(double) * (size_t)L.nt_max * s.hv * CHUNK);
  L.mw = off; off = align256(off + es * (size_t)L.nt_max * s.hv * CHUNK * CHUNK);
  L.pw = off; off = align256(off + es * (size_t)L.nt_max * s.hv * CHUNK * CHUNK);
  L.ww = off; off = align256(off + es_w * (size_t)L.nt_max * s.hv * CHUNK * s.dk);
  L.ktw = off; off = align256(off + es_w * (size_t)L.nt_max * s.hk * s.dk * CHUNK);
  L.q16w = off; off = align256(off + es_q * (size_t)L.nt_max * s.hk * CHUNK * s.dk);
  L.gw = off; off = align256(off + sizeof(float) * (size_t)L.nt_max * s.hv * CHUNK);
  L.dw = off; off = align256(off + sizeof(float) * (size_t)L.nt_max * s.hv * CHUNK);
  L.total_fwd = off;
  L.kb = off; off = align256(off + es * (size_t)L.nt_max * s.hk * CHUNK * s.dk);
  L.k16w = off; off = align256(off + (es == 2 ? 2 * (size_t)L.nt_max * s.hk * CHUNK * s.dk : 0));
  L.ktb = off; off = align256(off + es * (size_t)L.nt_max * s.hk * s.dk * CHUNK);
  L.qtb = off; off = align256(off + es * (size_t)L.nt_max * s.hk * s.dk * CHUNK);
  L.ptb = off; off = align256(off + es * (size_t)L.nt_max * s.hv * CHUNK * CHUNK);
  L.kkw = off; off = align256(off + es * (size_t)L.nt_max * s.hk * CHUNK * CHUNK);
  L.bw = off; off = align256(off + sizeof(float) * (size_t)L.nt_max * s.hv * CHUNK);
  L.tib = off; off = align256(off + es * (size_t)L.nt_max * s.hv * 2 * CHUNK * CHUNK);
  L.h = off; off = align256(off + es * (size_t)L.nt_max * s.hv * s.dk * s.dv);
  L.dh = off; off = align256(off + es * (size_t)L.nt_max * s.hv * s.dk * s.dv);
  const size_t rows = (size_t)L.nt_max * CHUNK * s.hv * s.dv;   // per-chunk token rows
  L.rw = off; off = align256(off + es * rows);
  L.dlw = off; off = align256(off + (es == 4 ? es * rows : 0));
  L.ddw = off; off = align256(off + es * rows);
  L.dl16w = off; off = align256(off + (es == 2 ? 2 * rows : 0));
  L.total_bwd = off;
  return L;
}

// The combine of the segmented scan (chunk_scan.hip): forward (rev false)
// from Sin = S0 (nullable) into the span start states and Sout = S_final
// (nullable); reverse from Sin = dS_final into the span end gradients and
// Sout = dS0.
hipError_t launch_span_combine(const gdn_shape& s, const ChunkLayout& Ly, char* ws, bool rev,
                               const float* Sin, float* Sout, hipStream_t st);

// Instantiation selector for the chunk kernels: bf16 storage at head dim 32
// or 128, fp32 storage at head dim 32 (the only combinations validated).
template <typename T, int D> struct ChunkCfg { typedef T type; static constexpr int d = D; };
template <typename F> hipError_t dispatch_chunk(const gdn_shape& s, F&& f) {
  if (s.dtype == GDN_BF16) return s.dk == 128 ? f(ChunkCfg<bf16, 128>{}) : f(ChunkCfg<bf16, 32>{});
  if (s.dtype == GDN_FP16) return s.dk == 128 ? f(ChunkCfg<fp16, 128>{}) : f(ChunkCfg<fp16, 32>{});
  return f(ChunkCfg<float, 32>{});
}

// Largest n in [0, n_seq) with off[n] <= c (off non-decreasing).
__device__ __forceinline__ int upper_index(const int32_t* off, int n_seq, int64_t c) {
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)off[mid] <= c) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Chunk c -> (first token, length) using the per-sequence chunk offsets.
__device__ __forceinline__ void chunk_span(const int32_t* seq_off, const int32_t* cu, int n_seq,
                                           int64_t c, int64_t& t0, int& L) {
  const int n = upper_index(seq_off, n_seq, c);
  t0 = (int64_t)cu[n] + (int64_t)CHUNK * (c - seq_off[n]);
  const int64_t rem = (int64_t)cu[n + 1] - t0;
  L = rem < CHUNK ? (int)rem : CHUNK;
}

// Stage rows [0, 64) x [0, W) of two token-major tensors into LDS (row
// stride ld_s), zero-filling rows >= L (1 <= L <= 64).  Source row r of
// tensor a is at sa + r * lda.  Every load is issued before the first store
// (rows >= L re-read row L - 1, which is valid memory, and are zeroed where
// stored), so their latencies overlap: a loop that stored each piece as it
// arrived waited for every load in turn.  The rows are read once, with the
// non-temporal hint.
template <typename TD, int W, typename TS>
__device__ __forceinline__ void stage_rows2(TD* da, const TS* sa, int64_t lda, TD* db,
                                            const TS* sb, int64_t ldb, int ld_s, int L, int tid) {
  constexpr int G8 = W / 8, ITEMS = CHUNK * G8;
  constexpr int N = (ITEMS + 255) / 256;
  constexpr int Q = (int)sizeof(TS) / 2;   // 16-byte words per 8 elements
  uint4 ra[N][Q], rb[N][Q];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int i = tid + 256 * j, r = i / G8, c8 = (i % G8) * 8;
    const int rr = r < L ? r : L - 1;
    if (ITEMS % 256 == 0 || i < ITEMS) {
      const uint4* pa = reinterpret_cast<const uint4*>(sa + (int64_t)rr * lda + c8);
      const uint4* pb = reinterpret_cast<const uint4*>(sb + (int64_t)rr * ldb + c8);
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        ra[j][q] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(pa) + q));
        rb[j][q] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(pb) + q));
      }
    }
  }
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int i = tid + 256 * j, r = i / G8, c8 = (i % G8) * 8;
    if (ITEMS % 256 == 0 || i < ITEMS) {
      f8 va = load8(reinterpret_cast<const TS*>(&ra[j][0]));
      f8 vb = load8(reinterpret_cast<const TS*>(&rb[j][0]));
      if (r >= L) {
#pragma unroll
        for (int e = 0; e < 8; ++e) va.v[e] = vb.v[e] = 0.f;
      }
      store8(da + r * ld_s + c8, va);
      store8(db + r * ld_s + c8, vb);
    }
  }
}

// ---- register prefetch ------------------------------------------------------
// The sequential kernels load chunk c+1 into registers while chunk c computes,
// so global-memory latency leaves the critical path.  Raw copies keep the
// storage type; conversion happens when the registers are consumed.

// Rows [0, 64) x [0, W) of a token-major tensor, 8 elements per item, items
// spread over the 256 threads.  Loads are unconditional (rows >= L re-read
// row L-1, which is valid memory) so that no wait is forced at load time;
// rows >= L are zeroed when the registers are stored.
// ROWFAST = false: consecutive lanes take consecutive 8-element column blocks
// of a row (coalesced loads; for row-major LDS staging).  ROWFAST = true:
// consecutive lanes take consecutive rows of one column block, so that a
// transposed LDS store writes consecutive addresses (no bank conflicts).
template <typename T, int W, bool ROWFAST = false> struct RowPrefetch {
  static constexpr int ITEMS = CHUNK * W / 8;
  static constexpr int NI = ITEMS / 256;
  static_assert(ITEMS % 256 == 0, "row prefetch covers whole rows per thread");
  Raw8<T> r[NI];
  int L;
  __device__ __forceinline__ static int row_of(int i) { return ROWFAST ? i % CHUNK : i / (W / 8); }
  __device__ __forceinline__ static int col_of(int i) {
    return ROWFAST ? (i / CHUNK) * 8 : (i % (W / 8)) * 8;
  }
  __device__ __forceinline__ void load(const T* src, int64_t ld, int L_, int tid) {
    L = L_;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int i = tid + 256 * j;
      const int row = row_of(i), c8 = col_of(i);
      r[j] = ld_raw8(src + (int64_t)(row < L ? row : L - 1) * ld + c8);
    }
  }
  __device__ __forceinline__ f8 value(int j, int row) const {
    f8 v = raw_f8(r[j]);
    if (row >= L) {
#pragma unroll
      for (int u = 0; u < 8; ++u) v.v[u] = 0.f;
    }
    return v;
  }
  template <typename TD>
  __device__ __forceinline__ void store(TD* dst, int ld_s, int tid) const {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int i = tid + 256 * j;
      const int row = row_of(i);
      store8(dst + row * ld_s + col_of(i), value(j, row));
    }
  }
};

// One MFMA A/B fragment read from memory with contiguous K, kept raw until
// use.  16-bit operands: 8 values (16 bytes) of storage type S converted to
// CT; fp32 operands: one value.
template <typename CT, typename S> struct FragKC {
  typedef uint4 raw;
  __device__ __forceinline__ static raw load(const S* row, int k0, int lane) {
    return *reinterpret_cast<const uint4*>(row + k0 + 8 * (lane >> 4));
  }
  __device__ __forceinline__ static typename Mma<CT>::frag cvt(const raw& r) {
    if constexpr (__is_same(S, CT)) {
      return __builtin_bit_cast(typename Mma<CT>::frag, r);
    } else {
      f8 v = load8(reinterpret_cast<const S*>(&r));
      typename Mma<CT>::frag f;
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = (CT)v.v[j];
      return f;
    }
  }
};
template <> struct FragKC<float, float> {
  typedef float raw;
  __device__ __forceinline__ static raw load(const float* row, int k0, int lane) {
    return row[k0 + (lane >> 4)];
  }
  __device__ __forceinline__ static float cvt(const raw& r) { return r; }
};

// Same, for a fragment whose K index is strided by ld in memory (8 scalar
// loads for 16-bit operands; the raw values stay untouched until use).
template <typename MT, typename S> struct FragKS {
  struct raw { S x[8]; };
  __device__ __forceinline__ static raw load(const S* col, int ld, int k0, int lane) {
    raw r;
    const S* p = col + (int64_t)(k0 + 8 * (lane >> 4)) * ld;
#pragma unroll
    for (int j = 0; j < 8; ++j) r.x[j] = p[(int64_t)j * ld];
    return r;
  }
  __device__ __forceinline__ static typename Mma<MT>::frag cvt(const raw& r) {
    typename Mma<MT>::frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (MT)to_f(r.x[j]);
    return f;
  }
};
template <typename S> struct FragKS<float, S> {
  typedef S raw;
  __device__ __forceinline__ static raw load(const S* col, int ld, int k0, int lane) {
    return col[(int64_t)(k0 + (lane >> 4)) * ld];
  }
  __device__ __forceinline__ static float cvt(const raw& r) { return to_f(r); }
};

// Transposed staging of prefetched rows: dst[col][row] (row stride ld_s).
template <typename T, int W, bool RF, typename TD>
__device__ __forceinline__ void store_rows_transposed(const RowPrefetch<T, W, RF>& p, TD* dst,
                                                      int ld_s, int tid) {
#pragma unroll
  for (int j = 0; j < RowPrefetch<T, W, RF>::NI; ++j) {
    const int i = tid + 256 * j;
    const int row = RowPrefetch<T, W, RF>::row_of(i), c8 = RowPrefetch<T, W, RF>::col_of(i);
    const f8 v = p.value(j, row);
#pragma unroll
    for (int u = 0; u < 8; ++u) dst[(c8 + u) * ld_s + row] = from_f<TD>(v.v[u]);
  }
}

// Keeps already-issued prefetch loads where they are: neither the optimizer
// nor the machine scheduler may move memory operations or instructions across
// it (otherwise the loads get sunk next to their first use).
__device__ __forceinline__ void issue_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup -> work item so that consecutive work items (the value-row
// blocks of one head) run on the same XCD: workgroups are dealt to the 8
// XCDs round-robin, so item = xcd * (n / 8) + (block / 8) when n % 8 == 0.
__device__ __forceinline__ int xcd_item(int block, int n) {
  return (n % 8 == 0) ? (block % 8) * (n / 8) + block / 8 : block;
}

// (I + A)^-1 for strictly lower-triangular A (64 x 64, fp32 in LDS, row
// stride 68), written to Ti.  Blocked: the four 16 x 16 diagonal blocks are
// inverted by forward substitution (one lane per column), then block
// (i, j), i > j, is  -Dinv_i * sum_{m=j}^{i-1} A_im Ti_mj,  level by level.
// Uses X (16 x 17 fp32) as scratch.  Ends with a barrier.
__device__ __forceinline__ void invert_unit_lower(const float (*A)[68], float (*Ti)[68],
                                                  float (*X)[17], int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  // zero the strictly upper block triangle
  for (int i = tid; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;
    if ((c >> 4) > (r >> 4)) Ti[r][c] = 0.f;
  }
  if (lane < 16) {
    const int b = wave * 16, j = lane;
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float acc = (t == j) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < t; ++s) acc -= A[b + t][b + s] * x[s];
      x[t] = acc;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) Ti[b + t][b + j] = x[t];
  }
  __syncthreads();
  const int r = tid >> 4, cc = tid & 15;
  for (int lv = 1; lv < 4; ++lv) {
    for (int i = lv; i < 4; ++i) {
      const int j = i - lv;
      float acc = 0.f;
      for (int m = j; m < i; ++m) {
#pragma unroll
        for (int u = 0; u < 16; ++u) acc += A[16 * i + r][16 * m + u] * Ti[16 * m + u][16 * j + cc];
      }
      X[r][cc] = acc;
      __syncthreads();
      float out = 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u) out += Ti[16 * i + r][16 * i + u] * X[u][cc];
      Ti[16 * i + r][16 * j + cc] = -out;
      __syncthreads();
    }
  }
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ double wave_incl_scan(double x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    double y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}


// The same sums without LDS: DPP shifts within rows of 16 lanes (lanes
// without a source read zero), then the other rows' totals, read from one
// lane of each row.  Inclusive prefix sum:
__device__ __forceinline__ float wave_prefix_dpp(float x, int lane) {
  x += dpp_f<0x111>(x);   // row_shr:1
  x += dpp_f<0x112>(x);   // row_shr:2
  x += dpp_f<0x114>(x);   // row_shr:4
  x += dpp_f<0x118>(x);   // row_shr:8
  const float t0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 15));
  const float t1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
  const float t2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 47));
  const int row = lane >> 4;
  float e = 0.f;   // the earlier rows' totals
  if (row >= 1) e = t0;
  if (row >= 2) e += t1;
  if (row >= 3) e += t2;
  return x + e;
}
// ... and inclusive suffix sum.
__device__ __forceinline__ float wave_suffix_dpp(float x, int lane) {
  x += dpp_f<0x101>(x);   // row_shl:1
  x += dpp_f<0x102>(x);   // row_shl:2
  x += dpp_f<0x104>(x);   // row_shl:4
  x += dpp_f<0x108>(x);   // row_shl:8
  const float t1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  const float t2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  const float t3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  const int row = lane >> 4;
  float e = 0.f;   // the later rows' totals
  if (row <= 2) e = t3;
  if (row <= 1) e += t2;
  if (row <= 0) e += t1;
  return x + e;
}
// ... and the sum over the wave, in every lane.
__device__ __forceinline__ float wave_sum_dpp(float x) {
  x = lane_group_sum<16>(x);
  const int v = __builtin_bit_cast(int, x);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(v, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(v, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(v, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(v, 48)));
}

}  // namespace gdn
