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
// Wave w owns value columns [32 w, 32 w + 32) for every token of the chunk.
// R and Delta then stay in MFMA accumulators and enter the next product as
// its B operand in accumulator order (M and P are stored with their columns
// in that order, acc_col).  S^T is the B operand of K S^T and Q S^T: the wave
// copies its d_k x 32 slice of S into its own LDS rows (padded so that the
// four lane groups of a column read hit different banks) and gathers each
// lane's reduction values from it.  K and Q rows are read straight from the
// conv output with range-checked buffer loads, which return zero for rows
// past the chunk's end.
#include "chunk_stream.h"

namespace gdn {

template <typename T, int D> struct alignas(16) OutWave {
  static constexpr int LDR = 32 + (sizeof(T) == 2 ? 2 : 1);   // padded row of 32 columns
  T hs[D][LDR];       // S^T slice: row k, value column
  T vs[CHUNK][LDR];   // V slice: row t, value column
};

// 32-bit words of the LDS slices: written as words, read as elements, so the
// word type must alias the element type.
typedef uint32_t __attribute__((may_alias)) word_alias;

// 16-byte (16-bit types) or 4-byte (fp32) MFMA operand from a buffer.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag buffer_frag(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  if constexpr (sizeof(T) == 2)
    return __builtin_bit_cast(typename Mma<T>::frag, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  else
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}

template <typename T, int D, bool WITH_O>
__global__ void __launch_bounds__(2 * D) chunk_out_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t ldq,
    int64_t ldk, int64_t ldv, const int32_t* __restrict__ cu, const int32_t* __restrict__ seq_off,
    int n_seq, int Hv, int G, float scale, const typename Compute<T>::type* __restrict__ Mw,
    const typename Compute<T>::type* __restrict__ Pw, const float* __restrict__ Gw,
    const T* __restrict__ hst, T* __restrict__ Rw, T* __restrict__ Dlw, T* __restrict__ o,
    int n_items) {
  typedef typename Compute<T>::type CT;
  typedef Mma<T> MS;     // products with S (storage-type operands)
  typedef Mma<CT> MC;    // products with R and Delta (accumulator order)
  typedef AccOrder<CT> AO;
  typedef OutWave<T, D> OW;
  constexpr int KS = MS::KS;
  static_assert(Mma<CT>::KS == KS, "both operand types step alike");
  constexpr int NW = D / 32;
  constexpr int NSD = D / KS, NSC = CHUNK / KS;
  constexpr int EPP = 16 / (int)sizeof(T), PPR = 32 / EPP;   // 16-byte pieces per 32-column row
  __shared__ OW wv[NW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int item = xcd_item(blockIdx.x, n_items);
  const int64_t c = item / Hv;
  const int h = item % Hv, kh = h / G;
  if (c >= seq_off[n_seq]) return;
  int64_t t0;
  int L;
  chunk_span(seq_off, cu, n_seq, c, t0, L);
  const int g = lane >> 4, g4 = 4 * g, c16 = lane & 15;
  const int v0 = 32 * wave;
  const int64_t ch = c * Hv + h, HvD = (int64_t)Hv * D;
  OW& W = wv[wave];

  // ---- the wave's slices of S^T and V into its LDS rows
  {
    const T* Sg = hst + ch * D * D + v0;
#pragma unroll
    for (int j = 0; j < D * PPR / 64; ++j) {
      const int i = lane + 64 * j, r = i / PPR, pc = i % PPR;
      const uint4 x = *reinterpret_cast<const uint4*>(Sg + (int64_t)r * D + pc * EPP);
      word_alias* d = reinterpret_cast<word_alias*>(&W.hs[r][pc * EPP]);
      d[0] = x.x; d[1] = x.y; d[2] = x.z; d[3] = x.w;
    }
    const uint32_t ldb = (uint32_t)(ldv * sizeof(T));
    const auto rs = buffer_of(v + t0 * ldv + (int64_t)h * D + v0, (uint32_t)L * ldb);
#pragma unroll
    for (int j = 0; j < CHUNK * PPR / 64; ++j) {
      const int i = lane + 64 * j, r = i / PPR, pc = i % PPR;
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)r * ldb + 16u * pc, 0, 0);
      word_alias* d = reinterpret_cast<word_alias*>(&W.vs[r][pc * EPP]);
      d[0] = x[0]; d[1] = x[1]; d[2] = x[2]; d[3] = x[3];
    }
  }
  // S^T as B operands: column 16 vt + c16 of the slice, reduction index
  // p KS + (8 g + j | g)
  typename MS::frag sb[2][NSD];
#pragma unroll
  for (int vt = 0; vt < 2; ++vt)
#pragma unroll
    for (int p = 0; p < NSD; ++p) {
      if constexpr (KS == 4) {
        sb[vt][p] = W.hs[p * KS + g][16 * vt + c16];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) sb[vt][p][j] = W.hs[p * KS + 8 * g + j][16 * vt + c16];
      }
    }

  // X S^T for the token rows of X (K or Q), rows past the chunk end zero
  auto rows_times_st = [&](const T* X, int64_t ldx, floatx4 (&acc)[2][4]) __attribute__((always_inline)) {
    const uint32_t ldb = (uint32_t)(ldx * sizeof(T));
    const auto rs = buffer_of(X + t0 * ldx + (int64_t)kh * D, (uint32_t)L * ldb);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      typename MS::frag a[NSD];
#pragma unroll
      for (int p = 0; p < NSD; ++p)
        a[p] = buffer_frag<T>(rs, (uint32_t)(16 * tt + c16) * ldb +
                                      (uint32_t)(p * KS + (KS == 4 ? g : 8 * g)) * sizeof(T));
#pragma unroll
      for (int vt = 0; vt < 2; ++vt) {
        acc[vt][tt] = zero4();
#pragma unroll
        for (int p = 0; p < NSD; ++p) acc[vt][tt] = MS::mma(a[p], sb[vt][p], acc[vt][tt]);
      }
    }
  };
  // A operand of accumulator-order step p from row 16 tt + c16 of a 64 x 64
  // operand stored with its columns in accumulator order
  auto acc_row = [&](const CT* base, int tt, int p) __attribute__((always_inline)) {
    const CT* r = base + (16 * tt + c16) * CHUNK;
    if constexpr (KS == 4) return r[16 * (p >> 2) + g4 + (p & 3)];
    else return *reinterpret_cast<const typename MC::frag*>(r + 32 * p + 8 * g);
  };

  const float4* gam4 = reinterpret_cast<const float4*>(Gw + ch * CHUNK);
  const uint32_t rowb = (uint32_t)(HvD * sizeof(T));
  const uint32_t so = (uint32_t)(((int64_t)g4 * HvD + v0 + c16) * sizeof(T));

  // ---- R = V - diag(Gam) K S^T
  floatx4 R[2][4];
  rows_times_st(k, ldk, R);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const float4 gm = gam4[4 * tt + g];
    const float gv[4] = {gm.x, gm.y, gm.z, gm.w};
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        R[vt][tt][i] = to_f(W.vs[16 * tt + g4 + i][16 * vt + c16]) - gv[i] * R[vt][tt][i];
  }
  // rows past the chunk end fall outside the store buffers: dropped
  const auto rr = buffer_of(Rw + t0 * HvD + (int64_t)h * D, (uint32_t)L * rowb);
#pragma unroll
  for (int vt = 0; vt < 2; ++vt)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store_elem<T>(rr, so + (uint32_t)(16 * tt + i) * rowb + 16u * vt * sizeof(T), R[vt][tt][i]);

  // ---- Delta = M R
  const CT* Mc = Mw + ch * CHUNK * CHUNK;
  floatx4 Dl[2][4];
#pragma unroll
  for (int vt = 0; vt < 2; ++vt) {
    typename MC::frag rb[NSC];
#pragma unroll
    for (int p = 0; p < NSC; ++p) rb[p] = AO::from_acc(R[vt], p);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      Dl[vt][tt] = zero4();
#pragma unroll
      for (int p = 0; p < NSC; ++p) Dl[vt][tt] = MC::mma(acc_row(Mc, tt, p), rb[p], Dl[vt][tt]);
    }
  }
  const auto rd = buffer_of(Dlw + t0 * HvD + (int64_t)h * D, (uint32_t)L * rowb);
#pragma unroll
  for (int vt = 0; vt < 2; ++vt)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store_elem<T>(rd, so + (uint32_t)(16 * tt + i) * rowb + 16u * vt * sizeof(T), Dl[vt][tt][i]);

  if constexpr (WITH_O) {
    // ---- O = diag(Gam) scale Q S^T + P Delta
    floatx4 O[2][4];
    rows_times_st(q, ldq, O);
    const CT* Pc = Pw + ch * CHUNK * CHUNK;
#pragma unroll
    for (int vt = 0; vt < 2; ++vt) {
      typename MC::frag db[NSC];
#pragma unroll
      for (int p = 0; p < NSC; ++p) db[p] = AO::from_acc(Dl[vt], p);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const float4 gm = gam4[4 * tt + g];
        const float gv[4] = {gm.x, gm.y, gm.z, gm.w};
        floatx4 pd = zero4();
#pragma unroll
        for (int p = 0; p < NSC; ++p) pd = MC::mma(acc_row(Pc, tt, p), db[p], pd);
#pragma unroll
        for (int i = 0; i < 4; ++i) O[vt][tt][i] = pd[i] + scale * gv[i] * O[vt][tt][i];
      }
    }
    const auto ro = buffer_of(o + t0 * HvD + (int64_t)h * D, (uint32_t)L * rowb);
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          store_elem<T>(ro, so + (uint32_t)(16 * tt + i) * rowb + 16u * vt * sizeof(T), O[vt][tt][i]);
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_chunk_outputs(const gdn_shape& s, const void* q, const void* k, const void* v,
                                int64_t ldq, int64_t ldk, int64_t ldv, float scale,
                                const int32_t* cu, void* o, void* wsv, hipStream_t st) {
  char* ws = (char*)wsv;
  const ChunkLayout Ly = chunk_layout(s);
  if (Ly.nt_max == 0 || s.total_tokens == 0) return hipSuccess;
  return dispatch_chunk(s, [&](auto cf) {
    using T = typename decltype(cf)::type;
    constexpr int D = decltype(cf)::d;
    typedef typename Compute<T>::type CT;
    const int n_items = (int)(Ly.nt_max * s.hv);
    auto kern = o ? chunk_out_kernel<T, D, true> : chunk_out_kernel<T, D, false>;
    hipLaunchKernelGGL(kern, dim3(n_items), dim3(2 * D), 0, st, (const T*)q, (const T*)k,
                       (const T*)v, ldq, ldk, ldv, cu, (const int32_t*)(ws + Ly.seq_off), s.n_seq,
                       s.hv, s.hv / s.hk, scale, (const CT*)(ws + Ly.mw), (const CT*)(ws + Ly.pw),
                       (const float*)(ws + Ly.gw), (const T*)(ws + Ly.h), (T*)(ws + Ly.rw),
                       (T*)(ws + Ly.dlw), (T*)o, n_items);
    return hipGetLastError();
  });
}

}  // namespace gdn
