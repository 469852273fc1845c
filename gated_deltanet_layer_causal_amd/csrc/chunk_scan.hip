// Segment-parallel state scan: the sequential combine over the segments of
// each sequence.
//
// Over the chunks of one segment the state map is affine,
//   S_end = S_start Phi + B,
// with Phi = A_1 ... A_L the product of the chunks' transitions
// A_c = Gam_L I - K^T diag(Gam) M^T diag(dec) K (d_k x d_k) and B the end
// state the segment reaches from a zero state; the first pass of the scan
// computes both per segment (B from the value rows, Phi from identity rows
// that carry no values).  The state gradient of the reverse pass maps through
// the transposes, dS_start = dS_end Phi^T + dB, with dB the gradient the
// reverse pass over the segment reaches from a zero dS_end.  Forward, this
// kernel chains S_0 = S0 (or 0), S_{s+1} = S_s Phi_s + B_s over the segments
// and stores every S_s (the start state of segment s) and S_final; reverse,
// it chains dS_last = dS_final (or 0), dS_{s-1} = dS_s Phi_s^T + dB_s from the
// last segment back and stores every dS_s (the gradient at the end of
// segment s) and dS0.  Plain fp32 products in a fixed order.

// One block per (sequence, value head, RB state rows) walks the segments in
// order.  Thread (row group, column group) keeps an RPT x 4 tile of the
// state rows in registers; per segment the block stages the state rows and
// Phi (transposed for the reverse, so both directions read Ph[k][4 cg .. +3]
// as one 16-byte piece) in LDS.  The next segment's Phi and B go to
// registers while the current one is multiplied, so the loads' latency stays
// off the chain.
#include "chunk_common.h"

namespace gdn {

template <int D, bool REV>
__global__ void __launch_bounds__(256) span_combine_kernel(
    const int32_t* __restrict__ segb, int Hv, const float* __restrict__ sumf,
    const float* __restrict__ sumr, const float* __restrict__ Sin, float* __restrict__ sspan,
    float* __restrict__ Sout) {
  constexpr int RB = D == 128 ? 16 : 32;   // state rows per block
  constexpr int NRB = D / RB;
  constexpr int CG = D / 4;            // column groups (four columns each)
  constexpr int RG = 256 / CG;         // row groups
  constexpr int RPT = RB / RG;         // rows per thread
  constexpr int PHI4 = D * D / 4 / 256;   // 16-byte pieces of Phi per thread
  constexpr int LDP = D + 4;           // padded LDS row (16-byte aligned)
  static_assert(RPT >= 1 && RB % RG == 0, "tile shape");
  __shared__ __align__(16) float Ph[D][LDP];
  __shared__ __align__(16) float Sx[RB][LDP];
  const int rb = blockIdx.x % NRB, h = (blockIdx.x / NRB) % Hv, n = blockIdx.x / (NRB * Hv);
  const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
  const int c0 = 4 * cg, lr0 = rg * RPT, r0 = rb * RB + lr0;   // this thread's columns and rows
  const int s_lo = segb[n], s_hi = segb[n + 1], ns = s_hi - s_lo;
  typedef float f4 __attribute__((ext_vector_type(4)));
  auto mat = [&](auto* base, int64_t block) __attribute__((always_inline)) {
    return base + block * D * D;   // D x D matrix number `block`
  };
  auto span_at = [&](int it) -> int64_t { return REV ? s_hi - 1 - it : s_lo + it; };

  f4 x[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j)
    x[j] = Sin ? *reinterpret_cast<const f4*>(mat(Sin, (int64_t)n * Hv + h) + (r0 + j) * D + c0)
               : f4{0.f, 0.f, 0.f, 0.f};
  // Phi of segment sp: rows [D, 2 D) of its summary; B (forward): rows [0, D)
  // of the summary, dB (reverse): its own array
  f4 phn[PHI4], bn[RPT];
  auto load_next = [&](int it) __attribute__((always_inline)) {
    const int64_t sh = span_at(it) * Hv + h;
    const float* phi = sumf + sh * 2 * D * D + D * D;
#pragma unroll
    for (int u = 0; u < PHI4; ++u) phn[u] = reinterpret_cast<const f4*>(phi)[tid + 256 * u];
    const float* b = REV ? mat(sumr, sh) : sumf + sh * 2 * D * D;
#pragma unroll
    for (int j = 0; j < RPT; ++j) bn[j] = *reinterpret_cast<const f4*>(b + (r0 + j) * D + c0);
  };
  if (ns > 0) load_next(0);
  for (int it = 0; it < ns; ++it) {
    const int64_t sh = span_at(it) * Hv + h;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      *reinterpret_cast<f4*>(mat(sspan, sh) + (r0 + j) * D + c0) = x[j];
      *reinterpret_cast<f4*>(&Sx[lr0 + j][c0]) = x[j];
    }
#pragma unroll
    for (int u = 0; u < PHI4; ++u) {
      const int e = 4 * (tid + 256 * u), pr = e / D, pc = e % D;   // Phi[pr][pc .. pc + 3]
      if constexpr (REV) {
#pragma unroll
        for (int i = 0; i < 4; ++i) Ph[pc + i][pr] = phn[u][i];
      } else {
        *reinterpret_cast<f4*>(&Ph[pr][pc]) = phn[u];
      }
    }
    f4 acc[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) acc[j] = bn[j];
    __syncthreads();
    if (it + 1 < ns) load_next(it + 1);
    for (int k = 0; k < D; ++k) {
      const f4 p = *reinterpret_cast<const f4*>(&Ph[k][c0]);
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const float a = Sx[lr0 + j][k];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] += a * p[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < RPT; ++j) x[j] = acc[j];
  }
  if (Sout) {
#pragma unroll
    for (int j = 0; j < RPT; ++j)
      *reinterpret_cast<f4*>(mat(Sout, (int64_t)n * Hv + h) + (r0 + j) * D + c0) = x[j];
  }
}

hipError_t launch_span_combine(const gdn_shape& s, const ChunkLayout& Ly, char* ws, bool rev,
                               const float* Sin, float* Sout, hipStream_t st) {
  const int32_t* segb = (const int32_t*)(ws + Ly.segb);
  const float* sumf = (const float*)(ws + Ly.sumf);
  const float* sumr = (const float*)(ws + Ly.sumr);
  float* sspan = (float*)(ws + (rev ? Ly.dse : Ly.sst));
  auto go = [&](auto kern, int D) {
    hipLaunchKernelGGL(kern, dim3((unsigned)(s.n_seq * s.hv * (D / (D == 128 ? 16 : 32)))), dim3(256), 0, st, segb,
                       s.hv, sumf, sumr, Sin, sspan, Sout);
    return hipGetLastError();
  };
  if (s.dk == 128)
    return rev ? go(span_combine_kernel<128, true>, 128) : go(span_combine_kernel<128, false>, 128);
  return rev ? go(span_combine_kernel<32, true>, 32) : go(span_combine_kernel<32, false>, 32);
}

}  // namespace gdn
