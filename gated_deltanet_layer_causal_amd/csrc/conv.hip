// Depthwise causal short convolution (4 taps) + SiLU + per-head L2
// normalisation of q and k, forward and backward.
//
// HBM-bound: every x / dy element is read once and every output written once.
// Mapping: a wave owns one run of CONV_TT consecutive tokens; each lane owns 8
// consecutive channels (one 16-byte bf16 vector) and walks the run keeping a
// 3-token sliding window in registers, so x is read once plus a 3-token halo
// per run.  A q or k head of D channels spans D/8 adjacent lanes; its L2 sum
// is a shuffle reduction over those lanes.  Four waves (four runs) share a
// workgroup so the backward's dw partial sums are combined in LDS before
// they go to memory; a second kernel adds the per-workgroup partials in a
// fixed order.
#include "common.h"
#include "launch.h"

namespace gdn {

// Sequence containing token t: largest n with cu[n] <= t (cu non-decreasing).
__device__ __forceinline__ int find_seq(const int32_t* cu, int n_seq, int64_t t) {
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <int D>
__device__ __forceinline__ float group_sum(float x) {
  // lanes of one head: D/8 consecutive lanes
  return lane_group_sum<D / 8>(x);
}

template <typename T>
__device__ __forceinline__ f8 load8_or_zero(const T* p, bool ok) {
  if (ok) return load8(p);
  f8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.v[i] = 0.f;
  return r;
}

template <typename T, int D>
__global__ void __launch_bounds__(256) conv_fwd_kernel(const T* __restrict__ x, int64_t ldx,
                                                       const float* __restrict__ w,
                                                       const int32_t* __restrict__ cu, int n_seq,
                                                       int64_t T_tok, int C, int n_l2, float eps,
                                                       T* __restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = (blockIdx.y * 64 + lane) * 8;
  const bool active = c0 < C;
  const int64_t run = (int64_t)blockIdx.x * CONV_RUNS_PER_BLOCK + wave;
  const int64_t tb = run * CONV_TT;
  if (tb >= T_tok) return;  // whole wave exits together
  const int64_t te = tb + CONV_TT < T_tok ? tb + CONV_TT : T_tok;
  const bool l2 = c0 < n_l2;

  float wr[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) wr[i][j] = active ? w[(int64_t)(c0 + i) * 4 + j] : 0.f;

  int n = find_seq(cu, n_seq, tb);
  int64_t ss = cu[n], se = cu[n + 1];
  f8 x1, x2, x3;  // x[t-1], x[t-2], x[t-3]
  x1 = load8_or_zero(x + (tb - 1) * ldx + c0, active && tb - 1 >= ss);
  x2 = load8_or_zero(x + (tb - 2) * ldx + c0, active && tb - 2 >= ss);
  x3 = load8_or_zero(x + (tb - 3) * ldx + c0, active && tb - 3 >= ss);

  for (int64_t t = tb; t < te; ++t) {
    while (t >= se) {  // next sequence (skips empty ones): restart the window
      ++n;
      ss = cu[n];
      se = cu[n + 1];
#pragma unroll
      for (int i = 0; i < 8; ++i) x1.v[i] = x2.v[i] = x3.v[i] = 0.f;
    }
    f8 x0 = load8_or_zero(x + t * ldx + c0, active);
    f8 a;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float u = wr[i][0] * x3.v[i] + wr[i][1] * x2.v[i] + wr[i][2] * x1.v[i] + wr[i][3] * x0.v[i];
      a.v[i] = u * sigmoidf_(u);
      sq += a.v[i] * a.v[i];
    }
    sq = group_sum<D>(sq);
    if (l2) {
      float r = rsqrtf(sq + eps);
#pragma unroll
      for (int i = 0; i < 8; ++i) a.v[i] *= r;
    }
    if (active) store8(y + t * ldy + c0, a);
    x3 = x2;
    x2 = x1;
    x1 = x0;
  }
}

// du for one token from its window x0..x3 (x[t], x[t-1], x[t-2], x[t-3]) and dy.
template <int D>
__device__ __forceinline__ f8 conv_du(const float (&wr)[8][4], const f8& x0, const f8& x1,
                                      const f8& x2, const f8& x3, const f8& dy, bool l2,
                                      float eps) {
  float u[8], a[8], sg[8];
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u[i] = wr[i][0] * x3.v[i] + wr[i][1] * x2.v[i] + wr[i][2] * x1.v[i] + wr[i][3] * x0.v[i];
    sg[i] = sigmoidf_(u[i]);
    a[i] = u[i] * sg[i];
    sq += a[i] * a[i];
  }
  sq = group_sum<D>(sq);
  float r = rsqrtf(sq + eps);
  float yd = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) yd += a[i] * r * dy.v[i];
  yd = group_sum<D>(yd);
  f8 du;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // L2: y = a r  ->  da = r (dy - y (y . dy));  SiLU': s (1 + u (1 - s))
    float da = l2 ? r * (dy.v[i] - a[i] * r * yd) : dy.v[i];
    du.v[i] = da * sg[i] * (1.f + u[i] * (1.f - sg[i]));
  }
  return du;
}

template <typename T, int D>
__global__ void __launch_bounds__(256) conv_bwd_kernel(
    const T* __restrict__ x, int64_t ldx, const float* __restrict__ w,
    const int32_t* __restrict__ cu, int n_seq, int64_t T_tok, int C, int n_l2, float eps,
    const T* __restrict__ dy, int64_t lddy, T* __restrict__ dx, int64_t lddx,
    float* __restrict__ partials) {
  __shared__ float red[CONV_RUNS_PER_BLOCK][64][33];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = (blockIdx.y * 64 + lane) * 8;
  const bool active = c0 < C;
  const bool l2 = c0 < n_l2;
  const int64_t run = (int64_t)blockIdx.x * CONV_RUNS_PER_BLOCK + wave;
  const int64_t tb = run * CONV_TT;
  const int64_t te = tb + CONV_TT < T_tok ? tb + CONV_TT : T_tok;

  float wr[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) wr[i][j] = active ? w[(int64_t)(c0 + i) * 4 + j] : 0.f;
  float dwa[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) dwa[i][j] = 0.f;

  if (tb < te) {
    int n = find_seq(cu, n_seq, te - 1);
    int64_t ss = cu[n], se = cu[n + 1];
    auto ldx8 = [&](int64_t t, int64_t s0) { return load8_or_zero(x + t * ldx + c0, active && t >= s0); };
    // du at te, te+1, te+2 (the tokens after the run) when in the same sequence
    f8 d1, d2, d3;  // du[s+1], du[s+2], du[s+3]
    {
      f8 h[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        int64_t t = te + j;
        bool in = t < se;  // wave-uniform
        if (in) {
          f8 dyv = load8_or_zero(dy + t * lddy + c0, active);
          h[j] = conv_du<D>(wr, ldx8(t, ss), ldx8(t - 1, ss), ldx8(t - 2, ss), ldx8(t - 3, ss), dyv,
                            l2, eps);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) h[j].v[i] = 0.f;
        }
      }
      d1 = h[0];
      d2 = h[1];
      d3 = h[2];
    }
    // window for s = te-1: x[s], x[s-1], x[s-2], x[s-3]
    int64_t s = te - 1;
    f8 x0 = ldx8(s, ss), x1 = ldx8(s - 1, ss), x2 = ldx8(s - 2, ss), x3 = ldx8(s - 3, ss);
    for (; s >= tb; --s) {
      if (s < ss) {  // moved into an earlier sequence: reset both windows
        while (s < ss) {
          --n;
          ss = cu[n];
          se = cu[n + 1];
        }
        x0 = ldx8(s, ss);
        x1 = ldx8(s - 1, ss);
        x2 = ldx8(s - 2, ss);
        x3 = ldx8(s - 3, ss);
#pragma unroll
        for (int i = 0; i < 8; ++i) d1.v[i] = d2.v[i] = d3.v[i] = 0.f;
      }
      f8 dyv = load8_or_zero(dy + s * lddy + c0, active);
      f8 d0 = conv_du<D>(wr, x0, x1, x2, x3, dyv, l2, eps);
      f8 o;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // x[s] feeds u[s+3-j] through tap j
        o.v[i] = wr[i][3] * d0.v[i] + wr[i][2] * d1.v[i] + wr[i][1] * d2.v[i] + wr[i][0] * d3.v[i];
        dwa[i][0] += d0.v[i] * x3.v[i];
        dwa[i][1] += d0.v[i] * x2.v[i];
        dwa[i][2] += d0.v[i] * x1.v[i];
        dwa[i][3] += d0.v[i] * x0.v[i];
      }
      if (active) store8(dx + s * lddx + c0, o);
      d3 = d2;
      d2 = d1;
      d1 = d0;
      x0 = x1;
      x1 = x2;
      x2 = x3;
      x3 = ldx8(s - 4, ss);
    }
  }
  // combine the four runs of this block in a fixed order
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wave][lane][i * 4 + j] = dwa[i][j];
  __syncthreads();
  if (wave == 0 && active) {
    float* out = partials + (int64_t)blockIdx.x * C * 4 + (int64_t)c0 * 4;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      float acc = red[0][lane][e];
#pragma unroll
      for (int r = 1; r < CONV_RUNS_PER_BLOCK; ++r) acc += red[r][lane][e];
      out[e] = acc;
    }
  }
}

// out[i] = sum over p of partials[p * width + i] in a fixed order: thread
// group j of RED_G adds p = j, j + RED_G, ... (eight loads in flight), then
// the group sums are added in group order.  Columns i < split go to out0[i],
// the rest to out1[i - split].
constexpr int RED_G = 16;

__global__ void __launch_bounds__(64 * RED_G) reduce_partials_kernel(
    const float* __restrict__ partials, int64_t n_part, int64_t width, float* __restrict__ out0,
    int64_t split, float* __restrict__ out1) {
  __shared__ float part[RED_G][64];
  const int col = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * 64 + col;
  float acc = 0.f;
  if (i < width) {
    int64_t p = grp;
    for (; p + 7 * RED_G < n_part; p += 8 * RED_G) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = partials[(p + u * RED_G) * width + i];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; p < n_part; p += RED_G) acc += partials[p * width + i];
  }
  part[grp][col] = acc;
  __syncthreads();
  if (grp == 0 && i < width) {
    float sum = 0.f;
#pragma unroll
    for (int g = 0; g < RED_G; ++g) sum += part[g][col];
    if (i < split) out0[i] = sum;
    else out1[i - split] = sum;
  }
}

hipError_t launch_reduce_partials(const float* partials, int64_t n_part, int64_t width,
                                  float* out0, int64_t split, float* out1, hipStream_t st) {
  if (width > 0)
    hipLaunchKernelGGL(reduce_partials_kernel, dim3((unsigned)((width + 63) / 64)),
                       dim3(64 * RED_G), 0, st, partials, n_part, width, out0, split, out1);
  return hipGetLastError();
}

hipError_t launch_reduce_partials(const float* partials, int64_t n_part, int64_t width,
                                  float* out, hipStream_t st) {
  return launch_reduce_partials(partials, n_part, width, out, width, out, st);
}

template <typename T, int D>
static hipError_t conv_fwd_t(const gdn_shape& s, const void* x, int64_t ldx, const float* w,
                             const int32_t* cu, int l2, float eps, void* y, int64_t ldy,
                             hipStream_t st) {
  const int C = 2 * s.hk * s.dk + s.hv * s.dv;
  const int n_l2 = l2 ? 2 * s.hk * s.dk : 0;
  const int64_t nT = s.total_tokens;
  if (nT == 0) return hipSuccess;
  dim3 grid((unsigned)conv_partials(nT), (C / 8 + 63) / 64);
  hipLaunchKernelGGL((conv_fwd_kernel<T, D>), grid, dim3(256), 0, st, (const T*)x, ldx, w, cu,
                     s.n_seq, nT, C, n_l2, eps, (T*)y, ldy);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t conv_bwd_t(const gdn_shape& s, const void* x, int64_t ldx, const float* w,
                             const int32_t* cu, int l2, float eps, const void* dy, int64_t lddy,
                             void* dx, int64_t lddx, float* dw, float* partials, hipStream_t st) {
  const int C = 2 * s.hk * s.dk + s.hv * s.dv;
  const int n_l2 = l2 ? 2 * s.hk * s.dk : 0;
  const int64_t nT = s.total_tokens;
  const int64_t np = conv_partials(nT);
  if (nT > 0) {
    dim3 grid((unsigned)np, (C / 8 + 63) / 64);
    hipLaunchKernelGGL((conv_bwd_kernel<T, D>), grid, dim3(256), 0, st, (const T*)x, ldx, w, cu,
                       s.n_seq, nT, C, n_l2, eps, (const T*)dy, lddy, (T*)dx, lddx, partials);
  }
  return launch_reduce_partials(partials, np, (int64_t)C * 4, dw, st);
}

hipError_t launch_conv_fwd(const gdn_shape& s, const void* x, int64_t ldx, const float* w,
                           const int32_t* cu, int l2, float eps, void* y, int64_t ldy,
                           hipStream_t st) {
  if (s.dtype == GDN_BF16)
    return s.dk == 128 ? conv_fwd_t<bf16, 128>(s, x, ldx, w, cu, l2, eps, y, ldy, st)
                       : conv_fwd_t<bf16, 32>(s, x, ldx, w, cu, l2, eps, y, ldy, st);
  return s.dk == 128 ? conv_fwd_t<float, 128>(s, x, ldx, w, cu, l2, eps, y, ldy, st)
                     : conv_fwd_t<float, 32>(s, x, ldx, w, cu, l2, eps, y, ldy, st);
}

hipError_t launch_conv_bwd(const gdn_shape& s, const void* x, int64_t ldx, const float* w,
                           const int32_t* cu, int l2, float eps, const void* dy, int64_t lddy,
                           void* dx, int64_t lddx, float* dw, float* partials, hipStream_t st) {
  if (s.dtype == GDN_BF16)
    return s.dk == 128
               ? conv_bwd_t<bf16, 128>(s, x, ldx, w, cu, l2, eps, dy, lddy, dx, lddx, dw, partials, st)
               : conv_bwd_t<bf16, 32>(s, x, ldx, w, cu, l2, eps, dy, lddy, dx, lddx, dw, partials, st);
  return s.dk == 128
             ? conv_bwd_t<float, 128>(s, x, ldx, w, cu, l2, eps, dy, lddy, dx, lddx, dw, partials, st)
             : conv_bwd_t<float, 32>(s, x, ldx, w, cu, l2, eps, dy, lddy, dx, lddx, dw, partials, st);
}

}  // namespace gdn
