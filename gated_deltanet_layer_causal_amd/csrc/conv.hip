// Depthwise causal short convolution (4 taps) + SiLU + per-head L2
// normalisation of q and k, forward and backward.
//
// HBM-bound: every x / dy element is read once and every output written once.
// Mapping: a wave owns one run of tt consecutive tokens (conv_tt); each lane owns 8
// consecutive channels (one 16-byte bf16 vector).  The run is cut where
// sequences start, and each piece is walked keeping the 4-token window in a
// 4-slot circular buffer, four tokens per loop iteration, so the window never
// moves between registers (token u sits in slot (u - u0) mod 4 for the
// group's first token u0).  Rows come through range-checked buffer accesses
// over the piece's sequence, which read zero before its start (the causal
// zero padding) and drop stores outside it.  A q or k head of D channels
// spans D/8 adjacent lanes; its L2 sum is a lane-group reduction.  Four
// waves (four runs) share a workgroup so the backward's dw partial sums are
// combined in LDS before they go to memory; a second kernel adds the
// per-workgroup partials in a fixed order.
#include <mutex>

#include "chunk_stream.h"

namespace gdn {

// Sequence containing token t: largest n with cu[n] <= t (cu non-decreasing).
// Called with wave-uniform t; the result and the bounds read from cu are
// made uniform explicitly so the row buffers built from them sit in scalar
// registers (a per-lane buffer descriptor turns each access into a loop over
// the distinct descriptors of the wave).
__device__ __forceinline__ int32_t uniform_i32(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int find_seq(const int32_t* cu, int n_seq, int64_t t) {
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)uniform_i32(cu[mid]) <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <int D>
__device__ __forceinline__ float group_sum(float x) {
  // lanes of one head: D/8 consecutive lanes
  return lane_group_sum<D / 8>(x);
}

// Which lanes of this block's channel group (512 channels) normalise: 1 all,
// 0 none, 2 some (the group that straddles the end of the q and k channels).
// Uniform over the block, so each conv kernel runs one of three bodies and the
// v channels (most of them) skip the L2 work instead of computing and
// discarding it.
__device__ __forceinline__ int l2_mode(int C, int n_l2) {
  const int lo = blockIdx.y * 512, hi = lo + 512 < C ? lo + 512 : C;
  return hi <= n_l2 ? 1 : lo >= n_l2 ? 0 : 2;
}

// Eight consecutive elements of row r (relative to the buffer's first row)
// at this lane's channel offset coff (bytes), as stored; zero outside the
// buffer.
template <typename T>
__device__ __forceinline__ Raw8<T> raw_row8(__amdgpu_buffer_rsrc_t rs, int64_t r, uint32_t ldb,
                                            uint32_t coff) {
  const uint32_t off = (uint32_t)r * ldb + coff;   // r < 0 wraps far past the range
  Raw8<T> raw;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i)
    raw.v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u * i, 0, 0));
  return raw;
}
template <typename T>
__device__ __forceinline__ f8 row8(__amdgpu_buffer_rsrc_t rs, int64_t r, uint32_t ldb, uint32_t coff) {
  return raw_f8(raw_row8<T>(rs, r, ldb, coff));
}
template <typename T>
__device__ __forceinline__ void put_row8(__amdgpu_buffer_rsrc_t rs, int64_t r, uint32_t ldb,
                                         uint32_t coff, const f8& v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const uint32_t off = (uint32_t)r * ldb + coff;
  if constexpr (sizeof(T) == 2) {
    const u32x4 w = {pack2<T>(v.v[0], v.v[1]), pack2<T>(v.v[2], v.v[3]),
                     pack2<T>(v.v[4], v.v[5]), pack2<T>(v.v[6], v.v[7])};
    __builtin_amdgcn_raw_buffer_store_b128(w, rs, off, 0, 0);
  } else {
    const u32x4 w0 = {__float_as_uint(v.v[0]), __float_as_uint(v.v[1]), __float_as_uint(v.v[2]),
                      __float_as_uint(v.v[3])};
    const u32x4 w1 = {__float_as_uint(v.v[4]), __float_as_uint(v.v[5]), __float_as_uint(v.v[6]),
                      __float_as_uint(v.v[7])};
    __builtin_amdgcn_raw_buffer_store_b128(w0, rs, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(w1, rs, off + 16u, 0, 0);
  }
}
// Buffer over rows [lo, hi) of a row-major tensor (row stride ldb bytes).
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_of(const T* base, int64_t ld, int64_t lo,
                                                          int64_t hi, uint32_t ldb) {
  return buffer_of(base + lo * ld, (uint32_t)(hi > lo ? hi - lo : 0) * ldb);
}

// HAS_STATE: cs_in [n_seq][3][C] holds the three input rows before each
// sequence (the carried conv state), read where a window reaches before the
// sequence start instead of the zero padding.
// L2M: the block's l2_mode.
template <typename T, int D, bool HAS_STATE, int L2M>
__device__ __forceinline__ void conv_fwd_run(const T* __restrict__ x, int64_t ldx,
                                             const float* __restrict__ w,
                                             const int32_t* __restrict__ cu, int n_seq,
                                             int64_t T_tok, int tt, int C, int n_l2, float eps,
                                             T* __restrict__ y, int64_t ldy,
                                             const T* __restrict__ cs_in) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = (blockIdx.y * 64 + lane) * 8;
  const bool active = c0 < C;
  const int64_t run = (int64_t)blockIdx.x * CONV_RUNS_PER_BLOCK + wave;
  const int64_t tb = run * tt;
  if (tb >= T_tok) return;  // whole wave exits together
  const int64_t te = tb + tt < T_tok ? tb + tt : T_tok;
  const bool l2 = c0 < n_l2;
  // lanes past the channels read zero and store nothing
  const uint32_t coff = active ? (uint32_t)c0 * sizeof(T) : 0x80000000u;
  const uint32_t ldxb = (uint32_t)(ldx * sizeof(T)), ldyb = (uint32_t)(ldy * sizeof(T));

  float wr[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) wr[i][j] = active ? w[(int64_t)(c0 + i) * 4 + j] : 0.f;

  // pieces [a, b) of the run, one per sequence, first to last
  int n = find_seq(cu, n_seq, tb);
  for (int64_t a = tb; a < te;) {
    const int64_t ss = uniform_i32(cu[n]), se = uniform_i32(cu[n + 1]);
    const int64_t b = se < te ? se : te;
    if (b > a) {
      const int64_t lo = a - 3 > ss ? a - 3 : ss;
      const auto rx = rows_of(x, ldx, lo, b, ldxb);
      const auto ry = rows_of(y, ldy, a, b, ldyb);
      // the rows before the piece: x, or (before the sequence start) the
      // carried state rows of sequence n, or the zero padding
      auto prev = [&](int64_t t) __attribute__((always_inline)) -> f8 {
        if constexpr (HAS_STATE) {
          if (t < ss)
            return row8<T>(buffer_of(cs_in + (int64_t)n * 3 * C, 3u * (uint32_t)C * sizeof(T)),
                           t - ss + 3, (uint32_t)C * sizeof(T), coff);
        }
        return row8<T>(rx, t - lo, ldxb, coff);
      };
      f8 xs[4];        // x[u] in slot (u - u0) mod 4
      Raw8<T> px[4];   // x[u + 4] in slot (u - u0) mod 4: rows load a group ahead
      xs[3] = prev(a - 1);
      xs[2] = prev(a - 2);
      xs[1] = prev(a - 3);
#pragma unroll
      for (int m = 0; m < 4; ++m) px[m] = raw_row8<T>(rx, a + m - lo, ldxb, coff);
      auto token = [&](const int m, const int64_t t) __attribute__((always_inline)) {
        xs[m] = raw_f8(px[m]);
        px[m] = raw_row8<T>(rx, t + 4 - lo, ldxb, coff);   // past the piece: zero, unused
        const f8 &x0 = xs[m], &x1 = xs[(m + 3) & 3], &x2 = xs[(m + 2) & 3], &x3 = xs[(m + 1) & 3];
        f8 av;
        float sq = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float u = wr[i][0] * x3.v[i] + wr[i][1] * x2.v[i] + wr[i][2] * x1.v[i] + wr[i][3] * x0.v[i];
          av.v[i] = u * sigmoidf_(u);
          if constexpr (L2M != 0) sq += av.v[i] * av.v[i];
        }
        if constexpr (L2M != 0) {
          sq = group_sum<D>(sq);
          if (L2M == 1 || l2) {
            const float r = rsqrtf(sq + eps);
#pragma unroll
            for (int i = 0; i < 8; ++i) av.v[i] *= r;
          }
        }
        put_row8<T>(ry, t - a, ldyb, coff, av);
      };
      // whole groups of four with no per-token test (so the loads stay a
      // group ahead across iterations), then the last one to three tokens
      int64_t u0 = a;
      for (; u0 + 4 <= b; u0 += 4) {
#pragma unroll
        for (int m = 0; m < 4; ++m) token(m, u0 + m);
      }
#pragma unroll
      for (int m = 0; m < 3; ++m)
        if (u0 + m < b) token(m, u0 + m);
    }
    a = b > a ? b : a;
    ++n;
  }
}

template <typename T, int D, bool HAS_STATE>
__global__ void __launch_bounds__(64 * CONV_RUNS_PER_BLOCK) conv_fwd_kernel(const T* __restrict__ x, int64_t ldx,
                                                       const float* __restrict__ w,
                                                       const int32_t* __restrict__ cu, int n_seq,
                                                       int64_t T_tok, int tt, int C, int n_l2, float eps,
                                                       T* __restrict__ y, int64_t ldy,
                                                       const T* __restrict__ cs_in) {
  const int mode = l2_mode(C, n_l2);
  if (mode == 1)
    conv_fwd_run<T, D, HAS_STATE, 1>(x, ldx, w, cu, n_seq, T_tok, tt, C, n_l2, eps, y, ldy, cs_in);
  else if (mode == 0)
    conv_fwd_run<T, D, HAS_STATE, 0>(x, ldx, w, cu, n_seq, T_tok, tt, C, n_l2, eps, y, ldy, cs_in);
  else
    conv_fwd_run<T, D, HAS_STATE, 2>(x, ldx, w, cu, n_seq, T_tok, tt, C, n_l2, eps, y, ldy, cs_in);
}

// du for one token from its window x0..x3 (x[t], x[t-1], x[t-2], x[t-3]) and
// dy.  With a = SiLU(u), s = sigmoid(u) and, on normalising lanes, y = a r
// with r = (|a|^2 + eps)^(-1/2) over the head:
//   da = r dy - a r^3 (a . dy),   du = da SiLU'(u),   SiLU'(u) = s + a (1 - s).
// L2M as l2_mode; with L2M = 2 the lanes that do not normalise take r = 1
// and r^3 (a . dy) = 0, so one formula serves every lane.
template <int D, int L2M>
__device__ __forceinline__ f8 conv_du(const float (&wr)[8][4], const f8& x0, const f8& x1,
                                      const f8& x2, const f8& x3, const f8& dy, bool l2,
                                      float eps) {
  float a[8], sg[8];
  float sq = 0.f, sd = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float u = wr[i][0] * x3.v[i] + wr[i][1] * x2.v[i] + wr[i][2] * x1.v[i] + wr[i][3] * x0.v[i];
    sg[i] = sigmoidf_(u);
    a[i] = u * sg[i];
    if constexpr (L2M != 0) {
      sq += a[i] * a[i];
      sd += a[i] * dy.v[i];
    }
  }
  float r = 1.f, c = 0.f;
  if constexpr (L2M != 0) {
    sq = group_sum<D>(sq);
    sd = group_sum<D>(sd);
    r = rsqrtf(sq + eps);
    c = r * r * r * sd;
    if constexpr (L2M == 2) {
      r = l2 ? r : 1.f;
      c = l2 ? c : 0.f;
    }
  }
  f8 du;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float da = L2M != 0 ? fmaf(-a[i], c, r * dy.v[i]) : dy.v[i];
    du.v[i] = da * fmaf(a[i], 1.f - sg[i], sg[i]);
  }
  return du;
}

// HAS_STATE: windows reaching before a sequence start read the carried state
// rows cs_in [n_seq][3][C], and dcs_out [n_seq][3][C] (nullable), the
// gradient of the final state (the last three input rows of each sequence),
// adds to dx of those rows.  The gradient of cs_in itself comes from
// conv_state_dgrad_kernel.
typedef float ConvRed[CONV_RUNS_PER_BLOCK][64][33];
template <typename T, int D, bool HAS_STATE, int L2M>
__device__ __forceinline__ void conv_bwd_run(
    const T* __restrict__ x, int64_t ldx, const float* __restrict__ w,
    const int32_t* __restrict__ cu, int n_seq, int64_t T_tok, int tt, int C, int n_l2, float eps,
    const T* __restrict__ dy, int64_t lddy, T* __restrict__ dx, int64_t lddx,
    float* __restrict__ partials, const T* __restrict__ cs_in, const T* __restrict__ dcs_out,
    ConvRed& red) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = (blockIdx.y * 64 + lane) * 8;
  const bool active = c0 < C;
  const bool l2 = c0 < n_l2;
  const int64_t run = (int64_t)blockIdx.x * CONV_RUNS_PER_BLOCK + wave;
  const int64_t tb = run * tt;
  const int64_t te = tb + tt < T_tok ? tb + tt : T_tok;
  // lanes past the channels read zero and store nothing
  const uint32_t coff = active ? (uint32_t)c0 * sizeof(T) : 0x80000000u;
  const uint32_t ldxb = (uint32_t)(ldx * sizeof(T)), ldyb = (uint32_t)(lddy * sizeof(T));
  const uint32_t ldob = (uint32_t)(lddx * sizeof(T));

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
    // pieces [a, b) of the run, one per sequence, last to first; each is
    // walked from its end
    int n = find_seq(cu, n_seq, te - 1);
    for (int64_t b = te; b > tb;) {
      const int64_t ss = uniform_i32(cu[n]), se = uniform_i32(cu[n + 1]);
      const int64_t a = ss > tb ? ss : tb;
      if (b > a) {
        // x rows [max(a - 3, ss), min(b + 3, se)); dy rows [a, min(b + 3, se))
        const int64_t lo = a - 3 > ss ? a - 3 : ss, hi = b + 3 < se ? b + 3 : se;
        const auto rx = rows_of(x, ldx, lo, hi, ldxb);
        const auto ry = rows_of(dy, lddy, a, hi, ldyb);
        const auto ro = rows_of(dx, lddx, a, b, ldob);
        const uint32_t ldsb = (uint32_t)C * sizeof(T);
        // x rows, or (before the sequence start) the carried state rows
        auto xraw = [&](int64_t t) __attribute__((always_inline)) -> Raw8<T> {
          if constexpr (HAS_STATE) {
            if (t < ss) return raw_row8<T>(buffer_of(cs_in + (int64_t)n * 3 * C, 3u * ldsb), t - ss + 3, ldsb, coff);
          }
          return raw_row8<T>(rx, t - lo, ldxb, coff);
        };
        auto xr = [&](int64_t t) __attribute__((always_inline)) { return raw_f8(xraw(t)); };
        // du at b, b + 1, b + 2 (the tokens after the piece) in slots 3, 2, 1
        f8 xs[4], ds[4];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int64_t t = b + j;
          if (t < se) {   // wave-uniform
            ds[3 - j] = conv_du<D, L2M>(wr, xr(t), xr(t - 1), xr(t - 2), xr(t - 3),
                                   row8<T>(ry, t - a, ldyb, coff), l2, eps);
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) ds[3 - j].v[i] = 0.f;
          }
        }
        // x[b - 1 - j] in slot j (u0 = b - 1; token u in slot (u0 - u) mod 4);
        // the rows of the next group (x[u - 4], dy[u]) load a group ahead
        // into raw slots; rows before the piece read zero and go unused
        Raw8<T> px[4], pd[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xs[j] = xr(b - 1 - j);
          px[j] = xraw(b - 5 - j);
          pd[j] = raw_row8<T>(ry, b - 1 - j - a, ldyb, coff);
        }
        auto token = [&](const int m, const int64_t s) __attribute__((always_inline)) {
          const f8 &x0 = xs[m], &x1 = xs[(m + 1) & 3], &x2 = xs[(m + 2) & 3], &x3 = xs[(m + 3) & 3];
          const f8 dyv = raw_f8(pd[m]);
          pd[m] = raw_row8<T>(ry, s - 4 - a, ldyb, coff);
          const f8 d0 = conv_du<D, L2M>(wr, x0, x1, x2, x3, dyv, l2, eps);
          const f8 &d1 = ds[(m + 3) & 3], &d2 = ds[(m + 2) & 3], &d3 = ds[(m + 1) & 3];
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
          if constexpr (HAS_STATE) {
            // the last three rows also feed the final state
            if (dcs_out && s >= se - 3) {
              const f8 gf = row8<T>(buffer_of(dcs_out + (int64_t)n * 3 * C, 3u * ldsb), s - se + 3, ldsb, coff);
#pragma unroll
              for (int i = 0; i < 8; ++i) o.v[i] += gf.v[i];
            }
          }
          put_row8<T>(ro, s - a, ldob, coff, o);
          ds[m] = d0;
          xs[m] = raw_f8(px[m]);
          px[m] = xraw(s - 8);
        };
        // whole groups of four with no per-token test, then the last one to
        // three tokens
        int64_t u0 = b - 1;
        for (; u0 - 3 >= a; u0 -= 4) {
#pragma unroll
          for (int m = 0; m < 4; ++m) token(m, u0 - m);
        }
#pragma unroll
        for (int m = 0; m < 3; ++m)
          if (u0 - m >= a) token(m, u0 - m);
      }
      b = a;
      --n;
    }
  }
  // combine the runs of this block in a fixed order
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

template <typename T, int D, bool HAS_STATE>
__global__ void __launch_bounds__(64 * CONV_RUNS_PER_BLOCK) conv_bwd_kernel(
    const T* __restrict__ x, int64_t ldx, const float* __restrict__ w,
    const int32_t* __restrict__ cu, int n_seq, int64_t T_tok, int tt, int C, int n_l2, float eps,
    const T* __restrict__ dy, int64_t lddy, T* __restrict__ dx, int64_t lddx,
    float* __restrict__ partials, const T* __restrict__ cs_in, const T* __restrict__ dcs_out) {
  __shared__ ConvRed red;
  const int mode = l2_mode(C, n_l2);
  if (mode == 1)
    conv_bwd_run<T, D, HAS_STATE, 1>(x, ldx, w, cu, n_seq, T_tok, tt, C, n_l2, eps, dy, lddy, dx,
                                     lddx, partials, cs_in, dcs_out, red);
  else if (mode == 0)
    conv_bwd_run<T, D, HAS_STATE, 0>(x, ldx, w, cu, n_seq, T_tok, tt, C, n_l2, eps, dy, lddy, dx,
                                     lddx, partials, cs_in, dcs_out, red);
  else
    conv_bwd_run<T, D, HAS_STATE, 2>(x, ldx, w, cu, n_seq, T_tok, tt, C, n_l2, eps, dy, lddy, dx,
                                     lddx, partials, cs_in, dcs_out, red);
}

// The final conv state: cs_out[n][r] = the input row at position
// cu[n + 1] - 3 + r, from x, or from cs_in (zeros when null) where that
// position precedes the sequence start.  One wave per (sequence, row, 512
// channels), 16-byte copies.
template <typename T>
__global__ void __launch_bounds__(64) conv_state_out_kernel(const T* __restrict__ x, int64_t ldx,
                                                            const int32_t* __restrict__ cu, int C,
                                                            const T* __restrict__ cs_in,
                                                            T* __restrict__ cs_out) {
  const int n = blockIdx.x, r = blockIdx.y, c0 = (blockIdx.z * 64 + threadIdx.x) * 8;
  if (c0 >= C) return;
  const int64_t ss = cu[n], se = cu[n + 1], t = se - 3 + r;
  Raw8<T> v;
  if (t >= ss) v = ld_raw8(x + t * ldx + c0);
  else if (cs_in) v = ld_raw8(cs_in + ((int64_t)n * 3 + (t - ss + 3)) * C + c0);
  else v = zero_raw8<T>();
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i)
    reinterpret_cast<uint4*>(cs_out + ((int64_t)n * 3 + r) * C + c0)[i] = v.v[i];
}

// Gradient of the carried state: input position p = cu[n] - 3 + r feeds u at
// tokens cu[n] + r - j through tap j, and the final state when the sequence
// is shorter than 3 - r.  du of the first three tokens is recomputed here from
// their windows (state rows included) and dy.  One wave per (sequence, 512
// channels), as the conv kernels lay out lanes.
template <typename T, int D>
__global__ void __launch_bounds__(64) conv_state_dgrad_kernel(
    const T* __restrict__ x, int64_t ldx, const float* __restrict__ w,
    const int32_t* __restrict__ cu, int C, int n_l2, float eps, const T* __restrict__ cs_in,
    const T* __restrict__ dy, int64_t lddy, const T* __restrict__ dcs_out, T* __restrict__ dcs_in) {
  const int lane = threadIdx.x, n = blockIdx.x;
  const int c0 = (blockIdx.y * 64 + lane) * 8;
  const bool active = c0 < C, l2 = c0 < n_l2;
  const uint32_t coff = active ? (uint32_t)c0 * sizeof(T) : 0x80000000u;
  const uint32_t ldxb = (uint32_t)(ldx * sizeof(T)), ldyb = (uint32_t)(lddy * sizeof(T));
  const uint32_t ldsb = (uint32_t)C * sizeof(T);
  const int64_t ss = uniform_i32(cu[n]), se = uniform_i32(cu[n + 1]);
  const int64_t L = se - ss;
  float wr[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) wr[i][j] = active ? w[(int64_t)(c0 + i) * 4 + j] : 0.f;
  const auto rx = rows_of(x, ldx, ss, se, ldxb);
  const auto ry = rows_of(dy, lddy, ss, se, ldyb);
  const auto rst = buffer_of(cs_in + (int64_t)n * 3 * C, cs_in ? 3u * ldsb : 0u);
  auto xrow = [&](int64_t t) __attribute__((always_inline)) -> f8 {
    return t >= ss ? row8<T>(rx, t - ss, ldxb, coff) : row8<T>(rst, t - ss + 3, ldsb, coff);
  };
  f8 du[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int64_t t = ss + k;
    if (k < L) {   // wave-uniform
      du[k] = conv_du<D, 2>(wr, xrow(t), xrow(t - 1), xrow(t - 2), xrow(t - 3), row8<T>(ry, t - ss, ldyb, coff),
                         l2, eps);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) du[k].v[i] = 0.f;
    }
  }
  const auto rdo = buffer_of(dcs_out + (int64_t)n * 3 * C, dcs_out ? 3u * ldsb : 0u);
  const auto rdi = buffer_of(dcs_in + (int64_t)n * 3 * C, 3u * ldsb);
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    f8 gsum;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j <= r; ++j) acc += wr[i][j] * du[r - j].v[i];
      gsum.v[i] = acc;
    }
    if (r >= L) {   // the position also sits in the final state
      const f8 gf = row8<T>(rdo, r - L, ldsb, coff);
#pragma unroll
      for (int i = 0; i < 8; ++i) gsum.v[i] += gf.v[i];
    }
    put_row8<T>(rdi, r, ldsb, coff, gsum);
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
                             const void* cs_in, void* cs_out, hipStream_t st) {
  const int C = 2 * s.hk * s.dk + s.hv * s.dv;
  const int n_l2 = l2 ? 2 * s.hk * s.dk : 0;
  const int64_t nT = s.total_tokens;
  if (nT > 0) {
    const int tt = conv_tt(nT, C);
    dim3 grid((unsigned)conv_partials(nT, tt), (C / 8 + 63) / 64);
    auto kern = cs_in ? conv_fwd_kernel<T, D, true> : conv_fwd_kernel<T, D, false>;
    hipLaunchKernelGGL(kern, grid, dim3(64 * CONV_RUNS_PER_BLOCK), 0, st, (const T*)x, ldx, w, cu,
                       s.n_seq, nT, tt, C, n_l2, eps, (T*)y, ldy, (const T*)cs_in);
  }
  if (cs_out)
    hipLaunchKernelGGL(conv_state_out_kernel<T>, dim3(s.n_seq, 3, (C / 8 + 63) / 64), dim3(64), 0,
                       st, (const T*)x, ldx, cu, C, (const T*)cs_in, (T*)cs_out);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t conv_bwd_t(const gdn_shape& s, const void* x, int64_t ldx, const float* w,
                             const int32_t* cu, int l2, float eps, const void* dy, int64_t lddy,
                             void* dx, int64_t lddx, float* dw, float* partials,
                             const void* cs_in, const void* dcs_out, void* dcs_in,
                             hipStream_t st) {
  const int C = 2 * s.hk * s.dk + s.hv * s.dv;
  const int n_l2 = l2 ? 2 * s.hk * s.dk : 0;
  const int64_t nT = s.total_tokens;
  const int tt = conv_tt(nT, C);
  const int64_t np = conv_partials(nT, tt);
  const bool stateful = cs_in || dcs_out || dcs_in;
  if (nT > 0) {
    dim3 grid((unsigned)np, (C / 8 + 63) / 64);
    auto kern = stateful ? conv_bwd_kernel<T, D, true> : conv_bwd_kernel<T, D, false>;
    hipLaunchKernelGGL(kern, grid, dim3(64 * CONV_RUNS_PER_BLOCK), 0, st, (const T*)x, ldx, w, cu,
                       s.n_seq, nT, tt, C, n_l2, eps, (const T*)dy, lddy, (T*)dx, lddx, partials,
                       (const T*)cs_in, (const T*)dcs_out);
  }
  if (dcs_in)
    hipLaunchKernelGGL((conv_state_dgrad_kernel<T, D>), dim3(s.n_seq, (C / 8 + 63) / 64), dim3(64), 0,
                       st, (const T*)x, ldx, w, cu, C, n_l2, eps, (const T*)cs_in, (const T*)dy,
                       lddy, (const T*)dcs_out, (T*)dcs_in);
  return launch_reduce_partials(partials, np, (int64_t)C * 4, dw, st);
}

hipError_t launch_conv_fwd(const gdn_shape& s, const void* x, int64_t ldx, const float* w,
                           const int32_t* cu, int l2, float eps, void* y, int64_t ldy,
                           const void* cs_in, void* cs_out, hipStream_t st) {
  if (s.dtype == GDN_FP16)
    return s.dk == 128 ? conv_fwd_t<fp16, 128>(s, x, ldx, w, cu, l2, eps, y, ldy, cs_in, cs_out, st)
                       : conv_fwd_t<fp16, 32>(s, x, ldx, w, cu, l2, eps, y, ldy, cs_in, cs_out, st);
  if (s.dtype == GDN_BF16)
    return s.dk == 128 ? conv_fwd_t<bf16, 128>(s, x, ldx, w, cu, l2, eps, y, ldy, cs_in, cs_out, st)
                       : conv_fwd_t<bf16, 32>(s, x, ldx, w, cu, l2, eps, y, ldy, cs_in, cs_out, st);
  return s.dk == 128 ? conv_fwd_t<float, 128>(s, x, ldx, w, cu, l2, eps, y, ldy, cs_in, cs_out, st)
                     : conv_fwd_t<float, 32>(s, x, ldx, w, cu, l2, eps, y, ldy, cs_in, cs_out, st);
}

hipError_t launch_conv_bwd(const gdn_shape& s, const void* x, int64_t ldx, const float* w,
                           const int32_t* cu, int l2, float eps, const void* dy, int64_t lddy,
                           void* dx, int64_t lddx, float* dw, float* partials, const void* cs_in,
                           const void* dcs_out, void* dcs_in, hipStream_t st) {
  if (s.dtype == GDN_FP16)
    return s.dk == 128 ? conv_bwd_t<fp16, 128>(s, x, ldx, w, cu, l2, eps, dy, lddy, dx, lddx, dw,
                                                partials, cs_in, dcs_out, dcs_in, st)
                       : conv_bwd_t<fp16, 32>(s, x, ldx, w, cu, l2, eps, dy, lddy, dx, lddx, dw,
                                               partials, cs_in, dcs_out, dcs_in, st);
  if (s.dtype == GDN_BF16)
    return s.dk == 128 ? conv_bwd_t<bf16, 128>(s, x, ldx, w, cu, l2, eps, dy, lddy, dx, lddx, dw,
                                                partials, cs_in, dcs_out, dcs_in, st)
                       : conv_bwd_t<bf16, 32>(s, x, ldx, w, cu, l2, eps, dy, lddy, dx, lddx, dw,
                                               partials, cs_in, dcs_out, dcs_in, st);
  return s.dk == 128 ? conv_bwd_t<float, 128>(s, x, ldx, w, cu, l2, eps, dy, lddy, dx, lddx, dw,
                                               partials, cs_in, dcs_out, dcs_in, st)
                     : conv_bwd_t<float, 32>(s, x, ldx, w, cu, l2, eps, dy, lddy, dx, lddx, dw,
                                              partials, cs_in, dcs_out, dcs_in, st);
}

// ---- the conv backward without a workspace argument -------------------------
// Its per-block dw partials go to `scratch`, a device array of this module
// (each GPU holds its own copy for the life of the process).  In host code
// the array's name stands for a host-side shadow, not a device address: the
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that pointer is handed to the kernels.  The
// backward kernel writes every partial that the reduction reads, so nothing
// needs clearing between calls.
static __device__ __align__(256) float scratch[CONV_BWD_NOALLOC_MAX_BYTES / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
float* scratch_dev[kMaxDevices] = {};

// This device's copy of `scratch`, looked up on the first call on the device.
hipError_t scratch_of_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = scratch_dev[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_conv_bwd_noalloc(const gdn_shape& s, const void* x, int64_t ldx, const float* w,
                                   const int32_t* cu, int l2, float eps, const void* dy,
                                   int64_t lddy, void* dx, int64_t lddx, float* dw,
                                   hipStream_t st) {
  float* partials = nullptr;
  const hipError_t e = scratch_of_current_device(&partials);
  if (e != hipSuccess) return e;
  return launch_conv_bwd(s, x, ldx, w, cu, l2, eps, dy, lddy, dx, lddx, dw, partials, nullptr,
                         nullptr, nullptr, st);
}

}  // namespace gdn
