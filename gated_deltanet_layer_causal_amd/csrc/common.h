// Device-side helpers shared by the libgdn kernels (gfx950 / CDNA4).
//
// Storage types: bf16 (__bf16) or fp32 for token tensors; all arithmetic is
// fp32.  Matrix products use MFMA: v_mfma_f32_16x16x32_bf16 for bf16 operands
// and v_mfma_f32_16x16x4_f32 for fp32 operands (true fp32 arithmetic).
//
// fp16 operands use v_mfma_f32_16x16x32_f16 (same rate, 11-bit mantissa).
// MFMA 16x16 output layout (all three instructions): lane l of the 64-wide wave
// holds C[4*(l/16) + i][l%16], i = 0..3.  Operand A is read row = l%16,
// operand B column = l%16; the K index a lane supplies is k0 + 8*(l/16) + j
// (bf16, j = 0..7) or k0 + l/16 (fp32).  A and B always use the same K map,
// so the contraction is exact whatever order the hardware sums in.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef _Float16 fp16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 fp16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(fp16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ fp16 from_f<fp16>(float x) { return (fp16)x; }

// Lane swaps within rows of 16 lanes (DPP), and the sum over aligned groups
// of N = 4, 8 or 16 lanes built from them (every lane gets the group sum).
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int N> __device__ __forceinline__ float lane_group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
  x += dpp_f<0xB1>(x);                         // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp_f<0x4E>(x);                         // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (N >= 8) x += dpp_f<0x141>(x);  // row_half_mirror: the other quad of 8
  if constexpr (N >= 16) x += dpp_f<0x140>(x); // row_mirror: the other half of 16
  return x;
}

// sigmoid with the hardware reciprocal (about 1 ulp) instead of an IEEE
// division sequence; e^-x = inf gives rcp(inf) = 0 as it should
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// ---- 8-element vector load/store of a storage type, converted to/from fp32
struct f8 { float v[8]; };

__device__ __forceinline__ f8 load8(const bf16* p) {
  uint4 raw = *reinterpret_cast<const uint4*>(p);
  f8 r;
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.v[2 * i] = __uint_as_float(w[i] << 16);
    r.v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
  return r;
}
__device__ __forceinline__ f8 load8(const fp16* p) {
  fp16x8 raw = *reinterpret_cast<const fp16x8*>(p);
  f8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.v[i] = (float)raw[i];
  return r;
}
__device__ __forceinline__ f8 load8(const float* p) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  f8 r;
  r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
  r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
  return r;
}
// Two floats to bf16 (round to nearest even) in one word, low half first.
// Converted as a pair, so that it is one v_cvt_pk_bf16_f32; two scalar
// conversions cost a conversion each plus a shift and an or.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}
// Two 16-bit storage elements (bf16 or fp16) in one 32-bit word, low half
// first: to floats, and from floats (round to nearest even).
template <typename T> __device__ __forceinline__ float lo16(uint32_t w) {
  if constexpr (__is_same(T, bf16)) return __uint_as_float(w << 16);
  else return (float)__builtin_bit_cast(fp16, (uint16_t)(w & 0xffffu));
}
template <typename T> __device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (__is_same(T, bf16)) return __uint_as_float(w & 0xffff0000u);
  else return (float)__builtin_bit_cast(fp16, (uint16_t)(w >> 16));
}
template <typename T> __device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (__is_same(T, bf16)) {
    return pack2_bf16(a, b);
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, h2{(fp16)a, (fp16)b});
  }
}
__device__ __forceinline__ void store8(bf16* p, const f8& r) {
  uint4 raw;
  raw.x = pack2_bf16(r.v[0], r.v[1]);
  raw.y = pack2_bf16(r.v[2], r.v[3]);
  raw.z = pack2_bf16(r.v[4], r.v[5]);
  raw.w = pack2_bf16(r.v[6], r.v[7]);
  *reinterpret_cast<uint4*>(p) = raw;
}
__device__ __forceinline__ void store8(fp16* p, const f8& r) {
  fp16x8 raw;
#pragma unroll
  for (int i = 0; i < 8; ++i) raw[i] = (fp16)r.v[i];
  *reinterpret_cast<fp16x8*>(p) = raw;
}
__device__ __forceinline__ void store8(float* p, const f8& r) {
  reinterpret_cast<float4*>(p)[0] = make_float4(r.v[0], r.v[1], r.v[2], r.v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(r.v[4], r.v[5], r.v[6], r.v[7]);
}
// 4 consecutive elements (used to write an MFMA column strip transposed)
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  uint2 raw;
  raw.x = pack2_bf16(a, b);
  raw.y = pack2_bf16(c, d);
  *reinterpret_cast<uint2*>(p) = raw;
}
__device__ __forceinline__ void store4(fp16* p, float a, float b, float c, float d) {
  typedef _Float16 fp16x4 __attribute__((ext_vector_type(4)));
  fp16x4 raw = {(fp16)a, (fp16)b, (fp16)c, (fp16)d};
  *reinterpret_cast<fp16x4*>(p) = raw;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// 8 consecutive storage elements (one 16-byte vector; two for fp32).
template <typename T> struct Raw8 { uint4 v[sizeof(T) / 2]; };
template <typename T> __device__ __forceinline__ Raw8<T> ld_raw8(const T* p) {
  Raw8<T> r;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i) r.v[i] = reinterpret_cast<const uint4*>(p)[i];
  return r;
}
template <typename T> __device__ __forceinline__ Raw8<T> zero_raw8() {
  Raw8<T> r;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i) r.v[i] = make_uint4(0, 0, 0, 0);
  return r;
}
template <typename T> __device__ __forceinline__ f8 raw_f8(const Raw8<T>& r) {
  return load8(reinterpret_cast<const T*>(&r.v[0]));
}

// The same 8-element loads and stores with the non-temporal hint, for global
// data that a kernel streams through once.  Only for stores that write whole
// 128-byte lines per wave: partial-line non-temporal stores measured several
// times slower than plain ones.
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ f8 load8_nt(const T* p) {
  Raw8<T> r;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i)
    r.v[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p) + i));
  return raw_f8(r);
}
template <typename T>
__device__ __forceinline__ void store4_nt(T* p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    typedef uint32_t nt_u32x2 __attribute__((ext_vector_type(2)));
    const nt_u32x2 w = {pack2<T>(a, b), pack2<T>(c, d)};
    __builtin_nontemporal_store(w, reinterpret_cast<nt_u32x2*>(p));
  } else {
    __builtin_nontemporal_store(nt_u32x4{__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)},
                                reinterpret_cast<nt_u32x4*>(p));
  }
}
template <typename T>
__device__ __forceinline__ void store16_nt(T* p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x4, v), reinterpret_cast<nt_u32x4*>(p));
}
template <typename T>
__device__ __forceinline__ void store8_nt(T* p, const f8& v) {
  Raw8<T> r;
  store8(reinterpret_cast<T*>(&r.v[0]), v);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i)
    __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x4, r.v[i]), reinterpret_cast<nt_u32x4*>(p) + i);
}

// ---- MFMA operand fragments -------------------------------------------------
// Mma<T>::frag is the per-lane operand of one MFMA step over KS values of K.
template <typename T> struct Mma;

// 16-bit operands (bf16 or fp16): same lane layout, 8 K values per lane.
template <typename E, typename V> struct Mma16 {
  static constexpr int KS = 32;
  typedef V frag;
  __device__ __forceinline__ static floatx4 mma(const frag& a, const frag& b, floatx4 c) {
    if constexpr (sizeof(E) == 2 && __is_same(E, bf16))
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // Element (r, k0 + kk) for this lane's K slots, r fixed, contiguous K.
  template <typename S>
  __device__ __forceinline__ static frag kc(const S* row, int k0, int lane) {
    const S* p = row + k0 + 8 * (lane >> 4);
    if constexpr (__is_same(S, E)) {
      return *reinterpret_cast<const frag*>(p);
    } else {
      f8 v = load8(p);
      frag f;
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = (E)v.v[j];
      return f;
    }
  }
  // K strided by ld: element (k) at col[k * ld].
  template <typename S>
  __device__ __forceinline__ static frag ks(const S* col, int ld, int k0, int lane) {
    const S* p = col + (int64_t)(k0 + 8 * (lane >> 4)) * ld;
    frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (E)to_f(p[(int64_t)j * ld]);
    return f;
  }
};
template <> struct Mma<bf16> : Mma16<bf16, bf16x8> {};
template <> struct Mma<fp16> : Mma16<fp16, fp16x8> {};

template <> struct Mma<float> {
  static constexpr int KS = 4;
  typedef float frag;
  __device__ __forceinline__ static floatx4 mma(const frag& a, const frag& b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  template <typename S>
  __device__ __forceinline__ static frag kc(const S* row, int k0, int lane) {
    return to_f(row[k0 + (lane >> 4)]);
  }
  template <typename S>
  __device__ __forceinline__ static frag ks(const S* col, int ld, int k0, int lane) {
    return to_f(col[(int64_t)(k0 + (lane >> 4)) * ld]);
  }
};

// One 16x16 output tile: acc += A[m0:m0+16, 0:K] * B[0:K, n0:n0+16].
// A is given as row pointers (KC: row-major, K contiguous) or column-strided
// (KS: element (m,k) at A[k*lda + m]); likewise B (KC: element (k,n) at
// B[n*ldb + k]; KS: at B[k*ldb + n]).
template <typename MT, bool A_KC, bool B_KC, typename SA, typename SB>
__device__ __forceinline__ floatx4 tile_mma(floatx4 acc, const SA* A, int lda, const SB* B, int ldb,
                                            int m0, int n0, int K, int lane) {
  typedef Mma<MT> M;
  const int r = lane & 15;
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += M::KS) {
    typename M::frag a, b;
    if constexpr (A_KC) a = M::kc(A + (int64_t)(m0 + r) * lda, k0, lane);
    else a = M::ks(A + (m0 + r), lda, k0, lane);
    if constexpr (B_KC) b = M::kc(B + (int64_t)(n0 + r) * ldb, k0, lane);
    else b = M::ks(B + (n0 + r), ldb, k0, lane);
    acc = M::mma(a, b, acc);
  }
  return acc;
}

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace gdn
