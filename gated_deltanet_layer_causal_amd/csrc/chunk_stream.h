// Pieces shared by the sequential chunk kernels (state pass and reverse
// pass): MFMA operands taken straight from accumulator tiles, LDS tiles that
// are filled by direct global -> LDS copies, and range-checked buffer stores.
#pragma once
#include <type_traits>

#include "chunk_common.h"

namespace gdn {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Reduction order of an MFMA step whose B operand comes from accumulator
// tiles x[0..] (rows = reduction index).
//  16-bit operands (32 per step): step p uses tiles 2p and 2p + 1; lane l's
//    slot j holds reduction index 16 (2p + j / 4) + 4 (l / 16) + j % 4.
//  fp32 operands (4 per step): step p holds index 16 (p / 4) + 4 (l / 16) + p % 4.
template <typename CT> struct AccOrder {
  typedef typename Mma<CT>::frag frag;
  __device__ __forceinline__ static frag from_acc(const floatx4* x, int p) {
    frag f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[j] = (CT)x[2 * p][j];
      f[4 + j] = (CT)x[2 * p + 1][j];
    }
    return f;
  }
};
template <> struct AccOrder<float> {
  typedef float frag;
  __device__ __forceinline__ static frag from_acc(const floatx4* x, int p) { return x[p >> 2][p & 3]; }
};

// Piece permutation of LDS row r (RP 16-byte pieces per row): reads by 16
// consecutive rows then touch RP (RP <= 8) or 16 different piece slots.
// With RP <= 8 it depends on r mod RP only, so a direct copy (64 pieces per
// wave = 64 / RP whole rows) needs the same per-lane source offset in every
// copy instruction.
template <int RP> __device__ __forceinline__ int row_swz(int r) {
  if constexpr (RP == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return r & (RP - 1);
}

// An LDS tile of ROWS rows of COLS elements of type E, unpadded, with the
// 16-byte pieces of row r permuted: piece q lives at slot q ^ swz(r), where
// swz = row_swz (SWZ_SHIFT = 0), (r >> SWZ_SHIFT) mod RP, or r mod RP
// (SWZ_SHIFT < 0: 16-byte reads of one piece column by 16 consecutive rows
// hit 16 different slots, which measured free of bank conflicts on gfx950,
// where row_swz with RP = 16 costs four extra cycles per wave read).
template <typename E, int ROWS, int COLS, int SWZ_SHIFT = 0> struct Tile {
  static constexpr int EPP = 16 / sizeof(E);         // elements per piece
  static constexpr int RP = COLS / EPP;              // pieces per row
  static constexpr int PIECES = ROWS * RP;
  static_assert(RP == 4 || RP == 8 || RP == 16, "pieces per row");
  __device__ __forceinline__ static int swz(int r) {
    if constexpr (SWZ_SHIFT == 0) return row_swz<RP>(r);
    else if constexpr (SWZ_SHIFT < 0) return r & (RP - 1);
    else return (r >> SWZ_SHIFT) & (RP - 1);
  }
  // element offset of (r, col)
  __device__ __forceinline__ static int at(int r, int col) {
    return (r * RP + ((col / EPP) ^ swz(r))) * EPP + col % EPP;
  }
  // byte offset, within the source tile, of the piece that LDS slot s holds
  __device__ __forceinline__ static uint32_t source_bytes(int s) {
    const int r = s / RP;
    return (uint32_t)(r * RP + ((s % RP) ^ swz(r))) * 16u;
  }
  // Copy J (64 slots from 64 J) reads source_bytes(64 J + lane) =
  // 1024 J + lane_bytes(J, lane); lane_bytes depends on J only through
  // J mod 4 for RP = 16 and not at all for RP <= 8 (row_swz tiles).
  __device__ __forceinline__ static uint32_t lane_bytes(int J, int lane) {
    return source_bytes(64 * (RP == 16 ? (J & 3) : 0) + lane) - 1024u * (RP == 16 ? (J & 3) : 0);
  }
};

// Transposing LDS read of 16-bit elements: within each group of 16 lanes,
// lane j passes the address of row k0 + j / 4, columns n0 + 4 (j % 4) .. + 3
// of a row-major tile (8-byte aligned), and lane i receives rows k0 .. k0 + 3
// of column n0 + i.  Two such reads give an MFMA operand of 16-bit values
// (eight consecutive reduction indices of one row or column) from a tile
// whose rows are the reduction index.
__device__ __forceinline__ u32x2 lds_read_tr4(const void* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p));
}

// Byte offset in LDS of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Direct copy of one 16-byte piece per lane from a buffer into LDS: the
// wave's 64 pieces land at consecutive 16-byte slots from `lds` (uniform).
// Buffer accesses are range-checked against the descriptor's size on the
// per-lane offset (loads past it read zero, stores past it are dropped).
// Cache policy of a buffer access (the instruction's aux bits on gfx950):
// non-temporal, for data streamed past the caches that no later access of
// the same kernel reads (rows stored for another kernel); and the sc1 scope
// bit, which with it writes through to memory (chosen per pass by
// measurement: the state pass's stores run faster with it, the reverse
// pass's slower).
constexpr int CACHE_NT = 2, CACHE_SC1 = 16;
template <int AUX = 0>
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voff,
                                            uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, soff, 0, AUX);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <typename T>
__device__ __forceinline__ void store_elem(__amdgpu_buffer_rsrc_t rs, uint32_t voff, float x) {
  if constexpr (sizeof(T) == 2) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, from_f<T>(x)), rs, voff, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, x), rs, voff, 0, 0);
  }
}

// 16-byte (16-bit types) or 4-byte (fp32) MFMA operand from a buffer.
template <typename T, int AUX = 0>
__device__ __forceinline__ typename Mma<T>::frag buffer_frag(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  if constexpr (sizeof(T) == 2)
    return __builtin_bit_cast(typename Mma<T>::frag, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, AUX));
  else
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, AUX));
}

// Four consecutive elements of type T as floats / from floats, through a
// range-checked buffer (8 bytes for 16-bit types, 16 for fp32).
template <typename T>
__device__ __forceinline__ floatx4 buffer_load4(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  if constexpr (sizeof(T) == 2) {
    const auto w = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
    return floatx4{lo16<T>(w[0]), hi16<T>(w[0]), lo16<T>(w[1]), hi16<T>(w[1])};
  } else {
    return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  }
}
template <typename T, int AUX = 0>
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t rs, uint32_t off, floatx4 x) {
  if constexpr (sizeof(T) == 2) {
    const u32x2 w = {pack2<T>(x[0], x[1]), pack2<T>(x[2], x[3])};
    __builtin_amdgcn_raw_buffer_store_b64(w, rs, off, 0, AUX);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rs, off, 0, AUX);
  }
}

// Stores of 16 x 16 MFMA accumulator tiles (lane l holds rows 4 (l / 16) + i,
// i < 4, of column l % 16) into a row-major matrix of the storage type, two
// adjacent columns per store: lanes l and l ^ 1 trade half their values
// (one DPP move), so lane l writes rows 4 (l / 16) + 2 (l & 1) + {0, 1} at
// columns (l % 16) & ~1 and + 1.  Half the store instructions of one store
// per element.
// 32-bit words of a paired row piece: two 16-bit elements, or two floats.

template <typename T> struct PairWord { typedef uint32_t type; };
template <> struct PairWord<float> { typedef u32x2 type; };

struct PairStore {
  uint32_t sel0, sel1;
  bool odd;
  __device__ __forceinline__ void init(int lane) {
    odd = lane & 1;
    // byte selectors of v_perm: (own, received) halves in column order
    sel0 = odd ? 0x01000504u : 0x05040100u;
    sel1 = odd ? 0x03020706u : 0x07060302u;
  }
  // byte offset of this lane's first element relative to the tile's
  // (row 0, column 0), for a row stride of ldb bytes
  template <typename T> __device__ __forceinline__ uint32_t lane_off(int lane, uint32_t ldb) const {
    return (uint32_t)(4 * (lane >> 4) + 2 * (lane & 1)) * ldb + (uint32_t)((lane & 15) & ~1) * sizeof(T);
  }
  // the tile's values for this lane's rows r0 = 4 (lane / 16) + 2 (lane % 2)
  // and r0 + 1, columns (lane % 16) & ~1 and the next: lanes 2j and 2j + 1
  // swap the halves of their four rows
  template <typename T>
  __device__ __forceinline__ void pair(floatx4 x, typename PairWord<T>::type& w0,
                                       typename PairWord<T>::type& w1) const {
    if constexpr (sizeof(T) == 2) {
      const uint32_t p01 = pack2<T>(x[0], x[1]), p23 = pack2<T>(x[2], x[3]);
      const uint32_t own = odd ? p23 : p01, send = odd ? p01 : p23;
      const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0xB1, 0xF, 0xF, false);
      w0 = __builtin_amdgcn_perm(recv, own, sel0);
      w1 = __builtin_amdgcn_perm(recv, own, sel1);
    } else {
      const float s0 = odd ? x[0] : x[2], s1 = odd ? x[1] : x[3];
      const float r0 = dpp_f<0xB1>(s0), r1 = dpp_f<0xB1>(s1);
      w0 = u32x2{__float_as_uint(odd ? r0 : x[0]), __float_as_uint(odd ? x[2] : r0)};
      w1 = u32x2{__float_as_uint(odd ? r1 : x[1]), __float_as_uint(odd ? x[3] : r1)};
    }
  }
  template <typename T>
  __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t ldb,
                                        floatx4 x) const {
    typename PairWord<T>::type w0, w1;
    pair<T>(x, w0, w1);
    if constexpr (sizeof(T) == 2) {
      __builtin_amdgcn_raw_buffer_store_b32(w0, rs, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(w1, rs, off + ldb, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b64(w0, rs, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b64(w1, rs, off + ldb, 0, 0);
    }
  }
};

// Output rows of a wave's 16 columns staged through LDS so that they leave
// in 16-byte stores (64 / PPR rows per store instead of the 8 rows of a
// PairStore pair).  Each wave owns its region of rows of 16 elements (SB
// bytes); a wave's LDS accesses complete in order, so no barrier is needed.
// The words go in through inline ds_write2 (two rows SB apart): the
// compiler would otherwise order every LDS store after all direct copies
// into LDS still in flight, not knowing that the region is apart from their
// buffers; the asm's memory clobber keeps the read-back after it.
template <typename T> struct StageRows {
  static constexpr int SB = 16 * (int)sizeof(T);   // bytes per staged row
  static constexpr int PPR = SB / 16;              // 16-byte pieces per row
  static constexpr int RPI = 64 / PPR;             // rows per store
  static_assert(SB / (int)sizeof(typename PairWord<T>::type) == 8, "ds_write2 offset1:8 is one row");
  typedef u32x4 __attribute__((may_alias)) piece;
  // store instructions per lane for n rows
  static constexpr int stores(int n) { return n / RPI; }
  // one 16 x 16 accumulator tile into rows row0.. of the region
  __device__ __forceinline__ static void put(char* region, int row0, const PairStore& ps, int lane,
                                             floatx4 x) {
    typename PairWord<T>::type w0, w1;
    ps.pair<T>(x, w0, w1);
    const uint32_t a = lds_offset(region) + (uint32_t)((row0 + 4 * (lane >> 4) + 2 * (lane & 1)) * SB) +
                       (uint32_t)(((lane & 15) & ~1) * (int)sizeof(T));
    if constexpr (sizeof(T) == 2)
      asm volatile("ds_write2_b32 %0, %1, %2 offset1:8" ::"v"(a), "v"(w0), "v"(w1) : "memory");
    else
      asm volatile("ds_write2_b64 %0, %1, %2 offset1:8" ::"v"(a), "v"(w0), "v"(w1) : "memory");
  }
  // rows [row0, row0 + n) of the region to rows 0.. of the buffer at byte
  // offset col (the wave's columns), row stride ldb bytes; rows outside the
  // buffer's range are dropped
  __device__ __forceinline__ static void flush(const char* region, int row0, int n,
                                               __amdgpu_buffer_rsrc_t rs, uint32_t col,
                                               uint32_t ldb, int lane) {
    const int r = lane / PPR, pc = lane % PPR;
#pragma unroll
    for (int j = 0; j < n / RPI; ++j) {
      const u32x4 v = *reinterpret_cast<const piece*>(region + (row0 + j * RPI + r) * SB + pc * 16);
      __builtin_amdgcn_raw_buffer_store_b128(v, rs, col + (uint32_t)(j * RPI + r) * ldb + (uint32_t)pc * 16u, 0, 0);
    }
  }
  // flush() for a wave with direct copies into other LDS regions in flight:
  // the reads are inline asm, which the compiler does not order after those
  // copies (a plain LDS read would wait for all of them, vmcnt(0)); each
  // asm block waits for its own reads before its outputs are used; AUX is
  // the stores' cache policy
  template <int AUX = 0>
  __device__ __forceinline__ static void flush_async(const char* region, int row0, int n,
                                                     __amdgpu_buffer_rsrc_t rs, uint32_t col,
                                                     uint32_t ldb, int lane) {
    const int r = lane / PPR, pc = lane % PPR;
    const uint32_t a = lds_offset(region) + (uint32_t)((row0 + r) * SB + pc * 16);
    constexpr uint32_t STEP = RPI * SB;   // LDS bytes between consecutive stores' rows
    auto store = [&](const u32x4& v, int j) __attribute__((always_inline)) {
      __builtin_amdgcn_raw_buffer_store_b128(v, rs, col + (uint32_t)(j * RPI + r) * ldb + (uint32_t)pc * 16u, 0, AUX);
    };
#pragma unroll
    for (int j = 0; j < n / RPI; j += 2) {
      u32x4 v0, v1;
      if (j + 1 < n / RPI) {
        asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:%3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(v0), "=&v"(v1)
                     : "v"(a + (uint32_t)j * STEP), "n"(STEP)
                     : "memory");
        store(v0, j);
        store(v1, j + 1);
      } else {
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(v0)
                     : "v"(a + (uint32_t)j * STEP)
                     : "memory");
        store(v0, j);
      }
    }
  }
};

// The same staging for 16-bit types with the region column-major: a lane
// puts its four rows of one column of an accumulator tile as one 8-byte LDS
// write (no trade of halves between lanes), and the mover turns the columns
// back into 16-byte row pieces with transposing reads (ds_read_b64_tr_b16
// gives lane i of a 16-lane group four consecutive columns of row r0 + i,
// lane j passing the address of column c0 + j / 4 at rows r0 + 4 (j % 4)
// .. + 3).  A wave's region holds its 16 columns of NR rows, CS bytes per
// column: NR 16-bit rows padded to CS / 4 = 10 (mod 64) dwords.  The LDS
// bank-conflict counter of a one-wave probe, per 64-lane instruction, for
// the puts (16 columns CS apart, four 8-byte pieces per column) and the
// movers' transposing reads, by CS / 4 mod 64: 2: 0 and 6 cycles; 4: 4 and
// 2; 6: 0 and 4; 8: 12 and 2; 10: 0 and 2; 12: 4 and 2 (the same at every
// base offset tried).
template <int NR> struct StageCols {
  static constexpr int CS = NR * 2 + 4 * ((10 - NR / 2 % 64 + 64) % 64);   // bytes per column
  static constexpr int BYTES = 16 * CS;                                     // per wave
  static_assert(NR % 32 == 0 && CS / 4 % 64 == 10, "padded columns");
  static constexpr int stores(int n) { return n / 32; }   // store instructions per lane for n rows
  // one 16 x 16 accumulator tile (lane l: rows 4 (l / 16) + i of column
  // l % 16) into rows row0.. of the region, as 16-bit E.  A plain store:
  // the waves that put issue no direct copies into LDS, so the compiler
  // needs no wait before it, keeps its own counts of outstanding LDS
  // operations exact (an asm write, which it cannot count, made it wait for
  // more than it had to at every later operand read) and pairs puts into
  // ds_write2_b64.
  template <typename E>
  __device__ __forceinline__ static void put(char* region, int row0, int lane, floatx4 x) {
    static_assert(sizeof(E) == 2, "16-bit staging");
    const u32x2 w = {pack2<E>(x[0], x[1]), pack2<E>(x[2], x[3])};
    *reinterpret_cast<u32x2*>(region + (lane & 15) * CS + (row0 + 4 * (lane >> 4)) * 2) = w;
  }
  // rows [row0, row0 + n) of the region to rows 0.. of the buffer at byte
  // offset col (the wave's columns), row stride ldb bytes, with cache policy
  // AUX; rows outside the buffer's range are dropped.  A store covers 32
  // rows: lane l takes row 16 ((l / 16) % 2) + l % 16 of them, columns
  // 8 (l / 32) .. + 7.  The reads are inline asm that waits for its own
  // results (a plain LDS read would wait for the direct copies in flight).
  template <int AUX = 0>
  __device__ __forceinline__ static void flush_async(const char* region, int row0, int n,
                                                     __amdgpu_buffer_rsrc_t rs, uint32_t col,
                                                     uint32_t ldb, int lane) {
    const int i = lane & 15, q = lane >> 4, rr = 16 * (q & 1) + i, o = q >> 1;
    const uint32_t a = lds_offset(region) + (uint32_t)((8 * o + i / 4) * CS + (row0 + 16 * (q & 1) + 4 * (i % 4)) * 2);
    constexpr uint32_t STEP = 64, HALF = 4 * CS;   // bytes to the next 32 rows; to columns + 4
    auto store = [&](const u32x2& lo, const u32x2& hi, int j) __attribute__((always_inline)) {
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{lo[0], lo[1], hi[0], hi[1]}, rs,
                                             col + (uint32_t)(32 * j + rr) * ldb + (uint32_t)o * 16u, 0, AUX);
    };
#pragma unroll
    for (int j = 0; j < n / 32; j += 2) {
      u32x2 a0, a1, b0, b1;
      if (j + 1 < n / 32) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %4\n\tds_read_b64_tr_b16 %1, %4 offset:%5\n\t"
            "ds_read_b64_tr_b16 %2, %4 offset:%6\n\tds_read_b64_tr_b16 %3, %4 offset:%7\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(a0), "=&v"(a1), "=&v"(b0), "=&v"(b1)
            : "v"(a + (uint32_t)j * STEP), "n"(HALF), "n"(STEP), "n"(STEP + HALF)
            : "memory");
        store(a0, a1, j);
        store(b0, b1, j + 1);
      } else {
        asm volatile("ds_read_b64_tr_b16 %0, %2\n\tds_read_b64_tr_b16 %1, %2 offset:%3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(a0), "=&v"(a1)
                     : "v"(a + (uint32_t)j * STEP), "n"(HALF)
                     : "memory");
        store(a0, a1, j);
      }
    }
  }
  // The rows of both compute waves' regions (wave 1's region BYTES after
  // wave 0's at w0), as whole 2 x 16-column rows: mover m of the two takes
  // rows [row0 + m n / 2, row0 + (m + 1) n / 2) to rows m n / 2.. of the
  // buffer, 16 rows per store, lane l row l % 16 of them and columns
  // 8 (l / 16) .. + 7 (wave (l / 16) / 2's columns), so that each store
  // writes whole lines.
  template <int AUX = 0>
  __device__ __forceinline__ static void flush_pair_async(const char* w0, int row0, int n,
                                                          __amdgpu_buffer_rsrc_t rs, uint32_t ldb,
                                                          int lane, int m) {
    const int i = lane & 15, p = lane >> 4, o = p & 1, h0 = m * (n / 2);
    const uint32_t a = lds_offset(w0) + (uint32_t)((p >> 1) * BYTES + (8 * o + i / 4) * CS +
                                                   (row0 + h0 + 4 * (i % 4)) * 2);
    constexpr uint32_t STEP = 32, HALF = 4 * CS;   // bytes to the next 16 rows; to columns + 4
    auto store = [&](const u32x2& lo, const u32x2& hi, int j) __attribute__((always_inline)) {
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{lo[0], lo[1], hi[0], hi[1]}, rs,
                                             (uint32_t)(h0 + 16 * j + i) * ldb + (uint32_t)p * 16u, 0, AUX);
    };
#pragma unroll
    for (int j = 0; j < n / 32; j += 2) {
      u32x2 a0, a1, b0, b1;
      if (j + 1 < n / 32) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %4\n\tds_read_b64_tr_b16 %1, %4 offset:%5\n\t"
            "ds_read_b64_tr_b16 %2, %4 offset:%6\n\tds_read_b64_tr_b16 %3, %4 offset:%7\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(a0), "=&v"(a1), "=&v"(b0), "=&v"(b1)
            : "v"(a + (uint32_t)j * STEP), "n"(HALF), "n"(STEP), "n"(STEP + HALF)
            : "memory");
        store(a0, a1, j);
        store(b0, b1, j + 1);
      } else {
        asm volatile("ds_read_b64_tr_b16 %0, %2\n\tds_read_b64_tr_b16 %1, %2 offset:%3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(a0), "=&v"(a1)
                     : "v"(a + (uint32_t)j * STEP), "n"(HALF)
                     : "memory");
        store(a0, a1, j);
      }
    }
  }
};

// Wait until at most N vector-memory operations of this wave are outstanding
// (they complete in issue order) and all its LDS operations are done, then
// meet the workgroup at a barrier.  Unlike __syncthreads() it leaves the
// newest N operations (copies still streaming ahead) in flight; as an asm
// statement with a memory clobber no memory access moves across it.
template <int N> __device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Barrier over LDS traffic only: this wave's LDS operations are done, while
// its vector-memory operations (direct copies into LDS among them) stay in
// flight.  For barriers that no copy still in flight needs to cross.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Per-lane source offsets of direct copies: copy J of a tile with RP pieces
// per row reads 1024 J + lane_pattern; the pattern depends only on RP (and on
// J mod 4 when RP = 16).  With copy J = j NW + wave, the RP = 16 pattern of
// copy j is q16[j mod 4], resolved once per wave.
struct CopyLanes {
  uint32_t q16[4], p8, p4;
  __device__ __forceinline__ void init(int lane, int wave, int NW) {
    uint32_t p16[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) p16[a] = Tile<float, 64, 64>::lane_bytes(a, lane);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int a = (m * NW + wave) & 3;
      q16[m] = a == 0 ? p16[0] : a == 1 ? p16[1] : a == 2 ? p16[2] : p16[3];
    }
    p8 = Tile<float, 64, 32>::lane_bytes(0, lane);
    p4 = Tile<float, 64, 16>::lane_bytes(0, lane);
  }
  template <int RP> __device__ __forceinline__ uint32_t get(int j) const {
    return RP == 16 ? q16[j & 3] : RP == 8 ? p8 : p4;
  }
};

// Copy a dense tile (rows contiguous in memory) into LDS with NW waves; the
// per-copy part of the source offset goes into the buffer base, so the range
// check sees only the per-lane offset.
template <typename TT, int NW, typename E>
__device__ __forceinline__ void copy_tile(E* dst, const E* src, const CopyLanes& cl, int wave) {
#pragma unroll
  for (int j = 0; j < TT::PIECES / (64 * NW); ++j) {
    const int J = j * NW + wave;
    const auto rs = buffer_of(reinterpret_cast<const char*>(src) + 1024 * J, 1024);
    copy_to_lds(rs, dst + J * 64 * TT::EPP, cl.template get<TT::RP>(j), 0);
  }
}

}  // namespace gdn
