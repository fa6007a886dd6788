// Device helpers shared by the matrix-core kernels: raw buffer loads whose
// out-of-range reads return zero, and the decode of packed CQ codes into
// 16-bit values through per-(row, group) tables of level * norm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "cq_internal.h"

namespace cqdev {

// Raw buffer resource over nbytes at base: loads at offsets >= nbytes return
// zero, which is how rows past the end of Xr and W read as zeros.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(nbytes),
                                           0x00020000);  // word 3: raw, 32-bit data format
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// N consecutive dwords at byte offset off, in as few loads as possible, with
// cache policy POLICY (0, or cq::kStreamLoad for data read once).
template <int N, int POLICY = 0>
__device__ inline void load_dwords(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t *d) {
#pragma unroll
  for (int q = 0; q + 4 <= N; q += 4) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * q, 0, POLICY);
    d[q] = v.x, d[q + 1] = v.y, d[q + 2] = v.z, d[q + 3] = v.w;
  }
  constexpr int q = N / 4 * 4;
  if constexpr (N - q == 3) {
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, off + 4 * q, 0, POLICY);
    d[q] = v.x, d[q + 1] = v.y, d[q + 2] = v.z;
  } else if constexpr (N - q == 2) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off + 4 * q, 0, POLICY);
    d[q] = v.x, d[q + 1] = v.y;
  } else if constexpr (N - q == 1) {
    d[q] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * q, 0, POLICY);
  }
}

// Two floats rounded to nearest-even 16-bit values of type T (__bf16 or
// _Float16), a in the low half.
template <typename T>
__device__ inline uint32_t pack2(float a, float b) {
  typedef T t2 __attribute__((ext_vector_type(2)));
  const t2 v = {static_cast<T>(a), static_cast<T>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ inline uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) { return __builtin_amdgcn_perm(hi, lo, sel); }

// b where mask bits are set, a elsewhere (one v_bfi_b32).
__device__ inline uint32_t select(uint32_t mask, uint32_t b, uint32_t a) { return (b & mask) | (a & ~mask); }

// Decoded values of one (row, group): T[c] = T16(level[c] * norm), rounded
// to nearest even, as the low and high byte planes of the 16-bit values (4
// entries per dword).
template <int SB, typename T16>
struct Table {
  static constexpr int L = 1 << SB;
  uint32_t lo[L / 4 > 0 ? L / 4 : 1], hi[L / 4 > 0 ? L / 4 : 1];
  uint32_t pair[2];  // SB == 2: T[0] | T[1] << 16, T[2] | T[3] << 16

  // Byte planes as cq::MmaLevels holds them: d[k] = low bytes, d[L/4 + k] =
  // high bytes of entries 4k..4k+3.
  __device__ void load(const uint32_t *d) {
#pragma unroll
    for (int k = 0; k < L / 4; ++k) lo[k] = d[k], hi[k] = d[L / 4 + k];
  }
  __device__ void build(const cq::CodeLevels &lev, float n) {
    if constexpr (SB == 2) {
      pair[0] = pack2<T16>(lev.v[0] * n, lev.v[1] * n);
      pair[1] = pack2<T16>(lev.v[2] * n, lev.v[3] * n);
    } else {
#pragma unroll
      for (int k = 0; k < L / 4; ++k) {
        const uint32_t p0 = pack2<T16>(lev.v[4 * k] * n, lev.v[4 * k + 1] * n);
        const uint32_t p1 = pack2<T16>(lev.v[4 * k + 2] * n, lev.v[4 * k + 3] * n);
        lo[k] = perm(p1, p0, 0x06040200u);
        hi[k] = perm(p1, p0, 0x07050301u);
      }
    }
  }
};

// 4-bit: the 8 codes of a dword -> 4 dwords of 16-bit pairs, codes in order.
template <typename T16>
__device__ inline void decode4(const Table<4, T16> &t, uint32_t d, uint32_t *o) {
  // Even codes (low nibbles) and odd codes (high nibbles), one per byte: the
  // low three bits select within an 8-entry half, bit 3 selects the half.
  const uint32_t se = d & 0x07070707u, so = (d >> 4) & 0x07070707u;
  const uint32_t me = ((d >> 3) & 0x01010101u) * 0xffu, mo = ((d >> 7) & 0x01010101u) * 0xffu;
  const uint32_t el = select(me, perm(t.lo[3], t.lo[2], se), perm(t.lo[1], t.lo[0], se));
  const uint32_t eh = select(me, perm(t.hi[3], t.hi[2], se), perm(t.hi[1], t.hi[0], se));
  const uint32_t ol = select(mo, perm(t.lo[3], t.lo[2], so), perm(t.lo[1], t.lo[0], so));
  const uint32_t oh = select(mo, perm(t.hi[3], t.hi[2], so), perm(t.hi[1], t.hi[0], so));
  // low bytes of codes 0,1,2,3 and high bytes of codes 0,1,2,3; then 4..7
  const uint32_t l03 = perm(ol, el, 0x05010400u), h03 = perm(oh, eh, 0x05010400u);
  const uint32_t l47 = perm(ol, el, 0x07030602u), h47 = perm(oh, eh, 0x07030602u);
  o[0] = perm(h03, l03, 0x05010400u);
  o[1] = perm(h03, l03, 0x07030602u);
  o[2] = perm(h47, l47, 0x05010400u);
  o[3] = perm(h47, l47, 0x07030602u);
}

// 3-bit: 8 codes in the low 24 bits of b (higher bits ignored) -> 4 dwords of
// 16-bit pairs.
template <typename T16>
__device__ inline void decode3(const Table<3, T16> &t, uint32_t b, uint32_t *o) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // four codes in bits 0..11 of f, spread to one per byte: the low 16 bits
    // in both halves, each half shifted by its own amount (packed 16-bit
    // shifts), then the bytes that hold codes 0, 1, 2, 3 in their low bits
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    const uint32_t f = b >> (12 * h);
    const u16x2 ff = __builtin_bit_cast(u16x2, perm(f, f, 0x01000100u));
    const uint32_t t02 = __builtin_bit_cast(uint32_t, ff >> u16x2{0, 6});  // codes 0 and 2 at bits 0 and 16
    const uint32_t t13 = __builtin_bit_cast(uint32_t, ff >> u16x2{3, 9});  // codes 1 and 3
    const uint32_t s = perm(t13, t02, 0x06020400u) & 0x07070707u;
    const uint32_t l = perm(t.lo[1], t.lo[0], s), hh = perm(t.hi[1], t.hi[0], s);
    o[2 * h] = perm(hh, l, 0x05010400u);
    o[2 * h + 1] = perm(hh, l, 0x07030602u);
  }
}

// 2-bit (CQ2 and ternary crumbs): the 16 codes of a dword -> 8 dwords.
template <typename T16>
__device__ inline void decode2(const Table<2, T16> &t, uint32_t d, uint32_t *o) {
  const uint32_t x0 = d & 0x03030303u, x1 = (d >> 2) & 0x03030303u;
  const uint32_t x2 = (d >> 4) & 0x03030303u, x3 = (d >> 6) & 0x03030303u;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    // codes 4b, 4b+1 sit in byte b of x0, x1; codes 4b+2, 4b+3 in x2, x3
    const uint32_t sa = perm(x1, x0, 0x04040000u + 0x01010101u * b) * 2u + 0x01000100u;
    const uint32_t sb = perm(x3, x2, 0x04040000u + 0x01010101u * b) * 2u + 0x01000100u;
    o[2 * b] = perm(t.pair[1], t.pair[0], sa);
    o[2 * b + 1] = perm(t.pair[1], t.pair[0], sb);
  }
}


// Byte-plane tables for every width (2-bit included): lo[k] / hi[k] hold the
// low / high bytes of entries 4k..4k+3.  The permuted decoders below return
// the values of 8 codes in an order that saves the final interleave; the
// consumer applies the same order to the other operand.
template <int SB, typename T16>
struct PlaneTable {
  static constexpr int L = 1 << SB;
  uint32_t lo[L / 4], hi[L / 4];
  __device__ void load(const uint32_t *d) {
#pragma unroll
    for (int k = 0; k < L / 4; ++k) lo[k] = d[k], hi[k] = d[L / 4 + k];
  }
  __device__ void build(const cq::CodeLevels &lev, float n) {
#pragma unroll
    for (int k = 0; k < L / 4; ++k) {
      const uint32_t p0 = pack2<T16>(lev.v[4 * k] * n, lev.v[4 * k + 1] * n);
      const uint32_t p1 = pack2<T16>(lev.v[4 * k + 2] * n, lev.v[4 * k + 3] * n);
      lo[k] = perm(p1, p0, 0x06040200u);
      hi[k] = perm(p1, p0, 0x07050301u);
    }
  }
};

// Binary (1-bit) values of one (row, group): fp16(-c * norm) and fp16(+c *
// norm) differ only in the sign bit, so their low bytes are equal.  src
// holds byte 0 = high byte of the code-0 value, byte 1 = high byte of the
// code-1 value, byte 2 = the common low byte.
template <typename T16>
struct BinTable {
  uint32_t src;
  __device__ void load(const uint32_t *d) { src = d[0]; }
  __device__ void build(const cq::CodeLevels &lev, float n) {
    const uint32_t v0 = pack2<T16>(lev.v[0] * n, lev.v[1] * n);  // code 0 low half, code 1 high half
    src = perm(0u, v0, 0x0c000301u);                             // bytes: hi(v0), hi(v1), lo(v1), 0
  }
};

// 1-bit: the 8 codes of byte b, as the pairs (0,4) (1,5) (2,6) (3,7): for
// pair t the selector takes the common low byte (index 2) for both halves
// and the code's high byte (index 0 or 1) from bit t / t + 4 of b.
template <typename T16>
__device__ inline void decode1_planes(const BinTable<T16> &t, uint32_t b, uint32_t *o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = (b >> i) & 0x11u;                                       // bits i and i + 4
    const uint32_t sel = ((x * 0x00100100u) & 0x01000100u) | 0x00020002u;  // x < 2^5: v_mul_u32_u24; bits 8, 24
    o[i] = perm(0u, t.src, sel);
  }
}

// 1-bit, natural order: the 8 codes of byte b as the pairs (0,1) (2,3) (4,5)
// (6,7) (the GEMM's B tile keeps k in order).
template <typename T16>
__device__ inline void decode1(const BinTable<T16> &t, uint32_t b, uint32_t *o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = (b >> (2 * i)) & 3u;                                  // bits 2i and 2i + 1
    const uint32_t sel = ((x * 0x00800100u) & 0x01000100u) | 0x00020002u;  // -> bits 8, 24
    o[i] = perm(0u, t.src, sel);
  }
}

// Binary codes as fp16 -1 / +1 (code 0 / 1; the level is applied in fp32 by
// the caller), for the batched matrix-core kernel: the four fp16 pairs of k
// step t (t < 4) of a 32-code piece x, pair u holding codes 4t + u and
// 4t + u + 16.  Bits i and i + 16 of ~x are 16 apart, so one shift puts them
// on the sign bits 15 and 31 of 0x3c003c00: two instructions per pair, no
// table.  The activation slots follow the same order (slot 8t + 2u + h holds
// column 4t + u + 16h of the piece).
__device__ inline void decode1_sign(uint32_t x, int t, uint32_t (&o)[4]) {
  const uint32_t nx = ~x;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = 4 * t + u;
    o[u] = ((nx & (0x00010001u << i)) << (15 - i)) | 0x3c003c00u;
  }
}

// Slot order of the permuted decoders: position t of an 8-value operand holds
// code perm_code<SB>(t) of its 8 consecutive codes (3-bit: natural order).
template <int SB>
__host__ __device__ constexpr int perm_code(int t) {
  return SB <= 2 ? (t >> 1) + 4 * (t & 1)                          // (0,4) (1,5) (2,6) (3,7)
       : SB == 4 ? (t & 4) + ((t >> 1) & 1) + 2 * (t & 1)          // (0,2) (1,3) (4,6) (5,7)
                 : t;
}

// 2-bit: the 16 codes of dword d.  x_i (i < 4) has codes i, i+4, i+8, i+12 in
// its bytes; one lookup per plane gives four codes' low or high bytes, and
// one interleave makes two values (27 instructions per 16 codes less the
// four selector ORs a single table pair would need: 23).  o[0..3] hold codes 0..7 as the pairs
// (0,4) (1,5) (2,6) (3,7); o[4..7] codes 8..15 as (8,12) (9,13) (10,14) (11,15).
template <typename T16>
__device__ inline void decode2_planes(const PlaneTable<2, T16> &t, uint32_t d, uint32_t *o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = (d >> (2 * i)) & 0x03030303u;
    // selectors 0..3 pick the second source's bytes: the low plane, then
    // with the sources swapped the high plane
    const uint32_t l = perm(t.hi[0], t.lo[0], x), h = perm(t.lo[0], t.hi[0], x);
    o[i] = perm(h, l, 0x05010400u);
    o[4 + i] = perm(h, l, 0x07030602u);
  }
}

// 4-bit: the 8 codes of dword d, as the pairs (0,2) (1,3) (4,6) (5,7).
template <typename T16>
__device__ inline void decode4_planes(const PlaneTable<4, T16> &t, uint32_t d, uint32_t *o) {
  const uint32_t se = d & 0x07070707u, so = (d >> 4) & 0x07070707u;
  const uint32_t me = ((d >> 3) & 0x01010101u) * 0xffu, mo = ((d >> 7) & 0x01010101u) * 0xffu;
  const uint32_t el = select(me, perm(t.lo[3], t.lo[2], se), perm(t.lo[1], t.lo[0], se));
  const uint32_t eh = select(me, perm(t.hi[3], t.hi[2], se), perm(t.hi[1], t.hi[0], se));
  const uint32_t ol = select(mo, perm(t.lo[3], t.lo[2], so), perm(t.lo[1], t.lo[0], so));
  const uint32_t oh = select(mo, perm(t.hi[3], t.hi[2], so), perm(t.hi[1], t.hi[0], so));
  o[0] = perm(eh, el, 0x05010400u);  // codes 0, 2
  o[1] = perm(oh, ol, 0x05010400u);  // codes 1, 3
  o[2] = perm(eh, el, 0x07030602u);  // codes 4, 6
  o[3] = perm(oh, ol, 0x07030602u);  // codes 5, 7
}

// Tables of the fp16 matrix-core matvec kernels: byte planes at 2 and 4
// bits, the plane pairs of Table at 3 bits.
template <int SB>
using MmaTable = typename std::conditional<
    SB == 1, BinTable<_Float16>,
    typename std::conditional<SB == 3, Table<3, _Float16>, PlaneTable<SB, _Float16>>::type>::type;

// B operand of k step s (s < 16) of one (row, group): codes 8s..8s+7 of the
// group's GROUP_DW code dwords, as four dwords of fp16 pairs in slot order
// perm_code<SB>.  The decoders work in units of 8 (4-bit), 8 (3-bit, one
// 24-bit field) or 16 codes (2-bit: half of one dword's decode).
template <int SB>
__device__ inline void decode_step(const MmaTable<SB> &tab, const uint32_t *codes, int s, uint32_t (&o)[4]) {
  if constexpr (SB == 1) {
    decode1_planes(tab, (codes[s >> 2] >> (8 * (s & 3))) & 0xffu, o);
  } else if constexpr (SB == 4) {
    decode4_planes(tab, codes[s], o);
  } else if constexpr (SB == 3) {
    constexpr int DW = 3 * 128 / 32;
    const int bit = 24 * s, w = bit >> 5, sh = bit & 31;
    const uint32_t f = sh <= 8 ? (codes[w] >> sh) : __builtin_amdgcn_alignbit(codes[(w + 1) % DW], codes[w], sh);
    decode3(tab, f, o);
  } else {
    uint32_t o8[8];
    decode2_planes(tab, codes[s >> 1], o8);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = o8[4 * (s & 1) + i];
  }
}

// B operand of k step t (t < 4) of one 32-code piece of a group (the codes a
// lane owns in the matvec kernels: SB dwords): codes 8t..8t+7 of the piece,
// four dwords of fp16 pairs in slot order perm_code<SB>.
template <int SB>
__device__ inline void decode_piece(const MmaTable<SB> &tab, const uint32_t *codes, int t, uint32_t (&o)[4]) {
  if constexpr (SB == 1) {
    decode1_planes(tab, (codes[0] >> (8 * t)) & 0xffu, o);
  } else if constexpr (SB == 4) {
    decode4_planes(tab, codes[t], o);
  } else if constexpr (SB == 3) {
    // 24-bit field t at bit 24t of the three dwords
    const uint32_t f = t == 0 ? codes[0]
                     : t == 1 ? __builtin_amdgcn_alignbit(codes[1], codes[0], 24)
                     : t == 2 ? __builtin_amdgcn_alignbit(codes[2], codes[1], 16)
                              : codes[2] >> 8;
    decode3(tab, f, o);
  } else {
    uint32_t o8[8];
    decode2_planes(tab, codes[t >> 1], o8);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = o8[4 * (t & 1) + i];
  }
}

// 2-bit, two tables at once (the level's high and low fp16 parts): codes
// 8h..8h+7 of dword d (h = 0 or 1) as the pairs (8h + i, 8h + i + 4), i < 4
// -- the slot order of decode2_planes.  One selector per pair serves both
// tables: bytes (c, c | 4, c', c' | 4) pick each code's low-plane byte (the
// second source) and high-plane byte (the first), so each table takes one
// permute per pair.  Per four codes (both halves h): 9 instructions for both
// tables, against 10 with decode2_planes per table sharing the extraction.
template <typename T16>
__device__ inline void decode2_pair2(const PlaneTable<2, T16> &ta, const PlaneTable<2, T16> &tb, uint32_t d, int h,
                                     uint32_t *oa, uint32_t *ob) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t m = (d >> (2 * i)) & 0x03030303u;  // codes i, i+4, i+8, i+12 in bytes 0..3
    const uint32_t mo = m | 0x04040404u;                // the same, as high-plane byte indices
    const uint32_t s = perm(mo, m, h ? 0x07030602u : 0x05010400u);
    oa[i] = perm(ta.hi[0], ta.lo[0], s);
    ob[i] = perm(tb.hi[0], tb.lo[0], s);
  }
}

// decode_piece for the high and low tables of the same codes.
template <int SB>
__device__ inline void decode_piece2(const MmaTable<SB> &thi, const MmaTable<SB> &tlo, const uint32_t *codes, int t,
                                     uint32_t (&ohi)[4], uint32_t (&olo)[4]) {
  if constexpr (SB == 2) {
    decode2_pair2(thi, tlo, codes[t >> 1], t & 1, ohi, olo);
  } else {
    decode_piece<SB>(thi, codes, t, ohi);
    decode_piece<SB>(tlo, codes, t, olo);
  }
}

// The pieces of a chunk of four groups, from whole groups: lane quarter q
// (lanes 16q..16q+15) holds group q of the chunk as four pieces of SB dwords
// (d[p*SB + i]: piece p), and afterwards holds piece q of every group (d[j*SB
// + i]: piece q of group j).  A 4x4 transpose across the quarters: the
// 16-lane swap exchanges quarter bit 0 with piece bit 0, the 32-lane swap
// quarter bit 1 with piece bit 1.
template <int SB>
__device__ inline void quarter_transpose(uint32_t *d) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const auto r = __builtin_amdgcn_permlane16_swap(d[(2 * h) * SB + i], d[(2 * h + 1) * SB + i], false, false);
      d[(2 * h) * SB + i] = r[0];
      d[(2 * h + 1) * SB + i] = r[1];
    }
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const auto r = __builtin_amdgcn_permlane32_swap(d[h * SB + i], d[(2 + h) * SB + i], false, false);
      d[h * SB + i] = r[0];
      d[(2 + h) * SB + i] = r[1];
    }
}

// Every quarter's value v of a 16-lane-quarter-uniform pattern, in every
// lane: out[j] = v of quarter j (lanes 16j..16j+15 at the same lane % 16).
__device__ inline void quarter_gather(uint32_t v, uint32_t (&out)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // quarters (q & 1) and (q & 1) + 2
  const auto lo = __builtin_amdgcn_permlane16_swap(a[0], a[0], false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(a[1], a[1], false, false);
  out[0] = lo[0], out[1] = lo[1], out[2] = hi[0], out[3] = hi[1];
}

// Activation operand of the fp16 matrix-core matvec kernels: batch rows
// 0..7 of the 16 MFMA rows carry fp16(a), rows 8..15 fp16(a - fp16(a)), with
// a the activation times a power of two; the products with the two rows add
// up to the product with a to about 2^-22.
__device__ inline void split_f16(float a, _Float16 &hi, _Float16 &lo) {
  hi = static_cast<_Float16>(a);
  lo = static_cast<_Float16>(a - static_cast<float>(hi));
}

}  // namespace cqdev
