// In-register decoding of the SBN-v1 packed planes (a K-bit meta bitmap per
// row, and the survivors' 2-bit codes 00 = 0, 01 = +1, 11 = -1 in position
// order) into int8 matrix-instruction operands.  Shared by the GEMM and the
// decode GEMV.
#pragma once

#include "sbn_internal.h"

namespace sbn {

// Unpack table entry e = nib | (c8 << 4): the four int8 weights of a group of
// four positions whose meta bits are `nib` and whose survivors' 2-bit codes
// start at the low end of `c8`.  The codes are spread to one byte each
// (01 -> +1, 11 -> -1, 00 -> 0), then byte k of the entry takes survivor
// number popcount(nib & ((1 << k) - 1)) if bit k of nib is set, else 0.
__device__ inline uint32_t unpack_entry(uint32_t e) {
  const uint32_t nib = e & 15u, c8 = (e >> 4) & 0xFFu;
  const uint32_t sp = (((c8 & 0x33u) * 0x1001u) & 0x00030003u) | (((c8 & 0xCCu) * 0x40040u) & 0x03000300u);
  const uint32_t v = sp | ((sp & 0x02020202u) * 0x7Eu);           // survivors, one per byte, in order
  const uint32_t t = (nib & 1u) | ((nib & 2u) << 7) | ((nib & 4u) << 14) | ((nib & 8u) << 21);   // byte k = bit k
  const uint32_t pre = t * 0x01010100u;                            // byte k = set bits below k
  const uint32_t msk = t * 0xFFu;
  const uint32_t sel = (pre & msk) | (0x0C0C0C0Cu & ~msk);        // byte select; 0x0C yields 0
  return __builtin_amdgcn_perm(0u, v, sel);
}

// bits [off, off+nb) of the word array w (off, nb compile-time after unrolling)
template <int NW>
__device__ inline uint32_t bits_at(const uint32_t (&w)[NW], int off, int nb) {
  const int i = off >> 5, s = off & 31;
  uint32_t v = w[i] >> s;
  if (s + nb > 32 && i + 1 < NW) v = __builtin_amdgcn_alignbit(w[i + 1], w[i], s);
  return nb >= 32 ? v : (v & ((1u << nb) - 1u));
}

// Sixteen consecutive positions of one row as int8 weights (one 16-byte
// operand of v_mfma_i32_16x16x64_i8), through the unpack table `lut`.
// mw16: the 16 meta bits of the positions (ignored when dense, n == M); c:
// the row's code bits from bit `cb0` on, where cb0 is the first code of the
// group containing the first position (positions start on a group boundary).
// M is the group size, n the survivors per group.
template <int M>
__device__ inline v4i unpack16(const uint32_t* lut, uint32_t mw16, bool dense, int n,
                               unsigned long long c, int cb0) {
  uint32_t e[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t nib = dense ? 0xFu : ((mw16 >> (4 * k)) & 0xFu);
    uint32_t c8;
    if (M == 4) {
      c8 = (uint32_t)(c >> (cb0 + 2 * n * k)) & 0xFFu;
    } else {
      const uint32_t gb = (uint32_t)(c >> (cb0 + 2 * n * (k >> 1)));
      if ((k & 1) == 0) {
        c8 = gb & 0xFFu;
      } else {
        const uint32_t low = dense ? 0xFu : ((mw16 >> (4 * (k - 1))) & 0xFu);
        c8 = (gb >> (2 * __builtin_popcount(low))) & 0xFFu;
      }
    }
    e[k] = lut[nib | (c8 << 4)];
  }
  return (v4i){(int)e[0], (int)e[1], (int)e[2], (int)e[3]};
}

// 2:4, one 32-position slice of a row: meta word mb (8 groups of 4 bits, two
// set) and code word cb (16 survivors x 2 bits, in position order) -> the 16
// compressed int8 values and the sixteen 2-bit position indices of
// v_smfmac_i32_16x16x128_i8's A operand (slot 2h, 2h+1 = group h's survivors).
__device__ inline void decode24(uint32_t mb, uint32_t cb, v4i& a, int& ix) {
  // indices, per nibble (m3 m2 m1 m0, two bits set): p0 = lowest set bit,
  // p1 = highest; p0 = (m1 & ~m0) + 2 (~m1 & ~m0), p1 = (m3 | ~m2) + 2 (m3 | m2),
  // each bit formed in place from the word shifted by one position
  const uint32_t L = mb << 1, Rr = mb >> 1, lx = L | mb;
  ix = (int)((~mb & Rr & 0x11111111u) | (~lx & 0x22222222u) | ((Rr | ~mb) & 0x44444444u) | (lx & 0x88888888u));
  // values: plane q holds, in byte d, the code of survivor 4d+q, turned into its
  // int8 weight by a byte permute against the table {00 -> 0, 01 -> +1, 11 -> -1};
  // words d and d+1 gather byte d and d+1 of the four planes
  constexpr uint32_t TAB = 0xFF000100u;
  const uint32_t e0 = __builtin_amdgcn_perm(0u, TAB, cb & 0x03030303u);
  const uint32_t o1 = __builtin_amdgcn_perm(0u, TAB, (cb >> 2) & 0x03030303u);
  const uint32_t e2 = __builtin_amdgcn_perm(0u, TAB, (cb >> 4) & 0x03030303u);
  const uint32_t o3 = __builtin_amdgcn_perm(0u, TAB, (cb >> 6) & 0x03030303u);
#pragma unroll
  for (int d = 0; d < 4; d += 2) {
    const uint32_t sel = ((uint32_t)(d + 5) << 24) | ((uint32_t)(d + 1) << 16) | ((uint32_t)(d + 4) << 8) | (uint32_t)d;
    const uint32_t lo = __builtin_amdgcn_perm(o1, e0, sel);   // [e0_d, o1_d, e0_d+1, o1_d+1]
    const uint32_t hi = __builtin_amdgcn_perm(o3, e2, sel);
    a[d] = (int)__builtin_amdgcn_perm(hi, lo, 0x05040100u);
    a[d + 1] = (int)__builtin_amdgcn_perm(hi, lo, 0x07060302u);
  }
}

// decode24 with the values as 64 * w: each survivor's code in the top two bits
// of its byte (0x40 = +64, 0xC0 = -64, 0 = 0), so the products sum to 64 times
// the accumulator.  Plane q = (cb << (6 - 2q)) & 0xC0C0C0C0 holds in byte d the
// code of survivor 4d + q; two rounds of byte permutes transpose the four
// planes into survivor order.
__device__ inline void decode24_x64(uint32_t mb, uint32_t cb, v4i& a, int& ix) {
  const uint32_t L = mb << 1, Rr = mb >> 1, lx = L | mb;
  ix = (int)((~mb & Rr & 0x11111111u) | (~lx & 0x22222222u) | ((Rr | ~mb) & 0x44444444u) | (lx & 0x88888888u));
  const uint32_t p0 = (cb << 6) & 0xC0C0C0C0u, p1 = (cb << 4) & 0xC0C0C0C0u;
  const uint32_t p2 = (cb << 2) & 0xC0C0C0C0u, p3 = cb & 0xC0C0C0C0u;
  const uint32_t q01l = __builtin_amdgcn_perm(p1, p0, 0x05010400u);   // [p0.0, p1.0, p0.1, p1.1]
  const uint32_t q01h = __builtin_amdgcn_perm(p1, p0, 0x07030602u);   // [p0.2, p1.2, p0.3, p1.3]
  const uint32_t q23l = __builtin_amdgcn_perm(p3, p2, 0x05010400u);
  const uint32_t q23h = __builtin_amdgcn_perm(p3, p2, 0x07030602u);
  a[0] = (int)__builtin_amdgcn_perm(q23l, q01l, 0x05040100u);         // survivors 0..3
  a[1] = (int)__builtin_amdgcn_perm(q23l, q01l, 0x07060302u);         // 4..7
  a[2] = (int)__builtin_amdgcn_perm(q23h, q01h, 0x05040100u);         // 8..11
  a[3] = (int)__builtin_amdgcn_perm(q23h, q01h, 0x07060302u);         // 12..15
}

}  // namespace sbn
