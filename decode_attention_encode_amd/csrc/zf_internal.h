// zf_internal.h - device-side helpers shared by the codec and attention kernels (gfx950).
//
// Format (ZipFusion video summary, chapter "Twelve Bits and One Addition"): per 64-value block
// a base exponent, per value a sign+mantissa byte and a 4-bit exponent offset; raw blocks keep
// exponent & 15 in the nibble plane and exponent >> 4 in a spill slot.  A bf16 is rebuilt as
// (s << 15 | nibble << 7 | m) + addend, the addend being base << 7 (compressed) or
// (exponent >> 4) << 11 (raw): one integer add.  Two values share one 32-bit add when they sit
// in the two halves of a register, which is how every kernel here rebuilds them.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/zf.h"

namespace zf {

constexpr int kBlock = 64;  // values per block

// Host-side layout strides of one cache, all in elements of their own array.
struct Geom {
  int32_t P, T, H, D;
  __host__ __device__ int nb() const { return D / kBlock; }              // blocks per head row
  __host__ __device__ int blocks_per_row() const { return 2 * H * nb(); }
  __host__ __device__ int64_t vals_per_page() const { return (int64_t)H * 2 * T * D; }
};

// ---------------------------------------------------------------- classification (encode)

// Exponent field of a bf16 word.
__device__ __forceinline__ uint32_t exp_of(uint32_t h) { return (h >> 7) & 0xFFu; }

// Per-lane partial window of 8 values held as 4 u32 words (two bf16 each).
struct Window {
  uint32_t emin, emax;
};

// Two 16-bit lanes at once (v_pk_min_u16, v_pk_max_u16).
typedef unsigned short zf_u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(zf_u16x2, a),
                                                                __builtin_bit_cast(zf_u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(zf_u16x2, a),
                                                                __builtin_bit_cast(zf_u16x2, b)));
}

// The exponent fields of the two values of a word, value 2k's in bits 0..7, value 2k + 1's in
// bits 16..23.
__device__ __forceinline__ uint32_t exp_pair(uint32_t w) { return (w >> 7) & 0x00FF00FFu; }

// Both values of a word at once: the minimum and maximum exponent fields of the two 16-bit
// halves, folded at the end.
__device__ __forceinline__ Window window8(const uint32_t w[4]) {
  uint32_t mn = 0x00FF00FFu, mx = 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t e = exp_pair(w[k]);
    mn = pk_min_u16(mn, e);
    mx = pk_max_u16(mx, e);
  }
  Window r;
  r.emin = min(mn & 0xFFFFu, mn >> 16);
  r.emax = max(mx & 0xFFFFu, mx >> 16);
  return r;
}

// The raw rule over a block's whole window: a value is special (zero or subnormal: field 0; Inf
// or NaN: field 255) exactly when the window reaches 0 or 255, so that needs no test per value.
__device__ __forceinline__ uint32_t is_raw(const Window& w) {
  return (uint32_t)(w.emin == 0u) | (uint32_t)(w.emax == 255u) | (uint32_t)(w.emax - w.emin > 15u);
}

// Two words of four 4-bit fields, one in the low bits of each byte (values 0..3 and 4..7),
// gathered into one word, value v at bits 4v: byte 0 of x | x >> 4 holds values 0 and 1, byte 2
// values 2 and 3.
__device__ __forceinline__ uint32_t gather_nibbles(uint32_t lo4, uint32_t hi4) {
  return __builtin_amdgcn_perm(hi4 | (hi4 >> 4), lo4 | (lo4 >> 4), 0x06040200u);
}

// Packs 8 values (4 words, value 2k in the low half of w[k]) into 8 sm bytes (two words)
// and 8 nibbles (one word, value k at bits 4k); `hi` gets every value's exponent >> 4 the same
// way (the spill nibbles, used for raw blocks).  `base` = 0 for raw blocks, whose nibbles are
// then the exponent's low 4 bits.  Four values at a time, one byte each: the exponent fields
// (bits 7..14 of a value) shifted down and gathered by a byte permute; a compressed block's
// offsets e - base lie in [0, 15], so one subtraction per four values serves both (the bytes
// never borrow from each other).
__device__ __forceinline__ void pack8(const uint32_t w[4], uint32_t base, uint32_t raw,
                                      uint32_t sm[2], uint32_t& nib, uint32_t& hi) {
  const uint32_t b4 = (raw ? 0u : base) * 0x01010101u;
  uint32_t n[2], h[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t e = __builtin_amdgcn_perm(w[2 * j + 1] >> 7, w[2 * j] >> 7, 0x06040200u);  // 4 fields
    n[j] = (e - b4) & 0x0F0F0F0Fu;
    h[j] = (e >> 4) & 0x0F0F0F0Fu;
    // sm byte of a value: its low byte (mantissa in bits 0..6) with bit 7 taken from its high
    // byte (the sign)
    const uint32_t lo = __builtin_amdgcn_perm(w[2 * j + 1], w[2 * j], 0x06040200u);  // low bytes
    const uint32_t hb = __builtin_amdgcn_perm(w[2 * j + 1], w[2 * j], 0x07050301u);  // high bytes
    sm[j] = (lo & 0x7F7F7F7Fu) | (hb & 0x80808080u);
  }
  nib = gather_nibbles(n[0], n[1]);
  hi = gather_nibbles(h[0], h[1]);
}

// ---------------------------------------------------------------- rebuild (decode, attention)

// Rebuilds the 8 values of a group as 4 pairs, pair r = (value r, value r + 4), value r in the
// low half.  s0 holds the sm bytes of values 0..3, s1 those of 4..7; `nib` the offset of value v
// at bits 4v; `hi` a raw block's exponent high nibbles the same way (zero for a compressed
// block); `base16` = base * 0x00010001 (zero for a raw block).
//
// First the exponent bytes, e = offset | high nibble << 4, for the even values (xe) and the odd
// values (xo).  Per pair, one byte permute spreads e of both values into the low bytes of the two
// halves, one add-and-shift puts (e + base) << 7 in bits 7..14 -- the single add of the method,
// done for two values -- and a bitfield select merges it with the sm bytes, which a second
// permute duplicates into both bytes of each half: bit 15 then carries the sign and bits 0..6
// the mantissa, the rest is replaced.
// v_bfi_b32: (a & mask) | (b & ~mask) in one instruction (the mask comes from an SGPR).
__device__ __forceinline__ uint32_t bitselect(uint32_t mask, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(mask), "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ void rebuild8(uint32_t s0, uint32_t s1, uint32_t nib, uint32_t hi,
                                         uint32_t base16, uint32_t out[4]) {
  const uint32_t xe = bitselect(0x0F0F0F0Fu, nib, hi << 4);  // e of values 0, 2, 4, 6
  const uint32_t xo = bitselect(0x0F0F0F0Fu, nib >> 4, hi);  // e of values 1, 3, 5, 7
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t k = (uint32_t)(r >> 1);  // byte of value r in xe / xo
    const uint32_t epair = __builtin_amdgcn_perm(0u, (r & 1) ? xo : xe, 0x0C000C00u | ((k + 2) << 16) | k);
    const uint32_t spair = __builtin_amdgcn_perm(s1, s0, (uint32_t)r * 0x0101u + (uint32_t)(r + 4) * 0x01010000u);
    out[r] = bitselect(0x7F807F80u, (epair + base16) << 7, spair);
  }
}

// Natural order (value 2k low, 2k+1 high in word k) from the (r, r+4) pair order.
__device__ __forceinline__ void pairs_to_natural(const uint32_t p[4], uint32_t w[4]) {
  w[0] = (p[0] & 0xFFFFu) | (p[1] << 16);          // v0 v1
  w[1] = (p[2] & 0xFFFFu) | (p[3] << 16);          // v2 v3
  w[2] = (p[0] >> 16) | (p[1] & 0xFFFF0000u);      // v4 v5
  w[3] = (p[2] >> 16) | (p[3] & 0xFFFF0000u);      // v6 v7
}

// (r, r+4) pair order from natural words w0..w3 (values 0..7).
__device__ __forceinline__ void natural_to_pairs(const uint32_t w[4], uint32_t p[4]) {
  p[0] = (w[0] & 0xFFFFu) | (w[2] << 16);          // v0 v4
  p[1] = (w[0] >> 16) | (w[2] & 0xFFFF0000u);      // v1 v5
  p[2] = (w[1] & 0xFFFFu) | (w[3] << 16);          // v2 v6
  p[3] = (w[1] >> 16) | (w[3] & 0xFFFF0000u);      // v3 v7
}

__device__ __forceinline__ void set_status(uint32_t* status, uint32_t bits) {
  if (bits) atomicOr(status, bits);
}

}  // namespace zf
