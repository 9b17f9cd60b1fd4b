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
  uint32_t emin, emax, special;
};

__device__ __forceinline__ Window window8(const uint32_t w[4]) {
  Window r{255u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint32_t e = exp_of(w[k] >> (16 * s));
      r.emin = min(r.emin, e);
      r.emax = max(r.emax, e);
      r.special |= (e == 0u) | (e == 255u);
    }
  }
  return r;
}

// Packs 8 values (4 words, value 2k in the low half of w[k]) into 8 sm bytes (two words)
// and 8 nibbles (one word, value k at bits 4k).  `base` = 0 for raw blocks.
__device__ __forceinline__ void pack8(const uint32_t w[4], uint32_t base, uint32_t raw,
                                      uint32_t sm[2], uint32_t& nib, uint32_t& hi) {
  sm[0] = sm[1] = 0u;
  nib = 0u;
  hi = 0u;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    uint32_t h = (w[v >> 1] >> (16 * (v & 1))) & 0xFFFFu;
    uint32_t e = exp_of(h);
    uint32_t smb = ((h >> 8) & 0x80u) | (h & 0x7Fu);
    sm[v >> 2] |= smb << (8 * (v & 3));
    uint32_t n = raw ? (e & 15u) : (e - base);
    nib |= n << (4 * v);
    hi |= (e >> 4) << (4 * v);
  }
}

// ---------------------------------------------------------------- rebuild (decode, attention)

// Rebuilds the pair (value r, value r + 4) of an 8-value group: the sm bytes of values 0..3
// are in s0, of 4..7 in s1 (s0x, s1x: the same words shifted left by 8); nibble of value v at
// bits 4v of `nib`; `hi` holds a raw block's exponent high nibbles the same way (0 for a
// compressed block) and `base_pair` = base * 0x00800080 (0 for a raw block).  Returns value r
// in the low half and value r + 4 in the high half.
//
// v_perm_b32 selectors 8..11 produce 0xFF or 0x00 from the sign bit of byte 1 or 3 of either
// source, which moves each sign to bit 15 of its half in the same instruction that spreads the
// sm bytes; the nibble and high-nibble fields are then inserted with bitfield selects, and a
// single add of the base completes both values.
// v_bfi_b32: (a & mask) | (b & ~mask) in one instruction (the mask comes from an SGPR).
__device__ __forceinline__ uint32_t bitselect(uint32_t mask, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(mask), "v"(a), "v"(b));
  return r;
}

template <int r>
__device__ __forceinline__ uint32_t rebuild_pair(uint32_t s0, uint32_t s1, uint32_t s0x,
                                                 uint32_t s1x, uint32_t nib, uint32_t hi,
                                                 uint32_t base_pair) {
  constexpr uint32_t sel = (r & 2) ? 0x0B070903u : 0x0A050801u;  // [b, sign(b), b', sign(b')]
  const uint32_t p = (r & 1) ? __builtin_amdgcn_perm(s1, s0, sel) : __builtin_amdgcn_perm(s1x, s0x, sel);
  const uint32_t n = (r <= 1) ? (nib << (7 - 4 * r)) : (nib >> (4 * r - 7));
  const uint32_t e = (r <= 2) ? (hi << (11 - 4 * r)) : (hi >> 1);
  uint32_t x = bitselect(0x07800780u, n, p);  // nibble -> bits 7..10 (and 23..26)
  x = bitselect(0x78007800u, e, x);           // high nibble -> bits 11..14
  return x + base_pair;                                  // the one add: + base << 7, twice
}

// The 4 pairs of one 8-value group, pair r = (value r, value r + 4).
__device__ __forceinline__ void rebuild8(uint32_t s0, uint32_t s1, uint32_t nib,
                                         uint32_t spill_hi, uint32_t base_pair,
                                         uint32_t out[4]) {
  const uint32_t s0x = s0 << 8, s1x = s1 << 8;
  out[0] = rebuild_pair<0>(s0, s1, s0x, s1x, nib, spill_hi, base_pair);
  out[1] = rebuild_pair<1>(s0, s1, s0x, s1x, nib, spill_hi, base_pair);
  out[2] = rebuild_pair<2>(s0, s1, s0x, s1x, nib, spill_hi, base_pair);
  out[3] = rebuild_pair<3>(s0, s1, s0x, s1x, nib, spill_hi, base_pair);
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
