// zf_attention.hip - fused GQA decode attention over the packed paged cache (gfx950).
//
// Method: ZipFusion video summary ("Run AI Faster With Lossless Compressed Memory"): the
// cache stays compressed in HBM and each bf16 is rebuilt in registers with one integer add
// (two values per 32-bit add here) right before it is used; decode is bound by the bytes
// read per step, so reading 12-bit values instead of 16-bit ones is the whole gain.
// Attention itself is the plain decode step (page "Open Weights: from files to tokens /
// second", section "03 / The inference loop": one new token per sequence attends over its
// KV cache).
//
// Mapping (head_dim 128, 16-token pages, G = 4 query heads per kv head; G = 8 differs only in
// the number of weight parts, see attn_k):
//   one workgroup of 8 waves per (split, kv head, sequence); wave w takes pages w, w+8, ...
//   of its split, one page per step of a software pipeline: row metadata (flags, first spill
//   slots, bases) six pages ahead, planes and spill slots two pages ahead, all staged in LDS by
//   direct loads; compute on the current page.  lane = (t = lane & 15, qd = lane >> 4).
//   K: lane holds 32 head_dim values (quarter qd) of token krow(t), read as 16-byte loads.
//   Scores as S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (rebuilt K pairs as A, the 4 query
//   heads replicated over the 16 columns of B): lane (t, qd) receives the scores of tokens
//   qd, qd + 4, qd + 8, qd + 12 for query head t >> 2 -- exactly the A-operand layout of the
//   p.V product.
//   p.V on v_mfma_f32_16x16x16_bf16: A row 4i + j carries part j of head i's weights (three
//   bf16 parts by truncation, hi + mid + lo = p exactly; row 4i + 3 zero), B is V with
//   k = token: lane (t, qd) rebuilds V rows qd + 4j at head_dim 8t..8t+7 straight into token
//   pairs.  The hi row goes to fp64 every page, mid and lo stay in the MFMA accumulators.
//   Softmax: running max in fp64, raised (with an fp64 rescale) only when a page exceeds it.
//   Precise path: every score whose weight may reach 2^-40 of the final maximum is recomputed
//   in fp64 from the exact bf16 products (on the fp64 matrix cores, v_mfma_f64_4x4x4_4b) and
//   weighted with an fp64 exp; the weight sums carry those fp64 weights.  An output that one large value dominates must be right to ~1e-9
//   before its one rounding (the 1e-3 bar is an fp32 ulp at 2^14), and the matrix cores' fp32
//   scores are only good to ~1e-6 of a weight.
//   Large values: a lane's 8 values of a V row holding a magnitude >= 2^4 leave the p.V MFMA
//   and are added in fp64 instead, with the fp64 weight, so the MFMA only ever sums products
//   below 2^4 (where the fp32 rounding of its weights stays below 1e-6 of the output).
//   Splits of the token axis write (acc, l, m) partials; a second small kernel merges them
//   in split order, so results do not depend on timing.
// One kernel body serves the packed cache and raw bf16 pages (the uncompressed twin): both
// loaders hand the same bf16 pairs to the same arithmetic, so the outputs match bit for bit.
#include <algorithm>
#include <mutex>
#include <hip/hip_ext.h>

#include "zf_internal.h"

namespace zf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One workgroup of 8 waves per CU (two per SIMD): with two smaller workgroups sharing a CU, the
// older one is issued first and the younger one then finishes alone at half occupancy.
constexpr int kD = 128, kT = 16, kWaves = 8, kThreads = 64 * kWaves;
constexpr double kLog2e = 1.4426950408889634;
// Exact-value path: V values whose product with their weight may reach 2^4 leave the p.V MFMA,
// which then only ever sums products below 2^4.  With the page's largest weight w in
// [2^e, 2^(e+1)), e <= 0, that is every value with a biased exponent >= max(131, 130 - e)
// (magnitude >= 2^4 while w can be 1).
constexpr uint32_t kLargeExp = 131;
// Which of the lane's four V rows (token qd + 4j) hold a value with biased exponent >= T among
// their 8 values (bit j), from the rebuilt pairs: vt[2n] holds rows 0 and 1 in its two halves,
// vt[2n + 1] rows 2 and 3.  Per half the largest magnitude (bf16 bits less the sign: exponent
// at bits 7..14); adding 0x8000 - (T << 7) sets bit 15 exactly when that exponent is >= T.
__device__ __forceinline__ uint32_t large_rows(const uint32_t (&vt)[16], uint32_t T) {
  uint32_t m01 = 0u, m23 = 0u;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    m01 = pk_max_u16(m01, vt[2 * n] & 0x7FFF7FFFu);
    m23 = pk_max_u16(m23, vt[2 * n + 1] & 0x7FFF7FFFu);
  }
  const uint32_t bias = (0x8000u - (T << 7)) * 0x00010001u;  // T <= 255: lanes stay below 0xBE80
  const uint32_t r01 = m01 + bias, r23 = m23 + bias;
  return ((r01 >> 15) & 1u) | ((r01 >> 30) & 2u) | ((r23 >> 13) & 4u) | ((r23 >> 28) & 8u);
}
// Precise path: tokens whose weight may reach 2^-kSigBits of the final maximum get fp64 scores
// and fp64 weights.  Below that, a weight's fp32 error cannot show: even 2^20 tokens with
// values of 2^17 move the output by less than 2^-40 * 2^20 * 2^17 * 2^-20 < 1e-7.
constexpr double kSigBits = 40.0;
// The hi row of p.V (below) sums this many pages in the MFMA's fp32 accumulator before it is
// added in fp64: each MFMA rounds to a few fp32 ulps of its largest term, so a few pages of
// weights <= 1 keep the row within ~2^-19 of its value.
constexpr int kFlushPages = 4;
// The exact-path test takes the largest score that the waves of the workgroup had seen
// kShareLag steps earlier as a lower bound of the final maximum (it depends on the data only,
// not on timing, so results stay bitwise repeatable), and on the first step the largest of
// the waves' first pages, which they exchange before any of them tests its own.  A wave waits
// when it gets more than kShareLag steps ahead of the slowest one; ring slots are reused after
// kShareRing steps.
constexpr int kShareLag = 1;
constexpr int kShareRing = 8;  // > 2 * kShareLag: no slot is rewritten while it may be read
constexpr uint32_t kDone = 0x7FFFFFFFu;  // progress of a wave that has finished its pages
constexpr int kOrderMaxBatch = 256;  // longest-first group order up to this batch (LDS scratch)
constexpr int kMaxPagesPerSplit = kWaves * 64;
constexpr uint32_t kXcds = 8;  // MI355X: workgroups are dispatched round-robin over 8 XCDs  // each wave keeps its page ids in one register
// One split's partial for G query heads per kv head, in doubles: acc[G][kD], l[G], m[G].
__host__ __device__ constexpr int part_doubles(int G) { return G * kD + 2 * G; }

struct AttnArgs {
  int32_t B, H, maxp, max_seq_len, pps, nsplit_max, num_pages;
  int32_t direct;  // one split per sequence: attn_k writes the output itself
  int32_t order;   // number the (sequence, split) groups longest sequence first
  const int32_t* pt;
  const int32_t* lens;
  const uint32_t* kmax;  // [B][H][maxp] largest K exponent field per page, or null
  const uint16_t* q;
  double scale_log2e;
  float scale_log2e_f32;  // the same in fp32
  float negl_f32;         // kSigBits / scale_log2e in fp32: scores further below the maximum
                          // than this weigh less than 2^-kSigBits of it
  float* out;
  double* part;  // [B][H][nsplit_max][part_doubles(G)]
  uint32_t* status;
};

// ---------------------------------------------------------------- LDS staging
// Pages travel HBM -> LDS with the direct global-to-LDS loads of gfx950 (each lane's bytes land
// at base + lane * size), so a wave keeps several pages in flight without holding them in
// VGPRs.  The loads are counted by hand: every wave issues a fixed number of them per page,
// and waits with an exact vmcnt for the oldest page only.  LDS reads are inline asm that wait
// for their own results, so the compiler never sees an LDS read it would have to fence against
// the whole DMA queue.

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)(uintptr_t)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)(uintptr_t)lds, 4, 0, 0);
}
// The same through a buffer resource: LDS dest = lds + lane * size, global = resource base +
// voff + soff (soff moves the global address only); reads outside the resource return zeros.
constexpr int32_t kRawBufferWord3 = 0x00020000;  // 32-bit data format, no swizzle (gfx9 raw buffer)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferWord3);
}
// Cache policy of a load: plain, or non-temporal (`nt`: the line is not kept for reuse).
// Page planes are read once per launch, so they stream; spill lines and metadata are shared
// by the kv heads of a sequence and stay cached.
constexpr int kKeep = 0, kStream = 2;
template <int Policy = kKeep>
__device__ __forceinline__ void dmab16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(uintptr_t)lds, 16, voff, soff, 0, Policy);
}
__device__ __forceinline__ void dmab4(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(uintptr_t)lds, 4, voff, soff, 0, 0);
}
// Progress of the waves of a workgroup, for the pair balancing below (LDS, asm so that the
// compiler does not fence these accesses against the page loads in flight).
__device__ __forceinline__ void lds_store_u32(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ uint32_t lds_load_u32(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ void lds_max_f64(uint32_t addr, double v) {
  asm volatile("ds_max_f64 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_add_u32(uint32_t addr, uint32_t v) {
  asm volatile("ds_add_u32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ double lds_load_f64(uint32_t addr) {
  double v;
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(addr) : "memory");
  return v;
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------- loaders
// A loader moves one page (16 tokens of kv head h) into an LDS slot and rebuilds it as bf16 pairs:
//   kp[4c + r]   K (head_dim 32*qd + 8c + r, same + 4) of token krow(t)
//   vt[2n], vt[2n + 1]   V (tokens qd, qd + 4) and (qd + 8, qd + 12) at head_dim vdim(n, t)
// with t = lane & 15, qd = lane >> 4.
// kMetaLoads / kPageLoads: direct loads per meta / page.
//
// Token order: row i of the score MFMA's A operand holds token krow(i), so its output row
// 4qd + r -- the r-th score of lane (t, qd) -- is token qd + 4r.  The p.V operands use the same
// order (k index 4qd + r is token qd + 4r), and the four V rows a lane needs, qd + 4j, are then
// four consecutive rows across the quarters of a wave: plain row-major V in LDS is read without
// bank conflicts.

__device__ __forceinline__ int krow(int i) { return (i >> 2) + 4 * (i & 3); }
__device__ __forceinline__ int vdim(int n, int t) { return 8 * t + (n & 3) + 4 * (n >> 2); }

// pr[j][r] = (value r, value r + 4) of V row j (8 values, 8t..8t+7) -> token pairs per dim
__device__ __forceinline__ void to_token_pairs(const uint32_t (&pr)[4][4], uint32_t (&vt)[16]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    vt[2 * r + 0] = __builtin_amdgcn_perm(pr[1][r], pr[0][r], 0x05040100u);
    vt[2 * r + 1] = __builtin_amdgcn_perm(pr[3][r], pr[2][r], 0x05040100u);
    vt[2 * (r + 4) + 0] = __builtin_amdgcn_perm(pr[1][r], pr[0][r], 0x07060302u);
    vt[2 * (r + 4) + 1] = __builtin_amdgcn_perm(pr[3][r], pr[2][r], 0x07060302u);
  }
}

constexpr uint32_t kSlotBytes = 8192;  // one page of either loader
constexpr uint32_t kMetaBytes = 256;   // one page's row metadata (packed loader)
constexpr int kMetaRing = 8;

// Packed page slot.  Every load is 16 bytes per lane; the reads of a quarter wave (16-byte
// reads) or of a half wave (8- and 4-byte reads) always hit distinct banks:
//   [0, 2048)     K sm rows 0..15, 128 B each; 16-byte chunk c of row r at c ^ ((r >> 1) & 7)
//   [2048, 4096)  V sm rows, 128 B each, as in memory
//   [4096, 5120)  K nibble rows, 64 B each; chunk c of row r at c ^ ((r >> 2) & 3)
//   [5120, 6144)  V nibble rows, 64 B each, as in memory
//   [6144, 7168)  V spill: row r's two V blocks of head h (32-byte slot each, zeros when the
//                 block is compressed), 64 B per row
//   [7168, 8192)  K spill the same way, chunk c of row r at c ^ ((r >> 2) & 3)
// Meta slot, one dword per lane of a 4-byte gather: words 2r, 2r + 1 = flags and first spill
// slot of row r (r < 16); words 32..39 the K base bytes of head h (row r at byte 2r + half),
// words 40..47 the V base words in the order 0, 2, 4, 6, 1, 3, 5, 7; words 48..63 unused.
struct PackedLoader {
  const uint8_t* sm;
  const uint8_t* nib;
  const uint8_t* base;
  const uint32_t* row_flags;
  const uint32_t* row_spill;
  const uint8_t* spill;  // a valid address even when the pool is empty
  uint32_t spill_bytes;  // spill_slots * 32 (below 2^32)

  static constexpr int kMetaLoads = 1, kPageLoads = 8;

  __device__ __forceinline__ void issue_meta(int64_t pid, int H, int h, int lane, uint32_t ms) const {
    // the lane's source: array and word are fixed per lane, only the page moves (arithmetic
    // selects, no divergent code)
    const bool is_spill = lane < 32 && (lane & 1), is_base = lane >= 32 && lane < 48;
    const int v = lane - 40;  // V base position v -> word 8 + 2 (v & 3) + (v >> 2)
    const uint32_t word = lane < 32 ? lane >> 1 : lane < 40 ? lane - 32 : lane < 48 ? 8 + 2 * (v & 3) + (v >> 2) : lane - 48;
    const uint64_t d_sp = (uint64_t)row_spill - (uint64_t)row_flags;
    const uint64_t d_bs = (uint64_t)(base + (int64_t)h * 2 * kT * 2) - (uint64_t)row_flags;
    const uint64_t delta = ((0ull - (uint64_t)is_spill) & d_sp) | ((0ull - (uint64_t)is_base) & d_bs);
    const uint64_t stride = is_base ? (uint64_t)H * 2 * kT * 2 : (uint64_t)kT * 4;
    dma4(reinterpret_cast<const void*>((uint64_t)row_flags + delta + 4ull * word + (uint64_t)pid * stride), ms);
  }

  // Byte offset of a spill piece in the pool: slot = first + popcount(lower raw blocks of the
  // row).  A compressed block gets an offset past the end, so its lanes load zeros; raw
  // blocks carry base 0.  The rebuild then needs no raw flag at all.
  __device__ __forceinline__ uint32_t spill_off(uint32_t flags, uint32_t first, int j, uint32_t piece) const {
    const uint32_t slot = (uint32_t)__popc(flags & ((1u << j) - 1u)) + first;
    const uint32_t raw = (uint32_t)__builtin_amdgcn_sbfe((int)flags, j, 1);  // all ones iff raw
    return bitselect(raw, slot * 32u + piece, 0xFFFFFFFFu);
  }

  // The row metadata issue_page needs, read from a meta slot ahead of time: flags and first
  // spill slot of row lane >> 2.
  struct Issue {
    u32x2 fs;
  };

  __device__ __forceinline__ Issue read_issue(int lane, uint32_t ms) const {
    Issue r;
    asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r.fs) : "v"(ms + 8 * (lane >> 2)) : "memory");
    return r;
  }

  // live = false: a step past the wave's last page; its loads still go out (the per-step load
  // count is fixed) but through empty resources, which return zeros without touching memory.
  __device__ __forceinline__ void issue_page(int64_t pid, int H, int h, int lane, uint32_t slot, const Issue& m,
                                             bool live) const {
    // spill: lane l loads 16 bytes of row l >> 2, chunk l & 3 of the row's 64 bytes (K chunks
    // swizzled); the pool as a bounds-checked buffer, so offsets past its end read zeros
    const __amdgpu_buffer_rsrc_t spr = buffer_of(spill, live ? spill_bytes : 0u);
    const int r = lane >> 2;
    const int ck = (lane & 3) ^ ((r >> 2) & 3), cv = lane & 3;
    dmab16(spr, slot + 7168, spill_off(m.fs.x, m.fs.y, (h * 2 + 0) * 2 + (ck >> 1), (ck & 1) * 16), 0);
    dmab16(spr, slot + 6144, spill_off(m.fs.x, m.fs.y, (h * 2 + 1) * 2 + (cv >> 1), (cv & 1) * 16), 0);
    // the planes of (page, h): sm of K rows then V rows (4 KB), nibbles likewise (2 KB)
    const int64_t row0 = ((pid * H + h) * 2) * kT;  // K row 0 of the page
    const __amdgpu_buffer_rsrc_t smr = buffer_of(sm + row0 * kD, live ? 2 * kT * kD : 0u);
    const __amdgpu_buffer_rsrc_t nbr = buffer_of(nib + row0 * (kD / 2), live ? 2 * kT * (kD / 2) : 0u);
    {  // K sm: gather i, lane l -> LDS chunk 64i + l = row 8i + (l >> 3), position l & 7
      const int r0 = lane >> 3, c0 = (lane & 7) ^ ((r0 >> 1) & 7);
      const int r1 = 8 + (lane >> 3), c1 = (lane & 7) ^ ((r1 >> 1) & 7);
      dmab16<kStream>(smr, slot, (uint32_t)(r0 * 128 + c0 * 16), 0);
      dmab16<kStream>(smr, slot + 1024, (uint32_t)(r1 * 128 + c1 * 16), 0);
    }
    {  // K nibbles: lane l -> row l >> 2, position l & 3
      const int rn = lane >> 2, cn = (lane & 3) ^ ((rn >> 2) & 3);
      dmab16<kStream>(nbr, slot + 4096, (uint32_t)(rn * 64 + cn * 16), 0);
    }
    // V sm and nibbles as they are in memory
    dmab16<kStream>(smr, slot + 2048, (uint32_t)(lane * 16), 2048);
    dmab16<kStream>(smr, slot + 3072, (uint32_t)(lane * 16), 3072);
    dmab16<kStream>(nbr, slot + 5120, (uint32_t)(lane * 16), 1024);
  }

  // One page's bytes as this lane needs them (read from LDS in one go): K row krow(t) (sm,
  // nibbles, spill piece, base byte), V rows qd + 4j (vs[j] sm, vn[j] nibbles, vh[j] spill, and
  // the base words vb, base of row qd + 4j in byte 2 (qd & 1) + half of word j).
  struct Page {
    u32x4 ks0, ks1, kn, kh;
    u32x4 vs01, vs23;
    u32x2 vn01, vn23, vh01, vh23;
    uint32_t kb;
    u32x4 vb;
  };

  // page n from its slot and meta slot ms, plus the issue metadata of a later page from ms2
  __device__ __forceinline__ Page read(int lane, uint32_t slot, uint32_t ms, uint32_t ms2, Issue& next) const {
    const int t = lane & 15, qd = lane >> 4;
    const int kr = krow(t);
    const int sk = (kr >> 1) & 7;
    Page p;
    asm volatile(
        "ds_read_b128 %0, %13\n\t"
        "ds_read_b128 %1, %14\n\t"
        "ds_read_b128 %2, %15\n\t"
        "ds_read_b128 %3, %16\n\t"
        "ds_read2st64_b64 %4, %17 offset0:0 offset1:1\n\t"
        "ds_read2st64_b64 %5, %17 offset0:2 offset1:3\n\t"
        "ds_read2st64_b32 %6, %18 offset0:0 offset1:1\n\t"
        "ds_read2st64_b32 %7, %18 offset0:2 offset1:3\n\t"
        "ds_read2st64_b32 %8, %18 offset0:4 offset1:5\n\t"
        "ds_read2st64_b32 %9, %18 offset0:6 offset1:7\n\t"
        "ds_read_u8 %10, %19\n\t"
        "ds_read_b128 %11, %20\n\t"
        "ds_read_b64 %12, %21\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(p.ks0), "=&v"(p.ks1), "=&v"(p.kn), "=&v"(p.kh), "=&v"(p.vs01), "=&v"(p.vs23),
          "=&v"(p.vn01), "=&v"(p.vn23), "=&v"(p.vh01), "=&v"(p.vh23), "=&v"(p.kb), "=&v"(p.vb),
          "=&v"(next.fs)
        : "v"(slot + kr * 128 + ((2 * qd) ^ sk) * 16), "v"(slot + kr * 128 + ((2 * qd + 1) ^ sk) * 16),
          "v"(slot + 4096 + kr * 64 + (qd ^ ((kr >> 2) & 3)) * 16),
          "v"(slot + 7168 + kr * 64 + (qd ^ ((kr >> 2) & 3)) * 16),
          "v"(slot + 2048 + qd * 128 + t * 8), "v"(slot + 5120 + qd * 64 + t * 4),
          "v"(ms + 128 + 2 * kr + (qd >> 1)), "v"(ms + 160 + 16 * (qd >> 1)), "v"(ms2 + 8 * (lane >> 2))
        : "memory");
    return p;
  }

  __device__ __forceinline__ void rebuild_k(const Page& p, int, int, uint32_t (&kp)[16]) const {
    // a raw block has base 0 and its spill piece, a compressed one its base and zeros
    const uint32_t bp = p.kb * 0x00010001u;
    const uint32_t smw[8] = {p.ks0.x, p.ks0.y, p.ks0.z, p.ks0.w, p.ks1.x, p.ks1.y, p.ks1.z, p.ks1.w};
    const uint32_t nw[4] = {p.kn.x, p.kn.y, p.kn.z, p.kn.w};
    const uint32_t hw[4] = {p.kh.x, p.kh.y, p.kh.z, p.kh.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) rebuild8(smw[2 * c], smw[2 * c + 1], nw[c], hw[c], bp, kp + 4 * c);
  }

  // V is rebuilt in groups of two rows: group (q, hh) takes dims 4hh..4hh+3 of rows j = 2q and
  // 2q + 1 (tokens qd + 8q and qd + 8q + 4) as the 8 values of rebuild8, so each rebuilt pair
  // is already the token pair the p.V operand wants.  The nibble and spill words of the two rows
  // are joined by one byte permute, and so are their base bytes.
  __device__ __forceinline__ void rebuild_v(const Page& p, int, int lane, uint32_t (&vt)[16]) const {
    const uint32_t t = (uint32_t)(lane & 15), qd = (uint32_t)(lane >> 4);
    const uint32_t by = 2u * (qd & 1u) + (t >> 3);  // base byte of the lane's rows in vb
    const uint32_t bsel = 0x0C000C00u | ((4u + by) << 16) | by;
    const uint32_t vsw[8] = {p.vs01.x, p.vs01.y, p.vs01.z, p.vs01.w, p.vs23.x, p.vs23.y, p.vs23.z, p.vs23.w};
    const uint32_t vna[4] = {p.vn01.x, p.vn01.y, p.vn23.x, p.vn23.y};
    const uint32_t vha[4] = {p.vh01.x, p.vh01.y, p.vh23.x, p.vh23.y};
    const uint32_t vbw[4] = {p.vb.x, p.vb.y, p.vb.z, p.vb.w};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t b16 = __builtin_amdgcn_perm(vbw[2 * q + 1], vbw[2 * q], bsel);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint32_t sel = hh ? 0x07060302u : 0x05040100u;
        uint32_t pr[4];
        rebuild8(vsw[4 * q + hh], vsw[4 * q + 2 + hh], __builtin_amdgcn_perm(vna[2 * q + 1], vna[2 * q], sel),
                 __builtin_amdgcn_perm(vha[2 * q + 1], vha[2 * q], sel), b16, pr);
#pragma unroll
        for (int r = 0; r < 4; ++r) vt[2 * (r + 4 * hh) + q] = pr[r];
      }
    }
  }
};

// Raw bf16 pages (the uncompressed twin): slot = K rows (256 B each, 16-byte chunk c of row r
// at c ^ r) then V rows.
struct RawLoader {
  const uint16_t* pages;

  static constexpr int kMetaLoads = 0, kPageLoads = 8;

  struct Issue {};
  __device__ __forceinline__ Issue read_issue(int, uint32_t) const { return Issue{}; }
  __device__ __forceinline__ void issue_meta(int64_t, int, int, int, uint32_t) const {}

  __device__ __forceinline__ void issue_page(int64_t pid, int H, int h, int lane, uint32_t slot, const Issue&,
                                             bool live) const {
    const __amdgpu_buffer_rsrc_t pr = buffer_of(pages + ((pid * H + h) * 2) * kT * kD, live ? 2 * kT * kD * 2 : 0u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // gather i, lane l -> row 4i + (l >> 4), position l & 15
      const int r = 4 * i + (lane >> 4), c = (lane & 15) ^ r;
      dmab16<kStream>(pr, slot + i * 1024, (uint32_t)(r * 256 + c * 16), 0);
    }
#pragma unroll
    for (int i = 4; i < 8; ++i) dmab16<kStream>(pr, slot + i * 1024, (uint32_t)(lane * 16), i * 1024);
  }

  struct Page {
    u32x4 k[4], v[4];
  };

  // K row krow(t) (quarter qd), V rows qd + 4j (head_dim 8t..8t+7)
  __device__ __forceinline__ Page read(int lane, uint32_t slot, uint32_t, uint32_t, Issue&) const {
    const int t = lane & 15, qd = lane >> 4;
    const int kr = krow(t);
    Page p;
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\t"
        "ds_read_b128 %5, %12 offset:1024\n\t"
        "ds_read_b128 %6, %12 offset:2048\n\t"
        "ds_read_b128 %7, %12 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(p.k[0]), "=&v"(p.k[1]), "=&v"(p.k[2]), "=&v"(p.k[3]), "=&v"(p.v[0]), "=&v"(p.v[1]),
          "=&v"(p.v[2]), "=&v"(p.v[3])
        : "v"(slot + kr * 256 + ((4 * qd + 0) ^ kr) * 16), "v"(slot + kr * 256 + ((4 * qd + 1) ^ kr) * 16),
          "v"(slot + kr * 256 + ((4 * qd + 2) ^ kr) * 16), "v"(slot + kr * 256 + ((4 * qd + 3) ^ kr) * 16),
          "v"(slot + 4096 + qd * 256 + t * 16)
        : "memory");
    return p;
  }

  __device__ __forceinline__ void rebuild_k(const Page& p, int, int, uint32_t (&kp)[16]) const {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t w[4] = {p.k[c].x, p.k[c].y, p.k[c].z, p.k[c].w};
      natural_to_pairs(w, kp + 4 * c);
    }
  }

  __device__ __forceinline__ void rebuild_v(const Page& p, int, int, uint32_t (&vt)[16]) const {
    uint32_t pr[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w[4] = {p.v[j].x, p.v[j].y, p.v[j].z, p.v[j].w};
      natural_to_pairs(w, pr[j]);
    }
    to_token_pairs(pr, vt);
  }
};

// ---------------------------------------------------------------- kernel

// Reductions across the four 16-lane rows of a wave64 without going through LDS, on gfx950's
// permlane swaps: a swap of v with itself leaves {v[l], v[l ^ 16]} (permlane16) or
// {v[l], v[l ^ 32]} (permlane32) in its two results, in a lane-dependent order that symmetric
// reductions (max, sum) never need to resolve.
// The two doubles {v[l], v[l ^ 16]} (or ^ 32) of a lane: both halves are swapped the same way,
// so the pairs stay whole.
template <bool k32>
__device__ __forceinline__ void pair_d(double v, double& a, double& b) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  const auto l = k32 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false) : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto h = k32 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false) : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  a = __longlong_as_double((int64_t)(((uint64_t)h[0] << 32) | l[0]));
  b = __longlong_as_double((int64_t)(((uint64_t)h[1] << 32) | l[1]));
}
// Maxima in plain C, never inline asm: the scores come straight out of the matrix cores, and
// a VALU read of an MFMA result needs wait states that the compiler inserts only for the
// instructions it can see (an asm max read them stale on full pages under some schedules).
__device__ __forceinline__ float max_f32(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ float max3_f32(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }
__device__ __forceinline__ double max_f64(double a, double b) { return fmax(a, b); }
// max / sum over the 4 rows (lanes l, l ^ 16, l ^ 32, l ^ 48) of a double
__device__ __forceinline__ double rows_max_d(double v) {
  double a, b;
  pair_d<false>(v, a, b);
  pair_d<true>(max_f64(a, b), a, b);
  return max_f64(a, b);
}
__device__ __forceinline__ double rows_sum_d(double v) {
  double a, b;
  pair_d<false>(v, a, b);
  pair_d<true>(a + b, a, b);
  return a + b;
}
// 2^x in fp64 for x <= 0 (weights and rescale factors).  x = n + f with n = rint(x) and
// |f| <= 1/2; 2^f = e^y, y = f ln 2, |y| < 0.35, from the Taylor series of e^y to degree 9
// (truncation below 0.35^10 / 10! < 8e-12 of the result); then 2^n by the exponent.  Written
// here rather than taken from the math library so that its coefficients come from the constant
// table below (scalar registers): as VGPRs they pushed the 8-head kernel past its register
// budget.  Exponents below -1075 give 0 (x = -inf included).
__constant__ double kExpTaylor[10] = {
    1.0, 1.0, 1.0 / 2, 1.0 / 6, 1.0 / 24, 1.0 / 120, 1.0 / 720, 1.0 / 5040, 1.0 / 40320,
    1.0 / 362880};
__device__ __forceinline__ double exp2_neg(double x) {
  const double n = rint(x);
  const double y = (x - n) * 0.69314718055994530942;
  double r = kExpTaylor[9];
#pragma unroll
  for (int k = 8; k >= 0; --k) r = fma(r, y, kExpTaylor[k]);
  return x < -1075.0 ? 0.0 : ldexp(r, (int)fmax(n, -1100.0));
}

// A double from lane I of the lane's quad (DPP quad_perm, both halves the same way).
template <int I0, int I1, int I2, int I3>
__device__ __forceinline__ double quad_pick(double v) {
  constexpr int ctrl = I0 | (I1 << 2) | (I2 << 4) | (I3 << 6);
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, ctrl, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), ctrl, 0xF, 0xF, false);
  return __longlong_as_double((int64_t)(((uint64_t)hi << 32) | lo));
}

// max over the 4 rows (lanes l, l ^ 16, l ^ 32, l ^ 48) of a float
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m1 = max_f32(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m1), __float_as_uint(m1), false, false);
  return max_f32(__uint_as_float(b[0]), __uint_as_float(b[1]));
}



// LDS per wave: two page slots and the meta ring; the end-of-split results reuse the wave's
// own region once its loads have drained.
constexpr uint32_t kWaveLds = 2 * kSlotBytes + kMetaRing * kMetaBytes;
static_assert(8 * kD * sizeof(double) + 2 * 8 * sizeof(double) <= kWaveLds, "results fit");
static_assert(2 * kOrderMaxBatch * sizeof(int32_t) <= kWaveLds, "order scratch fits");

// G query heads per kv head: 4 (Llama-3.1-8B) or 8 (Llama-3.1-70B).  The score MFMA's 16
// columns hold each head kParts = 16 / G times, and the p.V MFMA's 16 A rows hold kParts bf16
// parts of each head's weights: hi, mid, lo (exact, row 3 empty) for G = 4; hi and a rounded
// second part (within 2^-16 of p) for G = 8.
template <class Loader, int G>
__global__ __launch_bounds__(kThreads, 1) void attn_k(AttnArgs a, Loader ld) {
  static_assert(G == 4 || G == 8, "4 or 8 query heads per kv head");
  constexpr int kParts = 16 / G;           // score columns (and p.V rows) per head
  constexpr int kHeadsPerLane = G / 4;     // p.V output heads per lane
  // The job: a (sequence b, split s, kv head h).  Workgroup ids go round-robin over the 8
  // XCDs; in the plain order each XCD takes a contiguous run of jobs (split fastest, then kv
  // head, then sequence), so the kv heads of a sequence share one L2 for the page metadata and
  // spill lines they all read.
  const uint32_t per_xcd = gridDim.x / kXcds;
  const uint32_t xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const uint32_t job = xcd * per_xcd + local;
  const uint32_t units = (uint32_t)a.nsplit_max * (uint32_t)a.H * (uint32_t)a.B;  // <= maxp * B < 2^31
  if (!a.order && job >= units) return;
  int s = (int)(job % (uint32_t)a.nsplit_max);
  int h = (int)((job / (uint32_t)a.nsplit_max) % (uint32_t)a.H);
  int b = (int)(job / ((uint32_t)a.nsplit_max * (uint32_t)a.H));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = lane & 15, qd = lane >> 4;
  const int head = t / kParts;  // query head of this lane's scores (and of its p.V A-operand row)
  const int part = t % kParts;  // which bf16 part of the weights this lane's A row carries
  // masks of the weight split below: row 0 keeps p, row 1 takes p - hi, row 2 (p - hi) - mid,
  // row 3 p - p = 0; with two parts, row 1 keeps p - hi and rounds it (rnd)
  const uint32_t mask1 = part == 0 ? 0u : (G == 4 && part == 3) ? 0xFFFFFFFFu : 0xFFFF0000u;
  const uint32_t mask2 = (G == 4 && part == 2) ? 0xFFFF0000u : 0u;
  const bool rnd = G == 8 && part == 1;

  __shared__ __attribute__((aligned(16))) uint8_t s_ring[kWaves][kWaveLds];
  const int32_t cap = min(a.maxp * kT, a.max_seq_len);
  auto splits_of = [&](int32_t len) {  // splits of a sequence of `len` tokens (len clamped)
    len = len < 0 ? 0 : min(len, cap);
    return max(1, ((len + kT - 1) / kT + a.pps - 1) / a.pps);
  };
  if (a.order) {
    // More workgroups than CUs: when the lengths differ, the (sequence, split) groups are
    // dispatched largest first (longest-processing-time-first list scheduling), group g with
    // all its kv heads on XCD g % 8, so that long jobs start first and short ones fill the end.
    // A sequence's splits hold a.pps pages each except its last, which holds the rest: the
    // full splits come first in (sequence, split) order, then the partial last splits by size
    // (ties: lower sequence).  Each wave finds the same job on its own, with its LDS region as
    // scratch (no pages are in flight yet).
    int32_t* wl = reinterpret_cast<int32_t*>(&s_ring[wave][0]);  // [B] full splits, [B] rest
    int32_t lmin = 0x7FFFFFFF, lmax = -1;
    for (int i = lane; i < a.B; i += 64) {
      const int32_t li = max(0, min(a.lens[i], cap));
      const int32_t pages = (li + kT - 1) / kT;
      const int32_t full = pages / a.pps;
      // pages of the partial last split, -1 when there is none (an empty sequence still has
      // one split, of 0 pages)
      wl[i] = full;
      wl[kOrderMaxBatch + i] = full == splits_of(li) ? -1 : pages - full * a.pps;
      lmin = min(lmin, li);
      lmax = max(lmax, li);
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");  // the wave's stores above before its loads below
    for (int o = 32; o > 0; o >>= 1) {
      lmin = min(lmin, __shfl_xor(lmin, o, 64));
      lmax = max(lmax, __shfl_xor(lmax, o, 64));
    }
    if (lmin != lmax) {
      const uint32_t g = (local / (uint32_t)a.H) * kXcds + xcd;
      int mb = -1, ms = 0;
      uint32_t nfull = 0;  // full splits of all sequences
      for (int k = 0; k < a.B; ++k) nfull += (uint32_t)wl[k];
      for (int i = lane; i < a.B; i += 64) {
        const int32_t ri = wl[kOrderMaxBatch + i];
        uint32_t first = 0, before = 0;  // full splits of sequences < i; partials ranked before i's
        for (int k = 0; k < a.B; ++k) {
          const int32_t rk = wl[kOrderMaxBatch + k];
          if (k < i) first += (uint32_t)wl[k];
          if (rk > ri || (rk == ri && k < i)) before += 1u;
        }
        if (g >= first && g < first + (uint32_t)wl[i]) {
          mb = i;
          ms = (int)(g - first);
        } else if (ri >= 0 && g == nfull + before) {
          mb = i;
          ms = wl[i];
        }
      }
      const uint64_t found = __ballot(mb >= 0);
      if (!found) return;  // past the last group (every wave of the workgroup)
      const int src = __builtin_ffsll((long long)found) - 1;
      b = __builtin_amdgcn_readfirstlane(__shfl(mb, src, 64));
      s = __builtin_amdgcn_readfirstlane(__shfl(ms, src, 64));
      h = (int)(local % (uint32_t)a.H);
    } else if (job >= units) {
      return;
    }
  }

  // the job is the same for every lane: keep it in scalar registers
  b = __builtin_amdgcn_readfirstlane(b);
  s = __builtin_amdgcn_readfirstlane(s);
  h = __builtin_amdgcn_readfirstlane(h);

  // this wave's pages: p_first + 8n; lane n reads the page id (and hint) of page n.  The table row and q
  // are read together with the length, not after it (one memory round trip less before the
  // first page); table entries past the sequence's end are never used.
  const int p_first = s * a.pps + wave;
  int32_t pt_lane = 0;
  uint32_t km_lane = 0u;  // the page's K-exponent hint
  if (p_first + kWaves * lane < a.maxp) {
    pt_lane = a.pt[(int64_t)b * a.maxp + p_first + kWaves * lane];
    if (a.kmax) km_lane = a.kmax[((int64_t)b * a.H + h) * a.maxp + p_first + kWaves * lane];
  }
  // B operand of the score MFMA: column t is query head t / kParts (each head kParts times),
  // head_dim 32*qd + 8c + (0,4,1,5,2,6,3,7)[k]
  bf16x8 qb[4];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * a.H * G + h * G + head) * kD + qd * 32;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 x = *reinterpret_cast<const uint4*>(qrow + 8 * c);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
      uint32_t p[4];
      natural_to_pairs(w, p);
      qb[c] = __builtin_bit_cast(bf16x8, (u32x4){p[0], p[1], p[2], p[3]});
    }
  }
  int32_t L = a.lens[b];
  if (L < 0 || L > cap) {
    if (s == 0 && tid == 0) set_status(a.status, ZF_DEV_ELEN);
    L = L < 0 ? 0 : cap;
  }
  const int npages = (L + kT - 1) / kT;
  const int nsplit = max(1, (npages + a.pps - 1) / a.pps);
  if (s >= nsplit) return;

  // q in fp64, pair order, the B operand of the exact-score MFMA: [head][quarter][pair] =
  // (lo, hi) dims (rows of 17 pairs: the 16 (head, quarter) rows that one read instruction
  // touches fall in different banks)
  __shared__ double2 s_q64[G][4][17];
  if (tid < G * 64) {
    const int i = tid >> 6, qq = (tid >> 4) & 3, k = tid & 15;
    const int dlo = 32 * qq + 8 * (k >> 2) + (k & 3);
    const uint16_t* qrow = a.q + ((int64_t)b * a.H * G + h * G + i) * kD;
    s_q64[i][qq][k] = make_double2((double)__uint_as_float((uint32_t)qrow[dlo] << 16),
                                   (double)__uint_as_float((uint32_t)qrow[dlo + 4] << 16));
  }

  __shared__ uint32_t s_prog[kWaves];  // steps whose running maximum each wave has published
  const uint32_t ring = (uint32_t)(uintptr_t)&s_ring[wave][0];
  const uint32_t meta_ring = ring + 2 * kSlotBytes;

  // lane n holds the page id of page n < nmine
  const int p_end = min(npages, (s + 1) * a.pps);
  const int nmine = p_first < p_end ? (p_end - p_first + kWaves - 1) / kWaves : 0;
  const uint32_t nact = (uint32_t)max(0, min(kWaves, p_end - s * a.pps));  // waves with pages
  int32_t my_pid = 0;
  uint32_t err = 0;
  if (lane < nmine) {
    my_pid = pt_lane;
    if (my_pid < 0 || my_pid >= a.num_pages) {
      err = ZF_DEV_EPAGE;
      my_pid = -1;  // page skipped: read page 0, count no token
    }
  }
  // With the hint, the wave takes first its page with the largest K exponent (the lowest such
  // page on ties): its scores are the likeliest to be near the final maximum, so the running
  // maximum (and through the first-page exchange, every wave's bound) settles early and fewer
  // pages need the fp64 scores.  Steps 0 and `first` swap their pages.
  int first = 0;
  if (a.kmax) {
    uint32_t key = lane < nmine && my_pid >= 0 ? (km_lane << 6) | (63u - (uint32_t)lane) : 0u;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) key = max(key, (uint32_t)__shfl_xor((int)key, o, 64));
    first = __builtin_amdgcn_readfirstlane(key ? 63 - (int)(key & 63u) : 0);
    if (first > 0) {
      const int32_t p0 = __builtin_amdgcn_readlane(my_pid, 0), pf = __builtin_amdgcn_readlane(my_pid, first);
      my_pid = lane == 0 ? pf : (lane == first ? p0 : my_pid);
    }
  }
  // pin the q unpacking here: placed after the first page loads, its wait for q would also
  // wait for them
  asm volatile("" ::"v"(qb[0]), "v"(qb[1]), "v"(qb[2]), "v"(qb[3]));
  __shared__ double s_gmax[kShareRing][G];  // per step: max over the waves' running maxima
  if (tid < kShareRing * G) s_gmax[tid / G][tid % G] = -INFINITY;
  __shared__ double s_first_max[G];  // max over the waves' first pages
  __shared__ uint32_t s_first_count;  // waves that have added their first page to it
  if (tid < G) s_first_max[tid] = -INFINITY;
  if (tid == 0) s_first_count = 0u;
  if (lane == 0) s_prog[wave] = nmine > 0 ? 0u : kDone;
  __syncthreads();

  double m = -INFINITY;  // running max of head `head`'s unscaled scores (fp64)
  double l = 0.0;        // this lane's share of head `head`'s weight sum (tokens qd + 4i)
  // p.V output: lane (t, qd) receives rows 4qd..4qd+3 at head_dim vdim(n, t): for G = 4 the
  // hi, mid, lo parts (and an empty fourth row) of head qd; for G = 8 the hi and second parts
  // of heads 2qd and 2qd + 1.  The hi rows are summed here in fp64: with outlier values the
  // running sum reaches 1e4, where one fp32 rounding is already 5e-4.
  double acc[kHeadsPerLane][8];
  f32x4 cacc[8];  // the MFMA accumulators: rows 4qd + j kParts + r, part r of head slot j
#pragma unroll
  for (int n = 0; n < 8; ++n) {
#pragma unroll
    for (int j = 0; j < kHeadsPerLane; ++j) acc[j][n] = 0.0;
    cacc[n] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  const double c2 = a.scale_log2e;
  const float c2f = a.scale_log2e_f32;
  double mc2 = 0.0;        // m * c2 once m is finite
  float m32 = -INFINITY;   // m in fp32, for the exact-path test
  // from the kernel arguments, so it stays in a scalar register (computed here it sat in a VGPR
  // that was spilled and reloaded inside the page loop, behind a wait for every load in flight)
  const float negl32 = a.negl_f32;
  float shared32 = -INFINITY;  // the workgroup's maximum kShareLag steps ago (fp32)

  // page n of this wave; indices past the end repeat the last page (their metadata loads keep
  // the per-step load count fixed and are never used; their page loads read nothing)
  auto pid_at = [&](int n) -> int64_t {
    const int32_t v = __builtin_amdgcn_readlane(my_pid, min(n, nmine - 1));
    return v < 0 ? 0 : v;
  };
  auto ntok_at = [&](int n) -> int {
    if (__builtin_amdgcn_readlane(my_pid, n) < 0) return 0;
    const int ln = n == 0 ? first : (n == first ? 0 : n);  // the page's place in the sequence
    return min(kT, L - (p_first + kWaves * ln) * kT);
  };
  auto slot_of = [&](int n) -> uint32_t { return ring + (uint32_t)(n & 1) * kSlotBytes; };
  auto meta_of = [&](int n) -> uint32_t { return meta_ring + (uint32_t)(n & (kMetaRing - 1)) * kMetaBytes; };

  const uint32_t first_max_addr = (uint32_t)(uintptr_t)&s_first_max[head];
  const uint32_t first_count_addr = (uint32_t)(uintptr_t)&s_first_count;
  auto compute = [&](const int n, const typename Loader::Page& pg) {
    const int ntok = ntok_at(n);
    uint32_t kp[16];
    ld.rebuild_k(pg, h, lane, kp);
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 ka = __builtin_bit_cast(bf16x8, (u32x4){kp[4 * c], kp[4 * c + 1], kp[4 * c + 2], kp[4 * c + 3]});
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[c], sc, 0, 0, 0);
    }
    // sc[i]: token qd + 4i, head `head`; tokens past the end of the page count as -inf
    if (ntok < kT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = qd + 4 * i < ntok ? sc[i] : -INFINITY;
    }
    const float pm32 = rows_max(max_f32(max3_f32(sc[0], sc[1], sc[2]), sc[3]));
    if (n == 0) {
      // every wave with pages adds its first page's maximum, then waits for the others (they
      // all start together, so the wait is short) and takes the largest as its lower bound
      if (lane < 16 && part == 0) lds_max_f64(first_max_addr, (double)pm32);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the maximum lands before the count
      if (lane == 0) lds_add_u32(first_count_addr, 1u);
      while (lds_load_u32(first_count_addr) < nact) __builtin_amdgcn_s_sleep(1);
      shared32 = max_f32(shared32, (float)lds_load_f64(first_max_addr));
    }
    // A score is significant unless it lies more than kSigBits / c2 below a lower bound of the
    // final maximum (the wave's running maximum, this page's, and the workgroup's of a few steps
    // ago): only then is its weight sure to stay under 2^-kSigBits of the largest one.  The
    // fp32 score of the matrix cores is off by up to ~1e-6 of its weight, and an output that a
    // large value dominates needs its weights to ~1e-9, so significant scores are recomputed in
    // fp64 from the exact bf16 products (the margin covers the fp32 error of this test).
    const float floor32 = max_f32(max_f32(m32, pm32), shared32) - negl32;
    bool big = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) big |= sc[i] > floor32;
    double sd[4], pm;
    const bool exact = __any(big);
    if (exact) {
      // exact fp64 scores on the matrix cores (v_mfma_f64_4x4x4_4b: four independent 4x4x4
      // blocks per wave).  Block b = t >> 2 takes tokens b + 4r (r = 0..3) against 4 query
      // heads, k = the quarter qd: lane (t, qd) feeds A[r = t & 3][k = qd] = its own K value
      // (token krow(t) = b + 4 (t & 3)) and B[k = qd][j = t & 3] = query head j (+ 4 for the second
      // group of G = 8) at the same dim, and receives D[r = qd][j = t & 3]: the score of token
      // (t >> 2) + 4 qd, head t & 3.  Each step covers one dim of every quarter; the products
      // of two bf16 values are exact in fp64, so only the fp64 sums round.
      const uint64_t bm = __ballot(big);  // bit 16 qd + t: head t / kParts
      const uint32_t cols = (uint32_t)(bm | (bm >> 16) | (bm >> 32) | (bm >> 48)) & 0xFFFFu;
      constexpr int kGroups = G / 4;  // groups of 4 query heads (one MFMA chain set each)
      bool need[kGroups];  // wave-uniform: the group holds a significant score
#pragma unroll
      for (int g = 0; g < kGroups; ++g) need[g] = (cols >> (16 / kGroups) * g) & (0xFFFFu >> (16 - 16 / kGroups));
      double dsum[kGroups];
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        dsum[g] = 0.0;
        if (!need[g]) continue;
        double d0 = 0.0, d1 = 0.0, d2 = 0.0, d3 = 0.0;  // four chains: dims lo / hi of even / odd pairs
        const double2* qrow = &s_q64[4 * g + (t & 3)][qd][0];
#pragma unroll
        for (int n = 0; n < 16; n += 2) {
          const double2 qa = qrow[n], qb2 = qrow[n + 1];
          d0 = __builtin_amdgcn_mfma_f64_4x4x4f64((double)__uint_as_float(kp[n] << 16), qa.x, d0, 0, 0, 0);
          d1 = __builtin_amdgcn_mfma_f64_4x4x4f64((double)__uint_as_float(kp[n] & 0xFFFF0000u), qa.y, d1, 0, 0, 0);
          d2 = __builtin_amdgcn_mfma_f64_4x4x4f64((double)__uint_as_float(kp[n + 1] << 16), qb2.x, d2, 0, 0, 0);
          d3 = __builtin_amdgcn_mfma_f64_4x4x4f64((double)__uint_as_float(kp[n + 1] & 0xFFFF0000u), qb2.y, d3, 0, 0, 0);
        }
        dsum[g] = (d0 + d1) + (d2 + d3);
      }
      // lane (t, qd) reads token qd + 4i, head `head`: the D entry of lane (4 qd + (head & 3), i)
      // of group head >> 2.  Heads of a group without a significant score keep their fp32 ones.
      const bool mine = need[kGroups == 1 ? 0 : head >> 2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int src = 16 * i + 4 * qd + (head & 3);
        double x = __shfl(dsum[0], src, 64);
        if constexpr (G == 8) {
          const double x2 = __shfl(dsum[1], src, 64);
          x = head >= 4 ? x2 : x;
        }
        // tokens past the end stay out
        sd[i] = sc[i] == -INFINITY ? -INFINITY : mine ? x : (double)sc[i];
      }
      pm = rows_max_d(max_f64(max_f64(sd[0], sd[1]), max_f64(sd[2], sd[3])));
    } else {
      pm = (double)pm32;  // the same maximum
    }

    // V is rebuilt here, where its independent work can fill the latency of the maxima
    uint32_t vt[16];
    ld.rebuild_v(pg, h, lane, vt);
    // tokens past the end of the page: their weights are zero, but their rows hold whatever
    // the memory holds, and 0 * Inf or NaN would not be zero
    if (ntok < kT) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t keep = (qd + 8 * q < ntok ? 0x0000FFFFu : 0u) | (qd + 8 * q + 4 < ntok ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int nn = 0; nn < 8; ++nn) vt[2 * nn + q] &= keep;
      }
    }
    if (__any(pm > m)) {
      // rescale by alpha = 2^((m - mn) c2) in fp64: the factor applies to every earlier token,
      // so its error would act as a weight error of all of them
      const double mn = fmax(m, pm);
      const double alpha = exp2_neg((m - mn) * c2);  // m = -inf (no finite score yet): 0
      m = mn;
      m32 = (float)m;
      mc2 = m * c2;
      l *= alpha;
#pragma unroll
      for (int j = 0; j < kHeadsPerLane; ++j) {
        // acc slot j holds head kHeadsPerLane qd + j; lane head * kParts has that head's alpha
        const double al = __shfl(alpha, (kHeadsPerLane * qd + j) * kParts, 64);
        const float alf = (float)al;  // the MFMA sums only hold products below 2^4
#pragma unroll
        for (int nn = 0; nn < 8; ++nn) {
          acc[j][nn] *= al;
          cacc[nn][j * kParts] *= alf;
          cacc[nn][j * kParts + 1] *= alf;
          if constexpr (G == 4) cacc[nn][2] *= alf;
        }
      }
    }
    // weights 2^((s - m) c2); a page seen before any finite score leaves m = -inf and mc2 = 0.
    // On the precise path in fp64 (w64, which the weight sum and the exact-value path take);
    // p, their fp32 rounding, feeds the p.V MFMA, whose values all stay below 2^4.  Off it every
    // score is insignificant and fp32 is plenty.
    float p[4];
    double w64[4];
    if (exact) {
      // the kParts lanes of a quad that share a head hold the same four scores: each takes the
      // exp of 4 / kParts of them and the quad swaps the results
      if constexpr (G == 4) {
        const int x = t & 3;
        const double e = exp2_neg(fma(x == 0 ? sd[0] : x == 1 ? sd[1] : x == 2 ? sd[2] : sd[3], c2, -mc2));
        w64[0] = quad_pick<0, 0, 0, 0>(e);
        w64[1] = quad_pick<1, 1, 1, 1>(e);
        w64[2] = quad_pick<2, 2, 2, 2>(e);
        w64[3] = quad_pick<3, 3, 3, 3>(e);
      } else {
        const bool x = t & 1;
        const double e0 = exp2_neg(fma(x ? sd[1] : sd[0], c2, -mc2));
        const double e1 = exp2_neg(fma(x ? sd[3] : sd[2], c2, -mc2));
        w64[0] = quad_pick<0, 0, 2, 2>(e0);
        w64[1] = quad_pick<1, 1, 3, 3>(e0);
        w64[2] = quad_pick<0, 0, 2, 2>(e1);
        w64[3] = quad_pick<1, 1, 3, 3>(e1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = (float)w64[i];
      l += (w64[0] + w64[1]) + (w64[2] + w64[3]);
    } else {
      const float mc2f = (float)mc2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], c2f, -mc2f));
        w64[i] = (double)p[i];
      }
      l += (double)((p[0] + p[1]) + (p[2] + p[3]));
    }
    // Exact-value path: a lane's 8 values of row j holding a large value are added here, in
    // fp64, by the lanes that own those output columns, and leave the MFMA operand.  Lane
    // (t, qd) owns heads kHeadsPerLane qd + hh at head_dim vdim(n, t); the values of token
    // qs + 4j at those dims sit in lane (t, qs), its weight for head i in lane (i kParts, qs).
    // "Large" depends on the page's largest weight in the units of the final result: its heads'
    // page maxima against a lower bound of their final maxima (the running maximum and the
    // workgroup's of a few steps ago).  Once a far larger score has been seen, even outliers
    // stay in the MFMA: the sums they enter are scaled down by at least that much later.
    float wpage = 0.f;
    {
      const double mlb = fmax(m, (double)shared32);
      const float pw = __builtin_amdgcn_exp2f((float)((pm - mlb) * c2));  // this lane's head, <= 1
#pragma unroll
      for (int i = 0; i < G; ++i)  // lane i kParts holds head i (a NaN from an empty page drops out)
        wpage = fmaxf(wpage, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw), i * kParts)));
    }
    const int we = (int)((__float_as_uint(wpage) >> 23) & 0xFFu) - 127;  // floor(log2), -127 for 0
    const uint32_t vthr = (uint32_t)max((int)kLargeExp, 130 - we);  // wave-uniform
    // (rows past the end of the page are zero by now)
    const uint32_t vlarge = vthr <= 255u ? large_rows(vt, vthr) : 0u;
    if (__any(vlarge != 0u)) {
      uint64_t bw[4];     // bw[j]: lanes whose row j is large
      uint32_t toks = 0;  // bit qs + 4j: token qs + 4j has a large chunk in some lane
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bw[j] = __ballot((vlarge >> j) & 1u);
#pragma unroll
        for (int qs = 0; qs < 4; ++qs) toks |= ((bw[j] >> (16 * qs)) & 0xFFFFull) ? 1u << (qs + 4 * j) : 0u;
      }
      while (toks) {  // wave-uniform: one large token per iteration
        const int tok = __builtin_ctz(toks);
        toks &= toks - 1u;
        const int j = tok >> 2, qs = tok & 3, src = t + 16 * qs;
        const uint64_t bj = j == 0 ? bw[0] : j == 1 ? bw[1] : j == 2 ? bw[2] : bw[3];
        const bool take = ((uint32_t)(bj >> (16 * qs)) >> t) & 1u;
        const double wj = j == 0 ? w64[0] : j == 1 ? w64[1] : j == 2 ? w64[2] : w64[3];
        double wgt[kHeadsPerLane];
#pragma unroll
        for (int hh = 0; hh < kHeadsPerLane; ++hh)
          wgt[hh] = __shfl(wj, (kHeadsPerLane * qd + hh) * kParts + 16 * qs, 64);
        const uint32_t sh = (j & 1) ? 0u : 16u;  // row 2q in the low halves, 2q + 1 in the high
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const uint32_t x = __shfl((j >> 1) ? vt[2 * n + 1] : vt[2 * n], src, 64);
          if (take) acc[0][n] = fma(wgt[0], (double)__uint_as_float((x << sh) & 0xFFFF0000u), acc[0][n]);
          if constexpr (kHeadsPerLane == 2)
            if (take) acc[1][n] = fma(wgt[1], (double)__uint_as_float((x << sh) & 0xFFFF0000u), acc[1][n]);
        }
      }
      // this lane's large chunks leave the MFMA operand
      const uint32_t keep0 = ((vlarge & 1u) ? 0u : 0x0000FFFFu) | ((vlarge & 2u) ? 0u : 0xFFFF0000u);
      const uint32_t keep1 = ((vlarge & 4u) ? 0u : 0x0000FFFFu) | ((vlarge & 8u) ? 0u : 0xFFFF0000u);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) {
        vt[2 * nn] &= keep0;
        vt[2 * nn + 1] &= keep1;
      }
    }
    // A operand: this lane's row carries one bf16 part of the weights, p = hi + mid + lo, all
    // three by truncation: hi = the top 8 significant bits of p, mid those of x1 = p - hi,
    // lo = x1 - mid (at most 8 bits left).  The differences are exact, so the three parts
    // sum to p exactly.  Each row subtracts only the parts before its own (masks of 0 subtract
    // zero), so the truncation below leaves row `part` its part; row 3 subtracts p itself.
    uint32_t xb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x1 = p[i] - __uint_as_float(__float_as_uint(p[i]) & mask1);
      xb[i] = __float_as_uint(x1 - __uint_as_float(__float_as_uint(x1) & mask2));
      // two parts: the second one rounds to nearest even instead of truncating
      if constexpr (G == 8) xb[i] += rnd ? 0x7FFFu + ((xb[i] >> 16) & 1u) : 0u;
    }
    // the high halves (the truncated bf16 parts) of two values per register
    const s16x4 pa = __builtin_bit_cast(s16x4, (u32x2){__builtin_amdgcn_perm(xb[1], xb[0], 0x07060302u),
                                                        __builtin_amdgcn_perm(xb[3], xb[2], 0x07060302u)});
    // rows 4qd + j kParts + r: part r of head kHeadsPerLane qd + j.  The hi rows are moved to
    // fp64 every kFlushPages pages; the other parts (below 2^-8 of hi) accumulate in the MFMA
    // throughout.
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) {
      const s16x4 vb = __builtin_bit_cast(s16x4, (u32x2){vt[2 * nn], vt[2 * nn + 1]});
      cacc[nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, cacc[nn], 0, 0, 0);
    }
    if ((n & (kFlushPages - 1)) == kFlushPages - 1) {
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) {
#pragma unroll
        for (int j = 0; j < kHeadsPerLane; ++j) {
          acc[j][nn] += (double)cacc[nn][j * kParts];
          cacc[nn][j * kParts] = 0.f;
        }
      }
    }
  };

  // Pipeline: page n sits in slot n & 1, its row metadata in meta slot n & 7.  Step n issues
  // page n + 2 (planes and spill pieces; the spill addresses come from its metadata, read one
  // step earlier) and the metadata of page n + 6.  Every step issues exactly one page's and one
  // meta's worth of loads, so a fixed vmcnt finds everything of step n - 2 and earlier landed
  // at the top of step n.
  constexpr int kM = Loader::kMetaLoads, kP = Loader::kPageLoads;
  if (nmine > 0) {
    // virtual steps -6 .. -1 of the loop below: metas 0..5, pages 0 and 1
#pragma unroll
    for (int k = 0; k < 4; ++k) ld.issue_meta(pid_at(k), a.H, h, lane, meta_of(k));
    wait_vm<3 * kM>();
    ld.issue_page(pid_at(0), a.H, h, lane, slot_of(0), ld.read_issue(lane, meta_of(0)), true);
    ld.issue_meta(pid_at(4), a.H, h, lane, meta_of(4));
    wait_vm<kP + 2 * kM>();
    ld.issue_page(pid_at(1), a.H, h, lane, slot_of(1), ld.read_issue(lane, meta_of(1)), nmine > 1);
    typename Loader::Issue next = ld.read_issue(lane, meta_of(2));
    ld.issue_meta(pid_at(5), a.H, h, lane, meta_of(5));
    // Waves w and w + 4 share a SIMD, and the SIMD issues the older one first: left alone, w
    // finishes well before w + 4, which then runs by itself at half occupancy.  Each step, the
    // wave of the pair that is behind raises its priority (the pages each wave takes are fixed,
    // so the results do not depend on this).
    const uint32_t prog_base = (uint32_t)(uintptr_t)&s_prog[0];
    const uint32_t gmax_base = (uint32_t)(uintptr_t)&s_gmax[0][0];
    auto gmax_at = [&](int step) -> uint32_t {
      return gmax_base + (uint32_t)(((step & (kShareRing - 1)) * G + head) * 8);
    };
    for (int n = 0; n < nmine; ++n) {
      // step n's running maximum (pages before n) into the workgroup's maximum of step n
      if (lane < 16 && part == 0) lds_max_f64(gmax_at(n), m);
      lds_store_u32(prog_base + 4 * wave, (uint32_t)n + 1);
      uint32_t prog = lds_load_u32(prog_base + 4 * (lane & (kWaves - 1)));
      if (n > 0) {
        // the workgroup's maximum over the pages before step n - lag; on the first steps lag 0
        // (every wave has just published its first pages' maximum, and without it each wave
        // would take its first pages on the precise path), then kShareLag
        const int lag = n >= kShareLag ? kShareLag : 0;
        const uint32_t need = (uint32_t)(n - lag) + 1;  // every wave past step n - lag
        while (!__all(prog >= need)) {
          __builtin_amdgcn_s_sleep(1);
          prog = lds_load_u32(prog_base + 4 * (lane & (kWaves - 1)));
        }
        shared32 = max_f32(shared32, (float)lds_load_f64(gmax_at(n - lag)));
      }
      if ((uint32_t)n + 1 > __builtin_amdgcn_readlane(prog, wave ^ 4)) __builtin_amdgcn_s_setprio(0);
      else __builtin_amdgcn_s_setprio(2);
      // every load of step n - 2 and earlier has landed: page n, metas up to n + 4
      wait_vm<kP + kM>();
      // page n leaves its slot (LDS -> VGPRs) together with the issue metadata of page n + 3;
      // page n + 2's loads then go into the freed slot and the rebuild runs while they fly
      const typename Loader::Issue cur = next;
      const typename Loader::Page pg = ld.read(lane, slot_of(n), meta_of(n), meta_of(n + 3), next);
      ld.issue_page(pid_at(n + 2), a.H, h, lane, slot_of(n), cur, n + 2 < nmine);
      ld.issue_meta(pid_at(n + 6), a.H, h, lane, meta_of(n + 6));
      compute(n, pg);
    }
    wait_vm<0>();  // the loads past the end still target this wave's LDS
    if (lane < 16 && part == 0) lds_max_f64(gmax_at(nmine), m);  // the final maximum
    lds_store_u32(prog_base + 4 * wave, kDone);  // done: never hold the others back
    __builtin_amdgcn_s_setprio(0);
  }
  if (err) set_status(a.status, err);

  // ---- per-wave results to the wave's own LDS region: lane (t, qd) holds head qd at
  //      head_dim vdim(n, t)
#pragma unroll
  for (int nn = 0; nn < 8; ++nn) {
    if constexpr (G == 4) {
      acc[0][nn] += (double)cacc[nn][0] + (double)cacc[nn][1] + (double)cacc[nn][2];
    } else {
      acc[0][nn] += (double)cacc[nn][0] + (double)cacc[nn][1];
      acc[1][nn] += (double)cacc[nn][2] + (double)cacc[nn][3];
    }
  }
  l = rows_sum_d(l);
  double* w_acc = reinterpret_cast<double*>(&s_ring[wave][0]);  // [G][kD], then m[G], l[G]
#pragma unroll
  for (int nn = 0; nn < 8; ++nn) {
#pragma unroll
    for (int j = 0; j < kHeadsPerLane; ++j) w_acc[(kHeadsPerLane * qd + j) * kD + vdim(nn, t)] = acc[j][nn];
  }
  if (lane < 16 && part == 0) {  // lane i kParts holds head i
    w_acc[G * kD + head] = m;
    w_acc[G * kD + G + head] = l;
  }
  __syncthreads();

  // ---- merge the waves (fp64) into this split's partial acc[G][kD], l[G], m[G], or with
  //      a single split straight into the output
  auto wres = [&](int w2) { return reinterpret_cast<const double*>(&s_ring[w2][0]); };
  const int64_t unit = (int64_t)b * a.H + h;
  double* part_out = a.part + (unit * a.nsplit_max + s) * part_doubles(G);
  __shared__ double s_f[kWaves][G];
  __shared__ double s_lsum[G];
  if (tid < G * kWaves) {  // thread (head i, wave w2), in wave 0: lanes 8i..8i+7 hold head i
    const int i = tid >> 3, w2 = tid & (kWaves - 1);
    double mm = -INFINITY;
#pragma unroll
    for (int w3 = 0; w3 < kWaves; ++w3) mm = fmax(mm, wres(w3)[G * kD + i]);
    const double mw = wres(w2)[G * kD + i];
    const double f = mw == -INFINITY ? 0.0 : exp2((mw - mm) * c2);
    s_f[w2][i] = f;
    double lsum = f * wres(w2)[G * kD + G + i];
    lsum += __shfl_xor(lsum, 1, 64);
    lsum += __shfl_xor(lsum, 2, 64);
    lsum += __shfl_xor(lsum, 4, 64);
    if (w2 == 0) {
      s_lsum[i] = lsum;
      if (!a.direct) {
        part_out[G * kD + i] = lsum;
        part_out[G * kD + G + i] = mm;
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < G * kD; e += kThreads) {
    double sum = 0.0;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) sum += s_f[w2][e / kD] * wres(w2)[e];
    if (a.direct) {
      const double lsum = s_lsum[e / kD];
      a.out[((int64_t)b * a.H * G + h * G) * kD + e] = lsum > 0.0 ? (float)(sum / lsum) : 0.f;
    } else {
      part_out[e] = sum;
    }
  }
}

// Merges the split partials of one (sequence, kv head) in split order (a kernel of its own:
// the launch boundary makes every split's partial visible without device-wide fences).
// Each split's (m, l) pairs are staged in LDS in one parallel step, the per-split weights are
// formed once, and every thread then reads its accumulator column with independent loads.
constexpr int kMaxSplitsStaged = 256;

template <int G>
__global__ __launch_bounds__(kThreads) void combine_k(AttnArgs a) {
  constexpr int kPartDoubles = part_doubles(G);
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int32_t L = a.lens[b];
  const int32_t cap = min(a.maxp * kT, a.max_seq_len);
  L = L < 0 ? 0 : min(L, cap);
  const int npages = (L + kT - 1) / kT;
  const int nsplit = max(1, (npages + a.pps - 1) / a.pps);
  const int64_t unit = (int64_t)b * a.H + h;
  const double* base = a.part + unit * a.nsplit_max * kPartDoubles;
  const double c2 = a.scale_log2e;
  __shared__ double s_m[kMaxSplitsStaged][G];
  __shared__ double s_w[kMaxSplitsStaged][G];
  __shared__ double s_lsum[G];
  for (int e = tid; e < nsplit * G; e += kThreads) {
    const int x = e / G, i = e % G;
    s_m[x][i] = base[x * kPartDoubles + G * kD + G + i];
    s_w[x][i] = base[x * kPartDoubles + G * kD + i];  // l, turned into weights below
  }
  __syncthreads();
  if (tid < G) {
    const int i = tid;
    double mm = -INFINITY;
    for (int x = 0; x < nsplit; ++x) mm = fmax(mm, s_m[x][i]);
    double lsum = 0.0;
    for (int x = 0; x < nsplit; ++x) {
      const double f = s_m[x][i] == -INFINITY ? 0.0 : exp2((s_m[x][i] - mm) * c2);
      lsum += f * s_w[x][i];
      s_w[x][i] = f;
    }
    s_lsum[i] = lsum;
  }
  __syncthreads();
  for (int e = tid; e < G * kD; e += kThreads) {
    const int i = e / kD, d = e % kD;
    double sum = 0.0;
#pragma unroll 8
    for (int x = 0; x < nsplit; ++x) sum += s_w[x][i] * base[x * kPartDoubles + i * kD + d];
    const double lsum = s_lsum[i];
    a.out[((int64_t)b * a.H * G + h * G + i) * kD + d] = lsum > 0.0 ? (float)(sum / lsum) : 0.f;
  }
}

// ---------------------------------------------------------------- plan + launch

struct Plan {
  int pps, nsplit_max;
};

// Pages per split: about one workgroup per CU (256), at least one page per wave, at most 64
// per wave, and splits of one sequence as equal as the multiple of kWaves allows.
static Plan make_plan(int32_t B, int32_t H, int32_t max_seq_len) {
  const int maxpages = std::max(1, (max_seq_len + kT - 1) / kT);
  const int64_t units = std::max<int64_t>((int64_t)B * H, 1);
  int64_t splits = std::max<int64_t>(1, (256 + units - 1) / units);
  splits = std::min<int64_t>(splits, (maxpages + kWaves - 1) / kWaves);
  splits = std::max<int64_t>(splits, 1);
  int pps = (int)((maxpages + splits - 1) / splits);
  pps = (pps + kWaves - 1) / kWaves * kWaves;
  pps = std::min(std::max(pps, kWaves), kMaxPagesPerSplit);
  if ((maxpages + pps - 1) / pps > kMaxSplitsStaged)  // very long sequences: fewer, longer splits
    pps = std::min(kMaxPagesPerSplit, ((maxpages + kMaxSplitsStaged - 1) / kMaxSplitsStaged + kWaves - 1) / kWaves * kWaves);
  return Plan{pps, (maxpages + pps - 1) / pps};
}

// Workspace: a 256-byte header (unused, keeps the partials aligned), then the split partials.
size_t attention_workspace_bytes(int32_t B, int32_t H, int32_t G, int32_t max_seq_len) {
  Plan pl = make_plan(B, H, max_seq_len);
  return 256 + (size_t)B * H * pl.nsplit_max * part_doubles(G) * sizeof(double);
}

struct TimingEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
static thread_local TimingEvents t_timing;

void set_attention_timing(hipEvent_t start, hipEvent_t stop) { t_timing = TimingEvents{start, stop}; }

template <class Loader, int G>
static hipError_t launch(const Loader& ld, int32_t num_pages, int32_t H, const zf_seqs* q,
                         const uint16_t* qv, float scale, float* out, void* ws, uint32_t* status,
                         hipStream_t st) {
  Plan pl = make_plan(q->batch, H, q->max_seq_len);
  AttnArgs a;
  a.B = q->batch;
  a.H = H;
  a.maxp = q->max_pages_per_seq;
  a.max_seq_len = q->max_seq_len;
  a.pps = pl.pps;
  a.nsplit_max = pl.nsplit_max;
  a.num_pages = num_pages;
  a.direct = pl.nsplit_max == 1;
  int dev = 0, cus = 0;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  a.pt = q->page_table;
  a.lens = q->seq_lens;
  a.kmax = q->kmax;
  a.q = qv;
  a.scale_log2e = (double)scale * kLog2e;
  a.scale_log2e_f32 = (float)a.scale_log2e;
  a.negl_f32 = (float)(kSigBits / a.scale_log2e);
  a.out = out;
  a.part = reinterpret_cast<double*>(static_cast<char*>(ws) + 256);
  a.status = status;
  // groups (sequence, split) rounded up to a multiple of the XCD count, times the kv heads
  const uint32_t groups = (uint32_t)pl.nsplit_max * (uint32_t)q->batch;
  dim3 grid((groups + kXcds - 1) / kXcds * kXcds * (uint32_t)H);
  // the dispatch order only matters with more workgroups than CUs
  a.order = q->batch > 1 && q->batch <= kOrderMaxBatch && grid.x > (uint32_t)cus;
  if (t_timing.start) {  // one-shot device timestamps of this kernel (profiling aid)
    const TimingEvents ev = t_timing;
    t_timing = TimingEvents{};
    hipExtLaunchKernelGGL((attn_k<Loader, G>), grid, dim3(kThreads), 0, st, ev.start, ev.stop, 0, a, ld);
  } else {
    hipLaunchKernelGGL((attn_k<Loader, G>), grid, dim3(kThreads), 0, st, a, ld);
  }
  if (!a.direct) hipLaunchKernelGGL(combine_k<G>, dim3(H, q->batch), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <class Loader>
static hipError_t launch_g(const Loader& ld, int32_t num_pages, int32_t H, int32_t Hq,
                           const zf_seqs* q, const uint16_t* qv, float scale, float* out, void* ws,
                           uint32_t* status, hipStream_t st) {
  if (Hq == 8 * H) return launch<Loader, 8>(ld, num_pages, H, q, qv, scale, out, ws, status, st);
  return launch<Loader, 4>(ld, num_pages, H, q, qv, scale, out, ws, status, st);
}

hipError_t launch_attention_packed(const zf_cache* c, const zf_seqs* q, const uint16_t* qv,
                                   int32_t Hq, float scale, float* out, void* ws, hipStream_t st) {
  // the spill address of a compressed block is never used, but it must be readable
  const uint8_t* spill = c->spill_slots > 0 ? c->spill : c->sm;
  const uint32_t spill_bytes = (uint32_t)(c->spill_slots * 32);  // validated below 2^32
  PackedLoader ld{c->sm, c->nib, c->base, c->row_flags, c->row_spill, spill, spill_bytes};
  return launch_g(ld, c->num_pages, c->num_kv_heads, Hq, q, qv, scale, out, ws, c->status, st);
}

// ---------------------------------------------------------------- allocation-free scratch

// The split partials of zf_decode_attention_noalloc live here instead of in a caller's
// workspace: one array per GPU the library runs on, held until the process ends.  In host
// code `scratch` names a host-side stand-in, so its device address is looked up once per device
// and only that address is handed to kernels.  Calls on one device share the array.
static __device__ __align__(256) unsigned char scratch[ZF_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call there).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_attention_raw(const uint16_t* pages, int32_t num_pages, int32_t H,
                                const zf_seqs* q, const uint16_t* qv, int32_t Hq, float scale,
                                float* out, void* ws, uint32_t* status, hipStream_t st) {
  RawLoader ld{pages};
  return launch_g(ld, num_pages, H, Hq, q, qv, scale, out, ws, status, st);
}

// ---------------------------------------------------------------- workspace fill

__global__ void fill_zero_k(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_zero_k, dim3(blocks), dim3(256), 0, st, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace zf
