// zf_codec.hip - block codec kernels for gfx950: full-cache encode, per-step append, decode.
//
// Codec: ZipFusion video summary ("Run AI Faster With Lossless Compressed Memory", chapter
// "Twelve Bits and One Addition").  Paged cache: page "Open Weights: from files to tokens /
// second", section "09 / The optimization stack" (KV memory allocated in fixed-size blocks).
//
// Work split.  A raw page u16[H][2][T][D] is one contiguous 64 KB run (H = 8, T = 16,
// D = 128), so one workgroup owns one (sequence, logical page) and streams it with 16-byte
// loads: 8 lanes cover one 64-value block, a 256-thread group covers 32 blocks per sweep, and
// a thread issues the loads of 16 sweeps before it uses the first.  Spill slots follow an
// exclusive scan of raw-block counts in (sequence, token) order, which encode computes in the
// same pass by decoupled look-back (Merrill and Garland, "Single-pass Parallel Prefix Scan
// with Decoupled Look-back", NVIDIA technical report NVR-2016-002): each page publishes its
// raw count, then takes its prefix from the pages before it, so a raw block's spill nibbles
// are written from the registers that classified it and the raw input is read once.
#include <type_traits>

#include "zf_internal.h"

namespace zf {

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
size_t encode_workspace_bytes(const zf_seqs* q);

struct SeqView {
  int32_t B, maxp, max_seq_len;
  const int32_t* pt;
  int32_t* lens;
  uint32_t* kmax;  // [B][H][maxp] largest K exponent field per (sequence, kv head, page), or null
};

// The K-exponent hint of (sequence b, kv head h, logical page p).
__device__ __forceinline__ int64_t kmax_at(const SeqView& s, int H, int b, int h, int p) {
  return ((int64_t)b * H + h) * s.maxp + p;
}

// Whether `need` more slots fit in a pool of `slots` whose first `top` are taken (a top beyond
// the pool, which no call leaves behind, counts as full).
__device__ __forceinline__ bool fits_in_pool(uint64_t need, uint64_t top, uint64_t slots) {
  return top <= slots && need <= slots - top;
}

// Rows of logical page p of sequence b that hold tokens, or -1 when the length is invalid.
__device__ __forceinline__ int rows_in_page(const SeqView& s, const Geom& g, int b, int p,
                                            int32_t* len_out) {
  int32_t L = s.lens[b];
  *len_out = L;
  if (L < 0 || (int64_t)L > (int64_t)s.maxp * g.T) return -1;
  int64_t r = (int64_t)L - (int64_t)p * g.T;
  return r <= 0 ? 0 : (r > g.T ? g.T : (int)r);
}

// Streaming accesses: the codec reads and writes every plane byte once per call, so its loads
// and stores carry the non-temporal hint (lines are not kept for reuse).  Measured on gfx950, a
// plain 16-byte copy with the hint on both sides moves ~6.3 TB/s read plus written, without it
// ~5.4-5.9 TB/s.
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t nt_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_stream4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ uint2 ld_stream8(const void* p) {
  const nt_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st_stream16(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  __builtin_nontemporal_store((nt_u32x4){a, b, c, d}, reinterpret_cast<nt_u32x4*>(p));
}
__device__ __forceinline__ void st_stream8(void* p, uint32_t a, uint32_t b) {
  __builtin_nontemporal_store((nt_u32x2){a, b}, reinterpret_cast<nt_u32x2*>(p));
}

// ------------------------------------------------------------------------------ encode

// Look-back words, one per (sequence, logical page) in the workspace (zeroed before the pass):
// flag in bits 62..63 (0 nothing yet, 1 the page's own raw count, 2 the count of every page up
// to and including it), the count below.
constexpr uint64_t kLbAggregate = (uint64_t)1 << 62;
constexpr uint64_t kLbInclusive = (uint64_t)2 << 62;
constexpr uint64_t kLbValue = ((uint64_t)1 << 62) - 1u;
constexpr uint32_t kLbPolls = 1u << 22;  // bound on one look-back wait (~ seconds; none is expected)
// Pause between polls of a look-back word (units of 64 clocks): the words are read through the
// coherence point shared by all XCDs, and thousands of workgroups polling it back to back slow
// everyone's other traffic (encode: 302 us at 1, 288 us at 32, no better beyond)
constexpr int kLbSleep = 32;

// Pages of sequence b that hold tokens (0 for an invalid length).
__device__ __forceinline__ int pages_of(const SeqView& s, const Geom& g, int b) {
  const int32_t L = s.lens[b];
  if (L <= 0 || (int64_t)L > (int64_t)s.maxp * g.T) return 0;
  return (L + g.T - 1) / g.T;
}

// Raw blocks of every page before (b, p) in (sequence, page) order, from the look-back words
// (called by wave 0 of the workgroup; the result in every lane).  Lane l looks at the l-th page
// back within one sequence; the walk stops at the nearest page that has published an inclusive
// count and otherwise adds the pages' own counts, moving on to the previous sequence's last
// page when it has passed a sequence's first.  Every page waited for comes earlier in the grid,
// so it has been dispatched and publishes without waiting for this one.  *failed is set if a
// wait ran out (the sum is then incomplete).
__device__ uint64_t look_back(const SeqView& s, const Geom& g, const uint64_t* look, int b, int p,
                              uint32_t* failed) {
  const int lane = threadIdx.x & 63;
  uint64_t sum = 0;
  uint32_t ran_out = 0u;
  int pb = b, hi = p - 1;  // next page to look at: (pb, hi)
  while (true) {
    while (hi < 0) {  // on to the previous sequence's last page
      if (--pb < 0) {
        if (__any(ran_out)) *failed = 1u;  // in every lane
        return sum;
      }
      hi = pages_of(s, g, pb) - 1;
    }
    const int q = hi - lane;
    uint64_t w = kLbInclusive;  // before the sequence's first page: a stop with nothing in it
    if (q >= 0) {
      const uint64_t* a = look + (int64_t)pb * s.maxp + q;
      uint32_t n = 0;
      while (true) {
        w = __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((w >> 62) != 0u) break;
        if (++n == kLbPolls) {
          ran_out = 1u;
          w = kLbAggregate;
          break;
        }
        __builtin_amdgcn_s_sleep(kLbSleep);
      }
    }
    const uint64_t stop = __ballot((w >> 62) == 2u);
    const int k = stop ? __builtin_ctzll(stop) : 63;  // nearest stop, or the whole window
    uint64_t v = lane <= k ? (w & kLbValue) : 0u;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    sum += v;
    if (!stop) {
      hi -= 64;
      continue;
    }
    if (hi - k >= 0) {  // lane k holds an inclusive count: everything before is in it
      if (__any(ran_out)) *failed = 1u;
      return sum;
    }
    hi = -1;  // the window passed the sequence's first page
  }
}

// Encode of one (sequence, logical page): 4 lanes per 64-value block, 16 values each (two
// 16-byte loads).  The first kEncSweeps sweeps of kEncThreads chunks (a whole page of 512
// blocks) keep their raw blocks' spill nibbles in LDS until the page's slots are known; a
// larger page's later sweeps read their raw blocks again for them.  (512 threads with 4 sweeps
// measured 5 % slower than 256 with 8.)
constexpr int kEncThreads = 256;
constexpr int kEncSweeps = 8;
constexpr int kEncUnroll = 2;
// The encode is bound by how many loads are in flight, so by how many workgroups fit a CU: the
// raw blocks' spill nibbles wait for their slots in LDS rather than in VGPRs, and the register
// budget is held to 6 waves per SIMD (80 VGPRs, no spills; 8 waves spill and run slower).
constexpr int kEncWavesPerSimd = 6;

// x / d for x, d < 2^16 by one multiply: with M = floor((2^32 - 1) / d) + 1, x * M / 2^32 exceeds
// x / d by less than x / 2^32 < 1 / d, which never crosses the next integer (exact when d is a
// power of two).  The block index math of the encode divides by the blocks per head row and the
// page size once per chunk; a division there costs a dozen instructions, this one two.
struct SmallDiv {
  uint64_t m;
  __device__ explicit SmallDiv(uint32_t d) : m(0xFFFFFFFFull / d + 1u) {}
  __device__ uint32_t operator()(uint32_t x) const { return (uint32_t)((x * m) >> 32); }
};

__global__ __launch_bounds__(kEncThreads, kEncWavesPerSimd) void enc_k(
    Geom g, SeqView s, const uint16_t* __restrict__ raw, uint8_t* __restrict__ sm, uint8_t* __restrict__ nib,
    uint8_t* __restrict__ base, uint32_t* __restrict__ row_flags, uint32_t* __restrict__ row_spill,
    uint8_t* __restrict__ spill, const uint64_t* spill_top, uint64_t spill_slots, uint64_t* look, uint32_t* failed,
    uint32_t* status) {
  const int p = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int32_t L;
  int rows = rows_in_page(s, g, b, p, &L);
  if (rows < 0) {
    if (p == 0 && tid == 0) set_status(status, ZF_DEV_ELEN);
    return;  // the sequence counts as empty
  }
  if (rows == 0) {  // past the sequence's end: no page, no word, no K
    if (s.kmax && tid < g.H) s.kmax[kmax_at(s, g.H, b, tid, p)] = 0u;
    return;
  }
  const int32_t pid = s.pt[(int64_t)b * s.maxp + p];
  if (pid < 0 || pid >= g.P) {
    if (tid == 0) set_status(status, ZF_DEV_EPAGE);
    rows = 0;  // the page counts no raw block and writes nothing, but still takes part
  }

  __shared__ uint32_t s_flags[64], s_first[64];
  __shared__ uint32_t s_kmax[16];  // per kv head: the largest exponent field of the page's K rows
  if (tid < 64) s_flags[tid] = 0u;
  if (tid < 16) s_kmax[tid] = 0u;
  __syncthreads();

  const int nb = g.nb();
  const int blocks = 2 * g.H * g.T * nb;
  const int chunks = blocks * 4;  // 16 values each; chunk k: block k / 4, quarter k % 4
  const int64_t page0 = (int64_t)(rows > 0 ? pid : 0) * g.vals_per_page();
  const SmallDiv div_nb((uint32_t)nb), div_t((uint32_t)g.T);
  // block m of the page: half m % nb of head row rest = m / nb, which is slot rest % T of
  // K/V head row hk = rest / T
  auto slot_of_block = [&](int m) {
    const int rest = (int)div_nb((uint32_t)m);
    return rest - (int)div_t((uint32_t)rest) * g.T;
  };
  auto live = [&](int k) { return k < chunks && slot_of_block(k >> 2) < rows; };
  // Classify chunks k0 + kEncThreads u (u < kEncUnroll): loads first, then per chunk its 16 exponents,
  // the block's window over its 4 lanes (uniform over them), the planes and the row flag bit.
  // hio[u]: the chunk's spill nibbles (raw blocks); the return value: which chunks are raw.
  // (The loads and the bases' stores sit under no branch, so the compiler's waits before each
  // chunk's classification count only the loads it needs, never this lane's earlier stores:
  // encode of 4 x 131072 rows 928 -> 907 us.)
  auto classify = [&](int k0, uint2 (&hio)[kEncUnroll]) -> uint32_t {
    uint4 lo[kEncUnroll], hi[kEncUnroll];
#pragma unroll
    for (int u = 0; u < kEncUnroll; ++u) {  // a chunk outside the rows loads chunk 0 and drops it
      const int k = live(k0 + kEncThreads * u) ? k0 + kEncThreads * u : 0;
      const uint4* src = reinterpret_cast<const uint4*>(raw + page0 + (int64_t)(k >> 2) * kBlock + (k & 3) * 16);
      lo[u] = ld_stream16(src);
      hi[u] = ld_stream16(src + 1);
    }
    uint32_t raw_mask = 0u;
#pragma unroll
    for (int u = 0; u < kEncUnroll; ++u) {
      const int k = k0 + kEncThreads * u, m = k >> 2, qtr = k & 3;
      hio[u] = make_uint2(0u, 0u);
      if (!live(k)) continue;  // uniform over the 4 lanes of the block
      const uint32_t w0[4] = {lo[u].x, lo[u].y, lo[u].z, lo[u].w};
      const uint32_t w1[4] = {hi[u].x, hi[u].y, hi[u].z, hi[u].w};
      Window a = window8(w0);
      const Window c = window8(w1);
      a.emin = min(a.emin, c.emin);
      a.emax = max(a.emax, c.emax);
#pragma unroll
      for (int o = 1; o < 4; o <<= 1) {
        a.emin = min(a.emin, (uint32_t)__shfl_xor((int)a.emin, o, 4));
        a.emax = max(a.emax, (uint32_t)__shfl_xor((int)a.emax, o, 4));
      }
      const uint32_t raw_blk = is_raw(a);
      const uint32_t bexp = raw_blk ? 0u : a.emin;
      uint32_t sm0[2], sm1[2], n0, n1;
      pack8(w0, bexp, raw_blk, sm0, n0, hio[u].x);
      pack8(w1, bexp, raw_blk, sm1, n1, hio[u].y);
      const int64_t v0 = page0 + (int64_t)m * kBlock + qtr * 16;
      st_stream16(sm + v0, sm0[0], sm0[1], sm1[0], sm1[1]);
      st_stream8(nib + (v0 >> 1), n0, n1);
      raw_mask |= raw_blk << u;
      base[v0 / kBlock] = (uint8_t)bexp;  // the block's 4 lanes store the same byte
      if (qtr == 0) {
        const int rest = (int)div_nb((uint32_t)m), half = m - rest * nb;
        const int hk = (int)div_t((uint32_t)rest), slot = rest - hk * g.T;
        if (raw_blk) atomicOr(&s_flags[slot], 1u << (hk * nb + half));
        if (!(hk & 1)) atomicMax(&s_kmax[hk >> 1], a.emax);
      }
    }
    return raw_mask;
  };
  __shared__ uint2 s_hik[kEncSweeps][kEncThreads];  // LDS, not registers: more workgroups per CU
  uint32_t rawm = 0u;
#pragma unroll
  for (int gi = 0; gi < kEncSweeps / kEncUnroll; ++gi) {
    uint2 h[kEncUnroll];
    rawm |= classify(tid + kEncThreads * kEncUnroll * gi, h) << (kEncUnroll * gi);
#pragma unroll
    for (int u = 0; u < kEncUnroll; ++u) s_hik[kEncUnroll * gi + u][tid] = h[u];
  }
  for (int k0 = tid + kEncThreads * kEncSweeps; k0 < chunks; k0 += kEncThreads * kEncUnroll) {  // larger pages
    uint2 h[kEncUnroll];
    classify(k0, h);
  }
  __syncthreads();

  if (s.kmax && tid < g.H) s.kmax[kmax_at(s, g.H, b, tid, p)] = s_kmax[tid];
  // wave 0: row flags, the page's raw count, its prefix by look-back, row_spill
  if (tid < 64) {
    const uint32_t f = tid < rows ? s_flags[tid] : 0u;
    if (tid < rows) row_flags[(int64_t)pid * g.T + tid] = f;
    const uint32_t c = __popc(f);
    uint32_t incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t up = __shfl_up((int)incl, o, 64);
      if (tid >= o) incl += up;
    }
    const uint32_t total = __shfl((int)incl, 63, 64);
    uint64_t* my_word = look + (int64_t)b * s.maxp + p;
    if (tid == 0) __hip_atomic_store(my_word, kLbAggregate | total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t fail = 0u;
    const uint64_t before = look_back(s, g, look, b, p, &fail);
    if (tid == 0) {
      __hip_atomic_store(my_word, kLbInclusive | (before + total), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (fail) atomicOr(failed, 1u);
    }
    const uint64_t first = before + (incl - c);  // offset from spill_top
    if (tid < rows) row_spill[(int64_t)pid * g.T + tid] = (uint32_t)(*spill_top + first);
    s_first[tid] = (uint32_t)first;
  }
  __syncthreads();

  // spill slots: 8 bytes per chunk of a raw block
  const uint64_t top = *spill_top;
  auto slot_of = [&](int m) -> uint64_t {
    const int rest = (int)div_nb((uint32_t)m), half = m - rest * nb;
    const int hk = (int)div_t((uint32_t)rest), slot = rest - hk * g.T;
    const int j = hk * nb + half;
    return top + s_first[slot] + __popc(s_flags[slot] & ((1u << j) - 1u));
  };
#pragma unroll
  for (int i = 0; i < kEncSweeps; ++i) {
    if (!((rawm >> i) & 1u)) continue;
    const int k = tid + kEncThreads * i;
    const uint64_t idx = slot_of(k >> 2);
    if (idx < spill_slots)  // a pool too small for the call: slots past its end are skipped
      *reinterpret_cast<uint2*>(spill + idx * 32u + (k & 3) * 8) = s_hik[i][tid];
  }
  for (int k = tid + kEncThreads * kEncSweeps; k < chunks; k += kEncThreads) {  // larger pages
    const int m = k >> 2, rest = (int)div_nb((uint32_t)m), half = m - rest * nb;
    const int hk = (int)div_t((uint32_t)rest), slot = rest - hk * g.T;
    if (slot >= rows || !((s_flags[slot] >> (hk * nb + half)) & 1u)) continue;
    const uint64_t idx = slot_of(m);
    if (idx >= spill_slots) continue;
    const uint4* src = reinterpret_cast<const uint4*>(raw + page0 + (int64_t)m * kBlock + (k & 3) * 16);
    uint32_t hv[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const uint4 in = src[h2];
      const uint32_t w[4] = {in.x, in.y, in.z, in.w};
      hv[h2] = 0u;
#pragma unroll
      for (int v = 0; v < 8; ++v) hv[h2] |= (exp_of(w[v >> 1] >> (16 * (v & 1))) >> 4) << (4 * v);
    }
    *reinterpret_cast<uint2*>(spill + idx * 32u + (k & 3) * 8) = make_uint2(hv[0], hv[1]);
  }
}

// Ends an encode: spill_top += the raw blocks of all pages (the inclusive count of the last
// page that holds tokens) if the pool holds them, else ZF_DEV_ESPILL and spill_top kept;
// ZF_DEV_ESYNC instead if a look-back wait ran out.
__global__ void enc_finish_k(Geom g, SeqView s, const uint64_t* look, const uint32_t* failed,
                             uint64_t* spill_top, uint64_t spill_slots, uint32_t* status) {
  if (threadIdx.x != 0) return;
  if (*failed) {
    set_status(status, ZF_DEV_ESYNC);
    return;
  }
  uint64_t total = 0;
  for (int b = s.B - 1; b >= 0; --b) {
    const int np = pages_of(s, g, b);
    if (np > 0) {
      total = look[(int64_t)b * s.maxp + np - 1] & kLbValue;
      break;
    }
  }
  const uint64_t top = *spill_top;
  if (fits_in_pool(total, top, spill_slots)) *spill_top = top + total;
  else set_status(status, ZF_DEV_ESPILL);
}

// ------------------------------------------------------------------------------ encode: scan

// One workgroup.  Turns per-page raw counts into exclusive prefixes (offset by *top_in) in
// (sequence, page) order and stores the end in *top_out; flags the call as failed when the
// `spill_slots` slots of the target do not hold them.
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 8;

__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
  // Hillis-Steele over kScanThreads values in LDS (one value per thread).
  const int tid = threadIdx.x;
  s_tmp[tid] = v;
  __syncthreads();
  for (int o = 1; o < kScanThreads; o <<= 1) {
    uint32_t add = tid >= o ? s_tmp[tid - o] : 0u;
    __syncthreads();
    s_tmp[tid] += add;
    __syncthreads();
  }
  uint32_t incl = s_tmp[tid];
  *total = s_tmp[kScanThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kScanThreads) void enc_scan_k(Geom g, SeqView s,
                                                           uint32_t* __restrict__ page_count,
                                                           const uint64_t* top_in, uint64_t* top_out,
                                                           uint64_t spill_slots, uint32_t* ws_flag,
                                                           uint32_t* status) {
  extern __shared__ uint32_t s_off[];  // [B + 1] page offsets, then kScanThreads scratch
  uint32_t* s_tmp = s_off + s.B + 1;
  __shared__ uint32_t s_total;
  const int tid = threadIdx.x;
  // pages per sequence -> exclusive offsets (chunked over the batch)
  uint32_t carry = 0;
  for (int b0 = 0; b0 < s.B; b0 += kScanThreads) {
    int b = b0 + tid;
    uint32_t np = 0;
    if (b < s.B) {
      int32_t L = s.lens[b];
      if (L > 0 && (int64_t)L <= (int64_t)s.maxp * g.T) np = (uint32_t)((L + g.T - 1) / g.T);
    }
    uint32_t tot;
    uint32_t ex = block_exclusive_scan(np, s_tmp, &tot);
    if (b < s.B) s_off[b] = carry + ex;
    carry += tot;
  }
  if (tid == 0) s_off[s.B] = carry;
  __syncthreads();
  const uint32_t nchunks = s_off[s.B];
  const uint64_t top = *top_in;

  // two passes: total, then prefixes (only if the pool holds them)
  for (int pass = 0; pass < 2; ++pass) {
    uint64_t run = 0;
    for (uint32_t c0 = 0; c0 < nchunks; c0 += kScanThreads * kScanItems) {
      uint32_t vals[kScanItems];
      int64_t where[kScanItems];
      uint32_t mine = 0;
#pragma unroll
      for (int i = 0; i < kScanItems; ++i) {
        uint32_t c = c0 + (uint32_t)tid * kScanItems + i;
        vals[i] = 0;
        where[i] = -1;
        if (c < nchunks) {
          int lo = 0, hi = s.B - 1;  // last b with s_off[b] <= c
          while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= c) lo = mid; else hi = mid - 1;
          }
          where[i] = (int64_t)lo * s.maxp + (c - s_off[lo]);
          vals[i] = page_count[where[i]];
        }
        mine += vals[i];
      }
      uint32_t tot;
      uint32_t ex = block_exclusive_scan(mine, s_tmp, &tot);
      if (pass == 1) {
        uint64_t acc = top + run + ex;
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) {
          if (where[i] >= 0) page_count[where[i]] = (uint32_t)acc;
          acc += vals[i];
        }
      }
      run += tot;
    }
    if (pass == 0) {
      if (tid == 0) s_total = fits_in_pool(run, top, spill_slots) ? 0u : 1u;
      __syncthreads();
      if (s_total) {
        if (tid == 0) {
          *ws_flag = ZF_DEV_ESPILL;
          set_status(status, ZF_DEV_ESPILL);
        }
        return;
      }
      if (tid == 0) {
        *ws_flag = 0u;
        *top_out = top + run;
      }
    }
  }
}

// ------------------------------------------------------------------------------ append

// Append of n tokens per sequence; new row r = b * n + j is token j of sequence b, at position
// seq_lens[b] + j.  Packing: one workgroup per new row classifies its blocks and writes their
// sm/nib/base bytes and the row's flag word into the row's slot, which is not yet part of the
// sequence.  Commit: one workgroup validates every row, scans the rows' raw counts in row order
// ((sequence, token) order), and only if all of them fit in the spill pool writes the spill
// slots and row_spill and advances seq_lens and spill_top.  So a failed append changes no
// defined state: only slots at positions seq_lens[b] and later may be touched.
//
// Two forms.  Two launches: append_pack_k, then append_commit_k, which reads the flag words
// back from row_flags.  One launch (append_one_k, when the cache has sync words and there are
// at most 64 new rows): R packing workgroups and one commit workgroup (the last), handing
// their flag words to each other by decoupled look-back.  Packing workgroup r publishes one
// 64-bit word, its row's flag word and error bits tagged with the call's epoch (a counter in
// the sync area), stored only after its loads of the epoch, its length and spill_top have
// returned.  It then waits only for the words of rows 0 .. r-1, which take its prefix (their
// raw blocks) and their error bits, writes its spill slots and row_spill from spill_top plus
// that prefix, and marks its word done.  These writes land in slots that hold nothing yet
// (positions seq_lens[b] and later, spill slots from spill_top on, below spill_slots), so they
// are harmless if the call fails.  The commit waits until all R words are marked done, takes
// the all-or-nothing decision, and advances seq_lens and spill_top (every length was read
// before its word was stored); it always advances the epoch, so no word of this call can match
// the next one.  Every wait is for lower-numbered workgroups, which are dispatched first, so
// every wait ends without any assumption of co-residency.  A packing workgroup that still gives
// up waiting marks its word abandoned instead, and the commit then changes nothing
// (ZF_DEV_ESYNC).  Each word carries its data itself, so no fence orders it after other stores.
constexpr int kAppendThreads = 1024;
constexpr int kAppendMaxRows = 4096;  // two u32 per row in LDS (beyond: the grouped form)
constexpr int kAppendChunkedMaxRows = 1 << 24;  // new rows of one call
constexpr int kOneMaxRows = 64;       // new rows of a one-launch append (sync words 0 .. 63; 64: epoch)
constexpr uint32_t kSyncPolls = 1u << 20;  // bound on each wait for the words (about 1 s)
constexpr int kSyncEpoch = kOneMaxRows;      // sync word holding the epoch
constexpr int kSyncGiveUp = kOneMaxRows + 1; // sync word: nonzero makes waiting packing
                                             // workgroups give up at once (forces ZF_DEV_ESYNC)
constexpr uint64_t kTagMod = (1u << 27) - 1u;

// Where new token j of sequence b (n per sequence) goes when its length was read as L: its
// page and slot, and row = pid * T + slot; row -1 (with the error bit) when the sequence cannot
// take them.
struct NewPos {
  int64_t row;
  int32_t pid, slot, lp;  // lp: the logical page of the sequence
};

__device__ __forceinline__ NewPos append_pos_at(const Geom& g, const SeqView& s, int b, int j, int n, int32_t L,
                                                uint32_t* err) {
  if (L < 0 || (int64_t)L + n > (int64_t)s.maxp * g.T || (int64_t)L + n > s.max_seq_len) {
    *err = ZF_DEV_ELEN;
    return NewPos{-1, 0, 0, 0};
  }
  const int32_t t = L + j, p = t / g.T, slot = t - p * g.T;
  const int32_t pid = s.pt[(int64_t)b * s.maxp + p];
  if (pid < 0 || pid >= g.P) {
    *err = ZF_DEV_EPAGE;
    return NewPos{-1, 0, 0, 0};
  }
  *err = 0;
  return NewPos{(int64_t)pid * g.T + slot, pid, slot, p};
}

__device__ __forceinline__ int64_t append_row_at(const Geom& g, const SeqView& s, int b, int j, int n,
                                                 int32_t L, uint32_t* err) {
  return append_pos_at(g, s, b, j, n, L, err).row;
}

__device__ __forceinline__ NewPos append_pos(const Geom& g, const SeqView& s, int b, int j, int n, uint32_t* err) {
  return append_pos_at(g, s, b, j, n, s.lens[b], err);
}

__device__ __forceinline__ int64_t append_row(const Geom& g, const SeqView& s, int b, int j, int n,
                                              uint32_t* err) {
  return append_pos(g, s, b, j, n, err).row;
}

// Block j of a new row, classified and packed in registers (8 lanes, 8 values each).
struct NewBlock {
  uint32_t sm0, sm1, nib, hi, bexp, raw, emax;
};

// New row r is u16 [H][D] of K and of V; block j covers half j % nb of head j / nb / 2, K or V
// by (j / nb) & 1, the order of the row's flag bits.  load_new: this lane's 8 values of it.
__device__ __forceinline__ uint4 load_new(const Geom& g, int r, int j, int lane8, const uint16_t* __restrict__ k_new,
                                          const uint16_t* __restrict__ v_new) {
  const int nb = g.nb(), half = j % nb, hk = j / nb, h = hk >> 1, kv = hk & 1;
  return *reinterpret_cast<const uint4*>((kv ? v_new : k_new) + ((int64_t)r * g.H + h) * g.D + half * kBlock +
                                         lane8 * 8);
}

// The block's window over its 8 lanes, then this lane's planes.
__device__ __forceinline__ NewBlock classify_loaded(const uint4 in) {
  const uint32_t w[4] = {in.x, in.y, in.z, in.w};
  Window win = window8(w);
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    win.emin = min(win.emin, (uint32_t)__shfl_xor((int)win.emin, o, 8));
    win.emax = max(win.emax, (uint32_t)__shfl_xor((int)win.emax, o, 8));
  }
  NewBlock o;
  o.emax = win.emax;
  o.raw = is_raw(win);
  o.bexp = o.raw ? 0u : win.emin;
  uint32_t smw[2];
  pack8(w, o.bexp, o.raw, smw, o.nib, o.hi);
  o.sm0 = smw[0];
  o.sm1 = smw[1];
  return o;
}

__device__ __forceinline__ NewBlock classify_new(const Geom& g, int r, int j, int lane8,
                                                 const uint16_t* __restrict__ k_new,
                                                 const uint16_t* __restrict__ v_new) {
  return classify_loaded(load_new(g, r, j, lane8, k_new, v_new));
}

__device__ __forceinline__ void store_new(const Geom& g, const NewPos& at, int j, int lane8, const NewBlock& o,
                                          uint8_t* sm, uint8_t* nib, uint8_t* base) {
  const int nb = g.nb(), half = j % nb, hk = j / nb, h = hk >> 1, kv = hk & 1;
  const int64_t v0 = (((int64_t)at.pid * g.H + h) * 2 + kv) * g.T * g.D + (int64_t)at.slot * g.D + half * kBlock +
                     lane8 * 8;
  *reinterpret_cast<uint2*>(sm + v0) = make_uint2(o.sm0, o.sm1);
  *reinterpret_cast<uint32_t*>(nib + (v0 >> 1)) = o.nib;
  if (lane8 == 0) base[v0 / kBlock] = (uint8_t)o.bexp;
}

// The row's flag word (bit j = block j raw) from the blocks the workgroup classified (block j on
// threads 8j .. 8j + 7; the row has at most 32 blocks).  Every thread gets it.
__device__ __forceinline__ uint32_t row_flag_word(bool has, int j, int lane8, uint32_t raw) {
  __shared__ uint32_t s_f;
  if (threadIdx.x == 0) s_f = 0u;
  __syncthreads();
  if (has && lane8 == 0 && raw) atomicOr(&s_f, 1u << j);
  __syncthreads();
  return s_f;
}

// Grouped form of the append (below): rows per group, and the flags of a group's look-back word.
constexpr int kGroupRows = 16;
constexpr uint32_t kGlAggregate = 1u << 30;
constexpr uint32_t kGlInclusive = 2u << 30;
constexpr uint32_t kGlValue = (1u << 30) - 1u;  // raw blocks of a call: <= 2^24 rows x 32 < 2^30

// kPackRows new rows per workgroup, two at a time: 4 lanes per 64-value block, 16 values each
// (two 16-byte loads), so a row takes at most 128 lanes (32 blocks).  Every row's loads go out
// together, before the lookups of the rows' pages (dependent scalar round trips): the new
// values do not depend on where they go.  words: the grouped form's look-back words (the
// row_spill entries of each group's first row, which hold nothing yet), cleared here.
template <int kPackRows>
__global__ __launch_bounds__(256) void append_pack_k(Geom g, SeqView s, int n, const uint16_t* __restrict__ k_new,
                                                     const uint16_t* __restrict__ v_new, uint8_t* sm,
                                                     uint8_t* nib, uint8_t* base, uint32_t* row_flags,
                                                     uint32_t* words) {
  static_assert(kPackRows % 2 == 0, "two rows per pass");
  constexpr int kPasses = kPackRows / 2;
  const int R = s.B * n, r0 = blockIdx.x * kPackRows, tid = threadIdx.x;
  const int second = tid >> 7, j = (tid >> 2) & 31, qtr = tid & 3;  // row 2p + second of pass p
  const int nb = g.nb(), half = j % nb, hk = j / nb, h = hk >> 1, kv = hk & 1;
  const bool has = j < g.blocks_per_row();
  __shared__ uint32_t s_f[kPackRows];
  if (tid < kPackRows) s_f[tid] = 0u;
  uint4 lo[kPasses], hi[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int r = r0 + 2 * p + second;
    if (has && r < R) {
      const uint4* src = reinterpret_cast<const uint4*>((kv ? v_new : k_new) + ((int64_t)r * g.H + h) * g.D +
                                                        half * kBlock + qtr * 16);
      lo[p] = src[0];
      hi[p] = src[1];
    }
  }
  int32_t L[kPackRows];  // the lengths first, then the page-table entries they lead to
#pragma unroll
  for (int i = 0; i < kPackRows; ++i) L[i] = r0 + i < R ? s.lens[(r0 + i) / n] : 0;
  NewPos at[kPackRows];
#pragma unroll
  for (int i = 0; i < kPackRows; ++i) {
    const int r = r0 + i;
    at[i] = NewPos{-1, 0, 0, 0};  // past the last row, or a position the call cannot take
                               // (append_commit_k or append_group_finish_k reports it)
    if (r < R) {
      uint32_t err;
      at[i] = append_pos_at(g, s, r / n, r % n, n, L[i], &err);
    }
  }
  __syncthreads();  // s_f cleared
  uint32_t sm4[kPasses][4], nib2[kPasses][2], bexp[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const NewPos a = second ? at[2 * p + 1] : at[2 * p];
    if (!has || a.row < 0) continue;  // uniform over the block's 4 lanes
    const uint32_t w0[4] = {lo[p].x, lo[p].y, lo[p].z, lo[p].w};
    const uint32_t w1[4] = {hi[p].x, hi[p].y, hi[p].z, hi[p].w};
    Window wa = window8(w0);
    const Window wb = window8(w1);
    wa.emin = min(wa.emin, wb.emin);
    wa.emax = max(wa.emax, wb.emax);
#pragma unroll
    for (int o = 1; o < 4; o <<= 1) {
      wa.emin = min(wa.emin, (uint32_t)__shfl_xor((int)wa.emin, o, 4));
      wa.emax = max(wa.emax, (uint32_t)__shfl_xor((int)wa.emax, o, 4));
    }
    const uint32_t raw = is_raw(wa);
    if (qtr == 0 && !kv && s.kmax) atomicMax(&s.kmax[kmax_at(s, g.H, (r0 + 2 * p + second) / n, h, a.lp)], wa.emax);
    bexp[p] = raw ? 0u : wa.emin;
    uint32_t s0[2], s1[2], hio;
    pack8(w0, bexp[p], raw, s0, nib2[p][0], hio);
    pack8(w1, bexp[p], raw, s1, nib2[p][1], hio);
    sm4[p][0] = s0[0];
    sm4[p][1] = s0[1];
    sm4[p][2] = s1[0];
    sm4[p][3] = s1[1];
    if (qtr == 0 && raw) atomicOr(&s_f[2 * p + second], 1u << j);
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const NewPos a = second ? at[2 * p + 1] : at[2 * p];
    if (!has || a.row < 0) continue;
    const int64_t v0 = (((int64_t)a.pid * g.H + h) * 2 + kv) * g.T * g.D + (int64_t)a.slot * g.D + half * kBlock +
                       qtr * 16;
    *reinterpret_cast<uint4*>(sm + v0) = make_uint4(sm4[p][0], sm4[p][1], sm4[p][2], sm4[p][3]);
    *reinterpret_cast<uint2*>(nib + (v0 >> 1)) = make_uint2(nib2[p][0], nib2[p][1]);
    if (qtr == 0) base[v0 / kBlock] = (uint8_t)bexp[p];
  }
#pragma unroll
  for (int i = 0; i < kPackRows; ++i) {
    if (tid == i && at[i].row >= 0) {
      row_flags[at[i].row] = s_f[i];
      if (words && (r0 + i) % kGroupRows == 0) words[at[i].row] = 0u;
    }
  }
}

__global__ __launch_bounds__(kAppendThreads) void append_commit_k(Geom g, SeqView s, int n,
                                                                  const uint16_t* __restrict__ k_new,
                                                                  const uint16_t* __restrict__ v_new,
                                                                  const uint32_t* row_flags, uint32_t* row_spill,
                                                                  uint8_t* spill, uint64_t* spill_top,
                                                                  uint64_t spill_slots, uint32_t* status) {
  const int R = s.B * n;                 // new rows
  extern __shared__ uint32_t s_flags[];  // [R] row flags, then [R] exclusive prefixes
  uint32_t* s_pref = s_flags + R;
  __shared__ uint32_t s_err, s_total;
  const int tid = threadIdx.x;
  if (tid == 0) s_err = 0u;
  __syncthreads();
  for (int r = tid; r < R; r += kAppendThreads) {
    uint32_t e;
    const int64_t row = append_row(g, s, r / n, r % n, n, &e);
    if (e) atomicOr(&s_err, e);
    else s_flags[r] = row_flags[row];
  }
  __syncthreads();
  if (s_err) {
    if (tid == 0) set_status(status, s_err);
    return;
  }
  // exclusive scan of raw counts in row order (one wave)
  if (tid < 64) {
    uint32_t carry = 0;
    for (int r0 = 0; r0 < R; r0 += 64) {
      const int r = r0 + tid;
      const uint32_t c = r < R ? __popc(s_flags[r]) : 0u;
      uint32_t incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t up = __shfl_up((int)incl, o, 64);
        if (tid >= o) incl += up;
      }
      if (r < R) s_pref[r] = carry + incl - c;
      carry += __shfl((int)incl, 63, 64);
    }
    if (tid == 0) s_total = carry;
  }
  __syncthreads();
  const uint64_t top = *spill_top;
  const uint32_t total = s_total;
  if (!fits_in_pool(total, top, spill_slots)) {
    if (tid == 0) set_status(status, ZF_DEV_ESPILL);
    return;
  }
  // spill slots of the raw blocks: 8 lanes per block, blocks walked in (row, block) order
  const int nb = g.nb(), D = g.D, H = g.H;
  const uint32_t rb = 2u * H * nb, nblk = (uint32_t)R * rb;
  const int lane8 = tid & 7;
#pragma unroll 4
  for (uint32_t m = tid >> 3; m < nblk; m += kAppendThreads >> 3) {
    const uint32_t r = m / rb, j = m - r * rb;
    const uint32_t f = s_flags[r];
    if (!((f >> j) & 1u)) continue;
    const uint32_t hk = j / nb, half = j - hk * nb, h = hk >> 1, kv = hk & 1;
    const uint4 in = *reinterpret_cast<const uint4*>((kv ? v_new : k_new) + ((int64_t)r * H + h) * D +
                                                     half * kBlock + lane8 * 8);
    const uint32_t w[4] = {in.x, in.y, in.z, in.w};
    uint32_t hi = 0u;
#pragma unroll
    for (int v = 0; v < 8; ++v) hi |= (exp_of(w[v >> 1] >> (16 * (v & 1))) >> 4) << (4 * v);
    const uint64_t idx = top + s_pref[r] + __popc(f & ((1u << j) - 1u));
    *reinterpret_cast<uint32_t*>(spill + idx * 32u + lane8 * 4) = hi;
  }
  for (int r = tid; r < R; r += kAppendThreads) {
    uint32_t e;
    const int64_t row = append_row(g, s, r / n, r % n, n, &e);
    row_spill[row] = (uint32_t)(top + s_pref[r]);
  }
  __syncthreads();  // every length has been read before any is advanced
  for (int b = tid; b < s.B; b += kAppendThreads) s.lens[b] += n;
  if (tid == 0) *spill_top = top + total;
}

// ------------------------------------------------------------------ append: grouped form
// For more new rows than one commit workgroup holds (prefill written in chunks, long
// speculative runs), three launches and no workspace.  The rows are taken in groups of
// kGroupRows in row order; each group's first row's row_spill entry (which holds nothing yet)
// serves as the group's look-back word: append_pack_k clears it, append_group_commit_k
// publishes the group's raw count there, takes the count of every earlier group by decoupled
// look-back, publishes the inclusive count, and writes the group's other row_spill entries and
// its spill slots; append_group_finish_k checks the whole call (lengths, page ids, every group's
// word complete, room in the pool) and only then writes the first rows' entries and advances
// seq_lens and spill_top.  Until that last step only slots that hold nothing yet are written
// (rows at positions seq_lens[b] and later, spill slots from spill_top on within the pool), so
// a failed call changes no defined state.  A group whose first row has an invalid position has
// no word: the groups after it count it as an inclusive 0 (their prefixes are then wrong, and
// the call fails in the last step).

// Raw blocks of every group before group G (called by one wave; the result in every lane).
// Lane l looks at group G - 1 - l; the walk stops at the nearest group with an inclusive count.
// Every group waited for comes earlier in the grid, so it has been dispatched and publishes
// without waiting for this one.  *failed is set if a wait ran out (the sum is then incomplete).
__device__ uint32_t group_look_back(const Geom& g, const SeqView& s, int n, const uint32_t* row_spill, int G,
                                    uint32_t* failed) {
  const int lane = threadIdx.x & 63;
  uint32_t sum = 0, ran_out = 0u;
  for (int hi = G - 1; hi >= 0; hi -= 64) {
    const int q = hi - lane;
    uint32_t w = kGlInclusive;  // before group 0, or a group without a word: a stop with 0
    if (q >= 0) {
      uint32_t e;
      const int r = q * kGroupRows;
      const int64_t row = append_row(g, s, r / n, r % n, n, &e);
      if (row >= 0) {
        for (uint32_t k = 0;; ++k) {
          w = __hip_atomic_load(&row_spill[row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((w >> 30) != 0u) break;
          if (k + 1 == kLbPolls) {
            ran_out = 1u;
            w = kGlAggregate;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
    }
    const uint64_t stop = __ballot((w >> 30) == 2u);
    const int k = stop ? __builtin_ctzll(stop) : 63;
    uint32_t v = lane <= k ? (w & kGlValue) : 0u;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += (uint32_t)__shfl_xor((int)v, o, 64);
    sum += v;
    if (stop) break;
  }
  if (__any(ran_out)) *failed = 1u;  // in every lane
  return sum;
}

// One group per workgroup: its look-back, its rows' row_spill entries (but the first row's)
// and its raw blocks' spill slots.  Wave 0 reads the rows' flag words and then walks the
// look-back; meanwhile waves 1..3 load the new values of the raw blocks (their slots need the
// prefix, their nibbles do not), 8 lanes per block, every load out at once.
constexpr int kCommitItems = 22;  // blocks per 8-lane group of waves 1..3: 24 groups x 22 >= 16 x 32

__global__ __launch_bounds__(256) void append_group_commit_k(
    Geom g, SeqView s, int n, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const uint32_t* __restrict__ row_flags, uint32_t* row_spill, uint8_t* spill, const uint64_t* spill_top,
    uint64_t spill_slots, const uint64_t* sync) {
  static_assert(24 * kCommitItems >= kGroupRows * 32, "waves 1..3 cover a group's blocks");
  __shared__ uint32_t s_flags[kGroupRows], s_first[kGroupRows];
  __shared__ uint64_t s_base;
  const int R = s.B * n, G = blockIdx.x, r0 = G * kGroupRows, tid = threadIdx.x;
  const int rows = min(kGroupRows, R - r0);
  uint32_t e0;
  const int64_t row0 = append_row(g, s, r0 / n, r0 % n, n, &e0);
  if (row0 < 0) return;  // no word: the call fails in the last step
  int64_t row = -1;
  uint32_t f = 0u;
  if (tid < rows) {
    uint32_t e;
    const int r = r0 + tid;
    row = append_row(g, s, r / n, r % n, n, &e);
    if (row >= 0) f = row_flags[row];
  }
  if (tid < kGroupRows) s_flags[tid] = f;
  __syncthreads();
  const int nb = g.nb(), D = g.D, H = g.H;
  const uint32_t rb = 2u * H * nb, nblk = (uint32_t)rows * rb;
  const int lane8 = tid & 7, grp = (tid - 64) >> 3;  // waves 1..3: 24 groups of 8 lanes
  uint4 in[kCommitItems];
  uint32_t take = 0u;  // bit u: item u is a raw block's piece
  if (tid >= 64) {
#pragma unroll
    for (int u = 0; u < kCommitItems; ++u) {
      const uint32_t m = (uint32_t)grp + 24u * u;
      if (m >= nblk) continue;
      const uint32_t i = m / rb, j = m - i * rb;
      if (!((s_flags[i] >> j) & 1u)) continue;
      take |= 1u << u;
      const uint32_t hk = j / nb, half = j - hk * nb, h = hk >> 1, kv = hk & 1;
      in[u] = *reinterpret_cast<const uint4*>((kv ? v_new : k_new) + ((int64_t)(r0 + i) * H + h) * D + half * kBlock +
                                              lane8 * 8);
    }
  } else {
    const uint32_t c = __popc(f);
    uint32_t incl = c;
#pragma unroll
    for (int o = 1; o < kGroupRows; o <<= 1) {
      const uint32_t up = (uint32_t)__shfl_up((int)incl, o, 64);
      if (tid >= o) incl += up;
    }
    const uint32_t total = (uint32_t)__shfl((int)incl, kGroupRows - 1, 64);
    if (tid == 0) __hip_atomic_store(&row_spill[row0], kGlAggregate | total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the cache's give-up hook (a test of the failure path): every group with groups before it
    // acts as if its wait had run out
    uint32_t failed = G > 0 && sync && sync[kSyncGiveUp] != 0u ? 1u : 0u;
    const uint32_t before = failed ? 0u : group_look_back(g, s, n, row_spill, G, &failed);
    if (tid == 0) {
      // a wait that ran out leaves the word at its aggregate: the last step then fails the call
      if (!failed) __hip_atomic_store(&row_spill[row0], kGlInclusive | (before + total), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_base = *spill_top + before;
    }
    const uint32_t ex = incl - c;
    if (tid < kGroupRows) s_first[tid] = ex;
    if (tid > 0 && row >= 0) row_spill[row] = (uint32_t)(*spill_top + before + ex);
  }
  __syncthreads();
  if (tid < 64) return;
  const uint64_t base = s_base;
#pragma unroll
  for (int u = 0; u < kCommitItems; ++u) {
    if (!((take >> u) & 1u)) continue;
    const uint32_t m = (uint32_t)grp + 24u * u, i = m / rb, j = m - i * rb;
    const uint64_t idx = base + s_first[i] + __popc(s_flags[i] & ((1u << j) - 1u));
    if (idx >= spill_slots) continue;  // a slot past the pool: the call fails in the last step
    const uint32_t w[4] = {in[u].x, in[u].y, in[u].z, in[u].w};
    uint32_t hi = 0u;
#pragma unroll
    for (int v = 0; v < 8; ++v) hi |= (exp_of(w[v >> 1] >> (16 * (v & 1))) >> 4) << (4 * v);
    *reinterpret_cast<uint32_t*>(spill + idx * 32u + lane8 * 4) = hi;
  }
}

// The last step of the grouped form (one workgroup): every sequence's length and the page ids
// of its new rows, every group's word complete, then room in the pool; on success the first
// rows' row_spill entries, seq_lens and spill_top.
__global__ __launch_bounds__(kScanThreads) void append_group_finish_k(Geom g, SeqView s, int n,
                                                                      uint32_t* row_spill, uint64_t* spill_top,
                                                                      uint64_t spill_slots, uint32_t* status) {
  __shared__ uint32_t s_err, s_total;
  const int tid = threadIdx.x, R = s.B * n, ngroups = (R + kGroupRows - 1) / kGroupRows;
  if (tid == 0) {
    s_err = 0u;
    s_total = 0u;
  }
  __syncthreads();
  // 32 threads per sequence check the page ids of its new rows
  uint32_t err = 0u;
  for (int b = tid >> 5; b < s.B; b += kScanThreads >> 5) {
    const int32_t L = s.lens[b];
    if (L < 0 || (int64_t)L + n > (int64_t)s.maxp * g.T || (int64_t)L + n > s.max_seq_len) {
      err |= ZF_DEV_ELEN;
      continue;
    }
    const int p_lo = L / g.T, p_hi = (L + n - 1) / g.T;
    for (int p = p_lo + (tid & 31); p <= p_hi; p += 32) {
      const int32_t pid = s.pt[(int64_t)b * s.maxp + p];
      if (pid < 0 || pid >= g.P) err |= ZF_DEV_EPAGE;
    }
  }
  // every group's word inclusive (a look-back that ran out left one at its aggregate); the last
  // group's value is the call's total
  for (int G = tid; G < ngroups; G += kScanThreads) {
    uint32_t e;
    const int r = G * kGroupRows;
    const int64_t row = append_row(g, s, r / n, r % n, n, &e);
    if (row < 0) continue;  // reported above
    const uint32_t w = row_spill[row];
    if ((w >> 30) != 2u) err |= ZF_DEV_ESYNC;
    if (G == ngroups - 1) s_total = w & kGlValue;
  }
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  const uint64_t top = *spill_top, total = s_total;
  if (s_err) {
    if (tid == 0) set_status(status, s_err);
    return;
  }
  if (!fits_in_pool(total, top, spill_slots)) {
    if (tid == 0) set_status(status, ZF_DEV_ESPILL);
    return;
  }
  // first rows: a group's exclusive prefix is the inclusive count of the group before it; each
  // pass reads its groups' words before any of them is rewritten, and carries the last one on
  __shared__ uint32_t s_incl[kScanThreads], s_prev;
  if (tid == 0) s_prev = 0u;
  for (int G0 = 0; G0 < ngroups; G0 += kScanThreads) {
    const int G = G0 + tid;
    int64_t row = -1;
    uint32_t incl = 0u;
    if (G < ngroups) {
      uint32_t e;
      const int r = G * kGroupRows;
      row = append_row(g, s, r / n, r % n, n, &e);
      incl = row_spill[row] & kGlValue;
    }
    s_incl[tid] = incl;
    __syncthreads();
    const uint32_t ex = tid == 0 ? s_prev : s_incl[tid - 1];
    __syncthreads();  // every thread has its prefix before s_prev moves on
    if (row >= 0) row_spill[row] = (uint32_t)(top + ex);
    if (tid == kScanThreads - 1) s_prev = incl;
  }
  __syncthreads();  // every length was read above
  for (int b = tid; b < s.B; b += kScanThreads) s.lens[b] += n;
  if (tid == 0) *spill_top = top + total;
}

// Tag of a hand-over word published under epoch E: never 0, and different for consecutive
// epochs (a word left by an earlier call never matches).
__device__ __forceinline__ uint32_t sync_tag(uint64_t E) { return (uint32_t)(E % kTagMod) + 1u; }

// Hand-over word of one new row: tag << 37 | abandoned << 36 | done << 35 | error bits << 32 |
// flag word.  done: the row's workgroup has its prefix and has written its spill slots;
// abandoned: it gave up waiting for the rows before it.
__device__ __forceinline__ uint32_t word_tag(uint64_t w) { return (uint32_t)(w >> 37); }
constexpr uint64_t kDone = (uint64_t)1 << 35;
constexpr uint64_t kAbandoned = (uint64_t)1 << 36;
__device__ __forceinline__ uint64_t hand_over_word(uint32_t tag, uint32_t err, uint32_t flags) {
  return ((uint64_t)tag << 37) | ((uint64_t)err << 32) | flags;
}

// What a workgroup learns from the hand-over words of rows 0 .. n-1 (wave 0 polls them, lane
// i word i): whether all arrived (with the done or abandoned mark when `final`), their raw
// blocks, their error bits, and whether one was abandoned.
struct HandOver {
  uint32_t seen, err, total, abandoned;
};

__device__ __forceinline__ HandOver read_hand_over(const uint64_t* sync, int n, uint32_t tag, bool final,
                                                   uint32_t polls) {
  __shared__ HandOver s_h;
  const int tid = threadIdx.x;
  if (tid < 64) {
    uint64_t w = 0u;
    bool ok = tid >= n;
    for (uint32_t p = 0; !ok && p < polls; ++p) {
      w = __hip_atomic_load(&sync[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok = word_tag(w) == tag && (!final || (w & (kDone | kAbandoned)));
      if (!ok) __builtin_amdgcn_s_sleep(2);
    }
    uint32_t cnt = tid < n ? __popc((uint32_t)w) : 0u, err = tid < n ? (uint32_t)(w >> 32) & 7u : 0u;
    uint32_t miss = ok ? 0u : 1u, ab = tid < n && (w & kAbandoned) ? 1u : 0u;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      cnt += (uint32_t)__shfl_xor((int)cnt, o, 64);
      err |= (uint32_t)__shfl_xor((int)err, o, 64);
      miss |= (uint32_t)__shfl_xor((int)miss, o, 64);
      ab |= (uint32_t)__shfl_xor((int)ab, o, 64);
    }
    if (tid == 0) {
      s_h.total = cnt;
      s_h.err = err;
      s_h.seen = miss == 0u;
      s_h.abandoned = ab;
    }
  }
  __syncthreads();
  return s_h;
}

// Commit workgroup of the one-launch append: once every row's word carries this call's tag and
// its done (or abandoned) mark, it advances seq_lens and spill_top if the call succeeded, and
// moves to the next epoch in every case.
__device__ void commit_one(const SeqView& s, int n, uint64_t* spill_top, uint64_t spill_slots,
                           uint32_t* status, uint64_t* sync) {
  const int R = s.B * n, tid = threadIdx.x;
  const uint64_t E = sync[kSyncEpoch];  // written only by an earlier launch: a plain load
  const uint64_t top = *spill_top;
  const int32_t L = tid < s.B ? s.lens[tid] : 0;
  const HandOver h = read_hand_over(sync, R, sync_tag(E), true, kSyncPolls);
  const bool fits = fits_in_pool(h.total, top, spill_slots);
  if (tid == 0) {
    const uint32_t e = !h.seen || h.abandoned ? ZF_DEV_ESYNC : h.err ? h.err : fits ? 0u : ZF_DEV_ESPILL;
    set_status(status, e);
  }
  if (h.seen && !h.abandoned && !h.err && fits) {
    if (tid < s.B) s.lens[tid] = L + n;  // every packing workgroup read its length before its word
    if (tid == 0) *spill_top = top + h.total;
  }
  if (tid == 0) __hip_atomic_store(&sync[kSyncEpoch], E + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One-launch append: workgroups 0 .. R-1 pack new row blockIdx.x, workgroup R commits.
__global__ __launch_bounds__(256) void append_one_k(Geom g, SeqView s, int n, const uint16_t* __restrict__ k_new,
                                                    const uint16_t* __restrict__ v_new, uint8_t* sm,
                                                    uint8_t* nib, uint8_t* base, uint32_t* row_flags,
                                                    uint32_t* row_spill, uint8_t* spill, uint64_t* spill_top,
                                                    uint64_t spill_slots, uint32_t* status, uint64_t* sync) {
  const int R = s.B * n, r = blockIdx.x, tid = threadIdx.x, j = tid >> 3, lane8 = tid & 7;
  if (r == R) {
    commit_one(s, n, spill_top, spill_slots, status, sync);
    return;
  }
  const bool has = j < g.blocks_per_row();
  // the new values do not depend on where they go: their loads go out before the lookups
  // (unconditionally, from block 0 on lanes past the row's blocks: a load inside a branch is
  // waited for at the branch's end)
  const uint4 in = load_new(g, r, has ? j : 0, lane8, k_new, v_new);
  const uint64_t E = sync[kSyncEpoch];
  const uint32_t tag = sync_tag(E);
  const uint64_t top = *spill_top;
  const int b = r / n;
  uint32_t err;
  const NewPos at = append_pos(g, s, b, r - b * n, n, &err);
  const int64_t row = at.row;
  NewBlock o{};
  if (has) o = classify_loaded(in);
  const uint32_t f = row_flag_word(has, j, lane8, o.raw);
  if (tid == 0) {
    // the word is built from the epoch, the length (through err and row) and spill_top as
    // loaded, so it cannot be stored before those loads have returned
    uint32_t t = tag;
    asm volatile("" : "+v"(t) : "v"((uint32_t)row), "v"((uint32_t)top));
    __hip_atomic_store(&sync[r], hand_over_word(t, err, f), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (row >= 0) {
    if (has) store_new(g, at, j, lane8, o, sm, nib, base);
    if (tid == 0) row_flags[row] = f;
    const int hk = j / g.nb();
    if (has && lane8 == 0 && !(hk & 1) && s.kmax) atomicMax(&s.kmax[kmax_at(s, g.H, b, hk >> 1, at.lp)], o.emax);
  }
  // the rows before this one: their raw blocks are this row's prefix
  const bool give_up = r > 0 && sync[kSyncGiveUp] != 0u;
  const HandOver h = read_hand_over(sync, r, tag, false, give_up ? 0u : kSyncPolls);
  if (!h.seen) {  // the commit sees the mark and changes nothing
    if (tid == 0)
      __hip_atomic_store(&sync[r], hand_over_word(tag, err, f) | kAbandoned, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // A call that has already failed writes nothing more; otherwise the slots are written even if
  // a later row still makes the call fail (they hold nothing yet), within the pool
  if (!err && !h.err && row >= 0 && fits_in_pool(h.total + __popc(f), top, spill_slots)) {
    const uint64_t first_slot = top + h.total;
    if (has && o.raw) {
      const uint64_t slot = first_slot + __popc(f & ((1u << j) - 1u));
      *reinterpret_cast<uint32_t*>(spill + slot * 32u + lane8 * 4) = o.hi;
    }
    if (tid == 0) row_spill[row] = (uint32_t)first_slot;
  }
  if (tid == 0)
    __hip_atomic_store(&sync[r], hand_over_word(tag, err, f) | kDone, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------------ decode

// One workgroup per (sequence, logical page).  Each lane rebuilds 8 values (an eighth of a
// block) per step from 8 sm bytes, 4 nibble bytes and, for a raw block, 4 spill bytes, and
// writes 16 bytes; consecutive lanes take consecutive steps, so every load and every store
// instruction covers one contiguous run of the page.  Four steps per lane are unrolled so their
// loads fly together, and 1024 lanes cover a 16-token, 8-head page in one such round, so no
// lane waits for its own stores before loading again.  The page's row flags, spill indices and
// block bases go to LDS first, and the planes of the lane's first round, which need none of
// them, are loaded beside them: the page costs two round trips (metadata and planes, then
// spill bytes) before its values are written.  Measured on 4 x 131072 rows (the same bytes
// throughout): 16 values per step, 256 lanes in two rounds 855 us; one round of 512 lanes
// 742 us, its two 16-byte stores per lane leaving holes that the streaming stores wrote back
// as partial lines (5 % more bytes written); 8 values per step, 8 steps of 512 lanes 698 us
// (96 VGPRs, 5 waves per SIMD); this form 677 us (56 VGPRs, 8 waves per SIMD), the rate of
// the library's streaming copy, with the counters at 1.00x the algorithmic bytes.
constexpr int kDecSteps = 4;
constexpr int kDecThreads = 1024;  // 4 steps of 8 values per lane: one round covers a 16 x 8 x 128 page
constexpr int kMaxPageBlocks = 32 * 64;  // 32 blocks per row, 64 rows per page at most

__global__ __launch_bounds__(kDecThreads) void decode_k(Geom g, SeqView s, const uint8_t* __restrict__ sm,
                                                const uint8_t* __restrict__ nib, const uint8_t* __restrict__ base,
                                                const uint32_t* __restrict__ row_flags,
                                                const uint32_t* __restrict__ row_spill,
                                                const uint8_t* __restrict__ spill, uint64_t spill_slots,
                                                uint16_t* __restrict__ out, uint32_t* status) {
  const int p = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int32_t L;
  const int rows = rows_in_page(s, g, b, p, &L);
  if (rows < 0) {
    if (p == 0 && tid == 0) set_status(status, ZF_DEV_ELEN);
    return;
  }
  if (rows == 0) return;
  const int32_t pid = s.pt[(int64_t)b * s.maxp + p];
  if (pid < 0 || pid >= g.P) {
    if (tid == 0) set_status(status, ZF_DEV_EPAGE);
    return;
  }
  const int nb = g.nb();
  const int blocks = 2 * g.H * g.T * nb;
  const int64_t page0 = (int64_t)pid * g.vals_per_page();
  const int steps = blocks * 8;  // 8 values each
  // step k: eighth k & 7 of block m = k >> 3, which is half m % nb of head row m / nb, slot
  // (m / nb) % T of it
  const SmallDiv div_nb((uint32_t)nb), div_t((uint32_t)g.T);
  auto slot_of_block = [&](int m) {
    const int rest = (int)div_nb((uint32_t)m);
    return rest - (int)div_t((uint32_t)rest) * g.T;
  };
  // A full page whose steps fill whole rounds (every page but a sequence's last, at the usual
  // geometries) runs without any per-step test: with no load or store under a branch, the
  // compiler's waits count exactly the accesses they need and never wait for stores.
  const bool full = rows == g.T && steps % (kDecThreads * kDecSteps) == 0;
  auto live_at = [&](int k, auto whole) {
    if constexpr (decltype(whole)::value) return true;
    else return k < steps && slot_of_block(k >> 3) < rows;
  };
  // Loads without branches (a step outside the page's rows reads step 0 instead and drops it),
  // so that the waits for the metadata below count exactly the loads issued after it.
  // the page's planes from one wave-uniform base each and a 32-bit lane offset (no 64-bit
  // address per load in VGPRs)
  const uint8_t* const sm_pg = sm + page0;
  const uint8_t* const nib_pg = nib + page0 / 2;
  uint16_t* const out_pg = out + page0;
  auto load_planes = [&](int k0, uint2 (&smw)[kDecSteps], uint32_t (&nibw)[kDecSteps], auto whole) {
#pragma unroll
    for (int u = 0; u < kDecSteps; ++u) {
      const uint32_t k = live_at(k0 + kDecThreads * u, whole) ? (uint32_t)(k0 + kDecThreads * u) : 0u;
      smw[u] = ld_stream8(sm_pg + k * 8u);
      nibw[u] = ld_stream4(nib_pg + k * 4u);
    }
  };
  __shared__ uint32_t s_f[64], s_sp[64];
  __shared__ __align__(4) uint8_t s_base[kMaxPageBlocks];
  const bool word_bases = (blocks & 3) == 0;  // the page's bases as 4-byte words
  const int64_t row0 = (int64_t)pid * g.T + min(tid, rows - 1);
  const uint32_t f_in = row_flags[row0], sp_in = row_spill[row0];
  const uint8_t* bsrc = base + (int64_t)pid * blocks;
  const uint32_t b_in = *(word_bases ? reinterpret_cast<const uint32_t*>(bsrc) + min(tid, blocks / 4 - 1) : &row_flags[row0]);
  uint2 smw[kDecSteps];
  uint32_t nibw[kDecSteps];
  if (full) load_planes(tid, smw, nibw, std::true_type{});
  else load_planes(tid, smw, nibw, std::false_type{});
  if (tid < rows) {
    s_f[tid] = f_in;
    s_sp[tid] = sp_in;
  }
  if (word_bases) {
    uint32_t* s_bw = reinterpret_cast<uint32_t*>(s_base);
    if (tid < blocks / 4) s_bw[tid] = b_in;
    for (int m = tid + kDecThreads; m < blocks / 4; m += kDecThreads) s_bw[m] = reinterpret_cast<const uint32_t*>(bsrc)[m];
  } else {
    for (int m = tid; m < blocks; m += kDecThreads) s_base[m] = bsrc[m];
  }
  __syncthreads();
  uint32_t err = 0;
  auto rounds = [&](auto whole) {
    for (int k0 = tid; k0 < steps; k0 += kDecThreads * kDecSteps) {
      if (k0 != tid) load_planes(k0, smw, nibw, whole);
      // spill loads without branches as well (a block that is not raw reads the page's first
      // sm bytes and drops them), so a round's go out together and are waited for once
      uint32_t hiw[kDecSteps], bp[kDecSteps];
      bool spilled[kDecSteps];
#pragma unroll
      for (int u = 0; u < kDecSteps; ++u) {
        const int k = k0 + kDecThreads * u;
        const bool live = live_at(k, whole);
        const int m = live ? k >> 3 : 0, e8 = k & 7;
        const int rest = (int)div_nb((uint32_t)m), half = m - rest * nb;
        const int hk = (int)div_t((uint32_t)rest), slot = rest - hk * g.T;
        const int j = hk * nb + half;
        const uint32_t f = s_f[slot];
        const bool raw = live && ((f >> j) & 1u);
        const uint64_t idx = (uint64_t)s_sp[slot] + __popc(f & ((1u << j) - 1u));
        spilled[u] = raw && idx < spill_slots;
        if (raw && !spilled[u]) err = ZF_DEV_ESPILL;
        hiw[u] = *reinterpret_cast<const uint32_t*>(spilled[u] ? spill + idx * 32u + e8 * 4 : sm_pg);
        bp[u] = raw ? 0u : (uint32_t)s_base[m] * 0x00010001u;
      }
#pragma unroll
      for (int u = 0; u < kDecSteps; ++u)
        if (!spilled[u]) hiw[u] = 0u;
#pragma unroll
      for (int u = 0; u < kDecSteps; ++u) {
        const int k = k0 + kDecThreads * u;
        if (!live_at(k, whole)) continue;
        uint32_t pr[4], w[4];
        rebuild8(smw[u].x, smw[u].y, nibw[u], hiw[u], bp[u], pr);
        pairs_to_natural(pr, w);
        st_stream16(out_pg + (uint32_t)k * 8u, w[0], w[1], w[2], w[3]);
      }
    }
  };
  if (full) rounds(std::true_type{});
  else rounds(std::false_type{});
  if (err) set_status(status, err);
}

// ------------------------------------------------------------------------------ compaction

// Spill compaction for the sequences passed in: their raw blocks move to slots 0, 1, ... in
// (sequence, token) order, the order an encode into an empty pool takes (page "Open Weights:
// from files to tokens / second", section "09 / The optimization stack": pages return to the
// pool with their sequences; the spill pool is this format's own overflow area).  Runs as
// count -> scan -> gather -> copy back, through a staging area in the workspace, so the slots
// read and the slots written never overlap within a kernel.  All or nothing: the count pass
// checks every row (page id, length, slots inside [0, spill_top)) and the scan checks that the
// staging area holds the result; on any failure the gather and copy passes write nothing.
//
// Workspace header (256 bytes): word 0 scan failure, word 1 row failure, bytes 16..23 a zero
// u64 (the scan's start), bytes 24..31 the new spill_top.
struct CompactWs {
  uint32_t* scan_flag;
  uint32_t* row_err;
  const uint64_t* zero;
  uint64_t* new_top;
  uint32_t* page_count;
  uint8_t* staging;
  uint64_t staging_slots;
};

__global__ __launch_bounds__(64) void compact_count_k(Geom g, SeqView s, const uint32_t* __restrict__ row_flags,
                                                      const uint32_t* __restrict__ row_spill,
                                                      const uint64_t* spill_top, uint64_t spill_slots,
                                                      CompactWs w, uint32_t* status) {
  const int p = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int32_t L;
  const int rows = rows_in_page(s, g, b, p, &L);
  if (rows < 0) {
    if (p == 0 && tid == 0) {
      set_status(status, ZF_DEV_ELEN);
      atomicOr(w.row_err, ZF_DEV_ELEN);
    }
    return;
  }
  if (rows == 0) return;
  const int32_t pid = s.pt[(int64_t)b * s.maxp + p];
  if (pid < 0 || pid >= g.P) {
    if (tid == 0) {
      set_status(status, ZF_DEV_EPAGE);
      atomicOr(w.row_err, ZF_DEV_EPAGE);
      w.page_count[(int64_t)b * s.maxp + p] = 0u;
    }
    return;
  }
  const uint64_t top = min(*spill_top, spill_slots);  // the slots that hold data
  uint32_t n = 0u;
  bool bad = false;
  if (tid < rows) {
    const int64_t row = (int64_t)pid * g.T + tid;
    n = __popc(row_flags[row]);
    bad = n > 0u && (uint64_t)row_spill[row] + n > top;
  }
  if (__any(bad) && tid == 0) {
    set_status(status, ZF_DEV_ESPILL);
    atomicOr(w.row_err, ZF_DEV_ESPILL);
  }
  for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o, 64);
  if (tid == 0) w.page_count[(int64_t)b * s.maxp + p] = n;
}

__global__ __launch_bounds__(256) void compact_gather_k(Geom g, SeqView s, const uint32_t* __restrict__ row_flags,
                                                        uint32_t* __restrict__ row_spill,
                                                        const uint8_t* __restrict__ spill, CompactWs w) {
  if (*w.scan_flag != 0u || *w.row_err != 0u) return;
  const int p = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int32_t L;
  const int rows = rows_in_page(s, g, b, p, &L);
  if (rows <= 0) return;
  const int32_t pid = s.pt[(int64_t)b * s.maxp + p];  // checked by the count pass
  __shared__ uint32_t s_n[64], s_old[64], s_new[64];
  if (tid < 64) {
    const int64_t row = (int64_t)pid * g.T + tid;
    const uint32_t n = tid < rows ? (uint32_t)__popc(row_flags[row]) : 0u;
    uint32_t incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t up = __shfl_up(incl, o, 64);
      if (tid >= o) incl += up;
    }
    const uint32_t first = w.page_count[(int64_t)b * s.maxp + p] + (incl - n);
    s_n[tid] = n;
    s_new[tid] = first;
    if (tid < rows) {
      s_old[tid] = row_spill[row];  // this lane reads the row's old index, then replaces it
      row_spill[row] = first;
    }
  }
  __syncthreads();
  // 16-byte halves of the moved slots: row r, slot i, half k
  for (int m = tid; m < rows * 64; m += blockDim.x) {
    const int r = m >> 6, i = (m & 63) >> 1, k = m & 1;
    if ((uint32_t)i >= s_n[r]) continue;
    const uint64_t from = ((uint64_t)s_old[r] + i) * 32u + k * 16u;
    const uint64_t to = ((uint64_t)s_new[r] + i) * 32u + k * 16u;
    *reinterpret_cast<uint4*>(w.staging + to) = *reinterpret_cast<const uint4*>(spill + from);
  }
}

constexpr int kCopyBlocks = 1024;

__global__ __launch_bounds__(256) void compact_copy_k(CompactWs w, uint8_t* __restrict__ spill,
                                                      uint64_t* spill_top) {
  if (*w.scan_flag != 0u || *w.row_err != 0u) return;
  const uint64_t total = *w.new_top;
  const uint64_t n16 = total * 2u;  // 16-byte pieces
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (uint64_t)gridDim.x * blockDim.x)
    reinterpret_cast<uint4*>(spill)[i] = reinterpret_cast<const uint4*>(w.staging)[i];
  if (blockIdx.x == 0 && threadIdx.x == 0) *spill_top = total;
}

// ------------------------------------------------------------------------------ host launchers

static SeqView view(const zf_seqs* q) {
  return SeqView{q->batch, q->max_pages_per_seq, q->max_seq_len, q->page_table, q->seq_lens, q->kmax};
}

hipError_t launch_encode(const Geom& g, const zf_cache* c, const zf_seqs* q, const uint16_t* raw,
                         uint32_t* ws, hipStream_t st) {
  SeqView s = view(q);
  uint32_t* failed = ws;                                       // 256-byte header
  uint64_t* look = reinterpret_cast<uint64_t*>(ws + 64);       // one word per (sequence, page)
  hipError_t e = launch_fill_zero(ws, encode_workspace_bytes(q), st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(enc_k, dim3(q->max_pages_per_seq, q->batch), dim3(kEncThreads), 0, st, g, s, raw, c->sm,
                     c->nib, c->base, c->row_flags, c->row_spill, c->spill, c->spill_top, c->spill_slots,
                     look, failed, c->status);
  hipLaunchKernelGGL(enc_finish_k, dim3(1), dim3(64), 0, st, g, s, look, failed, c->spill_top,
                     c->spill_slots, c->status);
  return hipGetLastError();
}

size_t encode_workspace_bytes(const zf_seqs* q) {
  return 256 + (size_t)q->batch * (size_t)q->max_pages_per_seq * sizeof(uint64_t);
}

size_t encode_lds_bytes(int32_t batch) {
  return ((size_t)batch + 1 + kScanThreads) * sizeof(uint32_t);
}

int append_max_rows() { return kAppendChunkedMaxRows; }

hipError_t launch_append(const Geom& g, const zf_cache* c, const zf_seqs* q, int32_t n, const uint16_t* k_new,
                         const uint16_t* v_new, hipStream_t st) {
  SeqView s = view(q);
  const int rows = q->batch * n;
  if (c->append_sync && rows <= kOneMaxRows) {
    hipLaunchKernelGGL(append_one_k, dim3(rows + 1), dim3(256), 0, st, g, s, n, k_new, v_new, c->sm, c->nib,
                       c->base, c->row_flags, c->row_spill, c->spill, c->spill_top, c->spill_slots, c->status,
                       c->append_sync);
    return hipGetLastError();
  }
  if (rows > kAppendMaxRows) {
    const int ngroups = (rows + kGroupRows - 1) / kGroupRows;
    hipLaunchKernelGGL(append_pack_k<4>, dim3((rows + 3) / 4), dim3(256), 0, st, g, s, n, k_new, v_new, c->sm, c->nib,
                       c->base, c->row_flags, c->row_spill);
    hipLaunchKernelGGL(append_group_commit_k, dim3(ngroups), dim3(256), 0, st, g, s, n, k_new, v_new, c->row_flags,
                       c->row_spill, c->spill, c->spill_top, c->spill_slots, c->append_sync);
    hipLaunchKernelGGL(append_group_finish_k, dim3(1), dim3(kScanThreads), 0, st, g, s, n, c->row_spill,
                       c->spill_top, c->spill_slots, c->status);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(append_pack_k<2>, dim3((rows + 1) / 2), dim3(256), 0, st, g, s, n, k_new, v_new, c->sm, c->nib,
                     c->base, c->row_flags, nullptr);
  size_t lds = 2 * (size_t)rows * sizeof(uint32_t);
  hipLaunchKernelGGL(append_commit_k, dim3(1), dim3(kAppendThreads), lds, st, g, s, n, k_new, v_new,
                     c->row_flags, c->row_spill, c->spill, c->spill_top, c->spill_slots, c->status);
  return hipGetLastError();
}

static size_t compact_head_bytes(const zf_seqs* q) {
  const size_t counts = (size_t)q->batch * (size_t)q->max_pages_per_seq * sizeof(uint32_t);
  return 256 + (counts + 255) / 256 * 256;
}

size_t compact_workspace_bytes(const zf_cache* c, const zf_seqs* q) {
  return compact_head_bytes(q) + (size_t)c->spill_slots * 32u;
}

hipError_t launch_compact(const Geom& g, const zf_cache* c, const zf_seqs* q, void* ws, size_t ws_bytes,
                          hipStream_t st) {
  SeqView s = view(q);
  uint8_t* base = static_cast<uint8_t*>(ws);
  const size_t head = compact_head_bytes(q);
  CompactWs w;
  w.scan_flag = reinterpret_cast<uint32_t*>(base);
  w.row_err = reinterpret_cast<uint32_t*>(base) + 1;
  w.zero = reinterpret_cast<const uint64_t*>(base + 16);
  w.new_top = reinterpret_cast<uint64_t*>(base + 24);
  w.page_count = reinterpret_cast<uint32_t*>(base + 256);
  w.staging = base + head;
  // the live blocks must fit both the staging area and the pool (rows that alias each other's
  // slots could otherwise count more blocks than the pool has)
  w.staging_slots = std::min<uint64_t>((ws_bytes - head) / 32u, c->spill_slots);
  hipError_t e = launch_fill_zero(base, 256, st);
  if (e != hipSuccess) return e;
  dim3 grid(q->max_pages_per_seq, q->batch);
  if (q->batch > 0)
    hipLaunchKernelGGL(compact_count_k, grid, dim3(64), 0, st, g, s, c->row_flags, c->row_spill,
                       c->spill_top, c->spill_slots, w, c->status);
  size_t lds = ((size_t)q->batch + 1 + kScanThreads) * sizeof(uint32_t);
  hipLaunchKernelGGL(enc_scan_k, dim3(1), dim3(kScanThreads), lds, st, g, s, w.page_count, w.zero,
                     w.new_top, w.staging_slots, w.scan_flag, c->status);
  if (q->batch > 0)
    hipLaunchKernelGGL(compact_gather_k, grid, dim3(256), 0, st, g, s, c->row_flags, c->row_spill,
                       c->spill, w);
  hipLaunchKernelGGL(compact_copy_k, dim3(kCopyBlocks), dim3(256), 0, st, w, c->spill, c->spill_top);
  return hipGetLastError();
}

hipError_t launch_decode(const Geom& g, const zf_cache* c, const zf_seqs* q, uint16_t* out,
                         hipStream_t st) {
  SeqView s = view(q);
  dim3 grid(q->max_pages_per_seq, q->batch);
  hipLaunchKernelGGL(decode_k, grid, dim3(kDecThreads), 0, st, g, s, c->sm, c->nib, c->base, c->row_flags,
                     c->row_spill, c->spill, c->spill_slots, out, c->status);
  return hipGetLastError();
}

}  // namespace zf
