// zf_codec.hip - block codec kernels for gfx950: full-cache encode, per-step append, decode.
//
// Codec: ZipFusion video summary ("Run AI Faster With Lossless Compressed Memory", chapter
// "Twelve Bits and One Addition").  Paged cache: page "Open Weights: from files to tokens /
// second", section "09 / The optimization stack" (KV memory allocated in fixed-size blocks).
//
// Work split.  A raw page u16[H][2][T][D] is one contiguous 64 KB run (H = 8, T = 16,
// D = 128), so one workgroup owns one (sequence, logical page) and streams it with 16-byte
// loads: 8 lanes cover one 64-value block, a 256-thread group covers 32 blocks per sweep.
// Spill slots follow an exclusive scan of raw-block counts in (sequence, token) order, so
// encode runs as pack -> scan -> spill: the pack pass writes sm/nib/base/row_flags and a
// per-page raw count; one workgroup scans the page counts; the spill pass turns them into
// row_spill and writes the 32-byte spill slots of the raw blocks.
#include "zf_internal.h"

namespace zf {

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

struct SeqView {
  int32_t B, maxp, max_seq_len;
  const int32_t* pt;
  int32_t* lens;
};

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

// ------------------------------------------------------------------------------ encode: pack

__global__ __launch_bounds__(256) void enc_pack_k(Geom g, SeqView s, const uint16_t* __restrict__ raw,
                                                  uint8_t* __restrict__ sm, uint8_t* __restrict__ nib,
                                                  uint8_t* __restrict__ base, uint32_t* __restrict__ row_flags,
                                                  uint32_t* __restrict__ page_count, uint32_t* status) {
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
    if (tid == 0) {
      set_status(status, ZF_DEV_EPAGE);
      page_count[(int64_t)b * s.maxp + p] = 0u;
    }
    return;
  }
  __shared__ uint32_t s_flags[64];
  if (tid < g.T) s_flags[tid] = 0u;
  __syncthreads();

  const int nb = g.nb();
  const int blocks = 2 * g.H * g.T * nb;
  const int64_t page_vals = g.vals_per_page();
  const int lane8 = tid & 7;
  for (int m = tid >> 3; m < blocks; m += blockDim.x >> 3) {
    const int half = m % nb, rest = m / nb, slot = rest % g.T, hk = rest / g.T;
    if (slot >= rows) continue;  // uniform over the 8 lanes of the block
    const int64_t v0 = (int64_t)pid * page_vals + (int64_t)m * kBlock + lane8 * 8;
    uint4 in = *reinterpret_cast<const uint4*>(raw + v0);
    uint32_t w[4] = {in.x, in.y, in.z, in.w};
    Window win = window8(w);
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      win.emin = min(win.emin, (uint32_t)__shfl_xor((int)win.emin, o, 8));
      win.emax = max(win.emax, (uint32_t)__shfl_xor((int)win.emax, o, 8));
      win.special |= (uint32_t)__shfl_xor((int)win.special, o, 8);
    }
    const uint32_t raw_blk = win.special | (uint32_t)(win.emax - win.emin > 15u);
    const uint32_t bexp = raw_blk ? 0u : win.emin;
    uint32_t smw[2], nibw, hiw;
    pack8(w, bexp, raw_blk, smw, nibw, hiw);
    *reinterpret_cast<uint2*>(sm + v0) = make_uint2(smw[0], smw[1]);
    *reinterpret_cast<uint32_t*>(nib + (v0 >> 1)) = nibw;
    if (lane8 == 0) {
      base[v0 / kBlock] = (uint8_t)bexp;
      if (raw_blk) atomicOr(&s_flags[slot], 1u << (hk * nb + half));
    }
  }
  __syncthreads();
  if (tid < 64) {
    uint32_t f = tid < rows ? s_flags[tid] : 0u;
    if (tid < rows) row_flags[(int64_t)pid * g.T + tid] = f;
    uint32_t c = __popc(f);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) c += __shfl_xor((int)c, o, 64);
    if (tid == 0) page_count[(int64_t)b * s.maxp + p] = c;
  }
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

// ------------------------------------------------------------------------------ encode: spill

__global__ __launch_bounds__(256) void enc_spill_k(Geom g, SeqView s, const uint16_t* __restrict__ raw,
                                                   const uint32_t* __restrict__ row_flags,
                                                   uint32_t* __restrict__ row_spill, uint8_t* __restrict__ spill,
                                                   const uint32_t* __restrict__ page_prefix,
                                                   const uint32_t* ws_flag, uint64_t spill_slots) {
  if (*ws_flag != 0u) return;
  const int p = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int32_t L;
  const int rows = rows_in_page(s, g, b, p, &L);
  if (rows <= 0) return;
  const int32_t pid = s.pt[(int64_t)b * s.maxp + p];
  if (pid < 0 || pid >= g.P) return;
  __shared__ uint32_t s_flags[64], s_first[64];
  if (tid < 64) {
    uint32_t f = tid < rows ? row_flags[(int64_t)pid * g.T + tid] : 0u;
    uint32_t c = __popc(f), incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      uint32_t up = __shfl_up((int)incl, o, 64);
      if (tid >= o) incl += up;
    }
    uint32_t first = page_prefix[(int64_t)b * s.maxp + p] + (incl - c);
    s_flags[tid] = f;
    s_first[tid] = first;
    if (tid < rows) row_spill[(int64_t)pid * g.T + tid] = first;
  }
  __syncthreads();
  const int nb = g.nb();
  const int blocks = 2 * g.H * g.T * nb;
  const int lane8 = tid & 7;
  for (int m = tid >> 3; m < blocks; m += blockDim.x >> 3) {
    const int half = m % nb, rest = m / nb, slot = rest % g.T, hk = rest / g.T;
    if (slot >= rows) continue;
    const int j = hk * nb + half;
    const uint32_t f = s_flags[slot];
    if (!((f >> j) & 1u)) continue;
    const uint64_t idx = (uint64_t)s_first[slot] + __popc(f & ((1u << j) - 1u));
    if (idx >= spill_slots) continue;  // only reachable when two sequences share a page
    const int64_t v0 = (int64_t)pid * g.vals_per_page() + (int64_t)m * kBlock + lane8 * 8;
    uint4 in = *reinterpret_cast<const uint4*>(raw + v0);
    uint32_t w[4] = {in.x, in.y, in.z, in.w};
    uint32_t hi = 0u;
#pragma unroll
    for (int v = 0; v < 8; ++v) hi |= (exp_of(w[v >> 1] >> (16 * (v & 1))) >> 4) << (4 * v);
    *reinterpret_cast<uint32_t*>(spill + idx * 32u + lane8 * 4) = hi;
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
// at most 64 new rows): R packing workgroups and one commit workgroup.  Each packing workgroup
// publishes one 64-bit word, its row's flag word and error bits tagged with the call's epoch
// (a counter in the sync area), stored only after its loads of the epoch, its length and
// spill_top have returned.  Every packing workgroup then waits until all R words carry the tag,
// takes the all-or-nothing decision from them, marks its own word decided, and writes its
// row's spill slots (from spill_top plus the raw blocks of the rows before it) and row_spill.
// The commit waits until all R words are marked decided, takes the same decision, and advances
// seq_lens and spill_top (every length was read before its word was stored) and then the
// epoch; a workgroup that gives up waiting never marks its word, so the commit then changes
// nothing.  Each word carries its data itself, so no fence orders it after other stores.
constexpr int kAppendThreads = 1024;
constexpr int kAppendMaxRows = 4096;  // two u32 per row in LDS
constexpr int kOneMaxRows = 64;       // new rows of a one-launch append (sync words 0 .. 63; 64: epoch)
constexpr uint32_t kSyncPolls = 1u << 20;  // bound on each wait for the words (about 1 s);
                                           // the packing workgroups' bound can be lowered
constexpr uint64_t kTagMod = (1u << 28) - 1u;

// Row of new token j of sequence b (n per sequence) whose length was read as L, or -1 (with the
// error bit) when the sequence cannot take them.
__device__ __forceinline__ int64_t append_row_at(const Geom& g, const SeqView& s, int b, int j, int n,
                                                 int32_t L, uint32_t* err) {
  if (L < 0 || (int64_t)L + n > (int64_t)s.maxp * g.T || (int64_t)L + n > s.max_seq_len) {
    *err = ZF_DEV_ELEN;
    return -1;
  }
  const int32_t t = L + j;
  const int32_t pid = s.pt[(int64_t)b * s.maxp + t / g.T];
  if (pid < 0 || pid >= g.P) {
    *err = ZF_DEV_EPAGE;
    return -1;
  }
  *err = 0;
  return (int64_t)pid * g.T + t % g.T;
}

__device__ __forceinline__ int64_t append_row(const Geom& g, const SeqView& s, int b, int j, int n,
                                              uint32_t* err) {
  return append_row_at(g, s, b, j, n, s.lens[b], err);
}

// Block j of a new row, classified and packed in registers (8 lanes, 8 values each).
struct NewBlock {
  uint32_t sm0, sm1, nib, hi, bexp, raw;
};

// New row r is u16 [H][D] of K and of V; block j covers half j % nb of head j / nb / 2, K or V
// by (j / nb) & 1, the order of the row's flag bits.
__device__ __forceinline__ NewBlock classify_new(const Geom& g, int r, int j, int lane8,
                                                 const uint16_t* __restrict__ k_new,
                                                 const uint16_t* __restrict__ v_new) {
  const int nb = g.nb(), half = j % nb, hk = j / nb, h = hk >> 1, kv = hk & 1;
  const uint4 in = *reinterpret_cast<const uint4*>((kv ? v_new : k_new) + ((int64_t)r * g.H + h) * g.D +
                                                   half * kBlock + lane8 * 8);
  const uint32_t w[4] = {in.x, in.y, in.z, in.w};
  Window win = window8(w);
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    win.emin = min(win.emin, (uint32_t)__shfl_xor((int)win.emin, o, 8));
    win.emax = max(win.emax, (uint32_t)__shfl_xor((int)win.emax, o, 8));
    win.special |= (uint32_t)__shfl_xor((int)win.special, o, 8);
  }
  NewBlock o;
  o.raw = win.special | (uint32_t)(win.emax - win.emin > 15u);
  o.bexp = o.raw ? 0u : win.emin;
  uint32_t smw[2];
  pack8(w, o.bexp, o.raw, smw, o.nib, o.hi);
  o.sm0 = smw[0];
  o.sm1 = smw[1];
  return o;
}

__device__ __forceinline__ void store_new(const Geom& g, int64_t row, int j, int lane8, const NewBlock& o,
                                          uint8_t* sm, uint8_t* nib, uint8_t* base) {
  const int nb = g.nb(), half = j % nb, hk = j / nb, h = hk >> 1, kv = hk & 1;
  const int64_t pid = row / g.T, slot = row % g.T;
  const int64_t v0 = ((pid * g.H + h) * 2 + kv) * g.T * g.D + slot * g.D + half * kBlock + lane8 * 8;
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

__global__ __launch_bounds__(256) void append_pack_k(Geom g, SeqView s, int n, const uint16_t* __restrict__ k_new,
                                                     const uint16_t* __restrict__ v_new, uint8_t* sm,
                                                     uint8_t* nib, uint8_t* base, uint32_t* row_flags) {
  const int r = blockIdx.x, b = r / n, tid = threadIdx.x, j = tid >> 3, lane8 = tid & 7;
  uint32_t err;
  const int64_t row = append_row(g, s, b, r - b * n, n, &err);
  if (row < 0) return;  // reported by append_commit_k
  const bool has = j < g.blocks_per_row();
  NewBlock o{};
  if (has) o = classify_new(g, r, j, lane8, k_new, v_new);
  const uint32_t f = row_flag_word(has, j, lane8, o.raw);
  if (has) store_new(g, row, j, lane8, o, sm, nib, base);
  if (tid == 0) row_flags[row] = f;
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

// Tag of a hand-over word published under epoch E: never 0, and different for consecutive
// epochs (a word left by the previous call never matches).
__device__ __forceinline__ uint32_t sync_tag(uint64_t E) { return (uint32_t)(E % kTagMod) + 1u; }

// Hand-over word of one new row: tag << 36 | decided << 35 | error bits << 32 | flag word.
// `decided`: the row's workgroup has seen every word of the call (so it will write its spill
// slots if the call succeeds).
__device__ __forceinline__ uint32_t word_tag(uint64_t w) { return (uint32_t)(w >> 36); }
constexpr uint64_t kDecided = (uint64_t)1 << 35;

// What every workgroup learns from the R hand-over words (wave 0 polls them, lane i word i).
struct HandOver {
  uint32_t seen, err, total, pref;  // pref: raw blocks of the rows before row `me`
};

__device__ __forceinline__ HandOver read_hand_over(const uint64_t* sync, int R, int me, uint32_t tag,
                                                   bool need_decided, uint32_t polls) {
  __shared__ HandOver s_h;
  const int tid = threadIdx.x;
  if (tid < 64) {
    uint64_t w = 0u;
    bool ok = tid >= R;
    for (uint32_t p = 0; !ok && p < polls; ++p) {
      w = __hip_atomic_load(&sync[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok = word_tag(w) == tag && (!need_decided || (w & kDecided));
      if (!ok) __builtin_amdgcn_s_sleep(2);
    }
    const uint32_t cnt = tid < R ? __popc((uint32_t)w) : 0u;
    uint32_t incl = cnt, err = tid < R ? (uint32_t)(w >> 32) & 7u : 0u, miss = ok ? 0u : 1u;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t up = __shfl_up((int)incl, o, 64);
      if (tid >= o) incl += up;
      err |= (uint32_t)__shfl_xor((int)err, o, 64);
      miss |= (uint32_t)__shfl_xor((int)miss, o, 64);
    }
    if (tid == me) s_h.pref = incl - cnt;
    if (tid == 63) {
      s_h.total = incl;
      s_h.err = err;
      s_h.seen = miss == 0u;
    }
  }
  __syncthreads();
  return s_h;
}

// Commit workgroup of the one-launch append: once every row's word carries this call's tag and
// the decided mark, it advances seq_lens and spill_top, clears the words of unused rows and
// moves to the next epoch.
__device__ void commit_one(const SeqView& s, int n, uint64_t* spill_top, uint64_t spill_slots,
                           uint32_t* status, uint64_t* sync) {
  const int R = s.B * n, tid = threadIdx.x;
  const uint64_t E = sync[kOneMaxRows];  // written only by an earlier launch: a plain load
  const uint64_t top = *spill_top;
  const int32_t L = tid < s.B ? s.lens[tid] : 0;
  const HandOver h = read_hand_over(sync, R, -1, sync_tag(E), true, kSyncPolls);
  if (!h.seen) {  // some row's word never came or never got decided: change nothing
    if (tid == 0) set_status(status, ZF_DEV_ESYNC);
    return;
  }
  const bool fits = fits_in_pool(h.total, top, spill_slots);
  if (tid == 0) set_status(status, h.err ? h.err : (fits ? 0u : ZF_DEV_ESPILL));
  if (!h.err && fits) {
    if (tid < s.B) s.lens[tid] = L + n;  // every packing workgroup read its length before its word
    if (tid == 0) *spill_top = top + h.total;
  }
  if (tid >= R && tid < kOneMaxRows)
    __hip_atomic_store(&sync[tid], (uint64_t)0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) __hip_atomic_store(&sync[kOneMaxRows], E + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One-launch append: workgroups 0 .. R-1 pack new row blockIdx.x, workgroup R commits.
__global__ __launch_bounds__(256) void append_one_k(Geom g, SeqView s, int n, const uint16_t* __restrict__ k_new,
                                                    const uint16_t* __restrict__ v_new, uint8_t* sm,
                                                    uint8_t* nib, uint8_t* base, uint32_t* row_flags,
                                                    uint32_t* row_spill, uint8_t* spill, uint64_t* spill_top,
                                                    uint64_t spill_slots, uint32_t* status, uint64_t* sync,
                                                    uint32_t polls) {
  const int R = s.B * n, r = blockIdx.x, tid = threadIdx.x, j = tid >> 3, lane8 = tid & 7;
  if (r == R) {
    commit_one(s, n, spill_top, spill_slots, status, sync);
    return;
  }
  const uint64_t E = sync[kOneMaxRows];
  const uint64_t top = *spill_top;
  const int b = r / n;
  uint32_t err;
  const int64_t row = append_row(g, s, b, r - b * n, n, &err);
  const bool has = j < g.blocks_per_row();
  NewBlock o{};
  if (has) o = classify_new(g, r, j, lane8, k_new, v_new);
  const uint32_t f = row_flag_word(has, j, lane8, o.raw);
  if (tid == 0) {
    // the word is built from the epoch, the length (through err and row) and spill_top as
    // loaded, so it cannot be stored before those loads have returned
    uint32_t hi = (sync_tag(E) << 4) | err;
    asm volatile("" : "+v"(hi) : "v"((uint32_t)row), "v"((uint32_t)top));
    __hip_atomic_store(&sync[r], ((uint64_t)hi << 32) | f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (row >= 0) {
    if (has) store_new(g, row, j, lane8, o, sm, nib, base);
    if (tid == 0) row_flags[row] = f;
  }
  const HandOver h = read_hand_over(sync, R, r, sync_tag(E), false, polls);
  if (!h.seen) {  // the commit will not see this row decided, so the call changes nothing
    if (tid == 0) set_status(status, ZF_DEV_ESYNC);
    return;
  }
  if (tid == 0)
    __hip_atomic_store(&sync[r], ((uint64_t)((sync_tag(E) << 4) | err) << 32 | kDecided) | f,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the commit takes the same decision from the same words
  if (h.err || !fits_in_pool(h.total, top, spill_slots)) return;
  const uint64_t first = top + h.pref;
  if (has && o.raw) {
    const uint64_t slot = first + __popc(f & ((1u << j) - 1u));
    *reinterpret_cast<uint32_t*>(spill + slot * 32u + lane8 * 4) = o.hi;
  }
  if (tid == 0) row_spill[row] = (uint32_t)first;
}

// ------------------------------------------------------------------------------ decode

__global__ __launch_bounds__(256) void decode_k(Geom g, SeqView s, const uint8_t* __restrict__ sm,
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
  const int lane8 = tid & 7;
  uint32_t err = 0;
  for (int m = tid >> 3; m < blocks; m += blockDim.x >> 3) {
    const int half = m % nb, rest = m / nb, slot = rest % g.T, hk = rest / g.T;
    if (slot >= rows) continue;
    const int64_t v0 = (int64_t)pid * g.vals_per_page() + (int64_t)m * kBlock + lane8 * 8;
    const uint2 smw = *reinterpret_cast<const uint2*>(sm + v0);
    const uint32_t nibw = *reinterpret_cast<const uint32_t*>(nib + (v0 >> 1));
    const uint32_t f = row_flags[(int64_t)pid * g.T + slot];
    const int j = hk * nb + half;
    uint32_t base_pair = 0u, hi = 0u;
    if ((f >> j) & 1u) {
      const uint64_t idx = (uint64_t)row_spill[(int64_t)pid * g.T + slot] + __popc(f & ((1u << j) - 1u));
      if (idx < spill_slots) hi = *reinterpret_cast<const uint32_t*>(spill + idx * 32u + lane8 * 4);
      else err = ZF_DEV_ESPILL;
    } else {
      base_pair = (uint32_t)base[v0 / kBlock] * 0x00010001u;
    }
    uint32_t pr[4], w[4];
    rebuild8(smw.x, smw.y, nibw, hi, base_pair, pr);
    pairs_to_natural(pr, w);
    *reinterpret_cast<uint4*>(out + v0) = make_uint4(w[0], w[1], w[2], w[3]);
  }
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
  return SeqView{q->batch, q->max_pages_per_seq, q->max_seq_len, q->page_table, q->seq_lens};
}

hipError_t launch_encode(const Geom& g, const zf_cache* c, const zf_seqs* q, const uint16_t* raw,
                         uint32_t* ws, hipStream_t st) {
  SeqView s = view(q);
  uint32_t* ws_flag = ws;
  uint32_t* page_count = ws + 64;  // 256-byte header
  dim3 grid(q->max_pages_per_seq, q->batch);
  hipLaunchKernelGGL(enc_pack_k, grid, dim3(256), 0, st, g, s, raw, c->sm, c->nib, c->base,
                     c->row_flags, page_count, c->status);
  size_t lds = ((size_t)q->batch + 1 + kScanThreads) * sizeof(uint32_t);
  hipLaunchKernelGGL(enc_scan_k, dim3(1), dim3(kScanThreads), lds, st, g, s, page_count,
                     c->spill_top, c->spill_top, c->spill_slots, ws_flag, c->status);
  hipLaunchKernelGGL(enc_spill_k, grid, dim3(256), 0, st, g, s, raw, c->row_flags, c->row_spill,
                     c->spill, page_count, ws_flag, c->spill_slots);
  return hipGetLastError();
}

size_t encode_workspace_bytes(const zf_seqs* q) {
  return 256 + (size_t)q->batch * (size_t)q->max_pages_per_seq * sizeof(uint32_t);
}

size_t encode_lds_bytes(int32_t batch) {
  return ((size_t)batch + 1 + kScanThreads) * sizeof(uint32_t);
}

int append_max_rows() { return kAppendMaxRows; }

static uint32_t g_append_wait_polls = kSyncPolls;

void set_append_wait_polls(uint32_t polls) { g_append_wait_polls = polls; }

hipError_t launch_append(const Geom& g, const zf_cache* c, const zf_seqs* q, int32_t n, const uint16_t* k_new,
                         const uint16_t* v_new, hipStream_t st) {
  SeqView s = view(q);
  const int rows = q->batch * n;
  if (c->append_sync && rows <= kOneMaxRows) {
    hipLaunchKernelGGL(append_one_k, dim3(rows + 1), dim3(256), 0, st, g, s, n, k_new, v_new, c->sm, c->nib,
                       c->base, c->row_flags, c->row_spill, c->spill, c->spill_top, c->spill_slots, c->status,
                       c->append_sync, g_append_wait_polls);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(append_pack_k, dim3(rows), dim3(256), 0, st, g, s, n, k_new, v_new, c->sm, c->nib,
                     c->base, c->row_flags);
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
  hipLaunchKernelGGL(decode_k, grid, dim3(256), 0, st, g, s, c->sm, c->nib, c->base, c->row_flags,
                     c->row_spill, c->spill, c->spill_slots, out, c->status);
  return hipGetLastError();
}

}  // namespace zf
