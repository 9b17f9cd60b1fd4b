/*
 * zf.h - lossless compressed-KV decode attention for AMD Instinct MI355X (gfx950).
 *
 * The method (ZipFusion video summary, "Run AI Faster With Lossless Compressed Memory"):
 * the KV cache stays compressed in GPU memory; a block of BF16 values keeps one shared base
 * exponent and a 4-bit exponent offset per value next to each value's sign and mantissa
 * (12 bits per value, 75 % of BF16, chapter "Twelve Bits and One Addition"); blocks whose
 * exponents are too spread out stay raw; attention rebuilds every value in registers with a
 * single integer addition instead of unpacking the cache to a buffer inside the decode loop.
 * The cache is paged (page "Open Weights: from files to tokens / second": section "09 / The
 * optimization stack" allocates KV memory in blocks; section "03 / The inference loop" has
 * decode read the cache every step).
 *
 * ---------------------------------------------------------------------------------- format
 * Geometry: num_pages pages of page_size tokens; num_kv_heads heads; head_dim a multiple of
 * 64 with 2 * num_kv_heads * head_dim / 64 <= 32.  A block is 64 consecutive head_dim values
 * of one (token, kv head, K or V).  A token row is all blocks of one token; block j of a row
 * is j = (h * 2 + kv) * (head_dim / 64) + half  (kv = 0 for K, 1 for V).
 * For every value x (bf16 bits s|eeeeeeee|mmmmmmm):
 *   sm  byte  = s << 7 | m
 *   nibble    = e - base            (compressed block; base = smallest exponent of the block)
 *             = e & 15              (raw block)
 * A block is raw iff one of its exponents is 0 (zero, subnormal) or 255 (Inf, NaN), or its
 * exponents span more than 16 values.  A raw block has base 0, its bit set in the row's flag
 * word, and 32 spill bytes holding e >> 4 of each value (packed like the nibbles).
 * Rebuild: x = (s << 15 | nibble << 7 | m) + (base << 7)   or   + ((e >> 4) << 11) when raw.
 * Spill slots: a row's raw blocks occupy consecutive slots in block order starting at
 * row_spill[row]; zf_encode_kv and zf_append_kv_n take slots for rows in (sequence, token)
 * order, zf_append_kv in batch order, all starting at *spill_top, which they advance.  Only
 * zf_compact_spill gives slots back: it rewrites the pool for the sequences still live.
 *
 * Arrays (device memory, 256-byte aligned, caller-owned; the library allocates nothing):
 *   sm        u8 [num_pages][H][2][page_size][D]
 *   nib       u8 [num_pages][H][2][page_size][D/2]   two values per byte, low nibble first
 *   base      u8 [num_pages][H][2][page_size][D/64]  0 = raw
 *   row_flags u32[num_pages][page_size]              bit j = block j raw
 *   row_spill u32[num_pages][page_size]              slot of the row's first raw block
 *   spill     u8 [spill_slots][32]
 *   spill_top u64 (one counter)   status u32 (sticky device error bits, ZF_DEV_*)
 *   append_sync u64[66] (optional; the one-launch append's hand-over words, epoch, test hook)
 * Raw (uncompressed) pages use u16[num_pages][H][2][page_size][D], the same page ids.
 *
 * ---------------------------------------------------------------------------------- errors
 * Calls validate their host-side arguments and return ZF_EINVAL / ZF_EUNSUPPORTED without
 * enqueuing anything.  Otherwise they enqueue on `stream` and return at once (ZF_OK), or
 * ZF_EHIP if the launch failed.  Problems found on the device (a page id outside
 * [0, num_pages), a length beyond the page table or the host bound, an exhausted spill pool)
 * set ZF_DEV_* bits in *status, which stay set until the caller clears them; rows with a bad
 * page id are skipped.  zf_get_status reads the word (it synchronizes the stream).
 * Only rows t < seq_lens[b] are defined; other slots are never read as data.
 */
#ifndef ZF_H
#define ZF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* zf_stream_t; /* a hipStream_t; NULL = the default stream */

typedef enum {
  ZF_OK = 0,
  ZF_EINVAL = 1,        /* bad argument (null or misaligned pointer, bad sizes)        */
  ZF_EUNSUPPORTED = 2,  /* valid but outside what the kernels implement                */
  ZF_EHIP = 3,          /* a HIP runtime call failed                                   */
  ZF_EWORKSPACE = 4,    /* workspace missing or smaller than the matching _bytes query */
  ZF_ESCRATCH = 5       /* zf_decode_attention_noalloc: the call's split partials need more
                           than ZF_NOALLOC_SCRATCH_BYTES                                   */
} zf_status;

#define ZF_DEV_ESPILL 1u  /* spill pool exhausted: spill_top and the slots below it kept   */
#define ZF_DEV_EPAGE 2u   /* a page-table entry the call needed is out of range           */
#define ZF_DEV_ELEN 4u    /* a length is negative or beyond the page table / host bound   */
#define ZF_DEV_ESYNC 8u   /* one-launch append: a hand-over word did not arrive within the
                             bounded wait (about 1 s; none is expected) or the give-up hook
                             was set: the call changed no defined state                   */

typedef struct {
  int32_t num_pages, page_size, num_kv_heads, head_dim;
  uint8_t* sm;
  uint8_t* nib;
  uint8_t* base;
  uint32_t* row_flags;
  uint32_t* row_spill;
  uint8_t* spill;
  uint64_t spill_slots;
  uint64_t* spill_top;
  uint32_t* status;
  uint64_t* append_sync; /* device u64[ZF_APPEND_SYNC_WORDS], zero when the cache is set
                            up, or NULL: see zf_append_kv_n */
} zf_cache;

/* append_sync: [0, 64) hand-over words, [64] the epoch (calls so far), [65] a test hook: nonzero
 * makes the one-launch append's packing workgroups give up instead of waiting for the words of
 * the rows before theirs (and the grouped multi-token form's groups instead of walking their
 * look-back), so the call ends with ZF_DEV_ESYNC and changes nothing; zero in use. */
#define ZF_APPEND_SYNC_WORDS 66

typedef struct {
  int32_t batch, max_pages_per_seq;
  const int32_t* page_table; /* device [batch][max_pages_per_seq], physical page ids        */
  int32_t* seq_lens;         /* device [batch], tokens present                               */
  int32_t max_seq_len;       /* HOST bound on every seq_lens[b] when the call runs (after an
                                append: on the grown lengths); sizes grids and workspaces   */
  uint32_t* kmax;            /* optional device [batch][num_kv_heads][max_pages_per_seq]: per
                                (sequence, kv head, logical page) the largest bf16 exponent
                                field among the K values of the page's tokens, 0 for a page
                                with none.  zf_encode_kv writes every entry; the appends raise
                                the entries of the pages they write (a call that fails may
                                leave some raised).  Only a hint: zf_decode_attention takes
                                each wave's page with the largest entry first, which settles
                                the running score maximum early; any contents give a correct
                                result.  NULL: not kept, not used                            */
} zf_seqs;

/* Bytes of one cache's arrays except spill, for sizing a pool of pages (the paged KV memory of
 * page "Open Weights: from files to tokens / second", section "09 / The optimization stack"). */
size_t zf_cache_bytes(int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
                      int32_t head_dim);

/* Initial compression of a prefilled cache (ZipFusion video summary, "Run AI Faster With
 * Lossless Compressed Memory": the initial compression, which its timings leave out, in the
 * format of chapter "Twelve Bits and One Addition").  Encodes rows t < seq_lens[b] of every sequence from raw
 * pages into the packed planes, takes spill slots from *spill_top in (sequence, token) order
 * and advances it.  If the pool cannot hold them all: ZF_DEV_ESPILL and spill_top unchanged;
 * the rows' planes and row_spill and the spill slots from spill_top on (within the pool) are
 * then unspecified.  One pass over the raw pages (the slots by decoupled look-back over the
 * pages, which waits only for earlier pages of the grid); ZF_DEV_ESYNC if such a wait ran out
 * (none is expected; spill_top unchanged, the rest as for ESPILL).  Workspace: device memory
 * of zf_encode_workspace_bytes(seqs) bytes (8 per page of the page table, plus 256), any
 * contents.  Three launches: workspace clear, encode, finish. */
zf_status zf_encode_kv(const zf_cache* cache, const zf_seqs* seqs, const uint16_t* raw_pages,
                       void* workspace, size_t workspace_bytes, zf_stream_t stream);
size_t zf_encode_workspace_bytes(const zf_seqs* seqs);

/* Decode-step append (page "Open Weights: from files to tokens / second", section "03 / The
 * inference loop": every decode step adds one token's K and V to the cache; ZipFusion video
 * summary, "Run AI Faster With Lossless Compressed Memory": the cache stays compressed in GPU
 * memory, so the new row is encoded as it is written; chapter "Twelve Bits and One Addition"
 * gives the format).  Encodes one new token per sequence (k_new, v_new u16[batch][H][D])
 * into row seq_lens[b] of its page, spill slots from *spill_top in batch order, then
 * seq_lens[b] += 1 for every b.  All or nothing for defined state: on a device error
 * (ZF_DEV_*) seq_lens, spill_top, the spill slots below spill_top and every row
 * t < seq_lens[b] are left as they were; only the rows at position seq_lens[b] and the spill
 * slots from spill_top on, which hold nothing yet, may have been overwritten.  seqs->max_seq_len bounds the lengths after the append.
 * Launches as zf_append_kv_n with n_new = 1 (one launch for batch <= 64 with a sync area). */
zf_status zf_append_kv(const zf_cache* cache, const zf_seqs* seqs, const uint16_t* k_new,
                       const uint16_t* v_new, zf_stream_t stream);

/* Multi-token append (speculative or chunked decode; page "Open Weights: from files to
 * tokens / second", section "03 / The inference loop": the cache grows by the tokens each
 * forward pass processes, in the format of the ZipFusion video summary, "Run AI Faster With
 * Lossless Compressed Memory").  Encodes n_new tokens per sequence
 * (k_new, v_new u16[batch][n_new][H][D]) into rows seq_lens[b] .. seq_lens[b] + n_new - 1,
 * spill slots from *spill_top in (sequence, token) order, then seq_lens[b] += n_new for every
 * b.  All or nothing, as zf_append_kv (only slots at positions seq_lens[b] and later may have
 * been overwritten after a device error); seqs->max_seq_len bounds the grown lengths.
 * n_new == 0 does nothing; n_new < 0 is ZF_EINVAL.  Supports batch * n_new <= 2^24 new rows.
 * zf_append_kv is the case n_new == 1.
 * Launches: one when cache->append_sync is set and batch * n_new <= 64; two up to 4096 new
 * rows (pack, then one commit workgroup); three beyond (pack; per group of 16 rows a look-back
 * over the earlier groups and the group's slots; a last step that checks the whole call and
 * commits).  In the
 * one-launch form the new rows' workgroups hand their flag words to each other through
 * append_sync, words tagged with an epoch that append_sync[64] counts (every call advances it,
 * also one that fails); each workgroup waits only for lower-numbered ones, so no co-residency
 * is assumed.  The area is zero when the cache is set up, holds the last call's words between
 * calls (only these calls may write it; an ESYNC needs no clean-up), and appends sharing it
 * must not overlap (appends to one cache are ordered anyway: they advance one spill_top).
 * Both forms write the same bytes. */
zf_status zf_append_kv_n(const zf_cache* cache, const zf_seqs* seqs, int32_t n_new,
                         const uint16_t* k_new, const uint16_t* v_new, zf_stream_t stream);

/* Spill lifecycle (pages come and go with their sequences: page "Open Weights: from files to
 * tokens / second", section "09 / The optimization stack"; the spill pool is this format's
 * overflow area for raw blocks, and encode and append only ever grow it).  `seqs` lists the
 * sequences still live; a sequence that ended is freed by leaving it out.  Their raw blocks
 * move to spill slots 0, 1, ... in (sequence, token) order, the row spill index of each of
 * their rows follows (rows without raw blocks get the running count, as encode writes it), and
 * *spill_top becomes the number of those blocks: the layout an encode of just these sequences
 * into an empty pool produces.  Rows of other sequences are not touched; their slots are
 * given up.  Planes, bases and row flags are not touched.  The listed sequences must not share
 * pages (as for encode).  batch == 0 empties the pool.
 * All or nothing: if a listed row's page id or length is invalid (ZF_DEV_EPAGE, ZF_DEV_ELEN),
 * a listed row's raw blocks are not inside [0, min(spill_top, spill_slots)) (ZF_DEV_ESPILL),
 * or the live blocks outnumber the staging area's slots or the pool's (ZF_DEV_ESPILL; rows
 * that alias each other's slots can do that), the status word says so
 * and nothing else changes.  Workspace: device memory, any contents; a 256-byte header, the
 * page counts, then a staging area of 32 bytes per slot.  zf_compact_workspace_bytes gives
 * room for every slot of the pool; a smaller workspace (at least the header and counts) works
 * when its staging area holds the live blocks.  Five kernel launches, none allocates.
 * Supports batch <= 8192. */
zf_status zf_compact_spill(const zf_cache* cache, const zf_seqs* seqs, void* workspace,
                           size_t workspace_bytes, zf_stream_t stream);
size_t zf_compact_workspace_bytes(const zf_cache* cache, const zf_seqs* seqs);

/* Capacity model (page "Open Weights: from files to tokens / second": the memory left after
 * the weights, parameters x bits / 8, and a runtime reserve goes to the paged KV cache, and
 * more cache pages admit more concurrent sequences; the ZipFusion video summary puts most of
 * its gain there).  Returns how many sequences of `context` tokens fit in `kv_budget_bytes`
 * across `layers` layers: each sequence and layer holds ceil(context / page_size) pages;
 * raw_blocks_per_row < 0 prices them as bf16 pages (H x 2 x D values of 2 bytes per row),
 * otherwise as packed pages (zf_cache_bytes per page) plus ceil(raw_blocks_per_row x context)
 * spill slots of 32 bytes.  0 for a non-positive budget, layer count or context; -1 for an
 * unsupported geometry or more raw blocks per row than a row has.  Host only. */
int64_t zf_max_sequences(int64_t kv_budget_bytes, int32_t layers, int32_t context,
                         int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                         double raw_blocks_per_row);

/* Inverse of the codec (ZipFusion video summary, "Run AI Faster With Lossless Compressed
 * Memory", chapter "Lossless or FP8": the compression loses nothing, so the original values
 * come back exactly): writes rows t < seq_lens[b] as raw bf16 pages, the bits that were
 * encoded. */
zf_status zf_decode_kv(const zf_cache* cache, const zf_seqs* seqs, uint16_t* raw_pages_out,
                       zf_stream_t stream);

/* Fused decode attention over the packed cache (ZipFusion video summary, "Run AI Faster With
 * Lossless Compressed Memory": values rebuilt in registers by one integer add, no decompressed
 * copy; page "Open Weights: from files to tokens / second", section "03 / The inference loop":
 * the decode step's attention over the whole cache).  q: bf16 u16[batch][num_q_heads][D]; out:
 * f32 [batch][num_q_heads][D]; q head i uses kv head i / (num_q_heads / H).  out =
 * softmax(scale * q K^T) V over the sequence's tokens in logical order; zeros when
 * seq_lens[b] == 0.  Arithmetic: scores on the matrix cores in fp32, recomputed in fp64 from
 * the exact bf16 products wherever a weight may reach 2^-40 of the largest; weights, their
 * sum and the rescales in fp64; products of a value of 2^4 or more summed in fp64; the rest
 * of p.V on the matrix cores with each weight split into bf16 parts (three, exact, for 4
 * query heads per kv head; two, within 2^-17 of it, for 8).  With seqs->kmax the pages are
 * visited in another order (the sums are the same up to rounding order).  Workspace:
 * zf_attention_workspace_bytes(...) bytes of device memory, any contents (it holds per-split
 * partials); calls sharing one workspace must not overlap.
 * Requires D == 128, page_size == 16, num_q_heads == 4 * H or 8 * H (Llama-3.1-8B- and
 * 70B-shaped groups), max_seq_len <= 2^20 and
 * spill_slots < 2^27 (the pool is addressed with 32-bit byte offsets) in this
 * version (ZF_EUNSUPPORTED otherwise).  One kernel launch when max_seq_len fits one split per
 * (sequence, kv head), else two (split attention, split merge). */
zf_status zf_decode_attention(const zf_cache* cache, const zf_seqs* seqs, const uint16_t* q,
                              int32_t num_q_heads, float scale, float* out, void* workspace,
                              size_t workspace_bytes, zf_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): zf_decode_attention without a workspace argument.
 * The split partials live in a fixed device array inside the library, ZF_NOALLOC_SCRATCH_BYTES
 * per GPU (set up when the library's code is loaded on that GPU, held until the process ends);
 * the call itself allocates nothing.  Every call on one GPU uses that GPU's array, so calls that
 * overlap on one GPU (other streams, other threads) race: order them, as appends to one cache
 * are ordered anyway.  The partials are written before they are read, so the array's contents
 * from an earlier call never matter.  A shape whose partials need more than the array
 * (zf_attention_workspace_bytes(...) > ZF_NOALLOC_SCRATCH_BYTES) returns ZF_ESCRATCH and
 * enqueues nothing; other errors and the result are those of zf_decode_attention. */
#define ZF_NOALLOC_SCRATCH_BYTES (16u << 20)
zf_status zf_decode_attention_noalloc(const zf_cache* cache, const zf_seqs* seqs, const uint16_t* q,
                                      int32_t num_q_heads, float scale, float* out,
                                      zf_stream_t stream);

/* The same attention kernel reading an uncompressed bf16 cache: the comparator the ZipFusion
 * video summary ("Run AI Faster With Lossless Compressed Memory") measures its faster attention
 * against.  Same split plan and arithmetic, so its output is bitwise identical to
 * zf_decode_attention on the encoded copy of the same pages.  num_pages bounds the page ids;
 * status: device u32 for ZF_DEV_* bits (may not be NULL). */
zf_status zf_decode_attention_raw(const uint16_t* raw_pages, int32_t num_pages,
                                  int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                                  const zf_seqs* seqs, const uint16_t* q, int32_t num_q_heads,
                                  float scale, float* out, void* workspace,
                                  size_t workspace_bytes, uint32_t* status, zf_stream_t stream);

/* Sizing, outside the method: bytes of the split partials an attention call of this shape
 * needs (a 256-byte header and, per sequence, kv head and split, the running sums). */
size_t zf_attention_workspace_bytes(int32_t batch, int32_t num_kv_heads, int32_t num_q_heads,
                                    int32_t head_dim, int32_t max_seq_len);
/* Sizing aid, outside the method: zero-fills a workspace on `stream` (a kernel, no memset
 * node); optional. */
zf_status zf_attention_workspace_init(void* workspace, size_t workspace_bytes,
                                      zf_stream_t stream);

/* Profiling aid, outside the method: the next zf_decode_attention or zf_decode_attention_raw
 * call made by this host thread records `start_event` when its attention kernel begins
 * executing on the device and `stop_event` when it ends (the dispatch's own timestamps, the
 * interval a kernel trace reports, without launch overhead); the split merge, when there is
 * one, is not included.  One-shot: that call clears the setting.  Both are caller-created,
 * timing-enabled hipEvent_t handles, or both NULL (clears).  ZF_EINVAL if exactly one is NULL. */
zf_status zf_time_next_attention(void* start_event, void* stop_event);

/* Measurement aid, outside the method: reads `bytes` of device memory at `buf` once, with
 * 16-byte loads spread over up to ZF_PROBE_BLOCKS workgroups (a plain stream: the practically
 * achievable HBM read rate, context for the attention kernel's).  sink: device u32
 * [ZF_PROBE_BLOCKS], receives a checksum per workgroup.  bytes > 0, a multiple of 16, and buf
 * 16-byte aligned, else ZF_EINVAL.  One kernel launch. */
#define ZF_PROBE_BLOCKS 4096
zf_status zf_stream_read_probe(const void* buf, size_t bytes, uint32_t* sink, zf_stream_t stream);

/* Measurement aid, outside the method: copies `bytes` of device memory from `src` to `dst`
 * once, with 16-byte non-temporal loads and stores over up to ZF_COPY_PROBE_BLOCKS
 * workgroups (a plain stream: the practically achievable HBM read-plus-write rate, context for
 * the codec kernels', which read one cache form and write the other).  Both 16-byte aligned,
 * bytes > 0 and a multiple of 16, the two ranges disjoint, else ZF_EINVAL.  Caller-owned
 * memory; one kernel launch on `stream`. */
#define ZF_COPY_PROBE_BLOCKS 32768
zf_status zf_stream_copy_probe(const void* src, void* dst, size_t bytes, zf_stream_t stream);

/* Status, outside the method: copies the sticky status word to *host_status (synchronizes
 * `stream`); a cache's word or the twin's. */
zf_status zf_get_status(const uint32_t* status, uint32_t* host_status, zf_stream_t stream);
/* Status, outside the method: a short text for a return code. */
const char* zf_status_str(zf_status s);

#ifdef __cplusplus
}
#endif
#endif
