/*
 * zf_oracle.h - plain, slow CPU oracle for the lossless compressed-KV decode-attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link, load or call this
 * code; only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It shares no
 * code with the HIP library.
 *
 * What it computes, and where each part comes from:
 *  - Block codec (ZipFusion video summary, "Run AI Faster With Lossless Compressed Memory",
 *    chapter "Twelve Bits and One Addition"): a block of BF16 values keeps one shared base
 *    exponent and a 4-bit exponent offset per value next to each value's sign and mantissa,
 *    12 bits per value; blocks whose exponents are too spread out stay uncompressed; values are
 *    rebuilt with one integer addition.  Open points and the readings taken:
 *      block = 64 consecutive head_dim values of one (token, kv head, K or V);
 *      base  = the smallest exponent of the block (offsets 0..15, a 16-wide window);
 *      raw   = any exponent field 0 (zero, subnormal) or 255 (Inf, NaN), or max - min > 15;
 *      sm byte = sign << 7 | mantissa; nibble k of a block = offset (raw: exponent & 15),
 *      two per byte, low nibble first; raw blocks keep base 0 and park the exponents' high
 *      nibbles (exponent >> 4), packed the same way, in a 32-byte spill slot.
 *  - Spill slots: a token row's raw blocks take consecutive slots in block order; rows are
 *    numbered (sequence, token) ascending for a full encode and in batch order for an append.
 *  - Spill lifecycle: pages come and go with their sequences (paged cache: page "Open
 *    Weights: from files to tokens / second", section "09 / The optimization stack"), but the
 *    spill pool only grows; compaction rewrites it for the sequences still live, as if they had
 *    been encoded into an empty pool: slots from 0 in (sequence, token) order.
 *  - Capacity (same page, step "Spend the memory dividend" of its deployment checklist, and
 *    section "05 / Memory is the admission ticket"): the device memory left after the weights
 *    (parameters x bits / 8) and a reserve goes to the paged KV cache, and the number of
 *    sequences that fit is that budget over one sequence's cache across all layers.
 *  - Attention (page "Open Weights: from files to tokens / second", section
 *    "03 / The inference loop"): one query token per sequence attends over every cached token of its
 *    sequence; grouped-query heads share a KV head (q head -> q / (Hq / Hkv)); scaled dot
 *    product with scale 1/sqrt(D), softmax, weighted sum of V; computed in fp64 from the bf16
 *    inputs.
 *
 * Layout of the packed cache (all host memory here, same byte order as the format):
 *   sm        u8 [P][H][2][T][D]        sign << 7 | mantissa
 *   nib       u8 [P][H][2][T][D/2]      offsets (raw: exponent & 15), low nibble first
 *   base      u8 [P][H][2][T][D/64]     base exponent, 0 = raw block
 *   row_flags u32[P][T]                 bit j set = block j of the token row is raw,
 *                                        j = (h * 2 + kv) * (D/64) + half
 *   row_spill u32[P][T]                 spill slot of the row's first raw block
 *   spill     u8 [S][32]                raw blocks' exponent high nibbles
 */
#ifndef ZF_ORACLE_H
#define ZF_ORACLE_H
#include <stdint.h>

#define ORC_OK 0u
#define ORC_ESPILL 1u  /* spill pool exhausted: the call wrote no spill and kept spill_top   */
#define ORC_EPAGE 2u   /* a page-table entry needed by the call is outside [0, num_pages)     */
#define ORC_ELEN 4u    /* a sequence length is negative or exceeds its page-table row         */

typedef struct {
  int32_t num_pages, page_size, num_kv_heads, head_dim;
} orc_geom;

typedef struct {
  uint8_t* sm;
  uint8_t* nib;
  uint8_t* base;
  uint32_t* row_flags;
  uint32_t* row_spill;
  uint8_t* spill;
  uint64_t spill_slots;
  uint64_t spill_top;
} orc_cache;

/* One 64-value block.  Returns 1 if the block stays raw, 0 if compressed. */
int orc_block_encode(const uint16_t x[64], uint8_t sm[64], uint8_t nib[32], uint8_t* base,
                     uint8_t spill[32]);
/* Inverse; `spill` is read only when base == 0. */
void orc_block_decode(const uint8_t sm[64], const uint8_t nib[32], uint8_t base,
                      const uint8_t spill[32], uint16_t out[64]);

/* Encode tokens [0, seq_lens[b]) of every sequence from raw pages u16[P][H][2][T][D]. */
uint32_t orc_encode_kv(const orc_geom* g, orc_cache* c, int32_t batch, const int32_t* seq_lens,
                       const int32_t* page_table, int32_t max_pages, const uint16_t* raw_pages);
/* Encode one new token per sequence (k_new, v_new u16[B][H][D]) at position seq_lens[b];
 * on success every seq_lens[b] grows by one. */
uint32_t orc_append_kv(const orc_geom* g, orc_cache* c, int32_t batch, int32_t* seq_lens,
                       const int32_t* page_table, int32_t max_pages, const uint16_t* k_new,
                       const uint16_t* v_new);
/* Encode n_new tokens per sequence (k_new, v_new u16[B][n_new][H][D]) at positions
 * seq_lens[b] .. seq_lens[b] + n_new - 1, spill slots taken in (sequence, token) order; on
 * success every seq_lens[b] grows by n_new.  All or nothing.  n_new = 1 is orc_append_kv. */
uint32_t orc_append_kv_n(const orc_geom* g, orc_cache* c, int32_t batch, int32_t n_new,
                         int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                         const uint16_t* k_new, const uint16_t* v_new);
/* Rebuild tokens [0, seq_lens[b]) into raw pages u16[P][H][2][T][D]. */
uint32_t orc_decode_kv(const orc_geom* g, const orc_cache* c, int32_t batch,
                       const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                       uint16_t* raw_out);
/* Compaction of the spill pool for the listed sequences: the raw blocks of their rows
 * [0, seq_lens[b]) move to slots 0, 1, ... in (sequence, token) order, row_spill of those rows
 * follows, spill_top becomes their count.  Rows of other sequences are not touched (their
 * slots are given up).  All or nothing: a listed row whose slots are not inside
 * [0, spill_top) fails the call with ORC_ESPILL before anything is written. */
uint32_t orc_compact_spill(const orc_geom* g, orc_cache* c, int32_t batch,
                           const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages);
/* Capacity model: how many sequences of `context` tokens fit in `kv_budget` bytes of
 * device memory across `layers` layers.  Per sequence and layer: ceil(context / T) pages of
 * T token rows.  Uncompressed (raw_blocks_per_row < 0): a row is H x 2 x D bf16 values.
 * Packed: a row is its planes (sm D bytes, offsets D/2 bytes, one base byte per 64 values,
 * for H x 2 vectors) plus a flag word and a spill index (4 bytes each), and the sequence adds
 * ceil(raw_blocks_per_row x context) spill slots of 32 bytes. */
int64_t orc_max_sequences(int64_t kv_budget, int32_t layers, int32_t context, int32_t page_size,
                          int32_t num_kv_heads, int32_t head_dim, double raw_blocks_per_row);
/* fp64 decode attention over raw bf16 pages; q u16[B][Hq][D]; out f64[B][Hq][D].
 * `want` (u8[B][Hq], may be NULL = all) selects which (sequence, q head) rows to compute;
 * rows not wanted are not written.  `neff` (f64[B][Hq], may be NULL) receives each computed
 * row's effective number of tokens, (sum of weights)^2 / (sum of squared weights): 1 when one
 * token takes all the weight, L when all L tokens weigh the same (0 for L = 0). */
uint32_t orc_attention(const orc_geom* g, int32_t batch, int32_t num_q_heads,
                       const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                       const uint16_t* raw_pages, const uint16_t* q, double scale,
                       const uint8_t* want, double* out, double* neff);

#endif
