/*
 * zf_oracle.c - plain, slow CPU oracle (TEST INFRASTRUCTURE ONLY; see zf_oracle.h).
 *
 * Every loop here follows the definition directly: no blocking, no fusion, no reordering.
 * Codec: ZipFusion video summary, chapter "Twelve Bits and One Addition" (shared base
 * exponent, 4-bit offset, raw fallback, one-add rebuild).  Attention: page "Open Weights:
 * from files to tokens / second", section "03 / The inference loop" (softmax attention of one
 * query token over the cached tokens), computed in fp64.
 */
#include "zf_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define BLOCK 64

static int exponent_of(uint16_t x) { return (x >> 7) & 0xFF; }

int orc_block_encode(const uint16_t x[64], uint8_t sm[64], uint8_t nib[32], uint8_t* base,
                     uint8_t spill[32]) {
  /* Step 1: the exponent window of the block. */
  int emin = 255, emax = 0, special = 0;
  for (int i = 0; i < BLOCK; ++i) {
    int e = exponent_of(x[i]);
    if (e == 0 || e == 255) special = 1; /* zero / subnormal, Inf / NaN */
    if (e < emin) emin = e;
    if (e > emax) emax = e;
  }
  /* Step 2: eligible iff every offset from the smallest exponent fits in 4 bits. */
  int raw = special || (emax - emin > 15);
  /* Step 3: per-value fields. */
  memset(nib, 0, 32);
  for (int i = 0; i < BLOCK; ++i) {
    int s = x[i] >> 15, m = x[i] & 0x7F, e = exponent_of(x[i]);
    sm[i] = (uint8_t)((s << 7) | m);
    int n = raw ? (e & 15) : (e - emin);
    if (i % 2 == 0)
      nib[i / 2] = (uint8_t)n;
    else
      nib[i / 2] |= (uint8_t)(n << 4);
  }
  /* Step 4: base exponent, or the raw block's exponent high nibbles. */
  if (raw) {
    *base = 0;
    for (int k = 0; k < 32; ++k)
      spill[k] = (uint8_t)((exponent_of(x[2 * k]) >> 4) | ((exponent_of(x[2 * k + 1]) >> 4) << 4));
  } else {
    *base = (uint8_t)emin;
  }
  return raw;
}

void orc_block_decode(const uint8_t sm[64], const uint8_t nib[32], uint8_t base,
                      const uint8_t spill[32], uint16_t out[64]) {
  for (int i = 0; i < BLOCK; ++i) {
    int n = (i % 2 == 0) ? (nib[i / 2] & 15) : (nib[i / 2] >> 4);
    uint16_t fields = (uint16_t)(((sm[i] & 0x80) << 8) | (sm[i] & 0x7F) | (n << 7));
    uint16_t addend;
    if (base != 0) {
      addend = (uint16_t)(base << 7);
    } else {
      int hi = (i % 2 == 0) ? (spill[i / 2] & 15) : (spill[i / 2] >> 4);
      addend = (uint16_t)(hi << 11);
    }
    out[i] = (uint16_t)(fields + addend); /* the single integer addition */
  }
}

/* ------------------------------------------------------------------ cache-level helpers */

static int64_t raw_index(const orc_geom* g, int64_t page, int h, int kv, int slot) {
  return (((page * g->num_kv_heads + h) * 2 + kv) * g->page_size + slot) * (int64_t)g->head_dim;
}

static int popcount32(uint32_t v) {
  int n = 0;
  while (v) { n += (int)(v & 1u); v >>= 1; }
  return n;
}

/* Checks the rows [0, len + extra) of every sequence against the page table. */
static uint32_t check_rows(const orc_geom* g, int32_t batch, const int32_t* lens,
                           const int32_t* pt, int32_t max_pages, int extra) {
  uint32_t st = 0;
  for (int b = 0; b < batch; ++b) {
    int64_t n = (int64_t)lens[b] + extra;
    if (lens[b] < 0 || n > (int64_t)max_pages * g->page_size) { st |= ORC_ELEN; continue; }
    for (int64_t t = (extra ? lens[b] : 0); t < n; ++t) {
      int32_t p = pt[(int64_t)b * max_pages + t / g->page_size];
      if (p < 0 || p >= g->num_pages) st |= ORC_EPAGE;
    }
  }
  return st;
}

/* Encodes the token row (page, slot) from the 2*H*(D/64) blocks of raw_row(h, kv); returns
 * the number of spill slots used, starting at `first_slot`. */
static int encode_row(const orc_geom* g, orc_cache* c, int64_t page, int slot,
                      const uint16_t* const* src, uint64_t first_slot, int write) {
  const int H = g->num_kv_heads, D = g->head_dim, nb = D / BLOCK, T = g->page_size;
  uint32_t flags = 0;
  int used = 0;
  for (int h = 0; h < H; ++h)
    for (int kv = 0; kv < 2; ++kv)
      for (int half = 0; half < nb; ++half) {
        int j = (h * 2 + kv) * nb + half;
        const uint16_t* x = src[h * 2 + kv] + half * BLOCK;
        uint8_t sm[64], nib[32], base, spill[32];
        int raw = orc_block_encode(x, sm, nib, &base, spill);
        if (write) {
          int64_t e = raw_index(g, page, h, kv, slot) + half * BLOCK;
          memcpy(c->sm + e, sm, 64);
          memcpy(c->nib + e / 2, nib, 32);
          c->base[e / BLOCK] = base;
          if (raw) memcpy(c->spill + (first_slot + used) * 32u, spill, 32);
        }
        if (raw) { flags |= 1u << j; ++used; }
      }
  if (write) {
    c->row_flags[page * T + slot] = flags;
    c->row_spill[page * T + slot] = (uint32_t)first_slot;
  }
  return used;
}

uint32_t orc_encode_kv(const orc_geom* g, orc_cache* c, int32_t batch, const int32_t* seq_lens,
                       const int32_t* page_table, int32_t max_pages, const uint16_t* raw_pages) {
  uint32_t st = check_rows(g, batch, seq_lens, page_table, max_pages, 0);
  if (st) return st;
  const int H = g->num_kv_heads, T = g->page_size;
  const uint16_t** src = (const uint16_t**)malloc(sizeof(uint16_t*) * 2 * (size_t)H);
  /* Pass 1: how many spill slots the whole call needs. */
  uint64_t need = 0;
  for (int pass = 0; pass < 2; ++pass) {
    uint64_t next = c->spill_top;
    for (int b = 0; b < batch; ++b)
      for (int t = 0; t < seq_lens[b]; ++t) {
        int64_t page = page_table[(int64_t)b * max_pages + t / T];
        for (int h = 0; h < H; ++h)
          for (int kv = 0; kv < 2; ++kv) src[h * 2 + kv] = raw_pages + raw_index(g, page, h, kv, t % T);
        next += (uint64_t)encode_row(g, c, page, t % T, src, next, pass == 1);
      }
    if (pass == 0) {
      need = next - c->spill_top;
      /* a top beyond the pool leaves no free slot */
      if (c->spill_top > c->spill_slots || need > c->spill_slots - c->spill_top) { free(src); return ORC_ESPILL; }
    } else {
      c->spill_top = next;
    }
  }
  free(src);
  return ORC_OK;
}

uint32_t orc_append_kv_n(const orc_geom* g, orc_cache* c, int32_t batch, int32_t n_new,
                         int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                         const uint16_t* k_new, const uint16_t* v_new) {
  if (n_new < 0) return ORC_ELEN;
  if (n_new == 0) return ORC_OK;
  uint32_t st = check_rows(g, batch, seq_lens, page_table, max_pages, n_new);
  if (st) return st;
  const int H = g->num_kv_heads, D = g->head_dim, T = g->page_size;
  const uint16_t** src = (const uint16_t**)malloc(sizeof(uint16_t*) * 2 * (size_t)H);
  /* pass 0 counts the spill slots (all or nothing), pass 1 writes */
  for (int pass = 0; pass < 2; ++pass) {
    uint64_t next = c->spill_top;
    for (int b = 0; b < batch; ++b)     /* rows in (sequence, token) order, like an encode */
      for (int j = 0; j < n_new; ++j) {
        int t = seq_lens[b] + j;
        int64_t page = page_table[(int64_t)b * max_pages + t / T];
        for (int h = 0; h < H; ++h) {
          src[h * 2 + 0] = k_new + (((int64_t)b * n_new + j) * H + h) * D;
          src[h * 2 + 1] = v_new + (((int64_t)b * n_new + j) * H + h) * D;
        }
        next += (uint64_t)encode_row(g, c, page, t % T, src, next, pass == 1);
      }
    if (pass == 0) {
      if (c->spill_top > c->spill_slots || next - c->spill_top > c->spill_slots - c->spill_top) {
        free(src);
        return ORC_ESPILL;
      }
    } else {
      c->spill_top = next;
    }
  }
  for (int b = 0; b < batch; ++b) seq_lens[b] += n_new;
  free(src);
  return ORC_OK;
}

uint32_t orc_append_kv(const orc_geom* g, orc_cache* c, int32_t batch, int32_t* seq_lens,
                       const int32_t* page_table, int32_t max_pages, const uint16_t* k_new,
                       const uint16_t* v_new) {
  return orc_append_kv_n(g, c, batch, 1, seq_lens, page_table, max_pages, k_new, v_new);
}

uint32_t orc_decode_kv(const orc_geom* g, const orc_cache* c, int32_t batch,
                       const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                       uint16_t* raw_out) {
  uint32_t st = check_rows(g, batch, seq_lens, page_table, max_pages, 0);
  if (st) return st;
  const int H = g->num_kv_heads, D = g->head_dim, nb = D / BLOCK, T = g->page_size;
  for (int b = 0; b < batch; ++b)
    for (int t = 0; t < seq_lens[b]; ++t) {
      int64_t page = page_table[(int64_t)b * max_pages + t / T];
      uint32_t flags = c->row_flags[page * T + t % T];
      uint64_t first = c->row_spill[page * T + t % T];
      for (int h = 0; h < H; ++h)
        for (int kv = 0; kv < 2; ++kv)
          for (int half = 0; half < nb; ++half) {
            int j = (h * 2 + kv) * nb + half;
            int64_t e = raw_index(g, page, h, kv, t % T) + half * BLOCK;
            int raw = (flags >> j) & 1u;
            uint8_t base = raw ? 0 : c->base[e / BLOCK];
            const uint8_t* spill = NULL;
            if (raw) {
              uint64_t slot = first + (uint64_t)popcount32(flags & ((1u << j) - 1u));
              if (slot >= c->spill_slots) return ORC_ESPILL;
              spill = c->spill + slot * 32u;
            }
            orc_block_decode(c->sm + e, c->nib + e / 2, base, spill, raw_out + e);
          }
    }
  return ORC_OK;
}

uint32_t orc_compact_spill(const orc_geom* g, orc_cache* c, int32_t batch,
                           const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages) {
  uint32_t st = check_rows(g, batch, seq_lens, page_table, max_pages, 0);
  if (st) return st;
  const int T = g->page_size;
  /* Pass 1: every listed row's slots must be live ones; count them. */
  uint64_t total = 0;
  for (int b = 0; b < batch; ++b)
    for (int t = 0; t < seq_lens[b]; ++t) {
      int64_t row = (int64_t)page_table[(int64_t)b * max_pages + t / T] * T + t % T;
      uint64_t n = (uint64_t)popcount32(c->row_flags[row]);
      if (n > 0 && (uint64_t)c->row_spill[row] + n > c->spill_top) return ORC_ESPILL;
      total += n;
    }
  /* Pass 2: copy the slots out in the new order, then write them back from slot 0. */
  uint8_t* fresh = (uint8_t*)malloc(total * 32u + 1u);
  uint64_t next = 0;
  for (int b = 0; b < batch; ++b)
    for (int t = 0; t < seq_lens[b]; ++t) {
      int64_t row = (int64_t)page_table[(int64_t)b * max_pages + t / T] * T + t % T;
      uint64_t n = (uint64_t)popcount32(c->row_flags[row]);
      if (n > 0) memcpy(fresh + next * 32u, c->spill + (uint64_t)c->row_spill[row] * 32u, n * 32u);
      c->row_spill[row] = (uint32_t)next;
      next += n;
    }
  memcpy(c->spill, fresh, total * 32u);
  free(fresh);
  c->spill_top = total;
  return ORC_OK;
}

int64_t orc_max_sequences(int64_t kv_budget, int32_t layers, int32_t context, int32_t page_size,
                          int32_t num_kv_heads, int32_t head_dim, double raw_blocks_per_row) {
  if (kv_budget <= 0 || layers <= 0 || context <= 0) return 0;
  int64_t rows = (int64_t)(context + page_size - 1) / page_size * page_size;
  int64_t vectors = (int64_t)num_kv_heads * 2;
  int64_t per_layer;
  if (raw_blocks_per_row < 0) {
    per_layer = rows * vectors * head_dim * 2;
  } else {
    int64_t row_bytes = vectors * (head_dim + head_dim / 2 + head_dim / 64) + 4 + 4;
    int64_t slots = (int64_t)ceil(raw_blocks_per_row * (double)context);
    per_layer = rows * row_bytes + slots * 32;
  }
  return kv_budget / (per_layer * layers);
}

static double bf16_value(uint16_t x) {
  uint32_t u = (uint32_t)x << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

uint32_t orc_attention(const orc_geom* g, int32_t batch, int32_t num_q_heads,
                       const int32_t* seq_lens, const int32_t* page_table, int32_t max_pages,
                       const uint16_t* raw_pages, const uint16_t* q, double scale,
                       const uint8_t* want, double* out, double* neff) {
  uint32_t st = check_rows(g, batch, seq_lens, page_table, max_pages, 0);
  if (st) return st;
  const int H = g->num_kv_heads, D = g->head_dim, T = g->page_size;
  const int group = num_q_heads / H;
  int32_t maxlen = 0;
  for (int b = 0; b < batch; ++b) if (seq_lens[b] > maxlen) maxlen = seq_lens[b];
  double* s = (double*)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
  for (int b = 0; b < batch; ++b)
    for (int hq = 0; hq < num_q_heads; ++hq) {
      if (want && !want[(int64_t)b * num_q_heads + hq]) continue;
      const int hk = hq / group;
      const uint16_t* qv = q + ((int64_t)b * num_q_heads + hq) * D;
      double* o = out + ((int64_t)b * num_q_heads + hq) * D;
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      if (neff) neff[(int64_t)b * num_q_heads + hq] = 0.0;
      const int L = seq_lens[b];
      if (L == 0) continue;
      /* scores s_t = scale * <q, k_t> */
      double mx = -INFINITY;
      for (int t = 0; t < L; ++t) {
        int64_t page = page_table[(int64_t)b * max_pages + t / T];
        const uint16_t* k = raw_pages + raw_index(g, page, hk, 0, t % T);
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += bf16_value(qv[d]) * bf16_value(k[d]);
        s[t] = scale * acc;
        if (s[t] > mx) mx = s[t];
      }
      /* softmax weights and the weighted sum of V */
      double denom = 0.0, sq = 0.0;
      for (int t = 0; t < L; ++t) {
        double w = exp(s[t] - mx);
        denom += w;
        sq += w * w;
        int64_t page = page_table[(int64_t)b * max_pages + t / T];
        const uint16_t* v = raw_pages + raw_index(g, page, hk, 1, t % T);
        for (int d = 0; d < D; ++d) o[d] += w * bf16_value(v[d]);
      }
      for (int d = 0; d < D; ++d) o[d] /= denom;
      if (neff) neff[(int64_t)b * num_q_heads + hq] = denom * denom / sq;
    }
  free(s);
  return ORC_OK;
}
