/*
 * synth.c - seeded synthetic inputs for the compressed-KV decode-attention workloads.
 *
 * This module only draws numbers. It holds none of the codec's or attention's arithmetic:
 * it produces bf16 K/V tokens, bf16 queries, context lengths and page tables, and both the
 * HIP path and the CPU oracle consume exactly the bits it writes.
 *
 * Random numbers come from one counter-based generator: SplitMix64 (Steele, Lea and Flood,
 * "Fast Splittable Pseudorandom Number Generators", OOPSLA 2014), whose i-th output for a
 * state s is mix(s + (i + 1) * gamma).  Every draw is therefore a pure function of
 * (seed, stream, counter), so any element can be regenerated on its own and the fill loops
 * may run in any order or in parallel.
 *
 * Value recipe for one element (K or V, sequence b, token t, kv head h, dim d):
 *   x  = N(0,1) * s[kv][h][d], rounded fp64 -> fp32 -> bf16 (round to nearest even),
 *        N(0,1) by the cosine branch of Box-Muller, s = exp(U(ln lo, ln hi)) per channel;
 *   wide blocks     (probability p_wide per 64-value block): x *= 2^k per value, k uniform
 *                   integer in [-12, 12];
 *   outlier blocks  (probability p_outlier per block, in K and/or V as outlier_kinds says): the
 *                   value at one uniform position *= 2^10;
 *   zero values     (probability p_zero per value): x = +0.0.
 * K and V are perturbed alike.
 * A 64-value block is 64 consecutive head_dim values of one (token, head, K-or-V).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

enum {
  ST_KSCALE = 1, ST_VSCALE, ST_VALUE, ST_WIDE, ST_WIDE_K, ST_OUT, ST_OUT_POS, ST_ZERO,
  ST_QUERY, ST_LEN, ST_PAGES
};

typedef struct {
  int32_t batch, num_kv_heads, num_q_heads, head_dim, page_size;
  int32_t ctx_min, ctx_max;      /* cached tokens per sequence: uniform integer in [min, max] */
  int32_t extra_tokens;          /* tokens appended later (pages are reserved for them) */
  double k_scale_lo, k_scale_hi; /* per-channel scale, log-uniform in [lo, hi] */
  double v_scale_lo, v_scale_hi;
  double p_outlier_block, p_zero_value, p_wide_block;
  double pool_factor;            /* page pool size / pages needed (>= 1) */
  uint64_t seed;
  int32_t outlier_kinds;         /* which tensors get outlier blocks: bit 0 K, bit 1 V */
} synth_cfg;

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(seed * GAMMA + stream);
}

/* i-th SplitMix64 output of the state `key` */
static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

static inline double uniform01(uint64_t key, uint64_t i) {
  return (double)(draw(key, i) >> 11) * 0x1.0p-53;
}

static inline double normal01(uint64_t key, uint64_t i) {
  double u1 = uniform01(key, 2 * i), u2 = uniform01(key, 2 * i + 1);
  return sqrt(-2.0 * log(1.0 - u1)) * cos(6.283185307179586476925 * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static double channel_scale(const synth_cfg* c, int kv, int h, int d) {
  double lo = kv ? c->v_scale_lo : c->k_scale_lo, hi = kv ? c->v_scale_hi : c->k_scale_hi;
  if (lo == hi) return lo;
  uint64_t key = stream_key(c->seed, kv ? ST_VSCALE : ST_KSCALE);
  double u = uniform01(key, ((uint64_t)h * (uint64_t)c->head_dim) + (uint64_t)d);
  return exp(log(lo) + u * (log(hi) - log(lo)));
}

/* Unique counter of an element; blocks are 64 consecutive d. */
static inline uint64_t element_id(const synth_cfg* c, int kv, int b, int t, int h, int d) {
  uint64_t row = ((uint64_t)b << 24) | (uint64_t)t;
  return (((row * (uint64_t)c->num_kv_heads + (uint64_t)h) * 2u + (uint64_t)kv) *
          (uint64_t)c->head_dim) + (uint64_t)d;
}

/* One element's bf16 bits; `scale` is channel_scale(c, kv, h, d). */
static uint16_t element(const synth_cfg* c, int kv, int b, int t, int h, int d, double scale) {
  uint64_t eid = element_id(c, kv, b, t, h, d), bid = eid / 64u;
  uint64_t s = c->seed;
  uint16_t x = f32_to_bf16_rne((float)(normal01(stream_key(s, ST_VALUE), eid) * scale));
  if (c->p_wide_block > 0 && uniform01(stream_key(s, ST_WIDE), bid) < c->p_wide_block) {
    int k = (int)floor(uniform01(stream_key(s, ST_WIDE_K), eid) * 25.0) - 12;
    x = f32_to_bf16_rne(ldexpf(bf16_to_f32(x), k));
  }
  if (c->p_outlier_block > 0 && ((c->outlier_kinds >> kv) & 1) &&
      uniform01(stream_key(s, ST_OUT), bid) < c->p_outlier_block) {
    int pos = (int)floor(uniform01(stream_key(s, ST_OUT_POS), bid) * 64.0);
    if ((d & 63) == pos) x = f32_to_bf16_rne(bf16_to_f32(x) * 1024.0f);
  }
  if (c->p_zero_value > 0 && uniform01(stream_key(s, ST_ZERO), eid) < c->p_zero_value) x = 0;
  return x;
}

/* ---------------------------------------------------------------- exported API */

void synth_seq_lens(const synth_cfg* c, int32_t* lens) {
  uint64_t key = stream_key(c->seed, ST_LEN);
  for (int b = 0; b < c->batch; ++b) {
    if (c->ctx_max <= c->ctx_min) { lens[b] = c->ctx_min; continue; }
    int64_t span = (int64_t)c->ctx_max - c->ctx_min + 1;
    lens[b] = c->ctx_min + (int32_t)floor(uniform01(key, (uint64_t)b) * (double)span);
  }
}

/* Pages reserved for sequence b: enough for lens[b] + extra_tokens tokens. */
static int32_t pages_for(const synth_cfg* c, int32_t len) {
  int64_t tok = (int64_t)len + c->extra_tokens;
  return (int32_t)((tok + c->page_size - 1) / c->page_size);
}

/* Returns the pool size (number of physical pages) and the widest row of the page table. */
void synth_pool_shape(const synth_cfg* c, const int32_t* lens, int32_t* num_pages,
                      int32_t* max_pages_per_seq) {
  int64_t need = 0;
  int32_t mx = 0;
  for (int b = 0; b < c->batch; ++b) {
    int32_t p = pages_for(c, lens[b]);
    need += p;
    if (p > mx) mx = p;
  }
  double f = c->pool_factor < 1.0 ? 1.0 : c->pool_factor;
  *num_pages = (int32_t)ceil((double)need * f);
  *max_pages_per_seq = mx;
}

/* Page table [batch][max_pages_per_seq]: a random permutation of the pool handed out to the
 * sequences in order; pool pages left over stay unused; unused table entries are -1. */
void synth_page_table(const synth_cfg* c, const int32_t* lens, int32_t num_pages,
                      int32_t max_pages_per_seq, int32_t* perm_scratch, int32_t* table) {
  uint64_t key = stream_key(c->seed, ST_PAGES);
  for (int32_t i = 0; i < num_pages; ++i) perm_scratch[i] = i;
  for (int32_t i = num_pages - 1; i > 0; --i) { /* Fisher-Yates */
    int32_t j = (int32_t)floor(uniform01(key, (uint64_t)i) * (double)(i + 1));
    int32_t tmp = perm_scratch[i];
    perm_scratch[i] = perm_scratch[j];
    perm_scratch[j] = tmp;
  }
  int64_t next = 0;
  for (int b = 0; b < c->batch; ++b) {
    int32_t p = pages_for(c, lens[b]);
    for (int32_t k = 0; k < max_pages_per_seq; ++k)
      table[(int64_t)b * max_pages_per_seq + k] = k < p ? perm_scratch[next + k] : -1;
    next += p;
  }
}

/* Raw paged cache u16[num_pages][H][2][page_size][D]: writes tokens [t0, t1) of every sequence
 * (clipped to lens[b] when clip_to_len is set), leaving every other slot untouched. */
void synth_fill_pages(const synth_cfg* c, const int32_t* lens, const int32_t* table,
                      int32_t max_pages_per_seq, int32_t t0, int32_t t1, int clip_to_len,
                      uint16_t* pages) {
  const int H = c->num_kv_heads, D = c->head_dim, T = c->page_size;
  double* sc = (double*)malloc(sizeof(double) * 2 * (size_t)H * (size_t)D);
  if (!sc) return;
  for (int kv = 0; kv < 2; ++kv)
    for (int h = 0; h < H; ++h)
      for (int d = 0; d < D; ++d) sc[((size_t)kv * H + h) * D + d] = channel_scale(c, kv, h, d);
  for (int b = 0; b < c->batch; ++b) {
    int32_t end = t1;
    if (clip_to_len && lens[b] < end) end = lens[b];
    int32_t n = end - t0;
    if (n <= 0) continue;
#pragma omp parallel for schedule(static)
    for (int32_t i = 0; i < n; ++i) {
      int32_t t = t0 + i;
      int64_t page = table[(int64_t)b * max_pages_per_seq + t / T];
      int32_t slot = t % T;
      for (int h = 0; h < H; ++h)
        for (int kv = 0; kv < 2; ++kv) {
          uint16_t* dst = pages + ((((page * H + h) * 2 + kv) * T + slot) * (int64_t)D);
          for (int d = 0; d < D; ++d)
            dst[d] = element(c, kv, b, t, h, d, sc[((size_t)kv * H + h) * D + d]);
        }
    }
  }
  free(sc);
}

/* One token per sequence at position pos[b]: k_out, v_out u16[batch][H][D]. */
void synth_fill_tokens(const synth_cfg* c, const int32_t* pos, uint16_t* k_out, uint16_t* v_out) {
  const int H = c->num_kv_heads, D = c->head_dim;
#pragma omp parallel for schedule(static)
  for (int b = 0; b < c->batch; ++b)
    for (int h = 0; h < H; ++h)
      for (int kv = 0; kv < 2; ++kv) {
        uint16_t* dst = (kv ? v_out : k_out) + ((int64_t)b * H + h) * D;
        for (int d = 0; d < D; ++d) dst[d] = element(c, kv, b, pos[b], h, d, channel_scale(c, kv, h, d));
      }
}

/* Queries for decode step `step`: u16[batch][num_q_heads][D], N(0,1) rounded to bf16. */
void synth_fill_query(const synth_cfg* c, int32_t step, uint16_t* q) {
  uint64_t key = stream_key(c->seed, ST_QUERY);
  int64_t n = (int64_t)c->batch * c->num_q_heads * c->head_dim;
  uint64_t base = (uint64_t)step * (uint64_t)n;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) q[i] = f32_to_bf16_rne((float)normal01(key, base + (uint64_t)i));
}
