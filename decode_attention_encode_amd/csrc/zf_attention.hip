// zf_attention.hip - fused GQA decode attention over the packed paged cache (gfx950).
//
// Method: ZipFusion video summary ("Run AI Faster With Lossless Compressed Memory"): the
// cache stays compressed in HBM and each bf16 is rebuilt in registers with one integer add
// (two values per 32-bit add here) right before it is used; decode is bound by the bytes
// read per step, so reading 12-bit values instead of 16-bit ones is the whole gain.
// Attention itself is the plain decode step (essay "Open weights as an optimization
// surface": one new token per sequence attends over its KV cache).
//
// Mapping (head_dim 128, 16-token pages, 4 query heads per kv head):
//   grid (split, kv head, sequence); 4 waves per workgroup; a wave takes one page at a time.
//   lane = token (lane & 15) x quarter (lane >> 4): a lane owns 32 head_dim values of one
//   token of K and of V, read as 16-byte loads from the sm and nibble planes.
//   q.K^T: v_mfma_f32_16x16x32_bf16 with the rebuilt K pairs as B (k = head_dim, n = token)
//   and the 4 query heads replicated over the 16 rows of A, so that every lane receives the
//   4 scores of its own token with no cross-lane reduction.  Products of bf16 are exact and
//   sums are fp32.
//   softmax: running max per head kept per wave and only raised (with a rescale) when a page
//   exceeds it; p = exp2((s - m) * scale * log2 e).
//   p.V: fp32 FMAs, each lane accumulating its 32 dims x 4 heads over its token slot; one
//   reduce-scatter across the 16 token lanes per split, then the 4 waves merge in LDS.
//   Splits of the token axis write (m, l, acc) partials; the last workgroup of a (sequence,
//   kv head) to finish merges them in split order, so results do not depend on timing.
// The same kernel body reads either the packed planes or raw bf16 pages (the "twin"); both
// loaders hand identical bf16 pairs to identical arithmetic, so outputs match bit for bit.
#include <algorithm>
#include <stdlib.h>

#include "zf_internal.h"

namespace zf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128, kT = 16, kG = 4, kWaves = 4, kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  int32_t B, H, maxp, max_seq_len, pps, nsplit_max, num_pages;
  const int32_t* pt;
  const int32_t* lens;
  const uint16_t* q;
  float scale_log2e;
  float* out;
  float* part;        // [B][H][nsplit_max][kG * (kD + 2)]
  uint32_t* counter;  // [B][H]
  uint32_t* status;
};

// ---------------------------------------------------------------- loaders
// Both fill kp/vp with 16 bf16 pairs: pair 4c + r = (dim 32*qd + 8c + r, same + 4).

struct PackedLoader {
  const uint8_t* sm;
  const uint8_t* nib;
  const uint8_t* base;
  const uint32_t* row_flags;
  const uint32_t* row_spill;
  const uint8_t* spill;
  uint64_t spill_slots;

  __device__ __forceinline__ void load(int H, int64_t pid, int h, int t, int qd, bool valid,
                                       uint32_t kp[16], uint32_t vp[16]) const {
    const uint32_t flags = row_flags[pid * kT + t];
    const uint32_t first = row_spill[pid * kT + t];
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const int64_t hrow = ((pid * H + h) * 2 + kv) * kT + t;  // (page, head, kv, token)
      const uint4* smp = reinterpret_cast<const uint4*>(sm + hrow * kD + qd * 32);
      const uint4 s0 = smp[0], s1 = smp[1];
      const uint4 nb = *reinterpret_cast<const uint4*>(nib + hrow * (kD / 2) + qd * 16);
      const uint32_t bexp = base[hrow * 2 + (qd >> 1)];
      const int j = (h * 2 + kv) * 2 + (qd >> 1);
      const bool raw = valid && ((flags >> j) & 1u);
      uint4 hi = make_uint4(0u, 0u, 0u, 0u);
      if (raw) {
        const uint64_t slot = (uint64_t)first + __popc(flags & ((1u << j) - 1u));
        if (slot < spill_slots)
          hi = *reinterpret_cast<const uint4*>(spill + slot * 32u + (qd & 1) * 16);
      }
      const uint32_t bp = raw ? 0u : bexp * 0x00800080u;
      uint32_t* dst = kv ? vp : kp;
      const uint32_t smw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      const uint32_t nw[4] = {nb.x, nb.y, nb.z, nb.w};
      const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) rebuild8(smw[2 * c], smw[2 * c + 1], nw[c], hw[c], bp, dst + 4 * c);
    }
  }
};

struct RawLoader {
  const uint16_t* pages;

  __device__ __forceinline__ void load(int H, int64_t pid, int h, int t, int qd, bool /*valid*/,
                                       uint32_t kp[16], uint32_t vp[16]) const {
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const int64_t hrow = ((pid * H + h) * 2 + kv) * kT + t;
      const uint4* src = reinterpret_cast<const uint4*>(pages + hrow * kD + qd * 32);
      uint32_t* dst = kv ? vp : kp;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 x = src[c];
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        natural_to_pairs(w, dst + 4 * c);
      }
    }
  }
};

// ---------------------------------------------------------------- kernel

__device__ __forceinline__ float row_max16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 16));
  return v;
}

__device__ __forceinline__ float row_sum16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 16);
  return v;
}

// acc slot j (0..31) of a lane with quarter qd holds head_dim 32*qd + 8*(j/8) + (j%8)/2 + 4*(j%2).
__device__ __forceinline__ int slot_dim(int qd, int j) {
  return 32 * qd + 8 * (j >> 3) + ((j & 7) >> 1) + 4 * (j & 1);
}

template <class Loader>
__global__ __launch_bounds__(kThreads, 2) void attn_k(AttnArgs a, Loader ld) {
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t = lane & 15, qd = lane >> 4;

  int32_t L = a.lens[b];
  const int32_t cap = min(a.maxp * kT, a.max_seq_len);
  if (L < 0 || L > cap) {
    if (s == 0 && tid == 0) set_status(a.status, ZF_DEV_ELEN);
    L = L < 0 ? 0 : cap;
  }
  const int npages = (L + kT - 1) / kT;
  const int nsplit = max(1, (npages + a.pps - 1) / a.pps);
  if (s >= nsplit) return;

  // A operand: query head (lane & 15) & 3, head_dim 32*qd + 8c + (0,4,1,5,2,6,3,7)[k].
  bf16x8 qa[4];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * a.H * kG + h * kG + (t & 3)) * kD + qd * 32;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 x = *reinterpret_cast<const uint4*>(qrow + 8 * c);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
      uint32_t p[4];
      natural_to_pairs(w, p);
      qa[c] = __builtin_bit_cast(bf16x8, (u32x4){p[0], p[1], p[2], p[3]});
    }
  }

  float m[kG], l[kG], acc[kG][32];
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[i][j] = 0.f;
  }
  const float c2 = a.scale_log2e;
  const int p_end = min(npages, (s + 1) * a.pps);
  uint32_t err = 0;

  for (int p = s * a.pps + wave; p < p_end; p += kWaves) {
    const int32_t pid = a.pt[(int64_t)b * a.maxp + p];
    if (pid < 0 || pid >= a.num_pages) {
      err |= ZF_DEV_EPAGE;
      continue;
    }
    const int ntok = min(kT, L - p * kT);
    const bool valid = t < ntok;
    uint32_t kp[16], vp[16];
    ld.load(a.H, pid, h, t, qd, valid, kp, vp);

    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 kb = __builtin_bit_cast(bf16x8, (u32x4){kp[4 * c], kp[4 * c + 1], kp[4 * c + 2], kp[4 * c + 3]});
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[c], kb, sc, 0, 0, 0);
    }
    float sv[kG];
#pragma unroll
    for (int i = 0; i < kG; ++i) sv[i] = valid ? sc[i] : -INFINITY;
    if (ntok < kT) {
#pragma unroll
      for (int k = 0; k < 16; ++k) vp[k] = valid ? vp[k] : 0u;
    }

    bool raise = false;
#pragma unroll
    for (int i = 0; i < kG; ++i) raise |= sv[i] > m[i];
    if (__any(raise)) {
#pragma unroll
      for (int i = 0; i < kG; ++i) {
        const float mn = fmaxf(m[i], row_max16(sv[i]));
        const float alpha = exp2f((m[i] - mn) * c2);
        m[i] = mn;
        l[i] *= alpha;
#pragma unroll
        for (int j = 0; j < 32; ++j) acc[i][j] *= alpha;
      }
    }
    float pw[kG];
#pragma unroll
    for (int i = 0; i < kG; ++i) {
      pw[i] = exp2f((sv[i] - m[i]) * c2);
      l[i] += pw[i];
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float lo = __uint_as_float(vp[k] << 16), hi = __uint_as_float(vp[k] & 0xFFFF0000u);
#pragma unroll
      for (int i = 0; i < kG; ++i) {
        acc[i][2 * k] = fmaf(pw[i], lo, acc[i][2 * k]);
        acc[i][2 * k + 1] = fmaf(pw[i], hi, acc[i][2 * k + 1]);
      }
    }
  }
  if (err && lane == 0) set_status(a.status, err);

  // ---- reduce over the 16 token lanes: reduce-scatter, lane t ends with flat [8t, 8t + 8)
  float* flat = &acc[0][0];
#pragma unroll
  for (int step = 0; step < 4; ++step) {
    const int half = 64 >> step, mask = 8 >> step;
    const bool up = (t & mask) != 0;
#pragma unroll
    for (int k = 0; k < half; ++k) {
      const float send = up ? flat[k] : flat[k + half];
      const float keep = up ? flat[k + half] : flat[k];
      flat[k] = keep + __shfl_xor(send, mask, 16);
    }
  }
  // flat[0..7] of lane t = head t / 4, acc slots 8 * (t % 4) + k
  __shared__ float s_acc[kWaves][kG][kD];
  __shared__ float s_m[kWaves][kG], s_l[kWaves][kG];
  {
    const int i = t >> 2;
#pragma unroll
    for (int k = 0; k < 8; ++k) s_acc[wave][i][slot_dim(qd, 8 * (t & 3) + k)] = flat[k];
  }
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    const float lt = row_sum16(l[i]);
    if (lane == 0) {
      s_m[wave][i] = m[i];
      s_l[wave][i] = lt;
    }
  }
  __syncthreads();

  // ---- merge the 4 waves, write this split's partial
  const int64_t unit = (int64_t)b * a.H + h;
  float* part = a.part + (unit * a.nsplit_max + s) * (kG * (kD + 2));
  for (int e = tid; e < kG * kD; e += kThreads) {
    const int i = e / kD, d = e % kD;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, s_m[w][i]);
    float sum = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = s_m[w][i] == -INFINITY ? 0.f : exp2f((s_m[w][i] - mm) * c2);
      sum = fmaf(f, s_acc[w][i][d], sum);
      lsum = fmaf(f, s_l[w][i], lsum);
    }
    part[i * kD + d] = sum;
    if (d == 0) {
      part[kG * kD + i] = mm;
      part[kG * kD + kG + i] = lsum;
    }
  }

  // ---- last workgroup of this (sequence, kv head) merges the splits in order
  __shared__ uint32_t s_last;
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&a.counter[unit], 1u) == (uint32_t)(nsplit - 1)) ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const float* base = a.part + unit * a.nsplit_max * (kG * (kD + 2));
  for (int e = tid; e < kG * kD; e += kThreads) {
    const int i = e / kD, d = e % kD;
    float mm = -INFINITY;
    for (int x = 0; x < nsplit; ++x) mm = fmaxf(mm, base[x * (kG * (kD + 2)) + kG * kD + i]);
    float sum = 0.f, lsum = 0.f;
    for (int x = 0; x < nsplit; ++x) {
      const float* px = base + x * (kG * (kD + 2));
      const float mx = px[kG * kD + i];
      const float f = mx == -INFINITY ? 0.f : exp2f((mx - mm) * c2);
      sum = fmaf(f, px[i * kD + d], sum);
      lsum = fmaf(f, px[kG * kD + kG + i], lsum);
    }
    a.out[((int64_t)b * a.H * kG + h * kG + i) * kD + d] = lsum > 0.f ? sum / lsum : 0.f;
  }
  if (tid == 0) a.counter[unit] = 0u;
}

// ---------------------------------------------------------------- plan + launch

struct Plan {
  int pps, nsplit_max;
};

static int env_pps() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("ZF_PAGES_PER_SPLIT");
    v = e ? atoi(e) : 0;
    if (v < 0) v = 0;
  }
  return v;
}

// Pages per split: enough workgroups to fill 256 CUs several times over, at least 2 pages
// per wave, a multiple of the 4 waves.
static Plan make_plan(int32_t B, int32_t H, int32_t max_seq_len) {
  const int maxpages = std::max(1, (max_seq_len + kT - 1) / kT);
  int pps = env_pps();
  if (pps == 0) {
    const int64_t units = (int64_t)B * H;
    const int64_t target = 2048;
    int64_t want_splits = (target + units - 1) / std::max<int64_t>(units, 1);
    pps = (int)((maxpages + want_splits - 1) / std::max<int64_t>(want_splits, 1));
    pps = std::max(pps, 8);
  }
  pps = (pps + kWaves - 1) / kWaves * kWaves;
  return Plan{pps, (maxpages + pps - 1) / pps};
}

size_t attention_workspace_bytes(int32_t B, int32_t H, int32_t max_seq_len) {
  Plan pl = make_plan(B, H, max_seq_len);
  size_t part = (size_t)B * H * pl.nsplit_max * kG * (kD + 2) * sizeof(float);
  size_t cnt = (size_t)B * H * sizeof(uint32_t);
  return 256 + ((cnt + 255) / 256) * 256 + part;
}

template <class Loader>
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
  a.pt = q->page_table;
  a.lens = q->seq_lens;
  a.q = qv;
  a.scale_log2e = scale * kLog2e;
  a.out = out;
  size_t cnt = (size_t)q->batch * H * sizeof(uint32_t);
  a.counter = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + 256);
  a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + 256 + ((cnt + 255) / 256) * 256);
  a.status = status;
  dim3 grid(pl.nsplit_max, H, q->batch);
  hipLaunchKernelGGL(attn_k<Loader>, grid, dim3(kThreads), 0, st, a, ld);
  return hipGetLastError();
}

hipError_t launch_attention_packed(const zf_cache* c, const zf_seqs* q, const uint16_t* qv,
                                   float scale, float* out, void* ws, hipStream_t st) {
  PackedLoader ld{c->sm, c->nib, c->base, c->row_flags, c->row_spill, c->spill, c->spill_slots};
  return launch(ld, c->num_pages, c->num_kv_heads, q, qv, scale, out, ws, c->status, st);
}

hipError_t launch_attention_raw(const uint16_t* pages, int32_t num_pages, int32_t H,
                                const zf_seqs* q, const uint16_t* qv, float scale, float* out,
                                void* ws, uint32_t* status, hipStream_t st) {
  RawLoader ld{pages};
  return launch(ld, num_pages, H, q, qv, scale, out, ws, status, st);
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
