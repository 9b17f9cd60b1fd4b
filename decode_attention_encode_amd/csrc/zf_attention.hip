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
// Mapping (head_dim 128, 16-token pages, 4 query heads per kv head):
//   grid (split, kv head, sequence); 4 waves per workgroup; wave w takes pages w, w+4, ...
//   of its split, one page per step of a software pipeline: row metadata (flags, spill
//   base) two pages ahead, planes and spill slots one page ahead, compute on the current one.
//   K: lane = token (lane & 15) x quarter (lane >> 4), 32 head_dim values per lane read as
//   16-byte loads.  q.K^T runs on v_mfma_f32_16x16x32_bf16 with the rebuilt K pairs as B
//   (k = head_dim, n = token) and the 4 query heads replicated over the 16 rows of A, so
//   every lane receives the 4 scores of its own token without a cross-lane reduction.
//   V: lane = token (lane & 7, two passes of 8 tokens) x 16 head_dim values (lane >> 3);
//   p.V is fp32 FMAs into 4 heads x 16 dims per lane, reduced across the 8 token lanes once
//   per split, then across the 4 waves in LDS.
//   Softmax: running max per head in fp64, raised (with a rescale) only when a page exceeds
//   it.  Pages holding a score with |q.k| > kBigScore get exact fp64 scores: at that size one
//   fp32 ulp of a score is already a visible change of its weight.
//   Splits of the token axis write (acc, l, m) partials; a second small kernel merges them
//   in split order, so results do not depend on timing.
// One kernel body serves the packed cache and raw bf16 pages (the uncompressed twin): both
// loaders hand the same bf16 pairs to the same arithmetic, so the outputs match bit for bit.
#include <algorithm>
#include <stdlib.h>

#include "zf_internal.h"

namespace zf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128, kT = 16, kG = 4, kWaves = 4, kThreads = 64 * kWaves;
constexpr double kLog2e = 1.4426950408889634;
constexpr float kBigScore = 64.f;  // |q.k| above which a page's scores are recomputed in fp64
constexpr int kMaxPagesPerSplit = 4 * 64;  // each wave keeps its page ids in one register
// One split's partial: acc[kG][kD] f32, l[kG] f32, m[kG] f64 (8-byte aligned).
constexpr int kPartFloats = kG * kD + kG + 2 * kG;

struct AttnArgs {
  int32_t B, H, maxp, max_seq_len, pps, nsplit_max, num_pages;
  const int32_t* pt;
  const int32_t* lens;
  const uint16_t* q;
  double scale_log2e;
  float* out;
  float* part;        // [B][H][nsplit_max][kPartFloats]
  uint32_t* counter;  // [B][H]
  uint32_t* status;
};

// ---------------------------------------------------------------- loaders
// issue_meta / issue_bufs only start loads; rebuild turns one page's buffers into bf16 pairs:
//   kp[4c + r] = K (dim 32*qd + 8c + r, same + 4) of token lane & 15
//   vp[8ps + 4c + r] = V (dim 16*g + 8c + r, same + 4) of token 8*ps + (lane & 7), g = lane >> 3

struct PackedLoader {
  const uint8_t* sm;
  const uint8_t* nib;
  const uint8_t* base;
  const uint32_t* row_flags;
  const uint32_t* row_spill;
  const uint8_t* spill;  // a readable address even when spill_slots == 0
  uint64_t spill_slots;

  struct Meta {
    uint32_t fk, sk, fv[2], sv[2];  // flags and first spill slot of the rows this lane reads
  };
  struct Bufs {
    uint4 ks0, ks1, kn, kh;
    uint4 vs[2], vh2;  // vh2: the two passes' 8-byte spill pieces
    uint2 vn[2];
    uint32_t kb, vb[2], vmask;  // base bytes; bit ps of vmask = V block raw
    uint32_t kraw;
  };

  __device__ __forceinline__ Meta issue_meta(int64_t pid, int lane) const {
    const int t = lane & 15, tv = lane & 7;
    Meta m;
    m.fk = row_flags[pid * kT + t];
    m.sk = row_spill[pid * kT + t];
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      m.fv[ps] = row_flags[pid * kT + 8 * ps + tv];
      m.sv[ps] = row_spill[pid * kT + 8 * ps + tv];
    }
    return m;
  }

  // slot of block j of a row, or -1 when the block is compressed / out of the pool
  __device__ __forceinline__ int64_t slot_of(uint32_t flags, uint32_t first, int j) const {
    if (!((flags >> j) & 1u)) return -1;
    const uint64_t slot = (uint64_t)first + __popc(flags & ((1u << j) - 1u));
    return slot < spill_slots ? (int64_t)slot : -1;
  }

  __device__ __forceinline__ Bufs issue_bufs(int H, int64_t pid, int h, int lane, const Meta& m) const {
    const int t = lane & 15, qd = lane >> 4, tv = lane & 7, g = lane >> 3;
    Bufs b;
    const int64_t krow = ((pid * H + h) * 2 + 0) * kT + t;
    const uint4* kp = reinterpret_cast<const uint4*>(sm + krow * kD + qd * 32);
    b.ks0 = kp[0];
    b.ks1 = kp[1];
    b.kn = *reinterpret_cast<const uint4*>(nib + krow * (kD / 2) + qd * 16);
    b.kb = base[krow * 2 + (qd >> 1)];
    const int64_t ks = slot_of(m.fk, m.sk, (h * 2 + 0) * 2 + (qd >> 1));
    b.kraw = ks >= 0;
    b.kh = *reinterpret_cast<const uint4*>(spill + (ks >= 0 ? ks * 32 + (qd & 1) * 16 : 0));
    b.vmask = 0u;
    uint32_t vh[4];
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const int64_t vrow = ((pid * H + h) * 2 + 1) * kT + 8 * ps + tv;
      b.vs[ps] = *reinterpret_cast<const uint4*>(sm + vrow * kD + g * 16);
      b.vn[ps] = *reinterpret_cast<const uint2*>(nib + vrow * (kD / 2) + g * 8);
      b.vb[ps] = base[vrow * 2 + (g >> 2)];
      const int64_t vsl = slot_of(m.fv[ps], m.sv[ps], (h * 2 + 1) * 2 + (g >> 2));
      b.vmask |= (uint32_t)(vsl >= 0) << ps;
      const uint2 x = *reinterpret_cast<const uint2*>(spill + (vsl >= 0 ? vsl * 32 + (g & 3) * 8 : 0));
      vh[2 * ps] = x.x;
      vh[2 * ps + 1] = x.y;
    }
    b.vh2 = make_uint4(vh[0], vh[1], vh[2], vh[3]);
    return b;
  }

  __device__ __forceinline__ void rebuild(const Bufs& b, uint32_t kp[16], uint32_t vp[16]) const {
    {
      const uint32_t bp = b.kraw ? 0u : b.kb * 0x00800080u;
      const uint4 hi = b.kraw ? b.kh : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t smw[8] = {b.ks0.x, b.ks0.y, b.ks0.z, b.ks0.w, b.ks1.x, b.ks1.y, b.ks1.z, b.ks1.w};
      const uint32_t nw[4] = {b.kn.x, b.kn.y, b.kn.z, b.kn.w};
      const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) rebuild8(smw[2 * c], smw[2 * c + 1], nw[c], hw[c], bp, kp + 4 * c);
    }
    const uint32_t vh[4] = {b.vh2.x, b.vh2.y, b.vh2.z, b.vh2.w};
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const bool raw = (b.vmask >> ps) & 1u;
      const uint32_t bp = raw ? 0u : b.vb[ps] * 0x00800080u;
      const uint32_t smw[4] = {b.vs[ps].x, b.vs[ps].y, b.vs[ps].z, b.vs[ps].w};
      const uint32_t nw[2] = {b.vn[ps].x, b.vn[ps].y};
#pragma unroll
      for (int c = 0; c < 2; ++c)
        rebuild8(smw[2 * c], smw[2 * c + 1], nw[c], raw ? vh[2 * ps + c] : 0u, bp, vp + 8 * ps + 4 * c);
    }
  }
};

struct RawLoader {
  const uint16_t* pages;

  struct Meta {};
  struct Bufs {
    uint4 k[4];
    uint4 v[2][2];
  };

  __device__ __forceinline__ Meta issue_meta(int64_t, int) const { return Meta{}; }

  __device__ __forceinline__ Bufs issue_bufs(int H, int64_t pid, int h, int lane, const Meta&) const {
    const int t = lane & 15, qd = lane >> 4, tv = lane & 7, g = lane >> 3;
    Bufs b;
    const int64_t krow = ((pid * H + h) * 2 + 0) * kT + t;
    const uint4* kp = reinterpret_cast<const uint4*>(pages + krow * kD + qd * 32);
#pragma unroll
    for (int c = 0; c < 4; ++c) b.k[c] = kp[c];
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const int64_t vrow = ((pid * H + h) * 2 + 1) * kT + 8 * ps + tv;
      const uint4* vp = reinterpret_cast<const uint4*>(pages + vrow * kD + g * 16);
      b.v[ps][0] = vp[0];
      b.v[ps][1] = vp[1];
    }
    return b;
  }

  __device__ __forceinline__ void rebuild(const Bufs& b, uint32_t kp[16], uint32_t vp[16]) const {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t w[4] = {b.k[c].x, b.k[c].y, b.k[c].z, b.k[c].w};
      natural_to_pairs(w, kp + 4 * c);
    }
#pragma unroll
    for (int ps = 0; ps < 2; ++ps)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint32_t w[4] = {b.v[ps][c].x, b.v[ps][c].y, b.v[ps][c].z, b.v[ps][c].w};
        natural_to_pairs(w, vp + 8 * ps + 4 * c);
      }
  }
};

// ---------------------------------------------------------------- kernel

__device__ __forceinline__ double row_max16(double v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v = fmax(v, __shfl_xor(v, o, 16));
  return v;
}

__device__ __forceinline__ float row_sum16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 16);
  return v;
}

// V accumulator slot j (0..15) of lane group g holds head_dim 16*g + 8*(j/8) + (j%8)/2 + 4*(j%2).
__device__ __forceinline__ int vslot_dim(int g, int j) {
  return 16 * g + 8 * (j >> 3) + ((j & 7) >> 1) + 4 * (j & 1);
}

template <class Loader>
__global__ __launch_bounds__(kThreads, 2) void attn_k(AttnArgs a, Loader ld) {
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = lane & 15, qd = lane >> 4, tv = lane & 7, g = lane >> 3;

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
  // q in fp64, pair order, for the exact-score path: [head][quarter][pair] = (lo, hi) dims
  __shared__ double2 s_q64[kG][4][16];
  {
    const int i = tid >> 6, qq = (tid >> 4) & 3, k = tid & 15;
    const int dlo = 32 * qq + 8 * (k >> 2) + (k & 3);
    const uint16_t* qrow = a.q + ((int64_t)b * a.H * kG + h * kG + i) * kD;
    s_q64[i][qq][k] = make_double2((double)__uint_as_float((uint32_t)qrow[dlo] << 16),
                                   (double)__uint_as_float((uint32_t)qrow[dlo + 4] << 16));
  }

  // this wave's pages: p_first + 4n for n < nmine; lane n holds the page id of page n
  const int p_first = s * a.pps + wave;
  const int p_end = min(npages, (s + 1) * a.pps);
  const int nmine = p_first < p_end ? (p_end - p_first + kWaves - 1) / kWaves : 0;
  int32_t my_pid = 0;
  uint32_t err = 0;
  if (lane < nmine) {
    my_pid = a.pt[(int64_t)b * a.maxp + p_first + kWaves * lane];
    if (my_pid < 0 || my_pid >= a.num_pages) {
      err = ZF_DEV_EPAGE;
      my_pid = -1;  // page skipped: read page 0, count no token
    }
  }
  __syncthreads();

  double m[kG];  // running max of the unscaled scores, fp64
  float l[kG], acc[kG][16];
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
  }
  const double c2 = a.scale_log2e;

  auto pid_at = [&](int n) -> int64_t {
    const int32_t v = __builtin_amdgcn_readlane(my_pid, n);
    return v < 0 ? 0 : v;
  };
  auto ntok_at = [&](int n) -> int {
    if (__builtin_amdgcn_readlane(my_pid, n) < 0) return 0;
    return min(kT, L - (p_first + kWaves * n) * kT);
  };

  // One buffer slot per wave: page n is rebuilt into bf16 pairs first, which frees the slot
  // for page n + 1's planes and spill loads; those stay in flight while page n's MFMA,
  // softmax and p.V run.  Row metadata travels two pages ahead.  The last page is peeled so
  // that the loop's loads are unconditional (no buffer copies between iterations).
  auto compute = [&](const int n, const uint32_t (&kp)[16], const uint32_t (&vp)[16]) {
    const int ntok = ntok_at(n);
    const bool valid = t < ntok;

    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 kb = __builtin_bit_cast(bf16x8, (u32x4){kp[4 * c], kp[4 * c + 1], kp[4 * c + 2], kp[4 * c + 3]});
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[c], kb, sc, 0, 0, 0);
    }
    bool big = false;
#pragma unroll
    for (int i = 0; i < kG; ++i) big |= valid && fabsf(sc[i]) > kBigScore;
    double sd[kG];
    if (__any(big)) {
      double part[kG] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const double klo = (double)__uint_as_float(kp[k] << 16);
        const double khi = (double)__uint_as_float(kp[k] & 0xFFFF0000u);
#pragma unroll
        for (int i = 0; i < kG; ++i) {
          const double2 qq = s_q64[i][qd][k];
          part[i] = fma(qq.x, klo, part[i]);
          part[i] = fma(qq.y, khi, part[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < kG; ++i) {
        part[i] += __shfl_xor(part[i], 16, 64);
        part[i] += __shfl_xor(part[i], 32, 64);
        sd[i] = valid ? part[i] : -INFINITY;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kG; ++i) sd[i] = valid ? (double)sc[i] : -INFINITY;
    }

    bool raise = false;
#pragma unroll
    for (int i = 0; i < kG; ++i) raise |= sd[i] > m[i];
    if (__any(raise)) {
#pragma unroll
      for (int i = 0; i < kG; ++i) {
        const double mn = fmax(m[i], row_max16(sd[i]));
        const float alpha = exp2f((float)((m[i] - mn) * c2));
        m[i] = mn;
        l[i] *= alpha;
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] *= alpha;
      }
    }
    float pw[kG];
#pragma unroll
    for (int i = 0; i < kG; ++i) {
      pw[i] = exp2f((float)((sd[i] - m[i]) * c2));
      l[i] += pw[i];
    }
    // p.V: V lane (tv, g) needs the weights of token 8 * ps + tv (held by lane 8 * ps + tv)
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const bool vvalid = 8 * ps + tv < ntok;
      float pv[kG];
#pragma unroll
      for (int i = 0; i < kG; ++i) pv[i] = __shfl(pw[i], 8 * ps + tv, 64);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t x = vvalid ? vp[8 * ps + k] : 0u;
        const float lo = __uint_as_float(x << 16), hi = __uint_as_float(x & 0xFFFF0000u);
#pragma unroll
        for (int i = 0; i < kG; ++i) {
          acc[i][2 * k] = fmaf(pv[i], lo, acc[i][2 * k]);
          acc[i][2 * k + 1] = fmaf(pv[i], hi, acc[i][2 * k + 1]);
        }
      }
    }
  };

  typename Loader::Meta meta_n1{};
  typename Loader::Bufs buf{};
  if (nmine > 0) {
    const typename Loader::Meta meta0 = ld.issue_meta(pid_at(0), lane);
    meta_n1 = ld.issue_meta(pid_at(min(1, nmine - 1)), lane);
    buf = ld.issue_bufs(a.H, pid_at(0), h, lane, meta0);
  }
  for (int n = 0; n + 1 < nmine; ++n) {
    uint32_t kp[16], vp[16];
    ld.rebuild(buf, kp, vp);
    buf = ld.issue_bufs(a.H, pid_at(n + 1), h, lane, meta_n1);
    meta_n1 = ld.issue_meta(pid_at(min(n + 2, nmine - 1)), lane);
    compute(n, kp, vp);
  }
  if (nmine > 0) {
    uint32_t kp[16], vp[16];
    ld.rebuild(buf, kp, vp);
    compute(nmine - 1, kp, vp);
  }
  if (err) set_status(a.status, err);

  // ---- reduce over the 8 token lanes of each g: reduce-scatter, lane tv keeps [8tv, 8tv + 8)
  float* flat = &acc[0][0];
#pragma unroll
  for (int step = 0; step < 3; ++step) {
    const int half = 32 >> step, mask = 4 >> step;
    const bool up = (tv & mask) != 0;
#pragma unroll
    for (int k = 0; k < half; ++k) {
      const float send = up ? flat[k] : flat[k + half];
      const float keep = up ? flat[k + half] : flat[k];
      flat[k] = keep + __shfl_xor(send, mask, 8);
    }
  }
  // flat[0..7] of lane (tv, g) = head tv / 2, V slots 8 * (tv % 2) + k
  __shared__ float s_acc[kWaves][kG][kD];
  __shared__ double s_m[kWaves][kG];
  __shared__ float s_l[kWaves][kG];
  {
    const int i = tv >> 1;
#pragma unroll
    for (int k = 0; k < 8; ++k) s_acc[wave][i][vslot_dim(g, 8 * (tv & 1) + k)] = flat[k];
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

  // ---- merge the 4 waves, write this split's partial: acc[kG][kD] f32, l[kG] f32, m[kG] f64
  const int64_t unit = (int64_t)b * a.H + h;
  float* part = a.part + (unit * a.nsplit_max + s) * kPartFloats;
  for (int e = tid; e < kG * kD; e += kThreads) {
    const int i = e / kD, d = e % kD;
    double mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmax(mm, s_m[w][i]);
    float sum = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = s_m[w][i] == -INFINITY ? 0.f : exp2f((float)((s_m[w][i] - mm) * c2));
      sum = fmaf(f, s_acc[w][i][d], sum);
      lsum = fmaf(f, s_l[w][i], lsum);
    }
    part[i * kD + d] = sum;
    if (d == 0) {
      part[kG * kD + i] = lsum;
      reinterpret_cast<double*>(part + kG * kD + kG)[i] = mm;
    }
  }

}



// Merges the split partials of one (sequence, kv head) in split order (a kernel of its own:
// the launch boundary makes every split's partial visible without device-wide fences).
// Each split's (m, l) pairs are staged in LDS in one parallel step, the per-split weights are
// formed once, and every thread then reads its accumulator column with independent loads.
constexpr int kMaxSplitsStaged = 256;

__global__ __launch_bounds__(kThreads) void combine_k(AttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int32_t L = a.lens[b];
  const int32_t cap = min(a.maxp * kT, a.max_seq_len);
  L = L < 0 ? 0 : min(L, cap);
  const int npages = (L + kT - 1) / kT;
  const int nsplit = max(1, (npages + a.pps - 1) / a.pps);
  const int64_t unit = (int64_t)b * a.H + h;
  const float* base = a.part + unit * a.nsplit_max * kPartFloats;
  const double c2 = a.scale_log2e;
  __shared__ double s_m[kMaxSplitsStaged][kG];
  __shared__ float s_w[kMaxSplitsStaged][kG];
  __shared__ float s_lsum[kG];
  for (int e = tid; e < nsplit * kG; e += kThreads) {
    const int x = e / kG, i = e % kG;
    s_m[x][i] = reinterpret_cast<const double*>(base + x * kPartFloats + kG * kD + kG)[i];
    s_w[x][i] = base[x * kPartFloats + kG * kD + i];  // l, turned into weights below
  }
  __syncthreads();
  if (tid < kG) {
    const int i = tid;
    double mm = -INFINITY;
    for (int x = 0; x < nsplit; ++x) mm = fmax(mm, s_m[x][i]);
    float lsum = 0.f;
    for (int x = 0; x < nsplit; ++x) {
      const float f = s_m[x][i] == -INFINITY ? 0.f : exp2f((float)((s_m[x][i] - mm) * c2));
      lsum = fmaf(f, s_w[x][i], lsum);
      s_w[x][i] = f;
    }
    s_lsum[i] = lsum;
  }
  __syncthreads();
  for (int e = tid; e < kG * kD; e += kThreads) {
    const int i = e / kD, d = e % kD;
    float sum = 0.f;
#pragma unroll 8
    for (int x = 0; x < nsplit; ++x) sum = fmaf(s_w[x][i], base[x * kPartFloats + i * kD + d], sum);
    const float lsum = s_lsum[i];
    a.out[((int64_t)b * a.H * kG + h * kG + i) * kD + d] = lsum > 0.f ? sum / lsum : 0.f;
  }
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

// Pages per split: about 1024 workgroups (4 per CU on 256 CUs), at least 2 pages per
// wave, at most 64 per wave, and splits of one sequence as equal as the multiple of 4 allows.
static Plan make_plan(int32_t B, int32_t H, int32_t max_seq_len) {
  const int maxpages = std::max(1, (max_seq_len + kT - 1) / kT);
  int pps = env_pps();
  if (pps == 0) {
    const int64_t units = std::max<int64_t>((int64_t)B * H, 1);
    int64_t splits = std::max<int64_t>(1, (1024 + units - 1) / units);
    splits = std::min<int64_t>(splits, (maxpages + 7) / 8);
    splits = std::max<int64_t>(splits, 1);
    pps = (int)((maxpages + splits - 1) / splits);
  }
  pps = (pps + kWaves - 1) / kWaves * kWaves;
  pps = std::min(std::max(pps, 8), kMaxPagesPerSplit);
  if ((maxpages + pps - 1) / pps > kMaxSplitsStaged)  // very long sequences: fewer, longer splits
    pps = std::min(kMaxPagesPerSplit, ((maxpages + kMaxSplitsStaged - 1) / kMaxSplitsStaged + kWaves - 1) / kWaves * kWaves);
  return Plan{pps, (maxpages + pps - 1) / pps};
}

size_t attention_workspace_bytes(int32_t B, int32_t H, int32_t max_seq_len) {
  Plan pl = make_plan(B, H, max_seq_len);
  size_t part = (size_t)B * H * pl.nsplit_max * kPartFloats * sizeof(float);
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
  a.scale_log2e = (double)scale * kLog2e;
  a.out = out;
  size_t cnt = (size_t)q->batch * H * sizeof(uint32_t);
  a.counter = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + 256);
  a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + 256 + ((cnt + 255) / 256) * 256);
  a.status = status;
  dim3 grid(pl.nsplit_max, H, q->batch);
  hipLaunchKernelGGL(attn_k<Loader>, grid, dim3(kThreads), 0, st, a, ld);
  hipLaunchKernelGGL(combine_k, dim3(H, q->batch), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attention_packed(const zf_cache* c, const zf_seqs* q, const uint16_t* qv,
                                   float scale, float* out, void* ws, hipStream_t st) {
  // the spill address of a compressed block is never used, but it must be readable
  const uint8_t* spill = c->spill_slots > 0 ? c->spill : c->sm;
  PackedLoader ld{c->sm, c->nib, c->base, c->row_flags, c->row_spill, spill, c->spill_slots};
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
