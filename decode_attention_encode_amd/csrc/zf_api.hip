// zf_api.hip - the C ABI: argument checks, workspace sizing, kernel launches.
#include <math.h>
#include <string.h>

#include "zf_internal.h"

namespace zf {
hipError_t launch_encode(const Geom&, const zf_cache*, const zf_seqs*, const uint16_t*, uint32_t*,
                         hipStream_t);
size_t encode_workspace_bytes(const zf_seqs*);
int append_max_rows();
hipError_t launch_append(const Geom&, const zf_cache*, const zf_seqs*, int32_t, const uint16_t*,
                         const uint16_t*, hipStream_t);
hipError_t launch_decode(const Geom&, const zf_cache*, const zf_seqs*, uint16_t*, hipStream_t);
size_t compact_workspace_bytes(const zf_cache*, const zf_seqs*);
hipError_t launch_compact(const Geom&, const zf_cache*, const zf_seqs*, void*, size_t, hipStream_t);
hipError_t launch_attention_packed(const zf_cache*, const zf_seqs*, const uint16_t*, int32_t,
                                   float, float*, void*, hipStream_t);
hipError_t launch_attention_raw(const uint16_t*, int32_t, int32_t, const zf_seqs*,
                                const uint16_t*, int32_t, float, float*, void*, uint32_t*,
                                hipStream_t);
size_t attention_workspace_bytes(int32_t, int32_t, int32_t, int32_t);
hipError_t scratch_address(void**);
hipError_t launch_fill_zero(void*, size_t, hipStream_t);
void set_attention_timing(hipEvent_t, hipEvent_t);
}  // namespace zf

namespace {

constexpr int kMaxEncodeBatch = 8192;

bool aligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

// Geometry the format supports: whole 64-value blocks, at most 32 blocks per token row.
zf_status check_geom(int32_t P, int32_t T, int32_t H, int32_t D) {
  if (P <= 0 || T <= 0 || H <= 0 || D <= 0) return ZF_EINVAL;
  if (D % 64 != 0 || T > 64) return ZF_EUNSUPPORTED;
  if (2 * H * (D / 64) > 32) return ZF_EUNSUPPORTED;
  if ((int64_t)P * H * 2 * T * D > ((int64_t)1 << 40)) return ZF_EUNSUPPORTED;
  return ZF_OK;
}

zf_status check_cache(const zf_cache* c) {
  if (!c) return ZF_EINVAL;
  zf_status s = check_geom(c->num_pages, c->page_size, c->num_kv_heads, c->head_dim);
  if (s != ZF_OK) return s;
  if (!aligned(c->sm) || !aligned(c->nib) || !aligned(c->base) || !aligned(c->row_flags) ||
      !aligned(c->row_spill) || !c->spill_top || !c->status)
    return ZF_EINVAL;
  if (c->spill_slots > 0 && !aligned(c->spill)) return ZF_EINVAL;
  if (reinterpret_cast<uintptr_t>(c->append_sync) & 7u) return ZF_EINVAL;
  if (c->spill_slots >= ((uint64_t)1 << 32)) return ZF_EUNSUPPORTED;  // row_spill is 32-bit
  return ZF_OK;
}

zf_status check_seqs(const zf_seqs* q, int32_t T) {
  if (!q || q->batch < 0 || q->max_pages_per_seq < 0 || q->max_seq_len < 0) return ZF_EINVAL;
  if (q->batch == 0) return ZF_OK;
  if (q->max_pages_per_seq == 0 || !q->page_table || !q->seq_lens) return ZF_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q->page_table) & 3u) ||
      (reinterpret_cast<uintptr_t>(q->seq_lens) & 3u))
    return ZF_EINVAL;
  if ((int64_t)q->max_seq_len > (int64_t)q->max_pages_per_seq * T) return ZF_EINVAL;
  if ((int64_t)q->batch * q->max_pages_per_seq > ((int64_t)1 << 31)) return ZF_EUNSUPPORTED;
  return ZF_OK;
}

zf::Geom geom_of(const zf_cache* c) {
  return zf::Geom{c->num_pages, c->page_size, c->num_kv_heads, c->head_dim};
}

zf_status hip_status(hipError_t e) { return e == hipSuccess ? ZF_OK : ZF_EHIP; }

// The attention kernels are written for head_dim 128, 16-token pages and 4 or 8 query heads
// per kv head.
zf_status check_attention_shape(int32_t T, int32_t H, int32_t D, int32_t Hq) {
  if (Hq <= 0) return ZF_EINVAL;
  if (D != 128 || T != 16 || (Hq != 4 * H && Hq != 8 * H)) return ZF_EUNSUPPORTED;
  return ZF_OK;
}

// Longest sequence the split plan covers: 256 splits of at most 256 pages of 16 tokens.
constexpr int32_t kMaxAttentionLen = 256 * 256 * 16;
constexpr uint64_t kMaxAttentionSpillSlots = ((uint64_t)1 << 32) / 32 - 1;  // 32-bit byte offsets

}  // namespace

extern "C" {

size_t zf_cache_bytes(int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
                      int32_t head_dim) {
  if (check_geom(num_pages, page_size, num_kv_heads, head_dim) != ZF_OK) return 0;
  size_t vals = (size_t)num_pages * num_kv_heads * 2 * page_size * head_dim;
  return vals + vals / 2 + vals / 64 + 2 * (size_t)num_pages * page_size * sizeof(uint32_t);
}

size_t zf_encode_workspace_bytes(const zf_seqs* seqs) {
  if (!seqs || seqs->batch < 0 || seqs->max_pages_per_seq < 0) return 0;
  return zf::encode_workspace_bytes(seqs);
}

zf_status zf_encode_kv(const zf_cache* cache, const zf_seqs* seqs, const uint16_t* raw_pages,
                       void* workspace, size_t workspace_bytes, zf_stream_t stream) {
  zf_status s = check_cache(cache);
  if (s != ZF_OK) return s;
  if ((s = check_seqs(seqs, cache->page_size)) != ZF_OK) return s;
  if (seqs->batch == 0) return ZF_OK;
  if (seqs->batch > kMaxEncodeBatch) return ZF_EUNSUPPORTED;
  if (!aligned(raw_pages)) return ZF_EINVAL;
  if (!aligned(workspace) || workspace_bytes < zf::encode_workspace_bytes(seqs)) return ZF_EWORKSPACE;
  return hip_status(zf::launch_encode(geom_of(cache), cache, seqs, raw_pages,
                                      static_cast<uint32_t*>(workspace),
                                      static_cast<hipStream_t>(stream)));
}

zf_status zf_append_kv_n(const zf_cache* cache, const zf_seqs* seqs, int32_t n_new,
                         const uint16_t* k_new, const uint16_t* v_new, zf_stream_t stream) {
  zf_status s = check_cache(cache);
  if (s != ZF_OK) return s;
  if ((s = check_seqs(seqs, cache->page_size)) != ZF_OK) return s;
  if (n_new < 0) return ZF_EINVAL;
  if (seqs->batch == 0 || n_new == 0) return ZF_OK;
  if ((int64_t)seqs->batch * n_new > zf::append_max_rows()) return ZF_EUNSUPPORTED;
  if (!k_new || !v_new || (reinterpret_cast<uintptr_t>(k_new) & 15u) ||
      (reinterpret_cast<uintptr_t>(v_new) & 15u))
    return ZF_EINVAL;
  return hip_status(zf::launch_append(geom_of(cache), cache, seqs, n_new, k_new, v_new,
                                      static_cast<hipStream_t>(stream)));
}


zf_status zf_append_kv(const zf_cache* cache, const zf_seqs* seqs, const uint16_t* k_new,
                       const uint16_t* v_new, zf_stream_t stream) {
  return zf_append_kv_n(cache, seqs, 1, k_new, v_new, stream);
}

size_t zf_compact_workspace_bytes(const zf_cache* cache, const zf_seqs* seqs) {
  if (check_cache(cache) != ZF_OK || check_seqs(seqs, cache->page_size) != ZF_OK) return 0;
  return zf::compact_workspace_bytes(cache, seqs);
}

zf_status zf_compact_spill(const zf_cache* cache, const zf_seqs* seqs, void* workspace,
                           size_t workspace_bytes, zf_stream_t stream) {
  zf_status s = check_cache(cache);
  if (s != ZF_OK) return s;
  if ((s = check_seqs(seqs, cache->page_size)) != ZF_OK) return s;
  if (seqs->batch > kMaxEncodeBatch) return ZF_EUNSUPPORTED;
  // the header and the page counts at least; the staging area behind them may be smaller
  // than the pool (the device then checks that it holds the live slots)
  zf_cache head_only = *cache;
  head_only.spill_slots = 0;
  if (!aligned(workspace) || workspace_bytes < zf::compact_workspace_bytes(&head_only, seqs))
    return ZF_EWORKSPACE;
  return hip_status(zf::launch_compact(geom_of(cache), cache, seqs, workspace, workspace_bytes,
                                       static_cast<hipStream_t>(stream)));
}

int64_t zf_max_sequences(int64_t kv_budget_bytes, int32_t layers, int32_t context,
                         int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                         double raw_blocks_per_row) {
  if (kv_budget_bytes <= 0 || layers <= 0 || context <= 0) return 0;
  if (check_geom(1, page_size, num_kv_heads, head_dim) != ZF_OK) return -1;
  const int64_t pages = ((int64_t)context + page_size - 1) / page_size;
  const int64_t values = (int64_t)num_kv_heads * 2 * head_dim;  // per token row
  int64_t page_bytes, spill_bytes = 0;
  if (raw_blocks_per_row < 0) {
    page_bytes = (int64_t)page_size * values * 2;
  } else {
    const int64_t blocks = values / 64;
    if (raw_blocks_per_row > (double)blocks) return -1;
    page_bytes = (int64_t)zf_cache_bytes(1, page_size, num_kv_heads, head_dim);
    spill_bytes = 32 * (int64_t)ceil(raw_blocks_per_row * (double)context);
  }
  const int64_t per_seq = ((int64_t)pages * page_bytes + spill_bytes) * layers;
  return kv_budget_bytes / per_seq;
}

zf_status zf_decode_kv(const zf_cache* cache, const zf_seqs* seqs, uint16_t* raw_pages_out,
                       zf_stream_t stream) {
  zf_status s = check_cache(cache);
  if (s != ZF_OK) return s;
  if ((s = check_seqs(seqs, cache->page_size)) != ZF_OK) return s;
  if (seqs->batch == 0) return ZF_OK;
  if (!aligned(raw_pages_out)) return ZF_EINVAL;
  return hip_status(zf::launch_decode(geom_of(cache), cache, seqs, raw_pages_out,
                                      static_cast<hipStream_t>(stream)));
}

size_t zf_attention_workspace_bytes(int32_t batch, int32_t num_kv_heads, int32_t num_q_heads,
                                    int32_t head_dim, int32_t max_seq_len) {
  if (batch < 0 || num_kv_heads <= 0 || max_seq_len < 0 || max_seq_len > kMaxAttentionLen) return 0;
  if (check_attention_shape(16, num_kv_heads, head_dim, num_q_heads) != ZF_OK) return 0;
  return zf::attention_workspace_bytes(batch, num_kv_heads, num_q_heads / num_kv_heads, max_seq_len);
}

zf_status zf_attention_workspace_init(void* workspace, size_t workspace_bytes,
                                      zf_stream_t stream) {
  if (!aligned(workspace)) return ZF_EINVAL;
  return hip_status(zf::launch_fill_zero(workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

static zf_status check_attention_io(const zf_seqs* seqs, int32_t num_kv_heads, int32_t head_dim,
                                    const uint16_t* q, int32_t num_q_heads, float* out,
                                    void* workspace, size_t workspace_bytes) {
  if (!aligned(q) || !aligned(out)) return ZF_EINVAL;
  if (seqs->max_seq_len > kMaxAttentionLen) return ZF_EUNSUPPORTED;
  if (!aligned(workspace) ||
      workspace_bytes < zf::attention_workspace_bytes(seqs->batch, num_kv_heads,
                                                      num_q_heads / num_kv_heads, seqs->max_seq_len))
    return ZF_EWORKSPACE;
  (void)head_dim;
  return ZF_OK;
}

zf_status zf_decode_attention(const zf_cache* cache, const zf_seqs* seqs, const uint16_t* q,
                              int32_t num_q_heads, float scale, float* out, void* workspace,
                              size_t workspace_bytes, zf_stream_t stream) {
  zf_status s = check_cache(cache);
  if (s != ZF_OK) return s;
  if ((s = check_seqs(seqs, cache->page_size)) != ZF_OK) return s;
  if ((s = check_attention_shape(cache->page_size, cache->num_kv_heads, cache->head_dim,
                                 num_q_heads)) != ZF_OK)
    return s;
  // the kernel addresses the spill pool with 32-bit byte offsets
  if (cache->spill_slots > kMaxAttentionSpillSlots) return ZF_EUNSUPPORTED;
  if (seqs->batch == 0) return ZF_OK;
  if ((s = check_attention_io(seqs, cache->num_kv_heads, cache->head_dim, q, num_q_heads, out,
                              workspace, workspace_bytes)) != ZF_OK)
    return s;
  return hip_status(zf::launch_attention_packed(cache, seqs, q, num_q_heads, scale, out, workspace,
                                                static_cast<hipStream_t>(stream)));
}

zf_status zf_decode_attention_noalloc(const zf_cache* cache, const zf_seqs* seqs, const uint16_t* q,
                                      int32_t num_q_heads, float scale, float* out,
                                      zf_stream_t stream) {
  zf_status s = check_cache(cache);
  if (s != ZF_OK) return s;
  if ((s = check_seqs(seqs, cache->page_size)) != ZF_OK) return s;
  if ((s = check_attention_shape(cache->page_size, cache->num_kv_heads, cache->head_dim,
                                 num_q_heads)) != ZF_OK)
    return s;
  if (cache->spill_slots > kMaxAttentionSpillSlots) return ZF_EUNSUPPORTED;
  if (seqs->batch == 0) return ZF_OK;
  if (!aligned(q) || !aligned(out)) return ZF_EINVAL;
  if (seqs->max_seq_len > kMaxAttentionLen) return ZF_EUNSUPPORTED;
  const size_t need = zf::attention_workspace_bytes(seqs->batch, cache->num_kv_heads,
                                                    num_q_heads / cache->num_kv_heads,
                                                    seqs->max_seq_len);
  if (need > ZF_NOALLOC_SCRATCH_BYTES) return ZF_ESCRATCH;
  void* ws = nullptr;
  if (zf::scratch_address(&ws) != hipSuccess) return ZF_EHIP;
  return hip_status(zf::launch_attention_packed(cache, seqs, q, num_q_heads, scale, out, ws,
                                                static_cast<hipStream_t>(stream)));
}

zf_status zf_decode_attention_raw(const uint16_t* raw_pages, int32_t num_pages,
                                  int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                                  const zf_seqs* seqs, const uint16_t* q, int32_t num_q_heads,
                                  float scale, float* out, void* workspace,
                                  size_t workspace_bytes, uint32_t* status, zf_stream_t stream) {
  zf_status s = check_geom(num_pages, page_size, num_kv_heads, head_dim);
  if (s != ZF_OK) return s;
  if (!aligned(raw_pages) || !status) return ZF_EINVAL;
  if ((s = check_seqs(seqs, page_size)) != ZF_OK) return s;
  if ((s = check_attention_shape(page_size, num_kv_heads, head_dim, num_q_heads)) != ZF_OK) return s;
  if (seqs->batch == 0) return ZF_OK;
  if ((s = check_attention_io(seqs, num_kv_heads, head_dim, q, num_q_heads, out, workspace,
                              workspace_bytes)) != ZF_OK)
    return s;
  return hip_status(zf::launch_attention_raw(raw_pages, num_pages, num_kv_heads, seqs, q, num_q_heads, scale,
                                             out, workspace, status,
                                             static_cast<hipStream_t>(stream)));
}

zf_status zf_time_next_attention(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return ZF_EINVAL;
  zf::set_attention_timing(static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
  return ZF_OK;
}

zf_status zf_get_status(const uint32_t* status, uint32_t* host_status, zf_stream_t stream) {
  if (!status || !host_status) return ZF_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(host_status, status, sizeof(uint32_t), hipMemcpyDeviceToHost, st) != hipSuccess)
    return ZF_EHIP;
  return hip_status(hipStreamSynchronize(st));
}

const char* zf_status_str(zf_status s) {
  switch (s) {
    case ZF_OK: return "ok";
    case ZF_EINVAL: return "invalid argument";
    case ZF_EUNSUPPORTED: return "unsupported shape";
    case ZF_EHIP: return "HIP runtime error";
    case ZF_EWORKSPACE: return "workspace missing or too small";
    case ZF_ESCRATCH: return "the call needs more than the fixed scratch area (ZF_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

}  // extern "C"
