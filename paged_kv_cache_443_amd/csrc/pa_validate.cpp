// Host-side argument validation for the C ABI (no HIP calls).
//
// Checks run in a fixed order and the first failure is returned:
// cache descriptor, sizes, the no-op case, pointers, dtypes, alignment.
#include "pa_validate.h"

#include <cmath>
#include <cstdint>
#include <cstring>

namespace pa {
namespace {

// Dtype fields and arguments arrive from C callers as plain ints.  In C++
// reading an enum object that holds a value outside its enumerators is
// undefined, so validation reads them through their bytes.
static_assert(sizeof(pa_dtype) == sizeof(int32_t), "pa_dtype is passed as a 32-bit int");
int32_t raw(const pa_dtype &d) {
  int32_t v;
  std::memcpy(&v, &d, sizeof v);
  return v;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool supported_block_size(int32_t bs) { return bs == 16 || bs == 32 || bs == 64; }
bool supported_head_dim(int32_t d) { return d == 64 || d == 128; }

}  // namespace

pa_status check_cache(const pa_kv_cache *c) {
  if (c == nullptr || c->k_cache == nullptr || c->v_cache == nullptr) return PA_ERR_NULL_PTR;
  if (raw(c->kv_dtype) < PA_F32 || raw(c->kv_dtype) > PA_I4) return PA_ERR_UNSUPPORTED;
  const bool want_scales = c->kv_dtype == PA_I8 || c->kv_dtype == PA_I4;
  if (want_scales && (c->k_scale == nullptr || c->v_scale == nullptr)) return PA_ERR_NULL_PTR;
  if (!want_scales && (c->k_scale != nullptr || c->v_scale != nullptr)) return PA_ERR_NULL_PTR;
  if (c->num_blocks < 1 || c->num_kv_heads < 1 || c->block_size < 1 || c->head_dim < 1) return PA_ERR_BAD_SHAPE;
  if (!supported_block_size(c->block_size) || !supported_head_dim(c->head_dim)) return PA_ERR_UNSUPPORTED;
  // block * kv-head tile indices are formed in 32 bits on the device
  if (static_cast<int64_t>(c->num_blocks) * c->num_kv_heads > INT32_MAX) return PA_ERR_BAD_SHAPE;
  if (!aligned(c->k_cache, 16) || !aligned(c->v_cache, 16)) return PA_ERR_MISALIGNED;
  if (want_scales && (!aligned(c->k_scale, 16) || !aligned(c->v_scale, 16))) return PA_ERR_MISALIGNED;
  return PA_OK;
}

pa_status check_append(const void *key, const void *value, pa_dtype src_dtype, const int32_t *slot_mapping,
                       int32_t num_tokens, const pa_kv_cache *cache) {
  pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_ERR_BAD_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (key == nullptr || value == nullptr || slot_mapping == nullptr) return PA_ERR_NULL_PTR;
  const int32_t want = cache->kv_dtype == PA_F32 ? PA_F32 : PA_BF16;
  if (raw(src_dtype) != want) return PA_ERR_UNSUPPORTED;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(slot_mapping, 4)) return PA_ERR_MISALIGNED;
  return PA_OK;
}

pa_status check_decode_common(const void *q, pa_dtype q_dtype, int32_t num_seqs, int32_t num_heads,
                              const pa_kv_cache *cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                              const int32_t *context_lens, float scale) {
  pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_heads < 1 || max_blocks_per_seq < 1) return PA_ERR_BAD_SHAPE;
  if (num_heads % cache->num_kv_heads != 0) return PA_ERR_BAD_SHAPE;
  if (!std::isfinite(scale)) return PA_ERR_BAD_SHAPE;
  if (static_cast<int64_t>(max_blocks_per_seq) * cache->block_size > INT32_MAX) return PA_ERR_BAD_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (q == nullptr || block_tables == nullptr || context_lens == nullptr) return PA_ERR_NULL_PTR;
  if (raw(q_dtype) != PA_F32 && raw(q_dtype) != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(block_tables, 4) || !aligned(context_lens, 4)) return PA_ERR_MISALIGNED;
  return PA_OK;
}

pa_status check_out(const void *out, pa_dtype q_dtype, pa_dtype kv_dtype, pa_dtype out_dtype) {
  if (out == nullptr) return PA_ERR_NULL_PTR;
  const int32_t qd = raw(q_dtype), kd = raw(kv_dtype), od = raw(out_dtype);
  const bool ok = (qd == PA_F32 && kd == PA_F32 && od == PA_F32) ||
                  (qd == PA_BF16 && (kd == PA_BF16 || kd == PA_I8 || kd == PA_I4) && (od == PA_BF16 || od == PA_F32));
  if (!ok) return PA_ERR_UNSUPPORTED;
  if (!aligned(out, 16)) return PA_ERR_MISALIGNED;
  return PA_OK;
}

pa_status check_split(int32_t partition_size, int32_t max_num_partitions, int32_t block_size,
                      int32_t max_blocks_per_seq, const float *part_out, const float *part_lse) {
  if (partition_size < 1 || partition_size % block_size != 0 || max_num_partitions < 1) return PA_ERR_BAD_SHAPE;
  const int64_t max_len = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  const int64_t need = (max_len + partition_size - 1) / partition_size;
  if (max_num_partitions < need) return PA_ERR_BAD_WORKSPACE;
  if (part_out == nullptr || part_lse == nullptr) return PA_ERR_NULL_PTR;
  if (!aligned(part_out, 16) || !aligned(part_lse, 4)) return PA_ERR_MISALIGNED;
  return PA_OK;
}

pa_status check_multi(const int32_t *q_start, int32_t num_queries, int32_t max_q_len, int32_t num_seqs,
                      int32_t num_heads, const pa_kv_cache *cache) {
  if (num_queries < 0 || max_q_len < 1) return PA_ERR_BAD_SHAPE;
  // every sequence's query rows fit max_q_len, so the rows of all fit the bound
  if (static_cast<int64_t>(num_queries) > static_cast<int64_t>(num_seqs) * max_q_len) return PA_ERR_BAD_SHAPE;
  // rows (query token x head) of one kv head, and rows of q, in 32 bits
  const int64_t group = num_heads / cache->num_kv_heads;
  if (static_cast<int64_t>(max_q_len) * group + 15 > INT32_MAX) return PA_ERR_BAD_SHAPE;
  if (static_cast<int64_t>(num_queries) * num_heads > INT32_MAX) return PA_ERR_BAD_SHAPE;
  if (num_seqs == 0 || num_queries == 0) return PA_OK;
  if (q_start == nullptr) return PA_ERR_NULL_PTR;
  if (!aligned(q_start, 4)) return PA_ERR_MISALIGNED;
  return PA_OK;
}

pa_status check_reduce(const float *part_out, const float *part_lse, int32_t num_seqs, int32_t num_heads,
                       int32_t head_dim, int32_t max_num_partitions, const int32_t *context_lens,
                       int32_t partition_size, const void *out, pa_dtype out_dtype) {
  if (num_seqs < 0 || num_heads < 1 || head_dim < 1 || max_num_partitions < 1 || partition_size < 1)
    return PA_ERR_BAD_SHAPE;
  if (!supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (part_out == nullptr || part_lse == nullptr || context_lens == nullptr || out == nullptr)
    return PA_ERR_NULL_PTR;
  if (raw(out_dtype) != PA_F32 && raw(out_dtype) != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (!aligned(part_out, 16) || !aligned(part_lse, 4) || !aligned(context_lens, 4) || !aligned(out, 16))
    return PA_ERR_MISALIGNED;
  return PA_OK;
}

pa_status check_copy(const pa_kv_cache *cache, const int32_t *block_pairs, int32_t num_pairs) {
  pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return PA_ERR_BAD_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (block_pairs == nullptr) return PA_ERR_NULL_PTR;
  if (!aligned(block_pairs, 4)) return PA_ERR_MISALIGNED;
  return PA_OK;
}

pa_status check_swap(const pa_kv_cache *src, const pa_kv_cache *dst, const int32_t *block_pairs, int32_t num_pairs) {
  pa_status st = check_cache(src);
  if (st != PA_OK) return st;
  st = check_cache(dst);
  if (st != PA_OK) return st;
  if (src->kv_dtype != dst->kv_dtype || src->num_kv_heads != dst->num_kv_heads ||
      src->block_size != dst->block_size || src->head_dim != dst->head_dim)
    return PA_ERR_BAD_SHAPE;
  if (num_pairs < 0) return PA_ERR_BAD_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (block_pairs == nullptr) return PA_ERR_NULL_PTR;
  if (!aligned(block_pairs, 4)) return PA_ERR_MISALIGNED;
  return PA_OK;
}

pa_status check_probe(const void *buf, size_t bytes, int32_t mode, int32_t tile_bytes, const uint32_t *sink) {
  if (buf == nullptr || sink == nullptr) return PA_ERR_NULL_PTR;
  if (mode < 0 || mode > 3) return PA_ERR_UNSUPPORTED;
  if (bytes < 16 || bytes % 16 != 0) return PA_ERR_BAD_SHAPE;
  if (mode >= 2 && (tile_bytes < 16 || tile_bytes % 16 != 0 || static_cast<size_t>(tile_bytes) > bytes))
    return PA_ERR_BAD_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return PA_ERR_MISALIGNED;
  return PA_OK;
}

pa_status check_latent_cache(const pa_latent_cache *c) {
  if (c == nullptr || c->latent == nullptr) return PA_ERR_NULL_PTR;
  if (c->num_blocks < 1 || c->block_size < 1 || c->latent_dim < 1) return PA_ERR_BAD_SHAPE;
  if (!supported_block_size(c->block_size) || c->latent_dim != 512) return PA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(c->num_blocks) * c->block_size > INT32_MAX) return PA_ERR_BAD_SHAPE;  // int32 slots
  if (!aligned(c->latent, 16)) return PA_ERR_MISALIGNED;
  return PA_OK;
}

pa_status check_mla_append(const void *rows, const int32_t *slot_mapping, int32_t num_tokens,
                           const pa_latent_cache *cache) {
  pa_status st = check_latent_cache(cache);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_ERR_BAD_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (rows == nullptr || slot_mapping == nullptr) return PA_ERR_NULL_PTR;
  if (!aligned(rows, 16) || !aligned(slot_mapping, 4)) return PA_ERR_MISALIGNED;
  return PA_OK;
}

MlaWorkspace mla_workspace(int32_t num_seqs, int32_t num_heads, int32_t latent_dim, int32_t max_blocks_per_seq,
                           int32_t block_size, int32_t partition_size) {
  MlaWorkspace w{0, 0, 0, 0};
  if (num_seqs < 0 || num_heads < 1 || latent_dim < 1 || max_blocks_per_seq < 1 || block_size < 1 ||
      partition_size < 1)
    return w;
  const int64_t max_len = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  const int64_t pmax = (max_len + partition_size - 1) / partition_size;
  if (pmax > INT32_MAX) return w;
  const size_t rows = static_cast<size_t>(num_seqs) * num_heads;
  const size_t qlat = rows * latent_dim * sizeof(float);
  w.part_out_off = (qlat + 255) / 256 * 256;
  const size_t po = rows * static_cast<size_t>(pmax) * latent_dim * sizeof(float);
  w.part_lse_off = (w.part_out_off + po + 255) / 256 * 256;
  w.total = w.part_lse_off + rows * static_cast<size_t>(pmax) * sizeof(float);
  w.max_num_partitions = static_cast<int32_t>(pmax);
  return w;
}

pa_status check_mla_decode(const void *q, int32_t num_seqs, int32_t num_heads, int32_t head_dim, const void *w_uk,
                           const void *w_uv, const pa_latent_cache *cache, const int32_t *block_tables,
                           int32_t max_blocks_per_seq, const int32_t *context_lens, float scale,
                           int32_t partition_size, const void *workspace, size_t workspace_bytes, const void *out,
                           pa_dtype out_dtype) {
  pa_status st = check_latent_cache(cache);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_heads < 1 || head_dim < 1 || max_blocks_per_seq < 1) return PA_ERR_BAD_SHAPE;
  if (num_seqs > 4096) return PA_ERR_BAD_SHAPE;  // the persistent pass indexes its pieces in LDS
  if (!supported_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return PA_ERR_BAD_SHAPE;
  if (static_cast<int64_t>(max_blocks_per_seq) * cache->block_size > INT32_MAX) return PA_ERR_BAD_SHAPE;
  if (static_cast<int64_t>(num_heads) * head_dim > INT32_MAX / 512) return PA_ERR_BAD_SHAPE;
  if (partition_size < 64 || partition_size % 64 != 0 || partition_size % cache->block_size != 0 ||
      partition_size > 4096)
    return PA_ERR_BAD_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (q == nullptr || w_uk == nullptr || w_uv == nullptr || block_tables == nullptr || context_lens == nullptr ||
      workspace == nullptr || out == nullptr)
    return PA_ERR_NULL_PTR;
  if (raw(out_dtype) != PA_F32 && raw(out_dtype) != PA_BF16) return PA_ERR_UNSUPPORTED;
  const MlaWorkspace ws = mla_workspace(num_seqs, num_heads, cache->latent_dim, max_blocks_per_seq,
                                        cache->block_size, partition_size);
  if (ws.total == 0) return PA_ERR_BAD_SHAPE;
  if (workspace_bytes < ws.total) return PA_ERR_BAD_WORKSPACE;
  if (!aligned(q, 16) || !aligned(w_uk, 16) || !aligned(w_uv, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(workspace, 256))
    return PA_ERR_MISALIGNED;
  return PA_OK;
}

size_t split_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_num_partitions) {
  if (num_seqs < 0 || num_heads < 1 || head_dim < 1 || max_num_partitions < 1) return 0;
  const size_t rows = static_cast<size_t>(num_seqs) * num_heads * max_num_partitions;
  const size_t out_bytes = rows * head_dim * sizeof(float);
  const size_t lse_off = (out_bytes + 255) / 256 * 256;
  return lse_off + rows * sizeof(float);
}

}  // namespace pa
