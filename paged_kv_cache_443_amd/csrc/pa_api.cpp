// extern "C" entry points: validate, fill the kernel parameters, launch on
// the caller's stream.  No allocation, no synchronisation.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>

#include <hip/hip_runtime_api.h>

#include "pa.h"
#include "pa_internal.h"
#include "pa_probe.h"
#include "pa_validate.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

pa_status from_hip(hipError_t e) {
  g_last_hip_error = static_cast<int32_t>(e);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

constexpr float kLog2e = 1.4426950408889634f;

pa::DecodeParams make_decode_params(const void *q, int32_t num_seqs, int32_t num_heads, const pa_kv_cache *cache,
                                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                                    const int32_t *context_lens, float scale) {
  pa::DecodeParams p{};
  p.q = q;
  p.k_cache = cache->k_cache;
  p.v_cache = cache->v_cache;
  p.k_scale = static_cast<const uint16_t *>(cache->k_scale);
  p.v_scale = static_cast<const uint16_t *>(cache->v_scale);
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = cache->num_kv_heads;
  p.group = num_heads / cache->num_kv_heads;
  p.head_groups = (p.group + 15) / 16;
  p.rows_per_group = std::min(16, p.group);
  p.q_start = nullptr;
  p.num_queries = num_seqs;
  p.max_q_len = 1;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = cache->num_blocks;
  p.scale = scale;
  p.scale_log2 = scale * kLog2e;
  return p;
}

pa::AppendParams make_append_params(const void *key, const void *value, const int32_t *slot_mapping,
                                    int32_t num_tokens, const pa_kv_cache *cache) {
  pa::AppendParams p{};
  p.key = key;
  p.value = value;
  p.slot_mapping = slot_mapping;
  p.k_cache = cache->k_cache;
  p.v_cache = cache->v_cache;
  p.k_scale = static_cast<uint16_t *>(cache->k_scale);
  p.v_scale = static_cast<uint16_t *>(cache->v_scale);
  p.num_tokens = num_tokens;
  p.num_kv_heads = cache->num_kv_heads;
  p.block_size = cache->block_size;
  p.head_dim = cache->head_dim;
  p.num_blocks = cache->num_blocks;
  return p;
}

// Block-table entries a work-group stages at once: the whole range its unit
// can touch (the table row, or one partition), at most kMaxTableWindow.
constexpr int32_t kMaxTableWindow = 1024;

// PA_DECODE_VALU=1: single-token bf16 decodes run on the vector ALUs
// instead of the matrix cores (read at every call, so a process can time both).
bool valu_requested() {
  const char *v = std::getenv("PA_DECODE_VALU");
  return v != nullptr && v[0] == '1' && v[1] == '\0';
}

int32_t table_window(int32_t max_blocks_per_seq, int32_t partition_size, int32_t block_size) {
  int32_t w = max_blocks_per_seq;
  if (partition_size > 0) w = std::min(w, partition_size / block_size);
  w = std::min(std::max(w, 1), kMaxTableWindow);
  return (w + 3) / 4 * 4;
}

pa_status launch(pa::DecodeParams &p, const pa_kv_cache *cache, hipStream_t stream) {
  p.tbl_window = table_window(p.max_blocks_per_seq, p.partition_size, cache->block_size);
  // one work-group per (kv head, query-head group, sequence[, partition])
  const int64_t nparts = p.partition_size > 0 ? p.max_num_partitions : 1;
  const int64_t nwg = static_cast<int64_t>(p.num_kv_heads) * p.head_groups * p.num_seqs * nparts;
  if (nwg > INT32_MAX) return PA_ERR_BAD_SHAPE;
  hipError_t e;
  if (cache->kv_dtype == PA_F32)
    e = pa::launch_decode_f32(p, cache->head_dim, cache->block_size, stream);
  else if (valu_requested() && pa::decode_valu_applies(p, cache->kv_dtype, cache->head_dim))
    e = pa::launch_decode_valu(p, cache->head_dim, cache->block_size, stream);
  else
    e = pa::launch_decode_mfma(p, cache->kv_dtype, cache->head_dim, cache->block_size, stream);
  return from_hip(e);
}

pa_status launch_block_copies(const pa_kv_cache *src, const pa_kv_cache *dst, const int32_t *block_pairs,
                              int32_t num_pairs, hipStream_t stream) {
  if (static_cast<int64_t>(num_pairs) * src->num_kv_heads > INT32_MAX) return PA_ERR_BAD_SHAPE;
  static const int32_t kElemBits[] = {32, 16, 8, 4};  // PA_F32, PA_BF16, PA_I8, PA_I4
  pa::CopyParams p{};
  p.src_k = src->k_cache;
  p.src_v = src->v_cache;
  p.src_k_scale = src->k_scale;
  p.src_v_scale = src->v_scale;
  p.dst_k = dst->k_cache;
  p.dst_v = dst->v_cache;
  p.dst_k_scale = dst->k_scale;
  p.dst_v_scale = dst->v_scale;
  p.pairs = block_pairs;
  p.num_pairs = num_pairs;
  p.num_kv_heads = src->num_kv_heads;
  p.src_blocks = src->num_blocks;
  p.dst_blocks = dst->num_blocks;
  p.block_size = src->block_size;
  p.tile_bytes = static_cast<size_t>(src->block_size) * src->head_dim * kElemBits[src->kv_dtype] / 8;
  return from_hip(pa::launch_copy_blocks(p, stream));
}

}  // namespace

extern "C" {

pa_status pa_reshape_and_cache(const void *key, const void *value, pa_dtype src_dtype, const int32_t *slot_mapping,
                               int32_t num_tokens, const pa_kv_cache *cache, hipStream_t stream) {
  pa_status st = pa::check_append(key, value, src_dtype, slot_mapping, num_tokens, cache);
  if (st != PA_OK || num_tokens == 0) return st;
  if (static_cast<int64_t>(num_tokens) * cache->num_kv_heads > INT32_MAX) return PA_ERR_BAD_SHAPE;
  const pa::AppendParams p = make_append_params(key, value, slot_mapping, num_tokens, cache);
  return from_hip(pa::launch_append(p, cache->kv_dtype, stream));
}

pa_status pa_decode(const void *q, pa_dtype q_dtype, int32_t num_seqs, int32_t num_heads, const pa_kv_cache *cache,
                    const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens, float scale,
                    void *out, pa_dtype out_dtype, hipStream_t stream) {
  pa_status st = pa::check_decode_common(q, q_dtype, num_seqs, num_heads, cache, block_tables, max_blocks_per_seq,
                                         context_lens, scale);
  if (st != PA_OK || num_seqs == 0) return st;
  st = pa::check_out(out, q_dtype, cache->kv_dtype, out_dtype);
  if (st != PA_OK) return st;
  pa::DecodeParams p =
      make_decode_params(q, num_seqs, num_heads, cache, block_tables, max_blocks_per_seq, context_lens, scale);
  p.out = out;
  p.out_bf16 = out_dtype == PA_BF16;
  p.partition_size = 0;
  p.max_num_partitions = 1;
  return launch(p, cache, stream);
}

pa_status pa_decode_split(const void *q, pa_dtype q_dtype, int32_t num_seqs, int32_t num_heads,
                          const pa_kv_cache *cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                          const int32_t *context_lens, float scale, int32_t partition_size,
                          int32_t max_num_partitions, float *part_out, float *part_lse, hipStream_t stream) {
  pa_status st = pa::check_decode_common(q, q_dtype, num_seqs, num_heads, cache, block_tables, max_blocks_per_seq,
                                         context_lens, scale);
  if (st != PA_OK) return st;
  st = pa::check_split(partition_size, max_num_partitions, cache->block_size, max_blocks_per_seq, part_out, part_lse);
  if (st != PA_OK || num_seqs == 0) return st;
  // partials are fp32; the dtype combination is that of an fp32-output decode
  st = pa::check_out(part_out, q_dtype, cache->kv_dtype, PA_F32);
  if (st != PA_OK) return st;
  pa::DecodeParams p =
      make_decode_params(q, num_seqs, num_heads, cache, block_tables, max_blocks_per_seq, context_lens, scale);
  p.part_out = part_out;
  p.part_lse = part_lse;
  p.partition_size = partition_size;
  p.max_num_partitions = max_num_partitions;
  return launch(p, cache, stream);
}

pa_status pa_append_decode(const void *key, const void *value, pa_dtype src_dtype, const int32_t *slot_mapping,
                           const void *q, pa_dtype q_dtype, int32_t num_seqs, int32_t num_heads,
                           const pa_kv_cache *cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                           const int32_t *context_lens, float scale, void *out, pa_dtype out_dtype,
                           hipStream_t stream) {
  pa_status st = pa::check_append(key, value, src_dtype, slot_mapping, num_seqs, cache);
  if (st != PA_OK) return st;
  st = pa::check_decode_common(q, q_dtype, num_seqs, num_heads, cache, block_tables, max_blocks_per_seq,
                               context_lens, scale);
  if (st != PA_OK || num_seqs == 0) return st;
  st = pa::check_out(out, q_dtype, cache->kv_dtype, out_dtype);
  if (st != PA_OK) return st;
  if (static_cast<int64_t>(num_seqs) * cache->num_kv_heads > INT32_MAX) return PA_ERR_BAD_SHAPE;
  const int32_t group = num_heads / cache->num_kv_heads;
  // One kernel when every kv head has one work-group (at most 16 query heads
  // per kv head) and the cache is bf16, int8 or int4: the units take the new
  // row from the source (int8 / int4: quantised in the kernel exactly as the
  // append does) and append work-groups at the end of the grid write the
  // cache (measured against two launches: 70B-shaped workload 80.0 -> 72.9
  // us, LLaMA-13B-shaped 269.8 -> 261.4 us, int8 391.6 -> 379.9 us, int4
  // 237.7 -> 231.2 us).
  const bool fused = cache->kv_dtype != PA_F32 && group <= 16;
  if (!fused) {
    st = pa_reshape_and_cache(key, value, src_dtype, slot_mapping, num_seqs, cache, stream);
    if (st != PA_OK) return st;
    return pa_decode(q, q_dtype, num_seqs, num_heads, cache, block_tables, max_blocks_per_seq, context_lens, scale,
                     out, out_dtype, stream);
  }
  pa::DecodeParams p =
      make_decode_params(q, num_seqs, num_heads, cache, block_tables, max_blocks_per_seq, context_lens, scale);
  p.append = make_append_params(key, value, slot_mapping, num_seqs, cache);
  p.out = out;
  p.out_bf16 = out_dtype == PA_BF16;
  p.partition_size = 0;
  p.max_num_partitions = 1;
  return launch(p, cache, stream);
}

pa_status pa_append_decode_split(const void *key, const void *value, pa_dtype src_dtype, const int32_t *slot_mapping,
                                 const void *q, pa_dtype q_dtype, int32_t num_seqs, int32_t num_heads,
                                 const pa_kv_cache *cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                 const int32_t *context_lens, float scale, int32_t partition_size,
                                 int32_t max_num_partitions, float *part_out, float *part_lse, hipStream_t stream) {
  pa_status st = pa::check_append(key, value, src_dtype, slot_mapping, num_seqs, cache);
  if (st != PA_OK) return st;
  st = pa::check_decode_common(q, q_dtype, num_seqs, num_heads, cache, block_tables, max_blocks_per_seq,
                               context_lens, scale);
  if (st != PA_OK) return st;
  st = pa::check_split(partition_size, max_num_partitions, cache->block_size, max_blocks_per_seq, part_out, part_lse);
  if (st != PA_OK || num_seqs == 0) return st;
  st = pa::check_out(part_out, q_dtype, cache->kv_dtype, PA_F32);
  if (st != PA_OK) return st;
  if (static_cast<int64_t>(num_seqs) * cache->num_kv_heads > INT32_MAX) return PA_ERR_BAD_SHAPE;
  // One kernel for bf16 and int8 caches with at most 16 query heads per kv
  // head and a batch the persistent split pass indexes (pieces splice the
  // new row; the pass's work-groups write the rows after their last piece);
  // otherwise the two launches (int4: the fused pass needs 229 VGPRs, a
  // work-group per CU less than the plain one).
  const int32_t group = num_heads / cache->num_kv_heads;
  const bool fused = (cache->kv_dtype == PA_BF16 || cache->kv_dtype == PA_I8) && group <= 16 &&
                     num_seqs <= pa::kMaxFusedSplitSeqs;
  if (!fused) {
    st = pa_reshape_and_cache(key, value, src_dtype, slot_mapping, num_seqs, cache, stream);
    if (st != PA_OK) return st;
    return pa_decode_split(q, q_dtype, num_seqs, num_heads, cache, block_tables, max_blocks_per_seq, context_lens,
                           scale, partition_size, max_num_partitions, part_out, part_lse, stream);
  }
  pa::DecodeParams p =
      make_decode_params(q, num_seqs, num_heads, cache, block_tables, max_blocks_per_seq, context_lens, scale);
  p.append = make_append_params(key, value, slot_mapping, num_seqs, cache);
  p.part_out = part_out;
  p.part_lse = part_lse;
  p.partition_size = partition_size;
  p.max_num_partitions = max_num_partitions;
  return launch(p, cache, stream);
}

pa_status pa_decode_multi(const void *q, pa_dtype q_dtype, int32_t num_seqs, int32_t num_heads,
                          const int32_t *q_start, int32_t num_queries, int32_t max_q_len, const pa_kv_cache *cache,
                          const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                          float scale, void *out, pa_dtype out_dtype, hipStream_t stream) {
  pa_status st = pa::check_decode_common(q, q_dtype, num_seqs, num_heads, cache, block_tables, max_blocks_per_seq,
                                         context_lens, scale);
  if (st != PA_OK) return st;
  st = pa::check_multi(q_start, num_queries, max_q_len, num_seqs, num_heads, cache);
  if (st != PA_OK || num_seqs == 0 || num_queries == 0) return st;
  st = pa::check_out(out, q_dtype, cache->kv_dtype, out_dtype);
  if (st != PA_OK) return st;
  pa::DecodeParams p =
      make_decode_params(q, num_seqs, num_heads, cache, block_tables, max_blocks_per_seq, context_lens, scale);
  const int64_t rows = static_cast<int64_t>(max_q_len) * p.group;  // rows of one (sequence, kv head)
  p.head_groups = static_cast<int32_t>((rows + 15) / 16);
  p.rows_per_group = static_cast<int32_t>(std::min<int64_t>(16, rows));
  p.q_start = q_start;
  p.num_queries = num_queries;
  p.max_q_len = max_q_len;
  p.out = out;
  p.out_bf16 = out_dtype == PA_BF16;
  p.partition_size = 0;
  p.max_num_partitions = 1;
  return launch(p, cache, stream);
}

pa_status pa_reduce(const float *part_out, const float *part_lse, int32_t num_seqs, int32_t num_heads,
                    int32_t head_dim, int32_t max_num_partitions, const int32_t *context_lens,
                    int32_t partition_size, void *out, pa_dtype out_dtype, hipStream_t stream) {
  pa_status st = pa::check_reduce(part_out, part_lse, num_seqs, num_heads, head_dim, max_num_partitions,
                                  context_lens, partition_size, out, out_dtype);
  if (st != PA_OK || num_seqs == 0) return st;
  if (static_cast<int64_t>(num_seqs) * num_heads > INT32_MAX) return PA_ERR_BAD_SHAPE;
  pa::ReduceParams p{};
  p.part_out = part_out;
  p.part_lse = part_lse;
  p.context_lens = context_lens;
  p.out = out;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.head_dim = head_dim;
  p.max_num_partitions = max_num_partitions;
  p.partition_size = partition_size;
  p.out_bf16 = out_dtype == PA_BF16;
  return from_hip(pa::launch_reduce(p, stream));
}

pa_status pa_decode_split_noalloc(const void *q, pa_dtype q_dtype, int32_t num_seqs, int32_t num_heads,
                                  const pa_kv_cache *cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                  const int32_t *context_lens, float scale, int32_t partition_size, void *out,
                                  pa_dtype out_dtype, hipStream_t stream) {
  pa_status st = pa::check_decode_common(q, q_dtype, num_seqs, num_heads, cache, block_tables, max_blocks_per_seq,
                                         context_lens, scale);
  if (st != PA_OK) return st;
  if (partition_size < 1 || partition_size % cache->block_size != 0) return PA_ERR_BAD_SHAPE;
  if (num_seqs == 0) return PA_OK;
  st = pa::check_out(out, q_dtype, cache->kv_dtype, out_dtype);
  if (st != PA_OK) return st;
  // the fewest partitions that cover a table row; partials and lse must fit
  // the library's scratch
  const int64_t max_len = static_cast<int64_t>(max_blocks_per_seq) * cache->block_size;
  const int32_t pmax = static_cast<int32_t>((max_len + partition_size - 1) / partition_size);
  const size_t need = pa::split_workspace_bytes(num_seqs, num_heads, cache->head_dim, pmax);
  if (need == 0 || need > pa::kNoAllocScratchBytes) return PA_ERR_BAD_WORKSPACE;
  void *base = nullptr;
  st = from_hip(pa::noalloc_scratch(&base));
  if (st != PA_OK) return st;
  const size_t rows = static_cast<size_t>(num_seqs) * num_heads * pmax;
  const size_t lse_off = (rows * cache->head_dim * sizeof(float) + 255) / 256 * 256;
  float *part_out = static_cast<float *>(base);
  float *part_lse = reinterpret_cast<float *>(static_cast<unsigned char *>(base) + lse_off);
  st = pa_decode_split(q, q_dtype, num_seqs, num_heads, cache, block_tables, max_blocks_per_seq, context_lens, scale,
                       partition_size, pmax, part_out, part_lse, stream);
  if (st != PA_OK) return st;
  return pa_reduce(part_out, part_lse, num_seqs, num_heads, cache->head_dim, pmax, context_lens, partition_size, out,
                   out_dtype, stream);
}

pa_status pa_mla_append(const void *latent_rows, const int32_t *slot_mapping, int32_t num_tokens,
                        const pa_latent_cache *cache, hipStream_t stream) {
  const pa_status st = pa::check_mla_append(latent_rows, slot_mapping, num_tokens, cache);
  if (st != PA_OK || num_tokens == 0) return st;
  pa::MlaAppendParams p{};
  p.rows = static_cast<const uint16_t *>(latent_rows);
  p.slot_mapping = slot_mapping;
  p.cache = static_cast<uint16_t *>(cache->latent);
  p.num_tokens = num_tokens;
  p.num_blocks = cache->num_blocks;
  p.block_size = cache->block_size;
  return from_hip(pa::launch_mla_append(p, stream));
}

size_t pa_mla_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t latent_dim, int32_t max_blocks_per_seq,
                              int32_t block_size, int32_t partition_size) {
  return pa::mla_workspace(num_seqs, num_heads, latent_dim, max_blocks_per_seq, block_size, partition_size).total;
}

pa_status pa_mla_decode(const void *q, int32_t num_seqs, int32_t num_heads, int32_t head_dim, const void *w_uk,
                        const void *w_uv, const pa_latent_cache *cache, const int32_t *block_tables,
                        int32_t max_blocks_per_seq, const int32_t *context_lens, float scale, int32_t partition_size,
                        void *workspace, size_t workspace_bytes, void *out, pa_dtype out_dtype, hipStream_t stream) {
  const pa_status st = pa::check_mla_decode(q, num_seqs, num_heads, head_dim, w_uk, w_uv, cache, block_tables,
                                            max_blocks_per_seq, context_lens, scale, partition_size, workspace,
                                            workspace_bytes, out, out_dtype);
  if (st != PA_OK || num_seqs == 0) return st;
  const pa::MlaWorkspace ws = pa::mla_workspace(num_seqs, num_heads, cache->latent_dim, max_blocks_per_seq,
                                                cache->block_size, partition_size);
  unsigned char *base = static_cast<unsigned char *>(workspace);
  pa::MlaParams p{};
  p.q = static_cast<const uint16_t *>(q);
  p.w_uk = static_cast<const uint16_t *>(w_uk);
  p.w_uv = static_cast<const uint16_t *>(w_uv);
  p.cache = static_cast<const uint16_t *>(cache->latent);
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.q_lat = reinterpret_cast<float *>(base);
  p.part_out = reinterpret_cast<float *>(base + ws.part_out_off);
  p.part_lse = reinterpret_cast<float *>(base + ws.part_lse_off);
  p.out = out;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.head_dim = head_dim;
  p.block_size = cache->block_size;
  p.num_blocks = cache->num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.partition_size = partition_size;
  p.max_num_partitions = ws.max_num_partitions;
  p.head_groups = (num_heads + 15) / 16;
  p.scale_log2 = scale * kLog2e;
  p.out_bf16 = out_dtype == PA_BF16;
  return from_hip(pa::launch_mla_decode(p, stream));
}

pa_status pa_copy_blocks(const pa_kv_cache *cache, const int32_t *block_pairs, int32_t num_pairs,
                         hipStream_t stream) {
  pa_status st = pa::check_copy(cache, block_pairs, num_pairs);
  if (st != PA_OK || num_pairs == 0) return st;
  return launch_block_copies(cache, cache, block_pairs, num_pairs, stream);
}

pa_status pa_swap_blocks(const pa_kv_cache *src, const pa_kv_cache *dst, const int32_t *block_pairs,
                         int32_t num_pairs, hipStream_t stream) {
  pa_status st = pa::check_swap(src, dst, block_pairs, num_pairs);
  if (st != PA_OK || num_pairs == 0) return st;
  return launch_block_copies(src, dst, block_pairs, num_pairs, stream);
}

pa_status pa_probe_read(const void *buf, size_t bytes, int32_t mode, int32_t tile_bytes, uint32_t *sink,
                        hipStream_t stream) {
  const pa_status st = pa::check_probe(buf, bytes, mode, tile_bytes, sink);
  if (st != PA_OK) return st;
  return from_hip(pa::launch_probe_read(buf, bytes, mode, tile_bytes, sink, stream));
}

size_t pa_split_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_num_partitions) {
  return pa::split_workspace_bytes(num_seqs, num_heads, head_dim, max_num_partitions);
}

const char *pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL_PTR: return "a required pointer is null, or a pointer that must be null is not";
    case PA_ERR_BAD_SHAPE: return "a size is out of range or inconsistent";
    case PA_ERR_UNSUPPORTED: return "unsupported dtype, head_dim or block_size combination";
    case PA_ERR_MISALIGNED: return "a pointer is not aligned as required";
    case PA_ERR_BAD_WORKSPACE:
      return "split scratch too small: max_num_partitions below ceil(max_blocks_per_seq * block_size / "
             "partition_size), or partials beyond the fixed scratch of pa_decode_split_noalloc";
    case PA_ERR_HIP: return "HIP kernel launch failed (see pa_last_hip_error)";
    case PA_ERR_OUT_OF_BLOCKS: return "not enough free blocks";
    case PA_ERR_INVALID_BLOCK: return "a block id is out of range or not in use";
  }
  return "unknown status";
}

int32_t pa_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
