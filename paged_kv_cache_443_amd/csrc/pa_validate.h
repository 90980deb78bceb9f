// Host-side argument validation for the C ABI.  Pure C++ (no HIP calls), so
// it can be built and exercised without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

pa_status check_cache(const pa_kv_cache *c);
pa_status check_append(const void *key, const void *value, pa_dtype src_dtype, const int32_t *slot_mapping,
                       int32_t num_tokens, const pa_kv_cache *cache);
pa_status check_decode_common(const void *q, pa_dtype q_dtype, int32_t num_seqs, int32_t num_heads,
                              const pa_kv_cache *cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                              const int32_t *context_lens, float scale);
pa_status check_out(const void *out, pa_dtype q_dtype, pa_dtype kv_dtype, pa_dtype out_dtype);
pa_status check_split(int32_t partition_size, int32_t max_num_partitions, int32_t block_size,
                      int32_t max_blocks_per_seq, const float *part_out, const float *part_lse);
pa_status check_multi(const int32_t *q_start, int32_t num_queries, int32_t max_q_len, int32_t num_seqs,
                      int32_t num_heads, const pa_kv_cache *cache);
pa_status check_reduce(const float *part_out, const float *part_lse, int32_t num_seqs, int32_t num_heads,
                       int32_t head_dim, int32_t max_num_partitions, const int32_t *context_lens,
                       int32_t partition_size, const void *out, pa_dtype out_dtype);
pa_status check_copy(const pa_kv_cache *cache, const int32_t *block_pairs, int32_t num_pairs);
pa_status check_swap(const pa_kv_cache *src, const pa_kv_cache *dst, const int32_t *block_pairs, int32_t num_pairs);
pa_status check_probe(const void *buf, size_t bytes, int32_t mode, int32_t tile_bytes, const uint32_t *sink);
pa_status check_latent_cache(const pa_latent_cache *c);
pa_status check_mla_append(const void *rows, const int32_t *slot_mapping, int32_t num_tokens,
                           const pa_latent_cache *cache);
pa_status check_mla_decode(const void *q, int32_t num_seqs, int32_t num_heads, int32_t head_dim, const void *w_uk,
                           const void *w_uv, const pa_latent_cache *cache, const int32_t *block_tables,
                           int32_t max_blocks_per_seq, const int32_t *context_lens, float scale,
                           int32_t partition_size, const void *workspace, size_t workspace_bytes, const void *out,
                           pa_dtype out_dtype);
// Byte offsets of the MLA workspace parts (absorbed queries at 0); total 0 on invalid sizes.
struct MlaWorkspace {
  size_t part_out_off;
  size_t part_lse_off;
  size_t total;
  int32_t max_num_partitions;
};
MlaWorkspace mla_workspace(int32_t num_seqs, int32_t num_heads, int32_t latent_dim, int32_t max_blocks_per_seq,
                           int32_t block_size, int32_t partition_size);
size_t split_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_num_partitions);

}  // namespace pa
