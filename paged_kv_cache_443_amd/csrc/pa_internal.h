// Internal interface between the C ABI layer (pa_api.cpp) and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "pa.h"

namespace pa {

// Everything one cache append needs (also carried by a fused append + decode).
struct AppendParams {
  const void *key;
  const void *value;
  const int32_t *slot_mapping;
  void *k_cache;
  void *v_cache;
  uint16_t *k_scale;
  uint16_t *v_scale;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t head_dim;
  int32_t num_blocks;
};

// Everything one decode launch needs, passed by value to the kernel.
struct DecodeParams {
  const void *q;              // [B][Hq][D]
  const void *k_cache;        // K pool
  const void *v_cache;        // V pool
  const uint16_t *k_scale;    // fp16 bits, int8 caches only
  const uint16_t *v_scale;    // fp16 bits, int8 caches only
  const int32_t *block_tables;
  const int32_t *context_lens;
  void *out;                  // [B][Hq][D] (pa_decode)
  float *part_out;            // [B][Hq][Pmax][D] (pa_decode_split)
  float *part_lse;            // [B][Hq][Pmax]
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t group;              // num_heads / num_kv_heads
  int32_t head_groups;        // groups of <= 16 query rows per kv head: ceil(max query tokens * group / 16)
                              // (the causal launcher packs R of them per unit and stores ceil(groups / R))
  int32_t rows_per_group;     // min(16, max query tokens * group): LDS rows of a work-group
  const int32_t *q_start;     // causal multi-query: [num_seqs + 1] first query row of each sequence, else null
  int32_t num_queries;        // causal multi-query: rows of q and out
  int32_t max_q_len;          // causal multi-query: bound of any sequence's query tokens
  AppendParams append;        // fused append + decode: token b of each sequence b (slot_mapping null: none)
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t partition_size;     // 0: whole sequence (pa_decode)
  int32_t max_num_partitions;
  int32_t tbl_window;         // block-table entries staged in LDS at a time (multiple of 4)
  int32_t lpt;                // single pass: take sequences longest first (ranked in LDS)
  float scale;                // softmax scale as given
  float scale_log2;           // scale * log2(e)
  int32_t out_bf16;           // 1: bf16 output, 0: fp32 output
};

struct ReduceParams {
  const float *part_out;
  const float *part_lse;
  const int32_t *context_lens;
  void *out;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t head_dim;
  int32_t max_num_partitions;
  int32_t partition_size;
  int32_t out_bf16;
};



// Whole-block copies from one pool to another of the same layout (the same
// pool for copy-on-write; a GPU pool and a pinned host pool for a swap).
struct CopyParams {
  const void *src_k;
  const void *src_v;
  const void *src_k_scale;    // int8 caches only, else null
  const void *src_v_scale;
  void *dst_k;
  void *dst_v;
  void *dst_k_scale;
  void *dst_v_scale;
  const int32_t *pairs;       // [num_pairs][2] (source block, destination block)
  int32_t num_pairs;
  int32_t num_kv_heads;
  int32_t src_blocks;         // blocks in the source pool
  int32_t dst_blocks;         // blocks in the destination pool
  int32_t block_size;
  size_t tile_bytes;          // one (block, kv head) tile of one pool
};

// MLA decode over a paged latent cache (pa_mla_decode).
struct MlaParams {
  const uint16_t *q;          // [B][H][head_dim] bf16
  const uint16_t *w_uk;       // [latent_dim][H * head_dim] bf16: K = c W_uk
  const uint16_t *w_uv;       // [latent_dim][H * head_dim] bf16: V = c W_uv
  const uint16_t *cache;      // [num_blocks][block_size][latent_dim] bf16
  const int32_t *block_tables;
  const int32_t *context_lens;
  float *q_lat;               // workspace: [B][H][latent_dim] absorbed queries
  float *part_out;            // workspace: [B][H][Pmax][latent_dim] normalised partial latent outputs
  float *part_lse;            // workspace: [B][H][Pmax]
  void *out;                  // [B][H][head_dim]
  int32_t num_seqs;
  int32_t num_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t partition_size;
  int32_t max_num_partitions;
  int32_t head_groups;        // ceil(H / 16)
  float scale_log2;           // scale * log2(e)
  int32_t out_bf16;
};

// Latent rows written into their slots (pa_mla_append).
struct MlaAppendParams {
  const uint16_t *rows;       // [T][latent_dim] bf16
  const int32_t *slot_mapping;
  uint16_t *cache;
  int32_t num_tokens;
  int32_t num_blocks;
  int32_t block_size;
};

// Latent width the MLA kernels are built for (the pages' 512).
constexpr int32_t kMlaLatentDim = 512;
// Tokens per MLA chunk; partitions are a multiple of it.
constexpr int32_t kMlaChunk = 64;
// Largest MLA partition and batch (the persistent pass indexes pieces in LDS).
constexpr int32_t kMlaMaxPartition = 4096;
constexpr int32_t kMlaMaxSeqs = 4096;

// Largest batch the fused append + split pass takes (the persistent split
// pass indexes its sequences' pieces in LDS).
constexpr int32_t kMaxFusedSplitSeqs = 4096;

// Bytes of the library's own device scratch (pa_decode_split_noalloc): the
// partials and log-sum-exps of one KV-split decode.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;

// Device address of that scratch on the current device (looked up once per
// device with hipGetSymbolAddress, then cached; no allocation).
hipError_t noalloc_scratch(void **ptr);

// Launchers (one per kernel family); each returns the launch's hipError_t.
hipError_t launch_decode_mfma(const DecodeParams &p, pa_dtype kv_dtype, int head_dim, int block_size, hipStream_t s);
hipError_t launch_decode_f32(const DecodeParams &p, int head_dim, int block_size, hipStream_t s);
// Single-token decode of a bf16 cache on the vector ALUs (the arithmetic
// alternative to the matrix cores; pa_decode takes it when PA_DECODE_VALU=1).
bool decode_valu_applies(const DecodeParams &p, pa_dtype kv_dtype, int head_dim);
hipError_t launch_decode_valu(const DecodeParams &p, int head_dim, int block_size, hipStream_t s);
hipError_t launch_reduce(const ReduceParams &p, hipStream_t s);
hipError_t launch_append(const AppendParams &p, pa_dtype kv_dtype, hipStream_t s);
hipError_t launch_copy_blocks(const CopyParams &p, hipStream_t s);
hipError_t launch_mla_decode(const MlaParams &p, hipStream_t s);
hipError_t launch_mla_append(const MlaAppendParams &p, hipStream_t s);
hipError_t launch_probe_read(const void *buf, size_t bytes, int mode, int tile_bytes, uint32_t *sink, hipStream_t s);

}  // namespace pa
