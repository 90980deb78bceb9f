/*
 * pa.h -- C ABI of the MI355X (gfx950) paged-attention decode library.
 *
 * One new query token per sequence attends over that sequence's KV cache.
 * The cache is a pool of fixed-size physical blocks shared by all
 * sequences; sequence b reaches its tokens through row b of a block table
 * (logical block j of the sequence lives in physical block
 * block_tables[b][j]).  Sources: page "字节跳动 AI Infra (2)", question on
 * vLLM and PagedAttention (block pool of 16-token blocks, per-request block
 * tables, beams sharing prefix blocks with a copy-on-write last block, and
 * the kernel sketch that turns a block-table entry into a K/V address);
 * page "LLM推理优化", section 3.2 (fixed-size blocks, logical-to-physical
 * mapping, copy-on-write sharing).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument except `cache` and `stream` is a DEVICE pointer
 *   (HBM of the GPU that is current when the call is made).  `cache` is a
 *   host pointer to a descriptor holding device pointers.
 * - The caller owns all memory.  The library allocates no device memory,
 *   frees nothing of the caller's, copies nothing to the host and never
 *   synchronises; it keeps no state except a thread-local copy of the last
 *   HIP error.  (The host block manager's bookkeeping lives in host memory
 *   that pa_bm_create allocates and pa_bm_destroy frees; the one fixed
 *   device array of pa_decode_split_noalloc is part of the library's code
 *   object, not an allocation, and its address is looked up once per GPU.)
 * - Every call validates its host-visible arguments, then enqueues its
 *   kernels on `stream` and returns.  PA_OK means "valid and launched", not
 *   "finished".  On an error status nothing is launched and no output is
 *   touched.
 * - Device-resident values (context_lens, block-table entries, slots) are
 *   not visible to the host and are not validated; the preconditions are
 *   stated per call.  Kernels clamp out-of-range block ids and skip
 *   out-of-range slots so that bad device data gives wrong numbers, never an
 *   out-of-bounds access.
 * - Reduction order depends only on logical positions, never on physical
 *   block ids, and no floating-point atomics are used: results are bitwise
 *   reproducible run to run and invariant under relabelling of blocks.
 *
 * Cache layout (x = elements per storage vector: fp32 4, bf16 8, int8 16 in
 * 16 bytes; int4 16 codes in 8 bytes)
 * -----------------------------------------------------------------
 *   k_cache  [num_blocks][num_kv_heads][head_dim / x][block_size][x]
 *   v_cache  [num_blocks][num_kv_heads][block_size / x][head_dim][x]
 *   k_scale, v_scale (int8 / int4 caches only): fp16 [num_blocks][num_kv_heads][block_size]
 * K of (block pb, kv head h, in-block offset t, channel d) is
 * k_cache[pb][h][d / x][slot(t)][d % x] with slot(t) = t for fp32 and int8
 * caches and, for bf16 caches, t with its bits 2 and 3 exchanged (offsets
 * 0-3, 8-11, 4-7, 12-15 in every group of 16).  V of (pb, h, t, d) is
 * v_cache[pb][h][t / x][d][t % x].  Scales are indexed by t.  int4 caches
 * hold two 4-bit two's-complement codes per byte, element 2i of a vector in
 * the low nibble of byte i and element 2i + 1 in the high nibble (INT4 KV
 * cache: page "LLM推理优化", section 1.3; the packing is this library's).
 * Each (block, kv head) owns block_size * head_dim contiguous elements of
 * each pool, so with one kv head block pb starts at element
 * pb * block_size * head_dim, the address the pages' kernel sketch forms.
 * Inside a block, K is stored in 16-byte channel groups per token and V in
 * 16-byte token groups per channel, so that each lane of a wavefront loads
 * exactly the 16 bytes its matrix-core operand needs; the bf16 slot order
 * makes every K load instruction cover whole 128-byte lines.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL_PTR = 1,      /* a required pointer is NULL (or a forbidden one is not) */
  PA_ERR_BAD_SHAPE = 2,     /* a size is out of range or inconsistent */
  PA_ERR_UNSUPPORTED = 3,   /* a valid but unimplemented combination (dtype, head_dim, block_size) */
  PA_ERR_MISALIGNED = 4,    /* a pointer breaks the stated alignment */
  PA_ERR_BAD_WORKSPACE = 5, /* split scratch too small for the call */
  PA_ERR_HIP = 6,           /* the HIP launch failed; see pa_last_hip_error() */
  PA_ERR_OUT_OF_BLOCKS = 7, /* block manager: not enough free blocks (nothing changed) */
  PA_ERR_INVALID_BLOCK = 8  /* block manager: a block id out of range or not in use (nothing changed) */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_I8 = 2, PA_I4 = 3 } pa_dtype;

/* Descriptor of one paged KV cache (one layer).  Pointers are device pointers. */
typedef struct pa_kv_cache {
  void *k_cache;        /* see layout above; 16-byte aligned */
  void *v_cache;        /* see layout above; 16-byte aligned */
  void *k_scale;        /* fp16, int8 / int4 caches only (else NULL); 16-byte aligned */
  void *v_scale;        /* fp16, int8 / int4 caches only (else NULL); 16-byte aligned */
  int32_t num_blocks;   /* blocks in the pool, >= 1 */
  int32_t num_kv_heads; /* >= 1 */
  int32_t block_size;   /* tokens per block: 16, 32 or 64 */
  int32_t head_dim;     /* 64 or 128 */
  pa_dtype kv_dtype;    /* PA_F32, PA_BF16, PA_I8 or PA_I4 */
} pa_kv_cache;

/*
 * pa_reshape_and_cache -- write new tokens' K and V into their cache slots.
 *
 * The cache grows by one row per token before attention reads it (page
 * "字节跳动 AI Infra (2)", KV-cache question, step-t equations: the new K/V
 * row is concatenated onto the cached ones).  Token i goes to slot
 * s = slot_mapping[i]: physical block s / block_size, offset
 * s % block_size; s < 0 (conventionally -1) skips the token.
 *
 *   key, value    [num_tokens][num_kv_heads][head_dim], src_dtype, 16-byte aligned
 *   slot_mapping  int32 [num_tokens], 4-byte aligned
 *   src_dtype     PA_F32 for an fp32 cache; PA_BF16 for bf16, int8 and int4 caches
 *
 * fp32/bf16 caches store the source bits unchanged.  int8 caches (INT8
 * KV-cache quantisation: page "字节跳动 AI Infra (2)", optimisation table;
 * page "LLM推理优化", section 1.3) store per (token, kv head) the fp16 scale
 * s = fp16_rne(fp32(max|x| / 127)) and codes rint_even(fp32(x / s))
 * clamped to [-127, 127] (all codes 0 when s is 0).  int4 caches (page
 * "LLM推理优化", section 1.3, names INT4 beside INT8) do the same with
 * s = fp16_rne(fp32(max|x| / 7)) and codes clamped to [-7, 7].  Bit-exact.
 * Preconditions (device data): slots of one call are distinct; slots
 * >= num_blocks * block_size are skipped.  num_tokens == 0 is a no-op.
 */
pa_status pa_reshape_and_cache(const void *key, const void *value, pa_dtype src_dtype, const int32_t *slot_mapping,
                               int32_t num_tokens, const pa_kv_cache *cache, hipStream_t stream);

/*
 * pa_decode -- single-pass paged decode attention.
 *
 * For sequence b with L = context_lens[b] cached tokens (the newest one
 * included) and query head h, with kv head kv = h / (num_heads /
 * num_kv_heads) (consecutive query heads share one K/V head: GQA, MQA when
 * num_kv_heads == 1; page "LLM推理优化", section 1.3):
 *     out[b][h] = sum_t softmax_t(scale * q[b][h] . k_t) v_t,   t < L,
 * where token t lives in block block_tables[b][t / block_size] at offset
 * t % block_size (page "字节跳动 AI Infra (2)", KV-cache question step-t
 * equations and PagedAttention kernel sketch).  L == 0 gives a zero row.
 *
 *   q             [num_seqs][num_heads][head_dim], q_dtype, 16-byte aligned
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]; the whole row must
 *                 be readable memory.  Entries past ceil(L / block_size) may
 *                 be loaded (the row is staged in LDS in windows, with no
 *                 wait on L) but never form an address or influence the
 *                 result: they may hold anything
 *   context_lens  int32 [num_seqs]
 *   out           [num_seqs][num_heads][head_dim], out_dtype, 16-byte aligned
 *   (q, kv, out) dtypes: (F32, F32, F32), (BF16, BF16, BF16|F32),
 *                        (BF16, I8, BF16|F32), (BF16, I4, BF16|F32)
 * Accumulation is fp32; bf16 outputs are the round-to-nearest-even of the
 * fp32 result.  Tokens at positions >= L of the last block are never used,
 * whatever they hold (NaN included).
 * Preconditions (device data): 0 <= L <= max_blocks_per_seq * block_size;
 * the first ceil(L / block_size) entries of each row are < num_blocks.
 * num_seqs == 0 is a no-op.
 * Arithmetic unit: the products run on the matrix cores.  With the
 * environment variable PA_DECODE_VALU set to "1" (read at every call), a
 * bf16 cache with head_dim 128 and at most 16 query heads per kv head runs
 * them on the vector ALUs instead (v_dot2 over bf16 pairs, the same fp32
 * accumulation and results within the same tolerance): a measurement
 * switch, slower on every measured shape.
 */
pa_status pa_decode(const void *q, pa_dtype q_dtype, int32_t num_seqs, int32_t num_heads, const pa_kv_cache *cache,
                    const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens, float scale,
                    void *out, pa_dtype out_dtype, hipStream_t stream);

/*
 * pa_append_decode -- one decode step in one call: pa_reshape_and_cache of
 * each sequence's new token, then pa_decode over every sequence.
 *
 * Token b of key/value ([num_seqs][num_kv_heads][head_dim], src_dtype as for
 * pa_reshape_and_cache) goes to slot slot_mapping[b] (< 0 skips it), and
 * sequence b then attends over its L = context_lens[b] cached tokens, the new
 * one included (the concatenation of page "字节跳动 AI Infra (2)", KV-cache
 * question, step-t equations).  The results (cache contents and out) are
 * those of the two calls, bit for bit.  With a bf16, int8 or int4 cache and
 * at most 16 query heads per kv head it is one kernel (the append costs no
 * launch of its own): the work-group of each (sequence, kv head) takes
 * position L - 1's K and V from key/value (int8/int4: codes and scales,
 * quantised as the append quantises them; the bits the cache row receives)
 * and extra work-groups at the end of the grid write the rows.  Otherwise it
 * makes the two launches.
 * Preconditions (device data): those of both calls; the new token of
 * sequence b is its position L - 1, its slot in a block only b references.
 */
pa_status pa_append_decode(const void *key, const void *value, pa_dtype src_dtype, const int32_t *slot_mapping,
                           const void *q, pa_dtype q_dtype, int32_t num_seqs, int32_t num_heads,
                           const pa_kv_cache *cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                           const int32_t *context_lens, float scale, void *out, pa_dtype out_dtype,
                           hipStream_t stream);

/*
 * pa_append_decode_split -- one KV-split decode step in one call:
 * pa_reshape_and_cache of each sequence's new token, then pa_decode_split.
 *
 * Arguments as for pa_append_decode up to scale, then those of
 * pa_decode_split.  The results (cache contents, part_out, part_lse) are
 * those of the two calls, bit for bit; merge them with pa_reduce.  One kernel
 * for a bf16 or int8 cache with at most 16 query heads per kv head and at
 * most 4096 sequences: the piece holding position L - 1 takes that position's
 * K and V (int8: codes and scales, quantised as the append quantises them)
 * from key/value, and the split pass's work-groups write the new rows after
 * their last piece; otherwise the two launches.
 * Preconditions (device data): those of both calls; the new token of
 * sequence b is its position L - 1, its slot in a block only b references.
 */
pa_status pa_append_decode_split(const void *key, const void *value, pa_dtype src_dtype, const int32_t *slot_mapping,
                                 const void *q, pa_dtype q_dtype, int32_t num_seqs, int32_t num_heads,
                                 const pa_kv_cache *cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                 const int32_t *context_lens, float scale, int32_t partition_size,
                                 int32_t max_num_partitions, float *part_out, float *part_lse, hipStream_t stream);

/*
 * pa_decode_multi -- paged attention of several new query tokens per
 * sequence, causally masked (chunked prefill in small chunks, page
 * "vLLM框架是怎么做推理加速的", section 3; verification of several draft
 * tokens at once).
 *
 * Sequence b has n_b = q_start[b + 1] - q_start[b] new tokens, the last n_b
 * of its L = context_lens[b] cached tokens (their K/V rows already written
 * with pa_reshape_and_cache).  Its query token i is row q_start[b] + i of q
 * and out; it sits at position L - n_b + i and attends to the positions up
 * to and including its own:
 *     out[r][h] = sum_{t <= L - n_b + i} softmax_t(scale * q[r][h] . k_t) v_t
 * (the step-t attention of page "字节跳动 AI Infra (2)", KV-cache question,
 * taken for each new token in turn).  With max_q_len == 1 this is
 * pa_decode, bit for bit; a larger bound may change the fp32 summation
 * order (the launch shape depends on max_q_len * num_heads / num_kv_heads).
 *
 *   q             [num_queries][num_heads][head_dim], q_dtype (F32 for an
 *                 F32 cache, else BF16), 16-byte aligned
 *   q_start       int32 [num_seqs + 1], non-decreasing, q_start[0] == 0,
 *                 q_start[num_seqs] == num_queries (device memory)
 *   num_queries   rows of q and out; <= num_seqs * max_q_len
 *   max_q_len     an upper bound of every n_b (sets the launch size)
 *   out           [num_queries][num_heads][head_dim], out_dtype
 *   other arguments as for pa_decode; every cache kind is served (F32 on
 *   the vector ALUs, one wavefront per (query row, head); BF16, I8 and I4
 *   on the matrix cores).
 * Preconditions (device data): n_b <= max_q_len and n_b <= L; L as for
 * pa_decode.  A sequence whose q_start entries leave [0, num_queries], or
 * with n_b > max_q_len, is skipped (its rows are left as they are); rows of
 * a sequence with n_b > L are unspecified.  num_seqs == 0 or
 * num_queries == 0 is a no-op.
 */
pa_status pa_decode_multi(const void *q, pa_dtype q_dtype, int32_t num_seqs, int32_t num_heads,
                          const int32_t *q_start, int32_t num_queries, int32_t max_q_len, const pa_kv_cache *cache,
                          const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                          float scale, void *out, pa_dtype out_dtype, hipStream_t stream);

/*
 * pa_decode_split -- first pass of KV-split decode (FlashDecoding: split
 * along the KV length for long sequences; page "字节跳动 AI Infra (2)",
 * third question, layer-2 table).
 *
 * Partition p of sequence b covers positions [p * partition_size,
 * min((p + 1) * partition_size, L)).  For each (b, h, p) it writes the
 * normalised partial output o_p = softmax restricted to that range applied
 * to V, and lse_p = natural log of sum over the range of exp(scale * q.k_t).
 * Only partitions that hold tokens (p < ceil(L / partition_size)) are
 * written; the entries of the others are left as they are (pa_reduce never
 * reads them).  For L == 0 nothing of sequence b is written.
 *
 *   arguments up to `scale` as for pa_decode, then
 *   partition_size      tokens per partition, a positive multiple of block_size
 *   max_num_partitions  Pmax >= ceil(max_blocks_per_seq * block_size / partition_size)
 *   part_out            fp32 [num_seqs][num_heads][Pmax][head_dim], 16-byte aligned
 *   part_lse            fp32 [num_seqs][num_heads][Pmax], 4-byte aligned
 */
pa_status pa_decode_split(const void *q, pa_dtype q_dtype, int32_t num_seqs, int32_t num_heads,
                          const pa_kv_cache *cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                          const int32_t *context_lens, float scale, int32_t partition_size,
                          int32_t max_num_partitions, float *part_out, float *part_lse, hipStream_t stream);

/*
 * pa_reduce -- second pass of KV-split decode: log-sum-exp merge.
 *
 * With n = ceil(L / partition_size) used partitions, M = max_p lse_p and
 * w_p = exp(lse_p - M):  out[b][h] = sum_p w_p o_p / sum_p w_p  (online
 * softmax statistics combine this way; page "LLM推理优化", section 2).
 * L == 0 gives a zero row.  Arguments mirror pa_decode_split's; out as for
 * pa_decode (out_dtype PA_F32 or PA_BF16).
 */
pa_status pa_reduce(const float *part_out, const float *part_lse, int32_t num_seqs, int32_t num_heads,
                    int32_t head_dim, int32_t max_num_partitions, const int32_t *context_lens,
                    int32_t partition_size, void *out, pa_dtype out_dtype, hipStream_t stream);

/*
 * pa_decode_split_noalloc -- pa_decode_split followed by pa_reduce, with the
 * partials in the library's own device memory instead of a caller workspace.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The call
 * allocates nothing.  Arguments as for pa_decode_split up to partition_size,
 * then out / out_dtype as for pa_decode.  It uses max_num_partitions =
 * ceil(max_blocks_per_seq * block_size / partition_size), and the result is
 * that of pa_decode_split with that max_num_partitions followed by pa_reduce,
 * bit for bit.
 *
 * Scratch: one fixed array of 32 MiB per GPU (a file-scope device array of
 * the library, held by every GPU the library runs on until the process
 * ends).  It must hold num_seqs * num_heads * max_num_partitions * (head_dim
 * floats of partial output, placed first and padded to 256 bytes, then one
 * float of lse): pa_split_workspace_bytes() of those sizes <= 32 MiB, else
 * PA_ERR_BAD_WORKSPACE and nothing is launched.  Every call on a GPU uses
 * the same array and leaves its partials there: calls that overlap on one
 * GPU (on different streams without ordering between them) race and give
 * undefined results.  Calls ordered on one stream are safe.
 * Preconditions (device data): those of pa_decode_split.
 */
pa_status pa_decode_split_noalloc(const void *q, pa_dtype q_dtype, int32_t num_seqs, int32_t num_heads,
                                  const pa_kv_cache *cache, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                  const int32_t *context_lens, float scale, int32_t partition_size, void *out,
                                  pa_dtype out_dtype, hipStream_t stream);

/*
 * pa_copy_blocks -- copy whole physical blocks (the copy of copy-on-write).
 *
 * Sequences may share physical blocks (a forked beam shares its parent's
 * blocks); before one of them writes into a shared block, the block is
 * copied into a private one (page "字节跳动 AI Infra (2)", PagedAttention
 * question, block-pool figure: two beams share B1 and B3, the second writes
 * into B6', a copy of B6; page "LLM推理优化", section 3.2).  For each
 * i < num_pairs, block block_pairs[2i] (source) is copied to block
 * block_pairs[2i + 1] (destination): every K and V element of every kv head
 * and, for int8 and int4 caches, every scale.
 *
 *   cache        the pool (any dtype)
 *   block_pairs  int32 [num_pairs][2] (source, destination), device, 4-byte aligned
 * Preconditions (device data): destinations distinct, no destination also a
 * source in the same call (then every copy reads the pool as it was before
 * the call); pairs with an id outside [0, num_blocks) are skipped.
 * num_pairs == 0 is a no-op.
 */
pa_status pa_copy_blocks(const pa_kv_cache *cache, const int32_t *block_pairs, int32_t num_pairs, hipStream_t stream);

/*
 * pa_swap_blocks -- copy whole physical blocks from one pool to another of
 * the same layout: the GPU pool and a host pool, for preemption.
 *
 * When GPU memory runs short, or a request is preempted, its blocks are
 * moved to CPU memory and brought back before it runs again (page
 * "字节跳动 AI Infra (2)", PagedAttention question, scheduling list; page
 * "vLLM框架是怎么做推理加速的", section 2 and its second follow-up).  For
 * each i < num_pairs, block block_pairs[2i] of `src` is copied to block
 * block_pairs[2i + 1] of `dst`: every K and V element of every kv head and,
 * for int8 and int4 caches, every scale.  A block's contents do not depend on where
 * it lives: after swapping out and back in under new ids (and rewriting the
 * block table) a sequence decodes bit for bit as before.
 *
 *   src, dst     pools of the same kv_dtype, num_kv_heads, block_size and
 *                head_dim (else PA_ERR_BAD_SHAPE).  Either may be host memory
 *                that the GPU can address: allocated pinned (hipHostMalloc;
 *                torch's pin_memory=True), not registered after the fact.
 *                The kernel reads and writes it directly over the bus.
 *   block_pairs  int32 [num_pairs][2] (source id in src, destination id in
 *                dst), device memory or pinned host memory, 4-byte aligned
 * Preconditions (device data): destinations distinct; if src and dst are the
 * same pool, no destination is also a source.  Pairs with an id outside its
 * pool are skipped.  The copy is ordered on `stream` like any kernel: host
 * code reads a host destination only after synchronising with the stream.
 * num_pairs == 0 is a no-op.
 */
pa_status pa_swap_blocks(const pa_kv_cache *src, const pa_kv_cache *dst, const int32_t *block_pairs,
                         int32_t num_pairs, hipStream_t stream);

/*
 * MLA latent cache -- multi-head latent attention (page "字节跳动 AI Infra
 * (2)", question on KV-cache principles, the MLA paragraph and the MLA row
 * of its optimisation table).  Each token's K and V are compressed jointly
 * into one latent row c (latent_dim wide, 512 in the page's example); the
 * cache stores only c, and the heads' keys and values are recovered by the
 * up-projections K = c W_uk and V = c W_uv (latent_dim -> num_heads x
 * head_dim; head h is column block h, channel d of head h is column
 * h * head_dim + d).  The V projection is this library's reading: the page
 * writes out the K one and says K and V are compressed together.
 *
 * Layout: latent [num_blocks][block_size][latent_dim] bf16, the row of
 * logical position t of a sequence in block block_tables[b][t / block_size]
 * at offset t % block_size.  Pointers are device pointers.
 */
typedef struct pa_latent_cache {
  void *latent;         /* bf16, 16-byte aligned */
  int32_t num_blocks;   /* >= 1 */
  int32_t block_size;   /* 16, 32 or 64 */
  int32_t latent_dim;   /* 512 */
} pa_latent_cache;

/*
 * pa_mla_append -- write new tokens' latent rows into their slots.
 *
 *   latent_rows   bf16 [num_tokens][latent_dim], 16-byte aligned
 *   slot_mapping  int32 [num_tokens]: row i goes to block s / block_size,
 *                 offset s % block_size; s < 0 or s >= num_blocks *
 *                 block_size skips it.  Bit-exact copy.
 * num_tokens == 0 is a no-op.  Preconditions (device data): slots distinct.
 */
pa_status pa_mla_append(const void *latent_rows, const int32_t *slot_mapping, int32_t num_tokens,
                        const pa_latent_cache *cache, hipStream_t stream);

/* Workspace bytes of pa_mla_decode (absorbed queries, partial outputs and
 * log-sum-exps); 0 on invalid sizes. */
size_t pa_mla_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t latent_dim, int32_t max_blocks_per_seq,
                              int32_t block_size, int32_t partition_size);

/*
 * pa_mla_decode -- decode attention over an MLA latent cache.
 *
 * For sequence b with L = context_lens[b] cached tokens and query head h:
 *     K_t = c_t W_uk[:, h],  V_t = c_t W_uv[:, h],
 *     out[b][h] = sum_{t < L} softmax_t(scale * q[b][h] . K_t) V_t;
 * L == 0 gives a zero row.  Computed without forming K or V: the query is
 * moved into the latent space (q_lat = W_uk[:, h] q), attention runs over
 * the latent rows in partitions of partition_size tokens (normalised
 * partial latent outputs and log-sum-exps, merged as pa_reduce merges), and
 * the merged latent output is projected by W_uv[:, h].  fp32 accumulation;
 * bf16 out is the round-to-nearest-even of the fp32 result.
 *
 *   q               bf16 [num_seqs][num_heads][head_dim], 16-byte aligned
 *   head_dim        64 or 128;  num_heads >= 1;  num_seqs <= 4096
 *   w_uk, w_uv      bf16 [latent_dim][num_heads * head_dim], 16-byte aligned
 *   block_tables    int32 [num_seqs][max_blocks_per_seq] (whole row readable)
 *   context_lens    int32 [num_seqs]
 *   partition_size  a multiple of 64 and of block_size, at most 4096
 *   workspace       device memory, 256-byte aligned, workspace_bytes >=
 *                   pa_mla_workspace_bytes(...) (else PA_ERR_BAD_WORKSPACE)
 *   out             [num_seqs][num_heads][head_dim], out_dtype PA_F32 or PA_BF16
 * Preconditions (device data): 0 <= L <= max_blocks_per_seq * block_size;
 * the first ceil(L / block_size) entries of each row are < num_blocks.
 * num_seqs == 0 is a no-op.
 */
pa_status pa_mla_decode(const void *q, int32_t num_seqs, int32_t num_heads, int32_t head_dim, const void *w_uk,
                        const void *w_uv, const pa_latent_cache *cache, const int32_t *block_tables,
                        int32_t max_blocks_per_seq, const int32_t *context_lens, float scale, int32_t partition_size,
                        void *workspace, size_t workspace_bytes, void *out, pa_dtype out_dtype, hipStream_t stream);

/*
 * Block manager -- host bookkeeping of a block pool (no GPU work).
 *
 * Reference counts of num_blocks physical blocks of block_size tokens.  Blocks
 * are handed out on demand as sequences grow (page "LLM推理优化", section 3.2:
 * 100, 50 and 200 tokens take 7, 4 and 13 blocks of 16); a fork shares every
 * block of a table; a write into a block that another table still references
 * first moves the writer to a private copy (copy-on-write; the copy itself is
 * pa_copy_blocks).  Free blocks are handed out lowest id first.  All pointers
 * are HOST pointers.  A manager is not thread-safe; every call either
 * succeeds or leaves the manager unchanged.
 */
typedef struct pa_block_manager pa_block_manager;

/* Create a manager (host memory, owned by the caller until pa_bm_destroy).
 * PA_ERR_BAD_SHAPE unless num_blocks >= 1, block_size >= 1 and
 * num_blocks * block_size <= INT32_MAX (slots are int32). */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager **out);
void pa_bm_destroy(pa_block_manager *bm);
/* Free blocks; references held on block b (-1 if b is out of range). */
int32_t pa_bm_num_free(const pa_block_manager *bm);
int32_t pa_bm_refcount(const pa_block_manager *bm, int32_t block);
/* n free blocks, lowest ids first, one reference each, into ids_out[n]. */
pa_status pa_bm_allocate(pa_block_manager *bm, int32_t n, int32_t *ids_out);
/* Drop one reference to each of ids[n] (all must be in use). */
pa_status pa_bm_free(pa_block_manager *bm, const int32_t *ids, int32_t n);
/* One more reference to each of table[n] (all must be in use): a fork. */
pa_status pa_bm_fork(pa_block_manager *bm, const int32_t *table, int32_t n);
/*
 * Make room for the token at position `length` of a sequence whose block
 * table is table[*table_len] (capacity entries available).  A position that
 * starts a block takes a new block (appended, *table_len + 1); a position in
 * a block that another table also references moves this table to a fresh
 * block and reports the copy in copy_pair[0] (source), copy_pair[1]
 * (destination), else both are -1.  *slot_out = block * block_size + offset.
 */
pa_status pa_bm_append_slot(pa_block_manager *bm, int32_t *table, int32_t *table_len, int32_t capacity,
                            int32_t length, int32_t *slot_out, int32_t *copy_pair);

/* Bytes of part_out plus part_lse for pa_decode_split (lse placed at a
 * 256-byte aligned offset after part_out).  0 on invalid sizes. */
size_t pa_split_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_num_partitions);

/* Static, NUL-terminated description of a status code. */
const char *pa_status_string(pa_status status);

/* hipError_t value behind the calling thread's last PA_ERR_HIP (0 if none). */
int32_t pa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
