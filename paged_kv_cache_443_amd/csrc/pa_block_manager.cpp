// Host block manager: reference counts of a physical block pool, on-demand
// allocation, fork and copy-on-write (page "LLM推理优化", section 3.2; page
// "字节跳动 AI Infra (2)", PagedAttention question, block-pool figure).
// Pure C++ (no HIP calls).  Free blocks are kept in a min-heap so that the
// lowest free id is handed out first.
#include <algorithm>
#include <cstdint>
#include <functional>
#include <new>
#include <queue>
#include <vector>

#include "pa.h"

struct pa_block_manager {
  int32_t block_size = 0;
  std::vector<int32_t> refs;  // references per block
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_ids;

  bool in_use(int32_t b) const { return b >= 0 && b < static_cast<int32_t>(refs.size()) && refs[b] > 0; }

  int32_t take() {
    const int32_t b = free_ids.top();
    free_ids.pop();
    refs[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--refs[b] == 0) free_ids.push(b);
  }
};

extern "C" {

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager **out) {
  if (out == nullptr) return PA_ERR_NULL_PTR;
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1) return PA_ERR_BAD_SHAPE;
  // slots (block * block_size + offset) are int32, as slot_mapping is
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX) return PA_ERR_BAD_SHAPE;
  pa_block_manager *bm = new (std::nothrow) pa_block_manager();
  if (bm == nullptr) return PA_ERR_OUT_OF_BLOCKS;
  try {
    bm->block_size = block_size;
    bm->refs.assign(static_cast<size_t>(num_blocks), 0);
    std::vector<int32_t> ids(static_cast<size_t>(num_blocks));
    for (int32_t b = 0; b < num_blocks; ++b) ids[b] = b;
    bm->free_ids = decltype(bm->free_ids)(std::greater<int32_t>(), std::move(ids));
  } catch (...) {
    delete bm;
    return PA_ERR_OUT_OF_BLOCKS;
  }
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager *bm) { delete bm; }

int32_t pa_bm_num_free(const pa_block_manager *bm) {
  return bm == nullptr ? 0 : static_cast<int32_t>(bm->free_ids.size());
}

int32_t pa_bm_refcount(const pa_block_manager *bm, int32_t block) {
  if (bm == nullptr || block < 0 || block >= static_cast<int32_t>(bm->refs.size())) return -1;
  return bm->refs[block];
}

pa_status pa_bm_allocate(pa_block_manager *bm, int32_t n, int32_t *ids_out) {
  if (bm == nullptr || (n > 0 && ids_out == nullptr)) return PA_ERR_NULL_PTR;
  if (n < 0) return PA_ERR_BAD_SHAPE;
  if (static_cast<size_t>(n) > bm->free_ids.size()) return PA_ERR_OUT_OF_BLOCKS;
  for (int32_t i = 0; i < n; ++i) ids_out[i] = bm->take();
  return PA_OK;
}

pa_status pa_bm_free(pa_block_manager *bm, const int32_t *ids, int32_t n) {
  if (bm == nullptr || (n > 0 && ids == nullptr)) return PA_ERR_NULL_PTR;
  if (n < 0) return PA_ERR_BAD_SHAPE;
  // validate first (a block listed k times needs k references) so that a
  // rejected call changes nothing
  std::vector<int32_t> sorted(ids, ids + n);
  std::sort(sorted.begin(), sorted.end());
  for (int32_t i = 0; i < n;) {
    int32_t j = i;
    while (j < n && sorted[j] == sorted[i]) ++j;
    if (!bm->in_use(sorted[i]) || bm->refs[sorted[i]] < j - i) return PA_ERR_INVALID_BLOCK;
    i = j;
  }
  for (int32_t i = 0; i < n; ++i) bm->drop(ids[i]);
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager *bm, const int32_t *table, int32_t n) {
  if (bm == nullptr || (n > 0 && table == nullptr)) return PA_ERR_NULL_PTR;
  if (n < 0) return PA_ERR_BAD_SHAPE;
  for (int32_t i = 0; i < n; ++i)
    if (!bm->in_use(table[i])) return PA_ERR_INVALID_BLOCK;
  for (int32_t i = 0; i < n; ++i) ++bm->refs[table[i]];
  return PA_OK;
}

pa_status pa_bm_append_slot(pa_block_manager *bm, int32_t *table, int32_t *table_len, int32_t capacity,
                            int32_t length, int32_t *slot_out, int32_t *copy_pair) {
  if (bm == nullptr || table_len == nullptr || slot_out == nullptr || copy_pair == nullptr) return PA_ERR_NULL_PTR;
  const int32_t n = *table_len;
  if (n > 0 && table == nullptr) return PA_ERR_NULL_PTR;
  if (length < 0 || n < 0 || capacity < n) return PA_ERR_BAD_SHAPE;
  const int32_t bs = bm->block_size;
  const int32_t j = length / bs;
  const int32_t off = length % bs;
  // the position must follow the table: inside its blocks, or the first slot of the next one
  if (j > n || (j == n && off != 0)) return PA_ERR_BAD_SHAPE;
  copy_pair[0] = copy_pair[1] = -1;
  if (j == n) {
    if (n >= capacity || table == nullptr) return PA_ERR_BAD_SHAPE;
    if (bm->free_ids.empty()) return PA_ERR_OUT_OF_BLOCKS;
    table[n] = bm->take();
    *table_len = n + 1;
  } else {
    const int32_t b = table[j];
    if (!bm->in_use(b)) return PA_ERR_INVALID_BLOCK;
    if (bm->refs[b] > 1) {
      if (bm->free_ids.empty()) return PA_ERR_OUT_OF_BLOCKS;
      const int32_t fresh = bm->take();
      --bm->refs[b];  // still referenced by the other tables
      table[j] = fresh;
      copy_pair[0] = b;
      copy_pair[1] = fresh;
    }
  }
  // in range: pa_bm_create bounds num_blocks * block_size by INT32_MAX
  *slot_out = static_cast<int32_t>(static_cast<int64_t>(table[j]) * bs + off);
  return PA_OK;
}

}  // extern "C"
