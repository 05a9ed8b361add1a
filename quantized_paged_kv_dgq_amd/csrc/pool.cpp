// Host block pool: the block table's free list (PagedAttention article, "PagedAttention
// implementation": logical blocks map to physical blocks; blocks are allocated and released one
// block at a time from a free list).  Pure host code; no device work.
#include <cstdint>
#include <new>
#include <vector>

#include "dgq.h"

namespace {

struct Pool {
  std::vector<int32_t> free_list;  // stack: last freed is handed out first
  std::vector<uint8_t> is_free;    // 1 if the id is on the free list
};

}  // namespace

extern "C" dgq_status_t dgq_pool_create(int32_t num_blocks, void **pool) {
  if (pool == nullptr || num_blocks < 0) return DGQ_ERR_INVALID_ARG;
  *pool = nullptr;
  Pool *p = new (std::nothrow) Pool;
  if (p == nullptr) return DGQ_ERR_INVALID_ARG;
  try {
    p->free_list.resize((size_t)num_blocks);
    p->is_free.assign((size_t)num_blocks, 1);
  } catch (...) {
    delete p;
    return DGQ_ERR_INVALID_ARG;
  }
  // ids 0..n-1 are handed out in increasing order: the top of the stack is id 0
  for (int32_t i = 0; i < num_blocks; ++i) p->free_list[(size_t)i] = num_blocks - 1 - i;
  *pool = p;
  return DGQ_OK;
}

extern "C" dgq_status_t dgq_pool_destroy(void *pool) {
  delete static_cast<Pool *>(pool);
  return DGQ_OK;
}

extern "C" dgq_status_t dgq_block_alloc(void *pool, int32_t n, int32_t *ids) {
  Pool *p = static_cast<Pool *>(pool);
  if (p == nullptr || n < 0 || (n > 0 && ids == nullptr)) return DGQ_ERR_INVALID_ARG;
  if ((size_t)n > p->free_list.size()) return DGQ_ERR_POOL_EXHAUSTED;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = p->free_list.back();
    p->free_list.pop_back();
    p->is_free[(size_t)id] = 0;
    ids[i] = id;
  }
  return DGQ_OK;
}

extern "C" dgq_status_t dgq_block_free(void *pool, int32_t n, const int32_t *ids) {
  Pool *p = static_cast<Pool *>(pool);
  if (p == nullptr || n < 0 || (n > 0 && ids == nullptr)) return DGQ_ERR_INVALID_ARG;
  const size_t cap = p->is_free.size();
  // validate everything first so that a bad list leaves the pool unchanged
  std::vector<uint8_t> seen;
  try {
    seen.assign(cap, 0);
  } catch (...) {
    return DGQ_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || (size_t)id >= cap || p->is_free[(size_t)id] || seen[(size_t)id]) return DGQ_ERR_INVALID_ARG;
    seen[(size_t)id] = 1;
  }
  for (int32_t i = 0; i < n; ++i) {
    p->free_list.push_back(ids[i]);
    p->is_free[(size_t)ids[i]] = 1;
  }
  return DGQ_OK;
}

extern "C" int32_t dgq_pool_num_free(const void *pool) {
  const Pool *p = static_cast<const Pool *>(pool);
  return p == nullptr ? -1 : (int32_t)p->free_list.size();
}
