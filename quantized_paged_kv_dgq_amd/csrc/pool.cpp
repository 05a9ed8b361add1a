// Host block pool: the block table's free list (PagedAttention article, "PagedAttention
// implementation": logical blocks map to physical blocks; blocks are allocated and released one
// block at a time from a free list), with a reference count per block (Quantization article,
// section 3.2: a page-table entry carries a reference count so that several owners share one
// physical page).  Pure host code; no device work.
#include <cstdint>
#include <new>
#include <unordered_map>
#include <vector>

#include "dgq.h"

namespace {

struct Pool {
  std::vector<int32_t> free_list;  // stack: last freed is handed out first
  std::vector<int32_t> refs;       // 0 = on the free list
};

constexpr int32_t kMaxRefs = 1 << 30;

// Occurrences of each id in a host list, or false if an id is out of range.
bool count_ids(const Pool *p, int32_t n, const int32_t *ids, std::unordered_map<int32_t, int64_t> &cnt) {
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || (size_t)id >= p->refs.size()) return false;
    ++cnt[id];
  }
  return true;
}

}  // namespace

extern "C" dgq_status_t dgq_pool_create(int32_t num_blocks, void **pool) {
  if (pool == nullptr || num_blocks < 0) return DGQ_ERR_INVALID_ARG;
  *pool = nullptr;
  Pool *p = new (std::nothrow) Pool;
  if (p == nullptr) return DGQ_ERR_INVALID_ARG;
  try {
    p->free_list.resize((size_t)num_blocks);
    p->refs.assign((size_t)num_blocks, 0);
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
    p->refs[(size_t)id] = 1;
    ids[i] = id;
  }
  return DGQ_OK;
}

extern "C" dgq_status_t dgq_block_free(void *pool, int32_t n, const int32_t *ids) {
  Pool *p = static_cast<Pool *>(pool);
  if (p == nullptr || n < 0 || (n > 0 && ids == nullptr)) return DGQ_ERR_INVALID_ARG;
  // validate everything first so that a bad list leaves the pool unchanged
  std::unordered_map<int32_t, int64_t> cnt;
  try {
    if (!count_ids(p, n, ids, cnt)) return DGQ_ERR_INVALID_ARG;
  } catch (...) {
    return DGQ_ERR_INVALID_ARG;
  }
  for (const auto &kv : cnt)
    if (kv.second > p->refs[(size_t)kv.first]) return DGQ_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    int32_t &r = p->refs[(size_t)ids[i]];
    if (--r == 0) p->free_list.push_back(ids[i]);
  }
  return DGQ_OK;
}

extern "C" dgq_status_t dgq_block_share(void *pool, int32_t n, const int32_t *ids) {
  Pool *p = static_cast<Pool *>(pool);
  if (p == nullptr || n < 0 || (n > 0 && ids == nullptr)) return DGQ_ERR_INVALID_ARG;
  std::unordered_map<int32_t, int64_t> cnt;
  try {
    if (!count_ids(p, n, ids, cnt)) return DGQ_ERR_INVALID_ARG;
  } catch (...) {
    return DGQ_ERR_INVALID_ARG;
  }
  for (const auto &kv : cnt) {
    const int64_t r = p->refs[(size_t)kv.first];
    if (r == 0 || r + kv.second > kMaxRefs) return DGQ_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) ++p->refs[(size_t)ids[i]];
  return DGQ_OK;
}

extern "C" dgq_status_t dgq_block_cow(void *pool, int32_t n, const int32_t *ids, int32_t *out_ids) {
  Pool *p = static_cast<Pool *>(pool);
  if (p == nullptr || n < 0 || (n > 0 && (ids == nullptr || out_ids == nullptr))) return DGQ_ERR_INVALID_ARG;
  // Entries are served in order.  rem[id] = references of id not yet served: an entry that finds
  // more than one takes a fresh block and drops one; an entry that finds exactly one keeps the
  // block (rem becomes 0); an entry that finds none (a free block, or one already kept by an
  // earlier entry) is an error.  A dry run validates everything before the pool changes.
  std::unordered_map<int32_t, int64_t> rem;
  int64_t fresh = 0;
  try {
    for (int32_t i = 0; i < n; ++i) {
      const int32_t id = ids[i];
      if (id < 0 || (size_t)id >= p->refs.size()) return DGQ_ERR_INVALID_ARG;
      auto it = rem.find(id);
      if (it == rem.end()) it = rem.emplace(id, p->refs[(size_t)id]).first;
      if (it->second == 0) return DGQ_ERR_INVALID_ARG;
      if (it->second > 1) {
        --it->second;
        ++fresh;
      } else {
        it->second = 0;
      }
    }
  } catch (...) {
    return DGQ_ERR_INVALID_ARG;
  }
  if ((size_t)fresh > p->free_list.size()) return DGQ_ERR_POOL_EXHAUSTED;
  rem.clear();
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    auto it = rem.find(id);
    if (it == rem.end()) it = rem.emplace(id, p->refs[(size_t)id]).first;
    if (it->second > 1) {
      --it->second;
      --p->refs[(size_t)id];
      const int32_t nid = p->free_list.back();
      p->free_list.pop_back();
      p->refs[(size_t)nid] = 1;
      out_ids[i] = nid;
    } else {
      it->second = 0;
      out_ids[i] = id;
    }
  }
  return DGQ_OK;
}

extern "C" int32_t dgq_block_refcount(const void *pool, int32_t id) {
  const Pool *p = static_cast<const Pool *>(pool);
  if (p == nullptr || id < 0 || (size_t)id >= p->refs.size()) return -1;
  return p->refs[(size_t)id];
}

extern "C" int32_t dgq_pool_num_free(const void *pool) {
  const Pool *p = static_cast<const Pool *>(pool);
  return p == nullptr ? -1 : (int32_t)p->free_list.size();
}
