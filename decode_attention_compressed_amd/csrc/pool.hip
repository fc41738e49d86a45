// Page-pool packing: one device arena for the KV kinds of a layer stack, cut
// into size buckets of fixed-size pages (V4 page, section 3.1.3: a page is
// block size x compress ratio x bytes per element, and the pools of all KV
// kinds are packed into a few buckets by page size, each a pool of fixed-size
// pages; section 3.1.1: one 256-token logical block for every kind;
// vLLM-0.7.2 page, section 2.1: block tables map logical blocks to physical
// pages, which sequences that share a prefix share).
//
// Host-only bookkeeping (no device call): kinds with the same code and scale
// bytes per page share a bucket; a bucket's pages are allocated from a free
// stack, reference counted (a prefix page named by several block tables), and
// a full page can be published under a key so that a later sequence with the
// same prefix finds it; a released page that has a key stays cached until an
// allocation needs its memory (oldest released first).
#include <stdint.h>
#include <stdlib.h>

#include <iterator>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "hca.h"

namespace {

struct Bucket {
  size_t code_bytes = 0, scale_bytes = 0;  // per page
  size_t codes_off = 0, scales_off = 0;    // in the arena
  int32_t capacity = 0;
  std::vector<int32_t> free_stack;         // pages with no reference and no key
  std::vector<int32_t> refs;               // per page
  std::vector<uint64_t> key;               // per page (valid when has_key)
  std::vector<uint8_t> has_key;
  std::unordered_map<uint64_t, int32_t> by_key;
  std::list<int32_t> cached;               // released pages that keep a key, oldest first
  std::vector<std::list<int32_t>::iterator> cached_pos;
  std::vector<uint8_t> in_cache;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool kind_ok(const hca_kv_kind& k) {
  if (k.m < 1 || k.m > 256 || (256 % k.m) != 0 || k.dim < 1) return false;
  if (k.dtype == HCA_FP8_E4M3 || k.dtype == HCA_BF16) return true;
  return k.dtype == HCA_FP4_E2M1 && (k.dim % 32) == 0;
}

}  // namespace

struct hca_page_pool {
  std::vector<hca_kv_kind> kinds;
  std::vector<int32_t> kind_bucket;
  std::vector<Bucket> buckets;
  size_t arena_bytes = 0;
};

namespace {

// evict the oldest cached page of a bucket: its key is dropped and it is free
bool evict_one(Bucket& bk) {
  if (bk.cached.empty()) return false;
  const int32_t p = bk.cached.front();
  bk.cached.pop_front();
  bk.in_cache[p] = 0;
  bk.by_key.erase(bk.key[p]);
  bk.has_key[p] = 0;
  bk.free_stack.push_back(p);
  return true;
}

bool bucket_ok(const hca_page_pool* pool, int32_t bucket) {
  return pool != nullptr && bucket >= 0 && bucket < (int32_t)pool->buckets.size();
}

bool pages_ok(const Bucket& bk, const int32_t* pages, int32_t n) {
  if (n < 0 || (n > 0 && pages == nullptr)) return false;
  for (int32_t i = 0; i < n; ++i)
    if (pages[i] < 0 || pages[i] >= bk.capacity) return false;
  return true;
}

}  // namespace

extern "C" {

hca_status hca_page_bytes(hca_kv_kind kind, size_t* code_bytes, size_t* scale_bytes) {
  if (!kind_ok(kind) || code_bytes == nullptr || scale_bytes == nullptr) return HCA_ERR_INVALID;
  const size_t rows = 256 / (size_t)kind.m;
  switch (kind.dtype) {
    case HCA_FP8_E4M3: *code_bytes = rows * kind.dim; *scale_bytes = sizeof(float); break;
    case HCA_FP4_E2M1: *code_bytes = rows * (kind.dim / 2); *scale_bytes = rows * (kind.dim / 32); break;
    default: *code_bytes = rows * kind.dim * 2; *scale_bytes = 0; break;
  }
  return HCA_OK;
}

hca_status hca_pool_plan(const hca_kv_kind* kinds, int32_t n_kinds, int32_t* kind_bucket, int32_t* n_buckets) {
  if (n_kinds < 1 || kinds == nullptr || kind_bucket == nullptr || n_buckets == nullptr) return HCA_ERR_INVALID;
  std::vector<size_t> cb, sb;
  for (int32_t i = 0; i < n_kinds; ++i) {
    size_t c, s;
    if (hca_page_bytes(kinds[i], &c, &s) != HCA_OK) return HCA_ERR_INVALID;
    int32_t b = -1;
    for (size_t j = 0; j < cb.size(); ++j)
      if (cb[j] == c && sb[j] == s) b = (int32_t)j;
    if (b < 0) {
      b = (int32_t)cb.size();
      cb.push_back(c);
      sb.push_back(s);
    }
    kind_bucket[i] = b;
  }
  *n_buckets = (int32_t)cb.size();
  return HCA_OK;
}

hca_status hca_pool_create(const hca_kv_kind* kinds, int32_t n_kinds, const int32_t* capacity, size_t* arena_bytes,
                           hca_page_pool** out) {
  if (out == nullptr || arena_bytes == nullptr || capacity == nullptr) return HCA_ERR_INVALID;
  *out = nullptr;
  std::vector<int32_t> kb(n_kinds > 0 ? n_kinds : 1);
  int32_t nb = 0;
  const hca_status st = hca_pool_plan(kinds, n_kinds, kb.data(), &nb);
  if (st != HCA_OK) return st;
  for (int32_t b = 0; b < nb; ++b)
    if (capacity[b] < 0) return HCA_ERR_INVALID;
  hca_page_pool* p = new (std::nothrow) hca_page_pool;
  if (p == nullptr) return HCA_ERR_INVALID;
  p->kinds.assign(kinds, kinds + n_kinds);
  p->kind_bucket = kb;
  p->kind_bucket.resize(n_kinds);
  p->buckets.resize(nb);
  for (int32_t i = 0; i < n_kinds; ++i) {
    Bucket& bk = p->buckets[kb[i]];
    hca_page_bytes(kinds[i], &bk.code_bytes, &bk.scale_bytes);
  }
  size_t off = 0;
  for (int32_t b = 0; b < nb; ++b) {
    Bucket& bk = p->buckets[b];
    bk.capacity = capacity[b];
    bk.codes_off = off;
    off = align256(off + bk.code_bytes * (size_t)bk.capacity);
    bk.scales_off = off;
    off = align256(off + bk.scale_bytes * (size_t)bk.capacity);
    bk.refs.assign(bk.capacity, 0);
    bk.key.assign(bk.capacity, 0);
    bk.has_key.assign(bk.capacity, 0);
    bk.in_cache.assign(bk.capacity, 0);
    bk.cached_pos.resize(bk.capacity);
    bk.free_stack.reserve(bk.capacity);
    for (int32_t i = bk.capacity - 1; i >= 0; --i) bk.free_stack.push_back(i);  // page 0 first
  }
  p->arena_bytes = off;
  *arena_bytes = off;
  *out = p;
  return HCA_OK;
}

void hca_pool_destroy(hca_page_pool* pool) { delete pool; }

hca_status hca_pool_view(const hca_page_pool* pool, int32_t kind, void* arena, hca_paged_cache* out) {
  if (pool == nullptr || out == nullptr || kind < 0 || kind >= (int32_t)pool->kinds.size()) return HCA_ERR_INVALID;
  if (arena == nullptr || ((uintptr_t)arena % 256) != 0) return HCA_ERR_INVALID;
  const hca_kv_kind& k = pool->kinds[kind];
  const Bucket& bk = pool->buckets[pool->kind_bucket[kind]];
  uint8_t* base = static_cast<uint8_t*>(arena);
  out->codes = base + bk.codes_off;
  out->scales = bk.scale_bytes ? base + bk.scales_off : nullptr;
  out->num_pages = bk.capacity;
  out->epp = 256 / k.m;
  out->dim = k.dim;
  out->dtype = k.dtype;
  return HCA_OK;
}

int32_t hca_pool_bucket(const hca_page_pool* pool, int32_t kind) {
  if (pool == nullptr || kind < 0 || kind >= (int32_t)pool->kinds.size()) return -1;
  return pool->kind_bucket[kind];
}

hca_status hca_pool_alloc(hca_page_pool* pool, int32_t bucket, int32_t n, int32_t* pages) {
  if (!bucket_ok(pool, bucket) || n < 0 || (n > 0 && pages == nullptr)) return HCA_ERR_INVALID;
  Bucket& bk = pool->buckets[bucket];
  if ((size_t)n > bk.free_stack.size() + bk.cached.size()) return HCA_ERR_UNSUPPORTED;  // out of pages
  for (int32_t i = 0; i < n; ++i) {
    if (bk.free_stack.empty()) evict_one(bk);
    const int32_t p = bk.free_stack.back();
    bk.free_stack.pop_back();
    bk.refs[p] = 1;
    pages[i] = p;
  }
  return HCA_OK;
}

hca_status hca_pool_share(hca_page_pool* pool, int32_t bucket, const int32_t* pages, int32_t n) {
  if (!bucket_ok(pool, bucket)) return HCA_ERR_INVALID;
  Bucket& bk = pool->buckets[bucket];
  if (!pages_ok(bk, pages, n)) return HCA_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i)
    if (bk.refs[pages[i]] <= 0) return HCA_ERR_INVALID;  // only a held page can be shared
  for (int32_t i = 0; i < n; ++i) ++bk.refs[pages[i]];
  return HCA_OK;
}

hca_status hca_pool_release(hca_page_pool* pool, int32_t bucket, const int32_t* pages, int32_t n) {
  if (!bucket_ok(pool, bucket)) return HCA_ERR_INVALID;
  Bucket& bk = pool->buckets[bucket];
  if (!pages_ok(bk, pages, n)) return HCA_ERR_INVALID;
  {  // every release must drop a held reference (counting repeats in the list)
    std::unordered_map<int32_t, int32_t> cnt;
    for (int32_t i = 0; i < n; ++i)
      if (++cnt[pages[i]] > bk.refs[pages[i]]) return HCA_ERR_INVALID;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t p = pages[i];
    if (--bk.refs[p] > 0) continue;
    if (bk.has_key[p]) {
      bk.cached.push_back(p);
      bk.cached_pos[p] = std::prev(bk.cached.end());
      bk.in_cache[p] = 1;
    } else {
      bk.free_stack.push_back(p);
    }
  }
  return HCA_OK;
}

hca_status hca_pool_publish(hca_page_pool* pool, int32_t bucket, int32_t page, uint64_t key) {
  if (!bucket_ok(pool, bucket)) return HCA_ERR_INVALID;
  Bucket& bk = pool->buckets[bucket];
  if (page < 0 || page >= bk.capacity || bk.refs[page] <= 0) return HCA_ERR_INVALID;
  auto it = bk.by_key.find(key);
  if (it != bk.by_key.end() && it->second != page) return HCA_ERR_INVALID;  // the key names another page
  if (bk.has_key[page] && bk.key[page] != key) bk.by_key.erase(bk.key[page]);
  bk.key[page] = key;
  bk.has_key[page] = 1;
  bk.by_key[key] = page;
  return HCA_OK;
}

hca_status hca_pool_lookup(hca_page_pool* pool, int32_t bucket, uint64_t key, int32_t* page) {
  if (!bucket_ok(pool, bucket) || page == nullptr) return HCA_ERR_INVALID;
  Bucket& bk = pool->buckets[bucket];
  *page = -1;
  auto it = bk.by_key.find(key);
  if (it == bk.by_key.end()) return HCA_OK;
  const int32_t p = it->second;
  if (bk.in_cache[p]) {  // a released page comes back
    bk.cached.erase(bk.cached_pos[p]);
    bk.in_cache[p] = 0;
  }
  ++bk.refs[p];
  *page = p;
  return HCA_OK;
}

hca_status hca_pool_stats(const hca_page_pool* pool, int32_t bucket, int64_t* free_pages, int64_t* cached_pages,
                          int64_t* held_pages, size_t* codes_offset, size_t* scales_offset) {
  if (!bucket_ok(pool, bucket)) return HCA_ERR_INVALID;
  const Bucket& bk = pool->buckets[bucket];
  const int64_t fr = (int64_t)bk.free_stack.size(), ca = (int64_t)bk.cached.size();
  if (free_pages) *free_pages = fr;
  if (cached_pages) *cached_pages = ca;
  if (held_pages) *held_pages = bk.capacity - fr - ca;
  if (codes_offset) *codes_offset = bk.codes_off;
  if (scales_offset) *scales_offset = bk.scales_off;
  return HCA_OK;
}

}  // extern "C"
