// Host bookkeeping of a paged KV cache with zero-copy forks ("HPD-Parsing:
// Hierarchical Parallel Document Parsing" notes, prerequisites "KV cache and
// shared-prefix reuse" and Algorithm 1: a branch forked at a <FORK> shares
// its parent's KV blocks through a pointer, and KV is released by reference
// count when branches finish).  The device memory is the caller's cache of
// n_blocks x block_size token rows; the pool only decides which rows hold
// which sequence's tokens.
//
// A sequence is a root (its own tokens) or a fork: a read-only view of the
// first n tokens of a root's blocks, plus tokens of its own.  In the decode
// plan a fork's row reads the root's table up to its bound (segment A) and its
// own table (segment B), so a partially filled shared block is never written
// by the fork and needs no copy.
#include <algorithm>
#include <memory>
#include <climits>
#include <set>
#include <vector>

#include "ta_internal.h"

using namespace ta;

struct ta_kv_pool {
  struct Seq {
    bool live = false, root = false;
    std::vector<int32_t> view, own;
    int64_t view_len = 0, own_len = 0;
  };
  int32_t n_blocks = 0, block_size = 0;
  std::vector<int32_t> ref;
  std::set<int32_t> free_set;  // lowest id first
  std::vector<Seq> seqs;       // ids are indices, never reused

  Seq* get(int32_t id) {
    if (id < 0 || size_t(id) >= seqs.size() || !seqs[id].live) return nullptr;
    return &seqs[id];
  }
};

extern "C" int tree_attn_pool_create(int32_t n_blocks, int32_t block_size, ta_kv_pool** out) try {
  if (!out) return fail(TA_ERR_INVALID_ARG, "pool_create: out is NULL");
  if (n_blocks < 0 || block_size < 1) return fail(TA_ERR_INVALID_ARG, "pool_create: bad size");
  if (int64_t(n_blocks) * block_size >= INT32_MAX) return fail(TA_ERR_CAPACITY, "pool_create: token rows >= 2^31");
  std::unique_ptr<ta_kv_pool> owner(new ta_kv_pool());
  ta_kv_pool* p = owner.get();
  p->n_blocks = n_blocks;
  p->block_size = block_size;
  p->ref.assign(size_t(n_blocks), 0);
  for (int32_t b = 0; b < n_blocks; ++b) p->free_set.insert(p->free_set.end(), b);
  *out = owner.release();
  return TA_OK;
} catch (...) {
  return ta::fail_exception("pool_create");
}

extern "C" void tree_attn_pool_destroy(ta_kv_pool* pool) { delete pool; }

extern "C" int tree_attn_pool_new_seq(ta_kv_pool* pool, int32_t* seq) try {
  if (!pool || !seq) return fail(TA_ERR_INVALID_ARG, "pool_new_seq: NULL argument");
  if (pool->seqs.size() >= size_t(INT32_MAX)) return fail(TA_ERR_CAPACITY, "pool_new_seq: sequence ids exhausted");
  ta_kv_pool::Seq s;
  s.live = true;
  s.root = true;
  pool->seqs.push_back(std::move(s));
  *seq = int32_t(pool->seqs.size() - 1);
  return TA_OK;
} catch (...) {
  return ta::fail_exception("pool_new_seq");
}

extern "C" int tree_attn_pool_fork(ta_kv_pool* pool, int32_t parent, int32_t n_tokens, int32_t* child) try {
  if (!pool || !child) return fail(TA_ERR_INVALID_ARG, "pool_fork: NULL argument");
  const ta_kv_pool::Seq* p = pool->get(parent);
  if (!p || !p->root) return fail(TA_ERR_INVALID_ARG, "pool_fork: the parent must be a live root sequence");
  if (n_tokens < 0 || n_tokens > p->own_len) return fail(TA_ERR_INVALID_ARG, "pool_fork: fork point outside the parent");
  if (pool->seqs.size() >= size_t(INT32_MAX)) return fail(TA_ERR_CAPACITY, "pool_fork: sequence ids exhausted");
  ta_kv_pool::Seq s;
  s.live = true;
  s.root = false;
  const int64_t nb = (int64_t(n_tokens) + pool->block_size - 1) / pool->block_size;
  s.view.assign(p->own.begin(), p->own.begin() + nb);
  s.view_len = n_tokens;
  for (int32_t b : s.view) ++pool->ref[b];
  pool->seqs.push_back(std::move(s));
  *child = int32_t(pool->seqs.size() - 1);
  return TA_OK;
} catch (...) {
  return ta::fail_exception("pool_fork");
}

extern "C" int tree_attn_pool_append(ta_kv_pool* pool, int32_t seq, int32_t n_tokens, int64_t* slots) try {
  if (!pool) return fail(TA_ERR_INVALID_ARG, "pool_append: pool is NULL");
  ta_kv_pool::Seq* s = pool->get(seq);
  if (!s) return fail(TA_ERR_INVALID_ARG, "pool_append: unknown sequence");
  if (n_tokens < 0) return fail(TA_ERR_INVALID_ARG, "pool_append: negative count");
  if (n_tokens > 0 && !slots) return fail(TA_ERR_INVALID_ARG, "pool_append: slots is NULL");
  const int64_t bs = pool->block_size;
  const int64_t new_len = s->own_len + n_tokens;
  if (new_len >= INT32_MAX) return fail(TA_ERR_CAPACITY, "pool_append: sequence longer than 2^31");
  const int64_t need = (new_len + bs - 1) / bs - int64_t(s->own.size());
  if (need > int64_t(pool->free_set.size())) return fail(TA_ERR_CAPACITY, "pool_append: out of free blocks");
  for (int64_t i = 0; i < need; ++i) {
    const int32_t b = *pool->free_set.begin();
    pool->free_set.erase(pool->free_set.begin());
    pool->ref[b] = 1;
    s->own.push_back(b);
  }
  for (int64_t t = s->own_len; t < new_len; ++t) slots[t - s->own_len] = int64_t(s->own[t / bs]) * bs + t % bs;
  s->own_len = new_len;
  return TA_OK;
} catch (...) {
  return ta::fail_exception("pool_append");
}

extern "C" int tree_attn_pool_release(ta_kv_pool* pool, int32_t seq) try {
  if (!pool) return fail(TA_ERR_INVALID_ARG, "pool_release: pool is NULL");
  ta_kv_pool::Seq* s = pool->get(seq);
  if (!s) return fail(TA_ERR_INVALID_ARG, "pool_release: unknown sequence");
  for (const std::vector<int32_t>* list : {&s->view, &s->own})
    for (int32_t b : *list)
      if (--pool->ref[b] == 0) pool->free_set.insert(b);
  s->live = false;
  s->view.clear();
  s->own.clear();
  s->view.shrink_to_fit();
  s->own.shrink_to_fit();
  return TA_OK;
} catch (...) {
  return ta::fail_exception("pool_release");
}

extern "C" int tree_attn_pool_table(const ta_kv_pool* pool, int32_t seq, int32_t* view, int32_t view_cap,
                                    int32_t* view_tokens, int32_t* own, int32_t own_cap, int32_t* own_tokens) try {
  if (!pool || !view_tokens || !own_tokens) return fail(TA_ERR_INVALID_ARG, "pool_table: NULL argument");
  if (seq < 0 || size_t(seq) >= pool->seqs.size() || !pool->seqs[seq].live)
    return fail(TA_ERR_INVALID_ARG, "pool_table: unknown sequence");
  const ta_kv_pool::Seq& s = pool->seqs[seq];
  *view_tokens = int32_t(s.view_len);
  *own_tokens = int32_t(s.own_len);
  if (int64_t(s.view.size()) > view_cap || int64_t(s.own.size()) > own_cap)
    return fail(TA_ERR_WORKSPACE, "pool_table: table larger than the given capacity");
  if ((!s.view.empty() && !view) || (!s.own.empty() && !own)) return fail(TA_ERR_INVALID_ARG, "pool_table: NULL table");
  std::copy(s.view.begin(), s.view.end(), view);
  std::copy(s.own.begin(), s.own.end(), own);
  return TA_OK;
} catch (...) {
  return ta::fail_exception("pool_table");
}

extern "C" int tree_attn_pool_refs(const ta_kv_pool* pool, int32_t* refs, int32_t cap, int32_t* free_blocks) try {
  if (!pool || !free_blocks) return fail(TA_ERR_INVALID_ARG, "pool_refs: NULL argument");
  *free_blocks = int32_t(pool->free_set.size());
  if (refs) {
    if (cap < pool->n_blocks) return fail(TA_ERR_WORKSPACE, "pool_refs: cap < n_blocks");
    std::copy(pool->ref.begin(), pool->ref.end(), refs);
  }
  return TA_OK;
} catch (...) {
  return ta::fail_exception("pool_refs");
}
