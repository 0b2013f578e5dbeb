// Host block pool: LIFO free list, reference counts, per-sequence block
// tables, fork and copy-on-write.
//
// Follows "19.2 KV Cache 系统化管理" §19.2.3 (PhysicalBlockPool: the free list
// is taken from its end and a freshly allocated block gets count 1; release
// lowers the count and returns the block to the end of the list at 0;
// BlockTable: token n goes to logical block n / block_size, slot
// n % block_size, and a block is allocated when the logical block is not yet
// mapped; release_all frees the blocks in logical order) and §19.2.2 of the
// same page with §4 of "LLM 推理引擎的内存管理与调度" (sharing by reference
// count; the first write into a shared, partly filled block copies it to a
// new block, remaps the table and lowers the old count).
//
// Prefix cache ("LLM 推理引擎的内存管理与调度" §5.1-5.2; "19.2 KV Cache
// 系统化管理" §19.2.5): full blocks can be published under a chained key
// h_i = H(h_{i-1}, tokens_i, salt) (pa_prefix_hash: 64-bit FNV-1a); a new
// request maps the longest chain of published keys into its table, one more
// reference per hit; a published block whose count drops to zero becomes
// evictable instead of free, and allocation reclaims the least recently
// released evictable block once the free list is empty.
//
// All operations are O(1) per token or block and all-or-nothing: every
// failure is detected before the pool is touched.

#include <cstdint>
#include <cstring>
#include <list>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"
#include "pa_error.h"

struct pa_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_list;   // top of the stack is the back
  std::vector<int32_t> refcount;
  struct Seq {
    std::vector<int32_t> blocks;    // logical -> physical
    int64_t filled = 0;             // tokens written so far
  };
  std::unordered_map<int32_t, Seq> seqs;
  int32_t next_seq = 0;
  // prefix cache: key -> block; per block its key; evictable blocks, oldest first
  std::unordered_map<uint64_t, int32_t> cached;
  std::vector<uint64_t> key_of;
  std::vector<char> has_key;
  std::list<int32_t> evictable;
  std::vector<std::list<int32_t>::iterator> evict_pos;

  int64_t available() const { return (int64_t)free_list.size() + (int64_t)evictable.size(); }

  // Caller checked available() > 0.
  int32_t take() {
    int32_t b;
    if (!free_list.empty()) {
      b = free_list.back();
      free_list.pop_back();
    } else {  // reclaim the least recently released cached block
      b = evictable.front();
      evictable.pop_front();
      cached.erase(key_of[b]);
      has_key[b] = 0;
    }
    refcount[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--refcount[b] > 0) return;
    if (has_key[b]) {
      evictable.push_back(b);
      evict_pos[b] = std::prev(evictable.end());
    } else {
      free_list.push_back(b);
    }
  }
  // Blocks an append of n tokens would take (copy-on-write + new blocks).
  int64_t needed(const Seq& s, int64_t n) const {
    if (n <= 0) return 0;
    int64_t need = 0;
    const int64_t first = s.filled / block_size;
    if (first < (int64_t)s.blocks.size() && refcount[s.blocks[first]] > 1) need += 1;
    const int64_t last = (s.filled + n - 1) / block_size;
    const int64_t have = (int64_t)s.blocks.size();
    if (last + 1 > have) need += last + 1 - have;
    return need;
  }
};

namespace {

pa_pool::Seq* find(pa_pool* p, int32_t seq) {
  auto it = p->seqs.find(seq);
  return it == p->seqs.end() ? nullptr : &it->second;
}
const pa_pool::Seq* find(const pa_pool* p, int32_t seq) {
  auto it = p->seqs.find(seq);
  return it == p->seqs.end() ? nullptr : &it->second;
}

}  // namespace

extern "C" {

pa_status pa_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free,
                         pa_pool** out) {
  if (!out) return pa::fail(PA_ERR_INVALID_ARG, "pa_pool_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_pool_create: num_blocks and block_size must be > 0");
  pa_pool* p = new (std::nothrow) pa_pool();
  if (!p) return pa::fail(PA_ERR_INVALID_ARG, "pa_pool_create: out of host memory");
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->refcount.assign(num_blocks, 0);
  p->key_of.assign(num_blocks, 0);
  p->has_key.assign(num_blocks, 0);
  p->evict_pos.resize(num_blocks);
  p->free_list.resize(num_blocks);
  if (initial_free) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = initial_free[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        return pa::fail(PA_ERR_INVALID_ARG,
                        "pa_pool_create: initial_free is not a permutation of the block ids");
      }
      seen[b] = 1;
      p->free_list[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) p->free_list[i] = i;
  }
  *out = p;
  return PA_OK;
}

void pa_pool_destroy(pa_pool* pool) { delete pool; }

int32_t pa_pool_num_free(const pa_pool* pool) {
  return pool ? (int32_t)pool->available() : -1;
}

int32_t pa_pool_refcount(const pa_pool* pool, int32_t block) {
  if (!pool || block < 0 || block >= pool->num_blocks) return -1;
  return pool->refcount[block];
}

pa_status pa_pool_free_list(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n) {
  if (!pool || !n || (cap > 0 && !out))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_pool_free_list: NULL argument");
  const int32_t size = (int32_t)pool->free_list.size();
  if (cap < size) return pa::fail(PA_ERR_INVALID_ARG, "pa_pool_free_list: cap too small");
  if (size) std::memcpy(out, pool->free_list.data(), sizeof(int32_t) * size);
  *n = size;
  return PA_OK;
}

pa_status pa_seq_new(pa_pool* pool, int32_t* seq) {
  if (!pool || !seq) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_new: NULL argument");
  const int32_t id = pool->next_seq++;
  pool->seqs.emplace(id, pa_pool::Seq{});
  *seq = id;
  return PA_OK;
}

pa_status pa_seq_fork(pa_pool* pool, int32_t parent, int32_t* child) {
  if (!pool || !child) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_fork: NULL argument");
  const pa_pool::Seq* s = find(pool, parent);
  if (!s) return pa::fail(PA_ERR_NOT_FOUND, "pa_seq_fork: unknown parent sequence");
  pa_pool::Seq copy = *s;
  for (int32_t b : copy.blocks) pool->refcount[b] += 1;
  const int32_t id = pool->next_seq++;
  pool->seqs.emplace(id, std::move(copy));
  *child = id;
  return PA_OK;
}

pa_status pa_seq_blocks_needed(const pa_pool* pool, int32_t seq, int32_t n_tokens,
                               int32_t* needed) {
  if (!pool || !needed) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_blocks_needed: NULL");
  if (n_tokens < 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_blocks_needed: n_tokens < 0");
  const pa_pool::Seq* s = find(pool, seq);
  if (!s) return pa::fail(PA_ERR_NOT_FOUND, "pa_seq_blocks_needed: unknown sequence");
  *needed = (int32_t)pool->needed(*s, n_tokens);
  return PA_OK;
}

pa_status pa_seq_append(pa_pool* pool, int32_t seq, int32_t n_tokens, int32_t* slot_mapping_out,
                        int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow) {
  if (!pool || !n_cow) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append: NULL argument");
  if (n_tokens < 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append: n_tokens < 0");
  if (n_tokens > 0 && !slot_mapping_out)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append: slot_mapping_out is NULL");
  pa_pool::Seq* s = find(pool, seq);
  if (!s) return pa::fail(PA_ERR_NOT_FOUND, "pa_seq_append: unknown sequence");
  const int64_t bs = pool->block_size;
  if ((s->filled + n_tokens + bs - 1) / bs * bs > (int64_t)INT32_MAX ||
      (int64_t)pool->num_blocks * bs > (int64_t)INT32_MAX + 1)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append: slot index would overflow int32");
  const int64_t need = pool->needed(*s, n_tokens);
  if (need > pool->available())
    return pa::fail(PA_ERR_NO_FREE_BLOCKS, "pa_seq_append: not enough free blocks");
  // At most the first token can land in a shared block (later ones see a
  // private block), so one pair of room is enough.
  const int64_t first = s->filled / bs;
  const bool cow = n_tokens > 0 && first < (int64_t)s->blocks.size() &&
                   pool->refcount[s->blocks[first]] > 1;
  if (cow && (cow_cap < 1 || !cow_pairs_out))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append: no room for the copy-on-write pair");

  *n_cow = 0;
  if (cow) {
    const int32_t old = s->blocks[first];
    const int32_t fresh = pool->take();
    cow_pairs_out[0] = old;
    cow_pairs_out[1] = fresh;
    *n_cow = 1;
    pool->drop(old);
    s->blocks[first] = fresh;
  }
  int64_t pos = s->filled;
  for (int32_t t = 0; t < n_tokens; ++t, ++pos) {
    const int64_t logical = pos / bs;
    if (logical == (int64_t)s->blocks.size()) s->blocks.push_back(pool->take());
    slot_mapping_out[t] = (int32_t)(s->blocks[logical] * bs + pos % bs);
  }
  s->filled = pos;
  return PA_OK;
}

pa_status pa_seq_release(pa_pool* pool, int32_t seq) {
  if (!pool) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_release: pool is NULL");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return pa::fail(PA_ERR_NOT_FOUND, "pa_seq_release: unknown sequence");
  for (int32_t b : it->second.blocks) pool->drop(b);
  pool->seqs.erase(it);
  return PA_OK;
}

uint64_t pa_prefix_hash(uint64_t parent, const int32_t* tokens, int32_t n, uint64_t salt) {
  // 64-bit FNV-1a over parent (8 bytes LE), salt (8 bytes LE), token ids (4 bytes LE)
  uint64_t h = 0xCBF29CE484222325ull;
  auto eat = [&](uint64_t v, int bytes) {
    for (int i = 0; i < bytes; ++i) {
      h ^= (v >> (8 * i)) & 0xFFu;
      h *= 0x100000001B3ull;
    }
  };
  eat(parent, 8);
  eat(salt, 8);
  for (int32_t i = 0; tokens && i < n; ++i) eat((uint32_t)tokens[i], 4);
  return h;
}

pa_status pa_seq_match_prefix(pa_pool* pool, int32_t seq, const uint64_t* keys, int32_t n,
                              int32_t* n_hit) {
  if (!pool || !n_hit || (n > 0 && !keys))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_match_prefix: NULL argument");
  if (n < 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_match_prefix: n < 0");
  pa_pool::Seq* s = find(pool, seq);
  if (!s) return pa::fail(PA_ERR_NOT_FOUND, "pa_seq_match_prefix: unknown sequence");
  if (s->filled != 0 || !s->blocks.empty())
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_match_prefix: the sequence is not empty");
  if ((int64_t)n * pool->block_size > (int64_t)INT32_MAX)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_match_prefix: too many blocks");
  int32_t hits = 0;
  for (; hits < n; ++hits) {
    auto it = pool->cached.find(keys[hits]);
    if (it == pool->cached.end()) break;
    const int32_t b = it->second;
    if (pool->refcount[b] == 0) pool->evictable.erase(pool->evict_pos[b]);
    pool->refcount[b] += 1;
    s->blocks.push_back(b);
  }
  s->filled = (int64_t)hits * pool->block_size;
  *n_hit = hits;
  return PA_OK;
}

pa_status pa_seq_register_prefix(pa_pool* pool, int32_t seq, const uint64_t* keys, int32_t n) {
  if (!pool || (n > 0 && !keys))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_register_prefix: NULL argument");
  if (n < 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_register_prefix: n < 0");
  pa_pool::Seq* s = find(pool, seq);
  if (!s) return pa::fail(PA_ERR_NOT_FOUND, "pa_seq_register_prefix: unknown sequence");
  if (n > s->filled / pool->block_size)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_register_prefix: only full blocks can be registered");
  for (int32_t i = 0; i < n; ++i) {  // check first: all-or-nothing
    const int32_t b = s->blocks[i];
    if (pool->has_key[b] && pool->key_of[b] != keys[i])
      return pa::fail(PA_ERR_INVALID_ARG,
                      "pa_seq_register_prefix: block %d is already cached under another key", b);
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = s->blocks[i];
    if (pool->has_key[b] || pool->cached.count(keys[i])) continue;  // first holder stays
    pool->cached.emplace(keys[i], b);
    pool->key_of[b] = keys[i];
    pool->has_key[b] = 1;
  }
  return PA_OK;
}

pa_status pa_seq_len(const pa_pool* pool, int32_t seq, int32_t* len) {
  if (!pool || !len) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_len: NULL argument");
  const pa_pool::Seq* s = find(pool, seq);
  if (!s) return pa::fail(PA_ERR_NOT_FOUND, "pa_seq_len: unknown sequence");
  *len = (int32_t)s->filled;
  return PA_OK;
}

pa_status pa_block_tables(const pa_pool* pool, const int32_t* seqs, int32_t n, int32_t max_blocks,
                          int32_t fill, int32_t* out) {
  if (!pool || (n > 0 && (!seqs || !out)))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_block_tables: NULL argument");
  if (n < 0 || max_blocks < 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_block_tables: negative size");
  for (int32_t i = 0; i < n; ++i) {
    const pa_pool::Seq* s = find(pool, seqs[i]);
    if (!s) return pa::fail(PA_ERR_NOT_FOUND, "pa_block_tables: unknown sequence");
    if ((int64_t)s->blocks.size() > max_blocks)
      return pa::fail(PA_ERR_INVALID_ARG, "pa_block_tables: a sequence has more than max_blocks blocks");
  }
  for (int32_t i = 0; i < n; ++i) {
    const pa_pool::Seq* s = find(pool, seqs[i]);
    int32_t* row = out + (int64_t)i * max_blocks;
    const int32_t used = (int32_t)s->blocks.size();
    for (int32_t k = 0; k < used; ++k) row[k] = s->blocks[k];
    for (int32_t k = used; k < max_blocks; ++k) row[k] = fill;
  }
  return PA_OK;
}

}  // extern "C"
