// Host block allocator: FIFO free queue of block ids plus reference counts,
// the sequence-level operations built on it (fork, reserve with
// copy-on-write, release), and an optional block-level prefix cache.  Pure
// C++17, no GPU calls.
//
// The free queue is a ring buffer over all num_blocks ids: allocation pops the
// head and a block whose count reaches zero is pushed at the tail
// (hnwysp.cn/news/103996 §3.4), both O(1) — no scan of the pool, the point of
// the "watermark" tip in m.lqnn.cn/news/240480 §5.2.  Every public call checks
// its arguments before it changes anything, so a failed call leaves the
// allocator as it was.
#include <algorithm>
#include <array>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "sha256.h"
#include "status.h"

namespace {

using Key = std::array<uint8_t, 32>;

struct KeyHash {
  size_t operator()(const Key& k) const {
    uint64_t v;
    std::memcpy(&v, k.data(), sizeof v);  // a SHA-256 digest is already uniformly spread
    return static_cast<size_t>(v);
  }
};

// Chained block keys: key_i = SHA-256(key_{i-1} || tokens of block i as
// little-endian int32), key_{-1} = 32 zero bytes.  A key therefore names the
// whole token prefix ending with its block (keys extend block by block,
// icman.com.cn/news/78786 §4.4; SHA-256 as the collision-resistant hash of
// §3.2).
void next_key(const Key& prev, const int32_t* tokens, int32_t block_size, Key* out) {
  pkv::Sha256 h;
  h.update(prev.data(), prev.size());
  uint8_t le[256];   // tokens as little-endian bytes, 64 at a time
  for (int32_t i0 = 0; i0 < block_size; i0 += 64) {
    const int32_t n = std::min(64, block_size - i0);
    for (int32_t i = 0; i < n; ++i) {
      const uint32_t t = static_cast<uint32_t>(tokens[i0 + i]);
      le[4 * i] = static_cast<uint8_t>(t);
      le[4 * i + 1] = static_cast<uint8_t>(t >> 8);
      le[4 * i + 2] = static_cast<uint8_t>(t >> 16);
      le[4 * i + 3] = static_cast<uint8_t>(t >> 24);
    }
    h.update(le, 4 * static_cast<size_t>(n));
  }
  h.finish(out->data());
}

}  // namespace

struct pkv_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ring;  // free queue storage, capacity num_blocks
  int32_t head = 0;           // index of the queue head in `ring`
  int32_t count = 0;          // number of free blocks
  std::vector<int32_t> ref;   // reference count per block (0 = free or cached-evictable)

  // Prefix cache (off until enabled).  A cached block holds the key of the
  // token prefix ending with it; when its count falls to zero it joins an LRU
  // list (doubly linked through lru_prev / lru_next) instead of the free
  // queue, and stays matchable until the free queue is empty and it is the
  // least recently released.
  // Duplicate detection for rows handed to release and fork: stamp[b] ==
  // epoch marks an id already seen in the row being checked (one linear
  // pass; a new epoch per check, the stamps cleared when it wraps).
  mutable std::vector<uint32_t> stamp;
  mutable uint32_t epoch = 0;

  bool cache_on = false;
  std::vector<Key> key_of;
  std::vector<uint8_t> cached;
  std::unordered_map<Key, int32_t, KeyHash> index;
  std::vector<int32_t> lru_prev, lru_next;
  int32_t lru_head = -1, lru_tail = -1, n_lru = 0, n_cached = 0;

  // Blocks a reservation may take: the free queue, then evictable cached blocks.
  int32_t available() const { return count + n_lru; }

  void lru_unlink(int32_t b) {
    const int32_t p = lru_prev[b], n = lru_next[b];
    if (p >= 0) lru_next[p] = n; else lru_head = n;
    if (n >= 0) lru_prev[n] = p; else lru_tail = p;
    --n_lru;
  }
  void lru_append(int32_t b) {
    lru_prev[b] = lru_tail;
    lru_next[b] = -1;
    if (lru_tail >= 0) lru_next[lru_tail] = b; else lru_head = b;
    lru_tail = b;
    ++n_lru;
  }

  // Takes one block (callers check available() first): the free queue's head,
  // or else the least recently released cached block, whose key is dropped.
  int32_t pop() {
    int32_t b;
    if (count > 0) {
      b = ring[head];
      head = (head + 1 == num_blocks) ? 0 : head + 1;
      --count;
    } else {
      b = lru_head;
      lru_unlink(b);
      index.erase(key_of[b]);
      cached[b] = 0;
      --n_cached;
    }
    ref[b] = 1;
    return b;
  }
  // A block whose count reached zero: cached blocks wait in the LRU list,
  // others return to the tail of the free queue.
  void release_zero(int32_t b) {
    if (cache_on && cached[b]) lru_append(b); else push(b);
  }
  void push(int32_t b) {
    int32_t tail = head + count;
    if (tail >= num_blocks) tail -= num_blocks;
    ring[tail] = b;
    ++count;
  }
  bool in_range(int32_t b) const { return b >= 0 && b < num_blocks; }
};

namespace {

int32_t ceil_div(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }

// Checks that every id of a row is in range and referenced.  With
// `count_duplicates`, also that each block has at least as many references as
// the row holds it, so releasing the row cannot underflow a count (rows made
// by the allocator never repeat an id; only release and fork need the check).
int check_row(const pkv_allocator* a, const int32_t* row, int32_t n, const char* what, bool count_duplicates) {
  if (n < 0) return pkv::fail(PKV_ERR_INVALID, "%s: negative block count %d", what, n);
  if (n > 0 && row == nullptr) return pkv::fail(PKV_ERR_INVALID, "%s: null row", what);
  for (int32_t j = 0; j < n; ++j) {
    const int32_t b = row[j];
    if (!a->in_range(b)) return pkv::fail(PKV_ERR_BAD_BLOCK, "%s: block %d out of range [0,%d)", what, b, a->num_blocks);
    if (a->ref[b] < 1) return pkv::fail(PKV_ERR_REFCOUNT, "%s: block %d is free", what, b);
  }
  if (!count_duplicates || n < 2) return PKV_OK;
  if (++a->epoch == 0) {
    std::fill(a->stamp.begin(), a->stamp.end(), 0u);
    a->epoch = 1;
  }
  bool repeats = false;
  for (int32_t j = 0; j < n && !repeats; ++j) {
    repeats = a->stamp[row[j]] == a->epoch;
    a->stamp[row[j]] = a->epoch;
  }
  if (!repeats) return PKV_OK;  // each id once: referenced ids cannot underflow
  std::vector<int32_t> sorted(row, row + n);
  std::sort(sorted.begin(), sorted.end());
  for (int32_t j = 0; j < n;) {
    int32_t k = j;
    while (k < n && sorted[k] == sorted[j]) ++k;
    if (a->ref[sorted[j]] < k - j)
      return pkv::fail(PKV_ERR_REFCOUNT, "%s: block %d held %d times with count %d", what, sorted[j], k - j,
                       a->ref[sorted[j]]);
    j = k;
  }
  return PKV_OK;
}

// What one sequence's reservation needs: fresh blocks and whether the partly
// filled last block must be copied.  `ref_of` supplies the counts to judge
// sharing by (the live counts, or counts adjusted by earlier sequences of a
// batch).
struct Need {
  int32_t fresh = 0;
  int32_t cow = 0;
};

template <typename RefOf>
int plan_reserve(const pkv_allocator* a, const int32_t* row, int32_t row_capacity, int32_t n_blocks,
                 int32_t cur_len, int32_t n_new, RefOf ref_of, Need* need) {
  const int32_t bs = a->block_size;
  if (cur_len < 0 || n_new < 0) return pkv::fail(PKV_ERR_INVALID, "reserve: negative length (%d, %d)", cur_len, n_new);
  if (n_blocks != ceil_div(cur_len, bs))
    return pkv::fail(PKV_ERR_INVALID, "reserve: row holds %d blocks but cur_len %d needs %d", n_blocks, cur_len,
                     ceil_div(cur_len, bs));
  int st = check_row(a, row, n_blocks, "reserve", false);
  if (st != PKV_OK) return st;
  const int64_t end = static_cast<int64_t>(cur_len) + n_new;
  if (end > INT32_MAX) return pkv::fail(PKV_ERR_INVALID, "reserve: length overflow");
  const int32_t total = ceil_div(end, bs);
  if (total > row_capacity)
    return pkv::fail(PKV_ERR_INVALID, "reserve: %d blocks exceed row capacity %d", total, row_capacity);
  need->fresh = total - n_blocks;
  need->cow = 0;
  if (n_new > 0 && cur_len % bs != 0) {
    const int32_t b = row[cur_len / bs];
    if (ref_of(b) > 1) need->cow = 1;
  }
  return PKV_OK;
}

// Applies a planned reservation (resources already checked).
void apply_reserve(pkv_allocator* a, int32_t* row, int32_t* n_blocks, int32_t cur_len, int32_t n_new,
                   int64_t* slots_out, int32_t* cow_pair, int32_t* n_cow) {
  const int32_t bs = a->block_size;
  *n_cow = 0;
  for (int32_t i = 0; i < n_new; ++i) {
    const int32_t pos = cur_len + i;
    const int32_t j = pos / bs;
    if (j == *n_blocks) {
      row[j] = a->pop();
      ++*n_blocks;
    } else if (i == 0 && a->ref[row[j]] > 1) {
      // First write into a block other sequences still hold: copy it.
      const int32_t src = row[j];
      const int32_t dst = a->pop();
      cow_pair[0] = src;
      cow_pair[1] = dst;
      *n_cow = 1;
      --a->ref[src];  // stays >= 1: another holder remains
      row[j] = dst;
    }
    slots_out[i] = static_cast<int64_t>(row[j]) * bs + pos % bs;
  }
}

}  // namespace

extern "C" {

PKV_API int pkv_allocator_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free_order,
                                 pkv_allocator** out) {
  if (out == nullptr) return pkv::fail(PKV_ERR_INVALID, "allocator_create: null out");
  if (num_blocks <= 0 || block_size <= 0)
    return pkv::fail(PKV_ERR_INVALID, "allocator_create: num_blocks %d and block_size %d must be positive",
                     num_blocks, block_size);
  pkv_allocator* a = new (std::nothrow) pkv_allocator;
  if (a == nullptr) return pkv::fail(PKV_ERR_INVALID, "allocator_create: out of host memory");
  try {
    a->ring.resize(num_blocks);
    a->ref.assign(num_blocks, 0);
    a->stamp.assign(num_blocks, 0u);
  } catch (...) {
    delete a;
    return pkv::fail(PKV_ERR_INVALID, "allocator_create: out of host memory");
  }
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  if (initial_free_order != nullptr) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return pkv::fail(PKV_ERR_INVALID, "allocator_create: initial order is not a permutation (entry %d = %d)", i, b);
      }
      seen[b] = 1;
      a->ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) a->ring[i] = i;
  }
  a->head = 0;
  a->count = num_blocks;
  *out = a;
  return PKV_OK;
}

PKV_API void pkv_allocator_destroy(pkv_allocator* a) { delete a; }

PKV_API int pkv_block_alloc(pkv_allocator* a, int32_t* block_out) {
  if (a == nullptr || block_out == nullptr) return pkv::fail(PKV_ERR_INVALID, "block_alloc: null argument");
  if (a->available() == 0) return pkv::fail(PKV_ERR_NO_BLOCKS, "block_alloc: pool of %d blocks is full", a->num_blocks);
  *block_out = a->pop();
  return PKV_OK;
}

PKV_API int pkv_blocks_alloc(pkv_allocator* a, int32_t n, int32_t* blocks_out) {
  if (a == nullptr || n < 0 || (blocks_out == nullptr && n > 0))
    return pkv::fail(PKV_ERR_INVALID, "blocks_alloc: null argument or negative count");
  if (n > a->available())
    return pkv::fail(PKV_ERR_NO_BLOCKS, "blocks_alloc: %d blocks asked, %d available", n, a->available());
  for (int32_t i = 0; i < n; ++i) blocks_out[i] = a->pop();
  return PKV_OK;
}

PKV_API int pkv_block_incref(pkv_allocator* a, int32_t block) {
  if (a == nullptr) return pkv::fail(PKV_ERR_INVALID, "block_incref: null allocator");
  if (!a->in_range(block)) return pkv::fail(PKV_ERR_BAD_BLOCK, "block_incref: block %d out of range", block);
  if (a->ref[block] < 1) return pkv::fail(PKV_ERR_REFCOUNT, "block_incref: block %d is free", block);
  ++a->ref[block];
  return PKV_OK;
}

PKV_API int pkv_block_decref(pkv_allocator* a, int32_t block) {
  if (a == nullptr) return pkv::fail(PKV_ERR_INVALID, "block_decref: null allocator");
  if (!a->in_range(block)) return pkv::fail(PKV_ERR_BAD_BLOCK, "block_decref: block %d out of range", block);
  if (a->ref[block] < 1) return pkv::fail(PKV_ERR_REFCOUNT, "block_decref: block %d is already free", block);
  if (--a->ref[block] == 0) a->release_zero(block);
  return PKV_OK;
}

PKV_API int pkv_block_refcount(const pkv_allocator* a, int32_t block) {
  if (a == nullptr) return pkv::fail(PKV_ERR_INVALID, "block_refcount: null allocator");
  if (!a->in_range(block)) return pkv::fail(PKV_ERR_BAD_BLOCK, "block_refcount: block %d out of range", block);
  return a->ref[block];
}

PKV_API int32_t pkv_num_free(const pkv_allocator* a) { return a ? a->count : PKV_ERR_INVALID; }
PKV_API int32_t pkv_num_blocks(const pkv_allocator* a) { return a ? a->num_blocks : PKV_ERR_INVALID; }
PKV_API int32_t pkv_block_size(const pkv_allocator* a) { return a ? a->block_size : PKV_ERR_INVALID; }

PKV_API int pkv_free_list(const pkv_allocator* a, int32_t* out, int32_t capacity) {
  if (a == nullptr || (out == nullptr && capacity > 0)) return pkv::fail(PKV_ERR_INVALID, "free_list: null argument");
  const int32_t n = std::min(capacity, a->count);
  for (int32_t i = 0; i < n; ++i) {
    int32_t k = a->head + i;
    if (k >= a->num_blocks) k -= a->num_blocks;
    out[i] = a->ring[k];
  }
  return n;
}

PKV_API int pkv_seq_fork(pkv_allocator* a, const int32_t* src_row, int32_t n_blocks, int32_t* dst_row) {
  if (a == nullptr || (n_blocks > 0 && dst_row == nullptr)) return pkv::fail(PKV_ERR_INVALID, "seq_fork: null argument");
  int st = check_row(a, src_row, n_blocks, "seq_fork", true);
  if (st != PKV_OK) return st;
  for (int32_t j = 0; j < n_blocks; ++j) {
    ++a->ref[src_row[j]];
    dst_row[j] = src_row[j];
  }
  return PKV_OK;
}

PKV_API int pkv_seq_reserve(pkv_allocator* a, int32_t* row, int32_t row_capacity, int32_t* n_blocks, int32_t cur_len,
                            int32_t n_new, int64_t* slots_out, int32_t* cow_pairs_out, int32_t* n_cow_out) {
  if (a == nullptr || n_blocks == nullptr || n_cow_out == nullptr || cow_pairs_out == nullptr ||
      (row == nullptr && row_capacity > 0) || (slots_out == nullptr && n_new > 0))
    return pkv::fail(PKV_ERR_INVALID, "seq_reserve: null argument");
  Need need;
  int st = plan_reserve(a, row, row_capacity, *n_blocks, cur_len, n_new, [a](int32_t b) { return a->ref[b]; }, &need);
  if (st != PKV_OK) return st;
  if (need.fresh + need.cow > a->available())
    return pkv::fail(PKV_ERR_NO_BLOCKS, "seq_reserve: needs %d blocks, %d available", need.fresh + need.cow,
                     a->available());
  apply_reserve(a, row, n_blocks, cur_len, n_new, slots_out, cow_pairs_out, n_cow_out);
  return PKV_OK;
}

PKV_API int pkv_seq_reserve_batch(pkv_allocator* a, int32_t* tables, int32_t row_stride, int32_t* n_blocks,
                                  const int32_t* cur_lens, const int32_t* n_new, int32_t batch, int64_t* slots_out,
                                  int32_t* cow_pairs_out, int32_t cow_capacity, int32_t* n_cow_out) {
  if (a == nullptr || n_cow_out == nullptr || batch < 0 || row_stride < 0)
    return pkv::fail(PKV_ERR_INVALID, "seq_reserve_batch: bad argument");
  if (batch > 0 && (tables == nullptr || n_blocks == nullptr || cur_lens == nullptr || n_new == nullptr))
    return pkv::fail(PKV_ERR_INVALID, "seq_reserve_batch: null argument");
  // Dry run: validate every sequence and count the blocks the whole batch
  // takes, following how earlier copies lower the counts later sequences see.
  std::unordered_map<int32_t, int32_t> ref_drop;
  int64_t needed = 0, pairs = 0, total_slots = 0;
  for (int32_t i = 0; i < batch; ++i) {
    const int32_t* row = tables + static_cast<int64_t>(i) * row_stride;
    Need need;
    auto ref_of = [&](int32_t b) {
      auto it = ref_drop.find(b);
      return a->ref[b] - (it == ref_drop.end() ? 0 : it->second);
    };
    int st = plan_reserve(a, row, row_stride, n_blocks[i], cur_lens[i], n_new[i], ref_of, &need);
    if (st != PKV_OK) return st;
    if (need.cow) ++ref_drop[row[cur_lens[i] / a->block_size]];
    needed += need.fresh + need.cow;
    pairs += need.cow;
    total_slots += n_new[i];
  }
  if (total_slots > 0 && slots_out == nullptr) return pkv::fail(PKV_ERR_INVALID, "seq_reserve_batch: null slots_out");
  if (pairs > cow_capacity || (pairs > 0 && cow_pairs_out == nullptr))
    return pkv::fail(PKV_ERR_INVALID, "seq_reserve_batch: %lld copy pairs exceed capacity %d", (long long)pairs,
                     cow_capacity);
  if (needed > a->available())
    return pkv::fail(PKV_ERR_NO_BLOCKS, "seq_reserve_batch: needs %lld blocks, %d available", (long long)needed,
                     a->available());
  int64_t s = 0;
  int32_t n_cow = 0;
  for (int32_t i = 0; i < batch; ++i) {
    int32_t* row = tables + static_cast<int64_t>(i) * row_stride;
    int32_t one = 0;
    apply_reserve(a, row, &n_blocks[i], cur_lens[i], n_new[i], slots_out + s, cow_pairs_out + 2 * n_cow, &one);
    n_cow += one;
    s += n_new[i];
  }
  *n_cow_out = n_cow;
  return PKV_OK;
}

PKV_API int pkv_seq_release(pkv_allocator* a, const int32_t* row, int32_t n_blocks) {
  if (a == nullptr) return pkv::fail(PKV_ERR_INVALID, "seq_release: null allocator");
  int st = check_row(a, row, n_blocks, "seq_release", true);
  if (st != PKV_OK) return st;
  for (int32_t j = 0; j < n_blocks; ++j)
    if (--a->ref[row[j]] == 0) a->release_zero(row[j]);
  return PKV_OK;
}

// ---- prefix cache ------------------------------------------------------------

PKV_API int pkv_prefix_cache_enable(pkv_allocator* a) {
  if (a == nullptr) return pkv::fail(PKV_ERR_INVALID, "prefix_cache_enable: null allocator");
  if (a->cache_on) return PKV_OK;
  try {
    a->key_of.assign(a->num_blocks, Key{});
    a->cached.assign(a->num_blocks, 0);
    a->lru_prev.assign(a->num_blocks, -1);
    a->lru_next.assign(a->num_blocks, -1);
    a->index.reserve(static_cast<size_t>(a->num_blocks));
  } catch (...) {
    return pkv::fail(PKV_ERR_INVALID, "prefix_cache_enable: out of host memory");
  }
  a->cache_on = true;
  return PKV_OK;
}

PKV_API int pkv_prefix_block_keys(const int32_t* tokens, int32_t n_tokens, int32_t block_size, uint8_t* keys_out,
                                  int32_t capacity) {
  if (n_tokens < 0 || block_size <= 0 || capacity < 0 || (n_tokens > 0 && tokens == nullptr) ||
      (capacity > 0 && keys_out == nullptr))
    return pkv::fail(PKV_ERR_INVALID, "prefix_block_keys: bad argument");
  const int32_t n = std::min(n_tokens / block_size, capacity);
  Key k{};
  for (int32_t i = 0; i < n; ++i) {
    next_key(k, tokens + static_cast<int64_t>(i) * block_size, block_size, &k);
    std::memcpy(keys_out + 32 * static_cast<int64_t>(i), k.data(), 32);
  }
  return n;
}

PKV_API int pkv_prefix_match(pkv_allocator* a, const int32_t* tokens, int32_t n_tokens, int32_t* row_out,
                             int32_t row_capacity, int32_t* n_blocks_out) {
  if (a == nullptr || n_blocks_out == nullptr || n_tokens < 0 || row_capacity < 0 ||
      (n_tokens > 0 && tokens == nullptr) || (row_capacity > 0 && row_out == nullptr))
    return pkv::fail(PKV_ERR_INVALID, "prefix_match: bad argument");
  if (!a->cache_on) return pkv::fail(PKV_ERR_INVALID, "prefix_match: prefix cache not enabled");
  const int32_t bs = a->block_size;
  const int32_t limit = std::min(n_tokens / bs, row_capacity);
  int32_t hits = 0;
  Key k{};
  for (int32_t i = 0; i < limit; ++i) {
    next_key(k, tokens + static_cast<int64_t>(i) * bs, bs, &k);
    auto it = a->index.find(k);
    if (it == a->index.end()) break;   // the reusable prefix ends at the first miss
    row_out[hits++] = it->second;
  }
  for (int32_t i = 0; i < hits; ++i) {
    const int32_t b = row_out[i];
    if (a->ref[b] == 0) a->lru_unlink(b);   // revive an evictable block
    ++a->ref[b];
  }
  *n_blocks_out = hits;
  return PKV_OK;
}

PKV_API int pkv_prefix_register(pkv_allocator* a, const int32_t* tokens, int32_t n_tokens, const int32_t* row,
                                int32_t n_blocks, int32_t first_block, int32_t* n_new_out) {
  if (a == nullptr || n_tokens < 0 || n_blocks < 0 || first_block < 0 || (n_tokens > 0 && tokens == nullptr) ||
      (n_blocks > 0 && row == nullptr))
    return pkv::fail(PKV_ERR_INVALID, "prefix_register: bad argument");
  if (!a->cache_on) return pkv::fail(PKV_ERR_INVALID, "prefix_register: prefix cache not enabled");
  const int32_t bs = a->block_size;
  const int32_t n = std::min(n_blocks, n_tokens / bs);
  if (first_block > n) return pkv::fail(PKV_ERR_INVALID, "prefix_register: first_block %d beyond %d full blocks",
                                        first_block, n);
  // The chain resumes from the key of the last block the caller matched.
  Key k{};
  if (first_block > 0) {
    const int32_t b = row[first_block - 1];
    if (!a->in_range(b) || !a->cached[b])
      return pkv::fail(PKV_ERR_INVALID, "prefix_register: block %d before first_block is not cached", b);
    k = a->key_of[b];
  }
  std::vector<Key> keys(static_cast<size_t>(n - first_block));
  for (int32_t i = first_block; i < n; ++i) {   // validate everything before changing anything
    next_key(k, tokens + static_cast<int64_t>(i) * bs, bs, &k);
    keys[i - first_block] = k;
    const int32_t b = row[i];
    if (!a->in_range(b)) return pkv::fail(PKV_ERR_BAD_BLOCK, "prefix_register: block %d out of range", b);
    if (a->ref[b] < 1) return pkv::fail(PKV_ERR_REFCOUNT, "prefix_register: block %d is not held", b);
    if (a->cached[b] && a->key_of[b] != k)
      return pkv::fail(PKV_ERR_INVALID, "prefix_register: block %d already holds another prefix", b);
  }
  int32_t added = 0;
  for (int32_t i = first_block; i < n; ++i) {
    const int32_t b = row[i];
    const Key& key = keys[i - first_block];
    if (a->cached[b] || a->index.count(key)) continue;   // first block recorded for a key stays
    a->index.emplace(key, b);
    a->key_of[b] = key;
    a->cached[b] = 1;
    ++a->n_cached;
    ++added;
  }
  if (n_new_out) *n_new_out = added;
  return PKV_OK;
}

PKV_API int32_t pkv_prefix_cached_blocks(const pkv_allocator* a) { return a ? a->n_cached : PKV_ERR_INVALID; }

PKV_API int pkv_prefix_lru(const pkv_allocator* a, int32_t* out, int32_t capacity) {
  if (a == nullptr || capacity < 0 || (out == nullptr && capacity > 0))
    return pkv::fail(PKV_ERR_INVALID, "prefix_lru: bad argument");
  int32_t n = 0;
  for (int32_t b = a->cache_on ? a->lru_head : -1; b >= 0 && n < capacity; b = a->lru_next[b]) out[n++] = b;
  return n;
}

}  // extern "C"
