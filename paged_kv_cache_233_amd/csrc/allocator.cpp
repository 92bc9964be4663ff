// Host-side block allocator: the KV-cache manager of the paged pool.
//
// Policy (see pkv.h for the full contract) follows "vLLM: what PagedAttention
// turned into", section "The block pool, and the two tricks in it": the first
// block popped from the free queue becomes the null block; freed blocks
// without a content hash go to the front of the queue (LIFO), freed blocks
// with one to the back (FIFO, so cached prefixes are evicted least recently
// freed first), a request's blocks handed back tail first; the free queue is
// an intrusive doubly linked list with sentinel head and tail stored in two
// int32 arrays, so removal anywhere is O(1) and no per-operation heap objects
// are created. Sharing by refcount and copy-on-write follow "(2) vLLM
// Internals: From PagedAttention to Removing PagedAttention", section 1.2
// "Three Direct Wins".
//
// Prefix caching (optional; same page, sections "The block pool, and the two
// tricks in it" and "What a block hash actually is"): a full block whose
// token ids are known gets a chained content hash and enters a hash -> block
// map; when freed it keeps the hash and stays reusable until the free queue
// hands it out again, at which point it is evicted (lazily); a new sequence
// takes the longest run of cached full blocks of its prompt, stopping at the
// first miss.
#include <algorithm>
#include <array>
#include <cstring>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "host.h"

namespace {

typedef std::array<uint8_t, 32> Hash;
// Map key: the block hash followed by the KV-cache group id, 4 bytes big
// endian (one group here: 0).
typedef std::array<uint8_t, 36> Key;

struct KeyHasher {
  size_t operator()(const Key& k) const {
    uint64_t v;
    std::memcpy(&v, k.data(), sizeof(v));
    return (size_t)v;
  }
};

Key make_key(const Hash& h) {
  Key k{};
  std::copy(h.begin(), h.end(), k.begin());
  return k;
}

}  // namespace

struct pkv_allocator {
  int32_t nb = 0;
  // Free queue: nodes 0..nb-1 are blocks, nb is the head sentinel and nb+1
  // the tail sentinel. in_free[b] marks membership.
  std::vector<int32_t> next, prev;
  std::vector<uint8_t> in_free;
  int32_t nfree = 0;
  std::vector<int32_t> ref;
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t len = 0;
    // content-hash chain: token ids recorded so far, hash of the last full
    // recorded block, ids of the partly recorded block, the extra key of the
    // first block
    int64_t recorded = 0;
    bool has_parent = false;
    Hash parent{};
    int32_t pending[pkv::kBlock] = {};
    uint64_t salt = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;
  // prefix cache
  bool caching = false;
  std::vector<Hash> bhash;
  std::vector<uint8_t> hashed;
  std::unordered_map<Key, int32_t, KeyHasher> cached;
  int64_t lookups = 0, hit_blocks = 0;

  int32_t head() const { return nb; }
  int32_t tail() const { return nb + 1; }

  // Lazy eviction: a cached block leaves the map when it is reused.
  void evict(int32_t b) {
    auto it = cached.find(make_key(bhash[b]));
    if (it != cached.end() && it->second == b) cached.erase(it);
    hashed[b] = 0;
  }
  void clear_cache() {
    cached.clear();
    std::fill(hashed.begin(), hashed.end(), 0);
  }
  // A full block of a sequence got its hash: it enters the map unless
  // another block already holds the same content.
  void register_block(int32_t b, const Hash& h) {
    if (!caching || hashed[b]) return;
    Key k = make_key(h);
    if (cached.count(k)) return;
    bhash[b] = h;
    hashed[b] = 1;
    cached.emplace(k, b);
  }
  void link_after(int32_t at, int32_t b) {
    int32_t n = next[at];
    next[at] = b;
    prev[b] = at;
    next[b] = n;
    prev[n] = b;
    in_free[b] = 1;
    ++nfree;
  }
  void unlink(int32_t b) {
    int32_t p = prev[b], n = next[b];
    next[p] = n;
    prev[n] = p;
    in_free[b] = 0;
    --nfree;
  }
  int32_t pop_front() {
    int32_t b = next[head()];
    unlink(b);
    if (hashed[b]) evict(b);
    return b;
  }
  void reset_queue(const int32_t* order, int32_t n) {
    next[head()] = tail();
    prev[tail()] = head();
    std::fill(in_free.begin(), in_free.end(), 0);
    nfree = 0;
    int32_t at = head();
    for (int32_t i = 0; i < n; ++i) {
      link_after(at, order[i]);
      at = order[i];
    }
  }
  // Blocks needed to append n tokens: (copy-on-write?, new blocks).
  void needs(const Seq& s, int64_t n, bool* cow, int64_t* grow) const {
    *cow = n > 0 && (s.len % pkv::kBlock) != 0 && ref[s.blocks.back()] > 1;
    *grow = (s.len + n + pkv::kBlock - 1) / pkv::kBlock - (int64_t)s.blocks.size();
  }
};

namespace {

using pkv::fail;

int check_handle(pkv_allocator* a) {
  return a ? PKV_OK : fail(PKV_ERR_INVALID_ARG, "allocator handle is NULL");
}

// Performs one append whose feasibility was already checked.
void do_append(pkv_allocator* a, pkv_allocator::Seq& s, int32_t n, int64_t* slots,
               std::vector<int64_t>& pairs) {
  bool cow;
  int64_t grow;
  a->needs(s, n, &cow, &grow);
  if (cow) {
    int32_t old = s.blocks.back();
    int32_t b = a->pop_front();
    a->ref[b] = 1;
    a->ref[old] -= 1;
    s.blocks.back() = b;
    pairs.push_back(old);
    pairs.push_back(b);
  }
  for (int64_t i = 0; i < grow; ++i) {
    int32_t b = a->pop_front();
    a->ref[b] = 1;
    s.blocks.push_back(b);
  }
  for (int32_t i = 0; i < n; ++i) {
    int64_t p = s.len + i;
    slots[i] = (int64_t)s.blocks[p / pkv::kBlock] * pkv::kBlock + p % pkv::kBlock;
  }
  s.len += n;
}

}  // namespace

extern "C" {

int pkv_allocator_create(int32_t num_blocks, pkv_allocator** out) {
  pkv::clear_error();
  if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (num_blocks < 2) return fail(PKV_ERR_INVALID_ARG, "num_blocks must be >= 2, got %d", num_blocks);
  pkv_allocator* a = new (std::nothrow) pkv_allocator();
  if (!a) return fail(PKV_ERR_INVALID_ARG, "host allocation failed");
  a->nb = num_blocks;
  a->next.assign(num_blocks + 2, -1);
  a->prev.assign(num_blocks + 2, -1);
  a->in_free.assign(num_blocks, 0);
  a->ref.assign(num_blocks, 0);
  a->bhash.assign(num_blocks, Hash{});
  a->hashed.assign(num_blocks, 0);
  std::vector<int32_t> order(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) order[i] = i;
  a->reset_queue(order.data(), num_blocks);
  a->pop_front();  // block 0: the null block, never handed out
  *out = a;
  return PKV_OK;
}

int pkv_allocator_destroy(pkv_allocator* a) {
  pkv::clear_error();
  delete a;
  return PKV_OK;
}

int pkv_allocator_set_free_order(pkv_allocator* a, const int32_t* order, int32_t n) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  if (!a->seqs.empty() || a->nfree != a->nb - 1)
    return fail(PKV_ERR_INVALID_ARG, "free order can only be set while no block is in use");
  if (!order || n != a->nb - 1)
    return fail(PKV_ERR_INVALID_ARG, "order must hold num_blocks-1 = %d ids", a->nb - 1);
  std::vector<uint8_t> seen(a->nb, 0);
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = order[i];
    if (b < 1 || b >= a->nb || seen[b])
      return fail(PKV_ERR_INVALID_ARG, "order is not a permutation of 1..%d (entry %d = %d)",
                  a->nb - 1, i, b);
    seen[b] = 1;
  }
  a->clear_cache();
  a->reset_queue(order, n);
  return PKV_OK;
}

int pkv_allocator_shuffle_free_list(pkv_allocator* a, uint64_t seed) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  // Ids 1..nb-1 in ascending order, permuted by the Fisher-Yates shuffle in
  // Durstenfeld's form (for i = n-1 down to 1, swap entry i with entry
  // draw % (i+1)); the draws come from SplitMix64 (Steele, Lea and Flood,
  // "Fast splittable pseudorandom number generators", OOPSLA 2014): the
  // state advances by 0x9E3779B97F4A7C15 and each draw is that state mixed
  // by two xor-shift-multiply rounds and a final xor-shift.
  std::vector<int32_t> order(a->nb - 1);
  for (int32_t i = 0; i < a->nb - 1; ++i) order[i] = i + 1;
  uint64_t state = seed;
  for (int32_t i = a->nb - 2; i >= 1; --i) {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    std::swap(order[i], order[(size_t)(z % (uint64_t)(i + 1))]);
  }
  return pkv_allocator_set_free_order(a, order.data(), a->nb - 1);
}

int pkv_seq_add(pkv_allocator* a, int64_t seq_id) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  if (a->seqs.count(seq_id)) return fail(PKV_ERR_SEQ_EXISTS, "sequence %lld exists", (long long)seq_id);
  a->seqs.emplace(seq_id, pkv_allocator::Seq());
  return PKV_OK;
}

int pkv_batch_append(pkv_allocator* a, const int64_t* seq_ids, const int32_t* n_tokens,
                     int32_t n_seqs, int64_t* out_slots, int64_t* out_cow_pairs, int32_t max_pairs,
                     int32_t* out_n_pairs) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  if (n_seqs < 0 || (n_seqs > 0 && (!seq_ids || !n_tokens)))
    return fail(PKV_ERR_INVALID_ARG, "bad sequence list");
  if (max_pairs < 0 || (max_pairs > 0 && !out_cow_pairs))
    return fail(PKV_ERR_INVALID_ARG, "bad copy-pair buffer");
  // Feasibility first: nothing changes unless the whole batch fits.
  std::unordered_set<int64_t> seen;
  int64_t need = 0, total_tokens = 0, cows = 0;
  std::vector<pkv_allocator::Seq*> ss(n_seqs);
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", (long long)seq_ids[i]);
    if (!seen.insert(seq_ids[i]).second)
      return fail(PKV_ERR_INVALID_ARG, "sequence %lld appears twice", (long long)seq_ids[i]);
    if (n_tokens[i] < 0) return fail(PKV_ERR_INVALID_ARG, "negative token count");
    bool cow;
    int64_t grow;
    a->needs(it->second, n_tokens[i], &cow, &grow);
    need += grow + (cow ? 1 : 0);
    cows += cow ? 1 : 0;
    total_tokens += n_tokens[i];
    ss[i] = &it->second;
  }
  if (total_tokens > 0 && !out_slots) return fail(PKV_ERR_INVALID_ARG, "out_slots is NULL");
  if (cows > max_pairs)
    return fail(PKV_ERR_INVALID_ARG, "need room for %lld copy pairs, max_pairs = %d",
                (long long)cows, max_pairs);
  if (need > a->nfree)
    return fail(PKV_ERR_OUT_OF_BLOCKS, "need %lld blocks, %d free", (long long)need, a->nfree);
  std::vector<int64_t> pairs;
  int64_t off = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    do_append(a, *ss[i], n_tokens[i], out_slots + off, pairs);
    off += n_tokens[i];
  }
  for (size_t i = 0; i < pairs.size(); ++i) out_cow_pairs[i] = pairs[i];
  if (out_n_pairs) *out_n_pairs = (int32_t)(pairs.size() / 2);
  return PKV_OK;
}

int pkv_seq_append(pkv_allocator* a, int64_t seq_id, int32_t n_tokens, int64_t* out_slots,
                   int64_t* out_cow_pairs, int32_t max_pairs, int32_t* out_n_pairs) {
  return pkv_batch_append(a, &seq_id, &n_tokens, 1, out_slots, out_cow_pairs, max_pairs,
                          out_n_pairs);
}

int pkv_seq_fork(pkv_allocator* a, int64_t parent_id, int64_t child_id) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  auto it = a->seqs.find(parent_id);
  if (it == a->seqs.end()) return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", (long long)parent_id);
  if (a->seqs.count(child_id)) return fail(PKV_ERR_SEQ_EXISTS, "sequence %lld exists", (long long)child_id);
  pkv_allocator::Seq child = it->second;
  for (int32_t b : child.blocks) a->ref[b] += 1;
  a->seqs.emplace(child_id, std::move(child));
  return PKV_OK;
}

int pkv_seq_free(pkv_allocator* a, int64_t seq_id) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", (long long)seq_id);
  // Visit tail first. Released blocks without a hash go to the queue front
  // in visiting order, so the tail is handed out first and the first block
  // last; released blocks with a hash go to the back in visiting order, so
  // among cached blocks the tail is also evicted first.
  int32_t at = a->head();
  const std::vector<int32_t>& bl = it->second.blocks;
  for (size_t i = bl.size(); i-- > 0;) {
    int32_t b = bl[i];
    if (--a->ref[b] == 0) {
      if (a->hashed[b]) {
        a->link_after(a->prev[a->tail()], b);
      } else {
        a->link_after(at, b);
        at = b;
      }
    }
  }
  a->seqs.erase(it);
  return PKV_OK;
}

int pkv_allocator_enable_prefix_caching(pkv_allocator* a, int32_t enabled) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  if (!a->seqs.empty())
    return fail(PKV_ERR_INVALID_ARG, "prefix caching can only be switched while no sequence exists");
  a->clear_cache();
  a->caching = enabled != 0;
  return PKV_OK;
}

}  // extern "C"

// The cached blocks a prompt would attach (longest run of full blocks from
// its start whose chained hashes are in the map), and the hash of the last.
static void walk_cached(const pkv_allocator* a, const int32_t* tokens, int32_t n_tokens,
                        uint64_t extra_key, int32_t max_cached_tokens, std::vector<int32_t>* got,
                        Hash* last) {
  const int32_t limit = max_cached_tokens < 0 ? n_tokens : std::min(n_tokens, max_cached_tokens);
  const int32_t full = a->caching ? limit / pkv::kBlock : 0;
  Hash h;
  for (int32_t k = 0; k < full; ++k) {
    pkv::block_hash(k > 0 ? last->data() : nullptr, tokens + (int64_t)k * pkv::kBlock,
                    k == 0 ? extra_key : 0, h.data());
    auto it = a->cached.find(make_key(h));
    if (it == a->cached.end()) break;  // chained hashes: every later block misses too
    got->push_back(it->second);
    *last = h;
  }
}

extern "C" {

int pkv_prefix_lookup(pkv_allocator* a, const int32_t* tokens, int32_t n_tokens,
                      uint64_t extra_key, int32_t max_cached_tokens, int32_t* out_cached_tokens,
                      int32_t* out_revived_blocks) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  if (n_tokens < 0 || (n_tokens > 0 && !tokens)) return fail(PKV_ERR_INVALID_ARG, "bad token list");
  if (!out_cached_tokens || !out_revived_blocks) return fail(PKV_ERR_INVALID_ARG, "NULL output");
  std::vector<int32_t> got;
  Hash last;
  walk_cached(a, tokens, n_tokens, extra_key, max_cached_tokens, &got, &last);
  int32_t revived = 0;
  for (int32_t b : got) revived += a->ref[b] == 0;
  *out_cached_tokens = (int32_t)got.size() * pkv::kBlock;
  *out_revived_blocks = revived;
  return PKV_OK;
}

int pkv_seq_add_cached(pkv_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                       uint64_t extra_key, int32_t max_cached_tokens, int32_t* out_cached_tokens) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  if (n_tokens < 0 || (n_tokens > 0 && !tokens)) return fail(PKV_ERR_INVALID_ARG, "bad token list");
  if (a->seqs.count(seq_id)) return fail(PKV_ERR_SEQ_EXISTS, "sequence %lld exists", (long long)seq_id);
  pkv_allocator::Seq s;
  s.salt = extra_key;
  Hash last;
  walk_cached(a, tokens, n_tokens, extra_key, max_cached_tokens, &s.blocks, &last);
  for (int32_t b : s.blocks) {
    if (a->ref[b] == 0) a->unlink(b);  // free but cached: revived from the queue
    a->ref[b] += 1;
  }
  if (!s.blocks.empty()) {
    s.parent = last;
    s.has_parent = true;
  }
  s.len = s.recorded = (int64_t)s.blocks.size() * pkv::kBlock;
  a->lookups += 1;
  a->hit_blocks += (int64_t)s.blocks.size();
  if (out_cached_tokens) *out_cached_tokens = (int32_t)s.len;
  a->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

int pkv_seq_record_tokens(pkv_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t n) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", (long long)seq_id);
  pkv_allocator::Seq& s = it->second;
  if (n < 0 || (n > 0 && !tokens)) return fail(PKV_ERR_INVALID_ARG, "bad token list");
  if (s.recorded + n > s.len)
    return fail(PKV_ERR_INVALID_ARG, "sequence %lld: %lld recorded + %d > length %lld",
                (long long)seq_id, (long long)s.recorded, n, (long long)s.len);
  Hash h;
  for (int32_t i = 0; i < n; ++i) {
    s.pending[s.recorded % pkv::kBlock] = tokens[i];
    s.recorded += 1;
    if (s.recorded % pkv::kBlock == 0) {
      const int64_t k = s.recorded / pkv::kBlock - 1;
      pkv::block_hash(s.has_parent ? s.parent.data() : nullptr, s.pending, k == 0 ? s.salt : 0,
                      h.data());
      s.parent = h;
      s.has_parent = true;
      a->register_block(s.blocks[k], h);
    }
  }
  return PKV_OK;
}

int pkv_block_hash(pkv_allocator* a, int32_t block, uint8_t* out, int32_t* has_hash) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  if (!out || !has_hash || block < 0 || block >= a->nb)
    return fail(PKV_ERR_INVALID_ARG, "bad block query");
  *has_hash = a->hashed[block];
  std::memcpy(out, a->bhash[block].data(), 32);
  if (!*has_hash) std::memset(out, 0, 32);
  return PKV_OK;
}

int pkv_prefix_cache_stats(pkv_allocator* a, int32_t* cached_blocks, int64_t* lookups,
                           int64_t* hit_blocks) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  if (cached_blocks) *cached_blocks = (int32_t)a->cached.size();
  if (lookups) *lookups = a->lookups;
  if (hit_blocks) *hit_blocks = a->hit_blocks;
  return PKV_OK;
}

int pkv_seq_len(pkv_allocator* a, int64_t seq_id, int64_t* out) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", (long long)seq_id);
  *out = it->second.len;
  return PKV_OK;
}

int pkv_fill_block_table(pkv_allocator* a, const int64_t* seq_ids, int32_t n, int32_t* table,
                         int32_t max_blocks, int32_t* context_lens) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  if (n < 0 || max_blocks < 0 || (n > 0 && (!seq_ids || (!table && max_blocks > 0))))
    return fail(PKV_ERR_INVALID_ARG, "bad table arguments");
  // Check everything before writing anything.
  std::vector<const pkv_allocator::Seq*> ss(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return fail(PKV_ERR_NO_SUCH_SEQ, "no sequence %lld", (long long)seq_ids[i]);
    if ((int64_t)it->second.blocks.size() > max_blocks)
      return fail(PKV_ERR_INVALID_ARG, "sequence %lld has %zu blocks > max_blocks %d",
                  (long long)seq_ids[i], it->second.blocks.size(), max_blocks);
    if (context_lens && it->second.len > INT32_MAX)
      return fail(PKV_ERR_INVALID_ARG, "sequence too long for int32 context length");
    ss[i] = &it->second;
  }
  for (int32_t i = 0; i < n; ++i) {
    int32_t* row = table + (int64_t)i * max_blocks;
    const std::vector<int32_t>& bl = ss[i]->blocks;
    std::copy(bl.begin(), bl.end(), row);
    std::fill(row + bl.size(), row + max_blocks, 0);
    if (context_lens) context_lens[i] = (int32_t)ss[i]->len;
  }
  return PKV_OK;
}

int pkv_block_refcount(pkv_allocator* a, int32_t block, int32_t* out) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  if (!out || block < 0 || block >= a->nb) return fail(PKV_ERR_INVALID_ARG, "bad block id %d", block);
  *out = block == 0 ? 0 : a->ref[block];
  return PKV_OK;
}

int pkv_num_free_blocks(pkv_allocator* a, int32_t* out) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  *out = a->nfree;
  return PKV_OK;
}

int pkv_allocator_stats(pkv_allocator* a, pkv_stats* out) {
  pkv::clear_error();
  if (int e = check_handle(a)) return e;
  if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  std::vector<int32_t> filled(a->nb, 0);
  int64_t logical = 0;
  for (const auto& kv : a->seqs) {
    const auto& s = kv.second;
    logical += s.len;
    for (size_t i = 0; i < s.blocks.size(); ++i) {
      int64_t f = std::min<int64_t>(pkv::kBlock, s.len - (int64_t)i * pkv::kBlock);
      int32_t b = s.blocks[i];
      if (f > filled[b]) filled[b] = (int32_t)f;
    }
  }
  int32_t used = 0, shared = 0;
  int64_t stored = 0;
  for (int32_t b = 1; b < a->nb; ++b) {
    if (a->ref[b] > 0) ++used;
    if (a->ref[b] > 1) ++shared;
    stored += filled[b];
  }
  out->num_seqs = (int32_t)a->seqs.size();
  out->used_blocks = used;
  out->free_blocks = a->nfree;
  out->shared_blocks = shared;
  out->logical_tokens = logical;
  out->stored_tokens = stored;
  out->utilisation = used ? (double)stored / ((double)pkv::kBlock * used) : 0.0;
  return PKV_OK;
}

int pkv_blocks_for_bytes(int64_t bytes, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                         int32_t* out) {
  pkv::clear_error();
  if (!out || bytes < 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_ERR_INVALID_ARG, "bad pool sizing arguments");
  if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, "dtype %d", dtype);
  int64_t elem = dtype == PKV_F32 ? 4 : 2;
  int64_t per_block = 2 * (int64_t)num_kv_heads * pkv::kBlock * head_dim * elem;
  int64_t n = bytes / per_block;
  *out = (int32_t)std::min<int64_t>(n, INT32_MAX);
  return PKV_OK;
}

}  // extern "C"
