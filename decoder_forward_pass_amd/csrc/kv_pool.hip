// Host-side manager of the paged KV pool's block ids ("Candle model runner", section 2.2 "Candle
// tensors and Rust-owned state" and the KvPool interface of section 4): references per block,
// all-or-nothing allocation, a prefix index of full blocks, and an LRU cache of released full
// blocks (oldest evicted first when an allocation needs room). Host memory only; the blocks'
// K/V data are copied by dec_kv_export / dec_kv_import, next to the context that owns the pool.
#include <cstdint>
#include <list>
#include <set>
#include <string>
#include <unordered_map>
#include <vector>

#include "dec.h"

struct dec_block_pool {
  enum State : uint8_t { FREE = 0, USED = 1, CACHED = 2 };
  struct Block {
    int32_t ref = 0, fill = 0;
    State state = FREE;
    bool registered = false;
    uint64_t key = 0;
    std::list<int32_t>::iterator lru;
  };
  int32_t block_tokens = 0;
  bool prefix_cache = false;
  std::vector<Block> b;
  std::set<int32_t> free_ids;  // lowest id first
  std::list<int32_t> lru;      // cached blocks, oldest at the front
  std::unordered_map<uint64_t, int32_t> index;
  std::string err;
};

namespace {

int perr(dec_block_pool* p, int code, const char* msg) {
  if (p) p->err = msg;
  return code;
}

bool valid(const dec_block_pool* p, int32_t id) { return id >= 0 && id < (int32_t)p->b.size(); }

void make_free(dec_block_pool* p, int32_t id) {
  auto& k = p->b[id];
  if (k.registered) {
    auto it = p->index.find(k.key);
    if (it != p->index.end() && it->second == id) p->index.erase(it);
  }
  k = dec_block_pool::Block{};
  p->free_ids.insert(id);
}

}  // namespace

extern "C" {

int dec_pool_create(int32_t n_blocks, int32_t block_tokens, int32_t prefix_cache, dec_block_pool** out) {
  if (!out) return DEC_E_ARG;
  *out = nullptr;
  if (n_blocks < 1 || block_tokens < 1) return DEC_E_ARG;  // a pool without blocks is refused
  auto* p = new dec_block_pool();
  p->block_tokens = block_tokens;
  p->prefix_cache = prefix_cache != 0;
  p->b.resize(n_blocks);
  for (int32_t i = 0; i < n_blocks; ++i) p->free_ids.insert(i);
  *out = p;
  return DEC_OK;
}

void dec_pool_destroy(dec_block_pool* p) { delete p; }

const char* dec_pool_last_error(const dec_block_pool* p) { return p ? p->err.c_str() : ""; }

int dec_pool_alloc(dec_block_pool* p, int32_t n, int32_t* ids) {
  if (!p || !ids || n < 1) return perr(p, DEC_E_ARG, "alloc: NULL argument or n < 1");
  if ((size_t)n > p->free_ids.size() + p->lru.size()) return perr(p, DEC_E_CAPACITY, "alloc: not enough free or cached blocks");
  for (int32_t i = 0; i < n; ++i) {
    int32_t id;
    if (!p->free_ids.empty()) {
      id = *p->free_ids.begin();
      p->free_ids.erase(p->free_ids.begin());
    } else {  // evict the oldest cached block
      id = p->lru.front();
      p->lru.pop_front();
      p->b[id].state = dec_block_pool::FREE;
      make_free(p, id);
      p->free_ids.erase(id);
    }
    auto& k = p->b[id];
    k = dec_block_pool::Block{};
    k.state = dec_block_pool::USED;
    k.ref = 1;
    ids[i] = id;
  }
  return DEC_OK;
}

int dec_pool_retain(dec_block_pool* p, int32_t id) {
  if (!p || !valid(p, id) || p->b[id].state != dec_block_pool::USED) return perr(p, DEC_E_BLOCK, "retain: not an allocated block");
  ++p->b[id].ref;
  return DEC_OK;
}

int dec_pool_release(dec_block_pool* p, int32_t id) {
  if (!p || !valid(p, id) || p->b[id].state != dec_block_pool::USED) return perr(p, DEC_E_BLOCK, "release: not an allocated block");
  auto& k = p->b[id];
  if (--k.ref > 0) return DEC_OK;
  if (k.registered && p->prefix_cache) {
    k.state = dec_block_pool::CACHED;
    k.lru = p->lru.insert(p->lru.end(), id);  // newest at the back
  } else {
    make_free(p, id);
  }
  return DEC_OK;
}

int dec_pool_set_fill(dec_block_pool* p, int32_t id, int32_t n) {
  if (!p || !valid(p, id) || p->b[id].state != dec_block_pool::USED) return perr(p, DEC_E_BLOCK, "set_fill: not an allocated block");
  if (n < 0 || n > p->block_tokens) return perr(p, DEC_E_ARG, "set_fill: fill outside [0, block_tokens]");
  if (p->b[id].registered && n != p->block_tokens) return perr(p, DEC_E_ARG, "set_fill: a registered block stays full");
  p->b[id].fill = n;
  return DEC_OK;
}

int dec_pool_register(dec_block_pool* p, int32_t id, uint64_t key, int32_t* canonical) {
  if (!p || !valid(p, id) || p->b[id].state != dec_block_pool::USED) return perr(p, DEC_E_BLOCK, "register: not an allocated block");
  auto& k = p->b[id];
  if (k.fill != p->block_tokens) return perr(p, DEC_E_ARG, "register: only full blocks are registered");
  // a block holds one prefix, so it has one key: a second, different key would leave the first
  // key's entry naming the block after it is freed and handed to another sequence
  if (k.registered && k.key != key) return perr(p, DEC_E_ARG, "register: block already registered under another key");
  auto it = p->index.find(key);
  if (it != p->index.end() && it->second != id) {
    if (canonical) *canonical = it->second;  // the key's first block stays its entry
    return DEC_OK;
  }
  k.registered = true;
  k.key = key;
  p->index[key] = id;
  if (canonical) *canonical = id;
  return DEC_OK;
}

int dec_pool_lookup(dec_block_pool* p, uint64_t key, int32_t* id) {
  if (!p || !id) return perr(p, DEC_E_ARG, "lookup: NULL argument");
  *id = -1;
  auto it = p->index.find(key);
  if (it == p->index.end()) return DEC_OK;
  const int32_t i = it->second;
  auto& k = p->b[i];
  if (k.state == dec_block_pool::FREE || !k.registered || k.key != key) {
    // (an entry whose block was freed or re-keyed is stale: a miss, and it is dropped)
    p->index.erase(it);
    return DEC_OK;
  }
  if (k.state == dec_block_pool::CACHED) {  // reacquire a cached block
    p->lru.erase(k.lru);
    k.state = dec_block_pool::USED;
    k.ref = 1;
  } else {
    ++k.ref;
  }
  *id = i;
  return DEC_OK;
}

int dec_pool_block_info(const dec_block_pool* p, int32_t id, int32_t* state, int32_t* ref, int32_t* fill) {
  if (!p || !valid(p, id)) return DEC_E_BLOCK;
  if (state) *state = p->b[id].state;
  if (ref) *ref = p->b[id].ref;
  if (fill) *fill = p->b[id].fill;
  return DEC_OK;
}

void dec_pool_counts(const dec_block_pool* p, int32_t* n_free, int32_t* n_used, int32_t* n_cached) {
  if (!p) return;
  if (n_free) *n_free = (int32_t)p->free_ids.size();
  if (n_cached) *n_cached = (int32_t)p->lru.size();
  if (n_used) *n_used = (int32_t)(p->b.size() - p->free_ids.size() - p->lru.size());
}

uint64_t dec_prefix_key(uint64_t parent, const int32_t* tokens, int32_t n) {
  // FNV-1a over the parent key's and the tokens' little-endian bytes, then the splitmix64
  // finaliser (a block's key names its whole prefix: the parent key folds in every earlier block)
  uint64_t h = 1469598103934665603ull;
  auto eat = [&](uint64_t v, int bytes) {
    for (int i = 0; i < bytes; ++i) {
      h ^= (v >> (8 * i)) & 0xffu;
      h *= 1099511628211ull;
    }
  };
  eat(parent, 8);
  for (int32_t i = 0; i < n; ++i) eat((uint32_t)tokens[i], 4);
  h ^= h >> 30;
  h *= 0xBF58476D1CE4E5B9ull;
  h ^= h >> 27;
  h *= 0x94D049BB133111EBull;
  return h ^ (h >> 31);
}

}  // extern "C"
