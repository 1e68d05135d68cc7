// Host-side block manager of libpagedattn (plain C++17, no device code).
//
// Free pool, per-block reference counts, per-sequence block tables, fork and
// copy-on-write.  Blocks are taken on demand and given back as soon as a
// sequence ends (bmjup.com, "PagedAttention：大模型推理性能优化的核心技术解析",
// section "PagedAttention 的核心工作机制与创新", item 3 "动态内存分配"); one
// append walks the flowchart of wiblog.cn, "AI 推理系列（十六）：PagedAttention",
// section "PagedAttention 如何把连续序列映射到离散显存块" (a new physical block
// exactly when the last one is full); forked sequences share blocks with
// reference counts and copy a block only when they must write into a shared
// one (kongchang.com, "PagedAttention原理详解", section "PagedAttention的三大
// 核心优势", second advantage; wiblog.cn, section "Copy-on-Write、并行采样与
// Prefix Caching 不是同一件事").  A prefix cache on top of the block sharing
// lets a new request adopt full blocks whose exact token prefix another
// sequence already holds (the same wiblog.cn section: a cache key, exact
// token-sequence matching under one model configuration, a lifetime for the
// cached blocks, and the unmatched suffix still prefilled).
// The exact rules are stated with the declarations in pagedattn.h.
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pagedattn.h"

namespace {

struct Sequence {
  std::vector<int32_t> blocks;  // physical ids in logical order
  int32_t len = 0;              // tokens stored
};

// Prefix-cache key of a full block: a 128-bit hash of the cache
// configuration (the caller's salt: tokenizer, template, model) and of every
// token from the sequence start to the block's end, chained block by block.
// Two lanes of 64 bits with independent mixing; keys are compared whole.
struct Key {
  uint64_t a, b;
  bool operator==(const Key& o) const { return a == o.a && b == o.b; }
};
struct KeyHash {
  size_t operator()(const Key& k) const { return (size_t)(k.a ^ (k.b * 0x9E3779B97F4A7C15ull)); }
};

// splitmix64 finalizer (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", 2014).
uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

Key root_key(uint64_t salt) { return Key{mix64(salt ^ 0x6A09E667F3BCC908ull), mix64(salt + 0xBB67AE8584CAA73Bull)}; }

// Key of the block after `parent` holding tokens t[0 .. n).
Key next_key(Key parent, const int32_t* t, int32_t n) {
  uint64_t a = parent.a, b = parent.b;
  for (int32_t i = 0; i < n; ++i) {
    const uint64_t v = (uint32_t)t[i];
    a = mix64(a ^ (v + 0x3C6EF372FE94F82Bull));
    b = mix64(b + v * 0xA54FF53A5F1D36F1ull + 0x510E527FADE682D1ull);
  }
  return Key{mix64(a ^ (uint64_t)n), mix64(b + (uint64_t)n)};
}

}  // namespace

struct pa_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> stack;   // free pool; back() is handed out next
  std::vector<int32_t> ref;     // reference count per physical block
  std::unordered_map<int64_t, Sequence> seqs;
  // prefix cache: key of a full block's content -> the block holding it, and
  // back (a block is indexed under at most one key while it is referenced)
  std::unordered_map<Key, int32_t, KeyHash> prefix;
  std::unordered_map<int32_t, Key> key_of;

  // Length in blocks of the longest chain of indexed blocks that starts
  // tokens[0 .. n) (at most max_blocks), and their ids.
  int32_t match(const int32_t* tokens, int32_t n, uint64_t salt, int32_t max_blocks,
                std::vector<int32_t>* ids) const {
    Key k = root_key(salt);
    int32_t m = 0;
    while (m < max_blocks && (int64_t)(m + 1) * block_size <= n) {
      k = next_key(k, tokens + (int64_t)m * block_size, block_size);
      auto it = prefix.find(k);
      if (it == prefix.end()) break;
      if (ids) ids->push_back(it->second);
      ++m;
    }
    return m;
  }

  // Returns block b (refcount 0) to the free pool and removes it from the
  // prefix cache.
  void release(int32_t b) {
    stack.push_back(b);
    auto it = key_of.find(b);
    if (it != key_of.end()) {
      prefix.erase(it->second);
      key_of.erase(it);
    }
  }

  int32_t take() {
    int32_t b = stack.back();
    stack.pop_back();
    ref[b] = 1;
    return b;
  }

  // Number of fresh blocks one append to `s` needs, given the refcount that
  // its last block has at that moment.
  bool needs_block(const Sequence& s, int32_t tail_ref) const {
    if (s.len % block_size == 0) return true;
    return tail_ref > 1;
  }

  // Applies one append whose block need has already been checked.
  void append(Sequence& s, int64_t* slot, int32_t* cow_src, int32_t* cow_dst) {
    const int32_t pos = s.len % block_size;
    *cow_src = -1;
    *cow_dst = -1;
    if (pos == 0) {
      int32_t b = take();
      s.blocks.push_back(b);
      *slot = (int64_t)b * block_size;
    } else {
      int32_t tail = s.blocks.back();
      if (ref[tail] > 1) {
        int32_t fresh = take();
        ref[tail] -= 1;
        s.blocks.back() = fresh;
        *cow_src = tail;
        *cow_dst = fresh;
        *slot = (int64_t)fresh * block_size + pos;
      } else {
        *slot = (int64_t)tail * block_size + pos;
      }
    }
    s.len += 1;
  }
};

extern "C" {

PA_API pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size,
                                 const int32_t* init_free_order, pa_allocator** out) {
  if (!out) return PA_ERR_INVALID;
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0) return PA_ERR_INVALID;
  try {
    pa_allocator* a = new pa_allocator();
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->ref.assign(num_blocks, 0);
    a->stack.resize(num_blocks);
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = init_free_order ? init_free_order[i] : i;
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return PA_ERR_INVALID;
      }
      seen[b] = 1;
      a->stack[num_blocks - 1 - i] = b;  // element 0 of the order ends on top
    }
    *out = a;
    return PA_OK;
  } catch (...) {
    return PA_ERR_INVALID;
  }
}

PA_API void pa_alloc_destroy(pa_allocator* a) { delete a; }

PA_API int32_t pa_alloc_num_free(const pa_allocator* a) {
  return a ? (int32_t)a->stack.size() : -1;
}

PA_API int32_t pa_alloc_num_seqs(const pa_allocator* a) {
  return a ? (int32_t)a->seqs.size() : -1;
}

PA_API int32_t pa_block_refcount(const pa_allocator* a, int32_t block) {
  if (!a || block < 0 || block >= a->num_blocks) return -1;
  return a->ref[block];
}

PA_API pa_status pa_seq_add(pa_allocator* a, int64_t seq) {
  if (!a) return PA_ERR_INVALID;
  try {
    if (!a->seqs.emplace(seq, Sequence()).second) return PA_ERR_EXISTS;
  } catch (...) {
    return PA_ERR_INVALID;
  }
  return PA_OK;
}

PA_API pa_status pa_seq_fork(pa_allocator* a, int64_t parent, int64_t child) {
  if (!a) return PA_ERR_INVALID;
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  if (a->seqs.count(child)) return PA_ERR_EXISTS;
  try {
    Sequence copy = it->second;
    a->seqs.emplace(child, std::move(copy));
  } catch (...) {
    return PA_ERR_INVALID;
  }
  for (int32_t b : a->seqs[child].blocks) a->ref[b] += 1;
  return PA_OK;
}

PA_API pa_status pa_seq_append_slot(pa_allocator* a, int64_t seq, int64_t* slot,
                                    int32_t* cow_src, int32_t* cow_dst) {
  if (!a || !slot || !cow_src || !cow_dst) return PA_ERR_INVALID;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  Sequence& s = it->second;
  const int32_t tail_ref = s.blocks.empty() ? 0 : a->ref[s.blocks.back()];
  if (a->needs_block(s, tail_ref) && a->stack.empty()) return PA_ERR_NO_BLOCKS;
  a->append(s, slot, cow_src, cow_dst);
  return PA_OK;
}

PA_API pa_status pa_seq_append_slots(pa_allocator* a, const int64_t* seqs, int32_t n,
                                     int64_t* slots, int32_t* cow_pairs, int32_t* num_cow) {
  if (!a || n < 0 || (n > 0 && (!seqs || !slots || !cow_pairs)) || !num_cow)
    return PA_ERR_INVALID;
  *num_cow = 0;
  std::vector<Sequence*> targets;
  try {
    targets.reserve(n);
    std::unordered_set<int64_t> seen;
    for (int32_t i = 0; i < n; ++i) {
      auto it = a->seqs.find(seqs[i]);
      if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
      if (!seen.insert(seqs[i]).second) return PA_ERR_INVALID;
      targets.push_back(&it->second);
    }
    // Count the fresh blocks the whole step needs, replaying the refcount
    // drops of earlier copies in the batch (siblings sharing one tail: all
    // but the last holder copy).
    std::unordered_map<int32_t, int32_t> ref_now;
    int64_t need = 0;
    for (Sequence* s : targets) {
      int32_t tail_ref = 0;
      if (!s->blocks.empty()) {
        int32_t tail = s->blocks.back();
        auto r = ref_now.find(tail);
        tail_ref = r == ref_now.end() ? a->ref[tail] : r->second;
        if (s->len % a->block_size != 0 && tail_ref > 1) ref_now[tail] = tail_ref - 1;
      }
      if (a->needs_block(*s, tail_ref)) ++need;
    }
    if (need > (int64_t)a->stack.size()) return PA_ERR_NO_BLOCKS;
  } catch (...) {
    return PA_ERR_INVALID;
  }
  int32_t c = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src, dst;
    a->append(*targets[i], &slots[i], &src, &dst);
    if (src >= 0) {
      cow_pairs[2 * c] = src;
      cow_pairs[2 * c + 1] = dst;
      ++c;
    }
  }
  *num_cow = c;
  return PA_OK;
}

PA_API pa_status pa_seq_free(pa_allocator* a, int64_t seq) {
  if (!a) return PA_ERR_INVALID;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  for (int32_t b : it->second.blocks) {
    a->ref[b] -= 1;
    if (a->ref[b] == 0) a->release(b);
  }
  a->seqs.erase(it);
  return PA_OK;
}

PA_API pa_status pa_prefix_register(pa_allocator* a, int64_t seq, const int32_t* tokens,
                                    int32_t n_tokens, uint64_t salt, int32_t* n_registered) {
  if (!a || n_tokens < 0 || (n_tokens > 0 && !tokens) || !n_registered) return PA_ERR_INVALID;
  *n_registered = 0;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  const Sequence& s = it->second;
  const int32_t full = (n_tokens < s.len ? n_tokens : s.len) / a->block_size;
  try {
    Key k = root_key(salt);
    for (int32_t i = 0; i < full; ++i) {
      k = next_key(k, tokens + (int64_t)i * a->block_size, a->block_size);
      const int32_t b = s.blocks[i];
      if (a->prefix.count(k) || a->key_of.count(b)) continue;  // first registration wins
      a->prefix.emplace(k, b);
      a->key_of.emplace(b, k);
      ++*n_registered;
    }
  } catch (...) {
    return PA_ERR_INVALID;
  }
  return PA_OK;
}

PA_API int32_t pa_prefix_match(const pa_allocator* a, const int32_t* tokens, int32_t n_tokens,
                               uint64_t salt) {
  if (!a || n_tokens < 0 || (n_tokens > 0 && !tokens)) return -1;
  // at least one token stays out of the match: it must be prefilled
  const int32_t max_blocks = n_tokens > 0 ? (n_tokens - 1) / a->block_size : 0;
  return a->match(tokens, n_tokens, salt, max_blocks, nullptr) * a->block_size;
}

PA_API pa_status pa_seq_add_cached(pa_allocator* a, int64_t seq, const int32_t* tokens,
                                   int32_t n_tokens, uint64_t salt, int32_t* n_cached) {
  if (!a || n_tokens < 0 || (n_tokens > 0 && !tokens) || !n_cached) return PA_ERR_INVALID;
  *n_cached = 0;
  if (a->seqs.count(seq)) return PA_ERR_EXISTS;
  try {
    Sequence s;
    const int32_t max_blocks = n_tokens > 0 ? (n_tokens - 1) / a->block_size : 0;
    a->match(tokens, n_tokens, salt, max_blocks, &s.blocks);
    s.len = (int32_t)s.blocks.size() * a->block_size;
    a->seqs.emplace(seq, s);
    for (int32_t b : s.blocks) a->ref[b] += 1;
    *n_cached = s.len;
  } catch (...) {
    return PA_ERR_INVALID;
  }
  return PA_OK;
}

PA_API int32_t pa_prefix_num_entries(const pa_allocator* a) {
  return a ? (int32_t)a->prefix.size() : -1;
}

PA_API int32_t pa_seq_len(const pa_allocator* a, int64_t seq) {
  if (!a) return -1;
  auto it = a->seqs.find(seq);
  return it == a->seqs.end() ? -1 : it->second.len;
}

PA_API int32_t pa_seq_num_blocks(const pa_allocator* a, int64_t seq) {
  if (!a) return -1;
  auto it = a->seqs.find(seq);
  return it == a->seqs.end() ? -1 : (int32_t)it->second.blocks.size();
}

PA_API pa_status pa_seq_block_table(const pa_allocator* a, int64_t seq, int32_t* out,
                                    int32_t cap, int32_t* n) {
  if (!a || !n || cap < 0 || (cap > 0 && !out)) return PA_ERR_INVALID;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  const std::vector<int32_t>& b = it->second.blocks;
  *n = (int32_t)b.size();
  for (int32_t i = 0; i < cap && i < (int32_t)b.size(); ++i) out[i] = b[i];
  return PA_OK;
}

PA_API const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_NO_BLOCKS: return "no free KV blocks";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_UNKNOWN_SEQ: return "unknown sequence";
    case PA_ERR_EXISTS: return "sequence already exists";
  }
  return "unknown status";
}

}  // extern "C"
