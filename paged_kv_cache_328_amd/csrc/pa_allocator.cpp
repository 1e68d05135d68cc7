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
// Prefix Caching 不是同一件事").
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

}  // namespace

struct pa_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> stack;   // free pool; back() is handed out next
  std::vector<int32_t> ref;     // reference count per physical block
  std::unordered_map<int64_t, Sequence> seqs;

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
    if (a->ref[b] == 0) a->stack.push_back(b);
  }
  a->seqs.erase(it);
  return PA_OK;
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
