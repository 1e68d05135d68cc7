"""Reference model of the paged-KV block manager (pure Python, slow, plain).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT: only tests/ may use it.  The
native allocator in the HIP library is checked against this model on seeded
operation sequences; the two share no code.

Behaviour, with the passage each rule follows:
  * A sequence's KV lives in fixed-size blocks of `block_size` tokens; a
    per-sequence block table lists its physical block ids in logical order
    (wiblog.cn, "AI 推理系列（十六）：PagedAttention", section "PagedAttention
    如何把连续序列映射到离散显存块").
  * Appending one token (the same section's flowchart): if the current last
    block is full -- equivalently len % block_size == 0, which includes the
    empty sequence -- a new physical block is taken from the free pool and
    appended to the table; otherwise the token goes to the next slot of the
    last block.  The returned slot is block * block_size + len % block_size.
  * Blocks are taken on demand from a global free pool and returned to it as
    soon as a sequence finishes; the tables of running sequences are not
    touched (bmjup.com, "PagedAttention：大模型推理性能优化的核心技术解析",
    section "PagedAttention 的核心工作机制与创新", item 3 "动态内存分配";
    wiblog.cn, section "Continuous Batching 为什么依赖可快速回收的 KV Cache").
  * Sharing: a forked sequence references the same physical blocks and each
    block keeps a reference count (kongchang.com, "PagedAttention原理详解",
    section "PagedAttention的三大核心优势", second advantage: parallel
    sampling and beam search share prefix blocks with reference counts and
    copy-on-write).  A block is copied only when a sequence must write into a
    block that another sequence also references (bmjup.com, same section,
    item 2 "写入时拷贝（Copy-on-Write）"; wiblog.cn, section "Copy-on-Write、
    并行采样与 Prefix Caching 不是同一件事").
Readings where the pages are silent:
  * Copy-on-write is decided at append time: the writer whose last block is
    partly filled and has refcount > 1 takes a fresh block, the old block's
    refcount drops by one and (old, fresh) is reported as a copy pair; the
    slot then lands in the fresh block.  The last holder (refcount 1) writes
    in place.
  * Free-pool order: a stack.  It starts as `init_free_order` with element 0
    on top (handed out first); a freed block is pushed on top.  free() walks
    a table in logical order.
  * Out of blocks: the call fails and leaves the state unchanged.
Prefix cache (wiblog.cn, section "Copy-on-Write、并行采样与 Prefix Caching 不是
同一件事": a cache key, exact token-sequence matching under one model
configuration, a lifetime for cached blocks, and the unmatched suffix still
prefilled).  Readings where the page is silent:
  * Only full blocks are cached.  The key of block i of a sequence is
    (salt, the token ids 0 .. (i+1) * block_size - 1): the whole prefix up to
    the block's end, under the caller's configuration tag.
  * register(seq, tokens, salt) indexes the sequence's full blocks (those
    covered by both its length and `tokens`); a key already indexed, or a
    block already indexed under a key, is left alone (first one wins).
  * match(tokens, salt): the longest run of leading full blocks whose keys
    are indexed, leaving at least one token unmatched; returns tokens.
  * add_cached(seq, tokens, salt): a new sequence referencing the matched
    blocks (refcount + 1), of length match(tokens, salt).
  * An entry lives while its block is referenced: it is dropped when the
    block returns to the free pool.
"""


class NoBlocks(Exception):
    """The free pool cannot satisfy the request; state is unchanged."""


class BlockManagerModel:
    def __init__(self, num_blocks, block_size, init_free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if init_free_order is None else [int(b) for b in init_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("init_free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self._stack = list(reversed(order))  # top of the stack = end of the list
        self._ref = [0] * num_blocks
        self._seqs = {}  # seq id -> {"blocks": [...], "len": int}
        self._cache = {}   # (salt, token prefix tuple) -> block
        self._key_of = {}  # block -> its key in _cache

    # ---- queries ----
    def num_free(self):
        return len(self._stack)

    def refcount(self, block):
        return self._ref[block]

    def seq_len(self, seq):
        return self._seqs[seq]["len"]

    def block_table(self, seq):
        return list(self._seqs[seq]["blocks"])

    def has_seq(self, seq):
        return seq in self._seqs

    # ---- operations ----
    def _take(self):
        b = self._stack.pop()
        assert self._ref[b] == 0
        self._ref[b] = 1
        return b

    def add(self, seq):
        if seq in self._seqs:
            raise KeyError(f"sequence {seq} exists")
        self._seqs[seq] = {"blocks": [], "len": 0}

    def fork(self, parent, child):
        if parent not in self._seqs:
            raise KeyError(f"sequence {parent} unknown")
        if child in self._seqs:
            raise KeyError(f"sequence {child} exists")
        p = self._seqs[parent]
        for b in p["blocks"]:
            self._ref[b] += 1
        self._seqs[child] = {"blocks": list(p["blocks"]), "len": p["len"]}

    def append_slot(self, seq):
        """Returns (slot, cow_src, cow_dst); cow_* are -1 when nothing is copied."""
        if seq not in self._seqs:
            raise KeyError(f"sequence {seq} unknown")
        st = self._seqs[seq]
        bs = self.block_size
        pos = st["len"] % bs
        if pos == 0:  # last block full (or no block yet): take a new one
            if not self._stack:
                raise NoBlocks()
            b = self._take()
            st["blocks"].append(b)
            st["len"] += 1
            return b * bs, -1, -1
        tail = st["blocks"][-1]
        if self._ref[tail] > 1:  # shared partial tail: copy on write
            if not self._stack:
                raise NoBlocks()
            fresh = self._take()
            self._ref[tail] -= 1
            st["blocks"][-1] = fresh
            st["len"] += 1
            return fresh * bs + pos, tail, fresh
        st["len"] += 1
        return tail * bs + pos, -1, -1

    def free(self, seq):
        if seq not in self._seqs:
            raise KeyError(f"sequence {seq} unknown")
        for b in self._seqs.pop(seq)["blocks"]:
            self._ref[b] -= 1
            if self._ref[b] == 0:
                self._stack.append(b)
                if b in self._key_of:
                    del self._cache[self._key_of.pop(b)]

    # ---- prefix cache ----
    def register(self, seq, tokens, salt=0):
        if seq not in self._seqs:
            raise KeyError(f"sequence {seq} unknown")
        st, bs = self._seqs[seq], self.block_size
        tokens = [int(t) for t in tokens]
        added = 0
        for i in range(min(len(tokens), st["len"]) // bs):
            key = (salt, tuple(tokens[:(i + 1) * bs]))
            b = st["blocks"][i]
            if key in self._cache or b in self._key_of:
                continue
            self._cache[key] = b
            self._key_of[b] = key
            added += 1
        return added

    def _matched_blocks(self, tokens, salt):
        tokens = [int(t) for t in tokens]
        bs, out = self.block_size, []
        while (len(out) + 1) * bs <= len(tokens) - 1:  # at least one token left to prefill
            key = (salt, tuple(tokens[:(len(out) + 1) * bs]))
            if key not in self._cache:
                break
            out.append(self._cache[key])
        return out

    def match(self, tokens, salt=0):
        return len(self._matched_blocks(tokens, salt)) * self.block_size

    def add_cached(self, seq, tokens, salt=0):
        if seq in self._seqs:
            raise KeyError(f"sequence {seq} exists")
        blocks = self._matched_blocks(tokens, salt)
        for b in blocks:
            self._ref[b] += 1
        self._seqs[seq] = {"blocks": blocks, "len": len(blocks) * self.block_size}
        return len(blocks) * self.block_size

    def num_cache_entries(self):
        return len(self._cache)

    # ---- invariants ----
    def check_invariants(self):
        bs = self.block_size
        counted = [0] * self.num_blocks
        for st in self._seqs.values():
            assert len(st["blocks"]) == -(-st["len"] // bs), "blocks != ceil(len / block_size)"
            for b in st["blocks"]:
                counted[b] += 1
        assert counted == self._ref, "refcounts differ from table references"
        free = set(self._stack)
        assert len(free) == len(self._stack), "a block is on the free pool twice"
        for b in range(self.num_blocks):
            assert (b in free) == (self._ref[b] == 0), "free pool / refcount mismatch"
        assert len(self._cache) == len(self._key_of), "prefix cache maps differ"
        for key, b in self._cache.items():
            assert self._key_of[b] == key and self._ref[b] > 0, "cached block not referenced"
            assert len(key[1]) % bs == 0 and key[1], "cache key not a whole number of blocks"
