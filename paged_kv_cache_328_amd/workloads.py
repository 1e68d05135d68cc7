"""Seeded synthetic workloads for paged decode attention.

This module only draws inputs: context lengths, which physical blocks each
sequence owns, and N(0, 1) query / key / value data rounded to the storage
type.  It holds none of the attention arithmetic, imports nothing from the
kernels' binding or from the CPU oracle, and is shared by the tests, the
benchmark and the smoke check so that both sides see the same bits.

Workload shapes (no trained weights or serving traces are available, so the
shapes stand in for the pages' LLaMA workloads):
  tiny_f32        4 seqs, contexts {5,16,17,33}, 2 q = 2 KV heads, D 64, f32,
                  block 16, pool of 32 blocks (seeded permutation).
  llama13b_f16    batch 16, 40 q = 40 KV heads, D 128, f16, block 16,
                  contexts uniform in [1024, 1280], 20,000-block pool.
  mixed_gqa_bf16  batch 64, 32 q / 8 KV heads, D 128, bf16, block 16,
                  contexts log-uniform in [32, 8192], fragmented pool; the
                  step writes the 64 new tokens.
  cow_bf16        32 seqs sharing a 2048-token prefix + private suffixes of
                  uniform 1..512 tokens, 32 q / 8 KV heads, D 128, bf16,
                  block 32, 4096-block pool (built by driving a block
                  manager, see tests).
  long_bf16       batch 4, contexts {16384, 32768, 65536, 131072}, 64 q /
                  8 KV heads, D 128, bf16, block 16, split-K partitions of
                  512 tokens, 16,384-block pool.
Storage arrays: f32 -> float32, f16 -> float16, bf16 -> uint16 bit patterns.
Pool shapes: k [NB, Hkv, D/x, BS, x], v [NB, Hkv, D, BS], x = 16 B / element.
"""
from dataclasses import dataclass, field
import math

import numpy as np

NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
CONFIG_INDEX = {"tiny_f32": 1, "llama13b_f16": 2, "mixed_gqa_bf16": 3, "cow_bf16": 4, "long_bf16": 5,
                "prefill_llama13b_f16": 6}


def base_seed(name):
    return 328_000 + CONFIG_INDEX[name]


def round_to_storage(x32, dtype):
    """fp32 array -> storage array of `dtype`, rounding to nearest even."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f32":
        return x32
    if dtype == "f16":
        return x32.astype(np.float16)
    import torch  # bf16 rounding: torch's CPU cast is round-to-nearest-even
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def storage_to_f32(a, dtype):
    """Storage array -> float32 (exact for all three types)."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def nan_bits(dtype):
    return {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}[dtype]


def pool_shapes(NB, Hkv, D, BS, dtype):
    x = 16 // ELEM_BYTES[dtype]
    return (NB, Hkv, D // x, BS, x), (NB, Hkv, D, BS)


def kv_cache_bytes(layers, tokens, kv_heads, head_dim, elem_bytes):
    """KV cache size of `tokens` tokens: 2 (K and V) x layers x tokens x
    kv_heads x head_dim x element size (kongchang.com, "PagedAttention原理详解",
    section "显存消耗的三大来源")."""
    return 2 * layers * tokens * kv_heads * head_dim * elem_bytes


@dataclass
class DecodeCase:
    name: str
    dtype: str
    S: int
    Hq: int
    Hkv: int
    D: int
    BS: int
    NB: int
    scale: float
    partition_size: int
    context_lens: np.ndarray          # [S] int32 (includes the step's new token)
    block_tables: np.ndarray          # [R, S, max_blocks] int32
    q: np.ndarray                     # [R, S, Hq, D] storage
    k_cache: np.ndarray = None        # pool (storage) or None when filled on the device
    v_cache: np.ndarray = None
    new_k: np.ndarray = None          # [R, S, Hkv, D] storage: the step's new token
    new_v: np.ndarray = None
    slot_mapping: np.ndarray = None   # [R, S] int64: slot of each new token
    referenced: np.ndarray = None     # [NB] bool: block referenced by some table
    trap_block: int = 0               # unreferenced block used to pad table rows
    kv_dtype: str = None              # cache type: same as dtype, "i8" or "fp8" (8-bit pools)
    extra: dict = field(default_factory=dict)

    @property
    def replicas(self):
        return self.block_tables.shape[0]

    @property
    def max_blocks(self):
        return self.block_tables.shape[2]

    @property
    def max_context(self):
        return int(self.context_lens.max()) if self.S else 0

    def kv_bytes(self):
        """K + V bytes over every context (one replica); for 8-bit pools the
        codes plus each token's two fp32 scales."""
        tokens = int(self.context_lens.astype(np.int64).sum()) * self.Hkv
        if is_q8(self.kv_dtype):
            return 2 * tokens * (self.D + 4)
        return 2 * tokens * self.D * ELEM_BYTES[self.dtype]


def _blocks_needed(lens, BS):
    return [-(-int(c) // BS) for c in lens]


def _tables_from_lists(lists, max_blocks, pad):
    t = np.full((len(lists), max_blocks), pad, np.int32)
    for s, blocks in enumerate(lists):
        t[s, :len(blocks)] = blocks
    return t


def _fill_pool(rng_k, rng_v, NB, Hkv, D, BS, dtype, referenced, chunk_blocks=2048):
    """Pools with N(0,1) data in referenced blocks and NaN elsewhere."""
    ks, vs = pool_shapes(NB, Hkv, D, BS, dtype)
    k = np.full(ks, nan_bits(dtype), NP_STORAGE[dtype])
    v = np.full(vs, nan_bits(dtype), NP_STORAGE[dtype])
    ids = np.flatnonzero(referenced)
    for i in range(0, ids.size, chunk_blocks):
        sel = ids[i:i + chunk_blocks]
        k[sel] = round_to_storage(rng_k.standard_normal((sel.size,) + ks[1:], dtype=np.float32), dtype)
        v[sel] = round_to_storage(rng_v.standard_normal((sel.size,) + vs[1:], dtype=np.float32), dtype)
    return k, v


def is_q8(kv_dtype):
    """Whether a cache type is an 8-bit code format (INT8 or FP8 E4M3)."""
    return kv_dtype in ("i8", "fp8")


def i8_tile_bytes(D, BS):
    """Bytes of one (block, KV head) tile of an INT8 pool: D*BS codes, then
    BS fp32 scales."""
    return D * BS + 4 * BS


def _fp8_codes(rng, shape):
    """Random finite E4M3 codes: random sign, exponent field 4..13 (magnitudes
    2^-3 .. 2^6 * 1.875), or 0 (zeros and subnormals) for about 3% of them,
    random mantissa -- drawn as bits, no conversion."""
    e = np.where(rng.random(shape) < 0.03, 0, rng.integers(4, 14, size=shape))
    m = rng.integers(0, 8, size=shape)
    sgn = rng.integers(0, 2, size=shape)
    return ((sgn << 7) | (e << 3) | m).astype(np.uint8)


def _fill_pool_i8(rng_k, rng_v, NB, Hkv, D, BS, referenced, chunk_blocks=2048, fmt="i8"):
    """8-bit pools [NB, Hkv, tile] (uint8).  Referenced blocks get random codes
    (INT8: a rounded normal of spread 40, clipped to [-127, 127]; FP8: see
    _fp8_codes) and random scales uniform in [0.01, 0.04]; other blocks get
    code 0x7F (an FP8 NaN) and NaN scales.  Only random numbers are drawn
    here: no quantisation is performed."""
    tile = i8_tile_bytes(D, BS)
    out = []
    for rng in (rng_k, rng_v):
        pool = np.full((NB, Hkv, tile), 0x7F, np.uint8)
        pool[:, :, D * BS:] = np.frombuffer(np.full(BS, np.nan, np.float32).tobytes(), np.uint8)
        ids = np.flatnonzero(referenced)
        for i in range(0, ids.size, chunk_blocks):
            sel = ids[i:i + chunk_blocks]
            if fmt == "fp8":
                codes = _fp8_codes(rng, (sel.size, Hkv, D * BS))
            else:
                codes = np.clip(np.rint(40.0 * rng.standard_normal((sel.size, Hkv, D * BS))), -127,
                                127).astype(np.int8).view(np.uint8)
            scales = rng.uniform(0.01, 0.04, size=(sel.size, Hkv, BS)).astype(np.float32)
            pool[sel, :, :D * BS] = codes
            pool[sel, :, D * BS:] = scales.view(np.uint8).reshape(sel.size, Hkv, 4 * BS)
        out.append(pool)
    return out[0], out[1]


def _finish(name, dtype, S, Hq, Hkv, D, BS, NB, partition_size, lens, table_lists, rngs, fill,
            with_new_token, kv_dtype=None):
    """Common tail: tables, q, pools, new tokens."""
    R = len(table_lists)
    max_blocks = max(1, max(_blocks_needed(lens, BS)))
    referenced = np.zeros(NB, bool)
    for lists in table_lists:
        for blocks in lists:
            referenced[blocks] = True
    unref = np.flatnonzero(~referenced)
    trap = int(unref[0]) if unref.size else 0
    tables = np.stack([_tables_from_lists(lists, max_blocks, trap) for lists in table_lists])
    q = round_to_storage(rngs["q"].standard_normal((R, S, Hq, D), dtype=np.float32), dtype)
    case = DecodeCase(name=name, dtype=dtype, S=S, Hq=Hq, Hkv=Hkv, D=D, BS=BS, NB=NB,
                      scale=float(np.float32(1.0 / math.sqrt(D))), partition_size=partition_size,
                      context_lens=np.asarray(lens, np.int32), block_tables=tables, q=q,
                      referenced=referenced, trap_block=trap)
    case.kv_dtype = kv_dtype or dtype
    if fill and is_q8(case.kv_dtype):
        case.k_cache, case.v_cache = _fill_pool_i8(rngs["k"], rngs["v"], NB, Hkv, D, BS, referenced,
                                                   fmt=case.kv_dtype)
    elif fill:
        case.k_cache, case.v_cache = _fill_pool(rngs["k"], rngs["v"], NB, Hkv, D, BS, dtype, referenced)
    if with_new_token:
        case.new_k = round_to_storage(rngs["new"].standard_normal((R, S, Hkv, D), dtype=np.float32), dtype)
        case.new_v = round_to_storage(rngs["new"].standard_normal((R, S, Hkv, D), dtype=np.float32), dtype)
        # the new token is logical position c-1; slot numbering is block * BS + offset
        slots = np.empty((R, S), np.int64)
        for r in range(R):
            for s in range(S):
                t = int(lens[s]) - 1
                slots[r, s] = int(tables[r, s, t // BS]) * BS + t % BS if t >= 0 else -1
        case.slot_mapping = slots
    return case


def _rngs(seed):
    names = ["lens", "perm", "q", "k", "v", "new", "churn"]
    return dict(zip(names, [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(len(names))]))


def _permutation_tables(lens, BS, perm, replicas):
    """Replica r takes the next run of the permutation, in (seq, logical block) order."""
    need = sum(_blocks_needed(lens, BS))
    if replicas * need > perm.size:
        raise ValueError(f"pool too small: {replicas} replicas x {need} blocks > {perm.size}")
    out = []
    for r in range(replicas):
        it = iter(perm[r * need:(r + 1) * need].tolist())
        out.append([[next(it) for _ in range(n)] for n in _blocks_needed(lens, BS)])
    return out


def tiny_f32(seed=None, replicas=1, fill=True):
    name = "tiny_f32"
    rngs = _rngs(base_seed(name) if seed is None else seed)
    lens = [5, 16, 17, 33]
    NB, BS = 32, 16
    perm = rngs["perm"].permutation(NB)
    tables = _permutation_tables(lens, BS, perm, replicas)
    return _finish(name, "f32", 4, 2, 2, 64, BS, NB, 0, lens, tables, rngs, fill, True)


def llama13b_f16(seed=None, replicas=1, fill=True, num_blocks=None, kv_dtype=None, block_size=16):
    """num_blocks defaults to 20,000 blocks of 16 tokens (the same pool bytes
    at any block size)."""
    name = "llama13b_f16"
    rngs = _rngs(base_seed(name) if seed is None else seed)
    lens = rngs["lens"].integers(1024, 1280, size=16, endpoint=True).tolist()
    BS = block_size
    num_blocks = num_blocks or 20000 * 16 // BS
    perm = rngs["perm"].permutation(num_blocks)
    tables = _permutation_tables(lens, BS, perm, replicas)
    return _finish(name, "f16", 16, 40, 40, 128, BS, num_blocks, 0, lens, tables, rngs, fill, True,
                   kv_dtype)


def long_bf16(seed=None, replicas=1, fill=True, kv_dtype=None, block_size=16):
    name = "long_bf16"
    rngs = _rngs(base_seed(name) if seed is None else seed)
    lens = [16384, 32768, 65536, 131072]
    BS = block_size
    NB = 16384 * 16 // BS * replicas
    perm = rngs["perm"].permutation(NB)
    tables = _permutation_tables(lens, BS, perm, replicas)
    return _finish(name, "bf16", 4, 64, 8, 128, BS, NB, max(512, BS), lens, tables, rngs, fill, True,
                   kv_dtype)


def _log_uniform_lens(rng, n, lo, hi):
    return np.clip(np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))), lo, hi).astype(int).tolist()


def mixed_gqa_bf16(seed=None, replicas=1, fill=True, kv_dtype=None, block_size=16):
    """Fragmented pool: the free pool starts as a seeded permutation used as a
    stack; dummy sequences take blocks until 60% of the pool is in use, a
    seeded half of them is released, then the real sequences take their
    blocks round-robin, one block at a time.  The real sequences' blocks end up
    scattered between live dummy blocks and recycled holes."""
    name = "mixed_gqa_bf16"
    rngs = _rngs(base_seed(name) if seed is None else seed)
    S, BS = 64, block_size
    lens = _log_uniform_lens(rngs["lens"], S, 32, 8192)
    need_one = sum(_blocks_needed(lens, BS))
    NB = int(math.ceil(2.0 * need_one * replicas / 1024.0)) * 1024
    stack = rngs["perm"].permutation(NB).tolist()
    churn = rngs["churn"]
    table_lists = []
    budget = NB // replicas
    for _ in range(replicas):
        dummies, held = [], 0
        while held < 0.6 * budget:
            want = -(-int(_log_uniform_lens(churn, 1, 32, 8192)[0]) // BS)
            want = min(want, int(0.6 * budget) - held + 1)
            dummies.append([stack.pop() for _ in range(want)])
            held += want
        for i in churn.permutation(len(dummies))[: len(dummies) // 2]:
            stack.extend(dummies[i])
        lists = [[] for _ in range(S)]
        remaining = _blocks_needed(lens, BS)
        while any(remaining):
            for s in range(S):
                if remaining[s]:
                    if not stack:
                        raise RuntimeError("fragmented pool recipe ran out of blocks")
                    lists[s].append(stack.pop())
                    remaining[s] -= 1
        table_lists.append(lists)
    return _finish(name, "bf16", S, 32, 8, 128, BS, NB, 0, lens, table_lists, rngs, fill, True,
                   kv_dtype)


def cow_plan(seed=None):
    """Inputs of the shared-prefix / copy-on-write workload: the pool's
    initial free order, the suffix lengths and the data.  The block tables come
    from driving a block manager (see the tests) -- this only draws numbers."""
    name = "cow_bf16"
    rngs = _rngs(base_seed(name) if seed is None else seed)
    n, prefix, BS, NB = 32, 2048, 32, 4096
    Hq, Hkv, D = 32, 8, 128
    suffix = rngs["lens"].integers(1, 512, size=n, endpoint=True).tolist()
    init_free_order = rngs["perm"].permutation(NB).astype(np.int32)
    ks, vs = pool_shapes(NB, Hkv, D, BS, "bf16")
    k = round_to_storage(rngs["k"].standard_normal(ks, dtype=np.float32), "bf16")
    v = round_to_storage(rngs["v"].standard_normal(vs, dtype=np.float32), "bf16")
    q = round_to_storage(rngs["q"].standard_normal((n, Hq, D), dtype=np.float32), "bf16")
    new_k = round_to_storage(rngs["new"].standard_normal((n, Hkv, D), dtype=np.float32), "bf16")
    new_v = round_to_storage(rngs["new"].standard_normal((n, Hkv, D), dtype=np.float32), "bf16")
    return dict(name=name, dtype="bf16", n=n, prefix=prefix, suffix=suffix, BS=BS, NB=NB, Hq=Hq,
                Hkv=Hkv, D=D, scale=float(np.float32(1.0 / math.sqrt(D))),
                init_free_order=init_free_order, k_cache=k, v_cache=v, q=q, new_k=new_k, new_v=new_v)


def random_case(seed, S, Hq, Hkv, D, BS, dtype, lens, NB=None, partition_size=0, fill=True,
                kv_dtype=None):
    """A free-form case (edge cases and sweeps): seeded permutation pool."""
    rngs = _rngs(seed)
    need = sum(_blocks_needed(lens, BS))
    NB = NB if NB is not None else max(need + 2, 4)
    perm = rngs["perm"].permutation(NB)
    tables = _permutation_tables(lens, BS, perm, 1)
    return _finish("random", dtype, S, Hq, Hkv, D, BS, NB, partition_size, lens, tables, rngs, fill, True,
                   kv_dtype)


def shared_prefix_case(seed, groups, Hq, Hkv, D, BS, dtype, kv_dtype=None, fill=True):
    """Decode batch whose sequences share prefix blocks.  groups is a list of
    (shared_blocks, [suffix tokens of each member]): a group's members point
    their first shared_blocks table entries at the same physical blocks and
    have private blocks for their own suffix.  Sequences are numbered group
    by group.  Returns (DecodeCase, group_start, shared_tokens) with
    shared_tokens[g] = shared_blocks * BS."""
    rngs = _rngs(seed)
    lens, starts, shared = [], [0], []
    for nb, suffixes in groups:
        for x in suffixes:
            lens.append(nb * BS + int(x))
        starts.append(starts[-1] + len(suffixes))
        shared.append(nb * BS)
    need = sum(nb for nb, _ in groups) + sum(-(-int(x) // BS) for _, sfx in groups for x in sfx)
    NB = need + 4
    it = iter(rngs["perm"].permutation(NB).tolist())
    lists = []
    for nb, suffixes in groups:
        prefix = [next(it) for _ in range(nb)]
        for x in suffixes:
            lists.append(prefix + [next(it) for _ in range(-(-int(x) // BS))])
    case = _finish("shared_prefix", dtype, len(lens), Hq, Hkv, D, BS, NB, 0, lens, [lists], rngs,
                   fill, True, kv_dtype)
    return case, np.asarray(starts, np.int32), np.asarray(shared, np.int32)


@dataclass
class PrefillCase:
    """A paged (chunked) prefill step: sequence s has context_lens[s] cached
    tokens, the last chunks[s] of which are the chunk being prefilled (its
    K/V already in the pool); q holds the chunks' rows back to back."""
    name: str
    dtype: str
    kv_dtype: str
    S: int
    Hq: int
    Hkv: int
    D: int
    BS: int
    NB: int
    scale: float
    context_lens: np.ndarray
    query_start: np.ndarray
    block_tables: np.ndarray  # [S, max_blocks]
    q: np.ndarray             # [T, Hq, D] storage
    k_cache: np.ndarray = None
    v_cache: np.ndarray = None

    @property
    def max_query_len(self):
        return int(np.max(np.diff(self.query_start))) if self.S else 0

    @property
    def max_context(self):
        return int(self.context_lens.max()) if self.S else 0

    def flops(self):
        """Multiply-adds of QK and PV counted as 2 flops each: 4 * D per (row,
        head, key) pair, keys 0..p for a row at position p."""
        tot = 0
        for c, n in zip(self.context_lens.tolist(), np.diff(self.query_start).tolist()):
            tot += sum(range(c - n + 1, c + 1))  # keys seen by the chunk's rows
        return 4 * self.D * self.Hq * tot


def prefill_case(seed, priors, chunks, Hq, Hkv, D, BS, dtype, kv_dtype=None, NB=None, fill=True,
                 name="prefill"):
    """Sequence s: priors[s] earlier tokens plus a chunk of chunks[s] tokens
    (context = prior + chunk).  Seeded permutation pool as for decode."""
    rngs = _rngs(seed)
    lens = [int(a) + int(b) for a, b in zip(priors, chunks)]
    need = sum(_blocks_needed(lens, BS))
    NB = NB if NB is not None else max(need + 2, 4)
    perm = rngs["perm"].permutation(NB)
    tables = _permutation_tables(lens, BS, perm, 1)
    dec = _finish(name, dtype, len(lens), Hq, Hkv, D, BS, NB, 0, lens, tables, rngs, fill, False,
                  kv_dtype)
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = round_to_storage(rngs["q"].standard_normal((int(qs[-1]), Hq, D), dtype=np.float32), dtype)
    return PrefillCase(name=name, dtype=dtype, kv_dtype=dec.kv_dtype, S=len(lens), Hq=Hq, Hkv=Hkv,
                       D=D, BS=BS, NB=NB, scale=dec.scale, context_lens=dec.context_lens,
                       query_start=qs, block_tables=dec.block_tables[0], q=q, k_cache=dec.k_cache,
                       v_cache=dec.v_cache)


def prefill_llama13b_f16(seed=None, fill=True, kv_dtype=None, block_size=16):
    """Chunked prefill at LLaMA-13B shape: 8 sequences each prefill a 512-token
    chunk on top of 0..1536 earlier tokens (seeded), 40 heads, head_dim 128."""
    name = "prefill_llama13b_f16"
    seed = base_seed(name) if seed is None else seed
    rng = np.random.default_rng(seed)
    priors = rng.integers(0, 1536, size=8, endpoint=True).tolist()
    return prefill_case(seed + 1, priors, [512] * 8, 40, 40, 128, block_size, "f16", kv_dtype,
                        fill=fill, name=name)


BUILDERS = {
    "tiny_f32": tiny_f32,
    "llama13b_f16": llama13b_f16,
    "mixed_gqa_bf16": mixed_gqa_bf16,
    "long_bf16": long_bf16,
}
