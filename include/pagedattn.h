/*
 * pagedattn.h -- C ABI of libpagedattn: paged decode attention on MI355X
 * (gfx950) plus the host-side block manager that feeds it.
 *
 * Sources (web pages on PagedAttention; cited below by site and section):
 *   bmjup.com        "PagedAttention：大模型推理性能优化的核心技术解析"
 *   wiblog.cn        "AI 推理系列（十六）：PagedAttention——为什么 vLLM 能把 GPU
 *                    显存“像操作系统一样”管理？"
 *   kongchang.com    "PagedAttention原理详解：GPU显存优化与模型路由技术"
 *   intelliparadigm.com "vLLM的Paged Attention技术：高效注意力机制解析"
 *
 * The method (PagedAttention): a sequence's KV cache lives in fixed-size
 * physical blocks of block_size tokens that sit anywhere in one device pool;
 * a per-sequence block table maps logical block i to its physical block id
 * (wiblog.cn, section "PagedAttention 如何把连续序列映射到离散显存块").
 * Decode attention reads the blocks in place through the table, without
 * first concatenating them (wiblog.cn, section "非连续 KV 为什么需要专门的
 * Attention Kernel").  The attention formula itself is the ordinary one
 * (wiblog.cn, opening section: paging is not a new attention formula).
 *
 * Pool layout (intelliparadigm.com, section "2.2 内存布局优化"), row-major,
 * x = 16 bytes / element size:
 *     k_cache [num_blocks, num_kv_heads, head_dim / x, block_size, x]
 *     v_cache [num_blocks, num_kv_heads, head_dim,     block_size]
 * One (block, KV head) tile is one contiguous run of head_dim * block_size
 * elements in each pool.
 *
 * Conventions for every entry point:
 *   - Every pointer argument of a device op is device memory owned by the
 *     caller; the library allocates no device memory and frees none (the
 *     one exception: pa_decode_static's fixed scratch array, below).
 *   - Device ops are enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and return without synchronising it.  PA_ERR_HIP means the
 *     launch itself failed; errors inside a kernel surface on the caller's
 *     next synchronisation.
 *   - Host-side arguments (sizes, dtype, alignment, workspace size) are
 *     validated and rejected with PA_ERR_INVALID / PA_ERR_UNSUPPORTED /
 *     PA_ERR_WORKSPACE before anything is launched.  Device contents (block
 *     ids, context lengths, slots) are preconditions; a violation gives
 *     unspecified results for the affected sequence or token, but the kernels
 *     clamp every index so that no access leaves the arrays described here.
 *   - No function throws or aborts; nothing is thread-safe unless stated.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_API __attribute__((visibility("default")))

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID = 1,      /* bad argument: null pointer, non-positive size, misalignment, ... */
  PA_ERR_UNSUPPORTED = 2,  /* valid but not compiled in: head_dim, block_size, dtype, group size */
  PA_ERR_NO_BLOCKS = 3,    /* block manager: free pool exhausted (state unchanged) */
  PA_ERR_HIP = 4,          /* a HIP runtime call or kernel launch failed */
  PA_ERR_WORKSPACE = 5,    /* pa_decode: workspace missing or smaller than required */
  PA_ERR_UNKNOWN_SEQ = 6,  /* block manager: sequence id not present */
  PA_ERR_EXISTS = 7        /* block manager: sequence id already present */
} pa_status;

/* Element types.  PA_I8 is a cache type only: INT8 KV-cache quantisation
 * (kongchang.com, section "量化技术：与PagedAttention正交的显存优化路径": INT8
 * halves the KV memory, orthogonal to paging).  An INT8 pool is
 * [num_blocks, num_kv_heads, tile] bytes; each (block, KV head) tile holds
 * head_dim * block_size codes (K: [head_dim/16][block_size][16], the printed K
 * layout with x = 16; V: [head_dim][block_size]) followed by block_size fp32
 * scales, one per token: tile = head_dim * block_size + 4 * block_size bytes.
 * A cached value is code * scale.  Codes are made symmetric per (token, KV
 * head) in fp32: scale = max|x| / 127, code = rint(x / scale) clamped to
 * [-127, 127] (a zero row has scale 0).
 * PA_FP8 is the other 8-bit cache type: the same pools, tiles and scales
 * with codes in the OCP E4M3 8-bit float (sign, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; largest
 * finite magnitude 448; S.1111.111 is NaN): scale = max|x| / 448, code = the
 * E4M3 value nearest to x / scale, ties to an even mantissa, magnitudes of
 * 448 and more saturated to 448 (the writes never make a NaN code). */
typedef enum pa_dtype { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_I8 = 3, PA_FP8 = 4 } pa_dtype;

/* Static, never-NULL text for a status code. */
PA_API const char* pa_status_string(pa_status s);

/* ------------------------------------------------------------------------
 * pa_decode -- one decode step of attention for every sequence.
 *
 * For sequence s with context length c = context_lens[s] and query head h
 * (KV head g = floor(h / G), G = num_q_heads / num_kv_heads, consecutive
 * grouping):
 *     x_t = scale * <q[s,h,:], K_t>,  t = 0..c-1 in logical order, where
 *           K_t / V_t are row (t mod block_size) of physical block
 *           block_tables[s][t / block_size], KV head g;
 *     out[s,h,:] = sum_t exp(x_t - max x) V_t / sum_t exp(x_t - max x).
 * c counts every cached token including the one written this step; c == 0
 * writes zeros.  Arithmetic: fp32 accumulation; 16-bit inputs feed the
 * matrix cores with the softmax weights rounded to the input type; out is
 * rounded once to the element type.
 *
 * Long contexts are split into partitions of `partition_size` tokens (the
 * PARTITION_SIZE split of intelliparadigm.com, sections "3.1 核函数签名解析"
 * and "3.2 执行层次结构"); each
 * partition yields (running max, sum, unnormalised output) and a second pass
 * merges them with the log-sum-exp rule.  partition_size == 0 lets the
 * library choose; otherwise it must be a positive multiple of 32 tokens and
 * of block_size.
 *
 * Layouts: q, out [num_seqs, num_q_heads, head_dim] of `dtype`;
 * block_tables [num_seqs, max_blocks_per_seq] int32; context_lens
 * [num_seqs] int32 with 0 <= c <= max_context_len <= max_blocks_per_seq *
 * block_size.  Entries of a table row past ceil(c / block_size) are never
 * read.  All pointers 16-byte aligned.
 * Supported: dtype f16 / bf16 / f32, head_dim 64 or 128, block_size 8, 16,
 * 32 or 64, any G = num_q_heads / num_kv_heads >= 1.  The caches hold dtype, or
 * (kv_dtype PA_I8 or PA_FP8, f16 / bf16 only) 8-bit codes whose values
 * value(code) * scale stand for K_t and V_t: each code is widened exactly to dtype for the
 * matrix cores, K's scale multiplies the token's logit and V's scale the
 * token's softmax weight before that weight is rounded to dtype.
 * The workspace (caller-allocated device memory, any contents) holds the
 * split-K partials; its size comes from pa_decode_workspace_bytes (0 when no
 * context spans more than one partition).  Two calls in flight at once must
 * not share a workspace.
 * ------------------------------------------------------------------------ */
typedef struct pa_decode_args {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;  /* host-known upper bound of context_lens */
  float scale;              /* usually 1 / sqrt(head_dim) */
  int32_t dtype;            /* pa_dtype of q and out (PA_F32, PA_F16, PA_BF16) */
  int32_t partition_size;   /* 0 = library choice */
  void* workspace;
  size_t workspace_bytes;
  /* Optional fused cache write of the step's new token (NULL, NULL = none).
   * k_new, v_new: [num_seqs, num_kv_heads, head_dim] of dtype, 16-byte
   * aligned, both set or both NULL.  When set, sequence s's token at logical
   * position context_lens[s] - 1 is taken from k_new[s] / v_new[s] rather than
   * from the cache, and is also stored, bit for bit, into that position's slot
   * (physical block block_tables[s][(c - 1) / block_size], row (c - 1) %
   * block_size).  The pool afterwards equals that of pa_write_kv with those
   * slots; the output equals pa_decode after that write up to the rounding
   * order of the one new token's contribution.  Sequences with c == 0 append
   * nothing.  The slot of position c - 1 must not be shared with another
   * sequence (copy-on-write it first with pa_copy_blocks). */
  const void* k_new;
  const void* v_new;
  /* pa_dtype of k_cache / v_cache: equal to dtype, or PA_I8 / PA_FP8 (8-bit
   * pools, see pa_dtype) with f16 / bf16 queries.  With an 8-bit pool a fused
   * append quantises the new token as pa_write_kv_i8 / pa_write_kv_fp8 does;
   * k_new / v_new stay of dtype. */
  int32_t kv_dtype;
  /* Optional host copy of context_lens ([num_seqs] int32 in host memory,
   * NULL = none), read during the call.  From the device lengths the library
   * knows only the bound max_context_len, so it launches a workgroup for
   * every (sequence, partition) pair that bound allows and the surplus ones
   * exit at once; given the host copy, the 16-bit and INT8 kernels launch
   * only the pairs that exist, and the merge pass covers only the sequences
   * that span more than one partition (none: no merge launch).  Values
   * outside [0, max_context_len] return
   * PA_ERR_INVALID.  The values must equal the device ones: where they
   * differ, the outputs are undefined (no access leaves the arguments'
   * buffers either way).  A launch recorded into a graph keeps the shape it
   * was recorded with, so leave this NULL under capture. */
  const int32_t* context_lens_host;
  /* Which units compute the two products (q . K and weights . V) when every
   * KV head is read by one query head (num_q_heads == num_kv_heads) and the
   * caches are 16-bit: PA_PRODUCTS_MATRIX (the gfx950 matrix cores, the
   * query heads of a KV head as the columns of the tile), PA_PRODUCTS_VALU
   * (packed dot products on the vector ALU), or PA_PRODUCTS_AUTO (the
   * library's choice: the matrix cores, which measured on MI355X as fast as
   * the vector ALU or up to 2% faster at every block size).  With more query
   * heads per KV head the matrix cores always take the products;
   * PA_PRODUCTS_VALU there, or with INT8 or fp32 caches, returns
   * PA_ERR_UNSUPPORTED.  The results
   * agree within the same error bound (same rounding of the weights). */
  int32_t products;
} pa_decode_args;

enum { PA_PRODUCTS_AUTO = 0, PA_PRODUCTS_MATRIX = 1, PA_PRODUCTS_VALU = 2 };

/* Bytes of workspace pa_decode needs for these sizes (device pointers are
 * not read; a context_lens_host copy is checked).
 * 0 when the step needs none, or when the arguments are invalid. */
PA_API size_t pa_decode_workspace_bytes(const pa_decode_args* args);

/* The partition size pa_decode will use for these arguments, or -1 when
 * they are invalid. */
PA_API int32_t pa_decode_partition_size(const pa_decode_args* args);

/* The products pa_decode will use for these arguments (PA_PRODUCTS_MATRIX
 * or PA_PRODUCTS_VALU), or -1 when they are invalid. */
PA_API int32_t pa_decode_products(const pa_decode_args* args);

PA_API pa_status pa_decode(const pa_decode_args* args, void* stream);

/* ------------------------------------------------------------------------
 * pa_decode_static -- pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and results as pa_decode, with the
 * split-K partials in a scratch array the library holds in device memory
 * (PA_DECODE_STATIC_SCRATCH_BYTES per GPU it runs on, kept until the process
 * ends) instead of args->workspace, which is ignored.  It calls no hipMalloc,
 * hipFree or allocating routine.  The caller still owns every input and
 * output.  Returns PA_ERR_WORKSPACE when the step needs more partial storage
 * than the scratch holds (pa_decode_workspace_bytes(args) >
 * PA_DECODE_STATIC_SCRATCH_BYTES), PA_ERR_INVALID when `stream` belongs to
 * another device than the current one, otherwise as pa_decode.  Every call
 * on one GPU shares that GPU's scratch: calls that overlap in time on one
 * GPU (other streams, other threads) race; calls on one stream are ordered.
 * The scratch keeps the last call's partials; nothing in it must start at
 * zero (every partial read is written first by the same call).
 * ------------------------------------------------------------------------ */
#define PA_DECODE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
PA_API pa_status pa_decode_static(const pa_decode_args* args, void* stream);

/* ------------------------------------------------------------------------
 * pa_decode_prefix -- pa_decode for batches whose sequences share prefix
 * blocks (prefix caching and parallel sampling: wiblog.cn, section
 * "Copy-on-Write、并行采样与 Prefix Caching 不是同一件事"; kongchang.com,
 * section "PagedAttention的三大核心优势", second advantage).  Sequences are
 * ordered by group: group g is sequences [group_start[g], group_start[g+1])
 * and its members share their first prefix_len[g] tokens -- the same
 * physical slots through their tables, which the copy-on-write rules keep
 * true for whole shared blocks.  The shared prefix is attended once per
 * group (its K/V read once, every member's query heads as the matrix-core
 * columns, split into partitions like a long context), each member's
 * remaining tokens as in pa_decode in the same launch, and the parts merged
 * with the log-sum-exp rule by a second launch.  The output equals
 * pa_decode's up to rounding order.
 * Preconditions (device contents): group_start[0] = 0, non-decreasing,
 * group_start[num_groups] = num_seqs; 0 <= prefix_len[g] <= the context of
 * every member (minus the appended token when k_new is set); a group of one
 * or prefix_len 0 is allowed (that member decodes as in pa_decode).
 * max_group_size is a host-known bound of the group sizes.  Arguments of
 * pa_decode otherwise (f16 / bf16 queries; fp32 returns
 * PA_ERR_UNSUPPORTED); the workspace comes from
 * pa_decode_prefix_workspace_bytes (never 0 when num_groups > 0).
 * num_groups == 0 is pa_decode.
 * ------------------------------------------------------------------------ */
typedef struct pa_prefix_groups {
  const int32_t* group_start;   /* [num_groups + 1] device */
  const int32_t* prefix_len;    /* [num_groups] device, tokens */
  int32_t num_groups;
  int32_t max_group_size;       /* host bound of the group sizes */
  int32_t max_prefix_len;       /* host bound of prefix_len, <= max_context_len */
  int32_t min_prefix_len;       /* host lower bound of prefix_len, 0..max_prefix_len;
                                   0 = none.  A member's own tokens then span at
                                   most max_context_len - min_prefix_len tokens,
                                   which sizes their part of the grid; a prefix
                                   shorter than it is a precondition violation. */
} pa_prefix_groups;

PA_API size_t pa_decode_prefix_workspace_bytes(const pa_decode_args* args,
                                               const pa_prefix_groups* groups);
PA_API pa_status pa_decode_prefix(const pa_decode_args* args, const pa_prefix_groups* groups,
                                  void* stream);

/* ------------------------------------------------------------------------
 * pa_prefill -- paged (chunked) prefill: attention for the prompt tokens of
 * each sequence, read through its block table (the prefill / chunked
 * prefill of wiblog.cn, section "如何判断服务瓶颈是否真的来自
 * PagedAttention", where long prompts make prefill the bulk of the time to
 * first token).  Sequence s holds c = context_lens[s] cached tokens; the
 * last n_s = query_start[s+1] - query_start[s] of them are the chunk being
 * prefilled, their K/V already written (pa_write_kv / pa_write_kv_i8).
 * Query row r of the chunk (r in [query_start[s], query_start[s+1])) sits at
 * logical position p = c - n_s + (r - query_start[s]) and attends to
 * positions 0..p (causal):
 *     out[r,h,:] = sum_{t<=p} exp(x_t - max x) V_t / sum_{t<=p} exp(x_t - max x),
 *     x_t = scale * <q[r,h,:], K_t>, KV head floor(h / G),
 * with the arithmetic of pa_decode.  A chunk equal to the whole context is a
 * plain prompt prefill; a chunk of one row is one decode query.
 * Layouts: q, out [num_tokens, num_q_heads, head_dim] of dtype (f16 / bf16;
 * PA_F32 returns PA_ERR_UNSUPPORTED), rows of sequence s contiguous;
 * query_start [num_seqs + 1] int32 with query_start[0] = 0,
 * non-decreasing, query_start[num_seqs] = num_tokens and 0 <= n_s <=
 * min(c, max_query_len); the caches, tables and lengths as for pa_decode
 * (kv_dtype PA_I8 / PA_FP8 for 8-bit pools).  No workspace.  Device contents are
 * preconditions; out-of-range lengths are clamped, never read past.  Sizes
 * beyond the launch limits (num_seqs or num_kv_heads above 65535, or more
 * than 2^31 - 1 workgroups of 64 (row, head) slots per sequence and KV head)
 * return PA_ERR_UNSUPPORTED before anything is launched.
 * ------------------------------------------------------------------------ */
typedef struct pa_prefill_args {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;
  int32_t num_seqs;
  int32_t num_tokens;          /* rows of q and out */
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_query_len;       /* host-known upper bound of the chunk lengths */
  int32_t max_context_len;     /* host-known upper bound of context_lens */
  float scale;
  int32_t dtype;               /* pa_dtype of q and out */
  int32_t kv_dtype;            /* dtype, PA_I8 or PA_FP8 */
} pa_prefill_args;

PA_API pa_status pa_prefill(const pa_prefill_args* args, void* stream);

/* ------------------------------------------------------------------------
 * pa_write_kv -- cache write of the step's new tokens (the "追加 KV" (append
 * KV) box of the flowchart in wiblog.cn, section "PagedAttention 如何把连续序列
 * 映射到离散显存块").  For each token t with slot =
 * slot_mapping[t] >= 0: K and V rows of every KV head go to in-block
 * position slot % block_size of physical block slot / block_size, bit for
 * bit.  Negative slots are padding and are skipped; slots >= num_blocks *
 * block_size are skipped too.  k_new, v_new: [num_tokens, num_kv_heads,
 * head_dim] of dtype; slot_mapping: [num_tokens] int64.  Two tokens with the
 * same slot race.
 * ------------------------------------------------------------------------ */
PA_API pa_status pa_write_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             const int64_t* slot_mapping, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * pa_write_kv_i8 -- quantising cache write into INT8 pools (the append-KV
 * step above combined with KV-cache quantisation: wiblog.cn, section "非连续
 * KV 为什么需要专门的 Attention Kernel", mechanism table, row "KV Cache
 * Quantization"; kongchang.com, section "量化技术：与PagedAttention正交的显存
 * 优化路径").  For each token t with slot = slot_mapping[t] in [0,
 * num_blocks * block_size): the K row and the V row of every KV head are
 * quantised as pa_dtype states (one scale per row) and their codes and
 * scale stored at in-block position slot % block_size of block slot /
 * block_size; other slots are skipped.  k_new, v_new: [num_tokens,
 * num_kv_heads, head_dim] of src_dtype (PA_F32, PA_F16 or PA_BF16); the
 * pools are [num_blocks, num_kv_heads, head_dim * block_size + 4 *
 * block_size] bytes.  head_dim must be a multiple of 16.  Two tokens with
 * the same slot race.  The rows must hold finite values: a row with an
 * infinity or a NaN gets unspecified codes and scale (no access leaves the
 * buffers either way).
 * ------------------------------------------------------------------------ */
PA_API pa_status pa_write_kv_i8(const void* k_new, const void* v_new, int32_t src_dtype,
                                void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t num_blocks, void* stream);

/* ------------------------------------------------------------------------
 * pa_write_kv_fp8 -- pa_write_kv_i8 for FP8 pools (same passages): the rows
 * are quantised to E4M3 codes as pa_dtype states for PA_FP8; arguments,
 * layouts and errors as for pa_write_kv_i8.
 * ------------------------------------------------------------------------ */
PA_API pa_status pa_write_kv_fp8(const void* k_new, const void* v_new, int32_t src_dtype,
                                 void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, void* stream);

/* ------------------------------------------------------------------------
 * pa_copy_blocks -- copy-on-write block copies (bmjup.com, section
 * "PagedAttention 的核心工作机制与创新", item 2 "写入时拷贝（Copy-on-Write）";
 * wiblog.cn, section "Copy-on-Write、并行采样与 Prefix Caching 不是同一件
 * 事").  block_mapping is [num_pairs][2] int32 = {src, dst}: every element of
 * physical block dst (all KV heads, K and V) becomes a bit copy of block src.  A dst must not appear twice nor
 * as any pair's src (the pairs pa_seq_append_slot reports satisfy this).
 * Pairs with an id outside [0, num_blocks) are skipped.  dtype PA_I8 or
 * PA_FP8 copies whole 8-bit tiles, codes and scales (block_size must be a
 * multiple of 4).
 * ------------------------------------------------------------------------ */
PA_API pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                                int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t num_blocks, int32_t dtype,
                                void* stream);

/* ------------------------------------------------------------------------
 * pa_gather_kv -- test hook: copies each sequence's K and V through its block
 * table into contiguous k_out, v_out [num_seqs, max_context_len,
 * num_kv_heads, head_dim] of dtype, bit for bit, in logical token order.
 * Rows t >= context_lens[s] are left untouched.  This is the "concatenate
 * the blocks, then run ordinary attention" route that wiblog.cn (section
 * "非连续 KV 为什么需要专门的 Attention Kernel") warns costs extra copies; it
 * exists only to check addressing.  PA_I8 and PA_FP8 pools are not supported.
 * ------------------------------------------------------------------------ */
PA_API pa_status pa_gather_kv(const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              void* k_out, void* v_out, int32_t num_seqs, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t max_context_len, int32_t dtype,
                              void* stream);

/* ------------------------------------------------------------------------
 * pa_probe_read -- diagnostic, not a step of the decode path: the read
 * ceiling of an access pattern.  Decode is bound by reading the KV cache
 * from HBM (kongchang.com, "PagedAttention原理详解", section "GPU显存层次结构
 * 与带宽瓶颈"); this reads num_ranges byte ranges of range_bytes bytes at byte
 * offsets offs[i] (device, int64) of BOTH device buffers a and b (a K tile
 * and the V tile at the same offset), with the decode pass's non-temporal
 * 16-byte loads and no arithmetic.  Fed the (block, KV head) tiles of a
 * decode step it times the scattered-tile ceiling; fed consecutive offsets,
 * a streaming read.  buf_bytes: size of each buffer; a range that would
 * leave [0, buf_bytes) is skipped.  range_bytes: a multiple of 16, at most
 * 16384.  ranges_in_flight: 1, 2 or 4 ranges per wave per round.
 * workgroups: grid cap (0 = 2048).  sink: one device uint32 that is written
 * only when the xor of all bytes read equals a fixed value.  a, b 16-byte
 * aligned.  Caller-owned memory; asynchronous on `stream`.
 * ------------------------------------------------------------------------ */
PA_API pa_status pa_probe_read(const void* a, const void* b, size_t buf_bytes, const int64_t* offs,
                               int64_t num_ranges, int32_t range_bytes, int32_t ranges_in_flight,
                               int32_t workgroups, uint32_t* sink, void* stream);

/* ------------------------------------------------------------------------
 * Host block manager (the allocator, free pool, refcounts and block tables:
 * bmjup.com, section "PagedAttention 的核心工作机制与创新", item 3 "动态内存
 * 分配"; the wiblog.cn flowchart and its copy-on-write section; kongchang.com,
 * section "PagedAttention的三大核心优势", second advantage (shared prefix
 * blocks with reference counts and copy-on-write)).  Opaque, owned by the
 * caller, not thread-safe.  Rules:
 *   - append: when len % block_size == 0 a new block is taken from the free
 *     pool; otherwise the token goes to the next slot of the last block.  If
 *     that last block is partly filled AND shared (refcount > 1), the caller
 *     gets a fresh block instead: the old block's refcount drops by one and
 *     (old, fresh) is reported so that the caller copies it with
 *     pa_copy_blocks before writing.  slot = block * block_size + len %
 *     block_size.
 *   - fork: the child references every block of the parent (refcount + 1).
 *   - free: every block's refcount drops by one; blocks reaching 0 return to
 *     the free pool at once (in logical order).
 *   - free pool: a stack, initially init_free_order with element 0 on top
 *     (NULL = 0, 1, 2, ...); freed blocks are pushed on top.
 *   - PA_ERR_NO_BLOCKS leaves the state unchanged.
 * ------------------------------------------------------------------------ */
typedef struct pa_allocator pa_allocator;

/* init_free_order: NULL or a permutation of 0..num_blocks-1 (copied). */
PA_API pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size,
                                 const int32_t* init_free_order, pa_allocator** out);
PA_API void pa_alloc_destroy(pa_allocator* a);
PA_API int32_t pa_alloc_num_free(const pa_allocator* a);       /* -1 if a is NULL */
PA_API int32_t pa_alloc_num_seqs(const pa_allocator* a);       /* -1 if a is NULL */
PA_API int32_t pa_block_refcount(const pa_allocator* a, int32_t block); /* -1 if out of range */

PA_API pa_status pa_seq_add(pa_allocator* a, int64_t seq);
PA_API pa_status pa_seq_fork(pa_allocator* a, int64_t parent, int64_t child);
/* One token; *cow_src = *cow_dst = -1 when nothing must be copied. */
PA_API pa_status pa_seq_append_slot(pa_allocator* a, int64_t seq, int64_t* slot,
                                    int32_t* cow_src, int32_t* cow_dst);
/* One token for each of n distinct sequences (a decode step).  slots[n]
 * receives the slots; cow_pairs (room for n pairs, [n][2] int32) receives the
 * copy pairs in sequence order and *num_cow their count.  Either every
 * append happens or none (PA_ERR_NO_BLOCKS, PA_ERR_UNKNOWN_SEQ, or
 * PA_ERR_INVALID for a repeated sequence id). */
PA_API pa_status pa_seq_append_slots(pa_allocator* a, const int64_t* seqs, int32_t n,
                                     int64_t* slots, int32_t* cow_pairs, int32_t* num_cow);
PA_API pa_status pa_seq_free(pa_allocator* a, int64_t seq);
PA_API int32_t pa_seq_len(const pa_allocator* a, int64_t seq);          /* -1 if unknown */
PA_API int32_t pa_seq_num_blocks(const pa_allocator* a, int64_t seq);   /* -1 if unknown */
/* Copies the block table into out[0..cap); *n = its full length. */
PA_API pa_status pa_seq_block_table(const pa_allocator* a, int64_t seq, int32_t* out,
                                    int32_t cap, int32_t* n);

/* ------------------------------------------------------------------------
 * Prefix cache (wiblog.cn, section "Copy-on-Write、并行采样与 Prefix Caching
 * 不是同一件事": sharing physical blocks is not yet a cross-request prefix
 * cache, which also needs a cache key, exact matching of token sequences
 * under one model configuration, a lifetime for cached blocks, and normal
 * prefill of the unmatched suffix).  An index from the content of a FULL
 * block to the physical block holding it:
 *   - key of block i of a token sequence: a 128-bit hash chained from `salt`
 *     (the caller's tag of everything that changes the KV of the same tokens:
 *     model, tokenizer, chat template, positional configuration) over every
 *     token from the sequence start to the block's end, so two blocks share a
 *     key only when their whole prefixes are the same token ids under the
 *     same salt (up to a 2^-128-scale hash collision);
 *   - pa_prefix_register records the full blocks of a sequence whose KV is
 *     written (tokens: the sequence's token ids, at least its full blocks);
 *     a key already present, or a block already indexed, is left alone (the
 *     first registration wins);
 *   - pa_prefix_match gives how many leading tokens (whole blocks) of a new
 *     token sequence the index holds, leaving at least one token unmatched
 *     (it must be prefilled to give the next token);
 *   - pa_seq_add_cached creates a sequence that references those blocks
 *     (refcount + 1 each; its length is the matched token count): the caller
 *     prefills the rest through pa_seq_append_slot as usual;
 *   - an entry lives while its block is referenced: it is dropped when the
 *     block returns to the free pool (no retention of unreferenced blocks).
 * Full blocks are never written again (appends take a new block; copy-on-
 * write only copies partly filled tails), so an indexed block's content is
 * stable while it is indexed.
 * ------------------------------------------------------------------------ */
/* *n_registered: blocks newly indexed. */
PA_API pa_status pa_prefix_register(pa_allocator* a, int64_t seq, const int32_t* tokens,
                                    int32_t n_tokens, uint64_t salt, int32_t* n_registered);
/* Tokens (a multiple of block_size, < n_tokens) a new sequence could adopt;
 * -1 on bad arguments. */
PA_API int32_t pa_prefix_match(const pa_allocator* a, const int32_t* tokens, int32_t n_tokens,
                               uint64_t salt);
/* New sequence `seq` over the matched blocks; *n_cached = its length. */
PA_API pa_status pa_seq_add_cached(pa_allocator* a, int64_t seq, const int32_t* tokens,
                                   int32_t n_tokens, uint64_t salt, int32_t* n_cached);
PA_API int32_t pa_prefix_num_entries(const pa_allocator* a); /* -1 if a is NULL */

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
