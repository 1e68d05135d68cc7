"""ctypes front end of the fp64 C oracle (pa_oracle.c).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT: only tests/, the smoke entry
point and the CPU-baseline leg of the benchmark may import this module.

Array conventions (numpy, C-contiguous):
  * element types: "f32" -> float32, "f16" -> float16, "bf16" -> uint16
    holding the bfloat16 bit patterns (numpy has no bfloat16);
  * k_cache [NB, Hkv, D/x, BS, x] and v_cache [NB, Hkv, D, BS], x = 16 bytes /
    element size: the block layout printed by intelliparadigm.com,
    "vLLM的Paged Attention技术", section "2.2 内存布局优化";
  * q [S, Hq, D]; block_tables [S, max_blocks] int32; context_lens [S] int32;
    slot_mapping [T] int64; copy pairs [P, 2] int32 = (src, dst).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64


def lib():
    """Load liboracle.so (compiled by oracle/build_oracle.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: run python oracle/build_oracle.py")
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_k_index.restype = _I64
        L.oracle_k_index.argtypes = [_I64, _I, _I, _I, _I, _I, _I, _I]
        L.oracle_v_index.restype = _I64
        L.oracle_v_index.argtypes = [_I64, _I, _I, _I, _I, _I, _I]
        L.oracle_gather_raw.restype = _I
        L.oracle_gather_raw.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P]
        L.oracle_decode.restype = _I
        L.oracle_decode.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                    ctypes.c_float, _I, _I, _P, _P, _P, _P]
        L.oracle_prefill.restype = _I
        L.oracle_prefill.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                     ctypes.c_float, _I, _I, _P, _P, _P, _P]
        L.oracle_prefill_i8.restype = _I
        L.oracle_prefill_i8.argtypes = [_P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                        ctypes.c_float, _I, _P, _P, _P, _P]
        L.oracle_write_kv.restype = _I
        L.oracle_write_kv.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I]
        L.oracle_copy_blocks.restype = _I
        L.oracle_copy_blocks.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _I]
        for name in ("oracle_i8_k_offset", "oracle_i8_v_offset"):
            getattr(L, name).restype = _I64
            getattr(L, name).argtypes = [_I64, _I, _I, _I, _I, _I, _I]
        L.oracle_i8_scale_offset.restype = _I64
        L.oracle_i8_scale_offset.argtypes = [_I64, _I, _I, _I, _I, _I]
        L.oracle_i8_tile_bytes.restype = _I64
        L.oracle_i8_tile_bytes.argtypes = [_I, _I]
        L.oracle_quantize_row.restype = None
        L.oracle_quantize_row.argtypes = [_P, _I, _P, _P]
        L.oracle_write_kv_i8.restype = _I
        L.oracle_write_kv_i8.argtypes = [_P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I]
        L.oracle_copy_blocks_i8.restype = _I
        L.oracle_copy_blocks_i8.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I]
        L.oracle_decode_i8.restype = _I
        L.oracle_decode_i8.argtypes = [_P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                       ctypes.c_float, _I, _P, _P, _P, _P]
        L.oracle_fp8_value.restype = ctypes.c_double
        L.oracle_fp8_value.argtypes = [_I]
        L.oracle_fp8_encode.restype = _I
        L.oracle_fp8_encode.argtypes = [ctypes.c_float]
        L.oracle_quantize_row_fp8.restype = None
        L.oracle_quantize_row_fp8.argtypes = [_P, _I, _P, _P]
        L.oracle_write_kv_q8.restype = _I
        L.oracle_write_kv_q8.argtypes = [_P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I]
        L.oracle_decode_q8.restype = _I
        L.oracle_decode_q8.argtypes = [_P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                       ctypes.c_float, _I, _P, _P, _P, _P, _I]
        L.oracle_prefill_q8.restype = _I
        L.oracle_prefill_q8.argtypes = [_P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                        ctypes.c_float, _I, _P, _P, _P, _P, _I]
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


class Attention:
    """Oracle attention result with the ingredients of a per-element error
    bound (see pa_oracle.c, oracle_decode):
      out    [rows, Hq, D]  the attention output (fp64);
      spread [rows, Hq, D]  sum_t pi_t |v_t[d] - out[d]|;
      devmax [rows, Hq, D]  max_t |v_t[d] - out[d]|;
      lam    [rows, Hq]     max_t |scale| sum_d |q[d] k_t[d]|;
      keys   [rows]         how many keys each row attends to.
    Indexing by rows (an int array or a slice) selects the same rows of all."""

    def __init__(self, out, spread, devmax, lam, keys):
        self.out, self.spread, self.devmax, self.lam = out, spread, devmax, lam
        self.keys = np.asarray(keys, np.int64)

    def __getitem__(self, rows):
        return Attention(self.out[rows], self.spread[rows], self.devmax[rows], self.lam[rows],
                         self.keys[rows])


def _bound_buffers(rows, Hq, D, bound):
    """(spread, devmax, lam) output arrays, or three None."""
    if not bound:
        return None, None, None
    return np.empty((rows, Hq, D)), np.empty((rows, Hq, D)), np.empty((rows, Hq))


def _opt(a):
    return None if a is None else _ptr(a)


def _check(a, np_dtype, name):
    if a.dtype != np.dtype(np_dtype):
        raise TypeError(f"{name}: dtype {a.dtype}, expected {np.dtype(np_dtype)}")
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError(f"{name}: must be C-contiguous")


def cache_geometry(k_cache, v_cache, dtype):
    """(NB, Hkv, D, BS) from the two pool arrays; checks they agree."""
    x = 16 // ELEM_BYTES[dtype]
    if k_cache.ndim != 5 or v_cache.ndim != 4:
        raise ValueError("k_cache must be 5-D and v_cache 4-D")
    NB, Hkv, Dx, BS, kx = k_cache.shape
    if kx != x:
        raise ValueError(f"k_cache last dim {kx}, expected x={x} for {dtype}")
    D = Dx * x
    if v_cache.shape != (NB, Hkv, D, BS):
        raise ValueError(f"v_cache shape {v_cache.shape}, expected {(NB, Hkv, D, BS)}")
    _check(k_cache, NP_STORAGE[dtype], "k_cache")
    _check(v_cache, NP_STORAGE[dtype], "v_cache")
    return NB, Hkv, D, BS


def k_index(b, h, o, d, Hkv, D, BS, dtype):
    return lib().oracle_k_index(b, h, o, d, Hkv, D, BS, DTYPE_CODE[dtype])


def v_index(b, h, o, d, Hkv, D, BS):
    return lib().oracle_v_index(b, h, o, d, Hkv, D, BS)


def gather_raw(k_cache, v_cache, block_tables, context_lens, max_ctx, dtype, fill=0):
    """Bit copies of logical K, V [S, max_ctx, Hkv, D] in the cache's storage
    type; positions past a context keep `fill`."""
    NB, Hkv, D, BS = cache_geometry(k_cache, v_cache, dtype)
    _check(block_tables, np.int32, "block_tables")
    _check(context_lens, np.int32, "context_lens")
    S, max_blocks = block_tables.shape
    k = np.full((S, max_ctx, Hkv, D), fill, NP_STORAGE[dtype])
    v = np.full_like(k, fill)
    rc = lib().oracle_gather_raw(_ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                 _ptr(context_lens), S, Hkv, D, BS, max_blocks, max_ctx,
                                 DTYPE_CODE[dtype], _ptr(k), _ptr(v))
    if rc != 0:
        raise ValueError("oracle_gather_raw rejected its arguments")
    return k, v


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype, num_threads=1,
           bound=False):
    """Paged decode attention, fp64 output [S, Hq, D]; with bound=True an
    Attention (output plus the bound ingredients)."""
    NB, Hkv, D, BS = cache_geometry(k_cache, v_cache, dtype)
    _check(q, NP_STORAGE[dtype], "q")
    _check(block_tables, np.int32, "block_tables")
    _check(context_lens, np.int32, "context_lens")
    S, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q head_dim does not match the cache")
    out = np.empty((S, Hq, D), np.float64)
    spread, devmax, lam = _bound_buffers(S, Hq, D, bound)
    rc = lib().oracle_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                             _ptr(context_lens), S, Hq, Hkv, D, BS, block_tables.shape[1],
                             ctypes.c_float(scale), DTYPE_CODE[dtype], int(num_threads), _ptr(out),
                             _opt(spread), _opt(devmax), _opt(lam))
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return Attention(out, spread, devmax, lam, np.maximum(context_lens, 0)) if bound else out


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, dtype,
            num_threads=1, bound=False):
    """Paged (chunked) prefill: causal attention of each query row over its
    sequence's positions 0..p, fp64 output [T, Hq, D]; with bound=True an
    Attention."""
    NB, Hkv, D, BS = cache_geometry(k_cache, v_cache, dtype)
    _check(q, NP_STORAGE[dtype], "q")
    _check(block_tables, np.int32, "block_tables")
    _check(context_lens, np.int32, "context_lens")
    _check(query_start, np.int32, "query_start")
    S = context_lens.shape[0]
    T, Hq, Dq = q.shape
    if Dq != D or query_start.shape != (S + 1,) or int(query_start[-1]) != T:
        raise ValueError("q must be [T, Hq, D] with T = query_start[S]")
    out = np.empty((T, Hq, D), np.float64)
    spread, devmax, lam = _bound_buffers(T, Hq, D, bound)
    rc = lib().oracle_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                              _ptr(context_lens), _ptr(query_start), S, Hq, Hkv, D, BS,
                              block_tables.shape[1], ctypes.c_float(scale), DTYPE_CODE[dtype],
                              int(num_threads), _ptr(out), _opt(spread), _opt(devmax), _opt(lam))
    if rc != 0:
        raise ValueError("oracle_prefill rejected its arguments")
    return Attention(out, spread, devmax, lam, _row_keys(context_lens, query_start)) if bound else out


def write_kv(k_new, v_new, k_cache, v_cache, slot_mapping, dtype):
    """In-place cache write of k_new / v_new [T, Hkv, D] at slot_mapping [T]."""
    NB, Hkv, D, BS = cache_geometry(k_cache, v_cache, dtype)
    _check(k_new, NP_STORAGE[dtype], "k_new")
    _check(v_new, NP_STORAGE[dtype], "v_new")
    _check(slot_mapping, np.int64, "slot_mapping")
    T = slot_mapping.shape[0]
    if k_new.shape != (T, Hkv, D) or v_new.shape != (T, Hkv, D):
        raise ValueError("k_new / v_new must be [T, Hkv, D]")
    rc = lib().oracle_write_kv(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                               _ptr(slot_mapping), T, Hkv, D, BS, NB, DTYPE_CODE[dtype])
    if rc != 0:
        raise ValueError("oracle_write_kv rejected its arguments")


def copy_blocks(k_cache, v_cache, pairs, dtype):
    """In-place block copies; pairs [P, 2] int32 = (src, dst)."""
    NB, Hkv, D, BS = cache_geometry(k_cache, v_cache, dtype)
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    rc = lib().oracle_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(pairs), pairs.shape[0],
                                  Hkv, D, BS, NB, DTYPE_CODE[dtype])
    if rc != 0:
        raise ValueError("oracle_copy_blocks rejected its arguments")


# ---------------------------------------------------------------------------- INT8 KV cache
# Pools are uint8 arrays [NB, Hkv, tile_bytes] with tile_bytes = D*BS + 4*BS:
# codes ([D/16][BS][16] for K, [D][BS] for V) followed by BS fp32 scales (see
# the INT8 section of pa_oracle.c for the readings).

def i8_tile_bytes(D, BS):
    return int(lib().oracle_i8_tile_bytes(D, BS))


def i8_geometry(k_pool, v_pool, D, BS):
    """(NB, Hkv) of two INT8 pools; checks their shapes."""
    if k_pool.ndim != 3 or k_pool.shape != v_pool.shape or k_pool.shape[2] != i8_tile_bytes(D, BS):
        raise ValueError("INT8 pools must both be [NB, Hkv, D*BS + 4*BS] uint8")
    _check(k_pool, np.uint8, "k_pool")
    _check(v_pool, np.uint8, "v_pool")
    return k_pool.shape[0], k_pool.shape[1]


def i8_offsets(b, h, o, d, Hkv, D, BS):
    """Byte offsets (K code, V code, scale) of element (b, h, o, d)."""
    L = lib()
    return (L.oracle_i8_k_offset(b, h, o, d, Hkv, D, BS), L.oracle_i8_v_offset(b, h, o, d, Hkv, D, BS),
            L.oracle_i8_scale_offset(b, h, o, Hkv, D, BS))


# 8-bit code formats of a quantised pool: INT8, or FP8 (E4M3; see the FP8
# section of pa_oracle.c).  Both share the tile layout and the scales.
Q8_FORMAT = {"i8": 0, "fp8": 1}


def fp8_value(code):
    """Value of an E4M3 code (NaN for S.1111.111)."""
    return float(lib().oracle_fp8_value(int(code)))


def fp8_encode(r):
    """E4M3 code of the fp32 value r (nearest, ties to even, saturating)."""
    return int(lib().oracle_fp8_encode(ctypes.c_float(r)))


def quantize_row_fp8(x):
    """fp32 row -> (E4M3 codes as uint8, fp32 scale)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.empty(x.shape[0], np.uint8)
    sc = np.empty(1, np.float32)
    lib().oracle_quantize_row_fp8(_ptr(x), x.shape[0], _ptr(codes), _ptr(sc))
    return codes, sc[0]


def quantize_row(x):
    """fp32 row -> (int8 codes, fp32 scale)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.empty(x.shape[0], np.int8)
    sc = np.empty(1, np.float32)
    lib().oracle_quantize_row(_ptr(x), x.shape[0], _ptr(codes), _ptr(sc))
    return codes, sc[0]


def write_kv_i8(k_new, v_new, src_dtype, k_pool, v_pool, slot_mapping, D, BS, fmt="i8"):
    """Quantising cache write of k_new / v_new [T, Hkv, D] (src_dtype storage)
    into 8-bit pools of code format fmt ("i8" or "fp8")."""
    NB, Hkv = i8_geometry(k_pool, v_pool, D, BS)
    _check(k_new, NP_STORAGE[src_dtype], "k_new")
    _check(v_new, NP_STORAGE[src_dtype], "v_new")
    _check(slot_mapping, np.int64, "slot_mapping")
    T = slot_mapping.shape[0]
    if k_new.shape != (T, Hkv, D) or v_new.shape != (T, Hkv, D):
        raise ValueError("k_new / v_new must be [T, Hkv, D]")
    rc = lib().oracle_write_kv_q8(_ptr(k_new), _ptr(v_new), DTYPE_CODE[src_dtype], _ptr(k_pool),
                                  _ptr(v_pool), _ptr(slot_mapping), T, Hkv, D, BS, NB, Q8_FORMAT[fmt])
    if rc != 0:
        raise ValueError("oracle_write_kv_q8 rejected its arguments")


def copy_blocks_i8(k_pool, v_pool, pairs, D, BS):
    NB, Hkv = i8_geometry(k_pool, v_pool, D, BS)
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    rc = lib().oracle_copy_blocks_i8(_ptr(k_pool), _ptr(v_pool), _ptr(pairs), pairs.shape[0], Hkv, D,
                                     BS, NB)
    if rc != 0:
        raise ValueError("oracle_copy_blocks_i8 rejected its arguments")


def decode_i8(q, q_dtype, k_pool, v_pool, block_tables, context_lens, scale, D, BS, num_threads=1,
              bound=False, fmt="i8"):
    """Paged decode attention over 8-bit pools (code format fmt: "i8" or
    "fp8"), fp64 output [S, Hq, D]; with bound=True an Attention."""
    NB, Hkv = i8_geometry(k_pool, v_pool, D, BS)
    _check(q, NP_STORAGE[q_dtype], "q")
    _check(block_tables, np.int32, "block_tables")
    _check(context_lens, np.int32, "context_lens")
    S, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q head_dim does not match")
    out = np.empty((S, Hq, D), np.float64)
    spread, devmax, lam = _bound_buffers(S, Hq, D, bound)
    rc = lib().oracle_decode_q8(_ptr(q), DTYPE_CODE[q_dtype], _ptr(k_pool), _ptr(v_pool),
                                _ptr(block_tables), _ptr(context_lens), S, Hq, Hkv, D, BS,
                                block_tables.shape[1], ctypes.c_float(scale), int(num_threads),
                                _ptr(out), _opt(spread), _opt(devmax), _opt(lam), Q8_FORMAT[fmt])
    if rc != 0:
        raise ValueError("oracle_decode_q8 rejected its arguments")
    return Attention(out, spread, devmax, lam, np.maximum(context_lens, 0)) if bound else out


def prefill_i8(q, q_dtype, k_pool, v_pool, block_tables, context_lens, query_start, scale, D, BS,
               num_threads=1, bound=False, fmt="i8"):
    """Paged (chunked) prefill over 8-bit pools (code format fmt: "i8" or
    "fp8"), fp64 output [T, Hq, D]; with bound=True an Attention."""
    NB, Hkv = i8_geometry(k_pool, v_pool, D, BS)
    _check(q, NP_STORAGE[q_dtype], "q")
    _check(block_tables, np.int32, "block_tables")
    _check(context_lens, np.int32, "context_lens")
    _check(query_start, np.int32, "query_start")
    S = context_lens.shape[0]
    T, Hq, Dq = q.shape
    if Dq != D or query_start.shape != (S + 1,) or int(query_start[-1]) != T:
        raise ValueError("q must be [T, Hq, D] with T = query_start[S]")
    out = np.empty((T, Hq, D), np.float64)
    spread, devmax, lam = _bound_buffers(T, Hq, D, bound)
    rc = lib().oracle_prefill_q8(_ptr(q), DTYPE_CODE[q_dtype], _ptr(k_pool), _ptr(v_pool),
                                 _ptr(block_tables), _ptr(context_lens), _ptr(query_start), S, Hq,
                                 Hkv, D, BS, block_tables.shape[1], ctypes.c_float(scale),
                                 int(num_threads), _ptr(out), _opt(spread), _opt(devmax), _opt(lam),
                                 Q8_FORMAT[fmt])
    if rc != 0:
        raise ValueError("oracle_prefill_q8 rejected its arguments")
    return Attention(out, spread, devmax, lam, _row_keys(context_lens, query_start)) if bound else out


def _row_keys(context_lens, query_start):
    """Keys seen by each prefill row: position + 1 (chunk rows are the last
    query_start[s+1] - query_start[s] positions of sequence s)."""
    keys = []
    for s in range(context_lens.shape[0]):
        n = int(query_start[s + 1] - query_start[s])
        keys.extend(range(int(context_lens[s]) - n + 1, int(context_lens[s]) + 1))
    return np.asarray(keys, np.int64)
