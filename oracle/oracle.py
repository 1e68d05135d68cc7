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
        L.oracle_gather.restype = _I
        L.oracle_gather.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P]
        L.oracle_gather_raw.restype = _I
        L.oracle_gather_raw.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P]
        L.oracle_decode.restype = _I
        L.oracle_decode.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                    ctypes.c_float, _I, _I, _P]
        L.oracle_write_kv.restype = _I
        L.oracle_write_kv.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I]
        L.oracle_copy_blocks.restype = _I
        L.oracle_copy_blocks.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _I]
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


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


def gather(k_cache, v_cache, block_tables, context_lens, max_ctx, dtype):
    """Logical K, V [S, max_ctx, Hkv, D] fp64 (zero past each context)."""
    NB, Hkv, D, BS = cache_geometry(k_cache, v_cache, dtype)
    _check(block_tables, np.int32, "block_tables")
    _check(context_lens, np.int32, "context_lens")
    S, max_blocks = block_tables.shape
    k = np.empty((S, max_ctx, Hkv, D), np.float64)
    v = np.empty_like(k)
    rc = lib().oracle_gather(_ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
                             S, Hkv, D, BS, max_blocks, max_ctx, DTYPE_CODE[dtype], _ptr(k), _ptr(v))
    if rc != 0:
        raise ValueError("oracle_gather rejected its arguments")
    return k, v


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


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype, num_threads=1):
    """Paged decode attention, fp64 output [S, Hq, D]."""
    NB, Hkv, D, BS = cache_geometry(k_cache, v_cache, dtype)
    _check(q, NP_STORAGE[dtype], "q")
    _check(block_tables, np.int32, "block_tables")
    _check(context_lens, np.int32, "context_lens")
    S, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q head_dim does not match the cache")
    out = np.empty((S, Hq, D), np.float64)
    rc = lib().oracle_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                             _ptr(context_lens), S, Hq, Hkv, D, BS, block_tables.shape[1],
                             ctypes.c_float(scale), DTYPE_CODE[dtype], int(num_threads), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return out


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
