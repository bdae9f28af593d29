"""CPU oracle for sparse MLA forward over top-k indices (ctypes binding).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The GPU library never
imports, links or calls it, and this package imports nothing from the GPU
library: the two share only the seeded input generators.

The arithmetic lives in ``smla_oracle.c`` (plain C, double precision, OpenMP
over query tokens); this module only marshals numpy arrays. Every function
follows a passage of the vLLM ``flashmla_sparse.py`` page (FLASHMLA_SPARSE
backend source): the fp8_ds_mla cache-format note, the
``triton_convert_req_index_to_global_index`` docstring, and
``FlashMLASparseImpl.forward`` with its two kernel wrappers.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "smla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsmla_oracle.so")

BF16_CACHE = 0
FP8_CACHE = 1

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (plain C11, OpenMP). Returns the .so path."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", _SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # SMLA_ORACLE_LIB lets the mutation test load a deliberately broken copy.
    path = os.environ.get("SMLA_ORACLE_LIB")
    if not path:
        path = _LIB_PATH
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build()
    lib = ctypes.CDLL(path)
    i64, i32, dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    vp = ctypes.c_void_p
    lib.smla_oracle_num_threads.restype = ctypes.c_int
    lib.smla_oracle_num_threads.argtypes = []
    lib.smla_oracle_e4m3fn.restype = dbl
    lib.smla_oracle_e4m3fn.argtypes = [ctypes.c_uint8]
    lib.smla_oracle_bf16.restype = dbl
    lib.smla_oracle_bf16.argtypes = [ctypes.c_uint16]
    lib.smla_oracle_decode_fp8_row.restype = None
    lib.smla_oracle_decode_fp8_row.argtypes = [vp, vp]
    lib.smla_oracle_decode_bf16_row.restype = None
    lib.smla_oracle_decode_bf16_row.argtypes = [vp, vp]
    lib.smla_oracle_convert_one.restype = i32
    lib.smla_oracle_e4m3fn_encode.restype = ctypes.c_uint8
    lib.smla_oracle_e4m3fn_encode.argtypes = [ctypes.c_float]
    lib.smla_oracle_cache_write.restype = None
    lib.smla_oracle_cache_write.argtypes = [ctypes.c_int, vp, vp, vp, i64, vp, i64]
    lib.smla_oracle_convert_one.argtypes = [i32, i32, vp, i64, i64, i64]
    lib.smla_oracle_convert_indices.restype = None
    lib.smla_oracle_convert_indices.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64]
    lib.smla_oracle_attention.restype = ctypes.c_int
    lib.smla_oracle_attention.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, dbl,
                                          i64, i64, i64, i64, i64, i64, vp, i64, vp, vp, vp]
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loop uses."""
    return int(_load().smla_oracle_num_threads())


def e4m3fn(code: int) -> float:
    """Value of one OCP E4M3FN byte."""
    return _load().smla_oracle_e4m3fn(int(code) & 0xFF)


def bf16(bits: int) -> float:
    """Value of one bfloat16 bit pattern."""
    return _load().smla_oracle_bf16(int(bits) & 0xFFFF)


def decode_fp8_rows(rows: np.ndarray) -> np.ndarray:
    """[n, 656] uint8 fp8_ds_mla rows -> [n, 576] float64."""
    rows = _c(rows, np.uint8).reshape(-1, 656)
    out = np.empty((rows.shape[0], 576), dtype=np.float64)
    lib = _load()
    for i in range(rows.shape[0]):
        lib.smla_oracle_decode_fp8_row(rows[i].ctypes.data, out[i].ctypes.data)
    return out


def decode_bf16_rows(rows: np.ndarray) -> np.ndarray:
    """[n, 576] uint16 bf16 rows -> [n, 576] float64."""
    rows = _c(rows, np.uint16).reshape(-1, 576)
    out = np.empty((rows.shape[0], 576), dtype=np.float64)
    lib = _load()
    for i in range(rows.shape[0]):
        lib.smla_oracle_decode_bf16_row(rows[i].ctypes.data, out[i].ctypes.data)
    return out


def e4m3fn_encode(x: float) -> int:
    """float32 value -> E4M3FN byte, nearest with ties to even, saturating at 448."""
    return int(_load().smla_oracle_e4m3fn_encode(float(x)))


def cache_write(cache_format: int, k_c_bits: np.ndarray, k_pe_bits: np.ndarray,
                slot_mapping: np.ndarray, cache: np.ndarray) -> np.ndarray:
    """Write token rows into `cache` in place (the page's concat_and_cache_mla).
    k_c_bits uint16 [T, 512] and k_pe_bits uint16 [T, 64] are bf16 bit patterns;
    slot_mapping int64 [T]; cache uint16 [NB, 64, 576] (format 0, bf16) or uint8
    [NB, 64, 656] (format 1, fp8_ds_mla). Returns cache."""
    T = int(slot_mapping.shape[0])
    k_c = _c(k_c_bits.reshape(T, 512), np.uint16)
    k_pe = _c(k_pe_bits.reshape(T, 64), np.uint16)
    sm = _c(slot_mapping, np.int64)
    assert cache.flags["C_CONTIGUOUS"]
    want = np.uint16 if cache_format == BF16_CACHE else np.uint8
    assert cache.dtype == want
    _load().smla_oracle_cache_write(int(cache_format), _ptr(k_c), _ptr(k_pe), _ptr(sm), T, _ptr(cache),
                                    int(cache.shape[0]) * 64)
    return cache


def convert_indices(req_id_per_token, block_table, topk_indices, num_blocks: int) -> np.ndarray:
    """Logical top-k indices [T, K] -> physical slots [T, K] (int32, -1 = invalid)."""
    req = _c(req_id_per_token, np.int32).reshape(-1)
    bt = _c(block_table, np.int32)
    if bt.ndim != 2:
        raise ValueError("block_table must be 2-D")
    idx = _c(topk_indices, np.int32)
    if idx.ndim != 2 or idx.shape[0] != req.shape[0]:
        raise ValueError("topk_indices must be [num_tokens, topk]")
    out = np.empty_like(idx)
    _load().smla_oracle_convert_indices(req.ctypes.data, bt.ctypes.data, idx.ctypes.data,
                                        out.ctypes.data, idx.shape[0], idx.shape[1],
                                        bt.shape[0], bt.shape[1], int(num_blocks))
    return out


def attention(cache_format: int, q_bits, cache, block_table, req_id_per_token, topk_indices,
              sm_scale: float, tokens=None, want_weights: bool = False):
    """Sparse MLA forward on the CPU.

    q_bits: uint16 bf16 patterns [T, H, 576]. cache: uint16 [NB, 64, 576] (bf16) or
    uint8 [NB, 64, 656] (fp8_ds_mla). tokens: optional subset of query tokens.
    Returns (o [n, H, 512] float64, lse [n, H] float64[, weights [n, H, K]]).
    """
    q = _c(q_bits, np.uint16)
    if q.ndim != 3 or q.shape[2] != 576:
        raise ValueError("q must be [T, H, 576] bf16 bits")
    T, H = q.shape[0], q.shape[1]
    if cache_format == BF16_CACHE:
        c = cache if (cache.dtype == np.uint16 and cache.flags.c_contiguous) else _c(cache, np.uint16)
        if c.shape[-1] != 576:
            raise ValueError("bf16 cache rows must be 576 wide")
        nb = c.size // (64 * 576)
    elif cache_format == FP8_CACHE:
        c = cache if (cache.dtype == np.uint8 and cache.flags.c_contiguous) else _c(cache, np.uint8)
        if c.shape[-1] != 656:
            raise ValueError("fp8_ds_mla cache rows must be 656 bytes")
        nb = c.size // (64 * 656)
    else:
        raise ValueError("cache_format must be 0 (bf16) or 1 (fp8_ds_mla)")
    bt = _c(block_table, np.int32)
    req = _c(req_id_per_token, np.int32).reshape(-1)
    idx = _c(topk_indices, np.int32)
    if idx.ndim != 2 or idx.shape[0] != T or req.shape[0] != T:
        raise ValueError("topk_indices must be [T, K] and req_id_per_token [T]")
    K = idx.shape[1]
    if tokens is None:
        tok = None
        n = T
    else:
        tok = _c(tokens, np.int64).reshape(-1)
        n = tok.shape[0]
    o = np.empty((n, H, 512), dtype=np.float64)
    lse = np.empty((n, H), dtype=np.float64)
    w = np.empty((n, H, K), dtype=np.float64) if want_weights else None
    rc = _load().smla_oracle_attention(int(cache_format), q.ctypes.data, c.ctypes.data,
                                       bt.ctypes.data, req.ctypes.data, idx.ctypes.data,
                                       float(sm_scale), T, H, K, bt.shape[0], bt.shape[1], nb,
                                       _ptr(tok), n, o.ctypes.data, lse.ctypes.data, _ptr(w))
    if rc != 0:
        raise RuntimeError("oracle attention failed (bad token id or out of memory)")
    if want_weights:
        return o, lse, w
    return o, lse
