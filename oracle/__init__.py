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
``FlashMLASparseImpl.forward`` with its two kernel wrappers. The nvfp4_ds_mla
rows (352 bytes) follow the vLLM pull-request page "Support nvfp4_ds_mla on
FLASHINFER_MLA_SPARSE, with native NVFP4 decode" (row size, exact values in
native decode) with the layout reading stated in ``smla_oracle.c``.
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
NVFP4_CACHE = 2
NVFP4_ROW_BYTES = 352

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
    lib.smla_oracle_e2m1.restype = dbl
    lib.smla_oracle_e2m1.argtypes = [ctypes.c_uint8]
    lib.smla_oracle_e2m1_encode.restype = ctypes.c_uint8
    lib.smla_oracle_e2m1_encode.argtypes = [ctypes.c_float]
    lib.smla_oracle_decode_nvfp4_row.restype = None
    lib.smla_oracle_decode_nvfp4_row.argtypes = [vp, vp]
    lib.smla_oracle_convert_one.restype = i32
    lib.smla_oracle_e4m3fn_encode.restype = ctypes.c_uint8
    lib.smla_oracle_e4m3fn_encode.argtypes = [ctypes.c_float]
    lib.smla_oracle_cache_write.restype = None
    lib.smla_oracle_cache_write.argtypes = [ctypes.c_int, vp, vp, vp, i64, vp, i64]
    lib.smla_oracle_convert_one.argtypes = [i32, i32, vp, i64, i64, i64]
    lib.smla_oracle_convert_indices.restype = None
    lib.smla_oracle_convert_indices.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64]
    lib.smla_oracle_convert_indices_ws.restype = None
    lib.smla_oracle_convert_indices_ws.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64]
    lib.smla_oracle_bf16_rne.restype = ctypes.c_uint16
    lib.smla_oracle_bf16_rne.argtypes = [dbl]
    lib.smla_oracle_gather_upconvert.restype = None
    lib.smla_oracle_gather_upconvert.argtypes = [vp, i64, vp, i64, vp, vp, i64, vp, i64]
    lib.smla_oracle_gather_upconvert_nvfp4.restype = None
    lib.smla_oracle_gather_upconvert_nvfp4.argtypes = [vp, i64, vp, i64, vp, vp, i64, vp, i64]
    lib.smla_oracle_plan_prefill_chunks.restype = i64
    lib.smla_oracle_plan_prefill_chunks.argtypes = [vp, i64, i64, vp, vp]
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


def e2m1(code: int) -> float:
    """Value of one FP4 E2M1 code (low 4 bits)."""
    return _load().smla_oracle_e2m1(int(code) & 0xF)


def e2m1_encode(x: float) -> int:
    """float32 value -> E2M1 code, nearest with ties to even, saturating at 6."""
    return int(_load().smla_oracle_e2m1_encode(float(x)))


def decode_nvfp4_rows(rows: np.ndarray) -> np.ndarray:
    """[n, 352] uint8 nvfp4_ds_mla rows -> [n, 576] float64."""
    rows = _c(rows, np.uint8).reshape(-1, NVFP4_ROW_BYTES)
    out = np.empty((rows.shape[0], 576), dtype=np.float64)
    lib = _load()
    for i in range(rows.shape[0]):
        lib.smla_oracle_decode_nvfp4_row(rows[i].ctypes.data, out[i].ctypes.data)
    return out


def e4m3fn_encode(x: float) -> int:
    """float32 value -> E4M3FN byte, nearest with ties to even, saturating at 448."""
    return int(_load().smla_oracle_e4m3fn_encode(float(x)))


def cache_write(cache_format: int, k_c_bits: np.ndarray, k_pe_bits: np.ndarray,
                slot_mapping: np.ndarray, cache: np.ndarray) -> np.ndarray:
    """Write token rows into `cache` in place (the page's concat_and_cache_mla).
    k_c_bits uint16 [T, 512] and k_pe_bits uint16 [T, 64] are bf16 bit patterns;
    slot_mapping int64 [T]; cache uint16 [NB, 64, 576] (format 0, bf16), uint8
    [NB, 64, 656] (format 1, fp8_ds_mla) or uint8 [NB, 64, 352] (format 2,
    nvfp4_ds_mla). Returns cache."""
    T = int(slot_mapping.shape[0])
    k_c = _c(k_c_bits.reshape(T, 512), np.uint16)
    k_pe = _c(k_pe_bits.reshape(T, 64), np.uint16)
    sm = _c(slot_mapping, np.int64)
    assert cache.flags["C_CONTIGUOUS"]
    want = np.uint16 if cache_format == BF16_CACHE else np.uint8
    assert cache.dtype == want
    row = {BF16_CACHE: 576, FP8_CACHE: 656, NVFP4_CACHE: NVFP4_ROW_BYTES}[cache_format]
    assert cache.shape[-1] == row and cache.size % (64 * row) == 0
    _load().smla_oracle_cache_write(int(cache_format), _ptr(k_c), _ptr(k_pe), _ptr(sm), T, _ptr(cache),
                                    cache.size // row)
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


def convert_indices_workspace(req_id_per_token, block_table, topk_indices, num_blocks: int,
                              prefill_request_id, workspace_starts) -> np.ndarray:
    """Index conversion of the separate-prefill mode: tokens with a prefill request
    id r >= 0 map valid indices to workspace_starts[r] + idx, the others to cache
    slots. Returns int32 [T, K], -1 = invalid."""
    req = _c(req_id_per_token, np.int32).reshape(-1)
    bt = _c(block_table, np.int32)
    idx = _c(topk_indices, np.int32)
    pr = _c(prefill_request_id, np.int32).reshape(-1)
    ws = _c(workspace_starts, np.int32).reshape(-1)
    if bt.ndim != 2 or idx.ndim != 2 or idx.shape[0] != req.shape[0] or pr.shape[0] != req.shape[0]:
        raise ValueError("shapes: block_table [R, MB], topk_indices [T, K], req/prefill ids [T]")
    out = np.empty_like(idx)
    _load().smla_oracle_convert_indices_ws(req.ctypes.data, bt.ctypes.data, idx.ctypes.data,
                                           pr.ctypes.data, ws.ctypes.data if ws.size else None,
                                           out.ctypes.data, idx.shape[0], idx.shape[1], bt.shape[0],
                                           bt.shape[1], int(num_blocks), ws.shape[0])
    return out


def bf16_rne(x: float) -> int:
    """Bit pattern of the bfloat16 nearest to x (ties to even)."""
    return int(_load().smla_oracle_bf16_rne(float(x)))


def gather_upconvert(cache, block_table, seq_lens, workspace_starts, workspace_rows: int,
                     workspace=None, cache_format: int = FP8_CACHE) -> np.ndarray:
    """Upconvert the context rows of prefill requests from an fp8_ds_mla cache
    (uint8 [NB, 64, 656]) or an nvfp4_ds_mla cache (uint8 [NB, 64, 352],
    cache_format NVFP4_CACHE) into a bf16 workspace (uint16 bit patterns
    [workspace_rows, 576]); block_table [B, MB] holds the requests' rows, seq_lens
    and workspace_starts [B]. Rows no request covers keep their contents (zeros
    for a new workspace). Returns the workspace."""
    c = cache if (cache.dtype == np.uint8 and cache.flags.c_contiguous) else _c(cache, np.uint8)
    row = {FP8_CACHE: 656, NVFP4_CACHE: NVFP4_ROW_BYTES}[cache_format]
    if c.shape[-1] != row:
        raise ValueError(f"cache rows must be {row} bytes for this format")
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32).reshape(-1)
    st = _c(workspace_starts, np.int32).reshape(-1)
    if bt.ndim != 2 or bt.shape[0] != sl.shape[0] or st.shape[0] != sl.shape[0]:
        raise ValueError("block_table [B, MB], seq_lens [B], workspace_starts [B]")
    if workspace is None:
        workspace = np.zeros((workspace_rows, 576), dtype=np.uint16)
    assert workspace.dtype == np.uint16 and workspace.flags.c_contiguous
    fn = _load().smla_oracle_gather_upconvert if cache_format == FP8_CACHE else \
        _load().smla_oracle_gather_upconvert_nvfp4
    fn(c.ctypes.data, c.size // (64 * row), bt.ctypes.data, bt.shape[1], sl.ctypes.data, st.ctypes.data,
       sl.shape[0], workspace.ctypes.data, int(workspace_rows))
    return workspace


def plan_prefill_chunks(seq_lens, max_rows: int):
    """Greedy chunks of consecutive prefill requests that fit max_rows workspace
    rows. Returns (chunk_ends list, chunk-local workspace_starts int32 [B]); raises
    ValueError when a request alone does not fit."""
    sl = _c(seq_lens, np.int32).reshape(-1)
    ends = np.zeros(max(sl.shape[0], 1), dtype=np.int32)
    starts = np.zeros(sl.shape[0], dtype=np.int32)
    n = _load().smla_oracle_plan_prefill_chunks(sl.ctypes.data, sl.shape[0], int(max_rows),
                                                ends.ctypes.data, starts.ctypes.data)
    if n < 0:
        raise ValueError("a prefill request does not fit the workspace")
    return [int(e) for e in ends[:n]], starts


def attention(cache_format: int, q_bits, cache, block_table, req_id_per_token, topk_indices,
              sm_scale: float, tokens=None, want_weights: bool = False):
    """Sparse MLA forward on the CPU.

    q_bits: uint16 bf16 patterns [T, H, 576]. cache: uint16 [NB, 64, 576] (bf16),
    uint8 [NB, 64, 656] (fp8_ds_mla) or uint8 [NB, 64, 352] (nvfp4_ds_mla).
    tokens: optional subset of query tokens.
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
    elif cache_format == NVFP4_CACHE:
        c = cache if (cache.dtype == np.uint8 and cache.flags.c_contiguous) else _c(cache, np.uint8)
        if c.shape[-1] != NVFP4_ROW_BYTES:
            raise ValueError("nvfp4_ds_mla cache rows must be 352 bytes")
        nb = c.size // (64 * NVFP4_ROW_BYTES)
    else:
        raise ValueError("cache_format must be 0 (bf16), 1 (fp8_ds_mla) or 2 (nvfp4_ds_mla)")
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


def separate_prefill_attention(q_bits, cache, block_table, req_id_per_token, topk_indices, sm_scale: float,
                               num_decode_reqs: int, seq_lens, max_rows: int, cache_format: int = FP8_CACHE):
    """The separate-prefill mode of an fp8_ds_mla cache, end to end [flashmla_sparse.py page,
    _build_fp8_separate_prefill_decode and _forward_fp8_kv_separate_prefill_decode]
    (or of an nvfp4_ds_mla cache with cache_format NVFP4_CACHE, whose prefill the
    native-decode pull-request page stages through the same kind of gather):
    requests [0, num_decode_reqs) are decode requests, the rest prefill requests
    (prefill index r = request id - num_decode_reqs) with context length
    seq_lens[request]. Decode tokens attend over the fp8 cache; prefill tokens
    attend, chunk by chunk, over their chunk's context rows upconverted to bf16
    in a workspace of at most max_rows rows, through indices converted to
    workspace rows. Returns (o [T, H, 512] float64, lse [T, H] float64)."""
    q = _c(q_bits, np.uint16)
    T, H = q.shape[0], q.shape[1]
    bt = _c(block_table, np.int32)
    req = _c(req_id_per_token, np.int32).reshape(-1)
    idx = _c(topk_indices, np.int32)
    sl = _c(seq_lens, np.int32).reshape(-1)
    nb = cache.size // (64 * {FP8_CACHE: 656, NVFP4_CACHE: NVFP4_ROW_BYTES}[cache_format])
    R = bt.shape[0]
    nd = int(num_decode_reqs)
    prefill_id = np.where(req >= nd, req - nd, -1).astype(np.int32)
    ends, starts = plan_prefill_chunks(sl[nd:R], max_rows)
    phys = convert_indices_workspace(req, bt, idx, nb, prefill_id, starts)
    o = np.zeros((T, H, 512))
    lse = np.full((T, H), -np.inf)
    dec = np.nonzero(prefill_id < 0)[0]
    if dec.size:
        od, ld = attention(cache_format, q, cache, bt, req, idx, sm_scale, tokens=dec)
        o[dec], lse[dec] = od, ld
    c0 = 0
    for c1 in ends:
        rows = int(sl[nd + c0:nd + c1].sum())
        nbw = max(1, -(-rows // 64))
        ws = gather_upconvert(cache, bt[nd + c0:nd + c1], sl[nd + c0:nd + c1], starts[c0:c1], rows,
                              workspace=np.zeros((nbw * 64, 576), dtype=np.uint16), cache_format=cache_format)
        toks = np.nonzero((prefill_id >= c0) & (prefill_id < c1))[0]
        if toks.size:
            # workspace row w = block w // 64, offset w % 64 of a one-request table
            ident = np.arange(nbw, dtype=np.int32).reshape(1, nbw)
            op, lp = attention(BF16_CACHE, q[toks], ws.reshape(nbw, 64, 576), ident,
                               np.zeros(toks.size, dtype=np.int32), phys[toks], sm_scale)
            o[toks], lse[toks] = op, lp
        c0 = c1
    return o, lse

