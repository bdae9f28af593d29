"""Python binding of libsmla.so (argument marshalling only).

The functions carry the names of the C entry points in include/smla.h and pass
torch tensors' device pointers and the current HIP stream straight through. All
computation runs in the library's HIP kernels; there is no fallback path: if the
library is missing or fails to load, every call raises.

torch is imported before the library is opened, so libsmla.so binds to the HIP
runtime torch already loaded (both use the soname libamdhip64.so.7) and torch's
streams and device pointers are valid inside the library.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SMLA_LIB_PATH names another build of the same library (the sanitizer build of
# the host code); by default the in-tree libsmla.so.
LIB_PATH = os.environ.get("SMLA_LIB_PATH") or os.path.join(_PKG, "libsmla.so")

SMLA_OK = 0
STATUS_NAMES = {0: "SMLA_OK", 1: "SMLA_ERR_NULL", 2: "SMLA_ERR_SHAPE", 3: "SMLA_ERR_ALIGN",
                4: "SMLA_ERR_WORKSPACE", 5: "SMLA_ERR_HIP", 6: "SMLA_ERR_ARG"}
EXPORTS = ("smla_status_string", "smla_abi_version", "smla_plan", "smla_workspace_size",
           "smla_merge_partials", "smla_concat_and_cache_mla", "smla_convert_indices",
           "smla_prefill_workspace_rows", "smla_plan_prefill_chunks", "smla_convert_indices_workspace",
           "smla_gather_upconvert_fp8", "smla_gather_upconvert_nvfp4", "smla_prefill_bf16", "smla_decode_fp8",
           "smla_decode_nvfp4",
           "smla_decode_fp8_noalloc")
STATIC_WORKSPACE_BYTES = 64 << 20
CACHE_FORMATS = {"auto": 0, "bf16": 0, "fp8_ds_mla": 1, "nvfp4_ds_mla": 2}
NVFP4_ROW_BYTES = 352
FLAG_PARTIALS_ONLY = 0x1
FLAG_SLOT_INDICES = 0x2
FLAG_DEFER_MERGE = 0x4
FLAG_MERGE_ONLY = 0x8


class SmlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}")


class SmlaOptions(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("reserved", ctypes.c_int32 * 6)]


_lib = None


def library() -> ctypes.CDLL:
    """Open libsmla.so (built by `python -m sparse_mla_attention_indices_amd.build`)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_mla_attention_indices_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    fl = ctypes.c_float
    lib.smla_status_string.restype = ctypes.c_char_p
    lib.smla_status_string.argtypes = [ctypes.c_int]
    lib.smla_abi_version.restype = i32
    lib.smla_abi_version.argtypes = []
    lib.smla_plan.restype = ctypes.c_int
    lib.smla_plan.argtypes = [i32, i32, i32, i32, vp, ctypes.POINTER(i32), ctypes.POINTER(sz)]
    lib.smla_workspace_size.restype = ctypes.c_int
    lib.smla_workspace_size.argtypes = [i32, i32, i32, vp, ctypes.POINTER(sz)]
    lib.smla_merge_partials.restype = ctypes.c_int
    lib.smla_merge_partials.argtypes = [vp, sz, i32, i32, i32, vp, vp, vp]
    lib.smla_concat_and_cache_mla.restype = ctypes.c_int
    lib.smla_concat_and_cache_mla.argtypes = [vp, vp, vp, i32, vp, i64, i32, vp]
    lib.smla_convert_indices.restype = ctypes.c_int
    lib.smla_convert_indices.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i64, vp]
    lib.smla_prefill_workspace_rows.restype = i64
    lib.smla_prefill_workspace_rows.argtypes = [i64]
    lib.smla_plan_prefill_chunks.restype = ctypes.c_int
    lib.smla_plan_prefill_chunks.argtypes = [vp, i32, i64, vp, vp, ctypes.POINTER(i32)]
    lib.smla_convert_indices_workspace.restype = ctypes.c_int
    lib.smla_convert_indices_workspace.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i32, vp]
    for name in ("smla_gather_upconvert_fp8", "smla_gather_upconvert_nvfp4"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = [vp, i64, vp, i32, vp, vp, i32, i32, vp, i64, vp]
    attn = [vp, vp, vp, vp, vp, fl, i32, i32, i32, i32, i32, i64, vp, vp, vp, vp, sz, vp, vp]
    for name in ("smla_prefill_bf16", "smla_decode_fp8", "smla_decode_nvfp4"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = attn
    lib.smla_decode_fp8_noalloc.restype = ctypes.c_int
    lib.smla_decode_fp8_noalloc.argtypes = attn[:15] + attn[17:]
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != SMLA_OK:
        raise SmlaError(status, where)


def _options(num_splits: int, flags: int = 0):
    if not num_splits and not flags:
        return None
    o = SmlaOptions()
    o.num_splits = int(num_splits)
    o.flags = int(flags)
    return ctypes.byref(o)


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dev(t: torch.Tensor | None, name: str, dtype=None, ndim=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    return t.data_ptr()


def smla_abi_version() -> int:
    return int(library().smla_abi_version())


def smla_plan(num_tokens: int, h_q: int, topk: int, num_cus: int, num_splits: int = 0,
              partials_only: bool = False):
    """Host-only split plan: returns (num_splits, workspace_bytes)."""
    s = ctypes.c_int32()
    b = ctypes.c_size_t()
    flags = FLAG_PARTIALS_ONLY if partials_only else 0
    _check(library().smla_plan(num_tokens, h_q, topk, num_cus, _options(num_splits, flags),
                               ctypes.byref(s), ctypes.byref(b)), "smla_plan")
    return s.value, b.value


def smla_workspace_size(num_tokens: int, h_q: int, topk: int, num_splits: int = 0,
                        partials_only: bool = False) -> int:
    b = ctypes.c_size_t()
    flags = FLAG_PARTIALS_ONLY if partials_only else 0
    _check(library().smla_workspace_size(num_tokens, h_q, topk, _options(num_splits, flags),
                                         ctypes.byref(b)), "smla_workspace_size")
    return b.value


def partials_layout(num_tokens: int, h_q: int, num_parts: int):
    """Byte offsets and sizes of a partials buffer: (o_offset, total_bytes). lse is
    fp32 [T][F][H] at offset 0, o is fp32 [T][F][H][512] at o_offset."""
    rows = num_tokens * num_parts * h_q
    o_off = -(-rows * 4 // 256) * 256
    return o_off, o_off + rows * 512 * 4


def smla_merge_partials(partials: torch.Tensor, num_tokens: int, h_q: int, num_parts: int,
                        out=None, lse=None, stream=None, want_lse=True):
    """Log-sum-exp merge of a partials buffer (the workspace of a call made with
    partials_only=True, or parts assembled by the caller). Returns (out, lse)."""
    if out is None:
        out = torch.empty((num_tokens, h_q, 512), dtype=torch.bfloat16, device=partials.device)
    if lse is None and want_lse:
        lse = torch.empty((num_tokens, h_q), dtype=torch.float32, device=partials.device)
    _check(library().smla_merge_partials(_dev(partials, "partials"),
                                         partials.numel() * partials.element_size(), num_tokens, h_q,
                                         num_parts, _dev(out, "out", torch.bfloat16, 3),
                                         _dev(lse, "lse", torch.float32, 2), _stream(stream)),
           "smla_merge_partials")
    return out, lse


# Workspaces the binding allocates itself, one per (device, stream), grown on
# demand.
_own_workspaces: dict = {}


def _own_workspace(device: torch.device, stream, need: int) -> torch.Tensor:
    key = (device.index, _stream(stream))
    ws = _own_workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
        _own_workspaces[key] = ws
    return ws


def smla_concat_and_cache_mla(k_c_normed, k_pe, kv_cache, slot_mapping, kv_cache_dtype="fp8_ds_mla",
                              stream=None):
    """Write each token's latent ([T, 512] bf16) and RoPE ([T, 64] bf16) into its
    slot (int64 [T], block * 64 + offset; negative = skip) of kv_cache: uint8
    [NB, 64, 656] for "fp8_ds_mla", uint8 [NB, 64, 352] for "nvfp4_ds_mla",
    bf16 [NB, 64, 576] for "auto". Returns kv_cache."""
    fmt = CACHE_FORMATS[kv_cache_dtype]
    if fmt == 1 and (kv_cache.dtype != torch.uint8 or kv_cache.shape[1:] != (64, 656)):
        raise ValueError("an fp8_ds_mla cache is uint8 [num_blocks, 64, 656]")
    if fmt == 2 and (kv_cache.dtype != torch.uint8 or kv_cache.shape[1:] != (64, NVFP4_ROW_BYTES)):
        raise ValueError("an nvfp4_ds_mla cache is uint8 [num_blocks, 64, 352]")
    if fmt == 0 and (kv_cache.dtype != torch.bfloat16 or kv_cache.shape[1:] != (64, 576)):
        raise ValueError("a bf16 cache is bfloat16 [num_blocks, 64, 576]")
    T = slot_mapping.shape[0]
    _check(library().smla_concat_and_cache_mla(
        _dev(k_c_normed, "k_c_normed", torch.bfloat16, 2), _dev(k_pe, "k_pe", torch.bfloat16, 2),
        _dev(slot_mapping, "slot_mapping", torch.int64, 1), T, _dev(kv_cache, "kv_cache"),
        kv_cache.shape[0], fmt, _stream(stream)), "smla_concat_and_cache_mla")
    return kv_cache


def smla_convert_indices(req_id_per_token, block_table, topk_indices, num_blocks: int,
                         out=None, stream=None):
    """Logical top-k indices -> physical cache slots (int32, -1 = invalid)."""
    T, K = topk_indices.shape
    if out is None:
        out = torch.empty_like(topk_indices)
    _check(library().smla_convert_indices(
        _dev(req_id_per_token, "req_id_per_token", torch.int32, 1),
        _dev(block_table, "block_table", torch.int32, 2),
        _dev(topk_indices, "topk_indices", torch.int32, 2),
        _dev(out, "out", torch.int32, 2), T, K, block_table.shape[0], block_table.shape[1],
        int(num_blocks), _stream(stream)), "smla_convert_indices")
    return out


def _attention(name: str, q, kv_cache, block_table, req_id_per_token, topk_indices, sm_scale,
               out, lse, phys_indices_out, workspace, num_splits, stream, want_lse, partials_only=False,
               slot_indices=False, stage=None):
    T, H, D = q.shape
    if D != 576:
        raise ValueError("q must be [num_tokens, h_q, 576]")
    K = topk_indices.shape[1]
    flags = (FLAG_PARTIALS_ONLY if partials_only else 0) | (FLAG_SLOT_INDICES if slot_indices else 0)
    if stage is not None:
        if stage not in ("attention", "merge"):
            raise ValueError("stage must be None, 'attention' or 'merge'")
        if workspace is None:
            raise ValueError("a staged call needs the caller's workspace (it carries the parts)")
        flags |= FLAG_DEFER_MERGE if stage == "attention" else FLAG_MERGE_ONLY
    if slot_indices:
        block_table = req_id_per_token = None
    R, MB = (1, 1) if block_table is None else block_table.shape
    if partials_only:
        if workspace is None:
            raise ValueError("partials_only needs a workspace (the partial results go there)")
        out = lse = None
    else:
        if out is None:
            out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=q.device)
        if lse is None and want_lse:
            lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = smla_workspace_size(T, H, K, num_splits)
        if need > 0:
            workspace = _own_workspace(q.device, stream, need)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    fn = getattr(library(), name)
    _check(fn(_dev(q, "q", torch.bfloat16, 3), _dev(kv_cache, "kv_cache"),
              _dev(block_table, "block_table", torch.int32, 2),
              _dev(req_id_per_token, "req_id_per_token", torch.int32, 1),
              _dev(topk_indices, "topk_indices", torch.int32, 2), float(sm_scale), T, H, K,
              R, MB, kv_cache.shape[0],
              _dev(out, "out", torch.bfloat16, 3), _dev(lse, "lse", torch.float32, 2),
              _dev(phys_indices_out, "phys_indices_out", torch.int32, 2),
              ws_ptr, ws_bytes, _options(num_splits, flags), _stream(stream)), name)
    return out, lse


def smla_prefill_bf16(q, kv_cache, block_table, req_id_per_token, topk_indices, sm_scale,
                      out=None, lse=None, phys_indices_out=None, workspace=None, num_splits=0,
                      stream=None, want_lse=True, partials_only=False, slot_indices=False, stage=None):
    """Sparse MLA forward over a bf16 cache [num_blocks, 64, 576]. Returns (out, lse).

    workspace: uint8 device tensor of at least smla_workspace_size bytes (contents
    need not be initialised), or None for one the binding keeps per (device, stream).
    partials_only: write the per-part results into `workspace` (required) for
    smla_merge_partials and return (None, None).
    slot_indices: topk_indices already hold cache slots (block_table and
    req_id_per_token are not used and may be None).
    stage: None (the whole call), "attention" (a split call's attention kernel
    only, its merge deferred) or "merge" (only the merge of such a call, made
    with the same arguments and workspace)."""
    if kv_cache.dtype != torch.bfloat16 or kv_cache.shape[1:] != (64, 576):
        raise ValueError("kv_cache must be bf16 [num_blocks, 64, 576]")
    return _attention("smla_prefill_bf16", q, kv_cache, block_table, req_id_per_token, topk_indices,
                      sm_scale, out, lse, phys_indices_out, workspace, num_splits, stream, want_lse,
                      partials_only, slot_indices, stage)


def smla_decode_fp8(q, kv_cache, block_table, req_id_per_token, topk_indices, sm_scale,
                    out=None, lse=None, phys_indices_out=None, workspace=None, num_splits=0,
                    stream=None, want_lse=True, partials_only=False, slot_indices=False, stage=None):
    """Sparse MLA forward over an fp8_ds_mla cache uint8 [num_blocks, 64, 656]. Returns (out, lse).

    Other arguments as for smla_prefill_bf16."""
    if kv_cache.dtype != torch.uint8 or kv_cache.shape[1:] != (64, 656):
        raise ValueError("kv_cache must be uint8 [num_blocks, 64, 656]")
    return _attention("smla_decode_fp8", q, kv_cache, block_table, req_id_per_token, topk_indices,
                      sm_scale, out, lse, phys_indices_out, workspace, num_splits, stream, want_lse,
                      partials_only, slot_indices, stage)


def smla_decode_nvfp4(q, kv_cache, block_table, req_id_per_token, topk_indices, sm_scale,
                      out=None, lse=None, phys_indices_out=None, workspace=None, num_splits=0,
                      stream=None, want_lse=True, partials_only=False, slot_indices=False, stage=None):
    """Sparse MLA forward over an nvfp4_ds_mla cache uint8 [num_blocks, 64, 352],
    decoded natively (exact values, no staging copy). Returns (out, lse).

    Other arguments as for smla_prefill_bf16."""
    if kv_cache.dtype != torch.uint8 or kv_cache.shape[1:] != (64, NVFP4_ROW_BYTES):
        raise ValueError("kv_cache must be uint8 [num_blocks, 64, 352]")
    return _attention("smla_decode_nvfp4", q, kv_cache, block_table, req_id_per_token, topk_indices,
                      sm_scale, out, lse, phys_indices_out, workspace, num_splits, stream, want_lse,
                      partials_only, slot_indices, stage)


def smla_decode_fp8_noalloc(q, kv_cache, block_table, req_id_per_token, topk_indices, sm_scale, out,
                            lse=None, phys_indices_out=None, num_splits=0, stream=None, slot_indices=False):
    """smla_decode_fp8 with the split workspace in the library's static device
    array (no allocation by the library or here): out (bf16 [T, h_q, 512]) is
    required, lse (fp32 [T, h_q]) and phys_indices_out are optional. Calls that
    may overlap on one device share that array and race. Returns (out, lse)."""
    if kv_cache.dtype != torch.uint8 or kv_cache.shape[1:] != (64, 656):
        raise ValueError("kv_cache must be uint8 [num_blocks, 64, 656]")
    T, H, D = q.shape
    if D != 576:
        raise ValueError("q must be [num_tokens, h_q, 576]")
    K = topk_indices.shape[1]
    if slot_indices:
        block_table = req_id_per_token = None
    R, MB = (1, 1) if block_table is None else block_table.shape
    _check(library().smla_decode_fp8_noalloc(
        _dev(q, "q", torch.bfloat16, 3), _dev(kv_cache, "kv_cache"),
        _dev(block_table, "block_table", torch.int32, 2),
        _dev(req_id_per_token, "req_id_per_token", torch.int32, 1),
        _dev(topk_indices, "topk_indices", torch.int32, 2), float(sm_scale), T, H, K, R, MB, kv_cache.shape[0],
        _dev(out, "out", torch.bfloat16, 3), _dev(lse, "lse", torch.float32, 2),
        _dev(phys_indices_out, "phys_indices_out", torch.int32, 2),
        _options(num_splits, FLAG_SLOT_INDICES if slot_indices else 0), _stream(stream)),
        "smla_decode_fp8_noalloc")
    return out, lse


# ---- separate-prefill mode of an fp8_ds_mla or nvfp4_ds_mla cache (decode
# tokens over the cache, prefill requests chunk by chunk over an upconverted
# bf16 workspace)

def smla_prefill_workspace_rows(max_model_len: int) -> int:
    """bf16 workspace rows reserved for a model (5 x max_model_len)."""
    return int(library().smla_prefill_workspace_rows(int(max_model_len)))


def smla_plan_prefill_chunks(seq_lens, max_rows: int):
    """Host chunk plan: (chunk_ends list, chunk-local workspace starts int32 numpy [B])."""
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32).reshape(-1))
    n = sl.shape[0]
    ends = np.zeros(max(n, 1), dtype=np.int32)
    starts = np.zeros(max(n, 1), dtype=np.int32)
    nc = ctypes.c_int32()
    _check(library().smla_plan_prefill_chunks(sl.ctypes.data if n else None, n, int(max_rows),
                                              ends.ctypes.data, starts.ctypes.data, ctypes.byref(nc)),
           "smla_plan_prefill_chunks")
    return [int(e) for e in ends[:nc.value]], starts[:n]


def smla_convert_indices_workspace(req_id_per_token, block_table, topk_indices, prefill_request_id,
                                   workspace_starts, num_blocks: int, out=None, stream=None):
    """Index conversion of the separate-prefill mode: prefill tokens (id >= 0) get
    workspace rows workspace_starts[id] + index, decode tokens cache slots."""
    T, K = topk_indices.shape
    if out is None:
        out = torch.empty_like(topk_indices)
    P = 0 if workspace_starts is None else workspace_starts.shape[0]
    _check(library().smla_convert_indices_workspace(
        _dev(req_id_per_token, "req_id_per_token", torch.int32, 1),
        _dev(block_table, "block_table", torch.int32, 2),
        _dev(topk_indices, "topk_indices", torch.int32, 2),
        _dev(prefill_request_id, "prefill_request_id", torch.int32, 1),
        _dev(workspace_starts, "workspace_starts", torch.int32, 1) if P else None,
        _dev(out, "out", torch.int32, 2), T, K, block_table.shape[0], block_table.shape[1],
        int(num_blocks), P, _stream(stream)), "smla_convert_indices_workspace")
    return out


def _gather_upconvert(name, row_bytes, kv_cache, block_table, seq_lens, workspace_starts, max_seq_len, workspace,
                      stream):
    if kv_cache.dtype != torch.uint8 or kv_cache.shape[1:] != (64, row_bytes):
        raise ValueError(f"kv_cache must be uint8 [num_blocks, 64, {row_bytes}]")
    if workspace.dtype != torch.bfloat16 or workspace.dim() != 2 or workspace.shape[1] != 576:
        raise ValueError("workspace must be bf16 [rows, 576]")
    B = seq_lens.shape[0]
    _check(getattr(library(), name)(
        _dev(kv_cache, "kv_cache"), kv_cache.shape[0], _dev(block_table, "block_table", torch.int32, 2),
        block_table.shape[1], _dev(seq_lens, "seq_lens", torch.int32, 1),
        _dev(workspace_starts, "workspace_starts", torch.int32, 1), B, int(max_seq_len),
        _dev(workspace, "workspace"), workspace.shape[0], _stream(stream)), name)
    return workspace


def smla_gather_upconvert_fp8(kv_cache, block_table, seq_lens, workspace_starts, max_seq_len: int,
                              workspace, stream=None):
    """Upconvert the context rows of a chunk of prefill requests (block_table rows,
    seq_lens, workspace_starts: device int32) from an fp8_ds_mla cache into the
    bf16 workspace [rows, 576]. Returns workspace."""
    return _gather_upconvert("smla_gather_upconvert_fp8", 656, kv_cache, block_table, seq_lens, workspace_starts,
                             max_seq_len, workspace, stream)


def smla_gather_upconvert_nvfp4(kv_cache, block_table, seq_lens, workspace_starts, max_seq_len: int,
                                workspace, stream=None):
    """smla_gather_upconvert_fp8 over an nvfp4_ds_mla cache uint8 [num_blocks, 64,
    352]: the staged rows hold the exact values. Returns workspace."""
    return _gather_upconvert("smla_gather_upconvert_nvfp4", NVFP4_ROW_BYTES, kv_cache, block_table, seq_lens,
                             workspace_starts, max_seq_len, workspace, stream)


class SeparatePrefillPlan:
    """Per-batch metadata of the separate-prefill mode, built once per batch on
    the host (as the backend's metadata builder does) and reused by every call
    over that batch: the decode token range, the prefill chunks (request and
    token ranges, context rows, longest context), and three device arrays
    uploaded once: per-token prefill request ids (-1 for decode tokens), each
    prefill request's chunk-local workspace start, and its sequence length."""

    def __init__(self, num_tokens, num_decode_reqs, decode_tokens, chunks, prefill_request_id,
                 workspace_starts, seq_lens, workspace_rows):
        self.num_tokens = num_tokens
        self.num_decode_reqs = num_decode_reqs
        self.decode_tokens = decode_tokens          # (t0, t1)
        self.chunks = chunks                        # [(c0, c1, t0, t1, rows, max_seq_len)], c = prefill index
        self.prefill_request_id = prefill_request_id
        self.workspace_starts = workspace_starts
        self.seq_lens = seq_lens
        self.workspace_rows = workspace_rows


def smla_build_separate_prefill_plan(query_start_loc, seq_lens, num_decode_reqs: int, max_rows: int,
                                     device) -> SeparatePrefillPlan:
    """Host metadata of a batch for smla_forward_fp8_separate_prefill.

    query_start_loc: host sequence of R + 1 token offsets (request r owns tokens
    [query_start_loc[r], query_start_loc[r + 1]); decode requests come first).
    seq_lens: host sequence of R lengths (context + query). Requests
    [0, num_decode_reqs) are decode requests. The chunk plan is the library's
    host call smla_plan_prefill_chunks over the prefill lengths."""
    qsl = np.asarray(query_start_loc, dtype=np.int64).reshape(-1)
    sl = np.asarray(seq_lens, dtype=np.int64).reshape(-1)
    R = sl.shape[0]
    nd = int(num_decode_reqs)
    if qsl.shape[0] != R + 1 or qsl[0] != 0 or np.any(np.diff(qsl) < 0):
        raise ValueError("query_start_loc needs R + 1 non-decreasing offsets starting at 0")
    if not 0 <= nd <= R:
        raise ValueError("num_decode_reqs outside [0, R]")
    T = int(qsl[-1])
    counts = np.diff(qsl)
    pid = np.repeat(np.concatenate([np.full(nd, -1), np.arange(R - nd)]).astype(np.int32), counts)
    ends, starts = smla_plan_prefill_chunks(sl[nd:], max_rows)
    chunks = []
    c0 = 0
    for c1 in ends:
        rows = int(sl[nd + c0:nd + c1].sum())
        longest = int(sl[nd + c0:nd + c1].max()) if c1 > c0 else 0
        chunks.append((c0, c1, int(qsl[nd + c0]), int(qsl[nd + c1]), rows, longest))
        c0 = c1
    P = R - nd
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    return SeparatePrefillPlan(T, nd, (0, int(qsl[nd])), chunks, up(pid), up(starts) if P else None,
                               up(sl[nd:]) if P else None, -(-int(max_rows) // 64) * 64)


def smla_forward_fp8_separate_prefill(q, kv_cache, block_table, req_id_per_token, topk_indices, sm_scale,
                                      plan: SeparatePrefillPlan, out=None, lse=None, bf16_workspace=None,
                                      slots=None, stream=None):
    """The separate-prefill mode end to end, as library calls only: the
    workspace index conversion over the whole batch, smla_decode_fp8 over the
    fp8 cache for the decode tokens, then for each prefill chunk
    smla_gather_upconvert_fp8 (its requests' context rows into bf16_workspace)
    and smla_prefill_bf16 over that workspace with workspace-row indices.
    plan comes from smla_build_separate_prefill_plan. bf16_workspace: bf16
    [>= plan.workspace_rows, 576]; slots: int32 [T, topk] scratch for the
    converted indices; out, lse: results. Each is allocated when None. Returns
    (out, lse)."""
    return _forward_separate_prefill(smla_decode_fp8, smla_gather_upconvert_fp8, q, kv_cache, block_table,
                                     req_id_per_token, topk_indices, sm_scale, plan, out, lse, bf16_workspace,
                                     slots, stream)


def smla_forward_nvfp4_separate_prefill(q, kv_cache, block_table, req_id_per_token, topk_indices, sm_scale,
                                        plan: SeparatePrefillPlan, out=None, lse=None, bf16_workspace=None,
                                        slots=None, stream=None):
    """smla_forward_fp8_separate_prefill over an nvfp4_ds_mla cache: decode
    tokens through smla_decode_nvfp4, prefill chunks staged by
    smla_gather_upconvert_nvfp4 (exact values) and run by smla_prefill_bf16."""
    return _forward_separate_prefill(smla_decode_nvfp4, smla_gather_upconvert_nvfp4, q, kv_cache, block_table,
                                     req_id_per_token, topk_indices, sm_scale, plan, out, lse, bf16_workspace,
                                     slots, stream)


def _forward_separate_prefill(decode, upconvert, q, kv_cache, block_table, req_id_per_token, topk_indices,
                              sm_scale, plan, out, lse, bf16_workspace, slots, stream):
    """The steps of both separate-prefill entries; decode and upconvert are the
    format's library calls."""
    T, H, _ = q.shape
    if plan.num_tokens != T:
        raise ValueError("the plan was built for another batch")
    dev = q.device
    ws_rows = plan.workspace_rows
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    if bf16_workspace is None:
        bf16_workspace = torch.empty((ws_rows, 576), dtype=torch.bfloat16, device=dev)
    elif bf16_workspace.shape[0] < ws_rows:
        raise ValueError(f"bf16_workspace needs {ws_rows} rows")
    slots = smla_convert_indices_workspace(req_id_per_token, block_table, topk_indices, plan.prefill_request_id,
                                           plan.workspace_starts, kv_cache.shape[0], out=slots, stream=stream)
    d0, d1 = plan.decode_tokens
    if d1 > d0:
        decode(q[d0:d1], kv_cache, None, None, slots[d0:d1], sm_scale, out=out[d0:d1],
               lse=lse[d0:d1], stream=stream, slot_indices=True)
    ws_view = bf16_workspace[:ws_rows].view(ws_rows // 64, 64, 576)
    for c0, c1, t0, t1, rows, longest in plan.chunks:
        if rows > 0:
            nd = plan.num_decode_reqs
            upconvert(kv_cache, block_table[nd + c0:nd + c1], plan.seq_lens[c0:c1],
                      plan.workspace_starts[c0:c1], longest, bf16_workspace, stream=stream)
        if t1 > t0:
            smla_prefill_bf16(q[t0:t1], ws_view, None, None, slots[t0:t1], sm_scale, out=out[t0:t1],
                              lse=lse[t0:t1], stream=stream, slot_indices=True)
    return out, lse
