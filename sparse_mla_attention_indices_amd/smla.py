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
LIB_PATH = os.path.join(_PKG, "libsmla.so")

SMLA_OK = 0
STATUS_NAMES = {0: "SMLA_OK", 1: "SMLA_ERR_NULL", 2: "SMLA_ERR_SHAPE", 3: "SMLA_ERR_ALIGN",
                4: "SMLA_ERR_WORKSPACE", 5: "SMLA_ERR_HIP", 6: "SMLA_ERR_ARG"}
EXPORTS = ("smla_status_string", "smla_abi_version", "smla_plan", "smla_workspace_size",
           "smla_merge_partials", "smla_concat_and_cache_mla", "smla_convert_indices",
           "smla_prefill_workspace_rows", "smla_plan_prefill_chunks", "smla_convert_indices_workspace",
           "smla_gather_upconvert_fp8", "smla_prefill_bf16", "smla_decode_fp8")
CACHE_FORMATS = {"auto": 0, "bf16": 0, "fp8_ds_mla": 1}
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
    lib.smla_gather_upconvert_fp8.restype = ctypes.c_int
    lib.smla_gather_upconvert_fp8.argtypes = [vp, i64, vp, i32, vp, vp, i32, i32, vp, i64, vp]
    attn = [vp, vp, vp, vp, vp, fl, i32, i32, i32, i32, i32, i64, vp, vp, vp, vp, sz, vp, vp]
    for name in ("smla_prefill_bf16", "smla_decode_fp8"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = attn
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
    [NB, 64, 656] for "fp8_ds_mla", bf16 [NB, 64, 576] for "auto". Returns kv_cache."""
    fmt = CACHE_FORMATS[kv_cache_dtype]
    if fmt == 1 and (kv_cache.dtype != torch.uint8 or kv_cache.shape[1:] != (64, 656)):
        raise ValueError("an fp8_ds_mla cache is uint8 [num_blocks, 64, 656]")
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


# ---- separate-prefill mode of an fp8_ds_mla cache (decode tokens over the fp8
# cache, prefill requests chunk by chunk over an upconverted bf16 workspace)

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


def smla_gather_upconvert_fp8(kv_cache, block_table, seq_lens, workspace_starts, max_seq_len: int,
                              workspace, stream=None):
    """Upconvert the context rows of a chunk of prefill requests (block_table rows,
    seq_lens, workspace_starts: device int32) from an fp8_ds_mla cache into the
    bf16 workspace [rows, 576]. Returns workspace."""
    if kv_cache.dtype != torch.uint8 or kv_cache.shape[1:] != (64, 656):
        raise ValueError("kv_cache must be uint8 [num_blocks, 64, 656]")
    if workspace.dtype != torch.bfloat16 or workspace.dim() != 2 or workspace.shape[1] != 576:
        raise ValueError("workspace must be bf16 [rows, 576]")
    B = seq_lens.shape[0]
    _check(library().smla_gather_upconvert_fp8(
        _dev(kv_cache, "kv_cache"), kv_cache.shape[0], _dev(block_table, "block_table", torch.int32, 2),
        block_table.shape[1], _dev(seq_lens, "seq_lens", torch.int32, 1),
        _dev(workspace_starts, "workspace_starts", torch.int32, 1), B, int(max_seq_len),
        _dev(workspace, "workspace"), workspace.shape[0], _stream(stream)), "smla_gather_upconvert_fp8")
    return workspace


def smla_forward_fp8_separate_prefill(q, kv_cache, block_table, req_id_per_token, topk_indices, sm_scale,
                                      num_decode_reqs: int, seq_lens, max_rows: int, out=None, lse=None,
                                      bf16_workspace=None, stream=None):
    """The separate-prefill mode end to end. Requests [0, num_decode_reqs) are
    decode requests, the rest prefill requests; seq_lens (host sequence, one per
    request) gives each request's context + query length. Decode tokens run
    smla_decode_fp8 over the cache; prefill requests are cut into chunks of at
    most max_rows context rows, and for each chunk the rows are upconverted into
    bf16_workspace (bf16 [>= max_rows rounded up to 64, 576]; allocated when None)
    and its tokens run smla_prefill_bf16 over it with workspace-row indices.
    Tokens must be ordered by request. Returns (out, lse)."""
    T, H, _ = q.shape
    dev = q.device
    R = block_table.shape[0]
    nd = int(num_decode_reqs)
    sl = np.asarray(seq_lens, dtype=np.int64).reshape(-1)
    if sl.shape[0] != R:
        raise ValueError("seq_lens needs one length per request")
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    ends, starts = smla_plan_prefill_chunks(sl[nd:], max_rows)
    ws_rows = -(-int(max_rows) // 64) * 64
    if bf16_workspace is None:
        bf16_workspace = torch.empty((ws_rows, 576), dtype=torch.bfloat16, device=dev)
    elif bf16_workspace.shape[0] < ws_rows:
        raise ValueError(f"bf16_workspace needs {ws_rows} rows")
    req = req_id_per_token
    with torch.cuda.stream(stream) if stream is not None else torch.cuda.stream(torch.cuda.current_stream()):
        prefill_id = torch.where(req >= nd, req - nd, torch.full_like(req, -1))
        starts_d = torch.from_numpy(np.ascontiguousarray(starts, dtype=np.int32)).to(dev)
        sl_d = torch.from_numpy(sl[nd:].astype(np.int32)).to(dev)
    slots = smla_convert_indices_workspace(req, block_table, topk_indices, prefill_id,
                                           starts_d if len(starts) else None, kv_cache.shape[0],
                                           stream=stream)
    req_h = req.cpu().numpy()
    tok_of = [np.nonzero(req_h == r)[0] for r in range(R)]
    dec = np.concatenate(tok_of[:nd]) if nd else np.zeros(0, dtype=np.int64)
    if dec.size:
        d0, d1 = int(dec.min()), int(dec.max()) + 1
        if d1 - d0 != dec.size:
            raise ValueError("decode tokens must be contiguous")
        smla_decode_fp8(q[d0:d1], kv_cache, None, None, slots[d0:d1], sm_scale, out=out[d0:d1],
                        lse=lse[d0:d1], stream=stream, slot_indices=True)
    ws_view = bf16_workspace[:ws_rows].view(ws_rows // 64, 64, 576)
    c0 = 0
    for c1 in ends:
        toks = np.concatenate(tok_of[nd + c0:nd + c1])
        rows = int(sl[nd + c0:nd + c1].sum())
        if rows > 0:
            smla_gather_upconvert_fp8(kv_cache, block_table[nd + c0:nd + c1], sl_d[c0:c1], starts_d[c0:c1],
                                      int(sl[nd + c0:nd + c1].max()), bf16_workspace, stream=stream)
        if toks.size:
            t0, t1 = int(toks.min()), int(toks.max()) + 1
            if t1 - t0 != toks.size:
                raise ValueError("a chunk's tokens must be contiguous")
            smla_prefill_bf16(q[t0:t1], ws_view, None, None, slots[t0:t1], sm_scale, out=out[t0:t1],
                              lse=lse[t0:t1], stream=stream, slot_indices=True)
        c0 = c1
    return out, lse
