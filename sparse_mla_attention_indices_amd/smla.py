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

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsmla.so")

SMLA_OK = 0
STATUS_NAMES = {0: "SMLA_OK", 1: "SMLA_ERR_NULL", 2: "SMLA_ERR_SHAPE", 3: "SMLA_ERR_ALIGN",
                4: "SMLA_ERR_WORKSPACE", 5: "SMLA_ERR_HIP", 6: "SMLA_ERR_ARG"}
EXPORTS = ("smla_status_string", "smla_abi_version", "smla_plan", "smla_workspace_size",
           "smla_merge_partials", "smla_concat_and_cache_mla", "smla_convert_indices",
           "smla_prefill_bf16", "smla_decode_fp8")
CACHE_FORMATS = {"auto": 0, "bf16": 0, "fp8_ds_mla": 1}
FLAG_PARTIALS_ONLY = 0x1


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
               out, lse, phys_indices_out, workspace, num_splits, stream, want_lse, partials_only=False):
    T, H, D = q.shape
    if D != 576:
        raise ValueError("q must be [num_tokens, h_q, 576]")
    K = topk_indices.shape[1]
    flags = FLAG_PARTIALS_ONLY if partials_only else 0
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
              block_table.shape[0], block_table.shape[1], kv_cache.shape[0],
              _dev(out, "out", torch.bfloat16, 3), _dev(lse, "lse", torch.float32, 2),
              _dev(phys_indices_out, "phys_indices_out", torch.int32, 2),
              ws_ptr, ws_bytes, _options(num_splits, flags), _stream(stream)), name)
    return out, lse


def smla_prefill_bf16(q, kv_cache, block_table, req_id_per_token, topk_indices, sm_scale,
                      out=None, lse=None, phys_indices_out=None, workspace=None, num_splits=0,
                      stream=None, want_lse=True, partials_only=False):
    """Sparse MLA forward over a bf16 cache [num_blocks, 64, 576]. Returns (out, lse).

    workspace: uint8 device tensor of at least smla_workspace_size bytes (contents
    need not be initialised), or None for one the binding keeps per (device, stream).
    partials_only: write the per-part results into `workspace` (required) for
    smla_merge_partials and return (None, None)."""
    if kv_cache.dtype != torch.bfloat16 or kv_cache.shape[1:] != (64, 576):
        raise ValueError("kv_cache must be bf16 [num_blocks, 64, 576]")
    return _attention("smla_prefill_bf16", q, kv_cache, block_table, req_id_per_token, topk_indices,
                      sm_scale, out, lse, phys_indices_out, workspace, num_splits, stream, want_lse,
                      partials_only)


def smla_decode_fp8(q, kv_cache, block_table, req_id_per_token, topk_indices, sm_scale,
                    out=None, lse=None, phys_indices_out=None, workspace=None, num_splits=0,
                    stream=None, want_lse=True, partials_only=False):
    """Sparse MLA forward over an fp8_ds_mla cache uint8 [num_blocks, 64, 656]. Returns (out, lse).

    Other arguments as for smla_prefill_bf16."""
    if kv_cache.dtype != torch.uint8 or kv_cache.shape[1:] != (64, 656):
        raise ValueError("kv_cache must be uint8 [num_blocks, 64, 656]")
    return _attention("smla_decode_fp8", q, kv_cache, block_table, req_id_per_token, topk_indices,
                      sm_scale, out, lse, phys_indices_out, workspace, num_splits, stream, want_lse,
                      partials_only)
