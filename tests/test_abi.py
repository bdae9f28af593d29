"""C-ABI checks that need no GPU: the library loads, exports every function
include/smla.h declares, plans splits by host arithmetic, and rejects invalid
arguments before making any HIP call (every call here fails validation, so no
device is touched)."""

import ctypes
import os
import re

import pytest

from sparse_mla_attention_indices_amd import smla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smla.h")

A16 = 0x10000          # fake, 256-byte aligned addresses: never dereferenced
A16B = 0x20000
MIS = 0x10002          # misaligned
A256 = 0x30000


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(smla_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(smla.LIB_PATH):
        pytest.fail("libsmla.so not built (run __graft_entry__.build())")
    return smla.library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(smla.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version(lib):
    assert smla.smla_abi_version() == 8


def test_status_strings(lib):
    for code, name in smla.STATUS_NAMES.items():
        assert lib.smla_status_string(code).decode().startswith(name)


def test_plan_fills_the_chip_for_small_decode_batches(lib):
    # 64 tokens x 64 heads: one 64-head workgroup per token -> 4 top-k splits
    # fill 256 CUs once
    s, ws = smla.smla_plan(64, 64, 2048, 256)
    assert s == 4
    up = lambda v: -(-v // 256) * 256
    rows = 64 * 4 * 64
    o_off = up(rows * 4)                     # the partial lse first, then the partial o,
    assert ws == up(up(o_off + rows * 512 * 4) + 64 * 4 * 4)     # then a flag per (token, part)
    # two-wave workgroups (h_q = 16) fit two per CU: 256 tokens x 16 heads -> 2 splits
    assert smla.smla_plan(256, 16, 2048, 256)[0] == 2
    assert smla.smla_plan(256, 16, 1024, 256)[0] == 2
    # ... unless the list is short (<= 512) and every CU already has a workgroup
    assert smla.smla_plan(256, 16, 512, 256) == (1, 0)
    assert smla.smla_plan(255, 16, 512, 256)[0] == 3         # 255 < 256 CUs: split as before
    assert smla.smla_plan(256, 32, 512, 256) == (1, 0)
    # 32-head workgroups fit two per CU: 64 tokens x 32 heads -> 8 splits
    assert smla.smla_plan(64, 32, 2048, 256)[0] == 8
    # 128 heads, 32 tokens: one 128-head workgroup per token -> 8 splits
    assert smla.smla_plan(32, 128, 2048, 256)[0] == 8
    # enough (token, head-block) units already: no split, no workspace
    assert smla.smla_plan(512, 16, 2048, 256) == (1, 0)
    assert smla.smla_plan(16384, 128, 2048, 256) == (1, 0)
    # a split never exceeds the number of 64-row tiles of the list
    assert smla.smla_plan(1, 64, 100, 256)[0] == 2
    assert smla.smla_plan(1, 16, 64, 256)[0] == 1
    # forced splits, capped at topk
    assert smla.smla_plan(8, 16, 64, 256, num_splits=3)[0] == 3
    assert smla.smla_plan(8, 16, 5, 256, num_splits=9)[0] == 5
    assert smla.smla_plan(0, 16, 64, 256) == (1, 0)
    # never more than 32 parts, forced or planned
    assert smla.smla_plan(8, 16, 4096, 256, num_splits=100)[0] == 32
    assert smla.smla_plan(1, 16, 16384, 256)[0] == 32


def test_plan_workspace_layout_for_large_batches(lib):
    # [T][S][H] fp32 lse, then [T][S][H][512] fp32 partial outputs, then [T][S]
    # int32 flags, 256-B aligned; a partials-only call needs no flags
    up = lambda v: -(-v // 256) * 256
    s, ws = smla.smla_plan(5000, 16, 64, 256, num_splits=2)
    rows = 5000 * 2 * 16
    assert s == 2 and ws == up(up(up(rows * 4) + rows * 512 * 4) + 5000 * 2 * 4)
    s, ws = smla.smla_plan(5000, 16, 64, 256, num_splits=2, partials_only=True)
    assert s == 2 and ws == up(up(rows * 4) + rows * 512 * 4)


@pytest.mark.parametrize("args,code", [
    ((8, 48, 64, 256), 2),     # h_q not supported
    ((8, 16, 0, 256), 2),      # topk < 1
    ((-1, 16, 64, 256), 2),    # negative token count
    ((8, 16, 64, 0), 6),       # no compute units
])
def test_plan_rejects(lib, args, code):
    with pytest.raises(smla.SmlaError) as e:
        smla.smla_plan(*args)
    assert e.value.status == code


def test_plan_rejects_bad_options(lib):
    o = smla.SmlaOptions()
    o.reserved[3] = 1
    s, b = ctypes.c_int32(), ctypes.c_size_t()
    assert lib.smla_plan(8, 16, 64, 256, ctypes.byref(o), ctypes.byref(s), ctypes.byref(b)) == 6
    o = smla.SmlaOptions()
    o.num_splits = -2
    assert lib.smla_plan(8, 16, 64, 256, ctypes.byref(o), ctypes.byref(s), ctypes.byref(b)) == 6
    o = smla.SmlaOptions()
    for bit in (0x10, 0x80000000):           # unknown flag bits
        o.flags = bit
        assert lib.smla_plan(8, 16, 64, 256, ctypes.byref(o), ctypes.byref(s), ctypes.byref(b)) == 6
    # a deferred merge and a merge-only call exclude each other and partials-only
    for bits in (0xC, 0x5, 0x9):
        o.flags = bits
        assert lib.smla_plan(8, 16, 64, 256, ctypes.byref(o), ctypes.byref(s), ctypes.byref(b)) == 6
    for bits in (0x4, 0x8, 0x6, 0xA):
        o.flags = bits
        assert lib.smla_plan(8, 16, 64, 256, ctypes.byref(o), ctypes.byref(s), ctypes.byref(b)) == 0
    o.flags = smla.FLAG_PARTIALS_ONLY
    assert lib.smla_plan(8, 16, 64, 256, ctypes.byref(o), ctypes.byref(s), ctypes.byref(b)) == 0
    assert lib.smla_plan(8, 16, 64, 256, None, None, ctypes.byref(b)) == 1


def _attn(lib, name="smla_decode_fp8", q=A16, kv=A16, bt=A16, req=A16, idx=A16, scale=0.04,
          T=8, H=16, K=64, R=2, MB=4, NB=8, out=A16B, lse=A16, phys=None, ws=None, wsb=0, opts=None):
    return getattr(lib, name)(q, kv, bt, req, idx, scale, T, H, K, R, MB, NB, out, lse, phys,
                              ws, wsb, opts, None)


@pytest.mark.parametrize("name", ["smla_decode_fp8", "smla_decode_nvfp4", "smla_prefill_bf16"])
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(kv=None), 1), (dict(bt=None), 1), (dict(req=None), 1),
    (dict(idx=None), 1), (dict(out=None), 1),
    (dict(H=8), 2), (dict(H=96), 2), (dict(K=0), 2), (dict(K=(1 << 20) + 1), 2), (dict(T=-1), 2),
    (dict(R=0), 2), (dict(MB=0), 2), (dict(NB=0), 2), (dict(NB=(1 << 31) // 64 + 1), 2),
    (dict(q=MIS), 3), (dict(kv=MIS), 3), (dict(out=MIS), 3), (dict(bt=A16 + 2), 3),
    (dict(lse=A16 + 1), 3), (dict(phys=A16 + 2), 3), (dict(ws=A16 + 16, wsb=1024), 3),
    (dict(scale=0.0), 6), (dict(scale=-1.0), 6), (dict(scale=float("inf")), 6),
    (dict(scale=float("nan")), 6),
])
def test_attention_rejects_before_any_hip_call(lib, name, kw, code):
    assert _attn(lib, name, **kw) == code


@pytest.mark.parametrize("name", ["smla_decode_fp8", "smla_decode_nvfp4", "smla_prefill_bf16"])
def test_attention_rejects_bad_options(lib, name):
    o = smla.SmlaOptions()
    o.reserved[0] = 5
    assert _attn(lib, name, opts=ctypes.byref(o)) == 6
    o = smla.SmlaOptions()
    o.num_splits = -1
    assert _attn(lib, name, opts=ctypes.byref(o)) == 6
    o = smla.SmlaOptions()
    o.flags = 0x80000000
    assert _attn(lib, name, opts=ctypes.byref(o)) == 6


@pytest.mark.parametrize("name", ["smla_decode_fp8", "smla_decode_nvfp4", "smla_prefill_bf16"])
def test_zero_tokens_is_a_noop(lib, name):
    # no pointer is needed and nothing is launched
    assert _attn(lib, name, q=None, kv=None, bt=None, req=None, idx=None, out=None, T=0) == 0


def _noalloc(lib, q=A16, kv=A16, bt=A16, req=A16, idx=A16, scale=0.04, T=8, H=16, K=64, R=2, MB=4, NB=8,
             out=A16B, lse=A16, phys=None, opts=None):
    return lib.smla_decode_fp8_noalloc(q, kv, bt, req, idx, scale, T, H, K, R, MB, NB, out, lse, phys, opts, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(idx=None), 1), (dict(H=8), 2), (dict(K=0), 2),
    (dict(q=MIS), 3), (dict(out=MIS), 3), (dict(scale=0.0), 6),
])
def test_noalloc_rejects_before_any_hip_call(lib, kw, code):
    assert _noalloc(lib, **kw) == code


def test_noalloc_rejects_staged_and_parts_only_flags(lib):
    for bits in (smla.FLAG_PARTIALS_ONLY, smla.FLAG_DEFER_MERGE, smla.FLAG_MERGE_ONLY):
        o = smla.SmlaOptions()
        o.flags = bits
        assert _noalloc(lib, opts=ctypes.byref(o)) == 6
    assert _noalloc(lib, q=None, kv=None, bt=None, req=None, idx=None, out=None, T=0) == 0


def test_options_struct_layout():
    # num_splits, flags, reserved[6]: 32 bytes, as in include/smla.h
    assert ctypes.sizeof(smla.SmlaOptions) == 32
    assert smla.SmlaOptions.flags.offset == 4 and smla.SmlaOptions.reserved.offset == 8


def test_workspace_size_validation(lib):
    b = ctypes.c_size_t(123)
    assert lib.smla_workspace_size(4, 16, 64, None, None) == 1
    assert lib.smla_workspace_size(4, 20, 64, None, ctypes.byref(b)) == 2
    assert lib.smla_workspace_size(0, 16, 64, None, ctypes.byref(b)) == 0 and b.value == 0


@pytest.mark.parametrize("kw,code", [
    (dict(req=None), 1), (dict(out=None), 1), (dict(K=0), 2), (dict(T=-3), 2), (dict(R=0), 2),
    (dict(NB=(1 << 31) // 64 + 1), 2), (dict(out=A16 + 2), 3), (dict(idx=A16 + 1), 3),
])
def test_convert_rejects(lib, kw, code):
    a = dict(req=A16, bt=A16, idx=A16, out=A16B, T=4, K=7, R=3, MB=3, NB=6)
    a.update(kw)
    assert lib.smla_convert_indices(a["req"], a["bt"], a["idx"], a["out"], a["T"], a["K"],
                                    a["R"], a["MB"], a["NB"], None) == code


def test_convert_zero_tokens_is_a_noop(lib):
    assert lib.smla_convert_indices(None, None, None, None, 0, 7, 3, 3, 6, None) == 0


def test_plan_partials_only_needs_a_workspace_even_unsplit(lib):
    # 512 tokens x 16 heads fill the chip: one part, no workspace ...
    assert smla.smla_plan(512, 16, 2048, 256) == (1, 0)
    # ... but a partials-only call writes its one part there
    s, ws = smla.smla_plan(512, 16, 2048, 256, partials_only=True)
    o_off, total = smla.partials_layout(512, 16, 1)
    assert s == 1 and ws == total and o_off == 512 * 16 * 4


def test_partials_layout_matches_the_plan(lib):
    up = lambda v: -(-v // 256) * 256
    for T, H, K, S in ((64, 64, 2048, 4), (5, 16, 300, 3), (1000, 128, 64, 2)):
        s, ws = smla.smla_plan(T, H, K, 256, num_splits=S, partials_only=True)
        assert s == S and ws == smla.partials_layout(T, H, S)[1]
        # a call that merges its own parts also keeps one flag per (token, part)
        s, ws = smla.smla_plan(T, H, K, 256, num_splits=S)
        assert s == S and ws == up(smla.partials_layout(T, H, S)[1] + T * S * 4)


def _merge(lib, part=A256, pb=1 << 30, T=4, H=16, F=2, out=A16B, lse=A16):
    return lib.smla_merge_partials(part, pb, T, H, F, out, lse, None)


@pytest.mark.parametrize("kw,code", [
    (dict(part=None), 1), (dict(out=None), 1),
    (dict(H=48), 2), (dict(F=0), 2), (dict(F=4097), 2), (dict(T=-1), 2),
    (dict(part=A256 + 16), 3), (dict(out=MIS), 3), (dict(lse=A16 + 2), 3),
    (dict(pb=1024), 4),
])
def test_merge_rejects_before_any_hip_call(lib, kw, code):
    assert _merge(lib, **kw) == code


def test_merge_zero_tokens_is_a_noop(lib):
    assert _merge(lib, part=None, out=None, T=0) == 0


def _cw(lib, kc=A16, kpe=A16B, sm=A256, T=4, kv=A16, NB=8, fmt=1):
    return lib.smla_concat_and_cache_mla(kc, kpe, sm, T, kv, NB, fmt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(kc=None), 1), (dict(kpe=None), 1), (dict(sm=None), 1), (dict(kv=None), 1),
    (dict(T=-1), 2), (dict(NB=0), 2),
    (dict(kc=MIS), 3), (dict(kpe=A16 + 8), 3), (dict(sm=A256 + 4), 3), (dict(kv=A16 + 4), 3),
    (dict(fmt=3), 6), (dict(fmt=-1), 6),
])
def test_cache_write_rejects_before_any_hip_call(lib, kw, code):
    assert _cw(lib, **kw) == code


def test_cache_write_zero_tokens_is_a_noop(lib):
    assert _cw(lib, kc=None, kpe=None, sm=None, kv=None, T=0) == 0


# ------------------------------------------------------- separate-prefill mode

@pytest.mark.parametrize("name", ["smla_decode_fp8", "smla_decode_nvfp4", "smla_prefill_bf16"])
def test_slot_indices_need_no_table_or_request_ids(lib, name):
    o = smla.SmlaOptions()
    o.flags = smla.FLAG_SLOT_INDICES
    # validation passes the missing table / request ids and stops at the missing q
    assert _attn(lib, name, q=None, bt=None, req=None, R=0, MB=0, opts=ctypes.byref(o)) == 1
    assert _attn(lib, name, bt=None, req=None, T=0, opts=ctypes.byref(o)) == 0
    # without the flag a missing table is an error before anything runs
    assert _attn(lib, name, bt=None) == 1


def test_prefill_workspace_rows(lib):
    assert smla.smla_prefill_workspace_rows(163840) == 5 * 163840
    assert smla.smla_prefill_workspace_rows(0) == 0 and smla.smla_prefill_workspace_rows(-4) == 0


def test_prefill_chunk_plan_matches_the_oracle():
    import numpy as np
    import oracle
    rng = np.random.default_rng(3)
    for _ in range(200):
        n = int(rng.integers(0, 10))
        lens = rng.integers(0, 50, n)
        m = int(rng.integers(max(int(lens.max()) if n else 1, 1), 120))
        got = smla.smla_plan_prefill_chunks(lens, m)
        if n == 0:
            assert got[0] == [] and len(got[1]) == 0
            continue
        want = oracle.plan_prefill_chunks(lens, m)
        assert got[0] == want[0] and np.array_equal(got[1], want[1])


def test_prefill_chunk_plan_rejects(lib):
    with pytest.raises(smla.SmlaError):
        smla.smla_plan_prefill_chunks([5, 30], 20)          # a request longer than the workspace
    with pytest.raises(smla.SmlaError):
        smla.smla_plan_prefill_chunks([5, -1], 20)
    n = ctypes.c_int32()
    assert lib.smla_plan_prefill_chunks(None, 2, 10, A16, A16, ctypes.byref(n)) == 1
    assert lib.smla_plan_prefill_chunks(None, 0, 10, None, None, None) == 1
    assert lib.smla_plan_prefill_chunks(None, 0, 10, None, None, ctypes.byref(n)) == 0 and n.value == 0


def _convert_ws(lib, req=A16, bt=A16, idx=A16, pid=A16, st=A16, out=A16B, T=4, K=64, R=2, MB=4, NB=8, P=2):
    return lib.smla_convert_indices_workspace(req, bt, idx, pid, st, out, T, K, R, MB, NB, P, None)


@pytest.mark.parametrize("kw,code", [
    (dict(req=None), 1), (dict(bt=None), 1), (dict(idx=None), 1), (dict(pid=None), 1), (dict(out=None), 1),
    (dict(st=None), 1), (dict(K=0), 2), (dict(T=-1), 2), (dict(P=-1), 2), (dict(R=0), 2), (dict(NB=0), 2),
    (dict(pid=A16 + 2), 3), (dict(st=A16 + 1), 3), (dict(out=A16B + 2), 3),
])
def test_convert_workspace_rejects(lib, kw, code):
    assert _convert_ws(lib, **kw) == code


def test_convert_workspace_zero_tokens_and_no_prefills(lib):
    assert _convert_ws(lib, req=None, bt=None, idx=None, pid=None, st=None, out=None, T=0) == 0
    # no prefill requests: workspace_starts may be NULL (validation then stops at idx)
    assert _convert_ws(lib, st=None, P=0, idx=None) == 1


def _upconvert(lib, kv=A16, NB=8, bt=A16, MB=4, sl=A16, st=A16, B=2, L=100, ws=A16B, rows=256,
               name="smla_gather_upconvert_fp8"):
    return getattr(lib, name)(kv, NB, bt, MB, sl, st, B, L, ws, rows, None)


@pytest.mark.parametrize("kw,code", [
    (dict(kv=None), 1), (dict(bt=None), 1), (dict(sl=None), 1), (dict(st=None), 1), (dict(ws=None), 1),
    (dict(B=-1), 2), (dict(L=-1), 2), (dict(rows=-1), 2), (dict(MB=0), 2), (dict(NB=0), 2),
    (dict(NB=(1 << 31) // 64 + 1), 2), (dict(B=65536), 2),
    (dict(kv=MIS), 3), (dict(ws=A16B + 8), 3), (dict(bt=A16 + 2), 3), (dict(sl=A16 + 1), 3),
])
@pytest.mark.parametrize("name", ["smla_gather_upconvert_fp8", "smla_gather_upconvert_nvfp4"])
def test_upconvert_rejects(lib, kw, code, name):
    assert _upconvert(lib, name=name, **kw) == code


@pytest.mark.parametrize("name", ["smla_gather_upconvert_fp8", "smla_gather_upconvert_nvfp4"])
def test_upconvert_empty_batch_is_a_noop(lib, name):
    assert _upconvert(lib, kv=None, bt=None, sl=None, st=None, ws=None, B=0, name=name) == 0
    assert _upconvert(lib, kv=None, bt=None, sl=None, st=None, ws=None, L=0, name=name) == 0
