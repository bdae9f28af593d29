"""GPU parity of the separate-prefill mode of an fp8_ds_mla cache (the
flashmla_sparse.py page as changed for this mode): index conversion to
workspace rows (bit-exact), the gather-and-upconvert of prefill context rows
into a bf16 workspace (bit-exact, ties included), attention over cache slots
given directly (bit-identical to the logical path), and the mode end to end
against the oracle. The same mode over an nvfp4_ds_mla cache (the staged
prefill of the native-decode pull-request page): the exact upconvert bit for
bit, and the mode end to end."""

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_attention_indices_amd import smla, workloads as W
from tests.gpu_util import TOL, DeviceWorkload, bf16_tensor, errors, log

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ---------------------------------------------------------------- conversion

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_workspace_conversion_bit_exact(seed):
    rng = np.random.default_rng(seed)
    R, MB, T, K, NB = 6, 7, 40, 200, 30
    bt = rng.integers(-2, NB + 3, (R, MB)).astype(np.int32)
    req = rng.integers(-1, R + 1, T).astype(np.int32)
    idx = rng.integers(-70, MB * 64 + 70, (T, K)).astype(np.int32)
    pid = rng.integers(-1, 5, T).astype(np.int32)              # 4 prefill requests; id 4 is out of range
    starts = np.array([0, 300, 10, 777], dtype=np.int32)
    log(f"[case] workspace conversion seed={seed}")
    want = oracle.convert_indices_workspace(req, bt, idx, NB, pid, starts)
    got = smla.smla_convert_indices_workspace(_dev(req), _dev(bt), _dev(idx), _dev(pid), _dev(starts), NB)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), want)
    # no prefill requests at all: the plain conversion
    got0 = smla.smla_convert_indices_workspace(_dev(req), _dev(bt), _dev(idx), _dev(np.full(T, -1, np.int32)),
                                               None, NB)
    torch.cuda.synchronize()
    assert np.array_equal(got0.cpu().numpy(), oracle.convert_indices(req, bt, idx, NB))


# ----------------------------------------------------------------- upconvert

def _tie_rows(n_rows):
    """Rows whose float32 products land exactly halfway between two bf16 values
    while the exact products do not: group g holds one e4m3 value x and a scale s
    = float32(T / x) for a bf16 midpoint T, so x * s = T + (a residual of either sign)."""
    codes = [0x39, 0x3A, 0x3B, 0x3D, 0x3E, 0x3F, 0x41, 0x43]   # 1.125 .. 2.875, not powers of two
    rows = np.zeros((n_rows, 656), dtype=np.uint8)
    rng = np.random.default_rng(77)
    for r in range(n_rows):
        for g in range(4):
            c = codes[(r * 4 + g) % len(codes)]
            x = oracle.e4m3fn(c)
            tie = (1.0 + (2 * int(rng.integers(0, 64)) + 1) * 2.0 ** -8) * 2.0 ** int(rng.integers(-3, 4))
            rows[r, 128 * g:128 * (g + 1)] = c
            rows[r, 512 + 4 * g:516 + 4 * g] = np.array([tie / x], dtype="<f4").view(np.uint8)
        rows[r, 528:] = rng.integers(0, 256, 128).astype(np.uint8)
    return rows


@pytest.mark.parametrize("kind", ["random", "ties"])
def test_upconvert_bit_exact(kind):
    if kind == "random":
        cache = W.random_fp8_cache(5, 98, 12)
    else:
        cache = _tie_rows(12 * 64).reshape(12, 64, 656)
        fp32 = cache.reshape(-1, 656)[:, 512:528].copy().view("<f4")
        codes = cache.reshape(-1, 656)[:, 0:512:128]
        prods = np.float32(np.vectorize(oracle.e4m3fn)(codes)) * fp32
        assert ((prods.view(np.uint32) & 0xFFFF) == 0x8000).sum() >= 200     # many float32 ties
    NB = cache.shape[0]
    lens = np.array([150, 1, 64, 200], dtype=np.int32)
    bt = np.array([[3, 7, 1, 0], [5, 0, 0, 0], [11, 0, 0, 0], [2, 4, 6, NB + 5]], dtype=np.int32)  # last: bad
    starts = np.array([10, 0, 170, 300], dtype=np.int32)
    rows = 480                                                   # request 3 runs past the workspace end
    init = np.full((rows, 576), 0x7E57, dtype=np.uint16)
    want = oracle.gather_upconvert(cache, bt, lens, starts, rows, workspace=init.copy())
    ws = bf16_tensor(init)
    log(f"[case] upconvert {kind}")
    smla.smla_gather_upconvert_fp8(_dev(cache), _dev(bt), _dev(lens), _dev(starts), int(lens.max()), ws)
    torch.cuda.synchronize()
    got = ws.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, f"rows differ: {bad[:10]}"


def test_upconvert_negative_start_and_positions_past_the_table():
    """A request whose workspace start is negative (its first rows are not
    written) and whose length runs past its block-table row (those positions
    write zeros), next to one whose length ends inside a 16-row group."""
    cache = W.random_fp8_cache(5, 99, 9)
    lens = np.array([300, 37], dtype=np.int32)
    bt = np.array([[4, 8, 2, 6], [1, 0, 0, 0]], dtype=np.int32)
    starts = np.array([-21, 290], dtype=np.int32)
    rows = 330
    init = np.full((rows, 576), 0x7E57, dtype=np.uint16)
    want = oracle.gather_upconvert(cache, bt, lens, starts, rows, workspace=init.copy())
    assert (want[236:279] == 0).all() and (want[279:290] == 0x7E57).all()
    ws = bf16_tensor(init)
    log("[case] upconvert negative start, positions past the table")
    smla.smla_gather_upconvert_fp8(_dev(cache), _dev(bt), _dev(lens), _dev(starts), int(lens.max()), ws)
    torch.cuda.synchronize()
    got = ws.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, f"rows differ: {bad[:10]}"


def test_upconvert_full_size_prefill_part_sampled():
    """Config 5's prefill contexts (131072 and 65536 positions, 196608 rows) in one
    launch; sampled rows against the oracle, bit-exact."""
    lens = np.array([131072, 65536], dtype=np.int32)
    bt, nb = W.allocate_block_table(np.random.default_rng(70), lens)
    cache = W.random_fp8_cache(0, 70, nb)
    starts = np.array([0, lens[0]], dtype=np.int32)
    rows = int(lens.sum())
    ws = torch.empty((rows, 576), dtype=torch.bfloat16, device="cuda")
    log(f"[case] upconvert config 5 prefill part, {rows} rows")
    smla.smla_gather_upconvert_fp8(_dev(cache), _dev(bt), _dev(lens), _dev(starts), int(lens.max()), ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    for r in range(2):
        pos = np.concatenate([[0, 63, 64, lens[r] - 1], rng.integers(0, lens[r], 60)])
        for p in pos:
            # the oracle on a one-block cache holding the row of position p of request r
            blk = bt[r, p // 64]
            one_block = np.repeat(cache[blk, p % 64].reshape(1, 1, 656), 64, axis=1)
            one = oracle.gather_upconvert(one_block, np.zeros((1, 1), np.int32), [1], [0], 1)
            got = ws[starts[r] + p].view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(got, one[0]), (r, p)


def test_upconvert_nvfp4_bit_exact():
    """The nvfp4 gather: every staged value is exact, so the bf16 rows equal the
    oracle's bit for bit; a bad block writes zeros, rows past the workspace and
    rows no request covers are left alone."""
    cache = W.random_nvfp4_cache(5, 97, 12)
    NB = cache.shape[0]
    lens = np.array([150, 1, 64, 200], dtype=np.int32)
    bt = np.array([[3, 7, 1, 0], [5, 0, 0, 0], [11, 0, 0, 0], [2, 4, 6, NB + 5]], dtype=np.int32)  # last: bad
    starts = np.array([10, 0, 170, 300], dtype=np.int32)
    rows = 480
    init = np.full((rows, 576), 0x7E57, dtype=np.uint16)
    want = oracle.gather_upconvert(cache, bt, lens, starts, rows, workspace=init.copy(),
                                   cache_format=oracle.NVFP4_CACHE)
    ws = bf16_tensor(init)
    log("[case] upconvert nvfp4")
    smla.smla_gather_upconvert_nvfp4(_dev(cache), _dev(bt), _dev(lens), _dev(starts), int(lens.max()), ws)
    torch.cuda.synchronize()
    got = ws.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, f"rows differ: {bad[:10]}"


# ------------------------------------------------------------- slot indices

@pytest.mark.parametrize("fmt", ["bf16", "fp8", "nvfp4"])
def test_slot_indices_match_the_logical_path(fmt):
    w = W.build(f"slots_{fmt}", 1201, 3, [300, 700, 90], np.repeat([0, 1, 2], 4), np.repeat([300, 700, 90], 4),
                64, 160, fmt, p_invalid=0.2, max_blocks_per_req=13)
    dw = DeviceWorkload(w)
    fn = {"bf16": smla.smla_prefill_bf16, "fp8": smla.smla_decode_fp8, "nvfp4": smla.smla_decode_nvfp4}[fmt]
    for splits in (1, 3):
        log(f"[case] slot indices {fmt} splits={splits}")
        slots = smla.smla_convert_indices(dw.req, dw.bt, dw.idx, w.num_blocks)
        # out-of-cache slots count as invalid
        slots[0, :5] = w.num_blocks * 64
        slots[1, :5] = -3
        ref2 = dw.idx.clone()
        ref2[0, :5] = -1
        ref2[1, :5] = -1
        ref_o, ref_l = fn(dw.q, dw.cache, dw.bt, dw.req, ref2, w.sm_scale, num_splits=splits)
        o, l = fn(dw.q, dw.cache, None, None, slots, w.sm_scale, num_splits=splits, slot_indices=True)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


# ---------------------------------------------------------------- end to end

@pytest.mark.parametrize("h_q,topk,max_rows,fmt", [(16, 96, 300, "fp8"), (64, 128, 520, "fp8"),
                                                   (128, 64, 1000, "fp8"), (16, 96, 300, "nvfp4"),
                                                   (128, 64, 1000, "nvfp4")])
def test_separate_prefill_mode_end_to_end(h_q, topk, max_rows, fmt):
    w = W.mixed_batch(7 + h_q, h_q, topk, decode_ctx=[150, 300, 77], prefill_ctx=[200, 90, 260, 140],
                      prefill_queries=[5, 3, 4, 6], p_invalid=0.1, cache_format=fmt)
    nd = 3
    log(f"[case] separate prefill {fmt} h_q={h_q} topk={topk} max_rows={max_rows}")
    ofmt = oracle.FP8_CACHE if fmt == "fp8" else oracle.NVFP4_CACHE
    o_ref, l_ref = oracle.separate_prefill_attention(w.q, w.cache, w.block_table, w.req_id_per_token,
                                                     w.topk_indices, w.sm_scale, nd, w.ctx_lens, max_rows,
                                                     cache_format=ofmt)
    ends, _ = oracle.plan_prefill_chunks(w.ctx_lens[nd:], max_rows)
    log(f"  chunks {ends}")
    q = bf16_tensor(w.q)
    # the batch's host metadata, built once (tokens are grouped by request, decode first)
    counts = np.bincount(w.req_id_per_token, minlength=w.num_reqs)
    qsl = np.concatenate([[0], np.cumsum(counts)])
    plan = smla.smla_build_separate_prefill_plan(qsl, w.ctx_lens, nd, max_rows, "cuda")
    assert [c[1] for c in plan.chunks] == list(ends)
    forward = smla.smla_forward_fp8_separate_prefill if fmt == "fp8" else smla.smla_forward_nvfp4_separate_prefill
    o, l = forward(q, _dev(w.cache), _dev(w.block_table), _dev(w.req_id_per_token), _dev(w.topk_indices),
                   w.sm_scale, plan)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    l = l.cpu().numpy().astype(np.float64)
    dec = w.req_id_per_token < nd
    for sel, tfmt in ((dec, fmt), (~dec, "bf16")):
        om, orl = errors(o[sel], o_ref[sel])
        fin = np.isfinite(l_ref[sel])
        assert np.array_equal(fin, np.isfinite(l[sel]))
        lm, lrl = errors(l[sel][fin], l_ref[sel][fin])
        log(f"[parity] separate prefill {tfmt} tokens: o max_abs={om:.3e} rel_l2={orl:.3e} lse max_abs={lm:.3e}")
        assert om <= TOL[tfmt]["max_abs"] and orl <= TOL[tfmt]["rel_l2"]
        assert lm <= TOL[tfmt]["max_abs"] and lrl <= TOL[tfmt]["rel_l2"]


def test_config5_prefill_part_over_nvfp4_both_paths_sampled():
    """Config 5's prefill part (2 x 2048 query tokens, h_q 128, top-k 2048,
    contexts 131072 and 65536) over an nvfp4 cache, as the benchmark runs it:
    native decode and the staged mode, sampled tokens against the oracle."""
    w = W.config5_prefill(0, "nvfp4")
    dw = DeviceWorkload(w)
    counts = np.bincount(w.req_id_per_token, minlength=w.num_reqs)
    qsl = np.concatenate([[0], np.cumsum(counts)])
    plan = smla.smla_build_separate_prefill_plan(qsl, w.ctx_lens, 0, int(w.ctx_lens.sum()), "cuda")
    rng = np.random.default_rng(55)
    tokens = np.unique(np.concatenate([[0, 1, 2047, 2048, 4095], rng.choice(w.num_tokens, 19, replace=False)]))
    o_ref, l_ref = oracle.attention(oracle.NVFP4_CACHE, w.q, w.cache, w.block_table, w.req_id_per_token,
                                    w.topk_indices, w.sm_scale, tokens=tokens)
    for name in ("native", "staged"):
        log(f"[case] config 5 prefill part nvfp4 {name}")
        if name == "native":
            o, l = smla.smla_decode_nvfp4(dw.q, dw.cache, dw.bt, dw.req, dw.idx, w.sm_scale)
        else:
            o, l = smla.smla_forward_nvfp4_separate_prefill(dw.q, dw.cache, dw.bt, dw.req, dw.idx, w.sm_scale,
                                                            plan)
        torch.cuda.synchronize()
        sel = torch.from_numpy(tokens).cuda()
        og = o[sel].float().cpu().numpy().astype(np.float64)
        lg = l[sel].cpu().numpy().astype(np.float64)
        om, orl = errors(og, o_ref)
        lm, lrl = errors(lg, l_ref)
        log(f"[parity] config 5 prefill nvfp4 {name}: o max_abs={om:.3e} rel_l2={orl:.3e} lse max_abs={lm:.3e}")
        assert om <= TOL["nvfp4"]["max_abs"] and orl <= TOL["nvfp4"]["rel_l2"]
        assert lm <= TOL["nvfp4"]["max_abs"] and lrl <= TOL["nvfp4"]["rel_l2"]
