"""GPU parity: libsmla.so (through its C ABI) against the CPU oracle.

Index conversion is compared bit for bit. Attention outputs are compared element
by element with the stated tolerances: bf16 cache max-abs <= 1e-2 and rel-L2 <=
5e-3, fp8_ds_mla and nvfp4_ds_mla caches max-abs <= 2e-2 and rel-L2 <= 1e-2, for
o and for lse.
Small cases are checked in full; the full-size configurations run exactly as the
benchmark launches them and are checked on sampled tokens the oracle computes one
by one.
"""

import dataclasses
import json
import os

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_attention_indices_amd import smla
from sparse_mla_attention_indices_amd import workloads as W
from tests.gpu_util import (DeviceWorkload, assert_parity, assert_parity_up_to_output_rounding, entry_point, log,
                            oracle_run)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="session", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    smla.library()          # fail loudly if the HIP library is missing
    return torch.device("cuda")


def small(seed, fmt, h_q, topk, n_req=3, tok_per_req=3, ctx=(60, 700), p_invalid=0.2, mb_extra=2):
    rng = np.random.default_rng(seed)
    ctx_lens = rng.integers(ctx[0], ctx[1], size=n_req)
    req = np.repeat(np.arange(n_req), tok_per_req)
    vis = ctx_lens[req]
    mb = int(max(-(-ctx_lens // 64))) + mb_extra
    return W.build(f"small_{fmt}_h{h_q}_k{topk}_s{seed}", 1000 + seed, seed, ctx_lens, req, vis,
                   h_q, topk, fmt, p_invalid=p_invalid, max_blocks_per_req=mb)


# ------------------------------------------------------------- index convert

def test_convert_golden_bit_exact():
    g = json.load(open(os.path.join(GOLDEN, "index_convert_cases.json")))
    req = torch.tensor(g["req_id_per_token"], dtype=torch.int32, device="cuda")
    bt = torch.tensor(g["block_table"], dtype=torch.int32, device="cuda")
    idx = torch.tensor(g["topk_indices"], dtype=torch.int32, device="cuda")
    out = smla.smla_convert_indices(req, bt, idx, g["num_blocks"])
    torch.cuda.synchronize()
    assert out.cpu().tolist() == g["expected"]


@pytest.mark.parametrize("T,K", [(1, 1), (37, 129), (300, 777)])
def test_convert_random_bit_exact(T, K):
    rng = np.random.default_rng(T * 1000 + K)
    R, MB, NB = 9, 13, 50
    bt = rng.integers(-3, NB + 3, size=(R, MB)).astype(np.int32)     # includes bad entries
    req = rng.integers(-1, R + 1, size=T).astype(np.int32)           # includes bad request ids
    idx = rng.integers(-70, MB * 64 + 70, size=(T, K)).astype(np.int32)
    want = oracle.convert_indices(req, bt, idx, NB)
    got = smla.smla_convert_indices(torch.from_numpy(req).cuda(), torch.from_numpy(bt).cuda(),
                                    torch.from_numpy(idx).cuda(), NB)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), want)


# ------------------------------------------------------------ small matrix

@pytest.mark.parametrize("fmt", ["bf16", "fp8", "nvfp4"])
@pytest.mark.parametrize("h_q", [16, 32, 64, 128])
@pytest.mark.parametrize("topk", [1, 37, 64, 100, 200])
def test_small_parity(fmt, h_q, topk):
    w = small(h_q + topk, fmt, h_q, topk)
    dw = DeviceWorkload(w)
    want_phys = oracle.convert_indices(w.req_id_per_token, w.block_table, w.topk_indices, w.num_blocks)
    for splits in (0, 1, 3):
        log(f"[case] small {fmt} h_q={h_q} topk={topk} splits={splits}")
        out, lse, phys = dw.run(num_splits=splits, with_phys=True)
        assert np.array_equal(phys.cpu().numpy(), want_phys)
        assert_parity(w, out, lse, label=f"small {fmt} h{h_q} k{topk} s{splits}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "nvfp4"])
@pytest.mark.parametrize("h_q", [64, 128])
def test_long_list_crosses_the_lds_chunk(fmt, h_q):
    """topk 5000: several rounds of LDS compaction per list, a ragged tail, one
    split and several."""
    w = small(7, fmt, h_q, 5000, n_req=2, tok_per_req=2, ctx=(6000, 9000), p_invalid=0.1)
    dw = DeviceWorkload(w)
    for splits in (1, 2, 0):
        log(f"[case] long list {fmt} h_q={h_q} splits={splits}")
        out, lse, _ = dw.run(num_splits=splits)
        assert_parity(w, out, lse, label=f"long {fmt} h{h_q} s{splits}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "nvfp4"])
def test_logits_rising_past_the_first_tile_reference(fmt):
    """128-head workgroups (bf16 cache) weight every row against a reference per
    head taken from the max of the first tile (32 valid rows); when a later tile's
    max rises more than 64 log2 units above it, the workgroup redoes its list
    (exact maxima, then the full pass). The fp8 cache's 64-head workgroups rescale
    online instead and are held to the same bound on the same kind of input. Here the first 32 valid rows of every token are zero rows
    (logit 0) and q is scaled by 12 or 24 per head, so the later rows' maxima rise
    past that headroom for some heads of every token, which is checked on the
    oracle first: the lse of the whole list minus ln(rows) exceeds the lse of its
    first 32 valid rows by more than 64 ln 2. Such logits put nearly all weight on
    a few rows, so o is held to the bound for that case: exact up to the output's
    own rounding and the one bf16 rounding of each weight, unsplit and split."""
    w = small(81, fmt, 128, 1024, n_req=2, tok_per_req=2, ctx=(1100, 1500), p_invalid=0.05)
    rng = np.random.default_rng(81)
    gain = np.where(rng.random(128) < 0.5, 12.0, 24.0).astype(np.float32)
    w.q = W.to_bf16_bits(W.bf16_bits_to_f32(w.q) * gain[None, :, None])
    phys = oracle.convert_indices(w.req_id_per_token, w.block_table, w.topk_indices, w.num_blocks)
    first = np.full_like(w.topk_indices, -1)
    for t in range(w.num_tokens):
        valid = np.flatnonzero(phys[t] >= 0)[:32]
        first[t, valid] = w.topk_indices[t, valid]
        for slot in phys[t, valid]:
            w.cache[slot // 64, slot % 64, :] = 0        # zero latent, RoPE (and fp8 scales)
    _, lse_full = oracle_run(w)
    _, lse_first = oracle_run(dataclasses.replace(w, topk_indices=first))
    n_valid = (phys >= 0).sum(1)
    rise = lse_full - np.log(n_valid)[:, None] - lse_first
    log(f"[case] restart: heads past the headroom per token {(rise > 64 * np.log(2)).sum(1).tolist()}")
    assert (rise > 64 * np.log(2)).any(axis=1).all()
    dw = DeviceWorkload(w)
    for splits in (1, 0, 3):
        log(f"[case] rising logits {fmt} splits={splits}")
        out, lse, _ = dw.run(num_splits=splits)
        assert_parity_up_to_output_rounding(w, out, lse, label=f"rising logits {fmt} s{splits}",
                                            weights_rounded=True)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "nvfp4"])
@pytest.mark.parametrize("h_q", [32, 128])
def test_degenerate_rows(fmt, h_q):
    """Whole tokens without a valid slot, bad request ids, bad table entries, duplicates."""
    w = small(11, fmt, h_q, 96, n_req=3, tok_per_req=4, ctx=(100, 300), p_invalid=0.3)
    w.topk_indices[0, :] = -1                              # nothing valid
    w.topk_indices[1, :] = w.max_blocks_per_req * 64 + 5   # past the table: nothing valid
    w.req_id_per_token[2] = w.num_reqs + 4                 # request id outside the table
    w.block_table[1, 0] = -1                               # bad entries in request 1's table
    w.block_table[1, 1] = w.num_blocks + 10
    w.topk_indices[5, :10] = w.topk_indices[5, 10]         # duplicates count per occurrence
    w.topk_indices[6, :] = -1
    w.topk_indices[6, 50] = 3                              # exactly one valid slot
    dw = DeviceWorkload(w)
    for splits in (0, 2):
        log(f"[case] degenerate {fmt} h_q={h_q} splits={splits}")
        out, lse, phys = dw.run(num_splits=splits, with_phys=True)
        want = oracle.convert_indices(w.req_id_per_token, w.block_table, w.topk_indices, w.num_blocks)
        assert np.array_equal(phys.cpu().numpy(), want)
        assert_parity(w, out, lse, label=f"degenerate {fmt} h{h_q} s{splits}")


@pytest.mark.parametrize("h_q", [64, 128])
def test_valid_counts_across_tile_ring_and_short_list_bounds(h_q):
    """64-head fp8 workgroups (QK^T and PV waves, a ring of five 32-row tiles, or
    three for lists of at most 128 valid rows): per-token valid counts of 0, 1,
    around one tile, around the 128-row short-list bound, and past the ring's
    wrap; a token with a request id outside the table; unsplit, planned and
    3-way split calls."""
    counts = [0, 1, 31, 32, 33, 64, 96, 127, 128, 129, 160, 161, 224, 300, 500, 600]
    w = small(71 + h_q, "fp8", h_q, 600, n_req=4, tok_per_req=4, ctx=(700, 900), p_invalid=0.0)
    rng = np.random.default_rng(71 + h_q)
    for t, n in enumerate(counts):
        keep = rng.permutation(600)[:n]
        row = np.full(600, -1, dtype=np.int32)
        row[keep] = w.topk_indices[t, keep]
        w.topk_indices[t] = row
    w.req_id_per_token[3] = w.num_reqs + 2      # request id outside the table: nothing valid
    dw = DeviceWorkload(w)
    want = oracle.convert_indices(w.req_id_per_token, w.block_table, w.topk_indices, w.num_blocks)
    for splits in (1, 0, 3):
        log(f"[case] ring bounds fp8 h_q={h_q} splits={splits}")
        out, lse, phys = dw.run(num_splits=splits, with_phys=True)
        assert np.array_equal(phys.cpu().numpy(), want)
        assert_parity(w, out, lse, label=f"ring bounds h{h_q} s{splits}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "nvfp4"])
def test_short_lists_are_exact_up_to_output_rounding(fmt):
    """Tokens with 1..8 valid rows put large weights on few rows, so |o| can reach the
    bf16 range where half an ulp (0.0156 above 4) exceeds the stated max-abs bound by
    itself. There the kernel must be exact up to the output's own rounding: error <=
    half a bf16 ulp of the true value + 2e-3 (fp8: one more half ulp, for the one
    bf16 rounding of the dequantised rows), and the stated rel-L2 bound."""
    w = small(21, fmt, 128, 64, n_req=4, tok_per_req=8, ctx=(200, 400), p_invalid=0.0)
    rng = np.random.default_rng(21)
    for t in range(w.num_tokens):
        keep = 1 + t % 8
        w.topk_indices[t, keep:] = -1
        w.topk_indices[t] = rng.permutation(w.topk_indices[t])
    dw = DeviceWorkload(w)
    for splits in (0, 3):
        log(f"[case] short lists {fmt} splits={splits}")
        out, lse, _ = dw.run(num_splits=splits)
        assert_parity_up_to_output_rounding(w, out, lse, label=f"short lists {fmt} s{splits}")


@pytest.mark.parametrize("h_q", [16, 64, 128])
def test_wide_range_q_within_a_scale_group(h_q):
    """q whose magnitudes span 2^-20 .. 2^2 inside every 128-column group. The fp8
    QK^T writes q as hi + lo e4m3 terms under one power-of-two scale per head and
    group: elements within 2^13 of the group's largest are exact, smaller ones
    keep an absolute error below about 2^-21 of it. Results must still meet the
    fp8 bounds, unsplit and split."""
    w = small(61 + h_q, "fp8", h_q, 256, n_req=3, tok_per_req=3, ctx=(300, 900), p_invalid=0.1)
    rng = np.random.default_rng(61 + h_q)
    mag = np.exp2(rng.uniform(-20.0, 2.0, size=w.q.shape))
    sign = np.where(rng.random(w.q.shape) < 0.5, -1.0, 1.0)
    w.q = W.to_bf16_bits((sign * mag).astype(np.float32))
    dw = DeviceWorkload(w)
    for splits in (1, 0, 3):
        log(f"[case] wide-range q h_q={h_q} splits={splits}")
        out, lse, _ = dw.run(num_splits=splits)
        assert_parity(w, out, lse, label=f"wide-range q h{h_q} s{splits}")


# ------------------------------------------------------------ split merge

@pytest.mark.parametrize("fmt", ["bf16", "fp8", "nvfp4"])
@pytest.mark.parametrize("h_q", [16, 64, 128])
def test_split_merge_with_converted_indices(fmt, h_q):
    """Top-k splits merged by the second kernel, with invalid positions spread over
    the parts (some parts of a short list hold none): results match the oracle and
    the converted indices are written once, in full."""
    w = small(31 + h_q, fmt, h_q, 300, n_req=3, tok_per_req=3, ctx=(400, 900), p_invalid=0.15)
    dw = DeviceWorkload(w)
    want_phys = oracle.convert_indices(w.req_id_per_token, w.block_table, w.topk_indices, w.num_blocks)
    for splits in (2, 5):
        log(f"[case] split merge {fmt} h_q={h_q} splits={splits}")
        out, lse, phys = dw.run(num_splits=splits, with_phys=True)
        assert np.array_equal(phys.cpu().numpy(), want_phys)
        assert_parity(w, out, lse, label=f"split merge {fmt} h{h_q} s{splits}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "nvfp4"])
def test_workspace_reused_across_batch_sizes(fmt):
    """One workspace, filled with garbage once, then calls of changing token counts
    that share it: every call writes what it reads, so results depend neither on
    the initial contents nor on the calls before."""
    w = small(41, fmt, 16, 48, n_req=41, tok_per_req=100, ctx=(60, 300), p_invalid=0.2)
    dw = DeviceWorkload(w)
    need = max(smla.smla_workspace_size(T, 16, 48, num_splits=3) for T in (9, 4100))
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    for T in (9, 3, 4100, 9, 200, 4100, 5):
        log(f"[case] reused workspace {fmt} T={T}")
        out, lse, _ = dw.run(num_splits=3, num_tokens=T, workspace=ws)
        assert_parity(w, out, lse, tokens=np.arange(T), label=f"reused ws {fmt} T{T}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "nvfp4"])
def test_uninitialised_workspace(fmt):
    """A workspace full of 0xFF bytes (NaN patterns) gives the same results."""
    w = small(43, fmt, 64, 200, n_req=2, tok_per_req=4)
    dw = DeviceWorkload(w)
    ws = torch.full((smla.smla_workspace_size(w.num_tokens, 64, 200, num_splits=4),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    for _ in range(2):
        log(f"[case] garbage workspace {fmt}")
        out, lse, _ = dw.run(num_splits=4, workspace=ws)
        assert_parity(w, out, lse, label=f"garbage ws {fmt}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "nvfp4"])
def test_partials_only_then_merge_equals_the_call(fmt):
    """A call with partials_only followed by smla_merge_partials runs the same
    kernels as one ordinary call. The lse is bit-identical. So is the output for
    the bf16 and nvfp4 caches and for an unsplit list (one part). A split fp8 call of
    64-head workgroups keeps each part's O / l as bf16 rows (plus residual rows
    for a part of at most 128 valid rows), so there the output may differ from
    the fp32 parts' merge by one bf16 rounding of the largest part value plus
    one output ulp, and the call itself meets the oracle bounds."""
    w = small(51, fmt, 64, 300, n_req=3, tok_per_req=5, ctx=(200, 900), p_invalid=0.1)
    dw = DeviceWorkload(w)
    fn = entry_point(fmt)
    T, H, K = w.num_tokens, 64, 300
    for splits in (1, 3, 0):
        log(f"[case] partials then merge {fmt} splits={splits}")
        ref_out, ref_lse, _ = dw.run(num_splits=splits)
        S, need = smla.smla_plan(T, H, K, torch.cuda.get_device_properties(0).multi_processor_count,
                                 num_splits=splits, partials_only=True)
        ws = torch.full((need,), 0xEE, dtype=torch.uint8, device="cuda")
        assert fn(dw.q, dw.cache, dw.bt, dw.req, dw.idx, w.sm_scale, workspace=ws, num_splits=splits,
                  partials_only=True) == (None, None)
        out, lse = smla.smla_merge_partials(ws, T, H, S)
        torch.cuda.synchronize()
        assert torch.equal(lse, ref_lse)
        if fmt != "fp8" or S == 1:
            assert torch.equal(out, ref_out)
        else:
            o_off, _ = smla.partials_layout(T, H, S)
            parts = ws[o_off:o_off + T * S * H * 512 * 4].view(torch.float32).view(T, S, H, 512)
            bound = parts.abs().amax(1) * 2.0 ** -8 + ref_out.float().abs() * 2.0 ** -7
            diff = (out.float() - ref_out.float()).abs()
            assert bool((diff <= bound).all()), f"max excess {float((diff - bound).max()):.3e}"
            assert_parity(w, ref_out, ref_lse, label=f"split call {fmt} splits={splits}")


@pytest.mark.parametrize("fmt,h_q", [("fp8", 64), ("fp8", 16), ("bf16", 64), ("nvfp4", 16), ("nvfp4", 64)])
def test_deferred_merge_then_merge_only_equals_the_call(fmt, h_q):
    """The attention stage of a call (merge deferred) and then its merge stage,
    with the same arguments and workspace, write what one ordinary call writes,
    bit for bit: split, unsplit and planner-chosen."""
    w = small(52, fmt, h_q, 300, n_req=3, tok_per_req=5, ctx=(200, 900), p_invalid=0.1)
    dw = DeviceWorkload(w)
    fn = entry_point(fmt)
    T, H, K = w.num_tokens, h_q, 300
    for splits in (1, 3, 0):
        log(f"[case] deferred merge {fmt} h{h_q} splits={splits}")
        ref_out, ref_lse, _ = dw.run(num_splits=splits)
        ws = torch.full((max(smla.smla_workspace_size(T, H, K, splits), 256),), 0xEE, dtype=torch.uint8,
                        device="cuda")
        out = torch.full((T, H, 512), 7.0, dtype=torch.bfloat16, device="cuda")
        lse = torch.full((T, H), 7.0, dtype=torch.float32, device="cuda")
        for stage in ("attention", "merge"):
            fn(dw.q, dw.cache, dw.bt, dw.req, dw.idx, w.sm_scale, out=out, lse=lse, workspace=ws,
               num_splits=splits, stage=stage)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "nvfp4"])
def test_parts_of_a_list_merged_like_context_parallel(fmt):
    """Each token's top-k list cut in two halves, each half computed by its own
    call (as two devices would), the two parts stacked into one partials buffer
    and merged: the result is the attention over the whole list."""
    w = small(53, fmt, 32, 400, n_req=4, tok_per_req=4, ctx=(300, 1500), p_invalid=0.1)
    dw = DeviceWorkload(w)
    fn = entry_point(fmt)
    T, H, K = w.num_tokens, 32, 400
    halves = ((0, 160), (160, K))          # uneven cut
    o_off, total = smla.partials_layout(T, H, len(halves))
    merged = torch.empty(total, dtype=torch.uint8, device="cuda")
    lse_all = merged[:T * len(halves) * H * 4].view(torch.float32).view(T, len(halves), H)
    o_all = merged[o_off:].view(torch.float32).view(T, len(halves), H, 512)
    for f, (a, b) in enumerate(halves):
        idx = dw.idx[:, a:b].contiguous()
        s1, need = smla.smla_plan(T, H, b - a, 256, num_splits=1, partials_only=True)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        fn(dw.q, dw.cache, dw.bt, dw.req, idx, w.sm_scale, workspace=ws, num_splits=1, partials_only=True)
        po, _ = smla.partials_layout(T, H, 1)
        lse_all[:, f] = ws[:T * H * 4].view(torch.float32).view(T, H)
        o_all[:, f] = ws[po:po + T * H * 512 * 4].view(torch.float32).view(T, H, 512)
    out, lse = smla.smla_merge_partials(merged, T, H, len(halves))
    torch.cuda.synchronize()
    log(f"[case] two-part merge {fmt}")
    assert_parity(w, out, lse, label=f"two-part merge {fmt}")


def test_zero_tokens_writes_nothing():
    w = small(3, "fp8", 16, 64)
    dw = DeviceWorkload(w)
    out = torch.full((0, 16, 512), 1.0, dtype=torch.bfloat16, device="cuda")
    o, l = smla.smla_decode_fp8(dw.q[:0], dw.cache, dw.bt, dw.req[:0], dw.idx[:0], w.sm_scale, out=out)
    torch.cuda.synchronize()
    assert o.numel() == 0


def test_repeat_calls_are_bit_identical():
    w = W.config1_fp8()
    dw = DeviceWorkload(w)
    a, la, _ = dw.run(num_splits=2)
    b, lb, _ = dw.run(num_splits=2)
    assert torch.equal(a, b) and torch.equal(la, lb)


# ------------------------------------------------------------ named configs

@pytest.mark.parametrize("maker", [W.config1, W.config1_fp8, W.config1_nvfp4])
def test_config1(maker):
    w = maker()
    dw = DeviceWorkload(w)
    want_phys = oracle.convert_indices(w.req_id_per_token, w.block_table, w.topk_indices, w.num_blocks)
    for splits in (0, 2, 3):
        log(f"[case] {w.name} splits={splits}")
        out, lse, phys = dw.run(num_splits=splits, with_phys=True)
        assert np.array_equal(phys.cpu().numpy(), want_phys)
        assert_parity(w, out, lse, label=f"{w.name} s{splits}")


@pytest.fixture(scope="module")
def c2():
    return W.config2()


def test_config2_fp8_decode_full(c2):
    """The headline decode batch in the benchmark's launch configuration, every token checked."""
    dw = DeviceWorkload(c2)
    log("[case] config2 full")
    out, lse, phys = dw.run(with_phys=True)
    want = oracle.convert_indices(c2.req_id_per_token, c2.block_table, c2.topk_indices, c2.num_blocks)
    assert np.array_equal(phys.cpu().numpy(), want)
    assert_parity(c2, out, lse, label="config2 (64 tok, h64, k2048, fp8)")


def _sample_tokens(T, rng, extra=()):
    pick = set(int(x) for x in extra if 0 <= x < T)
    pick.update(int(x) for x in rng.choice(T, size=min(T, 24), replace=False))
    return np.array(sorted(pick), dtype=np.int64)


def test_config3_bf16_prefill_sampled():
    w = W.config3()
    dw = DeviceWorkload(w)
    log("[case] config3 full size")
    out, lse, _ = dw.run()
    # both ends of the causal ramp, the -1 / full boundary, and the last positions
    edges = [0, 1, 2, 63, 64, 2046, 2047, 2048, 4095, 4096, 4097, 6143, 16383]
    tokens = _sample_tokens(w.num_tokens, np.random.default_rng(3), edges)
    assert_parity(w, out, lse, tokens=tokens, label="config3 (16384 tok, h128, k2048, bf16) sampled")


@pytest.mark.parametrize("topk", [512, 1024, 2048])
def test_config4_spec_decode(topk):
    w = W.config4(topk=topk)
    dw = DeviceWorkload(w)
    log(f"[case] config4 topk={topk}")
    out, lse, _ = dw.run()
    tokens = None if topk == 512 else _sample_tokens(w.num_tokens, np.random.default_rng(topk), [0, 1, 255])
    assert_parity(w, out, lse, tokens=tokens, label=f"config4 (256 tok, h16, k{topk}, fp8)")


@pytest.mark.parametrize("topk", [512, 1024, 2048])
def test_config4_nvfp4_native_decode(topk):
    """Config 4's batch over an nvfp4_ds_mla cache: 16 heads and top-k 512, 1024
    or 2048, the shape the pull-request page runs native NVFP4 decode at, in the
    benchmark's launch configuration."""
    w = W.config4_nvfp4(topk=topk)
    dw = DeviceWorkload(w)
    log(f"[case] config4 nvfp4 topk={topk}")
    out, lse, phys = dw.run(with_phys=True)
    want = oracle.convert_indices(w.req_id_per_token, w.block_table, w.topk_indices, w.num_blocks)
    assert np.array_equal(phys.cpu().numpy(), want)
    tokens = None if topk == 512 else _sample_tokens(w.num_tokens, np.random.default_rng(topk), [0, 1, 255])
    assert_parity(w, out, lse, tokens=tokens, label=f"config4 nvfp4 (256 tok, h16, k{topk})")


def test_config5_long_mixed_sampled():
    w = W.config5()
    dw = DeviceWorkload(w)
    log("[case] config5 full size")
    out, lse, _ = dw.run()
    edges = list(range(32)) + [32, 33, 2079, 2080, 2081, 4127]
    tokens = _sample_tokens(w.num_tokens, np.random.default_rng(5), edges)
    assert_parity(w, out, lse, tokens=tokens, label="config5 (4128 tok, h128, k2048, fp8) sampled")
