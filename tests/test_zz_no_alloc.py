"""The allocation-free entry point (smla_decode_fp8_noalloc) against the entry it
varies (smla_decode_fp8 with the caller's workspace), through the C ABI: two
calls in a row on the library's static workspace, the second with a smaller
input, each equal bit for bit to the ordinary call; a plan larger than the
static workspace is rejected before anything is launched."""

import numpy as np
import pytest
import torch

from sparse_mla_attention_indices_amd import smla
from sparse_mla_attention_indices_amd import workloads as W
from tests.gpu_util import DeviceWorkload, assert_parity, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    smla.library()


def _pair(dw, T, splits):
    """(ordinary call with its own workspace, allocation-free call) over the first T tokens."""
    w = dw.w
    ref_out, ref_lse, _ = dw.run(num_splits=splits, num_tokens=T)
    out = torch.full((T, w.h_q, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, w.h_q), 3.0, dtype=torch.float32, device="cuda")
    smla.smla_decode_fp8_noalloc(dw.q[:T], dw.cache, dw.bt, dw.req[:T], dw.idx[:T], w.sm_scale, out, lse=lse,
                                 num_splits=splits)
    torch.cuda.synchronize()
    return ref_out, ref_lse, out, lse


def test_static_workspace_calls_match_the_ordinary_call():
    w = W.config2()
    dw = DeviceWorkload(w)
    T, H, K = w.num_tokens, w.h_q, w.topk
    # first call: the headline batch as planned (4 splits, 33.6 MB of parts);
    # second call: a smaller batch with another split count in the same array
    for t_count, splits in ((T, 0), (T // 4, 3)):
        need = smla.smla_workspace_size(t_count, H, K, num_splits=splits)
        assert 0 < need <= smla.STATIC_WORKSPACE_BYTES
        log(f"[case] no-alloc decode T={t_count} splits={splits} parts={need} B")
        ref_out, ref_lse, out, lse = _pair(dw, t_count, splits)
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        assert_parity(w, out, lse, tokens=np.arange(t_count) if t_count < T else None,
                      label=f"no-alloc T{t_count} s{splits}")


def test_static_workspace_too_small_is_rejected_before_launch():
    w = W.config1_fp8()
    dw = DeviceWorkload(w)
    T, H = 256, 64
    K = 2048
    q = torch.zeros((T, H, 576), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((T, K), dtype=torch.int32, device="cuda")
    req = torch.zeros((T,), dtype=torch.int32, device="cuda")
    assert smla.smla_workspace_size(T, H, K, num_splits=4) > smla.STATIC_WORKSPACE_BYTES
    out = torch.full((T, H, 512), 5.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(smla.SmlaError) as e:
        smla.smla_decode_fp8_noalloc(q, dw.cache, dw.bt, req, idx, w.sm_scale, out, num_splits=4)
    assert e.value.status == 4                      # SMLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())


def test_staged_and_parts_only_flags_are_rejected():
    lib = smla.library()
    w = W.config1_fp8()
    dw = DeviceWorkload(w)
    out = torch.empty((w.num_tokens, w.h_q, 512), dtype=torch.bfloat16, device="cuda")
    for flag in (smla.FLAG_PARTIALS_ONLY, smla.FLAG_DEFER_MERGE, smla.FLAG_MERGE_ONLY):
        st = lib.smla_decode_fp8_noalloc(dw.q.data_ptr(), dw.cache.data_ptr(), dw.bt.data_ptr(), dw.req.data_ptr(),
                                         dw.idx.data_ptr(), w.sm_scale, w.num_tokens, w.h_q, w.topk, w.num_reqs,
                                         w.max_blocks_per_req, w.num_blocks, out.data_ptr(), None, None,
                                         smla._options(2, flag), torch.cuda.current_stream().cuda_stream)
        assert st == 6                              # SMLA_ERR_ARG
