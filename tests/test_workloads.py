"""The seeded input generators: the shared-cache sweep of the speculative-decode
batch equals the batch built for each top-k on its own."""

import numpy as np
import pytest

from sparse_mla_attention_indices_amd import workloads as W


@pytest.mark.slow
def test_config4_sweep_equals_config4_per_topk():
    sweep = W.config4_sweep(0)
    assert [w.topk for w in sweep] == [512, 1024, 2048]
    one = W.config4(0, 512)
    a = sweep[0]
    for name in ("q", "cache", "block_table", "req_id_per_token", "topk_indices", "ctx_lens"):
        assert np.array_equal(getattr(a, name), getattr(one, name)), name
    assert a.name == one.name and a.sm_scale == one.sm_scale
    assert sweep[1].cache is sweep[2].cache


def test_nvfp4_rows_have_the_documented_byte_ranges():
    rows = W.random_nvfp4_rows(W._tgen(0, 1), 2000)
    assert rows.shape == (2000, W.NVFP4_ROW_BYTES) and rows.dtype == np.uint8
    # codes: every nibble value appears in both halves of the code bytes
    codes = rows[:, :256]
    assert set(np.unique(codes & 0xF)) == set(range(16))
    assert set(np.unique(codes >> 4)) == set(range(16))
    # scales: positive e4m3 codes of values in [1/6, 2/3], which round to
    # 0x23 (0.171875) .. 0x33 (0.6875)
    sc = rows[:, 256:288]
    assert sc.min() == 0x23 and sc.max() == 0x33
    # RoPE: e4m3 codes of N(0, 1) samples, both signs, never NaN
    rope = rows[:, 288:]
    assert np.any(rope & 0x80) and np.any(~rope & 0x80)
    assert not np.any((rope & 0x7F) == 0x7F)
