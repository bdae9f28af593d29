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
