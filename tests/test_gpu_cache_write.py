"""GPU parity of the cache writer (smla_concat_and_cache_mla) against the CPU
oracle's writer: the cache bytes must be identical, since the quantised codes and
scales are integer / bit-level results. Cases cover exact rounding ties, tiny and
subnormal inputs, signed zeros, all-zero groups, skipped slots and a
prefill-sized batch checked on sampled rows. The last test runs attention over a
cache the writer produced."""

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_attention_indices_amd import smla
from tests.gpu_util import DeviceWorkload, assert_parity, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    smla.library()


def bits_of(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def tricky_rows(rng, T):
    """Latent rows whose values hit e4m3 rounding ties exactly: each group holds
    448 (so its scale is exactly 1.0) and values on midpoints between codes."""
    vals = np.array([oracle.e4m3fn(c) for c in range(0x7F)])
    mids = (vals[:-1] + vals[1:]) / 2
    lat = rng.normal(0, 1, (T, 512)).astype(np.float32)
    for t in range(T):
        for g in range(4):
            grp = lat[t, 128 * g:128 * g + 128]
            kind = (t + g) % 5
            if kind == 0:           # exact ties, bf16-representable ones only
                m = mids[rng.integers(0, len(mids), 127)]
                grp[:127] = m * rng.choice([-1, 1], 127)
                grp[127] = 448.0
            elif kind == 1:         # tiny values: scale near the float32 subnormal range
                grp[:] *= 1e-38
            elif kind == 2:         # all zero, with signed zeros
                grp[:] = 0.0
                grp[::2] = -0.0
            elif kind == 3:         # large values
                grp[:] *= 1e4
            # kind 4: plain normal values
    return lat


@pytest.mark.parametrize("T", [300, 303, 1])
@pytest.mark.parametrize("fmt", ["fp8_ds_mla", "auto"])
def test_cache_write_bit_exact(fmt, T):
    """T = 303 ends inside a wave's group of tokens; T = 1 is a lone token."""
    rng = np.random.default_rng(11)
    NB = 16
    lat_b = bits_of(tricky_rows(rng, T))
    rope_b = bits_of(rng.normal(0, 2, (T, 64)))
    slots = rng.permutation(NB * 64)[:T].astype(np.int64)
    slots[::17] = -1                      # skipped
    slots[5:6] = NB * 64                  # past the cache: skipped
    slots[6:7] = NB * 64 + 1000
    f = oracle.FP8_CACHE if fmt == "fp8_ds_mla" else oracle.BF16_CACHE
    if fmt == "fp8_ds_mla":
        init = rng.integers(0, 256, (NB, 64, 656), dtype=np.uint8)
        dev_cache = torch.from_numpy(init.copy()).cuda()
    else:
        init = rng.integers(0, 1 << 16, (NB, 64, 576), dtype=np.uint16)
        dev_cache = torch.from_numpy(init.view(np.int16).copy()).cuda().view(torch.bfloat16)
    want = oracle.cache_write(f, lat_b, rope_b, slots, init.copy())
    log(f"[case] cache write {fmt} T={T}")
    smla.smla_concat_and_cache_mla(torch.from_numpy(lat_b.view(np.int16)).cuda().view(torch.bfloat16),
                                   torch.from_numpy(rope_b.view(np.int16)).cuda().view(torch.bfloat16),
                                   dev_cache, torch.from_numpy(slots).cuda(), kv_cache_dtype=fmt)
    torch.cuda.synchronize()
    got = dev_cache.cpu()
    got = got.numpy() if fmt == "fp8_ds_mla" else got.view(torch.int16).numpy().view(np.uint16)
    if not np.array_equal(got, want):
        bad = np.argwhere(got.reshape(NB * 64, -1) != want.reshape(NB * 64, -1))
        raise AssertionError(f"{len(bad)} bytes differ, first at (slot, byte) {bad[:5].tolist()}")


def test_cache_write_prefill_batch_sampled():
    """16384 tokens (a prefill batch) into a 2 GiB-class pool, checked on 512 sampled rows."""
    rng = np.random.default_rng(12)
    T, NB = 16384, 4096
    lat = torch.randn(T, 512, dtype=torch.float32, generator=torch.Generator().manual_seed(12)) * 3
    lat_d = lat.to(torch.bfloat16).cuda()
    rope_d = torch.randn(T, 64, generator=torch.Generator().manual_seed(13)).to(torch.bfloat16).cuda()
    slots = torch.from_numpy(rng.permutation(NB * 64)[:T].astype(np.int64)).cuda()
    cache = torch.zeros((NB, 64, 656), dtype=torch.uint8, device="cuda")
    log(f"[case] cache write prefill T={T}")
    smla.smla_concat_and_cache_mla(lat_d, rope_d, cache, slots, kv_cache_dtype="fp8_ds_mla")
    torch.cuda.synchronize()
    pick = rng.choice(T, 512, replace=False)
    lat_b = lat_d[pick].cpu().view(torch.int16).numpy().view(np.uint16)
    rope_b = rope_d[pick].cpu().view(torch.int16).numpy().view(np.uint16)
    sl = slots[pick].cpu().numpy()
    small = np.zeros((T // 64 + 1, 64, 656), dtype=np.uint8)
    want = oracle.cache_write(oracle.FP8_CACHE, lat_b, rope_b, np.arange(512, dtype=np.int64), small)
    got = cache.view(-1, 656)[torch.from_numpy(sl).cuda()].cpu().numpy()
    assert np.array_equal(got, want.reshape(-1, 656)[:512])


def test_attention_over_a_written_cache():
    """Rows written by smla_concat_and_cache_mla feed smla_decode_fp8; the result
    matches the oracle's attention over the oracle's bytes (identical by the test
    above, compared again here)."""
    from tests.test_gpu_parity import small
    w = small(61, "fp8", 16, 256, n_req=2, tok_per_req=4, ctx=(300, 600), p_invalid=0.1)
    rng = np.random.default_rng(61)
    NB = w.cache.shape[0]
    lat_b = bits_of(rng.normal(0, 1, (NB * 64, 512)))
    rope_b = bits_of(rng.normal(0, 1, (NB * 64, 64)))
    slots = np.arange(NB * 64, dtype=np.int64)
    w.cache = oracle.cache_write(oracle.FP8_CACHE, lat_b, rope_b, slots, np.zeros_like(w.cache))
    dw = DeviceWorkload(w)
    dw.cache.zero_()
    smla.smla_concat_and_cache_mla(torch.from_numpy(lat_b.view(np.int16)).cuda().view(torch.bfloat16),
                                   torch.from_numpy(rope_b.view(np.int16)).cuda().view(torch.bfloat16),
                                   dw.cache, torch.from_numpy(slots).cuda(), kv_cache_dtype="fp8_ds_mla")
    torch.cuda.synchronize()
    assert np.array_equal(dw.cache.cpu().numpy(), w.cache)
    out, lse, _ = dw.run()
    assert_parity(w, out, lse, label="attention over written cache")
