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


def tricky_nvfp4_rows(rng, T):
    """Latent rows for the nvfp4 writer. Each 16-value block is one kind: E2M1
    rounding ties under a scale of exactly 1.0 (the block holds 6.0), tiny values
    whose scale rounds to zero, signed zeros, large values whose amax / 6 passes
    448, scales on e4m3 rounding ties, or plain normal values."""
    e2m1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    ties = (e2m1[:-1] + e2m1[1:]) / 2                     # 0.25 .. 5.0, all bf16 values
    e4m3 = np.array([oracle.e4m3fn(c) for c in range(0x7F)])
    sc_ties = (e4m3[:-1] + e4m3[1:]) / 2
    lat = rng.normal(0, 1, (T, 512)).astype(np.float32)
    for t in range(T):
        for b in range(32):
            blk = lat[t, 16 * b:16 * b + 16]
            kind = (t + b) % 6
            if kind == 0:
                blk[:15] = ties[rng.integers(0, len(ties), 15)] * rng.choice([-1, 1], 15)
                blk[15] = 6.0
            elif kind == 1:
                blk[:] *= 1e-5
            elif kind == 2:
                blk[:] = 0.0
                blk[::2] = -0.0
            elif kind == 3:
                blk[:] *= 1e4
            elif kind == 4:
                # amax / 6 exactly halfway between two e4m3 values (bf16-exact ones)
                m = sc_ties[rng.integers(40, 100)]
                blk[:] = rng.uniform(-1, 1, 16) * m * 6
                blk[0] = m * 6
    return lat


@pytest.mark.parametrize("T", [300, 303, 1])
def test_cache_write_nvfp4_bit_exact(T):
    rng = np.random.default_rng(21)
    NB = 16
    lat_b = bits_of(tricky_nvfp4_rows(rng, T))
    rope = rng.normal(0, 2, (T, 64))
    rope[:, :4] = [600.0, -1000.0, 1e-6, -0.0]             # saturation, a tiny value, a signed zero
    rope_b = bits_of(rope)
    slots = rng.permutation(NB * 64)[:T].astype(np.int64)
    slots[::17] = -1
    slots[5:6] = NB * 64
    init = rng.integers(0, 256, (NB, 64, 352), dtype=np.uint8)
    want = oracle.cache_write(oracle.NVFP4_CACHE, lat_b, rope_b, slots, init.copy())
    dev_cache = torch.from_numpy(init.copy()).cuda()
    log(f"[case] cache write nvfp4_ds_mla T={T}")
    smla.smla_concat_and_cache_mla(torch.from_numpy(lat_b.view(np.int16)).cuda().view(torch.bfloat16),
                                   torch.from_numpy(rope_b.view(np.int16)).cuda().view(torch.bfloat16),
                                   dev_cache, torch.from_numpy(slots).cuda(), kv_cache_dtype="nvfp4_ds_mla")
    torch.cuda.synchronize()
    got = dev_cache.cpu().numpy()
    if not np.array_equal(got, want):
        bad = np.argwhere(got.reshape(NB * 64, -1) != want.reshape(NB * 64, -1))
        s, b = bad[0]
        raise AssertionError(f"{len(bad)} bytes differ, first at (slot, byte) {bad[:5].tolist()}: "
                             f"got {got.reshape(NB * 64, -1)[s, b]:#x} want {want.reshape(NB * 64, -1)[s, b]:#x}")


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


@pytest.mark.parametrize("fmt", ["fp8", "nvfp4"])
def test_attention_over_a_written_cache(fmt):
    """Rows written by smla_concat_and_cache_mla feed smla_decode_fp8 (or
    smla_decode_nvfp4); the result matches the oracle's attention over the
    oracle's bytes (identical by the tests above, compared again here)."""
    from tests.test_gpu_parity import small
    w = small(61, fmt, 16, 256, n_req=2, tok_per_req=4, ctx=(300, 600), p_invalid=0.1)
    rng = np.random.default_rng(61)
    NB = w.cache.shape[0]
    lat_b = bits_of(rng.normal(0, 1, (NB * 64, 512)))
    rope_b = bits_of(rng.normal(0, 1, (NB * 64, 64)))
    slots = np.arange(NB * 64, dtype=np.int64)
    ofmt = oracle.FP8_CACHE if fmt == "fp8" else oracle.NVFP4_CACHE
    w.cache = oracle.cache_write(ofmt, lat_b, rope_b, slots, np.zeros_like(w.cache))
    dw = DeviceWorkload(w)
    dw.cache.zero_()
    smla.smla_concat_and_cache_mla(torch.from_numpy(lat_b.view(np.int16)).cuda().view(torch.bfloat16),
                                   torch.from_numpy(rope_b.view(np.int16)).cuda().view(torch.bfloat16),
                                   dw.cache, torch.from_numpy(slots).cuda(), kv_cache_dtype=fmt + "_ds_mla")
    torch.cuda.synchronize()
    assert np.array_equal(dw.cache.cpu().numpy(), w.cache)
    out, lse, _ = dw.run()
    assert_parity(w, out, lse, label=f"attention over written {fmt} cache")
