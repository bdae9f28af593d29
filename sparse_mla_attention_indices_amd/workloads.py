"""Seeded synthetic workloads for sparse MLA forward.

This module only *generates inputs*: paged block tables (built by handing out
blocks from a shuffled free list, the way a cache allocator does), per-token
logical top-k index lists, bf16 queries and cache rows. It holds none of the
attention arithmetic and no logical-to-physical index conversion. It is the one
module that both the GPU path's tests/benchmark and the CPU oracle's tests read.

Values are produced as raw bit patterns (numpy ``uint16`` for bfloat16,
``uint8`` for fp8_ds_mla and nvfp4_ds_mla rows) so every consumer sees the same
bytes. Rounding to bfloat16 and encoding to e4m3 use PyTorch's own CPU casts;
nvfp4_ds_mla rows are drawn as random codes (no quantisation step).

Row formats follow the vLLM ``flashmla_sparse.py`` page (FLASHMLA_SPARSE
backend): bf16 cache rows are 576 values (512 latent + 64 RoPE); fp8_ds_mla rows
are 656 bytes = 512 e4m3 latent values, four float32 scales (scale i covers
latent values 128*i..128*i+127), 64 bfloat16 RoPE values. Block size is 64.
nvfp4_ds_mla rows are 352 bytes (the size on the vLLM pull-request page "Support
nvfp4_ds_mla on FLASHINFER_MLA_SPARSE, with native NVFP4 decode"), laid out as
256 bytes of E2M1 latent codes (two per byte, the even position in the low
nibble), 32 E4M3 scales (one per 16 latent values), 64 E4M3 RoPE bytes.

Five named configurations (the shapes the pages' serving setups run at):

  1 tiny        2 requests x 4 tokens, ctx 256, h_q 16, top-k 64, ~10% -1 slots, bf16 cache
  2 fp8 decode  64 requests x 1 token, ctx U{4096..8192}, h_q 64, top-k 2048, fp8 cache
  3 bf16 prefill 4 requests x 4096 tokens (causal, -1 tail below 2048), h_q 128, top-k 2048
  4 spec decode 128 requests x 2 tokens, ctx log-U[16k, 64k], h_q 16, top-k 512/1024/2048,
                5% -1 slots, fp8 cache
  5 long mixed  32 decode tokens + 2 prefill requests x 2048 tokens (ctx 131072 and 65536),
                h_q 128, top-k 2048, fp8 cache

and config 4's batches over an nvfp4_ds_mla cache (config4_nvfp4): the shape the
pull-request page runs its native NVFP4 decode at (16 heads, top-k 512, 1024 or
2048).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK = 64
D_QK = 576
D_V = 512
FP8_ROW_BYTES = 656
NVFP4_ROW_BYTES = 352
E4M3_MAX = 448.0
SM_SCALE_576 = 1.0 / math.sqrt(576.0)

# Rows generated per chunk when filling large caches (bounds peak host memory).
_CHUNK_ROWS = 1 << 18


@dataclass
class Workload:
    name: str
    cache_format: str                 # "bf16", "fp8" or "nvfp4"
    q: np.ndarray                     # uint16 [T, H, 576] bf16 bits
    cache: np.ndarray                 # uint16 [NB, 64, 576], uint8 [NB, 64, 656] or [NB, 64, 352]
    block_table: np.ndarray           # int32 [R, MB], padding entries 0
    req_id_per_token: np.ndarray      # int32 [T]
    topk_indices: np.ndarray          # int32 [T, K], logical, -1 = invalid
    sm_scale: float
    ctx_lens: np.ndarray              # int64 [R]
    info: dict = field(default_factory=dict)

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def h_q(self) -> int:
        return int(self.q.shape[1])

    @property
    def topk(self) -> int:
        return int(self.topk_indices.shape[1])

    @property
    def num_reqs(self) -> int:
        return int(self.block_table.shape[0])

    @property
    def max_blocks_per_req(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def num_blocks(self) -> int:
        return int(self.cache.shape[0])


# ----------------------------------------------------------------- helpers

def _rng(seed: int, *parts: int) -> np.random.Generator:
    """numpy generator for structure (block tables, index lists, context lengths)."""
    return np.random.default_rng(np.random.SeedSequence([int(seed), *[int(p) for p in parts]]))


def _tgen(seed: int, *parts: int):
    """torch CPU generator for bulk values (faster than numpy for 10^8-10^9 samples)."""
    import torch
    state = np.random.SeedSequence([int(seed), *[int(p) for p in parts]]).generate_state(1, np.uint64)[0]
    return torch.Generator().manual_seed(int(state) & ((1 << 63) - 1))


def to_bf16_bits(x) -> np.ndarray:
    """float32 values (numpy or torch) -> bfloat16 bit patterns (torch's RNE cast)."""
    import torch
    t = x if isinstance(x, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact widening)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(gen, shape) -> np.ndarray:
    """N(0, 1) samples rounded to bfloat16, as bit patterns."""
    import torch
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, 1 << 26):
        e = min(n, s + (1 << 26))
        out[s:e] = to_bf16_bits(torch.randn(e - s, generator=gen))
    return out.reshape(shape)


def pack_fp8_rows(latent, rope_bits: np.ndarray, gen) -> np.ndarray:
    """Encode rows into the 656-byte fp8_ds_mla format.

    latent: float32 [n, 512] (numpy or torch); rope_bits: uint16 [n, 64] bf16 bits,
    stored as is. Per 128-value group the scale is U(0.5, 2) * amax / 448 (float32),
    and each byte is e4m3(clamp(x / scale, -448, 448)) by torch's e4m3fn cast.
    """
    import torch
    lat = latent if isinstance(latent, torch.Tensor) else torch.from_numpy(
        np.ascontiguousarray(latent, dtype=np.float32))
    n = lat.shape[0]
    groups = lat.reshape(n, 4, 128)
    amax = groups.abs().amax(dim=2).clamp_min(1e-30)
    u = torch.rand((n, 4), generator=gen) * 1.5 + 0.5
    scale = (u * amax / E4M3_MAX).to(torch.float32)
    scaled = (groups / scale[:, :, None]).clamp(-E4M3_MAX, E4M3_MAX)
    codes = scaled.reshape(n, 512).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    rows = np.empty((n, FP8_ROW_BYTES), dtype=np.uint8)
    rows[:, 0:512] = codes
    rows[:, 512:528] = scale.numpy().astype("<f4").view(np.uint8).reshape(n, 16)
    rows[:, 528:656] = np.ascontiguousarray(rope_bits, dtype="<u2").view(np.uint8).reshape(n, 128)
    return rows


def random_bf16_cache(seed: int, cfg: int, num_blocks: int) -> np.ndarray:
    rows = num_blocks * BLOCK
    out = np.empty((rows, D_QK), dtype=np.uint16)
    for c, s in enumerate(range(0, rows, _CHUNK_ROWS)):
        e = min(rows, s + _CHUNK_ROWS)
        out[s:e] = normal_bf16(_tgen(seed, cfg, 2, c), (e - s, D_QK))
    return out.reshape(num_blocks, BLOCK, D_QK)


def random_fp8_cache(seed: int, cfg: int, num_blocks: int) -> np.ndarray:
    import torch
    rows = num_blocks * BLOCK
    out = np.empty((rows, FP8_ROW_BYTES), dtype=np.uint8)
    for c, s in enumerate(range(0, rows, _CHUNK_ROWS)):
        e = min(rows, s + _CHUNK_ROWS)
        gen = _tgen(seed, cfg, 2, c)
        latent = torch.randn((e - s, D_V), generator=gen)
        rope = normal_bf16(gen, (e - s, 64))
        out[s:e] = pack_fp8_rows(latent, rope, gen)
    return out.reshape(num_blocks, BLOCK, FP8_ROW_BYTES)


def random_nvfp4_rows(gen, n: int) -> np.ndarray:
    """n random nvfp4_ds_mla rows: every latent code uniform over the 16 E2M1
    codes (two random nibbles per byte), every block scale the e4m3 cast of
    U(0.5, 2) / 3 (a 16-value block of N(0, 1) samples has amax about 2, and
    amax / 6 is the usual NVFP4 scale), RoPE bytes the e4m3 cast of N(0, 1)."""
    import torch
    rows = np.empty((n, NVFP4_ROW_BYTES), dtype=np.uint8)
    rows[:, 0:256] = torch.randint(0, 256, (n, 256), generator=gen, dtype=torch.uint8).numpy()
    scale = (torch.rand((n, 32), generator=gen) * 1.5 + 0.5) / 3.0
    rows[:, 256:288] = scale.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    rows[:, 288:352] = torch.randn((n, 64), generator=gen).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return rows


def random_nvfp4_cache(seed: int, cfg: int, num_blocks: int) -> np.ndarray:
    rows = num_blocks * BLOCK
    out = np.empty((rows, NVFP4_ROW_BYTES), dtype=np.uint8)
    for c, s in enumerate(range(0, rows, _CHUNK_ROWS)):
        e = min(rows, s + _CHUNK_ROWS)
        out[s:e] = random_nvfp4_rows(_tgen(seed, cfg, 8, c), e - s)
    return out.reshape(num_blocks, BLOCK, NVFP4_ROW_BYTES)


def fp8_from_bf16_cache(cache_bf16: np.ndarray, seed: int, cfg: int) -> np.ndarray:
    """fp8_ds_mla packing of an existing bf16 cache (same latent values and RoPE bits)."""
    nb = cache_bf16.shape[0]
    flat = cache_bf16.reshape(-1, D_QK)
    latent = bf16_bits_to_f32(flat[:, :D_V])
    rows = pack_fp8_rows(latent, flat[:, D_V:], _tgen(seed, cfg, 5))
    return rows.reshape(nb, BLOCK, FP8_ROW_BYTES)


def allocate_block_table(rng: np.random.Generator, ctx_lens, max_blocks_per_req: int | None = None):
    """Give each request ceil(ctx/64) blocks, popped in order from a shuffled free list.

    Returns (block_table int32 [R, MB] with padding 0, num_blocks)."""
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    need = (ctx + BLOCK - 1) // BLOCK
    nb = int(need.sum())
    mb = int(need.max()) if max_blocks_per_req is None else int(max_blocks_per_req)
    if mb < int(need.max()):
        raise ValueError("max_blocks_per_req smaller than a request's block count")
    free_list = list(rng.permutation(nb))
    bt = np.zeros((len(ctx), mb), dtype=np.int32)
    for r in range(len(ctx)):
        for b in range(int(need[r])):
            bt[r, b] = free_list.pop()
    return bt, nb


def draw_indices(rng: np.random.Generator, visible, topk: int, p_invalid: float = 0.0) -> np.ndarray:
    """Per token: `topk` distinct logical positions in [0, visible) in random order.

    A token that sees fewer than `topk` positions gets all of them (shuffled) and
    -1 for the rest. Then every slot independently becomes -1 with p_invalid."""
    vis = np.asarray(visible, dtype=np.int64)
    out = np.full((len(vis), topk), -1, dtype=np.int32)
    for t, n in enumerate(vis):
        n = int(n)
        if n <= topk:
            out[t, :n] = rng.permutation(n)
        else:
            out[t] = rng.choice(n, size=topk, replace=False)
    if p_invalid > 0:
        drop = rng.random(out.shape) < p_invalid
        out[drop] = -1
    return out


def build(name: str, cfg: int, seed: int, ctx_lens, token_req, token_visible, h_q: int,
          topk: int, cache_format: str, p_invalid: float = 0.0,
          max_blocks_per_req: int | None = None, index_part: int = 3) -> Workload:
    """Generic builder: one request per entry of ctx_lens; one query token per entry of
    token_req (its request) / token_visible (how many leading positions it may pick)."""
    bt, nb = allocate_block_table(_rng(seed, cfg, 0), ctx_lens, max_blocks_per_req)
    req = np.asarray(token_req, dtype=np.int32)
    q = normal_bf16(_tgen(seed, cfg, 1), (len(req), h_q, D_QK))
    idx = draw_indices(_rng(seed, cfg, index_part), token_visible, topk, p_invalid)
    if cache_format == "bf16":
        cache = random_bf16_cache(seed, cfg, nb)
    elif cache_format == "fp8":
        cache = random_fp8_cache(seed, cfg, nb)
    elif cache_format == "nvfp4":
        cache = random_nvfp4_cache(seed, cfg, nb)
    else:
        raise ValueError(cache_format)
    return Workload(name=name, cache_format=cache_format, q=q, cache=cache, block_table=bt,
                    req_id_per_token=req, topk_indices=idx, sm_scale=SM_SCALE_576,
                    ctx_lens=np.asarray(ctx_lens, dtype=np.int64))


# ----------------------------------------------------------- named configs

def config1(seed: int = 0) -> Workload:
    """Tiny: 2 requests x 4 tokens, ctx 256, h_q 16, top-k 64 distinct, ~10% -1, bf16."""
    ctx = [256, 256]
    req = [0] * 4 + [1] * 4
    return build("c1_tiny", 1, seed, ctx, req, [256] * 8, 16, 64, "bf16", p_invalid=0.1)


def config1_fp8(seed: int = 0) -> Workload:
    """Config 1's inputs with the same kv packed as fp8_ds_mla rows."""
    w = config1(seed)
    w.cache = fp8_from_bf16_cache(w.cache, seed, 1)
    w.cache_format = "fp8"
    w.name = "c1_tiny_fp8"
    return w


def config1_nvfp4(seed: int = 0) -> Workload:
    """Config 1's block table, q and indices over an nvfp4_ds_mla cache."""
    w = config1(seed)
    w.cache = random_nvfp4_cache(seed, 1, w.cache.shape[0])
    w.cache_format = "nvfp4"
    w.name = "c1_tiny_nvfp4"
    return w


def config2(seed: int = 0) -> Workload:
    """FP8 decode: 64 requests x 1 token, ctx U{4096..8192}, h_q 64, top-k 2048."""
    ctx = _rng(seed, 2, 4).integers(4096, 8192, size=64, endpoint=True)
    return build("c2_fp8_decode", 2, seed, ctx, np.arange(64), ctx, 64, 2048, "fp8",
                 max_blocks_per_req=128)


def config3(seed: int = 0, tokens_per_req: int = 4096, num_reqs: int = 4) -> Workload:
    """BF16 prefill: 4 requests x 4096 tokens, causal (token p sees 0..p), h_q 128, top-k 2048."""
    ctx = [tokens_per_req] * num_reqs
    req = np.repeat(np.arange(num_reqs), tokens_per_req)
    vis = np.tile(np.arange(1, tokens_per_req + 1), num_reqs)
    return build("c3_bf16_prefill", 3, seed, ctx, req, vis, 128, 2048, "bf16")


def config4(seed: int = 0, topk: int = 2048, cache_format: str = "fp8") -> Workload:
    """Spec decode at h_q 16: 128 requests x 2 tokens, ctx log-U[16k, 64k], 5% -1."""
    if topk not in (512, 1024, 2048):
        raise ValueError("config 4 sweeps top-k over 512, 1024, 2048")
    u = _rng(seed, 4, 4).uniform(math.log(16384), math.log(65536), size=128)
    ctx = np.floor(np.exp(u)).astype(np.int64)
    req = np.repeat(np.arange(128), 2)
    vis = np.stack([ctx - 1, ctx], axis=1).reshape(-1)
    tag = "" if cache_format == "fp8" else f"_{cache_format}"
    return build(f"c4_spec_decode{tag}_k{topk}", 4, seed, ctx, req, vis, 16, topk, cache_format,
                 p_invalid=0.05, max_blocks_per_req=1024, index_part=10 + topk)


def config4_nvfp4(seed: int = 0, topk: int = 2048) -> Workload:
    """Config 4's batch (same block table, q and index lists) over an
    nvfp4_ds_mla cache."""
    return config4(seed, topk, "nvfp4")


def config4_sweep(seed: int = 0, cache_format: str = "fp8"):
    """config4 at top-k 512, 1024 and 2048, generated once: the three workloads
    share one cache array (the cache, q and block table do not depend on top-k;
    each index list comes from its own sub-seed), so each equals
    config4(seed, k, cache_format)."""
    base = config4(seed, 2048, cache_format)
    out = [base]
    for k in (512, 1024):
        u = _rng(seed, 4, 4).uniform(math.log(16384), math.log(65536), size=128)
        ctx = np.floor(np.exp(u)).astype(np.int64)
        vis = np.stack([ctx - 1, ctx], axis=1).reshape(-1)
        idx = draw_indices(_rng(seed, 4, 10 + k), vis, k, 0.05)
        tag = "" if cache_format == "fp8" else f"_{cache_format}"
        out.append(Workload(name=f"c4_spec_decode{tag}_k{k}", cache_format=cache_format, q=base.q,
                            cache=base.cache,
                            block_table=base.block_table, req_id_per_token=base.req_id_per_token,
                            topk_indices=idx, sm_scale=base.sm_scale, ctx_lens=base.ctx_lens))
    return sorted(out, key=lambda w: w.topk)


def config5(seed: int = 0) -> Workload:
    """Long mixed: 32 decode tokens (ctx U{8192..106496}) then 2 prefill requests
    (ctx 131072, 65536) whose last 2048 positions are query tokens; h_q 128, top-k 2048."""
    dec_ctx = _rng(seed, 5, 4).integers(8192, 106496, size=32, endpoint=True)
    pre_ctx = np.array([131072, 65536])
    ctx = np.concatenate([dec_ctx, pre_ctx])
    req = list(range(32))
    vis = list(dec_ctx)
    for r, c in zip((32, 33), pre_ctx):
        for p in range(int(c) - 2048, int(c)):
            req.append(r)
            vis.append(p + 1)
    return build("c5_long_mixed", 5, seed, ctx, req, vis, 128, 2048, "fp8",
                 max_blocks_per_req=2048)


def mixed_batch(seed: int, h_q: int, topk: int, decode_ctx, prefill_ctx, prefill_queries,
                p_invalid: float = 0.0, cache_format: str = "fp8") -> Workload:
    """A batch in the order a serving engine builds it: decode requests first
    (one query token each, seeing its whole context), then prefill requests whose
    last prefill_queries[r] positions are query tokens (position p sees 0..p).
    The Workload's ctx_lens are the requests' sequence lengths (context plus
    query)."""
    dec = [int(c) for c in decode_ctx]
    pre = [int(c) for c in prefill_ctx]
    ctx = dec + pre
    req = list(range(len(dec)))
    vis = list(dec)
    for r, (c, nq) in enumerate(zip(pre, prefill_queries)):
        for pos in range(c - int(nq), c):
            req.append(len(dec) + r)
            vis.append(pos + 1)
    return build("mixed", 6, seed, ctx, req, vis, h_q, topk, cache_format, p_invalid=p_invalid)


def config5_prefill(seed: int = 0, cache_format: str = "fp8") -> Workload:
    """Config 5's two prefill requests alone (ctx 131072 and 65536; query tokens are
    their last 2048 positions), h_q 128, top-k 2048, fp8 cache (or another
    format): the part the separate-prefill mode upconverts."""
    pre_ctx = np.array([131072, 65536])
    req, vis = [], []
    for r, c in enumerate(pre_ctx):
        for pos in range(int(c) - 2048, int(c)):
            req.append(r)
            vis.append(pos + 1)
    tag = "" if cache_format == "fp8" else f"_{cache_format}"
    return build(f"c5_prefill_part{tag}", 7, seed, pre_ctx, req, vis, 128, 2048, cache_format,
                 max_blocks_per_req=2048)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}
