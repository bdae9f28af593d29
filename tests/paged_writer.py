"""A paged-cache writer simulation used to pin the index conversion.

Tokens of every request are appended one at a time, round robin across
requests, into 64-slot blocks taken from a shuffled free list -- the way a
serving engine grows its KV cache. The writer records where each (request,
position) landed as a (block, offset) pair by iteration alone: it never divides
a position by the block size. A converter that maps (request, position) to the
slot the writer used is therefore checked against an independent construction.
"""

from __future__ import annotations

import numpy as np

BLOCK = 64


class PagedCache:
    def __init__(self, rng: np.random.Generator, ctx_lens, extra_blocks: int = 0,
                 max_blocks_per_req: int | None = None):
        ctx = [int(c) for c in ctx_lens]
        need = sum(-(-c // BLOCK) for c in ctx)
        self.num_blocks = need + int(extra_blocks)
        free = list(rng.permutation(self.num_blocks))
        self.blocks = [[] for _ in ctx]
        self.where = {}
        fill = [BLOCK] * len(ctx)
        written = [0] * len(ctx)
        remaining = True
        while remaining:
            remaining = False
            for r, c in enumerate(ctx):
                if written[r] == c:
                    continue
                remaining = True
                if fill[r] == BLOCK:
                    self.blocks[r].append(int(free.pop()))
                    fill[r] = 0
                self.where[(r, written[r])] = (self.blocks[r][-1], fill[r])
                fill[r] += 1
                written[r] += 1
        mb = max(len(b) for b in self.blocks) if max_blocks_per_req is None else max_blocks_per_req
        self.block_table = np.zeros((len(ctx), mb), dtype=np.int32)
        for r, bl in enumerate(self.blocks):
            self.block_table[r, :len(bl)] = bl
        self.ctx = ctx

    def logical_rows(self, cache: np.ndarray, r: int, positions) -> np.ndarray:
        """Rows of request r at the given logical positions, looked up in the writer's record."""
        return np.stack([cache[self.where[(r, int(p))]] for p in positions])
