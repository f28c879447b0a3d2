"""Cache append in logical token order -- TEST INFRASTRUCTURE ONLY.

Only ``tests/`` may use this module; the library never loads it.

Decoding appends the new token's cache entries before attending
("Attention Optimizations", "DSA: DeepSeek Sparse Attention", "Computation
Path": ``update_cache(cat(c_KV, k_pe))`` for the 576-value latent row and
``update_cache(k_i)`` for the indexer key; per KV head K and V rows for GQA).
Here a cache is held in logical order, one slot per token position, so an
append is a single indexed assignment; paging, page tables and rolling
buffers are layouts of this logical cache that the tests unfold back into it.

Parity status: pinned (tests compare with library index_put and with
attention over the appended token).
"""
from __future__ import annotations

import torch


def append(cache: torch.Tensor, positions, new: torch.Tensor) -> torch.Tensor:
    """Return a copy of the logical cache with each sequence's new entry written.

    cache      [B, S, X] (one row per token: latent or indexer cache) or
               [B, H, S, X] (one row per head and token: K or V cache)
    positions  int [B], the token position written; a negative entry leaves
               that sequence unchanged
    new        [B, X] or [B, H, X], the same dtype as cache
    """
    out = cache.clone()
    for b, p in enumerate(torch.as_tensor(positions).tolist()):
        if p < 0:
            continue
        if cache.dim() == 3:
            out[b, p] = new[b]
        else:
            out[b, :, p] = new[b]
    return out
