"""Query-aware page selection (Quest) for one decode query -- TEST INFRASTRUCTURE ONLY.

Only ``tests/`` may use this module; the library never loads it.

The steps follow the pages in their order ("Long context, KV eviction and
sparse attention", "Sparse attention: choosing dynamically at every step",
Quest; "Attention Optimizations", "Query-aware retrieval": a cheap per-page
summary, the top pages by it, attention over those only):

  1. summary: for every full page of 16 tokens and every KV head, the
     per-dimension minimum and maximum of the page's keys;
  2. bound: for query head h, upper[p] = sum_d max(q_d * kmin[p, d],
     q_d * kmax[p, d]), an upper bound on q . k for every key k of page p;
  3. choice: the `budget` pages with the largest bound per query head (ties
     go to the lower page; this build's reading, the pages leave ties open);
     the last, partial page is always kept;
  4. attention: softmax attention of the query head over the tokens of the
     chosen pages and the partial page, two passes in fp64.

Everything is fp64 (exact for the integer-valued inputs the tests use, so
the choice of pages is exact too).  Parity status: pinned (a hand-worked
mixed-sign bound in tests/golden/quest_bound_tiny.json, tightness on pages of
identical keys, the bound holding for every key, full budget equals full
attention through the C oracle, ties).
"""
from __future__ import annotations

import math

import torch

BLOCK = 16


def page_minmax(k: torch.Tensor, seq_lens):
    """k logical [B, Hkv, S, D] -> (kmin, kmax) [B, Hkv, n_blocks, D] fp64 over full pages."""
    B, Hkv, S, D = k.shape
    nb = S // BLOCK
    kk = k[:, :, : nb * BLOCK].double().reshape(B, Hkv, nb, BLOCK, D)
    return kk.amin(3), kk.amax(3)


def upper_bounds(q: torch.Tensor, kmin, kmax, seq_lens, G: int):
    """q [B, Hq, D] -> [B, Hq, n_blocks] fp64; -inf for pages that are not full."""
    B, Hq, D = q.shape
    nb = kmin.shape[2]
    out = torch.full((B, Hq, nb), -math.inf, dtype=torch.float64)
    for b, L in enumerate(torch.as_tensor(seq_lens).tolist()):
        n_full = min(L // BLOCK, nb)
        for h in range(Hq):
            qv = q[b, h].double()
            lo, hi = kmin[b, h // G, :n_full], kmax[b, h // G, :n_full]
            out[b, h, :n_full] = torch.maximum(qv * lo, qv * hi).sum(-1)
    return out


def choose(upper: torch.Tensor, seq_lens, budget: int):
    """Chosen full pages per (b, h): the `budget` largest bounds, ties to the
    lower page, as a sorted list."""
    B, Hq, nb = upper.shape
    sel = []
    for b, L in enumerate(torch.as_tensor(seq_lens).tolist()):
        n_full = min(L // BLOCK, nb)
        for h in range(Hq):
            order = sorted(range(n_full), key=lambda p: (-upper[b, h, p].item(), p))
            sel.append(sorted(order[:budget]))
    return sel


def attention(q, k, v, seq_lens, chosen, scale, G: int):
    """Attention of each query head over its chosen pages plus the partial
    last page; returns (out [B*Hq, D], lse [B*Hq]) fp64."""
    B, Hq, D = q.shape
    out = torch.zeros(B * Hq, D, dtype=torch.float64)
    lse = torch.full((B * Hq,), -math.inf, dtype=torch.float64)
    for b, L in enumerate(torch.as_tensor(seq_lens).tolist()):
        n_full = L // BLOCK
        for h in range(Hq):
            r = b * Hq + h
            toks = [BLOCK * p + i for p in chosen[r] for i in range(BLOCK)]
            toks += list(range(n_full * BLOCK, L))
            if not toks:
                continue
            kk = k[b, h // G, toks].double()
            vv = v[b, h // G, toks].double()
            s = scale * (kk @ q[b, h].double())
            m = s.max()
            p = torch.exp(s - m)
            out[r] = (p[:, None] * vv).sum(0) / p.sum()
            lse[r] = m + torch.log(p.sum())
    return out, lse


def decode(q, k, v, seq_lens, budget, scale=None):
    """The whole step: summaries, bounds, choice, attention."""
    B, Hq, D = q.shape
    G = Hq // k.shape[1]
    if scale is None:
        scale = D ** -0.5
    kmin, kmax = page_minmax(k, seq_lens)
    up = upper_bounds(q, kmin, kmax, seq_lens, G)
    chosen = choose(up, seq_lens, budget)
    return attention(q, k, v, seq_lens, chosen, scale, G), chosen
