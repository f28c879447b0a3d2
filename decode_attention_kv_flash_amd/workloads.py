"""Seeded synthetic inputs for decode attention over a KV cache.

This module draws random numbers and lays them out in memory; it computes
nothing of the attention method itself.  Both the HIP path and the CPU oracle
read the tensors it returns, so every comparison sees bit-identical inputs.

All values are drawn on the CPU with ``torch.Generator`` (seeded per workload),
rounded once to the storage dtype (fp32 -> bf16 is round-to-nearest-even), and
kept in two layouts:

* the *logical* layout the oracle reads: ``k[B, H_kv, S_max, D]`` with token
  ``t`` of sequence ``b`` at ``[b, :, t, :]``;
* the *physical* paged layout the kernels read: ``k_cache[num_pages, H_kv,
  page_size, D]`` plus ``page_table[B, max_pages]`` (PagedAttention's block
  table, "All the attentions", section 8).  Physical pages are a seeded random
  permutation, so logical neighbours are never physical neighbours.

Workload shapes follow the pages' model families: Llama-3-8B-shaped GQA
("All the attentions", "Why we need any of this"), Mistral-style window 4096
plus StreamingLLM sinks ("Attention Optimizations", "Attention sinks"), and
the DeepSeek-V3 MLA / DSA shapes ("Attention Optimizations", "DSA: DeepSeek
Sparse Attention", "Computation Path").
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

# Filler for cache slots that belong to no token (tail of a sequence's last
# page).  A kernel that reads them into a result is caught by the parity test.
TAIL_FILL = 3.0


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _normal(g, shape, dtype):
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    return x.to(dtype)


def _ints(g, lo, hi, shape, dtype):
    """Uniform integers in [lo, hi] (inclusive), stored in ``dtype``."""
    return torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int64).to(dtype)


@dataclass
class GQAInputs:
    """One decode step of (grouped-query) attention over a paged KV cache."""
    q: torch.Tensor               # [B, Hq, D]
    k: torch.Tensor               # logical [B, Hkv, S_max, D]
    v: torch.Tensor               # logical [B, Hkv, S_max, D]
    seq_lens: torch.Tensor        # int32 [B]
    k_cache: torch.Tensor         # physical [num_pages, Hkv, page_size, D]
    v_cache: torch.Tensor
    page_table: Optional[torch.Tensor]  # int32 [B, max_pages]; None = contiguous
    page_size: int
    window: int
    n_sink: int
    scale: float
    name: str = ""

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def Hq(self):
        return self.q.shape[1]

    @property
    def Hkv(self):
        return self.k.shape[1]

    @property
    def D(self):
        return self.q.shape[2]

    @property
    def S_max(self):
        return self.k.shape[2]

    @property
    def max_pages(self):
        return 1 if self.page_table is None else self.page_table.shape[1]

    def attended_tokens(self) -> int:
        """Number of (sequence, token) pairs a correct kernel must read."""
        total = 0
        for L in self.seq_lens.tolist():
            if self.window <= 0 or self.window >= L:
                total += L
            else:
                total += min(self.n_sink, L - self.window) + self.window
        return total

    def kv_bytes(self) -> int:
        """Algorithmic bytes: K and V rows of every attended token, all KV heads."""
        return self.attended_tokens() * 2 * self.Hkv * self.D * self.k.element_size()


def _paginate(g, k_log, v_log, seq_lens, page_size):
    """Scatter logical K/V into a randomly permuted paged cache."""
    B, Hkv, S_max, D = k_log.shape
    n_pages_b = [max(1, math.ceil(L / page_size)) for L in seq_lens]
    max_pages = max(n_pages_b)
    total = sum(n_pages_b)
    perm = torch.randperm(total, generator=g)
    page_table = torch.zeros(B, max_pages, dtype=torch.int32)
    kc = torch.full((total, Hkv, page_size, D), TAIL_FILL, dtype=k_log.dtype)
    vc = torch.full((total, Hkv, page_size, D), TAIL_FILL, dtype=v_log.dtype)
    off = 0
    for b, L in enumerate(seq_lens):
        for j in range(n_pages_b[b]):
            phys = int(perm[off + j])
            page_table[b, j] = phys
            t0, t1 = j * page_size, min((j + 1) * page_size, L)
            if t1 > t0:
                kc[phys, :, : t1 - t0] = k_log[b, :, t0:t1]
                vc[phys, :, : t1 - t0] = v_log[b, :, t0:t1]
        off += n_pages_b[b]
    return kc, vc, page_table


def make_gqa(*, B, Hq, Hkv, D, seq_lens, dtype=torch.bfloat16, page_size=16,
             paged=True, window=0, n_sink=0, sink_key_scale=1.0, scale=None,
             qk_int=0, seed=0, name="") -> GQAInputs:
    """Build a GQA/SWA decode workload.

    ``seq_lens`` is a list of per-sequence cached-token counts (the current
    token included).  ``sink_key_scale`` multiplies the key rows of tokens
    ``0..n_sink-1`` before rounding (a stand-in for the sink dominance of real
    models).  ``paged=False`` gives the contiguous cache ``[B, Hkv, S_max, D]``
    (one page per sequence, page_size = S_max, no page table).  ``qk_int`` > 0
    draws q and K as integers uniform in [-qk_int, qk_int] (V stays N(0,1)),
    so that dot products and page bounds are exact in fp32.
    """
    g = _gen(seed)
    seq_lens = [int(x) for x in seq_lens]
    assert len(seq_lens) == B
    S_max = max(1, max(seq_lens))
    if qk_int > 0:
        q = torch.randint(-qk_int, qk_int + 1, (B, Hq, D), generator=g).to(dtype)
    else:
        q = _normal(g, (B, Hq, D), dtype)
    k = torch.zeros(B, Hkv, S_max, D, dtype=dtype)
    v = torch.zeros(B, Hkv, S_max, D, dtype=dtype)
    for b, L in enumerate(seq_lens):
        if L == 0:
            continue
        if qk_int > 0:
            kb = torch.randint(-qk_int, qk_int + 1, (Hkv, L, D), generator=g).float()
        else:
            kb = torch.randn(Hkv, L, D, generator=g, dtype=torch.float32)
        if sink_key_scale != 1.0 and n_sink > 0:
            kb[:, : min(n_sink, L)] *= sink_key_scale
        k[b, :, :L] = kb.to(dtype)
        del kb
        v[b, :, :L] = torch.randn(Hkv, L, D, generator=g, dtype=torch.float32).to(dtype)
    if paged:
        kc, vc, pt = _paginate(g, k, v, seq_lens, page_size)
        psz = page_size
    else:
        kc, vc, pt, psz = k, v, None, S_max
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return GQAInputs(q=q, k=k, v=v, seq_lens=torch.tensor(seq_lens, dtype=torch.int32),
                     k_cache=kc, v_cache=vc, page_table=pt, page_size=psz,
                     window=int(window), n_sink=int(n_sink), scale=float(scale), name=name)


@dataclass
class MLAInputs:
    """One decode step of absorbed MLA over a 576-wide latent cache."""
    q: torch.Tensor            # [B, H, d_latent + d_rope] (absorbed query)
    latent: torch.Tensor       # [B, S_max, d_latent + d_rope] = [c_KV | k_pe]
    seq_lens: torch.Tensor     # int32 [B]
    d_latent: int
    d_rope: int
    scale: float
    name: str = ""

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def H(self):
        return self.q.shape[1]

    @property
    def S_max(self):
        return self.latent.shape[1]

    def kv_bytes(self) -> int:
        return int(self.seq_lens.sum()) * self.latent.shape[2] * self.latent.element_size()

    def flops(self) -> int:
        """2 FLOP per multiply-add: scores over d_latent+d_rope, output over d_latent."""
        return int(self.seq_lens.sum()) * 2 * self.H * (self.latent.shape[2] + self.d_latent)


def make_mla(*, B, H, seq_lens, d_latent=512, d_rope=64, dtype=torch.bfloat16,
             scale=None, seed=0, name="") -> MLAInputs:
    g = _gen(seed)
    seq_lens = [int(x) for x in seq_lens]
    S_max = max(1, max(seq_lens))
    Dq = d_latent + d_rope
    q = _normal(g, (B, H, Dq), dtype)
    lat = torch.zeros(B, S_max, Dq, dtype=dtype)
    for b, L in enumerate(seq_lens):
        if L:
            lat[b, :L] = torch.randn(L, Dq, generator=g, dtype=torch.float32).to(dtype)
        if L < S_max:
            lat[b, L:] = TAIL_FILL
    if scale is None:
        # qk head dim of the un-absorbed model: 128 "nope" + 64 RoPE dims
        scale = 1.0 / math.sqrt(192.0)
    return MLAInputs(q=q, latent=lat, seq_lens=torch.tensor(seq_lens, dtype=torch.int32),
                     d_latent=d_latent, d_rope=d_rope, scale=float(scale), name=name)


@dataclass
class DSAInputs:
    """Indexer inputs plus the MLA inputs the selected tokens feed."""
    q_i: torch.Tensor          # [B, Hi, Di] integer-valued
    w: torch.Tensor            # fp32 [B, Hi] integer-valued, positive
    k_i: torch.Tensor          # [B, S_max, Di] integer-valued
    seq_lens: torch.Tensor     # int32 [B]
    topk: int
    mla: MLAInputs
    name: str = ""

    @property
    def B(self):
        return self.q_i.shape[0]

    def indexer_bytes(self) -> int:
        return int(self.seq_lens.sum()) * self.k_i.shape[2] * self.k_i.element_size()

    def indexer_flops(self) -> int:
        return int(self.seq_lens.sum()) * 2 * self.q_i.shape[1] * self.q_i.shape[2]


def make_dsa(*, B, seq_lens, Hi=64, Di=128, topk=2048, H=128, d_latent=512, d_rope=64,
             qk_range=4, w_range=(1, 4), dtype=torch.bfloat16, seed=0, name="") -> DSAInputs:
    g = _gen(seed)
    seq_lens = [int(x) for x in seq_lens]
    S_max = max(1, max(seq_lens))
    q_i = _ints(g, -qk_range, qk_range, (B, Hi, Di), dtype)
    w = _ints(g, w_range[0], w_range[1], (B, Hi), torch.float32)
    k_i = torch.zeros(B, S_max, Di, dtype=dtype)
    for b, L in enumerate(seq_lens):
        if L:
            k_i[b, :L] = _ints(g, -qk_range, qk_range, (L, Di), dtype)
    mla = make_mla(B=B, H=H, seq_lens=seq_lens, d_latent=d_latent, d_rope=d_rope,
                   dtype=dtype, seed=seed + 1000, name=name + "/mla")
    return DSAInputs(q_i=q_i, w=w, k_i=k_i, seq_lens=torch.tensor(seq_lens, dtype=torch.int32),
                     topk=int(topk), mla=mla, name=name)


def make_scores(*, B, seq_lens, n_distinct=None, seed=0) -> torch.Tensor:
    """fp32 scores [B, S_max] for exercising the top-k select alone.

    ``n_distinct`` small forces many ties; negatives, +-0.0 and a spread of
    magnitudes are always present.
    """
    g = _gen(seed)
    S_max = max(1, max(seq_lens))
    if n_distinct is None:
        s = torch.randn(B, S_max, generator=g, dtype=torch.float32) * 100.0
    else:
        s = _ints(g, -(n_distinct // 2), n_distinct - n_distinct // 2 - 1, (B, S_max),
                  torch.float32)
    # sprinkle signed zeros so the select must treat them as equal
    z = torch.rand(B, S_max, generator=g) < 0.02
    sign = torch.rand(B, S_max, generator=g) < 0.5
    s[z & sign] = -0.0
    s[z & ~sign] = 0.0
    return s


def random_topk_indices(*, B, seq_lens, k, seed=0, pad_fraction=0.0) -> torch.Tensor:
    """Ascending distinct token indices [B, k], -1 padded (for sparse MLA alone)."""
    g = _gen(seed)
    out = torch.full((B, k), -1, dtype=torch.int32)
    for b, L in enumerate(seq_lens):
        n = min(k, L)
        n = n - int(n * pad_fraction)
        if n <= 0:
            continue
        sel = torch.randperm(L, generator=g)[:n].sort().values
        out[b, :n] = sel.to(torch.int32)
    return out


# --- the five workloads the library is measured on -------------------------

@dataclass
class Workload:
    key: str
    description: str
    seed: int
    build: object = field(repr=False, default=None)


def config1_tiny_gqa():
    """Tiny GQA, fp32: B2, 4 q heads / 2 KV heads, D64, 256 tokens, contiguous."""
    return make_gqa(B=2, Hq=4, Hkv=2, D=64, seq_lens=[256, 256], dtype=torch.float32,
                    paged=False, seed=1, name="tiny_gqa_fp32_b2_h4_kv2_d64_s256")


def config2_llama3_8b_gqa(B=16, L=8192):
    """Llama-3-8B-shaped layer: B16, 32/8 heads, D128, 8192 tokens, paged P16."""
    return make_gqa(B=B, Hq=32, Hkv=8, D=128, seq_lens=[L] * B, dtype=torch.bfloat16,
                    page_size=16, paged=True, seed=2,
                    name=f"gqa_llama3_8b_layer_bf16_b{B}_s{L}_paged16")


def config3_lens(B=32, lo=4096, hi=32768, seed=3):
    g = _gen(seed)
    return torch.randint(lo, hi + 1, (B,), generator=g).tolist()


def config3_swa_sinks(B=32, lo=4096, hi=32768, window=4096, n_sink=4):
    """Window 4096 + 4 sinks, 32/8 heads, D128, lengths U[4096, 32768], paged P16."""
    lens = config3_lens(B, lo, hi)
    return make_gqa(B=B, Hq=32, Hkv=8, D=128, seq_lens=lens, dtype=torch.bfloat16,
                    page_size=16, paged=True, window=window, n_sink=n_sink,
                    sink_key_scale=4.0, seed=3 + 100,
                    name=f"swa{window}_sinks{n_sink}_bf16_b{B}_s{lo}-{hi}_paged16")


def config4_mla(B=32, L=16384):
    """DeepSeek-V3-shaped MLA decode: B32, 128 heads, 576-wide latent, 16384 tokens."""
    return make_mla(B=B, H=128, seq_lens=[L] * B, seed=4,
                    name=f"mla_dsv3_bf16_b{B}_h128_s{L}")


def config5_dsa(B=8, L=65536, topk=2048):
    """DSA: indexer 64x128 over 65536 tokens, top-2048, then 128-head sparse MLA."""
    return make_dsa(B=B, seq_lens=[L] * B, topk=topk, seed=5,
                    name=f"dsa_bf16_b{B}_s{L}_top{topk}")
