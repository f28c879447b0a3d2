"""Cache append on the GPU (kv_append_gqa / kv_append_rows) against the
oracle's logical-order append, bit-exact, and the rolling buffer of a sliding
window: attention through the recycled page table against the oracle over the
whole logical cache."""
import math

import pytest
import torch

import oracle
from oracle import cache as ocache
from decode_attention_kv_flash_amd import api
from decode_attention_kv_flash_amd import workloads as wl
from _helpers import assert_rows_close, dev, say, tol_for

pytestmark = pytest.mark.gpu


def unfold(cache, page_table, S):
    """Physical paged cache [pages, H, P, X] (or [pages, P, X]) -> logical [B, H, S, X] ([B, S, X])."""
    P = cache.shape[-2]
    t = torch.arange(S)
    phys = page_table[:, t // P].long()  # [B, S]
    if cache.dim() == 4:
        return cache[phys, :, t % P].permute(0, 2, 1, 3)
    return cache[phys, t % P]


@pytest.mark.parametrize("dtype,D,paged", [
    (torch.bfloat16, 128, True),
    (torch.bfloat16, 64, False),
    (torch.float32, 128, True),
    (torch.float32, 64, False),
])
def test_append_gqa_matches_oracle(dtype, D, paged):
    B, Hkv, cap = 5, 8, 100
    x = wl.make_gqa(B=B, Hq=Hkv, Hkv=Hkv, D=D, seq_lens=[cap] * B, dtype=dtype, page_size=16,
                    paged=paged, seed=41, name="append")
    g = torch.Generator().manual_seed(42)
    k_new = torch.randn(B, Hkv, D, generator=g).to(dtype)
    v_new = torch.randn(B, Hkv, D, generator=g).to(dtype)
    pos = torch.tensor([0, 17, 99, -1, 64], dtype=torch.int32)  # -1: no append for sequence 3
    say(f"[append] gqa dtype={dtype} D={D} paged={paged} positions={pos.tolist()}")
    kc, vc = dev(x.k_cache), dev(x.v_cache)
    api.kv_append_gqa(dev(k_new), dev(v_new), kc, vc, dev(pos), dev(x.page_table))
    torch.cuda.synchronize()
    want_k = ocache.append(x.k, pos, k_new)
    want_v = ocache.append(x.v, pos, v_new)
    if paged:
        got_k, got_v = unfold(kc.cpu(), x.page_table, cap), unfold(vc.cpu(), x.page_table, cap)
    else:
        got_k, got_v = kc.cpu(), vc.cpu()
    assert torch.equal(got_k, want_k) and torch.equal(got_v, want_v)
    # nothing else in the physical cache changed
    changed = (kc.cpu() != x.k_cache).sum().item() + (vc.cpu() != x.v_cache).sum().item()
    assert changed <= 2 * 4 * Hkv * D


@pytest.mark.parametrize("row,paged", [(576, True), (576, False), (128, True), (128, False)])
def test_append_rows_matches_oracle(row, paged):
    """MLA latent rows (576 = 512 + 64) and indexer keys (128)."""
    B, cap, P = 4, 70, 16
    g = torch.Generator().manual_seed(43)
    logical = torch.randn(B, cap, row, generator=g).to(torch.bfloat16)
    new = torch.randn(B, row, generator=g).to(torch.bfloat16)
    pos = torch.tensor([69, 0, 33, 16], dtype=torch.int32)
    say(f"[append] rows row={row} paged={paged}")
    if paged:
        n_pages = B * math.ceil(cap / P)
        perm = torch.randperm(n_pages, generator=g)
        pt = perm.view(B, -1).to(torch.int32)
        phys = torch.zeros(n_pages, P, row, dtype=torch.bfloat16)
        for b in range(B):
            for t in range(cap):
                phys[pt[b, t // P], t % P] = logical[b, t]
        c = dev(phys)
        api.kv_append_rows(dev(new), c, dev(pos), dev(pt))
        torch.cuda.synchronize()
        got = unfold(c.cpu(), pt, cap)
    else:
        c = dev(logical)
        api.kv_append_rows(dev(new), c, dev(pos))
        torch.cuda.synchronize()
        got = c.cpu()
    want = ocache.append(logical, pos, new)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_positions_past_the_cache_are_skipped():
    B, Hkv, D = 2, 2, 64
    x = wl.make_gqa(B=B, Hq=Hkv, Hkv=Hkv, D=D, seq_lens=[32, 32], page_size=16, paged=True, seed=44)
    kc, vc = dev(x.k_cache), dev(x.v_cache)
    new = torch.ones(B, Hkv, D, dtype=torch.bfloat16)
    api.kv_append_gqa(dev(new), dev(new), kc, vc, dev(torch.tensor([32, 1000], dtype=torch.int32)),
                      dev(x.page_table))
    torch.cuda.synchronize()
    assert torch.equal(kc.cpu(), x.k_cache) and torch.equal(vc.cpu(), x.v_cache)


@pytest.mark.parametrize("window,n_sink,P", [(64, 4, 16), (100, 4, 16), (48, 0, 8)])
def test_rolling_buffer_window_attention(window, n_sink, P):
    """Token by token: append into a rolling buffer of fixed_pages + ring_pages
    physical pages per sequence, then attend with the window and sinks through
    the recycled page table; the result equals the oracle's window attention
    over the whole logical cache."""
    B, Hq, Hkv, D, T = 2, 8, 2, 64, 400
    fixed = math.ceil(n_sink / P)
    ring = math.ceil((window - 1) / P) + 1
    per_seq = fixed + ring
    max_pages = math.ceil(T / P)
    g = torch.Generator().manual_seed(45)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    k_log = torch.randn(B, Hkv, T, D, generator=g).to(torch.bfloat16)
    v_log = torch.randn(B, Hkv, T, D, generator=g).to(torch.bfloat16)
    phys_pages = B * per_seq
    kc = dev(torch.full((phys_pages, Hkv, P, D), 7.0, dtype=torch.bfloat16))
    vc = dev(torch.full((phys_pages, Hkv, P, D), 7.0, dtype=torch.bfloat16))
    pt = torch.full((B, max_pages), -1, dtype=torch.int32)
    perm = torch.randperm(phys_pages, generator=g).view(B, per_seq)
    pt[:, :per_seq] = perm.to(torch.int32)  # sink pages, then the ring; the rest is recycled
    pt_d = dev(pt)
    say(f"[append] rolling window={window} sinks={n_sink} P={P} ring={ring} fixed={fixed}")
    checks = 0
    for t in range(T):
        pos = dev(torch.full((B,), t, dtype=torch.int32))
        api.kv_append_gqa(dev(k_log[:, :, t].contiguous()), dev(v_log[:, :, t].contiguous()), kc, vc,
                          pos, pt_d, ring_pages=ring, fixed_pages=fixed)
        if t % 37 == 36 or t == T - 1:
            L = torch.full((B,), t + 1, dtype=torch.int32)
            out, _ = api.decode_attn_gqa(dev(q), kc, vc, dev(L), pt_d, window, n_sink, num_splits=0)
            torch.cuda.synchronize()
            want, _ = oracle.gqa(q, k_log[:, :, : t + 1].contiguous(), v_log[:, :, : t + 1].contiguous(),
                                 L, window=window, n_sink=n_sink)
            assert_rows_close(out.float().cpu().reshape(-1, D), want, tol_for(torch.bfloat16),
                              f"rolling t={t}")
            checks += 1
    assert checks >= 10
    # the table only ever names the sequence's own physical pages
    used = pt_d.cpu()[:, : math.ceil(T / P)]
    for b in range(B):
        assert set(used[b].tolist()) <= set(perm[b].tolist())
