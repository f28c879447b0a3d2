"""Quest query-aware page selection on the GPU against the oracle.

q and K are integer-valued, so the GPU's fp32 bounds equal the oracle's fp64
ones exactly: block summaries and chosen blocks must be bit-exact (ties to the
lower block on both sides); outputs are held to the fp32 / bf16 tolerances.
"""
import pytest
import torch

from decode_attention_kv_flash_amd import api
from decode_attention_kv_flash_amd import workloads as wl
from oracle import quest
from _helpers import assert_lse_close, assert_rows_close, dev, say, tol_for

pytestmark = pytest.mark.gpu


def summaries(x):
    kc = dev(x.k_cache)
    return api.quest_page_minmax(kc, dev(x.seq_lens), dev(x.page_table)), kc


def check_minmax(x):
    kmm, _ = summaries(x)
    torch.cuda.synchronize()
    kmin, kmax = quest.page_minmax(x.k, x.seq_lens)
    got = kmm.cpu().double()
    for b, L in enumerate(x.seq_lens.tolist()):
        nf = L // quest.BLOCK
        assert torch.equal(got[b, :, :nf, 0], kmin[b, :, :nf]), f"kmin b={b}"
        assert torch.equal(got[b, :, :nf, 1], kmax[b, :, :nf]), f"kmax b={b}"


def run_quest(x, budget, num_splits=0):
    kmm, kc = summaries(x)
    out, lse, sel = api.decode_attn_quest(dev(x.q), kc, dev(x.v_cache), kmm, dev(x.seq_lens), budget,
                                          dev(x.page_table), scale=x.scale, num_splits=num_splits,
                                          want_selected=True)
    torch.cuda.synchronize()
    return out.float().cpu().reshape(-1, x.D), lse.cpu().reshape(-1), sel.cpu()


def check_quest(x, budget, num_splits=0):
    say(f"[quest] {x.name} B={x.B} Hq={x.Hq} Hkv={x.Hkv} D={x.D} {x.q.dtype} lens={x.seq_lens.tolist()[:6]} "
        f"budget={budget} splits={num_splits} paged={x.page_table is not None}")
    got, glse, sel = run_quest(x, budget, num_splits)
    (want, wlse), chosen = quest.decode(x.q, x.k, x.v, x.seq_lens, budget, scale=x.scale)
    sel = sel.reshape(x.B * x.Hq, budget)
    for r, c in enumerate(chosen):
        row = sel[r].tolist()
        assert row[: len(c)] == c, f"{x.name}: row {r} chose {row[:len(c)]}, oracle {c}"
        assert all(v == -1 for v in row[len(c):]), f"{x.name}: row {r} padding {row[len(c):]}"
    err = assert_rows_close(got, want, tol_for(x.q.dtype), x.name)
    assert_lse_close(glse, wlse, 1e-5, x.name)
    return err


RAGGED = [0, 5, 16, 17, 250, 1029]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("paged", [True, False])
def test_minmax_bit_exact(dtype, D, paged):
    x = wl.make_gqa(B=6, Hq=8, Hkv=2, D=D, seq_lens=RAGGED, dtype=dtype, page_size=32, paged=paged,
                    seed=81, name="quest_minmax")
    check_minmax(x)


def test_minmax_first_block_leaves_earlier_slots():
    x = wl.make_gqa(B=2, Hq=4, Hkv=2, D=128, seq_lens=[200, 130], dtype=torch.bfloat16, page_size=16,
                    seed=82, name="quest_first_block")
    kc, sl, pt = dev(x.k_cache), dev(x.seq_lens), dev(x.page_table)
    n_blocks = kc.shape[2] * pt.shape[1] // 16
    kmm = torch.full((2, 2, n_blocks, 2, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    api.quest_page_minmax(kc, sl, pt, kminmax=kmm, first_block=5)
    torch.cuda.synchronize()
    kmin, kmax = quest.page_minmax(x.k, x.seq_lens)
    got = kmm.cpu().double()
    assert torch.all(got[:, :, :5] == 7.0)
    for b, L in enumerate([200, 130]):
        nf = L // 16
        assert torch.equal(got[b, :, 5:nf, 0], kmin[b, :, 5:nf])
        assert torch.equal(got[b, :, 5:nf, 1], kmax[b, :, 5:nf])
        assert torch.all(got[b, :, nf:] == 7.0)


@pytest.mark.parametrize("Hq,Hkv,D,dtype,paged", [
    (32, 8, 128, torch.bfloat16, True),
    (8, 8, 64, torch.bfloat16, False),
    (8, 1, 128, torch.float32, True),
    (4, 2, 64, torch.float32, False),
    (16, 2, 128, torch.bfloat16, True),  # eight bf16 heads per KV head: two register buffers per wave
])
@pytest.mark.parametrize("budget", [1, 4, 40])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_quest_ragged(Hq, Hkv, D, dtype, paged, budget, splits):
    x = wl.make_gqa(B=6, Hq=Hq, Hkv=Hkv, D=D, seq_lens=RAGGED, dtype=dtype, page_size=16, paged=paged,
                    qk_int=2, seed=83, name=f"quest_{Hq}_{Hkv}_{D}")
    check_quest(x, budget, splits)


def test_quest_budget_over_every_block_is_full_attention():
    # a budget above every sequence's block count reads the whole cache
    import oracle
    x = wl.make_gqa(B=3, Hq=8, Hkv=2, D=128, seq_lens=[33, 512, 700], dtype=torch.bfloat16, page_size=64,
                    qk_int=2, seed=84, name="quest_all")
    got, glse, _ = run_quest(x, 64)
    want, wlse = oracle.gqa(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    assert_rows_close(got, want, tol_for(x.q.dtype), x.name)
    assert_lse_close(glse, wlse, 1e-5, x.name)


def test_quest_ties_go_to_the_lower_block():
    # identical 16-token blocks everywhere: every bound ties, the lowest blocks win
    x = wl.make_gqa(B=2, Hq=4, Hkv=1, D=64, seq_lens=[160, 101], dtype=torch.float32, page_size=16,
                    qk_int=1, seed=85, name="quest_ties")
    for b in range(2):
        x.k[b, 0] = x.k[b, 0, :16].repeat(x.k.shape[2] // 16 + 1, 1)[: x.k.shape[2]]
    x.k_cache, x.v_cache, x.page_table = _repage(x)
    check_quest(x, 3)


def _repage(x):
    """Re-scatter x.k / x.v into x's page table after editing x.k."""
    kc, vc = x.k_cache.clone(), x.v_cache.clone()
    P = x.page_size
    for b, L in enumerate(x.seq_lens.tolist()):
        for j in range((L + P - 1) // P):
            phys = int(x.page_table[b, j])
            t1 = min((j + 1) * P, L)
            kc[phys, :, : t1 - j * P] = x.k[b, :, j * P: t1]
            vc[phys, :, : t1 - j * P] = x.v[b, :, j * P: t1]
    return kc, vc, x.page_table


def test_quest_llama_shape_sampled_sequences():
    """16 x 8192 tokens, 32 q / 8 KV heads, D128 bf16, pages of 16, budget 128
    blocks (2048 tokens): the full batch on the GPU, three sequences through
    the oracle (each sequence is independent)."""
    x = wl.make_gqa(B=16, Hq=32, Hkv=8, D=128, seq_lens=[8192] * 15 + [8183], dtype=torch.bfloat16,
                    page_size=16, qk_int=2, seed=86, name="quest_llama")
    got, glse, sel = run_quest(x, 128)
    for b in (0, 7, 15):
        (want, wlse), chosen = quest.decode(x.q[b:b + 1], x.k[b:b + 1], x.v[b:b + 1], x.seq_lens[b:b + 1],
                                            128, scale=x.scale)
        rows = slice(b * x.Hq, (b + 1) * x.Hq)
        s = sel.reshape(-1, 128)[rows]
        for h, c in enumerate(chosen):
            assert s[h].tolist() == c, f"b={b} h={h}"
        assert_rows_close(got[rows], want, tol_for(x.q.dtype), f"{x.name} b={b}")
        assert_lse_close(glse[rows], wlse, 1e-5, f"{x.name} b={b}")


def test_quest_per_head_lists_when_the_table_is_wide():
    """Above 8192 blocks per sequence the union bitmaps do not fit: each query
    head then runs its own workgroup over its own list (groups of 4 here)."""
    import torch.nn.functional as F
    x = wl.make_gqa(B=3, Hq=8, Hkv=2, D=128, seq_lens=[300, 17, 1029], dtype=torch.bfloat16, page_size=16,
                    qk_int=2, seed=87, name="quest_wide_table")
    x.page_table = F.pad(x.page_table, (0, 8200 - x.page_table.shape[1]))
    for budget in (3, 40):
        check_quest(x, budget)


def test_quest_union_at_the_bitmap_limit():
    """8192 blocks per sequence, the most the union bitmaps hold: 131067
    tokens, 4 query heads on one KV head, 700 blocks each."""
    x = wl.make_gqa(B=1, Hq=4, Hkv=1, D=64, seq_lens=[131067], dtype=torch.bfloat16, page_size=16,
                    qk_int=2, seed=88, name="quest_bitmap_limit")
    assert x.page_table.shape[1] == 8192
    check_quest(x, 700)
