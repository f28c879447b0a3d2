"""Absorbed MLA decode attention on the GPU against the oracle."""
import pytest
import torch

import oracle
from decode_attention_kv_flash_amd import api
from decode_attention_kv_flash_amd import workloads as wl
from _helpers import TOL_BF16, assert_lse_close, assert_rows_close, dev, rows_sample, say

pytestmark = pytest.mark.gpu


def run_gpu(x, num_splits=0, page_table=None, latent=None):
    out, lse = api.decode_attn_mla(dev(x.q), dev(latent if latent is not None else x.latent),
                                   dev(x.seq_lens), dev(page_table), scale=x.scale,
                                   num_splits=num_splits)
    torch.cuda.synchronize()
    return out.float().cpu().reshape(-1, 512), lse.cpu().reshape(-1)


def check(x, num_splits=0, rows=None, **kw):
    say(f"[mla] {x.name} B={x.B} H={x.H} lens={x.seq_lens.tolist()[:6]} splits={num_splits}")
    got, glse = run_gpu(x, num_splits, **kw)
    want, wlse = oracle.mla(x.q, x.latent, x.seq_lens, scale=x.scale, rows=rows)
    if rows is not None:
        got, glse = got[rows], glse[rows]
    assert_rows_close(got, want, TOL_BF16, x.name)
    assert_lse_close(glse, wlse, 1e-5, x.name)


@pytest.mark.parametrize("splits", [0, 1, 3, 8])
def test_mla_ragged(splits):
    x = wl.make_mla(B=3, H=128, seq_lens=[1, 33, 517], seed=41, name="mla_ragged")
    check(x, splits)


def test_mla_64_heads_and_long():
    x = wl.make_mla(B=2, H=64, seq_lens=[2048, 4000], seed=42, name="mla_h64")
    check(x)


def test_mla_empty_sequence():
    x = wl.make_mla(B=2, H=64, seq_lens=[0, 40], seed=43, name="mla_empty")
    got, lse = run_gpu(x)
    assert torch.all(got[:64] == 0)
    assert torch.all(torch.isinf(lse[:64]))
    check(x)


def test_mla_paged_equals_contiguous():
    x = wl.make_mla(B=2, H=64, seq_lens=[300, 129], seed=44, name="mla_paged")
    P = 16
    n_pages = [(L + P - 1) // P for L in x.seq_lens.tolist()]
    total = sum(n_pages)
    g = torch.Generator().manual_seed(0)
    perm = torch.randperm(total, generator=g)
    pt = torch.zeros(2, max(n_pages), dtype=torch.int32)
    cache = torch.zeros(total, P, 576, dtype=torch.bfloat16)
    off = 0
    for b, L in enumerate(x.seq_lens.tolist()):
        for j in range(n_pages[b]):
            phys = int(perm[off + j])
            pt[b, j] = phys
            t0, t1 = j * P, min(L, (j + 1) * P)
            cache[phys, : t1 - t0] = x.latent[b, t0:t1]
        off += n_pages[b]
    cont, _ = run_gpu(x, 2)
    paged, _ = run_gpu(x, 2, page_table=pt, latent=cache)
    assert torch.equal(cont, paged)
    check(x, 2, page_table=pt, latent=cache)


def _paged(x, P, seed):
    """x's latent rows scattered over shuffled pages of P rows (two spare
    pages, never referenced, at random places in the pool)."""
    lens = x.seq_lens.tolist()
    n_pages = [(L + P - 1) // P for L in lens]
    total = sum(n_pages) + 2
    perm = torch.randperm(total, generator=torch.Generator().manual_seed(seed))
    pt = torch.zeros(x.B, max(max(n_pages), 1), dtype=torch.int32)
    cache = torch.full((total, P, 576), 3.0, dtype=torch.bfloat16)
    off = 0
    for b, L in enumerate(lens):
        for j in range(n_pages[b]):
            phys = int(perm[off + j])
            pt[b, j] = phys
            t0, t1 = j * P, min(L, (j + 1) * P)
            cache[phys, : t1 - t0] = x.latent[b, t0:t1]
        off += n_pages[b]
    return pt, cache


@pytest.mark.parametrize("P", [4, 8, 16, 64, 256])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_mla_paged_128_heads(P, splits):
    """128 heads over pages of P rows: pages of 8 or more rows run the 32-row
    kernel, whose paged tiles must match its contiguous ones bit for bit;
    pages of 4 rows, and 2000 tokens in one split of 8-row pages (250 pages),
    take the 64-row kernel."""
    x = wl.make_mla(B=5, H=128, seq_lens=[1, 33, 517, 2000, 0], seed=46, name=f"mla_paged_p{P}")
    pt, cache = _paged(x, P, seed=P)
    check(x, splits, page_table=pt, latent=cache)
    # explicit splits: the 32-row kernel takes the call when a split spans at
    # most 126 pages (its 32-row multiple of cache positions, plus two)
    per = -(-(-(-P * pt.shape[1] // max(splits, 1)) // 32)) * 32
    if P >= 8 and splits > 0 and per // P + 2 <= 128:
        cont, clse = run_gpu(x, splits)
        paged, plse = run_gpu(x, splits, page_table=pt, latent=cache)
        assert torch.equal(cont, paged)
        assert torch.equal(clse, plse)


@pytest.mark.parametrize("H", [192, 256])
def test_mla_several_head_blocks(H):
    """More heads than one workgroup holds: 256 heads run as two 128-head
    blocks on the 32-row kernel, 192 as three 64-head blocks on the 16-row
    one; contiguous, paged and sparse."""
    x = wl.make_mla(B=3, H=H, seq_lens=[700, 1, 2100], seed=47, name=f"mla_h{H}")
    for splits in (0, 3):
        check(x, splits)
    pt, cache = _paged(x, 16, seed=47)
    check(x, 0, page_table=pt, latent=cache)
    idx = wl.random_topk_indices(B=3, seq_lens=x.seq_lens.tolist(), k=512, seed=48)
    got, glse = api.sparse_mla_attn(dev(x.q), dev(x.latent), dev(idx), scale=x.scale)
    torch.cuda.synchronize()
    want, wlse = oracle.mla(x.q, x.latent, idx=idx, scale=x.scale)
    assert_rows_close(got.float().cpu().reshape(-1, 512), want, TOL_BF16, f"{x.name} sparse")
    assert_lse_close(glse.cpu().reshape(-1), wlse, 1e-5, f"{x.name} sparse")


@pytest.fixture(scope="module")
def cfg4():
    say("[mla] generating DeepSeek-V3-shaped MLA decode: B32 H128 576-wide latent 16384 tokens")
    return wl.config4_mla()


def test_config4_full_size_sampled(cfg4):
    x = cfg4
    rows = rows_sample(x.B * x.H, 48, seed=4)
    check(x, 0, rows=rows)


# --- balanced splits: the library's own plan for 128-head calls cuts every
# sequence into items of about equal token counts (at most 3840 each)

@pytest.mark.parametrize("P", [0, 32, 64, 256])
def test_mla_balanced_items_on_skewed_lengths(P):
    """One long sequence among short and empty ones: contiguous, balanced
    items (the long one takes many, the short ones one each, the empty one
    none); paged with 32-, 64- and 256-row pages, equal splits per
    sequence; sampled rows of every sequence."""
    lens = [40000, 1, 0, 5000, 33, 2047, 320, 321]
    x = wl.make_mla(B=len(lens), H=128, seq_lens=lens, seed=49, name=f"mla_skew_p{P}")
    rows = sorted(set(rows_sample(x.B * x.H, 40, seed=7) + [128 * b + 5 for b in range(x.B)]))
    if P == 0:
        check(x, 0, rows=rows)
    else:
        pt, cache = _paged(x, P, seed=P)
        check(x, 0, rows=rows, page_table=pt, latent=cache)
    got, lse = run_gpu(x)
    assert torch.all(got[256:384] == 0) and torch.all(torch.isinf(lse[256:384]))  # the empty sequence


def test_mla_balanced_items_all_empty_and_many_sequences():
    """Every sequence empty (no item at all: the combine writes zeros and
    -inf); 300 short sequences (one item each, more items than CUs); and 513
    sequences, past the balanced plan's 512, on the split grid."""
    x = wl.make_mla(B=4, H=128, seq_lens=[0, 0, 0, 0], seed=50, name="mla_all_empty")
    got, lse = run_gpu(x)
    assert torch.all(got == 0) and torch.all(torch.isinf(lse))
    for B in (300, 513):
        g = torch.Generator().manual_seed(B)
        lens = torch.randint(0, 60, (B,), generator=g).tolist()
        x = wl.make_mla(B=B, H=128, seq_lens=lens, seed=51, name=f"mla_{B}_short")
        check(x, 0, rows=rows_sample(x.B * x.H, 48, seed=B))


def test_mla_balanced_items_without_lse_and_reused_workspace():
    """A balanced call without lse writes the same output; a workspace reused
    by a call with other lengths (a different item table) holds no state."""
    x = wl.make_mla(B=5, H=128, seq_lens=[9000, 5, 0, 3000, 700], seed=53, name="mla_nolse")
    y = wl.make_mla(B=5, H=128, seq_lens=[100, 9000, 4000, 0, 1], seed=54, name="mla_nolse2")
    nbytes = api.lib().decode_attn_mla_workspace(5, 128, 512, max(x.S_max, y.S_max), 0)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda")
    for m in (x, y):
        ref, _ = api.decode_attn_mla(dev(m.q), dev(m.latent), dev(m.seq_lens), scale=m.scale, workspace=ws)
        got, lse = api.decode_attn_mla(dev(m.q), dev(m.latent), dev(m.seq_lens), scale=m.scale, want_lse=False,
                                       workspace=ws)
        torch.cuda.synchronize()
        assert lse is None and torch.equal(got, ref)
        want, _ = oracle.mla(m.q, m.latent, m.seq_lens, scale=m.scale)
        assert_rows_close(got.float().cpu().reshape(-1, 512), want, TOL_BF16, m.name)


def test_mla_balanced_items_in_several_rounds():
    """512 sequences (the balanced plan's limit) of up to 4000 tokens: items
    are capped at 3840 tokens, so there are about four items per CU and the
    grid runs several rounds; sampled rows against the oracle."""
    g = torch.Generator().manual_seed(512)
    lens = torch.randint(3000, 4001, (512,), generator=g).tolist()
    lens[7], lens[300] = 3840, 3841  # one item exactly, and one token over
    x = wl.make_mla(B=512, H=128, seq_lens=lens, seed=52, name="mla_512_rounds")
    check(x, 0, rows=sorted(set(rows_sample(x.B * x.H, 40, seed=9) + [7 * 128 + 3, 300 * 128 + 100])))


@pytest.mark.parametrize("splits", [0, 35])
def test_mla_long_context_sampled(splits):
    """Sequences of 131072 and 100000 tokens: the automatic plan (many splits
    per sequence for two sequences), and the fewest splits the 3840-token
    split capacity allows (35), on sampled rows."""
    x = wl.make_mla(B=2, H=128, seq_lens=[131072, 100000], seed=48, name="mla_long")
    check(x, splits, rows=rows_sample(x.B * x.H, 16, seed=5))


def test_mla_score_jumps_restart_the_split():
    """Scores far above the first ones of a split (more than 2^64 apart in
    exp2 units): rows whose latent is a multiple of one head's query."""
    x = wl.make_mla(B=2, H=128, seq_lens=[3000, 700], seed=45, name="mla_spikes")
    q = x.q.float()
    x.latent[0, 100] = (1.5 * q[0, 0]).to(torch.bfloat16)    # ~60 nats above the rest
    x.latent[0, 1500] = (3.0 * q[0, 0]).to(torch.bfloat16)   # ~60 nats above that
    x.latent[1, 650] = (2.0 * q[1, 70]).to(torch.bfloat16)
    for splits in (1, 0):
        check(x, splits)
    # the same jumps read through 16-row pages, and through a sparse list of
    # every row (the 32-row kernel's paged and sparse tiles)
    pt, cache = _paged(x, 16, seed=45)
    for splits in (1, 3):
        check(x, splits, page_table=pt, latent=cache)
    idx = torch.stack([torch.arange(x.S_max, dtype=torch.int32)] * x.B)
    idx[1, 700:] = -1
    got, glse = api.sparse_mla_attn(dev(x.q), dev(x.latent), dev(idx), scale=x.scale)
    torch.cuda.synchronize()
    want, wlse = oracle.mla(x.q, x.latent, x.seq_lens, scale=x.scale)
    assert_rows_close(got.float().cpu().reshape(-1, 512), want, TOL_BF16, "mla_spikes sparse")
    assert_lse_close(glse.cpu().reshape(-1), wlse, 1e-5, "mla_spikes sparse")


# A split holds at most 3840 tokens (120 tiles of 32 in its LDS row table).
SPLIT_CAP = 3840


@pytest.mark.parametrize("H", [64, 128])
@pytest.mark.parametrize("lens,splits", [
    ([31, 32, 96, 97, SPLIT_CAP], 1),   # one split holds exactly the capacity: a full row table
    ([31, 32, 96, 97, SPLIT_CAP], 0),
    ([33, SPLIT_CAP + 1], 1),           # one token past it: the request for one split is raised to two
    ([SPLIT_CAP + 1], 0),
])
def test_mla_tile_and_split_capacity_boundaries(H, lens, splits):
    """Lengths at a 32-token tile and at the split capacity.  S_max is the
    longest length, so with splits=1 the first case runs one split of
    exactly 3840 tokens (n_tiles at its maximum) and the third is raised to
    two splits."""
    x = wl.make_mla(B=len(lens), H=H, seq_lens=lens, seed=46, name=f"mla_bounds_h{H}")
    assert x.S_max == max(lens)
    check(x, splits)
