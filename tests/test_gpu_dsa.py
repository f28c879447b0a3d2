"""DSA indexer, top-k select and sparse MLA on the GPU against the oracle.

Indexer inputs are integer-valued, so scores are exact on both sides and the
selected index sets must match bit for bit (ties to the lower index).
"""
import pytest
import torch

import oracle
from decode_attention_kv_flash_amd import api
from decode_attention_kv_flash_amd import workloads as wl
from _helpers import TOL_BF16, assert_lse_close, assert_rows_close, dev, rows_sample, say

pytestmark = pytest.mark.gpu


def gpu_indexer(x, k):
    idx, scores = api.dsa_indexer_topk(dev(x.q_i), dev(x.w), dev(x.k_i), dev(x.seq_lens), k,
                                       return_scores=True)
    torch.cuda.synchronize()
    return idx.cpu(), scores.cpu()


def check_indexer(x, k):
    say(f"[dsa] indexer B={x.B} Hi={x.q_i.shape[1]} lens={x.seq_lens.tolist()[:4]} k={k}")
    idx, scores = gpu_indexer(x, k)
    want = oracle.indexer(x.q_i, x.w, x.k_i, x.seq_lens)
    for b, L in enumerate(x.seq_lens.tolist()):
        assert torch.equal(scores[b, :L].double(), want[b, :L].double()), f"scores row {b}"
        assert torch.all(torch.isinf(scores[b, L:]))
    want_idx = oracle.topk(want, x.seq_lens, k)
    assert torch.equal(idx, want_idx)
    return idx, want_idx


FP8 = torch.float8_e4m3fn


def check_indexer_fp8(x, k):
    """The indexer with q_i and k_i in fp8 e4m3 (exact for the integer inputs)
    against the oracle on the same fp8 values."""
    say(f"[dsa] indexer fp8 B={x.B} Hi={x.q_i.shape[1]} lens={x.seq_lens.tolist()[:4]} k={k}")
    q8, k8 = x.q_i.to(FP8), x.k_i.to(FP8)
    idx, scores = api.dsa_indexer_topk(dev(q8), dev(x.w), dev(k8), dev(x.seq_lens), k,
                                       return_scores=True)
    torch.cuda.synchronize()
    idx, scores = idx.cpu(), scores.cpu()
    want = oracle.indexer(q8, x.w, k8, x.seq_lens)
    for b, L in enumerate(x.seq_lens.tolist()):
        assert torch.equal(scores[b, :L].double(), want[b, :L].double()), f"fp8 scores row {b}"
        assert torch.all(torch.isinf(scores[b, L:]))
    assert torch.equal(idx, oracle.topk(want, x.seq_lens, k))


@pytest.mark.parametrize("Hi", [32, 64, 96, 128])
def test_indexer_fp8_small(Hi):
    x = wl.make_dsa(B=3, seq_lens=[5, 700, 3001], Hi=Hi, topk=64, H=64, seed=61)
    check_indexer_fp8(x, 64)


@pytest.mark.parametrize("k", [1, 2048, 5000])
def test_indexer_fp8_topk_sizes(k):
    x = wl.make_dsa(B=2, seq_lens=[4096, 2500], topk=k, H=64, seed=62)
    check_indexer_fp8(x, k)


def test_indexer_fp8_hand_worked_example():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "indexer_tiny.json")))
    q = torch.zeros(1, 32, 128, dtype=torch.float32)
    q[0, :2, :3] = torch.tensor(g["q_i"], dtype=torch.float32)
    w = torch.zeros(1, 32)
    w[0, :2] = torch.tensor(g["w"], dtype=torch.float32)
    k = torch.zeros(1, 5, 128, dtype=torch.float32)
    k[0, :, :3] = torch.tensor(g["k_i"], dtype=torch.float32)
    for kk, want in g["topk"].items():
        idx, sc = api.dsa_indexer_topk(dev(q.to(FP8)), dev(w), dev(k.to(FP8)),
                                       dev(torch.tensor([5], dtype=torch.int32)), int(kk), return_scores=True)
        torch.cuda.synchronize()
        assert idx.cpu()[0].tolist() == want
        assert sc.cpu()[0].tolist() == [float(v) for v in g["scores"]]


def test_indexer_fp8_full_size(cfg5):
    """The DSA workload's indexer (B8 x 65536 tokens, 64 heads, top-2048) in fp8."""
    check_indexer_fp8(cfg5, cfg5.topk)


@pytest.mark.parametrize("Hi", [32, 64, 128])
def test_indexer_small(Hi):
    x = wl.make_dsa(B=3, seq_lens=[5, 700, 3001], Hi=Hi, topk=64, H=64, seed=51)
    check_indexer(x, 64)


@pytest.mark.parametrize("k", [1, 16, 2048, 5000])
def test_indexer_topk_sizes(k):
    x = wl.make_dsa(B=2, seq_lens=[4096, 2500], topk=k, H=64, seed=52)
    check_indexer(x, k)


def test_indexer_hand_worked_example():
    """The golden tiny example, padded to the built head width (extra heads weigh 0)."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "indexer_tiny.json")))
    q = torch.zeros(1, 32, 128, dtype=torch.bfloat16)
    q[0, :2, :3] = torch.tensor(g["q_i"], dtype=torch.bfloat16)
    w = torch.zeros(1, 32)
    w[0, :2] = torch.tensor(g["w"], dtype=torch.float32)
    k = torch.zeros(1, 5, 128, dtype=torch.bfloat16)
    k[0, :, :3] = torch.tensor(g["k_i"], dtype=torch.bfloat16)
    for kk, want in g["topk"].items():
        idx, sc = api.dsa_indexer_topk(dev(q), dev(w), dev(k), dev(torch.tensor([5], dtype=torch.int32)),
                                       int(kk), return_scores=True)
        assert sc.cpu()[0].tolist() == g["scores"]
        assert idx.cpu()[0].tolist() == want


@pytest.mark.parametrize("fp8", [False, True])
def test_indexer_hands_the_select_its_first_level(fp8):
    """B x S_max = 4 x 131072 on 256 CUs: every indexer workgroup covers one
    2048-token chunk of the select and counts its scores' top key bytes, so
    the select skips its first launch.  Ragged rows, one shorter than k and
    an empty one; the selection must equal the oracle's select over the same
    scores, and the scores the oracle indexer on the first 4096 tokens."""
    lens = [131072, 1000, 70001, 0]
    x = wl.make_dsa(B=4, seq_lens=lens, Hi=32, topk=2048, H=64, seed=63, name="dsa_first_level")
    say(f"[dsa] indexer + top-k, first level from the indexer, lens={lens} fp8={fp8}")
    q, k = (x.q_i.to(torch.float8_e4m3fn), x.k_i.to(torch.float8_e4m3fn)) if fp8 else (x.q_i, x.k_i)
    idx, sc = api.dsa_indexer_topk(dev(q), dev(x.w), dev(k), dev(x.seq_lens), 2048, return_scores=True)
    torch.cuda.synchronize()
    sc, idx = sc.cpu(), idx.cpu()
    assert torch.equal(idx, oracle.topk(sc, x.seq_lens, 2048))
    head = torch.clamp(x.seq_lens, max=4096)
    want = oracle.indexer(x.q_i, x.w, x.k_i[:, :4096].contiguous(), head)
    for b in range(4):
        n = int(head[b])
        assert torch.equal(sc[b, :n].double(), want[b, :n].double())


def test_indexer_six_rows_of_65536():
    """6 rows: 42 token ranges of 1568 tokens per row (one round of 252
    workgroups; the ranges are not the select's chunks, so the select counts
    its own first level), ragged lengths; scores and selection bit-exact."""
    x = wl.make_dsa(B=6, seq_lens=[65536, 60000, 65536, 1000, 65536, 33333], Hi=64, topk=2048, H=64, seed=64,
                    name="dsa_six_rows")
    check_indexer(x, 2048)


@pytest.mark.parametrize("n_distinct", [None, 3, 50])
@pytest.mark.parametrize("k", [1, 100, 2048])
def test_topk_alone(n_distinct, k):
    lens = [0, 1, 99, 100, 2048, 2049, 65536]
    s = wl.make_scores(B=len(lens), seq_lens=lens, n_distinct=n_distinct, seed=k)
    sl = torch.tensor(lens, dtype=torch.int32)
    got = api.dsa_topk(dev(s), dev(sl), k).cpu()
    want = oracle.topk(s, sl, k)
    assert torch.equal(got, want)


@pytest.mark.parametrize("n_distinct", [None, 1, 2])
@pytest.mark.parametrize("k", [2048, 16384])
def test_topk_long_and_ragged_rows(n_distinct, k):
    """Rows of several 2048-token chunks with a ragged last chunk, longer than
    65536, shorter than k, empty, and all-equal rows (every key ties)."""
    lens = [131073, 70001, 16384, 16385, 2047, 0, 40000]
    say(f"[dsa] topk lens={lens} k={k} n_distinct={n_distinct}")
    s = wl.make_scores(B=len(lens), seq_lens=lens, n_distinct=n_distinct, seed=k + 7)
    sl = torch.tensor(lens, dtype=torch.int32)
    got = api.dsa_topk(dev(s), dev(sl), k).cpu()
    want = oracle.topk(s, sl, k)
    assert torch.equal(got, want)


@pytest.mark.parametrize("n_distinct", [None, 1, 3])
@pytest.mark.parametrize("k", [1, 100, 2047, 2048])
def test_topk_rows_within_one_chunk(n_distinct, k):
    """S_max <= 2048: one workgroup per row runs the whole select in one
    launch; ragged, empty, all-equal and k >= length rows."""
    lens = [0, 1, 99, 100, 1500, 2047, 2048]
    say(f"[dsa] topk one chunk lens={lens} k={k} n_distinct={n_distinct}")
    s = wl.make_scores(B=len(lens), seq_lens=lens, n_distinct=n_distinct, seed=k + 11)
    assert s.shape[1] == 2048
    sl = torch.tensor(lens, dtype=torch.int32)
    got = api.dsa_topk(dev(s), dev(sl), k).cpu()
    want = oracle.topk(s, sl, k)
    assert torch.equal(got, want)


@pytest.mark.parametrize("n_distinct", [None, 1, 3])
@pytest.mark.parametrize("k", [1, 100, 511, 512])
def test_topk_rows_of_512_blocks(n_distinct, k):
    """S_max = 512 (the selection over the 16-token blocks of 8192 tokens, as
    Quest makes it): ragged, empty, all-equal and k >= length rows."""
    lens = [0, 1, 99, 100, 300, 511, 512]
    say(f"[dsa] topk 512 lens={lens} k={k} n_distinct={n_distinct}")
    s = wl.make_scores(B=len(lens), seq_lens=lens, n_distinct=n_distinct, seed=k + 13)
    assert s.shape[1] == 512
    sl = torch.tensor(lens, dtype=torch.int32)
    got = api.dsa_topk(dev(s), dev(sl), k).cpu()
    want = oracle.topk(s, sl, k)
    assert torch.equal(got, want)


def _ordered_scores(order, lens, seed):
    if order == "crowded":
        return wl.make_scores(B=len(lens), seq_lens=lens, n_distinct=3, seed=seed)
    if order == "many_ties":
        return wl.make_scores(B=len(lens), seq_lens=lens, n_distinct=20000, seed=seed)
    s = wl.make_scores(B=len(lens), seq_lens=lens, seed=seed)
    if order in ("ascending", "descending"):
        for b, L in enumerate(lens):
            s[b, :L] = torch.sort(s[b, :L], descending=order == "descending").values
    return s


@pytest.mark.parametrize("order", ["random", "many_ties", "ascending", "descending", "crowded"])
@pytest.mark.parametrize("k", [1, 2048, 8192, 8193])
def test_topk_sorted_and_crowded_rows(order, k):
    """Rows of up to 65536 tokens (32 chunks) in random order with or without
    many ties, sorted either way (the taken keys sit in a few chunks, at the
    start or the end of the row), and with three distinct values; lengths on
    and off chunk boundaries, one more than k, equal to k, and empty."""
    lens = [65536, 65535, 40000, 20481, 16385, 16384, 9000, k + 1, k, 0]
    say(f"[dsa] topk sorted/crowded rows order={order} k={k}")
    s = _ordered_scores(order, lens, seed=k + 17)
    assert s.shape[1] == 65536
    sl = torch.tensor(lens, dtype=torch.int32)
    got = api.dsa_topk(dev(s), dev(sl), k).cpu()
    assert torch.equal(got, oracle.topk(s, sl, k))


def test_topk_ignores_workspace_contents():
    """The workspace holds no state between calls: garbage in it changes nothing."""
    lens = [9000, 20000, 5]
    s = wl.make_scores(B=3, seq_lens=lens, n_distinct=40, seed=3)
    sl = dev(torch.tensor(lens, dtype=torch.int32))
    k = 1000
    nbytes = api.lib().dsa_topk_workspace(3, s.shape[1], k)
    ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")
    out = torch.empty(3, k, dtype=torch.int32, device="cuda")
    api._check(api.lib().dsa_topk(api._ptr(dev(s)), api._ptr(sl), k, api._ptr(out), 3, s.shape[1],
                                  api._ptr(ws), nbytes, None))
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), oracle.topk(s, sl.cpu(), k))


def test_topk_run_to_run_identical():
    s = wl.make_scores(B=4, seq_lens=[30000] * 4, n_distinct=7, seed=9)
    sl = torch.tensor([30000] * 4, dtype=torch.int32)
    a = api.dsa_topk(dev(s), dev(sl), 2048).cpu()
    b = api.dsa_topk(dev(s), dev(sl), 2048).cpu()
    assert torch.equal(a, b)


def run_sparse(m, idx, num_splits=0):
    out, lse = api.sparse_mla_attn(dev(m.q), dev(m.latent), dev(idx), scale=m.scale,
                                   num_splits=num_splits)
    torch.cuda.synchronize()
    return out.float().cpu().reshape(-1, 512), lse.cpu().reshape(-1)


# 3 sequences x 128 heads: up to 85 splits leave CUs idle with 128-head
# workgroups, so the call takes 64-head ones; 96 splits keep 128 heads
@pytest.mark.parametrize("splits", [0, 1, 5, 96])
def test_sparse_mla_random_indices(splits):
    m = wl.make_mla(B=3, H=128, seq_lens=[50, 4000, 3000], seed=53, name="sparse")
    idx = wl.random_topk_indices(B=3, seq_lens=[50, 4000, 3000], k=256, seed=5, pad_fraction=0.1)
    got, glse = run_sparse(m, idx, splits)
    want, wlse = oracle.mla(m.q, m.latent, idx=idx, scale=m.scale)
    assert_rows_close(got, want, TOL_BF16, "sparse")
    assert_lse_close(glse, wlse, 1e-5, "sparse")


@pytest.mark.parametrize("splits", [0, 1])
def test_sparse_mla_empty_lists_and_holes(splits):
    """Empty slots anywhere in the list: a sequence with none selected (zero
    output, lse -inf), holes between selected tokens, and a list whose first
    tiles are all empty."""
    lens = [500, 500, 500, 3000]
    m = wl.make_mla(B=4, H=128, seq_lens=lens, seed=56, name="sparse_holes")
    idx = wl.random_topk_indices(B=4, seq_lens=lens, k=512, seed=57)
    idx[1] = -1
    idx[2, ::3] = -1
    idx[3, :200] = -1
    got, glse = run_sparse(m, idx, splits)
    rows1 = slice(128, 256)
    assert torch.all(got[rows1] == 0)
    assert torch.all(torch.isinf(glse[rows1])) and torch.all(glse[rows1] < 0)
    want, wlse = oracle.mla(m.q, m.latent, idx=idx, scale=m.scale)
    keep = torch.ones(4 * 128, dtype=torch.bool)
    keep[rows1] = False
    assert_rows_close(got[keep], want[keep], TOL_BF16, "sparse holes")
    assert_lse_close(glse[keep], wlse[keep], 1e-5, "sparse holes")


@pytest.mark.parametrize("k_sel", [3840, 3841])
def test_sparse_mla_split_capacity(k_sel):
    """One split asked for k_sel listed rows: 3840 fills a split's row table
    exactly; 3841 is raised to two splits.  A few holes in the list, and the
    list in descending order (order does not matter to the set)."""
    m = wl.make_mla(B=2, H=128, seq_lens=[6000, 5000], seed=58, name="sparse_cap")
    idx = wl.random_topk_indices(B=2, seq_lens=[6000, 5000], k=k_sel, seed=59)
    idx[0, 7::97] = -1
    idx[1] = idx[1].flip(0)
    got, glse = run_sparse(m, idx, 1)
    want, wlse = oracle.mla(m.q, m.latent, idx=idx, scale=m.scale)
    assert_rows_close(got, want, TOL_BF16, f"sparse k={k_sel}")
    assert_lse_close(glse, wlse, 1e-5, f"sparse k={k_sel}")


@pytest.mark.parametrize("k_sel", [2048, 1000])
def test_sparse_mla_128_heads_tile32_holes(k_sel):
    """The automatic plan for 128 heads runs sparse MLA on the 32-row kernel
    (splits of at most 256 positions).  Holes that empty whole 32-row tiles in
    the middle of a split, a split whose only valid row is its last position,
    a split whose first tile has no valid row, repeated rows (counted twice), and a list length that is not a multiple of
    32."""
    lens = [9000, 7000, 3000, 5000]
    m = wl.make_mla(B=4, H=128, seq_lens=lens, seed=64, name="sparse_tile32")
    idx = wl.random_topk_indices(B=4, seq_lens=lens, k=k_sel, seed=65)
    idx[0, 32:96] = -1          # two whole tiles
    idx[1, 64:127] = -1         # all but the last position of a 64-position split
    idx[1, 256:300] = -1        # a split whose first tile has no row (splits of 128 or 256)
    idx[1, 384:420] = -1        # the same for splits of 96, 128 or 192 positions
    idx[2, 5::7] = -1           # scattered holes
    idx[3, 10:20] = idx[3, 100:110]  # repeated rows
    got, glse = run_sparse(m, idx, 0)
    want, wlse = oracle.mla(m.q, m.latent, idx=idx, scale=m.scale)
    assert_rows_close(got, want, TOL_BF16, f"sparse tile32 k={k_sel}")
    assert_lse_close(glse, wlse, 1e-5, f"sparse tile32 k={k_sel}")


def test_sparse_with_all_tokens_equals_dense():
    m = wl.make_mla(B=2, H=64, seq_lens=[256, 256], seed=54)
    idx = torch.arange(256, dtype=torch.int32).repeat(2, 1)
    sp, _ = run_sparse(m, idx, 2)
    de, _ = api.decode_attn_mla(dev(m.q), dev(m.latent), dev(m.seq_lens), scale=m.scale, num_splits=2)
    assert oracle.rel_err_rows(sp, de.float().cpu().reshape(-1, 512)) <= 1e-6


@pytest.fixture(scope="module")
def cfg5():
    say("[dsa] generating DSA decode: B8, 65536 tokens, indexer 64x128, top-2048, 128-head MLA")
    return wl.config5_dsa()


def test_config5_full_pipeline(cfg5):
    x = cfg5
    idx, want_idx = check_indexer(x, x.topk)
    m = x.mla
    got, glse = run_sparse(m, dev(idx))
    rows = rows_sample(m.B * m.H, 48, seed=5)
    want, wlse = oracle.mla(m.q, m.latent, idx=want_idx, scale=m.scale, rows=rows)
    assert_rows_close(got[rows], want, TOL_BF16, "config5 sparse")
    assert_lse_close(glse[rows], wlse, 1e-5, "config5 sparse")
