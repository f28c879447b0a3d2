"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formula: each compares it with something
independent -- numbers the pages print, closed forms, a library routine
(torch's fp64 scaled_dot_product_attention), a different construction of the
same set (StreamingLLM's keep list), the un-absorbed MLA, or invariants that
characterise the result.
"""
import json
import math
import os
import random

import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import accounting as acc
from decode_attention_kv_flash_amd import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# accounting against the pages' printed numbers


def test_kv_bytes_per_token_llama3_8b():
    g = gold("page_numbers.json")["kv_bytes_per_token_llama3_8b"]
    assert acc.kv_cache_bytes(1, **g["shape"]) == g["value"]


def test_mla_values_per_token():
    g = gold("page_numbers.json")["mla_values_per_token"]
    assert acc.mla_values_per_token(**g["shape"]) == g["value"]


def test_mha_to_gqa_at_8k():
    g = gold("page_numbers.json")["mha_to_gqa_cache_8k"]
    s = g["shape"]
    mha = acc.kv_cache_bytes(s["S"], s["n_layers"], s["n_heads"], s["d_head"], s["n_bytes"])
    gqa = acc.kv_cache_bytes(s["S"], s["n_layers"], s["n_kv_heads"], s["d_head"], s["n_bytes"])
    assert mha / 2**30 == g["value_gb"][0]
    assert gqa / 2**30 == g["value_gb"][1]


def test_mistral_window_cache():
    g = gold("page_numbers.json")["mistral_swa_cache_32k"]
    s = g["shape"]
    full = acc.kv_cache_bytes(s["S"], s["n_layers"], s["n_kv_heads"], s["d_head"], s["n_bytes"])
    win = acc.kv_cache_bytes(s["W"], s["n_layers"], s["n_kv_heads"], s["d_head"], s["n_bytes"])
    assert round(full / 1e9) == g["value"]["full_gb"]
    assert win / 2**20 == g["value"]["window_mb"]


def test_crossover_and_128k_cache():
    g = gold("page_numbers.json")["crossover"]
    for name in ("Qwen2.5-7B", "LLaMA-3-70B"):
        m = g[name]
        c = acc.attention_linear_crossover(m["params"], m["layers"], m["heads"], m["head_dim"])
        assert round(c / 1000) == m["crossover_k"]
        kv = acc.kv_cache_bytes(131072, m["layers"], m["kv_heads"], m["head_dim"], 2)
        assert round(kv / 1e9, 1) == m["kv_128k_gb"]


def test_attention_flops_counts_a_naive_decode():
    # brute force: run one decode step with plain loops on tiny sizes and
    # count each multiply and each add of QK^T and PV (the page counts
    # those two products, not the softmax)
    S, nh, dh = 5, 3, 4
    g = torch.Generator().manual_seed(0)
    q, k, v = (torch.randn(*shape, generator=g).tolist()
               for shape in ((nh, dh), (nh, S, dh), (nh, S, dh)))
    n = 0
    for h in range(nh):
        s = []
        for t in range(S):
            acc_ = 0.0
            for d in range(dh):
                acc_ += q[h][d] * k[h][t][d]
                n += 2
            s.append(acc_)
        m = max(s)
        p = [math.exp(x - m) for x in s]
        o = [0.0] * dh
        for t in range(S):
            for d in range(dh):
                o[d] += p[t] * v[h][t][d]
                n += 2
    assert acc.attention_flops(S, nh, dh) == n


def test_dsa_selected_cache_per_layer():
    g = gold("page_numbers.json")["dsa_selected_cache_per_layer"]
    s, v = g["shape"], g["value_decimal_mb"]
    gqa = acc.kv_cache_bytes(s["S_sel"], 1, s["gqa_kv_heads"], s["d_head"], s["n_bytes"])
    mla = acc.mla_cache_bytes(s["S_sel"], s["d_latent"], s["d_rope"], s["n_bytes"])
    wts = acc.mla_kv_up_projection_bytes(s["d_latent"], s["mla_heads"], s["d_nope"], s["d_v"],
                                         s["n_bytes"])
    assert round(gqa / 1e6, 2) == v["gqa_per_bsz"]
    assert round(mla / 1e6, 2) == v["mla_per_bsz"]
    assert round(wts / 1e6, 1) == v["mla_weights"]


def test_mla_equals_gqa_with_225_groups():
    assert acc.mla_over_gqa_groups(128) == gold("page_numbers.json")["mla_equiv_gqa_groups"]["value"]


# --------------------------------------------------------------------------
# attention: closed forms and brute force on tiny inputs


def _tiny(B=1, Hq=1, Hkv=1, D=4, L=3, seed=0, dtype=torch.float32):
    return wl.make_gqa(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_lens=[L] * B, dtype=dtype,
                       paged=False, seed=seed)


def test_single_token_returns_its_value():
    x = _tiny(L=1)
    out, lse = oracle.gqa(x.q, x.k, x.v, x.seq_lens)
    assert torch.equal(out[0], x.v[0, 0, 0].double())
    s0 = float((x.q[0, 0].double() * x.k[0, 0, 0].double()).sum()) * x.scale
    assert lse[0].item() == pytest.approx(s0, abs=1e-14)


def test_two_tokens_sigmoid():
    x = _tiny(L=2, D=8, seed=3)
    out, _ = oracle.gqa(x.q, x.k, x.v, x.seq_lens)
    q, k, v = x.q[0, 0].double(), x.k[0, 0].double(), x.v[0, 0].double()
    s0, s1 = float(q @ k[0]) * x.scale, float(q @ k[1]) * x.scale
    a = 1.0 / (1.0 + math.exp(s1 - s0))
    want = a * v[0] + (1 - a) * v[1]
    assert torch.allclose(out[0], want, rtol=0, atol=1e-14)


def test_equal_keys_average_values_and_lse_is_log_count():
    x = _tiny(L=37, D=16, seed=5)
    x.k.zero_()
    out, lse = oracle.gqa(x.q, x.k, x.v, x.seq_lens)
    assert torch.allclose(out[0], x.v[0, 0, :37].double().mean(0), rtol=0, atol=1e-14)
    assert lse[0].item() == pytest.approx(math.log(37), abs=1e-14)


def test_dominant_score_picks_its_value():
    x = _tiny(L=9, D=4, seed=7)
    x.q[0, 0] = torch.tensor([1.0, 0, 0, 0])
    x.k[0, 0] = 0.0
    x.k[0, 0, 5, 0] = 200.0  # score 100 after scale 1/2
    out, _ = oracle.gqa(x.q, x.k, x.v, x.seq_lens)
    assert torch.allclose(out[0], x.v[0, 0, 5].double(), atol=1e-30)


def test_empty_sequence_gives_zeros_and_minus_inf():
    x = wl.make_gqa(B=2, Hq=2, Hkv=1, D=8, seq_lens=[0, 5], dtype=torch.float32,
                    paged=False, seed=1)
    out, lse = oracle.gqa(x.q, x.k, x.v, x.seq_lens)
    assert torch.all(out[:2] == 0) and torch.all(torch.isinf(lse[:2])) and torch.all(lse[:2] < 0)
    assert torch.all(torch.isfinite(lse[2:]))


# --------------------------------------------------------------------------
# explicit sink logit: one more softmax-denominator term with a zero value


def test_sink_single_token_sigmoid():
    # one token and a sink logit c: o = sigmoid(s0 - c) v0, lse = log(e^s0 + e^c)
    x = _tiny(L=1, D=8, seed=4)
    c = 0.37
    out, lse = oracle.gqa(x.q, x.k, x.v, x.seq_lens, sink_logits=[c])
    s0 = float((x.q[0, 0].double() * x.k[0, 0, 0].double()).sum()) * x.scale
    a = 1.0 / (1.0 + math.exp(c - s0))
    assert torch.allclose(out[0], a * x.v[0, 0, 0].double(), rtol=0, atol=1e-14)
    assert lse[0].item() == pytest.approx(math.log(math.exp(s0) + math.exp(c)), abs=1e-13)


def test_sink_on_empty_sequence():
    # no token: the output is zero and the denominator is the sink term alone
    x = wl.make_gqa(B=1, Hq=2, Hkv=1, D=8, seq_lens=[0], dtype=torch.float32, paged=False, seed=2)
    out, lse = oracle.gqa(x.q, x.k, x.v, x.seq_lens, sink_logits=[-1.5, 2.0])
    assert torch.all(out == 0)
    assert lse.tolist() == [-1.5, 2.0]


def test_very_negative_sink_equals_no_sink():
    # e^{sink} with sink = -1e4 underflows to zero next to any score here, so
    # the extra denominator term vanishes and the result is plain attention
    x = wl.make_gqa(B=2, Hq=4, Hkv=2, D=16, seq_lens=[1, 37], dtype=torch.float32, paged=False, seed=19)
    out, lse = oracle.gqa(x.q, x.k, x.v, x.seq_lens, sink_logits=[-1e4] * 4)
    want, wlse = oracle.gqa(x.q, x.k, x.v, x.seq_lens)
    assert torch.equal(out, want) and torch.equal(lse, wlse)


def _sdpa_with_sink_token(q, k, v, scale, L, sink, keep=None):
    """Library attention over the cache plus one token whose key and value are
    zero vectors and whose logit is raised by the head's sink (an additive
    mask); q [Hq, D], k/v [Hkv, S, D] (fp64)."""
    Hq, Hkv, D = q.shape[0], k.shape[0], q.shape[1]
    kk = k[:, :L] if keep is None else k[:, keep]
    vv = v[:, :L] if keep is None else v[:, keep]
    n = kk.shape[1]
    kk = torch.cat([kk, torch.zeros(Hkv, 1, D, dtype=kk.dtype)], dim=1).repeat_interleave(Hq // Hkv, 0)
    vv = torch.cat([vv, torch.zeros(Hkv, 1, D, dtype=vv.dtype)], dim=1).repeat_interleave(Hq // Hkv, 0)
    bias = torch.zeros(Hq, 1, n + 1, dtype=q.dtype)
    bias[:, 0, n] = torch.as_tensor(sink, dtype=q.dtype)
    return F.scaled_dot_product_attention(q[:, None, :], kk, vv, attn_mask=bias, scale=scale)[:, 0, :]


def test_zero_sink_equals_library_attention_with_a_zero_token():
    # softmax-off-by-one: a sink logit of 0 is a token whose key and value are zero
    lens = [1, 9, 150]
    x = wl.make_gqa(B=3, Hq=4, Hkv=2, D=32, seq_lens=lens, dtype=torch.float32, paged=False, seed=21)
    out, _ = oracle.gqa(x.q, x.k, x.v, x.seq_lens, sink_logits=[0.0] * 4)
    out = out.view(3, 4, 32)
    for b, L in enumerate(lens):
        want = _sdpa_with_sink_token(x.q[b].double(), x.k[b].double(), x.v[b].double(), x.scale, L, [0.0] * 4)
        assert torch.allclose(out[b], want, rtol=1e-12, atol=1e-12)


def test_learned_sink_with_window_equals_library_attention():
    lens, window, n_sink = [40, 300], 64, 4
    sinks = [-3.0, 0.5, 2.5, 7.0]
    x = wl.make_gqa(B=2, Hq=4, Hkv=1, D=16, seq_lens=lens, dtype=torch.bfloat16, paged=False, seed=22)
    out, lse = oracle.gqa(x.q, x.k, x.v, x.seq_lens, window=window, n_sink=n_sink, sink_logits=sinks)
    out = out.view(2, 4, 16)
    for b, L in enumerate(lens):
        keep = _keep_list(L, window, n_sink)
        want = _sdpa_with_sink_token(x.q[b].double(), x.k[b].double(), x.v[b].double(), x.scale, L,
                                     sinks, keep=keep)
        assert torch.allclose(out[b], want, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# cache append in logical order


def test_append_matches_library_index_put():
    from oracle import cache as ocache
    g = torch.Generator().manual_seed(9)
    for shape, new_shape in (((3, 2, 11, 5), (3, 2, 5)), ((3, 11, 7), (3, 7))):
        c = torch.randn(*shape, generator=g)
        new = torch.randn(*new_shape, generator=g)
        pos = torch.tensor([10, -1, 0])
        got = ocache.append(c, pos, new)
        want = c.clone()
        keep = pos >= 0
        b = torch.arange(3)[keep]
        if c.dim() == 4:
            want.permute(0, 2, 1, 3).index_put_((b, pos[keep]), new[keep])
        else:
            want.index_put_((b, pos[keep]), new[keep])
        assert torch.equal(got, want)
        assert torch.equal(got[1], c[1])  # a negative position appends nothing


def test_attention_after_append_sees_the_new_token():
    # appending a token whose key dominates every score makes it the output
    from oracle import cache as ocache
    x = wl.make_gqa(B=1, Hq=1, Hkv=1, D=4, seq_lens=[6], dtype=torch.float32, paged=False, seed=12)
    x.q[0, 0] = torch.tensor([1.0, 0, 0, 0])
    k_new = torch.tensor([[[400.0, 0, 0, 0]]])
    v_new = torch.tensor([[[1.0, 2.0, 3.0, 4.0]]])
    k = ocache.append(x.k, [5], k_new)
    v = ocache.append(x.v, [5], v_new)
    out, _ = oracle.gqa(x.q, k, v, x.seq_lens)
    assert torch.allclose(out[0], v_new[0, 0].double(), atol=1e-30)


# --------------------------------------------------------------------------
# Quest: query-aware page selection


def test_quest_bound_holds_for_every_key():
    from oracle import quest
    x = wl.make_gqa(B=2, Hq=4, Hkv=2, D=32, seq_lens=[70, 160], dtype=torch.float32, paged=False, seed=71)
    kmin, kmax = quest.page_minmax(x.k, x.seq_lens)
    up = quest.upper_bounds(x.q, kmin, kmax, x.seq_lens, 2)
    for b, L in enumerate([70, 160]):
        for h in range(4):
            s = x.k[b, h // 2, : L // 16 * 16].double() @ x.q[b, h].double()
            best = s.view(-1, 16).amax(1)
            assert torch.all(best <= up[b, h, : L // 16] + 1e-12)
            assert torch.all(torch.isinf(up[b, h, L // 16:]))


def test_quest_bound_hand_worked_example():
    # the page's bound on a mixed-sign query, worked by hand in the fixture;
    # a looser valid bound (sum |q| max(|kmin|, |kmax|)) or a sign slip
    # changes both values and the page chosen at budget 1
    from oracle import quest
    g = gold("quest_bound_tiny.json")
    pages = torch.tensor(g["pages"], dtype=torch.float64)        # [2, 16, 4]
    k = pages.reshape(1, 1, 32, 4)
    q = torch.tensor(g["q"], dtype=torch.float64).reshape(1, 1, 4)
    kmin, kmax = quest.page_minmax(k, [32])
    assert kmin[0, 0].tolist() == g["kmin"] and kmax[0, 0].tolist() == g["kmax"]
    up = quest.upper_bounds(q, kmin, kmax, [32], 1)
    assert up[0, 0].tolist() == g["upper"]
    assert quest.choose(up, [32], 1) == [g["chosen_budget_1"]]


def test_quest_bound_is_tight_on_identical_keys():
    # a page whose 16 keys are one vector k has kmin = kmax = k, and the
    # bound must then be exactly q . k, for queries and keys of any sign
    from oracle import quest
    g = torch.Generator().manual_seed(75)
    D = 8
    k = torch.randint(-4, 5, (1, 1, 3, D), generator=g).double()
    k = k.repeat_interleave(16, dim=2)                              # 3 pages of identical keys
    q = torch.randint(-4, 5, (1, 2, D), generator=g).double()
    kmin, kmax = quest.page_minmax(k, [48])
    up = quest.upper_bounds(q, kmin, kmax, [48], 2)
    for h in range(2):
        for p in range(3):
            assert up[0, h, p].item() == float(k[0, 0, 16 * p] @ q[0, h])


def test_quest_full_budget_equals_full_attention():
    # every full page chosen plus the partial one is the whole cache
    from oracle import quest
    x = wl.make_gqa(B=2, Hq=4, Hkv=1, D=16, seq_lens=[37, 100], dtype=torch.bfloat16, paged=False, seed=72)
    (out, lse), chosen = quest.decode(x.q, x.k, x.v, x.seq_lens, budget=100)
    want, wlse = oracle.gqa(x.q, x.k, x.v, x.seq_lens)
    assert torch.allclose(out, want, rtol=1e-12, atol=1e-12)
    assert torch.allclose(lse, wlse, rtol=1e-12, atol=1e-12)
    assert chosen[0] == [0, 1] and chosen[4] == list(range(6))


def test_quest_picks_the_page_that_points_along_the_query():
    # page 3's keys are a large multiple of the query: its bound dominates, so a
    # budget of one page picks it, and the output is close to its values' mix
    from oracle import quest
    x = wl.make_gqa(B=1, Hq=1, Hkv=1, D=8, seq_lens=[90], dtype=torch.float32, paged=False, seed=73)
    x.k[0, 0, 48:64] = 20.0 * x.q[0, 0]
    (out, _), chosen = quest.decode(x.q, x.k, x.v, x.seq_lens, budget=1)
    assert chosen == [[3]]
    assert torch.allclose(out[0], x.v[0, 0, 48:64].double().mean(0), atol=1e-6)


def test_quest_ties_go_to_the_lower_page():
    from oracle import quest
    x = wl.make_gqa(B=1, Hq=2, Hkv=1, D=4, seq_lens=[96], dtype=torch.float32, paged=False, seed=74)
    x.k[0, 0, :96] = x.k[0, 0, :16].repeat(6, 1)  # six identical pages
    (_, _), chosen = quest.decode(x.q, x.k, x.v, x.seq_lens, budget=3)
    assert chosen == [[0, 1, 2], [0, 1, 2]]


# --------------------------------------------------------------------------
# attention against the library routine (fp64 SDPA, CPU math path)


def _sdpa_rows(q, k, v, scale, L, keep=None):
    """Library attention for one sequence: q [Hq, D], k/v [Hkv, S, D] (fp64)."""
    Hq, Hkv = q.shape[0], k.shape[0]
    kk = k[:, :L] if keep is None else k[:, keep]
    vv = v[:, :L] if keep is None else v[:, keep]
    kk = kk.repeat_interleave(Hq // Hkv, dim=0)
    vv = vv.repeat_interleave(Hq // Hkv, dim=0)
    return F.scaled_dot_product_attention(q[:, None, :], kk, vv, scale=scale)[:, 0, :]


@pytest.mark.parametrize("Hq,Hkv,D,dtype", [
    (4, 2, 64, torch.float32),    # the tiny fp32 workload's shape
    (8, 8, 32, torch.float32),    # G = H: MHA
    (8, 1, 32, torch.bfloat16),   # one KV head: MQA
    (32, 8, 128, torch.bfloat16), # Llama-3-8B-shaped
])
def test_gqa_matches_library_sdpa(Hq, Hkv, D, dtype):
    lens = [1, 17, 300]
    x = wl.make_gqa(B=3, Hq=Hq, Hkv=Hkv, D=D, seq_lens=lens, dtype=dtype, paged=False, seed=11)
    out, _ = oracle.gqa(x.q, x.k, x.v, x.seq_lens)
    out = out.view(3, Hq, D)
    for b, L in enumerate(lens):
        want = _sdpa_rows(x.q[b].double(), x.k[b].double(), x.v[b].double(), x.scale, L)
        assert torch.allclose(out[b], want, rtol=1e-12, atol=1e-12)


def test_gqa_equals_mha_on_repeated_kv():
    x = wl.make_gqa(B=2, Hq=8, Hkv=2, D=16, seq_lens=[40, 23], dtype=torch.float32,
                    paged=False, seed=4)
    out_g, lse_g = oracle.gqa(x.q, x.k, x.v, x.seq_lens)
    k4 = x.k.repeat_interleave(4, dim=1).contiguous()
    v4 = x.v.repeat_interleave(4, dim=1).contiguous()
    out_m, lse_m = oracle.gqa(x.q, k4, v4, x.seq_lens)
    assert torch.equal(out_g, out_m) and torch.equal(lse_g, lse_m)


def test_sliding_window_mask_example():
    """Token 3 of T=6 with W=3 sees tokens 1, 2, 3 ('All the attentions', section 4)."""
    g = gold("page_numbers.json")["sliding_window_mask_example"]
    L = g["query"] + 1           # the cache holds tokens 0..query
    D = 8
    q = torch.zeros(1, 1, D)
    k = torch.zeros(1, 1, L, D)  # equal scores: the output is the mean of the seen values
    v = torch.zeros(1, 1, L, D)
    for t in range(L):
        v[0, 0, t, t] = 1.0      # one-hot value marks which token was seen
    out, _ = oracle.gqa(q, k, v, torch.tensor([L]), window=g["W"], n_sink=0)
    seen = [t for t in range(L) if out[0, t] > 0]
    assert seen == g["sees"]
    assert torch.allclose(out[0, seen], torch.full((len(seen),), 1.0 / len(seen), dtype=torch.float64))


def _keep_list(L, window, n_sink):
    """StreamingLLM keep list ('Long context...', 'KV eviction: StreamingLLM'):
    the first sinks plus the last window tokens; a union when they overlap."""
    return sorted(set(range(min(n_sink, L))) | set(range(max(0, L - window), L)))


def test_keep_list_fixture():
    g = gold("page_numbers.json")["streamingllm_keep_list"]
    keep = _keep_list(g["S"], g["budget"] - g["sinks"], g["sinks"])
    assert keep[:4] == g["keep_first"] and keep[4] == g["keep_window_start"]
    assert len(keep) == g["keep_len"]


@pytest.mark.parametrize("lens,window,n_sink", [
    ([300], 252, 4),             # the page's budget 256 = 4 sinks + 252 window
    ([4, 5, 9, 100], 5, 4),      # window shorter than, equal to, overlapping the sinks
    ([50, 70], 64, 0),           # window, no sinks
    ([50, 70], 80, 4),           # window >= length: full attention
    ([33], 1, 2),                # window of one token
])
def test_window_and_sinks_equal_attention_on_compacted_cache(lens, window, n_sink):
    x = wl.make_gqa(B=len(lens), Hq=4, Hkv=2, D=16, seq_lens=lens, dtype=torch.float32,
                    paged=False, window=window, n_sink=n_sink, sink_key_scale=4.0, seed=8)
    out, _ = oracle.gqa(x.q, x.k, x.v, x.seq_lens, window=window, n_sink=n_sink)
    out = out.view(len(lens), 4, 16)
    for b, L in enumerate(lens):
        keep = _keep_list(L, window, n_sink)
        want = _sdpa_rows(x.q[b].double(), x.k[b].double(), x.v[b].double(), x.scale, L, keep)
        assert torch.allclose(out[b], want, rtol=1e-12, atol=1e-12)


def test_row_subset_matches_full():
    x = wl.make_gqa(B=3, Hq=4, Hkv=2, D=32, seq_lens=[20, 31, 7], dtype=torch.bfloat16,
                    paged=False, seed=9)
    full, lse_full = oracle.gqa(x.q, x.k, x.v, x.seq_lens, window=9, n_sink=2)
    rows = [11, 0, 5]
    part, lse_part = oracle.gqa(x.q, x.k, x.v, x.seq_lens, window=9, n_sink=2, rows=rows)
    assert torch.equal(part, full[rows]) and torch.equal(lse_part, lse_full[rows])


def test_lse_merges_two_halves():
    """Splitting the tokens in two and merging by log-sum-exp gives the whole."""
    x = _tiny(L=64, D=16, seed=12)
    out, lse = oracle.gqa(x.q, x.k, x.v, x.seq_lens)
    lo = wl.make_gqa(B=1, Hq=1, Hkv=1, D=16, seq_lens=[30], dtype=torch.float32, paged=False)
    lo.q.copy_(x.q); lo.k.copy_(x.k[:, :, :30]); lo.v.copy_(x.v[:, :, :30])
    o1, l1 = oracle.gqa(lo.q, lo.k, lo.v, lo.seq_lens)
    k2 = x.k[:, :, 30:].contiguous(); v2 = x.v[:, :, 30:].contiguous()
    o2, l2 = oracle.gqa(x.q, k2, v2, torch.tensor([34]))
    L = torch.logaddexp(l1, l2)
    merged = torch.exp(l1 - L)[:, None] * o1 + torch.exp(l2 - L)[:, None] * o2
    assert torch.allclose(merged, out, rtol=1e-13, atol=1e-13)
    assert torch.allclose(L, lse, rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------------
# MLA: absorbed (what the oracle computes) against expanded (what the model does)


def test_absorbed_mla_equals_expanded_mla():
    """W_UK folded into q and W_UV applied after attention equal the per-head
    keys/values rebuilt from the latent ('Overview of Attention Mechanism', MLA;
    'Attention Optimizations', 'Computation Path')."""
    torch.manual_seed(0)
    H, d_nope, d_rope, d_c, d_v, S = 4, 16, 8, 32, 16, 23
    c_kv = torch.randn(S, d_c).double()
    k_pe = torch.randn(S, d_rope).double()
    q_nope = torch.randn(H, d_nope).double()
    q_pe = torch.randn(H, d_rope).double()
    W_UK = torch.randn(H, d_nope, d_c).double() / d_c ** 0.5
    W_UV = torch.randn(H, d_v, d_c).double() / d_c ** 0.5
    scale = (d_nope + d_rope) ** -0.5
    # expanded: per-head keys [W_UK c ; k_pe] and values W_UV c, then library SDPA
    k_h = torch.cat([torch.einsum("hnc,sc->hsn", W_UK, c_kv), k_pe.expand(H, S, d_rope)], -1)
    v_h = torch.einsum("hvc,sc->hsv", W_UV, c_kv)
    q_h = torch.cat([q_nope, q_pe], -1)
    want = F.scaled_dot_product_attention(q_h[:, None], k_h, v_h, scale=scale)[:, 0]
    # absorbed: q~ = [W_UK^T q_nope ; q_pe] against the latent rows [c_KV ; k_pe]
    q_abs = torch.cat([torch.einsum("hnc,hn->hc", W_UK, q_nope), q_pe], -1)
    latent = torch.cat([c_kv, k_pe], -1)
    o_lat, _ = oracle.mla(q_abs[None].float(), latent[None].float(), torch.tensor([S]),
                          d_latent=d_c, scale=scale)
    got = torch.einsum("hvc,hc->hv", W_UV, o_lat)
    # agreement up to the fp32 rounding of the oracle's inputs
    assert torch.allclose(got, want, rtol=2e-5, atol=2e-5)
    # a wrong scale, split or concatenation order is off by O(1)
    o_bad, _ = oracle.mla(q_abs[None].float(), latent[None].float(), torch.tensor([S]),
                          d_latent=d_c, scale=d_c ** -0.5)
    assert not torch.allclose(torch.einsum("hvc,hc->hv", W_UV, o_bad), want, rtol=1e-3, atol=1e-3)


def test_mla_value_is_the_latent_prefix_only():
    """The RoPE part of the row scores but never enters the output."""
    x = wl.make_mla(B=1, H=2, seq_lens=[10], d_latent=16, d_rope=8, dtype=torch.float32, seed=2)
    out, _ = oracle.mla(x.q, x.latent, x.seq_lens, d_latent=16, scale=0.3)
    lat2 = x.latent.clone()
    lat2[..., 16:] = 0
    q2 = x.q.clone()
    q2[..., 16:] = 0
    # zero RoPE parts in both q and the rows: scores lose that term, values unchanged
    out2, _ = oracle.mla(q2, lat2, x.seq_lens, d_latent=16, scale=0.3)
    want2 = F.scaled_dot_product_attention(q2[0].double()[:, None], lat2[0].double().expand(2, 10, 24),
                                           lat2[0, :, :16].double().expand(2, 10, 16), scale=0.3)[:, 0]
    assert torch.allclose(out2, want2, rtol=1e-12, atol=1e-12)
    assert not torch.allclose(out, out2)


def test_sparse_mla_with_all_tokens_equals_dense():
    x = wl.make_mla(B=2, H=3, seq_lens=[12, 7], d_latent=32, d_rope=8, dtype=torch.bfloat16, seed=3)
    dense, lse_d = oracle.mla(x.q, x.latent, x.seq_lens, d_latent=32)
    idx = torch.full((2, 12), -1, dtype=torch.int32)
    idx[0] = torch.arange(12)
    idx[1, :7] = torch.arange(7)
    sparse, lse_s = oracle.mla(x.q, x.latent, idx=idx, d_latent=32)
    assert torch.allclose(sparse, dense, rtol=1e-14, atol=1e-14)
    assert torch.allclose(lse_s, lse_d, rtol=1e-14, atol=1e-14)


def test_sparse_mla_equals_dense_on_gathered_rows():
    x = wl.make_mla(B=1, H=4, seq_lens=[50], d_latent=32, d_rope=8, dtype=torch.bfloat16, seed=4)
    sel = [3, 9, 10, 41, 49]
    idx = torch.tensor([sel + [-1, -1]], dtype=torch.int32)
    sparse, _ = oracle.mla(x.q, x.latent, idx=idx, d_latent=32)
    gathered = x.latent[:, sel].contiguous()
    dense, _ = oracle.mla(x.q, gathered, torch.tensor([len(sel)]), d_latent=32)
    assert torch.allclose(sparse, dense, rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------------
# indexer


def test_indexer_hand_worked_example():
    g = gold("indexer_tiny.json")
    q = torch.tensor([g["q_i"]], dtype=torch.bfloat16)
    k = torch.tensor([g["k_i"]], dtype=torch.bfloat16)
    w = torch.tensor([g["w"]], dtype=torch.float32)
    s = oracle.indexer(q, w, k, torch.tensor([5]))
    assert s[0].tolist() == g["scores"]
    for kk, want in g["topk"].items():
        assert oracle.topk(s, torch.tensor([5]), int(kk))[0].tolist() == want


def _small_dsa(seed, B=2, L=(40, 33), Hi=4, Di=8):
    return wl.make_dsa(B=B, seq_lens=list(L), Hi=Hi, Di=Di, topk=8, H=2, d_latent=16,
                       d_rope=8, seed=seed)


def test_indexer_brute_force():
    x = _small_dsa(1)
    s = oracle.indexer(x.q_i, x.w, x.k_i, x.seq_lens)
    q, k, w = x.q_i.tolist(), x.k_i.tolist(), x.w.tolist()
    for b, L in enumerate(x.seq_lens.tolist()):
        for t in range(k[b].__len__()):
            if t >= L:
                assert s[b, t] == torch.iinfo(torch.int64).min
                continue
            tot = 0
            for h in range(len(q[b])):
                dot = 0
                for d in range(len(q[b][h])):
                    dot += int(q[b][h][d]) * int(k[b][t][d])
                tot += int(w[b][h]) * max(0, dot)
            assert s[b, t] == tot


def test_indexer_relu_identity():
    """I(q) - I(-q) = sum_h w_h q_h . k_t: pins the ReLU, its sign and the weights."""
    x = _small_dsa(2)
    s_pos = oracle.indexer(x.q_i, x.w, x.k_i, x.seq_lens)
    s_neg = oracle.indexer(-x.q_i, x.w, x.k_i, x.seq_lens)
    lin = torch.einsum("bh,bhd,btd->bt", x.w.double(), x.q_i.double(), x.k_i.double())
    for b, L in enumerate(x.seq_lens.tolist()):
        assert torch.equal((s_pos[b, :L] - s_neg[b, :L]).double(), lin[b, :L])
        assert torch.all(s_pos[b, :L] >= 0)


def test_indexer_weight_and_head_permutation():
    x = _small_dsa(3)
    s = oracle.indexer(x.q_i, x.w, x.k_i, x.seq_lens)
    s2 = oracle.indexer(x.q_i, 2 * x.w, x.k_i, x.seq_lens)
    perm = torch.randperm(x.q_i.shape[1], generator=torch.Generator().manual_seed(0))
    s3 = oracle.indexer(x.q_i[:, perm].contiguous(), x.w[:, perm].contiguous(), x.k_i, x.seq_lens)
    for b, L in enumerate(x.seq_lens.tolist()):
        assert torch.equal(s2[b, :L], 2 * s[b, :L])
        assert torch.equal(s3[b, :L], s[b, :L])


def test_e4m3_decoding_matches_library_for_every_code():
    # the oracle's own decoder of the fp8 format against torch's float8_e4m3fn
    codes = torch.arange(256, dtype=torch.uint8)
    lib_vals = codes.view(torch.float8_e4m3fn).to(torch.float64)
    for c in range(256):
        got, want = oracle.e4m3_value(c), lib_vals[c].item()
        assert (math.isnan(got) and math.isnan(want)) or got == want, (c, got, want)
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9


def test_indexer_fp8_equals_bf16_on_the_same_integers():
    # integers in [-4, 4] are exact in e4m3: the scores cannot depend on the encoding
    d = _small_dsa(31)
    s16 = oracle.indexer(d.q_i, d.w, d.k_i, d.seq_lens)
    s8 = oracle.indexer(d.q_i.to(torch.float8_e4m3fn), d.w, d.k_i.to(torch.float8_e4m3fn), d.seq_lens)
    assert torch.equal(s16, s8)


def test_indexer_rejects_non_integers():
    x = _small_dsa(4)
    q = x.q_i.float()
    q[0, 0, 0] = 0.5
    with pytest.raises(RuntimeError):
        oracle.indexer(q, x.w, x.k_i.float(), x.seq_lens)


# --------------------------------------------------------------------------
# top-k: the properties that make the answer unique


def _check_topk_properties(scores, lens, k, idx):
    for b, L in enumerate(lens):
        row = idx[b].tolist()
        n = min(k, L)
        sel = row[:n]
        assert row[n:] == [-1] * (k - n)
        assert sel == sorted(sel) and len(set(sel)) == n and all(0 <= t < L for t in sel)
        if n == L or n == 0:
            continue
        vals = [float(scores[b, t]) for t in range(L)]
        chosen = set(sel)
        lo_sel = min(vals[t] for t in chosen)
        hi_rest = max(vals[t] for t in range(L) if t not in chosen)
        assert lo_sel >= hi_rest
        if lo_sel == hi_rest:  # tie at the threshold: lower indices win
            tied_sel = [t for t in chosen if vals[t] == lo_sel]
            tied_rest = [t for t in range(L) if t not in chosen and vals[t] == lo_sel]
            assert max(tied_sel) < min(tied_rest)


@pytest.mark.parametrize("n_distinct", [None, 3, 40])
@pytest.mark.parametrize("k", [1, 7, 64, 500])
def test_topk_properties(n_distinct, k):
    lens = [0, 1, 63, 64, 257, 1000]
    s = wl.make_scores(B=len(lens), seq_lens=lens, n_distinct=n_distinct, seed=k)
    idx = oracle.topk(s, torch.tensor(lens), k)
    _check_topk_properties(s, lens, k, idx)


def test_topk_brute_force_tiny():
    rng = random.Random(0)
    for trial in range(200):
        L = rng.randint(1, 12)
        k = rng.randint(1, 14)
        vals = [float(rng.randint(-3, 3)) for _ in range(L)]
        s = torch.tensor([vals], dtype=torch.float32)
        got = oracle.topk(s, torch.tensor([L]), k)[0].tolist()
        order = sorted(range(L), key=lambda t: (-vals[t], t))[: min(k, L)]
        assert got == sorted(order) + [-1] * (k - min(k, L))


def test_topk_signed_zeros_tie():
    s = torch.tensor([[-0.0, 0.0, -1.0, 0.0]], dtype=torch.float32)
    assert oracle.topk(s, torch.tensor([4]), 2)[0].tolist() == [0, 1]


def test_topk_int64_and_fp32_agree_on_integers():
    x = _small_dsa(5, L=(40, 40))
    s = oracle.indexer(x.q_i, x.w, x.k_i, x.seq_lens)
    a = oracle.topk(s, x.seq_lens, 8)
    b = oracle.topk(s.float(), x.seq_lens, 8)
    assert torch.equal(a, b)


# --------------------------------------------------------------------------
# error metric used by the parity tests


def test_rel_err_rows_metric():
    y = torch.tensor([[1.0, -2.0], [0.5, 0.25]])
    x = y + torch.tensor([[0.02, 0.0], [0.0, 0.001]])
    assert oracle.rel_err_rows(x, y) == pytest.approx(0.01)
    assert oracle.norm_rel_err(y, y) == 0.0
