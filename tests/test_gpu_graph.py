"""The entry points under HIP graph capture: every launch goes to the caller's
stream and nothing is read back on the host, so a captured call replays to
the eager result.  Each graph is replayed several times with eager work of
the library and synchronisations in between, and every replay is compared
with the eager run bit for bit (the kernels are deterministic)."""
import pytest
import torch

from decode_attention_kv_flash_amd import api
from decode_attention_kv_flash_amd import workloads as wl
from _helpers import dev, say

pytestmark = pytest.mark.gpu


def replay_and_check(run, outs, eager, n=3):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm once on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for i in range(n):
        for o in outs:
            o.fill_(0)
        eager()  # eager library work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        yield i


def test_gqa_sink_and_combine_replay():
    x = wl.make_gqa(B=3, Hq=32, Hkv=8, D=128, seq_lens=[700, 5000, 33], dtype=torch.bfloat16,
                    page_size=16, window=1024, n_sink=4, seed=91, name="graph_gqa")
    q, kc, vc, sl, pt = dev(x.q), dev(x.k_cache), dev(x.v_cache), dev(x.seq_lens), dev(x.page_table)
    sk = dev(torch.linspace(-1, 1, 32))
    nb = api.lib().decode_attn_gqa_workspace(3, 32, 8, 128, 16, pt.shape[1], 1024, 4, 0)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(3, 32, dtype=torch.float32, device="cuda")

    def run():
        api.decode_attn_gqa(q, kc, vc, sl, pt, 1024, 4, scale=x.scale, out=out, lse=lse, workspace=ws,
                            sink_logits=sk)

    run()
    torch.cuda.synchronize()
    want_o, want_l = out.clone(), lse.clone()
    other = wl.make_gqa(B=2, Hq=8, Hkv=2, D=64, seq_lens=[100, 300], dtype=torch.bfloat16, seed=92)
    eager = lambda: api.decode_attn_gqa(dev(other.q), dev(other.k_cache), dev(other.v_cache),
                                        dev(other.seq_lens), dev(other.page_table))
    for i in replay_and_check(run, [out, lse], eager):
        say(f"[graph] gqa replay {i}")
        assert torch.equal(out, want_o) and torch.equal(lse, want_l)


def test_mla_dsa_replay():
    d = wl.make_dsa(B=2, seq_lens=[5000, 3000], Hi=64, topk=512, H=128, seed=93, name="graph_dsa")
    m = d.mla
    qi, w, ki, sl = dev(d.q_i), dev(d.w), dev(d.k_i), dev(d.seq_lens)
    q, lat = dev(m.q), dev(m.latent)
    L = api.lib()
    iws = torch.empty(L.dsa_indexer_topk_workspace(2, d.k_i.shape[1], 512), dtype=torch.uint8, device="cuda")
    idx = torch.empty(2, 512, dtype=torch.int32, device="cuda")
    nb = L.sparse_mla_attn_workspace(2, 128, 512, 512, 0)
    sws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    nd = L.decode_attn_mla_workspace(2, 128, 512, m.S_max, 0)
    dws = torch.empty(max(nd, 1), dtype=torch.uint8, device="cuda")
    sout = torch.empty(2, 128, 512, dtype=torch.bfloat16, device="cuda")
    dout = torch.empty_like(sout)
    slse = torch.empty(2, 128, dtype=torch.float32, device="cuda")
    dlse = torch.empty_like(slse)

    def run():
        api.dsa_indexer_topk(qi, w, ki, sl, 512, topk_idx=idx, workspace=iws)
        api.sparse_mla_attn(q, lat, idx, scale=m.scale, out=sout, lse=slse, workspace=sws)
        api.decode_attn_mla(q, lat, sl, scale=m.scale, out=dout, lse=dlse, workspace=dws)

    run()
    torch.cuda.synchronize()
    want_i, want_s, want_d = idx.clone(), sout.clone(), dout.clone()
    want_sl, want_dl = slse.clone(), dlse.clone()
    eager = lambda: api.dsa_topk(dev(torch.randn(2, 3000)), dev(torch.tensor([3000, 10], dtype=torch.int32)), 64)
    for i in replay_and_check(run, [idx, sout, dout, slse, dlse], eager):
        say(f"[graph] mla + dsa replay {i}")
        assert torch.equal(idx, want_i)
        assert torch.equal(sout, want_s) and torch.equal(dout, want_d)
        assert torch.equal(slse, want_sl) and torch.equal(dlse, want_dl)


def test_quest_replay():
    x = wl.make_gqa(B=2, Hq=32, Hkv=8, D=128, seq_lens=[3000, 1029], dtype=torch.bfloat16, page_size=16,
                    qk_int=2, seed=94, name="graph_quest")
    q, kc, vc, sl, pt = dev(x.q), dev(x.k_cache), dev(x.v_cache), dev(x.seq_lens), dev(x.page_table)
    kmm = api.quest_page_minmax(kc, sl, pt)
    L = api.lib()
    nb = L.decode_attn_quest_workspace(2, 32, 8, 128, 16, pt.shape[1], 40, 1, 0)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(2, 32, dtype=torch.float32, device="cuda")

    def run():
        api.quest_page_minmax(kc, sl, pt, kminmax=kmm)
        api.decode_attn_quest(q, kc, vc, kmm, sl, 40, pt, scale=x.scale, out=out, lse=lse, workspace=ws)

    run()
    torch.cuda.synchronize()
    want_o, want_l = out.clone(), lse.clone()
    eager = lambda: api.quest_page_minmax(kc, sl, pt)
    for i in replay_and_check(run, [out, lse], eager):
        say(f"[graph] quest replay {i}")
        assert torch.equal(out, want_o) and torch.equal(lse, want_l)
