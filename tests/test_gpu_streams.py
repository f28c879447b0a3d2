"""Calls launched on a side stream while the current stream allocates and
writes: the binding's workspace and outputs must belong to the launch stream,
so that the caching allocator does not hand them to the other stream's work
while the split and combine kernels still use them."""
import pytest
import torch

import oracle
from decode_attention_kv_flash_amd import api
from decode_attention_kv_flash_amd import workloads as wl
from _helpers import TOL_BF16, assert_lse_close, assert_rows_close, say

pytestmark = pytest.mark.gpu


def _scribble(nbytes, rounds=24):
    """Allocate and fill blocks on the current stream, as other work would."""
    for _ in range(rounds):
        t = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        t.fill_(0xFF)
        del t


def test_gqa_on_side_stream():
    x = wl.make_gqa(B=8, Hq=32, Hkv=8, D=128, seq_lens=[4096] * 8, dtype=torch.bfloat16, seed=91,
                    name="gqa_side_stream")
    say(f"[streams] {x.name}")
    q, kc, vc = x.q.cuda(), x.k_cache.cuda(), x.v_cache.cuda()
    sl, pt = x.seq_lens.cuda(), x.page_table.cuda()
    ws_bytes = api.lib().decode_attn_gqa_workspace(x.B, x.Hq, x.Hkv, x.D, x.page_size, pt.shape[1], 0, 0, 0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    outs = []
    for _ in range(3):
        outs.append(api.decode_attn_gqa(q, kc, vc, sl, pt, scale=x.scale, stream=side))
        _scribble(max(ws_bytes, 1 << 20))
    side.synchronize()
    torch.cuda.synchronize()
    want, wlse = oracle.gqa(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    for out, lse in outs:
        assert_rows_close(out.float().cpu().reshape(-1, x.D), want, TOL_BF16, x.name)
        assert_lse_close(lse.cpu(), wlse, 1e-5, x.name)


def test_mla_on_side_stream():
    m = wl.make_mla(B=4, H=128, seq_lens=[3000, 2048, 1500, 4000], seed=92, name="mla_side_stream")
    say(f"[streams] {m.name}")
    q, lat, sl = m.q.cuda(), m.latent.cuda(), m.seq_lens.cuda()
    ws_bytes = api.lib().decode_attn_mla_workspace(m.B, m.H, 512, m.S_max, 0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    outs = []
    for _ in range(3):
        outs.append(api.decode_attn_mla(q, lat, sl, scale=m.scale, stream=side))
        _scribble(ws_bytes)
    side.synchronize()
    torch.cuda.synchronize()
    want, wlse = oracle.mla(m.q, m.latent, m.seq_lens, scale=m.scale)
    for out, lse in outs:
        assert_rows_close(out.float().cpu().reshape(-1, 512), want, TOL_BF16, m.name)
        assert_lse_close(lse.cpu(), wlse, 1e-5, m.name)


def test_calls_from_two_host_threads():
    """Two host threads, each with its own stream, call the library at once
    (the C calls release the GIL): every result equals the single-threaded one."""
    import threading
    x = wl.make_gqa(B=4, Hq=32, Hkv=8, D=128, seq_lens=[3000, 17, 4096, 1000], dtype=torch.bfloat16,
                    seed=95, name="gqa_threads")
    m = wl.make_mla(B=2, H=128, seq_lens=[2500, 700], seed=96, name="mla_threads")
    say("[streams] two host threads, GQA and MLA")
    q, kc, vc, sl, pt = x.q.cuda(), x.k_cache.cuda(), x.v_cache.cuda(), x.seq_lens.cuda(), x.page_table.cuda()
    mq, lat, msl = m.q.cuda(), m.latent.cuda(), m.seq_lens.cuda()
    ref_g, _ = api.decode_attn_gqa(q, kc, vc, sl, pt, scale=x.scale)
    ref_m, _ = api.decode_attn_mla(mq, lat, msl, scale=m.scale)
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(tid):
        try:
            s = torch.cuda.Stream()
            outs = []
            with torch.cuda.stream(s):
                for _ in range(20):
                    if tid == 0:
                        outs.append(api.decode_attn_gqa(q, kc, vc, sl, pt, scale=x.scale, stream=s)[0])
                    else:
                        outs.append(api.decode_attn_mla(mq, lat, msl, scale=m.scale, stream=s)[0])
            s.synchronize()
            results[tid] = outs
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    assert all(torch.equal(o, ref_g) for o in results[0])
    assert all(torch.equal(o, ref_m) for o in results[1])
    want, _ = oracle.gqa(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    assert_rows_close(ref_g.float().cpu().reshape(-1, x.D), want, TOL_BF16, x.name)
