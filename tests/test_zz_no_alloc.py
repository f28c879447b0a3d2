"""decode_attn_gqa_noalloc, the allocation-free entry point, through the C ABI:
its output against decode_attn_gqa's (and the oracle's) on two calls in a
row, the second smaller, so the second reads the library's scratch array
after the first left its partials there."""
import pytest
import torch

import oracle
from decode_attention_kv_flash_amd import api
from decode_attention_kv_flash_amd import workloads as wl
from _helpers import assert_lse_close, assert_rows_close, say, tol_for

pytestmark = pytest.mark.gpu


def _both(x, num_splits=0, sink=None):
    q, kc, vc, sl = x.q.cuda(), x.k_cache.cuda(), x.v_cache.cuda(), x.seq_lens.cuda()
    pt = x.page_table.cuda() if x.page_table is not None else None
    sk = sink.cuda() if sink is not None else None
    ref, ref_lse = api.decode_attn_gqa(q, kc, vc, sl, pt, x.window, x.n_sink, scale=x.scale,
                                       num_splits=num_splits, sink_logits=sk)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((x.B, x.Hq), float("nan"), dtype=torch.float32, device="cuda")
    api.decode_attn_gqa_noalloc(q, kc, vc, sl, pt, x.window, x.n_sink, out=out, lse=lse, scale=x.scale,
                                num_splits=num_splits, sink_logits=sk)
    torch.cuda.synchronize()
    return ref, ref_lse, out, lse


def _check(x, ref, ref_lse, out, lse, sink=None):
    tol = tol_for(x.q.dtype)
    assert_rows_close(out.float().cpu().reshape(-1, x.D), ref.double().cpu().reshape(-1, x.D), tol, x.name)
    assert_lse_close(lse.cpu(), ref_lse.cpu(), 1e-6, x.name)
    want, wlse = oracle.gqa(x.q, x.k, x.v, x.seq_lens, window=x.window, n_sink=x.n_sink, scale=x.scale,
                            sink_logits=None if sink is None else sink.tolist())
    assert_rows_close(out.float().cpu().reshape(-1, x.D), want, tol, x.name)
    assert_lse_close(lse.cpu(), wlse, 1e-5, x.name)


def test_noalloc_matches_the_workspace_entry_point_twice():
    x = wl.make_gqa(B=8, Hq=32, Hkv=8, D=128, seq_lens=[4096, 3000, 17, 0, 4096, 2048, 1, 4000],
                    dtype=torch.bfloat16, seed=95, name="noalloc_first")
    say(f"[noalloc] {x.name}: paged bf16, automatic splits")
    _check(x, *_both(x))
    # second call, smaller: fp32, contiguous, window + sinks + sink logits,
    # a requested split count; the scratch still holds the first call's partials
    y = wl.make_gqa(B=3, Hq=8, Hkv=2, D=64, seq_lens=[300, 33, 129], dtype=torch.float32, paged=False,
                    window=64, n_sink=4, seed=96, name="noalloc_second")
    sink = torch.linspace(-1.0, 2.0, 8, dtype=torch.float32)
    say(f"[noalloc] {y.name}: contiguous fp32, window 64 + 4 sinks, sink logits, 5 splits")
    _check(y, *_both(y, num_splits=5, sink=sink), sink=sink)


def test_noalloc_refuses_a_split_count_past_the_scratch():
    # 16 x 32 rows x 64 splits x 129 fp32 values exceed the 16 MiB array:
    # refused on the host, before any launch
    x = wl.make_gqa(B=16, Hq=32, Hkv=8, D=128, seq_lens=[64] * 16, dtype=torch.bfloat16, seed=97,
                    name="noalloc_refuse")
    q = x.q.cuda()
    out = torch.empty_like(q)
    say(f"[noalloc] {x.name}: 64 splits requested")
    with pytest.raises(api.DattnError, match="scratch") as e:
        api.decode_attn_gqa_noalloc(q, x.k_cache.cuda(), x.v_cache.cuda(), x.seq_lens.cuda(),
                                    x.page_table.cuda(), out=out, num_splits=64)
    assert e.value.code == -3
