"""DATTN_DEBUG mode: the device-resident tables are copied to the host and
checked before any launch.  The malformed cases here are rejected by that
check and never reach a kernel; each is also chosen so that, were the check
to let it through, the kernels would still read only this test's memory
(page -1 of a cache placed one page into a larger buffer; lengths past the
table, which the kernels clamp to the cache)."""
import pytest
import torch

import oracle
from decode_attention_kv_flash_amd import api
from decode_attention_kv_flash_amd import workloads as wl
from _helpers import TOL_BF16, assert_rows_close, say

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_mode():
    api.debug_enable(True)
    try:
        yield
    finally:
        api.debug_enable(False)


def _gqa_inputs():
    x = wl.make_gqa(B=3, Hq=8, Hkv=2, D=128, seq_lens=[40, 200, 17], dtype=torch.bfloat16, seed=93,
                    name="gqa_debug")
    return x, x.q.cuda(), x.k_cache.cuda(), x.v_cache.cuda(), x.seq_lens.cuda(), x.page_table.cuda()


def test_debug_mode_passes_a_valid_call(debug_mode):
    x, q, kc, vc, sl, pt = _gqa_inputs()
    say(f"[debug] {x.name} valid tables")
    out, _ = api.decode_attn_gqa(q, kc, vc, sl, pt, scale=x.scale)
    torch.cuda.synchronize()
    want, _ = oracle.gqa(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    assert_rows_close(out.float().cpu().reshape(-1, x.D), want, TOL_BF16, x.name)


def _padded(cache):
    """The cache as a view one page into a buffer with a spare page on each
    side, so that page -1 is still memory of this test."""
    buf = torch.zeros((cache.shape[0] + 2,) + tuple(cache.shape[1:]), dtype=cache.dtype, device="cuda")
    buf[1:-1].copy_(cache)
    return buf, buf[1:-1]


def test_debug_mode_rejects_a_negative_page(debug_mode):
    x, q, kc, vc, sl, pt = _gqa_inputs()
    kbuf, kc = _padded(kc)
    vbuf, vc = _padded(vc)
    bad = pt.clone()
    bad[1, 3] = -1                       # a page the 200-token sequence reads
    out = torch.full_like(q, 7.0)
    say(f"[debug] {x.name} negative page_table entry")
    with pytest.raises(api.DattnError, match=r"page_table\[1\]\[3\] = -1"):
        api.decode_attn_gqa(q, kc, vc, sl, bad, scale=x.scale, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)         # nothing was launched
    # the same cache and a valid table pass the check
    out, _ = api.decode_attn_gqa(q, kc, vc, sl, pt, scale=x.scale)
    torch.cuda.synchronize()
    want, _ = oracle.gqa(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    assert_rows_close(out.float().cpu().reshape(-1, x.D), want, TOL_BF16, x.name)


def test_debug_mode_rejects_a_length_past_the_table(debug_mode):
    x, q, kc, vc, sl, pt = _gqa_inputs()
    bad = sl.clone()
    bad[2] = pt.shape[1] * x.page_size + 1
    say(f"[debug] {x.name} seq_lens past the table")
    with pytest.raises(api.DattnError, match=r"seq_lens\[2\]"):
        api.decode_attn_gqa(q, kc, vc, bad, pt, scale=x.scale)


def test_debug_mode_checks_mla_and_indexer_lengths(debug_mode):
    m = wl.make_mla(B=2, H=64, seq_lens=[100, 64], seed=94, name="mla_debug")
    sl = m.seq_lens.clone()
    sl[0] = m.S_max + 1
    say("[debug] mla and indexer lengths past the cache")
    with pytest.raises(api.DattnError, match=r"seq_lens\[0\]"):
        api.decode_attn_mla(m.q.cuda(), m.latent.cuda(), sl.cuda(), scale=m.scale)
    qi = torch.zeros(2, 64, 128, dtype=torch.bfloat16, device="cuda")
    ki = torch.zeros(2, 300, 128, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(2, 64, dtype=torch.float32, device="cuda")
    lens = torch.tensor([300, 301], dtype=torch.int32, device="cuda")
    with pytest.raises(api.DattnError, match=r"seq_lens\[1\]"):
        api.dsa_indexer_topk(qi, w, ki, lens, 16)
