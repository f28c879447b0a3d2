"""The seeded input generator: determinism and layout consistency."""
import torch

from decode_attention_kv_flash_amd import workloads as wl


def test_generator_is_deterministic():
    a = wl.make_gqa(B=2, Hq=4, Hkv=2, D=16, seq_lens=[33, 70], seed=5)
    b = wl.make_gqa(B=2, Hq=4, Hkv=2, D=16, seq_lens=[33, 70], seed=5)
    for x, y in [(a.q, b.q), (a.k_cache, b.k_cache), (a.page_table, b.page_table)]:
        assert torch.equal(x, y)
    c = wl.make_gqa(B=2, Hq=4, Hkv=2, D=16, seq_lens=[33, 70], seed=6)
    assert not torch.equal(a.q, c.q)


def test_paged_cache_gathers_back_to_logical():
    x = wl.make_gqa(B=3, Hq=4, Hkv=2, D=8, seq_lens=[1, 16, 45], page_size=16, seed=2)
    assert x.page_table.dtype == torch.int32
    used = set()
    for b, L in enumerate(x.seq_lens.tolist()):
        for t in range(L):
            phys = int(x.page_table[b, t // 16])
            used.add(phys)
            assert torch.equal(x.k_cache[phys, :, t % 16], x.k[b, :, t])
            assert torch.equal(x.v_cache[phys, :, t % 16], x.v[b, :, t])
    assert len(used) == x.k_cache.shape[0]  # every physical page belongs to one sequence


def test_pages_are_permuted():
    x = wl.make_gqa(B=4, Hq=4, Hkv=2, D=8, seq_lens=[160] * 4, page_size=16, seed=3)
    flat = x.page_table.flatten().tolist()
    assert sorted(flat) == list(range(40)) and flat != list(range(40))


def test_sink_keys_scaled_before_rounding():
    a = wl.make_gqa(B=1, Hq=2, Hkv=1, D=8, seq_lens=[10], n_sink=4, window=3,
                    sink_key_scale=4.0, seed=1, paged=False)
    b = wl.make_gqa(B=1, Hq=2, Hkv=1, D=8, seq_lens=[10], n_sink=4, window=3,
                    sink_key_scale=1.0, seed=1, paged=False)
    assert torch.equal(a.k[0, 0, :4], (b.k[0, 0, :4].float() * 4).to(torch.bfloat16))
    assert torch.equal(a.k[0, 0, 4:], b.k[0, 0, 4:])


def test_attended_token_count():
    x = wl.make_gqa(B=4, Hq=2, Hkv=1, D=8, seq_lens=[3, 6, 7, 100], window=4, n_sink=2,
                    paged=False, seed=0)
    # L=3: all 3; L=6: [0,2) u [2,6) = 6; L=7: [0,2) u [3,7) = 6; L=100: 2 + 4
    assert x.attended_tokens() == 3 + 6 + 6 + 6


def test_config_shapes():
    lens = wl.config3_lens()
    assert len(lens) == 32 and min(lens) >= 4096 and max(lens) <= 32768
    d = wl.make_dsa(B=1, seq_lens=[100], topk=16, H=2, d_latent=16, d_rope=8, seed=0)
    assert d.q_i.abs().max() <= 4 and d.k_i.abs().max() <= 4
    assert d.w.min() >= 1 and d.w.max() <= 4
    assert torch.equal(d.q_i.float().round(), d.q_i.float())
