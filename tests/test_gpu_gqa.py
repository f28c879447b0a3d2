"""GQA and sliding-window + sinks decode attention on the GPU against the oracle."""
import pytest
import torch

import oracle
from decode_attention_kv_flash_amd import api
from decode_attention_kv_flash_amd import workloads as wl
from _helpers import (TOL_BF16, TOL_F32, assert_lse_close, assert_rows_close, dev, rows_sample,
                      say, tol_for)

pytestmark = pytest.mark.gpu


def run_gpu(x, num_splits=0):
    out, lse = api.decode_attn_gqa(dev(x.q), dev(x.k_cache), dev(x.v_cache), dev(x.seq_lens),
                                   dev(x.page_table), x.window, x.n_sink, scale=x.scale,
                                   num_splits=num_splits)
    torch.cuda.synchronize()
    return out.float().cpu().reshape(-1, x.D), lse.cpu().reshape(-1)


def check_full(x, num_splits=0):
    say(f"[gqa] {x.name or 'case'} B={x.B} Hq={x.Hq} Hkv={x.Hkv} D={x.D} lens={x.seq_lens.tolist()[:6]} "
        f"window={x.window} sinks={x.n_sink} splits={num_splits}")
    got, glse = run_gpu(x, num_splits)
    want, wlse = oracle.gqa(x.q, x.k, x.v, x.seq_lens, window=x.window, n_sink=x.n_sink,
                            scale=x.scale)
    tol = tol_for(x.q.dtype)
    err = assert_rows_close(got, want, tol, x.name)
    assert_lse_close(glse, wlse, 1e-5, x.name)
    return err


def test_tiny_gqa_fp32_config():
    """B2, 4 q heads / 2 KV heads, D64, 256 tokens, contiguous, fp32: tolerance 1e-5."""
    x = wl.config1_tiny_gqa()
    for splits in (0, 1, 2, 4, 7):
        err = check_full(x, splits)
        assert err <= TOL_F32


def check_sink(x, sinks, num_splits=0):
    """decode_attn_gqa_sink against the oracle with the same fp32 sink logits."""
    say(f"[gqa-sink] {x.name or 'case'} B={x.B} Hq={x.Hq} Hkv={x.Hkv} D={x.D} "
        f"lens={x.seq_lens.tolist()[:6]} window={x.window} sinks={x.n_sink} splits={num_splits}")
    sk = torch.tensor(sinks, dtype=torch.float32)
    out, lse = api.decode_attn_gqa(dev(x.q), dev(x.k_cache), dev(x.v_cache), dev(x.seq_lens),
                                   dev(x.page_table), x.window, x.n_sink, scale=x.scale,
                                   num_splits=num_splits, sink_logits=dev(sk))
    torch.cuda.synchronize()
    got, glse = out.float().cpu().reshape(-1, x.D), lse.cpu().reshape(-1)
    want, wlse = oracle.gqa(x.q, x.k, x.v, x.seq_lens, window=x.window, n_sink=x.n_sink,
                            scale=x.scale, sink_logits=sk.double())
    err = assert_rows_close(got, want, tol_for(x.q.dtype), x.name)
    assert_lse_close(glse, wlse, 1e-5, x.name)
    return err


@pytest.mark.parametrize("splits", [0, 1, 2, 4])
def test_zero_sink_tiny_fp32(splits):
    """softmax-off-by-one (all sinks 0) on the tiny fp32 workload, 1e-5."""
    x = wl.config1_tiny_gqa()
    assert check_sink(x, [0.0] * x.Hq, splits) <= TOL_F32


@pytest.mark.parametrize("Hq,Hkv,D,dtype,paged", [
    (32, 8, 128, torch.bfloat16, True),
    (8, 1, 64, torch.float32, False),
    (8, 2, 64, torch.float32, True),
    (64, 8, 64, torch.bfloat16, True),
])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_learned_sinks_ragged(Hq, Hkv, D, dtype, paged, splits):
    x = wl.make_gqa(B=4, Hq=Hq, Hkv=Hkv, D=D, seq_lens=[1, 17, 300, 1029], dtype=dtype,
                    page_size=16, paged=paged, seed=31, name=f"sinks_{Hq}_{Hkv}_{D}")
    g = torch.Generator().manual_seed(5)
    # logits spanning well below to well above the scores (N(0,1) data)
    sinks = (torch.rand(Hq, generator=g) * 16 - 6).tolist()
    check_sink(x, sinks, splits)


@pytest.mark.parametrize("splits", [0, 2])
def test_learned_sinks_with_window(splits):
    x = wl.make_gqa(B=3, Hq=32, Hkv=8, D=128, seq_lens=[3, 700, 5000], dtype=torch.bfloat16,
                    page_size=16, paged=True, window=512, n_sink=4, seed=32, name="sinks_window")
    check_sink(x, [float(h % 7) - 3.0 for h in range(32)], splits)


@pytest.mark.parametrize("splits", [0, 2])
def test_learned_sinks_window_d64_eight_heads(splits):
    """64 q / 8 KV heads, D64 bf16, a 128-token window and a sink logit per
    head: the eight-head transposed softmax at 8 lanes per token row."""
    x = wl.make_gqa(B=3, Hq=64, Hkv=8, D=64, seq_lens=[5, 130, 2000], dtype=torch.bfloat16,
                    page_size=16, paged=True, window=128, seed=35, name="sinks_window_d64")
    check_sink(x, [float(h % 9) - 4.0 for h in range(64)], splits)


def test_sink_on_empty_sequences():
    """No token: zero output and lse equal to the head's sink logit."""
    x = wl.make_gqa(B=3, Hq=8, Hkv=2, D=64, seq_lens=[0, 40, 0], dtype=torch.bfloat16,
                    page_size=16, paged=True, seed=33, name="sinks_empty")
    for splits in (1, 2):
        check_sink(x, [0.5 * h - 2.0 for h in range(8)], splits)


@pytest.mark.parametrize("Hq,Hkv,D,dtype,paged", [
    (32, 8, 128, torch.bfloat16, True),
    (8, 8, 64, torch.bfloat16, True),     # MHA
    (8, 1, 128, torch.bfloat16, False),   # MQA
    (16, 2, 64, torch.float32, True),     # G = 8
    (4, 2, 128, torch.float32, False),
    (6, 3, 64, torch.bfloat16, True),     # G = 2, odd head counts
    (8, 2, 64, torch.float32, True),      # G = 4 at 16 lanes per row in fp32: the transposed softmax
    (16, 4, 128, torch.bfloat16, False),  # G = 4, contiguous
    (8, 2, 64, torch.bfloat16, True),     # G = 4 at 8 lanes per row: the transposed softmax
    (64, 8, 64, torch.bfloat16, False),   # G = 8 at 8 lanes per row, contiguous
    (64, 8, 128, torch.bfloat16, True),   # G = 8 at 16 lanes per row
])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_gqa_ragged(Hq, Hkv, D, dtype, paged, splits):
    x = wl.make_gqa(B=4, Hq=Hq, Hkv=Hkv, D=D, seq_lens=[1, 17, 300, 1029], dtype=dtype,
                    page_size=16, paged=paged, seed=21, name=f"ragged_{Hq}_{Hkv}_{D}")
    check_full(x, splits)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("splits", [1, 2, 5, 16])
def test_eight_heads_double_buffer_edges(D, splits):
    """Eight bf16 heads per KV head keep two register buffers per wave; short
    and ragged sequences over many splits give waves none, one, two or three
    blocks, whole and partial, so every exit of the two-buffer loop runs."""
    x = wl.make_gqa(B=6, Hq=64, Hkv=8, D=D, seq_lens=[1, 16, 17, 64, 65, 200], dtype=torch.bfloat16,
                    page_size=16, seed=36, name=f"g8_edges_d{D}")
    check_full(x, splits)


@pytest.mark.parametrize("page_size", [1, 4, 32, 64])
def test_gqa_page_sizes(page_size):
    x = wl.make_gqa(B=3, Hq=8, Hkv=2, D=128, seq_lens=[5, 129, 700], page_size=page_size,
                    seed=22, name=f"pages{page_size}")
    check_full(x)


@pytest.mark.parametrize("page_size", [2, 8, 128, 256, 1024])
@pytest.mark.parametrize("D", [64, 128])
def test_window_and_sinks_on_small_and_large_pages(page_size, D):
    """Pages of 2 and 8 tokens (several per 16-token step) and of 128 to 1024
    (a window spanning one to eight pages, sinks and window in one page),
    ragged lengths, 4 query heads per KV head, automatic and 3 splits."""
    lens = [1, 300, 2049, 5000]
    x = wl.make_gqa(B=4, Hq=16, Hkv=4, D=D, seq_lens=lens, page_size=page_size, window=1000, n_sink=4,
                    sink_key_scale=4.0, seed=28 + page_size, name=f"swa_pages{page_size}_d{D}")
    check_full(x, 0)
    check_full(x, 3)


@pytest.mark.parametrize("window,n_sink,lens", [
    (64, 4, [1, 4, 60, 64, 65, 68, 69, 1000]),   # window >= L, sinks inside / overlapping / apart
    (16, 0, [15, 16, 17, 500]),
    (1, 3, [1, 2, 3, 4, 100]),
    (100, 4, [2000, 3333]),
])
@pytest.mark.parametrize("splits", [0, 2])
def test_window_and_sinks(window, n_sink, lens, splits):
    x = wl.make_gqa(B=len(lens), Hq=8, Hkv=2, D=128, seq_lens=lens, window=window, n_sink=n_sink,
                    sink_key_scale=4.0, seed=23, name=f"swa{window}_s{n_sink}")
    check_full(x, splits)


def test_empty_sequences():
    x = wl.make_gqa(B=3, Hq=8, Hkv=2, D=64, seq_lens=[0, 7, 0], seed=24, name="empty")
    got, lse = run_gpu(x)
    got = got.view(3, 8, 64)
    assert torch.all(got[0] == 0) and torch.all(got[2] == 0)
    lse = lse.view(3, 8)
    assert torch.all(torch.isinf(lse[0])) and torch.all(lse[0] < 0)
    check_full(x)


def test_window_of_whole_cache_equals_full_attention():
    full = wl.make_gqa(B=2, Hq=8, Hkv=2, D=128, seq_lens=[300, 301], seed=25)
    o_full, _ = run_gpu(full)
    full.window, full.n_sink = 301, 4
    o_win, _ = run_gpu(full)
    assert torch.equal(o_full, o_win)


def test_paged_equals_contiguous_bitwise():
    """Paging does not change the output ("All the attentions", section 8)."""
    p = wl.make_gqa(B=2, Hq=8, Hkv=2, D=128, seq_lens=[512, 512], page_size=16, paged=True, seed=26)
    c = wl.make_gqa(B=2, Hq=8, Hkv=2, D=128, seq_lens=[512, 512], paged=False, seed=26)
    assert torch.equal(p.k, c.k)
    op, _ = run_gpu(p, 4)
    oc, _ = run_gpu(c, 4)
    assert torch.equal(op, oc)


def test_aliased_pages():
    """Several sequences may point at the same physical pages (copy-on-write prefixes)."""
    x = wl.make_gqa(B=2, Hq=8, Hkv=2, D=128, seq_lens=[64, 64], page_size=16, seed=27)
    x.page_table[1] = x.page_table[0]
    x.k[1] = x.k[0]
    x.v[1] = x.v[0]
    got, _ = run_gpu(x)
    got = got.view(2, 8, 128)
    want, _ = oracle.gqa(x.q, x.k, x.v, x.seq_lens)
    assert_rows_close(got.reshape(-1, 128), want, TOL_BF16)


def test_workspace_needs_no_initialisation_and_is_reusable():
    """Garbage in the workspace and back-to-back calls that share it, with
    different split counts, all give the oracle's result."""
    x = wl.make_gqa(B=3, Hq=16, Hkv=4, D=128, seq_lens=[700, 1, 2222], seed=29, name="ws")
    want, _ = oracle.gqa(x.q, x.k, x.v, x.seq_lens)
    ws = torch.full((1 << 22,), 0xFF, dtype=torch.uint8, device="cuda")
    for splits in (4, 4, 3, 8, 4):
        out, _ = api.decode_attn_gqa(dev(x.q), dev(x.k_cache), dev(x.v_cache), dev(x.seq_lens),
                                     dev(x.page_table), num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert_rows_close(out.float().cpu().reshape(-1, 128), want, TOL_BF16, f"splits {splits}")


def test_deterministic():
    x = wl.make_gqa(B=2, Hq=32, Hkv=8, D=128, seq_lens=[999, 2048], seed=28)
    a, _ = run_gpu(x)
    b, _ = run_gpu(x)
    assert torch.equal(a, b)


# --- full-size workloads, sampled rows, in the launch configuration the benchmark times ---

@pytest.fixture(scope="module")
def cfg2():
    say("[gqa] generating Llama-3-8B-shaped layer: B16 32/8 heads D128 8192 tokens paged16")
    return wl.config2_llama3_8b_gqa()


def test_config2_full_size_sampled(cfg2):
    x = cfg2
    got, glse = run_gpu(x)
    rows = rows_sample(x.B * x.Hq, 48, seed=2)
    want, wlse = oracle.gqa(x.q, x.k, x.v, x.seq_lens, rows=rows)
    assert_rows_close(got[rows], want, TOL_BF16, "config2")
    assert_lse_close(glse[rows], wlse, 1e-5, "config2")


def test_config2_split_invariance(cfg2):
    x = cfg2
    a, _ = run_gpu(x, 0)
    b, _ = run_gpu(x, 3)
    assert oracle.rel_err_rows(a, b) <= 2 * TOL_BF16


@pytest.mark.parametrize("window,n_sink", [(0, 0), (8192, 4)])
def test_gqa_long_context_sampled(window, n_sink):
    """Sequences of 131072 and 70001 tokens (Llama-3-8B heads, 16-token
    pages in a random order): many splits per (sequence, KV head); full
    attention, and an 8192-token window with 4 sinks."""
    x = wl.make_gqa(B=2, Hq=32, Hkv=8, D=128, seq_lens=[131072, 70001], window=window, n_sink=n_sink,
                    sink_key_scale=4.0 if n_sink else 1.0, seed=29, name=f"gqa_long_w{window}")
    say(f"[gqa] {x.name} lens={x.seq_lens.tolist()} window={window} sinks={n_sink}")
    got, glse = run_gpu(x)
    rows = rows_sample(x.B * x.Hq, 24, seed=6)
    want, wlse = oracle.gqa(x.q, x.k, x.v, x.seq_lens, window=window, n_sink=n_sink, scale=x.scale,
                            rows=rows)
    assert_rows_close(got[rows], want, TOL_BF16, x.name)
    assert_lse_close(glse[rows], wlse, 1e-5, x.name)


@pytest.fixture(scope="module")
def cfg3():
    say("[swa] generating window 4096 + 4 sinks: B32 32/8 heads D128 lens U[4096,32768] paged16")
    return wl.config3_swa_sinks()


def test_config3_full_size_sampled(cfg3):
    x = cfg3
    got, glse = run_gpu(x)
    rows = rows_sample(x.B * x.Hq, 48, seed=3)
    want, wlse = oracle.gqa(x.q, x.k, x.v, x.seq_lens, window=x.window, n_sink=x.n_sink,
                            scale=x.scale, rows=rows)
    assert_rows_close(got[rows], want, TOL_BF16, "config3")
    assert_lse_close(glse[rows], wlse, 1e-5, "config3")
