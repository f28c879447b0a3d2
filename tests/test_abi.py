"""The C-ABI library: it loads, exports what include/dattn.h declares, and
rejects malformed arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

from decode_attention_kv_flash_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    with open(os.path.join(ROOT, "include", "dattn.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"DATTN_EXPORT\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    syms = declared_symbols()
    for name in ("decode_attn_gqa", "decode_attn_mla", "dsa_indexer_topk", "sparse_mla_attn"):
        assert name in syms


def test_library_exports_every_declared_symbol():
    L = api.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name
    assert set(declared_symbols()) == set(api.EXPORTS)
    assert L.dattn_version() == 1


def _gqa(**kw):
    args = dict(q=256, k=256, v=256, seq_lens=256, page_table=None, window=0, n_sink=0, out=256, lse=None,
                B=2, Hq=8, Hkv=2, D=128, page_size=16, max_pages=4, dtype=1, scale=0.0,
                num_splits=0, ws=None, ws_bytes=0)
    args.update(kw)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return api.lib().decode_attn_gqa(
        P(args["q"]), P(args["k"]), P(args["v"]), P(args["seq_lens"]), P(args["page_table"]),
        args["window"], args["n_sink"], P(args["out"]), P(args["lse"]), args["B"], args["Hq"],
        args["Hkv"], args["D"], args["page_size"], args["max_pages"], args["dtype"],
        args["scale"], args["num_splits"], P(args["ws"]), args["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1),
    (dict(seq_lens=None), -1),
    (dict(out=None), -1),
    (dict(B=0), -1),
    (dict(Hq=6, Hkv=4), -1),          # not a multiple
    (dict(Hq=48, Hkv=2), -2),         # group 24 not built
    (dict(D=96), -2),
    (dict(dtype=7), -2),
    (dict(page_table=256, page_size=24), -2),  # paged needs power-of-two pages
    (dict(page_table=256, max_pages=0), -1),
    (dict(n_sink=-1), -1),
    (dict(num_splits=-3), -1),
    (dict(scale=float("nan")), -1),
    (dict(page_table=256, num_splits=8), -3),  # 8 splits need a workspace
    (dict(k=264), -1),                          # not 16-byte aligned
    (dict(out=258), -1),
])
def test_gqa_validation(kw, code):
    rc = _gqa(**kw)
    assert rc == code, api.lib().dattn_last_error()
    assert api.lib().dattn_last_error()


def test_gqa_workspace_sizes():
    L = api.lib()
    # one split: no workspace
    assert L.decode_attn_gqa_workspace(2, 4, 2, 64, 256, 1, 0, 0, 1) == 0
    # explicit 8 splits on 16 x 32 heads x 128: o and lse partials, each 256-aligned
    n = L.decode_attn_gqa_workspace(16, 32, 8, 128, 16, 512, 0, 0, 8)
    assert n == 16 * 32 * 8 * 128 * 4 + 16 * 32 * 8 * 4
    # window + sinks cap the planned splits below the cache capacity
    full = L.decode_attn_gqa_workspace(32, 32, 8, 128, 16, 2048, 0, 0, 0)
    win = L.decode_attn_gqa_workspace(32, 32, 8, 128, 16, 2048, 64, 4, 0)
    assert win <= full


def test_mla_and_sparse_validation():
    L = api.lib()
    P = ctypes.c_void_p
    # bad latent width
    rc = L.decode_attn_mla(P(256), P(256), P(256), None, P(256), None, 2, 128, 256, 64, 100, 100, 1, 1,
                           0.0, 0, None, 0, None)
    assert rc == -2
    # fp32 MLA is not built
    rc = L.decode_attn_mla(P(256), P(256), P(256), None, P(256), None, 2, 128, 512, 64, 100, 100, 1, 0,
                           0.0, 0, None, 0, None)
    assert rc == -2
    # the latent cache must be 16-byte aligned
    rc = L.decode_attn_mla(P(256), P(258), P(256), None, P(256), None, 2, 128, 512, 64, 100, 100, 1, 1,
                           0.0, 0, None, 0, None)
    assert rc == -1
    # heads not a multiple of 64
    rc = L.decode_attn_mla(P(256), P(256), P(256), None, P(256), None, 2, 96, 512, 64, 100, 100, 1, 1,
                           0.0, 0, None, 0, None)
    assert rc == -2
    # paged: S_max must be the capacity page_size * max_pages, the quantity
    # decode_attn_mla_workspace plans from
    rc = L.decode_attn_mla(P(256), P(256), P(256), P(256), P(256), None, 2, 128, 512, 64, 100, 16, 8, 1,
                           0.0, 0, P(256), 1 << 30, None)
    assert rc == -1 and b"page_size * max_pages" in L.dattn_last_error()
    # sparse: k must be >= 1 and idx non-null
    rc = L.sparse_mla_attn(P(256), P(256), None, 16, P(256), None, 2, 128, 512, 64, 100, 1, 0.0, 0,
                           None, 0, None)
    assert rc == -1
    rc = L.sparse_mla_attn(P(256), P(256), P(256), 0, P(256), None, 2, 128, 512, 64, 100, 1, 0.0, 0,
                           None, 0, None)
    assert rc == -1


def test_mla_plan_stays_in_one_round_of_workgroups():
    """The MLA split grid, read back from the workspace size (rows x splits x
    (512 + 2) fp32) of 64-head calls, which always take it, on the 256-CU
    default the library assumes without a device: at most one workgroup per
    CU for every batch size (a count rounded up gave 258 workgroups at 6
    sequences), splits of at least 320 tokens, and never more than the
    3840-token split capacity allows.  128-head calls reserve room for
    balanced items too: one per CU plus one per sequence."""
    L = api.lib()
    S = 16384
    for B in list(range(1, 65)) + [96, 128, 255, 256, 300]:
        rows = B * 64
        nb = L.decode_attn_mla_workspace(B, 64, 512, S, 0)
        assert nb % (rows * 2056) == 0
        splits = nb // (rows * 2056)
        assert splits >= (S + 3839) // 3840
        assert splits * 320 <= S + 319
        if B <= 256 and splits > (S + 3839) // 3840:
            assert B * splits <= 256, (B, splits)
    # 8 to 32 sequences of 16384 tokens keep 256 / B splits; 64 take the 5
    # that the split capacity needs
    for B, want in ((8, 32), (16, 16), (32, 8), (64, 5)):
        assert L.decode_attn_mla_workspace(B, 64, 512, S, 0) == B * 64 * 2056 * want
    for B in (1, 6, 32, 512):
        assert L.decode_attn_mla_workspace(B, 128, 512, S, 0) >= (256 + B) * 128 * 2056


def test_dsa_validation():
    L = api.lib()
    P = ctypes.c_void_p
    args = lambda **kw: dict(dict(k=2048, Hi=64, Di=128, dt=1), **kw)
    def call(a, scores=None, ws=None, ws_bytes=0):
        return L.dsa_indexer_topk(P(256), P(256), P(256), P(256), a["k"], P(256), scores, 8, a["Hi"],
                                  a["Di"], 65536, a["dt"], ws, ws_bytes, None)
    assert call(args(k=0)) == -1
    assert call(args(k=20000)) == -1
    assert call(args(Di=64)) == -2
    assert call(args(Hi=48)) == -2
    assert call(args(dt=0)) == -2
    assert call(args()) == -3                     # no scores buffer, no workspace
    assert L.dsa_indexer_topk(P(264), P(256), P(256), P(256), 2048, P(256), None, 8, 64, 128, 65536, 1,
                              None, 0, None) == -1   # q_i not 16-byte aligned
    assert call(args(), scores=P(256)) == -3        # the selection always needs one
    # top-k workspace per row: 4 x 256 + 1 words per 2048-token chunk + 8, rounded to 64 words
    topk_ws = 8 * (((32 * 1025 + 8) + 63) // 64 * 64) * 4
    assert L.dsa_topk_workspace(8, 65536, 2048) == topk_ws
    assert L.dsa_indexer_topk_workspace(8, 65536, 2048) == 8 * 65536 * 4 + topk_ws
    assert L.dsa_topk(P(256), P(256), 0, P(256), 8, 100, None, 0, None) == -1
    assert L.dsa_topk(None, P(256), 4, P(256), 8, 100, None, 0, None) == -1
    assert L.dsa_topk(P(256), P(256), 4, P(256), 70000, 100, None, 0, None) == -1   # B > 65535
    assert L.dsa_topk(P(256), P(256), 4, P(256), 8, (1 << 30) + 1, None, 0, None) == -1
    assert L.dsa_topk(P(256), P(256), 4, P(256), 8, 100, None, 0, None) == -3     # no workspace
    assert L.dsa_topk(P(256), P(256), 4, P(256), 8, 100, P(256), 16, None) == -3  # too small


def test_profile_calls_without_gpu():
    api.profile_enable(True)
    api.profile_reset()
    assert api.profile_read("gqa") == (0.0, 0)
    api.profile_enable(False)


def _append(**kw):
    args = dict(k_new=256, v_new=256, k_cache=256, v_cache=256, positions=256, page_table=None,
                B=2, Hkv=8, D=128, page_size=16, max_pages=4, ring=0, fixed=0, dtype=1)
    args.update(kw)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return api.lib().kv_append_gqa(
        P(args["k_new"]), P(args["v_new"]), P(args["k_cache"]), P(args["v_cache"]),
        P(args["positions"]), P(args["page_table"]), args["B"], args["Hkv"], args["D"],
        args["page_size"], args["max_pages"], args["ring"], args["fixed"], args["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(k_new=None), -1),
    (dict(positions=None), -1),
    (dict(v_cache=264), -1),                 # not 16-byte aligned
    (dict(B=0), -1),
    (dict(Hkv=0), -1),
    (dict(dtype=5), -2),
    (dict(D=4), -2),                         # a row of 8 bytes
    (dict(D=100), -2),                       # 200 bytes, not a multiple of 16
    (dict(page_table=256, page_size=24), -2),
    (dict(page_table=256, max_pages=0), -1),
    (dict(ring=3), -1),                      # rolling buffer without a page table
    (dict(page_table=256, ring=-1), -1),
])
def test_append_validation(kw, code):
    rc = _append(**kw)
    assert rc == code, api.lib().dattn_last_error()
    assert api.lib().dattn_last_error()


def test_append_rows_validation():
    L = api.lib()
    P = ctypes.c_void_p
    # a latent row of 577 bf16 values is not a multiple of 16 bytes
    assert L.kv_append_rows(P(256), P(256), P(256), None, 2, 577, 100, 1, 1, None) == -2
    assert L.kv_append_rows(None, P(256), P(256), None, 2, 576, 100, 1, 1, None) == -1


def _quest(**kw):
    args = dict(q=256, k=256, v=256, kmm=256, seq_lens=256, page_table=256, budget=8, out=256,
                lse=None, sel=None, B=2, Hq=8, Hkv=2, D=128, page_size=16, max_pages=64, dtype=1,
                scale=0.0, num_splits=0, ws=None, ws_bytes=0)
    args.update(kw)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return api.lib().decode_attn_quest(
        P(args["q"]), P(args["k"]), P(args["v"]), P(args["kmm"]), P(args["seq_lens"]),
        P(args["page_table"]), args["budget"], P(args["out"]), P(args["lse"]), P(args["sel"]),
        args["B"], args["Hq"], args["Hkv"], args["D"], args["page_size"], args["max_pages"],
        args["dtype"], args["scale"], args["num_splits"], P(args["ws"]), args["ws_bytes"], None)


# Every case fails before a launch: the last ones for want of a workspace.
@pytest.mark.parametrize("kw,code", [
    (dict(kmm=None), -1),
    (dict(q=None), -1),
    (dict(budget=0), -1),
    (dict(budget=16385), -1),
    (dict(page_size=8), -2),                 # a 16-token block would straddle pages
    (dict(kmm=260), -1),                     # summaries not 16-byte aligned
    (dict(D=96), -2),
    (dict(Hq=48, Hkv=2), -2),
    (dict(B=4096, Hq=32, Hkv=8), -1),        # B * Hq rows above the select's grid
    (dict(), -3),                            # bounds, select and partials need a workspace
    (dict(page_table=None, page_size=1000, max_pages=1), -3),
])
def test_quest_validation(kw, code):
    rc = _quest(**kw)
    assert rc == code, api.lib().dattn_last_error()
    assert api.lib().dattn_last_error()


def test_quest_minmax_validation():
    L = api.lib()
    P = ctypes.c_void_p
    # k_cache, seq_lens, page_table, kminmax, first_block, B, Hkv, D, page_size, max_pages, dtype
    assert L.quest_page_minmax(None, P(256), None, P(256), 0, 2, 2, 128, 64, 1, 1, None) == -1
    assert L.quest_page_minmax(P(256), P(256), None, P(256), -1, 2, 2, 128, 64, 1, 1, None) == -1
    assert L.quest_page_minmax(P(256), P(256), P(256), P(256), 0, 2, 2, 128, 8, 4, 1, None) == -2
    assert L.quest_page_minmax(P(256), P(256), None, P(256), 0, 2, 2, 128, 64, 1, 2, None) == -2


def test_quest_workspace_sizes():
    L = api.lib()
    # rows x blocks fp32 bounds + per-row counts + selection + select workspace + partials
    one = L.decode_attn_quest_workspace(2, 8, 2, 128, 16, 64, 8, 1, 1)
    more = L.decode_attn_quest_workspace(2, 8, 2, 128, 16, 64, 8, 1, 4)
    assert one >= 16 * 64 * 4 + 16 * 4 + 16 * 8 * 4
    assert more - one == 16 * 4 * 128 * 4 + 256    # the split partials (o, then lse aligned)
    assert L.decode_attn_quest_workspace(0, 8, 2, 128, 16, 64, 8, 1, 1) == 0


# --------------------------------------------------------------------------
# debug checking of the device-resident tables, on host arrays


def _tables(lens, pt=None):
    i32 = ctypes.c_int32
    L = (i32 * len(lens))(*lens)
    if pt is None:
        return L, None
    flat = [e for row in pt for e in row]
    return L, (i32 * len(flat))(*flat)


@pytest.mark.parametrize("lens,pt,page_size,max_pages,num_pages,ok,what", [
    ([32, 17], [[3, 1], [0, 2]], 16, 2, 4, True, ""),
    ([32, 0], [[3, 1], [-1, -1]], 16, 2, 4, True, ""),             # an empty sequence uses no page
    ([17, 16], [[0, 5], [1, -7]], 16, 2, 6, True, ""),             # entries past the length are never read
    ([33, 16], [[0, 1], [2, 3]], 16, 2, 4, False, "seq_lens[0] = 33"),
    ([-1, 16], [[0, 1], [2, 3]], 16, 2, 4, False, "seq_lens[0] = -1"),
    ([32, 17], [[3, 1], [0, 4]], 16, 2, 4, False, "page_table[1][1] = 4"),
    ([32, 17], [[3, -2], [0, 2]], 16, 2, 4, False, "page_table[0][1] = -2"),
    ([32, 17], [[3, -2], [0, 2]], 16, 2, -1, False, "page_table[0][1] = -2"),
    ([32, 17], [[3, 99], [0, 2]], 16, 2, -1, True, ""),            # page count unknown: only >= 0
    ([256, 100], None, 256, 1, -1, True, ""),                      # contiguous: L <= S_max
    ([257, 100], None, 256, 1, -1, False, "seq_lens[0] = 257"),
])
def test_check_tables(lens, pt, page_size, max_pages, num_pages, ok, what):
    L = api.lib()
    sl, tab = _tables(lens, pt)
    rc = L.dattn_check_tables(sl, tab, len(lens), page_size, max_pages, num_pages)
    if ok:
        assert rc == 0, L.dattn_last_error()
    else:
        assert rc == -1 and what.encode() in L.dattn_last_error(), L.dattn_last_error()


def test_debug_toggle_without_gpu():
    L = api.lib()
    assert L.dattn_debug_enable(1) == 0
    assert L.dattn_debug_enable(0) == 0
