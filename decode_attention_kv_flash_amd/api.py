"""Python binding of the dattn C ABI (include/dattn.h).

Argument marshalling only: every computation happens in the HIP kernels of
``libdattn.so``.  Torch supplies device memory (outputs, workspace) and the
current HIP stream.  There is no fallback: if the library is missing or a call
fails, this module raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdattn.so")

DATTN_F32, DATTN_BF16, DATTN_FP8_E4M3 = 0, 1, 2
STATUS = {0: "OK", -1: "EINVAL", -2: "EUNSUPPORTED", -3: "EWORKSPACE", -4: "EHIP"}

EXPORTS = (
    "decode_attn_gqa", "decode_attn_gqa_sink", "decode_attn_gqa_workspace", "decode_attn_gqa_noalloc",
    "decode_attn_mla", "decode_attn_mla_workspace",
    "dsa_indexer_topk", "dsa_indexer_topk_workspace",
    "dsa_topk", "dsa_topk_workspace",
    "sparse_mla_attn", "sparse_mla_attn_workspace",
    "kv_append_gqa", "kv_append_rows",
    "quest_page_minmax", "decode_attn_quest", "decode_attn_quest_workspace",
    "dattn_last_error", "dattn_version", "dattn_debug_enable", "dattn_check_tables",
    "dattn_profile_enable", "dattn_profile_read", "dattn_profile_reset", "dattn_stream_read_probe",
)

_lib = None


class DattnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dattn {STATUS.get(code, code)}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libdattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m decode_attention_kv_flash_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    L.decode_attn_gqa.argtypes = [P, P, P, P, P, I32, I32, P, P, I32, I32, I32, I32, I32, I32,
                                  I32, F, I32, P, SZ, P]
    L.decode_attn_gqa_sink.argtypes = [P, P, P, P, P, I32, I32, P, P, P, I32, I32, I32, I32, I32,
                                       I32, I32, F, I32, P, SZ, P]
    L.decode_attn_gqa_workspace.argtypes = [I32] * 9
    L.decode_attn_gqa_noalloc.argtypes = [P, P, P, P, P, I32, I32, P, P, P, I32, I32, I32, I32, I32,
                                          I32, I32, F, I32, P]
    L.kv_append_gqa.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, I32, P]
    L.kv_append_rows.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, P]
    L.quest_page_minmax.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, I32, I32, P]
    L.decode_attn_quest.argtypes = [P, P, P, P, P, P, I32, P, P, P, I32, I32, I32, I32, I32, I32,
                                    I32, F, I32, P, SZ, P]
    L.decode_attn_quest_workspace.argtypes = [I32] * 9
    L.decode_attn_mla.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, I32, F, I32,
                                  P, SZ, P]
    L.decode_attn_mla_workspace.argtypes = [I32] * 5
    L.dsa_indexer_topk.argtypes = [P, P, P, P, I32, P, P, I32, I32, I32, I32, I32, P, SZ, P]
    L.dsa_indexer_topk_workspace.argtypes = [I32] * 3
    L.dsa_topk.argtypes = [P, P, I32, P, I32, I32, P, SZ, P]
    L.dsa_topk_workspace.argtypes = [I32] * 3
    L.sparse_mla_attn.argtypes = [P, P, P, I32, P, P, I32, I32, I32, I32, I32, I32, F, I32, P, SZ, P]
    L.sparse_mla_attn_workspace.argtypes = [I32] * 5
    for name in ("decode_attn_gqa_workspace", "decode_attn_mla_workspace", "decode_attn_quest_workspace",
                 "dsa_indexer_topk_workspace", "dsa_topk_workspace", "sparse_mla_attn_workspace"):
        getattr(L, name).restype = SZ
    for name in ("decode_attn_gqa", "decode_attn_gqa_sink", "decode_attn_gqa_noalloc", "decode_attn_mla", "dsa_indexer_topk", "dsa_topk",
                 "kv_append_gqa", "kv_append_rows", "quest_page_minmax", "decode_attn_quest",
                 "sparse_mla_attn", "dattn_profile_enable", "dattn_profile_read",
                 "dattn_profile_reset"):
        getattr(L, name).restype = ctypes.c_int
    L.dattn_last_error.restype = ctypes.c_char_p
    L.dattn_last_error.argtypes = []
    L.dattn_version.restype = I32
    L.dattn_stream_read_probe.argtypes = [P, SZ, P, I32, I32, P]
    L.dattn_stream_read_probe.restype = ctypes.c_int
    L.dattn_debug_enable.argtypes = [I32]
    L.dattn_debug_enable.restype = ctypes.c_int
    L.dattn_check_tables.argtypes = [P, P, I32, I32, I32, ctypes.c_int64]
    L.dattn_check_tables.restype = ctypes.c_int
    L.dattn_profile_enable.argtypes = [I32]
    L.dattn_profile_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int64)]
    _lib = L
    return L


def _check(rc: int):
    if rc != 0:
        raise DattnError(rc, lib().dattn_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DATTN_F32
    if t.dtype == torch.bfloat16:
        return DATTN_BF16
    if t.dtype == torch.float8_e4m3fn:
        return DATTN_FP8_E4M3
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _empty(shape, dtype, device, stream) -> torch.Tensor:
    """torch.empty on the stream the call launches on.  The caching allocator
    ties a block to the stream it was allocated on, so a workspace freed when
    the binding returns is not handed to other streams' work while this
    call's kernels may still use it; outputs follow the same rule."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _workspace(nbytes: int, device, stream) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return _empty((nbytes,), torch.uint8, device, stream)


def decode_attn_gqa(q, k_cache, v_cache, seq_lens, page_table=None, window=0, n_sink=0, *,
                    scale=None, num_splits=0, out=None, lse=None, want_lse=True, workspace=None,
                    stream=None, sink_logits=None):
    """GQA / sliding-window + sinks decode attention.  Returns (out, lse).

    sink_logits: optional device fp32 [Hq] explicit sink logits (decode_attn_gqa_sink).
    """
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (seq_lens, "seq_lens")):
        _dev(t, n)
    if sink_logits is not None:
        _dev(sink_logits, "sink_logits")
        if sink_logits.dtype != torch.float32 or sink_logits.shape != (q.shape[1],):
            raise ValueError("sink_logits must be fp32 [Hq]")
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    page_size = k_cache.shape[2]
    if page_table is not None:
        _dev(page_table, "page_table")
        max_pages = page_table.shape[1]
    else:
        max_pages = 1
    if out is None:
        out = _empty(q.shape, q.dtype, q.device, stream)
    if lse is None and want_lse:
        lse = _empty((B, Hq), torch.float32, q.device, stream)
    nbytes = lib().decode_attn_gqa_workspace(B, Hq, Hkv, D, page_size, max_pages, int(window),
                                             int(n_sink), int(num_splits))
    if workspace is not None:
        _dev(workspace, "workspace")
        ws, nbytes = workspace, workspace.numel() * workspace.element_size()
    else:
        ws = _workspace(nbytes, q.device, stream)
    if sink_logits is None:
        _check(lib().decode_attn_gqa(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(page_table),
            int(window), int(n_sink), _ptr(out), _ptr(lse), B, Hq, Hkv, D, page_size, max_pages,
            _dtype_code(q), float(scale or 0.0), int(num_splits), _ptr(ws), nbytes, _stream(stream)))
    else:
        _check(lib().decode_attn_gqa_sink(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(page_table),
            int(window), int(n_sink), _ptr(sink_logits.contiguous()), _ptr(out), _ptr(lse), B, Hq,
            Hkv, D, page_size, max_pages, _dtype_code(q), float(scale or 0.0), int(num_splits),
            _ptr(ws), nbytes, _stream(stream)))
    return out, lse


def decode_attn_gqa_noalloc(q, k_cache, v_cache, seq_lens, page_table=None, window=0, n_sink=0, *,
                            out, lse=None, scale=None, num_splits=0, stream=None, sink_logits=None):
    """decode_attn_gqa whose split partials live in the library's own device
    array: the caller passes every output (out, and lse or None) and nothing
    is allocated.  Calls that overlap on one GPU race (one shared array)."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (seq_lens, "seq_lens"), (out, "out")):
        _dev(t, n)
    if lse is not None:
        _dev(lse, "lse")
    if sink_logits is not None:
        _dev(sink_logits, "sink_logits")
        if sink_logits.dtype != torch.float32 or sink_logits.shape != (q.shape[1],):
            raise ValueError("sink_logits must be fp32 [Hq]")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    B, Hq, D = q.shape
    Hkv, page_size = k_cache.shape[1], k_cache.shape[2]
    max_pages = 1
    if page_table is not None:
        _dev(page_table, "page_table")
        max_pages = page_table.shape[1]
    _check(lib().decode_attn_gqa_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(page_table), int(window), int(n_sink),
        _ptr(sink_logits), _ptr(out), _ptr(lse), B, Hq, Hkv, D, page_size, max_pages, _dtype_code(q),
        float(scale or 0.0), int(num_splits), _stream(stream)))
    return out, lse


def kv_append_gqa(k_new, v_new, k_cache, v_cache, positions, page_table=None, *, ring_pages=0,
                  fixed_pages=0, stream=None):
    """Write each sequence's new K/V rows [B, Hkv, D] at positions[b] of the
    (paged) caches; with ring_pages > 0 the page table is a rolling buffer."""
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (positions, "positions")):
        _dev(t, n)
    B, Hkv, D = k_new.shape
    page_size = k_cache.shape[2]
    max_pages = 1
    if page_table is not None:
        _dev(page_table, "page_table")
        max_pages = page_table.shape[1]
    _check(lib().kv_append_gqa(
        _ptr(k_new.contiguous()), _ptr(v_new.contiguous()), _ptr(k_cache), _ptr(v_cache),
        _ptr(positions), _ptr(page_table), B, Hkv, D, page_size, max_pages, int(ring_pages),
        int(fixed_pages), _dtype_code(k_new), _stream(stream)))


def kv_append_rows(rows_new, cache, positions, page_table=None, *, stream=None):
    """Write each sequence's new row [B, X] (MLA latent or indexer key) at
    positions[b] of a cache [pages, page_size, X] or [B, S_max, X]."""
    for t, n in ((rows_new, "rows_new"), (cache, "cache"), (positions, "positions")):
        _dev(t, n)
    B, X = rows_new.shape
    page_size = cache.shape[1]
    max_pages = 1
    if page_table is not None:
        _dev(page_table, "page_table")
        max_pages = page_table.shape[1]
    _check(lib().kv_append_rows(
        _ptr(rows_new.contiguous()), _ptr(cache), _ptr(positions), _ptr(page_table), B, X,
        page_size, max_pages, _dtype_code(rows_new), _stream(stream)))


QUEST_BLOCK = 16  # tokens per summarised block


def quest_page_minmax(k_cache, seq_lens, page_table=None, *, kminmax=None, first_block=0,
                      stream=None):
    """Per-block key summaries [B, Hkv, n_blocks, 2, D] (kmin, kmax) of a
    decode_attn_gqa K cache; blocks [first_block, L_b // 16) are (re)written.
    Returns kminmax (allocated when not given)."""
    for t, n in ((k_cache, "k_cache"), (seq_lens, "seq_lens")):
        _dev(t, n)
    Hkv, page_size, D = k_cache.shape[1], k_cache.shape[2], k_cache.shape[3]
    B = seq_lens.shape[0]
    max_pages = 1
    if page_table is not None:
        _dev(page_table, "page_table")
        max_pages = page_table.shape[1]
    n_blocks = page_size * max_pages // QUEST_BLOCK
    if kminmax is None:
        kminmax = _empty((B, Hkv, n_blocks, 2, D), k_cache.dtype, k_cache.device, stream)
    else:
        _dev(kminmax, "kminmax")
        if tuple(kminmax.shape) != (B, Hkv, n_blocks, 2, D) or kminmax.dtype != k_cache.dtype:
            raise ValueError(f"kminmax must be {k_cache.dtype} [{B}, {Hkv}, {n_blocks}, 2, {D}]")
    _check(lib().quest_page_minmax(
        _ptr(k_cache), _ptr(seq_lens), _ptr(page_table), _ptr(kminmax), int(first_block), B, Hkv, D,
        page_size, max_pages, _dtype_code(k_cache), _stream(stream)))
    return kminmax


def decode_attn_quest(q, k_cache, v_cache, kminmax, seq_lens, budget, page_table=None, *,
                      scale=None, num_splits=0, out=None, lse=None, want_lse=True,
                      want_selected=False, workspace=None, stream=None):
    """Quest decode: per query head the `budget` 16-token blocks with the
    largest key bounds plus the partial last block.  Returns (out, lse) or,
    with want_selected, (out, lse, selected [B, Hq, budget] int32, -1 padded)."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (kminmax, "kminmax"),
                 (seq_lens, "seq_lens")):
        _dev(t, n)
    B, Hq, D = q.shape
    Hkv, page_size = k_cache.shape[1], k_cache.shape[2]
    max_pages = 1
    if page_table is not None:
        _dev(page_table, "page_table")
        max_pages = page_table.shape[1]
    if kminmax.dtype != k_cache.dtype or kminmax.shape[:2] != (B, Hkv):
        raise ValueError("kminmax must come from quest_page_minmax on this cache")
    if out is None:
        out = _empty(q.shape, q.dtype, q.device, stream)
    if lse is None and want_lse:
        lse = _empty((B, Hq), torch.float32, q.device, stream)
    sel = _empty((B, Hq, int(budget)), torch.int32, q.device, stream) if want_selected else None
    dt = _dtype_code(q)
    nbytes = lib().decode_attn_quest_workspace(B, Hq, Hkv, D, page_size, max_pages, int(budget), dt,
                                               int(num_splits))
    if workspace is not None:
        _dev(workspace, "workspace")
        ws, nbytes = workspace, workspace.numel() * workspace.element_size()
    else:
        ws = _workspace(nbytes, q.device, stream)
    _check(lib().decode_attn_quest(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kminmax), _ptr(seq_lens), _ptr(page_table),
        int(budget), _ptr(out), _ptr(lse), _ptr(sel), B, Hq, Hkv, D, page_size, max_pages, dt,
        float(scale or 0.0), int(num_splits), _ptr(ws), nbytes, _stream(stream)))
    return (out, lse, sel) if want_selected else (out, lse)


def decode_attn_mla(q_absorbed, latent_cache, seq_lens, page_table=None, *, d_latent=512,
                    scale=None, num_splits=0, out=None, lse=None, want_lse=True, workspace=None,
                    stream=None):
    """Absorbed MLA decode attention.  latent_cache [B, S_max, 576] (contiguous)
    or [num_pages, page_size, 576] with page_table.  Returns (out [B,H,512], lse)."""
    for t, n in ((q_absorbed, "q_absorbed"), (latent_cache, "latent_cache"), (seq_lens, "seq_lens")):
        _dev(t, n)
    B, H, Dq = q_absorbed.shape
    d_rope = Dq - d_latent
    if page_table is not None:
        _dev(page_table, "page_table")
        page_size, max_pages = latent_cache.shape[1], page_table.shape[1]
        S_max = page_size * max_pages
    else:
        S_max, page_size, max_pages = latent_cache.shape[1], latent_cache.shape[1], 1
    if out is None:
        out = _empty((B, H, d_latent), q_absorbed.dtype, q_absorbed.device, stream)
    if lse is None and want_lse:
        lse = _empty((B, H), torch.float32, q_absorbed.device, stream)
    nbytes = lib().decode_attn_mla_workspace(B, H, d_latent, S_max, int(num_splits))
    if workspace is not None:
        _dev(workspace, "workspace")
        ws, nbytes = workspace, workspace.numel() * workspace.element_size()
    else:
        ws = _workspace(nbytes, q_absorbed.device, stream)
    _check(lib().decode_attn_mla(
        _ptr(q_absorbed), _ptr(latent_cache), _ptr(seq_lens), _ptr(page_table), _ptr(out),
        _ptr(lse), B, H, d_latent, d_rope, S_max, page_size, max_pages, _dtype_code(q_absorbed),
        float(scale or 0.0), int(num_splits), _ptr(ws), nbytes, _stream(stream)))
    return out, lse


def dsa_indexer_topk(q_i, w, k_i_cache, seq_lens, k, *, topk_idx=None, return_scores=False,
                     workspace=None, stream=None):
    """Indexer scores + top-k.  Returns topk_idx [B,k] (and scores [B,S_max])."""
    for t, n in ((q_i, "q_i"), (w, "w"), (k_i_cache, "k_i_cache"), (seq_lens, "seq_lens")):
        _dev(t, n)
    if w.dtype != torch.float32:
        raise ValueError("w must be fp32")
    B, Hi, Di = q_i.shape
    S_max = k_i_cache.shape[1]
    if q_i.dtype != k_i_cache.dtype:
        raise ValueError("q_i and k_i_cache must have one dtype")
    if topk_idx is None:
        topk_idx = _empty((B, k), torch.int32, q_i.device, stream)
    scores = _empty((B, S_max), torch.float32, q_i.device, stream) if return_scores else None
    nbytes = lib().dsa_indexer_topk_workspace(B, S_max, k)
    if workspace is not None:
        _dev(workspace, "workspace")
        ws, nbytes = workspace, workspace.numel() * workspace.element_size()
    else:
        ws = _workspace(nbytes, q_i.device, stream)
    _check(lib().dsa_indexer_topk(
        _ptr(q_i), _ptr(w), _ptr(k_i_cache), _ptr(seq_lens), int(k), _ptr(topk_idx), _ptr(scores),
        B, Hi, Di, S_max, _dtype_code(q_i), _ptr(ws), nbytes, _stream(stream)))
    return (topk_idx, scores) if return_scores else topk_idx


def dsa_topk(scores, seq_lens, k, *, topk_idx=None, workspace=None, stream=None):
    """Top-k of fp32 scores [B, S_max]; ties to the lower index; ascending; -1 padded."""
    _dev(scores, "scores")
    _dev(seq_lens, "seq_lens")
    if scores.dtype != torch.float32:
        raise ValueError("scores must be fp32")
    B, S_max = scores.shape
    if topk_idx is None:
        topk_idx = _empty((B, k), torch.int32, scores.device, stream)
    nbytes = lib().dsa_topk_workspace(B, S_max, k)
    if workspace is not None:
        _dev(workspace, "workspace")
        ws, nbytes = workspace, workspace.numel() * workspace.element_size()
    else:
        ws = _workspace(nbytes, scores.device, stream)
    _check(lib().dsa_topk(_ptr(scores), _ptr(seq_lens), int(k), _ptr(topk_idx), B, S_max,
                          _ptr(ws), nbytes, _stream(stream)))
    return topk_idx


def sparse_mla_attn(q, latent_cache, topk_idx, *, d_latent=512, scale=None, num_splits=0,
                    out=None, lse=None, want_lse=True, workspace=None, stream=None):
    """MLA over the rows listed in topk_idx [B,k] (-1 = skip).  Returns (out, lse)."""
    for t, n in ((q, "q"), (latent_cache, "latent_cache"), (topk_idx, "topk_idx")):
        _dev(t, n)
    B, H, Dq = q.shape
    S_max = latent_cache.shape[1]
    k = topk_idx.shape[1]
    if out is None:
        out = _empty((B, H, d_latent), q.dtype, q.device, stream)
    if lse is None and want_lse:
        lse = _empty((B, H), torch.float32, q.device, stream)
    nbytes = lib().sparse_mla_attn_workspace(B, H, d_latent, k, int(num_splits))
    if workspace is not None:
        _dev(workspace, "workspace")
        ws, nbytes = workspace, workspace.numel() * workspace.element_size()
    else:
        ws = _workspace(nbytes, q.device, stream)
    _check(lib().sparse_mla_attn(
        _ptr(q), _ptr(latent_cache), _ptr(topk_idx), k, _ptr(out), _ptr(lse), B, H, d_latent,
        Dq - d_latent, S_max, _dtype_code(q), float(scale or 0.0), int(num_splits), _ptr(ws),
        nbytes, _stream(stream)))
    return out, lse


# ---- debug checking of the device-resident tables ---------------------------

def debug_enable(on: bool = True):
    """Check seq_lens / page_table on the host before each launch (synchronous)."""
    _check(lib().dattn_debug_enable(1 if on else 0))


# ---- per-kernel timing (HIP events recorded inside the library) -------------

def profile_enable(on: bool = True):
    _check(lib().dattn_profile_enable(1 if on else 0))


def profile_reset():
    _check(lib().dattn_profile_reset())


def profile_read(name: str = ""):
    """(total milliseconds, launch count) of kernels whose name contains ``name``."""
    tot, cnt = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(lib().dattn_profile_read(name.encode() if name else None, ctypes.byref(tot),
                                    ctypes.byref(cnt)))
    return tot.value, cnt.value
