"""CPU oracle for decode attention over a KV cache -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library's product path never loads
it: the HIP path and the oracle share no code, and neither imports the other.
The only thing both sides use is the seeded input generator
(``decode_attention_kv_flash_amd.workloads``), which holds none of the
method's arithmetic.

The arithmetic lives in ``dattn_oracle.c`` (plain C, fp64 / int64, OpenMP over
output rows); this module compiles it with gcc and marshals torch CPU tensors
into it.  Closed-form byte and FLOP accounting lives in ``accounting.py``.

Parity status per function (what pins each one is listed in the tests):
  gqa        pinned (library SDPA in fp64, keep-list compaction, brute force)
  mla        pinned (expanded, un-absorbed MLA through library SDPA)
  indexer    pinned (hand-computed fixture, invariants, brute force); its fp8
             e4m3 decoding pinned code by code against torch.float8_e4m3fn
  topk       pinned (characterising invariants, brute force on tiny inputs)
  accounting pinned (numbers printed on the pages, tests/golden)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dattn_oracle.c")
_LIB = os.path.join(_HERE, "libdattn_oracle.so")
_lib = None

F32, BF16, FP8_E4M3 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math, no -march)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_gqa.argtypes = [P, P, P, I, I, I, I, I, I, P, I, I, D, P, I64, P, P]
        lib.oracle_gqa_sink.argtypes = [P, P, P, I, I, I, I, I, I, P, I, I, P, D, P, I64, P, P]
        lib.oracle_mla.argtypes = [P, P, I, I, I, I, I, I, P, P, I, D, P, I64, P, P]
        lib.oracle_indexer.argtypes = [P, P, P, I, I, I, I, I, P, P]
        lib.oracle_topk.argtypes = [P, I, I, I, P, I, P]
        lib.oracle_e4m3_value.argtypes = [I]
        lib.oracle_e4m3_value.restype = D
        for f in (lib.oracle_gqa, lib.oracle_gqa_sink, lib.oracle_mla, lib.oracle_indexer, lib.oracle_topk):
            f.restype = I
        _lib = lib
    return _lib


def threads() -> int:
    """Threads OpenMP will use (OMP_NUM_THREADS, else the cores of this host)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env:
        return int(env)
    return len(os.sched_getaffinity(0))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float8_e4m3fn:
        return FP8_E4M3
    raise TypeError(f"oracle takes fp32, bf16 or fp8 e4m3, got {t.dtype}")


def e4m3_value(code: int) -> float:
    """The oracle's decoding of one fp8 e4m3 byte (for pinning the decoder)."""
    return float(_load().oracle_e4m3_value(int(code)))


def _ptr(t: torch.Tensor):
    assert t.device.type == "cpu" and t.is_contiguous()
    return ctypes.c_void_p(t.data_ptr())


def _rows(rows):
    if rows is None:
        return None, 0
    r = torch.as_tensor(np.asarray(rows, dtype=np.int64)).contiguous()
    return r, r.numel()


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def gqa(q, k, v, seq_lens, *, window=0, n_sink=0, scale=None, rows=None, sink_logits=None):
    """Grouped-query decode attention in fp64.

    q [B,Hq,D]; k, v logical [B,Hkv,S_max,D] (fp32 or bf16, same dtype);
    sink_logits: None, or [Hq] per-head sink logits (an extra softmax
    denominator term exp(sink) with a zero value).
    Returns (out [n_rows, D] fp64, lse [n_rows] fp64) for flat rows b*Hq+h.
    """
    lib = _load()
    if sink_logits is not None:
        return _gqa_sink(lib, q, k, v, seq_lens, window, n_sink, scale, rows, sink_logits)
    B, Hq, D = q.shape
    _, Hkv, S_max, _ = k.shape
    assert k.dtype == v.dtype == q.dtype
    if scale is None:
        scale = D ** -0.5
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    sl = seq_lens.to(torch.int32).contiguous()
    r, n = _rows(rows)
    n_out = n if r is not None else B * Hq
    out = torch.empty(n_out, D, dtype=torch.float64)
    lse = torch.empty(n_out, dtype=torch.float64)
    rc = lib.oracle_gqa(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, D, S_max,
                        _ptr(sl), int(window), int(n_sink), float(scale),
                        _ptr(r) if r is not None else None, n, _ptr(out), _ptr(lse))
    _check(rc, "gqa")
    return out, lse


def _gqa_sink(lib, q, k, v, seq_lens, window, n_sink, scale, rows, sink_logits):
    B, Hq, D = q.shape
    _, Hkv, S_max, _ = k.shape
    assert k.dtype == v.dtype == q.dtype
    if scale is None:
        scale = D ** -0.5
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    sl = seq_lens.to(torch.int32).contiguous()
    sk = torch.as_tensor(sink_logits, dtype=torch.float64).contiguous()
    assert sk.shape == (Hq,)
    r, n = _rows(rows)
    n_out = n if r is not None else B * Hq
    out = torch.empty(n_out, D, dtype=torch.float64)
    lse = torch.empty(n_out, dtype=torch.float64)
    rc = lib.oracle_gqa_sink(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, D, S_max,
                             _ptr(sl), int(window), int(n_sink), _ptr(sk), float(scale),
                             _ptr(r) if r is not None else None, n, _ptr(out), _ptr(lse))
    _check(rc, "gqa_sink")
    return out, lse


def mla(q, latent, seq_lens=None, *, d_latent=512, scale=None, idx=None, rows=None):
    """Absorbed MLA decode attention in fp64 (dense, or over ``idx`` when given).

    q [B,H,Dc+Dr]; latent [B,S_max,Dc+Dr]; idx int32 [B,k] (-1 = empty slot).
    Returns (out [n_rows, Dc] fp64, lse [n_rows] fp64).
    """
    lib = _load()
    B, H, Dq = q.shape
    S_max = latent.shape[1]
    Dc, Dr = d_latent, Dq - d_latent
    if scale is None:
        scale = 1.0 / (192.0 ** 0.5)
    q, latent = q.contiguous(), latent.contiguous()
    sl = seq_lens.to(torch.int32).contiguous() if seq_lens is not None else None
    ix = idx.to(torch.int32).contiguous() if idx is not None else None
    k_sel = ix.shape[1] if ix is not None else 0
    r, n = _rows(rows)
    n_out = n if r is not None else B * H
    out = torch.empty(n_out, Dc, dtype=torch.float64)
    lse = torch.empty(n_out, dtype=torch.float64)
    rc = lib.oracle_mla(_ptr(q), _ptr(latent), _dtype_code(q), B, H, Dc, Dr, S_max,
                        _ptr(sl) if sl is not None else None,
                        _ptr(ix) if ix is not None else None, k_sel, float(scale),
                        _ptr(r) if r is not None else None, n, _ptr(out), _ptr(lse))
    _check(rc, "mla")
    return out, lse


def indexer(q_i, w, k_i, seq_lens):
    """Exact int64 indexer scores [B, S_max]; INT64_MIN past each sequence's end."""
    lib = _load()
    B, Hi, Di = q_i.shape
    S_max = k_i.shape[1]
    q_i, k_i = q_i.contiguous(), k_i.contiguous()
    w = w.to(torch.float32).contiguous()
    sl = seq_lens.to(torch.int32).contiguous()
    scores = torch.empty(B, S_max, dtype=torch.int64)
    rc = lib.oracle_indexer(_ptr(q_i), _ptr(w), _ptr(k_i), _dtype_code(q_i), B, Hi, Di, S_max,
                            _ptr(sl), _ptr(scores))
    _check(rc, "indexer")
    return scores


def topk(scores, seq_lens, k):
    """Top-k indices [B, k] int32, ascending, -1 padded; ties to the lower index."""
    lib = _load()
    B, S_max = scores.shape
    if scores.dtype == torch.int64:
        kind = 0
    elif scores.dtype == torch.float32:
        kind = 1
    else:
        raise TypeError("scores must be int64 or fp32")
    scores = scores.contiguous()
    sl = seq_lens.to(torch.int32).contiguous()
    idx = torch.empty(B, k, dtype=torch.int32)
    rc = lib.oracle_topk(_ptr(scores), kind, B, S_max, _ptr(sl), int(k), _ptr(idx))
    _check(rc, "topk")
    return idx


def rel_err_rows(x, y):
    """max over rows of ||x-y||_inf / ||y||_inf (rows of an [n, d] pair).

    Rows whose reference is all-zero (an empty token set) compare absolutely.
    """
    x = torch.as_tensor(x, dtype=torch.float64).reshape(-1, x.shape[-1])
    y = torch.as_tensor(y, dtype=torch.float64).reshape(-1, y.shape[-1])
    num = (x - y).abs().amax(dim=1)
    den = y.abs().amax(dim=1)
    den = torch.where(den > 0, den, torch.ones_like(den))
    return float((num / den).max()) if num.numel() else 0.0


def norm_rel_err(x, y):
    """||x-y||_2 / ||y||_2 over the whole output."""
    x = torch.as_tensor(x, dtype=torch.float64)
    y = torch.as_tensor(y, dtype=torch.float64)
    d = float(torch.linalg.vector_norm(y))
    return float(torch.linalg.vector_norm(x - y)) / (d if d > 0 else 1.0)
