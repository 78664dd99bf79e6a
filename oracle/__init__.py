"""Double-precision CPU oracle of the DashAttention forward pass (ctypes binding).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; the product package never does.
The arithmetic lives in ``dash_oracle.c`` (see its header for the equations it follows, from
"DashAttention: Differentiable and Adaptive Sparse Hierarchical Attention", arXiv 2605.18753v1).

Inputs are numpy arrays or CPU torch tensors in float32 or bfloat16; both reach the C code
unchanged (bf16 as raw 16-bit patterns) and convert to double exactly there.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dash_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP over query rows)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i, d, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_int64
        L.orc_pool_keys.argtypes = [vp, i, i, i, i, i, i, vp]
        L.orc_pool_keys_query.argtypes = [vp, i, vp, i, i, i, i, i, vp]
        L.orc_pool_keys_query_ex.argtypes = [vp, i, vp, i64, i64, i, i, i, i, i, vp]
        L.orc_pool_keys_query_backward.argtypes = [vp, i, vp, i64, i64, vp, i, i, i, i, i, vp, vp]
        L.orc_entmax_tau_sort.argtypes = [vp, i, d]
        L.orc_entmax_tau_sort.restype = d
        L.orc_entmax_tau_bisect.argtypes = [vp, i, d, i]
        L.orc_entmax_tau_bisect.restype = d
        L.orc_entmax_tau.argtypes = [vp, i, d]
        L.orc_entmax_tau.restype = d
        L.orc_entmax_probs.argtypes = [vp, i, d, d, vp]
        L.orc_block_entmax.argtypes = [vp, i, vp, i, i, i, i, i, i, i, i, d, d, d, i, vp, i64,
                                       vp, vp, vp, vp, vp]
        L.orc_sparse_attn.argtypes = [vp, vp, vp, i, vp, vp, i, i, i, i, i, i, i, i, d, vp, i64,
                                      vp, vp]
        L.orc_sparse_attn_prior.argtypes = [vp, vp, vp, i, vp, i, i, i, i, i, i, i, i, d, d, vp,
                                            i64, vp]
        L.orc_backward.argtypes = [vp, vp, vp, i, vp, i, i, i, i, i, i, d, d, d, i, d, vp, vp, vp,
                                   vp]
        L.orc_sparse_attn_backward.argtypes = [vp, vp, vp, i, vp, vp, vp, i, i, i, i, i, i, d, vp,
                                               vp, vp, vp]
        L.orc_sparse_attn_backward_rows.argtypes = [vp, vp, vp, i, vp, vp, vp, i, i, i, i, i, i, d,
                                                    vp, ctypes.c_int64, vp, vp]
        L.orc_block_entmax_backward.argtypes = [vp, i, vp, vp, i, i, i, i, i, i, d, d, d, i, vp,
                                                ctypes.c_int64, vp, vp]
        L.orc_num_threads.restype = i
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().orc_num_threads())


def _host(a):
    """(contiguous numpy array, dtype code) for a numpy array or a CPU torch tensor."""
    if hasattr(a, "detach"):  # torch tensor
        import torch
        t = a.detach()
        if t.device.type != "cpu":
            raise ValueError("oracle inputs must live in host memory")
        t = t.contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16), BF16
        if t.dtype == torch.float32:
            return t.numpy(), F32
        if t.dtype == torch.float64:
            return t.numpy(), F64
        raise TypeError(f"unsupported dtype {t.dtype}")
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.float64:
        return a, F64
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"unsupported dtype {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, name: str):
    if rc != 0:
        raise ValueError(f"{name}: invalid arguments (rc={rc})")


def _rows(rows, total):
    if rows is None:
        return None, total
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if r.ndim != 1 or (r.size and (r.min() < 0 or r.max() >= total)):
        raise ValueError("rows out of range")
    return r, r.size


def pool_keys(k, block: int) -> np.ndarray:
    """Stage 0 at summary query zero: kbar [B, Tc, Hkv, D] (float64)."""
    ka, dt = _host(k)
    b, n, hkv, d = ka.shape
    out = np.zeros((b, n // block, hkv, d), dtype=np.float64)
    _check(lib().orc_pool_keys(_ptr(ka), dt, b, n, hkv, d, block, _ptr(out)), "pool_keys")
    return out


def pool_keys_query(k, qbar, block: int) -> np.ndarray:
    """Stage 0 with learned summary queries (Eq. 3): qbar [Hkv, D] (one per KV head), [Tc, Hkv, D]
    (one per chunk, Alg. 1) or [B, Tc, Hkv, D] (one per sequence and chunk)."""
    ka, dt = _host(k)
    qb = np.ascontiguousarray(np.asarray(qbar, dtype=np.float64))
    b, n, hkv, d = ka.shape
    tc = n // block
    if qb.shape == (hkv, d):
        sb, sc = 0, 0
    elif qb.shape == (tc, hkv, d):
        sb, sc = 0, hkv * d
    elif qb.shape == (b, tc, hkv, d):
        sb, sc = tc * hkv * d, hkv * d
    else:
        raise ValueError(f"qbar shape {qb.shape} is none of [Hkv, D], [Tc, Hkv, D], [B, Tc, Hkv, D]")
    out = np.zeros((b, tc, hkv, d), dtype=np.float64)
    _check(lib().orc_pool_keys_query_ex(_ptr(ka), dt, _ptr(qb), sb, sc, b, n, hkv, d, block,
                                        _ptr(out)), "pool_keys_query")
    return out


def _qbar_strides(qb, b, tc, hkv, d):
    if qb.shape == (hkv, d):
        return 0, 0
    if qb.shape == (tc, hkv, d):
        return 0, hkv * d
    if qb.shape == (b, tc, hkv, d):
        return tc * hkv * d, hkv * d
    raise ValueError(f"qbar shape {qb.shape} is none of [Hkv, D], [Tc, Hkv, D], [B, Tc, Hkv, D]")


def pool_keys_query_backward(k, qbar, dkbar, block: int) -> dict:
    """Gradients of Stage 0 with learned summary queries (Eq. 3) for dL/dkbar [B, Tc, Hkv, D]:
    dict(dk [B, n, Hkv, D], dqbar in qbar's shape, each summed over the chunks and sequences that
    share a query) in float64."""
    ka, dt = _host(k)
    qb = np.ascontiguousarray(np.asarray(qbar, dtype=np.float64))
    b, n, hkv, d = ka.shape
    tc = n // block
    sb, sc = _qbar_strides(qb, b, tc, hkv, d)
    dkb = np.ascontiguousarray(np.asarray(dkbar, dtype=np.float64).reshape(b, tc, hkv, d))
    dk = np.zeros((b, n, hkv, d))
    full = np.zeros((b, tc, hkv, d))
    _check(lib().orc_pool_keys_query_backward(_ptr(ka), dt, _ptr(qb), sb, sc, _ptr(dkb), b, n, hkv,
                                              d, block, _ptr(dk), _ptr(full)),
           "pool_keys_query_backward")
    if qb.shape == (hkv, d):
        dq = full.sum(axis=(0, 1))
    elif qb.shape == (tc, hkv, d):
        dq = full.sum(axis=0)
    else:
        dq = full
    return dict(dk=dk, dqbar=dq)


def entmax_tau(x, alpha: float, method: str = "auto", iters: int = 200) -> float:
    xa = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if method == "sort":
        return lib().orc_entmax_tau_sort(_ptr(xa), xa.size, alpha)
    if method == "bisect":
        return lib().orc_entmax_tau_bisect(_ptr(xa), xa.size, alpha, iters)
    return lib().orc_entmax_tau(_ptr(xa), xa.size, alpha)


def entmax(x, alpha: float, method: str = "auto") -> np.ndarray:
    """alpha-entmax of scores already multiplied by (alpha - 1), i.e. [x - tau]_+^(1/(alpha-1))."""
    xa = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    tau = entmax_tau(xa, alpha, method)
    p = np.zeros_like(xa)
    lib().orc_entmax_probs(_ptr(xa), xa.size, alpha, tau, _ptr(p))
    return p


def block_entmax(q, kbar, *, n_kv: int, block: int, alpha: float, gamma: float, sigma: float,
                 q_pos0: int = 0, h_kv: int | None = None, rows=None, window: int = 1):
    """Stage 1. Returns dict(mask uint32 [R,Hkv,W], bias [R,Hkv,Nc], tau [R,Hq], x [R,Hq,Nc],
    w [R,Hkv,Nc]) for the listed rows rho = b * n_q + t (all rows when rows is None).
    window: blocks always attended (the query's own and window - 1 before it, DA App. B.1.1)."""
    qa, dt = _host(q)
    kb = np.ascontiguousarray(np.asarray(kbar, dtype=np.float64))
    b, n_q, hq, d = qa.shape
    hkv = kb.shape[2] if h_kv is None else h_kv
    nc = math.ceil(n_kv / block)
    nw = math.ceil(nc / 32)
    r, nr = _rows(rows, b * n_q)
    mask = np.zeros((nr, hkv, nw), dtype=np.uint32)
    bias = np.zeros((nr, hkv, nc), dtype=np.float64)
    tau = np.zeros((nr, hq), dtype=np.float64)
    x = np.zeros((nr, hq, nc), dtype=np.float64)
    w = np.zeros((nr, hkv, nc), dtype=np.float64)
    _check(lib().orc_block_entmax(
        _ptr(qa), dt, _ptr(kb), b, n_q, q_pos0, n_kv, hq, hkv, d, block, alpha, gamma, sigma,
        int(window), None if r is None else _ptr(r), nr, _ptr(mask), _ptr(bias), _ptr(tau),
        _ptr(x), _ptr(w)),
        "block_entmax")
    return dict(mask=mask, bias=bias, tau=tau, x=x, w=w)


def sparse_attn(q, k, v, mask, bias, *, block: int, scale: float | None = None, q_pos0: int = 0,
                rows=None):
    """Stage 2, bias form. mask/bias are the compact per-row arrays block_entmax returns for the
    same rows. Returns (o [R, Hq, D], lse [R, Hq]) in float64."""
    qa, dt = _host(q)
    ka, dtk = _host(k)
    va, dtv = _host(v)
    if not (dt == dtk == dtv):
        raise TypeError("q, k, v must share a dtype")
    b, n_q, hq, d = qa.shape
    n_kv, hkv = ka.shape[1], ka.shape[2]
    r, nr = _rows(rows, b * n_q)
    m = np.ascontiguousarray(mask, dtype=np.uint32)
    bi = np.ascontiguousarray(bias, dtype=np.float64)
    nc = math.ceil(n_kv / block)
    if m.shape != (nr, hkv, math.ceil(nc / 32)) or bi.shape != (nr, hkv, nc):
        raise ValueError("mask/bias shape does not match the row list")
    o = np.zeros((nr, hq, d), dtype=np.float64)
    lse = np.zeros((nr, hq), dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(lib().orc_sparse_attn(
        _ptr(qa), _ptr(ka), _ptr(va), dt, _ptr(m), _ptr(bi), b, n_q, q_pos0, n_kv, hq, hkv, d,
        block, scale, None if r is None else _ptr(r), nr, _ptr(o), _ptr(lse)), "sparse_attn")
    return o, lse


def sparse_attn_prior(q, k, v, w, *, block: int, sigma: float, scale: float | None = None,
                      q_pos0: int = 0, rows=None) -> np.ndarray:
    """Stage 2, prior form (Eq. 7 with g of Eq. 8-10) from the GQA-averaged probabilities w."""
    qa, dt = _host(q)
    ka, _ = _host(k)
    va, _ = _host(v)
    b, n_q, hq, d = qa.shape
    n_kv, hkv = ka.shape[1], ka.shape[2]
    r, nr = _rows(rows, b * n_q)
    wa = np.ascontiguousarray(w, dtype=np.float64)
    o = np.zeros((nr, hq, d), dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(lib().orc_sparse_attn_prior(
        _ptr(qa), _ptr(ka), _ptr(va), dt, _ptr(wa), b, n_q, q_pos0, n_kv, hq, hkv, d, block,
        scale, sigma, None if r is None else _ptr(r), nr, _ptr(o)), "sparse_attn_prior")
    return o


def forward(q, k, v, *, block: int, alpha: float, gamma: float, sigma: float,
            scale: float | None = None, q_pos0: int = 0, rows=None, window: int = 1):
    """The whole forward pass for the listed rows: pool, route, attend (bias form)."""
    kbar = pool_keys(k, block)
    n_kv = (k.shape[1])
    st1 = block_entmax(q, kbar, n_kv=n_kv, block=block, alpha=alpha, gamma=gamma, sigma=sigma,
                       q_pos0=q_pos0, h_kv=k.shape[2], rows=rows, window=window)
    o, lse = sparse_attn(q, k, v, st1["mask"], st1["bias"], block=block, scale=scale,
                         q_pos0=q_pos0, rows=rows)
    return dict(kbar=kbar, o=o, lse=lse, **st1)


def backward(q, k, v, dout, *, block: int, alpha: float, gamma: float, sigma: float,
             window: int = 1, scale: float | None = None) -> dict:
    """Gradients of the prefill forward (pool, route, attend; every query row) for dL/do = dout
    [B, n, Hq, D]: dict(dq, dk, dv, dbias) in float64 (see orc_backward)."""
    qa, dt = _host(q)
    ka, dtk = _host(k)
    va, dtv = _host(v)
    if not (dt == dtk == dtv):
        raise TypeError("q, k, v must share a dtype")
    b, n, hq, d = qa.shape
    hkv = ka.shape[2]
    do = np.ascontiguousarray(np.asarray(dout, dtype=np.float64))
    if do.shape != qa.shape:
        raise ValueError("dout must have q's shape")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nc = math.ceil(n / block)
    dq = np.zeros((b, n, hq, d))
    dk = np.zeros((b, n, hkv, d))
    dv = np.zeros((b, n, hkv, d))
    dbias = np.zeros((b, n, hkv, nc))
    _check(lib().orc_backward(_ptr(qa), _ptr(ka), _ptr(va), dt, _ptr(do), b, n, hq, hkv, d, block,
                              alpha, gamma, sigma, int(window), scale, _ptr(dq), _ptr(dk), _ptr(dv),
                              _ptr(dbias)), "backward")
    return dict(dq=dq, dk=dk, dv=dv, dbias=dbias)


def sparse_attn_backward(q, k, v, mask, bias, dout, *, block: int, scale: float | None = None) -> dict:
    """Stage 2 gradients for prefill with the selection held fixed: mask [B, n, Hkv, W] uint32 and
    bias [B, n, Hkv, Nc] as Stage 1 writes them; dout [B, n, Hq, D]. Returns dict(dq, dk, dv,
    dbias) in float64 (dbias [B, n, Hkv, Nc], 0 off the routed chunks)."""
    qa, dt = _host(q)
    ka, _ = _host(k)
    va, _ = _host(v)
    b, n, hq, d = qa.shape
    hkv = ka.shape[2]
    nc = math.ceil(n / block)
    m = np.ascontiguousarray(np.asarray(mask).view(np.uint32).reshape(b * n, hkv, -1))
    bi = np.ascontiguousarray(np.asarray(bias, dtype=np.float64).reshape(b * n, hkv, nc))
    do = np.ascontiguousarray(np.asarray(dout, dtype=np.float64))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = np.zeros((b, n, hq, d))
    dk = np.zeros((b, n, hkv, d))
    dv = np.zeros((b, n, hkv, d))
    dbias = np.zeros((b, n, hkv, nc))
    _check(lib().orc_sparse_attn_backward(_ptr(qa), _ptr(ka), _ptr(va), dt, _ptr(m), _ptr(bi),
                                          _ptr(do), b, n, hq, hkv, d, block, scale, _ptr(dq),
                                          _ptr(dk), _ptr(dv), _ptr(dbias)), "sparse_attn_backward")
    return dict(dq=dq, dk=dk, dv=dv, dbias=dbias)


def sparse_attn_backward_rows(q, k, v, mask, bias, dout, rows, *, block: int,
                              scale: float | None = None) -> dict:
    """dq and dL/dd of the listed rows (rho = b * n + t) only, the selection held fixed: mask
    [R, Hkv, W], bias [R, Hkv, Nc] and dout [R, Hq, D] hold the listed rows in list order.
    Returns dict(dq [R, Hq, D], dbias [R, Hkv, Nc]) in float64."""
    qa, dt = _host(q)
    ka, _ = _host(k)
    va, _ = _host(v)
    b, n, hq, d = qa.shape
    hkv = ka.shape[2]
    nc = math.ceil(n / block)
    r, nr = _rows(rows, b * n)
    if r is None or nr == 0:
        raise ValueError("rows must list at least one row")
    m = np.ascontiguousarray(np.asarray(mask).view(np.uint32).reshape(nr, hkv, -1))
    bi = np.ascontiguousarray(np.asarray(bias, dtype=np.float64).reshape(nr, hkv, nc))
    do = np.ascontiguousarray(np.asarray(dout, dtype=np.float64).reshape(nr, hq, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = np.zeros((nr, hq, d))
    dbias = np.zeros((nr, hkv, nc))
    _check(lib().orc_sparse_attn_backward_rows(_ptr(qa), _ptr(ka), _ptr(va), dt, _ptr(m),
                                               _ptr(bi), _ptr(do), b, n, hq, hkv, d, block, scale,
                                               _ptr(r), nr, _ptr(dq), _ptr(dbias)),
           "sparse_attn_backward_rows")
    return dict(dq=dq, dbias=dbias)


def block_entmax_backward(q, kbar, dd, *, n_kv: int, block: int, alpha: float, gamma: float,
                          sigma: float, window: int = 1, rows=None, want_dkbar: bool = False):
    """Routing gradients for prefill with the selection held fixed: dd = dL/dd [R, Hkv, Nc] of
    the listed rows (all rows when rows is None). Returns dict(dq [R, Hq, D]: the routing part of
    dq, dkbar [B, Tc, Hkv, D] or None) in float64."""
    qa, dt = _host(q)
    kb = np.ascontiguousarray(np.asarray(kbar, dtype=np.float64))
    b, n, hq, d = qa.shape
    hkv = kb.shape[2]
    nc = math.ceil(n_kv / block)
    r, nr = _rows(rows, b * n)
    ddv = np.ascontiguousarray(np.asarray(dd, dtype=np.float64).reshape(nr, hkv, nc))
    dq = np.zeros((nr, hq, d))
    dkbar = np.zeros(kb.shape) if want_dkbar else None
    _check(lib().orc_block_entmax_backward(
        _ptr(qa), dt, _ptr(kb), _ptr(ddv), b, n, hq, hkv, d, block, alpha, gamma, sigma,
        int(window), None if r is None else _ptr(r), nr, _ptr(dq), _ptr(dkbar)),
        "block_entmax_backward")
    return dict(dq=dq, dkbar=dkbar)
