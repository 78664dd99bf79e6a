"""libdash: the DashAttention forward pass on AMD Instinct MI355X (gfx950).

A thin ctypes binding of the C ABI in ``include/dash.h``; the functions carry the C names.
Arguments are torch tensors on the GPU: torch only supplies device memory and the current HIP
stream, every step of the computation runs in libdash's own kernels. There is no fallback: if
``libdash.so`` is not built, or an argument is rejected, a call raises.

Method: "DashAttention: Differentiable and Adaptive Sparse Hierarchical Attention"
(arXiv 2605.18753v1), Stage 0 (§3.1), Stage 1 (§3.2) and Stage 2 (§3.3-3.4, Prop. 1).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "DashError", "lib", "library_path",
    "dash_pool_keys", "dash_pool_keys_query", "dash_pool_keys_append", "dash_block_entmax",
    "dash_pool_keys_query_ex", "dash_pool_keys_append_ex",
    "dash_block_entmax_ex", "dash_block_entmax_workspace_bytes", "dash_sparse_attn_prefill",
    "dash_sparse_attn_prefill_ex",
    "dash_decode_workspace_bytes", "dash_sparse_attn_decode", "dash_sparse_attn_decode_varlen",
    "dash_sparse_attn_backward_workspace_bytes", "dash_sparse_attn_prefill_backward",
    "dash_block_entmax_backward_workspace_bytes", "dash_block_entmax_backward",
    "dash_block_entmax_backward_query_workspace_bytes", "dash_block_entmax_backward_query",
    "dash_decode_step_workspace_bytes", "dash_decode_step", "dash_decode_step_noalloc",
    "dash_version", "backward", "forward", "decode_step",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libdash.so")
_lib = None

DASH_F32, DASH_BF16 = 0, 1


class DashError(RuntimeError):
    """A libdash call returned a non-OK status."""

    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.status_name = name


def lib():
    """The loaded libdash.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"libdash is not built ({library_path} missing); run "
                "`python -m sparse_hierarchical_attention_amd.build` first")
        L = ctypes.CDLL(library_path)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.dash_status_string.argtypes = [i]
        L.dash_status_string.restype = ctypes.c_char_p
        L.dash_last_error.restype = ctypes.c_char_p
        L.dash_version.restype = i
        L.dash_pool_keys.argtypes = [vp, i, vp, i, i, i, i, i, vp]
        i64 = ctypes.c_int64
        L.dash_pool_keys_query.argtypes = [vp, i, vp, vp, i, i, i, i, i, vp]
        L.dash_pool_keys_query_ex.argtypes = [vp, i, vp, i64, i64, vp, i, i, i, i, i, vp]
        L.dash_pool_keys_append.argtypes = [vp, i, vp, vp, vp, i, i, i, i, i, vp]
        L.dash_pool_keys_append_ex.argtypes = [vp, i, vp, i64, i64, vp, vp, i, i, i, i, i, vp]
        L.dash_block_entmax_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i]
        L.dash_block_entmax_workspace_bytes.restype = sz
        L.dash_block_entmax.argtypes = [vp, i, vp, i, i, i, i, i, i, i, i, f, f, f, vp, vp, vp,
                                        vp, sz, vp]
        L.dash_block_entmax_ex.argtypes = [vp, i, vp, vp, i, i, i, i, i, i, i, i, f, f, f, i, vp,
                                           vp, vp, vp, sz, vp]
        L.dash_sparse_attn_prefill.argtypes = [vp, vp, vp, i, vp, vp, vp, vp, i, i, i, i, i, i,
                                               f, vp]
        L.dash_sparse_attn_prefill_ex.argtypes = [vp, vp, vp, i, vp, vp, vp, vp, i, i, i, i, i, i,
                                                  i, i, f, vp]
        L.dash_decode_workspace_bytes.argtypes = [i, i, i, i, i, i]
        L.dash_decode_workspace_bytes.restype = sz
        L.dash_sparse_attn_decode.argtypes = [vp, vp, vp, i, vp, vp, vp, i, i, i, i, i, i, f,
                                              vp, sz, vp]
        L.dash_sparse_attn_decode_varlen.argtypes = [vp, vp, vp, i, vp, vp, vp, vp, i, i, i, i,
                                                     i, i, f, vp, sz, vp]
        L.dash_sparse_attn_backward_workspace_bytes.argtypes = [i, i, i]
        L.dash_sparse_attn_backward_workspace_bytes.restype = sz
        L.dash_sparse_attn_prefill_backward.argtypes = [vp, vp, vp, vp, vp, i, vp, vp, vp, vp, vp,
                                                        vp, i, i, i, i, i, i, f, vp, sz, vp]
        L.dash_block_entmax_backward_workspace_bytes.argtypes = [i, i, i, i]
        L.dash_block_entmax_backward_workspace_bytes.restype = sz
        L.dash_block_entmax_backward.argtypes = [vp, i, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i,
                                                 f, f, f, i, vp, sz, vp]
        L.dash_block_entmax_backward.restype = i
        L.dash_block_entmax_backward_query_workspace_bytes.argtypes = [i, i, i, i, i, i]
        L.dash_block_entmax_backward_query_workspace_bytes.restype = sz
        L.dash_block_entmax_backward_query.argtypes = [vp, vp, i, vp, vp, i64, i64, vp, vp, vp, vp,
                                                       vp, vp, i, i, i, i, i, i, f, f, f, i, vp,
                                                       sz, vp]
        L.dash_block_entmax_backward_query.restype = i
        L.dash_decode_step_workspace_bytes.argtypes = [i, i, i, i, i, i]
        L.dash_decode_step_workspace_bytes.restype = sz
        L.dash_decode_step.argtypes = [vp, vp, vp, i, vp, vp, i, i, i, i, i, i, f, f, f, i, f, vp,
                                       vp, vp, vp, sz, vp]
        L.dash_decode_step.restype = i
        L.dash_decode_step_noalloc.argtypes = [vp, vp, vp, i, vp, vp, i, i, i, i, i, i, f, f, f,
                                               i, f, vp, vp, vp, vp]
        L.dash_decode_step_noalloc.restype = i
        for fn in ("dash_pool_keys", "dash_pool_keys_query", "dash_pool_keys_append",
                   "dash_pool_keys_query_ex", "dash_pool_keys_append_ex",
                   "dash_block_entmax", "dash_block_entmax_ex", "dash_sparse_attn_prefill",
                   "dash_sparse_attn_prefill_ex", "dash_sparse_attn_decode", "dash_sparse_attn_decode_varlen",
                   "dash_sparse_attn_prefill_backward"):
            getattr(L, fn).restype = i
        _lib = L
    return _lib


def dash_version() -> int:
    return int(lib().dash_version())


def _check(status: int):
    if status != 0:
        L = lib()
        raise DashError(status, L.dash_status_string(status).decode(),
                        L.dash_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DASH_BF16
    if t.dtype == torch.float32:
        return DASH_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _dev(*ts: torch.Tensor) -> torch.device:
    dev = ts[0].device
    for t in ts:
        if t is None:
            continue
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError("all tensors must live on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _f32(**ts):
    """Raise unless every given tensor (None skipped) is float32."""
    for name, t in ts.items():
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32 (got {t.dtype})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def dash_pool_keys(k: torch.Tensor, block: int, kbar: torch.Tensor | None = None) -> torch.Tensor:
    """Stage 0 (mean pooling): k [B, n, Hkv, D] -> kbar [B, n // block, Hkv, D] fp32."""
    _f32(kbar=kbar)
    b, n, hkv, d = k.shape
    if kbar is None:
        kbar = torch.empty((b, n // block, hkv, d), dtype=torch.float32, device=k.device)
    dev = _dev(k, kbar)
    _check(lib().dash_pool_keys(_ptr(k), _dtype_code(k), _ptr(kbar), b, n, hkv, d, block,
                                _stream(dev)))
    return kbar


def _qbar_strides(qbar: torch.Tensor, batch: int, tc: int, hkv: int, d: int) -> tuple[int, int]:
    """Strides (in floats) of summary queries [Hkv, D], [Tc, Hkv, D] or [B, Tc, Hkv, D]."""
    if tuple(qbar.shape) == (hkv, d):
        return 0, 0
    if tuple(qbar.shape) == (tc, hkv, d):
        return 0, hkv * d
    if tuple(qbar.shape) == (batch, tc, hkv, d):
        return tc * hkv * d, hkv * d
    raise ValueError(f"qbar shape {tuple(qbar.shape)} is none of [Hkv, D], [Tc, Hkv, D], "
                     f"[B, Tc, Hkv, D] (B={batch}, Tc={tc}, Hkv={hkv}, D={d})")


def dash_pool_keys_query(k: torch.Tensor, qbar: torch.Tensor, block: int,
                         kbar: torch.Tensor | None = None) -> torch.Tensor:
    """Stage 0 with learned summary queries (Eq. 3), fp32: qbar [Hkv, D] (one per KV head),
    [Tc, Hkv, D] (one per chunk, as Alg. 1 takes it) or [B, Tc, Hkv, D]."""
    _f32(qbar=qbar, kbar=kbar)
    b, n, hkv, d = k.shape
    if kbar is None:
        kbar = torch.empty((b, n // block, hkv, d), dtype=torch.float32, device=k.device)
    sb, sc = _qbar_strides(qbar, b, n // block, hkv, d)
    dev = _dev(k, qbar, kbar)
    _check(lib().dash_pool_keys_query_ex(_ptr(k), _dtype_code(k), _ptr(qbar), sb, sc, _ptr(kbar),
                                         b, n, hkv, d, block, _stream(dev)))
    return kbar


def dash_block_entmax_workspace_bytes(dtype, batch, n_q, q_pos0, n_kv, h_q, h_kv, head_dim,
                                      block) -> int:
    """Workspace bytes dash_block_entmax needs; dtype is a torch dtype (bf16 / fp32)."""
    code = DASH_BF16 if dtype == torch.bfloat16 else DASH_F32
    return int(lib().dash_block_entmax_workspace_bytes(code, batch, n_q, q_pos0, n_kv, h_q, h_kv,
                                                       head_dim, block))


def dash_pool_keys_append(k_cache: torch.Tensor, ctx_lens: torch.Tensor, kbar: torch.Tensor,
                          block: int, qbar: torch.Tensor | None = None) -> torch.Tensor:
    """Streaming Stage 0: write the summary of the chunk each sequence's newest token completed
    (ctx_lens int32 [B] a positive multiple of block) into kbar [B, n_cap // block, Hkv, D].
    qbar: None (mean), or summary queries [Hkv, D], [Tc, Hkv, D] or [B, Tc, Hkv, D] for the
    cache's Tc = n_cap // block chunks."""
    _f32(kbar=kbar, qbar=qbar)
    b, n_cap, hkv, d = k_cache.shape
    if ctx_lens.dtype != torch.int32:
        raise TypeError("ctx_lens must be int32")
    sb, sc = (0, 0) if qbar is None else _qbar_strides(qbar, b, n_cap // block, hkv, d)
    dev = _dev(k_cache, ctx_lens, kbar, qbar)
    _check(lib().dash_pool_keys_append_ex(_ptr(k_cache), _dtype_code(k_cache), _ptr(qbar), sb, sc,
                                          _ptr(ctx_lens), _ptr(kbar), b, n_cap, hkv, d, block,
                                          _stream(dev)))
    return kbar


def _route_outputs(q, n_kv, block, hkv, mask, bias, tau, want_tau):
    b, n_q, hq, _ = q.shape
    nc = -(-n_kv // block)
    nw = -(-nc // 32)
    dev = q.device
    if mask is None:
        mask = torch.empty((b, n_q, hkv, nw), dtype=torch.int32, device=dev)
    if bias is None:
        bias = torch.empty((b, n_q, hkv, nc), dtype=torch.float32, device=dev)
    if tau is None and want_tau:
        tau = torch.empty((b, n_q, hq), dtype=torch.float32, device=dev)
    return mask, bias, tau


def dash_block_entmax_ex(q: torch.Tensor, kbar: torch.Tensor, *, n_kv: int, block: int,
                         alpha: float, gamma: float, sigma: float, q_pos0: int = 0,
                         h_kv: int | None = None, ctx_lens: torch.Tensor | None = None,
                         window_blocks: int = 1, mask: torch.Tensor | None = None,
                         bias: torch.Tensor | None = None, tau: torch.Tensor | None = None,
                         want_tau: bool = True, workspace: torch.Tensor | None = None):
    """Stage 1 with the attention window (window_blocks blocks always attended: the query's own
    and the window_blocks - 1 before it) and, for decode (n_q = 1), per-sequence context lengths
    ctx_lens int32 [B] in a cache of capacity n_kv. Outputs as dash_block_entmax."""
    _f32(kbar=kbar, bias=bias, tau=tau)
    b, n_q, hq, d = q.shape
    hkv = kbar.shape[2] if h_kv is None else h_kv
    mask, bias, tau = _route_outputs(q, n_kv, block, hkv, mask, bias, tau, want_tau)
    if ctx_lens is not None:
        if ctx_lens.dtype != torch.int32:
            raise TypeError("ctx_lens must be int32")
        q_pos0 = n_kv - 1
    need = dash_block_entmax_workspace_bytes(q.dtype, b, n_q, q_pos0, n_kv, hq, hkv, d, block)
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dev = _dev(q, kbar, ctx_lens, mask, bias, tau, workspace)
    _check(lib().dash_block_entmax_ex(
        _ptr(q), _dtype_code(q), _ptr(kbar), _ptr(ctx_lens), b, n_q, q_pos0, n_kv, hq, hkv, d,
        block, float(alpha), float(gamma), float(sigma), int(window_blocks), _ptr(mask),
        _ptr(bias), _ptr(tau), _ptr(workspace), wsb, _stream(dev)))
    return mask, bias, tau


def dash_block_entmax(q: torch.Tensor, kbar: torch.Tensor, *, n_kv: int, block: int, alpha: float,
                      gamma: float, sigma: float, q_pos0: int = 0, h_kv: int | None = None,
                      mask: torch.Tensor | None = None, bias: torch.Tensor | None = None,
                      tau: torch.Tensor | None = None, want_tau: bool = True,
                      workspace: torch.Tensor | None = None):
    """Stage 1: q [B, n_q, Hq, D], kbar [B, Tc, Hkv, D] fp32 ->
    mask int32 [B, n_q, Hkv, W] (uint32 bit patterns), bias fp32 [B, n_q, Hkv, Nc],
    tau fp32 [B, n_q, Hq] (None unless want_tau)."""
    _f32(kbar=kbar, bias=bias, tau=tau)
    b, n_q, hq, d = q.shape
    hkv = kbar.shape[2] if h_kv is None else h_kv
    nc = -(-n_kv // block)
    nw = -(-nc // 32)
    dev = q.device
    if mask is None:
        mask = torch.empty((b, n_q, hkv, nw), dtype=torch.int32, device=dev)
    if bias is None:
        bias = torch.empty((b, n_q, hkv, nc), dtype=torch.float32, device=dev)
    if tau is None and want_tau:
        tau = torch.empty((b, n_q, hq), dtype=torch.float32, device=dev)
    need = dash_block_entmax_workspace_bytes(q.dtype, b, n_q, q_pos0, n_kv, hq, hkv, d, block)
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dev = _dev(q, kbar, mask, bias, tau, workspace)
    _check(lib().dash_block_entmax(
        _ptr(q), _dtype_code(q), _ptr(kbar), b, n_q, q_pos0, n_kv, hq, hkv, d, block,
        float(alpha), float(gamma), float(sigma), _ptr(mask), _ptr(bias), _ptr(tau),
        _ptr(workspace), wsb, _stream(dev)))
    return mask, bias, tau


def dash_sparse_attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                             mask: torch.Tensor, bias: torch.Tensor, *, block: int,
                             scale: float | None = None, o: torch.Tensor | None = None,
                             lse: torch.Tensor | None = None, want_lse: bool = True,
                             q_pos0: int = 0):
    """Stage 2 prefill: -> (o [B, n_q, Hq, D] in q's dtype, lse fp32 [B, n_q, Hq] or None).
    q holds the rows at positions q_pos0 .. q_pos0 + n_q - 1 of sequences of k.shape[1] tokens
    (all of them by default); mask and bias hold the same rows."""
    _f32(bias=bias, lse=lse)
    b, n_q, hq, d = q.shape
    n_kv, hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((b, n_q, hq), dtype=torch.float32, device=q.device)
    dev = _dev(q, k, v, mask, bias, o, lse)
    if q_pos0 == 0 and n_q == n_kv:  # whole sequences: the plain entry point
        _check(lib().dash_sparse_attn_prefill(
            _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(mask), _ptr(bias), _ptr(o),
            _ptr(lse), b, n_kv, hq, hkv, d, block, float(scale), _stream(dev)))
    else:
        _check(lib().dash_sparse_attn_prefill_ex(
            _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(mask), _ptr(bias), _ptr(o),
            _ptr(lse), b, n_q, int(q_pos0), n_kv, hq, hkv, d, block, float(scale), _stream(dev)))
    return o, lse


def dash_sparse_attn_backward_workspace_bytes(batch, n, h_q) -> int:
    return int(lib().dash_sparse_attn_backward_workspace_bytes(batch, n, h_q))


def dash_sparse_attn_prefill_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                      lse: torch.Tensor, dout: torch.Tensor, mask: torch.Tensor,
                                      bias: torch.Tensor, *, block: int,
                                      scale: float | None = None, want_dbias: bool = True,
                                      workspace: torch.Tensor | None = None):
    """Stage 2 prefill gradients with the selection held fixed: lse from
    dash_sparse_attn_prefill, dout in q's dtype. -> (dq, dk, dv, dbias or None), fp32."""
    _f32(lse=lse, bias=bias)
    b, n, hq, d = q.shape
    hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if dout.dtype != q.dtype:
        raise TypeError("dout must have q's dtype")
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty((b, n, hq, d), **f32)
    dk = torch.empty((b, n, hkv, d), **f32)
    dv = torch.empty((b, n, hkv, d), **f32)
    dbias = torch.empty(bias.shape, **f32) if want_dbias else None
    need = dash_sparse_attn_backward_workspace_bytes(b, n, hq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dev = _dev(q, k, v, lse, dout, mask, bias, workspace)
    _check(lib().dash_sparse_attn_prefill_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _dtype_code(q), _ptr(mask),
        _ptr(bias), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias), b, n, hq, hkv, d, block,
        float(scale), _ptr(workspace), workspace.numel(), _stream(dev)))
    return dq, dk, dv, dbias


def dash_block_entmax_backward_workspace_bytes(batch, n, h_q, h_kv) -> int:
    return int(lib().dash_block_entmax_backward_workspace_bytes(batch, n, h_q, h_kv))


def dash_block_entmax_backward(q: torch.Tensor, kbar: torch.Tensor, tau: torch.Tensor,
                               mask: torch.Tensor, dbias: torch.Tensor, dq: torch.Tensor,
                               dk: torch.Tensor, *, block: int, alpha: float, gamma: float,
                               sigma: float, window_blocks: int = 1,
                               workspace: torch.Tensor | None = None) -> None:
    """Routing and pooling gradients for prefill, added in place to dq [B, n, Hq, D] and dk
    [B, n, Hkv, D] (fp32), from dbias = dL/dd of dash_sparse_attn_prefill_backward."""
    _f32(kbar=kbar, tau=tau, dbias=dbias, dq=dq, dk=dk)
    b, n, hq, d = q.shape
    hkv = dk.shape[2]
    need = dash_block_entmax_backward_workspace_bytes(b, n, hq, hkv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dev = _dev(q, kbar, tau, mask, dbias, dq, dk, workspace)
    _check(lib().dash_block_entmax_backward(
        _ptr(q), _dtype_code(q), _ptr(kbar), _ptr(tau), _ptr(mask), _ptr(dbias), _ptr(dq),
        _ptr(dk), b, n, hq, hkv, d, block, float(alpha), float(gamma), float(sigma),
        int(window_blocks), _ptr(workspace), workspace.numel(), _stream(dev)))


def dash_block_entmax_backward_query_workspace_bytes(batch, n, h_q, h_kv, head_dim, block) -> int:
    return int(lib().dash_block_entmax_backward_query_workspace_bytes(batch, n, h_q, h_kv, head_dim,
                                                                      block))


def dash_block_entmax_backward_query(q: torch.Tensor, k: torch.Tensor, kbar: torch.Tensor,
                                     qbar: torch.Tensor, tau: torch.Tensor, mask: torch.Tensor,
                                     dbias: torch.Tensor, dq: torch.Tensor, dk: torch.Tensor, *,
                                     block: int, alpha: float, gamma: float, sigma: float,
                                     window_blocks: int = 1, dqbar: torch.Tensor | None = None,
                                     workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Routing and learned-query pooling gradients for prefill: adds to dq and dk (fp32) and
    returns dqbar, qbar's shape ([Hkv, D], [Tc, Hkv, D] or [B, Tc, Hkv, D]), fp32."""
    _f32(kbar=kbar, qbar=qbar, tau=tau, dbias=dbias, dq=dq, dk=dk, dqbar=dqbar)
    b, n, hq, d = q.shape
    hkv = k.shape[2]
    sb, sc = _qbar_strides(qbar, b, n // block, hkv, d)
    if dqbar is None:
        dqbar = torch.empty_like(qbar)
    need = dash_block_entmax_backward_query_workspace_bytes(b, n, hq, hkv, d, block)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dev = _dev(q, k, kbar, qbar, tau, mask, dbias, dq, dk, dqbar, workspace)
    _check(lib().dash_block_entmax_backward_query(
        _ptr(q), _ptr(k), _dtype_code(q), _ptr(kbar), _ptr(qbar), sb, sc, _ptr(tau), _ptr(mask),
        _ptr(dbias), _ptr(dq), _ptr(dk), _ptr(dqbar), b, n, hq, hkv, d, block, float(alpha),
        float(gamma), float(sigma), int(window_blocks), _ptr(workspace), workspace.numel(),
        _stream(dev)))
    return dqbar


def dash_decode_workspace_bytes(batch, n_ctx, h_q, h_kv, head_dim, block) -> int:
    return int(lib().dash_decode_workspace_bytes(batch, n_ctx, h_q, h_kv, head_dim, block))


def dash_sparse_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            mask: torch.Tensor, bias: torch.Tensor, *, block: int,
                            scale: float | None = None, o: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Stage 2 decode: q [B, Hq, D] (or [B, 1, Hq, D]) -> o of the same shape."""
    _f32(bias=bias)
    b, n_ctx, hkv, d = k_cache.shape
    hq = q.shape[-2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    need = dash_decode_workspace_bytes(b, n_ctx, hq, hkv, d, block)
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dev = _dev(q, k_cache, v_cache, mask, bias, o, workspace)
    _check(lib().dash_sparse_attn_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(q), _ptr(mask), _ptr(bias), _ptr(o),
        b, n_ctx, hq, hkv, d, block, float(scale), _ptr(workspace), wsb, _stream(dev)))
    return o


def dash_sparse_attn_decode_varlen(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                   ctx_lens: torch.Tensor, mask: torch.Tensor, bias: torch.Tensor,
                                   *, block: int, scale: float | None = None,
                                   o: torch.Tensor | None = None,
                                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Stage 2 decode with per-sequence lengths ctx_lens int32 [B] in a cache of capacity
    k_cache.shape[1]: q [B, Hq, D] (or [B, 1, Hq, D]) -> o of the same shape."""
    _f32(bias=bias)
    b, n_cap, hkv, d = k_cache.shape
    hq = q.shape[-2]
    if ctx_lens.dtype != torch.int32:
        raise TypeError("ctx_lens must be int32")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    need = dash_decode_workspace_bytes(b, n_cap, hq, hkv, d, block)
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dev = _dev(q, k_cache, v_cache, ctx_lens, mask, bias, o, workspace)
    _check(lib().dash_sparse_attn_decode_varlen(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(q), _ptr(ctx_lens), _ptr(mask),
        _ptr(bias), _ptr(o), b, n_cap, hq, hkv, d, block, float(scale), _ptr(workspace), wsb,
        _stream(dev)))
    return o


def forward(q, k, v, *, block: int, alpha: float, gamma: float, sigma: float,
            scale: float | None = None, window: int = 1, qbar: torch.Tensor | None = None):
    """Whole prefill forward: pool -> route -> sparse attention. Returns a dict of every
    intermediate (kbar, mask, bias, tau, o, lse). window: blocks always attended (the query's
    own and window - 1 before it). qbar: learned summary queries (see dash_pool_keys_query);
    None for mean pooling."""
    kbar = dash_pool_keys(k, block) if qbar is None else dash_pool_keys_query(k, qbar, block)
    if window == 1:
        mask, bias, tau = dash_block_entmax(q, kbar, n_kv=k.shape[1], block=block, alpha=alpha,
                                            gamma=gamma, sigma=sigma, h_kv=k.shape[2])
    else:
        mask, bias, tau = dash_block_entmax_ex(q, kbar, n_kv=k.shape[1], block=block,
                                               alpha=alpha, gamma=gamma, sigma=sigma,
                                               h_kv=k.shape[2], window_blocks=window)
    o, lse = dash_sparse_attn_prefill(q, k, v, mask, bias, block=block, scale=scale)
    return dict(kbar=kbar, mask=mask, bias=bias, tau=tau, o=o, lse=lse)


def backward(q, k, v, dout, fwd: dict, *, block: int, alpha: float, gamma: float, sigma: float,
             scale: float | None = None, window: int = 1,
             qbar: torch.Tensor | None = None) -> dict:
    """Gradients of the prefill forward (pool, route, attend) for dL/do = dout, given the dict
    that forward() returned with the same arguments: dict(dq, dk, dv, dbias), fp32, plus dqbar
    when qbar (learned summary queries) is given. The selection is held fixed (no gradient flows
    through which chunks are selected)."""
    dq, dk, dv, dbias = dash_sparse_attn_prefill_backward(q, k, v, fwd["lse"], dout, fwd["mask"],
                                                          fwd["bias"], block=block, scale=scale)
    out = dict(dq=dq, dk=dk, dv=dv, dbias=dbias)
    if qbar is None:
        dash_block_entmax_backward(q, fwd["kbar"], fwd["tau"], fwd["mask"], dbias, dq, dk,
                                   block=block, alpha=alpha, gamma=gamma, sigma=sigma,
                                   window_blocks=window)
    else:
        out["dqbar"] = dash_block_entmax_backward_query(
            q, k, fwd["kbar"], qbar, fwd["tau"], fwd["mask"], dbias, dq, dk, block=block,
            alpha=alpha, gamma=gamma, sigma=sigma, window_blocks=window)
    return out


def dash_decode_step_workspace_bytes(batch, n_ctx, h_q, h_kv, head_dim, block) -> int:
    return int(lib().dash_decode_step_workspace_bytes(batch, n_ctx, h_q, h_kv, head_dim, block))


def dash_decode_step(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     kbar: torch.Tensor, *, block: int, alpha: float, gamma: float, sigma: float,
                     ctx_lens: torch.Tensor | None = None, window_blocks: int = 1,
                     scale: float | None = None, mask: torch.Tensor | None = None,
                     bias: torch.Tensor | None = None, o: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None):
    """One decode step (Stage 1 routing and Stage 2 attention, one call) for a new token per
    sequence whose key/value are already in the cache: q [B, Hq, D] (or [B, 1, Hq, D]) ->
    (o, mask, bias).
    ctx_lens int32 [B] gives per-sequence lengths in a cache of capacity k_cache.shape[1]. A
    workspace passed in must be zero-filled when allocated (it keeps its ticket counters zero)."""
    _f32(kbar=kbar, bias=bias)
    b, n_ctx, hkv, d = k_cache.shape
    hq = q.shape[-2]
    if ctx_lens is not None and ctx_lens.dtype != torch.int32:
        raise TypeError("ctx_lens must be int32")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nc = -(-n_ctx // block)
    if mask is None:
        mask = torch.empty((b, 1, hkv, -(-nc // 32)), dtype=torch.int32, device=q.device)
    if bias is None:
        bias = torch.empty((b, 1, hkv, nc), dtype=torch.float32, device=q.device)
    if o is None:
        o = torch.empty_like(q)
    need = dash_decode_step_workspace_bytes(b, n_ctx, hq, hkv, d, block)
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    wsb = workspace.numel() * workspace.element_size()
    dev = _dev(q, k_cache, v_cache, kbar, ctx_lens, mask, bias, o, workspace)
    _check(lib().dash_decode_step(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(q), _ptr(kbar), _ptr(ctx_lens), b,
        n_ctx, hq, hkv, d, block, float(alpha), float(gamma), float(sigma), int(window_blocks),
        float(scale), _ptr(mask), _ptr(bias), _ptr(o), _ptr(workspace), wsb, _stream(dev)))
    return o, mask, bias


def dash_decode_step_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                             kbar: torch.Tensor, *, mask: torch.Tensor, bias: torch.Tensor,
                             o: torch.Tensor, block: int, alpha: float, gamma: float,
                             sigma: float, ctx_lens: torch.Tensor | None = None,
                             window_blocks: int = 1, scale: float | None = None) -> None:
    """dash_decode_step on the library's own device scratch: nothing is allocated, so the
    caller passes every output (mask, bias, o) in. Calls that overlap on one GPU race."""
    _f32(kbar=kbar, bias=bias)
    b, n_ctx, hkv, d = k_cache.shape
    hq = q.shape[-2]
    if ctx_lens is not None and ctx_lens.dtype != torch.int32:
        raise TypeError("ctx_lens must be int32")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dev = _dev(q, k_cache, v_cache, kbar, ctx_lens, mask, bias, o)
    _check(lib().dash_decode_step_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(q), _ptr(kbar), _ptr(ctx_lens), b,
        n_ctx, hq, hkv, d, block, float(alpha), float(gamma), float(sigma), int(window_blocks),
        float(scale), _ptr(mask), _ptr(bias), _ptr(o), _stream(dev)))


def decode_step(q, k_cache, v_cache, kbar, *, block: int, alpha: float, gamma: float,
                sigma: float, scale: float | None = None, route_ws=None, attn_ws=None,
                fused: bool = True, workspace=None):
    """One decode step for a new token per sequence whose key/value are already in the cache:
    route with the cached summaries, then the split sparse attention. q [B, 1, Hq, D].
    fused: one dash_decode_step call (workspace), else dash_block_entmax and
    dash_sparse_attn_decode (route_ws, attn_ws). Returns (o, mask, bias)."""
    n_ctx = k_cache.shape[1]
    if fused:
        return dash_decode_step(q, k_cache, v_cache, kbar, block=block, alpha=alpha, gamma=gamma,
                                sigma=sigma, scale=scale, workspace=workspace)
    mask, bias, _ = dash_block_entmax(q, kbar, n_kv=n_ctx, block=block, alpha=alpha, gamma=gamma,
                                      sigma=sigma, q_pos0=n_ctx - 1, h_kv=k_cache.shape[2],
                                      want_tau=False, workspace=route_ws)
    o = dash_sparse_attn_decode(q, k_cache, v_cache, mask, bias, block=block, scale=scale,
                                workspace=attn_ws)
    return o, mask, bias
