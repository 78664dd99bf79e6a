"""GPU parity of the Stage 2 prefill backward (the selection held fixed) against the oracle's
float64 gradients, through the C ABI, on seeded random inputs and random selections.

Tolerance: the gradients have no fixed scale, so each tensor's error is measured against its
largest reference magnitude: at most 1e-4 of it for fp32 inputs and 2e-2 (max) / 1e-2 (mean,
against the mean magnitude) for bf16 inputs, the forward output's bars applied to the
normalised gradients. bf16 adds one rounding of o (2^-9 relative) inside rowsum(dout * o)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def dash():
    import sparse_hierarchical_attention_amd as d
    d.lib()
    return d


def _compare(name, gpu, ref, dtype):
    gpu = np.asarray(gpu, dtype=np.float64)
    scale = float(np.abs(ref).max())
    if scale == 0.0:  # e.g. dq and dk of a one-token sequence: p = 1, so ds = 0 exactly
        assert float(np.abs(gpu).max()) <= 1e-5, name
        return
    err = np.abs(gpu - ref)
    max_rel = float(err.max()) / scale
    mean_rel = float(err.mean()) / float(np.abs(ref).mean())
    print(f"{name}: max {max_rel:.2e} mean {mean_rel:.2e} (scale {scale:.3g})", flush=True)
    if dtype == "f32":
        assert max_rel <= 1e-4, (name, max_rel)
    else:
        assert max_rel <= 2e-2 and mean_rel <= 1e-2, (name, max_rel, mean_rel)


def run_backward(dash, orc, w: wl.Workload, sparsity: float, seed: int, want_dbias=True):
    print(f"case: {w.name} sparsity {sparsity} seed {seed}", flush=True)
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    mask, bias = wl.random_selection(w.batch, w.n_q, 0, w.n_kv, w.h_kv, w.block, sparsity,
                                     seed=seed, device=DEV, bias_std=0.5)
    o, lse = dash.dash_sparse_attn_prefill(q, k, v, mask, bias, block=w.block)
    dout = wl.output_gradient(q.shape, seed + 1, q.dtype, DEV)
    dq, dk, dv, dbias = dash.dash_sparse_attn_prefill_backward(q, k, v, o, lse, dout, mask, bias,
                                                                block=w.block,
                                                                want_dbias=want_dbias)
    torch.cuda.synchronize()
    m = parity.to_host(mask).view(np.uint32)
    ref = orc.sparse_attn_backward(q.cpu(), k.cpu(), v.cpu(), m, parity.to_host(bias),
                                   parity.to_host(dout).astype(np.float64), block=w.block)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        _compare(name, parity.to_host(g), ref[name], w.dtype)
    if want_dbias:
        db = parity.to_host(dbias)
        # bit-exact zeros off the routed chunks below each row's own
        np.testing.assert_array_equal(db[ref["dbias"] == 0.0], 0.0)
        if np.any(ref["dbias"] != 0.0):  # else no row routes a chunk: all zero, checked above
            _compare("dbias", db, ref["dbias"], w.dtype)
    return dict(dq=dq, dk=dk, dv=dv, dbias=dbias)


CASES = [
    # batch, n, hq, hkv, d, block, dtype
    (2, 300, 4, 4, 128, 32, "f32"),
    (1, 531, 16, 1, 128, 64, "bf16"),
    (2, 300, 8, 2, 64, 32, "bf16"),
    (1, 600, 32, 2, 128, 128, "bf16"),
    (1, 389, 8, 1, 64, 64, "f32"),
    (1, 260, 4, 2, 128, 64, "bf16"),
    (1, 1500, 4, 1, 64, 32, "bf16"),
]


@pytest.mark.parametrize("batch,n,hq,hkv,d,block,dtype", CASES)
@pytest.mark.parametrize("sparsity", [0.0, 0.75])
def test_backward_small(dash, orc, batch, n, hq, hkv, d, block, dtype, sparsity):
    """Every gradient of every row against the oracle: groups of 1 to 16, head dims 64 and 128,
    chunks of 32 to 128 with a ragged tail, more tokens than one column-scan block (256)."""
    w = wl.Workload(f"backward B{batch} n{n} {hq}q/{hkv}kv D{d} block {block} {dtype}", batch, n,
                    hq, hkv, d, block, 1.5, 0.5, 1e8, dtype=dtype, seed=90 + n)
    run_backward(dash, orc, w, sparsity, seed=n)


def test_backward_without_dbias(dash, orc):
    w = wl.Workload("backward no dbias", 1, 333, 8, 2, 128, 32, 1.5, 0.5, 1e8, seed=95)
    run_backward(dash, orc, w, 0.5, seed=96, want_dbias=False)


def test_backward_single_chunk_and_token(dash, orc):
    """n below one chunk (only the causal own chunk) and n = 1."""
    for n in (20, 1):
        w = wl.Workload(f"backward n{n}", 1, n, 8, 2, 128, 32, 1.5, 0.5, 1e8, seed=97)
        run_backward(dash, orc, w, 0.5, seed=98)


def test_backward_deterministic(dash):
    w = wl.Workload("backward determinism", 1, 1000, 16, 1, 128, 64, 1.5, 0.5, 1e8, seed=99)
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    mask, bias = wl.random_selection(1, w.n_q, 0, w.n_kv, 1, 64, 0.5, seed=5, device=DEV,
                                     bias_std=0.5)
    o, lse = dash.dash_sparse_attn_prefill(q, k, v, mask, bias, block=64)
    dout = wl.output_gradient(q.shape, 6, q.dtype, DEV)
    a = dash.dash_sparse_attn_prefill_backward(q, k, v, o, lse, dout, mask, bias, block=64)
    b = dash.dash_sparse_attn_prefill_backward(q, k, v, o, lse, dout, mask, bias, block=64)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_prefill_32k(dash, orc):
    """The 32K prefill (32 query heads over 8 KV heads, D 128, chunks of 64) with the selection
    its own forward pass routes: sampled rows of dq and dL/dd against the oracle, and dk, dv by
    two sums that hold at any size: every row's probabilities add up to one, so the dv of all
    keys of a KV head adds up to the sum of dout over all rows and heads of its group, and every
    row's ds adds up to zero, so the dk of all keys adds up to zero."""
    from tests.test_gpu_parity import flat_rows, sample_rows
    w = wl.PREFILL_32K
    print(f"case: {w.name}", flush=True)
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    res = dash.forward(q, k, v, block=w.block, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma)
    dout = wl.output_gradient(q.shape, 77, q.dtype, DEV)
    dq, dk, dv, dbias = dash.dash_sparse_attn_prefill_backward(q, k, v, res["o"], res["lse"], dout,
                                                                res["mask"], res["bias"],
                                                                block=w.block)
    torch.cuda.synchronize()
    rows = sample_rows(w.n_q, w.block, 40, seed=78)
    ref = orc.sparse_attn_backward_rows(q.cpu(), k.cpu(), v.cpu(),
                                        flat_rows(res["mask"], rows).view(np.uint32),
                                        flat_rows(res["bias"], rows), flat_rows(dout, rows), rows,
                                        block=w.block)
    _compare("dq rows", flat_rows(dq, rows), ref["dq"], w.dtype)
    db = flat_rows(dbias, rows)
    np.testing.assert_array_equal(db[ref["dbias"] == 0.0], 0.0)
    _compare("dbias rows", db, ref["dbias"], w.dtype)

    g = w.h_q // w.h_kv
    d64 = parity.to_host(dout).astype(np.float64).reshape(w.n_q, w.h_kv, g, w.head_dim)
    dv_sum = parity.to_host(dv).astype(np.float64).sum(axis=(0, 1))
    want = d64.sum(axis=(0, 2))
    dv_scale = float(np.abs(parity.to_host(dv)).astype(np.float64).sum(axis=(0, 1)).max())
    err_v = float(np.abs(dv_sum - want).max()) / dv_scale
    dk_h = parity.to_host(dk).astype(np.float64)
    err_k = float(np.abs(dk_h.sum(axis=(0, 1))).max()) / float(np.abs(dk_h).sum(axis=(0, 1)).max())
    print(f"sum rules: dv {err_v:.2e}, dk {err_k:.2e} (of the summed magnitudes)", flush=True)
    assert err_v <= 1e-4 and err_k <= 1e-3
