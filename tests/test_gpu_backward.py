"""GPU parity of the prefill backward against the oracle's float64 gradients, through the C ABI,
on seeded random inputs: Stage 2 on random selections, and the whole chain (pool, route, attend).

Tolerance: the gradients have no fixed scale, so each tensor's error is measured against its
largest (max) and mean (mean) reference magnitude. fp32 inputs run in fp32 throughout: 1e-4.
bf16 inputs run on the matrix cores, whose dV, dK and dQ products take p and ds rounded to bf16
(2^-9), as the forward's P V does: the forward's bf16 bars, 2e-2 (max) and 1e-2 (mean). dL/dd
sums ds in fp32 and keeps 1e-4 for both. The routing part is loosened by its condition (the
rounding of x - tau relative to x - tau, see _row_condition) times 1e-6, and rows whose condition
exceeds 1e4 are left out."""
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


def _bars(name, dtype):
    """(max, mean) bars for a gradient tensor."""
    if dtype == "f32" or name.startswith("dbias"):
        return 1e-4, 1e-4
    return 2e-2, 1e-2


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
    bmax, bmean = _bars(name, dtype)
    assert max_rel <= bmax and mean_rel <= bmean, (name, max_rel, mean_rel)


def run_backward(dash, orc, w: wl.Workload, sparsity: float, seed: int, want_dbias=True):
    print(f"case: {w.name} sparsity {sparsity} seed {seed}", flush=True)
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    mask, bias = wl.random_selection(w.batch, w.n_q, 0, w.n_kv, w.h_kv, w.block, sparsity,
                                     seed=seed, device=DEV, bias_std=0.5)
    o, lse = dash.dash_sparse_attn_prefill(q, k, v, mask, bias, block=w.block)
    dout = wl.output_gradient(q.shape, seed + 1, q.dtype, DEV)
    dq, dk, dv, dbias = dash.dash_sparse_attn_prefill_backward(q, k, v, lse, dout, mask, bias,
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
    a = dash.dash_sparse_attn_prefill_backward(q, k, v, lse, dout, mask, bias, block=64)
    b = dash.dash_sparse_attn_prefill_backward(q, k, v, lse, dout, mask, bias, block=64)
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
    dq, dk, dv, dbias = dash.dash_sparse_attn_prefill_backward(q, k, v, res["lse"], dout,
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
    assert err_v <= 1e-3 and err_k <= 1e-3  # bf16 rounding of p and ds in the dV, dK products


# ------------------------------------------------------------- the whole chain: pool, route, attend

def _row_condition(st, q, w: wl.Workload) -> np.ndarray:
    """Condition of each query row's routing gradient [R]: the largest, over its heads and routed
    chunks, of S / |x - tau| with S = coef sum_d |q_d kbar_d| + |tau| the scale of the rounding
    error in x - tau (fp32 x is a 128-term dot product; fp32 tau). The routing gradient grows
    like 1 / (x - tau) near the edge of a head's support (and, for alpha = 2, jumps there), so a
    row whose condition is k can move by ~1e-7 k relative under fp32 rounding alone."""
    x, tau, kbar, wts = st["x"], st["tau"], st["kbar"], st["w"]
    R = w.batch * w.n_q
    tc = kbar.shape[1]
    cond = np.zeros(R)
    if tc == 0:
        return cond
    g = w.h_q // w.h_kv
    coef = (w.alpha - 1.0) * w.gamma / np.sqrt(w.head_dim)
    qa = np.abs(q.reshape(w.batch, w.n_q, w.h_q, w.head_dim))
    ka = np.abs(kbar)  # [B, Tc, Hkv, D]
    for b in range(w.batch):
        kh = np.repeat(ka[b], g, axis=1)  # [Tc, Hq, D]
        s = coef * np.einsum("thd,chd->thc", qa[b], kh)  # [n, Hq, Tc]
        rows = slice(b * w.n_q, (b + 1) * w.n_q)
        s = s + np.abs(tau[rows])[..., None]
        routed = np.repeat(wts[rows, :, :tc] > 0.0, g, axis=1)  # [n, Hq, Tc]
        with np.errstate(invalid="ignore", divide="ignore"):
            k = np.where(routed, s / np.abs(x[rows, :, :tc] - tau[rows][..., None]), 0.0)
        cond[rows] = np.nan_to_num(k, nan=np.inf).max(axis=(1, 2))
    return cond


def _compare_cond(name, gpu, ref, dtype, cond):
    base_max, base_mean = _bars(name, dtype)
    gpu = np.asarray(gpu, dtype=np.float64)
    scale = float(np.abs(ref).max())
    if scale == 0.0:
        assert float(np.abs(gpu).max()) <= 1e-5, name
        return
    err = np.abs(gpu - ref)
    max_rel = float(err.max()) / scale
    mean_rel = float(err.mean()) / float(np.abs(ref).mean())
    tol = base_max + 1e-6 * cond  # rounding of x - tau, scaled by the condition (at most 1e4)
    print(f"{name}: max {max_rel:.2e} (tol {tol:.1e}) mean {mean_rel:.2e} (scale {scale:.3g})",
          flush=True)
    assert max_rel <= tol and mean_rel <= base_mean + 1e-6 * cond, (name, max_rel, mean_rel, tol)


def _as_gpu_selection(st, w):
    """The oracle's selection in the layouts Stage 1 writes (mask int32, bias and tau fp32)."""
    nw = st["mask"].shape[-1]
    mask = torch.from_numpy(st["mask"].view(np.int32).reshape(w.batch, w.n_q, w.h_kv, nw).copy())
    bias = torch.from_numpy(st["bias"].astype(np.float32).reshape(w.batch, w.n_q, w.h_kv, -1))
    tau = torch.from_numpy(st["tau"].astype(np.float32).reshape(w.batch, w.n_q, w.h_q))
    return mask.to(DEV), bias.to(DEV), tau.to(DEV)


def run_full_backward(dash, orc, w: wl.Workload, window: int, own_selection: bool):
    """dash.backward against the oracle's gradient of the whole forward. own_selection: the GPU
    forward routes (and must select exactly the oracle's chunks); else the oracle's selection (its
    mask, bias and threshold) is handed to the GPU, so that both differentiate the same branch."""
    print(f"case: {w.name} window {window} own selection {own_selection}", flush=True)
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    kw = dict(block=w.block, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma)
    st = orc.forward(q.cpu(), k.cpu(), v.cpu(), window=window, **kw)
    # rows whose routing gradient is ill-conditioned are skipped in dq, and the keys of their
    # routed chunks (which those rows feed) in dk
    row_cond = _row_condition(st, parity.to_host(q).astype(np.float64), w)
    skip_rows = row_cond > 1e4
    skip_keys = np.zeros((w.batch, w.n_kv, w.h_kv), dtype=bool)
    for rho in np.flatnonzero(skip_rows):
        for r, c in zip(*np.nonzero(st["w"][rho] > 0.0)):
            skip_keys[rho // w.n_q, c * w.block:(c + 1) * w.block, r] = True
    cond = float(row_cond[~skip_rows].max()) if (~skip_rows).any() else 0.0
    if own_selection:
        fwd = dash.forward(q, k, v, window=window, **kw)
        got = parity.to_host(fwd["mask"]).view(np.uint32).reshape(st["mask"].shape)
        assert np.array_equal(got, st["mask"]), "the GPU routed other chunks than the oracle"
    else:
        mask, bias, tau = _as_gpu_selection(st, w)
        kbar = dash.dash_pool_keys(k, w.block)
        o, lse = dash.dash_sparse_attn_prefill(q, k, v, mask, bias, block=w.block)
        fwd = dict(kbar=kbar, mask=mask, bias=bias, tau=tau, o=o, lse=lse)
    dout = wl.output_gradient(q.shape, w.seed + 5, q.dtype, DEV)
    g = dash.backward(q, k, v, dout, fwd, window=window, **kw)
    torch.cuda.synchronize()
    ref = orc.backward(q.cpu(), k.cpu(), v.cpu(), parity.to_host(dout).astype(np.float64),
                       window=window, **kw)
    s2 = orc.sparse_attn_backward(q.cpu(), k.cpu(), v.cpu(), st["mask"], st["bias"],
                                  parity.to_host(dout).astype(np.float64), block=w.block)
    route = np.abs(ref["dq"] - s2["dq"]).max() / np.abs(ref["dq"]).max()
    print(f"routing share of dq: {route:.2e}, condition of the kept rows {cond:.3g}, "
          f"ill-conditioned rows skipped: {int(skip_rows.sum())}", flush=True)
    err_row = np.abs(parity.to_host(g["dq"]) - ref["dq"]).reshape(len(row_cond), -1).max(axis=1)
    for rho in np.argsort(err_row)[-3:]:
        print(f"  row {rho}: dq max-abs error {err_row[rho]:.3g}, condition {row_cond[rho]:.3g}",
              flush=True)
    assert skip_rows.mean() <= 0.05
    dq_ok = ~skip_rows.reshape(w.batch, w.n_q)
    dk_ok = ~skip_keys
    _compare_cond("dq", parity.to_host(g["dq"])[dq_ok], ref["dq"][dq_ok], w.dtype, cond)
    _compare_cond("dk", parity.to_host(g["dk"])[dk_ok], ref["dk"][dk_ok], w.dtype, cond)
    _compare_cond("dv", parity.to_host(g["dv"]), ref["dv"], w.dtype, cond)
    routed = ref["dbias"] != 0.0  # the routed chunks (the window's chunks carry no gradient)
    _compare_cond("dbias", parity.to_host(g["dbias"])[routed], ref["dbias"][routed], w.dtype, cond)
    return route


FULL_CASES = [
    # batch, n, hq, hkv, d, block, dtype, alpha, gamma, sigma, window
    (1, 256, 8, 2, 64, 32, "f32", 1.5, 8.0, 0.5, 1),
    (1, 300, 8, 2, 128, 32, "bf16", 2.0, 8.0, 0.5, 1),
    (1, 260, 4, 4, 64, 32, "f32", 1.25, 8.0, 0.5, 2),
    (2, 200, 16, 1, 128, 32, "bf16", 1.5, 8.0, 1.0, 1),
    (1, 400, 8, 1, 128, 64, "bf16", 1.5, 16.0, 0.5, 3),
]


@pytest.mark.parametrize("batch,n,hq,hkv,d,block,dtype,alpha,gamma,sigma,window", FULL_CASES)
def test_full_backward_on_oracle_selection(dash, orc, batch, n, hq, hkv, d, block, dtype, alpha,
                                           gamma, sigma, window):
    w = wl.Workload(f"full backward B{batch} n{n} {hq}q/{hkv}kv D{d} block {block} {dtype} "
                    f"alpha {alpha}", batch, n, hq, hkv, d, block, alpha, gamma, sigma,
                    dtype=dtype, seed=300 + n)
    route = run_full_backward(dash, orc, w, window, own_selection=False)
    assert route > 1e-2  # the routing gradient is a visible part of dq


@pytest.mark.parametrize("dtype,alpha", [("f32", 1.5), ("bf16", 1.5), ("bf16", 2.0)])
def test_full_backward_on_own_selection(dash, orc, dtype, alpha):
    w = wl.Workload(f"full backward, own routing, {dtype} alpha {alpha}", 1, 320, 8, 2, 128, 32,
                    alpha, 8.0, 0.5, dtype=dtype, seed=330)
    run_full_backward(dash, orc, w, 1, own_selection=True)


def test_full_backward_sigma_inf_is_stage2_only(dash):
    """With sigma = inf the bias is 0 whatever w is: the routing adds nothing to dq and dk."""
    w = wl.Workload("sigma inf", 1, 300, 8, 2, 128, 32, 1.5, 8.0, float("inf"), seed=340)
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    kw = dict(block=32, alpha=1.5, gamma=8.0, sigma=float("inf"))
    fwd = dash.forward(q, k, v, **kw)
    dout = wl.output_gradient(q.shape, 341, q.dtype, DEV)
    g = dash.backward(q, k, v, dout, fwd, **kw)
    dq, dk, dv, _ = dash.dash_sparse_attn_prefill_backward(q, k, v, fwd["lse"], dout, fwd["mask"],
                                                            fwd["bias"], block=32)
    assert torch.equal(g["dq"], dq) and torch.equal(g["dk"], dk) and torch.equal(g["dv"], dv)


# ------------------------------------------------- learned summary queries: the pooling's gradient

QBAR_SHAPES = {"head": lambda b, tc, hkv, d: (hkv, d), "chunk": lambda b, tc, hkv, d: (tc, hkv, d),
               "sequence_chunk": lambda b, tc, hkv, d: (b, tc, hkv, d)}


def _learned_case(w: wl.Workload, per: str, seed: int):
    inp = wl.make_inputs(w, DEV)
    tc = w.n_kv // w.block
    g = torch.Generator().manual_seed(seed)
    qbar = (torch.randn(QBAR_SHAPES[per](w.batch, tc, w.h_kv, w.head_dim), generator=g) * 0.15)
    return inp["q"], inp["k"], inp["v"], qbar.to(DEV)


@pytest.mark.parametrize("per", list(QBAR_SHAPES))
@pytest.mark.parametrize("dtype,d,block", [("f32", 64, 32), ("bf16", 128, 64), ("bf16", 128, 32)])
def test_learned_query_routing_backward(dash, orc, per, dtype, d, block):
    """dash_block_entmax_backward_query against the oracle's routing gradient (dq, dkbar) chained
    into its learned-pooling gradient (dk, dqbar), on the oracle's selection and a random dL/dd.
    Rows whose routing gradient is ill-conditioned get dL/dd = 0 on both sides. The route
    backward runs in fp32 for either input dtype: 1e-4 of each tensor's scale, plus the rounding
    of x - tau scaled by the kept rows' condition."""
    n = 300 if block == 32 else 520
    w = wl.Workload(f"learned-query routing backward {per} {dtype} D{d} block {block}", 2, n, 8, 2,
                    d, block, 1.5, 8.0, 0.5, dtype=dtype, seed=360 + d + block)
    print(f"case: {w.name}", flush=True)
    q, k, _, qbar = _learned_case(w, per, 361)
    kbar = dash.dash_pool_keys_query(k, qbar, w.block)
    kbar_ref = orc.pool_keys_query(k.cpu(), qbar.cpu().numpy(), w.block)
    np.testing.assert_allclose(kbar.cpu().numpy(), kbar_ref, rtol=1e-5, atol=1e-5)
    kw = dict(block=w.block, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma)
    st = orc.block_entmax(q.cpu(), kbar_ref, n_kv=w.n_kv, h_kv=w.h_kv, **kw)
    st["kbar"] = kbar_ref
    cond = _row_condition(st, parity.to_host(q).astype(np.float64), w)
    ill = cond > 1e4
    rng = np.random.default_rng(362)
    dd = rng.standard_normal(st["bias"].shape)
    dd[ill] = 0.0
    nw = st["mask"].shape[-1]
    mask = torch.from_numpy(st["mask"].view(np.int32).reshape(w.batch, w.n_q, w.h_kv, nw).copy()).to(DEV)
    tau = torch.from_numpy(st["tau"].astype(np.float32).reshape(w.batch, w.n_q, w.h_q)).to(DEV)
    dbias = torch.from_numpy(dd.astype(np.float32).reshape(w.batch, w.n_q, w.h_kv, -1)).to(DEV)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=DEV)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=DEV)
    dqbar = dash.dash_block_entmax_backward_query(q, k, kbar, qbar, tau, mask, dbias, dq, dk, **kw)
    torch.cuda.synchronize()
    r1 = orc.block_entmax_backward(q.cpu(), kbar_ref, dd, n_kv=w.n_kv, want_dkbar=True, **kw)
    r0 = orc.pool_keys_query_backward(k.cpu(), qbar.cpu().numpy(), r1["dkbar"], w.block)
    kept = float(cond[~ill].max()) if (~ill).any() else 0.0
    print(f"ill-conditioned rows zeroed: {int(ill.sum())}, condition of the rest {kept:.3g}",
          flush=True)
    assert ill.mean() <= 0.05
    _compare_cond("dq", parity.to_host(dq), r1["dq"].reshape(q.shape), "f32", kept)
    _compare_cond("dk", parity.to_host(dk), r0["dk"], "f32", kept)
    _compare_cond("dqbar", parity.to_host(dqbar), r0["dqbar"], "f32", kept)
    # the incomplete tail chunk has no summary: its keys get no pooling gradient
    tail = w.n_kv // w.block * w.block
    if tail < w.n_kv:
        assert float(dk[:, tail:].abs().max()) == 0.0
    # deterministic: a second call gives the same bits
    dq2 = torch.zeros_like(dq)
    dk2 = torch.zeros_like(dk)
    dqbar2 = dash.dash_block_entmax_backward_query(q, k, kbar, qbar, tau, mask, dbias, dq2, dk2, **kw)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dqbar, dqbar2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_learned_query_full_backward(dash, orc, dtype):
    """dash.backward with per-chunk summary queries, on the oracle's selection, against the
    oracle's Stage 2 gradient chained into its routing and learned-pooling gradients. Rows whose
    routing gradient is ill-conditioned get dL/do = 0 (so dL/dd = 0 too) on both sides."""
    w = wl.Workload(f"full backward, per-chunk summary queries, {dtype}", 1, 320, 8, 2, 128, 32,
                    1.5, 8.0, 0.5, dtype=dtype, seed=370)
    print(f"case: {w.name}", flush=True)
    q, k, v, qbar = _learned_case(w, "chunk", 371)
    kw = dict(block=w.block, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma)
    kbar_ref = orc.pool_keys_query(k.cpu(), qbar.cpu().numpy(), w.block)
    st = orc.block_entmax(q.cpu(), kbar_ref, n_kv=w.n_kv, h_kv=w.h_kv, **kw)
    st["kbar"] = kbar_ref
    cond = _row_condition(st, parity.to_host(q).astype(np.float64), w)
    ill = cond > 1e4
    assert ill.mean() <= 0.05
    mask, bias, tau = _as_gpu_selection(st, w)
    kbar = dash.dash_pool_keys_query(k, qbar, w.block)
    o, lse = dash.dash_sparse_attn_prefill(q, k, v, mask, bias, block=w.block)
    fwd = dict(kbar=kbar, mask=mask, bias=bias, tau=tau, o=o, lse=lse)
    dout = wl.output_gradient(q.shape, 372, q.dtype, DEV)
    dout.view(-1, w.h_q, w.head_dim)[torch.from_numpy(ill).to(DEV)] = 0
    g = dash.backward(q, k, v, dout, fwd, qbar=qbar, **kw)
    torch.cuda.synchronize()
    dout_h = parity.to_host(dout).astype(np.float64)
    s2 = orc.sparse_attn_backward(q.cpu(), k.cpu(), v.cpu(), st["mask"], st["bias"], dout_h,
                                  block=w.block)
    r1 = orc.block_entmax_backward(q.cpu(), kbar_ref, s2["dbias"].reshape(st["bias"].shape),
                                   n_kv=w.n_kv, want_dkbar=True, **kw)
    r0 = orc.pool_keys_query_backward(k.cpu(), qbar.cpu().numpy(), r1["dkbar"], w.block)
    ref_dq = s2["dq"] + r1["dq"].reshape(q.shape)
    ref_dk = s2["dk"] + r0["dk"]
    c = float(cond[~ill].max())
    print(f"ill-conditioned rows given dL/do = 0: {int(ill.sum())}, condition of the rest {c:.3g}",
          flush=True)
    _compare_cond("dq", parity.to_host(g["dq"]), ref_dq, w.dtype, c)
    _compare_cond("dk", parity.to_host(g["dk"]), ref_dk, w.dtype, c)
    _compare_cond("dv", parity.to_host(g["dv"]), s2["dv"], w.dtype, c)
    _compare_cond("dqbar", parity.to_host(g["dqbar"]), r0["dqbar"], "f32", c)


@pytest.mark.parametrize("alpha,gamma", [(2.0, 0.002), (1.5, 0.01)])
def test_routing_backward_many_routed_chunks(dash, orc, alpha, gamma):
    """The routing gradient of rows that route more chunks than the row kernel keeps in LDS between
    its passes (it then scores them again): 16384 tokens in chunks of 32 with a routing scale so
    small that every candidate chunk is in every head's support with nearly equal weight (about 500
    routed chunks per late row, each well above the threshold, so the gradient is well
    conditioned). Sampled late rows of dq (routing part) against the oracle on the GPU's own
    selection, for a random dL/dd."""
    from tests.test_gpu_parity import flat_rows, sample_rows
    w = wl.Workload(f"routing backward, 16384 tokens, chunk 32, alpha {alpha}, gamma {gamma}", 1,
                    16384, 8, 2, 128, 32, alpha, gamma, 1.0, seed=380)
    print(f"case: {w.name}", flush=True)
    inp = wl.make_inputs(w, DEV)
    q, k = inp["q"], inp["k"]
    kw = dict(block=w.block, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma)
    kbar = dash.dash_pool_keys(k, w.block)
    mask, bias, tau = dash.dash_block_entmax(q, kbar, n_kv=w.n_kv, h_kv=w.h_kv, **kw)
    nc = -(-w.n_kv // w.block)
    dd = torch.randn((1, w.n_q, w.h_kv, nc), generator=torch.Generator(device=DEV).manual_seed(381),
                     device=DEV, dtype=torch.float32)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=DEV)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=DEV)
    dash.dash_block_entmax_backward(q, kbar, tau, mask, dd, dq, dk, **kw)
    torch.cuda.synchronize()
    rows = sample_rows(w.n_q, w.block, 24, seed=382)
    rows = rows[rows % w.n_q >= 14000]
    kbar_h = kbar.cpu().numpy().astype(np.float64)
    st = orc.block_entmax(q.cpu(), kbar_h, n_kv=w.n_kv, h_kv=w.h_kv, rows=rows, **kw)
    st["kbar"] = kbar_h
    gm = flat_rows(mask, rows).view(np.uint32)
    same = np.array([np.array_equal(gm[i], st["mask"][i]) for i in range(len(rows))])
    routed = (st["w"] > 0.0).sum(axis=2).min(axis=1)  # routed chunks of the row (per group)
    print(f"rows {len(rows)}, same selection {int(same.sum())}, routed chunks per row "
          f"{int(routed.min())}..{int(routed.max())}", flush=True)
    assert same.all() and routed.min() > 2048 // 5  # past the row kernel's LDS cache (g = 4)
    ref = orc.block_entmax_backward(q.cpu(), kbar_h, flat_rows(dd, rows).astype(np.float64),
                                    n_kv=w.n_kv, rows=rows, **kw)
    _compare_cond("dq (routing) rows", flat_rows(dq, rows), ref["dq"], "f32", 0.0)
