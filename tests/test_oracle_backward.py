"""Pins of the oracle's gradients of the forward pass ("DashAttention", arXiv 2605.18753v1:
§3.2-3.4 and App. A give the forward; its gradients follow by the chain rule through a fixed
selection). Each pin is independent of the backward code: central differences of the oracle's own
forward in float64, and torch autograd of plain causal attention where the routing cannot move."""
import math

import numpy as np
import pytest
import torch


def case(seed, n=96, hq=4, hkv=2, d=8, block=8):
    """Random inputs whose rows route several chunks with unequal weights, so that the bias and
    the gradient through the routing are far from zero."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, n, hq, d))
    k = rng.standard_normal((1, n, hkv, d))
    v = rng.standard_normal((1, n, hkv, d))
    dout = rng.standard_normal((1, n, hq, d))
    return q, k, v, dout


def loss(orc, q, k, v, dout, **kw):
    res = orc.forward(q, k, v, **kw)
    return float((res["o"] * dout.reshape(res["o"].shape)).sum()), res["mask"]


@pytest.mark.parametrize("alpha,gamma,window", [(1.5, 8.0, 1), (2.0, 4.0, 1), (1.25, 8.0, 1),
                                                (1.5, 8.0, 2)])
def test_gradients_match_central_differences(orc, alpha, gamma, window):
    kw = dict(block=8, alpha=alpha, gamma=gamma, sigma=2.0, window=window)
    q, k, v, dout = case(11)
    g = orc.backward(q, k, v, dout, **kw)
    base = orc.forward(q, k, v, **kw)
    # rows route several chunks with unequal weights: the bias, and the gradient through it, live
    assert (base["w"] > 0).sum(axis=2).max() >= 3 and np.ptp(base["bias"]) > 1.0
    rng = np.random.default_rng(7)
    eps = 1e-6
    checked = 0
    for name, arr, grad in (("q", q, g["dq"]), ("k", k, g["dk"]), ("v", v, g["dv"])):
        idx = rng.choice(arr.size, size=40, replace=False)
        for i in idx:
            plus, minus = arr.copy(), arr.copy()
            plus.flat[i] += eps
            minus.flat[i] -= eps
            args = {"q": q, "k": k, "v": v}
            lp, mp = loss(orc, **{**args, name: plus}, dout=dout, **kw)
            lm, mm = loss(orc, **{**args, name: minus}, dout=dout, **kw)
            if not (np.array_equal(mp, base["mask"]) and np.array_equal(mm, base["mask"])):
                continue  # the step moved the selection: no derivative there
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad.flat[i]) <= 1e-5 * max(1.0, abs(fd)), (name, i, fd, grad.flat[i])
            checked += 1
    assert checked >= 100


def test_routing_gradient_is_not_negligible(orc):
    """The case above exercises the chain through the routing: with sigma = inf (constant bias)
    the gradients differ by a large margin."""
    q, k, v, dout = case(11)
    kw = dict(block=8, alpha=1.5, gamma=8.0, window=1)
    a = orc.backward(q, k, v, dout, sigma=2.0, **kw)
    b = orc.backward(q, k, v, dout, sigma=math.inf, **kw)
    assert np.abs(a["dq"] - b["dq"]).max() > 0.1 * np.abs(a["dq"]).max()
    assert np.abs(a["dk"] - b["dk"]).max() > 0.1 * np.abs(a["dk"]).max()


def causal_sdpa_grads(q, k, v, dout):
    """Gradients of plain causal SDPA (Eq. 1) by torch autograd, K/V shared by each query group."""
    g = q.shape[2] // k.shape[2]
    f64 = dict(dtype=torch.float64)
    qt = torch.tensor(q[0], **f64).transpose(0, 1).requires_grad_()
    kt = torch.tensor(k[0], **f64).transpose(0, 1).requires_grad_()
    vt = torch.tensor(v[0], **f64).transpose(0, 1).requires_grad_()
    o = torch.nn.functional.scaled_dot_product_attention(
        qt[None], kt.repeat_interleave(g, 0)[None], vt.repeat_interleave(g, 0)[None], is_causal=True)[0]
    o.backward(torch.tensor(dout[0], **f64).transpose(0, 1))
    return (qt.grad.transpose(0, 1).numpy()[None], kt.grad.transpose(0, 1).numpy()[None],
            vt.grad.transpose(0, 1).numpy()[None])


def test_dense_routing_without_bias_is_causal_sdpa(orc):
    """alpha -> 1 routes every chunk and sigma = inf removes the bias: the forward is causal SDPA,
    and no gradient flows through the routing."""
    q, k, v, dout = case(4, n=48)
    g = orc.backward(q, k, v, dout, block=8, alpha=1.0 + 1e-5, gamma=1.0, sigma=math.inf)
    dq, dk, dv = causal_sdpa_grads(q, k, v, dout)
    for a, b in ((g["dq"], dq), (g["dk"], dk), (g["dv"], dv)):
        np.testing.assert_allclose(a, b, atol=1e-10)


def test_window_over_every_chunk_is_causal_sdpa(orc):
    """A window reaching chunk 0 for every query routes nothing: causal SDPA and its gradients."""
    q, k, v, dout = case(5, n=48)
    g = orc.backward(q, k, v, dout, block=8, alpha=1.5, gamma=3.0, sigma=1.0, window=7)
    dq, dk, dv = causal_sdpa_grads(q, k, v, dout)
    for a, b in ((g["dq"], dq), (g["dk"], dk), (g["dv"], dv)):
        np.testing.assert_allclose(a, b, atol=1e-10)
    assert np.all(g["dbias"] == 0.0)


def test_stage2_gradients_match_central_differences(orc):
    """Stage 2 alone with a fixed selection and bias: central differences of the bias-form
    attention for q, k, v and the bias entries."""
    q, k, v, dout = case(12)
    kw = dict(block=8, alpha=1.5, gamma=8.0, sigma=0.5)
    st = orc.forward(q, k, v, **kw)
    mask, bias = st["mask"], st["bias"]
    g = orc.sparse_attn_backward(q, k, v, mask, bias, dout, block=8)

    def loss(q_, k_, v_, bias_):
        o, _ = orc.sparse_attn(q_, k_, v_, mask, bias_, block=8)
        return float((o * dout.reshape(o.shape)).sum())

    rng = np.random.default_rng(8)
    eps = 1e-6
    for name, arr, grad in (("q", q, g["dq"]), ("k", k, g["dk"]), ("v", v, g["dv"])):
        for i in rng.choice(arr.size, size=30, replace=False):
            plus, minus = arr.copy(), arr.copy()
            plus.flat[i] += eps
            minus.flat[i] -= eps
            args = dict(q_=q, k_=k, v_=v, bias_=bias)
            fd = (loss(**{**args, name + "_": plus}) - loss(**{**args, name + "_": minus})) / (2 * eps)
            assert abs(fd - grad.flat[i]) <= 1e-5 * max(1.0, abs(fd)), (name, i)
    # the bias: only routed chunks below the query's own chunk move the output
    nc = bias.shape[-1]
    bits = ((mask[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(mask.shape[:2] + (-1,))[..., :nc]
    rows, heads, chunks = np.nonzero(bits)
    own = chunks == (rows // 8)
    pick = rng.choice(np.flatnonzero(~own), size=30, replace=False)
    for j in pick:
        rr, hh, cc = rows[j], heads[j], chunks[j]
        plus, minus = bias.copy(), bias.copy()
        plus[rr, hh, cc] += eps
        minus[rr, hh, cc] -= eps
        fd = (loss(q, k, v, plus) - loss(q, k, v, minus)) / (2 * eps)
        assert abs(fd - g["dbias"].reshape(bias.shape)[rr, hh, cc]) <= 1e-5 * max(1.0, abs(fd))
    assert np.all(g["dbias"].reshape(bias.shape)[rows[own], heads[own], chunks[own]] == 0.0)


def test_stage2_row_gradients_match_the_full_pass(orc):
    """The row-subset form (dq and dL/dd of listed rows, used to check sampled rows of long
    sequences) against the full pass on a batch of two with a ragged tail, rows listed out of
    order."""
    q, k, v, dout = case(13, n=45)
    q, k, v, dout = (np.concatenate([a, a[:, ::-1].copy()], axis=0) for a in (q, k, v, dout))
    kw = dict(block=8, alpha=1.5, gamma=8.0, sigma=0.5)
    st = orc.forward(q, k, v, **kw)
    mask, bias = st["mask"], st["bias"]
    full = orc.sparse_attn_backward(q, k, v, mask, bias, dout, block=8)
    rows = np.array([89, 3, 44, 45, 0, 60, 17])
    part = orc.sparse_attn_backward_rows(q, k, v, mask[rows], bias[rows],
                                         dout.reshape(-1, 4, 8)[rows], rows, block=8)
    np.testing.assert_allclose(part["dq"], full["dq"].reshape(-1, 4, 8)[rows], rtol=1e-12,
                               atol=1e-12)
    np.testing.assert_allclose(part["dbias"], full["dbias"].reshape(90, 2, -1)[rows], rtol=1e-12,
                               atol=1e-12)


def test_routing_gradient_rows_match_the_full_chain(orc):
    """The routing part on its own (listed rows, and every row with dkbar) against the full
    chain minus the Stage 2 part, with a window of two blocks."""
    q, k, v, dout = case(14, n=80)
    kw = dict(block=8, alpha=1.5, gamma=8.0, sigma=0.5, window=2)
    full = orc.backward(q, k, v, dout, **kw)
    st = orc.forward(q, k, v, **kw)
    s2 = orc.sparse_attn_backward(q, k, v, st["mask"], st["bias"], dout, block=8)
    dd = s2["dbias"].reshape(st["w"].shape)
    rk = dict(n_kv=80, block=8, alpha=1.5, gamma=8.0, sigma=0.5, window=2)
    rows = np.array([79, 40, 17, 63, 5])
    part = orc.block_entmax_backward(q, st["kbar"], dd[rows], rows=rows, **rk)
    route_dq = (full["dq"] - s2["dq"]).reshape(80, 4, 8)
    np.testing.assert_allclose(part["dq"], route_dq[rows], rtol=1e-10, atol=1e-12)
    assert np.abs(route_dq).max() > 1e-3  # the routing part is present
    every = orc.block_entmax_backward(q, st["kbar"], dd, want_dkbar=True, **rk)
    np.testing.assert_allclose(every["dq"], route_dq, rtol=1e-10, atol=1e-12)
    dk_route = np.repeat(every["dkbar"], 8, axis=1) / 8  # mean pooling: each key gets dkbar / Bc
    np.testing.assert_allclose(dk_route, full["dk"] - s2["dk"], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("per", ["head", "chunk", "sequence_chunk"])
def test_learned_pooling_gradients_match_central_differences(orc, per):
    """Eq. 3's local attention, differentiated: dk and dqbar of <dkbar, kbar(k, qbar)> against
    central differences of the oracle's own pooling, for one query per KV head, per chunk, and per
    sequence and chunk (a shared query collects the sum over what shares it)."""
    rng = np.random.default_rng(21)
    b, n, hkv, d, block = 2, 40, 2, 4, 8
    tc = n // block
    k = rng.standard_normal((b, n, hkv, d))
    shape = {"head": (hkv, d), "chunk": (tc, hkv, d), "sequence_chunk": (b, tc, hkv, d)}[per]
    qbar = rng.standard_normal(shape) * 1.5
    dkbar = rng.standard_normal((b, tc, hkv, d))
    g = orc.pool_keys_query_backward(k, qbar, dkbar, block)
    f = lambda kk, qq: float((orc.pool_keys_query(kk, qq, block) * dkbar).sum())
    eps = 1e-6
    for idx in [(0, 3, 1, 2), (1, 17, 0, 0), (1, 39, 1, 3), (0, 8, 0, 1)]:
        kp, km = k.copy(), k.copy()
        kp[idx] += eps
        km[idx] -= eps
        num = (f(kp, qbar) - f(km, qbar)) / (2 * eps)
        if idx[1] >= tc * block:   # the incomplete tail has no summary, so no gradient
            assert g["dk"][idx] == 0.0
        assert abs(num - g["dk"][idx]) <= 1e-7 * max(1.0, abs(num))
    flat = qbar.reshape(-1)
    for j in range(0, flat.size, max(1, flat.size // 6)):
        qp, qm = flat.copy(), flat.copy()
        qp[j] += eps
        qm[j] -= eps
        num = (f(k, qp.reshape(shape)) - f(k, qm.reshape(shape))) / (2 * eps)
        assert abs(num - g["dqbar"].reshape(-1)[j]) <= 1e-7 * max(1.0, abs(num))


def test_learned_pooling_gradient_at_zero_query_is_the_mean_pooling_gradient(orc):
    """At qbar = 0 every weight is 1 / B, so dk_t = dkbar_c / B plus the logit term ds_t qbar = 0;
    and dqbar_c = sum_t (1/B)(g_t - mean g) k_t / sqrt(D), the covariance of g and k in the chunk."""
    rng = np.random.default_rng(22)
    k = rng.standard_normal((1, 16, 1, 4))
    dkbar = rng.standard_normal((1, 2, 1, 4))
    g = orc.pool_keys_query_backward(k, np.zeros((1, 4)), dkbar, 8)
    np.testing.assert_allclose(g["dk"][0, :8, 0], np.broadcast_to(dkbar[0, 0, 0] / 8, (8, 4)), atol=1e-15)
    np.testing.assert_allclose(g["dk"][0, 8:, 0], np.broadcast_to(dkbar[0, 1, 0] / 8, (8, 4)), atol=1e-15)
    want = np.zeros(4)
    for c in range(2):
        kc = k[0, 8 * c:8 * c + 8, 0]
        gt = kc @ dkbar[0, c, 0]
        want += ((gt - gt.mean())[:, None] * kc).sum(axis=0) / 8 / 2.0
    np.testing.assert_allclose(g["dqbar"][0], want, atol=1e-14)
