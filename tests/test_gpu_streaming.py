"""GPU parity of the incremental-decoding features: the attention window of the pages'
training setup ("DashAttention", App. B.1.1), per-sequence context lengths in one cache, and
chunk summaries written as decoding completes each chunk (§3.1, §3.5). Every case is checked
against the oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from tests import parity
from tests.test_gpu_parity import flat_rows, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def dash():
    import sparse_hierarchical_attention_amd as d
    d.lib()
    return d


def window_bias_is_zero(gpu_bias, ref_mask, ref_w, nc):
    """Bias entries of the window's chunks (mask bit set, not routed) are exactly 0."""
    ob = parity.bits(ref_mask, nc)
    win = ob & ~(ref_w > 0)
    assert np.all(gpu_bias[win] == 0.0)


@pytest.mark.parametrize("window", [2, 3])
@pytest.mark.parametrize("dtype,n,hq,hkv,d,block", [("bf16", 2000, 8, 2, 128, 64),
                                                     ("bf16", 1500, 32, 2, 128, 64),
                                                     ("f32", 1024, 2, 1, 64, 64)])
def test_window_prefill(dash, orc, window, dtype, n, hq, hkv, d, block):
    w = wl.Workload("window prefill", 1, n, hq, hkv, d, block, 1.5, 0.5 if dtype == "bf16" else 8.0,
                    1.0, dtype=dtype, plant="span" if dtype == "bf16" else "none",
                    plant_args=dict(span=8, per_span=2), seed=81)
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    kbar = dash.dash_pool_keys(k, block)
    mask, bias, tau = dash.dash_block_entmax_ex(q, kbar, n_kv=n, block=block, alpha=w.alpha,
                                                gamma=w.gamma, sigma=w.sigma, h_kv=hkv,
                                                window_blocks=window)
    o, lse = dash.dash_sparse_attn_prefill(q, k, v, mask, bias, block=block)
    torch.cuda.synchronize()
    ref = orc.forward(host(q), host(k), host(v), block=block, alpha=w.alpha, gamma=w.gamma,
                      sigma=w.sigma, window=window)
    rows = np.arange(n)
    parity.check_forward(orc, host(q), host(k), host(v), ref, mask=flat_rows(mask, rows),
                         bias=flat_rows(bias, rows), tau=flat_rows(tau, rows), o=flat_rows(o, rows),
                         lse=flat_rows(lse, rows), rows=rows, n_kv=n, block=block, h_kv=hkv,
                         q_pos=rows, alpha=w.alpha, sigma=w.sigma, dtype=dtype,
                         vmax=float(v.abs().max()))
    window_bias_is_zero(flat_rows(bias, rows), ref["mask"], ref["w"], -(-n // block))


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("window", [1, 2, 4])
def test_window_decode(dash, orc, window, fused):
    n, block = 4096 + 40, 64
    w = wl.Workload("window decode", 3, n, 8, 2, 128, block, 1.5, 1.5, 1.0, decode=True,
                    plant="decode", plant_args=dict(lo=1, hi=8), seed=82)
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    kbar = dash.dash_pool_keys(k, block)
    if fused:
        o, mask, bias = dash.dash_decode_step(q, k, v, kbar, block=block, alpha=1.5, gamma=1.5,
                                              sigma=1.0, window_blocks=window)
        tau = None
    else:
        mask, bias, tau = dash.dash_block_entmax_ex(q, kbar, n_kv=n, block=block, alpha=1.5,
                                                    gamma=1.5, sigma=1.0, q_pos0=n - 1, h_kv=2,
                                                    window_blocks=window)
        o = dash.dash_sparse_attn_decode(q, k, v, mask, bias, block=block)
    torch.cuda.synchronize()
    ref = orc.forward(host(q), host(k), host(v), block=block, alpha=1.5, gamma=1.5, sigma=1.0,
                      q_pos0=n - 1, window=window)
    rows = np.arange(w.batch)
    parity.check_forward(orc, host(q), host(k), host(v), ref, mask=flat_rows(mask, rows),
                         bias=flat_rows(bias, rows), tau=None if tau is None else flat_rows(tau, rows),
                         o=flat_rows(o, rows), rows=rows, n_kv=n, block=block, h_kv=2,
                         q_pos=np.full(w.batch, n - 1),
                         q_pos0=n - 1, alpha=1.5, sigma=1.0, dtype="bf16",
                         vmax=float(v.abs().max()), max_flip_frac=0.34)
    window_bias_is_zero(flat_rows(bias, rows), ref["mask"], ref["w"], -(-n // block))


def _varlen_reference(orc, q, k, v, lens, block, alpha, gamma, sigma, window=1):
    """The oracle on each sequence alone, cut to its own length."""
    out = []
    for b, n_b in enumerate(lens):
        out.append(orc.forward(host(q[b:b + 1]), host(k[b:b + 1, :n_b]), host(v[b:b + 1, :n_b]),
                               block=block, alpha=alpha, gamma=gamma, sigma=sigma,
                               q_pos0=n_b - 1, window=window))
    return out


def _check_varlen_rows(q, k, v, gpu_mask, gpu_bias, gpu_tau, gpu_o, refs, lens, block, hkv, alpha,
                       sigma, vmax):
    """Each sequence b against the oracle on its first lens[b] tokens (ref = refs[b])."""
    nw_cap = gpu_mask.shape[-1]
    for b, (ref, n_b) in enumerate(zip(refs, lens)):
        nc_b = -(-n_b // block)
        nw_b = -(-nc_b // 32)
        gm = np.ascontiguousarray(gpu_mask[b:b + 1, :, :nw_b])
        assert not np.any(gpu_mask[b, :, nw_b:nw_cap]), "bits past the sequence"
        gbias = np.ascontiguousarray(gpu_bias[b:b + 1, :, :nc_b])
        parity.check_forward(orc_module(), host(q[b:b + 1]), host(k[b:b + 1, :n_b]),
                             host(v[b:b + 1, :n_b]), ref, mask=gm, bias=gbias,
                             tau=None if gpu_tau is None else gpu_tau[b:b + 1], o=gpu_o[b:b + 1],
                             rows=np.array([0]), n_kv=n_b, block=block, h_kv=hkv,
                             q_pos=np.array([n_b - 1]), q_pos0=n_b - 1, alpha=alpha, sigma=sigma,
                             dtype="bf16", vmax=vmax, max_flip_frac=1.0)


def orc_module():
    import oracle
    return oracle


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("window", [1, 2])
def test_varlen_decode(dash, orc, window, fused):
    """One cache of capacity 5000 holding sequences of different lengths: a single token, chunk
    edges on both sides, a ragged middle length and a full cache."""
    cap, block = 5000, 64
    lens = [1, 63, 64, 65, 129, 3000, 4097, 5000]
    w = wl.Workload("varlen decode", len(lens), cap, 8, 2, 128, block, 1.5, 1.5, 1.0,
                    decode=True, plant="decode", plant_args=dict(lo=1, hi=8), seed=83)
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    ctx = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kbar = dash.dash_pool_keys(k, block)  # summaries past a sequence's length are never read
    if fused:
        o, mask, bias = dash.dash_decode_step(q, k, v, kbar, block=block, alpha=1.5, gamma=1.5,
                                              sigma=1.0, ctx_lens=ctx, window_blocks=window)
        tau = None
    else:
        mask, bias, tau = dash.dash_block_entmax_ex(q, kbar, n_kv=cap, block=block, alpha=1.5,
                                                    gamma=1.5, sigma=1.0, h_kv=2, ctx_lens=ctx,
                                                    window_blocks=window)
        o = dash.dash_sparse_attn_decode_varlen(q, k, v, ctx, mask, bias, block=block)
    torch.cuda.synchronize()
    refs = _varlen_reference(orc, q, k, v, lens, block, 1.5, 1.5, 1.0, window)
    rows = np.arange(len(lens))
    _check_varlen_rows(q, k, v, flat_rows(mask, rows), flat_rows(bias, rows),
                       None if tau is None else flat_rows(tau, rows), flat_rows(o, rows), refs,
                       lens, block, 2, 1.5, 1.0, float(v.abs().max()))


@pytest.mark.parametrize("learned", [False, True, "per_chunk"])
def test_streaming_decode(dash, orc, learned):
    """Decode steps that append one token per sequence: the summary of each chunk the new token
    completes is written by the append call (and nothing else is), and every step's route and
    attention match the oracle on the sequences as they stand."""
    cap, block, steps = 1024, 32, 70
    start = [100, 127, 128, 31]
    w = wl.Workload("streaming decode", len(start), cap, 8, 2, 128, block, 1.5, 1.5, 1.0,
                    decode=True, plant="decode", plant_args=dict(lo=1, hi=6), seed=84)
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    tc = cap // block
    qshape = (tc, 2, 128) if learned == "per_chunk" else (2, 128)
    qbar = (torch.randn(qshape, generator=torch.Generator().manual_seed(9)) * 0.3).to(DEV) if learned else None
    kbar = torch.full((len(start), tc, 2, 128), float("nan"), dtype=torch.float32, device=DEV)
    # summaries of the chunks complete before the first step, written by the full pooling
    full = dash.dash_pool_keys_query(k, qbar, block) if learned else dash.dash_pool_keys(k, block)
    for b, n0 in enumerate(start):
        kbar[b, :n0 // block] = full[b, :n0 // block]
    lens = list(start)
    ctx = torch.tensor(lens, dtype=torch.int32, device=DEV)
    for step in range(steps):
        lens = [n + 1 for n in lens]
        ctx.copy_(torch.tensor(lens, dtype=torch.int32))
        dash.dash_pool_keys_append(k, ctx, kbar, block, qbar=qbar)
        if step % 23 == 0 or step == steps - 1:
            mask, bias, tau = dash.dash_block_entmax_ex(q, kbar, n_kv=cap, block=block, alpha=1.5,
                                                        gamma=1.5, sigma=1.0, h_kv=2, ctx_lens=ctx)
            o = dash.dash_sparse_attn_decode_varlen(q, k, v, ctx, mask, bias, block=block)
            torch.cuda.synchronize()
            rows = np.arange(len(lens))
            if learned:
                refs = []
                for b, n_b in enumerate(lens):
                    qb = host(qbar).double().numpy()
                    if learned == "per_chunk":
                        qb = qb[:n_b // block]
                    kb_ref = orc.pool_keys_query(host(k[b:b + 1, :n_b]), qb, block)
                    st1 = orc.block_entmax(host(q[b:b + 1]), kb_ref, n_kv=n_b, block=block, alpha=1.5,
                                           gamma=1.5, sigma=1.0, q_pos0=n_b - 1, h_kv=2)
                    ob, _ = orc.sparse_attn(host(q[b:b + 1]), host(k[b:b + 1, :n_b]),
                                            host(v[b:b + 1, :n_b]), st1["mask"], st1["bias"],
                                            block=block, q_pos0=n_b - 1)
                    refs.append(dict(o=ob, **st1))
            else:
                refs = _varlen_reference(orc, q, k, v, lens, block, 1.5, 1.5, 1.0)
            _check_varlen_rows(q, k, v, flat_rows(mask, rows), flat_rows(bias, rows),
                               flat_rows(tau, rows), flat_rows(o, rows), refs, lens, block, 2, 1.5, 1.0,
                               float(v.abs().max()))
    torch.cuda.synchronize()
    kb = kbar.cpu().numpy()
    for b, n_b in enumerate(lens):
        t_b = n_b // block
        qb = None if not learned else host(qbar).double().numpy()
        if learned == "per_chunk":
            qb = qb[:t_b]
        ref = (orc.pool_keys_query(host(k[b:b + 1, :t_b * block]), qb, block)
               if learned else orc.pool_keys(host(k[b:b + 1, :t_b * block]), block))
        np.testing.assert_allclose(kb[b:b + 1, :t_b], ref, rtol=1e-5, atol=1e-5)
        assert np.all(np.isnan(kb[b, t_b:])), "a summary was written for an open chunk"
