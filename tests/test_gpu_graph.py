"""The decode step captured in a HIP graph and replayed, as the benchmark times it: every replay,
with eager work and synchronisations between the replays, gives the eager step's output bit for
bit (fixed context and per-sequence lengths)."""
from __future__ import annotations

import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def dash():
    import sparse_hierarchical_attention_amd as d
    d.lib()
    return d


def capture(step):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("varlen", [False, True])
def test_decode_step_graph_replays(dash, varlen, fused):
    w = wl.Workload("graph decode", 4, 4096 + 17, 32, 8, 128, 64, 1.5, 1.5, 1.0, decode=True,
                    plant="decode", plant_args=dict(lo=1, hi=8), seed=41)
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    kbar = dash.dash_pool_keys(k, w.block)
    nc = -(-w.n_kv // w.block)
    mask = torch.empty((w.batch, 1, w.h_kv, -(-nc // 32)), dtype=torch.int32, device=DEV)
    bias = torch.empty((w.batch, 1, w.h_kv, nc), dtype=torch.float32, device=DEV)
    o = torch.empty_like(q)
    rws = torch.zeros(max(1, dash.dash_block_entmax_workspace_bytes(
        q.dtype, w.batch, 1, w.n_kv - 1, w.n_kv, w.h_q, w.h_kv, w.head_dim, w.block)),
        dtype=torch.uint8, device=DEV)
    awb = dash.dash_decode_workspace_bytes(w.batch, w.n_kv, w.h_q, w.h_kv, w.head_dim, w.block)
    aws = torch.zeros(awb, dtype=torch.uint8, device=DEV) if awb else None
    sws = torch.zeros(dash.dash_decode_step_workspace_bytes(w.batch, w.n_kv, w.h_q, w.h_kv,
                                                            w.head_dim, w.block),
                      dtype=torch.uint8, device=DEV)
    lens = wl.ragged_lengths(w.batch, w.n_kv, 42, DEV)
    kw = dict(block=w.block, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma)

    def step():
        if fused:
            if varlen:
                dash.dash_pool_keys_append(k, lens, kbar, w.block)
            dash.dash_decode_step(q, k, v, kbar, ctx_lens=lens if varlen else None, mask=mask,
                                  bias=bias, o=o, workspace=sws, **kw)
        elif varlen:
            dash.dash_pool_keys_append(k, lens, kbar, w.block)
            dash.dash_block_entmax_ex(q, kbar, n_kv=w.n_kv, h_kv=w.h_kv, ctx_lens=lens, mask=mask,
                                      bias=bias, want_tau=False, workspace=rws, **kw)
            dash.dash_sparse_attn_decode_varlen(q, k, v, lens, mask, bias, block=w.block, o=o,
                                                workspace=aws)
        else:
            dash.dash_block_entmax(q, kbar, n_kv=w.n_kv, q_pos0=w.n_kv - 1, mask=mask, bias=bias,
                                   want_tau=False, workspace=rws, **kw)
            dash.dash_sparse_attn_decode(q, k, v, mask, bias, block=w.block, o=o, workspace=aws)

    step()
    torch.cuda.synchronize()
    want_o, want_mask = o.clone(), mask.clone()
    g = capture(step)
    for i in range(4):
        o.zero_()
        mask.zero_()
        # eager work between the replays: the same step run eagerly on other outputs' buffers is
        # not needed; an unrelated kernel and a synchronisation are
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, want_o), f"replay {i}: output differs"
        assert torch.equal(mask, want_mask), f"replay {i}: mask differs"
        del junk
