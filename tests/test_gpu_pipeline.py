"""Row blocks: routing and attending the query rows of a prefill in blocks (as the benchmark's
pipelined step does, routing one block while attending the previous one on another stream)
gives every row the mask of one call over all rows bit for bit, and its output and lse up to
rounding: the 128-row tile a row falls into decides whether a chunk's exponent is evaluated as one
fused multiply-add or two (the path of the tile's own chunks), so the last bit may differ."""
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


@pytest.mark.parametrize("dtype,d,block,hq,hkv", [("bf16", 128, 64, 32, 8), ("bf16", 64, 32, 16, 1),
                                                  ("bf16", 128, 128, 8, 2), ("f32", 128, 64, 8, 4)])
def test_row_blocks_match_one_call(dash, dtype, d, block, hq, hkv):
    n = 3000
    w = wl.Workload(f"row blocks {dtype} D{d} block {block}", 1, n, hq, hkv, d, block, 1.5, 0.5, 1.0,
                    dtype=dtype, plant="span", plant_args=dict(span=8, per_span=2), seed=51)
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    kw = dict(n_kv=n, block=block, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma, h_kv=hkv)
    kbar = dash.dash_pool_keys(k, block)
    mask, bias, _ = dash.dash_block_entmax(q, kbar, want_tau=False, **kw)
    o, lse = dash.dash_sparse_attn_prefill(q, k, v, mask, bias, block=block)
    for t0, t1 in [(0, 700), (700, 1234), (1234, 2048), (2048, 2999), (2999, 3000)]:
        qs = q[:, t0:t1].contiguous()
        ms, bs, _ = dash.dash_block_entmax(qs, kbar, q_pos0=t0, want_tau=False, **kw)
        os_, ls = dash.dash_sparse_attn_prefill(qs, k, v, ms, bs, block=block, q_pos0=t0)
        torch.cuda.synchronize()
        assert torch.equal(ms, mask[:, t0:t1]), (t0, t1)
        ref_o = o[:, t0:t1].float()
        d_o = (os_.float() - ref_o).abs().max().item()
        d_l = (ls - lse[:, t0:t1]).abs().max().item()
        # end to end, the block's own routing included (a one-row block routes through the decode
        # solver, whose tau can differ in the last bit): one rounding step of the output's type at
        # its largest magnitude; lse in fp32
        ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -20
        assert d_o <= ulp * ref_o.abs().max().item(), (t0, t1, d_o)
        assert d_l <= 1e-5, (t0, t1, d_l)
        if dtype == "bf16":
            # Stage 2 alone on the single call's own mask and bias rows: one softmax path for every
            # tile, so a row's result does not depend on the row tiling
            o2, l2 = dash.dash_sparse_attn_prefill(qs, k, v, mask[:, t0:t1].contiguous(),
                                                   bias[:, t0:t1].contiguous(), block=block, q_pos0=t0)
            torch.cuda.synchronize()
            assert torch.equal(o2, o[:, t0:t1]) and torch.equal(l2, lse[:, t0:t1]), (t0, t1)


def test_row_block_rejects_rows_past_the_sequence(dash):
    q = torch.zeros(1, 10, 8, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16, device=DEV)
    mask = torch.zeros(1, 10, 2, 1, dtype=torch.int32, device=DEV)
    bias = torch.zeros(1, 10, 2, 1, dtype=torch.float32, device=DEV)
    with pytest.raises(dash.DashError, match="q_pos0"):
        dash.dash_sparse_attn_prefill(q, k, k, mask, bias, block=64, q_pos0=60)
