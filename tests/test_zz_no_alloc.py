"""dash_decode_step_noalloc (the decode step on the library's own device scratch, for callers
that cannot allocate) against dash_decode_step on its own workspace: two calls in a row, the
second on a smaller input, each bit for bit equal; per-sequence lengths too."""
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


def _outputs(w, inp):
    nc = -(-w.n_kv // w.block)
    return (torch.zeros((w.batch, 1, w.h_kv, -(-nc // 32)), dtype=torch.int32, device=DEV),
            torch.zeros((w.batch, 1, w.h_kv, nc), dtype=torch.float32, device=DEV),
            torch.zeros_like(inp["q"]))


@pytest.mark.parametrize("varlen", [False, True])
def test_noalloc_matches_workspace_entry(dash, varlen):
    big = wl.Workload("noalloc decode", 6, 8192 + 40, 32, 8, 128, 64, 1.5, 1.5, 1.0, decode=True,
                      plant="decode", plant_args=dict(lo=1, hi=8), seed=47)
    small = big.with_(batch=2, n_kv=3000, seed=48)
    for w in (big, small):  # two calls in a row, the second smaller
        inp = wl.make_inputs(w, DEV)
        q, k, v = inp["q"], inp["k"], inp["v"]
        kbar = dash.dash_pool_keys(k, w.block)
        lens = wl.ragged_lengths(w.batch, w.n_kv, 49, DEV) if varlen else None
        kw = dict(block=w.block, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma, ctx_lens=lens)
        want_o, want_m, want_b = dash.dash_decode_step(q, k, v, kbar, **kw)
        m, b, o = _outputs(w, inp)
        dash.dash_decode_step_noalloc(q, k, v, kbar, mask=m, bias=b, o=o, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o, want_o), f"{w.batch} x {w.n_kv}: outputs differ"
        assert torch.equal(m, want_m), f"{w.batch} x {w.n_kv}: masks differ"
        bits = ((want_m.view(torch.int32).unsqueeze(-1) >> torch.arange(32, device=DEV)) & 1)
        sel = bits.flatten(-2)[..., :b.shape[-1]].bool()
        assert torch.equal(b[sel], want_b[sel]), f"{w.batch} x {w.n_kv}: biases differ"


def test_noalloc_rejects_calls_past_its_scratch(dash):
    """A call that needs more than the scratch holds is rejected before anything launches."""
    w = wl.Workload("noalloc too big", 64, 131072, 32, 8, 128, 64, 1.5, 1.5, 1.0, decode=True)
    need = dash.dash_decode_step_workspace_bytes(w.batch, w.n_kv, 32, 8, 128, 64)
    assert need > 32 << 20
    q = torch.zeros((w.batch, 1, 32, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((1, 1, 1, 1), dtype=torch.bfloat16, device=DEV).expand(w.batch, w.n_kv, 8, 128)
    kbar = torch.zeros((1,), dtype=torch.float32, device=DEV)
    m = torch.zeros((1,), dtype=torch.int32, device=DEV)
    b = torch.zeros((1,), dtype=torch.float32, device=DEV)
    L = dash.lib()
    import ctypes
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = L.dash_decode_step_noalloc(p(q), p(kv), p(kv), 1, p(kbar), None, w.batch, w.n_kv, 32, 8,
                                    128, 64, 1.5, 1.5, 1.0, 1, 0.088, p(m), p(b), p(q), None)
    assert st == 3 and b"scratch" in L.dash_last_error()
