"""GPU parity: libdash (through its C ABI) against the double-precision oracle on the same seeded
inputs. Small cases compare every row; full-size workloads compare sampled rows."""
from __future__ import annotations

import math

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


def host(t):
    return t.detach().cpu()


def sample_rows(n_q: int, block: int, count: int, seed: int, batch: int = 1) -> np.ndarray:
    """Query rows to check: chunk edges, the first and last rows, and random rows."""
    rng = np.random.default_rng(seed)
    fixed = {0, 1, block - 1, block, block + 1, 2 * block - 1, n_q // 2, n_q - 2, n_q - 1}
    fixed |= set(range(0, n_q, max(1, n_q // 8)))
    rows = sorted(r for r in fixed if 0 <= r < n_q)
    extra = rng.choice(n_q, size=min(count, n_q), replace=False)
    rows = sorted(set(rows) | set(int(e) for e in extra))
    return np.array([b * n_q + r for b in range(batch) for r in rows], dtype=np.int64)


def flat_rows(t: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    """[B, n_q, ...] GPU tensor -> host array of the listed rows rho = b * n_q + t (gathered on
    the device, so that a multi-GiB bias never crosses to the host whole)."""
    flat = t.reshape((-1,) + tuple(t.shape[2:]))
    idx = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=t.device)
    return parity.to_host(flat.index_select(0, idx))


def run_and_compare(dash, orc, w: wl.Workload, alpha, gamma, sigma, rows=None, max_flip_frac=0.02):
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    res = dash.forward(q, k, v, block=w.block, alpha=alpha, gamma=gamma, sigma=sigma)
    torch.cuda.synchronize()
    qh, kh, vh = host(q), host(k), host(v)
    ref = orc.forward(qh, kh, vh, block=w.block, alpha=alpha, gamma=gamma, sigma=sigma, rows=rows)
    all_rows = np.arange(w.batch * w.n_q) if rows is None else rows
    # Stage 0 in full
    kb_ref = ref["kbar"]
    kb = res["kbar"].cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(kb, kb_ref, rtol=1e-6, atol=1e-6)
    rep = parity.check_forward(orc, qh, kh, vh, ref, mask=flat_rows(res["mask"], all_rows),
                               bias=flat_rows(res["bias"], all_rows),
                               tau=flat_rows(res["tau"], all_rows), o=flat_rows(res["o"], all_rows),
                               lse=flat_rows(res["lse"], all_rows), rows=all_rows, n_kv=w.n_kv,
                               block=w.block, h_kv=w.h_kv, q_pos=all_rows % w.n_q, alpha=alpha,
                               sigma=sigma, dtype=w.dtype, vmax=float(v.abs().max()),
                               max_flip_frac=max_flip_frac)
    return rep


# ------------------------------------------------------------------------------ Stage 0

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n,hkv,d,block", [(1024, 1, 64, 64), (1000, 3, 128, 32), (333, 8, 128, 128),
                                           (64, 2, 64, 64)])
def test_pool_keys(dash, orc, dtype, n, hkv, d, block):
    w = wl.Workload("pool", 2, n, hkv, hkv, d, block, 1.5, 1.0, 1.0, dtype=dtype, seed=21)
    inp = wl.make_inputs(w, DEV)
    kb = dash.dash_pool_keys(inp["k"], block)
    torch.cuda.synchronize()
    np.testing.assert_allclose(kb.cpu().numpy(), orc.pool_keys(host(inp["k"]), block), rtol=1e-6,
                               atol=1e-6)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pool_keys_learned_query(dash, orc, dtype):
    w = wl.Workload("poolq", 2, 640, 4, 4, 128, 64, 1.5, 1.0, 1.0, dtype=dtype, seed=22)
    inp = wl.make_inputs(w, DEV)
    qbar = torch.randn(4, 128, generator=torch.Generator().manual_seed(5)) * 0.3
    kb = dash.dash_pool_keys_query(inp["k"], qbar.to(DEV), 64)
    torch.cuda.synchronize()
    ref = orc.pool_keys_query(host(inp["k"]), qbar.double().numpy(), 64)
    np.testing.assert_allclose(kb.cpu().numpy(), ref, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("per", ["chunk", "sequence_chunk"])
@pytest.mark.parametrize("d,block", [(128, 64), (64, 32), (128, 128)])
def test_pool_keys_per_chunk_query(dash, orc, dtype, per, d, block):
    """Stage 0 with one summary query per chunk (Alg. 1's qbar [Tc, Hkv, D]) or per sequence and
    chunk, against the oracle; a ragged tail chunk gets no summary."""
    w = wl.Workload("poolq chunks", 2, 5 * block + 7, 4, 4, d, block, 1.5, 1.0, 1.0, dtype=dtype,
                    seed=23)
    inp = wl.make_inputs(w, DEV)
    tc = w.n_kv // block
    shape = (tc, 4, d) if per == "chunk" else (2, tc, 4, d)
    qbar = torch.randn(shape, generator=torch.Generator().manual_seed(6)) * 0.4
    kb = dash.dash_pool_keys_query(inp["k"], qbar.to(DEV), block)
    torch.cuda.synchronize()
    ref = orc.pool_keys_query(host(inp["k"]), qbar.double().numpy(), block)
    np.testing.assert_allclose(kb.cpu().numpy(), ref, rtol=1e-5, atol=1e-5)
    # equal queries in every chunk give the per-head result
    same = qbar.reshape(-1, 4, d)[:1].expand(shape[:-2] + (4, d)).contiguous()
    a = dash.dash_pool_keys_query(inp["k"], same.to(DEV), block)
    bq = dash.dash_pool_keys_query(inp["k"], qbar.reshape(-1, 4, d)[0].contiguous().to(DEV), block)
    torch.cuda.synchronize()
    assert torch.equal(a, bq)


# ------------------------------------------------------------------ tiny fp32 workload, in full

@pytest.mark.parametrize("gamma", [1.0, 8.0, 32.0])
@pytest.mark.parametrize("sigma", [1.0, 10.0, 1e8])
def test_tiny_fp32_alpha15(dash, orc, gamma, sigma):
    run_and_compare(dash, orc, wl.TINY, 1.5, gamma, sigma)


@pytest.mark.parametrize("alpha", [1.25, 2.0])
@pytest.mark.parametrize("gamma", [1.0, 8.0, 32.0])
def test_tiny_fp32_other_alpha(dash, orc, alpha, gamma):
    run_and_compare(dash, orc, wl.TINY, alpha, gamma, 10.0)


def test_tiny_fp32_sigma_inf(dash, orc):
    run_and_compare(dash, orc, wl.TINY, 1.5, 8.0, math.inf)


# ------------------------------------------------------------- bf16, several tiles, ragged tail

SMALL_BF16 = [
    # batch, n, hq, hkv, d, block
    (1, 2048, 8, 2, 128, 64),
    (2, 2000, 8, 2, 128, 64),     # ragged tail chunk of 16 tokens
    (1, 1536, 16, 1, 64, 32),     # group of 16
    (1, 1500, 16, 2, 128, 64),    # group of 8, ragged
    (1, 1100, 4, 4, 128, 128),    # group of 1, ragged
    (1, 777, 4, 2, 64, 64),
    (1, 40, 4, 2, 128, 64),       # shorter than one chunk: diagonal only
    (1, 64, 2, 1, 128, 64),       # exactly one chunk
]


@pytest.mark.parametrize("shape", SMALL_BF16)
@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_small_bf16_planted(dash, orc, shape, alpha):
    b, n, hq, hkv, d, block = shape
    w = wl.Workload("small bf16", b, n, hq, hkv, d, block, alpha, 0.5, 1.0, plant="span",
                    plant_args=dict(span=8, per_span=2), seed=31)
    run_and_compare(dash, orc, w, alpha, 0.5 if alpha != 2.0 else 1.0, 1.0)


@pytest.mark.parametrize("sigma", [1.0, 1e8, math.inf])
def test_small_bf16_unplanted(dash, orc, sigma):
    w = wl.Workload("small bf16 noise", 1, 1500, 8, 2, 128, 64, 1.5, 4.0, sigma, seed=32)
    run_and_compare(dash, orc, w, 1.5, 4.0, sigma)


def test_stage2_on_oracle_selection(dash, orc):
    """Stage 2 alone: the GPU kernel fed with the oracle's own mask and bias matches the oracle
    on every row (no near-threshold exclusions)."""
    w = wl.Workload("stage2", 1, 1200, 8, 2, 128, 64, 1.5, 0.5, 1.0, plant="span",
                    plant_args=dict(span=8, per_span=2), seed=33)
    inp = wl.make_inputs(w, DEV)
    qh, kh, vh = host(inp["q"]), host(inp["k"]), host(inp["v"])
    ref = orc.forward(qh, kh, vh, block=w.block, alpha=1.5, gamma=0.5, sigma=1.0)
    mask = torch.from_numpy(ref["mask"].view(np.int32)).reshape(1, w.n_q, w.h_kv, -1).to(DEV)
    bias = torch.from_numpy(ref["bias"].astype(np.float32)).reshape(1, w.n_q, w.h_kv, -1).to(DEV)
    o, lse = dash.dash_sparse_attn_prefill(inp["q"], inp["k"], inp["v"], mask, bias, block=w.block)
    torch.cuda.synchronize()
    parity.compare_output(parity.to_host(o)[0], ref["o"], "bf16", gpu_lse=parity.to_host(lse)[0],
                          ref_lse=ref["lse"])


# --------------------------------------------- keys past a sequence's end are never read

@pytest.mark.parametrize("n,hq,hkv,block", [(2000, 8, 2, 64), (1000 + 7, 32, 2, 128),
                                            (777, 4, 4, 32)])
def test_prefill_tail_stays_inside_sequence(dash, orc, n, hq, hkv, block):
    """The last key tile of a sequence whose length is not a multiple of the tile reads nothing
    past that sequence. One sequence: K and V are the first n rows of a buffer whose following
    rows hold NaN. Two sequences: the second one's K and V are all NaN, and the first one's
    outputs must still be finite and match the oracle on every row."""
    w = wl.Workload("tail", 1, n, hq, hkv, 128, block, 1.5, 0.5, 1e8, seed=36)
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    mask, bias = wl.random_selection(1, n, 0, n, hkv, block, 0.5, seed=9, device=DEV,
                                     bias_std=0.5)
    nan = float("nan")
    kb = torch.full((1, n + 64, hkv, 128), nan, dtype=torch.bfloat16, device=DEV)
    vb = torch.full((1, n + 64, hkv, 128), nan, dtype=torch.bfloat16, device=DEV)
    kb[:, :n] = k
    vb[:, :n] = v
    o1, lse1 = dash.dash_sparse_attn_prefill(q, kb[:, :n], vb[:, :n], mask, bias, block=block)
    # two sequences, the second all NaN
    q2 = torch.cat([q, q]).contiguous()
    k2 = torch.cat([k, torch.full_like(k, nan)]).contiguous()
    v2 = torch.cat([v, torch.full_like(v, nan)]).contiguous()
    o2, lse2 = dash.dash_sparse_attn_prefill(q2, k2, v2, torch.cat([mask, mask]).contiguous(),
                                             torch.cat([bias, bias]).contiguous(), block=block)
    torch.cuda.synchronize()
    m, bi = _compact(mask, bias)
    ref_o, ref_lse = orc.sparse_attn(host(q), host(k), host(v), m, bi, block=block)
    for o, lse in ((o1[0], lse1[0]), (o2[0], lse2[0])):
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        parity.compare_output(parity.to_host(o), ref_o, "bf16", gpu_lse=parity.to_host(lse),
                              ref_lse=ref_lse)


# ------------------------------------------------- injected random selections (g = 16, Hkv = 2)

def _compact(mask: torch.Tensor, bias: torch.Tensor):
    """[B, n_q, Hkv, W] / [B, n_q, Hkv, Nc] GPU tensors -> the oracle's per-row host arrays."""
    m = parity.to_host(mask).view(np.uint32)
    bi = parity.to_host(bias).astype(np.float64)
    return m.reshape((-1,) + m.shape[2:]), bi.reshape((-1,) + bi.shape[2:])


@pytest.mark.parametrize("sparsity", [0.0, 0.75, 0.9375])
def test_stage2_random_selection_prefill(dash, orc, sparsity):
    """Stage 2 fed a random selection, as the pages' efficiency sweep injects it (32 query heads
    over 2 KV heads, so groups of 16), with a random bias: every row against the oracle."""
    w = wl.Workload("random selection", 1, 2000, 32, 2, 128, 64, 1.5, 0.5, 1e8, seed=34)
    inp = wl.make_inputs(w, DEV)
    mask, bias = wl.random_selection(1, w.n_q, 0, w.n_kv, w.h_kv, w.block, sparsity, seed=7,
                                     device=DEV, bias_std=0.5)
    o, lse = dash.dash_sparse_attn_prefill(inp["q"], inp["k"], inp["v"], mask, bias, block=w.block)
    torch.cuda.synchronize()
    m, bi = _compact(mask, bias)
    ref_o, ref_lse = orc.sparse_attn(host(inp["q"]), host(inp["k"]), host(inp["v"]), m, bi,
                                     block=w.block)
    parity.compare_output(parity.to_host(o)[0], ref_o, "bf16", gpu_lse=parity.to_host(lse)[0],
                          ref_lse=ref_lse)


@pytest.mark.parametrize("n_ctx", [3000, 4096 + 17])
def test_decode_random_selection(dash, orc, n_ctx):
    """Decode at batch 24 with groups of 16 on a random selection at sparsity 87.5 %."""
    w = wl.Workload("decode random selection", 24, n_ctx, 32, 2, 128, 64, 1.5, 0.5, 1e8,
                    decode=True, seed=43)
    inp = wl.make_inputs(w, DEV)
    mask, bias = wl.random_selection(w.batch, 1, n_ctx - 1, n_ctx, w.h_kv, w.block, 0.875, seed=8,
                                     device=DEV, bias_std=0.5)
    o = dash.dash_sparse_attn_decode(inp["q"], inp["k"], inp["v"], mask, bias, block=w.block)
    torch.cuda.synchronize()
    m, bi = _compact(mask, bias)
    ref_o, _ = orc.sparse_attn(host(inp["q"]), host(inp["k"]), host(inp["v"]), m, bi,
                               block=w.block, q_pos0=n_ctx - 1)
    parity.compare_output(parity.to_host(o).reshape(w.batch, w.h_q, -1), ref_o, "bf16")


# ------------------------------------------------------------------------------ decode

@pytest.mark.parametrize("n_ctx,block", [(4096 + 17, 64), (3000, 32), (1024, 128)])
def test_decode_small(dash, orc, n_ctx, block):
    w = wl.Workload("decode small", 3, n_ctx, 8, 2, 128, block, 1.5, 1.5, 1.0, decode=True,
                    plant="decode", plant_args=dict(lo=1, hi=8), seed=41)
    inp = wl.make_inputs(w, DEV)
    kbar = dash.dash_pool_keys(inp["k"], block)
    o, mask, bias = dash.decode_step(inp["q"], inp["k"], inp["v"], kbar, block=block, alpha=1.5,
                                     gamma=1.5, sigma=1.0)
    torch.cuda.synchronize()
    qh, kh, vh = host(inp["q"]), host(inp["k"]), host(inp["v"])
    ref = orc.forward(qh, kh, vh, block=block, alpha=1.5, gamma=1.5, sigma=1.0, q_pos0=n_ctx - 1)
    rows = np.arange(w.batch)
    parity.check_forward(orc, qh, kh, vh, ref, mask=flat_rows(mask, rows), bias=flat_rows(bias, rows),
                         tau=None, o=flat_rows(o, rows), rows=rows, n_kv=n_ctx, block=block,
                         h_kv=w.h_kv, q_pos=np.full(w.batch, n_ctx - 1), q_pos0=n_ctx - 1,
                         alpha=1.5, sigma=1.0, dtype="bf16", vmax=float(inp["v"].abs().max()),
                         max_flip_frac=0.34)


@pytest.mark.parametrize("fused", [False, True])
def test_decode_tickets_reset_between_calls(dash, fused):
    """Decode attention hands the merge to the last workgroup of each (sequence, group) through
    ticket counters kept in its workspace: calls that reuse the same workspaces, with another
    batch size in between, give bit for bit the outputs of calls on fresh workspaces (the two
    separate calls, and the fused decode step)."""
    big = wl.Workload("decode tickets", 6, 4096 + 17, 32, 8, 128, 64, 1.5, 1.5, 1.0, decode=True,
                      plant="decode", plant_args=dict(lo=1, hi=8), seed=44)
    small = big.with_(batch=2, seed=45)
    if fused:
        ws = torch.zeros(dash.dash_decode_step_workspace_bytes(big.batch, big.n_kv, 32, 8, 128, 64),
                         dtype=torch.uint8, device=DEV)
        kw = lambda: dict(workspace=ws)
    else:
        rws = torch.zeros(dash.dash_block_entmax_workspace_bytes(
            torch.bfloat16, big.batch, 1, big.n_kv - 1, big.n_kv, 32, 8, 128, 64),
            dtype=torch.uint8, device=DEV)
        ws = torch.zeros(dash.dash_decode_workspace_bytes(big.batch, big.n_kv, 32, 8, 128, 64),
                         dtype=torch.uint8, device=DEV)
        kw = lambda: dict(route_ws=rws, attn_ws=ws)

    def run(w, reuse):
        inp = wl.make_inputs(w, DEV)
        kbar = dash.dash_pool_keys(inp["k"], w.block)
        o, mask, bias = dash.decode_step(inp["q"], inp["k"], inp["v"], kbar, block=w.block,
                                         alpha=w.alpha, gamma=w.gamma, sigma=w.sigma,
                                         fused=fused, **(kw() if reuse else {}))
        torch.cuda.synchronize()
        return o.clone(), mask.clone()

    fresh_big, fresh_small = run(big, False), run(small, False)
    for _ in range(2):
        for w, want in ((big, fresh_big), (small, fresh_small), (big, fresh_big)):
            got = run(w, True)
            assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1])
    # the ticket words at the start of the attention workspace are zero again after the calls
    assert not torch.any(ws[:4 * big.batch * 8]) and torch.any(ws[4 * big.batch * 8:])


def test_decode_step_matches_two_calls(dash):
    """dash_decode_step gives bit for bit the outputs of dash_block_entmax followed by
    dash_sparse_attn_decode."""
    w = wl.Workload("decode step", 5, 8192 + 33, 32, 8, 128, 64, 1.5, 1.5, 1.0, decode=True,
                    plant="decode", plant_args=dict(lo=1, hi=8), seed=46)
    inp = wl.make_inputs(w, DEV)
    kbar = dash.dash_pool_keys(inp["k"], w.block)
    a = dash.decode_step(inp["q"], inp["k"], inp["v"], kbar, block=w.block, alpha=w.alpha,
                         gamma=w.gamma, sigma=w.sigma, fused=True)
    b = dash.decode_step(inp["q"], inp["k"], inp["v"], kbar, block=w.block, alpha=w.alpha,
                         gamma=w.gamma, sigma=w.sigma, fused=False)
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1]), "masks differ"
    m = parity.bits(parity.to_host(a[1]), -(-w.n_kv // w.block))
    assert np.array_equal(parity.to_host(a[2])[m], parity.to_host(b[2])[m])
    assert torch.equal(a[0], b[0])


# ------------------------------------------------------------------------------ properties

def test_deterministic(dash):
    w = wl.Workload("det", 1, 2048, 8, 2, 128, 64, 1.5, 0.5, 1.0, plant="span",
                    plant_args=dict(span=8, per_span=2), seed=51)
    inp = wl.make_inputs(w, DEV)
    a = dash.forward(inp["q"], inp["k"], inp["v"], block=64, alpha=1.5, gamma=0.5, sigma=1.0)
    b = dash.forward(inp["q"], inp["k"], inp["v"], block=64, alpha=1.5, gamma=0.5, sigma=1.0)
    torch.cuda.synchronize()
    for key in ("kbar", "mask", "tau", "o", "lse"):
        assert torch.equal(a[key], b[key]), key


def test_errors_raise(dash):
    q = torch.zeros(1, 64, 4, 96, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(dash.DashError, match="head_dim"):
        dash.dash_pool_keys(q, 64)
    k = torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16, device=DEV)
    kb = dash.dash_pool_keys(k, 64)
    q = torch.zeros(1, 64, 4, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(dash.DashError, match="alpha"):
        dash.dash_block_entmax(q, kb, n_kv=64, block=64, alpha=2.5, gamma=1.0, sigma=1.0)
    with pytest.raises(dash.DashError, match="DASH_ERR_WORKSPACE"):
        # one query per sequence scores through the workspace; one byte is too small
        dash.dash_block_entmax(q[:, :1], kb, n_kv=64, block=64, alpha=1.5, gamma=1.0, sigma=1.0,
                               q_pos0=63, workspace=torch.empty(1, dtype=torch.uint8, device=DEV))
