"""GPU parity at the full workload sizes, in the launch configuration the benchmark times:
the whole GPU pass runs at full size and sampled rows are checked against the oracle, which
computes those rows one by one (Stage 0 in full, since every row depends on it)."""
from __future__ import annotations

import json
import os
import time

import numpy as np
import pytest
import torch

import workloads as wl
from tests import parity
from tests.test_gpu_parity import flat_rows, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def dash():
    import sparse_hierarchical_attention_amd as d
    d.lib()
    return d


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def prefill_parity(dash, orc, w: wl.Workload, sigma: float, rows: np.ndarray):
    log(f"{w.name}: generating inputs")
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    log("GPU forward")
    res = dash.forward(q, k, v, block=w.block, alpha=w.alpha, gamma=w.gamma, sigma=sigma)
    torch.cuda.synchronize()
    log(f"oracle on {len(rows)} rows")
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    ref = orc.forward(qh, kh, vh, block=w.block, alpha=w.alpha, gamma=w.gamma, sigma=sigma,
                      rows=rows)
    np.testing.assert_allclose(res["kbar"].cpu().numpy(), ref["kbar"], rtol=1e-6, atol=1e-6)
    rep = parity.check_forward(orc, qh, kh, vh, ref, mask=flat_rows(res["mask"], rows),
                               bias=flat_rows(res["bias"], rows), tau=flat_rows(res["tau"], rows),
                               o=flat_rows(res["o"], rows), lse=flat_rows(res["lse"], rows),
                               rows=rows, n_kv=w.n_kv, block=w.block, h_kv=w.h_kv,
                               q_pos=rows % w.n_q, alpha=w.alpha, sigma=sigma, dtype=w.dtype,
                               vmax=float(v.abs().max()))
    out = rep["e2e"]
    log(f"support {rep['support_frac']:.4f} flips {rep['flips']} own {rep['own']} e2e {out}")
    return rep, out


@pytest.mark.parametrize("sigma", [1e8, 1.0])
def test_prefill_32k(dash, orc, sigma):
    w = wl.PREFILL_32K
    prefill_parity(dash, orc, w, sigma, sample_rows(w.n_q, w.block, 160, seed=61))


def test_prefill_long_rows(dash, orc):
    """Rows of more than 512 chunks (the widest fused Stage 1 shape): 30017 tokens in chunks of
    32, so 938 complete chunks and a one-token tail chunk."""
    w = wl.PREFILL_32K.with_(n_kv=30017, block=32, name="prefill 30017 tokens, chunk 32")
    prefill_parity(dash, orc, w, 1.0, sample_rows(w.n_q, w.block, 64, seed=64))


def _sweep_points():
    with open(os.path.join(GOLDEN, "sweep_gamma.json")) as f:
        return [(p["alpha"], p["block"], p["gamma"]) for p in json.load(f)["points"]]


@pytest.mark.parametrize("alpha,block,gamma", _sweep_points())
def test_sweep_16k(dash, orc, alpha, block, gamma):
    w = wl.sweep_workload(alpha, block, gamma)
    rep, _ = prefill_parity(dash, orc, w, 1.0, sample_rows(w.n_q, w.block, 64, seed=62))


@pytest.mark.parametrize("n,hq,hkv,block", [(40000, 32, 8, 32), (36000, 32, 2, 32), (34000, 8, 8, 32),
                                           (34000, 16, 2, 32), (2048 * 32 + 17, 8, 2, 32)])
def test_prefill_rows_past_1024_chunks(dash, orc, n, hq, hkv, block):
    """bf16 prefill whose rows reach 1025 to 2048 chunks (the long-row route), groups of 1 to 16
    and a ragged tail whose 2049th chunk slot spills into a 65th mask word."""
    w = wl.Workload(f"prefill {n} tokens, {hq}q/{hkv}kv heads, D 128, block {block}", 1, n, hq, hkv,
                    128, block, 1.5, 0.5, 1.0, plant="span", plant_args=dict(span=16, per_span=4),
                    seed=67)
    prefill_parity(dash, orc, w, w.sigma, sample_rows(w.n_q, w.block, 40, seed=68))


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.25])
def test_prefill_long_rows_packed_candidates(dash, orc, alpha):
    """Rows of 1025 to 2048 chunks whose support is small (2 planted of every 16 chunks): the
    long-row route solves the threshold on the entries above the bound from the lanes' maxima
    (at most 256 of them) instead of the whole row; sampled rows against the oracle for the three
    kinds of exponent."""
    w = wl.Workload(f"prefill 40000 tokens, chunk 32, 2 planted of every 16 chunks, alpha {alpha}",
                    1, 40000, 32, 8, 128, 32, alpha, 0.5, 1.0, plant="span",
                    plant_args=dict(span=16, per_span=2), seed=71)
    prefill_parity(dash, orc, w, w.sigma, sample_rows(w.n_q, w.block, 40, seed=72))


def test_prefill_bf16_rows_past_2048_chunks(dash, orc):
    """bf16 prefill whose rows reach 2049 to 8192 chunks: 160K tokens in chunks of 64 (2560
    complete chunks) leave the fused Stage 1 for the score workspace, routed in slabs of query
    rows; sampled rows against the oracle."""
    w = wl.Workload("prefill 160K, 32q/8kv heads, D 128, block 64, 4 planted of every 16 chunks",
                    1, 163840, 32, 8, 128, 64, 1.5, 0.5, 1e8, plant="span",
                    plant_args=dict(span=16, per_span=4), seed=69)
    need = dash.dash_block_entmax_workspace_bytes(torch.bfloat16, 1, w.n_q, 0, w.n_kv, 32, 8, 128, 64)
    row_bytes = 32 * (w.n_kv // 64) * 4
    assert need == (512 << 20) // row_bytes * row_bytes  # slabs of whole score rows
    prefill_parity(dash, orc, w, w.sigma, sample_rows(w.n_q, w.block, 32, seed=70))


def test_prefill_slabs_across_sequences(dash, orc):
    """Two fp32 sequences of 16K whose score rows (2 GiB) exceed the workspace: Stage 1 runs in
    four slabs of query rows, two per sequence; sampled rows of both against the oracle."""
    w = wl.Workload("prefill fp32 2 x 16K, 32q/8kv heads, D 128, block 32", 2, 16384, 32, 8, 128, 32,
                    1.5, 0.5, 1.0, dtype="f32", plant="span", plant_args=dict(span=16, per_span=4),
                    seed=65)
    assert dash.dash_block_entmax_workspace_bytes(torch.float32, 2, w.n_q, 0, w.n_kv, 32, 8, 128, 32) == 512 << 20
    rows = sample_rows(w.n_q, w.block, 24, seed=66, batch=2)
    rows = np.union1d(rows, [8191, 8192, 16383, 16384, 16385, 24575, 24576])  # slab edges
    prefill_parity(dash, orc, w, w.sigma, rows)


def test_prefill_256k(dash, orc):
    w = wl.PREFILL_256K
    prefill_parity(dash, orc, w, w.sigma, sample_rows(w.n_q, w.block, 48, seed=63))


@pytest.mark.parametrize("sigma", [1e8, 1.0])
def test_decode_128k(dash, orc, sigma):
    w = wl.DECODE_128K
    log(f"{w.name}: generating inputs")
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    kbar = dash.dash_pool_keys(k, w.block)
    o, mask, bias = dash.decode_step(q, k, v, kbar, block=w.block, alpha=w.alpha, gamma=w.gamma,
                                     sigma=sigma)
    torch.cuda.synchronize()
    for b in (0, 7, 15):  # the oracle regenerates nothing: it reads these sequences' inputs
        log(f"oracle on sequence {b}")
        qh, kh, vh = q[b:b + 1].cpu(), k[b:b + 1].cpu(), v[b:b + 1].cpu()
        ref = orc.forward(qh, kh, vh, block=w.block, alpha=w.alpha, gamma=w.gamma, sigma=sigma,
                          q_pos0=w.n_kv - 1)
        np.testing.assert_allclose(kbar[b:b + 1].cpu().numpy(), ref["kbar"], rtol=1e-6, atol=1e-6)
        parity.check_forward(orc, qh, kh, vh, ref, mask=parity.to_host(mask[b]),
                             bias=parity.to_host(bias[b]), tau=None, o=parity.to_host(o[b]),
                             rows=np.array([0]), n_kv=w.n_kv, block=w.block, h_kv=w.h_kv,
                             q_pos=np.array([w.n_kv - 1]), q_pos0=w.n_kv - 1, alpha=w.alpha,
                             sigma=sigma, dtype="bf16", vmax=float(v[b].abs().max()),
                             max_flip_frac=1.0)
        # the planted chunks are what the router finds
        routed = parity.bits(ref["mask"], -(-w.n_kv // w.block))[0]
        for r in range(w.h_kv):
            sel = set(np.flatnonzero(routed[r][:-1]).tolist())
            assert set(inp["planted"][b][r].tolist()) <= sel


# ------------------------------------------- the pages' efficiency sweep: injected random selection

def test_table5_prefill_16k_random_selection(dash, orc):
    """Stage 2 at the sweep's 16K prefill shape (32 query heads over 2 KV heads) on a random
    selection at sparsity 75 %, sampled rows against the oracle."""
    w = wl.table5_workload(16384, decode=False)
    log(f"{w.name}: generating inputs")
    inp = wl.make_inputs(w, DEV)
    mask, bias = wl.random_selection(1, w.n_q, 0, w.n_kv, w.h_kv, w.block, 0.75, seed=11,
                                     device=DEV, bias_std=0.5)
    o, lse = dash.dash_sparse_attn_prefill(inp["q"], inp["k"], inp["v"], mask, bias, block=w.block)
    torch.cuda.synchronize()
    rows = sample_rows(w.n_q, w.block, 96, seed=71)
    log(f"oracle on {len(rows)} rows")
    m = flat_rows(mask, rows).view(np.uint32)
    ref_o, ref_lse = orc.sparse_attn(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), m,
                                     flat_rows(bias, rows).astype(np.float64), block=w.block,
                                     rows=rows)
    out = parity.compare_output(flat_rows(o, rows), ref_o, "bf16", gpu_lse=flat_rows(lse, rows),
                                ref_lse=ref_lse)
    log(f"out {out}")


def test_table5_decode_96k_random_selection(dash, orc):
    """Decode at the sweep's largest shape, 24 sequences of 96K context with groups of 16, on a
    random selection at sparsity 93.75 %, every sequence against the oracle."""
    w = wl.table5_workload(98304, decode=True)
    log(f"{w.name}: generating inputs")
    inp = wl.make_inputs(w, DEV)
    mask, bias = wl.random_selection(w.batch, 1, w.n_kv - 1, w.n_kv, w.h_kv, w.block, 0.9375,
                                     seed=12, device=DEV, bias_std=0.5)
    o = dash.dash_sparse_attn_decode(inp["q"], inp["k"], inp["v"], mask, bias, block=w.block)
    torch.cuda.synchronize()
    log("oracle")
    m = parity.to_host(mask).view(np.uint32).reshape(w.batch, w.h_kv, -1)
    bi = parity.to_host(bias).astype(np.float64).reshape(w.batch, w.h_kv, -1)
    ref_o, _ = orc.sparse_attn(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), m, bi,
                               block=w.block, q_pos0=w.n_kv - 1)
    out = parity.compare_output(parity.to_host(o).reshape(w.batch, w.h_q, -1), ref_o, "bf16")
    log(f"out {out}")


# ------------------------------------------------------------------ the documented chunk limit

def test_decode_at_the_chunk_limit(dash, orc):
    """Decode with 8192 chunk slots, the most the ABI accepts: 2 sequences of 262144 tokens in
    chunks of 32 (the full length, and a length that ends one token into the last chunk)."""
    w = wl.Workload("decode 2 x 256K, chunk 32 (8192 chunks)", 2, 8192 * 32, 32, 8, 128, 32, 1.5,
                    1.5, 1.0, decode=True, plant="decode", plant_args=dict(lo=1, hi=16), seed=72)
    log(f"{w.name}: generating inputs")
    inp = wl.make_inputs(w, DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    kbar = dash.dash_pool_keys(k, w.block)
    lens = [w.n_kv, 8191 * 32 + 1]
    ctx = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, mask, bias = dash.dash_decode_step(q, k, v, kbar, block=w.block, alpha=w.alpha,
                                          gamma=w.gamma, sigma=w.sigma, ctx_lens=ctx)
    torch.cuda.synchronize()
    for b, n_b in enumerate(lens):
        log(f"oracle on sequence {b} ({n_b} tokens)")
        qh, kh, vh = q[b:b + 1].cpu(), k[b:b + 1, :n_b].cpu(), v[b:b + 1, :n_b].cpu()
        ref = orc.forward(qh, kh, vh, block=w.block, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma,
                          q_pos0=n_b - 1)
        nc_b = -(-n_b // w.block)
        m = parity.to_host(mask[b]).view(np.uint32)[..., :-(-nc_b // 32)].copy()
        words = -(-nc_b // 32)
        if nc_b % 32:
            m[..., words - 1] &= np.uint32((1 << (nc_b % 32)) - 1)
        parity.check_forward(orc, qh, kh, vh, ref, mask=m, bias=parity.to_host(bias[b])[..., :nc_b],
                             tau=None, o=parity.to_host(o[b]), rows=np.array([0]), n_kv=n_b,
                             block=w.block, h_kv=w.h_kv, q_pos=np.array([n_b - 1]),
                             q_pos0=n_b - 1, alpha=w.alpha, sigma=w.sigma, dtype="bf16",
                             vmax=float(v[b].abs().max()), max_flip_frac=1.0)


def test_prefill_at_the_chunk_limit(dash, orc):
    """bf16 prefill with 8192 chunk slots: 262144 tokens in chunks of 32, 32 query heads over 2 KV
    heads (routed in slabs of query rows through the score workspace); sampled rows, the last ones
    included, against the oracle."""
    w = wl.Workload("prefill 256K, chunk 32 (8192 chunks), 32q/2kv heads, D 128", 1, 8192 * 32, 32, 2,
                    128, 32, 1.5, 0.5, 1e8, plant="span", plant_args=dict(span=16, per_span=4),
                    seed=73)
    rows = np.union1d(sample_rows(w.n_q, w.block, 10, seed=74), [w.n_q - 33, w.n_q - 1])
    prefill_parity(dash, orc, w, w.sigma, rows)
