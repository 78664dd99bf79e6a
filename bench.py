"""Benchmark of the DashAttention forward pass (libdash) on one MI355X.

One step = the whole hot path once: the 32K prefill forward (pool keys, route with alpha-entmax,
sparse attention) on the 32K workload, plus one decode step (route against the cached chunk
summaries, split sparse attention) on the 16 x 128K workload. Inputs are seeded synthetic
tensors already resident in HBM; the decode cache's summaries are pooled once before timing, as a
decode loop would keep them.

Prints one JSON line. `value` is the prefill's effective TFLOP/s: the FLOPs the method must do on
the selected (query head, key) pairs, 4 * D per pair, over the time of its three stages. The
decode rate and the per-kernel rooflines are reported beside it.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "prefill eff. TFLOP/s @32K + decode tok/s @128K; % of MFMA / HBM roofline"
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def popcount32(a: np.ndarray) -> np.ndarray:
    a = a.astype(np.uint32)
    a = a - ((a >> 1) & 0x55555555)
    a = (a & 0x33333333) + ((a >> 2) & 0x33333333)
    a = (a + (a >> 4)) & 0x0F0F0F0F
    return ((a * 0x01010101) & 0xFFFFFFFF) >> 24


def selected_pairs_prefill(mask: torch.Tensor, w: wl.Workload) -> tuple[int, float]:
    """Number of selected (query head, key) pairs of a prefill and the routed fraction of the
    candidate chunks. Routed chunks hold `block` keys each; the query's own chunk contributes its
    causal prefix. Every head of a group shares the group's selection."""
    m = mask.cpu().numpy().view(np.uint32)                  # [B, n, Hkv, W]
    g = w.h_q // w.h_kv
    pos = np.arange(w.n_q)
    cp = pos // w.block
    bits = popcount32(m).sum(axis=-1).astype(np.int64)      # routed + diagonal, per (b, t, r)
    routed = bits - 1
    pairs = (routed * w.block).sum() * g + w.batch * w.h_q * (pos - cp * w.block + 1).sum()
    cand = w.batch * w.h_kv * np.minimum(cp, w.n_kv // w.block).sum()
    return int(pairs), float(routed.sum() / max(1, cand))


def issued_pairs_prefill(mask: torch.Tensor, w: wl.Workload, rows_per_wg: int = 128,
                         rows_per_wave: int = 32, tile_keys: int = 32) -> int:
    """(query head, key) pairs the bf16 D = 128 prefill kernel multiplies on its matrix cores for
    this mask: a workgroup of rows_per_wg rows (tokens x the group's heads) walks the union of its
    tokens' chunks (their own chunks included) in tiles of tile_keys keys, and a wave of
    rows_per_wave rows multiplies a tile unless none of its tokens selected the chunk; each
    multiplied tile costs rows_per_wave x tile_keys pairs (masked causal keys and rows that did not
    select the chunk included)."""
    m = mask.cpu().numpy().view(np.uint32)                  # [B, n, Hkv, W]
    g = w.h_q // w.h_kv
    nc = -(-w.n_kv // w.block)
    cw = np.arange(nc)
    bits = ((m[..., cw // 32] >> (cw % 32).astype(np.uint32)) & 1).astype(bool)  # [B, n, Hkv, Nc]
    pos = np.arange(w.n_q)
    cp = pos // w.block
    bits &= cw[None, None, None, :] <= cp[None, :, None, None]
    bits[:, pos, :, cp] = True                              # the own chunk
    tw = rows_per_wave // g                                 # tokens per wave
    n_pad = -(-w.n_q // tw) * tw
    if n_pad != w.n_q:
        bits = np.concatenate([bits, np.zeros((bits.shape[0], n_pad - w.n_q) + bits.shape[2:], bool)], 1)
    wave_sel = bits.reshape(bits.shape[0], n_pad // tw, tw, w.h_kv, nc).any(axis=2)
    sub = max(1, w.block // tile_keys)
    return int(wave_sel.sum()) * sub * rows_per_wave * min(tile_keys, w.block)


def decode_bytes(mask: torch.Tensor, w: wl.Workload) -> tuple[int, float]:
    """Algorithmic HBM bytes of one decode step: the cached summaries of the complete chunks
    before the new token's chunk (fp32), the selected K and V chunks including the new token's
    own chunk, and q / o. Also the mean number of routed chunks per (sequence, group)."""
    m = mask.cpu().numpy().view(np.uint32)                  # [B, 1, Hkv, W]
    bits = popcount32(m).sum(axis=-1).astype(np.int64)
    pos = w.n_kv - 1
    cp = pos // w.block
    kbar_bytes = w.batch * min(cp, w.n_kv // w.block) * w.h_kv * w.head_dim * 4
    routed = (bits - 1).sum()
    diag_tokens = pos - cp * w.block + 1
    kv_bytes = (routed * w.block + w.batch * w.h_kv * diag_tokens) * w.head_dim * 2 * 2
    qo_bytes = 2 * w.batch * w.h_q * w.head_dim * 2
    return int(kbar_bytes + kv_bytes + qo_bytes), float(routed / (w.batch * w.h_kv))


def decode_bytes_varlen(mask: torch.Tensor, lens: np.ndarray, w: wl.Workload) -> int:
    """decode_bytes for one new token per sequence at position lens[b] - 1 of a cache of capacity
    w.n_kv: the summaries of the complete chunks before each token's chunk, the routed K and V
    chunks, the token's own chunk up to it, and q / o."""
    m = mask.cpu().numpy().view(np.uint32)                  # [B, 1, Hkv, W]
    bits = popcount32(m).sum(axis=-1).astype(np.int64)[:, 0]  # [B, Hkv] routed + own
    pos = lens.astype(np.int64) - 1
    cp = pos // w.block
    kbar_bytes = int((np.minimum(cp, w.n_kv // w.block) * w.h_kv * w.head_dim * 4).sum())
    routed = int((bits - 1).sum())
    diag = int(((pos - cp * w.block + 1) * w.h_kv).sum())
    kv_bytes = (routed * w.block + diag) * w.head_dim * 2 * 2
    qo_bytes = 2 * w.batch * w.h_q * w.head_dim * 2
    return kbar_bytes + kv_bytes + qo_bytes


def decode_graph(step):
    """step() captured once in a HIP graph (after a warm run on a side stream of default priority);
    every buffer it touches is allocated beforehand."""
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


def extras_leg(dash, pre, dec, wp: wl.Workload, wd: wl.Workload, reps: int) -> dict:
    """The learned summary query (Stage 0 as the local attention of a learned q per KV head) over
    the 32K prefill keys and the 16 x 128K decode cache, and the streaming paths: a decode step
    with per-sequence lengths (seeded, ragged over the cache's second half) and the 32K prefill
    with a window of two blocks. Each timed with HIP events over `reps` calls after one warm call."""
    dev = pre["q"].device
    out = {}
    k, kd = pre["k"], dec["k"]
    qbar = wl.summary_query(wp.h_kv, wp.head_dim, 91, dev)
    pool = {}
    for name, kk, blk, per_chunk in (("prefill_32k", k, wp.block, False),
                                     ("prefill_32k_per_chunk_query", k, wp.block, True),
                                     ("decode_cache_16x128k", kd, wd.block, False)):
        kb = torch.empty((kk.shape[0], kk.shape[1] // blk, kk.shape[2], kk.shape[3]),
                         dtype=torch.float32, device=dev)
        qb = qbar
        if per_chunk:  # one query per chunk and KV head, as Alg. 1 takes it
            qb = (torch.randn((kk.shape[1] // blk,) + tuple(qbar.shape),
                              generator=torch.Generator().manual_seed(93)) * 0.3).to(dev)
        t = _time_ms(lambda: dash.dash_pool_keys_query(kk, qb, blk, kbar=kb), reps)
        nbytes = kk.numel() * kk.element_size() + kb.numel() * 4 + (qb.numel() * 4 if per_chunk else 0)
        gbs = nbytes / (t * 1e-3) / 1e9
        pool[name] = {"ms": round(t, 4), "algorithmic_bytes": nbytes, "gb_per_s": round(gbs, 1),
                      "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBPS,
                                   "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBPS, 4)}}
    out["learned_summary_query"] = pool

    # decode with a length per sequence: append the newest token's completed chunk (if any),
    # route with the lengths, split attention with the lengths
    qd, vd = dec["q"], dec["v"]
    lens = wl.ragged_lengths(wd.batch, wd.n_kv, 92, dev)
    kbar_d = dash.dash_pool_keys(kd, wd.block)
    ncd = -(-wd.n_kv // wd.block)
    mask_d = torch.empty((wd.batch, 1, wd.h_kv, -(-ncd // 32)), dtype=torch.int32, device=dev)
    bias_d = torch.empty((wd.batch, 1, wd.h_kv, ncd), dtype=torch.float32, device=dev)
    o_d = torch.empty_like(qd)
    wsb = dash.dash_block_entmax_workspace_bytes(qd.dtype, wd.batch, 1, wd.n_kv - 1, wd.n_kv,
                                                 wd.h_q, wd.h_kv, wd.head_dim, wd.block)
    rws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)
    awb = dash.dash_decode_workspace_bytes(wd.batch, wd.n_kv, wd.h_q, wd.h_kv, wd.head_dim, wd.block)
    aws = torch.zeros(awb, dtype=torch.uint8, device=dev) if awb else None

    sws = torch.zeros(dash.dash_decode_step_workspace_bytes(wd.batch, wd.n_kv, wd.h_q, wd.h_kv,
                                                            wd.head_dim, wd.block),
                      dtype=torch.uint8, device=dev)

    def varlen_step():
        dash.dash_pool_keys_append(kd, lens, kbar_d, wd.block)
        dash.dash_decode_step(qd, kd, vd, kbar_d, block=wd.block, alpha=wd.alpha, gamma=wd.gamma,
                              sigma=wd.sigma, ctx_lens=lens, mask=mask_d, bias=bias_d, o=o_d,
                              workspace=sws)

    def varlen_two_calls():
        dash.dash_pool_keys_append(kd, lens, kbar_d, wd.block)
        dash.dash_block_entmax_ex(qd, kbar_d, n_kv=wd.n_kv, block=wd.block, alpha=wd.alpha,
                                  gamma=wd.gamma, sigma=wd.sigma, h_kv=wd.h_kv, ctx_lens=lens,
                                  mask=mask_d, bias=bias_d, want_tau=False, workspace=rws)
        dash.dash_sparse_attn_decode_varlen(qd, kd, vd, lens, mask_d, bias_d, block=wd.block,
                                            o=o_d, workspace=aws)

    t_two = _time_ms(decode_graph(varlen_two_calls).replay, reps)
    t_eager = _time_ms(varlen_step, reps)
    # the step's three calls cost more host time than the GPU spends on them, so it is also
    # captured once in a HIP graph and replayed (no allocation or memset inside the step)
    t = _time_ms(decode_graph(varlen_step).replay, reps)
    nbytes = decode_bytes_varlen(mask_d, lens.cpu().numpy(), wd)
    gbs = nbytes / (t * 1e-3) / 1e9
    out["varlen_decode"] = {
        "lengths": "uniform over [64K, 128K] per sequence", "us_per_step": round(t * 1e3, 2),
        "us_per_step_eager": round(t_eager * 1e3, 2),
        "us_per_step_two_calls": round(t_two * 1e3, 2), "tok_per_s": round(wd.batch / (t * 1e-3), 1),
        "algorithmic_bytes": nbytes, "gb_per_s": round(gbs, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBPS, 4)}}

    # prefill with a window of two blocks (the own block and the one before it always attended)
    q, v = pre["q"], pre["v"]
    kbar = dash.dash_pool_keys(k, wp.block)
    nc = -(-wp.n_kv // wp.block)
    mask = torch.empty((1, wp.n_q, wp.h_kv, -(-nc // 32)), dtype=torch.int32, device=dev)
    bias = torch.empty((1, wp.n_q, wp.h_kv, nc), dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((1, wp.n_q, wp.h_q), dtype=torch.float32, device=dev)
    wsb = dash.dash_block_entmax_workspace_bytes(q.dtype, 1, wp.n_q, 0, wp.n_kv, wp.h_q, wp.h_kv,
                                                 wp.head_dim, wp.block)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    t_pool = _time_ms(lambda: dash.dash_pool_keys(k, wp.block, kbar=kbar), reps)
    t_route = _time_ms(lambda: dash.dash_block_entmax_ex(
        q, kbar, n_kv=wp.n_kv, block=wp.block, alpha=wp.alpha, gamma=wp.gamma, sigma=wp.sigma,
        h_kv=wp.h_kv, window_blocks=2, mask=mask, bias=bias, want_tau=False, workspace=ws), reps)
    t_attn = _time_ms(lambda: dash.dash_sparse_attn_prefill(q, k, v, mask, bias, block=wp.block,
                                                            o=o, lse=lse), reps)
    pairs, frac = selected_pairs_prefill(mask, wp)
    flops = 4.0 * wp.head_dim * pairs
    at = flops / (t_attn * 1e-3) / 1e12
    out["window2_prefill"] = {
        "ms": {"pool": round(t_pool, 4), "entmax": round(t_route, 4), "attn": round(t_attn, 4)},
        "selected_pairs": pairs, "selected_fraction_of_candidates": round(frac, 4),
        "end_to_end_tflops": round(flops / ((t_pool + t_route + t_attn) * 1e-3) / 1e12, 3),
        "roofline": {"bound": "mfma", "achieved": round(at, 3), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(at / MFMA_BF16_PEAK_TFLOPS, 4)}}
    return out


def config_point(dash, w: wl.Workload, dev, reps: int, oracle_rows: int) -> dict:
    """One prefill workload through the three stages (pool, route, attend), each timed as the
    median of `reps` HIP-event spans, with its selected-pair work, roofline, and the oracle timed
    on `oracle_rows` sampled query rows of the same inputs (its TFLOP/s on those rows' pairs)."""
    import oracle
    inp = wl.make_inputs(w, dev)
    q, k, v = inp["q"], inp["k"], inp["v"]
    nc = -(-w.n_kv // w.block)
    kbar = torch.empty((w.batch, w.n_kv // w.block, w.h_kv, w.head_dim), dtype=torch.float32,
                       device=dev)
    mask = torch.empty((w.batch, w.n_q, w.h_kv, -(-nc // 32)), dtype=torch.int32, device=dev)
    bias = torch.empty((w.batch, w.n_q, w.h_kv, nc), dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.batch, w.n_q, w.h_q), dtype=torch.float32, device=dev)
    wsb = dash.dash_block_entmax_workspace_bytes(q.dtype, w.batch, w.n_q, 0, w.n_kv, w.h_q, w.h_kv,
                                                 w.head_dim, w.block)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)
    t = Timer()
    for i in range(reps + 1):
        spans = [t.span(n) if i else (None, None) for n in ("pool", "entmax", "attn")]
        spans[0][0] and spans[0][0].record()
        dash.dash_pool_keys(k, w.block, kbar=kbar)
        spans[0][1] and spans[0][1].record()
        spans[1][0] and spans[1][0].record()
        dash.dash_block_entmax(q, kbar, n_kv=w.n_kv, block=w.block, alpha=w.alpha, gamma=w.gamma,
                               sigma=w.sigma, mask=mask, bias=bias, want_tau=False, workspace=ws)
        spans[1][1] and spans[1][1].record()
        spans[2][0] and spans[2][0].record()
        dash.dash_sparse_attn_prefill(q, k, v, mask, bias, block=w.block, o=o, lse=lse)
        spans[2][1] and spans[2][1].record()
    torch.cuda.synchronize()
    ms = {n: t.median_ms(n) for n in ("pool", "entmax", "attn")}
    pairs, frac = selected_pairs_prefill(mask, w)
    flops = 4.0 * w.head_dim * pairs
    at = flops / (ms["attn"] * 1e-3) / 1e12
    fp32 = w.dtype == "f32"
    peak = 157.3 if fp32 else MFMA_BF16_PEAK_TFLOPS  # fp32 runs on the vector ALUs
    # the oracle on sampled rows (the chunk edges and the last rows, then spread), Stage 0 in full
    rng = np.random.default_rng(w.seed)
    rows = np.unique(np.concatenate([np.arange(w.n_q - 4, w.n_q),
                                     rng.choice(w.n_q, size=max(0, oracle_rows - 4), replace=False)]))
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    t0 = time.perf_counter()
    ref = oracle.forward(qh, kh, vh, block=w.block, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma,
                         rows=rows)
    t_orc = time.perf_counter() - t0
    pos = rows % w.n_q
    cp = pos // w.block
    routed = popcount32(ref["mask"]).sum(axis=-1).astype(np.int64) - 1
    orc_pairs = (routed * w.block).sum() * (w.h_q // w.h_kv) + w.h_q * (pos - cp * w.block + 1).sum()
    del inp, q, k, v, kbar, mask, bias, o, lse, ws, qh, kh, vh, ref
    torch.cuda.empty_cache()
    return {
        "workload": w.name, "alpha": w.alpha, "block": w.block, "gamma": w.gamma,
        "dtype": w.dtype, "ms": {n: round(x, 4) for n, x in ms.items()},
        "selected_pairs": pairs, "routed_fraction": round(frac, 4),
        "algorithmic_tflop": round(flops / 1e12, 4),
        "attn_tflops": round(at, 3),
        "end_to_end_tflops": round(flops / (sum(ms.values()) * 1e-3) / 1e12, 3),
        "roofline": {"bound": "alu" if fp32 else "mfma", "achieved": round(at, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(at / peak, 4)},
        "cpu_baseline": {"kind": "oracle", "cores": oracle.num_threads(), "rows": int(len(rows)),
                         "seconds": round(t_orc, 3),
                         "tflops": round(4.0 * w.head_dim * orc_pairs / t_orc / 1e12, 6)},
    }


def configs_leg(dash, dev, reps: int) -> dict:
    """The other workloads of the measurement plan, each timed on its own: the tiny fp32
    workload, the nine alpha / block points of the sweep at 16K and the 256K prefill."""
    out = {}
    print("[bench] configs: tiny fp32", file=sys.stderr, flush=True)
    out["tiny_fp32"] = config_point(dash, wl.TINY, dev, reps, oracle_rows=1024)
    with open(os.path.join(ROOT, "tests", "golden", "sweep_gamma.json")) as f:
        points = json.load(f)["points"]
    sweep = []
    for pt in points:
        w = wl.sweep_workload(pt["alpha"], pt["block"], pt["gamma"])
        print(f"[bench] configs: {w.name}", file=sys.stderr, flush=True)
        sweep.append(config_point(dash, w, dev, reps, oracle_rows=32))
    out["sweep_16k"] = sweep
    print("[bench] configs: prefill 256K", file=sys.stderr, flush=True)
    out["prefill_256k"] = config_point(dash, wl.PREFILL_256K, dev, max(2, reps // 4), oracle_rows=16)
    return out


# Sources each measured launch is built from: a counter summary taken on other sources is stale.
KERNEL_SOURCES = {
    "sparse_attn_prefill": ["common.h", "kernels.h", "sparse_attn_dma.hip"],
    "decode_step": ["common.h", "kernels.h", "entmax.h", "route_common.h", "block_entmax.hip",
                    "decode_common.h", "decode.hip"],
    "sparse_attn_backward": ["common.h", "kernels.h", "sparse_attn_bwd_mfma.hip"],
}


def source_hash(kernel: str) -> str:
    """Hash of the code (comments and whitespace dropped) of the sources a kernel is built from."""
    csrc = os.path.join(ROOT, "sparse_hierarchical_attention_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(f.encode() + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy) from the
    committed counter summary, if it was taken on the current sources of that kernel; else None."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel)
    if not ent or ent.get("source_sha") != source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


class Timer:
    """HIP events on the stream the library launches on (torch's current stream)."""

    def __init__(self):
        self.spans = {}

    def span(self, name):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        self.spans.setdefault(name, []).append((s, e))
        return s, e

    def median_ms(self, name):
        return float(np.median([s.elapsed_time(e) for s, e in self.spans[name]]))


def cpu_baseline(pre_inp, dec_inp, wp: wl.Workload, wd: wl.Workload, pre_pairs_per_row: float):
    """The oracle, as it stands, on a bounded sample of the same workloads, on this host."""
    import oracle
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(np.arange(wp.n_q // 2, wp.n_q), size=384, replace=False))
    qh, kh, vh = pre_inp["q"].cpu(), pre_inp["k"].cpu(), pre_inp["v"].cpu()
    t0 = time.perf_counter()
    ref = oracle.forward(qh, kh, vh, block=wp.block, alpha=wp.alpha, gamma=wp.gamma,
                         sigma=wp.sigma, rows=rows)
    t_pre = time.perf_counter() - t0
    nc = -(-wp.n_kv // wp.block)
    m = ref["mask"]
    pos = rows % wp.n_q
    cp = pos // wp.block
    routed = popcount32(m).sum(axis=-1).astype(np.int64) - 1
    pairs = (routed * wp.block).sum() * (wp.h_q // wp.h_kv) + wp.h_q * (pos - cp * wp.block + 1).sum()
    tflops = 4.0 * wp.head_dim * pairs / t_pre / 1e12
    # decode: two sequences, summaries pooled by the oracle beforehand (a decode loop's cache)
    seqs = [0, 1]
    tok_s = []
    for b in seqs:
        qb, kb_, vb = dec_inp["q"][b:b + 1].cpu(), dec_inp["k"][b:b + 1].cpu(), dec_inp["v"][b:b + 1].cpu()
        kbar = oracle.pool_keys(kb_, wd.block)
        t0 = time.perf_counter()
        st = oracle.block_entmax(qb, kbar, n_kv=wd.n_kv, block=wd.block, alpha=wd.alpha,
                                 gamma=wd.gamma, sigma=wd.sigma, q_pos0=wd.n_kv - 1, h_kv=wd.h_kv)
        oracle.sparse_attn(qb, kb_, vb, st["mask"], st["bias"], block=wd.block, q_pos0=wd.n_kv - 1)
        tok_s.append(1.0 / (time.perf_counter() - t0))
    del nc, ref
    return {"value": round(tflops, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"prefill: {len(rows)} query rows of the 32K workload (Stage 0 in full, "
                      f"all heads), {t_pre:.1f} s; decode: sequences {seqs} of the 16 x 128K "
                      f"workload with summaries pooled beforehand",
            "decode_tok_per_s": round(float(np.mean(tok_s)), 3)}


def _time_ms(fn, reps: int, warm: int = 1) -> float:
    """Mean HIP-event time of fn() on torch's current stream (the stream the library launches on)."""
    for _ in range(warm):
        fn()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def _sdpa_ms(q, k, v, causal: bool, reps: int):
    """torch's fused scaled-dot-product attention (flash or memory-efficient kernel only, never
    the math path) on [B, H, n, D] views, or None where the installed torch offers neither for the
    shape."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    import torch.nn.functional as F
    qt, kt, vt = (x.transpose(1, 2) for x in (q, k, v))
    for backend in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
        try:
            with sdpa_kernel([backend]):
                return _time_ms(lambda: F.scaled_dot_product_attention(
                    qt, kt, vt, is_causal=causal, enable_gqa=True), reps), backend.name
        except RuntimeError:
            continue
    return None, None


def random_mask_sweep(dash, dev, reps: int):
    """The pages' efficiency sweep: Hq 32, Hkv 2, D 128, chunk 64, N in {16, 32, 64, 96}K, chunk
    sparsity s in {75, 87.5, 93.75} %, prefill at batch 1 and decode at batch 24, with Stage 2
    given a random selection at sparsity s in place of the router's (Stages 0 and 1 still run
    in full, their cost does not depend on s). Prints one JSON line per (mode, N) with each
    stage's time, the speedup over dense causal attention through the same Stage 2 kernel (every
    chunk selected) and over torch's fused attention kernel, where the installed torch has one."""
    rows = []
    for n in wl.TABLE5_CONTEXTS:
        for decode in (False, True):
            w = wl.table5_workload(n, decode)
            print(f"[bench] sweep: {w.name}", file=sys.stderr, flush=True)
            inp = wl.make_inputs(w, dev)
            q, k, v = inp["q"], inp["k"], inp["v"]
            nc = -(-n // w.block)
            nw = -(-nc // 32)
            kbar = dash.dash_pool_keys(k, w.block)
            mask = torch.empty((w.batch, w.n_q, w.h_kv, nw), dtype=torch.int32, device=dev)
            bias = torch.empty((w.batch, w.n_q, w.h_kv, nc), dtype=torch.float32, device=dev)
            wsb = dash.dash_block_entmax_workspace_bytes(q.dtype, w.batch, w.n_q, w.q_pos0, n,
                                                         w.h_q, w.h_kv, w.head_dim, w.block)
            ws = torch.zeros(wsb, dtype=torch.uint8, device=dev) if wsb else None
            o = torch.empty_like(q)
            lse = torch.empty((w.batch, w.n_q, w.h_q), dtype=torch.float32, device=dev)
            t_pool = 0.0 if decode else _time_ms(lambda: dash.dash_pool_keys(k, w.block, kbar=kbar), reps)
            t_route = _time_ms(lambda: dash.dash_block_entmax(
                q, kbar, n_kv=n, block=w.block, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma,
                q_pos0=w.q_pos0, mask=mask, bias=bias, want_tau=False, workspace=ws), reps)
            del ws
            if decode:
                awb = dash.dash_decode_workspace_bytes(w.batch, n, w.h_q, w.h_kv, w.head_dim, w.block)
                aws = torch.zeros(awb, dtype=torch.uint8, device=dev) if awb else None

                def stage2(m, bi):
                    dash.dash_sparse_attn_decode(q, k, v, m, bi, block=w.block, o=o, workspace=aws)
            else:
                def stage2(m, bi):
                    dash.dash_sparse_attn_prefill(q, k, v, m, bi, block=w.block, o=o, lse=lse)
            point = {"mode": "decode" if decode else "prefill", "n": n, "batch": w.batch,
                     "ms": {"pool": round(t_pool, 4), "route": round(t_route, 4)}, "sparsity": {}}
            for s in (0.0,) + wl.TABLE5_SPARSITY:
                m, bi = wl.random_selection(w.batch, w.n_q, w.q_pos0, n, w.h_kv, w.block, s,
                                            seed=1000 + int(s * 1e4), device=dev)
                t = _time_ms(lambda: stage2(m, bi), reps)
                ent = {"stage2_ms": round(t, 4)}
                if not decode:
                    pairs, frac = selected_pairs_prefill(m, w)
                    ent["selected_fraction"] = round(frac, 4)
                    ent["stage2_tflops"] = round(4.0 * w.head_dim * pairs / (t * 1e-3) / 1e12, 2)
                point["sparsity"][str(s)] = ent
                del m, bi
            t_dense = point["sparsity"]["0.0"]["stage2_ms"]
            t_sdpa, backend = _sdpa_ms(q, k, v, causal=not decode, reps=reps)
            point["dense_ms"] = {"same_kernel": t_dense,
                                 "torch_sdpa": None if t_sdpa is None else round(t_sdpa, 4),
                                 "torch_backend": backend}
            for s in wl.TABLE5_SPARSITY:
                ent = point["sparsity"][str(s)]
                total = t_pool + t_route + ent["stage2_ms"]
                ent["total_ms"] = round(total, 4)
                ent["speedup_vs_same_kernel_dense"] = round(t_dense / total, 3)
                ent["speedup_vs_torch_sdpa"] = None if t_sdpa is None else round(t_sdpa / total, 3)
            print(json.dumps(point), flush=True)
            rows.append(point)
            del inp, q, k, v, kbar, mask, bias, o, lse
            torch.cuda.empty_cache()
    print("mode     N     " + "  ".join(f"s={s:<6}" for s in wl.TABLE5_SPARSITY)
          + "  (speedup over dense causal, same Stage 2 kernel / torch fused attention)",
          file=sys.stderr)
    for p in rows:
        cells = []
        for s in wl.TABLE5_SPARSITY:
            e = p["sparsity"][str(s)]
            t = e["speedup_vs_torch_sdpa"]
            cells.append(f"{e['speedup_vs_same_kernel_dense']:.2f}/{'-' if t is None else f'{t:.2f}'}")
        print(f"{p['mode']:8} {p['n'] // 1024:3}K  " + "  ".join(f"{c:8}" for c in cells),
              file=sys.stderr, flush=True)


def backward_leg(dash, pre, wp: wl.Workload, args) -> dict:
    """Gradients of the 32K prefill (Stage 2 with the selection held fixed, then the routing and
    pooling chain) for a seeded dL/do, timed with HIP events over `steps` passes after `warmup`
    untimed ones. The forward that produces the selection, lse and tau runs once, untimed.
    Algorithmic work of Stage 2: the five products of attention's backward (S = QK^T, dP = dO V^T,
    dV = P^T dO, dQ = dS K, dK = dS^T Q), 2 D flops each per selected (query head, key) pair; they
    run on bf16 MFMA, so the roofline is the bf16 matrix peak."""
    q, k, v = pre["q"], pre["k"], pre["v"]
    kw = dict(block=wp.block, alpha=wp.alpha, gamma=wp.gamma, sigma=wp.sigma)
    fwd = dash.forward(q, k, v, **kw)
    dout = wl.output_gradient(q.shape, 77, q.dtype, q.device)
    hq, hkv, d = wp.h_q, wp.h_kv, wp.head_dim
    ws2 = torch.empty(dash.dash_sparse_attn_backward_workspace_bytes(1, wp.n_q, hq),
                      dtype=torch.uint8, device=q.device)
    wsr = torch.empty(dash.dash_block_entmax_backward_workspace_bytes(1, wp.n_q, hq, hkv),
                      dtype=torch.uint8, device=q.device)
    timer = Timer()

    def one(t):
        s, e = t.span("bwd_attn") if t else (None, None)
        s and s.record()
        dq, dk, dv, dbias = dash.dash_sparse_attn_prefill_backward(
            q, k, v, fwd["lse"], dout, fwd["mask"], fwd["bias"], block=wp.block, workspace=ws2)
        e and e.record()
        s, e = t.span("bwd_route") if t else (None, None)
        s and s.record()
        dash.dash_block_entmax_backward(q, fwd["kbar"], fwd["tau"], fwd["mask"], dbias, dq, dk,
                                        workspace=wsr, **kw)
        e and e.record()

    print(f"[bench] backward: warmup {args.warmup}, timing {args.steps}", file=sys.stderr,
          flush=True)
    for _ in range(args.warmup):
        one(None)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        one(timer)
    torch.cuda.synchronize()
    pairs, _ = selected_pairs_prefill(fwd["mask"], wp)
    flops = 10.0 * d * pairs
    t_attn, t_route = timer.median_ms("bwd_attn"), timer.median_ms("bwd_route")
    tf = flops / (t_attn * 1e-3) / 1e12

    # the routing and pooling gradients with learned summary queries, one per chunk (Alg. 1's
    # form), on the selection the forward with those queries makes
    tc = wp.n_kv // wp.block
    g = torch.Generator(device=q.device).manual_seed(78)
    qbar = torch.randn((tc, hkv, d), generator=g, device=q.device, dtype=torch.float32) * 0.15
    fq = dash.forward(q, k, v, qbar=qbar, **kw)
    dq_q, dk_q, _, dbias_q = dash.dash_sparse_attn_prefill_backward(
        q, k, v, fq["lse"], dout, fq["mask"], fq["bias"], block=wp.block, workspace=ws2)
    wsq = torch.empty(dash.dash_block_entmax_backward_query_workspace_bytes(1, wp.n_q, hq, hkv, d,
                                                                           wp.block),
                      dtype=torch.uint8, device=q.device)
    dqbar = torch.empty_like(qbar)
    tq = Timer()
    for it in range(args.warmup + args.steps):
        s, e = tq.span("q") if it >= args.warmup else (None, None)
        s and s.record()
        dash.dash_block_entmax_backward_query(q, k, fq["kbar"], qbar, fq["tau"], fq["mask"],
                                              dbias_q, dq_q, dk_q, dqbar=dqbar, workspace=wsq,
                                              **kw)
        e and e.record()
    torch.cuda.synchronize()
    return {
        "ms": {"attn": round(t_attn, 3), "route": round(t_route, 3),
               "route_learned_query_per_chunk": round(tq.median_ms("q"), 3)},
        "algorithmic_tflop": round(flops / 1e12, 4),
        "tflops": round(flops / ((t_attn + t_route) * 1e-3) / 1e12, 3),
        "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("sparse_attn_backward")},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=200,
                    help="decode steps timed on their own (median), each from a cold cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode"], default=None,
                    help="run one half of the step (for profiling); no JSON line is printed")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB `steps` times: the "
                         "reference for scaling HBM byte counters; no JSON line is printed")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward leg (gradients of the 32K prefill, timed on their own "
                         "after the step)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the learned-summary-query and streaming legs (timed on their own "
                         "after the step)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (tiny fp32, the 16K alpha / block sweep, the "
                         "256K prefill), each timed on its own after the step with an oracle "
                         "baseline on sampled rows")
    ap.add_argument("--random-mask-sweep", action="store_true",
                    help="run the pages' random-selection efficiency sweep instead of the step "
                         "(Hq 32, Hkv 2, N 16-96K, three sparsities); one JSON line per point")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(the path runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copied {n} bytes x {args.steps}", file=sys.stderr, flush=True)
        return

    import sparse_hierarchical_attention_amd as dash
    dash.lib()
    if args.random_mask_sweep:
        random_mask_sweep(dash, dev, reps=max(1, args.steps // 2))
        return
    wp, wd = wl.PREFILL_32K, wl.DECODE_128K
    print(f"[bench] generating inputs", file=sys.stderr, flush=True)
    pre = wl.make_inputs(wp, dev)
    dec = wl.make_inputs(wd, dev)
    q, k, v = pre["q"], pre["k"], pre["v"]
    qd, kd, vd = dec["q"], dec["k"], dec["v"]

    # outputs and workspaces, allocated once
    nc = -(-wp.n_kv // wp.block)
    kbar = torch.empty((1, wp.n_kv // wp.block, wp.h_kv, wp.head_dim), dtype=torch.float32, device=dev)
    mask = torch.empty((1, wp.n_q, wp.h_kv, -(-nc // 32)), dtype=torch.int32, device=dev)
    bias = torch.empty((1, wp.n_q, wp.h_kv, nc), dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((1, wp.n_q, wp.h_q), dtype=torch.float32, device=dev)
    ws_b = dash.dash_block_entmax_workspace_bytes(q.dtype, 1, wp.n_q, 0, wp.n_kv, wp.h_q, wp.h_kv,
                                                  wp.head_dim, wp.block)
    route_ws = torch.empty(ws_b, dtype=torch.uint8, device=dev) if ws_b else None
    kbar_d = dash.dash_pool_keys(kd, wd.block)          # the decode cache's summaries
    ncd = -(-wd.n_kv // wd.block)
    mask_d = torch.empty((wd.batch, 1, wd.h_kv, -(-ncd // 32)), dtype=torch.int32, device=dev)
    bias_d = torch.empty((wd.batch, 1, wd.h_kv, ncd), dtype=torch.float32, device=dev)
    o_d = torch.empty_like(qd)
    wsd_b = dash.dash_block_entmax_workspace_bytes(qd.dtype, wd.batch, 1, wd.n_kv - 1, wd.n_kv,
                                                   wd.h_q, wd.h_kv, wd.head_dim, wd.block)
    route_ws_d = torch.zeros(max(wsd_b, 1), dtype=torch.uint8, device=dev)
    attn_ws_b = dash.dash_decode_workspace_bytes(wd.batch, wd.n_kv, wd.h_q, wd.h_kv, wd.head_dim,
                                                 wd.block)
    attn_ws_d = torch.zeros(attn_ws_b, dtype=torch.uint8, device=dev) if attn_ws_b else None
    step_ws_d = torch.zeros(dash.dash_decode_step_workspace_bytes(wd.batch, wd.n_kv, wd.h_q, wd.h_kv,
                                                                  wd.head_dim, wd.block),
                            dtype=torch.uint8, device=dev)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB: more than the MALL
    flush_sum = torch.empty((), dtype=torch.float32, device=dev)

    def step(timer: Timer | None):
        def ev(name):
            return timer.span(name) if timer else (None, None)
        if args.only != "decode":
            prefill_step(ev)
        if args.only != "prefill":
            decode_step(ev)

    def prefill_step(ev):
        s, e = ev("pool")
        s and s.record()
        dash.dash_pool_keys(k, wp.block, kbar=kbar)
        e and e.record()
        s, e = ev("entmax")
        s and s.record()
        dash.dash_block_entmax(q, kbar, n_kv=wp.n_kv, block=wp.block, alpha=wp.alpha,
                               gamma=wp.gamma, sigma=wp.sigma, mask=mask, bias=bias,
                               want_tau=False, workspace=route_ws)
        e and e.record()
        s, e = ev("attn")
        s and s.record()
        dash.dash_sparse_attn_prefill(q, k, v, mask, bias, block=wp.block, o=o, lse=lse)
        e and e.record()

    def decode_step(ev):
        s, e = ev("decode")
        s and s.record()
        dash.dash_decode_step(qd, kd, vd, kbar_d, block=wd.block, alpha=wd.alpha, gamma=wd.gamma,
                              sigma=wd.sigma, mask=mask_d, bias=bias_d, o=o_d,
                              workspace=step_ws_d)
        e and e.record()

    def decode_two_calls():
        dash.dash_block_entmax(qd, kbar_d, n_kv=wd.n_kv, block=wd.block, alpha=wd.alpha,
                               gamma=wd.gamma, sigma=wd.sigma, q_pos0=wd.n_kv - 1, mask=mask_d,
                               bias=bias_d, want_tau=False, workspace=route_ws_d)
        dash.dash_sparse_attn_decode(qd, kd, vd, mask_d, bias_d, block=wd.block, o=o_d,
                                     workspace=attn_ws_d)

    def decode_cold(fn, n):
        """Median HIP-event time of fn() over n runs, each after a 1 GiB read (outside the
        events) that leaves none of the step's data in the L2 caches or the 256 MB MALL, and no
        dirty lines to write back either."""
        t = Timer()
        for i in range(n):
            torch.sum(flush, dim=0, out=flush_sum)
            s_ev, e_ev = t.span("x")
            s_ev.record()
            fn()
            e_ev.record()
        torch.cuda.synchronize()
        return t.median_ms("x")

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    timer = Timer()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(timer)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    if args.only:
        print(f"[bench] {args.only} only: {ms_step:.3f} ms per step", file=sys.stderr, flush=True)
        return
    backward = None if args.no_backward else backward_leg(dash, pre, wp, args)
    extras = None if args.no_extras else extras_leg(dash, pre, dec, wp, wd, max(1, args.steps))
    if extras is not None and not args.no_configs:
        extras["configs"] = configs_leg(dash, dev, reps=max(3, args.steps // 2))

    pairs, frac = selected_pairs_prefill(mask, wp)
    issued = issued_pairs_prefill(mask, wp)
    flops = 4.0 * wp.head_dim * pairs
    t_pool, t_ent, t_attn = timer.median_ms("pool"), timer.median_ms("entmax"), timer.median_ms("attn")
    t_pre = t_pool + t_ent + t_attn
    pre_tflops = flops / (t_pre * 1e-3) / 1e12
    attn_tflops = flops / (t_attn * 1e-3) / 1e12
    dbytes, mean_routed = decode_bytes(mask_d, wd)
    # the decode step on its own, from a cold cache, as the median of --decode-steps runs: the
    # fused step (headline), the same step as a HIP graph replay, and the two separate calls
    print(f"[bench] decode: {args.decode_steps} cold steps each way", file=sys.stderr, flush=True)
    n_dec = max(1, args.decode_steps)
    t_dec = decode_cold(lambda: decode_step(lambda name: (None, None)), n_dec)
    dec_graph = decode_graph(lambda: decode_step(lambda name: (None, None)))
    t_dec_graph = decode_cold(dec_graph.replay, n_dec)
    t_dec_two = decode_cold(decode_two_calls, n_dec)
    decode_step(lambda name: (None, None))  # leave the step's own mask in mask_d
    torch.cuda.synchronize()
    t_dec_in_step = timer.median_ms("decode")
    dec_gbps = dbytes / (t_dec * 1e-3) / 1e9
    traffic = measured_traffic("sparse_attn_prefill")
    dec_traffic = measured_traffic("decode_step")

    out = {
        "metric": METRIC,
        "value": round(pre_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, planted chunks; see workloads.py)",
        "config": {
            "workload": f"{wp.name} + {wd.name}",
            "prefill": {"batch": wp.batch, "seq_len": wp.n_kv, "h_q": wp.h_q, "h_kv": wp.h_kv,
                        "head_dim": wp.head_dim, "block": wp.block, "alpha": wp.alpha,
                        "gamma": wp.gamma, "sigma": wp.sigma},
            "decode": {"batch": wd.batch, "context": wd.n_kv, "h_q": wd.h_q, "h_kv": wd.h_kv,
                       "head_dim": wd.head_dim, "block": wd.block, "alpha": wd.alpha,
                       "gamma": wd.gamma, "sigma": wd.sigma},
        },
        "prefill": {
            "selected_pairs": pairs, "routed_fraction": round(frac, 4),
            "issued_pairs": issued, "useful_fraction_of_issued": round(pairs / issued, 4),
            "algorithmic_tflop": round(flops / 1e12, 4),
            "ms": {"pool": round(t_pool, 4), "entmax": round(t_ent, 4), "attn": round(t_attn, 4)},
            "attn_tflops": round(attn_tflops, 3),
            "end_to_end_tflops": round(pre_tflops, 3),
        },
        "decode": {
            "tok_per_s": round(wd.batch / (t_dec * 1e-3), 1),
            "us_per_step": round(t_dec * 1e3, 2),
            "us_per_step_graph": round(t_dec_graph * 1e3, 2),
            "us_per_step_two_calls": round(t_dec_two * 1e3, 2),
            "us_per_step_after_prefill": round(t_dec_in_step * 1e3, 2),
            "timing": f"median of {n_dec} steps, each after a 1 GiB read (cold L2 and MALL)",
            "algorithmic_bytes": dbytes,
            "mean_routed_chunks": round(mean_routed, 3),
            "gb_per_s": round(dec_gbps, 1),
            "roofline": {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                         "traffic": dec_traffic},
        },
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 3),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic},
        "cpu_baseline": None,
        "backward": backward,
        "extras": extras,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(pre, dec, wp, wd, pairs / wp.n_q)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
