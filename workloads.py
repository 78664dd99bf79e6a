"""Seeded synthetic inputs for the DashAttention forward pass.

This module only draws numbers: it holds none of the method's arithmetic and is shared, unchanged,
by the GPU library's tests and benchmark and by the CPU oracle's tests. Every tensor comes from
its own seeded stream, so a run is reproducible on a given device.

Recipe (the pages run their efficiency benchmark on synthetic inputs, with no dataset; these
shapes follow their long-context settings: 32 query heads, 8 KV heads, head dim 128, chunk 64):
  * values are drawn in float32 and rounded to the working dtype (bf16 round-to-nearest-even);
  * "plain" workloads: Q, K, V ~ N(0, 1);
  * "planted" workloads: for every (sequence b, KV head r) a unit direction u[b, r] is drawn;
    every query of the heads in group r is sqrt(D) * u + N(0, I); keys inside planted chunks are
    3 * u + N(0, I); every other key and every value is N(0, 1). Planted chunks are chosen
      - "span":   `per_span` chunks drawn without replacement inside every run of `span` chunks,
      - "global": `count` chunks drawn without replacement over all complete chunks,
      - "decode": a count m ~ U{lo..hi} per (b, r), positions uniform over the complete chunks
                  before the newest token's chunk.
Bulk N(0, 1) noise is drawn by torch on the target device (Philox on a GPU, so that multi-GiB
caches are cheap to make); the small planted structure is drawn by numpy's PCG64 on the host.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_kv: int              # keys per sequence (prefill: also the number of queries)
    h_q: int
    h_kv: int
    head_dim: int
    block: int
    alpha: float
    gamma: float
    sigma: float
    dtype: str = "bf16"    # "bf16" or "f32"
    decode: bool = False   # one new query per sequence at position n_kv - 1
    plant: str = "none"    # "none" | "span" | "global" | "decode"
    plant_args: dict = field(default_factory=dict)
    seed: int = 0

    @property
    def n_q(self) -> int:
        return 1 if self.decode else self.n_kv

    @property
    def q_pos0(self) -> int:
        return self.n_kv - 1 if self.decode else 0

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: tiny fp32, 32K prefill, 16 x 128K decode, the alpha / block sweep at 16K,
# and the 256K prefill.
TINY = Workload("tiny fp32 causal, 2q/1kv heads, seq 1024, D 64, block 64", 1, 1024, 2, 1, 64, 64,
                1.5, 8.0, 10.0, dtype="f32", seed=1)
PREFILL_32K = Workload("prefill 32K, 32q/8kv heads, D 128, block 64, 4 planted of every 16 chunks",
                       1, 32768, 32, 8, 128, 64, 1.5, 0.5, 1e8, plant="span",
                       plant_args=dict(span=16, per_span=4), seed=2)
DECODE_128K = Workload("decode 16 x 128K context, 32q/8kv heads, D 128, block 64, 1-16 planted chunks",
                       16, 131072, 32, 8, 128, 64, 1.5, 1.5, 1e8, decode=True, plant="decode",
                       plant_args=dict(lo=1, hi=16), seed=3)
SWEEP_16K = Workload("alpha/block sweep at 16K, 32q/8kv heads, D 128", 1, 16384, 32, 8, 128, 64,
                     1.5, 0.5, 1e8, plant="span", plant_args=dict(span=16, per_span=4), seed=4)
PREFILL_256K = Workload("prefill 256K, 32q/8kv heads, D 128, block 128, 128 planted of 2048 chunks",
                        1, 262144, 32, 8, 128, 128, 1.5, 0.5, 1e8, plant="global",
                        plant_args=dict(count=128), seed=5)

# alpha / block points of the sweep, each with the routing scale gamma used for it
SWEEP_POINTS = [(a, b) for a in (1.25, 1.5, 2.0) for b in (32, 64, 128)]


def sweep_workload(alpha: float, block: int, gamma: float) -> Workload:
    return SWEEP_16K.with_(alpha=alpha, block=block, gamma=gamma,
                           name=f"sweep 16K alpha {alpha} block {block} gamma {gamma}")


def _streams(seed: int, n: int):
    return np.random.SeedSequence(seed).spawn(n)


def _torch_seed(ss: np.random.SeedSequence) -> int:
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _randn(shape, ss, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(ss))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def planted_chunks(w: Workload) -> list[list[np.ndarray]]:
    """Planted chunk indices per (b, r); empty lists for unplanted workloads."""
    tc = w.n_kv // w.block
    ss = _streams(w.seed, 6)[3]
    rng = np.random.Generator(np.random.PCG64(ss))
    out = []
    for _b in range(w.batch):
        row = []
        for _r in range(w.h_kv):
            if w.plant == "span":
                span, per = w.plant_args["span"], w.plant_args["per_span"]
                sel = [s + rng.choice(min(span, tc - s), size=min(per, tc - s), replace=False)
                       for s in range(0, tc, span)]
                row.append(np.sort(np.concatenate(sel)) if sel else np.zeros(0, np.int64))
            elif w.plant == "global":
                row.append(np.sort(rng.choice(tc, size=min(w.plant_args["count"], tc),
                                              replace=False)))
            elif w.plant == "decode":
                visible = (w.n_kv - 1) // w.block  # complete chunks before the newest token's
                m = int(rng.integers(w.plant_args["lo"], w.plant_args["hi"] + 1))
                row.append(np.sort(rng.choice(visible, size=min(m, visible), replace=False)))
            else:
                row.append(np.zeros(0, np.int64))
        out.append(row)
    return out


def directions(w: Workload) -> np.ndarray:
    """Unit directions u[b, r] (float32) of the planted workloads."""
    ss = _streams(w.seed, 6)[4]
    rng = np.random.Generator(np.random.PCG64(ss))
    u = rng.standard_normal((w.batch, w.h_kv, w.head_dim))
    return (u / np.linalg.norm(u, axis=-1, keepdims=True)).astype(np.float32)


def make_inputs(w: Workload, device="cpu") -> dict:
    """q [B, n_q, Hq, D], k, v [B, n_kv, Hkv, D] in the workload's dtype on `device`."""
    s_q, s_k, s_v, _, _, _ = _streams(w.seed, 6)
    dt = w.torch_dtype
    B, n, nq, hq, hkv, d = w.batch, w.n_kv, w.n_q, w.h_q, w.h_kv, w.head_dim
    gq = hq // hkv
    planted = planted_chunks(w)
    u = torch.from_numpy(directions(w)).to(device) if w.plant != "none" else None

    q = _randn((B, nq, hq, d), s_q, device)
    if u is not None:
        # every head of group r gets sqrt(D) * u[b, r]
        q += math.sqrt(d) * u.repeat_interleave(gq, dim=1)[:, None, :, :]
    q = q.to(dt)

    # keys and values are drawn one sequence at a time to bound temporary memory
    k = torch.empty((B, n, hkv, d), dtype=dt, device=device)
    v = torch.empty((B, n, hkv, d), dtype=dt, device=device)
    ks, vs = s_k.spawn(B), s_v.spawn(B)
    for b in range(B):
        kb = _randn((n, hkv, d), ks[b], device)
        if u is not None:
            for r in range(hkv):
                for c in planted[b][r]:
                    kb[c * w.block:(c + 1) * w.block, r, :] += 3.0 * u[b, r]
        k[b] = kb.to(dt)
        del kb
        v[b] = _randn((n, hkv, d), vs[b], device).to(dt)
    return dict(q=q, k=k, v=v, planted=planted)


# ------------------------------------------------------------------ injected random selections
# The pages' efficiency benchmark sweeps Stage 2 at a set chunk sparsity s by replacing the
# router's selection with a random bit-packed mask: Hq = 32, Hkv = 2, D = 128, chunk 64,
# N in {16, 32, 64, 96}K, s in {75, 87.5, 93.75} %, prefill at batch 1 and decode at batch 24.
TABLE5_CONTEXTS = (16384, 32768, 65536, 98304)
TABLE5_SPARSITY = (0.75, 0.875, 0.9375)


def table5_workload(n: int, decode: bool) -> Workload:
    kind = "decode 24 x" if decode else "prefill"
    return Workload(f"{kind} {n // 1024}K, 32q/2kv heads, D 128, block 64, random selection",
                    24 if decode else 1, n, 32, 2, 128, 64, 1.5, 0.5, 1e8, decode=decode,
                    seed=6 + (1 if decode else 0))


def output_gradient(shape, seed: int, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """A seeded upstream gradient dL/dO ~ N(0, 1) of the given shape, rounded to dtype."""
    return _randn(tuple(shape), np.random.SeedSequence(seed), device).to(dtype)


def summary_query(h_kv: int, head_dim: int, seed: int, device="cpu", scale: float = 0.3) -> torch.Tensor:
    """A seeded learned summary query qbar [Hkv, D] fp32 ~ N(0, scale^2) for Stage 0's local
    attention over each chunk."""
    return _randn((h_kv, head_dim), np.random.SeedSequence(seed), device) * scale


def ragged_lengths(batch: int, n_cap: int, seed: int, device="cpu") -> torch.Tensor:
    """Seeded per-sequence context lengths int32 [B], uniform over [n_cap / 2, n_cap]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    lens = rng.integers(n_cap // 2, n_cap + 1, size=batch)
    return torch.from_numpy(lens.astype(np.int32)).to(device)


def random_selection(batch: int, n_q: int, q_pos0: int, n_kv: int, h_kv: int, block: int,
                     sparsity: float, seed: int, device="cpu", bias_std: float = 0.0,
                     slab: int = 4096) -> tuple[torch.Tensor, torch.Tensor]:
    """A random selection in the layout Stage 1 writes: mask [B, n_q, Hkv, ceil(Nc / 32)] int32
    (chunk c is bit c % 32 of word c // 32) and bias [B, n_q, Hkv, Nc] float32, Nc = ceil(n_kv /
    block). For the query at position p, each complete chunk before its own chunk c_p = p // block
    is selected independently with probability 1 - sparsity; c_p itself is always selected, and
    no chunk after it. Selected chunks before c_p get bias ~ N(0, bias_std^2) (0 when bias_std is
    0); every other entry is 0. Queries are drawn in slabs of `slab` rows, each from its own
    stream, to bound temporary memory."""
    nc = -(-n_kv // block)
    nw = -(-nc // 32)
    mask = torch.empty((batch, n_q, h_kv, nw), dtype=torch.int32, device=device)
    bias = torch.zeros((batch, n_q, h_kv, nc), dtype=torch.float32, device=device)
    weights = (torch.ones(32, dtype=torch.int64, device=device) << torch.arange(32, device=device))
    chunk = torch.arange(nw * 32, device=device)
    n_slabs = -(-n_q // slab)
    streams = np.random.SeedSequence(seed).spawn(batch * n_slabs)
    for b in range(batch):
        for si in range(n_slabs):
            t0, t1 = si * slab, min(n_q, (si + 1) * slab)
            ss_sel, ss_bias = streams[b * n_slabs + si].spawn(2)
            g = torch.Generator(device=device)
            g.manual_seed(_torch_seed(ss_sel))
            u = torch.rand((t1 - t0, h_kv, nw * 32), generator=g, device=device)
            cp = (q_pos0 + torch.arange(t0, t1, device=device)) // block
            before = chunk[None, :] < torch.minimum(cp, torch.tensor(n_kv // block, device=device))[:, None]
            sel = (u >= sparsity) & before[:, None, :]
            if bias_std > 0.0:
                d = _randn((t1 - t0, h_kv, nw * 32), ss_bias, device) * bias_std
                bias[b, t0:t1] = torch.where(sel, d, torch.zeros_like(d))[..., :nc]
            sel |= (chunk[None, :] == cp[:, None])[:, None, :]
            words = (sel.view(t1 - t0, h_kv, nw, 32).to(torch.int64) * weights).sum(-1)
            mask[b, t0:t1] = (words - ((words >> 31) << 32)).to(torch.int32)  # two's complement
            del u, sel, words
    return mask, bias
