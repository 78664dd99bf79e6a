"""Seeded input generators: the random selection that the pages' efficiency sweep injects at
Stage 2 follows the layout and rules Stage 1 writes (CPU only)."""
from __future__ import annotations

import numpy as np
import pytest

import workloads as wl


def _bits(mask) -> np.ndarray:
    m = mask.numpy().view(np.uint32)
    return ((m[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(m.shape[:-1] + (-1,))


@pytest.mark.parametrize("sparsity", [0.0, 0.75, 0.9375])
def test_random_selection_layout(sparsity):
    n, block, hkv = 1000, 16, 3
    mask, bias = wl.random_selection(2, n, 0, n, hkv, block, sparsity, seed=3, bias_std=1.0,
                                     slab=256)
    nc = -(-n // block)
    assert mask.shape == (2, n, hkv, -(-nc // 32)) and bias.shape == (2, n, hkv, nc)
    bits = _bits(mask)
    pos = np.arange(n)
    cp = pos // block
    chunk = np.arange(bits.shape[-1])
    # own chunk always set, nothing after it
    assert np.all(bits[:, pos, :, cp] == 1)
    assert not np.any(bits & (chunk[None, None, None, :] > cp[None, :, None, None]))
    # bias only on selected chunks before the own chunk
    before = (chunk[:nc][None, :] < cp[:, None])[None, :, None, :]
    sel = bits[..., :nc].astype(bool) & before
    assert np.all(bias.numpy()[~sel] == 0.0)
    assert np.all(bias.numpy()[sel] != 0.0)
    # density of the candidates
    cand = before.sum() * 2 * hkv
    frac = sel.sum() / cand
    assert abs(frac - (1.0 - sparsity)) < 0.01, frac


def test_random_selection_seeded():
    a = wl.random_selection(1, 300, 0, 300, 2, 32, 0.5, seed=9)[0]
    b = wl.random_selection(1, 300, 0, 300, 2, 32, 0.5, seed=9)[0]
    c = wl.random_selection(1, 300, 0, 300, 2, 32, 0.5, seed=10)[0]
    assert np.array_equal(a.numpy(), b.numpy()) and not np.array_equal(a.numpy(), c.numpy())


def test_random_selection_decode_row():
    """One query at the end of a ragged context: its own (partial) chunk is the last one."""
    n = 4096 + 17
    mask, bias = wl.random_selection(4, 1, n - 1, n, 2, 64, 0.875, seed=4)
    bits = _bits(mask)
    nc = -(-n // 64)
    assert np.all(bits[:, 0, :, nc - 1] == 1) and not np.any(bits[..., nc:])
    assert np.all(bias.numpy() == 0.0)


def test_table5_shapes():
    for n in wl.TABLE5_CONTEXTS:
        p, d = wl.table5_workload(n, False), wl.table5_workload(n, True)
        assert (p.batch, p.h_q, p.h_kv, p.head_dim, p.block) == (1, 32, 2, 128, 64)
        assert (d.batch, d.decode, d.n_q, d.q_pos0) == (24, True, 1, n - 1)
