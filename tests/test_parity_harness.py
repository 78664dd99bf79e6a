"""The GPU-vs-oracle comparison helpers themselves, on the CPU: the oracle's own results (rounded
to fp32, as a GPU returns them) pass every check, and planted mistakes in the "GPU" side fail the
check meant to catch them. No GPU and no libdash are involved."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from tests import parity


@pytest.fixture(scope="module")
def case(orc):
    w = wl.Workload("harness", 1, 640, 4, 2, 64, 64, 1.5, 8.0, 1.0, dtype="f32", seed=91)
    inp = wl.make_inputs(w, "cpu")
    q, k, v = inp["q"], inp["k"], inp["v"]
    ref = orc.forward(q, k, v, block=w.block, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma)
    return w, q, k, v, ref


def _gpu_like(ref):
    return dict(mask=ref["mask"].copy(), bias=ref["bias"].astype(np.float32),
                tau=ref["tau"].astype(np.float32), o=ref["o"].astype(np.float32),
                lse=ref["lse"].astype(np.float32))


def _check(orc, w, q, k, v, ref, g, **kw):
    rows = np.arange(w.n_q)
    return parity.check_forward(orc, q, k, v, ref, mask=g["mask"], bias=g["bias"], tau=g["tau"],
                                o=g["o"], lse=g["lse"], rows=rows, n_kv=w.n_kv, block=w.block,
                                h_kv=w.h_kv, q_pos=rows, alpha=w.alpha, sigma=w.sigma,
                                dtype=w.dtype, vmax=float(v.abs().max()), **kw)


def test_oracle_results_pass(orc, case):
    w, q, k, v, ref = case
    rep = _check(orc, w, q, k, v, ref, _gpu_like(ref))
    assert rep["own"]["compared"] == w.n_q
    assert rep["e2e"]["compared"] + rep["e2e"]["ill_rows"] == w.n_q
    assert rep["own"]["max_abs"] < 1e-6 and rep["e2e"]["max_abs"] < 1e-6


def test_wrong_output_fails(orc, case):
    w, q, k, v, ref = case
    g = _gpu_like(ref)
    g["o"][w.n_q // 2, 1, 3] += 5e-4
    with pytest.raises(AssertionError, match="output max-abs"):
        _check(orc, w, q, k, v, ref, g)


def test_wrong_bias_fails(orc, case):
    """A bias off by a constant over one row's routed chunks: Stage 1 rejects it (the bias must
    have zero mean over R), and Stage 2 on that selection alone would not see it."""
    w, q, k, v, ref = case
    g = _gpu_like(ref)
    row = w.n_q - 1
    routed = ref["w"][row, 0] > 0
    assert routed.sum() >= 2
    g["bias"][row, 0, routed] += 0.05
    with pytest.raises(AssertionError, match="bias"):
        _check(orc, w, q, k, v, ref, g)


def test_flipped_row_checked_on_own_selection(orc, case):
    """A row whose support gains a chunk (as a near-threshold flip would) is compared against the
    oracle's Stage 2 on that very selection: the right output for the flipped selection passes,
    the oracle's output for its own selection does not."""
    w, q, k, v, ref = case
    row = w.n_q - 1
    nc = -(-w.n_kv // w.block)
    ob = parity.bits(ref["mask"], nc)[row, 0]
    off = [c for c in range(row // w.block) if not ob[c]]
    assert off, "the row routes every chunk"
    c = off[0]
    g = _gpu_like(ref)
    g["mask"][row, 0, c // 32] |= np.uint32(1 << (c % 32))
    g["bias"][row, 0, c] = 0.0
    # make the chunk "near tau" for the Stage 1 check: move the oracle's score onto its threshold
    ref2 = dict(ref)
    ref2["x"] = ref["x"].copy()
    ref2["x"][row, 0:w.h_q // w.h_kv, c] = ref["tau"][row, 0:w.h_q // w.h_kv]
    with pytest.raises(AssertionError, match="output max-abs|lse"):
        _check(orc, w, q, k, v, ref2, g, max_flip_frac=1.0)
    o_flip, lse_flip = orc.sparse_attn(q, k, v, g["mask"], g["bias"].astype(np.float64),
                                       block=w.block, rows=np.arange(w.n_q))
    g["o"] = o_flip.astype(np.float32)
    g["lse"] = lse_flip.astype(np.float32)
    rep = _check(orc, w, q, k, v, ref2, g, max_flip_frac=1.0)
    assert rep["rows_with_flips"] == 1 and rep["own"]["compared"] == w.n_q


def test_widening_is_capped_and_counted():
    """Rows whose allowance would widen the tolerance past the cap are left out of the
    end-to-end comparison and counted; the others widen by at most the cap."""
    o_ref = np.zeros((4, 2, 8))
    o_gpu = o_ref.copy()
    o_gpu[1] += 0.03            # within 2e-2 * (1 + widening 0.6)
    o_gpu[2] += 1.0             # ill-conditioned row, past the cap
    allow = np.array([0.0, 0.6 * 2e-2, 10.0, 0.0])
    rep = parity.compare_output(o_gpu.astype(np.float32), o_ref, "bf16", widen_o=allow)
    assert rep["ill_rows"] == 1 and rep["widened_rows"] == 1 and rep["compared"] == 3
    assert rep["max_widen"] == pytest.approx(0.6)
    o_gpu[1] += 0.02            # now beyond the widened tolerance
    with pytest.raises(AssertionError, match="output max-abs"):
        parity.compare_output(o_gpu.astype(np.float32), o_ref, "bf16", widen_o=allow)
