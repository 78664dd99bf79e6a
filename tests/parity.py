"""Comparison helpers for GPU-vs-oracle parity (tolerances as the method's checks demand).

Support sets: identical except for chunks within 1e-4 (x-units) of some head's threshold,
as decided on the oracle's values. tau: |diff| <= 1e-5 * max(1, |tau|) (fp32 resolves tau only
relative to its size; large routing scales put tau near 100).

Bias d = (log w_c - mu) / sigma, on chunks in both supports of rows whose supports match:
|diff| <= 1e-4 * max(1, |d|) plus the error the bias inherits from its conditioning. With
p = (x - tau)^e, e = 1/(alpha-1), an error eps in x - tau moves log p by e * eps / (x - tau), so a
chunk just above its threshold has an ill-conditioned log-weight, and mu, the mean over the routed
chunks, passes a share of every such error on to the whole row. With eps = 1e-6 * max(1, |x|,
|tau|) (fp32 scores and thresholds), the allowed difference is
    (kappa_c + mean_{c' in R} kappa_c') * eps / sigma + 1e-4 * max(1, |d_c|),
    kappa_c = max over the group's heads with p_c > 0 of e / (x_c - tau).
Outputs: fp32 max-abs <= 1e-4; bf16 max-abs <= 2e-2 and mean-abs <= 1e-2, compared on every
row whose support matches exactly (rows with a near-threshold flip have a different, equally
valid token set and are counted instead). A row whose bias carries a conditioning error of up to
delta (the first term above, maximised over its routed chunks) may see its lse move by delta and
its output by 2 * delta * max|v| (softmax weights move by at most a factor e^(+-2 delta)); those
amounts are added to the row's tolerances.
"""
from __future__ import annotations

import numpy as np
import torch

NEAR_TAU = 1e-4
TAU_TOL = 1e-5
BIAS_TOL = 1e-4
F32_MAX_ABS = 1e-4
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 1e-2
EPS_REL = 1e-6


def bits(mask_words: np.ndarray, n_chunks: int) -> np.ndarray:
    """uint32 words [..., W] -> bool [..., n_chunks] (chunk c = bit c % 32 of word c // 32)."""
    w = mask_words.astype(np.uint32)
    c = np.arange(n_chunks)
    return ((w[..., c // 32] >> (c % 32).astype(np.uint32)) & 1).astype(bool)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    return t.float().numpy() if t.dtype == torch.bfloat16 else t.numpy()


def compare_stage1(gpu_mask, gpu_bias, gpu_tau, ref, *, n_kv, block, h_kv, q_pos, alpha,
                   sigma):
    """gpu_* are host arrays for the same listed rows as `ref` (oracle dict). q_pos: absolute
    position of each listed row. Returns a report dict and asserts the tolerances."""
    nc = -(-n_kv // block)
    gb = bits(gpu_mask, nc)
    ob = bits(ref["mask"], nc)
    nrows, hkv, _ = ob.shape
    hq = ref["tau"].shape[1]
    g = hq // hkv
    x, tau = ref["x"], ref["tau"]
    with np.errstate(invalid="ignore"):
        gap = x - tau[:, :, None]                                   # [R, Hq, Nc], NaN past c_p
        near = (np.abs(gap) < NEAR_TAU).reshape(nrows, hkv, g, nc).any(axis=2)
    diff = gb != ob
    bad = diff & ~near
    assert not bad.any(), f"support mismatch away from tau at {np.argwhere(bad)[:5].tolist()}"
    row_flip = diff.any(axis=(1, 2))
    finite = np.isfinite(tau)
    if gpu_tau is not None:
        assert np.array_equal(np.isfinite(gpu_tau), finite), "tau finiteness differs"
        if finite.any():
            dt = np.abs(gpu_tau[finite] - tau[finite]) / np.maximum(1.0, np.abs(tau[finite]))
            assert dt.max() <= TAU_TOL, f"tau max relative diff {dt.max():.3g}"
    # bias, on rows whose supports agree
    routed = ref["w"] > 0                                           # R (excludes the diagonal)
    e = 1.0 / (alpha - 1.0)
    inv_sigma = 0.0 if np.isinf(sigma) else 1.0 / sigma
    with np.errstate(invalid="ignore", divide="ignore"):
        eps = EPS_REL * np.maximum(1.0, np.maximum(np.abs(np.nan_to_num(x)),
                                                   np.abs(np.nan_to_num(tau, posinf=0))[:, :, None]))
        kap_h = np.where(gap > 0, e * eps / np.where(gap > 0, gap, 1.0), 0.0)
    kap = kap_h.reshape(nrows, hkv, g, nc).max(axis=2)               # [R, Hkv, Nc]
    n_r = np.maximum(1, routed.sum(axis=2))
    kap_mu = (kap * routed).sum(axis=2) / n_r                        # [R, Hkv]
    both = gb & ob & routed & ~row_flip[:, None, None]
    cond = (kap + kap_mu[:, :, None]) * inv_sigma                    # conditioning part of |dd|
    cond_row = np.where(routed, cond, 0.0).max(axis=(1, 2)) if routed.any() else np.zeros(nrows)
    worst = 0.0
    if both.any():
        gd, od = gpu_bias[both], ref["bias"][both]
        tol = cond[both] + BIAS_TOL * np.maximum(1.0, np.abs(od))
        ratio = np.abs(gd - od) / tol
        worst = float(ratio.max())
        assert worst <= 1.0, (f"bias diff {np.abs(gd - od)[ratio.argmax()]:.3g} exceeds its "
                              f"tolerance {tol[ratio.argmax()]:.3g}")
        # the bias has zero mean over the routed chunks (mu is their mean log-weight)
        gsum = np.where(gb & routed, np.nan_to_num(gpu_bias), 0.0).sum(axis=2)
        gabs = np.where(gb & routed, np.abs(np.nan_to_num(gpu_bias)), 0.0).sum(axis=2)
        with np.errstate(divide="ignore"):
            mu_ref = np.where(routed, np.log(np.where(routed, ref["w"], 1.0)), 0.0).sum(axis=2) / n_r
        bound = 1e-5 * np.maximum(1.0, gabs) + 1e-6 * n_r * inv_sigma * np.maximum(1.0, np.abs(mu_ref))
        ok = ~row_flip[:, None] & np.ones_like(gsum, dtype=bool)
        assert np.all(np.abs(gsum[ok]) <= bound[ok]), "bias does not have zero mean over R"
    return dict(rows_with_flips=int(row_flip.sum()), flips=int(diff.sum()),
                support_frac=float(routed.sum() / max(1, (np.isfinite(x)).reshape(nrows, hkv, g, nc)[:, :, 0].sum())),
                bias_tol_ratio=worst, row_flip=row_flip, cond_row=cond_row)


def compare_output(gpu_o, ref_o, dtype: str, *, exclude_rows=None, gpu_lse=None, ref_lse=None,
                   cond_row=None, vmax=0.0):
    """Outputs [R, Hq, D] and lse [R, Hq] of the listed rows; cond_row / vmax widen the
    tolerance of rows whose bias is ill-conditioned (see the module docstring)."""
    go = np.asarray(gpu_o, dtype=np.float64)
    ro = np.asarray(ref_o, dtype=np.float64)
    keep = np.ones(go.shape[0], dtype=bool) if exclude_rows is None else ~exclude_rows
    extra = np.zeros(go.shape[0]) if cond_row is None else np.asarray(cond_row, np.float64)
    d = np.abs(go[keep] - ro[keep])
    if d.size == 0:
        return dict(max_abs=0.0, mean_abs=0.0)
    base = F32_MAX_ABS if dtype == "f32" else BF16_MAX_ABS
    tol = base + 2.0 * extra[keep] * vmax
    excess = d.reshape(d.shape[0], -1).max(axis=1) / tol
    assert excess.max() <= 1.0, (f"{dtype} output max-abs {d.max():.3g} "
                                 f"(tolerance {tol[excess.argmax()]:.3g})")
    if dtype != "f32":
        assert d.mean() <= BF16_MEAN_ABS, f"bf16 output mean-abs {d.mean():.3g}"
    rep = dict(max_abs=float(d.max()), mean_abs=float(d.mean()))
    if gpu_lse is not None and ref_lse is not None:
        dl = np.abs(np.asarray(gpu_lse, np.float64)[keep] - np.asarray(ref_lse, np.float64)[keep])
        ltol = (1e-4 if dtype == "f32" else 2e-3) + extra[keep]
        lex = dl.max(axis=1) / ltol
        assert lex.max() <= 1.0, f"lse max diff {dl.max():.3g} (tolerance {ltol[lex.argmax()]:.3g})"
        rep["lse_max_abs"] = float(dl.max())
    return rep
