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
Outputs are checked twice, and every listed row is compared at least once at the fixed
tolerances (fp32 max-abs <= 1e-4; bf16 max-abs <= 2e-2 and mean-abs <= 1e-2; lse 1e-4 / 2e-3):
1. Stage 2 on the GPU's own selection: the oracle's Stage 2 run on the mask and bias the GPU
   produced, for every listed row, near-threshold flips included, with no widening. The bias the
   GPU produced is itself checked against the oracle's in Stage 1 (above).
2. End to end against the oracle's own selection, on rows whose support matches. There the two
   token sets are equal and the outputs differ by the Stage 2 error (check 1) plus the effect of
   the bias difference, which the oracle measures in double precision as its Stage 2 on the GPU's
   selection minus its Stage 2 on its own. That effect is first checked against what the bias
   difference allows (logits moved by at most delta move softmax weights by a factor within
   e^(+-2 delta), so the output by at most (e^(2 delta) - 1) * max|v| and lse by delta), then
   added to the row's tolerance. The widening is reported and capped: it may at most double a
   row's tolerance (WIDEN_CAP); rows past the cap are ill-conditioned (their bias moves the output
   more than the base tolerance), left to check 1, counted, and at most 2 % of the listed rows
   (MAX_ILL_FRAC) may be such rows.
Rows whose support differs only inside the near-threshold band hold a different, equally valid
token set: check 1 compares them, and on the chunks both supports route their bias must differ
from the oracle's by one constant (the two mean log-weights differ; the rest is unique).
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
WIDEN_CAP = 1.0       # widening at most this multiple of the base tolerance
MAX_ILL_FRAC = 0.02   # rows past the cap, as a share of the listed rows
MAX_FLIP_FRAC = 0.02  # rows with a near-threshold support flip, as a share of the listed rows


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
    bias_dev_row = np.where(both, np.abs(np.nan_to_num(gpu_bias) - ref["bias"]), 0.0).max(axis=(1, 2)) \
        if nrows else np.zeros(0)
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
    # rows with a near-threshold flip: on the chunks both supports route, the bias differs from
    # the oracle's by the same constant (the mean log-weights differ), up to the tolerance
    shift_worst = 0.0
    for ri in np.flatnonzero(row_flip):
        for r in range(hkv):
            com = gb[ri, r] & ob[ri, r] & routed[ri, r]
            if com.sum() < 2:
                continue
            dd = gpu_bias[ri, r][com] - ref["bias"][ri, r][com]
            tol = 2.0 * (cond[ri, r][com].max() + BIAS_TOL * np.maximum(1.0, np.abs(ref["bias"][ri, r][com]).max()))
            spread = float(np.abs(dd - np.median(dd)).max())
            shift_worst = max(shift_worst, spread / tol)
            assert spread <= tol, (f"row {ri} group {r}: bias is not a constant shift of the "
                                   f"oracle's on the common chunks ({spread:.3g} > {tol:.3g})")
    return dict(rows_with_flips=int(row_flip.sum()), flips=int(diff.sum()),
                flip_shift_ratio=shift_worst,
                support_frac=float(routed.sum() / max(1, (np.isfinite(x)).reshape(nrows, hkv, g, nc)[:, :, 0].sum())),
                bias_tol_ratio=worst, row_flip=row_flip, cond_row=cond_row,
                bias_dev_row=bias_dev_row)


def compare_output(gpu_o, ref_o, dtype: str, *, exclude_rows=None, gpu_lse=None, ref_lse=None,
                   widen_o=None, widen_l=None):
    """Outputs [R, Hq, D] and lse [R, Hq] of the listed rows against the oracle's.

    Without widen_* this is the fixed-tolerance check. widen_o / widen_l add a per-row allowance
    (absolute, as in the module docstring) to the output / lse tolerance; a row whose allowance
    exceeds WIDEN_CAP times the base tolerance is left out and counted in 'ill_rows'.
    exclude_rows leaves rows out as well (a different valid token set)."""
    go = np.asarray(gpu_o, dtype=np.float64)
    ro = np.asarray(ref_o, dtype=np.float64)
    nrows = go.shape[0]
    keep = np.ones(nrows, dtype=bool) if exclude_rows is None else ~np.asarray(exclude_rows)
    base = F32_MAX_ABS if dtype == "f32" else BF16_MAX_ABS
    lbase = 1e-4 if dtype == "f32" else 2e-3
    wo = np.zeros(nrows) if widen_o is None else np.asarray(widen_o, np.float64) / base
    wl_ = np.zeros(nrows) if widen_l is None or gpu_lse is None else np.asarray(widen_l, np.float64) / lbase
    widen = np.maximum(wo, wl_)                          # in units of the base tolerance
    ill = keep & (widen > WIDEN_CAP)
    keep = keep & ~ill
    widened = keep & (widen > 1e-3)
    rep = dict(rows=int(nrows), compared=int(keep.sum()), ill_rows=int(ill.sum()),
               widened_rows=int(widened.sum()),
               max_widen=float(widen[keep].max()) if keep.any() else 0.0,
               max_abs=0.0, mean_abs=0.0)
    if not keep.any():
        return rep
    d = np.abs(go[keep] - ro[keep])
    tol = base * (1.0 + wo[keep])
    excess = d.reshape(d.shape[0], -1).max(axis=1) / tol
    assert excess.max() <= 1.0, (f"{dtype} output max-abs {d.max():.3g} "
                                 f"(tolerance {tol[excess.argmax()]:.3g})")
    if dtype != "f32":
        assert d.mean() <= BF16_MEAN_ABS, f"bf16 output mean-abs {d.mean():.3g}"
    rep.update(max_abs=float(d.max()), mean_abs=float(d.mean()))
    if gpu_lse is not None and ref_lse is not None:
        dl = np.abs(np.asarray(gpu_lse, np.float64)[keep] - np.asarray(ref_lse, np.float64)[keep])
        ltol = lbase * (1.0 + wl_[keep])
        lex = dl.max(axis=1) / ltol
        assert lex.max() <= 1.0, f"lse max diff {dl.max():.3g} (tolerance {ltol[lex.argmax()]:.3g})"
        rep["lse_max_abs"] = float(dl.max())
    return rep


def check_forward(orc, q, k, v, ref, *, mask, bias, tau, o, lse=None, rows, n_kv, block, h_kv,
                  q_pos, q_pos0=0, alpha, sigma, dtype, vmax, max_flip_frac=MAX_FLIP_FRAC):
    """Every check of one forward pass on the listed rows.

    q, k, v: host tensors the oracle reads; ref: the oracle's forward on the same rows; mask,
    bias, tau, o, lse: the GPU's results for the listed rows (host arrays, tau and lse may be
    None); rows: the listed rows (rho = b * n_q + t) in q's row numbering; q_pos: each listed
    row's absolute position. Returns a report with the Stage 1, own-selection and end-to-end
    statistics; asserts the tolerances of the module docstring."""
    rep = compare_stage1(mask, bias, tau, ref, n_kv=n_kv, block=block, h_kv=h_kv, q_pos=q_pos,
                         alpha=alpha, sigma=sigma)
    nrows = len(rows)
    assert rep["rows_with_flips"] <= max(1, max_flip_frac * nrows), \
        f"{rep['rows_with_flips']} of {nrows} rows have a near-threshold flip"
    own_o, own_lse = orc.sparse_attn(q, k, v, np.asarray(mask).view(np.uint32),
                                     np.asarray(bias, np.float64), block=block, q_pos0=q_pos0,
                                     rows=rows)
    own = compare_output(o, own_o, dtype, gpu_lse=lse, ref_lse=None if lse is None else own_lse)
    assert own["compared"] == nrows
    # the effect of the bias difference on rows whose token sets agree, measured in double, and
    # checked against what that difference allows
    same = ~rep["row_flip"]
    eff_o = np.abs(own_o - ref["o"]).reshape(nrows, -1).max(axis=1)
    eff_l = np.abs(own_lse - ref["lse"]).max(axis=1) if "lse" in ref else np.zeros(nrows)
    dev = rep["bias_dev_row"]
    allow_o = np.expm1(2.0 * dev) * vmax * (1 + 1e-6) + 1e-9
    allow_l = dev * (1 + 1e-6) + 1e-9
    assert np.all(eff_o[same] <= allow_o[same]), "the oracle's Stage 2 moved more than its bias did"
    if "lse" in ref:
        assert np.all(eff_l[same] <= allow_l[same]), "the oracle's lse moved more than its bias did"
    e2e = compare_output(o, ref["o"], dtype, exclude_rows=rep["row_flip"], gpu_lse=lse,
                         ref_lse=None if lse is None else ref["lse"], widen_o=eff_o,
                         widen_l=eff_l)
    assert e2e["ill_rows"] <= max(1, MAX_ILL_FRAC * nrows), \
        f"{e2e['ill_rows']} of {nrows} rows are ill-conditioned past the widening cap"
    out = dict(rows=nrows, support_frac=rep["support_frac"], flips=rep["flips"],
               rows_with_flips=rep["rows_with_flips"], flip_shift_ratio=rep["flip_shift_ratio"],
               bias_tol_ratio=rep["bias_tol_ratio"], own=own, e2e=e2e)
    log_stats(out)
    return out


def log_stats(rep: dict) -> None:
    """Append a parity report to the file named by DASH_PARITY_LOG (one JSON line per check)."""
    import json
    import os
    path = os.environ.get("DASH_PARITY_LOG")
    if not path:
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    with open(path, "a") as f:
        f.write(json.dumps(dict(test=test, **rep)) + "\n")
