"""Pins of the oracle's three stages against the pages' own statements and library routines.

DashAttention paper (arXiv 2605.18753v1): §3.1 Eq. 3 (chunk summaries; mean pooling when the
summary query is zero), §3.2 Eq. 4 (entmax routing, GQA mean, union support), §3.3-3.4 Eq. 7-10
and Prop. 1 (prior-induced softmax and its bias form, with App. D's proof), §3.4 (sigma -> inf
limit), §5.1 (chunk size 1 gives entmax routing followed by softmax), §2 Eq. 1 (plain SDPA).
"""
import math

import numpy as np
import pytest
import torch

import workloads as wl


def sdpa_reference(q, k, v, add_mask, scale):
    """Plain SDPA of Eq. 1 through torch's own routine, in float64, with an explicit additive
    mask matrix (-inf where a key is not attended)."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(q)[None, None], torch.as_tensor(k)[None, None],
        torch.as_tensor(v)[None, None], attn_mask=torch.as_tensor(add_mask)[None, None],
        scale=scale)
    return out[0, 0].numpy()


def token_mask_matrix(mask_row, bias_row, pos, block):
    """Additive mask over tokens 0..pos for one query row from its chunk mask and bias."""
    ci = pos // block
    m = np.full(pos + 1, -np.inf)
    for c in range(ci + 1):
        bit = (int(mask_row[c // 32]) >> (c % 32)) & 1
        lo, hi = c * block, min((c + 1) * block, pos + 1)
        if c == ci:
            m[lo:hi] = 0.0
        elif bit:
            m[lo:hi] = bias_row[c]
    return m


def small_case(seed, n=256, hq=4, hkv=2, d=16, block=16, plant=True):
    w = wl.Workload("small", 1, n, hq, hkv, d, block, 1.5, 2.0, 1.0, dtype="f32",
                    plant="span" if plant else "none", plant_args=dict(span=4, per_span=1),
                    seed=seed)
    return w, wl.make_inputs(w, "cpu")


# ------------------------------------------------------------------------------- Stage 0

def test_pool_is_the_mean_at_zero_summary_query(orc):
    """Eq. 3 with qbar = 0: the local softmax is uniform, so the summary is the mean."""
    rng = np.random.default_rng(0)
    k = rng.normal(size=(2, 96, 3, 8)).astype(np.float32)
    kb = orc.pool_keys(k, 32)
    kq = orc.pool_keys_query(k, np.zeros((3, 8)), 32)
    np.testing.assert_allclose(kb, kq, atol=1e-15)
    assert kb.shape == (2, 3, 3, 8)


def test_pool_closed_forms(orc):
    """A ramp k_t = t pools to the chunk midpoint c*B + (B-1)/2; a constant pools to itself;
    an incomplete tail chunk has no summary (Tc = floor(n / B))."""
    n, block = 100, 16
    k = np.broadcast_to(np.arange(n, dtype=np.float32)[None, :, None, None], (1, n, 2, 4)).copy()
    kb = orc.pool_keys(k, block)
    assert kb.shape[1] == n // block
    for c in range(n // block):
        np.testing.assert_array_equal(kb[0, c], c * block + (block - 1) / 2)
    kc = np.full((1, 64, 1, 4), 0.375, dtype=np.float32)
    np.testing.assert_array_equal(orc.pool_keys(kc, 32), 0.375)


def test_pool_bf16_reads_exact_values(orc):
    k = torch.randn(1, 64, 2, 8).to(torch.bfloat16)
    np.testing.assert_allclose(orc.pool_keys(k, 16), orc.pool_keys(k.float().numpy(), 16), atol=0)


def test_learned_summary_query_selects_a_key(orc):
    """A summary query far along one key's direction puts (almost) all local weight on it."""
    k = np.zeros((1, 8, 1, 4), dtype=np.float32)
    k[0, :, 0, :] = np.eye(4, dtype=np.float32)[[0, 1, 2, 3, 0, 1, 2, 3]] * [[1], [1], [1], [1], [-1], [-1], [-1], [-1]]
    qbar = np.array([[0.0, 0.0, 400.0, 0.0]])
    kb = orc.pool_keys_query(k, qbar, 4)
    np.testing.assert_allclose(kb[0, 0, 0], [0, 0, 1, 0], atol=1e-12)
    # chunk 1 holds -e0..-e3: logit -200 for -e2, three ties at 0 share the weight
    np.testing.assert_allclose(kb[0, 1, 0], [-1 / 3, -1 / 3, 0, -1 / 3], atol=1e-12)


def test_per_chunk_summary_queries_closed_form(orc):
    """One summary query per chunk (and per sequence): two keys per chunk, D = 4 (sqrt(D) = 2),
    each chunk's own query sets its logits to (ln 3, 0) / (0, ln 4) / ..., so the weights are
    3/4, 1/4 and 1/5, 4/5 by hand; a query taken from the wrong chunk or sequence gives other
    weights."""
    e = np.eye(4)
    k = np.zeros((2, 4, 1, 4))
    k[:, 0, 0], k[:, 1, 0], k[:, 2, 0], k[:, 3, 0] = e[0], e[1], e[2], e[3]
    q = np.zeros((2, 2, 1, 4))
    q[0, 0, 0, 0] = 2 * np.log(3.0)      # seq 0, chunk 0: logits (ln 3, 0)
    q[0, 1, 0, 3] = 2 * np.log(4.0)      # seq 0, chunk 1: logits (0, ln 4)
    q[1, 0, 0, 1] = 2 * np.log(9.0)      # seq 1, chunk 0: logits (0, ln 9)
    q[1, 1, 0, 2] = -2 * np.log(2.0)     # seq 1, chunk 1: logits (-ln 2, 0)
    kb = orc.pool_keys_query(k, q, 2)
    np.testing.assert_allclose(kb[0, 0, 0], [0.75, 0.25, 0, 0], atol=1e-15)
    np.testing.assert_allclose(kb[0, 1, 0], [0, 0, 0.2, 0.8], atol=1e-15)
    np.testing.assert_allclose(kb[1, 0, 0], [0.1, 0.9, 0, 0], atol=1e-15)
    np.testing.assert_allclose(kb[1, 1, 0], [0, 0, 1 / 3, 2 / 3], atol=1e-15)
    # one query per chunk shared by both sequences: sequence 1 takes sequence 0's queries
    kc = orc.pool_keys_query(k, q[0], 2)
    np.testing.assert_allclose(kc[1], kb[0], atol=1e-15)


def test_per_chunk_queries_equal_across_chunks_give_the_per_head_form(orc):
    rng = np.random.default_rng(3)
    k = rng.normal(size=(2, 96, 3, 8)).astype(np.float32)
    qh = rng.normal(size=(3, 8))
    per_head = orc.pool_keys_query(k, qh, 32)
    per_chunk = orc.pool_keys_query(k, np.broadcast_to(qh, (3, 3, 8)), 32)
    per_seq_chunk = orc.pool_keys_query(k, np.broadcast_to(qh, (2, 3, 3, 8)), 32)
    np.testing.assert_array_equal(per_head, per_chunk)
    np.testing.assert_array_equal(per_head, per_seq_chunk)


# ------------------------------------------------------------------------------- Stage 1

@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_route_scores_probabilities_mask_bias(orc, alpha):
    w, inp = small_case(3)
    q, k = inp["q"], inp["k"]
    block, gamma, sigma = w.block, 2.0, 3.0
    kbar = orc.pool_keys(k, block)
    st = orc.block_entmax(q, kbar, n_kv=w.n_kv, block=block, alpha=alpha, gamma=gamma, sigma=sigma)
    n, hq, hkv, d = w.n_kv, w.h_q, w.h_kv, w.head_dim
    gq = hq // hkv
    qn = q.numpy().astype(np.float64)[0]
    # scores via a library matmul: x = (alpha - 1) gamma <q_h, kbar_{h // gq}> / sqrt(D)
    for t in range(0, n, 7):
        ci = t // block
        for h in range(hq):
            ref = (alpha - 1) * gamma * (kbar[0, :ci, h // gq, :] @ qn[t, h]) / math.sqrt(d)
            np.testing.assert_allclose(st["x"][t, h, :ci], ref, rtol=1e-12, atol=1e-14)
            assert np.all(np.isnan(st["x"][t, h, ci:]))
        for r in range(hkv):
            wr = st["w"][t, r, :ci]
            heads = range(r * gq, (r + 1) * gq)
            ps = [orc.entmax(st["x"][t, h, :ci], alpha) for h in heads]
            np.testing.assert_allclose(wr, np.mean(ps, axis=0), atol=1e-14)
            if ci == 0:
                continue
            assert abs(wr.sum() - 1.0) <= 1e-12                       # a distribution
            union = np.any([p > 0 for p in ps], axis=0)
            np.testing.assert_array_equal(wr > 0, union)              # union of supports
            bits = np.array([(int(st["mask"][t, r, c // 32]) >> (c % 32)) & 1
                             for c in range(w.n_kv // block)])
            np.testing.assert_array_equal(bits[:ci], union)
            assert bits[ci] == 1 and not bits[ci + 1:].any()          # diagonal bit only beyond
            d_r = st["bias"][t, r, :ci][union]
            assert abs(d_r.sum()) <= 1e-9                             # d has zero mean over R
            np.testing.assert_allclose(d_r * sigma, np.log(wr[union]) - np.log(wr[union]).mean(),
                                       atol=1e-12)
            assert st["bias"][t, r, ci] == 0.0


def test_route_sigma_infinite_gives_zero_bias(orc):
    w, inp = small_case(4)
    kbar = orc.pool_keys(inp["k"], w.block)
    st = orc.block_entmax(inp["q"], kbar, n_kv=w.n_kv, block=w.block, alpha=1.5, gamma=2.0,
                          sigma=math.inf)
    assert np.all(st["bias"] == 0.0)


def test_route_first_chunk_rows_attend_to_themselves_only(orc):
    w, inp = small_case(5)
    kbar = orc.pool_keys(inp["k"], w.block)
    st = orc.block_entmax(inp["q"], kbar, n_kv=w.n_kv, block=w.block, alpha=1.5, gamma=2.0, sigma=1.0)
    for t in range(w.block):
        assert np.all(st["mask"][t, :, 0] == 1) and np.all(np.isinf(st["tau"][t]))


# ---------------------------------------------- the attention window [DA App. B.1.1]

def test_window_of_one_block_is_the_default(orc):
    w, inp = small_case(14)
    kbar = orc.pool_keys(inp["k"], w.block)
    a = orc.block_entmax(inp["q"], kbar, n_kv=w.n_kv, block=w.block, alpha=1.5, gamma=2.0, sigma=3.0)
    b = orc.block_entmax(inp["q"], kbar, n_kv=w.n_kv, block=w.block, alpha=1.5, gamma=2.0, sigma=3.0,
                         window=1)
    for key in ("mask", "bias", "tau"):
        np.testing.assert_array_equal(a[key], b[key])


@pytest.mark.parametrize("window", [2, 3])
def test_window_blocks_always_attended_and_not_routed(orc, window):
    """The window's blocks (the query's own and window - 1 before it) carry their mask bit and
    d = 0; routing sees only the complete chunks before them, and its threshold solves Eq. 2 on
    exactly those candidates."""
    w, inp = small_case(15)
    kbar = orc.pool_keys(inp["k"], w.block)
    alpha, sigma = 1.5, 3.0
    st = orc.block_entmax(inp["q"], kbar, n_kv=w.n_kv, block=w.block, alpha=alpha, gamma=2.0,
                          sigma=sigma, window=window)
    gq = w.h_q // w.h_kv
    for t in range(0, w.n_kv, 3):
        ci = t // w.block
        lo = max(0, ci - window + 1)
        for h in range(w.h_q):
            x = st["x"][t, h]
            assert np.all(np.isnan(x[lo:]))                       # window and later: no score
            if lo == 0:
                assert np.isinf(st["tau"][t, h])
                continue
            assert not np.any(np.isnan(x[:lo]))
            resid = np.sum(np.maximum(x[:lo] - st["tau"][t, h], 0.0) ** (1 / (alpha - 1))) - 1
            assert abs(resid) < 1e-10                             # Eq. 2 on c < lo
        for r in range(w.h_kv):
            bits = np.array([(int(st["mask"][t, r, c // 32]) >> (c % 32)) & 1
                             for c in range(-(-w.n_kv // w.block))])
            assert bits[lo:ci + 1].all() and not bits[ci + 1:].any()
            assert np.all(st["bias"][t, r, lo:ci + 1] == 0.0)
            np.testing.assert_array_equal(bits[:lo], st["w"][t, r, :lo] > 0)
            assert np.all(st["w"][t, r, lo:] == 0.0)


@pytest.mark.parametrize("window", [2, 3])
def test_window_attention_matches_brute_force_sdpa(orc, window):
    """Stage 2 on a window's selection vs Eq. 1 with an explicit token-level mask and bias."""
    w, inp = small_case(16)
    q, k, v = (inp[x] for x in ("q", "k", "v"))
    res = orc.forward(q, k, v, block=w.block, alpha=1.5, gamma=2.0, sigma=1.0, window=window)
    gq = w.h_q // w.h_kv
    scale = 1 / math.sqrt(w.head_dim)
    qd, kd, vd = (x.double()[0] for x in (q, k, v))
    for t in range(0, w.n_kv, 7):
        for h in range(w.h_q):
            r = h // gq
            am = token_mask_matrix(res["mask"][t, r], res["bias"][t, r], t, w.block)
            lo = max(0, t // w.block - window + 1)
            assert np.all(am[lo * w.block:] == 0.0)               # the window, unbiased, in full
            ref = sdpa_reference(qd[t:t + 1, h], kd[:t + 1, r], vd[:t + 1, r], am[None], scale)
            np.testing.assert_allclose(res["o"][t, h], ref[0], atol=1e-12)


def test_window_over_every_chunk_is_causal_sdpa(orc):
    """A window reaching chunk 0 for every query leaves nothing to route: causal SDPA."""
    w, inp = small_case(17, plant=False)
    q, k, v = (inp[x] for x in ("q", "k", "v"))
    res = orc.forward(q, k, v, block=w.block, alpha=1.5, gamma=2.0, sigma=1.0,
                      window=w.n_kv // w.block + 1)
    gq = w.h_q // w.h_kv
    qd = q.double()[0].transpose(0, 1)[None]
    kd = k.double()[0].transpose(0, 1).repeat_interleave(gq, 0)[None]
    vd = v.double()[0].transpose(0, 1).repeat_interleave(gq, 0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, is_causal=True)[0]
    np.testing.assert_allclose(res["o"], ref.transpose(0, 1).numpy(), atol=1e-12)


# ------------------------------------------------------------------------------- Stage 2

@pytest.mark.parametrize("sigma", [1.0, 10.0, 1e8])
def test_attend_matches_brute_force_sdpa(orc, sigma):
    """Bias form vs Eq. 1 evaluated by torch with an explicit token-level additive mask."""
    w, inp = small_case(6)
    q, k, v = (inp[x] for x in ("q", "k", "v"))
    res = orc.forward(q, k, v, block=w.block, alpha=1.5, gamma=2.0, sigma=sigma)
    gq = w.h_q // w.h_kv
    scale = 1 / math.sqrt(w.head_dim)
    qd, kd, vd = (x.double()[0] for x in (q, k, v))
    for t in range(0, w.n_kv, 5):
        for h in range(w.h_q):
            r = h // gq
            am = token_mask_matrix(res["mask"][t, r], res["bias"][t, r], t, w.block)
            ref = sdpa_reference(qd[t:t + 1, h], kd[:t + 1, r], vd[:t + 1, r], am[None], scale)
            np.testing.assert_allclose(res["o"][t, h], ref[0], atol=1e-12)
            lg = scale * (kd[:t + 1, r] @ qd[t, h]).numpy() + am
            assert abs(res["lse"][t, h] - torch.logsumexp(torch.as_tensor(lg), 0).item()) < 1e-12


@pytest.mark.parametrize("sigma", [0.5, 1.0, 10.0, 1e8, math.inf])
@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_proposition_1_prior_form_equals_bias_form(orc, alpha, sigma):
    """Prop. 1 (proved in App. D): Eq. 7 with the prior of Eq. 8-10 equals softmax(z + d) V."""
    w, inp = small_case(7)
    q, k, v = (inp[x] for x in ("q", "k", "v"))
    res = orc.forward(q, k, v, block=w.block, alpha=alpha, gamma=2.0, sigma=sigma)
    o2 = orc.sparse_attn_prior(q, k, v, res["w"], block=w.block, sigma=sigma)
    np.testing.assert_allclose(res["o"], o2, atol=1e-10, rtol=0)


def test_sigma_infinite_is_softmax_on_selected_tokens(orc):
    """sigma -> inf: the prior is uniform over the routed support and lambda -> |R|/(|R|+|D|),
    i.e. plain softmax over the selected tokens (§3.4)."""
    w, inp = small_case(8)
    q, k, v = (inp[x] for x in ("q", "k", "v"))
    res = orc.forward(q, k, v, block=w.block, alpha=1.5, gamma=2.0, sigma=math.inf)
    scale = 1 / math.sqrt(w.head_dim)
    qd, kd, vd = (x.double()[0] for x in (q, k, v))
    gq = w.h_q // w.h_kv
    for t in range(w.block, w.n_kv, 9):
        for h in range(w.h_q):
            r = h // gq
            sel = np.zeros(t + 1, dtype=bool)
            for c in range(t // w.block + 1):
                if (int(res["mask"][t, r, c // 32]) >> (c % 32)) & 1:
                    sel[c * w.block:min((c + 1) * w.block, t + 1)] = True
            lg = scale * (kd[:t + 1, r] @ qd[t, h]).numpy()
            p = np.where(sel, np.exp(lg - lg[sel].max()), 0.0)
            np.testing.assert_allclose(res["o"][t, h], (p / p.sum()) @ vd[:t + 1, r].numpy(),
                                       atol=1e-12)


def test_dense_limit_is_causal_sdpa(orc):
    """alpha -> 1 routes to every chunk (softmax is dense) and sigma = inf removes the bias:
    the output is causal SDPA (Eq. 1 with a causal mask)."""
    w, inp = small_case(9, plant=False)
    q, k, v = (inp[x] for x in ("q", "k", "v"))
    res = orc.forward(q, k, v, block=w.block, alpha=1.0 + 1e-5, gamma=1.0, sigma=math.inf)
    gq = w.h_q // w.h_kv
    qd = q.double()[0].transpose(0, 1)[None]
    kd = k.double()[0].transpose(0, 1).repeat_interleave(gq, 0)[None]
    vd = v.double()[0].transpose(0, 1).repeat_interleave(gq, 0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, is_causal=True)[0]
    np.testing.assert_allclose(res["o"], ref.transpose(0, 1).numpy(), atol=1e-12)


def test_chunk_size_one_is_entmax_then_softmax(orc):
    """§5.1: with chunk size 1 the method is alpha-entmax over tokens followed by softmax on its
    support (plus the query itself); with sigma = inf there is no bias."""
    w, inp = small_case(10, n=48, block=1)
    q, k, v = (inp[x] for x in ("q", "k", "v"))
    alpha, gamma = 1.5, 4.0
    res = orc.forward(q, k, v, block=1, alpha=alpha, gamma=gamma, sigma=math.inf)
    qd, kd, vd = (x.double()[0].numpy() for x in (q, k, v))
    gq, d = w.h_q // w.h_kv, w.head_dim
    for t in range(1, w.n_kv):
        for r in range(w.h_kv):
            sup = np.zeros(t, dtype=bool)
            for h in range(r * gq, (r + 1) * gq):
                z = kd[:t, r] @ qd[t, h] / math.sqrt(d)
                sup |= orc.entmax((alpha - 1) * gamma * z, alpha) > 0
            sel = np.append(sup, True)
            for h in range(r * gq, (r + 1) * gq):
                lg = kd[:t + 1, r] @ qd[t, h] / math.sqrt(d)
                p = np.where(sel, np.exp(lg - lg[sel].max()), 0.0)
                np.testing.assert_allclose(res["o"][t, h], (p / p.sum()) @ vd[:t + 1, r], atol=1e-12)


def test_decode_row_equals_prefill_last_row(orc):
    """A single query at position n - 1 (decode) gives the prefill result of that row."""
    w, inp = small_case(11)
    q, k, v = (inp[x] for x in ("q", "k", "v"))
    full = orc.forward(q, k, v, block=w.block, alpha=1.5, gamma=2.0, sigma=10.0)
    last = orc.forward(q[:, -1:], k, v, block=w.block, alpha=1.5, gamma=2.0, sigma=10.0,
                       q_pos0=w.n_kv - 1)
    np.testing.assert_array_equal(last["mask"][0], full["mask"][-1])
    np.testing.assert_allclose(last["o"][0], full["o"][-1], atol=1e-15)


def test_row_subset_equals_full_run(orc):
    w, inp = small_case(12)
    q, k, v = (inp[x] for x in ("q", "k", "v"))
    full = orc.forward(q, k, v, block=w.block, alpha=1.5, gamma=2.0, sigma=1.0)
    rows = [0, 17, 100, 255]
    sub = orc.forward(q, k, v, block=w.block, alpha=1.5, gamma=2.0, sigma=1.0, rows=rows)
    np.testing.assert_array_equal(sub["mask"], full["mask"][rows])
    np.testing.assert_array_equal(sub["o"], full["o"][rows])
