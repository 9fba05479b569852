"""Pins of the oracle's attention parts against library routines and closed
forms (no GPU).

Zipage (arXiv 2603.08743): Sec. 6 (decode attention is ordinary softmax
attention over the resident tokens), App. C.2 / Alg. 1 (window logits, causal
mask on the last block, softmax, GQA max, window mean).
"""
import math

import numpy as np
import pytest
import torch

from oracle import zipage as Z


def _sdpa(q, K, V):
    """torch's scaled_dot_product_attention on the CPU in float64, GQA by
    repeating kv-heads (library routine used as the independent pin)."""
    h_q, d = q.shape
    h_kv = K.shape[0]
    g = h_q // h_kv
    qt = torch.from_numpy(q).double()[:, None, :]               # [h_q][1][d]
    Kt = torch.from_numpy(K).double().repeat_interleave(g, 0)   # [h_q][n][d]
    Vt = torch.from_numpy(V).double().repeat_interleave(g, 0)
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt)[:, 0].numpy()


@pytest.mark.parametrize("h_q,h_kv,d,n", [(4, 1, 64, 1), (4, 1, 64, 208), (32, 8, 128, 300), (8, 8, 16, 7)])
def test_decode_matches_sdpa(h_q, h_kv, d, n):
    rng = np.random.default_rng([1, h_q, d, n])
    q = rng.standard_normal((h_q, d))
    K = rng.standard_normal((h_kv, n, d))
    V = rng.standard_normal((h_kv, n, d))
    o, lse = Z.decode_attention(q, K, V)
    np.testing.assert_allclose(o, _sdpa(q, K, V), rtol=1e-12, atol=1e-12)
    # lse against a direct logsumexp of one head
    j = h_q - 1
    logits = K[j // (h_q // h_kv)] @ q[j] / math.sqrt(d)
    assert abs(lse[j] - torch.logsumexp(torch.from_numpy(logits), 0).item()) < 1e-12


def test_paged_decode_equals_dense_when_budget_covers_context():
    """Budget >= context: no compression ever fires, and attention over the
    paged cache read through a scrambled block table equals dense attention
    over the contiguous K/V (the identity the method must keep)."""
    rng = np.random.default_rng(7)
    b, d, h_kv, h_q, n = 16, 32, 2, 8, 75
    N = -(-n // b)
    assert not Z.should_compress(n, b, n_max=N + 1)
    pool = 11
    table = rng.permutation(pool)[:N]
    Kd = rng.standard_normal((h_kv, n, d))
    Vd = rng.standard_normal((h_kv, n, d))
    Kp = rng.standard_normal((pool, h_kv, b, d))
    Vp = rng.standard_normal((pool, h_kv, b, d))
    for t in range(n):
        Kp[table[t // b], :, t % b] = Kd[:, t]
        Vp[table[t // b], :, t % b] = Vd[:, t]
    Kg = np.stack([Z.gather_sequence(Kp[:, h], table, n, b) for h in range(h_kv)])
    Vg = np.stack([Z.gather_sequence(Vp[:, h], table, n, b) for h in range(h_kv)])
    q = rng.standard_normal((h_q, d))
    np.testing.assert_array_equal(Kg, Kd)
    np.testing.assert_allclose(Z.decode_attention(q, Kg, Vg)[0], _sdpa(q, Kd, Vd), atol=1e-12)


def test_post_compaction_decode_is_attention_over_kept_subset():
    """After compaction, decode over the packed pages equals dense attention
    over the kept tokens taken from the pre-compression K/V."""
    rng = np.random.default_rng(11)
    b, d, n_max = 4, 8, 4
    n = 6 * b
    table = [9, 2, 7, 0, 5, 3]
    Kp = rng.standard_normal((10, b, d))
    Vp = rng.standard_normal((10, b, d))
    K = Z.gather_sequence(Kp, table, n, b)
    V = Z.gather_sequence(Vp, table, n, b)
    S = rng.standard_normal(n)
    kept = Z.topk_keep(S, (n_max - 1) * b)
    tag = np.zeros(n, bool)
    tag[kept] = True
    dst = table[:n_max - 1]
    Kc = Z.compact_pages(Kp, table, n, dst, tag, b)
    Vc = Z.compact_pages(Vp, table, n, dst, tag, b)
    q = rng.standard_normal((2, d))
    k_res = Z.gather_sequence(Kc, dst, len(kept), b)
    v_res = Z.gather_sequence(Vc, dst, len(kept), b)
    o = Z.decode_attention(q, k_res[None], v_res[None])[0]
    np.testing.assert_allclose(o, _sdpa(q, K[kept][None], V[kept][None]), atol=1e-12)


def _window_case(seed, g=4, w=8, b=16, N=3, d=16):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((g, w, d)), rng.standard_normal((N * b, d)), b


def test_window_mask_hides_only_later_keys_and_rows_sum_to_one():
    Qw, K, b = _window_case(3)
    g, w, _ = Qw.shape
    n = K.shape[0]
    A = Z.window_logits(Qw, K, b)
    P = Z.softmax_last(A)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-13)
    for u in range(w):
        pos = n - w + u
        assert np.all(np.isneginf(A[:, u, pos + 1:]))
        assert np.all(np.isfinite(A[:, u, :pos + 1]))
    # the last window query sees everything
    assert np.all(np.isfinite(A[:, w - 1]))


def test_attention_score_single_head_single_query_is_softmax():
    """g = 1, w = 1: S0 is just the softmax row of the one window query."""
    rng = np.random.default_rng(5)
    b, d, N = 8, 16, 4
    Qw = rng.standard_normal((1, 1, d))
    K = rng.standard_normal((N * b, d))
    S0 = Z.attention_score(Qw, K, b)
    ref = torch.softmax(torch.from_numpy(K @ Qw[0, 0] / math.sqrt(d)), 0).numpy()
    np.testing.assert_allclose(S0, ref, atol=1e-14)


def test_attention_score_identical_heads_reduce_to_mean_of_causal_softmax():
    """If all g query heads of the group are equal, the GQA max is the common
    value and S0 is the window mean of causal softmax rows."""
    rng = np.random.default_rng(6)
    g, w, b, N, d = 4, 4, 8, 3, 16
    q1 = rng.standard_normal((w, d))
    Qw = np.repeat(q1[None], g, axis=0)
    K = rng.standard_normal((N * b, d))
    n = N * b
    S0 = Z.attention_score(Qw, K, b)
    ref = np.zeros(n)
    for u in range(w):
        vis = n - w + u + 1
        row = torch.softmax(torch.from_numpy(K[:vis] @ q1[u] / math.sqrt(d)), 0).numpy()
        ref[:vis] += row / w
    np.testing.assert_allclose(S0, ref, atol=1e-14)


def test_attention_score_equal_keys_closed_form():
    """All keys equal: each window query spreads 1/(visible count) uniformly."""
    g, w, b, N, d = 2, 4, 8, 2, 4
    n = N * b
    rng = np.random.default_rng(2)
    Qw = rng.standard_normal((g, w, d))
    K = np.tile(rng.standard_normal(d), (n, 1))
    S0 = Z.attention_score(Qw, K, b)
    ref = np.zeros(n)
    for u in range(w):
        vis = n - w + u + 1
        ref[:vis] += 1.0 / vis / w
    np.testing.assert_allclose(S0, ref, atol=1e-15)


@pytest.mark.parametrize("g", [1, 2, 4])
def test_attention_score_mass_between_one_and_g(g):
    Qw, K, b = _window_case(10 + g, g=g)
    S0 = Z.attention_score(Qw, K, b)
    assert 1.0 - 1e-12 <= S0.sum() <= g + 1e-12
    assert np.all(S0 >= 0)


def test_attention_score_heavy_key_dominates():
    """A key aligned with every query and of large norm takes almost all the
    mass (sanity check of the orientation of the logits)."""
    rng = np.random.default_rng(4)
    g, w, b, N, d = 2, 4, 8, 2, 16
    K = rng.standard_normal((N * b, d)) * 0.1
    Qw = np.tile(np.eye(d)[0], (g, w, 1))
    K[5] = 40.0 * np.eye(d)[0]
    S0 = Z.attention_score(Qw, K, b)
    assert S0.argmax() == 5 and S0[5] > 0.99


def test_attention_score_group_reduction_is_max_closed_form():
    """Two query heads, one window query, four keys. Head 0 aims at key 0,
    head 1 at key 1, so with a = s/sqrt(2):
      head 0 probs: (e^a, 1, 1, 1) / (e^a + 3), head 1: (1, e^a, 1, 1) / (e^a + 3)
    and the group max is (e^a, e^a, 1, 1) / (e^a + 3). A mean over the group
    would give (e^a + 1)/2 on the first two, a sum e^a + 1."""
    s = 3.0
    Qw = np.array([[[s, 0.0]], [[0.0, s]]])          # [g=2][w=1][d=2]
    K = np.array([[1.0, 0.0], [0.0, 1.0], [0.0, 0.0], [0.0, 0.0]])
    ea = math.exp(s / math.sqrt(2))
    ref = np.array([ea, ea, 1.0, 1.0]) / (ea + 3)
    np.testing.assert_allclose(Z.attention_score(Qw, K, 4), ref, atol=1e-15)


def _sdpa_causal(Q, K, V, ctx):
    """torch SDPA on the CPU in float64 with the bottom-right causal mask of
    a chunk of T queries after ctx resident tokens (library routine)."""
    T, h_q, d = Q.shape
    h_kv = K.shape[0]
    g = h_q // h_kv
    qt = torch.from_numpy(Q).double().permute(1, 0, 2)          # [h_q][T][d]
    Kt = torch.from_numpy(K).double().repeat_interleave(g, 0)   # [h_q][n][d]
    Vt = torch.from_numpy(V).double().repeat_interleave(g, 0)
    n = K.shape[1]
    mask = torch.arange(n)[None, :] <= (ctx + torch.arange(T))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask)
    lse = torch.logsumexp(torch.where(mask, qt @ Kt.transpose(1, 2) / math.sqrt(d),
                                      torch.tensor(-math.inf, dtype=torch.float64)), -1)
    return o.permute(1, 0, 2).numpy(), lse.T.numpy()


@pytest.mark.parametrize("h_q,h_kv,d,ctx,T", [(4, 1, 64, 0, 37), (32, 8, 128, 0, 70),
                                              (8, 2, 64, 45, 20), (4, 4, 16, 300, 5)])
def test_prefill_matches_causal_sdpa(h_q, h_kv, d, ctx, T):
    rng = np.random.default_rng([2, h_q, d, ctx, T])
    Q = rng.standard_normal((T, h_q, d))
    K = rng.standard_normal((h_kv, ctx + T, d))
    V = rng.standard_normal((h_kv, ctx + T, d))
    O, L = Z.prefill_attention(Q, K, V, ctx)
    Oref, Lref = _sdpa_causal(Q, K, V, ctx)
    np.testing.assert_allclose(O, Oref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L, Lref, rtol=1e-12, atol=1e-12)
    # a subset of rows is the same rows
    O2, L2 = Z.prefill_attention(Q, K, V, ctx, rows=[T - 1, 0])
    np.testing.assert_array_equal(O2, O[[T - 1, 0]])
    np.testing.assert_array_equal(L2, L[[T - 1, 0]])


def test_prefill_first_token_without_context_returns_its_own_value():
    """Position 0 sees only itself: softmax over one key is 1, so o = v_0."""
    rng = np.random.default_rng(5)
    Q = rng.standard_normal((3, 4, 8))
    K = rng.standard_normal((2, 3, 8))
    V = rng.standard_normal((2, 3, 8))
    O, L = Z.prefill_attention(Q, K, V, 0, rows=[0])
    np.testing.assert_allclose(O[0], np.repeat(V[:, 0], 2, axis=0), rtol=0, atol=1e-15)
    # and the log-sum-exp of one logit is that logit
    k0 = np.repeat(K[:, 0], 2, axis=0)
    np.testing.assert_allclose(L[0], np.einsum("hd,hd->h", Q[0], k0) / math.sqrt(8), rtol=1e-14)
