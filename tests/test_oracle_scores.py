"""Pins of the oracle's global score, pooling and redundancy scores (no GPU).

Zipage (arXiv 2603.08743): App. C.3 / Alg. 2 (global score), App. C.4 eq. (3)
(pooling), App. C.5 / Fig. 11 (original redundancy), Alg. 3 / Fig. 12 (flash
redundancy), App. C.7 / Fig. 15 (lightning redundancy), App. C.8 (tempered
softmax, eq. (4) combination).
"""
import numpy as np
import pytest
import torch

from oracle import zipage as Z


# --- global score -----------------------------------------------------------

def test_global_first_compression_stores_scores():
    S0 = np.array([0.1, 0.2, 0.3, 0.4, 0.5, 0.6])
    S1, F = Z.global_score(S0, np.full(6, 99.0), True, 0.8, 2)
    np.testing.assert_array_equal(S1, S0)
    np.testing.assert_array_equal(F, S0)


def test_global_worked_example():
    """Hand-computed: b = 2, N = 3, alpha = 0.5. Blocks 0 and 1 have history,
    block 2 is the last (fresh) block.
      t:      0    1    2    3    4    5
      F_old:  0.8  0.1  0.6  0.2  7.0  7.0
      S0:     0.3  0.3  0.4  0.05 0.2  0.1
      aF:     0.4  0.05 0.3  0.1   -    -
      S1:     0.4  0.3  0.4  0.1  0.2  0.1
    """
    F_old = np.array([0.8, 0.1, 0.6, 0.2, 7.0, 7.0])
    S0 = np.array([0.3, 0.3, 0.4, 0.05, 0.2, 0.1])
    S1, F = Z.global_score(S0, F_old, False, 0.5, 2)
    np.testing.assert_allclose(S1, [0.4, 0.3, 0.4, 0.1, 0.2, 0.1], atol=1e-15)
    np.testing.assert_allclose(F, S1, atol=1e-15)


def test_global_alpha_zero_is_identity_and_alpha_one_never_decreases_history():
    rng = np.random.default_rng(1)
    S0 = rng.random(12)
    F_old = rng.random(12)
    S1, _ = Z.global_score(S0, F_old, False, 0.0, 4)
    np.testing.assert_array_equal(S1, S0)
    S1, F = Z.global_score(S0, F_old, False, 1.0, 4)
    assert np.all(F[:8] >= F_old[:8])
    np.testing.assert_array_equal(F[8:], S0[8:])


def test_global_sum_worked_example():
    """Decayed sum-reduce (App. C.3's second form), same inputs as the max
    example: S1 = 0.5 F_old + S0 on blocks 0 and 1, the last block as is.
      aF + S0:  0.7  0.35 0.7  0.15 | 0.2  0.1
    """
    F_old = np.array([0.8, 0.1, 0.6, 0.2, 7.0, 7.0])
    S0 = np.array([0.3, 0.3, 0.4, 0.05, 0.2, 0.1])
    S1, F = Z.global_score(S0, F_old, False, 0.5, 2, reduce="sum")
    np.testing.assert_allclose(S1, [0.7, 0.35, 0.7, 0.15, 0.2, 0.1], atol=1e-15)
    np.testing.assert_allclose(F, S1, atol=1e-15)
    S1, F = Z.global_score(S0, F_old, True, 0.5, 2, reduce="sum")
    np.testing.assert_array_equal(S1, S0)                # no history yet


def test_global_sum_of_a_constant_score_is_a_geometric_series():
    """A token that scores s at every compression carries, after its k-th
    compression with history, s (1 + a + ... + a^k) = s (1 - a^(k+1)) / (1 - a);
    the max-reduce keeps s (a < 1)."""
    s, a, b = 0.3, 0.8, 4
    S0 = np.full(3 * b, s)
    F = None
    Fm = None
    for k in range(6):
        _, F = Z.global_score(S0, F, k == 0, a, b, reduce="sum")
        _, Fm = Z.global_score(S0, Fm, k == 0, a, b, reduce="max")
        np.testing.assert_allclose(F[:2 * b], s * (1 - a ** (k + 1)) / (1 - a), rtol=1e-14)
        np.testing.assert_array_equal(F[2 * b:], s)      # the last block has no history
        np.testing.assert_allclose(Fm, s, rtol=0)


def test_global_sum_bounds_the_max_for_nonnegative_scores():
    rng = np.random.default_rng(4)
    S0, F_old = rng.random(16), rng.random(16)
    Ss, _ = Z.global_score(S0, F_old, False, 0.7, 4, reduce="sum")
    Sm, _ = Z.global_score(S0, F_old, False, 0.7, 4, reduce="max")
    assert np.all(Ss >= Sm) and np.all(Ss <= 2 * Sm + 1e-15)
    with pytest.raises(ValueError):
        Z.global_score(S0, F_old, False, 0.7, 4, reduce="mean")


# --- pooling ------------------------------------------------------------------

@pytest.mark.parametrize("kernel", [1, 3, 5, 7])
def test_max_pool_matches_torch(kernel):
    rng = np.random.default_rng(kernel)
    S = rng.random(37)
    ref = torch.nn.functional.max_pool1d(torch.from_numpy(S)[None, None], kernel, 1,
                                         kernel // 2)[0, 0].numpy()
    np.testing.assert_array_equal(Z.max_pool(S, kernel), ref)


def test_max_pool_kernel_one_is_identity():
    S = np.random.default_rng(0).random(9)
    np.testing.assert_array_equal(Z.max_pool(S, 1), S)


# --- redundancy ---------------------------------------------------------------

def _clustered_keys(rng, n, d, n_dirs, noise):
    """Keys drawn around a few random directions so that many cosine values
    exceed the usual thresholds and the zero-out rule is exercised."""
    dirs = rng.standard_normal((n_dirs, d))
    lab = rng.integers(0, n_dirs, n)
    scale = rng.uniform(0.5, 3.0, n)[:, None]
    return (dirs[lab] + noise * rng.standard_normal((n, d))) * scale


@pytest.mark.parametrize("N,b,p", [(1, 8, 0.5), (2, 4, 0.9), (3, 8, 0.5), (4, 4, 0.0), (3, 5, 0.95)])
def test_flash_equals_original(N, b, p):
    """Alg. 3 is a re-organisation of Fig. 11's computation: same row sums."""
    rng = np.random.default_rng([N, b])
    K = _clustered_keys(rng, N * b, 16, 3, 0.3)
    np.testing.assert_allclose(Z.redundancy_rows_flash(K, b, p),
                               Z.redundancy_rows_original(K, p), atol=1e-12)


@pytest.mark.parametrize("b,p", [(8, 0.5), (16, 0.9), (5, 0.0)])
def test_lightning_equals_original_for_one_block(b, p):
    rng = np.random.default_rng(b)
    K = _clustered_keys(rng, b, 16, 2, 0.2)
    np.testing.assert_allclose(Z.redundancy_rows_lightning(K, b, p),
                               Z.redundancy_rows_original(K, p), atol=1e-13)


def _planted(b, N, d, clusters, rng):
    """Keys along orthogonal basis directions with random positive scales.
    ``clusters`` lists position sets; every other key gets a direction of its
    own. Cosines are exactly 1 inside a cluster and 0 elsewhere."""
    n = N * b
    K = np.zeros((n, d))
    used = 0
    owner = {}
    for c in clusters:
        for t in c:
            owner[t] = used
        used += 1
    for t in range(n):
        if t not in owner:
            owner[t] = used
            used += 1
    assert used <= d
    for t in range(n):
        K[t, owner[t]] = rng.uniform(0.3, 5.0)
    return K


def _planted_closed_form(n, clusters):
    """Row sums for clusters of identical directions, any p in [0, 1):
    with m members at ascending positions, every member but the two newest
    keeps m - 1, the second newest keeps m - 2 and the newest keeps 0 (the
    newest loses its entry in every other member's column; the second newest
    loses the one in the newest's column). Singletons keep 0."""
    r = np.zeros(n)
    for c in clusters:
        c = sorted(c)
        m = len(c)
        for t in c[:-2]:
            r[t] = m - 1
        if m >= 2:
            r[c[-2]] = m - 2
            r[c[-1]] = 0
    return r


@pytest.mark.parametrize("p", [0.0, 0.1, 0.5, 0.9])
def test_original_and_lightning_planted_clusters(p):
    rng = np.random.default_rng(int(p * 10))
    b, N, d = 8, 3, 32
    # clusters inside one block (lightning sees them whole) ...
    clusters = [[0, 2, 5, 7], [9, 10], [17, 19, 20]]
    K = _planted(b, N, d, clusters, rng)
    ref = _planted_closed_form(N * b, clusters)
    np.testing.assert_allclose(Z.redundancy_rows_original(K, p), ref, atol=1e-12)
    np.testing.assert_allclose(Z.redundancy_rows_lightning(K, b, p), ref, atol=1e-12)
    np.testing.assert_allclose(Z.redundancy_rows_flash(K, b, p), ref, atol=1e-12)


def test_lightning_ignores_cross_block_similarity():
    """A cluster split across blocks counts only inside each block for the
    lightning score, but fully for the original one."""
    rng = np.random.default_rng(3)
    b, N, d = 4, 2, 16
    clusters = [[1, 2, 5, 6]]
    K = _planted(b, N, d, clusters, rng)
    np.testing.assert_allclose(Z.redundancy_rows_original(K, 0.5),
                               _planted_closed_form(N * b, clusters), atol=1e-12)
    per_block = [[1, 2], [5, 6]]
    np.testing.assert_allclose(Z.redundancy_rows_lightning(K, b, 0.5),
                               _planted_closed_form(N * b, per_block), atol=1e-12)


def test_threshold_above_one_keeps_everything_but_the_diagonal():
    """With p >= 1 nothing is zeroed besides the diagonal: row sums are
    the plain off-diagonal cosine sums."""
    rng = np.random.default_rng(8)
    K = rng.standard_normal((12, 8))
    U = K / np.linalg.norm(K, axis=1, keepdims=True)
    C = U @ U.T
    ref = C.sum(1) - np.diag(C)
    np.testing.assert_allclose(Z.redundancy_rows_original(K, 1.0), ref, atol=1e-12)


def test_zero_norm_key_has_no_similarity():
    K = np.random.default_rng(0).standard_normal((8, 4))
    K[3] = 0
    r = Z.redundancy_rows_lightning(K, 8, 2.0)
    assert r[3] == 0.0


def test_redundancy_score_is_a_distribution_and_temperature_sharpens():
    rng = np.random.default_rng(9)
    r = rng.random(64) * 30
    n = 64
    R1 = Z.redundancy_score(r, n, 1.0)
    R2 = Z.redundancy_score(r, n, 0.1)
    assert abs(R1.sum() - 1) < 1e-14 and abs(R2.sum() - 1) < 1e-14
    assert R2.max() > R1.max()
    ref = torch.softmax(torch.from_numpy(r / n / 0.4), 0).numpy()
    np.testing.assert_allclose(Z.redundancy_score(r, n, 0.4), ref, atol=1e-15)


# --- whole chain --------------------------------------------------------------

def test_score_chain_order_and_window():
    """Parts compose in the paper's order, window entries are +inf, and with
    every optional part switched off the final score is S0."""
    rng = np.random.default_rng(12)
    g, w, b, N, d = 4, 8, 16, 5, 32
    Qw = rng.standard_normal((g, w, d))
    K = rng.standard_normal((N * b, d))
    F_old = rng.random(N * b) * 0.01
    P = Z.ScoreParams()
    S, F_new, parts = Z.score_tokens(Qw, K, F_old, False, b, P, return_parts=True)
    n = N * b
    assert np.all(np.isinf(S[n - w:])) and np.all(np.isfinite(S[:n - w]))
    np.testing.assert_allclose(parts["S1"], Z.global_score(parts["S0"], F_old, False, P.alpha, b)[0])
    np.testing.assert_array_equal(parts["S2"], parts["S1"])   # not first: no pooling
    np.testing.assert_allclose(parts["S3"], parts["S2"] - P.lam * parts["R"])
    np.testing.assert_allclose(F_new, parts["S1"])
    S_first, _, pf = Z.score_tokens(Qw, K, F_old, True, b, P, return_parts=True)
    np.testing.assert_array_equal(pf["S2"], Z.max_pool(pf["S0"], P.pool_kernel))
    off = Z.ScoreParams(use_global=False, use_pool=False, use_redundancy=False)
    S_off, F_off = Z.score_tokens(Qw, K, F_old, True, b, off)
    assert F_off is None
    np.testing.assert_array_equal(S_off[:n - w], Z.attention_score(Qw, K, b)[:n - w])


def test_pooling_every_compression_comes_after_the_global_score():
    """With pooling on every compression, S2 = pool(S1) where S1 already
    carries the decayed history (eq. (3) follows Alg. 2)."""
    rng = np.random.default_rng(13)
    g, w, b, N, d = 2, 4, 8, 4, 16
    Qw = rng.standard_normal((g, w, d))
    K = rng.standard_normal((N * b, d))
    F_old = rng.random(N * b)          # large history so that it dominates
    P = Z.ScoreParams(pool_first_only=False, use_redundancy=False)
    _, _, parts = Z.score_tokens(Qw, K, F_old, False, b, P, return_parts=True)
    S1 = Z.global_score(parts["S0"], F_old, False, P.alpha, b)[0]
    np.testing.assert_array_equal(parts["S2"], Z.max_pool(S1, P.pool_kernel))
    assert not np.array_equal(parts["S2"], Z.max_pool(parts["S0"], P.pool_kernel))
