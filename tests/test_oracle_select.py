"""Pins of the oracle's selection, compaction, trigger and capacity rules
(no GPU).

Zipage (arXiv 2603.08743): Sec. 4.1 (cap, trigger, reserved block, Fig. 1),
Sec. 4.2 (top-k budget k = (N_max - 1) b, +inf window, eq. (1)), Sec. 4.4
(shared-prefix targets, reference counts), App. C.3 eq. (2), App. C.6 / Alg. 4
(top-k tag, two-pointer compaction).
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import planner as PL
from oracle import zipage as Z

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_keep(S, k):
    """Token t is kept iff fewer than k tokens beat it, where u beats t when
    its score is higher or equal with a higher index (pairwise definition,
    independent of any sort)."""
    n = len(S)
    keep = []
    for t in range(n):
        beaten = sum(1 for u in range(n)
                     if S[u] > S[t] or (S[u] == S[t] and u > t))
        if beaten < k:
            keep.append(t)
    return keep


@pytest.mark.parametrize("seed", range(20))
def test_topk_matches_pairwise_definition(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 14))
    k = int(rng.integers(0, n + 1))
    S = rng.integers(0, 4, n).astype(float)          # many exact ties
    if seed % 3 == 0:
        S[-2:] = np.inf
    kept = Z.topk_keep(S, k)
    assert list(kept) == _brute_keep(S, k)
    assert len(kept) == k and np.all(np.diff(kept) > 0)


def test_topk_is_the_best_subset_by_exhaustion():
    """On a tiny tie-free input the kept set maximises the score sum over all
    subsets of size k."""
    rng = np.random.default_rng(3)
    S = rng.random(9)
    k = 4
    best = max(itertools.combinations(range(9), k), key=lambda c: S[list(c)].sum())
    assert tuple(Z.topk_keep(S, k)) == best


def test_window_is_always_kept():
    rng = np.random.default_rng(4)
    b, w, n_max = 16, 8, 4
    n = 13 * b
    S = rng.random(n)
    S[:50] = 1e9                                      # huge but finite scores
    S[n - w:] = np.inf
    kept = Z.topk_keep(S, (n_max - 1) * b)
    assert set(range(n - w, n)) <= set(kept.tolist())


def test_fig1_compaction_golden():
    """Fig. 1: 16 tokens in 4 blocks, N_max = 4, b = 4, w = 2; the kept 12
    entries are packed in order into the first three blocks and the window
    (tokens 15, 16) is among them; the fourth block takes token 17."""
    with open(os.path.join(GOLDEN, "fig1_compaction.json")) as f:
        G = json.load(f)
    b, n_max, w = G["b"], G["n_max"], G["w"]
    n = len(G["tokens_one_based"])
    kept = [t - 1 for t in G["kept_one_based"]]
    assert len(kept) == (n_max - 1) * b
    assert set(range(n - w, n)) <= set(kept)
    # scores that rank exactly these tokens first; window gets +inf
    S = np.zeros(n)
    S[kept] = 1.0 + np.arange(len(kept))
    S[n - w:] = np.inf
    sel = Z.topk_keep(S, (n_max - 1) * b)
    assert sel.tolist() == kept
    tag = np.zeros(n, bool)
    tag[sel] = True
    table = [0, 1, 2, 3]                              # blocks a, b, c, d
    pages = np.array(G["tokens_one_based"], float).reshape(4, b)[..., None]
    plan = PL.plan_targets(table, {p: 1 for p in table}, n_max)
    assert plan["dst"] == [0, 1, 2] and plan["new_table"][-1] == 3 and plan["release"] == []
    out = Z.compact_pages(pages, table, n, plan["dst"], tag, b)
    packed = out[:3, :, 0].reshape(-1)
    assert packed.tolist() == G["kept_one_based"]
    # next token goes to slot 0 of the reserved block
    nxt = len(kept)
    assert plan["new_table"][nxt // b] == 3 and nxt % b == 0


def test_compaction_all_kept_is_identity_and_out_of_place_matches_gather():
    rng = np.random.default_rng(5)
    b, d = 4, 3
    pages = rng.standard_normal((8, b, d))
    table = [5, 1, 6]
    n = 12
    tag = np.ones(n, bool)
    np.testing.assert_array_equal(Z.compact_pages(pages, table, n, table, tag, b), pages)
    tag = rng.random(n) < 0.5
    dst = [7, 0, 2]
    out = Z.compact_pages(pages, table, n, dst, tag, b)
    src_rows = Z.gather_sequence(pages, table, n, b)[tag]
    got = Z.gather_sequence(out, dst, int(tag.sum()), b)
    np.testing.assert_array_equal(got, src_rows)


def test_trigger_rule():
    b, n_max = 16, 4
    assert not Z.should_compress(63, b, n_max)
    assert Z.should_compress(64, b, n_max)
    assert not Z.should_compress(65, b, n_max)
    assert Z.should_compress(208, b, n_max)       # prefill may exceed the cap
    assert not Z.should_compress(48, b, n_max)     # N = 3 < N_max
    assert Z.window_row(200, 16, 8) == 0 and Z.window_row(207, 16, 8) == 7
    assert Z.window_row(199, 16, 8) == -1


# --- target rule (Sec. 4.4) -------------------------------------------------

def test_plan_without_sharing_keeps_own_blocks_in_place():
    table = [10, 11, 12, 13, 14, 15, 16, 17, 18, 19]
    plan = PL.plan_targets(table, {p: 1 for p in table}, 8)
    assert plan["dst"] == table[:7] and plan["new_table"] == table[:8]
    assert plan["n_new"] == 0 and plan["release"] == [18, 19] and plan["decref"] == []


def test_plan_short_prefix_allocates_prefix_count():
    """N_prefix < N_max - 1: N_prefix new blocks plus reused own blocks."""
    table = [1, 2, 3, 4, 20, 21, 22, 23]
    rc = {1: 128, 2: 128, 3: 128, 4: 128, 20: 1, 21: 1, 22: 1, 23: 1}
    plan = PL.plan_targets(table, rc, 8)
    assert plan["dst"] == ["new0", "new1", "new2", "new3", 20, 21, 22]
    assert plan["new_table"][-1] == 23 and plan["n_new"] == 4
    assert plan["decref"] == [1, 2, 3, 4] and plan["release"] == []


def test_plan_long_prefix_allocates_all_targets():
    """N_prefix >= N_max - 1: N_max - 1 new blocks."""
    table = [1, 2, 3, 4, 5, 30, 31]
    rc = {p: 2 for p in [1, 2, 3, 4, 5]} | {30: 1, 31: 1}
    plan = PL.plan_targets(table, rc, 4)
    assert plan["dst"] == ["new0", "new1", "new2"] and plan["n_new"] == 3
    assert plan["new_table"][-1] == 30 and plan["release"] == [31]
    assert plan["decref"] == [1, 2, 3, 4, 5]
    # everything shared: the reserved block is new as well
    plan = PL.plan_targets([1, 2, 3, 4], {p: 3 for p in [1, 2, 3, 4]}, 4)
    assert plan["n_new"] == 4 and plan["new_table"] == ["new0", "new1", "new2", "new3"]


# --- capacity (eq. (1), eq. (2)) ----------------------------------------------

def _lp_bruteforce(m_avail, m_blk, m_q, n_max):
    """Vertices of the 2-variable LP {m_blk N + m_q M <= A, N_max M <= N,
    M >= 0, N >= 0}, enumerated exactly with fractions; return the vertex with
    the largest M."""
    A = Fraction(m_avail)
    lines = [(Fraction(m_blk), Fraction(m_q), A),     # a N + c M = rhs
             (Fraction(1), Fraction(-n_max), Fraction(0)),
             (Fraction(1), Fraction(0), Fraction(0)),
             (Fraction(0), Fraction(1), Fraction(0))]
    best = None
    for (a1, c1, r1), (a2, c2, r2) in itertools.combinations(lines, 2):
        det = a1 * c2 - a2 * c1
        if det == 0:
            continue
        N = (r1 * c2 - r2 * c1) / det
        M = (a1 * r2 - a2 * r1) / det
        if N < 0 or M < 0 or m_blk * N + m_q * M > A or n_max * M > N:
            continue
        if best is None or M > best[0]:
            best = (M, N)
    return best


@pytest.mark.parametrize("m_avail,m_kv,m_q,n_max,m_f", [
    (1000, 10, 5, 4, 0), (124, 10, 5, 2, 0), (97, 3, 7, 8, 0), (5000, 64, 3, 8, 1),
    (10, 20, 1, 4, 0), (999, 7, 0, 3, 2)])
def test_capacity_is_floored_lp_optimum(m_avail, m_kv, m_q, n_max, m_f):
    M, Nt = PL.capacity(m_avail, m_kv, m_q, n_max, m_f)
    Mopt, Nopt = _lp_bruteforce(m_avail, m_kv + m_f, m_q, n_max)
    assert M == int(Mopt) and Nt == int(Nopt)
    assert (m_kv + m_f) * Nt + M * m_q <= m_avail and M * n_max <= Nt
    # and M is the best feasible integer concurrency
    best = max((m for m in range(0, m_avail + 1)
                if (m_kv + m_f) * n_max * m + m * m_q <= m_avail), default=0)
    assert M == best


def test_capacity_eq2_global_score_fraction():
    """eq. (2): with F in the KV element size the block cost is (1 + 1/(2d))
    m_kv; here F's bytes per block are m_kv / (2 d)."""
    d, m_kv = 128, 2 * 256 * 8 * 128 * 2
    m_f = m_kv // (2 * d)
    assert Fraction(m_kv + m_f) == (1 + Fraction(1, 2 * d)) * m_kv
    M, Nt = PL.capacity(10**11, m_kv, 10**6, 8, m_f)
    assert M == 10**11 // ((m_kv + m_f) * 8 + 10**6)


# --- whole-request simulation ------------------------------------------------

def test_simulation_without_compression_is_dense_decode():
    """Budget above the context: every step is dense attention over prompt +
    decoded tokens (Sec. 6), no event fires."""
    rng = np.random.default_rng(30)
    L, h_q, h_kv, d, n0, T, b = 2, 4, 2, 8, 10, 5, 4
    pk, pv = rng.standard_normal((L, h_kv, n0, d)), rng.standard_normal((L, h_kv, n0, d))
    sq = rng.standard_normal((T, L, h_q, d))
    sk, sv = rng.standard_normal((T, L, h_kv, d)), rng.standard_normal((T, L, h_kv, d))
    res = Z.simulate_request(pk, pv, None, sq, sk, sv, b, 2, n_max=8, params=Z.ScoreParams())
    assert res["events"] == []
    for s in range(T):
        for l in range(L):
            K = np.concatenate([pk[l], np.moveaxis(sk[:s + 1, l], 0, 1)], axis=1)
            V = np.concatenate([pv[l], np.moveaxis(sv[:s + 1, l], 0, 1)], axis=1)
            np.testing.assert_allclose(res["outputs"][s, l], Z.decode_attention(sq[s, l], K, V)[0],
                                       atol=1e-13)


def test_simulation_events_keep_budget_and_gather_kept_rows():
    """An event keeps exactly (N_max - 1) b rows per (layer, kv-head), the
    window among them, and the resident rows are the kept pre-event rows in
    order; the next token lands in the reserved block."""
    rng = np.random.default_rng(31)
    L, h_q, h_kv, d, b, w, n_max = 1, 4, 2, 8, 4, 2, 3
    n0, T = 10, 3           # 12 tokens = 3 full blocks after 2 steps -> event
    pk, pv = rng.standard_normal((L, h_kv, n0, d)), rng.standard_normal((L, h_kv, n0, d))
    sq = rng.standard_normal((T, L, h_q, d))
    sk, sv = rng.standard_normal((T, L, h_kv, d)), rng.standard_normal((T, L, h_kv, d))
    res = Z.simulate_request(pk, pv, None, sq, sk, sv, b, w, n_max, Z.ScoreParams())
    assert len(res["events"]) == 1
    ev = res["events"][0]
    keep = (n_max - 1) * b
    assert ev["n"] == 12 and ev["kept"].shape == (L, h_kv, keep)
    full_K = np.concatenate([pk[0], np.moveaxis(sk[:2, 0], 0, 1)], axis=1)   # [h_kv][12][d]
    for h in range(h_kv):
        kept = ev["kept"][0, h]
        assert {10, 11} <= set(kept.tolist())
        np.testing.assert_array_equal(res["K"][0][h][:keep], full_K[h][kept])
        np.testing.assert_array_equal(res["K"][0][h][keep], sk[2, 0, h])
