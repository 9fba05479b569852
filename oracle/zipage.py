"""Float64 CPU oracle of Compressed PagedAttention's data-parallel hot path.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): slow, plain NumPy,
float64 arithmetic, one request / layer / kv-head at a time. Inputs in bf16 or
fp32 arrive as float32 or float64 arrays and are upcast exactly.

Source of every definition: "Zipage: Maintain High Request Concurrency for LLM
Reasoning through Compressed PagedAttention" (Liao et al., arXiv 2603.08743),
cited below as "Zipage" with the section, algorithm, equation or figure.

Readings taken where the paper is silent or garbled:
  * causal mask of the window logits: a window query never sees a key that
    comes after it (the printed inequality of Alg. 1 is inverted);
  * GQA grouping is contiguous: query head j belongs to kv-head j // g;
  * order of reductions in the attention score: softmax per query head over
    all n tokens, then max over the group, then mean over the window;
  * the global score cache holds the pre-pooling score; alpha is applied once
    per compression event;
  * pooling is a stride-1 max over a centred window of odd width, clipped at
    the sequence ends;
  * the redundancy threshold test is strict (C > p), the diagonal is zeroed
    first, "last" means the highest token index, and every variant divides the
    row sums by the full length n before the tempered softmax;
  * a zero-norm key has cosine 0 with everything;
  * top-k ties are broken towards the newer (higher-index) token.
"""
from __future__ import annotations

from dataclasses import dataclass
import math

import numpy as np

_F = np.float64


def _f64(x):
    return np.asarray(x, dtype=_F)


# ---------------------------------------------------------------------------
# Paged layout (Zipage Sec. 3 "Pre-allocated memory" / "KV cache management")
# ---------------------------------------------------------------------------

def gather_sequence(pages, table, n, b):
    """Logical token rows [n][...] of one request from its block table.

    ``pages`` is one (layer, kv-head) slice of the cache, shaped
    [num_blocks][b][...]; token t lives in page ``table[t // b]`` at slot
    ``t % b`` (Zipage Sec. 3: a request's sequence is cut into blocks of b
    tokens, recorded in order in its block table).
    """
    out = [np.asarray(pages[table[t // b]][t % b]) for t in range(n)]
    return _f64(np.stack(out)) if n else _f64(np.zeros((0,) + np.shape(pages)[2:]))


# ---------------------------------------------------------------------------
# Decode attention (Zipage Sec. 6: eviction leaves the attention forward as
# ordinary softmax attention over whatever tokens are resident)
# ---------------------------------------------------------------------------

def decode_attention(q, K, V, scale=None):
    """Grouped-query softmax attention of one decode token.

    q: [h_q][d]; K, V: [h_kv][n][d]. Query head j reads kv-head j // g with
    g = h_q / h_kv. Returns (o [h_q][d], lse [h_q]) where
    o_j = sum_t softmax_t(q_j . k_t * scale) v_t and lse_j = log sum_t exp(.).
    The scale is 1/sqrt(d), the factor Zipage Alg. 1 uses for its logits.
    """
    q, K, V = _f64(q), _f64(K), _f64(V)
    h_q, d = q.shape
    h_kv = K.shape[0]
    g = h_q // h_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((h_q, d), _F)
    lse = np.zeros(h_q, _F)
    for j in range(h_q):
        logits = K[j // g] @ q[j] * scale
        m = logits.max()
        e = np.exp(logits - m)
        s = e.sum()
        o[j] = (e / s) @ V[j // g]
        lse[j] = m + math.log(s)
    return o, lse


def prefill_attention(Q, K, V, ctx, rows=None, scale=None):
    """Causal attention of a prompt chunk over a request's resident tokens.

    Q: [T][h_q][d], the queries of the T new tokens, which sit at positions
    ctx .. ctx+T-1 after the ctx tokens already resident (a shared prefix or
    an earlier chunk). K, V: [h_kv][ctx+T][d], every resident token including
    the new ones. Token i attends to positions 0 .. ctx+i: ordinary causal
    softmax attention, which the paper runs with FlashAttention over the
    paged cache before any eviction (Zipage Sec. 3 and Sec. 6; the prompt may
    exceed the N_max-block cap until its first compression, Sec. 4.1). Each
    row is the decode attention of that token over its causal prefix.
    ``rows`` restricts the computation to some token indices i. Returns
    (O [len(rows)][h_q][d], lse [len(rows)][h_q]).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    T = Q.shape[0]
    rows = range(T) if rows is None else rows
    O, L = [], []
    for i in rows:
        o, lse = decode_attention(Q[i], K[:, :ctx + i + 1], V[:, :ctx + i + 1], scale)
        O.append(o)
        L.append(lse)
    h_q, d = Q.shape[1], Q.shape[2]
    if not O:
        return np.zeros((0, h_q, d), _F), np.zeros((0, h_q), _F)
    return np.stack(O), np.stack(L)


# ---------------------------------------------------------------------------
# Attention score (Zipage App. C.2, Alg. 1)
# ---------------------------------------------------------------------------

def window_logits(Qw, K, b, scale=None):
    """Block attention logits of the observation window, all blocks.

    Qw: [g][w][d] window queries of the g query heads of one kv-head (query u
    sits at position n - w + u, the last w slots of the full last block,
    Zipage Sec. 4.2). K: [n][d] with n = N*b. Follows Alg. 1 block by block:
    A'_i = Qw K_i^T / sqrt(d) of shape [g][w][b]; only the last block gets the
    causal mask, which hides key slot v from query u when v > b - w + u
    (reading: key after query). Returns A: [g][w][N*b] (blocks laid out
    contiguously, as the paper stores A before its softmax).
    """
    Qw, K = _f64(Qw), _f64(K)
    g, w, d = Qw.shape
    n = K.shape[0]
    assert n % b == 0 and n >= b, "compression runs on full blocks only"
    N = n // b
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    A = np.empty((g, w, n), _F)
    for i in range(N):
        Ki = K[i * b:(i + 1) * b]
        Ai = np.einsum("guk,vk->guv", Qw, Ki) * scale
        if i == N - 1:
            u = np.arange(w)[:, None]
            v = np.arange(b)[None, :]
            Ai = np.where(v > b - w + u, -np.inf, Ai)
        A[:, :, i * b:(i + 1) * b] = Ai
    return A


def softmax_last(x):
    """Softmax along the last axis in float64 (max-shifted)."""
    x = _f64(x)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def attention_score(Qw, K, b, scale=None, return_probs=False):
    """S0 of Zipage App. C.2.

    The logits are reshaped to [w][N*b] per query head and normalised with a
    softmax over the sequence; the g query heads sharing a kv-head are
    max-reduced; the result is averaged over the window. S0: [n].
    """
    A = window_logits(Qw, K, b, scale)
    P = softmax_last(A)                 # [g][w][n]
    S0 = P.max(axis=0).mean(axis=0)     # max over the group, mean over window
    return (S0, P) if return_probs else S0


# ---------------------------------------------------------------------------
# Global score (Zipage App. C.3, Alg. 2)
# ---------------------------------------------------------------------------

def global_score(S0, F_old, first_compression, alpha, b, reduce="max"):
    """Decayed reduction with the stored history, block by block (App. C.3,
    Alg. 2).

    A request that was never compressed stores its scores in F unchanged.
    Otherwise every block but the last combines the decayed history with the
    new score, max(alpha * F_old, S) (Alg. 2's max-reduce) or, with
    reduce="sum", alpha * F_old + S (the decayed sum-reduce the appendix
    names beside it), and the result both replaces S and is stored in F; the
    last block (new tokens, no history) stores S as is. Returns (S1, F_new),
    both [n].
    """
    if reduce not in ("max", "sum"):
        raise ValueError(reduce)
    S = _f64(S0).copy()
    n = S.shape[0]
    N = n // b
    F_new = np.empty(n, _F)
    if first_compression:
        F_new[:] = S
        return S, F_new
    F_old = _f64(F_old)
    for i in range(N):
        blk = slice(i * b, (i + 1) * b)
        s = S[blk]
        if i != N - 1:
            if reduce == "max":
                s = np.maximum(alpha * F_old[blk], s)
            else:
                s = alpha * F_old[blk] + s
            S[blk] = s
        F_new[blk] = s
    return S, F_new


# ---------------------------------------------------------------------------
# Pooling along the sequence (Zipage App. C.4, eq. (3))
# ---------------------------------------------------------------------------

def max_pool(S, kernel):
    """Stride-1 max pooling of width ``kernel`` (odd), same-length output.

    Padding behaves like -inf, so the window is clipped at both ends.
    """
    S = _f64(S)
    assert kernel >= 1 and kernel % 2 == 1
    r = kernel // 2
    n = S.shape[0]
    out = np.empty(n, _F)
    for t in range(n):
        out[t] = S[max(0, t - r):min(n, t + r + 1)].max()
    return out


# ---------------------------------------------------------------------------
# Redundancy of key states (Zipage App. C.5 Fig. 11, Alg. 3; App. C.7)
# ---------------------------------------------------------------------------

def _unit_rows(K):
    K = _f64(K)
    nrm = np.sqrt((K * K).sum(axis=-1))
    inv = np.where(nrm > 1e-30, 1.0 / np.where(nrm > 1e-30, nrm, 1.0), 0.0)
    return K * inv[:, None]


def cosine_matrix(Ka, Kb):
    """Cosine similarity of every row of Ka with every row of Kb (0 for a
    zero-norm key)."""
    return _unit_rows(Ka) @ _unit_rows(Kb).T


def _zero_last_above(C, p):
    """In each column, zero the entry of the highest row that exceeds p (the
    newest similar token keeps its similarity, Zipage App. C.5). Modifies C
    in place."""
    above = C > p
    has = above.any(axis=0)
    last = C.shape[0] - 1 - np.argmax(above[::-1, :], axis=0)   # highest row above p
    j = np.nonzero(has)[0]
    C[last[j], j] = 0.0
    return C


def redundancy_rows_original(K, p):
    """Row sums of the full similarity matrix (Zipage App. C.5, Fig. 11).

    Cosine similarity of all n keys with each other, diagonal set to zero,
    then in every column the last entry above p is zeroed (newer tokens are
    favoured); the rows are summed. Returns the un-normalised sums r: [n].
    """
    C = cosine_matrix(K, K)
    np.fill_diagonal(C, 0.0)
    _zero_last_above(C, p)
    return C.sum(axis=1)


def redundancy_rows_flash(K, b, p):
    """Row sums of the flash redundancy (Zipage App. C.5, Alg. 3, Fig. 12).

    Alg. 3 computes the full similarity matrix of Fig. 11 without holding it:
    one column block of b keys at a time, against every row block. Its
    result is the original one: in every column the diagonal and the entry
    of the highest row whose cosine exceeds p (over the whole sequence) are
    zeroed, then rows are summed. Here, per column block m, the n x b cosine
    slab is formed from the b x b blocks, its diagonal entries zeroed, each
    column's highest row above p located and zeroed, and the slab's row sums
    added to r. Returns r: [n].
    """
    K = _f64(K)
    n = K.shape[0]
    N = n // b
    r = np.zeros(n, _F)
    for m in range(N):
        Km = K[m * b:(m + 1) * b]
        slab = np.concatenate([cosine_matrix(K[i * b:(i + 1) * b], Km) for i in range(N)])
        cols = np.arange(b)
        slab[m * b + cols, cols] = 0.0            # k_j against itself
        _zero_last_above(slab, p)
        r += slab.sum(axis=1)
    return r


def redundancy_rows_lightning(K, b, p):
    """Row sums of the lightning redundancy (Zipage App. C.7, Fig. 15).

    Similarity is computed only among keys of the same block; inside each
    b x b block the diagonal is zeroed and each column's last entry above p is
    zeroed, then rows are summed. Returns r: [n].
    """
    K = _f64(K)
    n = K.shape[0]
    r = np.empty(n, _F)
    for i in range(n // b):
        Ki = K[i * b:(i + 1) * b]
        C = cosine_matrix(Ki, Ki)
        np.fill_diagonal(C, 0.0)
        _zero_last_above(C, p)
        r[i * b:(i + 1) * b] = C.sum(axis=1)
    return r


def redundancy_score(r_rows, n, tau):
    """R = softmax_t(r_t / n / tau): length normalisation (App. C.5) and the
    tempered softmax without max-normalisation (App. C.8)."""
    return softmax_last(_f64(r_rows) / n / tau)


# ---------------------------------------------------------------------------
# The whole scoring chain for one (request, layer, kv-head)
# ---------------------------------------------------------------------------

@dataclass
class ScoreParams:
    """Hyper-parameters of the scoring chain.

    Defaults are the configuration Zipage App. C.8 recommends (lambda 0.2,
    tau 0.4, alpha 0.8, pooling at the first compression only) with the
    lightning redundancy (the engine's default). ``p`` and ``pool_kernel``
    are not given by the paper (readings: 0.9 and 7).
    """
    alpha: float = 0.8
    lam: float = 0.2
    tau: float = 0.4
    p: float = 0.9
    pool_kernel: int = 7
    use_global: bool = True
    global_reduce: str = "max"      # or "sum" (App. C.3's decayed sum-reduce)
    use_pool: bool = True
    pool_first_only: bool = True
    use_redundancy: bool = True
    redundancy: str = "lightning"   # or "flash", "original"


def redundancy_rows(K, b, p, variant):
    if variant == "lightning":
        return redundancy_rows_lightning(K, b, p)
    if variant == "flash":
        return redundancy_rows_flash(K, b, p)
    if variant == "original":
        return redundancy_rows_original(K, p)
    raise ValueError(variant)


def score_tokens(Qw, K, F_old, first_compression, b, params: ScoreParams,
                 scale=None, return_parts=False):
    """Final per-token scores of one (request, layer, kv-head).

    Steps, in the paper's order: attention score (App. C.2), global score
    (App. C.3), pooling after the global score (App. C.4), redundancy
    subtracted after pooling, S - lambda R (eq. (4), App. C.5/C.7/C.8), and
    +inf on the observation window (Sec. 4.2, App. C.6). Returns
    (scores [n], F_new [n] or None) and, with ``return_parts``, a dict of the
    intermediate vectors.
    """
    K = _f64(K)
    n = K.shape[0]
    w = np.shape(Qw)[1]
    S0 = attention_score(Qw, K, b, scale)
    F_new = None
    if params.use_global:
        S1, F_new = global_score(S0, F_old, first_compression, params.alpha, b,
                                 params.global_reduce)
    else:
        S1 = S0.copy()
    if params.use_pool and (first_compression or not params.pool_first_only):
        S2 = max_pool(S1, params.pool_kernel)
    else:
        S2 = S1.copy()
    if params.use_redundancy:
        r = redundancy_rows(K, b, params.p, params.redundancy)
        R = redundancy_score(r, n, params.tau)
        S3 = S2 - params.lam * R
    else:
        r = R = None
        S3 = S2.copy()
    S = S3.copy()
    S[n - w:] = np.inf
    if return_parts:
        return S, F_new, dict(S0=S0, S1=S1, S2=S2, r=r, R=R, S3=S3)
    return S, F_new


# ---------------------------------------------------------------------------
# Selection (Zipage Sec. 4.2, App. C.6)
# ---------------------------------------------------------------------------

def topk_keep(S, k):
    """Indices of the k highest scores, returned in ascending order.

    Ties are ordered by index, newer first. (The paper marks the top-k with a
    library routine and does not say how ties fall; this is the reading.)
    """
    S = _f64(S)
    n = S.shape[0]
    assert 0 <= k <= n
    idx = np.arange(n)
    order = np.lexsort((-idx, -S))     # score descending, then index descending
    return np.sort(order[:k]).astype(np.int64)


def topk_tag(S, k):
    """The top-k tag T of App. C.6: 1 for kept tokens, 0 otherwise."""
    T = np.zeros(np.shape(S)[0], np.int8)
    T[topk_keep(S, k)] = 1
    return T


# ---------------------------------------------------------------------------
# Compaction (Zipage App. C.6, Alg. 4; Sec. 4.4 target blocks)
# ---------------------------------------------------------------------------

def compact_pages(pages, src_table, n, dst_table, tag, b):
    """Move the tagged tokens of one request into its target blocks.

    ``pages`` is one (layer, kv-head) slice [num_blocks][b][...] of K, V or
    the global-score cache F (element size d or 1, App. C.6). A read cursor
    walks the n source slots in block-table order and a write cursor walks
    the target blocks, advancing only when the current token is tagged, so the
    kept tokens end up densely packed and in their original order (Alg. 4's
    two-pointer move). Target blocks are the request's own blocks or fresh
    ones (Sec. 4.4). Returns a modified copy of ``pages``.
    """
    out = np.array(pages, copy=True)
    s = 0
    for ell in range(n):
        if tag[ell]:
            src = (src_table[ell // b], ell % b)
            dst = (dst_table[s // b], s % b)
            out[dst] = out[src]
            s += 1
    return out


# ---------------------------------------------------------------------------
# Trigger (Zipage Sec. 4.1)
# ---------------------------------------------------------------------------

def should_compress(n_tokens, b, n_max):
    """True when the request holds N >= N_max blocks and the last is full."""
    N = -(-n_tokens // b)
    return N >= n_max and n_tokens % b == 0 and n_tokens > 0


def window_row(pos, b, w):
    """Row of the query cache that the query at resident position ``pos``
    fills, or -1 if it is not among the last w slots of its block
    (Zipage Sec. 4.2: the observation window is the last w tokens of the final
    block)."""
    off = pos % b
    return off - (b - w) if off >= b - w else -1


# ---------------------------------------------------------------------------
# End-to-end logical simulation of one request (used for the small cases)
# ---------------------------------------------------------------------------

def simulate_request(prompt_K, prompt_V, prompt_Q_tail, steps_q, steps_k, steps_v,
                     b, w, n_max, params: ScoreParams, scale=None, choose=None):
    """Run one request through prompt, decode steps and compressions.

    prompt_K/V: [L][h_kv][n0][d]; prompt_Q_tail: [L][h_q][m][d] with the
    queries of the last m prompt positions, or None (needed only when the
    window falls inside the prompt);
    steps_q: [T][L][h_q][d]; steps_k/v: [T][L][h_kv][d]. Each decode step
    appends k/v to every layer, runs decode attention over the resident tokens
    and records the window query; after every step that leaves N >= N_max full
    blocks the request is compressed to k = (N_max - 1) b tokens per
    (layer, kv-head) (Sec. 4.1). The prompt itself is checked for the trigger
    too (reading: the trigger follows any step that appends KV).

    ``choose(event, layer, head, S, k)``, if given, returns the kept indices
    of that (event, layer, kv-head) from its scores S instead of
    ``topk_keep``. It exists for ties: where several tokens share the k-th
    score within the tie tolerance, several kept sets are equally correct,
    and the caller may continue the simulation from another one of them
    (the caller is responsible for checking that its choice is one).

    Returns dict(outputs [T][L][h_q][d], events: list of per-event dicts with
    the kept indices [L][h_kv][k] and scores [L][h_kv][n], and the final
    resident K, V, F as lists [L][h_kv] of arrays).
    """
    prompt_K, prompt_V = _f64(prompt_K), _f64(prompt_V)
    L, h_kv, n0, d = prompt_K.shape
    T = len(steps_q)
    h_q = np.shape(steps_q)[2] if T else np.shape(prompt_Q_tail)[1]
    g = h_q // h_kv
    cap = n0 + T
    # resident tokens of every (layer, kv-head), in logical order, plus F
    K = np.zeros((L, h_kv, cap, d))
    V = np.zeros((L, h_kv, cap, d))
    F = np.zeros((L, h_kv, cap))
    K[:, :, :n0] = prompt_K
    V[:, :, :n0] = prompt_V
    n = n0
    qwin = np.zeros((L, h_kv, g, w, d), _F)
    if prompt_Q_tail is not None:
        m = np.shape(prompt_Q_tail)[2]
        for pos in range(n0 - m, n0):
            row = window_row(pos, b, w)
            if row >= 0:
                for l in range(L):
                    for j in range(h_q):
                        qwin[l, j // g, j % g, row] = prompt_Q_tail[l][j][pos - (n0 - m)]
    first = True
    events = []
    outputs = np.zeros((T, L, h_q, d), _F)

    def maybe_compress():
        nonlocal first, n
        if not should_compress(n, b, n_max):
            return
        keep = (n_max - 1) * b
        ev = dict(n=n, kept=np.zeros((L, h_kv, keep), np.int64),
                  scores=np.zeros((L, h_kv, n), _F), first=first)
        for l in range(L):
            for h in range(h_kv):
                S, F_new = score_tokens(qwin[l, h], K[l, h, :n], F[l, h, :n], first, b,
                                        params, scale)
                kept = (topk_keep(S, keep) if choose is None
                        else np.asarray(choose(len(events), l, h, S, keep), np.int64))
                ev["kept"][l, h] = kept
                ev["scores"][l, h] = S
                K[l, h, :keep] = K[l, h, kept]
                V[l, h, :keep] = V[l, h, kept]
                F[l, h, :keep] = F_new[kept] if F_new is not None else 0.0
        n = keep
        first = False
        events.append(ev)

    maybe_compress()
    for s in range(T):
        K[:, :, n] = steps_k[s]
        V[:, :, n] = steps_v[s]
        F[:, :, n] = 0.0
        n += 1
        for l in range(L):
            outputs[s, l] = decode_attention(steps_q[s][l], K[l, :, :n], V[l, :, :n], scale)[0]
            row = window_row(n - 1, b, w)
            if row >= 0:
                for j in range(h_q):
                    qwin[l, j // g, j % g, row] = steps_q[s][l][j]
        maybe_compress()
    return dict(outputs=outputs, events=events,
                K=[[K[l, h, :n].copy() for h in range(h_kv)] for l in range(L)],
                V=[[V[l, h, :n].copy() for h in range(h_kv)] for l in range(L)],
                F=[[F[l, h, :n].copy() for h in range(h_kv)] for l in range(L)])
