"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

This module only draws numbers: it holds none of the method's arithmetic.
Every array is produced on the host with NumPy's PCG64 generator seeded by a
tuple (seed, config, layer, purpose), so the HIP path and the CPU oracle can
be fed identical values. Keys get the "heavy token" pattern of the workloads:
each (layer, kv-head, token) is heavy with probability ``heavy_frac`` and its
key is then multiplied by ``heavy_scale``. For bf16 workloads the values are
rounded to bf16 once here (round to nearest even), so both sides see exactly
the same numbers.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

PURPOSE = {"prompt_k": 1, "prompt_v": 2, "prompt_q": 3, "step_q": 4, "step_k": 5,
           "step_v": 6, "heavy": 7, "gscore": 8, "scores": 9, "lengths": 10, "misc": 11,
           "serve": 12, "serve_stream": 13, "prompt_lengths": 14}


def rng(seed, config, layer, purpose):
    return np.random.default_rng([int(seed), int(config), int(layer), PURPOSE[purpose]])


def round_bf16(x):
    """Rounds float32 values to the nearest bf16 (ties to even), returned as
    float32. Pure integer manipulation of the bit pattern."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    out = r.view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = np.where(nan, np.float32(np.nan), out)
    return out


def cast(x, dtype):
    return round_bf16(x) if dtype == "bf16" else np.asarray(x, np.float32)


@dataclass
class RequestInputs:
    prompt_k: np.ndarray   # [L][h_kv][n0][d]
    prompt_v: np.ndarray   # [L][h_kv][n0][d]
    prompt_q: np.ndarray   # [L][h_q][m][d]: queries of the last m prompt positions, or None
    steps_q: np.ndarray    # [T][L][h_q][d]
    steps_k: np.ndarray    # [T][L][h_kv][d]
    steps_v: np.ndarray    # [T][L][h_kv][d]


def request_inputs(seed, config, L, h_q, h_kv, d, n_prompt, n_steps, dtype="f32",
                   heavy_frac=0.02, heavy_scale=4.0, prompt_q_last=0):
    """Q/K/V ~ N(0, 1) for one request: its prompt and its decode steps.

    ``prompt_q_last`` = m > 0 also draws queries for the last m prompt
    positions (the observation window when compression fires right after the
    prompt), shaped [L][h_q][m][d].
    """
    pk = np.empty((L, h_kv, n_prompt, d), np.float32)
    pv = np.empty_like(pk)
    m = min(prompt_q_last, n_prompt)
    pq = np.zeros((L, h_q, m, d), np.float32) if prompt_q_last else None
    sq = np.empty((n_steps, L, h_q, d), np.float32)
    sk = np.empty((n_steps, L, h_kv, d), np.float32)
    sv = np.empty_like(sk)
    for l in range(L):
        pk[l] = rng(seed, config, l, "prompt_k").standard_normal((h_kv, n_prompt, d))
        pv[l] = rng(seed, config, l, "prompt_v").standard_normal((h_kv, n_prompt, d))
        hv = rng(seed, config, l, "heavy").random((h_kv, n_prompt + n_steps)) < heavy_frac
        pk[l] *= np.where(hv[:, :n_prompt], heavy_scale, 1.0)[..., None]
        if prompt_q_last:
            pq[l] = rng(seed, config, l, "prompt_q").standard_normal((h_q, m, d))
        sq[:, l] = rng(seed, config, l, "step_q").standard_normal((n_steps, h_q, d))
        sk[:, l] = rng(seed, config, l, "step_k").standard_normal((n_steps, h_kv, d))
        sv[:, l] = rng(seed, config, l, "step_v").standard_normal((n_steps, h_kv, d))
        sk[:, l] *= np.where(hv[:, n_prompt:].T, heavy_scale, 1.0)[..., None]
    c = lambda a: None if a is None else cast(a, dtype)
    return RequestInputs(c(pk), c(pv), c(pq), c(sq), c(sk), c(sv))


def scores_with_ties(seed, config, n, n_window, levels=None):
    """fp32 score vectors for selection tests: either continuous values or a
    few discrete levels (many exact ties), with +inf on the last n_window."""
    g = rng(seed, config, 0, "scores")
    if levels:
        s = g.integers(0, levels, n).astype(np.float32) * np.float32(0.125)
    else:
        s = g.random(n).astype(np.float32)
    s[n - n_window:] = np.inf
    return s


def log_uniform_lengths(seed, config, count, lo, hi):
    """Prompt lengths drawn log-uniformly in [lo, hi]."""
    g = rng(seed, config, 0, "lengths")
    return np.floor(np.exp(g.uniform(np.log(lo), np.log(hi), count))).astype(np.int64)
