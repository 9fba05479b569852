"""Acceptance of a kept-token set against the oracle's scores, under the tie
rule of the parity bar (kept sets bit-exact except at score ties within 1e-6
relative).

Let S be the oracle's final scores of one (request, layer, kv-head)
(float64, +inf on the window) and s_k its k-th largest value. The tie zone is
every token t with |S[t] - s_k| <= 1e-6 |s_k|. A kept set is accepted when it
holds exactly k distinct indices in [0, n), contains every token scoring
above the zone and none scoring below it. Tokens inside the zone are
interchangeable: any k - #above of them may be kept. An accepted set is
therefore one of the top-k sets of S under that tolerance, and the oracle's
simulation may continue from it (the Zipage paper marks the top-k with a
library routine and says nothing of ties, App. C.6).

Pure NumPy; no part of the method is computed here.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from oracle import zipage as Z

TIE_REL = 1e-6


@dataclass
class KeptCheck:
    ok: bool             # the set is a valid top-k of S under the tie zone
    same: bool           # the set equals the oracle's own top-k (tie rule: newer first)
    n_diff: int          # tokens in exactly one of the two sets
    max_rel: float       # largest |S - s_k| / |s_k| over those tokens (0 if none)
    n_zone: int          # tokens inside the tie zone
    n_above_missing: int # tokens above the zone that the set lacks
    n_below_taken: int   # tokens below the zone that the set holds
    s_k: float

    def describe(self):
        return (f"{self.n_diff} tokens differ (max |S-s_k|/|s_k| {self.max_rel:.2e}), "
                f"zone {self.n_zone}, above-zone missing {self.n_above_missing}, "
                f"below-zone taken {self.n_below_taken}, s_k {self.s_k:.6e}")


def check_kept(kept, S, k, rel=TIE_REL) -> KeptCheck:
    S = np.asarray(S, np.float64)
    n = S.shape[0]
    kept = np.asarray(kept).astype(np.int64).reshape(-1)
    uniq = np.unique(kept)
    if len(kept) != k or len(uniq) != k or (k and (uniq[0] < 0 or uniq[-1] >= n)):
        return KeptCheck(False, False, -1, np.inf, 0, 0, 0, np.nan)
    sk = np.sort(S)[::-1][k - 1]
    if np.isinf(sk):
        above, below = np.zeros(n, bool), S < sk
    else:
        delta = rel * abs(sk)
        above, below = S > sk + delta, S < sk - delta
    zone = ~above & ~below
    g = np.zeros(n, bool)
    g[kept] = True
    r = np.zeros(n, bool)
    r[Z.topk_keep(S, k)] = True
    diff = g != r
    rel_d = np.abs(S[diff] - sk) / abs(sk) if diff.any() and np.isfinite(sk) and sk != 0 else []
    missing = int(np.sum(above & ~g))
    taken = int(np.sum(below & g))
    return KeptCheck(ok=missing == 0 and taken == 0, same=not diff.any(), n_diff=int(diff.sum()),
                     max_rel=float(np.max(rel_d)) if len(rel_d) else 0.0,
                     n_zone=int(zone.sum()), n_above_missing=missing, n_below_taken=taken,
                     s_k=float(sk))
