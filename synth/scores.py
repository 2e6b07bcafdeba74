"""Seeded page-score arrays with hard tie structure, for tests of the page
select on given scores.  Only random draws and placements: no part of the
method's arithmetic."""
from __future__ import annotations

import numpy as np


def tie_scores(seed: int, batch: int, n_kv_heads: int, max_pages: int, n_pages, keep) -> np.ndarray:
    """fp64 scores [batch][n_kv_heads][max_pages] (0 past n_pages[b]).  Each (b, h) draws background
    scores in [-2, 2] and a cluster, at random pages, whose values straddle the keep boundary, cycling
    through these cluster kinds by (b * n_kv_heads + h) mod 5:
      0: 300 distinct fp64 values that all round to the same fp32 value;
      1: 200 copies of one fp64 value;
      2: 40 distinct fp64 values that round to one fp32 value;
      3: signed zeros and values of the smallest magnitudes (denormals included);
      4: every score equal.
    Above the cluster sit keep[b] - (cluster size) / 2 larger distinct scores, so the keep boundary falls
    inside it."""
    rng = np.random.default_rng(seed)
    out = np.zeros((batch, n_kv_heads, max_pages), np.float64)
    tiny = np.array([0.0, -0.0, 5e-324, -5e-324, 1e-310, -1e-310, 1e-300, -1e-300])
    for b in range(batch):
        NP = int(n_pages[b])
        kp = int(keep[b])
        for h in range(n_kv_heads):
            kind = (b * n_kv_heads + h) % 5
            if kind == 0:
                c = 3.0 + np.arange(300) * 2.0 ** -40
            elif kind == 1:
                c = np.full(200, 3.0)
            elif kind == 2:
                c = 3.0 + np.arange(40) * 2.0 ** -38
            elif kind == 3:
                c = np.concatenate([tiny, np.full(80, 0.0), np.full(80, -0.0)])
            else:
                c = np.full(NP, 1.0)
            c = c[:NP]
            n_top = min(max(kp - len(c) // 2, 0), NP - len(c))
            s = rng.uniform(-2.0, 2.0, NP) if kind != 3 else rng.uniform(-2.0, -1.0, NP)
            perm = rng.permutation(NP)
            s[perm[:n_top]] = 10.0 + rng.uniform(0.0, 1.0, n_top)
            s[perm[n_top:n_top + len(c)]] = rng.permutation(c)
            out[b, h, :NP] = s
    return out
