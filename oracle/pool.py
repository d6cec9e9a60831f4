"""Oracle for the batch-level decode expert-pool cap (test infrastructure).

Source: "ExFold: Unified Expert Folding for Training-Free MoE Prefill-Decode
Acceleration" (listing page), abstract: decode is bound by the memory traffic
of the expert set a batch activates, and decode acceleration retains a pool of
at most m experts per batch ("D m", Tables 1 and 6; retained experts ranked by
a score S_i, Table 5).  The folding of excluded experts into retained ones
needs calibrated projectors and is not part of this function.

Readings where the page is silent (also listed in the design notes):
  * S_e = the sum of the gates of the batch's kept slots routed to e,
    accumulated in float32 in slot order (t ascending, then i), the same
    precision and order as the kernel, since it decides an integer ranking;
  * every expert that is some token's top-1 is retained (the ACE rule keeps
    top-1 slots), so the pool holds max(m, #distinct top-1 experts) experts:
    top-1 experts first, then by S_e descending, lower index first on ties;
  * a kept slot whose expert is outside the pool is skipped; nothing is
    folded or renormalised.

Pins (tests/test_oracle_pool.py): brute force over all pools on tiny cases,
m >= #active experts is the identity, top-1 slots stay kept, the active set
never exceeds max(m, #top-1 experts), nesting in m, and a hand-worked case.
"""
from __future__ import annotations

import numpy as np


def pool_scores(idx: np.ndarray, gate: np.ndarray, keep: np.ndarray, E: int) -> np.ndarray:
    """S_e over the batch: float32, slots in order."""
    S = np.zeros(E, dtype=np.float32)
    T, k = idx.shape
    for t in range(T):
        for i in range(k):
            if keep[t, i]:
                e = int(idx[t, i])
                S[e] = np.float32(S[e] + np.float32(gate[t, i]))
    return S


def expert_pool(idx: np.ndarray, gate: np.ndarray, keep: np.ndarray, E: int, m: int) -> np.ndarray:
    """Boolean [E]: the retained experts."""
    S = pool_scores(idx, gate, keep, E)
    top1 = set(int(e) for e in idx[:, 0]) if idx.shape[0] else set()
    order = sorted(range(E), key=lambda e: (e not in top1, -float(S[e]), e))
    size = max(int(m), len(top1))
    pool = np.zeros(E, dtype=bool)
    pool[order[:size]] = True
    return pool


def cap_expert_pool(idx: np.ndarray, gate: np.ndarray, keep: np.ndarray, E: int, m: int) -> np.ndarray:
    """The keep mask after the cap: kept and retained."""
    pool = expert_pool(idx, gate, keep, E, m)
    return np.asarray(keep, dtype=bool) & pool[np.asarray(idx, dtype=np.int64)]
