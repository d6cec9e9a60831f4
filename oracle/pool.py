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
  * every expert that is some token's top-1 (slot 0) is retained (the ACE
    rule keeps top-1 slots), so the pool can exceed m when the batch has more
    distinct top-1 experts; the remaining places go to the other experts that
    have a kept slot, by S_e descending, lower index first on ties;
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
    """Boolean [E]: the retained experts.  Every top-1 expert (slot 0 of some
    token), then, while the pool holds fewer than m experts, the other
    experts with a kept slot by S_e descending, lower index first."""
    S = pool_scores(idx, gate, keep, E)
    keep = np.asarray(keep, dtype=bool)
    top1 = set(int(e) for e in idx[:, 0]) if idx.shape[0] else set()
    active = set(int(e) for e in np.asarray(idx)[keep])
    others = sorted((e for e in active if e not in top1), key=lambda e: (-float(S[e]), e))
    pool = np.zeros(E, dtype=bool)
    for e in top1:
        pool[e] = True
    for e in others[:max(int(m) - len(top1), 0)]:
        pool[e] = True
    return pool


def cap_expert_pool(idx: np.ndarray, gate: np.ndarray, keep: np.ndarray, E: int, m: int) -> np.ndarray:
    """The keep mask after the cap: kept and retained."""
    pool = expert_pool(idx, gate, keep, E, m)
    return np.asarray(keep, dtype=bool) & pool[np.asarray(idx, dtype=np.int64)]
