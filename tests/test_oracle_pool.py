"""Pins of the decode expert-pool cap oracle ("ExFold: Unified Expert Folding
for Training-Free MoE Prefill-Decode Acceleration", abstract and Tables 1, 5, 6)."""
import itertools

import numpy as np

import oracle


def _batch(rng, T, E, k, skip=0.4):
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    gate = rng.dirichlet(np.ones(k), size=T).astype(np.float32)
    gate = -np.sort(-gate, axis=1)
    keep = rng.random((T, k)) > skip
    keep[:, 0] = True
    return idx, gate, keep


def test_hand_case():
    # two tokens, E = 5, k = 2.  Top-1 experts {0, 3}; other kept slots go to
    # 1 (gate 0.3) and 4 (gate 0.4).  m = 3: pool = {0, 3} + the larger of
    # S_1 = 0.3, S_4 = 0.4 -> {0, 3, 4}; the slot to expert 1 is skipped.
    idx = np.array([[0, 1], [3, 4]], dtype=np.int32)
    gate = np.array([[0.7, 0.3], [0.6, 0.4]], dtype=np.float32)
    keep = np.ones((2, 2), dtype=bool)
    assert oracle.expert_pool(idx, gate, keep, 5, 3).tolist() == [True, False, False, True, True]
    assert oracle.cap_expert_pool(idx, gate, keep, 5, 3).tolist() == [[True, False], [True, True]]
    # m below the number of top-1 experts: the top-1 experts alone
    assert oracle.cap_expert_pool(idx, gate, keep, 5, 1).tolist() == [[True, False], [True, False]]
    # equal scores: the lower index wins
    gate2 = np.array([[0.6, 0.4], [0.6, 0.4]], dtype=np.float32)
    assert oracle.expert_pool(idx, gate2, keep, 5, 3).tolist() == [True, True, False, True, False]
    # a top-1 expert counts even when its slot is not kept; experts without a
    # kept slot never take a place
    keep2 = np.array([[False, True], [True, False]])
    assert oracle.expert_pool(idx, gate, keep2, 5, 3).tolist() == [True, True, False, True, False]


def test_brute_force_best_pool():
    """Among all pools made of every top-1 expert plus the allowed number of
    other experts with a kept slot, the chosen one maximises the retained
    gate mass (float32 scores), lower indices first on equal mass; the kept
    slots are exactly those inside it."""
    rng = np.random.default_rng(3)
    for trial in range(40):
        T, E, k = int(rng.integers(1, 5)), int(rng.integers(3, 8)), 2
        idx, gate, keep = _batch(rng, T, E, k)
        m = int(rng.integers(1, E + 1))
        S = oracle.pool_scores(idx, gate, keep, E)
        top1 = set(idx[:, 0].tolist())
        cands = sorted(set(idx[keep].tolist()) - top1)
        extra = min(max(m - len(top1), 0), len(cands))
        best = None
        for c in itertools.combinations(cands, extra):
            mass = sum(float(S[e]) for e in c)
            key = (mass, [-e for e in c])
            if best is None or key > best[0]:
                best = (key, set(c) | top1)
        pool = oracle.expert_pool(idx, gate, keep, E, m)
        assert set(np.flatnonzero(pool).tolist()) == best[1]
        new = oracle.cap_expert_pool(idx, gate, keep, E, m)
        assert np.array_equal(new, keep & pool[idx])


def test_invariants():
    rng = np.random.default_rng(4)
    T, E, k = 16, 32, 4
    idx, gate, keep = _batch(rng, T, E, k)
    active = set(idx[keep].tolist())
    top1 = set(idx[:, 0].tolist())
    prev = None
    for m in range(1, E + 1):
        new = oracle.cap_expert_pool(idx, gate, keep, E, m)
        assert new[:, 0].all()                       # top-1 slots stay kept
        assert not (new & ~keep).any()               # nothing skipped comes back
        assert len(set(idx[new].tolist())) <= max(m, len(top1))
        if prev is not None:
            assert not (prev & ~new).any()           # nesting: a larger pool keeps a superset
        prev = new
        if m >= len(active):
            assert np.array_equal(new, keep)         # no cap when the pool holds every active expert


def test_scores_follow_slot_order_in_float32():
    idx = np.array([[2, 1], [2, 0], [2, 1]], dtype=np.int32)
    gate = np.array([[0.1, 0.2], [np.float32(1e8), 0.3], [np.float32(-1e8), 0.4]], dtype=np.float32)
    keep = np.ones((3, 2), dtype=bool)
    S = oracle.pool_scores(idx, gate, keep, 3)
    # ((0.1 + 1e8) + -1e8) in float32 loses the 0.1
    assert S[2] == np.float32(np.float32(np.float32(0.1) + np.float32(1e8)) - np.float32(1e8))
