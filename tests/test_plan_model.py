"""Host model of the device plan's slot claiming (plan_count, plan_scan and
plan_scatter in bit_moe_amd/csrc/plan.hip), checked against oracle.moe.plan.

The scatter walks a 64-token chunk in token order; in each step the k lanes of
one token read their expert's next slot from an LDS counter and write it back
plus one, all at once.  That is race-free only if the lanes of a step name
distinct experts.  The model replays those steps, records any two lanes of a
step that share a counter, and marks the perm slots never written.  With the
serving rule of the kernels (an id in [0, E) that does not repeat an earlier
slot of its token) no step has a collision and the perm equals the oracle's;
with the range check alone, a token naming one expert twice makes two lanes
claim one slot and leaves the group's last slot unwritten -- the stale index
the grouped GEMMs would then read and write through."""
import numpy as np

from oracle import moe


def _served(row, j, E):
    e = int(row[j])
    return 0 <= e < E and e not in [int(v) for v in row[:j]]


def _in_range(row, j, E):
    return 0 <= int(row[j]) < E


def claim_slots(ids, E, rule, chunk=64):
    ids = np.asarray(ids)
    T, k = ids.shape
    n_chunks = (T + chunk - 1) // chunk
    # plan_count: per-chunk histogram of the pairs the rule serves
    hist = np.zeros((n_chunks, E), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if rule(ids[t], j, E):
                hist[t // chunk, ids[t, j]] += 1
    # plan_scan: per-expert base of each chunk, exclusive offsets over experts
    counts = hist.sum(0)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    base = np.cumsum(hist, axis=0) - hist
    perm = np.full(int(offsets[-1]), -1, dtype=np.int64)
    collisions = 0
    for c in range(n_chunks):
        s_pos = offsets[:-1] + base[c]
        for t in range(c * chunk, min(T, (c + 1) * chunk)):
            lanes = [j for j in range(k) if rule(ids[t], j, E)]
            reads = {j: int(s_pos[ids[t, j]]) for j in lanes}   # every lane reads ...
            seen = {}
            for j in lanes:
                e = int(ids[t, j])
                collisions += e in seen
                seen[e] = j
            for j in lanes:                                     # ... then every lane writes
                s_pos[ids[t, j]] = reads[j] + 1
                perm[reads[j]] = t * k + j
    return counts, offsets, perm, collisions


def _ids_with_repeats(rng, T, k, E):
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    for t in rng.choice(T, size=max(1, T // 7), replace=False):
        j = int(rng.integers(1, k))
        ids[t, j] = ids[t, int(rng.integers(0, j))]      # a repeat of an earlier slot
    ids[rng.integers(0, T), rng.integers(0, k)] = E + 3  # and one id out of range
    return ids


def test_serving_rule_makes_the_claiming_race_free_and_equal_to_the_oracle():
    rng = np.random.default_rng(0)
    for T, k, E in [(1, 6, 384), (5, 6, 384), (300, 6, 384), (129, 2, 16), (700, 8, 64)]:
        ids = _ids_with_repeats(rng, T, k, E)
        counts, offsets, perm, collisions = claim_slots(ids, E, _served)
        ref = moe.plan(ids, E)
        assert collisions == 0
        assert np.array_equal(counts, ref.counts) and np.array_equal(offsets, ref.offsets)
        assert np.array_equal(perm, ref.perm)


def test_range_check_alone_lets_repeats_collide_and_leaves_stale_slots():
    ids = np.array([[4, 1, 4], [2, 4, 0]])
    counts, offsets, perm, collisions = claim_slots(ids, 5, _in_range)
    assert collisions == 1
    assert counts[4] == 3 and (perm == -1).sum() == 1  # one slot of expert 4's group never written
