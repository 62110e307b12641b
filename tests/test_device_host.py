"""Host-side logic of the device driver (no GPU): when a step meets the
contract of paged_append_attn_step (append and attention in one call)."""
import numpy as np

from paged_kv_cache_286_amd.device import append_fusable


def _slots(tables, lens, qlens):
    out = []
    for i, (L, Q) in enumerate(zip(lens, qlens)):
        for pos in range(L - Q, L):
            out.append(int(tables[i, pos // 16]) * 16 + pos % 16)
    return np.array(out, dtype=np.int32)


def test_private_last_blocks_meet_the_contract():
    # blocks 0 and 1 shared by both sequences, each appends into its own block
    t = np.array([[0, 1, 2, -1], [0, 1, 3, -1]])
    assert append_fusable(t, [40, 45], [1, 1], _slots(t, [40, 45], [1, 1]))
    # several rows of one sequence in its own blocks
    assert append_fusable(t, [40, 45], [2, 1], _slots(t, [40, 45], [2, 1]))


def test_an_appended_slot_another_sequence_reads_breaks_it():
    # both tables end in block 2: the second sequence reads the first one's new row
    t = np.array([[0, 1, 2], [0, 1, 2]])
    assert not append_fusable(t, [40, 45], [1, 1], np.array([2 * 16 + 7, 2 * 16 + 12]))
    # a row appended into a prefix block another sequence also holds
    t = np.array([[5, 6, -1], [5, 7, -1]])
    assert not append_fusable(t, [16, 20], [1, 1], np.array([5 * 16 + 15, 7 * 16 + 3]))


def test_a_slot_other_than_the_tables_breaks_it():
    t = np.array([[0, 1, 2, -1], [0, 1, 3, -1]])
    good = _slots(t, [40, 45], [1, 1])
    for bad in ([-1, good[1]], [good[0], good[1] + 1], [good[1], good[0]]):
        assert not append_fusable(t, [40, 45], [1, 1], np.array(bad))
    # one slot per query row, no more, no fewer
    assert not append_fusable(t, [40, 45], [1, 1], good[:1])
    assert not append_fusable(t, [40, 45], [1, 1], np.concatenate([good, good[:1]]))


def _fusable_by_definition(tables, lens, qlens, slots):
    # the contract written out row by row and block by block
    rows = [(s, L - Q + r) for s, (L, Q) in enumerate(zip(lens, qlens)) for r in range(Q)]
    if len(rows) != len(slots) or not rows:
        return False
    reads = {s: [int(b) for b in tables[s][:(L + 15) // 16]] for s, L in enumerate(lens)}
    if any(b < 0 for bs in reads.values() for b in bs):
        return False
    for (s, p), slot in zip(rows, slots):
        b = int(tables[s][p // 16])
        if b < 0 or slot != b * 16 + p % 16:
            return False
        if any(b in reads[t] for t in reads if t != s):
            return False
    return True


def test_fusable_check_matches_its_definition_on_random_steps():
    rng = np.random.default_rng(17)
    for trial in range(300):
        S = int(rng.integers(1, 7))
        lens = rng.integers(1, 70, S)
        qlens = np.minimum(rng.integers(1, 4, S), lens)
        width = int(((lens + 15) // 16).max()) + int(rng.integers(0, 2))
        nb = 24
        tables = np.full((S, width), -1, np.int64)
        for s in range(S):
            n = (int(lens[s]) + 15) // 16
            tables[s, :n] = rng.choice(nb, n, replace=False)
        if rng.random() < 0.4 and S > 1:               # a shared block
            a, b = rng.choice(S, 2, replace=False)
            tables[b, 0] = tables[a, int(rng.integers(0, (lens[a] + 15) // 16))]
        slots = _slots(tables, lens, qlens)
        if rng.random() < 0.2:                          # a wrong slot
            slots[int(rng.integers(0, len(slots)))] += 1
        if rng.random() < 0.1:                          # an invalid entry in use
            tables[0, 0] = -1
        want = _fusable_by_definition(tables, lens.tolist(), qlens.tolist(), slots.tolist())
        assert append_fusable(tables, lens, qlens, slots) == want, trial
