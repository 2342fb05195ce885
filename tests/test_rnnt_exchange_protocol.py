"""CPU: the clustered RNNT decoder's exchange protocol, checked over every interleaving.

Each of G cluster members, at step s = 1, 2, ..., writes its word (tagged s) into slot
s % 2 of its own column, then reads every member's word of that step, waiting while a
word carries an older tag. The decoder relies on two facts that this exhaustive search
over all interleavings of small clusters confirms: a reader never finds a word already
overwritten by step s + 2 (a member is never two steps ahead of another), and the protocol
never deadlocks (some member can always move until all are done). The search also shows
that a single slot would not do: with one slot a fast member overwrites a word that a slow
one has not read yet."""
from collections import deque

import pytest


def explore(G, steps, slots):
    # member state: (step, read_mask); step == steps + 1 means done; read_mask None means
    # "still has to write this step's word"
    start = (tuple((1, None) for _ in range(G)), tuple((0,) * G for _ in range(slots)))
    seen, todo = {start}, deque([start])
    overwritten = False
    while todo:
        members, mem = todo.popleft()
        moves = []
        for m, (s, mask) in enumerate(members):
            if s > steps:
                continue
            slot = s % slots
            if mask is None:                         # write: tag s into slot, own column
                row = list(mem[slot])
                row[m] = s
                nm = list(mem)
                nm[slot] = tuple(row)
                nmem = list(members)
                nmem[m] = (s, 0)
                moves.append((tuple(nmem), tuple(nm)))
                continue
            for p in range(G):                       # read peer p's word of step s
                if mask >> p & 1:
                    continue
                tag = mem[slot][p]
                if tag > s:
                    overwritten = True
                if tag == s:
                    nmask = mask | 1 << p
                    nmem = list(members)
                    nmem[m] = (s + 1, None) if nmask == (1 << G) - 1 else (s, nmask)
                    moves.append((tuple(nmem), mem))
        if not moves and any(s <= steps for s, _ in members):
            return "deadlock", overwritten
        for st in moves:
            if st not in seen:
                seen.add(st)
                todo.append(st)
    return "done", overwritten


@pytest.mark.parametrize("G,steps", [(2, 5), (3, 4), (4, 3)])
def test_two_parity_slots_never_lose_a_word_and_never_deadlock(G, steps):
    end, overwritten = explore(G, steps, slots=2)
    assert end == "done" and not overwritten


def test_one_slot_would_lose_words():
    end, overwritten = explore(2, 3, slots=1)
    assert overwritten
