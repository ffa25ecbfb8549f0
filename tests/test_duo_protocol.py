"""CPU model check of the two-workgroup form's protocol (the producer and the
consumer workgroup of one (sequence, head) pair, gated_delta_rule_tok_amd/
csrc/kda_duo.hip).

Producer workgroup: ten producer waves fill five single-buffered chunk slots
in LDS (two halves a chunk); two copy waves (even and odd chunks) copy each
finished package into the pair's ring of RING packages in global memory and
publish the count of their chunks.  Consumer workgroup: two loader waves (even
and odd chunks) load each published package into an LDS ring of two buffers
of four slots and acknowledge it; the state waves read the packages in chunk
order.  Counters and flags:

  half[c], rdy[c]   producer halves of slot c past their first phase / done
  copied[c]         packages copied out of producer slot c
  pub[p], ack[p]    (nonce, count) flag words in global memory: chunks of
                    parity p published by its copy wave / loaded by its loader
  lrdy[b][c]        packages loaded into consumer slot (b, c)
  done[c][s]        rounds state wave s is done with on consumer slot c

This test runs the same waits and counts as Python generators under random
interleavings, over consecutive calls that share the ring and the flag words
(flag words holding garbage before the first call; the same nonce twice, as a
replayed graph does), and checks that every state wave reads every chunk of
its call complete and in order, that no slot (LDS or ring) is overwritten
while it is read, that a package is loaded only once its stores are complete,
that every run ends, that planted mistakes are caught, and that a wait which
gives up lets every wave finish with the error recorded.
"""
from __future__ import annotations

import random

import pytest

SLOTS, HALVES, COPY, ROUND = 5, 2, 2, 4


class Violation(Exception):
    pass


def run(nc_per_call, nsw: int, seed: int, nonces, ring: int = 4, bug: str | None = None,
        spin: int | None = None) -> int:
    """Consecutive calls (chunk count and nonce each) of one pair under one
    random interleaving per call; returns the error flag of the last call."""
    rng = random.Random(seed)
    # global memory, kept across calls: ring slots (call, chunk, complete)
    # and the four flag words, which start as garbage
    gring = {i: (-1, -1, True) for i in range(ring)}
    flags = {k: (rng.randrange(1, 1 << 16) + 1000, rng.randrange(0, 50))
             for k in ("pub0", "pub1", "ack0", "ack1")}
    err = 0
    for call, (nc, nonce) in enumerate(zip(nc_per_call, nonces)):
        err = _one_call(call, nc, nonce, nsw, rng, gring, flags, ring, bug, spin)
    return err


def _one_call(call, nc, nonce, nsw, rng, gring, flags, ring, bug, spin):
    st = {"err": 0}

    def fail(msg):
        if not st["err"]:  # after a give-up the results are void
            raise Violation(f"call {call}: {msg}")

    def wait(cond):
        if st["err"]:
            return
        it = 0
        while not cond():
            it += 1
            if spin is not None and it > spin:
                st["err"] = 1
                return
            yield "blocked"

    def flag_count(word, nonce_):
        n, cnt = flags[word]
        return cnt if n == nonce_ else -1

    # producer workgroup LDS
    pk = {(c, hf): (-1, False) for c in range(SLOTS) for hf in range(HALVES)}
    kg = {(c, hf): -1 for c in range(SLOTS) for hf in range(HALVES)}
    half = [0] * SLOTS
    rdy = [0] * SLOTS
    copied = [0] * SLOTS
    copy_reading = {}
    kg_reading = {}
    # consumer workgroup LDS
    lpk = {(b, c): (-1, -1) for b in range(2) for c in range(ROUND)}
    lrdy = [[0] * ROUND for _ in range(2)]
    done = [[0] * nsw for _ in range(ROUND)]
    state_reading = {}
    ring_reading = {}

    def producer(c, hf):
        r = 0
        while SLOTS * r + c < nc:
            j = SLOTS * r + c
            if r >= 1:
                tgt = r - 1 if bug == "early_overwrite" else r
                yield from wait(lambda: copied[c] >= tgt)
            if copy_reading.get(c) not in (None, j):
                fail(f"producer slot {c} overwritten with chunk {j} while chunk {copy_reading[c]} is copied")
            for h_j in kg_reading.get(c, set()):
                if h_j[1] != j:
                    fail(f"kg of slot {c} overwritten while half {h_j[0]} reads chunk {h_j[1]}")
            pk[(c, hf)] = (j, False)
            kg[(c, hf)] = j
            yield "run"
            half[c] += 1
            yield "run"
            yield from wait(lambda: half[c] >= HALVES * (r + 1))
            kg_reading.setdefault(c, set()).add((hf, j))
            for h in range(HALVES):
                if kg[(c, h)] != j:
                    fail(f"half {hf} of chunk {j} reads kg of chunk {kg[(c, h)]}")
            yield "run"
            kg_reading[c].discard((hf, j))
            pk[(c, hf)] = (j, True)
            yield "run"
            rdy[c] += 1
            yield "run"
            r += 1

    def copier(cw):
        acked = 0
        for j in range(cw, nc, COPY):
            c, r = j % SLOTS, j // SLOTS
            tgt = HALVES * (r + 1) - (1 if bug == "early_copy" else 0)
            yield from wait(lambda: rdy[c] >= tgt)
            need = (j - ring) // COPY + 1
            if j >= ring and acked < need and bug != "ring_overrun":
                yield from wait(lambda: flag_count(f"ack{cw}", nonce) >= need)
                acked = max(acked, flag_count(f"ack{cw}", nonce))
            copy_reading[c] = j
            for hf in range(HALVES):
                if pk[(c, hf)] != (j, True):
                    fail(f"copy of chunk {j} reads slot {c} half {hf} holding {pk[(c, hf)]}")
            yield "run"
            for hf in range(HALVES):
                if pk[(c, hf)] != (j, True):
                    fail(f"slot {c} changed while chunk {j} is copied")
            copy_reading.pop(c, None)
            copied[c] += 1
            slot = j % ring
            if ring_reading.get(slot) not in (None, (call, j)):
                fail(f"ring slot {slot} overwritten with chunk {j} while {ring_reading[slot]} is loaded")
            gring[slot] = (call, j, False)  # stores issued
            if bug == "early_publish":
                flags[f"pub{cw}"] = (nonce, j // COPY + 1)
            yield "run"
            gring[slot] = (call, j, True)   # the stores complete (vmcnt)
            yield "run"
            flags[f"pub{cw}"] = (nonce, j // COPY + 1)
            yield "run"

    def loader(lw):
        known = 0
        for j in range(lw, nc, COPY):
            r, c = j // ROUND, j % ROUND
            b = r & 1
            if r >= 2:
                tgt = r - 2 if bug == "lds_overrun" else r - 1
                yield from wait(lambda: min(done[c]) >= tgt)
            need = j // COPY + 1
            if known < need:
                yield from wait(lambda: flag_count(f"pub{lw}", nonce) >= need)
                known = max(known, flag_count(f"pub{lw}", nonce))
            slot = j % ring
            ring_reading[slot] = (call, j)
            if gring[slot] != (call, j, True):
                fail(f"loader {lw} loads chunk {j} from ring slot {slot} holding {gring[slot]}")
            for s_j in state_reading.get((b, c), set()):
                if s_j[1] != j:
                    fail(f"LDS slot {(b, c)} overwritten with chunk {j} while wave {s_j[0]} reads chunk {s_j[1]}")
            lpk[(b, c)] = (call, j)
            yield "run"
            if gring[slot] != (call, j, True):
                fail(f"ring slot {slot} changed while chunk {j} is loaded")
            ring_reading.pop(slot, None)
            lrdy[b][c] += 1
            yield "run"
            flags[f"ack{lw}"] = (nonce, j // COPY + 1)
            yield "run"
        if bug != "no_clear":
            flags[f"pub{lw}"] = (0, 0)
            flags[f"ack{lw}"] = (0, 0)

    def state(s):
        r = 0
        while ROUND * r < nc:
            b = r & 1
            for c in range(ROUND):
                j = ROUND * r + c
                if j >= nc:
                    break
                tgt = (r >> 1) + 1 - (1 if bug == "early_state" else 0)
                yield from wait(lambda: lrdy[b][c] >= tgt)
                state_reading.setdefault((b, c), set()).add((s, j))
                if lpk[(b, c)] != (call, j):
                    fail(f"state wave {s} reads chunk {j} from LDS slot {(b, c)} holding {lpk[(b, c)]}")
                yield "run"
                if lpk[(b, c)] != (call, j):
                    fail(f"LDS slot {(b, c)} changed under state wave {s} at chunk {j}")
                state_reading[(b, c)].discard((s, j))
                done[c][s] += 1
                yield "run"
            r += 1

    waves = ([producer(c, hf) for hf in range(HALVES) for c in range(SLOTS)]
             + [copier(cw) for cw in range(COPY)] + [loader(lw) for lw in range(COPY)]
             + [state(s) for s in range(nsw)])
    live = list(range(len(waves)))
    blocked = 0
    while live:
        i = rng.choice(live)
        try:
            ev = next(waves[i])
        except StopIteration:
            live.remove(i)
            blocked = 0
            continue
        if ev == "blocked":
            blocked += 1
            if blocked > 50 * len(live) + 2000:
                raise Violation(f"call {call}: deadlock")
        else:
            blocked = 0
    return st["err"]


@pytest.mark.parametrize("nsw", [1, 2, 8])
def test_protocol_is_safe_and_ends(nsw):
    """Chunk counts 0..23 and longer runs that wrap both rings many times, in
    pairs of calls with distinct nonces and with the same nonce (a replayed
    graph), after garbage flag words."""
    for nc in list(range(0, 24)) + [37, 64]:
        for seed in range(3):
            run([nc, nc], nsw, seed, nonces=[77, 78])
            run([nc, (nc * 7) % 29], nsw, seed + 10, nonces=[5, 5])


@pytest.mark.parametrize("ring", [2, 4, 8])
def test_ring_sizes(ring):
    for nc in (1, 2, 9, 30):
        for seed in range(4):
            run([nc, nc], 2, seed, nonces=[3, 3], ring=ring)


@pytest.mark.parametrize("bug,nonces", [("early_copy", [1, 2]), ("ring_overrun", [1, 2]),
                                        ("early_publish", [1, 2]), ("lds_overrun", [1, 2]),
                                        ("early_state", [1, 2]), ("early_overwrite", [1, 2]),
                                        ("no_clear", [4, 4])])
def test_planted_mistakes_are_caught(bug, nonces):
    caught = 0
    for seed in range(40):
        try:
            run([24, 24], 2, seed, nonces=nonces, bug=bug)
        except Violation:
            caught += 1
    assert caught > 0, f"the model does not catch the planted mistake {bug}"


def test_give_up_ends_every_wave():
    """With a tiny poll bound some wait gives up: every wave still finishes
    (later waits return at once) and the error is recorded."""
    seen = 0
    for seed in range(20):
        seen += run([24], 2, seed, nonces=[9], spin=2)
    assert seen > 0
