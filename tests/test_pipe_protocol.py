"""CPU model check of the LDS counter protocol of the pipelined chunk kernel.

The kernel (gated_delta_rule_tok_amd/csrc/kda_pipe.hip) has no workgroup
barrier in its main loops.  Eight producer waves (two channel halves for each
of four chunk slots) fill double-buffered packages; the state waves read them
in chunk order.  Three kinds of LDS counters order them:

  done[c][s]  chunks of slot c that state wave s has finished (one 16-byte row,
              polled by a producer before it overwrites a buffer of slot c);
  half[c]     producer halves of slot c that formed their first-phase operands
              (the second phase of a round waits for both halves);
  rdy[b][c]   producer halves that finished their package part on buffer b of
              slot c (a state wave waits for both halves of its round).

This test runs the same waits and counts as Python generators under random
interleavings and checks that no wave reads a buffer that is incomplete or
from another round, that no producer overwrites what a wave still reads, that
the run always ends, that planted off-by-one mistakes are caught, and that
a wait which gives up (a bound on the number of polls) lets every wave finish
with the error recorded.
"""
from __future__ import annotations

import random

import pytest

KPW, KPH = 4, 2


class Violation(Exception):
    pass


def run(nc: int, nsw: int, seed: int, bug: str | None = None, spin: int | None = None) -> int:
    """One random interleaving of the protocol for nc chunks and nsw state waves;
    returns the error flag (a wait gave up after spin polls)."""
    st = {"err": 0}

    def fail(msg):
        # after a give-up the results are void: only the ending is checked
        if not st["err"]:
            raise Violation(msg)
    nr = (nc + KPW - 1) // KPW
    done = [[0] * 4 for _ in range(KPW)]
    half = [0] * KPW
    rdy = [[0] * KPW for _ in range(2)]
    # content of each buffer part: (round, complete) per producer half;
    # kg scratch of each buffer: round and which halves have read it
    pkg = {(b, c, hf): (-1, False) for b in range(2) for c in range(KPW) for hf in range(KPH)}
    kg = {(b, c, hf): -1 for b in range(2) for c in range(KPW) for hf in range(KPH)}
    reading = {}  # (b, c) -> set of (state wave, round) reading it now
    kg_reading = {}  # (b, c) -> set of (half, round) reading kg now

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

    def producer(c, hf):
        for r in range(nr):
            j = KPW * r + c
            if j >= nc:
                break
            b = r & 1
            if r >= 2:
                tgt = r - 2 if bug == "early_overwrite" else r - 1
                yield from wait(lambda: min(done[c][:nsw]) >= tgt)
            # first phase: this half's operands of round r, and its kg part
            for s_r in reading.get((b, c), set()):
                if s_r[1] != r:
                    fail(f"slot {c} buffer {b}: overwritten (round {r}) while wave {s_r[0]} reads round {s_r[1]}")
            pkg[(b, c, hf)] = (r, False)
            yield "run"
            for h_r in kg_reading.get((b, c), set()):
                if h_r[1] != r:
                    fail(f"slot {c} buffer {b}: kg overwritten while half {h_r[0]} reads round {h_r[1]}")
            kg[(b, c, hf)] = r
            yield "run"
            half[c] += 1
            yield "run"
            tgt = KPH * (r + 1) - (1 if bug == "early_half" else 0)
            yield from wait(lambda: half[c] >= tgt)
            # second phase: read both halves' kg, finish the package part
            kg_reading.setdefault((b, c), set()).add((hf, r))
            for h in range(KPH):
                if kg[(b, c, h)] != r:
                    fail(f"slot {c} buffer {b}: half {hf} reads kg of round {kg[(b, c, h)]} for round {r}")
            yield "run"
            for h in range(KPH):
                if kg[(b, c, h)] != r:
                    fail(f"slot {c} buffer {b}: kg changed under half {hf} in round {r}")
            kg_reading[(b, c)].discard((hf, r))
            pkg[(b, c, hf)] = (r, True)
            yield "run"
            rdy[b][c] += 1
            yield "run"

    def state(s):
        for r in range(nr):
            b = r & 1
            for c in range(KPW):
                j = KPW * r + c
                if j >= nc:
                    break
                tgt = KPH * ((r >> 1) + 1) - (1 if bug == "early_read" else 0)
                yield from wait(lambda: rdy[b][c] >= tgt)
                reading.setdefault((b, c), set()).add((s, r))
                for hf in range(KPH):
                    if pkg[(b, c, hf)] != (r, True):
                        fail(f"wave {s} reads slot {c} buffer {b} for round {r}: half {hf} holds {pkg[(b, c, hf)]}")
                yield "run"
                for hf in range(KPH):
                    if pkg[(b, c, hf)] != (r, True):
                        fail(f"slot {c} buffer {b} changed under wave {s} in round {r}")
                reading[(b, c)].discard((s, r))
                done[c][s] += 1
                yield "run"

    rng = random.Random(seed)
    waves = [producer(c, hf) for hf in range(KPH) for c in range(KPW)] + [state(s) for s in range(nsw)]
    live = list(range(len(waves)))
    blocked_rounds = 0
    while live:
        i = rng.choice(live)
        try:
            ev = next(waves[i])
        except StopIteration:
            live.remove(i)
            blocked_rounds = 0
            continue
        if ev == "blocked":
            blocked_rounds += 1
            if blocked_rounds > 50 * len(live) + 1000:
                # every live wave has been polled many times without progress
                raise Violation("deadlock")
        else:
            blocked_rounds = 0
    return st["err"]


@pytest.mark.parametrize("nsw", [1, 2, 4])
def test_protocol_is_safe_and_ends(nsw):
    for nc in list(range(0, 20)) + [31, 32, 33, 47, 64, 69]:
        for seed in range(6):
            run(nc, nsw, seed)


@pytest.mark.parametrize("bug", ["early_read", "early_overwrite", "early_half"])
def test_planted_mistakes_are_caught(bug):
    caught = 0
    for seed in range(40):
        try:
            run(24, 4, seed, bug)
        except Violation:
            caught += 1
    assert caught > 0, f"the model does not catch the planted mistake {bug}"


def test_give_up_ends_every_wave():
    """With a tiny poll bound some wait gives up: every wave still finishes
    (later waits return at once) and the error is recorded."""
    seen = 0
    for seed in range(20):
        seen += run(24, 4, seed, spin=2)
    assert seen > 0
