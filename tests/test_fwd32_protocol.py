"""CPU model check of the LDS counter protocol of the 32-token pipelined kernel.

The kernel (gated_delta_rule_tok_amd/csrc/kda_fwd32.hip) has no workgroup
barrier in its main loops.  Four producer waves form two slots; the two
waves (halves HF) of slot k build chunks k, k + 2, ..  Packages live in
buffers (c, bf) = (chunk & 1, (chunk >> 1) & 1) with a scratch per slot; the
state waves read the packages in chunk order.  LDS counters order them:

  opnd[k]     halves of producer slot k whose operands are in LDS (two per chunk)
  rdy[c][bf]  four per complete package: the two product waves add two each
  done[c][w]  chunks of parity c that state wave w has finished

The model runs the same waits and counts as Python generators under random
interleavings (every wave at its own random speed) and checks that every read
sees the right chunk's data, that nothing is overwritten while still being
read, that the run ends, that a planted off-by-one mistake is caught, and that
a wait which gives up (a bound on the number of polls) makes every wave finish
with the error set.
"""
from __future__ import annotations

import random

import pytest

NH = 2  # producer waves per slot


class Violation(Exception):
    pass


class Deadlock(Exception):
    pass


def run(nc: int, nsw: int, seed: int, bug: str | None = None, spin: int | None = None) -> int:
    """One random interleaving; returns the error flag of the workgroup."""
    rng = random.Random(seed)
    st = {"err": 0}
    opnd = [0, 0]
    rdy = [[0, 0] for _ in range(2)]
    done = [[0] * 4 for _ in range(2)]
    # LDS contents: per package buffer, the chunk each half's operand part and
    # each product holds; per slot scratch, the chunk each half wrote
    pk_opnd = {(c, b, q): -1 for c in range(2) for b in range(2) for q in range(NH)}
    pk_prod = {(c, b, x): -1 for c in range(2) for b in range(2) for x in ("l", "m")}
    sc = {(k, q): -1 for k in range(2) for q in range(NH)}
    reading = {}  # (c, bf) -> set of (reader, chunk)

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

    def ok(c, b, j):
        return (pk_prod[(c, b, "l")] == j and pk_prod[(c, b, "m")] == j and
                all(pk_opnd[(c, b, q)] == j for q in range(NH)))

    def producer(k, q):
        for j in range(k, nc, 2):
            u, bf = j >> 1, (j >> 1) & 1
            if j >= 4:
                tgt = u - 1 - (1 if bug == "early_overwrite" else 0)
                yield from wait(lambda: min(done[k][:nsw]) >= tgt)
            if j >= 2:
                tgt = 4 * (((u - 1) >> 1) + 1) - (2 if bug == "early_scratch" else 0)
                yield from wait(lambda: rdy[k][bf ^ 1] >= tgt)
            if not st["err"]:
                for rd in reading.get((k, bf), set()):
                    if rd[1] != j:
                        raise Violation(f"slot {k} buffer {bf} overwritten with chunk {j} "
                                        f"while {rd[0]} reads chunk {rd[1]}")
            pk_opnd[(k, bf, q)] = j
            sc[(k, q)] = j
            yield "run"
            opnd[k] += 1
            tgt = 2 * (u + 1) - (1 if bug == "early_opnd" else 0)
            yield from wait(lambda: opnd[k] >= tgt)
            # the products read both halves' operands and scratch
            if not st["err"]:
                for qq in range(NH):
                    if sc[(k, qq)] != j or pk_opnd[(k, bf, qq)] != j:
                        raise Violation(f"products of chunk {j}: half {qq} holds "
                                        f"{sc[(k, qq)]}/{pk_opnd[(k, bf, qq)]}")
            yield "run"
            if not st["err"]:
                for qq in range(NH):
                    if sc[(k, qq)] != j:
                        raise Violation(f"scratch of chunk {j} changed under its products")
            pk_prod[(k, bf, "l" if q == (u & 1) else "m")] = j
            rdy[k][bf] += 2
            yield "run"

    def state(w):
        """Loads chunk j's operands once it is ready, reads its K' while
        updating, says it is done with it, and only then waits for chunk j + 1."""
        def begin(j):
            c, bf = j & 1, (j >> 1) & 1
            tgt = 4 * ((j >> 2) + 1) - (2 if bug == "early_read" else 0)
            yield from wait(lambda: rdy[c][bf] >= tgt)
            reading.setdefault((c, bf), set()).add((f"state wave {w}", j))
            if not st["err"] and not ok(c, bf, j):
                raise Violation(f"state wave {w} reads an incomplete package for chunk {j}")

        if nc > 0:
            yield from begin(0)
        for j in range(nc):
            c, bf = j & 1, (j >> 1) & 1
            yield "run"
            if not st["err"] and not ok(c, bf, j):
                raise Violation(f"package of chunk {j} changed under state wave {w}")
            reading[(c, bf)].discard((f"state wave {w}", j))
            done[c][w] += 1
            if j + 1 < nc:
                yield from begin(j + 1)
            yield "run"

    gens = [producer(k, q) for k in range(2) for q in range(NH)] + [state(w) for w in range(nsw)]
    speed = [rng.uniform(0.05, 1.0) for _ in gens]
    live = list(range(len(gens)))
    stalled = 0
    while live:
        i = rng.choice(live)
        if rng.random() > speed[i]:
            continue
        try:
            r = next(gens[i])
        except StopIteration:
            live.remove(i)
            stalled = 0
            continue
        if r == "blocked":
            stalled += 1
            if stalled > 200 * len(live) + 2000:
                raise Deadlock(f"deadlock (nc={nc}, nsw={nsw})")
        else:
            stalled = 0
    return st["err"]


@pytest.mark.parametrize("nsw", [1, 2, 4])
def test_protocol_is_safe_and_ends(nsw):
    for nc in list(range(0, 14)) + [31, 32, 33, 64]:
        for seed in range(6):
            assert run(nc, nsw, seed) == 0


@pytest.mark.parametrize("bug", ["early_read", "early_overwrite", "early_opnd", "early_scratch"])
def test_planted_mistakes_are_caught(bug):
    caught = 0
    for seed in range(40):
        try:
            run(20, 4, seed, bug)
        except (Violation, Deadlock):
            caught += 1
    assert caught > 0, f"the model does not catch the planted mistake {bug}"


def test_give_up_ends_every_wave():
    """With a tiny poll bound some wait gives up: every wave still finishes
    (later waits return at once) and the error is recorded."""
    seen = 0
    for seed in range(20):
        seen += run(24, 4, seed, spin=2)
    assert seen > 0
