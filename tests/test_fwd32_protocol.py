"""CPU model check of the counter protocol of the 32-token pipelined kernel.

The kernel (gated_delta_rule_tok_amd/csrc/kda_fwd32.hip) has no workgroup
barrier in its main loops.  Four producer waves (quarter Q = 2 CH + HF: token
half HF, channel half CH) build each chunk's package in one of two slots
(c = chunk & 1), double-buffered (bf = (chunk >> 1) & 1); the state waves read
the packages in chunk order.  LDS counters order them:

  nrm[c][HF]  partial norms of half HF written (two per chunk: both channel halves)
  opnd[c]     quarters whose operands are in LDS (four per chunk)
  rdy[c][bf]  four per complete package: the two product waves add two each, or
              each producer wave adds one for a package copied from the partner
  done[c][w]  chunks of slot c that state wave w has finished

With a value split of two and a ring, the two workgroups of a (sequence, head)
build alternate chunks (slice s builds chunks 2 r + s in round r) and hand each
finished package to the other through a two-slot ring in global memory:
flag[pub][slot][Q] = chunk + 1 once wave Q's blocks are stored.  A slot needs
no acknowledgement: the partner raises its next flag only after its copy of
the slot's previous image is complete.  Stores and copies are asynchronous and
complete in issue order per wave (the vector memory count).

The model runs the same waits, counts and flags as Python generators under
random interleavings, with asynchronous memory operations completing at random
(in order per wave), and checks that every read sees the right chunk's data,
that nothing is overwritten while still being read, that the run ends, that a
planted off-by-one mistake is caught, and that a wait which gives up (a bound
on the number of polls) makes every wave finish quickly with the error set.
"""
from __future__ import annotations

import random

import pytest

NQ = 4  # producer waves


class Violation(Exception):
    pass


class Deadlock(Exception):
    pass


def run(nc: int, nsw: int, seed: int, shared: bool, bug: str | None = None, spin: int | None = None):
    """One random interleaving; returns the error flags of the workgroups."""
    rng = random.Random(seed)
    nwg = 2 if shared else 1
    g_flag = {}  # (pub, slot, q) -> value
    g_ring = {}  # (pub, slot, q) -> chunk whose blocks are stored there
    class WG:
        def __init__(self, s):
            self.s = s
            self.nrm = [[0, 0] for _ in range(2)]
            self.opnd = [0, 0]
            self.rdy = [[0, 0] for _ in range(2)]
            self.done = [[0] * 4 for _ in range(2)]
            self.err = 0
            # LDS contents: package (c, bf) -> per quarter, the chunk its operand
            # part / its copied blocks hold; products -> chunk
            self.pk_opnd = {(c, b, q): -1 for c in range(2) for b in range(2) for q in range(NQ)}
            self.pk_blocks = {(c, b, q): -1 for c in range(2) for b in range(2) for q in range(NQ)}
            self.pk_prod = {(c, b, k): -1 for c in range(2) for b in range(2) for k in ("l", "m")}
            self.sc = {(c, q): -1 for c in range(2) for q in range(NQ)}
            self.nr = {(c, hf, ch): -1 for c in range(2) for hf in range(2) for ch in range(2)}
            self.reading = {}  # (c, bf) -> set of (reader, chunk)

    wgs = [WG(s) for s in range(nwg)]

    def wait(wg, cond, what):
        if wg.err:
            return
        it = 0
        while not cond():
            it += 1
            if spin is not None and it > spin:
                wg.err = 1
                return
            yield ("blocked", what)

    def poll(wg, cond, what):
        if wg.err:
            return
        it = 0
        while not cond():
            it += 1
            if spin is not None and it > spin:
                wg.err = 2
                return
            yield ("blocked", what)

    def check_free(wg, c, b, j, who):
        if wg.err:
            return
        for rd in wg.reading.get((c, b), set()):
            if rd[1] != j:
                raise Violation(f"wg {wg.s} {who}: package ({c},{b}) overwritten with chunk {j} "
                                f"while {rd[0]} reads chunk {rd[1]}")

    def package_ok(wg, c, b, j):
        if wg.pk_prod[(c, b, "l")] == j and wg.pk_prod[(c, b, "m")] == j and \
                all(wg.pk_opnd[(c, b, q)] == j for q in range(NQ)):
            return True
        return all(wg.pk_blocks[(c, b, q)] == j for q in range(NQ))

    def producer(wg, q, vmq):
        hf, ch = q & 1, q >> 1
        s = wg.s

        def own_chunk(j, c, bf, rot, nrm_target, opnd_target, between):
            # the package buffer is free once the state waves are done with chunk j - 4,
            # the scratch once the products of chunk j - 2 are
            if j >= 4:
                tgt = (j >> 1) - 1 - (1 if bug == "early_overwrite" else 0)
                yield from wait(wg, lambda: min(wg.done[c][:nsw]) >= tgt, "done")
            if j >= 2:
                pb = ((j - 2) >> 1) & 1
                yield from wait(wg, lambda: wg.rdy[c][pb] >= 4 * (((j - 2) >> 2) + 1), "scratch")
            # partial norms
            wg.nr[(c, hf, ch)] = j
            yield ("run", None)
            wg.nrm[c][hf] += 1
            yield from between()
            tgt = nrm_target - (1 if bug == "early_norm" else 0)
            yield from wait(wg, lambda: wg.nrm[c][hf] >= tgt, "nrm")
            if not wg.err and wg.nr[(c, hf, ch ^ 1)] != j:
                raise Violation(f"wg {s} wave {q}: norms of chunk {wg.nr[(c, hf, ch ^ 1)]} for chunk {j}")
            check_free(wg, c, bf, j, f"wave {q}")
            wg.pk_opnd[(c, bf, q)] = j
            wg.pk_blocks[(c, bf, q)] = -2
            wg.sc[(c, q)] = j
            yield ("run", None)
            wg.opnd[c] += 1
            yield from wait(wg, lambda: wg.opnd[c] >= opnd_target, "opnd")
            for kind, sel in (("l", rot & 3), ("m", (rot + 2) & 3)):
                if q == sel:
                    if not wg.err:
                        for qq in range(NQ):
                            if wg.sc[(c, qq)] != j or wg.pk_opnd[(c, bf, qq)] != j:
                                raise Violation(f"wg {s} products of chunk {j}: quarter {qq} holds "
                                                f"{wg.sc[(c, qq)]}/{wg.pk_opnd[(c, bf, qq)]}")
                    yield ("run", None)
                    wg.pk_prod[(c, bf, kind)] = j
                    wg.rdy[c][bf] += 2

        if not shared:
            for j in range(nc):
                c, bf = j & 1, (j >> 1) & 1

                def nothing():
                    return
                    yield
                yield from own_chunk(j, c, bf, j, 2 * (j >> 1) + 2, 4 * (j >> 1) + 4, nothing)
            return

        nr = (nc + 1) >> 1
        for r in range(nr + 1):
            j, jq, jo = 2 * r + s, 2 * (r - 1) + 1 - s, 2 * (r - 1) + s
            own = r < nr and j < nc
            rcv = r >= 1 and jq < nc

            def between(r=r, j=j, jq=jq, jo=jo, rcv=rcv, after_gate=True):
                if r >= 1 and jo < nc:
                    # the previous own chunk's stores are complete: flag them
                    if bug != "early_flag":
                        # all but the gate loads just issued (the youngest entry)
                        while len(vmq) > (1 if after_gate else 0):
                            yield from complete_one(vmq)
                    g_flag[(s, (r - 1) & 1, q)] = jo + 1
                    yield ("run", None)
                if rcv:
                    yield from poll(wg, lambda: g_flag.get((1 - s, (r - 1) & 1, q), 0) >= jq + 1, "flag")
                    cq, bq = jq & 1, (jq >> 1) & 1
                    if jq >= 4:
                        yield from wait(wg, lambda: min(wg.done[cq][:nsw]) >= (jq >> 1) - 1, "done(copy)")
                    check_free(wg, cq, bq, jq, f"copy by wave {q}")
                    wg.pk_blocks[(cq, bq, q)] = -2  # being written
                    vmq.append(("copy", (wg, cq, bq, q, jq, (1 - s, (r - 1) & 1, q))))

            if own:
                bf = r & 1

                def gate_between():
                    vmq.append(("gate", None))
                    yield from between()
                yield from own_chunk(j, s, bf, r, 2 * r + 2, 4 * r + 4, gate_between)
                yield from wait(wg, lambda: wg.rdy[s][bf] >= 4 * ((r >> 1) + 1), "rdy(publish)")
                if not wg.err and not package_ok(wg, s, bf, j):
                    raise Violation(f"wg {s} wave {q}: publishes an incomplete package of chunk {j}")
                # the data is read from LDS now, stored at completion
                vmq.append(("qk", None))
                vmq.append(("store", (s, bf, q, j)))
                if rcv:
                    # the copy is older than the q/k loads and the stores
                    while vmq and any(op[0] == "copy" for op in vmq):
                        yield from complete_one(vmq)
                    wg.rdy[jq & 1][(jq >> 1) & 1] += 1
            else:
                yield from between(after_gate=False)
                if rcv:
                    while vmq:
                        yield from complete_one(vmq)
                    wg.rdy[jq & 1][(jq >> 1) & 1] += 1
        while vmq:
            yield from complete_one(vmq)

    def complete_one(vmq):
        """The wave's oldest memory operation completes: a store lands in the
        ring; a copy reads the ring (now) and its data is in LDS."""
        kind, arg = vmq.pop(0)
        if kind == "store":
            pub, slot, q, j = arg
            g_ring[(pub, slot, q)] = j
        elif kind == "copy":
            wg, c, b, q, j, src = arg
            if not any(w.err for w in wgs) and g_ring.get(src, -1) != j:
                raise Violation(f"wg {wg.s} wave {q} copies chunk {j}: ring {src} holds {g_ring.get(src, -1)}")
            wg.pk_blocks[(c, b, q)] = j
        yield ("run", None)

    def state(wg, w):
        """A state wave loads chunk j's operands once chunk j is ready, reads
        the rest of its package (K') while updating, and then says it is done
        with it; only then does it wait for chunk j + 1.  (Waiting for chunk
        j + 1 before saying done with chunk j, the planted "done_after_next",
        deadlocks the shared ring: the partner's chunk j + 1 may only be
        copied in after this workgroup's producers got a buffer back.)"""
        def begin(j):
            c, bf = j & 1, (j >> 1) & 1
            tgt = 4 * ((j >> 2) + 1) - (2 if bug == "early_read" else 0)
            yield from wait(wg, lambda: wg.rdy[c][bf] >= tgt, "rdy(state)")
            wg.reading.setdefault((c, bf), set()).add((f"state {w}", j))
            if not wg.err and not package_ok(wg, c, bf, j):
                raise Violation(f"wg {wg.s} state wave {w} reads an incomplete package for chunk {j}")

        def end(j):
            c, bf = j & 1, (j >> 1) & 1
            if not wg.err and not package_ok(wg, c, bf, j):
                raise Violation(f"wg {wg.s} package of chunk {j} changed under state wave {w}")
            wg.reading[(c, bf)].discard((f"state {w}", j))
            wg.done[c][w] += 1

        if nc > 0:
            yield from begin(0)
        for j in range(nc):
            yield ("run", None)
            if bug == "done_after_next":
                if j + 1 < nc:
                    yield from begin(j + 1)
                end(j)
            else:
                end(j)
                if j + 1 < nc:
                    yield from begin(j + 1)
            yield ("run", None)

    gens = []
    for wg in wgs:
        for q in range(NQ):
            vmq = []
            gens.append((producer(wg, q, vmq), vmq))
        for w in range(nsw):
            gens.append((state(wg, w), None))
    live = list(range(len(gens)))
    stalled = 0
    while live:
        # producers (those with a memory queue) run three times as often: they
        # get ahead, which is where an early overwrite would show
        i = rng.choice(live)
        if gens[i][1] is None and rng.random() < 0.67:
            continue
        gen, vmq = gens[i]
        # asynchronous completion of the oldest memory operation of the wave
        if vmq and rng.random() < 0.3:
            for _ in complete_one(vmq):
                pass
        try:
            st = next(gen)
        except StopIteration:
            live.remove(i)
            stalled = 0
            continue
        if st[0] == "blocked":
            stalled += 1
            if stalled > 200 * len(live) + 2000:
                raise Deadlock(f"deadlock (nc={nc}, nsw={nsw}, shared={shared})")
        else:
            stalled = 0
    return [wg.err for wg in wgs]


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("nsw", [1, 2, 4])
def test_protocol_is_safe_and_ends(nsw, shared):
    for nc in list(range(0, 14)) + [31, 32, 33, 64]:
        for seed in range(4):
            assert run(nc, nsw, seed, shared) == [0] * (2 if shared else 1)


@pytest.mark.parametrize("shared,bug", [(False, "early_read"), (False, "early_overwrite"), (False, "early_norm"),
                                        (True, "early_read"), (True, "early_overwrite"), (True, "early_norm"),
                                        (True, "early_flag"), (True, "done_after_next")])
def test_planted_mistakes_are_caught(bug, shared):
    caught = 0
    for seed in range(30):
        try:
            run(20, 4, seed, shared, bug)
        except (Violation, Deadlock):
            caught += 1
    assert caught > 0, f"the model does not catch the planted mistake {bug}"


@pytest.mark.parametrize("shared", [False, True])
def test_give_up_ends_every_wave(shared):
    """With a tiny poll bound some wait gives up: every wave still finishes
    (later waits return at once) and the error is recorded."""
    seen = 0
    for seed in range(20):
        errs = run(24, 4, seed, shared, spin=2)
        seen += any(errs)
    assert seen > 0
