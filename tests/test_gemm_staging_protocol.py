"""CPU model of the grouped GEMM's staging protocol (gemm.hip, K loop).

The kernel keeps three LDS stages in a ring.  Four producer waves only
issue direct-to-LDS loads; eight consumer waves in two groups only read
LDS fragments and multiply, alternating read and matrix phases one phase
apart.  Every phase ends with a workgroup barrier taken by all twelve waves.
A workgroup's work items (whole tiles, then possibly one K-split piece of a
tile) form one stream of stages.  In the two phases of stream stage G a
producer issues its loads of stage G + 2 (first half, barrier, second half)
and then waits (vmcnt) until its loads of stage G + 1 have landed.  Producer 0 issues one extra load per stage (the FP8 weight scales),
first.  This test replays that program order for every role, for 1, 2 and
5 tiles of many stage counts, and checks the properties the kernel relies
on:

* every role passes the same number of barriers;
* every read of stage s by either consumer group comes after a barrier that
  follows every producer's wait for all of its loads of s;
* a slot is only re-staged after a barrier that follows every read of the
  stage it held.

Loads complete in issue order (vmcnt(n) = all but the last n loads landed)."""
import pytest

NST = 3          # LDS ring depth


def _items(K, tiles, piece=0):
    """A workgroup's work items: (stages, whole tile?).  `tiles` whole tiles of
    K stages, then optionally one K-split piece of `piece` stages (pieces
    store raw partial sums and skip the FP8 epilogue's row-amax barrier)."""
    return [(K, True)] * tiles + ([(piece, False)] if piece else [])


def consumer_program(group, K, tiles=1, fp8_epilogue=True, piece=0):
    items = _items(K, tiles, piece)
    stream = K >= 2
    ev, base = [], 0
    for ti, (nks, whole) in enumerate(items):
        if ti == 0 or not stream:
            ev += [("bar", None), ("bar", None)]      # producers fill stage 0
        if group == 1:
            ev.append(("bar", None))                  # group 1 sits out the item's phase 0
        for ks in range(nks):
            ev.append(("read", base + ks))
            ev.append(("bar", None))                  # end of read phase (reads complete)
            ev.append(("bar", None))                  # end of matrix phase
        if group == 0:
            ev.append(("bar", None))                  # group 0 sits out the last phase
        if fp8_epilogue and whole:
            ev.append(("bar", None))                  # row-amax exchange of the FP8 Z epilogue
        base += nks
    return ev


def producer_program(K, tiles=1, fp8=True, first=False, fp8_epilogue=True, piece=0):
    """One producer wave.  FP8: 7 + 6 loads per stage (+1 weight-scale load
    issued first by producer 0); otherwise 6 + 6."""
    items = _items(K, tiles, piece)
    stream = K >= 2
    total = sum(n for n, _ in items)
    halves = (7, 6) if fp8 else (6, 6)
    nload = sum(halves)
    ev, base = [], 0

    def issue(g, half):
        n = halves[half] + (1 if (fp8 and first and half == 0) else 0)
        return [("issue", g)] * n

    for ti, (nks, whole) in enumerate(items):
        def staged(g):
            return g < total and (stream or g < base + nks)
        if ti == 0 or not stream:
            ev += [("wait", 0), ("bar", None)]
            ev += issue(base, 0) + issue(base, 1)
            if staged(base + 1):
                ev += issue(base + 1, 0) + issue(base + 1, 1) + [("wait", nload)]
            else:
                ev.append(("wait", 0))
            ev.append(("bar", None))
        for ks in range(nks):
            g = base + ks
            s2 = staged(g + 2)
            if s2:
                ev += issue(g + 2, 0)
            ev.append(("bar", None))
            if s2:
                ev += issue(g + 2, 1) + [("wait", nload)]
            elif staged(g + 1):
                ev.append(("wait", 0))
            ev.append(("bar", None))
        ev.append(("bar", None))                      # the item's last phase
        if fp8_epilogue and whole:
            ev.append(("bar", None))
        base += nks
    return ev


def replay_consumer(prog):
    b, reads = 0, []
    for kind, a in prog:
        if kind == "bar":
            b += 1
        elif kind == "read":
            reads.append((a, b))
    return b, reads


def replay_producer(prog):
    """-> (barriers, {stage: barrier count at the wait that landed all of
    its loads}, [(stage, barrier count at issue)])"""
    from collections import Counter
    b, issued, landed, issues = 0, [], 0, []
    n_issued, n_landed = Counter(), Counter()
    landed_at = {}
    for kind, a in prog:
        if kind == "bar":
            b += 1
        elif kind == "issue":
            issued.append(a)
            n_issued[a] += 1
            issues.append((a, b))
        else:
            upto = max(landed, len(issued) - a)
            newly = set(issued[landed:upto])
            for s in issued[landed:upto]:
                n_landed[s] += 1
            landed = upto
            for s in newly:                           # only these can have just completed
                if s not in landed_at and n_landed[s] == n_issued[s]:
                    landed_at[s] = b
    return b, landed_at, issues


def check(K, tiles, fp8, fp8_epilogue, programs=None, piece=0):
    progs = programs or {
        "c0": consumer_program(0, K, tiles, fp8_epilogue, piece),
        "c1": consumer_program(1, K, tiles, fp8_epilogue, piece),
        "p0": producer_program(K, tiles, fp8, True, fp8_epilogue, piece),
        "p1": producer_program(K, tiles, fp8, False, fp8_epilogue, piece),
    }
    cons = {k: replay_consumer(v) for k, v in progs.items() if k[0] == "c"}
    prod = {k: replay_producer(v) for k, v in progs.items() if k[0] == "p"}
    bars = {k: v[0] for k, v in cons.items()} | {k: v[0] for k, v in prod.items()}
    assert len(set(bars.values())) == 1, ("barrier counts differ", bars)
    for ck, (_, reads) in cons.items():
        for s, b in reads:
            for pk, (_, landed_at, _) in prod.items():
                lb = landed_at.get(s)
                assert lb is not None and lb < b, (K, ck, s, pk, lb, b)
    last_read = {}                                    # (consumer, stage) -> barrier count of its read
    for ck, (_, reads) in cons.items():
        for s2, b2 in reads:
            last_read[ck, s2] = max(b2, last_read.get((ck, s2), -1))
    for pk, (_, _, issues) in prod.items():
        for s, b in issues:
            if s >= NST:
                for ck in cons:
                    b2 = last_read.get((ck, s - NST))
                    assert b2 is None or b2 < b, (K, pk, s, ck, b2, b)


@pytest.mark.parametrize("fp8,fp8_epilogue", [(True, True), (True, False), (False, False)])
@pytest.mark.parametrize("tiles", [1, 2, 5])
@pytest.mark.parametrize("K", list(range(1, 40)) + [56, 64, 112, 128])
def test_staging_protocol(K, tiles, fp8, fp8_epilogue):
    check(K, tiles, fp8, fp8_epilogue)


@pytest.mark.parametrize("fp8,fp8_epilogue", [(True, True), (False, False)])
@pytest.mark.parametrize("tiles", [0, 1, 3])
@pytest.mark.parametrize("K", [2, 3, 4, 7, 16, 56, 112])
def test_staging_protocol_with_k_piece(K, tiles, fp8, fp8_epilogue):
    """Whole tiles followed by one K-split piece of the last round (every
    piece length the kernel can choose: at least 2 stages, at most K)."""
    for piece in sorted({2, 3, K // 2, K} - {0, 1}):
        if piece <= K:
            check(K, tiles, fp8, fp8_epilogue, piece=piece)


def test_protocol_model_detects_a_missing_wait():
    """The checker fails when a producer skips its wait for stage G + 1."""
    K, tiles = 8, 2
    p1 = producer_program(K, tiles, True, False)
    i = next(n for n, e in enumerate(p1) if e == ("wait", 13) and n > 40)
    broken = {
        "c0": consumer_program(0, K, tiles), "c1": consumer_program(1, K, tiles),
        "p0": producer_program(K, tiles, True, True), "p1": p1[:i] + p1[i + 1:],
    }
    with pytest.raises(AssertionError):
        check(K, tiles, True, True, broken)


def test_protocol_model_detects_early_restaging():
    """The checker fails when a producer issues stage G + 2 one phase early."""
    K, tiles = 8, 1
    p0 = producer_program(K, tiles, True, True)
    # move the first in-loop barrier behind the second half of stage 4
    # (stage 4 re-stages the slot of stage 1, which group 1 is still reading)
    bars = [n for n, e in enumerate(p0) if e == ("bar", None)]
    n = bars[3]                                   # closes group 0's read of stage 1
    broken_p0 = p0[:n] + p0[n + 1:]
    broken_p0.insert(len(broken_p0) - 1, ("bar", None))
    broken = {
        "c0": consumer_program(0, K, tiles), "c1": consumer_program(1, K, tiles),
        "p0": broken_p0, "p1": producer_program(K, tiles, True, False),
    }
    with pytest.raises(AssertionError):
        check(K, tiles, True, True, broken)
