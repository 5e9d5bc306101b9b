"""CPU model of the grouped GEMM's staging protocol (gemm.hip, K loop).

The kernel keeps three LDS stages in a ring and splits its 8 waves into two
groups that alternate read and matrix phases, one phase apart; every phase
ends with a workgroup barrier.  In its read phase for stage ks a wave issues
its direct-to-LDS loads of stage ks + 2 and, before the closing barrier,
waits (vmcnt) until its own loads of stage ks + 1 have landed.  This test
replays that program order for both groups and every stage count up to 129
and checks the two properties the kernel relies on:

* every read of stage s by either group comes after a barrier that follows
  every wave's wait for stage s;
* a slot is only re-staged after every read of the stage it held.

Loads complete in issue order (vmcnt(n) = all but the last n loads landed)."""
import pytest

NST = 3          # LDS ring depth


def wave_program(group, K):
    ev = [("issue", 0)]
    if K > 1:
        ev += [("issue", 1), ("wait", 1)]      # stage 0 landed, stage 1 may be in flight
    else:
        ev += [("wait", 0)]
    ev.append(("bar", None))
    if group == 1:
        ev.append(("bar", None))               # group 1 sits out phase 0
    for ks in range(K):
        if ks + 2 < K:
            ev.append(("issue", ks + 2))
        ev.append(("read", ks))
        if ks + 2 < K:
            ev.append(("wait", 1))
        elif ks + 1 < K:
            ev.append(("wait", 0))
        ev.append(("bar", None))               # end of read phase
        ev.append(("bar", None))               # end of matrix phase
    if group == 0:
        ev.append(("bar", None))               # group 0 sits out the last phase
    return ev


def replay(K):
    info = {}
    for g in (0, 1):
        b, issued, landed_at, reads, issues = 0, [], {}, [], []
        for kind, a in wave_program(g, K):
            if kind == "bar":
                b += 1
            elif kind == "issue":
                issued.append(a)
                issues.append((a, b))
            elif kind == "wait":
                for s in (issued[:len(issued) - a] if a else issued):
                    landed_at.setdefault(s, b)
            else:
                reads.append((a, b))
        info[g] = (b, landed_at, reads, issues)
    return info


@pytest.mark.parametrize("K", list(range(1, 130)))
def test_staging_protocol(K):
    info = replay(K)
    assert info[0][0] == info[1][0], "both groups must pass the same number of barriers"
    for g in (0, 1):
        for s, b in info[g][2]:
            for g2 in (0, 1):
                lb = info[g2][1].get(s)
                assert lb is not None and lb < b, (K, g, s, g2)
        for s, b in info[g][3]:
            if s >= NST:
                for g2 in (0, 1):
                    for s2, b2 in info[g2][2]:
                        if s2 == s - NST:
                            assert b2 < b, (K, g, s, g2)


def test_protocol_model_detects_a_missing_wait():
    """The checker itself fails when a wave skips its wait for stage ks + 1."""
    global wave_program
    orig = wave_program

    def broken(group, K):
        return [e for e in orig(group, K) if not (group == 1 and e == ("wait", 1))]

    try:
        wave_program = broken
        with pytest.raises(AssertionError):
            test_staging_protocol(8)
    finally:
        wave_program = orig
