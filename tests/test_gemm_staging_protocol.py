"""CPU model of the grouped GEMM's staging protocol (gemm.hip, K loop).

The kernel keeps three LDS stages in a ring and splits its 8 waves into two
groups that alternate read and matrix phases, one phase apart; every phase
ends with a workgroup barrier.  A workgroup's tiles form one stream of
stages; in its read phase for stream stage G a wave issues its
direct-to-LDS loads of stage G + 2 (possibly the next tile's) and, before the
closing barrier, waits (vmcnt) until its own loads of stage G + 1 have
landed.  This test replays that program order for both groups, for 1, 2 and
5 tiles of many stage counts, and checks the two properties the kernel
relies on:

* every read of stage s by either group comes after a barrier that follows
  every wave's wait for stage s;
* a slot is only re-staged after every read of the stage it held.

Loads complete in issue order (vmcnt(n) = all but the last n loads landed)."""
import pytest

NST = 3          # LDS ring depth


def wave_program(group, K, tiles=1):
    """Program order of one wave over `tiles` tiles of K stages each.  The
    stages of all tiles form one stream (stage g = K stage g % K of tile
    g // K, slot g % NST); with K >= 2 the next tile's first stages are
    staged during the current tile, otherwise each tile refills the ring."""
    total = tiles * K
    stream = K >= 2
    ev = []
    for ti in range(tiles):
        base = ti * K

        def staged(g):
            return g < total and (stream or g < base + K)

        if ti == 0 or not stream:
            ev += [("wait", 0), ("bar", None)]         # ring idle
            ev.append(("issue", base))
            if staged(base + 1):
                ev += [("issue", base + 1), ("wait", 1)]
            else:
                ev.append(("wait", 0))
            ev.append(("bar", None))
        if group == 1:
            ev.append(("bar", None))                  # group 1 sits out the tile's phase 0
        for ks in range(K):
            g = base + ks
            if staged(g + 2):
                ev.append(("issue", g + 2))
            ev.append(("read", g))
            if staged(g + 2):
                ev.append(("wait", 1))
            elif staged(g + 1):
                ev.append(("wait", 0))
            ev.append(("bar", None))                  # end of read phase
            ev.append(("bar", None))                  # end of matrix phase
        if group == 0:
            ev.append(("bar", None))                  # group 0 sits out the last phase
        ev.append(("bar", None))                      # epilogue barrier (FP8 Z amax)
    return ev


def replay(K, tiles=1):
    info = {}
    for g in (0, 1):
        b, issued, landed_at, reads, issues = 0, [], {}, [], []
        for kind, a in wave_program(g, K, tiles):
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


@pytest.mark.parametrize("tiles", [1, 2, 5])
@pytest.mark.parametrize("K", list(range(1, 40)) + [56, 64, 112, 128])
def test_staging_protocol(K, tiles):
    info = replay(K, tiles)
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

    def broken(group, K, tiles=1):
        return [e for e in orig(group, K, tiles) if not (group == 1 and e == ("wait", 1))]

    try:
        wave_program = broken
        with pytest.raises(AssertionError):
            test_staging_protocol(8, 2)
    finally:
        wave_program = orig
