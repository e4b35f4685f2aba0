"""CPU model of the decode kernel's stage layouts: the 1 KB loads of a stage
fill every (row, chunk) of the weight and activation areas exactly once, at
the LDS position the MFMA fragment reads expect, and the waves' k-steps cover
every chunk of a stage row.  Covers 512 k and 1024 k stages (16 rows) and the
paired gate+up stage (16 + 16 rows x 256 k); the kernel maps LDS chunk P of a
stage to row P // CPR, position swz(P % CPR, row)."""
import pytest


def swz(c, r):
    return (c & ~15) | ((c ^ r) & 15)


@pytest.mark.parametrize("MC,CPR", [(1, 128), (4, 128), (16, 64), (1, 64)])
def test_single_stage_maps(MC, CPR):
    WCH = 16 * CPR
    NL = WCH // 64 // 8
    NT = CPR // 32
    XI = (MC * CPR // 64 + 7) // 8
    lds, xl = {}, {}
    for w in range(8):
        for i in range(NL):
            for L in range(64):
                P = 64 * (NL * w + i) + L
                r = P // CPR
                assert P not in lds
                lds[P] = (r, swz(P % CPR, r))
        for j in range(XI):
            if w + 8 * j >= MC * CPR // 64:
                continue
            for L in range(64):
                P = 64 * (w + 8 * j) + L
                r = P // CPR
                xl[P] = (r, swz(P % CPR, r))
    assert set(lds.values()) == {(r, c) for r in range(16) for c in range(CPR)}
    assert set(xl.values()) == {(r, c) for r in range(MC) for c in range(CPR)}
    cover = set()
    for w in range(8):
        for t in range(NT):
            for lane in range(64):
                li, lg = lane & 15, lane >> 4
                kc = w * (CPR // 8) + 4 * t + lg
                assert lds[li * CPR + swz(kc, li)] == (li, kc)
                if li < MC:
                    assert xl[li * CPR + swz(kc, li)] == (li, kc)
                cover.add((li, kc))
    assert cover == {(r, c) for r in range(16) for c in range(CPR)}


def test_paired_stage_maps():
    MC, CPR, cpr = 16, 64, 32
    NL = 16 * CPR // 64 // 8
    lds, xl = {}, {}
    for w in range(8):
        for i in range(NL):
            for L in range(64):
                P = 64 * (NL * w + i) + L
                r = P // cpr
                assert (r >= 16) == (w >= 4)   # waves 4-7 load the up rows
                lds[P] = (r >> 4, r & 15, swz(P % cpr, r))
        for L in range(64):
            P = 64 * w + L
            r = P // cpr
            xl[P] = (r, swz(P % cpr, r))
    assert set(lds.values()) == {(m, r, c) for m in (0, 1) for r in range(16) for c in range(32)}
    assert set(xl.values()) == {(r, c) for r in range(MC) for c in range(32)}
    for w in range(8):
        for lane in range(64):
            li, lg = lane & 15, lane >> 4
            kcp = 4 * w + lg
            assert lds[li * 32 + swz(kcp, li)] == (0, li, kcp)
            assert lds[512 + li * 32 + swz(kcp, li)] == (1, li, kcp)
            assert xl[li * 32 + swz(kcp, li)] == (li, kcp)
