"""CPU model of the one-launch gated block's LDS layouts (the index formulas
of csrc/glu_fused.hip, restated): a stage's 40 load instructions (5 per wave)
fill every (row, 16-byte chunk) of the 64 activation rows and 256 weight rows
exactly once; every MFMA fragment read (activation, gate/up weights, down
weights, m) finds the global chunk it needs; gate and up fragments of a wave
cover the same hidden units; the m tile written by the epilogue is read back
at the same (token, hidden) place; and every 16-lane cycle of a fragment read
touches 16 distinct bank groups under gfx950's four-cycle ds_read_b128 model
(the cycle of lane l is set by l >> 5 and the parity of (l >> 2) & 7)."""
import itertools


def sw8(r):            # 128-byte stage rows
    return (r >> 1) & 7


def sw16(r):           # 256-byte m rows
    return r & 15


XROWS, WROWS, HS = 64, 256, 128


def load_map():
    """LDS chunk index of a stage -> (area, row, global chunk)."""
    lds = {}
    for w in range(8):
        for lane in range(64):
            pos = lane & 7
            rx = 8 * w + (lane >> 3)
            cx = pos ^ sw8(rx)
            P = w * 64 + lane                     # byte offset w * 1024 + 16 * lane
            assert P not in lds
            lds[P] = ("x", rx, cx)
            for j in range(4):
                rw = 8 * (4 * w + j) + (lane >> 3)
                cw = pos ^ sw8(rw)
                P = XROWS * 8 + (4 * w + j) * 64 + lane
                assert P not in lds
                lds[P] = ("w", rw, cw)
    return lds


def test_stage_filled_exactly_once():
    lds = load_map()
    assert len(lds) == (XROWS + WROWS) * 8
    assert {v for v in lds.values() if v[0] == "x"} == {("x", r, c) for r in range(XROWS) for c in range(8)}
    assert {v for v in lds.values() if v[0] == "w"} == {("w", r, c) for r in range(WROWS) for c in range(8)}
    # waves 0-3 load gate rows (0-127), waves 4-7 up rows (128-255)
    for w in range(8):
        for j in range(4):
            rows = {8 * (4 * w + j) + (lane >> 3) for lane in range(64)}
            assert all((r >= HS) == (w >= 4) for r in rows)


def _cycles():
    """lanes of each of the four 16-lane cycles of a ds_read_b128"""
    cyc = {}
    for l in range(64):
        key = (l >> 5, bin((l >> 2) & 7).count("1") & 1)
        cyc.setdefault(key, []).append(l)
    assert all(len(v) == 16 for v in cyc.values())
    return list(cyc.values())


def _conflict_free(addr_of_lane):
    for lanes in _cycles():
        banks = [addr_of_lane(l) % 16 for l in lanes]
        assert len(set(banks)) == 16


def test_fragment_reads():
    lds = load_map()
    for wave, ks in itertools.product(range(8), range(2)):
        wm, wn = wave >> 2, wave & 3
        xa = {}
        for f in range(2):
            def x_addr(l, f=f):
                r = 32 * wm + 16 * f + (l & 15)
                return r * 8 + ((4 * ks + (l >> 4)) ^ sw8(r))
            for l in range(64):
                r, c = 32 * wm + 16 * f + (l & 15), 4 * ks + (l >> 4)
                assert lds[x_addr(l)] == ("x", r, c)
            _conflict_free(x_addr)
        for j in range(4):
            def g_addr(l, j=j):
                rg = (32 * wn + 16 * j if j < 2 else HS + 32 * wn + 16 * (j - 2)) + (l & 15)
                return (XROWS + rg) * 8 + ((4 * ks + (l >> 4)) ^ sw8(rg))

            def d_addr(l, j=j):
                rd = 64 * wn + 16 * j + (l & 15)
                return (XROWS + rd) * 8 + ((4 * ks + (l >> 4)) ^ sw8(rd))
            for l in range(64):
                li, lg = l & 15, l >> 4
                rg = (32 * wn + 16 * j if j < 2 else HS + 32 * wn + 16 * (j - 2)) + li
                assert lds[g_addr(l)] == ("w", rg, 4 * ks + lg)
                rd = 64 * wn + 16 * j + li
                assert lds[d_addr(l)] == ("w", rd, 4 * ks + lg)
            _conflict_free(g_addr)
            _conflict_free(d_addr)
        # gate fragment j and up fragment j + 2 cover the same hidden units
        for j in range(2):
            gate = {32 * wn + 16 * j + li for li in range(16)}
            up = {HS + 32 * wn + 16 * j + li - HS for li in range(16)}
            assert gate == up


def test_m_tile_round_trip_and_reads():
    # epilogue: lane (li, lg) of wave (wm, wn) writes 8 bytes (hidden units
    # 32 wn + 16 gi + 4 lg .. + 3 of token 32 wm + 16 f + li)
    mbuf = {}
    for wave, f, gi, lane in itertools.product(range(8), range(2), range(2), range(64)):
        wm, wn, li, lg = wave >> 2, wave & 3, lane & 15, lane >> 4
        t = 32 * wm + 16 * f + li
        hcol = 32 * wn + 16 * gi + 4 * lg
        chunk = t * 16 + ((hcol >> 3) ^ sw16(t))
        half = lg & 1
        assert hcol % 8 == 4 * half
        for e in range(4):
            key = (chunk, 4 * half + e)
            assert key not in mbuf
            mbuf[key] = (t, hcol + e)
    assert set(mbuf.values()) == {(t, h) for t in range(64) for h in range(HS)}
    # down k-steps: token fragment f, hidden chunk 8 kh + 4 ks + lg
    for wave, kh, ks, f in itertools.product(range(8), range(2), range(2), range(2)):
        wm = wave >> 2

        def m_addr(l):
            r = 32 * wm + 16 * f + (l & 15)
            return r * 16 + ((8 * kh + 4 * ks + (l >> 4)) ^ sw16(r))
        for l in range(64):
            t = 32 * wm + 16 * f + (l & 15)
            c = 8 * kh + 4 * ks + (l >> 4)
            for e in range(8):
                assert mbuf[(m_addr(l), e)] == (t, 8 * c + e)
        _conflict_free(m_addr)


def test_output_ownership():
    """Every y element of a 64-token tile (D up to 4 x 256 columns) is held by
    exactly one lane of one wave: rows 256 nb + 64 wn + 16 j + 4 lg + r."""
    for ND in range(1, 5):
        owner = {}
        for wave, nb, f, j, lane, r in itertools.product(range(8), range(ND), range(2), range(4), range(64),
                                                         range(4)):
            wm, wn, li, lg = wave >> 2, wave & 3, lane & 15, lane >> 4
            key = (32 * wm + 16 * f + li, 256 * nb + 64 * wn + 16 * j + 4 * lg + r)
            assert key not in owner
            owner[key] = wave
        assert len(owner) == 64 * 256 * ND
