"""CPU model of the GEMM's k-major operand tiles (the backward's contractions
over the rows of both operands): the 1 KB loads of a stage place every
(k-row, chunk) of the 64 x 256 tile exactly once, and the transposing
fragment reads then hand each lane the 8 consecutive k of its MFMA column,
in the order a row-major fragment read gives them.

The transposing read (ds_read_b64_tr_b16) is modelled by its measured lane
map: within each 16-lane group, lane j gets element j % 4 of the 8-byte
pieces addressed by lanes 4 r + j // 4 of the group, r = 0..3 (an in-bounds
probe on gfx950 with LDS element i holding i).  The bank model: 64 banks of 4
bytes, a half-wave's 256 bytes per cycle."""
import pytest

NW, WM, WN, TM, TN = 8, 2, 4, 128, 64   # the 256 x 256 tile: 2 x 4 waves of 128 x 64
CPR = 32                                 # 16-byte chunks per k-row of 256 columns


def kswz(k):
    return 2 * ((k & 7) ^ (((k >> 3) & 1) << 2))


def stage_lds():
    """unit (16 B) of the operand region -> (k-row, first column) it holds"""
    lds = {}
    for w in range(NW):
        for i in range(4):
            for lane in range(64):
                unit = (i * NW + w) * 64 + lane
                kr = 16 * i + 2 * w + (lane >> 5)
                c = (lane & 31) ^ kswz(kr)
                assert unit not in lds
                lds[unit] = (kr, 8 * c)
    return lds


def element_at(lds, byte):
    """(k, column) of the bf16 element at a byte offset of the region"""
    kr, col0 = lds[byte // 16]
    return kr, col0 + (byte % 16) // 2


def tr_read(lds, addrs):
    """the measured lane map of ds_read_b64_tr_b16 over one wave"""
    out = []
    for lane in range(64):
        g, j = lane >> 4, lane & 15
        out.append([element_at(lds, addrs[16 * g + 4 * r + j // 4] + 2 * (j % 4)) for r in range(4)])
    return out


def frag_addrs(kind, wave, ks, f, h):
    """the kernel's address of each lane for fragment f, k-step ks, half h"""
    wm, wn = wave // WN, wave % WN
    addrs = []
    for lane in range(64):
        kq, s16 = lane >> 4, lane & 15
        row = ks * 32 + 8 * kq + (s16 >> 2) + 4 * h
        row0 = 8 * kq + (s16 >> 2)            # k-step 0, half 0: the one per-lane register
        if kind == "x":
            a0 = (row0 * 512 + (((wm * 16 + ((s16 & 3) >> 1)) ^ kswz(row0)) << 4) + ((s16 & 1) << 3)) ^ (32 * f)
            half = 0
        else:
            a0 = (row0 * 512 + (((wn * 8 + (s16 & 3)) ^ kswz(row0)) << 4)) ^ (64 * (f >> 1))
            half = 8 * (f & 1)
        # k-step ks: + 16384; half h = 1: (a0 ^ 128) + 2048
        addrs.append(16384 * ks + half + (a0 if h == 0 else (a0 ^ 128) + 2048))
        assert row == row0 + 32 * ks + 4 * h
    return addrs


def expected_col(kind, wave, f, j):
    wm, wn = wave // WN, wave % WN
    if kind == "x":                      # activation fragment: 16 consecutive tile rows
        return wm * TM + 16 * f + j
    # weight fragment: the pair permutation that gives each lane runs of 8 output columns
    return wn * TN + 32 * (f >> 1) + 8 * (j >> 2) + 4 * (f & 1) + (j & 3)


def test_stage_loads_fill_the_tile_once():
    lds = stage_lds()
    assert sorted(lds.values()) == sorted((k, 8 * c) for k in range(64) for c in range(CPR))
    # the swizzle reads only row bits 0-3, so a lane's chunk is the same for all 4 loads
    for w in range(NW):
        for lane in range(64):
            assert len({kswz(16 * i + 2 * w + (lane >> 5)) for i in range(4)}) == 1


@pytest.mark.parametrize("kind,nfrag", [("x", TM // 16), ("w", TN // 16)])
def test_fragment_reads_give_the_mfma_operand(kind, nfrag):
    lds = stage_lds()
    for wave in range(NW):
        for ks in range(2):
            for f in range(nfrag):
                lo = tr_read(lds, frag_addrs(kind, wave, ks, f, 0))
                hi = tr_read(lds, frag_addrs(kind, wave, ks, f, 1))
                for lane in range(64):
                    kq, j = lane >> 4, lane & 15
                    got = lo[lane] + hi[lane]
                    col = expected_col(kind, wave, f, j)
                    assert got == [(32 * ks + 8 * kq + e, col) for e in range(8)], (kind, wave, ks, f, lane, got)


def bank_passes(addrs):
    """LDS cycles a half-wave's 8-byte reads need: the largest number of
    distinct 8-byte words it asks of one bank"""
    worst = 0
    for half in range(2):
        per_bank = {}
        for a in addrs[32 * half:32 * half + 32]:
            for b in (a // 4, a // 4 + 1):
                per_bank.setdefault(b % 64, set()).add(a // 8)
        worst = max(worst, max(len(v) for v in per_bank.values()))
    return worst


def test_activation_reads_are_conflict_free_and_weight_reads_take_two_passes():
    for wave in range(NW):
        for ks in range(2):
            for h in range(2):
                for f in range(TM // 16):
                    assert bank_passes(frag_addrs("x", wave, ks, f, h)) == 1
                for f in range(TN // 16):
                    assert bank_passes(frag_addrs("w", wave, ks, f, h)) == 2
