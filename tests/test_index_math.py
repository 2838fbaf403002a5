"""Host model of the GEMM kernel's index arithmetic (csrc/gemm.hpp), checked
for every instantiated configuration without a GPU: the formulas are restated
here and each access is bounds-checked.

- workgroup -> logical tile (the XCD chunk dealing, with its contiguous tail)
  is a bijection onto [0, totalTiles) for every tile count;
- logical tile -> (bi, bj): the upper-triangle walk and the 4-row groups are
  bijections onto the tile grid they cover;
- the direct-to-LDS copy plan fills every 16-byte slot of a stage exactly once,
  inside the ring, with the swizzle the fragment reads assume, for 4 and 8
  waves and both operand layouts;
- fragment reads, epilogue strips and the mirror pass's transposed reads stay
  inside the LDS ring.
"""
import itertools

import pytest


def xcd_logical(b, tot, S):
    xcd, loc = b & 7, b >> 3
    full = tot // (8 * S)
    if loc < full * S:
        return (loc // S) * 8 * S + xcd * S + loc % S
    rest = tot - full * 8 * S
    q, r = rest >> 3, rest & 7
    return full * 8 * S + xcd * q + min(xcd, r) + (loc - full * S)


@pytest.mark.parametrize("S", [32, 64, 8 * 16, 8 * 56, 8 * 4, 8 * 6])
def test_xcd_mapping_is_a_bijection(S):
    for tot in list(range(1, 700)) + [8704, 8704 + 5, 57344, 4096, 640, 136 * 32 + 7]:
        got = sorted(xcd_logical(b, tot, S) for b in range(tot))
        assert got == list(range(tot)), (S, tot)


def upper_tile(t, T):
    i = 0
    while t >= T - i:
        t -= T - i
        i += 1
    return i, i + t


def group_tile(tt, tilesM, tilesN, GROUP=4):
    per_group = GROUP * tilesN
    g = tt // per_group
    first = g * GROUP
    gm = min(tilesM - first, GROUP)
    w = tt - g * per_group
    return first + w % gm, w // gm


@pytest.mark.parametrize("T", [1, 2, 3, 4, 6, 11, 16, 56])
def test_upper_triangle_walk(T):
    got = [upper_tile(t, T) for t in range(T * (T + 1) // 2)]
    assert sorted(got) == sorted((i, j) for i in range(T) for j in range(i, T))


@pytest.mark.parametrize("tilesM,tilesN", [(1, 1), (3, 3), (4, 16), (5, 7), (16, 16), (56, 16), (16, 56), (6, 8)])
def test_four_row_groups(tilesM, tilesN):
    got = [group_tile(tt, tilesM, tilesN) for tt in range(tilesM * tilesN)]
    assert sorted(got) == [(i, j) for i in range(tilesM) for j in range(tilesN)]


CONFIGS = [(BM, NW, ES, TR) for BM, NW, ES, TR in itertools.product((128, 256), (4, 8), (2, 4), (False, True))
           if not (BM == 128 and NW == 8) and not (ES == 4 and NW == 8)]


@pytest.mark.parametrize("BM,NW,ES,TRANS", CONFIGS)
def test_lds_plan_in_bounds(BM, NW, ES, TRANS):
    BN = BM
    EPC = 16 // ES
    CPR, NSTG = 8, 2
    BK = CPR * EPC
    WGN = WPO = NW // 2
    WTM = BM // 64
    WN = BN // WGN
    WTN = WN // 32
    STG = (BM + BN) * CPR
    NQ = STG // (64 * NW)
    assert NQ * 8 * WPO == BM
    CR = BM * ES // 16
    SROW, RS16 = WN + 8, WN * 2 + 32
    ring_bytes = NSTG * STG * 16
    assert NW * 32 * SROW * 4 <= ring_bytes
    if ES == 2:
        assert NW * 32 * SROW * 4 + NW * 32 * RS16 <= ring_bytes
    filled = [0] * STG
    for wid in range(NW):
        copies_l, cw = wid < WPO, wid % WPO
        region = 0 if copies_l else BM * CPR
        slot_off = region + cw * (BM // WPO) * CPR
        for q in range(NQ):
            for lane in range(64):
                slot = slot_off + q * 64 + lane
                assert 0 <= slot < STG
                filled[slot] += 1
                if not TRANS:
                    row = cw * (BM // WPO) + 8 * q + lane // 8
                    assert row < BM
                    swz = (row & 7) ^ ((row >> 3) & 1)
                    assert slot - region == row * CPR + lane % 8
                    # the chunk this lane copies is the logical chunk its slot holds
                    assert ((lane & 7) ^ (lane >> 3) ^ (q & 1)) == (lane % 8) ^ swz
                else:
                    slot_in = slot - region
                    krow = slot_in // CR
                    assert krow < BK
                    if ES == 2:
                        RPC = 64 // CR
                        assert krow == (cw * NQ + q) * RPC + lane // CR
                        # the K-row's swizzle (k & 3) depends on the copy index by parity only
                        assert (cw * NQ * RPC) % 4 == 0 and (2 * RPC) % 4 == 0
    assert all(f == 1 for f in filled)
    for wid in range(NW):
        wm, wn = wid // WGN, wid % WGN
        for r in range(WTM + WTN):
            rb = wm * (BM // 2) + r * 32 if r < WTM else wn * WN + (r - WTM) * 32
            assert rb + 31 < (BM if r < WTM else BN)
        assert (wid + 1) * 32 * SROW * 4 <= NW * 32 * SROW * 4
        if ES == 2:
            assert NW * 32 * SROW * 4 + (wid + 1) * 32 * RS16 <= ring_bytes
    NT, CW = 32 * WN // 8 // 64, WN // 8
    DRS = 64 // CW
    assert 64 % CW == 0 and NT * DRS == 32
    # mirror pass positions: every (strip column, 8-row group) once; 16-bit
    # strips: the 16-lane groups of one store share the columns (output rows)
    for mir16 in (True, False):
        seen = set()
        for t in range(NT):
            rows_of_store = {}
            for lane in range(64):
                if mir16:
                    jj, c8 = 16 * t + (lane & 15), 8 * (lane >> 4)
                else:
                    qq = t * 64 + lane
                    jj, c8 = qq % WN, (qq // WN) * 8
                assert jj < WN and c8 + 7 < 32
                seen.add((jj, c8))
                rows_of_store.setdefault(jj, set()).add(c8)
                if mir16:
                    L = lane & 15
                    assert jj - L == 16 * t  # a transposed read serves 16 consecutive columns at one c8
                    off = (c8 + (L >> 2)) * RS16 + (jj - L + 4 * (L & 3)) * 2
                    assert 0 <= off and off + 4 * RS16 + 8 <= 32 * RS16
            if mir16:
                assert all(v == {0, 8, 16, 24} for v in rows_of_store.values()) and len(rows_of_store) == 16
        assert len(seen) == WN * 4


@pytest.mark.parametrize("WTM,WTN", [(4, 4), (4, 2), (2, 2)])
def test_fragment_read_order(WTM, WTN):
    """The row-major read order is a permutation of the fragments, and each
    MFMA of the sequence (j fastest) finds both its fragments among the reads
    issued before the first MFMA that needs a later one."""
    ro = [0 if p == 0 else (WTM + p - 1 if p <= WTN else p - WTN) for p in range(WTM + WTN)]
    assert sorted(ro) == list(range(WTM + WTN))
    pos = {r: k for k, r in enumerate(ro)}
    need = 0
    for q in range(WTM * WTN):
        i, j = q // WTN, q % WTN
        need = max(need, pos[i], pos[WTM + j])
        # reads needed by the first q + 1 MFMAs are a prefix no longer than
        # the fragments those MFMAs touch
        touched = {i2 for i2 in range(q // WTN + 1)} | {WTM + j2 for j2 in range(min(q + 1, WTN))}
        assert need + 1 == len(touched)

