"""Model check of the kernels' LDS tile layouts (CPU only).

The kernels stage 16-byte chunks of K, V, Q and dO rows in LDS with
direct-to-LDS loads and read them back in two patterns:

  * fragment reads (ds_read_b128): lane (c, g) of a wave reads chunk 2t + g of
    tile row sigma(c) (+ 32 hh), 16 lanes served per cycle;
  * transposed reads (ds_read_b64_tr_b16): in 16-lane group G = 2 gg + h,
    source lane s reads 8 bytes of chunk (d / 16)(s & 1) + 2 i + h, half
    (s >> 1) & 1, of row 8 gg + e0 + s / 4 (+ a multiple of 16), 32 lanes per
    cycle.

Each layout places row r's chunk k at an address of its own; this file
re-derives those addresses from the layout definitions (the XOR swizzles of
the forward's K and V tiles and of the backward's two-way tiles; the padded
288-byte row slots of the d = 128 dK/dV kernel and its 272-byte V rows) and
checks, under the LDS model of 64 four-byte banks, that every read pattern is
free of bank conflicts (the kernels' SQ_LDS_BANK_CONFLICT counters read 0),
that every data chunk lands exactly once, that the padded layouts' spare
bytes are the only positions the loads fill with out-of-range zeros, and
that no read leaves its tile.  A planted slip (the unshifted 288-byte slot)
must fail.
"""
from __future__ import annotations

import pytest

BANKS = 64


def sigma32(s):
    """Key-slot order: bits 2 and 3 swapped."""
    return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1)


def conflict_degree(addrs, width):
    """Largest number of distinct dwords that one bank must serve for these lane addresses."""
    banks = {}
    for a in addrs:
        for off in range(0, width, 4):
            dw = (a + off) // 4
            banks.setdefault(dw % BANKS, set()).add(dw)
    return max(len(v) for v in banks.values())


def worst(addrs, width, lanes_per_cycle):
    return max(conflict_degree(addrs[i:i + lanes_per_cycle], width) for i in range(0, 64, lanes_per_cycle))


# ---- layouts: byte address of chunk k (16 bytes) of tile row r ------------------------------

def xor_layout(D, swz):
    rowb = 2 * D
    return lambda r, k: r * rowb + 16 * (k ^ swz(r))


def k_swz(D):     # forward K tile (rows in key-slot order)
    return (lambda r: r & 15) if D == 128 else (lambda r: ((r & 31) ^ ((r & 31) >> 3)) & 7)


def v_swz(D):     # forward V tile
    return (lambda r: 2 * (r & 3)) if D == 128 else (lambda r: 2 * ((r >> 1) & 1))


def dual_swz(D):  # backward tiles read both ways
    if D == 128:
        return lambda r: ((r & 15 & 3) << 1) | (((r & 15) >> 2) & 1) | ((r & 15) & 8)
    return lambda r: ((((r & 15) >> 1) & 1) << 1) | (((r & 15) >> 2) & 1) | (((r & 15) >> 1) & 4)


SLOT = 288


def pad_row(r):   # d = 128 dK/dV Q/dO tiles
    return SLOT * r + 16 * ((r >> 3) & 1)


def pad_layout(r, k):
    return pad_row(r) + 16 * k


# ---- read patterns --------------------------------------------------------------------------

def fragment_addrs(layout, D, hh, t, rowperm):
    out = []
    for lane in range(64):
        c, g = lane & 31, lane >> 5
        out.append(layout(32 * hh + rowperm(c), 2 * t + g))
    return out


def transposed_addrs(layout, D, base_row, i):
    out = []
    for lane in range(64):
        G, s = lane >> 4, lane & 15
        h, gg = G & 1, G >> 1
        r = base_row + 8 * gg + (s >> 2)
        lc = (D // 16) * (s & 1) + 2 * i + h
        out.append(layout(r, lc) + 8 * ((s >> 1) & 1))
    return out


def check_both_patterns(layout, D, rowperm, rows=64):
    frag = max(worst(fragment_addrs(layout, D, hh, t, rowperm), 16, 16)
               for hh in range(rows // 32) for t in range(D // 16))
    tr = max(worst(transposed_addrs(layout, D, kb + e0, i), 8, 32)
             for kb in range(0, rows, 16) for e0 in (0, 4) for i in range(D // 32))
    return frag, tr


@pytest.mark.parametrize("D", [64, 128])
def test_forward_k_fragments_and_v_transposed_reads_are_conflict_free(D):
    # K: rows in key-slot order, lane c reads row c; V: transposed reads of consecutive key rows
    kf, _ = check_both_patterns(xor_layout(D, k_swz(D)), D, lambda c: c)
    _, vt = check_both_patterns(xor_layout(D, v_swz(D)), D, lambda c: c)
    assert (kf, vt) == (1, 1)


@pytest.mark.parametrize("D", [64, 128])
def test_backward_two_way_tiles_are_conflict_free_both_ways(D):
    assert check_both_patterns(xor_layout(D, dual_swz(D)), D, sigma32) == (1, 1)


def test_padded_dkdv_tiles_are_conflict_free_both_ways():
    assert check_both_patterns(pad_layout, 128, sigma32) == (1, 1)


def test_a_slot_without_the_shift_would_conflict():
    plain = lambda r, k: SLOT * r + 16 * k
    frag, tr = check_both_patterns(plain, 128, sigma32)
    assert max(frag, tr) > 1


def test_padded_v_rows_are_conflict_free():
    for w in range(8):
        for t in range(8):
            addrs = [(32 * w + (l & 31)) * 272 + 16 * (2 * t + (l >> 5)) for l in range(64)]
            assert worst(addrs, 16, 16) == 1


def padded_source(pos, pad):
    """The padded tile's load source for tile byte `pos` (row-major 256-byte rows), or pad."""
    r = pos // SLOT
    k = pos - pad_row(r)
    return r * 256 + k if 0 <= k < 256 else pad


def test_padded_tile_loads_place_every_chunk_once_and_fill_only_the_gaps():
    PAD = 64 * 256
    seen = {}
    for pos in range(0, 64 * SLOT, 16):
        src = padded_source(pos, PAD)
        if src == PAD:
            continue
        r, k = divmod(src, 256)
        assert (r, k // 16) not in seen
        seen[(r, k // 16)] = pos
    assert len(seen) == 64 * 16
    # each chunk sits where the reads look for it, and the pad offset lies past any tile's range
    for (r, k), pos in seen.items():
        assert pos == pad_layout(r, k)
    assert PAD >= 64 * 256
    # 288 = 256 + 32: two spare chunks per row
    assert 64 * SLOT // 16 - len(seen) == 64 * 2


def test_padded_v_rows_place_every_chunk_once():
    seen = set()
    for pos in range(0, 256 * 272, 16):
        r, k = divmod(pos, 272)
        if k < 256:
            assert (r, k // 16) not in seen
            seen.add((r, k // 16))
    assert len(seen) == 256 * 16


def test_every_read_stays_inside_its_tile():
    tile = 64 * SLOT
    for hh in range(2):
        for t in range(8):
            assert all(0 <= a and a + 16 <= tile for a in fragment_addrs(pad_layout, 128, hh, t, sigma32))
    for kb in range(0, 64, 16):
        for e0 in (0, 4):
            for i in range(4):
                assert all(0 <= a and a + 8 <= tile for a in transposed_addrs(pad_layout, 128, kb + e0, i))
    for D in (64, 128):
        for layout in (xor_layout(D, dual_swz(D)), xor_layout(D, k_swz(D)), xor_layout(D, v_swz(D))):
            end = 64 * 2 * D
            assert all(0 <= layout(r, k) < end for r in range(64) for k in range(D // 8))
