"""Bounds of every LDS and row-id access of the matrix-core kernels, replayed on the CPU.

The k=3 kernel (k_subm_lds) and the k=1 streaming kernel (k_linear_stream) compute their LDS
offsets from compile-time shapes and the lane index.  This test repeats that arithmetic for
every instantiated shape (the channel pairs the kernels are built for, both output widths) and
checks that each access lies inside its region and each row id it reads lies inside the tile:
the class of mistake that once sent a partial epilogue pass past the row-id table.  No GPU.
"""
import itertools

import pytest

SHAPES = [(ci, co) for ci in (32, 64, 128) for co in (16, 32, 64, 128)]
TAPS = 27


def lds_cfg(cin, cout):
    """LdsPick + LdsCfg of the k=3 kernel."""
    wc = 4 if cout >= 64 else cout // 16
    wr = 4 // wc
    nb = 8
    c = dict(CIN=cin, COUT=cout, NB=nb, WR=wr, WC=wc, WAVES=wr * wc, THREADS=wr * wc * 64,
             CPR=cin // 8, A_BLOCK=16 * cin, CS=cout // wc, KS=cin // 32, BPW=nb // wr)
    c["RPW"] = 16 // c["WAVES"]
    c["NCT"] = c["CS"] // 16
    c["ABUF"] = nb * c["A_BLOCK"] * 2
    c["OFF_G"] = 2 * c["ABUF"]
    c["OFF_P"] = c["OFF_G"] + TAPS * nb * 16 * 4
    c["SMEM"] = c["OFF_P"] + nb * 16 * 4
    return c


def swz(r, cpr):
    return ((r * cpr) >> 4) & (cpr - 1)


@pytest.mark.parametrize("cin,cout", SHAPES)
def test_k3_gather_and_fragment_offsets(cin, cout):
    C = lds_cfg(cin, cout)
    assert C["SMEM"] <= 160 * 1024
    cpr, nb = C["CPR"], C["NB"]
    # gather copies: each (wave, lane) of a block's pieces writes 16 bytes inside its block slot,
    # and together they cover every byte of the slot exactly once
    for b in range(nb):
        written = set()
        for wave in range(C["WAVES"]):
            if cin < 128:
                rpi = 64 // cpr
                pieces = 16 // rpi
                ppw = nb * pieces // C["WAVES"]
                for i in range(ppw):
                    piece = i * C["WAVES"] + wave
                    if piece // pieces != b:
                        continue
                    base = b * C["A_BLOCK"] * 2 + (piece % pieces) * 1024
                    for lane in range(64):
                        written.add(base + 16 * lane)
            else:
                base = b * C["A_BLOCK"] * 2 + wave * C["RPW"] * cin * 2
                for lane in range(64):
                    written.add(base + 16 * lane)
        lo, hi = b * C["A_BLOCK"] * 2, (b + 1) * C["A_BLOCK"] * 2
        assert written == set(range(lo, hi, 16))
    # fragment reads: lane l reads row l & 15, logical chunk (l >> 4) + 4 s, swizzled
    for lane, s in itertools.product(range(64), range(C["KS"])):
        r, chunk = lane & 15, (lane >> 4) + 4 * s
        assert chunk < cpr
        off = (r * cpr + (chunk ^ swz(r, cpr))) * 16
        assert 0 <= off and off + 16 <= C["A_BLOCK"] * 2
    # the swizzle is a permutation of each row's chunks (no two logical chunks collide)
    for r in range(16):
        assert sorted(c ^ swz(r, cpr) for c in range(cpr)) == list(range(cpr))


@pytest.mark.parametrize("cin,cout", SHAPES)
def test_k3_index_copies(cin, cout):
    C = lds_cfg(cin, cout)
    nb = C["NB"]
    tpc = 64 // (nb * 4)
    # up to 27 present taps, tpc per copy; lane serves tap sub = lane / (nb*4) of the copy
    for ntaps in range(1, TAPS + 1):
        q = 0
        while q < ntaps:
            for lane in range(64):
                sub, off = lane // (nb * 4), (lane % (nb * 4)) * 4
                if q + sub >= ntaps:
                    continue   # the copy's tap slot is absent: the lane is switched off
                dst = C["OFF_G"] + q * nb * 16 * 4 + sub * nb * 16 * 4 + off * 4
                assert C["OFF_G"] <= dst and dst + 16 <= C["OFF_P"]
            q += tpc
    # row ids: NB * 4 lanes x 4 ids
    assert C["OFF_P"] + nb * 4 * 16 <= C["SMEM"]


@pytest.mark.parametrize("cin,cout,out16", [(ci, co, o) for ci, co in SHAPES
                                            for o in (False, True)])
def test_k3_epilogue_passes(cin, cout, out16):
    C = lds_cfg(cin, cout)
    nb, wr, wc = C["NB"], C["WR"], C["WC"]
    esz = 2 if out16 else 4
    rowb = cout * esz
    chunks = rowb // 16
    swm = min(chunks, 16) - 1
    stage = C["OFF_P"]
    bpp_raw = stage // (16 * rowb)
    bpp = nb if bpp_raw >= nb else 8 if bpp_raw >= 8 else 4 if bpp_raw >= 4 else \
        2 if bpp_raw >= 2 else 1
    assert bpp_raw >= 1 and nb % bpp == 0
    for p0 in range(0, nb, bpp):
        # staging writes: lane's piece of channels col .. col + 3 of site row (l & 15)
        for wave in range(C["WAVES"]):
            wrow, wcol = wave // wc, wave % wc
            for bl in range(C["BPW"]):
                b = bl * wr + wrow
                if b < p0 or b >= p0 + bpp:
                    continue
                for c, lane in itertools.product(range(C["NCT"]), range(64)):
                    col = wcol * C["CS"] + c * 16 + 4 * (lane >> 4)
                    row = (b - p0) * 16 + (lane & 15)
                    byte = col * esz
                    dst = row * rowb + (((byte >> 4) ^ (row & swm)) << 4) + (byte & 15)
                    assert 0 <= dst and dst + 4 * esz <= bpp * 16 * rowb <= stage
                    assert (byte & 15) + 4 * esz <= 16       # the piece stays in one chunk
        # store loop: row ids read at p0 * 16 + row with row < bpp * 16
        for idx in range(0, bpp * 16 * chunks):
            row, ch = idx // chunks, idx % chunks
            assert p0 * 16 + row < nb * 16
            assert row * rowb + ((ch ^ (row & swm)) << 4) + 16 <= stage
    # group-norm reduction space (waves that share columns)
    if wr > 1:
        assert bpp * 16 * rowb + wr * cout * 2 * 4 <= C["OFF_P"]


@pytest.mark.parametrize("cin,cout,out16", [(ci, co, o) for ci, co in SHAPES
                                            for o in (False, True)])
def test_k1_stream_offsets(cin, cout, out16):
    esz = 2 if out16 else 4
    rowb = cout * esz
    tr = 64 if rowb >= 64 else 128
    nb = tr // 16
    wc = 4 if cout >= 64 else cout // 16
    waves, threads = 4, 256
    xbuf, obuf = tr * cin * 2, tr * rowb
    smem = 2 * xbuf + obuf
    assert smem <= 160 * 1024
    copies = xbuf // 1024
    assert copies % waves == 0 and obuf % (16 * threads) == 0
    stores = obuf // 16 // threads
    assert 1 <= stores <= 63
    rpi = 512 // cin
    cpw = copies // waves
    for wave, i in itertools.product(range(waves), range(cpw)):
        k = i * waves + wave
        for lane in range(64):
            r = k * rpi + lane // (cin // 8)
            assert r < tr and k * 1024 + 16 * lane < xbuf
    # residual copies into the staging tile: whole 1 KB copies inside it
    assert obuf % (1024 * waves) == 0
    chunks = rowb // 16
    swm = min(chunks, 16) - 1
    for it, t in itertools.product(range(stores), range(threads)):
        idx = t + it * threads
        row, ch = idx // chunks, idx % chunks
        assert row < tr and row * rowb + ((ch ^ (row & swm)) << 4) + 16 <= obuf
    assert nb * 16 == tr and wc * (4 // wc) == 4
