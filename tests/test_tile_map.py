"""CPU model of the grouped GEMMs' workgroup -> tile mapping.

The kernels map blockIdx.x to a tile with integer arithmetic only
(csrc/gemm_tile.h: group_tile_prefix, xcd_tile, band_order, group_band_order,
resolve_tile and the launch grids in csrc/gemm_bf16.hip). This file restates that arithmetic
in Python and checks, over many group layouts and CU counts, what the
kernels rely on:

* every tile of every group is computed exactly once, and surplus
  workgroups find no tile;
* a RAG_M group's tiles are contiguous in the tile order, and a group of at
  most 12 m-tiles is one band: its n-tiles advance together over all its
  m-tiles;
* with the split-K of each XCD's last, partial round of tiles, every split
  tile gets exactly its S parts, each once; its counter slot and its partial
  sums stay inside the workspace and no two tiles share them; the parts'
  k-step ranges cover the tile's k-steps exactly;
* the group prefix gives the total tile count for every G up to the
  library's limit of 1024 groups (its 256 threads cover 4 groups each).

Pure integer arithmetic on the CPU: no GPU is involved.
"""
import random

import pytest

TAIL_CUS_MAX = 32          # the library sizes the split-K workspace for 32 CUs per XCD
BAND_M = 8                 # m-tiles per band
GROUP_BAND_MAX = 12        # a RAG_M group of at most this many m-tiles is one band


def cdiv(a, b):
    return (a + b - 1) // b


def group_tile_prefix(counts, BM):
    """s_tiles[0..G]: the kernel's 256 threads x 4 slots, slot i = group 4*tid + i."""
    G = len(counts)
    assert G <= 1024
    slot = [cdiv(counts[g], BM) if g < G else 0 for g in range(1024)]
    s_tiles = [None] * (G + 1)
    # per thread: exclusive prefix of its 4 slots; per wave: shuffle scan; waves summed in order
    per_thread = [sum(slot[4 * t:4 * t + 4]) for t in range(256)]
    incl = []
    run = 0
    for t in range(256):
        run += per_thread[t]
        incl.append(run)
    for t in range(256):
        ex = incl[t] - per_thread[t]
        for i in range(4):
            gi = 4 * t + i
            if gi < G:
                s_tiles[gi] = ex
            ex += slot[gi]
    s_tiles[G] = incl[255]      # written by the last thread
    return s_tiles


def xcd_tile(bid, valid):
    x, i = bid & 7, bid >> 3
    lo, hi = x * valid // 8, (x + 1) * valid // 8
    return lo + i if lo + i < hi else -1


def band_order(L, mt_total, nt):
    band = L // (BAND_M * nt)
    within = L - band * BAND_M * nt
    rem = mt_total - band * BAND_M
    h = rem if rem < BAND_M else BAND_M
    return band * BAND_M + within % h, within // h


def group_band_order(u, mtg, nt):
    if mtg <= GROUP_BAND_MAX:
        return u % mtg, u // mtg
    return band_order(u, mtg, nt)


def find_group(s_tiles, G, mt):
    lo, hi = 0, G - 1
    while lo < hi:
        mid = (lo + hi + 1) >> 1
        if s_tiles[mid] <= mt:
            lo = mid
        else:
            hi = mid - 1
    return lo


def resolve_rag_m(bid, offsets, BM, BNo, N, tail_cus, s_tiles, with_L=False):
    """One workgroup of a RAG_M launch: (g, m0, n0, S, part, slot, item) or None
    (with_L: also the logical tile index).
    s_tiles: group_tile_prefix of the offsets (every workgroup computes the
    same prefix, so the model computes it once per launch)."""
    G = len(offsets) - 1
    nt = cdiv(N, BNo)
    total = s_tiles[G]
    S, part, slot, item = 1, 0, 0, 0
    if tail_cus:
        V = total * nt
        x, i, cus = bid & 7, bid >> 3, tail_cus
        lo = x * V // 8
        n = (x + 1) * V // 8 - lo
        r = n % cus
        full = n - r
        if r > 0 and 2 * r <= cus:
            Sx = cus // r if cus // r < 4 else 4
            if i < full:
                L = lo + i
            elif i < full + r * Sx:
                j = (i - full) // Sx
                L = lo + full + j
                S, part = Sx, (i - full) % Sx
                slot, item = x * cus + j, x * cus + j * Sx
            else:
                return None
        else:
            if i >= n:
                return None
            L = lo + i
    else:
        L = xcd_tile(bid, total * nt)
        if L < 0:
            return None
    g = find_group(s_tiles, G, L // nt)
    first = s_tiles[g]
    mt, ntile = group_band_order(L - first * nt, s_tiles[g + 1] - first, nt)
    r = (g, mt * BM, ntile * BNo, S, part, slot, item)
    return r + (L,) if with_L else r


def grid_rag_m(max_rows, G, BM, BNo, N, tail_cus):
    nt = cdiv(N, BNo)
    tiles = (cdiv(max_rows, BM) + G) * nt
    nb = cdiv(tiles, 8) * 8
    return nb + (8 * tail_cus if tail_cus else 0)


def expected_tiles(offsets, BM, BNo, N):
    out = set()
    for g in range(len(offsets) - 1):
        M = offsets[g + 1] - offsets[g]
        for m in range(cdiv(M, BM)):
            for n in range(cdiv(N, BNo)):
                out.add((g, m * BM, n * BNo))
    return out


def check_rag_m(offsets, max_rows, BM, BNo, N, tail_cus):
    G = len(offsets) - 1
    nb = grid_rag_m(max_rows, G, BM, BNo, N, tail_cus)
    s_tiles = group_tile_prefix([offsets[g + 1] - offsets[g] for g in range(G)], BM)
    parts = {}
    for bid in range(nb):
        r = resolve_rag_m(bid, offsets, BM, BNo, N, tail_cus, s_tiles)
        if r is None:
            continue
        g, m0, n0, S, part, slot, item = r
        parts.setdefault((g, m0, n0), []).append((S, part, slot, item))
    assert set(parts) == expected_tiles(offsets, BM, BNo, N)
    used_slots, used_items = set(), set()
    for tile, items in parts.items():
        S = items[0][0]
        assert all(it[0] == S for it in items)
        assert sorted(it[1] for it in items) == list(range(S)), (tile, items)
        if S > 1:
            slots = {it[2] for it in items}
            bases = {it[3] for it in items}
            assert len(slots) == 1 and len(bases) == 1
            slot, base = slots.pop(), bases.pop()
            # counters: 8 * cus ints; partials: 8 * cus items of 256 KiB
            assert 0 <= slot < 8 * tail_cus <= 8 * TAIL_CUS_MAX
            assert 0 <= base and base + S <= 8 * tail_cus
            assert slot not in used_slots
            used_slots.add(slot)
            for p in range(S):
                assert base + p not in used_items
                used_items.add(base + p)
    return parts


def split_k_ranges(nk, S):
    """k-steps of each part, as the kernel computes them."""
    per = cdiv(nk, S)
    out = []
    for part in range(S):
        kbase = per * part
        n = 0 if kbase >= nk else min(nk - kbase, per)
        out.append((kbase, n))
    return out


@pytest.mark.parametrize("cus", [1, 2, 3, 5, 8, 13, 16, 24, 30, 31, 32])
def test_tail_split_covers_every_tile_once(cus):
    """One group of V m-tiles (nt = 1), V = 0..299: every count of tiles per
    XCD modulo the CUs, with and without the tail split."""
    for V in range(0, 300):
        offsets = [0, V * 256]
        check_rag_m(offsets, V * 256, 256, 256, 256, cus)
        if cus == 32:
            check_rag_m(offsets, V * 256, 256, 256, 256, 0)


def test_tail_split_on_ragged_groups():
    rng = random.Random(7)
    for _ in range(150):
        G = rng.randint(1, 40)
        counts = [rng.choice([0, rng.randint(1, 600), rng.randint(1, 3000)]) for _ in range(G)]
        offsets = [0]
        for c in counts:
            offsets.append(offsets[-1] + c)
        max_rows = offsets[-1] + rng.randint(0, 500)
        N = 8 * rng.randint(1, 300)
        cus = rng.choice([0, 1, 4, 8, 16, 32])
        for BNo in (128, 256):
            check_rag_m(offsets, max_rows, 256, BNo, N, cus)


def test_split_k_parts_cover_the_k_steps():
    for nk in range(0, 80):
        for S in (1, 2, 3, 4):
            covered = []
            for kbase, n in split_k_ranges(nk, S):
                covered.extend(range(kbase, kbase + n))
            assert covered == list(range(nk))


def resolve_rag_k(bid, G, M, N, BM, BN):
    nt = cdiv(N, BN)
    per = cdiv(M, BM) * nt
    x, i = bid & 7, bid >> 3
    lo = x * per // 8
    n = (x + 1) * per // 8 - lo
    if n == 0 or i >= n * G:
        return None
    g = i // n
    Lg = lo + i % n
    mt, ntile = band_order(Lg, cdiv(M, BM), nt)
    return g, mt * BM, ntile * BN


@pytest.mark.parametrize("G,M,N", [(1, 256, 256), (8, 28672, 4096), (8, 4096, 14336),
                                   (256, 4096, 7168), (3, 300, 72), (1024, 256, 8), (5, 8, 8)])
def test_weight_gradient_map_covers_every_tile_once(G, M, N):
    nt = cdiv(N, 256)
    per = cdiv(M, 256) * nt
    nb = 8 * G * cdiv(per, 8)
    seen = {}
    for bid in range(nb):
        r = resolve_rag_k(bid, G, M, N, 256, 256)
        if r is not None:
            seen[r] = seen.get(r, 0) + 1
    want = {(g, m * 256, n * 256) for g in range(G) for m in range(cdiv(M, 256))
            for n in range(nt)}
    assert set(seen) == want and all(v == 1 for v in seen.values())


@pytest.mark.parametrize("G", [1, 255, 256, 257, 1023, 1024])
def test_group_prefix_total_up_to_1024_groups(G):
    rng = random.Random(G)
    counts = [rng.randint(0, 700) for _ in range(G)]
    s = group_tile_prefix(counts, 256)
    want = [0]
    for c in counts:
        want.append(want[-1] + cdiv(c, 256))
    assert s == want


@pytest.mark.parametrize("seed", range(6))
def test_rag_m_groups_are_contiguous_and_small_groups_one_band(seed):
    rng = random.Random(seed)
    G, BM, BNo, N = rng.choice([(9, 256, 256, 1024), (40, 256, 128, 2048), (256, 256, 256, 7168)])
    counts = [rng.choice([0, rng.randrange(1, 600), rng.randrange(2000, 3300)]) for _ in range(G)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    s_tiles = group_tile_prefix(counts, BM)
    nt = cdiv(N, BNo)
    order = {}
    for bid in range(grid_rag_m(offsets[-1], G, BM, BNo, N, 0)):
        r = resolve_rag_m(bid, offsets, BM, BNo, N, 0, s_tiles, with_L=True)
        if r is not None:
            order[r[-1]] = r[:3]
    assert sorted(order) == list(range(s_tiles[G] * nt))
    for g in range(G):
        Ls = sorted(L for L, t in order.items() if t[0] == g)
        mtg = cdiv(counts[g], BM)
        assert len(Ls) == mtg * nt
        if Ls:
            assert Ls == list(range(Ls[0], Ls[0] + len(Ls)))
        if 0 < mtg <= GROUP_BAND_MAX:
            # consecutive tiles: all m-tiles of n-tile 0, then of n-tile 1, ...
            seq = [order[L][1:] for L in Ls]
            assert seq == [(m * BM, n * BNo) for n in range(nt) for m in range(mtg)]
