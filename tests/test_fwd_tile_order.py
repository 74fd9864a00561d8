"""Host replay of the 256 x 256 forward kernel's tile order (k_fwd_lds4 in
csrc/gemm_fwd.hip): every live tile must be run exactly once,
by the persistent grid (one workgroup per compute unit, each looping over
its XCD's list, reversed in odd rounds) and by the one-tile-per-workgroup
grid (round 0 only), with and without the short tails left to the streaming
kernel. The formulas restate the kernel's: five parts (full m-tiles, then
partial last m-tiles with 4, 3, 2, 1 blocks of 64 rows), each split into
nx contiguous ranges, nx = 8 when the grid is a multiple of 8."""

import random

import pytest

LT = 256
PARTS = 5


def tiles_in_part(m, part):
    rem = m % LT
    if part == 0:
        return m // LT
    return int(rem != 0 and (rem + 63) // 64 == PARTS - part)


def prefix(counts, ntn):
    G = len(counts)
    cnt = [tiles_in_part(counts[e % G], e // G) * ntn for e in range(PARTS * G)]
    pre = [0]
    for c in cnt:
        pre.append(pre[-1] + c)
    return pre


def xcd_list_tile(pre, G, nparts, x, nx, i):
    for p in range(nparts):
        a = pre[p * G]
        n = pre[(p + 1) * G] - a
        q, r = divmod(n, nx)
        c = q + (1 if x < r else 0)
        if i < c:
            return a + x * q + min(x, r) + i
        i -= c
    return -1


def one_tile_grid(tiles):
    return (tiles + 8 * PARTS + 7) // 8 * 8


def run(counts, ntn, grid, persist, tail_cus):
    G = len(counts)
    pre = prefix(counts, ntn)
    nbig, allt = pre[3 * G], pre[PARTS * G]
    nparts = 3 if (tail_cus > 0 and nbig <= tail_cus and allt > tail_cus) else PARTS
    nx = 8 if grid % 8 == 0 else 1
    per = grid // nx
    seen = []
    for b in range(grid):
        xcd, j0 = b % nx, b // nx
        rnd = 0
        while True:
            j = per - 1 - j0 if rnd & 1 else j0
            tt = xcd_list_tile(pre, G, nparts, xcd, nx, rnd * per + j)
            if tt < 0:
                break
            assert 0 <= tt < pre[nparts * G]
            seen.append((tt, rnd))
            if not persist:
                break
            rnd += 1
    expect = pre[nparts * G]
    return seen, expect


def ragged(seed, G, lo, hi):
    rng = random.Random(seed)
    return [rng.randrange(lo, hi) for _ in range(G)]


CASES = [
    ("expert share shape", [11629, 3867, 2266, 1585, 1249, 961, 806, 639, 623, 561, 492, 447,
                            400, 347, 335, 324, 293, 289, 248, 245, 229, 224, 213, 188, 186,
                            181, 176, 173, 164, 153, 151, 145, 141, 138, 134, 123, 122, 117,
                            112, 111, 110, 109, 108, 106, 104, 98, 88, 86]),
    ("uniform 8 x 1024", [1024] * 8),
    ("ragged 8", ragged(1, 8, 0, 3000)),
    ("ragged 48", ragged(2, 48, 0, 1200)),
    ("ragged 300", ragged(3, 300, 0, 700)),
    ("all tails", [64, 1, 127, 128, 129, 192, 193, 255]),
    ("empty groups", [0, 0, 513, 0, 7, 0]),
]


@pytest.mark.parametrize("ntn", [1, 6, 16])
@pytest.mark.parametrize("name,counts", CASES)
@pytest.mark.parametrize("tails", [False, True])
def test_every_tile_once(name, counts, ntn, tails):
    cus = 256
    tail_cus = cus if tails else 0
    G = len(counts)
    bound = ((sum(counts) + LT - 1) // LT + G) * ntn
    for grid, persist in ((cus, True), (one_tile_grid(bound), False), (cus - 4, True)):
        seen, expect = run(counts, ntn, grid, persist, tail_cus)
        tiles = sorted(t for t, _ in seen)
        assert tiles == list(range(expect)), (name, grid, persist)


def test_snake_balances_the_expert_share():
    """The reversed odd rounds lower the most loaded compute unit's share of
    row blocks at the expert share's up-projection (6 n-tiles), by the cost
    a partial tile has: its 32-row blocks split over two wavefront rows."""
    counts = CASES[0][1]
    ntn, cus = 6, 256
    G = len(counts)
    pre = prefix(counts, ntn)

    def size(tt):
        e = max(i for i in range(PARTS * G) if pre[i] <= tt)
        m = counts[e % G]
        return LT if e < G else m % LT

    def cost(r):
        nb = (r + 31) // 32
        return 2 * ((nb + 1) // 2)

    def loads(snake):
        out = [0] * cus
        for b in range(cus):
            xcd, j0 = b % 8, b // 8
            rnd = 0
            while True:
                j = 31 - j0 if (snake and rnd & 1) else j0
                tt = xcd_list_tile(pre, G, PARTS, xcd, 8, rnd * 32 + j)
                if tt < 0:
                    break
                out[b] += cost(size(tt))
                rnd += 1
        return out

    plain, snake = loads(False), loads(True)
    assert sum(plain) == sum(snake)
    assert max(snake) < max(plain)
