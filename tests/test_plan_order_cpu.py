"""The work order the one-launch path computes in place of the plan kernel's sort.

For a one-request batch each attention workgroup of the one-launch path works out the unit the
plan kernel gives its grid slot without the plan's ranking of the groups: it relies on a
group's work depending only on its split block gs and never growing with gs.  Split 0 does the
tree's tiles too.  A tree of more than one 64-key tile has places of its own in the range the
splits cut (its whole tiles, then the committed keys), so the full blocks, block 0 among them,
come first; a one-tile tree has none and block 0, its tree keys on top of a full share, comes
alone before the full blocks.  Then come at most one partly filled block and the blocks past
the last split; equal work forms runs of consecutive gs ordered by group index.  This test
states both orders in Python -- the plan's (rank groups by a unique key: has work, 64-key
tiles, 2047 - index; deal ranks to grid slots in snake order over the 8 XCD lanes) and the
closed form -- and checks that every grid slot gets the same unit, over random one-request
shapes, cache bounds and lengths (rejected lengths included).  The GPU tests then hold the
kernel's unit list to the plan kernel's byte for byte."""
import random

import pytest


def _tree_keys(N):
    """Places of the tree in the range the splits cut: its whole 64-key tiles for trees of more than
    one tile, else none (make_geometry)."""
    return 64 * -(-N // 64) if N > 64 else 0


def _geometry(rows, max_len, N, cus=256, tile_rows=64, min_chunk=256):
    """The host geometry of a one-request batch (make_geometry): splits cut the tree's places then
    the committed keys; split blocks of 2 on 64-row tiles, 4 on 128-row tiles."""
    bs_many = 2 if tile_rows == 64 else 4
    rt = -(-rows // tile_rows)
    T = _tree_keys(N)
    lv = max_len + T
    S = 1
    if rt < 2 * cus and max_len > min_chunk:
        S = max(1, min(-(-cus // rt), -(-lv // min_chunk)))
    chunk = max(T, 64, -(-(-(-lv // S)) // 64) * 64) if lv > 0 else 64
    S = max(1, -(-lv // chunk))
    bs = bs_many if (S >= 4 and rt >= 16) else 1
    bt = -(-rt // 4) if bs > 1 else rt
    groups = lambda: (-(-rt // bt)) * (-(-S // bs))
    while groups() < 8 and bt > 1:
        bt = (bt + 1) // 2
    units = -(-groups() // 8) * 8 * bt * bs
    return rt, S, chunk, bt, bs, units


def _splits(L, T, chunk, S):
    return max(1, min(-(-(max(L, 0) + T) // chunk), S))


def _deal(u, per):
    x, k = u & 7, u >> 3
    rnd, i = divmod(k, per)
    return rnd * 8 + (7 - x if rnd & 1 else x), i


def _unit(gr, gs, i, L, T, RT, chunk, bt, bs, sb):
    ib = i // bs
    rt, sp = gr * bt + ib, gs * bs + (i - ib * bs)
    if rt < RT and sp < sb:
        v0 = sp * chunk - T
        k0 = max(v0, 0)
        return (rt, sp, sb, k0, max(min(v0 + chunk, L), k0))
    return None


def plan_units(L, N, RT, S, chunk, bt, bs, U, max_len):
    """The plan kernel's order: sort the groups by their key (work in virtual keys, plus N for
    split 0 when the tree has no places), deal the ranks."""
    ok = 0 <= L <= max_len
    T = _tree_keys(N)
    sb = _splits(L, T, chunk, S)
    GR, GS = -(-RT // bt), -(-S // bs)
    lv = max(L, 0) + T
    keys = []
    for g in range(GR * GS):
        gs = g % GS
        w = -1
        if ok:
            for sp in range(gs * bs, min(gs * bs + bs, sb)):
                left = lv - sp * chunk
                w = max(w, 0) + (max(left, 0) if left < chunk else chunk) + (N if sp == 0 and T == 0 else 0)
        tiles = 0 if w < 0 else (w + 63) // 64
        keys.append(((w >= 0) << 31) | (min(tiles, 0xfffff) << 11) | (2047 - g))
    order = sorted(range(GR * GS), key=lambda g: -keys[g])
    out = []
    for u in range(U):
        p, i = _deal(u, bt * bs)
        un = None
        if ok and p < len(order):
            gr, gs = divmod(order[p], GS)
            un = _unit(gr, gs, i, L, T, RT, chunk, bt, bs, sb)
        out.append(un)
    return out


def _runs(lv, sb, bs, chunk, GS, c, alone):
    """The run of equal work holding split block c: block 0 alone (a tree without places), the
    full blocks up to fe, the partial block, or the blocks past the last split."""
    E = -(-sb // bs)                       # blocks with a split
    span = bs * chunk
    fe = E - 1 if lv - (E - 1) * span > span - 64 else E - 2
    if alone and c == 0:
        return 0, 0
    if c <= fe:
        return (1 if alone else 0), fe
    if c < E:
        return E - 1, E - 1
    return E, GS - 1


def closed_form_units(L, N, RT, S, chunk, bt, bs, U, max_len):
    """The one-launch path's order: the run of equal work that holds gs = p / GR."""
    ok = 0 <= L <= max_len
    T = _tree_keys(N)
    sb = _splits(L, T, chunk, S)
    GR, GS = -(-RT // bt), -(-S // bs)
    lv = max(L, 0) + T
    out = []
    for u in range(U):
        p, i = _deal(u, bt * bs)
        un = None
        if ok and p < GR * GS:
            lo, hi = _runs(lv, sb, bs, chunk, GS, p // GR, T == 0)
            m = hi - lo + 1
            q = p - GR * lo
            un = _unit(q // m, lo + q % m, i, L, T, RT, chunk, bt, bs, sb)
        out.append(un)
    return out


def _cases():
    rng = random.Random(7)
    shapes = [(4096, 64, 4096), (64, 1, 32768), (448, 7, 4096), (2560, 40, 2999), (8192, 128, 8192), (480, 10, 3000),
              (1024, 16, 32768), (16384, 256, 4096), (16384, 256, 32768), (1000, 125, 5000)]
    while len(shapes) < 400:
        N = rng.randint(1, 256)
        rows = N * rng.choice([1, 2, 8, 16, 48, 64, 128])
        if rows <= 16384:
            shapes.append((rows, N, rng.choice([0, 1, 64, 65, 256, 257, 1000, 4096, 8192, rng.randint(0, 40000)])))
    for rows, N, max_len in shapes:
        for L in sorted({0, 1, max_len, max(0, max_len - 1), max_len // 2, max_len + 1, -1,
                         rng.randint(0, max(max_len, 1))}):
            yield rows, N, max_len, L


def test_closed_form_equals_plan_order():
    n = 0
    for rows, N, max_len, L in _cases():
        for tile_rows in (64, 128):
            RT, S, chunk, bt, bs, U = _geometry(rows, max_len, N, tile_rows=tile_rows)
            a = plan_units(L, N, RT, S, chunk, bt, bs, U, max_len)
            b = closed_form_units(L, N, RT, S, chunk, bt, bs, U, max_len)
            assert a == b, (rows, N, max_len, L, tile_rows)
            n += 1
    assert n > 4000


@pytest.mark.parametrize("wrong", ["ties_by_split", "no_partial_run", "block0_alone", "block0_joined",
                                   "tree_without_places"])
def test_a_plausible_mistake_is_caught(wrong):
    """Wrong closed forms disagree with the plan on some shape: ties broken split-major; a partly
    filled last block kept in the run of full blocks; block 0 ranked as a run of its own also when
    the tree has places; block 0 ranked with the full blocks also when its tree keys come on top;
    the units of a tree with places cut over the committed keys alone."""
    def bad_units(L, N, RT, S, chunk, bt, bs, U, max_len):
        ok = 0 <= L <= max_len
        T = 0 if wrong == "tree_without_places" else _tree_keys(N)
        sb = _splits(L, T, chunk, S)
        GR, GS = -(-RT // bt), -(-S // bs)
        lv = max(L, 0) + T
        E = -(-sb // bs)
        alone = {"block0_alone": True, "block0_joined": False}.get(wrong, T == 0)
        out = []
        for u in range(U):
            p, i = _deal(u, bt * bs)
            un = None
            if ok and p < GR * GS:
                c = p // GR
                if wrong == "ties_by_split":
                    gs, gr = divmod(p, GR)
                else:
                    if wrong == "no_partial_run":
                        lo, hi = _runs(lv, sb, bs, chunk, GS, c, alone)
                        if c < E and (not alone or c > 0):
                            lo, hi = (1 if alone else 0), E - 1
                    else:
                        lo, hi = _runs(lv, sb, bs, chunk, GS, c, alone)
                    m = hi - lo + 1
                    q = p - GR * lo
                    gr, gs = q // m, lo + q % m
                un = _unit(gr, gs, i, L, T, RT, chunk, bt, bs, sb)
            out.append(un)
        return out
    for rows, N, max_len, L in _cases():
        for tile_rows in (64, 128):
            RT, S, chunk, bt, bs, U = _geometry(rows, max_len, N, tile_rows=tile_rows)
            if bad_units(L, N, RT, S, chunk, bt, bs, U, max_len) != plan_units(L, N, RT, S, chunk, bt, bs, U, max_len):
                return
    pytest.fail(f"the mistake {wrong} was not caught")
