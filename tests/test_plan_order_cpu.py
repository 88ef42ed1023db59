"""The work order the one-launch path computes in place of the plan kernel's sort.

For a one-request batch each attention workgroup of the one-launch path works out the unit the
plan kernel gives its grid slot without the plan's ranking of the groups: it relies on a
group's work depending only on its split block gs and never growing with gs (block 0 holds
split 0 and the tree keys, then the full blocks, at most one partly filled block, then blocks
past the last split), so equal work forms runs of consecutive gs ordered by group index.  This
test states both orders in Python -- the plan's (rank groups by a unique key: has work, 64-key
tiles, 2047 - index; deal ranks to grid slots in snake order over the 8 XCD lanes) and the
closed form -- and checks that every grid slot gets the same unit, over random one-request
shapes, cache bounds and lengths (rejected lengths included).  The GPU tests then hold the
kernel's unit list to the plan kernel's byte for byte."""
import random

import pytest


def _geometry(rows, max_len, cus=256, tile_rows=64, min_chunk=256):
    """The host geometry of a one-request batch (make_geometry): split blocks of 2 on 64-row
    tiles, 4 on 128-row tiles."""
    bs_many = 2 if tile_rows == 64 else 4
    rt = -(-rows // tile_rows)
    S = 1
    if rt < 2 * cus and max_len > min_chunk:
        S = max(1, min(-(-cus // rt), -(-max_len // min_chunk)))
    chunk = max(64, -(-(-(-max_len // S) if max_len > 0 else 64) // 64) * 64)
    S = max(1, -(-max_len // chunk)) if max_len > 0 else 1
    bs = bs_many if (S >= 4 and rt >= 16) else 1
    bt = -(-rt // 4) if bs > 1 else rt
    groups = lambda: (-(-rt // bt)) * (-(-S // bs))
    while groups() < 8 and bt > 1:
        bt = (bt + 1) // 2
    units = -(-groups() // 8) * 8 * bt * bs
    return rt, S, chunk, bt, bs, units


def _splits(L, chunk, S):
    return 1 if L <= 0 else min(-(-L // chunk), S)


def _deal(u, per):
    x, k = u & 7, u >> 3
    rnd, i = divmod(k, per)
    return rnd * 8 + (7 - x if rnd & 1 else x), i


def _unit(gr, gs, i, L, RT, chunk, bt, bs, sb):
    ib = i // bs
    rt, sp = gr * bt + ib, gs * bs + (i - ib * bs)
    if rt < RT and sp < sb:
        k0 = sp * chunk
        return (rt, sp, sb, k0, min(k0 + chunk, L))
    return None


def plan_units(L, N, RT, S, chunk, bt, bs, U, max_len):
    """The plan kernel's order: sort the groups by their key, deal the ranks."""
    ok = 0 <= L <= max_len
    sb = _splits(L, chunk, S)
    GR, GS = -(-RT // bt), -(-S // bs)
    keys = []
    for g in range(GR * GS):
        gs = g % GS
        w = -1
        if ok:
            for sp in range(gs * bs, min(gs * bs + bs, sb)):
                left = L - sp * chunk
                w = max(w, 0) + (max(left, 0) if left < chunk else chunk) + (N if sp == 0 else 0)
        tiles = 0 if w < 0 else (w + 63) // 64
        keys.append(((w >= 0) << 31) | (min(tiles, 0xfffff) << 11) | (2047 - g))
    order = sorted(range(GR * GS), key=lambda g: -keys[g])
    out = []
    for u in range(U):
        p, i = _deal(u, bt * bs)
        un = None
        if ok and p < len(order):
            gr, gs = divmod(order[p], GS)
            un = _unit(gr, gs, i, L, RT, chunk, bt, bs, sb)
        out.append(un)
    return out


def closed_form_units(L, N, RT, S, chunk, bt, bs, U, max_len):
    """The one-launch path's order: the run of equal work that holds gs = p / GR."""
    ok = 0 <= L <= max_len
    sb = _splits(L, chunk, S)
    GR, GS = -(-RT // bt), -(-S // bs)
    E = -(-sb // bs)                       # blocks with a split
    span = bs * chunk
    out = []
    for u in range(U):
        p, i = _deal(u, bt * bs)
        un = None
        if ok and p < GR * GS:
            c = p // GR
            if c == 0:
                lo = hi = 0
            elif c < E:
                fe = E - 1 if L - (E - 1) * span > span - 64 else E - 2
                lo, hi = (1, fe) if c <= fe else (E - 1, E - 1)
            else:
                lo, hi = E, GS - 1
            m = hi - lo + 1
            q = p - GR * lo
            un = _unit(q // m, lo + q % m, i, L, RT, chunk, bt, bs, sb)
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
            RT, S, chunk, bt, bs, U = _geometry(rows, max_len, tile_rows=tile_rows)
            a = plan_units(L, N, RT, S, chunk, bt, bs, U, max_len)
            b = closed_form_units(L, N, RT, S, chunk, bt, bs, U, max_len)
            assert a == b, (rows, N, max_len, L, tile_rows)
            n += 1
    assert n > 4000


@pytest.mark.parametrize("wrong", ["ties_by_split", "no_partial_run"])
def test_a_plausible_mistake_is_caught(wrong):
    """Two wrong closed forms (ties broken split-major; a partly filled last block kept in the
    run of full blocks) disagree with the plan on some shape."""
    def bad_units(L, N, RT, S, chunk, bt, bs, U, max_len):
        ok = 0 <= L <= max_len
        sb = _splits(L, chunk, S)
        GR, GS = -(-RT // bt), -(-S // bs)
        E = -(-sb // bs)
        out = []
        for u in range(U):
            p, i = _deal(u, bt * bs)
            un = None
            if ok and p < GR * GS:
                if wrong == "ties_by_split":
                    gs, gr = divmod(p, GR)
                else:
                    c = p // GR
                    lo, hi = (0, 0) if c == 0 else ((1, E - 1) if c < E else (E, GS - 1))
                    m = hi - lo + 1
                    q = p - GR * lo
                    gr, gs = q // m, lo + q % m
                un = _unit(gr, gs, i, L, RT, chunk, bt, bs, sb)
            out.append(un)
        return out
    for rows, N, max_len, L in _cases():
        RT, S, chunk, bt, bs, U = _geometry(rows, max_len)
        if bad_units(L, N, RT, S, chunk, bt, bs, U, max_len) != plan_units(L, N, RT, S, chunk, bt, bs, U, max_len):
            return
    pytest.fail(f"the mistake {wrong} was not caught")
