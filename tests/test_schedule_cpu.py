"""Host-side check of the tile kernels' schedules (no GPU): for every product shape below, the schedule the
planner returns (sgd_gemm_plan) is run through the work partition the product kernel and its stream-K fixup
derive from it, and must cover every (tile, 16-deep k-slice) exactly once, give each tile shared between
blocks a fixup slot list that is the pieces' slots in k order, and meet the kernel's preconditions (grouped
ranges inside an XCD's run of blocks, 32-bit range arithmetic, the fixup's 1024-slot list).

The partition below restates the kernel's indexing: the stream-K range of block (or block group) q is
[q * S / Q, (q + 1) * S / Q) of the flattened (tile or column group, k-slice) space; whole tiles go
round-robin first; a range's first piece goes to slot 2b and its last to 2b + 1; wide unpermuted products
order their tiles in bands of 8 tile columns; one-block-per-tile launches with ragged edges put each XCD
run's share of the edge tiles last.
"""
import random

import pytest

import sgd_cnns_amd as S

FORMS = {"nt": (0, 0), "tn": (1, 1), "nn": (0, 1), "tt": (1, 0)}
BAND = 8


def sk_start(b, s, g):
    return b * s // g


def sk_block_of(x, s, g):
    b = (x * g + g - 1) // s
    while b > 0 and sk_start(b, s, g) > x:
        b -= 1
    while b + 1 < g and sk_start(b + 1, s, g) <= x:
        b += 1
    return b


def tile_coords(t, tm, tn):
    """(row, column) of tile t: along M, or in bands of 8 tile columns (N first) when wider than 8."""
    if tn <= BAND:
        return t % tm, t // tm
    band, inb = divmod(t, tm * BAND)
    cols = min(BAND, tn - band * BAND)
    r, c = divmod(inb, cols)
    return r, band * BAND + c


def edge_last_coords(b, g, tm, tn, ragged):
    runs = 8 if g % 8 == 0 else 1
    run = g // runs
    x, j = divmod(b, run)
    rowr, colr = ragged & 1, ragged >> 1
    im, icn = tm - rowr, tn - colr
    ne = g - im * icn
    e0 = x * ne // runs
    ix = run - ((x + 1) * ne // runs - e0)
    if j < ix:
        return tile_coords(x * run - e0 + j, im, icn)
    e = e0 + j - ix
    if e < colr * im:
        return e, tn - 1
    return tm - 1, e - colr * im


def check_schedule(m, n, k, form):
    p = S.gemm_plan(m, n, k, *FORMS[form])
    g, dp, s, rg, cg, edge = p["grid"], p["dp"], p["sk_iters"], p["rg"], p["cg"], p["edge_last"]
    tm, tn, ipt = p["tiles_m"], p["tiles_n"], p["ipt"]
    T = tm * tn
    assert tm == -(-m // p["bm"]) and tn == -(-n // p["bn"]) and ipt == -(-k // 16)
    assert 1 <= g and 0 <= dp <= T
    gsz = rg * cg
    if s:
        assert g <= 1024, "the fixup's slot list holds 1024 blocks"
        assert s * g < 2 ** 31, "32-bit range arithmetic"
    if gsz > 1:
        assert dp == 0 and rg == tm and tn % cg == 0 and cg <= 8
        assert g % 8 == 0 and (g // 8) % gsz == 0, "a block group lies inside one XCD's run"
        assert s == tn // cg * ipt
    else:
        assert s == (T - dp) * ipt
    q_count = g // gsz
    assert s == 0 or s >= q_count, "every range holds at least one k-slice"
    if edge:
        assert s == 0 and dp == T == g and g > p["cus"] * 3
        assert (edge & 1) == (1 if m % p["bm"] else 0) and (edge >> 1) == (1 if n % p["bn"] else 0)

    covered = {}
    whole = {}
    pieces = {}  # tile -> [(k0, slot)]
    for b in range(g):
        t = b
        while t < dp:  # whole tiles, round-robin
            rc = edge_last_coords(t, g, tm, tn, edge) if edge else tile_coords(t, tm, tn)
            assert rc not in whole, f"tile {rc} done whole twice"
            whole[rc] = b
            t += g
        if not s:
            continue
        grp, mem = divmod(b, gsz)
        g_r, g_c = divmod(mem, cg)
        it, end = sk_start(grp, s, q_count), sk_start(grp + 1, s, q_count)
        first = True
        while it < end:
            tt, k0 = divmod(it, ipt)
            k1 = min(ipt, k0 + end - it)
            rc = tile_coords(dp + tt, tm, tn) if gsz == 1 else (g_r, tt * cg + g_c)
            assert 0 <= rc[0] < tm and 0 <= rc[1] < tn
            for kk in range(k0, k1):
                assert (rc, kk) not in covered, f"tile {rc} slice {kk} twice"
                covered[rc, kk] = b
            if k0 == 0 and k1 == ipt:
                assert rc not in whole
                whole[rc] = b
            else:
                pieces.setdefault(rc, []).append((k0, 2 * b if first else 2 * b + 1))
            first = False
            it += k1 - k0
    assert len(whole) + len(pieces) == T, "every tile is stored whole or completed by the fixup"
    assert len(covered) == (T - dp) * ipt
    # the fixup: tile j of the stream-K part, its ranges and slots
    for j in range(T - dp):
        if gsz == 1:
            rc, u, mem = tile_coords(dp + j, tm, tn), j, 0
        else:
            rc = (j % rg, j // rg)
            u = rc[1] // cg
            mem = rc[0] * cg + (rc[1] - u * cg)
        lo, hi = sk_block_of(u * ipt, s, q_count), sk_block_of(u * ipt + ipt - 1, s, q_count)
        if lo == hi:
            assert rc in whole and rc not in pieces
            continue
        slots = [2 * (qq * gsz + mem) + (0 if sk_start(qq, s, q_count) // ipt == u else 1)
                 for qq in range(lo, hi + 1)]
        assert slots == [sl for _, sl in sorted(pieces[rc])], f"fixup slots of tile {rc}"
        assert max(slots) < 2 * g
    return p


# The benchmark networks' product shapes (m, n with the bias column for weight gradients, k) and others
# that reach every schedule form: grouped stream-K, whole-tile rounds with edge tiles last (961 tiles: no
# XCD runs), plain stream-K, hybrid whole tiles + stream-K.
SHAPES = [("nt", 512, 5000, 5000), ("nn", 512, 5000, 5000), ("tn", 5000, 5001, 512), ("nt", 512, 5000, 3072),
          ("tn", 5000, 3073, 512), ("nt", 8192, 256, 2304), ("nn", 2048, 512, 4608), ("tn", 512, 4609, 2048),
          ("tn", 256, 2305, 8192), ("nt", 512, 512, 4608), ("tn", 128, 1153, 32768), ("nt", 32768, 128, 1152),
          ("nt", 3900, 3950, 200), ("nt", 4000, 4000, 64), ("nt", 500, 1000, 3000), ("nn", 1000, 600, 4000),
          ("nt", 256, 192, 4096), ("nt", 256, 2100, 4096), ("nt", 128, 128, 30000), ("nt", 6272, 512, 4608),
          ("tn", 512, 4609, 6272), ("nn", 32, 25088, 4096), ("nt", 2000, 3000, 2000), ("tt", 700, 900, 5000),
          ("nt", 3000, 3001, 1024), ("nt", 5000, 5001, 1024)]


@pytest.mark.parametrize("form,m,n,k", SHAPES)
def test_benchmark_shapes_schedule(form, m, n, k):
    check_schedule(m, n, k, form)


def test_schedule_forms_are_reached():
    """The shapes above exercise grouped stream-K, edge tiles last (with and without XCD runs) and hybrid
    whole-tile + stream-K plans."""
    plans = [S.gemm_plan(m, n, k, *FORMS[f]) for f, m, n, k in SHAPES]
    assert any(p["rg"] * p["cg"] > 1 for p in plans)
    assert any(p["edge_last"] and p["grid"] % 8 == 0 for p in plans)
    assert any(p["edge_last"] and p["grid"] % 8 for p in plans)
    assert any(p["dp"] > 0 and p["sk_iters"] > 0 for p in plans)


def test_random_shapes_schedule():
    rng = random.Random(20261202)
    done = 0
    while done < 150:
        m, n, k = rng.randint(1, 4500), rng.randint(1, 4500), rng.randint(1, 20000)
        form = rng.choice(list(FORMS))
        if (-(-m // 64)) * (-(-n // 64)) * (-(-k // 16)) > 400_000:
            continue  # keeps the Python model of the partition fast
        check_schedule(m, n, k, form)
        done += 1


def test_plan_rejects_bad_arguments():
    with pytest.raises(S.SgdError):
        S.gemm_plan(0, 10, 10)
    with pytest.raises(S.SgdError):
        S.gemm_plan(10, 10, -1)
