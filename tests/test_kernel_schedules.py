"""Host-side replays of the tiled kernels' work distribution and pipeline
waits (CPU).  They restate, in Python, the index arithmetic of tile_of and
the issue/wait schedule of the integer-format tiled kernel, and check the
invariants those rely on: every tile is computed exactly once for any grid at
least as large as the live tile count, and every wait leaves the stage about
to be used complete.  A change to either piece of device code must keep these
invariants; update the replay with it."""
import itertools

XCDS = 8
LDS = 160 * 1024


def tile_of(pid, m_tiles, n_tiles, group_m):
    total = m_tiles * n_tiles
    per = (total + XCDS - 1) // XCDS
    if pid // XCDS >= per:
        return None
    t = (pid % XCDS) * per + pid // XCDS
    if t >= total:
        return None
    group = group_m * n_tiles
    first = (t // group) * group_m
    gm = min(group_m, m_tiles - first)
    r = t % group
    return first + r % gm, r // gm


def test_raster_visits_every_tile_once_for_oversized_grids():
    for m, n, gm, extra in itertools.product([1, 2, 3, 7, 32, 33, 264], [1, 3, 8, 24, 32, 112],
                                             [1, 4, 8], [0, 1, 300]):
        grid = (((m + extra) * n + XCDS - 1) // XCDS) * XCDS
        live = [s for s in (tile_of(p, m, n, gm) for p in range(grid)) if s is not None]
        assert len(live) == m * n and len(set(live)) == m * n, (m, n, gm, extra)
        assert all(0 <= a < m and 0 <= b < n for a, b in live)


def a16_rings(bm, bits, zp, group, waves=4, small=False, bn=128):
    """Ring depths and per-stage load counts of the integer-format tiled kernel
    (small: one wave per 16 columns, rings within half of LDS)."""
    gpb = 128 // group
    nblk = bn // 16
    a_stage = bm * 256 + gpb * max(bm, 64) * 4
    b_stage = nblk * 64 * (16 if bits == 4 else 12) + bn * 16 + (bn * 4 if zp else 0)
    cap = LDS // 2 if small else LDS
    na = 2 if small else (3 if 3 * a_stage + (3 if bn > 128 else 2) * b_stage <= cap else 2)
    nb = min(6, (cap - na * a_stage) // b_stage)
    a_loads = bm * 256 // 1024 // waves
    b_loads = (nblk if bits == 4 else 3 * nblk) // waves
    # per wave kind: the first waves also copy the row sums (+ gpb) and the
    # scales / zero points (+ 1 + zp)
    kinds = [(a_loads + sx, b_loads + ss) for sx in (0, gpb) for ss in (0, 1 + (1 if zp else 0))]
    return na, nb, kinds, na * a_stage + nb * b_stage, cap


def a16_after(na, nb, ai, bi):
    return (bi if nb > na else 0) + (na - 2) * (ai + bi)


def test_a16_tiled_ring_waits_cover_each_stage():
    # 128- and 256-row tiles (4 or 8 waves) and the 32- and 64-row small tiles (8 waves)
    shapes = [(bm, w, False, 128) for bm in (128, 256) for w in (4, 8)] + \
             [(32, 8, True, 128), (64, 8, True, 128), (128, 8, False, 256)]
    for (bm, waves, small, bn), bits, zp, group in itertools.product(shapes, [3, 4], [False, True],
                                                                   [32, 64, 128]):
        na, nb, kinds, lds, cap = a16_rings(bm, bits, zp, group, waves, small, bn)
        assert 2 <= na <= nb and lds <= cap
        for (ai, bi), kbs in itertools.product(kinds, range(1, 13)):
            after = a16_after(na, nb, ai, bi)
            assert after <= 63
            seq = []
            for s in range(nb - 1):
                if s < na - 1 and s < kbs:
                    seq += [("A", s)] * ai
                if s < kbs:
                    seq += [("B", s)] * bi
            for kb in range(kbs):
                if kb + nb - 2 < kbs:
                    w = after
                elif na == 3 and kb + 1 < kbs:
                    w = ai
                else:
                    w = 0
                outstanding = seq[len(seq) - w:] if w else []
                assert ("A", kb) in seq and ("B", kb) in seq
                assert ("A", kb) not in outstanding and ("B", kb) not in outstanding, (bm, bits, zp, group, kbs, kb)
                if kb + na - 1 < kbs:
                    seq += [("A", kb + na - 1)] * ai
                if kb + nb - 1 < kbs:
                    seq += [("B", kb + nb - 1)] * bi


def test_moe_tile_list_capacity_bounds_the_tiles():
    """tiles <= pairs / 128 + min(E, pairs / min_rows) + 1 for any split of the
    pairs over experts (one partial tile per expert that has tiles)."""
    import numpy as np
    r = np.random.default_rng(0)
    for _ in range(200):
        e = int(r.integers(1, 300))
        pairs = int(r.integers(1, 40000))
        min_rows = int(r.choice([1, 12, 64]))
        cuts = np.sort(r.integers(0, pairs + 1, e - 1))
        counts = np.diff(np.concatenate([[0], cuts, [pairs]]))
        tiles = sum(-(-c // 128) for c in counts if c >= min_rows)
        cap = pairs // 128 + min(e, pairs // min_rows) + 1
        assert tiles <= cap


def test_moe_small_tile_list_capacity_bounds_the_tiles():
    """Small tiles (experts with 1 .. min_rows - 1 rows, 64-row tiles):
    tiles <= pairs / 64 + min(E, pairs) + 1."""
    import numpy as np
    r = np.random.default_rng(1)
    for _ in range(200):
        e = int(r.integers(1, 300))
        pairs = int(r.integers(1, 40000))
        min_rows = int(r.choice([2, 12, 64, 1000]))
        cuts = np.sort(r.integers(0, pairs + 1, e - 1))
        counts = np.diff(np.concatenate([[0], cuts, [pairs]]))
        tiles = sum(-(-c // 64) for c in counts if 1 <= c < min_rows)
        assert tiles <= pairs // 64 + min(e, pairs) + 1


def test_tile_epilogue_stores_every_row_chunk_once():
    """The tiled kernels' epilogue moves a 16-row block of a wave tile of 16 NJ
    columns out in passes: lane l takes 16-byte chunk l % cpr of row
    pass * (64 // cpr) + l // cpr (cpr = chunks per row), lanes past the
    pass's rows idle.  Every (row, chunk) must be stored exactly once for
    every width the kernels use (NJ = 1 .. 8, bf16 and fp32 outputs), also
    where cpr does not divide 64 (NJ = 3, 5, 6, 7)."""
    for nj in range(1, 9):
        for el in (2, 4):
            cpr = 16 * nj * el // 16
            rpp = 64 // cpr
            seen = {}
            for p in range((16 + rpp - 1) // rpp):
                for lane in range(64):
                    rr, c = p * rpp + lane // cpr, lane % cpr
                    if lane >= rpp * cpr or rr >= 16:
                        continue
                    seen[(rr, c)] = seen.get((rr, c), 0) + 1
            assert sorted(seen) == [(r, c) for r in range(16) for c in range(cpr)], (nj, el)
            assert set(seen.values()) == {1}, (nj, el)


def test_mx_tiled_waits_cover_each_stage():
    """MX tiled kernel: stage kb = A_LOADS + B_LOADS copies, + 1 SA copy on
    the SA waves, + 1 weight-scale copy on the SW waves when kb % 4 == 0 (it
    fills the scale ring slot of steps kb .. kb + 3).  Stages 0 and 1 go out
    in the prologue, stage kb + 2 after the barrier of step kb; step kb waits
    until only this wave's loads of stage kb + 1 are outstanding.  Replayed
    per wave kind: every load of stage kb (and of the scale group of step kb)
    has retired at the wait of step kb."""
    # sar: the activation scales also travel in a ring filled every fourth step
    for ab, sa_wave, sw_wave, sar in itertools.product((6, 5, 4, 12), (True, False), (True, False),
                                                       (False, True)):
        def stage(kb):
            return [("AB", kb)] * ab + ([("SA", kb)] if (sa_wave and (kb % 4 == 0 or not sar)) else []) + \
                   ([("SW", kb)] if (kb % 4 == 0 and sw_wave) else [])
        for kbs in range(1, 14):
            seq = stage(0) + (stage(1) if kbs > 1 else [])
            for kb in range(kbs):
                if kb + 1 < kbs:
                    ring_next = (kb + 1) % 4 == 0
                    w = ab + (1 if (sa_wave and (ring_next or not sar)) else 0) + \
                        (1 if (ring_next and sw_wave) else 0)
                else:
                    w = 0
                assert w <= 63
                outstanding = seq[len(seq) - w:] if w else []
                assert all(t[1] != kb for t in outstanding), (ab, sa_wave, sw_wave, sar, kbs, kb)
                # the ring slots of step kb were filled with stage kb - kb % 4
                assert all(t[1] != kb - kb % 4 or t[0] not in ("SW", "SA") for t in outstanding)
                if kb + 2 < kbs:
                    seq += stage(kb + 2)
