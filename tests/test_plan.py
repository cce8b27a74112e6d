"""Host-side launch planning (no GPU): configuration choice, whole-tile waves,
and the Stream-K partition of (tile, K chunk) steps.

The work mapping below restates, for checking, how each workgroup of a
launch walks its share (logical id, tile order, Stream-K range, partial
slot); coverage and slot uniqueness are then checked on the planner's own
numbers for many shapes and grids.
"""
import os
from collections import Counter, defaultdict

import numpy as np
import pytest

import fp32_sgemm_f32_amd as sg

OCC = [0, 1, 2, 1, 1, 2, 1, 2, 4, 2, 2, 1, 1, 2, 1, 1, 1, 2, 1, 1, 2, 2, 2, 1, 2, 2]
EDGE_CFGS = {sg.CFG_DL_64x64x32, sg.CFG_DL_64x64x64, sg.CFG_DL_128x128x32, sg.CFG_DL_256x256x16,
             sg.CFG_GENERIC_64x64x16}


def logical_ids(p):
    g = p["grid"]
    ids = []
    for b in range(g):
        if p["xcd_remap"]:
            per = g >> 3
            ids.append((b & 7) * per + (b >> 3))
        else:
            ids.append(b)
    return ids


def tile_coords(p, t):
    gsz = p["group_m"] * p["tiles_n"]
    g = t // gsz
    first = g * p["group_m"]
    rows = min(p["tiles_m"] - first, p["group_m"])
    r = t - g * gsz
    return first + r % rows, r // rows


def sk_begin(p, w):
    return w * p["sk_iters"] // p["sk_grid"]


def sk_owner(p, i):
    return ((i + 1) * p["sk_grid"] - 1) // p["sk_iters"]


def walk(p):
    """Yield (logical wg, tile_m, tile_n, k0, k1, kind, slot) for every piece of work."""
    ipt = p["iters_per_tile"]
    for w in sorted(logical_ids(p)):
        t = w
        while t < p["dp_tiles"]:
            tm, tn = tile_coords(p, t)
            yield w, tm, tn, 0, ipt, "whole", None
            t += p["grid"]
        if w >= p["sk_grid"]:
            continue
        s, e = sk_begin(p, w), sk_begin(p, w + 1)
        while s < e:
            tl = s // ipt
            k0 = s - tl * ipt
            k1 = k0 + min(e - s, ipt - k0)
            tm, tn = tile_coords(p, p["dp_tiles"] + tl)
            first, last = sk_owner(p, tl * ipt), sk_owner(p, (tl + 1) * ipt - 1)
            if first == last:
                yield w, tm, tn, k0, k1, "whole", None
            else:
                slot = 0 if sk_begin(p, w) // ipt == tl else 1
                yield w, tm, tn, k0, k1, "partial", slot
            s += k1 - k0


def ceil_div(a, b):
    return -(-a // b)


def check_plan(p, M, N, K):
    assert p["tiles_m"] == ceil_div(M, p["tile_m"]) and p["tiles_n"] == ceil_div(N, p["tile_n"])
    assert p["iters_per_tile"] == ceil_div(K, p["tile_k"])
    assert sorted(logical_ids(p)) == list(range(p["grid"]))        # remap is a bijection
    assert p["sk_grid"] <= p["grid"]
    if p["sk_tiles"]:
        assert 1 <= p["sk_grid"] <= p["sk_iters"]
        assert (p["sk_iters"] + 1) * p["sk_grid"] < 2 ** 31
    cover = Counter()
    slots = set()
    per_tile = defaultdict(set)
    for w, tm, tn, k0, k1, kind, slot in walk(p):
        assert 0 <= tm < p["tiles_m"] and 0 <= tn < p["tiles_n"] and 0 <= k0 < k1 <= p["iters_per_tile"]
        for k in range(k0, k1):
            cover[(tm, tn, k)] += 1
        if kind == "partial":
            assert (w, slot) not in slots, "two partials in one slot"
            slots.add((w, slot))
            per_tile[(tm, tn)].add(w)
    tiles = p["tiles_m"] * p["tiles_n"]
    assert len(cover) == tiles * p["iters_per_tile"]
    assert set(cover.values()) == {1}, "a (tile, K chunk) step is missing or repeated"
    # Contributors of a split tile are consecutive workgroups.
    for ws in per_tile.values():
        assert sorted(ws) == list(range(min(ws), max(ws) + 1))
    # Two partial slots per split workgroup; one for the skinny kernel, whose
    # workgroups each own a single (strip, split) step.
    slots = 1 if p["config"] in (sg.CFG_SKINNY_16x256, sg.CFG_ROWDOT_N8) else 2
    need = p["sk_grid"] * slots * p["tile_m"] * p["tile_n"] * 4 if p["sk_tiles"] else 0
    assert p["workspace_bytes"] >= need
    return per_tile


SHAPES = [(128, 128, 32), (256, 256, 256), (512, 384, 96), (1024, 1024, 1024), (1024, 1024, 16384),
          (2048, 2048, 2048), (4096, 4096, 4096), (1280, 768, 640), (3072, 2048, 352),
          (1, 1, 1), (7, 13, 5), (100, 196, 36), (1000, 1000, 1000), (4095, 4096, 4092), (300, 17, 9000),
          (16, 4096, 4096), (1, 256, 1), (5, 1028, 300), (16, 256, 65536),
          (4096, 1, 4096), (300, 8, 20000), (7, 3, 12), (100000, 5, 64)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("config", range(sg.NUM_CFGS))
@pytest.mark.parametrize("sched", [sg.SCHED_AUTO, sg.SCHED_DP, sg.SCHED_STREAMK])
@pytest.mark.parametrize("cus", [256, 132, 7])
def test_every_step_covered_once(shape, config, sched, cus):
    M, N, K = shape
    try:
        p = sg.plan(M, N, K, config, sched, num_cus=cus, occupancy=OCC)
    except sg.SgemmError as e:
        # Only a forced configuration that cannot run the shape may be
        # refused: a tile that does not divide it on a kernel without edge
        # masking, or the vector kernels when N or K is not a multiple of 4.
        assert e.status == sg.ERR_CONFIG and config != sg.CFG_AUTO
        if config == sg.CFG_SKINNY_16x256:   # at most 16 rows
            assert M > 16
            return
        if config == sg.CFG_ROWDOT_N8:       # at most 8 columns; B's whole K range in LDS for DP
            cols = 1 if N <= 1 else 2 if N == 2 else 4 if N <= 4 else 8
            assert N > 8 or (sched == sg.SCHED_DP and K > 16384 // cols)
            return
        bm, bn, bk = sg.CFG_TILES[config]
        divides = M % bm == 0 and N % bn == 0 and K % bk == 0
        vector = N % 4 == 0 and K % 4 == 0
        assert config != sg.CFG_GENERIC_64x64x16
        assert not vector or (not divides and config not in EDGE_CFGS)
        return
    check_plan(p, M, N, K)
    if sched == sg.SCHED_DP:
        assert p["sk_tiles"] == 0 and p["grid"] == p["tiles_m"] * p["tiles_n"]
    if sched == sg.SCHED_STREAMK:
        assert p["dp_tiles"] == 0


@pytest.mark.parametrize("shape", [(1, 16385, 16384), (8, 12288, 8192), (4, 20000, 8192), (2, 11008, 4096),
                                   (1, 16384, 16384), (16, 700, 4096), (3000, 1, 4096), (1000, 3, 1000),
                                   (1500, 8, 4096), (16384, 1, 16384), (40, 5, 300000)])
@pytest.mark.parametrize("cus", [256, 132])
def test_thin_grids_fit_one_resident_round(shape, cus):
    """A split count chosen freely never adds a second, nearly empty round of
    workgroups: the skinny kernel holds one workgroup per CU, the row-dot
    kernel two.  Only the row-dot kernel's LDS limit on B's split may force
    more splits than that."""
    M, N, K = shape
    for config, per_cu in ((sg.CFG_SKINNY_16x256, 1), (sg.CFG_ROWDOT_N8, 2)):
        try:
            p = sg.plan(M, N, K, config, sg.SCHED_AUTO, num_cus=cus, occupancy=OCC)
        except sg.SgemmError:
            continue
        check_plan(p, M, N, K)
        slots = cus * per_cu
        strips = p["tiles_m"] * p["tiles_n"]
        if config == sg.CFG_ROWDOT_N8:
            cols = 1 if N <= 1 else 2 if N == 2 else 4 if N <= 4 else 8
            forced = -(-K // (16384 // cols))
            assert p["grid"] <= max(slots, strips * forced)
        else:
            assert p["grid"] <= max(slots, strips)
        # Still splits K where a single pass would leave most CUs idle.
        if strips * 2 <= slots and K >= 4 * 256:
            assert p["iters_per_tile"] >= 2


def test_stream_k_example_from_the_page():
    """n = 1024, 128x128 tiles, 264 resident blocks: all 64 tiles split, each
    shared by roughly four blocks."""
    path = os.path.join(os.path.dirname(__file__), "golden", "streamk_p4_example.txt")
    g = dict(ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#"))
    n, tile = int(g["n"]), int(g["tile"])
    # The 128x128 tile with K chunks of 8, as on the page's FFMA kernels.
    cfg = sg.CFG_VALU_128x128x8
    occ = [0] * sg.NUM_CFGS
    occ[cfg] = int(g["blocks_per_sm"])
    p = sg.plan(n, n, n, cfg, sg.SCHED_AUTO, num_cus=int(g["sms"]), occupancy=occ,
                sk_wg_per_cu=int(g["blocks_per_sm"]))
    assert p["tile_m"] == p["tile_n"] == tile
    assert p["tiles_m"] * p["tiles_n"] == int(g["tiles"])
    assert p["grid"] == int(g["resident_blocks"])
    assert p["dp_tiles"] == 0 and p["sk_tiles"] == int(g["tiles"])
    per_tile = check_plan(p, n, n, n)
    counts = [len(v) for v in per_tile.values()]
    assert len(counts) == int(g["tiles"])
    # "Roughly four" blocks per tile: each tile holds grid / tiles = 4.125
    # blocks' worth of K chunks.  A tile's K range therefore meets that many
    # block ranges, plus one wherever the range boundaries fall inside it.
    share = p["grid"] / (p["tiles_m"] * p["tiles_n"])
    assert round(share) == int(g["blocks_per_tile_approx"])
    assert all(int(share) <= c <= int(share) + 2 for c in counts)
    mean = sum(counts) / len(counts)
    assert share <= mean <= share + 1.0


def test_full_waves_first_then_split():
    # 1.25 waves of 128x128 tiles on 64 CUs x 2 = 128 resident workgroups:
    # one full wave of whole tiles, the other 32 tiles split over the grid.
    occ = [0] * sg.NUM_CFGS
    occ[sg.CFG_MFMA_128x128x32] = 2
    p = sg.plan(128 * 16, 128 * 10, 1024, sg.CFG_MFMA_128x128x32, sg.SCHED_AUTO, num_cus=64,
                occupancy=occ, sk_wg_per_cu=2)
    assert p["tiles_m"] * p["tiles_n"] == 160
    assert p["dp_tiles"] == 128 and p["sk_tiles"] == 32 and p["grid"] == 128
    check_plan(p, 128 * 16, 128 * 10, 1024)


def test_auto_choices_on_256_cus():
    occ = OCC
    p = sg.plan(4096, 4096, 4096, num_cus=256, occupancy=occ)
    assert (p["config"], p["sched"], p["grid"]) == (sg.CFG_DL_256x256x16, sg.SCHED_DP, 256)
    p = sg.plan(6144, 6144, 6144, num_cus=256, occupancy=occ)
    assert p["config"] == sg.CFG_DL_256x256x16
    p = sg.plan(2048, 2048, 2048, num_cus=256, occupancy=occ)
    assert (p["config"], p["sched"], p["grid"]) == (sg.CFG_DL_128x128x32, sg.SCHED_DP, 256)
    p = sg.plan(2048, 4096, 2048, num_cus=256, occupancy=occ)
    assert (p["config"], p["sched"], p["grid"]) == (sg.CFG_DL_128x128x32, sg.SCHED_DP, 512)
    # 576 tiles of 128 x 128 at 3072^3: two full waves, the 64 left split
    # (measured 3-5% faster than 2304 whole 64 x 64 tiles).
    p = sg.plan(3072, 3072, 3072, num_cus=256, occupancy=occ)
    assert (p["config"], p["dp_tiles"], p["sk_tiles"]) == (sg.CFG_DL_128x128x32, 512, 64)
    p = sg.plan(1024, 1024, 1024, num_cus=256, occupancy=occ)
    assert (p["config"], p["sched"], p["grid"]) == (sg.CFG_DL_64x64x64, sg.SCHED_DP, 256)
    p = sg.plan(1024, 1024, 16384, num_cus=256, occupancy=occ)
    assert (p["config"], p["sched"], p["grid"]) == (sg.CFG_DL_64x64x64, sg.SCHED_DP, 256)
    p = sg.plan(1024, 1024, 1056, num_cus=256, occupancy=occ)     # K not a multiple of 64
    assert p["config"] == sg.CFG_DL_64x64x32
    p = sg.plan(256, 256, 256, num_cus=256, occupancy=occ)     # 1-2% ahead of 64-deep chunks
    assert (p["config"], p["sched"]) == (sg.CFG_DL_64x64x32, sg.SCHED_DP)
    # 41 chunks of 32 (odd): 32-deep chunks; 441 tiles fill 86% of the 512
    # resident slots, so every tile runs at once, data-parallel.
    p = sg.plan(1292, 1292, 1292, num_cus=256, occupancy=occ)
    assert (p["config"], p["sched"], p["grid"]) == (sg.CFG_DL_64x64x32, sg.SCHED_DP, 441)
    # One full wave of 64x64 tiles and 16 more, 32 chunks each: the
    # remainder alone would spread over only 64 workgroups, so every tile is
    # split over the full grid instead.
    p = sg.plan(1024, 1028, 2048, num_cus=256, occupancy=occ)
    assert (p["config"], p["dp_tiles"], p["sk_tiles"], p["sk_grid"]) == (sg.CFG_DL_64x64x64, 0, 272, 256)
    # With 256 chunks per tile the remainder spreads over the whole grid:
    # one wave of whole tiles, then the 16 split.
    p = sg.plan(4096, 4100, 4096, sg.CFG_DL_256x256x16, num_cus=256, occupancy=occ)
    assert (p["config"], p["dp_tiles"], p["sk_tiles"], p["sk_grid"]) == (sg.CFG_DL_256x256x16, 256, 16, 256)
    # The automatic choice there: four waves of 128 x 128 tiles and 32 split
    # (measured 1.7-2% faster).
    p = sg.plan(4096, 4100, 4096, num_cus=256, occupancy=occ)
    assert (p["config"], p["dp_tiles"], p["sk_tiles"], p["sk_grid"]) == (sg.CFG_DL_128x128x32, 1024, 32, 256)
    # Small K: whole tiles.  A split there costs a second kernel and more
    # than the little work it balances (measured, back to back: 4224 x 448 x
    # 384 in 17.2 us against 25.9 split; 304 x 5632 x 64 in 8.0 against 30.8;
    # 3984 x 3712 x 80 on 256 x 256 tiles in 33.4 against 61.5 split).
    for shape, config in (((4224, 448, 384), sg.CFG_DL_64x64x32), ((304, 5632, 64), sg.CFG_DL_64x64x32),
                          ((3984, 3712, 80), sg.CFG_DL_256x256x16)):
        p = sg.plan(*shape, num_cus=256, occupancy=occ)
        assert (p["config"], p["sched"]) == (config, sg.SCHED_DP), shape
    # A side much narrower than the tile: tiles at most half inside C are
    # passed over for ones that fit (256 columns of 128: 128x128 tiles).
    p = sg.plan(65536, 128, 2048, num_cus=256, occupancy=occ)
    assert (p["config"], p["sched"], p["tiles_m"], p["tiles_n"]) == (sg.CFG_DL_128x128x32, sg.SCHED_DP, 512, 1)
    p = sg.plan(128, 65536, 2048, num_cus=256, occupancy=occ)
    assert p["config"] == sg.CFG_DL_128x128x32
    p = sg.plan(65536, 320, 2048, num_cus=256, occupancy=occ)   # 83% inside 128-wide tiles
    assert p["config"] in (sg.CFG_DL_64x64x64, sg.CFG_DL_64x64x32)
    # Narrow C with a small B: row by row (tiles sharing an A panel side by
    # side); few tile rows with a small A: column by column.
    assert p["group_m"] == 1
    p = sg.plan(49152, 192, 4096, num_cus=256, occupancy=occ)
    assert (p["config"], p["tiles_n"], p["group_m"]) == (sg.CFG_DL_64x64x32, 3, 1)
    # Narrow but few tiles (64): the 64-deep chunks.
    assert sg.plan(512, 512, 8192, num_cus=256, occupancy=occ)["config"] == sg.CFG_DL_64x64x64
    p = sg.plan(192, 49152, 4096, num_cus=256, occupancy=occ)
    assert (p["tiles_m"], p["group_m"]) == (3, 3)
    check_plan(p, 192, 49152, 4096)
    # Few rows: the skinny kernel up to 16 (N and K at least 256); for 9-16
    # rows only once B has more than 2^22 elements, unless the layout rules
    # out the tiled kernels.
    for shape in [(1, 16384, 16384), (8, 4096, 4096), (8, 256, 256), (12, 16384, 16384), (16, 50257, 1024),
                  (13, 4096, 4094), (16, 16384, 16384), (16, 2049, 2048), (9, 4096, 2048)]:
        assert sg.plan(*shape, num_cus=256, occupancy=occ)["config"] == sg.CFG_SKINNY_16x256, shape
    for shape in [(17, 16384, 16384), (12, 255, 4096), (12, 4096, 252), (13, 2048, 2048), (9, 256, 256)]:
        assert sg.plan(*shape, num_cus=256, occupancy=occ)["config"] != sg.CFG_SKINNY_16x256, shape
    # Ragged shapes: the edge-masking kernels of the same regimes, or the
    # general kernel when N or K is not a multiple of 4.
    p = sg.plan(4000, 4000, 4000, num_cus=256, occupancy=occ)
    assert (p["config"], p["tiles_m"], p["iters_per_tile"]) == (sg.CFG_DL_256x256x16, 16, 250)
    p = sg.plan(2000, 2000, 2000, num_cus=256, occupancy=occ)
    assert p["config"] == sg.CFG_DL_128x128x32
    p = sg.plan(1000, 1000, 1000, num_cus=256, occupancy=occ)
    assert p["config"] == sg.CFG_DL_64x64x64
    p = sg.plan(100, 101, 100, num_cus=256, occupancy=occ)
    assert (p["config"], p["repacked"]) == (sg.CFG_GENERIC_64x64x16, 0)
    p = sg.plan(7, 13, 5, num_cus=256, occupancy=occ)
    assert p["config"] == sg.CFG_GENERIC_64x64x16
    # At least 2^25 multiply-adds (M, N, K >= 64): the call runs on padded
    # copies, and the plan is the padded product's.
    p = sg.plan(1000, 1001, 1000, num_cus=256, occupancy=occ)
    assert (p["config"], p["repacked"], p["tiles_n"]) == (sg.CFG_DL_64x64x64, 1, 16)
    p = sg.plan(4096, 4097, 4096, num_cus=256, occupancy=occ)
    assert (p["config"], p["repacked"], p["tiles_n"]) == (sg.CFG_DL_128x128x32, 1, 33)
    p = sg.plan(1000, 1001, 1000, sg.CFG_GENERIC_64x64x16, num_cus=256, occupancy=occ)   # forced: as asked
    assert (p["config"], p["repacked"]) == (sg.CFG_GENERIC_64x64x16, 0)


def test_automatic_choice_is_the_least_modelled_time():
    """The automatic choice's modelled time is no more than that of any
    data-parallel plan of the four configurations it weighs (each is one of
    its candidates); other configurations report no model (-1)."""
    occ = OCC
    tiled = (sg.CFG_DL_256x256x16, sg.CFG_DL_128x128x32, sg.CFG_DL_64x64x64, sg.CFG_DL_64x64x32)
    rng = np.random.default_rng(5)
    for _ in range(300):
        M, N, K = (int(x) * 16 for x in rng.integers(1, 513, size=3))
        ta, tb = int(rng.integers(0, 2)), int(rng.integers(0, 2))
        p = sg.plan(M, N, K, num_cus=256, occupancy=occ, trans_a=ta, trans_b=tb)
        if p["config"] not in tiled:
            assert p["model_us"] == -1.0
            continue
        assert p["model_us"] > 0
        for cfg in tiled:
            q = sg.plan(M, N, K, cfg, sg.SCHED_DP, num_cus=256, occupancy=occ, trans_a=ta, trans_b=tb)
            assert q["model_us"] > 0
            assert p["model_us"] <= q["model_us"] * (1 + 1e-12), ((M, N, K, ta, tb), cfg)
    # More K costs more; the vector-ALU and general kernels are not modelled.
    a = sg.plan(1024, 1024, 1024, sg.CFG_DL_64x64x64, sg.SCHED_DP, num_cus=256, occupancy=occ)["model_us"]
    b = sg.plan(1024, 1024, 2048, sg.CFG_DL_64x64x64, sg.SCHED_DP, num_cus=256, occupancy=occ)["model_us"]
    assert 0 < a < b
    for cfg in (sg.CFG_VALU_128x128x8, sg.CFG_GENERIC_64x64x16, sg.CFG_MFMA_256x256x16):
        assert sg.plan(1024, 1024, 1024, cfg, num_cus=256, occupancy=occ)["model_us"] == -1.0


def test_cost_model_coefficients_are_the_committed_fit():
    """plan.cpp's cost-model coefficients are what the committed fitting
    script computes from the committed sweep timings."""
    import re
    pytest.importorskip("scipy")
    from fp32_sgemm_f32_amd.tuning import fit_cost_model as fit
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = open(os.path.join(root, "fp32_sgemm_f32_amd", "csrc", "plan.cpp")).read()
    coef = {m.group(1): (float(m.group(2)), float(m.group(3)))
            for m in re.finditer(r"\{SGEMM_CFG_(DL_\w+), ([0-9.e+-]+), ([0-9.e+-]+)\}", src)}
    const = {m.group(1): float(m.group(2))
             for m in re.finditer(r"constexpr double (k\w+) = ([0-9.e+-]+);", src)}
    th = fit.fit(fit.load(os.path.join(root, "fp32_sgemm_f32_amd", "tuning", "plan_sweeps.csv")))
    for i, name in enumerate(fit.NAMES):
        eff, tile = coef["DL_" + name[3:]]   # dl_256x256x16 -> SGEMM_CFG_DL_256x256x16
        assert eff == pytest.approx(th[i], rel=1e-3) and tile == pytest.approx(th[4 + i], rel=1e-3), name
    assert const["kSumLaunchUs"] == pytest.approx(th[9], rel=1e-3)
    assert const["kSumBytesPerUs"] == pytest.approx(th[10], rel=1e-3)
    assert const["kStoreBytesPerUs"] == pytest.approx(th[11], rel=1e-3)
    assert const["kNarrowEff64x64x32"] == pytest.approx(th[12], rel=1e-3)


def test_automatic_choice_cache_is_keyed_on_the_whole_request():
    """The per-thread cache of the automatic choice returns what the first
    call computed for the same request, across more shapes than it holds,
    and never a plan computed for another occupancy or CU count."""
    occ = OCC
    shapes = [(1000, 1028, 1024), (4224, 448, 384), (2688, 1472, 256), (1292, 1292, 1292), (131072, 64, 1024),
              (4096, 4096, 4096), (512, 512, 512), (3072, 3072, 3072)]
    first = {s: sg.plan(*s, num_cus=256, occupancy=occ) for s in shapes}
    for rep in range(3):
        for s in (shapes if rep % 2 == 0 else shapes[::-1]):
            assert sg.plan(*s, num_cus=256, occupancy=occ) == first[s], s
    # 1292^3: 441 64x64 tiles all resident with two workgroups per CU on the
    # 32-deep kernel; with one, the 64-deep kernel.
    occ1 = list(occ)
    occ1[sg.CFG_DL_64x64x32] = 1
    a = sg.plan(1292, 1292, 1292, num_cus=256, occupancy=occ)
    b = sg.plan(1292, 1292, 1292, num_cus=256, occupancy=occ1)
    assert (a["config"], b["config"]) == (sg.CFG_DL_64x64x32, sg.CFG_DL_64x64x64)
    assert a["model_us"] < b["model_us"]
    assert sg.plan(1292, 1292, 1292, num_cus=256, occupancy=occ) == a
    c = sg.plan(4096, 4096, 4096, num_cus=128, occupancy=occ)
    assert c["model_us"] > 1.9 * first[(4096, 4096, 4096)]["model_us"]


# Configurations that also run A stored K x M and / or B stored N x K.
LAYOUT_CFGS = EDGE_CFGS


@pytest.mark.parametrize("layout", [(1, 0), (0, 1), (1, 1)], ids=["TN", "NT", "TT"])
def test_auto_choices_for_transposed_storage(layout):
    """The same choices as for A M x K, B K x N (the direct-to-LDS kernels
    load every storage order), and the general kernel when a stored row
    length is not a multiple of 4."""
    ta, tb = layout
    occ = OCC

    def cfg(M, N, K):
        return sg.plan(M, N, K, num_cus=256, occupancy=occ, trans_a=ta, trans_b=tb)["config"]

    assert cfg(4096, 4096, 4096) == sg.CFG_DL_256x256x16
    assert cfg(2048, 2048, 2048) == sg.CFG_DL_128x128x32
    assert cfg(1024, 1024, 1024) == sg.CFG_DL_64x64x64
    assert cfg(1024, 1024, 16384) == sg.CFG_DL_64x64x64
    assert cfg(1024, 1024, 96) == sg.CFG_DL_64x64x32
    # A stored K x M has rows of M floats; B stored N x K rows of K floats.
    # Below 2^25 multiply-adds such a layout runs on the general kernel:
    tiled64 = (sg.CFG_DL_64x64x64, sg.CFG_DL_64x64x32)
    assert cfg(254, 256, 256) == sg.CFG_GENERIC_64x64x16 if ta else cfg(254, 256, 256) in tiled64
    assert cfg(256, 256, 254) in tiled64 if (ta and not tb) else cfg(256, 256, 254) == sg.CFG_GENERIC_64x64x16
    assert cfg(256, 254, 256) == sg.CFG_GENERIC_64x64x16          # C rows
    # at or above it, on padded copies (the plan of the padded product).
    for shape, misaligned in (((1022, 1024, 1024), ta), ((1024, 1024, 1022), not (ta and not tb)),
                              ((1024, 1022, 1024), True)):
        p = sg.plan(*shape, num_cus=256, occupancy=occ, trans_a=ta, trans_b=tb)
        assert p["repacked"] == (1 if misaligned else 0), shape
        assert p["config"] == sg.CFG_DL_64x64x64
    p = sg.plan(4096, 4096, 4096, num_cus=256, occupancy=occ, trans_a=ta, trans_b=tb)
    assert p["tiles_m"] == 16 and p["sched"] == sg.SCHED_DP


@pytest.mark.parametrize("config", range(1, sg.NUM_CFGS))
def test_transposed_storage_runs_only_on_layout_configs(config):
    for ta, tb in [(1, 0), (0, 1), (1, 1)]:
        if config in LAYOUT_CFGS:
            p = sg.plan(512, 512, 512, config, num_cus=256, occupancy=OCC, trans_a=ta, trans_b=tb)
            check_plan(p, 512, 512, 512)
        else:
            with pytest.raises(sg.SgemmError) as e:
                sg.plan(512, 512, 512, config, num_cus=256, occupancy=OCC, trans_a=ta, trans_b=tb)
            assert e.value.status == sg.ERR_CONFIG
    with pytest.raises(sg.SgemmError) as e:
        sg.plan(512, 512, 512, config, trans_a=2)
    assert e.value.status == sg.ERR_CONFIG


def test_xcd_grouping_for_the_headline_shape():
    """4096^3 on 256 CUs: each XCD's 32 consecutive tiles form a 4 x 8 block."""
    p = sg.plan(4096, 4096, 4096, num_cus=256, occupancy=OCC)
    assert p["xcd_remap"] == 1 and p["group_m"] == 4
    ids = logical_ids(p)
    for x in range(8):
        tiles = {tile_coords(p, ids[b]) for b in range(p["grid"]) if b % 8 == x}
        rows = {t[0] for t in tiles}
        cols = {t[1] for t in tiles}
        assert len(tiles) == 32 and len(rows) == 4 and len(cols) == 8


def test_plan_errors():
    with pytest.raises(sg.SgemmError) as e:
        sg.plan(-1, 128, 32)
    assert e.value.status == sg.ERR_SHAPE
    with pytest.raises(sg.SgemmError) as e:
        sg.plan(128, 128, 32, config=sg.CFG_MFMA_256x256x16)
    assert e.value.status == sg.ERR_CONFIG
    with pytest.raises(sg.SgemmError) as e:      # vector kernel, N not a multiple of 4
        sg.plan(128, 130, 32, config=sg.CFG_DL_64x64x32)
    assert e.value.status == sg.ERR_CONFIG
    with pytest.raises(sg.SgemmError) as e:
        sg.plan(128, 128, 32, config=42)
    assert e.value.status == sg.ERR_CONFIG


def test_empty_shapes_plan_no_work():
    for shape in [(0, 128, 32), (128, 0, 32), (128, 128, 0)]:
        p = sg.plan(*shape, num_cus=256, occupancy=OCC)
        assert p["sk_tiles"] == 0 and p["workspace_bytes"] == 0


def test_thin_products_in_other_storage_orders_run_transposed():
    """Few rows with B stored N x K go to the row-dot kernel, and few
    columns with A stored K x M to the skinny kernel, as the transposed
    product (C^T = op(B)^T op(A)^T), where that kernel's own rule would take
    the transposed shape; the plan is the transposed product's."""
    occ = OCC

    def plan(M, N, K, ta, tb, sched=sg.SCHED_AUTO, config=sg.CFG_AUTO):
        return sg.plan(M, N, K, config, sched, num_cus=256, occupancy=occ, trans_a=ta, trans_b=tb)

    # x W^T: at most 2 rows, B of 2^26 elements or more, or an unaligned layout.
    for shape in [(1, 16384, 16384), (2, 4096, 1024), (8, 16384, 8192), (5, 1000, 777), (8, 4096, 4095)]:
        p = plan(*shape, 0, 1)
        assert (p["config"], p["transposed"]) == (sg.CFG_ROWDOT_N8, 1), shape
        M, N, K = shape
        assert p["tiles_m"] * p["tile_m"] >= N and p["tiles_n"] == 1   # rows of the transposed product: N
        check_plan(p, N, M, K)
    # Not taken: more than 8 rows, a small aligned B with 3-8 rows, N or K
    # under 256, B stored K x N, a forced configuration, or the data-parallel
    # schedule with B's K range beyond LDS.
    for shape, ta, tb, sched, config in [((9, 16384, 16384), 0, 1, 0, 0), ((4, 4096, 4096), 0, 1, 0, 0),
                                         ((1, 255, 4096), 0, 1, 0, 0), ((1, 4096, 255), 0, 1, 0, 0),
                                         ((1, 16384, 16384), 0, 0, 0, 0),
                                         ((1, 16384, 16384), 0, 1, 0, sg.CFG_DL_64x64x64),
                                         ((1, 4096, 32768), 0, 1, sg.SCHED_DP, 0)]:
        assert plan(*shape, ta, tb, sched, config)["transposed"] == 0, (shape, ta, tb, sched, config)
    # X^T v: at most 8 columns, A above 2^22 elements, or an unaligned layout.
    for shape, tb in [((16384, 1, 16384), 0), ((4096, 12, 4096), 0), ((1000, 3, 1000), 1), ((4099, 16, 3000), 0)]:
        p = plan(*shape, 1, tb)
        assert (p["config"], p["transposed"]) == (sg.CFG_SKINNY_16x256, 1), shape
        M, N, K = shape
        check_plan(p, N, M, K)
    for shape, tb in [((300, 12, 300), 0), ((16384, 17, 16384), 0), ((255, 1, 4096), 0), ((16384, 1, 16384), 1)]:
        p = plan(*shape, 0 if shape == (16384, 1, 16384) else 1, tb)
        assert p["transposed"] == 0, shape


FIXED_SHAPES = [((4096, 4096, 4096), sg.CFG_DL_256x256x16), ((2048, 2048, 2048), sg.CFG_DL_128x128x32),
                ((1024, 1024, 1024), sg.CFG_DL_64x64x64), ((1024, 1024, 16384), sg.CFG_DL_64x64x64)]


@pytest.mark.parametrize("shape,config", FIXED_SHAPES, ids=lambda x: "x".join(map(str, x)) if isinstance(x, tuple) else "")
def test_compile_time_shape_plans(shape, config):
    """SGEMM_SCHED_FIXED: the automatic choice's configuration, data-parallel,
    with the same grid and tile order as the runtime plan of the shape."""
    p = sg.plan(*shape, sched=sg.SCHED_FIXED)
    q = sg.plan(*shape, sched=sg.SCHED_DP)
    assert p["fixed_shape"] == 1 and q["fixed_shape"] == 0
    assert p["config"] == config and p["sched"] == sg.SCHED_DP and p["sk_tiles"] == 0
    for k in ("config", "grid", "group_m", "xcd_remap", "tiles_m", "tiles_n", "iters_per_tile"):
        assert p[k] == q[k], k
    assert sg.plan(*shape)["fixed_shape"] == 0      # the automatic choice keeps the runtime kernels


@pytest.mark.parametrize("case", ["other_shape", "ragged", "forced_other_config", "transposed_a", "transposed_b",
                                  "thin"])
def test_compile_time_shape_refused_elsewhere(case):
    kw = {}
    shape = (4096, 4096, 4096)
    if case == "other_shape":
        shape = (4096, 4096, 2048)
    elif case == "ragged":
        shape = (1000, 1024, 1024)
    elif case == "forced_other_config":
        kw["config"] = sg.CFG_DL_128x128x32
    elif case == "transposed_a":
        kw["trans_a"] = 1
    elif case == "transposed_b":
        kw["trans_b"] = 1
    elif case == "thin":
        shape = (8, 4096, 4096)
    with pytest.raises(sg.SgemmError) as e:
        sg.plan(*shape, sched=sg.SCHED_FIXED, **kw)
    assert e.value.status == sg.ERR_CONFIG
