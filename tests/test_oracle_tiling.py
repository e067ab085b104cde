"""Pins for oracle/tiling.py: hand-worked shrink paths and choices, geometry
limits, dim collapse cases, coverage by brute force, and the header/range
invariants (no GPU)."""
import numpy as np
import pytest

from oracle import tiling as TL
from oracle.tiling import Operand


def f32(s_r=0, s_c=1):
    return Operand(4, s_r, s_c, 0)


def test_had():
    assert TL.had(528903, 2, 512) == 264704
    assert TL.had(528903, 2048, 512) == 512
    assert TL.had(1000, 1, 512) == 1024
    assert TL.had(7, 3, 1) == 3


def test_sqrt_add_workload_choice_by_hand():
    # c = sqrt(a + b) over (513, 1031) fp32, three contiguous operands
    R, C, st = TL.collapse(TL.ELEMWISE, (513, 1031), [(1031, 1)] * 3)
    assert (R, C) == (1, 528903) and st == [(0, 1)] * 3
    ops = [Operand(4, s, c) for s, c in st]
    p = TL.plan(TL.ELEMWISE, R, C, ops)
    assert [tc for _, tc in p.path] == [528903, 264704, 132608, 66560, 33280, 16896, 8704,
                                        4608, 2560, 1536, 1024, 512]
    # one 256-lane row holds at most 5 * 256 * 8 = 10240 columns; costs worked
    # by hand: ceil(tiles / 512) * (78125 + 12 * tc) for the feasible tail
    # (61, 115, 207, 345, 517, 1034 tiles)
    assert p.costs[:6] == [None] * 6
    assert p.costs[6:] == [182573, 133421, 108845, 96557, 2 * 90413, 3 * 84269]
    assert (p.tr, p.tc, p.block_dim, p.body_tile, p.grid) == (1, 1536, 345, 1, 345)
    assert (p.P, p.g, p.nv, p.pad) == (1, 256, 1, 0)


def test_layernorm_rows_choice_by_hand():
    x = Operand(2, 5120, 1)
    y = Operand(2, 5120, 1)
    gam = Operand(4, 0, 1)
    bet = Operand(4, 0, 1)
    p = TL.plan(TL.ROWREDUCE, 1000, 5120, [x, gam, bet, y])
    # ceil(R / k) for k = 1, 2, 4, ..., each followed by its power-of-two floor
    assert [tr for tr, _ in p.path] == [1000, 512, 500, 256, 250, 128, 125, 64, 63, 32, 16, 8, 4, 2, 1]
    # 4 rows of 5120 need 10 chunks per lane; 2 rows need 5 (g = 128)
    assert p.costs[:-2] == [None] * 13
    # tr=2: 500 tiles in one round, x and y vary (2*5120*2 bytes each), gamma
    # and beta are invariant (5120*4 bytes each); tr=1: 1000 tiles, two rounds
    assert p.costs[-2:] == [(78125 + 40960) + 40960, 2 * (78125 + 20480) + 40960]
    assert (p.tr, p.tc, p.block_dim, p.body_tile, p.grid, p.g, p.nv) == (2, 5120, 500, 1, 500, 128, 5)


def test_row_tiles_fill_their_lane_groups():
    # 34640 rows of 5120 bf16 on the wide build: ceil(R / 8192) = 5 rows need 8
    # lane groups of 32 lanes (20 chunks each, infeasible), ceil(R / 16384) = 3
    # rows leave one of 4 groups idle; its floor 4 fills them and costs fewer
    # rounds: 8660 tiles in 17 rounds against 11547 in 23
    x, y = Operand(2, 5120, 1), Operand(2, 5120, 1)
    p = TL.plan(TL.ROWREDUCE, 34640, 5120, [x, y], TL.NV_WIDE)
    trs = [tr for tr, _ in p.path]
    assert trs[trs.index(5):trs.index(5) + 4] == [5, 4, 3, 2]
    c4, c3 = p.costs[trs.index(4)], p.costs[trs.index(3)]
    assert c4 == 17 * (78125 + 4 * 5120 * 4) and c3 == 23 * (78125 + 3 * 5120 * 4)
    assert (p.tr, p.block_dim, p.g, p.nv) == (4, 8660, 64, 10)


def test_softmax_misaligned_rows_by_hand():
    s = Operand(2, 3001, 1)
    o = Operand(2, 3001, 1)
    assert TL.alignment_pad(280, [s, o]) == 7
    assert TL.geometry(2, 3001, 7) == (2, 128, 3, True)
    assert TL.geometry(3, 3001, 7) == (4, 64, 6, False)
    p = TL.plan(TL.ROWREDUCE, 280, 3001, [s, o])
    # tr=2: 140 tiles, 1 round of (78125 + 2*3001*2*2); tr=1: 280 tiles, still
    # 1 round, of (78125 + 3001*2*2): the smaller tile wins
    assert p.costs[-2:] == [102133, 90129]
    assert p.tr == 1 and p.block_dim == 280
    # with 4000 rows the rounds differ (4 against 8) and the 2-row tile wins
    p = TL.plan(TL.ROWREDUCE, 4000, 3001, [s, o])
    i2 = [tr for tr, _ in p.path].index(2)
    assert p.costs[i2] == 4 * 102133 and p.costs[-1] == 8 * 90129
    assert p.tr == 2 and p.block_dim == 2000


def test_feasibility_edges():
    assert TL.geometry(1, 10240, 0)[3] is True
    assert TL.geometry(1, 10240, 7)[3] is False
    assert TL.geometry(1, 10233, 7)[3] is True
    assert TL.geometry(1, 10241, 0)[3] is False
    assert TL.geometry(256, 8, 0) == (256, 1, 1, True)
    assert TL.geometry(128, 8, 0) == (128, 2, 1, True)
    assert TL.geometry(257, 8, 0)[3] is False
    with pytest.raises(ValueError):
        TL.plan(TL.ROWREDUCE, 10, 10240, [Operand(2, 10241, 1)])   # misaligned 10240-wide rows


def test_alignment_pad_rules():
    assert TL.alignment_pad(5, [Operand(4, 4, 1)]) == 0        # 16-byte rows
    assert TL.alignment_pad(5, [Operand(4, 6, 1)]) == 7        # 24-byte rows
    assert TL.alignment_pad(1, [Operand(4, 6, 1)]) == 0        # a single row
    assert TL.alignment_pad(5, [Operand(2, 8, 1, 4)]) == 7      # base off by 4 bytes
    assert TL.alignment_pad(5, [Operand(2, 3, 7)]) == 0        # strided inner: element path


def test_collapse_cases():
    # [C] broadcast operand keeps two dims
    assert TL.collapse(TL.ELEMWISE, (4, 6), [(6, 1), (0, 1)]) == (4, 6, [(6, 1), (0, 1)])
    # swapped outer dims cannot merge
    assert TL.collapse(TL.ROWREDUCE, (4, 6, 8), [(8, 32, 1)]) is None
    # unit dims dropped; contiguous -> 1-D
    assert TL.collapse(TL.ELEMWISE, (1, 4, 1, 6), [(24, 6, 6, 1)]) == (1, 24, [(0, 1)])
    # row reduce over a 3-D shape, with a [.., 1] row output
    assert TL.collapse(TL.ROWREDUCE, (2, 3, 5), [(15, 5, 1), (3, 1, 0)]) == (6, 5, [(5, 1), (1, 0)])
    # scalar operand
    assert TL.collapse(TL.ELEMWISE, (3, 3), [(3, 1), (0, 0)]) == (1, 9, [(0, 1), (0, 0)])
    # empty
    assert TL.collapse(TL.ELEMWISE, (0, 5), [(5, 1)])[:2] == (0, 0)


def test_coverage_and_ranges_brute_force():
    g = np.random.default_rng(7)
    for _ in range(40):
        tmpl = [TL.ELEMWISE, TL.ROWREDUCE][int(g.integers(0, 2))]
        R = int(g.integers(1, 700))
        C = int(g.integers(1, 3000))
        if tmpl == TL.ELEMWISE and g.random() < 0.5:
            R, C = 1, R * C
        ops = [Operand(4, C if R > 1 else 0, 1), Operand(2, 0, 1)]
        p = TL.plan(tmpl, R, C, ops)
        tiles, wgs = TL.element_tile_map(p)
        assert (tiles >= 0).all()
        # workgroup tile sets are strided by grid, disjoint, at most
        # body_tile long and together cover [0, block_dim) once
        seen = []
        for b in range(p.grid):
            ts = list(TL.workgroup_tiles(b, p.grid, p.block_dim))
            assert 0 < len(ts) <= p.body_tile and ts[0] == b
            assert all(t1 - t0 == p.grid for t0, t1 in zip(ts, ts[1:]))
            seen.extend(ts)
        assert sorted(seen) == list(range(p.block_dim))
        assert p.grid <= TL.G_WG
        # the choice is a least-cost feasible candidate, earliest on ties
        feas = [(c, i) for i, c in enumerate(p.costs) if c is not None]
        cmin = min(c for c, _ in feas)
        first = min(i for c, i in feas if c == cmin)
        assert p.path[first] == (p.tr, p.tc)


def test_header_formula_cases():
    assert TL.header(0) == (0, 0)
    assert TL.header(1) == (1, 1)
    assert TL.header(512) == (1, 512)
    assert TL.header(513) == (2, 257)
    assert TL.header(1024) == (2, 512)
    assert TL.header(1025) == (3, 342)


def test_matmul_plan_by_hand():
    bias = Operand(4, 0, 1)
    y = Operand(2, 17408, 1)
    # per-tile ticks of a 128 x 128 tile (G = 512), worked by hand:
    #   7812 + (128*5120*2 + 5120*128*2 + 128*128*2 + 128*4) + 2*128*128*5120/312.5
    #   = 7812 + 2654720 + 536871 = 3199403
    t128 = 3199403
    p = TL.plan_matmul(1, 17408, 5120, 2, 2, [bias, y])
    assert p.costs == [t128]
    assert (p.tr, p.tc, p.n_r, p.n_c, p.block_dim, p.body_tile, p.grid) == (128, 128, 1, 136, 136, 1, 136)
    # 8192 rows: 64 x 136 = 8704 tiles, 17 rounds of 512, 17 per workgroup
    p = TL.plan_matmul(8192, 17408, 5120, 2, 2, [bias, y])
    assert p.costs == [17 * t128]
    assert (p.n_r, p.n_c, p.block_dim, p.body_tile, p.grid) == (64, 136, 8704, 17, 512)
    # the per-entry residency: a variant with G_e = 256 resident workgroups pays
    # half a tick per byte and G_e / 160000 per flop (worked by hand)
    saved = TL.MM_TILES
    try:
        TL.MM_TILES = [(256, 256, 256)]
        p = TL.plan_matmul(8192, 17408, 5120, 2, 2, [bias, y])
        assert p.costs == [9 * (7812 + 2687488 + 1073742)]
        assert (p.block_dim, p.body_tile, p.grid) == (2176, 9, 242)
    finally:
        TL.MM_TILES = saved
    # ragged edges: 300 x 1000 -> 3 x 8 tiles, the last row and column tiles partial
    p = TL.plan_matmul(300, 1000, 64, 2, 2, [])
    assert (p.tr, p.n_r, p.n_c, p.block_dim) == (128, 3, 8, 24)
    tiles, wgs = TL.element_tile_map(p)
    assert tiles[299, 999] == 23 and tiles[256, 0] == 16 and tiles[0, 896] == 7
    assert (tiles >= 0).all()
    assert TL.plan_matmul(0, 5, 8, 2, 2, []).block_dim == 0


# ---------------------------------------------------------------------------
# MIX tile order (grouped rows, XCD-aware starting positions)
# ---------------------------------------------------------------------------
def test_mix_order_hand_worked():
    # 10 row tiles x 3 column tiles: the first group holds rows 0..7, the
    # second rows 8..9; inside a group the order walks column by column
    order = [TL.mix_tile_coords(v, 10, 3) for v in range(30)]
    assert order[:9] == [(0, 0), (1, 0), (2, 0), (3, 0), (4, 0), (5, 0), (6, 0), (7, 0), (0, 1)]
    assert order[23] == (7, 2)
    assert order[24:] == [(8, 0), (9, 0), (8, 1), (9, 1), (8, 2), (9, 2)]
    # grid 500: grid8 = 496, 62 positions per XCD; workgroup 8k + x starts at 62x + k
    assert [TL.mix_first_position(b, 500) for b in (0, 1, 7, 8, 9, 495, 496, 499)] == \
        [0, 62, 434, 1, 63, 495, 496, 499]


@pytest.mark.parametrize("n_r,n_c,grid", [(10, 3, 30), (64, 136, 512), (16, 136, 512), (3, 5, 15), (1, 1, 1),
                                          (9, 7, 63)])
def test_mix_order_is_a_bijection(n_r, n_c, grid):
    block_dim = n_r * n_c
    body_tile = -(-block_dim // min(512, block_dim))
    seen = set()
    for b in range(grid):
        pos = list(TL.mix_workgroup_positions(b, grid, block_dim))
        assert len(pos) <= body_tile
        seen.update(TL.mix_tile_coords(v, n_r, n_c) for v in pos)
    assert seen == {(r, c) for r in range(n_r) for c in range(n_c)}
    assert sorted(TL.mix_first_position(b, grid) for b in range(grid)) == list(range(grid))


def test_mix_element_map_covers_ragged_output():
    p = TL.plan_matmul(300, 1000, 64, 2, 2, [])
    tiles, wgs = TL.mix_element_tile_map(p)
    assert (tiles >= 0).all() and (wgs >= 0).all()
    assert tiles[299, 999] == (p.n_r - 1) * p.n_c + p.n_c - 1


@pytest.mark.parametrize("grid,bds", [(512, [3000, 1, 517, 9000]), (7, [3, 4, 5]), (5, [12]), (64, [0, 70, 0, 3])])
def test_temporal_stack_tiles_cover_once_and_balance(grid, bds):
    """Temporal stack order: every (segment, tile) runs exactly once; each
    workgroup walks the segments in order; workgroups get the stack's tiles
    as evenly as the count allows (floor or ceil of total / grid)."""
    seen = {}
    counts = []
    for b in range(grid):
        run = TL.temporal_stack_tiles(b, grid, bds)
        assert [s for s, _ in run] == sorted(s for s, _ in run)
        for st in run:
            assert st not in seen
            seen[st] = b
        counts.append(len(run))
    assert set(seen) == {(s, t) for s, bd in enumerate(bds) for t in range(bd)}
    total = sum(bds)
    assert min(counts) >= total // grid and max(counts) <= -(-total // grid)
    # tile u of the stack's space runs on workgroup u mod grid
    base = 0
    for s, bd in enumerate(bds):
        for t in range(bd):
            assert seen[(s, t)] == (base + t) % grid
        base += bd


def test_wide_grid_rule_hand_worked():
    """Long wide-build programs run as workgroups of about 8 tiles (up to
    8192 of them).  Hand-worked: the 126576-row LayerNorm over 5120 columns
    tiles as 4 x 5120 (31644 tiles); 31644 / 512 would give 62 tiles per
    workgroup, more than 8, so the header is taken with min(8192, 31644 // 8)
    = 3955 workgroups: ceil(31644 / 3955) = 9 tiles each (3955 * 8 = 31640 <
    31644), ceil(31644 / 9) = 3516 workgroups."""
    ops = [Operand(2, 5120, 1), Operand(4, 0, 1), Operand(4, 0, 1), Operand(2, 5120, 1)]
    p = TL.plan(TL.ROWREDUCE, 126576, 5120, ops, TL.NV_WIDE)
    assert (p.tr, p.tc, p.block_dim, p.body_tile, p.grid) == (4, 5120, 31644, 9, 3516)
    # 16384 rows: 4096 tiles, 8 per workgroup at 512: the rule does not apply
    p = TL.plan(TL.ROWREDUCE, 16384, 5120, ops, TL.NV_WIDE)
    assert (p.block_dim, p.body_tile, p.grid) == (4096, 8, 512)
    # 200000 rows: 50000 tiles, min(8192, 6250) = 6250 workgroups of 8
    p = TL.plan(TL.ROWREDUCE, 200000, 5120, ops, TL.NV_WIDE)
    assert (p.block_dim, p.body_tile, p.grid) == (50000, 8, 6250)
    # 400000 rows: 100000 tiles, at the cap: 8192 workgroups of ceil(100000 / 8192) = 13,
    # ceil(100000 / 13) = 7693 of them used
    p = TL.plan(TL.ROWREDUCE, 400000, 5120, ops, TL.NV_WIDE)
    assert (p.block_dim, p.body_tile, p.grid) == (100000, 13, 7693)
    # the standard build keeps G: 126576 x 1024 (one row per tile) stays at 512 workgroups
    q = TL.plan(TL.ROWREDUCE, 126576, 1024, [Operand(2, 1024, 1), Operand(2, 1024, 1)])
    assert q.grid <= TL.G_WG and q.body_tile > TL.WIDE_WG_TILES


def test_wide_grid_rule_invariants():
    g = np.random.default_rng(11)
    for _ in range(60):
        R = int(g.integers(1, 400000))
        ops = [Operand(2, 5120, 1), Operand(4, 0, 1), Operand(2, 5120, 1)]
        p = TL.plan(TL.ROWREDUCE, R, 5120, ops, TL.NV_WIDE)
        if p.block_dim <= 8 * TL.G_WG:
            assert p.grid <= TL.G_WG and p.body_tile <= TL.WIDE_WG_TILES
        else:
            assert TL.G_WG <= p.grid <= TL.WIDE_GRID_MAX
            assert p.body_tile <= max(TL.WIDE_WG_TILES + 1, -(-p.block_dim // TL.WIDE_GRID_MAX))
        # the strided sets still cover every tile once, at most body_tile each
        seen = []
        for b in range(p.grid):
            ts = list(TL.workgroup_tiles(b, p.grid, p.block_dim))
            assert 0 < len(ts) <= p.body_tile
            seen.extend(ts)
        assert sorted(seen) == list(range(p.block_dim))
