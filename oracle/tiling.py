"""Shape tiling, header, tile ranges and the element -> tile map
(test infrastructure; an independent statement of the encoder's rules).

Source: the DVM paper review page, section 4.2 (shape tiling: find the
dominant shape S_d, start from the largest tile L = S_d, shrink tiles from the
outer dims inward, prune candidates by hardware resource limits and a
lightweight cost model; hardware_align_div takes the least-cost tile size and
rounds it up to a multiple of the hardware instruction width), section 4.3
(header: tile count block_dim, tiles per core body_tile, kernel type) and
section 4.4 (each core computes its tile count and its tile range, then runs
the bytecode per tile).  Section 7 of that page adds that tiling uses
dedicated templates and needs no measurement on hardware.

Readings taken where the page leaves a step open (each also listed in the
design notes):

* Iteration space.  The dominant shape is collapsed to two dims [R, C]: C is
  the innermost dim, R the product of the outer dims.  Elementwise graphs whose
  every operand is contiguous (or a scalar) collapse further to [1, numel].
* Per-core resource.  A core is one workgroup of T = 256 lanes, two of them
  resident per compute unit; a tile row is spread over g lanes, each holding
  up to NV_MAX = 5 chunks of V = 8 elements in registers.  Rows of a tile go
  to P = next_pow2(tr) lane groups of g = T / P lanes.  A tile is feasible iff
  P <= T and NV = ceil((tc + pad) / (g V)) <= NV_MAX.
* Wide variant.  The VM also comes as a wide build whose one tile register
  holds NV_WIDE = 10 chunks per lane (the same per-lane register budget spent
  on one tile value instead of three): the same rules with NV_MAX replaced by
  NV_WIDE.  The encoder uses it for programs that keep every tile value in
  the accumulator and reduce rows, where the standard plan has no feasible
  tile, or where the wide plan puts more rows in a tile and either keeps the
  LDS staging or runs one tile per workgroup.  plan() takes the variant's
  chunk limit.
* Alignment pad.  pad = V - 1 if some unit-stride operand does not start every
  row on a 16-byte boundary, else 0: a misaligned row may need one more chunk.
* hardware_align_div(n, k, W) = W * ceil(ceil(n / k) / W) with W = 64 V = 512
  (one wave of 16-byte vectors of the narrowest type), clamped to C.
* Shrink path (outer -> inner).  Row-reduce graphs pin tc = C and try
  tr = ceil(R / k) for k = 1, 2, 4, ... down to 1, each followed by its
  power-of-two floor: rows go to next_pow2(tr) lane groups, so that floor is
  the largest tile whose rows fill their groups (tr = 3 leaves one group of
  four idle; on MI355X LayerNorm calls tiled 3 rows at a time ran at 4.8
  TB/s against 5.3 for 4).  Elementwise and
  reduce-all graphs first try the same row counts with the widest aligned tc,
  then, at tr = 1, tc = min(C, had(C, k, W)) for k = 2, 4, ... until tc stops
  changing or reaches W.  Consecutive duplicates are dropped.
* Cost (integer "ticks", 1 tick = 1/15625 us): G = 512 resident workgroups
  (two per compute unit), A = 78125 ticks (5 us) of fixed time per round of
  tiles, and 1 tick per byte a workgroup moves (8 TB/s shared by G workgroups
  is 15625 bytes/us each).  A is measured on MI355X: on latency-bound calls
  (LayerNorm over 1385 rows of 5120) one more round of tiles cost 6.4 us, of
  which the bytes account for about 1.3 us:
  cost = ceil(n_tiles / G) * (A + var_bytes) + inv_bytes, where
  var_bytes are the bytes one tile touches in operands that change from tile
  to tile and inv_bytes those of tile-invariant operands, loaded once per
  workgroup.  The least cost wins; ties go to the earlier candidate (the
  larger tile).
* MATMUL graphs (a matmul [M, K] x [K, N] first, elementwise ops on its [M, N]
  output after it): K is pinned (every tile runs the whole K loop) and the
  output is tiled tm x tn from the MIX kernel's tile menu MM_TILES (multiples
  of 32, the MFMA block; the matrix-core analogue of hardware_align_div).
  Each entry runs with its own number G_e of resident workgroups, which share
  the chip's 8 TB/s and 2.5 PFLOP/s (bf16 matrix peak).  In the same ticks a
  byte costs G_e / 512 and a flop G_e / 160000, so a candidate costs
  ceil(n_tiles / G_e) * (A_MM + ceil(var_bytes G_e / 512) + ceil(flops G_e / 160000))
  + ceil(inv_bytes G_e / 512), with A_MM = 7812 ticks (0.5 us; a MIX tile's
  fixed work is small next to its K loop), var_bytes the A and B panels one tile reads
  (tm K + K tn elements) plus its varying epilogue operand and output bytes and
  flops = 2 tm tn K.  The least cost wins; ties go to the earlier (larger)
  entry.
* Header: block_dim = n_tiles; body_tile = ceil(block_dim / min(G,
  block_dim)); grid = ceil(block_dim / body_tile).  Tile id -> (ir, ic) is
  row-major with the column index fastest.  A wide-build plan (nv_max =
  NV_WIDE) whose body_tile would exceed WIDE_WG_TILES = 8 is re-headed with
  min(WIDE_GRID_MAX = 8192, block_dim // 8) in place of G: about 8 tiles per
  workgroup and more workgroups than are resident (see the deviation below).

Deviations from the page (stated here because the tile maps follow them):

* Tile range of a core (section 4.4).  The page has each core compute its
  tile range, which reads most plainly as the contiguous range [b body_tile,
  (b + 1) body_tile).  This build gives workgroup b the strided set b,
  b + grid, b + 2 grid, ... below block_dim instead: still at most body_tile
  tiles, but at any moment the resident workgroups run neighbouring tiles, so
  their streams advance together through memory (on MI355X 6% faster on the
  LayerNorm stream and up to 14% on copy-like graphs).
* More workgroups than cores for long wide-build programs.  The page's core
  count is the grid.  On MI355X the two workgroups that share a compute unit
  stream at different rates (the older one wins issue arbitration: measured
  12% apart on a 126576-row LayerNorm), so equal static shares leave the
  faster half idle at the end.  A wide-build program with more than 8 tiles
  per workgroup therefore runs as up to 8192 workgroups of about 8 tiles,
  and the hardware dispatcher hands the next one to whichever slot frees
  first (LayerNorm stream +3 to 5%; standard-build and reduce-all programs
  measured no better or worse, so they keep G).  The cap was 4096 at first;
  8192 lets the op stream's softmax over 69740 tiles run 9 tiles per
  workgroup instead of 18 (op stream +1.9%; the LayerNorm calls stay below
  either cap).
* MIX tile order.  The MIX kernel keeps block_dim, body_tile and grid, and
  walks the [M, N] output tiles in a grouped order for the L2 caches of the
  eight XCDs: row tiles go in groups of MM_GROUP = 8; inside a group the
  order runs column by column with the group's row tiles fastest.  Workgroups
  are dispatched to the XCDs in turn (b to XCD b mod 8), and the kernel gives
  the workgroups of one XCD consecutive starting positions in that order:
  with grid8 = grid rounded down to a multiple of 8, workgroup b = 8 k + x
  (b < grid8) starts at position x (grid8 / 8) + k, a workgroup past grid8 at
  position b; each then takes every grid-th position below block_dim.
"""
from __future__ import annotations

from dataclasses import dataclass, field

T_LANES = 256
VEC = 8
NV_MAX = 5
NV_WIDE = 10
W_ALIGN = 64 * VEC
G_WG = 512
WIDE_WG_TILES = 8       # tiles per workgroup of a long wide-build program
WIDE_GRID_MAX = 8192    # workgroups of such a program, at most
A_TICKS = 78125
A_MM_TICKS = 7812
BYTE_TICKS = 1

ELEMWISE, ROWREDUCE, ALLREDUCE, MATMUL = "elemwise", "rowreduce", "allreduce", "matmul"

# (tm, tn, resident workgroups) of the MIX kernel's tile variants, largest first
MM_TILES = [(128, 128, 512)]
MM_GROUP = 8        # row tiles per group of the MIX tile order
N_XCD = 8           # accelerator complex dies (each with its own L2)


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def next_pow2(x: int) -> int:
    p = 1
    while p < x:
        p *= 2
    return p


def had(n: int, k: int, w: int) -> int:
    """hardware_align_div: ceil(n / k) rounded up to a multiple of w."""
    return w * cdiv(cdiv(n, k), w)


@dataclass
class Operand:
    """A global operand in the collapsed [R, C] space (strides in elements)."""
    esize: int
    s_r: int
    s_c: int
    base_mod16: int = 0


@dataclass
class Plan:
    template: str
    R: int
    C: int
    pad: int
    path: list
    tr: int = 0
    tc: int = 0
    g: int = 0
    nv: int = 0
    P: int = 0
    n_r: int = 0
    n_c: int = 0
    block_dim: int = 0
    body_tile: int = 0
    grid: int = 0
    costs: list = field(default_factory=list)


# ---------------------------------------------------------------------------
# Dim collapse
# ---------------------------------------------------------------------------
def _drop_unit(shape, strides):
    keep = [i for i, d in enumerate(shape) if d != 1]
    return [shape[i] for i in keep], [[s[i] for i in keep] for s in strides]


def collapse(template, shape, op_strides):
    """Collapse the dominant shape to [R, C].

    ``op_strides``: per global operand, its strides over ``shape`` (0 on a
    broadcast dim).  Returns (R, C, [(s_r, s_c)]) or None when some operand's
    outer dims cannot be merged into one row index.
    """
    numel = 1
    for d in shape:
        numel *= d
    if numel == 0:
        return 0, 0, [(0, 0) for _ in op_strides]
    dims, strides = _drop_unit(list(shape), [list(s) for s in op_strides])
    if not dims:
        return 1, 1, [(0, 0) for _ in op_strides]

    def mergeable(s, lo, hi):
        # dims lo..hi-1 of one operand merge into one index
        return all(s[i] == s[i + 1] * dims[i + 1] for i in range(lo, hi - 1))

    if template in (ELEMWISE, ALLREDUCE) and all(mergeable(s, 0, len(dims)) for s in strides):
        return 1, numel, [(0, s[-1]) for s in strides]
    # two dims: innermost dim of the dominant shape (even if it has size 1)
    C = shape[-1] if len(shape) else 1
    if C == 1:
        outer_dims = dims
        outer_strides = strides
    else:
        outer_dims = dims[:-1]
        outer_strides = [s[:-1] for s in strides]
    R = 1
    for d in outer_dims:
        R *= d
    out = []
    for s_full, s in zip(strides, outer_strides):
        if not all(s[i] == s[i + 1] * outer_dims[i + 1] for i in range(len(outer_dims) - 1)):
            return None
        s_r = s[-1] if outer_dims else 0
        s_c = s_full[-1] if C != 1 else 0
        out.append((s_r, s_c))
    return R, C, out


# ---------------------------------------------------------------------------
# Geometry, path, cost, choice
# ---------------------------------------------------------------------------
def alignment_pad(R: int, ops) -> int:
    for o in ops:
        if o.s_c != 1:
            continue
        if o.base_mod16 % 16 != 0:
            return VEC - 1
        if R > 1 and (o.s_r * o.esize) % 16 != 0:
            return VEC - 1
    return 0


def geometry(tr: int, tc: int, pad: int, nv_max: int = NV_MAX):
    """(P, g, NV, feasible) of a tr x tc tile."""
    P = next_pow2(tr)
    if P > T_LANES:
        return P, 0, 0, False
    g = T_LANES // P
    nv = cdiv(tc + pad, g * VEC)
    return P, g, nv, nv <= nv_max


def shrink_path(template: str, R: int, C: int):
    path = []

    def push(t):
        if not path or path[-1] != t:
            path.append(t)

    def push_rows(tr, tc):
        push((tr, tc))
        f = 1
        while 2 * f <= tr:
            f *= 2
        push((f, tc))

    if template == ROWREDUCE:
        k = 1
        while True:
            tr = cdiv(R, k)
            push_rows(tr, C)
            if tr <= 1:
                break
            k *= 2
        return path
    tc0 = min(C, had(C, 1, W_ALIGN))
    k = 1
    while True:
        tr = cdiv(R, k)
        push_rows(tr, tc0)
        if tr <= 1:
            break
        k *= 2
    prev = tc0
    k = 2
    while prev > W_ALIGN:
        tc = min(C, had(C, k, W_ALIGN))
        if tc == prev:
            break
        push((1, tc))
        prev = tc
        k *= 2
    return path


def cost(R: int, C: int, tr: int, tc: int, ops) -> int:
    n_r, n_c = cdiv(R, tr), cdiv(C, tc)
    n_tiles = n_r * n_c
    var_b, inv_b = 0, 0
    for o in ops:
        touched = (tr if o.s_r != 0 else 1) * (tc if o.s_c != 0 else 1) * o.esize
        invariant = (o.s_r == 0 or n_r == 1) and (o.s_c == 0 or n_c == 1)
        if invariant:
            inv_b += touched
        else:
            var_b += touched
    rounds = cdiv(n_tiles, G_WG)
    return rounds * (A_TICKS + BYTE_TICKS * var_b) + BYTE_TICKS * inv_b


def plan(template: str, R: int, C: int, ops, nv_max: int = NV_MAX) -> Plan:
    """Tile choice and header for a vector-template graph over [R, C], for
    the VM variant whose tile register holds nv_max chunks per lane."""
    pad = alignment_pad(R, ops)
    p = Plan(template, R, C, pad, [])
    if R == 0 or C == 0:
        return p
    p.path = shrink_path(template, R, C)
    best = None
    for (tr, tc) in p.path:
        P, g, nv, ok = geometry(tr, tc, pad, nv_max)
        if not ok:
            p.costs.append(None)
            continue
        c = cost(R, C, tr, tc, ops)
        p.costs.append(c)
        if best is None or c < best[0]:
            best = (c, tr, tc, P, g, nv)
    if best is None:
        raise ValueError("no feasible tile")
    _, p.tr, p.tc, p.P, p.g, p.nv = best
    p.n_r, p.n_c = cdiv(R, p.tr), cdiv(C, p.tc)
    p.block_dim = p.n_r * p.n_c
    p.body_tile, p.grid = header(p.block_dim)
    if nv_max == NV_WIDE and p.body_tile > WIDE_WG_TILES:
        p.body_tile, p.grid = header(p.block_dim, min(WIDE_GRID_MAX, p.block_dim // WIDE_WG_TILES))
    return p


def plan_matmul(M: int, N: int, K: int, a_esize: int, b_esize: int, epi_ops) -> Plan:
    """Tile choice and header for a MATMUL graph over its [M, N] output.
    ``epi_ops``: the epilogue's global operands (inputs and stored outputs) in
    the [M, N] space, as Operand(esize, s_r, s_c)."""
    p = Plan(MATMUL, M, N, 0, [])
    if M == 0 or N == 0:
        return p
    p.path = [(tm, tn) for tm, tn, _ in MM_TILES]
    best = None
    for (tm, tn, ge) in MM_TILES:
        n_r, n_c = cdiv(M, tm), cdiv(N, tn)
        var_b = tm * K * a_esize + K * tn * b_esize
        inv_b = 0
        for o in epi_ops:
            touched = (tm if o.s_r != 0 else 1) * (tn if o.s_c != 0 else 1) * o.esize
            invariant = (o.s_r == 0 or n_r == 1) and (o.s_c == 0 or n_c == 1)
            if invariant:
                inv_b += touched
            else:
                var_b += touched
        per_tile = A_MM_TICKS + cdiv(var_b * ge, 512) + cdiv(2 * tm * tn * K * ge, 160000)
        c = cdiv(n_r * n_c, ge) * per_tile + cdiv(inv_b * ge, 512)
        p.costs.append(c)
        if best is None or c < best[0]:
            best = (c, tm, tn, ge)
    _, p.tr, p.tc, ge = best
    p.n_r, p.n_c = cdiv(M, p.tr), cdiv(N, p.tc)
    p.block_dim = p.n_r * p.n_c
    p.body_tile, p.grid = header(p.block_dim, ge)
    return p


def header(block_dim: int, g_res: int = G_WG):
    if block_dim == 0:
        return 0, 0
    gp = min(g_res, block_dim)
    body_tile = cdiv(block_dim, gp)
    grid = cdiv(block_dim, body_tile)
    return body_tile, grid


def workgroup_tiles(b: int, grid: int, block_dim: int):
    """Tile ids run by workgroup b: b, b + grid, b + 2 grid, ... below
    block_dim (at most body_tile of them)."""
    return range(b, block_dim, grid)


def temporal_stack_tiles(b: int, grid: int, block_dims):
    """(segment, tile) pairs run, in order, by workgroup b of a temporally
    stacked launch of `grid` workgroups over programs of block_dims tiles
    (stacking-based fusion, temporal: tiles of different graphs run on one
    core in sequence).  The segments' tiles are numbered as one space in
    segment order; tile u of that space runs on workgroup u mod grid.  Inside
    segment s workgroup b then plays workgroup (b - base_s) mod grid of the
    segment's own strided order (base_s = tiles of the segments before it)."""
    out, base = [], 0
    for s, bd in enumerate(block_dims):
        t0 = (b - base) % grid
        out += [(s, t) for t in workgroup_tiles(t0, grid, bd)]
        base += bd
    return out


def tile_box(tile_id: int, tr: int, tc: int, R: int, C: int, n_c: int):
    ir, ic = divmod(tile_id, n_c)
    return (ir * tr, min(ir * tr + tr, R)), (ic * tc, min(ic * tc + tc, C))


def element_tile_map(p: Plan):
    """For every element (r, c) of [R, C]: the id of the tile that holds it
    and the workgroup that runs that tile, built by walking every tile's box
    (no closed form, so it checks coverage independently)."""
    import numpy as np
    tiles = np.full((p.R, p.C), -1, dtype=np.int64)
    wgs = np.full((p.R, p.C), -1, dtype=np.int64)
    for b in range(p.grid):
        for t in workgroup_tiles(b, p.grid, p.block_dim):
            (r0, r1), (c0, c1) = tile_box(t, p.tr, p.tc, p.R, p.C, p.n_c)
            if (tiles[r0:r1, c0:c1] != -1).any():
                raise AssertionError("element covered twice")
            tiles[r0:r1, c0:c1] = t
            wgs[r0:r1, c0:c1] = b
    return tiles, wgs


# ---------------------------------------------------------------------------
# MIX tile order
# ---------------------------------------------------------------------------
def mix_tile_coords(v: int, n_r: int, n_c: int):
    """(row tile, column tile) at position v of the grouped order."""
    per_group = MM_GROUP * n_c
    grp, w = divmod(v, per_group)
    r0 = grp * MM_GROUP
    rows = min(MM_GROUP, n_r - r0)
    return r0 + w % rows, w // rows


def mix_first_position(b: int, grid: int) -> int:
    """Starting position of workgroup b in the grouped order."""
    grid8 = grid - grid % N_XCD
    if b >= grid8:
        return b
    k, x = divmod(b, N_XCD)
    return x * (grid8 // N_XCD) + k


def mix_workgroup_positions(b: int, grid: int, block_dim: int):
    return range(mix_first_position(b, grid), block_dim, grid)


def mix_element_tile_map(p: Plan):
    """For every element (m, n) of a MATMUL plan's [M, N] output: the
    row-major id of the tile that holds it and the workgroup that runs it,
    built by walking every workgroup's positions (so it also checks that the
    order covers every element exactly once)."""
    import numpy as np
    tiles = np.full((p.R, p.C), -1, dtype=np.int64)
    wgs = np.full((p.R, p.C), -1, dtype=np.int64)
    for b in range(p.grid):
        for v in mix_workgroup_positions(b, p.grid, p.block_dim):
            ir, ic = mix_tile_coords(v, p.n_r, p.n_c)
            r0, r1 = ir * p.tr, min(ir * p.tr + p.tr, p.R)
            c0, c1 = ic * p.tc, min(ic * p.tc + p.tc, p.C)
            if (tiles[r0:r1, c0:c1] != -1).any():
                raise AssertionError("element covered twice")
            tiles[r0:r1, c0:c1] = ir * p.n_c + ic
            wgs[r0:r1, c0:c1] = b
    return tiles, wgs
