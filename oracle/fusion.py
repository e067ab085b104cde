"""Streaming-fusion partition rules (test infrastructure; an independent
statement of the fuser's rules).

Source: the DVM paper review page, section 5.2 (dynamic-graph fusion: ops are
added to a buffer in order; the fusion conditions -- shape compatibility and
dependence -- are checked; fusible ops are fused; when a new op cannot be fused
or a communication condition holds, the buffered ops are flushed to the
compiler; the decisions need no cache), and the MindSpore DVM summary page,
sections 3.2-3.3 (capture and incremental graph building; a flush happens on an
op that cannot be fused, at a fusion boundary or at a synchronisation
interface; streaming fusion decides at run time, e.g. when two expressions
turn out to have equal shapes; pattern fusion covers elemwise-elemwise,
reduce forward fusion and MatMul+elemwise).

Readings taken (the pages give only "shape compatibility and dependence"):

* Unit of decision.  A *group* is either one primitive op or a composite the
  caller brackets (LayerNorm, RMSNorm, softmax, ...).  The decision is taken
  when the group is complete: the whole group joins the buffered graph or the
  graph is flushed and the group starts a new one.  Values made and released
  inside a group never need storage.
* Iteration shape.  Elementwise op: its output shape; row reduce: its input
  shape; reduce-all: its input shape; matmul: its [M, N] output.
* Dominant shape S_d: the iteration shape of largest rank, then largest numel,
  then the earliest op.  row(S_d) = S_d with its last dim set to 1.
* Pattern (F2/F3).  Every row or all reduce iterates over S_d.  Every other op
  iterates over S_d or row(S_d).  A matmul may only be a graph's first op; a
  matmul graph holds no reduce.  A reduce-all (sum or max over all axes) must be
  the graph's last op, the graph holds no row reduce, and the graph is flushed
  as soon as it is added.  Every external operand's strides over S_d must
  collapse to the [R, C] space of the tiling rules.
* Dependence (F4), through memory: the group may not write storage that the
  buffered graph reads from an external tensor (WAR), may not read storage the
  buffered graph may still write (RAW not carried by a value), and may not
  write storage the buffered graph may still write (WAW).  A value is carried
  on chip only when the consumer names the producer's value.
* Resources (F7): at most 64 ops; at most 24 distinct external tensors; at
  every op at most 3 tile-shaped values in flight (live values plus the op's
  output: the device keeps a tile in at most three register sets) and at most
  4 row values in flight; and a feasible tile exists.
* A value is stored when its graph is flushed if it is marked live, or if the
  caller has not released it by then.
"""
from __future__ import annotations

import numpy as np

from . import tiling as TL

MAX_OPS = 64
MAX_EXT = 24
MAX_TILE_VALUES = 3
MAX_ROW_VALUES = 4

ESIZE = {"f32": 4, "bf16": 2, "u8": 1}
ELEMWISE_OPS = {"add", "sub", "mul", "div", "max", "min", "pow", "sqrt", "abs", "log", "exp",
                "round", "floor", "isfinite", "neg", "recip", "cast", "copy"}
REDUCE_OPS = {"reduce_sum", "reduce_max"}


def row_shape(s):
    return tuple(s[:-1]) + (1,) if len(s) else ()


def numel(s):
    n = 1
    for d in s:
        n *= d
    return n


def bcast_strides(shape, strides, target):
    """Strides of a tensor broadcast (numpy rules) to ``target``."""
    nd = len(target)
    out = [0] * nd
    off = nd - len(shape)
    for i, (d, s) in enumerate(zip(shape, strides)):
        j = off + i
        out[j] = 0 if (d == 1 and target[j] != 1) else s
    return out


class Stream:
    """Replays a stream of events and records the graph partition.

    Events (tuples):
      ("input", name, shape, strides, dtype, addr)   external tensor
      ("group", [op, ...])                           ops; see below
      ("release", name)
      ("flush",)                                     explicit flush
      ("sync",)                                      synchronisation point
    An op is a dict {"op", "in": [names or floats], "out", "shape", "dtype",
    "axis" (reduces: -1 or None), "live": bool, "addr" (storage or None),
    "nbytes"}.
    """

    def __init__(self):
        self.ext = {}          # name -> dict(shape, strides, dtype, addr, nbytes)
        self.vals = {}         # op output name -> op dict
        self.released = set()
        self.buf = []          # ops of the buffered graph
        self.graphs = []       # (list of op outs, reason, stored outs)
        self.unsupported = []
        self.lost = set()      # values whose graph was flushed without storing them

    # -- events ---------------------------------------------------------
    def run(self, events):
        for ev in events:
            kind = ev[0]
            if kind == "input":
                _, name, shape, strides, dtype, addr = ev
                nb = (max((d - 1) * s for d, s in zip(shape, strides)) + 1 if numel(shape) else 0) * ESIZE[dtype] if len(shape) else ESIZE[dtype]
                self.ext[name] = dict(shape=tuple(shape), strides=tuple(strides), dtype=dtype, addr=addr, nbytes=nb)
            elif kind == "group":
                self.add_group(ev[1])
            elif kind == "release":
                self.released.add(ev[1])
            elif kind in ("flush", "sync"):
                self.flush("explicit" if kind == "flush" else "sync")
        return self.graphs

    def flush(self, reason):
        if not self.buf:
            return
        stored = [o["out"] for o in self.buf if o["live"] or o["out"] not in self.released]
        self.graphs.append(([o["out"] for o in self.buf], reason, stored))
        # a stored value is read back from its storage by later graphs
        for o in self.buf:
            if o["out"] in stored and o.get("addr") is not None:
                shape = tuple(o["shape"])
                st, acc = [], 1
                for d in reversed(shape):
                    st.append(acc)
                    acc *= d
                self.ext[o["out"]] = dict(shape=shape, strides=tuple(reversed(st)), dtype=o["dtype"],
                                          addr=o["addr"], nbytes=o["nbytes"])
            elif o["out"] not in stored:
                self.lost.add(o["out"])
            else:
                raise ValueError(f"value {o['out']} must be stored but has no storage")
        self.buf = []

    # -- group decision -------------------------------------------------
    def add_group(self, grp):
        for o in grp:
            for x in o["in"]:
                if isinstance(x, str) and x in self.lost:
                    raise ValueError(f"value {x} was flushed without storage")
            self.vals[o["out"]] = o
        if self.buf:
            why = self.check(self.buf + list(grp), len(self.buf))
            if why is None:
                self.buf.extend(grp)
                self._close_if_reduce_all()
                return
            self.flush(why)
        why = self.check(list(grp), 0)
        if why is not None:
            self.unsupported.append(([o["out"] for o in grp], why))
            return
        self.buf = list(grp)
        self._close_if_reduce_all()

    def _close_if_reduce_all(self):
        if self.buf and self.buf[-1]["op"] in REDUCE_OPS and self.buf[-1].get("axis", -1) is None:
            self.flush("reduce_all")

    # -- legality of a candidate graph ------------------------------------
    def iter_shape(self, o):
        if o["op"] in REDUCE_OPS:
            return self.shape_of(o["in"][0])
        return tuple(o["shape"])

    def shape_of(self, x):
        if isinstance(x, (int, float)):
            return ()
        if x in self.ext:
            return self.ext[x]["shape"]
        return tuple(self.vals[x]["shape"])

    def check(self, ops, n_old):
        r = self.check_pattern(ops)
        if r:
            return r
        r = self.check_dependence(ops, n_old)
        if r:
            return r
        return self.check_resources(ops)

    def dominant(self, ops):
        best, key = None, None
        for o in ops:
            s = self.iter_shape(o)
            k = (len(s), numel(s))
            if key is None or k > key:
                best, key = s, k
        return best

    def template(self, ops):
        if ops[0]["op"] == "matmul":
            return TL.MATMUL
        if any(o["op"] in REDUCE_OPS and o.get("axis", -1) is None for o in ops):
            return TL.ALLREDUCE
        if any(o["op"] in REDUCE_OPS for o in ops):
            return TL.ROWREDUCE
        return TL.ELEMWISE

    def check_pattern(self, ops):
        sd = self.dominant(ops)
        rs = row_shape(sd)
        n_all = 0
        n_row = 0
        for i, o in enumerate(ops):
            name = o["op"]
            if name == "matmul":
                if i != 0:
                    return "pattern"
                continue
            if name in REDUCE_OPS:
                if self.iter_shape(o) != sd:
                    return "shape"
                if o.get("axis", -1) is None:
                    n_all += 1
                    if i != len(ops) - 1:
                        return "pattern"
                else:
                    n_row += 1
                continue
            s = tuple(o["shape"])
            if s != sd and s != rs:
                return "shape"
        if ops[0]["op"] == "matmul" and (n_all or n_row):
            return "pattern"
        if n_all and n_row:
            return "pattern"
        if n_all > 1:
            return "pattern"
        if self.collapse(ops, sd) is None:
            return "shape"
        return None

    def ext_operands(self, ops):
        """External tensors read by the graph, in first-use order."""
        seen = []
        for o in ops:
            if o["op"] == "matmul":
                continue
            for x in o["in"]:
                if isinstance(x, str) and x in self.ext and x not in seen:
                    seen.append(x)
        return seen

    def collapse(self, ops, sd):
        tmpl = self.template(ops)
        if tmpl == TL.MATMUL:
            sd2 = sd
        else:
            sd2 = sd
        strides = []
        for x in self.ext_operands(ops):
            e = self.ext[x]
            if len(e["shape"]) > len(sd2):
                return None
            try:
                np.broadcast_shapes(e["shape"], sd2)
            except ValueError:
                return None
            strides.append(bcast_strides(e["shape"], e["strides"], sd2))
        # stored outputs are dense tensors of their own shape
        for o in ops:
            if o["op"] == "matmul" or o.get("addr") is None:
                continue
            s = tuple(o["shape"])
            if o["op"] in REDUCE_OPS and o.get("axis", -1) is None:
                continue
            dense = [0] * len(s)
            acc = 1
            for j in range(len(s) - 1, -1, -1):
                dense[j] = acc
                acc *= s[j]
            strides.append(bcast_strides(s, dense, sd2))
        if tmpl == TL.MATMUL:
            return (sd2[0], sd2[1], strides)
        return TL.collapse(tmpl, sd2, strides)

    def _writes(self, ops):
        out = []
        for o in ops:
            if o.get("addr") is not None and (o["live"] or o["out"] not in self.released):
                out.append((o["addr"], o["nbytes"]))
        return out

    @staticmethod
    def _overlap(a, b):
        return a[0] < b[0] + b[1] and b[0] < a[0] + a[1]

    def check_dependence(self, ops, n_old):
        if n_old == 0:
            return None
        old, new = ops[:n_old], ops[n_old:]
        old_reads = [(self.ext[x]["addr"], self.ext[x]["nbytes"]) for x in self.ext_operands(old)
                     if self.ext[x]["nbytes"]]
        for o in old:
            if o["op"] == "matmul":
                for x in o["in"]:
                    if x in self.ext:
                        old_reads.append((self.ext[x]["addr"], self.ext[x]["nbytes"]))
        old_writes = self._writes(old)
        new_reads = []
        for o in new:
            for x in o["in"]:
                if isinstance(x, str) and x in self.ext and self.ext[x]["nbytes"]:
                    new_reads.append((self.ext[x]["addr"], self.ext[x]["nbytes"]))
        new_writes = [(o["addr"], o["nbytes"]) for o in new if o.get("addr") is not None]
        for w in new_writes:
            if any(self._overlap(w, r) for r in old_reads):
                return "dependence"
            if any(self._overlap(w, r) for r in old_writes):
                return "dependence"
        for r in new_reads:
            if any(self._overlap(r, w) for w in old_writes):
                return "dependence"
        return None

    def value_class(self, ops, sd):
        """'tile' or 'row' for every value (op outputs and external inputs)."""
        rs = row_shape(sd)
        tmpl = self.template(ops)
        cls = {}
        for o in ops:
            if tmpl == TL.ROWREDUCE and (o["op"] in REDUCE_OPS or
                                         (tuple(o["shape"]) == rs and rs != sd)):
                oc = "row"
            elif o["op"] in REDUCE_OPS and o.get("axis", -1) is None:
                oc = "none"
            else:
                oc = "tile"
            cls[o["out"]] = oc
            for x in o["in"]:
                if isinstance(x, str) and x in self.ext and x not in cls:
                    if o["op"] == "matmul":
                        cls[x] = "none"
                    elif oc == "row" and o["op"] not in REDUCE_OPS:
                        cls[x] = "row"
                    else:
                        cls[x] = "tile"
        return cls

    def demand(self, ops, sd):
        cls = self.value_class(ops, sd)
        first, last = {}, {}
        for i, o in enumerate(ops):
            for x in o["in"]:
                if isinstance(x, str):
                    first.setdefault(x, i)
                    last[x] = i
        start = {}
        for v in last:
            if v in self.ext:
                start[v] = first[v]
            else:
                d = next(i for i, o in enumerate(ops) if o["out"] == v)
                start[v] = d + 1
        peak = {"tile": 0, "row": 0}
        for i, o in enumerate(ops):
            for kind in ("tile", "row"):
                n = sum(1 for v in last if cls.get(v) == kind and start[v] <= i <= last[v])
                if cls.get(o["out"]) == kind:
                    n += 1
                peak[kind] = max(peak[kind], n)
        return peak

    def check_resources(self, ops):
        if len(ops) > MAX_OPS:
            return "resource"
        exts = set()
        for o in ops:
            for x in o["in"]:
                if isinstance(x, str) and x in self.ext:
                    exts.add(x)
        if len(exts) > MAX_EXT:
            return "resource"
        sd = self.dominant(ops)
        pk = self.demand(ops, sd)
        if pk["tile"] > MAX_TILE_VALUES or pk["row"] > MAX_ROW_VALUES:
            return "resource"
        tmpl = self.template(ops)
        if tmpl == TL.MATMUL:
            return None
        col = self.collapse(ops, sd)
        R, C, strides = col
        opnds = []
        names = self.ext_operands(ops)
        i = 0
        for x in names:
            e = self.ext[x]
            s_r, s_c = strides[i]
            opnds.append(TL.Operand(ESIZE[e["dtype"]], s_r, s_c, e["addr"] % 16))
            i += 1
        for o in ops:
            if o["op"] == "matmul" or o.get("addr") is None:
                continue
            if o["op"] in REDUCE_OPS and o.get("axis", -1) is None:
                continue
            s_r, s_c = strides[i]
            opnds.append(TL.Operand(ESIZE[o["dtype"]], s_r, s_c, o["addr"] % 16))
            i += 1
        # feasible on the standard VM or on its wide variant
        for nv_max in (TL.NV_MAX, TL.NV_WIDE):
            try:
                TL.plan(tmpl, R, C, opnds, nv_max)
                return None
            except ValueError:
                pass
        return "resource"
