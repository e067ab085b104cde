"""MI355X-native DVM hot path: streaming fuser, tile-level bytecode encoder and
resident VM kernels, behind the C ABI of include/dvm.h.

This package is a thin binding: argument marshalling only.  PyTorch supplies
device memory and streams.  Every computation runs in libdvm.so (host C++ for
fusion, tiling and encoding; HIP kernels on gfx950 for execution).
"""
from __future__ import annotations

import contextlib
import ctypes as C
from dataclasses import dataclass

from . import _lib as L
from ._lib import DvmError, check, lib

__all__ = ["Context", "Graph", "Program", "Value", "TensorDesc", "DvmError", "lib", "stack_programs", "Template"]


@dataclass
class TensorDesc:
    """A tensor described without torch: device address, dtype name, shape and
    element strides (used by encode-only callers and tests)."""
    addr: int
    dtype: str
    shape: tuple
    strides: tuple = None

    def __post_init__(self):
        self.shape = tuple(int(d) for d in self.shape)
        if self.strides is None:
            st, acc = [], 1
            for d in reversed(self.shape):
                st.append(acc)
                acc *= d
            self.strides = tuple(reversed(st))
        self.strides = tuple(int(s) for s in self.strides)


def _torch_dtype_code(t):
    import torch
    m = {torch.float32: L.F32, torch.bfloat16: L.BF16, torch.uint8: L.U8}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def to_c(t, dtype=None, shape=None) -> L.DvmTensor:
    """dvm_tensor from a torch tensor, a TensorDesc, or (None, dtype, shape)."""
    d = L.DvmTensor()
    if t is None:
        d.data = None
        d.dtype = L.DTYPE_CODES[dtype]
        shape = tuple(shape)
        d.ndim = len(shape)
        acc = 1
        for i in range(len(shape) - 1, -1, -1):
            d.shape[i] = shape[i]
            d.stride[i] = acc
            acc *= shape[i]
        return d
    if isinstance(t, TensorDesc):
        d.data = t.addr or None
        d.dtype = L.DTYPE_CODES[t.dtype]
        d.ndim = len(t.shape)
        for i, (n, s) in enumerate(zip(t.shape, t.strides)):
            d.shape[i] = n
            d.stride[i] = s
        return d
    d.data = t.data_ptr() or None
    d.dtype = _torch_dtype_code(t)
    d.ndim = t.dim()
    if d.ndim > 4:
        raise ValueError("at most 4 dims")
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


class Context:
    """device >= 0: launches on that HIP device; device < 0: encode-only."""

    def __init__(self, device: int = 0):
        h = C.c_void_p()
        check(lib.dvm_context_create(int(device), C.byref(h)))
        self.h = h
        self.device = device

    def close(self):
        if self.h:
            lib.dvm_context_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


@dataclass
class Value:
    h: int
    shape: tuple
    dtype: str
    storage: object = None  # keeps the storage tensor alive


class Program:
    def __init__(self, h, ctx):
        self.h = h
        self.ctx = ctx
        self._keep = []   # tensors the program reads or writes (kept alive with it)

    def header(self) -> dict:
        hd = L.DvmHeader()
        check(lib.dvm_program_header(self.h, C.byref(hd)))
        return {f: getattr(hd, f) for f, _ in L.DvmHeader._fields_}

    def words(self) -> list:
        n = C.c_size_t(0)
        check(lib.dvm_program_words(self.h, None, C.byref(n)))
        buf = (C.c_uint32 * n.value)()
        cap = C.c_size_t(n.value)
        check(lib.dvm_program_words(self.h, buf, C.byref(cap)))
        return list(buf)

    def verify(self):
        """The bytecode verifier: None if the program passes, else the first
        violation it finds."""
        buf = C.create_string_buffer(512)
        st = lib.dvm_program_verify(self.h, buf, 512)
        return None if st == L.OK else buf.value.decode()

    @staticmethod
    def from_words(words, ctx=None) -> "Program":
        arr = (C.c_uint32 * len(words))(*[int(w) & 0xFFFFFFFF for w in words])
        q = C.c_void_p()
        check(lib.dvm_program_from_words(arr, len(words), C.byref(q)))
        return Program(q, ctx)

    def launch(self, stream=None, ctx=None):
        """Launch on `ctx` (default: the context that encoded the program)."""
        check(lib.dvm_launch((ctx or self.ctx).h, self.h, _stream_handle(stream)))

    def launch_noalloc(self, stream=None, ctx=None):
        """dvm_launch_noalloc: no device allocation; a reduce-all uses the
        library's static scratch array (at most 65536 workgroup partials)."""
        check(lib.dvm_launch_noalloc((ctx or self.ctx).h, self.h, _stream_handle(stream)))

    PROF_COUNTERS = 5

    def launch_profiled(self, counters, stream=None):
        """Profiling launch (same results as launch) that fills `counters`, a
        device uint64 tensor of at least 5 * grid values, with each
        workgroup's total, decode, execute and tile-change cycles and its
        dispatch count."""
        check(lib.dvm_launch_profiled(self.ctx.h, self.h, _stream_handle(stream), C.c_void_p(counters.data_ptr()),
                                      counters.numel()))

    def launch_stress(self, seed, counters, stream=None):
        """Race-stress launch (profiling twin with seeded per-wave delays):
        the same stored results as launch, for a correctly synchronised
        program.  counters as for launch_profiled."""
        check(lib.dvm_launch_stress(self.ctx.h, self.h, _stream_handle(stream), int(seed) & 0xFFFFFF,
                                    C.c_void_p(counters.data_ptr()), counters.numel()))

    def debug_tilemap(self, tile_out, wg_out) -> "Program":
        q = C.c_void_p()
        a, b = to_c(tile_out), to_c(wg_out)
        check(lib.dvm_program_debug_tilemap(self.h, C.byref(a), C.byref(b), C.byref(q)))
        return Program(q, self.ctx)

    def __del__(self):
        try:
            if self.h:
                lib.dvm_program_free(self.h)
                self.h = None
        except Exception:
            pass


def stack_programs(programs, temporal: bool = False) -> "Program":
    """dvm_program_stack (dvm_program_stack_temporal if temporal): one launch
    of 2..7 independent VECTOR programs."""
    arr = (C.c_void_p * len(programs))(*[p.h.value if isinstance(p.h, C.c_void_p) else p.h for p in programs])
    q = C.c_void_p()
    fn = lib.dvm_program_stack_temporal if temporal else lib.dvm_program_stack
    check(fn(arr, len(programs), C.byref(q)))
    prog = Program(q, programs[0].ctx)
    for p in programs:
        prog._keep.extend(p._keep)
    return prog


def _stream_handle(stream):
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return C.c_void_p(torch.cuda.current_stream().cuda_stream)
        except Exception:
            pass
        return None
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


class Graph:
    """A streaming fusion buffer (DVM: capture ops in order, fuse while the
    conditions hold, flush at boundaries) bound to a stream."""

    def __init__(self, ctx: Context, stream=None):
        self.ctx = ctx
        h = C.c_void_p()
        self._stream = _stream_handle(stream) if ctx.device >= 0 else None
        check(lib.dvm_graph_create(ctx.h, self._stream, C.byref(h)))
        self.h = h
        self._in_group = False
        self.flushes = 0
        # Tensors the buffered ops borrow: held until the graph is launched (or
        # handed to a Program), so the caching allocator cannot reuse their
        # memory while the device still has to read or write it.
        self._keep = []

    def close(self):
        if self.h:
            lib.dvm_graph_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- values ----------------------------------------------------------
    def input(self, t) -> Value:
        self._keep.append(t)
        d = to_c(t)
        v = C.c_int64()
        check(lib.dvm_graph_input(self.h, C.byref(d), C.byref(v)))
        shape = tuple(d.shape[i] for i in range(d.ndim))
        return Value(v.value, shape, L.DTYPE_NAMES[d.dtype], t)

    def infer_shape(self, name, *ins, axis=-1):
        hs, n_in, attrs = self._inputs(name, ins, axis)
        out = L.DvmTensor()
        check(lib.dvm_graph_infer_shape(self.h, L.OP_CODES[name], hs, n_in, C.byref(attrs), C.byref(out)))
        return tuple(out.shape[i] for i in range(out.ndim))

    def _inputs(self, name, ins, axis):
        attrs = L.DvmAttrs(axis, -1, 0.0)
        vals = []
        for pos, x in enumerate(ins):
            if isinstance(x, Value):
                vals.append(x.h)
            else:
                if name not in L.BINARY or attrs.scalar_pos != -1:
                    raise TypeError(f"{name}: scalar operand not allowed here")
                attrs.scalar_pos = pos
                attrs.scalar = float(x)
        hs = (C.c_int64 * max(len(vals), 1))(*vals)
        return hs, len(vals), attrs

    def op(self, name, *ins, out=None, dtype=None, live=False, axis=-1) -> Value:
        """Append a primitive op.  ins: Values or one python float (binary ops).
        out: storage (torch tensor / TensorDesc) or None (no storage; the value
        must be released before its graph is flushed)."""
        hs, n_in, attrs = self._inputs(name, ins, axis)
        if out is None:
            shape = self.infer_shape(name, *ins, axis=axis)
            if dtype is None:
                dtype = "u8" if name == "isfinite" else next(x.dtype for x in ins if isinstance(x, Value))
            d = to_c(None, dtype, shape)
        else:
            self._keep.append(out)
            d = to_c(out)
            shape = tuple(d.shape[i] for i in range(d.ndim))
            dtype = L.DTYPE_NAMES[d.dtype]
        v = C.c_int64()
        st = lib.dvm_graph_add_op(self.h, L.OP_CODES[name], hs, n_in, C.byref(attrs), C.byref(d),
                                  L.OUT_LIVE if live else 0, C.byref(v))
        check(st)
        return Value(v.value, shape, dtype, out)

    def release(self, *vals):
        for v in vals:
            check(lib.dvm_graph_release(self.h, v.h))

    @contextlib.contextmanager
    def group(self):
        check(lib.dvm_graph_begin_group(self.h))
        self._in_group = True
        try:
            yield self
        finally:
            self._in_group = False
            fl = C.c_int32(0)
            check(lib.dvm_graph_end_group(self.h, C.byref(fl)))
            self.flushes += fl.value

    # -- flushing --------------------------------------------------------
    def flush(self):
        """Encode the buffered graph (no launch); returns a Program or None."""
        q = C.c_void_p()
        check(lib.dvm_flush(self.h, C.byref(q)))
        keep, self._keep = self._keep, []
        if not q.value:
            return None
        prog = Program(q, self.ctx)
        prog._keep = keep
        return prog

    def set_stacking(self, max_segments: int, temporal: bool = False):
        """Pack up to max_segments independent encoded graphs into one launch
        (1: launch every graph when it is flushed); temporal: the launch runs
        the segments in sequence on every workgroup (dvm_graph_set_stack_order)."""
        check(lib.dvm_graph_set_stacking(self.h, int(max_segments)))
        check(lib.dvm_graph_set_stack_order(self.h, 1 if temporal else 0))

    # -- device-side control flow -----------------------------------------
    def begin_branch(self, cond: "Value", threshold: float = 0.0):
        """Ops until else_branch() form the then-body, run iff cond > threshold
        (cond: one fp32 value, read on the device)."""
        check(lib.dvm_graph_begin_branch(self.h, cond.h, float(threshold)))

    def begin_branch_reduce(self, x: "Value", out, threshold: float = 0.0, kind: str = "sum") -> "Value":
        """A reduce-all of x ("sum" or "max") into the 0-d fp32 storage out,
        then begin_branch on it (dvm_graph_begin_branch_reduce: the branch
        program folds the reduce-all's partials itself).  Returns the value."""
        self._keep.append(out)
        d = to_c(out)
        v = C.c_int64()
        check(lib.dvm_graph_begin_branch_reduce(self.h, x.h, L.OP_CODES["reduce_" + kind], C.byref(d),
                                                float(threshold), C.byref(v)))
        return Value(v.value, (), "f32", out)

    def else_branch(self):
        check(lib.dvm_graph_else_branch(self.h))

    def end_branch(self) -> bool:
        """Encodes both bodies into one branch program and launches it."""
        fl = C.c_int32(0)
        check(lib.dvm_graph_end_branch(self.h, C.byref(fl)))
        return bool(fl.value)

    def take_program(self):
        """The oldest program an encode-only context flushed implicitly (at a
        fusion boundary or a reduce-all), or None."""
        q = C.c_void_p()
        check(lib.dvm_graph_take_program(self.h, C.byref(q)))
        if not q.value:
            return None
        prog = Program(q, self.ctx)
        prog._keep = list(self._keep)   # the tensors it reads or writes stay alive with it
        return prog

    def flush_launch(self) -> bool:
        fl = C.c_int32(0)
        check(lib.dvm_graph_flush_launch(self.h, C.byref(fl)))
        # launched on the graph's stream: later reuse of the memory is ordered after it
        self._keep = []
        return bool(fl.value)

    def sync(self):
        check(lib.dvm_sync(self.h))
        self._keep = []

    def flush_log(self, detail=False) -> list:
        """[(n_ops, reason name)] for every graph flushed so far; with
        detail=True [(n_ops, reason, encode_us, bytes)]."""
        n = C.c_size_t(0)
        check(lib.dvm_graph_flush_log(self.h, None, None, None, None, C.byref(n)))
        k = n.value
        ops = (C.c_int32 * max(k, 1))()
        rs = (C.c_int32 * max(k, 1))()
        us = (C.c_float * max(k, 1))()
        by = (C.c_uint64 * max(k, 1))()
        cap = C.c_size_t(k)
        check(lib.dvm_graph_flush_log(self.h, ops, rs, us, by, C.byref(cap)))
        if detail:
            return [(ops[i], L.FLUSH_REASONS[rs[i]], float(us[i]), int(by[i])) for i in range(k)]
        return [(ops[i], L.FLUSH_REASONS[rs[i]]) for i in range(k)]

    def stats(self) -> dict:
        s = L.DvmStats()
        check(lib.dvm_graph_stats(self.h, C.byref(s)))
        return {
            "graphs": s.graphs, "launches": s.launches, "ops": s.ops, "groups": s.groups,
            "unsupported": s.unsupported,
            "flush_reason": {L.FLUSH_REASONS[i]: s.flush_reason[i] for i in range(8)},
            "encode_us_total": s.encode_us_total, "encode_us_max": s.encode_us_max, "bytes": s.bytes,
            "fuse_us_total": s.fuse_us_total, "launch_us_total": s.launch_us_total, "stacked": s.stacked,
        }


class _TemplateGraph(Graph):
    """The graph a template runs through (not owned: the template frees it)."""

    def __init__(self, ctx, h):
        self.ctx = ctx
        self.h = h
        self._in_group = False
        self.flushes = 0
        self._keep = []

    def close(self):
        self.h = None


class Output:
    """An output slot of a template op (out= in Template.op): its dtype; the
    shape follows from the op."""

    def __init__(self, dtype):
        self.dtype = dtype


class Template:
    """Static-graph symbolic fusion: ops recorded once over symbolic dims
    (strings) and concrete dims (ints); finalize() decides the fusion
    partition once; run() binds tensors and only tiles, encodes and launches.
    The interface of Graph for building (input / op / group / release), so the
    composites build templates too."""

    def __init__(self, ctx: Context, stream=None):
        self.ctx = ctx
        h = C.c_void_p()
        check(lib.dvm_template_create(ctx.h, _stream_handle(stream) if ctx.device >= 0 else None, C.byref(h)))
        self.h = h
        gh = C.c_void_p()
        check(lib.dvm_template_graph(h, C.byref(gh)))
        self.graph = _TemplateGraph(ctx, gh)
        self.symbols = {}
        self.n_inputs = 0
        self.n_outputs = 0

    def close(self):
        if self.h:
            lib.dvm_template_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _dims(self, dims):
        out = []
        for d in dims:
            if isinstance(d, str):
                k = self.symbols.setdefault(d, len(self.symbols))
                out.append(-(k + 1))
            else:
                out.append(int(d))
        return out

    def input(self, dtype, dims=None) -> Value:
        """A template input: input(dtype, dims), dims holding ints and symbol
        names."""
        dv = self._dims(dims or ())
        arr = (C.c_int64 * max(len(dv), 1))(*dv)
        v = C.c_int64()
        check(lib.dvm_template_input(self.h, L.DTYPE_CODES[dtype], len(dv), arr, C.byref(v)))
        self.n_inputs += 1
        return Value(v.value, tuple(dims or ()), dtype)

    def output(self, dtype) -> Output:
        return Output(dtype)

    def op(self, name, *ins, out=None, dtype=None, live=False, axis=-1) -> Value:
        attrs = L.DvmAttrs(axis, -1, 0.0)
        vals = []
        for pos, x in enumerate(ins):
            if isinstance(x, Value):
                vals.append(x.h)
            else:
                attrs.scalar_pos = pos
                attrs.scalar = float(x)
        hs = (C.c_int64 * max(len(vals), 1))(*vals)
        if isinstance(out, Output):
            dtype = out.dtype
            live = True
        if dtype is None:
            dtype = "u8" if name == "isfinite" else next(x.dtype for x in ins if isinstance(x, Value))
        v = C.c_int64()
        check(lib.dvm_template_add_op(self.h, L.OP_CODES[name], hs, len(vals), C.byref(attrs), L.DTYPE_CODES[dtype],
                                      L.OUT_LIVE if live else 0, C.byref(v)))
        if live:
            self.n_outputs += 1
        first = next(x for x in ins if isinstance(x, Value))
        shape = first.shape
        if name in ("reduce_sum", "reduce_max"):
            shape = () if axis == L.AXIS_ALL else tuple(shape[:-1]) + (1,)
        return Value(v.value, shape, dtype)

    def release(self, *vals):
        pass    # internal values are the template's to manage

    @contextlib.contextmanager
    def group(self):
        check(lib.dvm_template_begin_group(self.h))
        try:
            yield self
        finally:
            check(lib.dvm_template_end_group(self.h))

    def finalize(self) -> int:
        n = C.c_int32(0)
        check(lib.dvm_template_finalize(self.h, C.byref(n)))
        return n.value

    def partition(self):
        """(graph index of every op, host microseconds finalize took)."""
        n = C.c_size_t(0)
        check(lib.dvm_template_partition(self.h, None, C.byref(n), None))
        arr = (C.c_int32 * max(n.value, 1))()
        cap = C.c_size_t(n.value)
        us = C.c_double(0)
        check(lib.dvm_template_partition(self.h, arr, C.byref(cap), C.byref(us)))
        return [arr[i] for i in range(n.value)], us.value

    def run(self, inputs, outputs) -> bool:
        ia = (L.DvmTensor * max(len(inputs), 1))(*[to_c(x) for x in inputs])
        oa = (L.DvmTensor * max(len(outputs), 1))(*[to_c(x) for x in outputs])
        fl = C.c_int32(0)
        check(lib.dvm_template_run(self.h, ia, len(inputs), oa, len(outputs), C.byref(fl)))
        self.graph._keep.extend(list(inputs) + list(outputs))
        return bool(fl.value)
