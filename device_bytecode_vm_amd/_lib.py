"""ctypes binding of include/dvm.h (argument marshalling only).

Every step of the hot path -- fusion decisions, tiling, bytecode encoding and
the VM kernels -- runs inside libdvm.so.  This module only converts Python
objects (torch tensors, plain descriptors) into the C structs and checks the
returned status.  If the library is missing, importing fails: there is no
fallback.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdvm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(or python device_bytecode_vm_amd/build.py)")

# libdvm.so shares streams and device allocations with PyTorch, so it must
# bind to the HIP runtime PyTorch loads.  torch's libamdhip64 carries the same
# soname (libamdhip64.so.7) as the system one libdvm.so names, so loading torch
# first makes the dynamic linker reuse it; loading libdvm.so first would bring
# in a second, separate runtime.
import torch  # noqa: E402,F401  (load order only)

lib = C.CDLL(LIB_PATH)

# dvm_status
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_SHAPE, ERR_RESOURCE, ERR_DEVICE, ERR_INTERNAL = range(7)
STATUS_NAMES = ["OK", "INVALID_ARG", "UNSUPPORTED", "SHAPE", "RESOURCE", "DEVICE", "INTERNAL"]

F32, BF16, U8 = 0, 1, 2
DTYPE_CODES = {"f32": F32, "bf16": BF16, "u8": U8}
DTYPE_NAMES = {v: k for k, v in DTYPE_CODES.items()}
ESIZE = {F32: 4, BF16: 2, U8: 1}

OPS = ["add", "sub", "mul", "div", "max", "min", "pow", "sqrt", "abs", "log", "exp", "round", "floor",
       "isfinite", "neg", "recip", "cast", "copy", "reduce_sum", "reduce_max", "matmul"]
OP_CODES = {n: i for i, n in enumerate(OPS)}
BINARY = set(OPS[:7])
AXIS_ALL = 0x7FFFFFFF
OUT_LIVE = 1

FLUSH_REASONS = ["explicit", "sync", "reduce_all", "shape", "pattern", "dependence", "resource", "branch"]


class DvmTensor(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int32), ("ndim", C.c_int32),
                ("shape", C.c_int64 * 4), ("stride", C.c_int64 * 4)]


class DvmAttrs(C.Structure):
    _fields_ = [("axis", C.c_int32), ("scalar_pos", C.c_int32), ("scalar", C.c_float)]


class DvmHeader(C.Structure):
    _fields_ = [("kernel_type", C.c_uint32), ("tmpl", C.c_uint32), ("block_dim", C.c_uint32),
                ("body_tile", C.c_uint32), ("grid", C.c_uint32), ("tr", C.c_uint32), ("tc", C.c_uint32),
                ("g", C.c_uint32), ("nv", C.c_uint32), ("p", C.c_uint32), ("R", C.c_int64), ("C", C.c_int64),
                ("n_instr", C.c_uint32), ("n_args", C.c_uint32), ("pad", C.c_uint32), ("n_words", C.c_uint32),
                ("bytes", C.c_uint64), ("segments", C.c_uint32)]


class DvmStats(C.Structure):
    _fields_ = [("graphs", C.c_uint64), ("launches", C.c_uint64), ("ops", C.c_uint64), ("groups", C.c_uint64),
                ("unsupported", C.c_uint64), ("flush_reason", C.c_uint64 * 8),
                ("encode_us_total", C.c_double), ("encode_us_max", C.c_double), ("bytes", C.c_uint64),
                ("fuse_us_total", C.c_double), ("launch_us_total", C.c_double), ("stacked", C.c_uint64)]


VP = C.c_void_p
P = C.POINTER
_sigs = {
    "dvm_context_create": (C.c_int, [C.c_int, P(VP)]),
    "dvm_context_destroy": (None, [VP]),
    "dvm_graph_create": (C.c_int, [VP, VP, P(VP)]),
    "dvm_graph_destroy": (None, [VP]),
    "dvm_graph_take_program": (C.c_int, [VP, P(VP)]),
    "dvm_graph_input": (C.c_int, [VP, P(DvmTensor), P(C.c_int64)]),
    "dvm_graph_begin_group": (C.c_int, [VP]),
    "dvm_graph_end_group": (C.c_int, [VP, P(C.c_int32)]),
    "dvm_graph_add_op": (C.c_int, [VP, C.c_int32, P(C.c_int64), C.c_int32, P(DvmAttrs), P(DvmTensor),
                                   C.c_uint32, P(C.c_int64)]),
    "dvm_graph_release": (C.c_int, [VP, C.c_int64]),
    "dvm_graph_infer_shape": (C.c_int, [VP, C.c_int32, P(C.c_int64), C.c_int32, P(DvmAttrs), P(DvmTensor)]),
    "dvm_flush": (C.c_int, [VP, P(VP)]),
    "dvm_launch": (C.c_int, [VP, VP, VP]),
    "dvm_launch_noalloc": (C.c_int, [VP, VP, VP]),
    "dvm_launch_profiled": (C.c_int, [VP, VP, VP, VP, C.c_size_t]),
    "dvm_launch_stress": (C.c_int, [VP, VP, VP, C.c_uint32, VP, C.c_size_t]),
    "dvm_graph_flush_launch": (C.c_int, [VP, P(C.c_int32)]),
    "dvm_graph_set_stacking": (C.c_int, [VP, C.c_int32]),
    "dvm_program_stack": (C.c_int, [P(VP), C.c_size_t, P(VP)]),
    "dvm_graph_set_stack_order": (C.c_int, [VP, C.c_int32]),
    "dvm_program_stack_temporal": (C.c_int, [P(VP), C.c_size_t, P(VP)]),
    "dvm_graph_begin_branch": (C.c_int, [VP, C.c_int64, C.c_float]),
    "dvm_graph_begin_branch_reduce": (C.c_int, [VP, C.c_int64, C.c_int32, P(DvmTensor), C.c_float, P(C.c_int64)]),
    "dvm_graph_else_branch": (C.c_int, [VP]),
    "dvm_graph_end_branch": (C.c_int, [VP, P(C.c_int32)]),
    "dvm_sync": (C.c_int, [VP]),
    "dvm_program_header": (C.c_int, [VP, P(DvmHeader)]),
    "dvm_program_words": (C.c_int, [VP, P(C.c_uint32), P(C.c_size_t)]),
    "dvm_program_free": (None, [VP]),
    "dvm_program_verify": (C.c_int, [VP, C.c_char_p, C.c_size_t]),
    "dvm_program_from_words": (C.c_int, [P(C.c_uint32), C.c_size_t, P(VP)]),
    "dvm_program_debug_tilemap": (C.c_int, [VP, P(DvmTensor), P(DvmTensor), P(VP)]),
    "dvm_graph_stats": (C.c_int, [VP, P(DvmStats)]),
    "dvm_graph_flush_log": (C.c_int, [VP, P(C.c_int32), P(C.c_int32), P(C.c_float), P(C.c_uint64),
                                      P(C.c_size_t)]),
    "dvm_template_create": (C.c_int, [VP, VP, P(VP)]),
    "dvm_template_destroy": (None, [VP]),
    "dvm_template_graph": (C.c_int, [VP, P(VP)]),
    "dvm_template_input": (C.c_int, [VP, C.c_int32, C.c_int32, P(C.c_int64), P(C.c_int64)]),
    "dvm_template_begin_group": (C.c_int, [VP]),
    "dvm_template_end_group": (C.c_int, [VP]),
    "dvm_template_add_op": (C.c_int, [VP, C.c_int32, P(C.c_int64), C.c_int32, P(DvmAttrs), C.c_int32, C.c_uint32,
                                      P(C.c_int64)]),
    "dvm_template_finalize": (C.c_int, [VP, P(C.c_int32)]),
    "dvm_template_partition": (C.c_int, [VP, P(C.c_int32), P(C.c_size_t), P(C.c_double)]),
    "dvm_template_run": (C.c_int, [VP, P(DvmTensor), C.c_int32, P(DvmTensor), C.c_int32, P(C.c_int32)]),
    "dvm_last_error": (C.c_char_p, []),
}
for _name, (_res, _args) in _sigs.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_sigs)


class DvmError(RuntimeError):
    def __init__(self, status, msg):
        self.status = status
        super().__init__(f"{STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else status}: {msg}")


def check(status):
    if status != OK:
        raise DvmError(status, lib.dvm_last_error().decode())
    return status
