"""The tiling and fusion constants as each side states them.

The oracle and the encoder share no code, no tables and no constant
generators: each states the constants of the tiling and fusion rules in its
own source.  This host test reads the encoder's and kernels' statements from
their C++ text and checks that they equal the oracle's, so a constant cannot
change on one side only.  Each constant's provenance (a passage of the pages
or a measurement on MI355X) is listed in the design notes.
"""
import os
import re

from oracle import fusion as FU
from oracle import tiling as TL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "device_bytecode_vm_amd", "csrc")


def cxx(*names):
    return "\n".join(open(os.path.join(CSRC, n)).read() for n in names)


def const(src, name):
    """Value of `constexpr <type> name = <int>;` (also `name = a * b`) in src."""
    m = re.search(r"\b" + name + r"\s*=\s*([0-9 *A-Z_]+)[,;]", src)
    assert m, name
    expr = m.group(1)
    for tok in re.findall(r"[A-Z_]+", expr):
        expr = expr.replace(tok, str(const(src, tok)))
    return eval(expr)


def test_tiling_constants_agree():
    src = cxx("bytecode.h", "dvm_host.cpp")
    assert const(src, "T_LANES") == TL.T_LANES
    assert const(src, "VEC") == TL.VEC
    assert const(src, "NV_MAX") == TL.NV_MAX
    assert const(src, "NV_WIDE") == TL.NV_WIDE
    ns = src[src.index("namespace tiling {"):]
    assert const(ns, "G") == TL.G_WG
    assert const(ns, "A") == TL.A_TICKS
    assert const(ns, "A_MM") == TL.A_MM_TICKS
    assert const(ns, "BT") == TL.BYTE_TICKS
    assert const(ns, "WIDE_WG_TILES") == TL.WIDE_WG_TILES
    assert const(ns, "WIDE_GRID_MAX") == TL.WIDE_GRID_MAX
    assert eval(re.search(r"\bW = ([0-9 *A-Z_]+),", ns).group(1).replace("VEC", str(TL.VEC))) == TL.W_ALIGN
    menu = re.search(r"MM_TILES\[\] = \{(.*?)\};", ns).group(1)
    tiles = [tuple(int(x) for x in t.split(",")) for t in re.findall(r"\{([0-9, ]+)\}", menu)]
    assert tiles == TL.MM_TILES


def test_fusion_constants_agree():
    src = cxx("dvm_host.cpp")
    assert const(src, "MAX_OPS") == FU.MAX_OPS
    assert const(src, "MAX_EXT") == FU.MAX_EXT
    assert const(src, "MAX_TILE_VALUES") == FU.MAX_TILE_VALUES
    assert const(src, "MAX_ROW_VALUES") == FU.MAX_ROW_VALUES


def test_mix_order_constants_agree():
    src = cxx("vm_mix.hip")
    assert const(src, "GM") == TL.MM_GROUP
    # the XCD count appears in the slot rule as "& 7" / ">> 3" (8 = 2^3)
    body = src[src.index("xcd_slot(uint32_t b, uint32_t G)"):]
    body = body[:body.index("}")]
    assert "& ~7u" in body and "(b & 7u)" in body and ">> 3" in body and TL.N_XCD == 8
