// Static checks of an encoded program (host side): the bytecode verifier.
//
// The encoder inserts the syncs and the staging of a program (the DVM review
// page, section 4.3: the code body carries the synchronisation the encoder
// adds); the VM trusts them.  This pass re-derives, from the words alone, the
// conditions the VM relies on and reports the first one a program breaks:
//  * layout: magic, version, kernel type, word ranges in order and in bounds,
//    instruction pairs at even words;
//  * geometry: the tile fits the VM build (lanes per row, chunks per lane),
//    and block_dim, column tiles, body_tile and grid follow from R, C and the
//    tile as the tiling rules make them;
//  * operands: every operand index names a table entry of a known dtype, and
//    vector access (AF_VEC) only on unit-stride, aligned operands;
//  * registers: every tile or row register an instruction reads was written
//    earlier in the same tile's body (the VM's registers carry the previous
//    tile's values otherwise), and the wide build names only the
//    accumulator;
//  * staging: prefetch slots read in the body were filled by the prologue
//    with the same operand, are read before the body refills them and are
//    refilled exactly once per tile; invariant slots read were loaded;
//  * cross-wave reduction buffers: over consecutive tiles, no buffer is
//    written while a read of it is not yet fenced by a barrier.
// Branch programs check both bodies; stacked programs their directory and
// every segment.
#include <algorithm>
#include <cstdio>
#include <string>
#include <vector>

#include "bytecode.h"

namespace dvmbc {
namespace {

struct Effect {
  unsigned t_rd = 0, t_wr = 0;  // tile register masks
  unsigned r_rd = 0, r_wr = 0;  // row register masks
  int arg_rd = -1, arg_wr = -1; // operands read / written through word 1
  int pf = -1;                  // prefetch slot read
  bool pf_issue = false;        // ... then refilled with the next tile
  int inv[2] = {-1, -1};        // invariant slots read
  unsigned buf_wr = 0, buf_rd = 0;  // cross-wave reduction buffers written / read (masks)
  bool barrier_mid = false;     // a barrier between the buffer write and read (REDX)
  bool barrier = false;         // a workgroup barrier (SYNC)
  bool prologue_only = false;
  bool valid = true;
};

Effect effect(uint32_t w0, uint32_t w1) {
  Effect e;
  const uint32_t h = f_op(w0), d = f_dst(w0), a = f_a(w0), b = f_b(w0), bk = f_bk(w0), fl = f_flags(w0);
  auto mem_src = [&](uint32_t flags) {
    e.arg_rd = (int)w1;
    if (flags & FL_INV) e.inv[0] = (int)(b & 1u);
    else if (flags & FL_PF) {
      e.pf = (int)(b & 1u);
      e.pf_issue = (flags & FL_ISSUE) != 0;
    }
  };
  if (h == HD_END) {
  } else if (h >= HD_LD_DIR && h < HD_LD_DIR + 3) {
    e.t_wr = 1u << (h - HD_LD_DIR);
    e.arg_rd = (int)w1;
  } else if (h >= HD_LD_PF16 && h < HD_LD_PF16 + 6) {
    e.t_wr = 1u << ((h - HD_LD_PF16) % 3);
    e.arg_rd = (int)w1;
    e.pf = (int)(b & 1u);
    e.pf_issue = (fl & FL_ISSUE) != 0;
  } else if (h >= HD_LD_INV && h < HD_LD_INV + 3) {
    e.t_wr = 1u << (h - HD_LD_INV);
    e.inv[0] = (int)(b & 1u);
  } else if (h >= HD_ST_DIR && h < HD_ST_DIR + 3) {
    e.t_rd = 1u << (h - HD_ST_DIR);
    e.arg_wr = (int)w1;
  } else if (h == HD_ST_BF16 || h == HD_ST_F32) {
    e.t_rd = 1u;
    e.arg_wr = (int)w1;
  } else if (h >= HD_COPY && h < HD_COPY + 9) {
    const uint32_t dd = (h - HD_COPY) / 3, aa = (h - HD_COPY) % 3;
    if (dd == aa) e.valid = false;
    e.t_rd = 1u << aa;
    e.t_wr = 1u << dd;
  } else if ((h >= HD_UN && h < HD_UN + 11) || h == HD_SILU) {
    e.t_rd = e.t_wr = 1u;
  } else if (h == HD_SOFTMAX) {
    // rows across waves (the caller drops these for rows inside a wave): the
    // buffer pair b, b + 1 written, a barrier, both read
    e.t_rd = e.t_wr = 1u;
    if (b + 1 >= (uint32_t)N_LDSBUF) e.valid = false;
    e.buf_wr = e.buf_rd = 3u << b;
    e.barrier_mid = true;
  } else if (h >= HD_BIN && h < HD_BIN + 70) {
    const uint32_t form = ((h - HD_BIN) % 10) % 5;
    e.t_wr = 1u;
    e.t_rd = 1u;
    if (form <= BF_T2) e.t_rd |= 1u << form;
    else if (form == BF_SCALAR && bk == BK_RREG) e.r_rd = 1u << b;
    else if (form != BF_SCALAR) e.valid = false;
  } else if (h >= HD_RED && h < HD_RED + 9) {
    e.t_rd = 1u << ((h - HD_RED) % 3);
    e.r_wr = 1u << d;
  } else if (h >= HD_REDX && h < HD_REDX + 9) {
    e.t_rd = 1u << ((h - HD_REDX) % 3);
    e.r_wr = 1u << d;
    e.buf_wr = e.buf_rd = 1u << b;
    e.barrier_mid = true;
  } else if (h >= HD_ALL && h < HD_ALL + 6) {
    // the lane's running partial: no LDS buffer, no barrier
    e.t_rd = 1u << ((h - HD_ALL) % 3);
  } else if (h >= HD_BCAST && h < HD_BCAST + 3) {
    e.r_rd = 1u << a;
    e.t_wr = 1u << (h - HD_BCAST);
  } else if (h == HD_RBIN) {
    e.r_rd = 1u << a;
    if (bk == BK_RREG) e.r_rd |= 1u << b;
    e.r_wr = 1u << d;
  } else if (h == HD_RUN) {
    e.r_rd = 1u << a;
    e.r_wr = 1u << d;
  } else if (h == HD_SYNC) {
    e.barrier = true;
  } else if (h == HD_LD_ROW) {
    e.r_wr = 1u << d;
    e.arg_rd = (int)w1;
  } else if (h == HD_ST_ROW) {
    e.r_rd = 1u << a;
    e.arg_wr = (int)w1;
  } else if (h == HD_DBG) {
    e.t_wr = 1u << d;
  } else if (h == HD_LDS_INV || h == HD_PF) {
    e.prologue_only = true;
    e.arg_rd = (int)w1;
  } else if (h == HD_BIN_POW) {
    e.t_rd = e.t_wr = 1u;
    if (bk == BK_TREG) e.t_rd |= 1u << b;
    else if (bk == BK_RREG) e.r_rd = 1u << b;
  } else if (h == HD_BIN_MEM) {
    e.t_rd = e.t_wr = 1u;
    mem_src(fl);
  } else if (h == HD_DIV_T) {
    e.t_rd = 1u | (1u << b);
    e.t_wr = 1u;
  } else if (h == HD_FMA_INV) {
    e.t_rd = e.t_wr = 1u;
    e.inv[0] = (int)(b & 1u);
    e.inv[1] = (int)(a & 1u);
    if (bk == BK_RREG) e.r_rd = 1u << d;
  } else {
    e.valid = false;
  }
  return e;
}

struct Ctx {
  const uint32_t* W;
  uint32_t n_args;
  std::string* err;
  bool fail(const char* fmt, uint32_t a = 0, uint32_t b = 0) {
    char buf[256];
    snprintf(buf, sizeof buf, fmt, a, b);
    *err = buf;
    return false;
  }
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool check_arg_index(Ctx& c, int arg, uint32_t pc) {
  if (arg < 0) return true;
  if ((uint32_t)arg >= c.n_args) return c.fail("word %u: operand %u outside the table", pc, (uint32_t)arg);
  return true;
}

bool verify_vector(Ctx& c) {
  const uint32_t* W = c.W;
  const uint32_t kt = W[H_KTYPE];
  const int nvk = kt == KT_VECTOR_WIDE ? NV_WIDE : NV_MAX;
  const unsigned treg_ok = kt == KT_VECTOR_WIDE ? 1u : (1u << N_TREG) - 1u;
  // geometry
  const int64_t R = ((int64_t)W[H_R_HI] << 32) | W[H_R_LO], C = ((int64_t)W[H_C_HI] << 32) | W[H_C_LO];
  const uint32_t tr = W[H_TR], tc = W[H_TC], g = W[H_G], nv = W[H_NV], P = W[H_P];
  const uint32_t block_dim = W[H_BLOCK_DIM], body_tile = W[H_BODY_TILE], grid = W[H_GRID];
  if (R > 0 && C > 0) {
    if (g == 0 || (g & (g - 1)) || g > (uint32_t)T_LANES || P * g != (uint32_t)T_LANES)
      return c.fail("lanes per row %u and row groups %u do not split a workgroup", g, P);
    if (tr == 0 || tr > P) return c.fail("tile rows %u exceed the row groups %u", tr, P);
    if (nv == 0 || nv > (uint32_t)nvk) return c.fail("chunks per lane %u outside the build's %u", nv, (uint32_t)nvk);
    if (tc == 0 || (int64_t)tc > (int64_t)g * VEC * nv) return c.fail("tile columns %u exceed a row's lanes (%u chunks)", tc, nv);
    const int64_t n_r = cdiv(R, tr), n_c = cdiv(C, tc);
    if ((int64_t)block_dim != n_r * n_c || (int64_t)W[H_NC] != n_c) return c.fail("block_dim %u is not the tile count", block_dim);
    // 512 resident workgroups; a wide-build program with more than 8 tiles
    // per workgroup runs as min(8192, block_dim / 8) workgroups instead
    int64_t gp = std::min<int64_t>(512, block_dim);
    if (W[H_KTYPE] == KT_VECTOR_WIDE && cdiv(block_dim, gp) > 8) gp = std::min<int64_t>(8192, block_dim / 8);
    if ((int64_t)body_tile != cdiv(block_dim, gp) || (int64_t)grid != cdiv(block_dim, body_tile))
      return c.fail("body_tile %u / grid %u do not follow from block_dim", body_tile, grid);
  } else if (block_dim != 0) {
    return c.fail("an empty iteration space with %u tiles", block_dim);
  }
  // LDS staging areas
  const uint32_t budget = LDS_BUDGET;
  if (W[H_LDS_BYTES] > budget) return c.fail("dynamic LDS %u exceeds %u", W[H_LDS_BYTES], budget);
  // prologue
  int pf_arg[2] = {-1, -1}, inv_arg[2] = {-1, -1};
  // staging areas [begin, end) in the dynamic LDS, checked disjoint below
  std::vector<std::pair<uint32_t, uint32_t>> areas;
  for (uint32_t pc = W[H_PRO_BEGIN]; pc < W[H_PRO_END]; pc += 2) {
    const uint32_t w0 = W[pc], w1 = W[pc + 1];
    const uint32_t h = f_op(w0);
    if (h == HD_PF) {
      const int s = (int)(f_b(w0) & 1u);
      if (pf_arg[s] >= 0) return c.fail("word %u: prefetch slot %u filled twice", pc, (uint32_t)s);
      pf_arg[s] = (int)w1;
      if (w1 >= c.n_args) return c.fail("word %u: operand %u outside the table", pc, w1);
      if (f_a(w0) != 0) return c.fail("word %u: a prefetch of a tile other than the workgroup's first", pc);
      // the tile's nv chunks x 256 lanes x 16 bytes per 16-bit half of the element
      const uint32_t halves = W[ARG_BASE + w1 * ARG_WORDS + A_DTYPE] == DT_F32 ? 2u : 1u;
      const uint32_t sz = W[H_NV] * T_LANES * 16u * halves;
      if (W[H_PF_OFF0 + s] + sz > W[H_LDS_BYTES])
        return c.fail("prefetch slot %u outside the dynamic LDS (%u bytes)", (uint32_t)s, W[H_LDS_BYTES]);
      areas.push_back({W[H_PF_OFF0 + s], W[H_PF_OFF0 + s] + sz});
    } else if (h == HD_LDS_INV) {
      const int s = (int)(f_dst(w0) & 1u);
      inv_arg[s] = (int)w1;
      // nvk chunks x (one row's lanes, or all 256) x 32 bytes
      const uint32_t lanes = W[H_INV_SHARED0 + s] ? g : (uint32_t)T_LANES;
      if (W[H_INV_OFF0 + s] + (uint32_t)nvk * lanes * 32u > W[H_LDS_BYTES])
        return c.fail("invariant slot %u outside the dynamic LDS (%u bytes)", (uint32_t)s, W[H_LDS_BYTES]);
      areas.push_back({W[H_INV_OFF0 + s], W[H_INV_OFF0 + s] + (uint32_t)nvk * lanes * 32u});
    } else {
      return c.fail("word %u: handler %u in the prologue", pc, h);
    }
    if (!check_arg_index(c, (int)w1, pc)) return false;
  }
  // the cross-wave reduction buffers (rows across waves, a fused softmax
  // across waves, the reduce-all epilogue) need their area too
  {
    bool red = W[H_TEMPLATE] == TM_ALLREDUCE;
    auto scan = [&](uint32_t b0, uint32_t b1) {
      for (uint32_t pc = b0; pc + 1 < b1; pc += 2) {
        const uint32_t h = f_op(W[pc]);
        red = red || (h >= HD_REDX && h < HD_REDX + 9) || (h == HD_SOFTMAX && g > 64);
      }
    };
    scan(W[H_BODY_BEGIN], W[H_BODY_END]);
    if (W[H_FLAGS] & HF_BRANCH) scan(W[H_ALT_BEGIN], W[H_ALT_END]);
    if (red) {
      if (W[H_RED_OFF] + RED_LDS_BYTES > W[H_LDS_BYTES])
        return c.fail("reduction buffers outside the dynamic LDS (%u bytes)", W[H_LDS_BYTES]);
      areas.push_back({W[H_RED_OFF], W[H_RED_OFF] + RED_LDS_BYTES});
    }
    std::sort(areas.begin(), areas.end());
    for (size_t k = 1; k < areas.size(); ++k)
      if (areas[k].first < areas[k - 1].second)
        return c.fail("LDS staging areas overlap at byte %u", areas[k].first);
  }
  // the bodies: registers, staging and operands per tile; reduction buffers
  // over three consecutive tiles
  // under HF_RED_ALT the workgroup's tiles alternate reduction buffers b and
  // b ^ 2 (tile parity)
  const bool red_alt = (W[H_FLAGS] & HF_RED_ALT) != 0;
  auto swap2 = [](unsigned m) { return ((m & 0x33u) << 2) | ((m & 0xCCu) >> 2); };
  auto body = [&](uint32_t b0, uint32_t b1) -> bool {
    unsigned reads_since_barrier = 0;
    for (int tile = 0; tile < 3; ++tile) {
      unsigned t_def = 0, r_def = 0;
      bool pf_done[2] = {false, false};
      for (uint32_t pc = b0; pc < b1; pc += 2) {
        const uint32_t w0 = W[pc], w1 = W[pc + 1];
        Effect e = effect(w0, w1);
        if (!e.valid) return c.fail("word %u: unknown handler %u", pc, f_op(w0));
        if (f_op(w0) == HD_SOFTMAX && g <= 64) {  // rows inside a wave: no exchange
          e.buf_wr = e.buf_rd = 0;
          e.barrier_mid = false;
        }
        if (red_alt && (tile & 1)) {
          e.buf_wr = swap2(e.buf_wr);
          e.buf_rd = swap2(e.buf_rd);
        }
        if (e.prologue_only) return c.fail("word %u: prologue handler %u in the body", pc, f_op(w0));
        if ((e.t_rd | e.t_wr) & ~treg_ok) return c.fail("word %u: tile register outside the build (handler %u)", pc, f_op(w0));
        if ((e.r_rd | e.r_wr) >> N_RREG) return c.fail("word %u: row register outside the file", pc);
        if (e.t_rd & ~t_def) return c.fail("word %u: reads a tile register not written in this tile", pc);
        if (e.r_rd & ~r_def) return c.fail("word %u: reads a row register not written in this tile", pc);
        if (!check_arg_index(c, e.arg_rd, pc) || !check_arg_index(c, e.arg_wr, pc)) return false;
        if (e.pf >= 0) {
          if (pf_arg[e.pf] < 0) return c.fail("word %u: reads prefetch slot %u that the prologue never fills", pc, (uint32_t)e.pf);
          if (pf_arg[e.pf] != e.arg_rd) return c.fail("word %u: prefetch slot %u holds another operand", pc, (uint32_t)e.pf);
          if (pf_done[e.pf]) return c.fail("word %u: reads prefetch slot %u after refilling it", pc, (uint32_t)e.pf);
          if (e.pf_issue) pf_done[e.pf] = true;
        }
        for (int k = 0; k < 2; ++k)
          if (e.inv[k] >= 0 && inv_arg[e.inv[k]] < 0)
            return c.fail("word %u: reads invariant slot %u that the prologue never loads", pc, (uint32_t)e.inv[k]);
        if (e.buf_wr & reads_since_barrier)
          return c.fail("word %u: writes reduction buffer %u before every wave read it (no barrier)", pc,
                        (uint32_t)__builtin_ctz(e.buf_wr & reads_since_barrier));
        if (e.barrier_mid) reads_since_barrier = 0;
        reads_since_barrier |= e.buf_rd;
        if (e.barrier) reads_since_barrier = 0;
        t_def |= e.t_wr;
        r_def |= e.r_wr;
      }
      for (int s = 0; s < 2; ++s)
        if (pf_arg[s] >= 0 && !pf_done[s] && b1 > b0)
          return c.fail("the body never refills prefetch slot %u for the next tile", (uint32_t)s);
    }
    return true;
  };
  if (!body(W[H_BODY_BEGIN], W[H_BODY_END])) return false;
  // a reduce-all body folds exactly one operand into the lanes' running
  // partials, of the kind the epilogue combines; an ALL in any other program
  // would have no epilogue to deliver it
  {
    int n_all = 0;
    bool kind_ok = true;
    for (uint32_t pc = W[H_BODY_BEGIN]; pc + 1 < W[H_BODY_END]; pc += 2) {
      const uint32_t h = f_op(W[pc]);
      if (h >= HD_ALL && h < HD_ALL + 6) {
        ++n_all;
        kind_ok = kind_ok && (h - HD_ALL) / 3 == W[H_ALL_KIND];
      }
    }
    if (W[H_TEMPLATE] == TM_ALLREDUCE ? n_all != 1 || !kind_ok : n_all != 0)
      return c.fail("%d reduce-all instructions in a program of template %u", n_all, W[H_TEMPLATE]);
  }
  if ((W[H_FLAGS] & HF_COND_FOLD) && !(W[H_FLAGS] & HF_BRANCH)) return c.fail("a folded condition without a branch");
  if (W[H_FLAGS] & HF_BRANCH) {
    if (W[H_COND_ARG] >= c.n_args || c.W[ARG_BASE + W[H_COND_ARG] * ARG_WORDS + A_DTYPE] != DT_F32)
      return c.fail("the branch condition is no fp32 operand");
    if (W[H_FLAGS] & HF_COND_FOLD) {
      // the partials: fp32, a whole number of them, at most 2 T_LANES (the
      // VM folds them in one pass), not the condition the program writes
      const uint32_t k = W[H_ALL_SCRATCH];
      const uint32_t* a = c.W + ARG_BASE + k * ARG_WORDS;
      const uint64_t ext = k < c.n_args ? arg_extent(a[A_FLAGS], a[A_EXTENT]) : 0;
      if (k >= c.n_args || k == W[H_COND_ARG] || a[A_DTYPE] != DT_F32 || ext == 0 || ext % 4 ||
          ext > 8u * T_LANES)
        return c.fail("the folded partials are no fp32 operand of their own");
      if (W[H_ALL_KIND] != RK_SUM && W[H_ALL_KIND] != RK_MAX) return c.fail("fold kind %u", W[H_ALL_KIND]);
    }
    if (!body(W[H_ALT_BEGIN], W[H_ALT_END])) return false;
  }
  return true;
}

bool verify_mix(Ctx& c) {
  const uint32_t* W = c.W;
  // (an empty output has no tiles and no tile size)
  if (W[H_BLOCK_DIM] != 0 && (W[H_TR] != 128 || W[H_TC] != 128))
    return c.fail("MIX tile %u x %u is not a kernel variant", W[H_TR], W[H_TC]);
  if (W[H_BLOCK_DIM] != 0) {
    const int64_t M = ((int64_t)W[H_R_HI] << 32) | W[H_R_LO], N = ((int64_t)W[H_C_HI] << 32) | W[H_C_LO];
    if ((int64_t)W[H_BLOCK_DIM] != cdiv(M, 128) * cdiv(N, 128) || (int64_t)W[H_NC] != cdiv(N, 128))
      return c.fail("MIX block_dim %u is not the tile count", W[H_BLOCK_DIM]);
  }
  if (c.n_args < 2 || W[H_MM_A] != 0 || W[H_MM_B] != 1) return c.fail("MIX operands A and B must be operands 0 and 1");
  for (int k = 0; k < 2; ++k)
    if (W[ARG_BASE + k * ARG_WORDS + A_DTYPE] != DT_BF16) return c.fail("MIX operand %u is not bf16", (uint32_t)k);
  unsigned def = 1u;  // register 0 starts as the matmul result
  for (uint32_t pc = W[H_BODY_BEGIN]; pc < W[H_BODY_END]; pc += 2) {
    const uint32_t w0 = W[pc], w1 = W[pc + 1];
    const uint32_t op = f_op(w0), d = f_dst(w0), a = f_a(w0), b = f_b(w0);
    if (d >= (uint32_t)N_TREG || a >= (uint32_t)N_TREG || b >= (uint32_t)N_TREG) return c.fail("word %u: register outside the epilogue's three", pc);
    switch (op) {
      case OP_LOAD: if (!check_arg_index(c, (int)w1, pc)) return false; def |= 1u << d; break;
      case OP_STORE: if (!(def >> a & 1u)) return c.fail("word %u: stores an unwritten register", pc);
        if (!check_arg_index(c, (int)w1, pc)) return false; break;
      case OP_COPY: if (!(def >> a & 1u)) return c.fail("word %u: copies an unwritten register", pc); def |= 1u << d; break;
      case OP_BIN: if (f_bk(w0) == BK_TREG && !(def >> b & 1u)) return c.fail("word %u: reads an unwritten register", pc);
        if (f_bk(w0) == BK_MEM && !check_arg_index(c, (int)w1, pc)) return false; break;
      case OP_UN: case OP_DBG: def |= 1u << d; break;
      default: return c.fail("word %u: opcode %u in a MIX epilogue", pc, op);
    }
  }
  return true;
}

bool verify_one(const uint32_t* W, uint32_t n_words, std::string* err) {
  Ctx c{W, 0, err};
  if (W[H_MAGIC] != MAGIC || W[H_VERSION] != VERSION) return c.fail("bad magic or version");
  const uint32_t kt = W[H_KTYPE];
  if (kt != KT_VECTOR && kt != KT_MIX && kt != KT_VECTOR_WIDE) return c.fail("kernel type %u", kt);
  c.n_args = W[H_NARGS];
  if (c.n_args > (uint32_t)MAX_ARGS) return c.fail("%u operands", c.n_args);
  const uint32_t base = ARG_BASE + c.n_args * ARG_WORDS;
  uint32_t end = W[H_BODY_END];
  if (W[H_FLAGS] & HF_BRANCH) {
    if (W[H_ALT_BEGIN] != W[H_BODY_END] || W[H_ALT_END] < W[H_ALT_BEGIN]) return c.fail("else-body range");
    end = W[H_ALT_END];
  }
  if (W[H_PRO_BEGIN] != base || W[H_PRO_END] < W[H_PRO_BEGIN] || W[H_BODY_BEGIN] != W[H_PRO_END] ||
      W[H_BODY_END] < W[H_BODY_BEGIN] || end + PAD_WORDS > (uint32_t)MAX_WORDS || end > n_words)
    return c.fail("word ranges out of order or out of bounds (end %u)", end);
  if ((W[H_PRO_BEGIN] | W[H_BODY_BEGIN] | W[H_BODY_END] | end) & 1u) return c.fail("instructions at odd words");
  for (uint32_t k = 0; k < c.n_args; ++k) {
    const uint32_t* a = W + ARG_BASE + k * ARG_WORDS;
    if (a[A_DTYPE] > DT_U8) return c.fail("operand %u: dtype %u", k, a[A_DTYPE]);
    if (arg_flag_bits(a[A_FLAGS]) & AF_VEC) {
      const uint64_t p = ((uint64_t)a[A_PTR_HI] << 32) | a[A_PTR_LO];
      const uint32_t al = a[A_DTYPE] == DT_BF16 ? 2u : 4u;
      if ((int32_t)a[A_SC] != 1 || p % al) return c.fail("operand %u: vector access without unit stride and alignment", k);
    }
  }
  return kt == KT_MIX ? verify_mix(c) : verify_vector(c);
}

}  // namespace

// Verifies a program's words (a single program, or a stacked one: its
// directory and every segment).  Returns true, or false with the first
// violation in *err.
bool verify_words(const uint32_t* W, uint32_t n_words, std::string* err) {
  if (n_words > (uint32_t)MAX_WORDS) {
    *err = "program longer than the kernel argument";
    return false;
  }
  if (W[0] != STACK_MAGIC && W[0] != TSTACK_MAGIC) return verify_one(W, n_words, err);
  // spatial stacks list each segment's first workgroup, temporal ones its
  // first tile in the stack's tile space: both the running sum over the
  // segments before it
  const bool temporal = W[0] == TSTACK_MAGIC;
  const uint32_t n = W[S_NSEG];
  if (n < 2 || n > (uint32_t)MAX_SEGS) {
    *err = "stack directory: segment count";
    return false;
  }
  uint32_t wg = 0, prev_end = STACK_DIR_WORDS;
  for (uint32_t s = 0; s < n; ++s) {
    const uint32_t off = W[S_DIR + 2 * s], first = W[S_DIR + 2 * s + 1];
    if ((off & 1u) || off < prev_end || off + HDR_WORDS > n_words || first != wg) {
      *err = "stack directory: segment " + std::to_string(s) + (temporal ? " offset or first tile" : " offset or first workgroup");
      return false;
    }
    const uint32_t* S = W + off;
    std::string e;
    if (!verify_one(S, n_words - off, &e)) {
      *err = "segment " + std::to_string(s) + ": " + e;
      return false;
    }
    if (S[H_KTYPE] != W[W[S_DIR] + H_KTYPE] || S[H_KTYPE] == KT_MIX || S[H_TEMPLATE] == TM_ALLREDUCE) {
      *err = "segment " + std::to_string(s) + ": not stackable with the first";
      return false;
    }
    const uint32_t seg_end = (S[H_FLAGS] & HF_BRANCH) ? S[H_ALT_END] : S[H_BODY_END];
    prev_end = off + seg_end + PAD_WORDS;
    wg += temporal ? S[H_BLOCK_DIM] : S[H_GRID];
  }
  return true;
}

}  // namespace dvmbc
