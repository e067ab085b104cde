// Tile-level bytecode program format shared by the host encoder and the
// device VM kernels.
//
// A program is one flat array of 32-bit words that travels to the device as
// the VM kernel's argument (the kernarg segment), so the kernel reads it with
// wave-uniform scalar loads.  Layout:
//
//   words [0, HDR_WORDS)                  code header
//   words [ARG_BASE, ARG_BASE + 8 n_args) argument table (global operands)
//   words [instr_base, ...)               code body, 2 words per instruction
//
// The header holds the fields the DVM paper review page names for its code
// header (section 4.3: tile count block_dim, tiles per core body_tile, kernel
// type) plus the tile geometry the VM needs; the body holds one instruction
// per tile-level virtual instruction (Table 1 of that page: Load/Store, Copy,
// Broadcast, elementwise ops; plus the binary ops, reductions and the syncs
// the encoder inserts).
#pragma once
#include <stdint.h>

namespace dvmbc {

constexpr uint32_t MAGIC = 0x314d5644u;  // "DVM1"
constexpr uint32_t VERSION = 3;

// Device geometry constants: one workgroup of T lanes runs a tile; a tile row
// is spread over g lanes, each holding up to NV_MAX chunks of V elements.  Two
// workgroups are resident per compute unit (their waves share each SIMD and
// run different tiles, so one wave's scalar decode overlaps the other's
// vector work).
constexpr int T_LANES = 256;
constexpr int VEC = 8;
constexpr int NV_MAX = 5;
constexpr int E_MAX = VEC * NV_MAX;   // elements per lane per tile register
// The wide VM variant: one tile register of NV_WIDE chunks per lane, for
// programs that never hold a second tile value (twice the columns per lane).
constexpr int NV_WIDE = 10;
constexpr int N_TREG = 3;             // tile registers: 0 = ACC, 1..2 slots
constexpr int N_RREG = 4;             // row registers
constexpr int N_LDSBUF = 8;           // cross-wave reduction buffers
constexpr int MAX_WORDS = 1000;       // whole program, <= 4000 bytes of kernarg
constexpr int PAD_WORDS = 2;          // unused words after the body (the VM reads one instruction ahead)
constexpr int HDR_WORDS = 44;
constexpr int ARG_BASE = HDR_WORDS;
constexpr int ARG_WORDS = 8;
constexpr int MAX_ARGS = 32;

enum KernelType : uint32_t { KT_VECTOR = 0, KT_MIX = 1, KT_VECTOR_WIDE = 2 };
enum Template : uint32_t { TM_ELEMWISE = 0, TM_ROWREDUCE = 1, TM_ALLREDUCE = 2, TM_MATMUL = 3 };

// Header word offsets.
enum Hdr : int {
  H_MAGIC = 0,
  H_VERSION = 1,
  H_KTYPE = 2,
  H_TEMPLATE = 3,
  H_BLOCK_DIM = 4,   // number of tiles
  H_BODY_TILE = 5,   // tiles per workgroup
  H_GRID = 6,        // workgroups launched
  H_TR = 7,          // tile rows
  H_TC = 8,          // tile columns
  H_G = 9,           // lanes per tile row
  H_NV = 10,         // chunks per lane
  H_P = 11,          // lane groups (rows) per workgroup
  H_NC = 12,         // column tiles
  H_NARGS = 13,
  H_PRO_BEGIN = 14,  // prologue (tile-invariant) instruction word range
  H_PRO_END = 15,
  H_BODY_BEGIN = 16, // per-tile instruction word range
  H_BODY_END = 17,
  H_R_LO = 18,
  H_R_HI = 19,
  H_C_LO = 20,
  H_C_HI = 21,
  H_ALL_KIND = 22,   // reduce-all: 0 sum, 1 max (and a branch program with HF_COND_FOLD)
  H_ALL_OUT = 23,    // reduce-all: arg index of the scalar output
  H_ALL_SCRATCH = 24,// reduce-all: arg index of the scratch (partials from byte 256);
                     //   HF_COND_FOLD: arg index of the partials themselves
  H_N_INSTR = 25,
  H_FLAGS = 26,      // HF_* bits
  H_LDS_BYTES = 27,  // dynamic LDS of the launch (staging areas below)
  H_PF_OFF0 = 28,    // byte offset of prefetch slot 0 / 1 (next-tile loads)
  H_PF_OFF1 = 29,
  H_INV_OFF0 = 30,   // byte offset of LDS-resident invariant operand 0 / 1
  H_INV_OFF1 = 31,
  H_INV_SHARED0 = 32,// 1: invariant slot 0 / 1 is one row shared by all row groups
  H_INV_SHARED1 = 33,
  H_MM_K = 34,       // MIX: contraction length K
  H_MM_A = 35,       // MIX: arg index of A [M, K] (bf16, unit stride along K)
  H_MM_B = 36,       // MIX: arg index of B [K, N] (bf16, unit stride along N)
  H_PROF_LO = 37,    // profiling launches only: device address of the per-workgroup
  H_PROF_HI = 38,    //   cycle counters (5 x uint64 per workgroup)
  H_RED_OFF = 39,    // byte offset of the cross-wave reduction buffers in dynamic LDS
  H_COND_ARG = 40,   // branch programs (HF_BRANCH): arg index of the condition (0-d fp32)
  H_COND_THR = 41,   //   the then-body runs iff condition > threshold (fp32 bits), strictly
  H_ALT_BEGIN = 42,  //   word range of the else-body (the then-body is H_BODY_BEGIN..END)
  H_ALT_END = 43,
};

// MIX kernel geometry: the output tile (header H_TR x H_TC) is one of the MIX
// kernel's variants (128 x 128 per 256-lane workgroup, two workgroups per
// compute unit); K runs in stages of MM_KT through a ring of MM_STAGES LDS
// stages, each holding tm x MM_KT of A and MM_KT x tn of B (bf16).  After
// the K loop the fp32 output tile is staged in LDS with rows of tn + MM_OPAD
// values; the ring and the staged tile share the same bytes.
constexpr int MM_KT = 64;
constexpr int MM_STAGES = 2;
constexpr int MM_OPAD = 8;
__host__ __device__ constexpr int mm_lds_bytes(int tm, int tn) {
  return MM_STAGES * (tm + tn) * MM_KT * 2 > tm * (tn + MM_OPAD) * 4 ? MM_STAGES * (tm + tn) * MM_KT * 2
                                                                    : tm * (tn + MM_OPAD) * 4;
}

// LDS staging (per workgroup, dynamic):
//  * prefetch slot: NVK chunks x T lanes x 16 bytes x (element size / 2)
//    (NVK = the VM build's chunk count, NV_MAX or NV_WIDE, whatever the
//    tile's NV: every chunk position has its bytes)
//    halves; lane t's data for chunk j, half h sits at ((j * halves + h) * T +
//    t) * 16, written by a direct-to-LDS buffer load of that lane and read back
//    by the same lane, which then issues the next tile's load into the same
//    bytes (one buffer: the read completes before the refill is issued);
//  * invariant slot: an operand that is the same for every tile, held as fp32,
//    8 elements (32 bytes) per index and chunk, in 2 x NVK planes of 16-byte
//    cells: index i's elements 4h..4h+3 of chunk j sit at ((2j + h) * stride
//    + i) * 16.  A slot shared by the row groups (the operand does not vary
//    along rows) holds one row: stride g, indexed by the lane's position in
//    its row; otherwise stride T, indexed by the lane.  An fp32 operand with
//    contiguous whole-chunk columns is staged with direct-to-LDS loads when
//    each wave's indices are 64 consecutive values (lane-private slots, or
//    g a multiple of 64); others go through registers.
// The budget keeps two workgroups resident per compute unit (160 KB of LDS).
// Both VM builds keep their cross-wave reduction buffers in the dynamic area,
// reserved only by programs that use them (16 bytes of the reservation are
// spare), so two workgroups may take the whole 160 KB (two fp32 prefetch
// slots of 40 KB).
constexpr uint32_t LDS_BUDGET = 80u * 1024u;
constexpr uint32_t RED_LDS_BYTES = N_LDSBUF * (T_LANES / 64) * 4 + 16;

// Argument table entry (8 words): pointer, dtype, flags, column stride, row
// stride (elements, in the collapsed [R, C] iteration space) and the byte
// extent of the tensor (one past its last element), which bounds every access
// the VM makes to it.
enum ArgW : int { A_PTR_LO = 0, A_PTR_HI = 1, A_DTYPE = 2, A_FLAGS = 3, A_SR_LO = 4, A_SR_HI = 5,
                  A_SC = 6, A_EXTENT = 7 };
// The operand's byte extent is 64-bit: bits [31:0] in word A_EXTENT, bits
// [55:32] in bits [31:8] of word A_FLAGS (whose bits [7:0] hold the flags).
// The VM addresses one tile through a buffer resource based at the tile with
// 32-bit lane offsets, so a tile must span < EXTENT_CAP bytes; the resource's
// record count is the extent left after the tile start, capped the same way.
constexpr uint32_t EXTENT_CAP = 0x80000000u;
__host__ __device__ constexpr uint32_t arg_flag_bits(uint32_t w_flags) { return w_flags & 0xffu; }
__host__ __device__ constexpr uint64_t arg_extent(uint32_t w_flags, uint32_t w_extent) {
  return ((uint64_t)(w_flags >> 8) << 32) | (uint64_t)w_extent;
}
__host__ __device__ constexpr uint32_t arg_flags_word(uint32_t flags, uint64_t extent) {
  return (flags & 0xffu) | ((uint32_t)(extent >> 32) << 8);
}
enum DType : uint32_t { DT_F32 = 0, DT_BF16 = 1, DT_U8 = 2 };
enum HdrFlag : uint32_t {
  // tile operands and outputs move with the streaming (non-temporal) cache
  // policy: set for programs that touch at least STREAM_BYTES, except
  // reduce-all programs, whose input the host-resolved branch after them
  // usually reads again.  Smaller programs keep the default policy, so data
  // they share with the launches around them can stay in the last-level
  // cache.  (Measured on MI355X: 16 MiB rather than 64 leaves the kernels'
  // own throughput unchanged and shortens the wait of a host sync after a
  // launch, e.g. 9% end to end on the if-else stream.)
  HF_STREAM = 1u,
  // a branch program: two bodies over one tiling, prologue and operand table;
  // the VM reads the condition operand once and every tile runs the body it
  // selects (device-side control flow: no host round trip between the launch
  // that writes the condition and this one)
  HF_BRANCH = 2u,
  // race-stress launches (profiling twin only): before every dispatch a wave
  // sleeps a pseudo-random, wave-uniform number of intervals drawn from the
  // seed in bits [31:8], so waves drift apart and a missing barrier shows as
  // a changed result
  HF_STRESS = 4u,
  // cross-wave reductions alternate between LDS buffers b and b ^ 2 by the
  // parity of the workgroup's tile count: set instead of an end-of-body
  // barrier when a tile's cross-wave reductions use only buffers 0 and 1 and
  // its last one reads a buffer that the next tile's first one writes, which
  // would otherwise overwrite it while slower waves still read it (the next
  // tile's own barrier fences the reads before the buffers come round again)
  HF_RED_ALT = 8u,
  // a branch program whose condition is the scalar of the reduce-all launched
  // just before it, whose combine launch it replaces: each wave folds the
  // workgroup partials (operand H_ALL_SCRATCH, at most 2 T_LANES of them, kind
  // H_ALL_KIND) in the combine's order, and workgroup 0 writes the scalar to
  // the condition operand
  HF_COND_FOLD = 16u,
};
constexpr uint64_t STREAM_BYTES = 16ull << 20;
enum ArgFlag : uint32_t {
  AF_VEC = 1u,       // chunk starts aligned (bf16: to the element, else the dword): 64/128-bit path
};

// Opcodes (bits [7:0] of word 0).
enum Op : uint32_t {
  OP_END = 0,
  OP_LOAD = 1,       // treg[dst] <- arg[w1] tile           (Load / ViewLoad)
  OP_LOAD_ROW = 2,   // rreg[dst] <- arg[w1] row value
  OP_STORE = 3,      // arg[w1] <- treg[a] tile              (Store / ViewStore)
  OP_STORE_ROW = 4,  // arg[w1] <- rreg[a]
  OP_COPY = 5,       // treg[dst] <- treg[a]                 (Copy)
  OP_BIN = 6,        // treg[0] <- treg[0] (op) B, or B (op) treg[0]
  OP_UN = 7,         // treg[0] <- f(treg[0])
  OP_RBIN = 8,       // rreg[dst] <- rreg[a] (op) (rreg[b] | imm)
  OP_RUN = 9,        // rreg[dst] <- f(rreg[a])
  OP_RED = 10,       // row reduce of treg[a]: rreg[dst] (and LDS buffer b if the row spans waves)
  OP_RED_FIN = 11,   // (unused: cross-wave row reductions are OP_REDX)
  OP_SYNC = 12,      // workgroup barrier inserted by the encoder
  OP_ALL = 13,       // reduce-all: treg[a]'s lane partial folded into the lane's running
                     //   partial (the VM's reduce-all epilogue combines the lanes, waves
                     //   and workgroups)
  OP_ALL_FIN = 14,   // (retired: reduce-all partials are per workgroup, in the epilogue)
  OP_BCAST = 15,     // treg[dst] <- rreg[a] broadcast along the row (Broadcast)
  OP_DBG = 16,       // treg[dst] <- tile id (sub 0) / workgroup id (sub 1)
  OP_LDS_INV = 17,   // prologue: invariant slot dst <- arg[w1] (fp32, lane-private)
  OP_PF = 18,        // prologue: prefetch slot b <- arg[w1] for the first tile
  OP_REDX = 19,      // row reduce of treg[a] across waves: partial into LDS buffer b,
                     //   workgroup barrier, combine of the row's partials into rreg[dst]
  OP_FMA_INV = 20,   // treg[0] <- (treg[0] * r) * inv[b] + inv[a]: a multiply by one tile-
                     //   invariant operand and an add of another in one rounding, r =
                     //   rreg[dst] if bk == BK_RREG (a row scale applied first) else 1
  OP_COUNT
};

// Handler ids.  The encoder emits the generic opcodes above and, as its last
// step, rewrites bits [7:0] of every word 0 into the id of the specialised VM
// routine that runs it: register numbers, ALU op, operand form and dtype are
// folded into the id, so the VM decodes one byte with one switch and the
// routine itself has no further branches on them.  The other fields keep their
// meaning (staging slot, wait count, row register, scalar / argument word).
enum Handler : uint32_t {
  HD_END = 0,
  HD_LD_DIR = 1,     // + d: treg[d] <- arg[w1] tile, straight from memory (any dtype)
  HD_LD_PF16 = 10,   // + d: bf16 from prefetch slot b (then refill it, if FL_ISSUE)
  HD_LD_PF32 = 13,   // + d: f32 from prefetch slot b
  HD_LD_INV = 16,    // + d: from invariant slot b
  HD_ST_DIR = 19,    // + a: arg[w1] <- treg[a] (any dtype)
  HD_ST_BF16 = 22,   // arg[w1] <- ACC, bf16
  HD_ST_F32 = 23,    // arg[w1] <- ACC, f32
  HD_COPY = 28,      // + 3 d + a: treg[d] <- treg[a]
  HD_UN = 37,        // + f (Una): ACC <- f(ACC)
  HD_BIN = 48,       // + 10 alu + form: ACC <- ACC (op) B; forms 0..2: B = treg[form],
                     //   3: B = row register b or the immediate w1; + 5: reversed,
                     //   B (op) ACC (pow, division by a register and memory operands
                     //   have handlers of their own)
  HD_RED = 118,      // + 3 kind + a: row reduce of treg[a] into rreg[dst] (rows inside a wave)
  HD_REDX = 127,     // + 3 kind + a: OP_REDX (rows across waves)
  HD_ALL = 136,      // + 3 kind + a: OP_ALL (sum, max)
  HD_ALL_FIN = 142,  // (retired with OP_ALL_FIN; the ids stay reserved)
  HD_BCAST = 144,    // + d
  HD_RBIN = 147,
  HD_RUN = 148,
  HD_SYNC = 149,
  HD_LD_ROW = 150,
  HD_ST_ROW = 151,
  HD_DBG = 152,
  HD_LDS_INV = 153,
  HD_PF = 154,
  HD_BIN_POW = 155,  // ACC <- ACC pow B (or B pow ACC), B of forms 0..3 (from bk, b)
  HD_BIN_MEM = 156,  // ACC <- ACC (op) B for a memory operand, any ALU op (sub, FL_REV)
  HD_DIV_T = 157,    // ACC <- ACC / treg[b] (or treg[b] / ACC)
  HD_FMA_INV = 158,  // OP_FMA_INV
  HD_SILU = 159,     // ACC <- ACC / (exp(-ACC) + 1) (OP_UN, UN_SILU)
  HD_SOFTMAX = 160,  // ACC <- row softmax of ACC (OP_UN, UN_SOFTMAX); rows across waves use
                     //   LDS buffers b and b + 1 and one barrier
  HD_COUNT = 161
};
enum BinForm : uint32_t { BF_T0 = 0, BF_T1 = 1, BF_T2 = 2, BF_SCALAR = 3, BF_MEM = 4, BF_REV = 5 };

// ALU sub-ops (bits [23:20]).
enum Alu : uint32_t {
  ALU_ADD = 0, ALU_SUB = 1, ALU_MUL = 2, ALU_DIV = 3, ALU_MAX = 4, ALU_MIN = 5, ALU_POW = 6,
};
enum Una : uint32_t {
  UN_SQRT = 0, UN_ABS = 1, UN_LOG = 2, UN_EXP = 3, UN_ROUND = 4, UN_FLOOR = 5, UN_ISFINITE = 6,
  UN_NEG = 7, UN_RECIP = 8, UN_TOBF16 = 9, UN_IDENT = 10,
  UN_SILU = 11,  // z / (exp(-z) + 1): a fused SiLU chain, the chain's own operations in registers
  // exp(z - max) / sum(exp(z - max)) over the row: a fused softmax chain.  Rows
  // inside a wave: the chain's own operations in order.  Rows across waves:
  // each wave's max m_w and sum s_w of exp(z - m_w) cross in one exchange;
  // then M = max m_k, S = sum s_k exp(m_k - M) and the output exp(z - m_w)
  // exp(m_w - M) / S (fp32 reordering only)
  UN_SOFTMAX = 12,
};
enum BKind : uint32_t { BK_TREG = 0, BK_RREG = 1, BK_IMM = 2, BK_MEM = 3 };  // BK_MEM: B loaded from arg[w1]
// RK_SUMSQ: sum of the squares of treg[a] (a reduce of x * x whose product is
// not needed otherwise; row reduces only).
enum RedKind : uint32_t { RK_SUM = 0, RK_MAX = 1, RK_SUMSQ = 2 };

// Word 0 fields.
__host__ __device__ constexpr uint32_t enc0(uint32_t op, uint32_t dst, uint32_t a, uint32_t b,
                                            uint32_t sub, uint32_t bk, uint32_t flags) {
  return (op & 0xffu) | ((dst & 0xfu) << 8) | ((a & 0xfu) << 12) | ((b & 0xfu) << 16) |
         ((sub & 0xfu) << 20) | ((bk & 0xfu) << 24) | ((flags & 0xfu) << 28);
}
__host__ __device__ constexpr uint32_t f_op(uint32_t w) { return w & 0xffu; }
__host__ __device__ constexpr uint32_t f_dst(uint32_t w) { return (w >> 8) & 0xfu; }
__host__ __device__ constexpr uint32_t f_a(uint32_t w) { return (w >> 12) & 0xfu; }
__host__ __device__ constexpr uint32_t f_b(uint32_t w) { return (w >> 16) & 0xfu; }
__host__ __device__ constexpr uint32_t f_sub(uint32_t w) { return (w >> 20) & 0xfu; }
__host__ __device__ constexpr uint32_t f_bk(uint32_t w) { return (w >> 24) & 0xfu; }
__host__ __device__ constexpr uint32_t f_flags(uint32_t w) { return (w >> 28) & 0xfu; }
constexpr uint32_t FL_REV = 1u;    // BIN: B (op) ACC instead of ACC (op) B
constexpr uint32_t FL_PF = 2u;     // LOAD / BIN BK_MEM: read the operand from prefetch slot b
constexpr uint32_t FL_ISSUE = 4u;  // ... then prefetch the workgroup's next tile into the same slot
constexpr uint32_t FL_INV = 8u;    // LOAD / BIN BK_MEM: read the operand from invariant slot b

// Prefetch reads wait with vmcnt(n), n = a lower bound (computed by the
// encoder for full tiles) on the vector-memory instructions this wave issued
// after the prefetch being read; vmcnt retires in issue order, so the wait
// covers the prefetch without waiting for later stores.  LOAD keeps n in
// fields a | sub << 4, BIN (memory operand) in dst | a << 4.
__host__ __device__ constexpr uint32_t vmc_load(uint32_t w) { return ((w >> 12) & 0xfu) | (((w >> 20) & 0xfu) << 4); }
__host__ __device__ constexpr uint32_t vmc_bin(uint32_t w) { return ((w >> 8) & 0xfu) | (((w >> 12) & 0xfu) << 4); }
constexpr uint32_t VMC_MAX = 63;

// Stacked launches (the stacking-based fusion of the DVM review page, section
// 5.1: independent graphs packed into one launch, each on its own
// workgroups).  The kernel argument then starts with a directory instead of a
// header: word 0 STACK_MAGIC, word 1 the number of segments, then per segment
// s the word offset of its program (a complete program: header, operand
// table, prologue, body, whose word indices are relative to its own start) and
// the first workgroup that runs it.  Workgroup b belongs to the segment with
// the largest first workgroup <= b and runs that program as workgroup b -
// first of a grid that ends where the next segment starts.  Segment offsets
// are even (instructions are fetched as 8-byte pairs) and each segment is
// followed by PAD_WORDS spare words.
constexpr uint32_t STACK_MAGIC = 0x4b545344u;  // "DSTK"
// Temporal stacking (the same section: different graphs' tiles run on the same
// core in sequence): word 0 TSTACK_MAGIC, the same directory layout with
// each segment's second word the index of its first tile in one tile space
// that numbers the segments' tiles in order (its first tile = the sum of the
// earlier segments' block_dim).  A launch of G workgroups runs tile u of that
// space on workgroup u mod G, so every workgroup walks the segments in order;
// a barrier separates its segments.
constexpr uint32_t TSTACK_MAGIC = 0x4b535454u;  // "TTSK"
constexpr int S_NSEG = 1;
constexpr int S_DIR = 2;                        // (offset, first workgroup) pairs from here
constexpr int MAX_SEGS = 7;
constexpr int STACK_DIR_WORDS = S_DIR + 2 * MAX_SEGS;

struct Program {
  uint32_t w[MAX_WORDS];
};

}  // namespace dvmbc
