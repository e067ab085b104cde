// The resident VM kernel for VECTOR programs (elementwise, row-reduce and
// reduce-all templates) on gfx950.
//
// It follows the VM algorithm of the DVM paper review page (section 4.4):
// each workgroup finds its tiles from the code header (workgroup b runs
// tiles b, b + grid, ..., at most body_tile of them), and for every tile
// decodes the body instruction by instruction and runs the matching
// virtual-instruction routine.  Decoding is wave-uniform:
// the program sits in the kernarg segment and every word is read with a scalar
// load (the next instruction's words are fetched while the current one runs),
// so the dispatch is a tree of scalar compares on one pre-decoded handler byte
// (the counterpart of the page's decode on the Scalar unit), and the routines
// run on the vector ALUs, the LDS and the vector memory pipeline.
//
// Tiles are staged in registers: each lane owns up to NVK chunks of VEC
// consecutive columns of its row, so elementwise chains never leave the VGPR
// file (the page's "intermediate results stay in local memory" of section
// 5.1, with the register file as that local memory).  Every register number
// is folded into the handler id, so each routine names its registers
// statically; compute has the two-address form ACC <- ACC (op) B.
//
// The interpreter loop branches only on wave-uniform values.  Lane masks are
// selects over values every lane computes (out-of-range buffer offsets for
// memory), so the compiler keeps the tile registers in place across the
// dispatch instead of merging copies of them at divergent joins.
//
// Global memory is reached through buffer resources: one scalar descriptor
// per operand and tile (base = the tile's first element, size = the bytes left
// in the tensor), 32-bit lane offsets, and an out-of-range offset for masked
// elements, so loads and stores are branch-free (a masked load returns 0 and a
// masked store is dropped) and never touch memory outside the operand.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bytecode.h"

using namespace dvmbc;

// Two builds of this source: the standard VM (three tile registers of NV_MAX
// chunks per lane) and, with DVM_WIDE defined, the wide VM (one tile register
// of NV_WIDE chunks), for programs whose values all pass through the
// accumulator and whose rows are too long for two of them to share a
// standard tile.  Every symbol of the wide build carries a _wide suffix.
#ifdef DVM_WIDE
#define DVM_SYM(name) name##_wide
#else
#define DVM_SYM(name) name
#endif

namespace {

#ifdef DVM_WIDE
constexpr int NVK = NV_WIDE;  // chunks per lane per tile register
constexpr int TREGS = 1;      // tile registers
#else
constexpr int NVK = NV_MAX;
constexpr int TREGS = N_TREG;
#endif

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float V8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef __attribute__((address_space(3))) void lds_void;
// Program words are read in place in the kernarg segment (constant address
// space, scalar loads); the kernel never takes a copy of its argument.
typedef const __attribute__((address_space(4))) uint32_t KW;
typedef uint32_t u2w __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(4))) u2w KW2;

// The two words of the instruction at word pc (even, so 8-byte aligned in the
// kernarg segment) with one scalar load.
__device__ __forceinline__ void fetch2(KW* W, uint32_t pc, uint32_t& a, uint32_t& b) {
  const u2w v = *(KW2*)(W + pc);
  a = v.x;
  b = v.y;
}

constexpr int OOB = 0x7fffffff;                 // lane offset beyond any descriptor size
// Cache policy of the streaming accesses (tile operands and outputs) of
// programs flagged HF_STREAM: non-temporal, so a stream passing through does
// not evict what is reused (tile-invariant operands, the program).  Measured
// on the LayerNorm stream: 6% less time per launch.
constexpr int CP_STREAM = 2;                    // gfx950 cache-policy bit nt
__device__ __forceinline__ bool streaming(KW* W) { return (W[H_FLAGS] & HF_STREAM) != 0; }
constexpr int RSRC_W3 = 0x00020000;             // raw buffer, 32-bit data format

// One tile register: NVK chunks of VEC fp32 values per lane.
struct Ch {
  V8 c[NVK];
};

struct ArgD {
  const char* p;
  uint32_t dt, fl;
  int64_t sr;
  int32_t sc;
  uint64_t extent;
};

struct Geo {
  int g, nv, tr, tc, nc, lg;  // lg = log2(g)
  int64_t R, C;
};

// The tile's chunk count for a per-chunk pass, opaque to the optimiser so the
// pass compares it chunk by chunk (one scalar branch each) instead of keeping
// a condition per chunk live across the interpreter loop.  Chunks at or past
// nv hold only columns past every row end: passes skip them, reductions mask
// their columns, and the encoder's wait counts assume nv chunks per access.
__device__ __forceinline__ int nv_pass(const Geo& G) {
  int n = G.nv;
  asm volatile("" : "+s"(n));
  return n;
}

struct Tile {
  int64_t r0;   // first row of the tile
  int64_t c0;   // first column of the tile
  int tce;      // valid columns in this tile
  int tre;      // valid rows in this tile
  uint32_t id;
};

// Lane coordinates inside the tile.
struct Lane {
  int tid;
  int row;   // row group of the lane (row inside the tile)
  int lane;  // position inside the row group
  bool rok;  // the row exists
};

__device__ __forceinline__ uint64_t w64(KW* w, int lo) {
  return ((uint64_t)w[lo + 1] << 32) | (uint64_t)w[lo];
}

// Bytes of reduce-all partials a program of block_dim tiles writes into a
// scratch operand of `extent` bytes (counter at byte 0, partials from 256).
__device__ __forceinline__ uint32_t part_bytes(uint64_t extent, uint32_t block_dim) {
  const uint64_t room = extent > 256u ? extent - 256u : 0u;
  const uint64_t need = 4ull * block_dim;
  return (uint32_t)(need < room ? need : room);
}

__device__ __forceinline__ ArgD read_arg(KW* W, uint32_t i) {
  KW* a = W + ARG_BASE + i * ARG_WORDS;
  ArgD d;
  d.p = reinterpret_cast<const char*>(w64(a, A_PTR_LO));
  d.dt = a[A_DTYPE];
  d.fl = arg_flag_bits(a[A_FLAGS]);
  d.sr = (int64_t)w64(a, A_SR_LO);
  d.sc = (int32_t)a[A_SC];
  d.extent = arg_extent(a[A_FLAGS], a[A_EXTENT]);
  return d;
}

template <uint32_t DT>
constexpr int esize_c() { return DT == DT_F32 ? 4 : DT == DT_BF16 ? 2 : 1; }
__device__ __forceinline__ int esize(uint32_t dt) { return dt == DT_F32 ? 4 : dt == DT_BF16 ? 2 : 1; }

// Byte offset of the tile's first element in the operand, and the bytes of
// the operand from there on (capped): the size of the tile's descriptor.
__device__ __forceinline__ int64_t tile_offset(const ArgD& a, const Tile& tl, int es) {
  return (tl.r0 * a.sr + tl.c0 * (int64_t)a.sc) * es;
}

__device__ __forceinline__ int tile_records(const ArgD& a, const Tile& tl, int es) {
  const int64_t left = (int64_t)a.extent - tile_offset(a, tl, es);
  return left <= 0 ? 0 : (left >= (int64_t)EXTENT_CAP ? (int)(EXTENT_CAP - 1) : (int)left);
}

// Descriptor over the operand's part of the tile: base at the tile's first
// element, size = bytes left in the tensor (capped).
__device__ __forceinline__ Rsrc tile_rsrc(const ArgD& a, const Tile& tl, int es) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a.p + tile_offset(a, tl, es)), 0,
                                           tile_records(a, tl, es), RSRC_W3);
}

// The same descriptor as four scalar words (for inline assembly).
__device__ __forceinline__ u4 tile_rsrc_words(const ArgD& a, const Tile& tl, int es) {
  const uint64_t base = (uint64_t)(uintptr_t)(a.p + tile_offset(a, tl, es));
  u4 r;
  r.x = (uint32_t)base;
  r.y = (uint32_t)(base >> 32) & 0xffffu;  // stride 0
  r.z = (uint32_t)tile_records(a, tl, es);
  r.w = (uint32_t)RSRC_W3;
  return r;
}

__device__ __forceinline__ Tile make_tile(const Geo& G, uint32_t id) {
  Tile tl;
  const uint32_t ir = id / (uint32_t)G.nc;
  const uint32_t ic = id - ir * (uint32_t)G.nc;
  tl.id = id;
  tl.r0 = (int64_t)ir * G.tr;
  tl.c0 = (int64_t)ic * G.tc;
  const int64_t remc = G.C - tl.c0;
  tl.tce = remc < G.tc ? (int)remc : G.tc;
  const int64_t remr = G.R - tl.r0;
  tl.tre = remr < G.tr ? (int)remr : G.tr;
  return tl;
}

// a tile whose columns end on a chunk boundary moves whole chunks
__device__ __forceinline__ bool tile_full(const Tile& tl) { return (tl.tce & (VEC - 1)) == 0; }

// Lane masks: selects over values computed on every lane (the arguments are
// evaluated before the call), so no lane-dependent branch is formed.
__device__ __forceinline__ int lane_off(bool ok, int off) { return ok ? off : OOB; }
__device__ __forceinline__ float lane_sel(bool ok, float v, float other) { return ok ? v : other; }

// ---------------------------------------------------------------------------
// element conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint32_t f2bf_pack(float lo, float hi) {
  f2 v = {lo, hi};
  bf2 b = __builtin_convertvector(v, bf2);  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float round_bf16(float x) { return bf2f(f2bf_pack(x, 0.f) & 0xffffu); }

// A chunk a pass skips: a fresh definition with no instructions (its value
// is never used), so the register keeps no older value alive.
__device__ __forceinline__ V8 skipped_chunk() {
  V8 v;
  asm volatile("" : "=v"(v));
  return v;
}

__device__ __forceinline__ V8 unpack_bf16(u4 v) {
  V8 r;
  r[0] = bf2f(v.x & 0xffffu); r[1] = __uint_as_float(v.x & 0xffff0000u);
  r[2] = bf2f(v.y & 0xffffu); r[3] = __uint_as_float(v.y & 0xffff0000u);
  r[4] = bf2f(v.z & 0xffffu); r[5] = __uint_as_float(v.z & 0xffff0000u);
  r[6] = bf2f(v.w & 0xffffu); r[7] = __uint_as_float(v.w & 0xffff0000u);
  return r;
}

__device__ __forceinline__ V8 unpack_f32(u4 a, u4 b) {
  V8 r;
  r[0] = __uint_as_float(a.x); r[1] = __uint_as_float(a.y); r[2] = __uint_as_float(a.z); r[3] = __uint_as_float(a.w);
  r[4] = __uint_as_float(b.x); r[5] = __uint_as_float(b.y); r[6] = __uint_as_float(b.z); r[7] = __uint_as_float(b.w);
  return r;
}

// ---------------------------------------------------------------------------
// ALU
// ---------------------------------------------------------------------------
template <uint32_t OPK>
__device__ __forceinline__ float alu(float x, float y) {
  if constexpr (OPK == ALU_ADD) return x + y;
  else if constexpr (OPK == ALU_SUB) return x - y;
  else if constexpr (OPK == ALU_MUL) return x * y;
  else if constexpr (OPK == ALU_DIV) return x / y;
  // NaN-propagating (IEEE 754-2019 maximum / minimum: v_maximum3_f32 / v_minimum3_f32)
  else if constexpr (OPK == ALU_MAX) return __builtin_elementwise_maximum(x, y);
  else if constexpr (OPK == ALU_MIN) return __builtin_elementwise_minimum(x, y);
  else return powf(x, y);
}

__device__ __forceinline__ float alu_rt(uint32_t k, float x, float y) {
  switch (k) {
    case ALU_ADD: return x + y;
    case ALU_SUB: return x - y;
    case ALU_MUL: return x * y;
    case ALU_DIV: return x / y;
    case ALU_MAX: return alu<ALU_MAX>(x, y);
    case ALU_MIN: return alu<ALU_MIN>(x, y);
    default: return powf(x, y);
  }
}

template <uint32_t F>
__device__ __forceinline__ float una(float x) {
  if constexpr (F == UN_SQRT) return sqrtf(x);
  else if constexpr (F == UN_ABS) return fabsf(x);
  else if constexpr (F == UN_LOG) return logf(x);
  else if constexpr (F == UN_EXP) return __expf(x);  // v_exp_f32 of x log2(e)
  else if constexpr (F == UN_ROUND) return rintf(x);
  else if constexpr (F == UN_FLOOR) return floorf(x);
  else if constexpr (F == UN_ISFINITE) return isfinite(x) ? 1.f : 0.f;
  else if constexpr (F == UN_NEG) return -x;
  else if constexpr (F == UN_RECIP) return 1.f / x;
  else if constexpr (F == UN_TOBF16) return round_bf16(x);
  else if constexpr (F == UN_SILU) return x / (__expf(-x) + 1.f);  // the chain's operations, in order
  else return x;
}

__device__ __forceinline__ float una_rt(uint32_t f, float x) {
  switch (f) {
    case UN_SQRT: return sqrtf(x);
    case UN_ABS: return fabsf(x);
    case UN_LOG: return logf(x);
    case UN_EXP: return __expf(x);
    case UN_ROUND: return rintf(x);
    case UN_FLOOR: return floorf(x);
    case UN_ISFINITE: return isfinite(x) ? 1.f : 0.f;
    case UN_NEG: return -x;
    case UN_RECIP: return 1.f / x;
    case UN_TOBF16: return round_bf16(x);
    case UN_SILU: return x / (__expf(-x) + 1.f);
    default: return x;
  }
}

// Row registers: one value per lane (the lane's row).  Four named variables,
// not an array, so that a wave-uniform index selects among registers instead
// of becoming an indexed private (scratch) access.
struct RowRegs {
  float r0, r1, r2, r3;
};
__device__ __forceinline__ float rget(const RowRegs& rw, uint32_t i) {
  const float a = (i & 1u) ? rw.r1 : rw.r0;
  const float b = (i & 1u) ? rw.r3 : rw.r2;
  return (i & 2u) ? b : a;
}
__device__ __forceinline__ void rset(RowRegs& rw, uint32_t i, float v) {
  if (i == 0) rw.r0 = v;
  else if (i == 1) rw.r1 = v;
  else if (i == 2) rw.r2 = v;
  else rw.r3 = v;
}

__device__ __forceinline__ void fill(Ch& d, float v) {
#pragma unroll
  for (int j = 0; j < NVK; ++j) d.c[j] = (V8)v;
}

// Make every value of a freshly loaded tile register available before the
// routine returns (an empty use of each value).  A routine that left loads
// outstanding into its destination would make the compiler wait, in every
// routine after the dispatch merge, for all outstanding vector memory.
__device__ __forceinline__ void settle(Ch& d) {
#pragma unroll
  for (int j = 0; j < NVK; ++j) {
    float x0 = d.c[j][0], x1 = d.c[j][1], x2 = d.c[j][2], x3 = d.c[j][3];
    float x4 = d.c[j][4], x5 = d.c[j][5], x6 = d.c[j][6], x7 = d.c[j][7];
    asm volatile("" : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3), "+v"(x4), "+v"(x5), "+v"(x6), "+v"(x7));
    d.c[j][0] = x0; d.c[j][1] = x1; d.c[j][2] = x2; d.c[j][3] = x3;
    d.c[j][4] = x4; d.c[j][5] = x5; d.c[j][6] = x6; d.c[j][7] = x7;
  }
}

// ---------------------------------------------------------------------------
// Ragged tiles: the tile's columns do not end on a chunk boundary.
//
// Every row's last column lies in chunk q = (tce - 1) / VEC of its row, held
// by lane q mod g of the row group, in chunk slot q / g.  tce and g are the
// same on every lane, so that slot, that lane and the number of valid columns
// in the chunk are wave-uniform: the per-element work on the row-end chunk
// sits behind scalar branches and runs on one chunk, not on every slot.
//
// Reads take the row-end chunk with the same 128-bit access as the others
// when those bytes lie inside the operand's extent: the bytes past the row's
// end then belong to the next row or to the gap between rows, and their values
// are never used (stores and reductions mask them).  Only where the tile's
// last row ends within one chunk of the extent's end is the chunk completed
// element by element.
// ---------------------------------------------------------------------------
struct Tail {
  int slot;  // chunk slot holding every row's last column
  int lane;  // lane, inside its row group, that holds it
  int col;   // first column of that chunk
  int r;     // valid columns in it (1..VEC-1)
};

__device__ __forceinline__ Tail tail_of(const Geo& G, const Tile& tl) {
  static_assert(VEC == 8, "chunk index below divides by eight");
  const int q = (tl.tce - 1) >> 3;
  return {q >> G.lg, q & (G.g - 1), q * VEC, tl.tce & (VEC - 1)};
}

// Columns of the tile that whole-chunk reads may cover, for rows 0..rows-1
// at row stride a.sr >= 0: up to the end of the row-end chunk when the last
// row's copy of that chunk lies inside the extent (then every row's does),
// else the whole chunks only.
__device__ __forceinline__ int chunk_cols(const ArgD& a, const Tile& tl, int es, int rows) {
  const int full = tl.tce & ~(VEC - 1);
  if (full == tl.tce) return full;
  const int64_t end = ((int64_t)(rows - 1) * a.sr + (full + VEC)) * es;
  return end <= (int64_t)tile_records(a, tl, es) ? full + VEC : full;
}

template <uint32_t DT>
__device__ __forceinline__ float load_elem(const Rsrc& rs, int off) {
  if constexpr (DT == DT_F32) return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
  else if constexpr (DT == DT_BF16) return bf2f(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
  else return (float)__builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0);
}

// Complete the row-end chunk element by element (for reads whose whole-chunk
// accesses stopped short of it).
template <uint32_t DT>
__device__ __forceinline__ void load_tail(Ch& d, const Rsrc& rs, int roff, const Geo& G, const Tile& tl,
                                          const Lane& L, bool rok) {
  constexpr int ES = esize_c<DT>();
  const Tail T = tail_of(G, tl);
  const bool mine = rok & (L.lane == T.lane);
  float v[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) v[i] = load_elem<DT>(rs, lane_off(mine & (i < T.r), (roff + T.col + i) * ES));
  // wait for these loads on this path: left pending, they would make the
  // compiler wait at the join for all outstanding vector memory (a prefetch
  // issued later included), also on the path that skips them
  asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
#pragma unroll
  for (int j = 0; j < NVK; ++j)
    if (j == T.slot)
#pragma unroll
      for (int i = 0; i < VEC; ++i) d.c[j][i] = lane_sel(mine, v[i], d.c[j][i]);
}

// Store the first r (1..VEC-1) values of chunk x at byte offset off as pieces
// of four, two and one elements.
template <uint32_t DT>
__device__ __forceinline__ void store_part(const V8& x, const Rsrc& rs, int off, int r) {
  constexpr int ES = esize_c<DT>();
  // the two-element piece starts at element r&4, the one-element piece at r&6
  const int o2 = off == OOB ? OOB : off + (r & 4) * ES;
  const int o1 = off == OOB ? OOB : off + (r & 6) * ES;
  const bool h4 = (r & 4) != 0, h2 = (r & 2) != 0;
  const float y0 = h4 ? x[4] : x[0], y1 = h4 ? x[5] : x[1];
  const float z = h4 ? (h2 ? x[6] : x[4]) : (h2 ? x[2] : x[0]);
  if constexpr (DT == DT_F32) {
    if (r & 4) {
      u4 v;
      v.x = __float_as_uint(x[0]); v.y = __float_as_uint(x[1]); v.z = __float_as_uint(x[2]); v.w = __float_as_uint(x[3]);
      __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 0);
    }
    if (r & 2) {
      u2 v;
      v.x = __float_as_uint(y0); v.y = __float_as_uint(y1);
      __builtin_amdgcn_raw_buffer_store_b64(v, rs, o2, 0, 0);
    }
    if (r & 1) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(z), rs, o1, 0, 0);
  } else if constexpr (DT == DT_BF16) {
    if (r & 4) {
      u2 v;
      v.x = f2bf_pack(x[0], x[1]); v.y = f2bf_pack(x[2], x[3]);
      __builtin_amdgcn_raw_buffer_store_b64(v, rs, off, 0, 0);
    }
    if (r & 2) __builtin_amdgcn_raw_buffer_store_b32(f2bf_pack(y0, y1), rs, o2, 0, 0);
    if (r & 1) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(f2bf_pack(z, 0.f) & 0xffffu), rs, o1, 0, 0);
  } else {
    if (r & 4) {
      uint32_t v = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) v |= ((uint32_t)x[i] & 0xffu) << (8 * i);
      __builtin_amdgcn_raw_buffer_store_b32(v, rs, off, 0, 0);
    }
    if (r & 2)
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(((uint32_t)y0 & 0xffu) | (((uint32_t)y1 & 0xffu) << 8)), rs, o2, 0, 0);
    if (r & 1) __builtin_amdgcn_raw_buffer_store_b8((uint8_t)z, rs, o1, 0, 0);
  }
}

template <uint32_t DT>
__device__ __forceinline__ void store_tail(const Ch& s, const Rsrc& rs, int roff, const Geo& G, const Tile& tl,
                                           const Lane& L) {
  constexpr int ES = esize_c<DT>();
  if (tile_full(tl)) return;
  const Tail T = tail_of(G, tl);
  const int off = lane_off(L.rok & (L.lane == T.lane), (roff + T.col) * ES);
#pragma unroll
  for (int j = 0; j < NVK; ++j)
    if (j == T.slot) store_part<DT>(s.c[j], rs, off, T.r);
}

// ---------------------------------------------------------------------------
// Load / Store (Table 1: Load/ViewLoad/Store/ViewStore)
// ---------------------------------------------------------------------------
// Fill d (one tile register) from operand a for this tile.  `any_row` loads
// as if every row of the tile existed (for operands that do not vary along
// rows, whose row offset is zero).
// The 128-bit chunk loads of load_dir: all chunks (ALL) or the first nv.
template <uint32_t DT, int CP, bool ALL>
__device__ __forceinline__ void load_chunks(Ch& d, const Rsrc& rs, int roff, bool rok, int lim, int nv, const Geo& G,
                                            const Lane& L) {
  constexpr int ES = esize_c<DT>();
#pragma unroll
  for (int j = 0; j < NVK; ++j) {
    const int ct = (j * G.g + L.lane) * VEC;
    const int off = lane_off(rok & (ct + VEC <= lim), (roff + ct) * ES);
    if constexpr (DT == DT_F32) {
      if (ALL || j < nv) {
        const u4 v0 = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, CP);
        const u4 v1 = __builtin_amdgcn_raw_buffer_load_b128(rs, off == OOB ? OOB : off + 16, 0, CP);
        d.c[j] = unpack_f32(v0, v1);
      } else {
        d.c[j] = skipped_chunk();
      }
    } else if constexpr (DT == DT_BF16) {
      if (ALL || j < nv) d.c[j] = unpack_bf16(__builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, CP));
      else d.c[j] = skipped_chunk();
    } else {
      const u2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, CP);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d.c[j][i] = (float)((v.x >> (8 * i)) & 0xffu);
        d.c[j][4 + i] = (float)((v.y >> (8 * i)) & 0xffu);
      }
    }
  }
}

template <uint32_t DT, int CP = CP_STREAM>
__device__ __forceinline__ void load_dir(Ch& d, const ArgD& a, const Geo& G, const Tile& tl, const Lane& L,
                                         bool any_row = false) {
  constexpr int ES = esize_c<DT>();
  const Rsrc rs = tile_rsrc(a, tl, ES);
  const int roff = L.row * (int)a.sr;  // a tile spans < 2^31 bytes (host checked)
  const bool rok = any_row | L.rok;
  if (a.sc == 0) {
    // broadcast along the row: one element per row
    const int off = lane_off(rok, roff * ES);
    float v;
    if constexpr (DT == DT_F32) v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
    else if constexpr (DT == DT_BF16) v = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
    else v = (float)__builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0);
    fill(d, v);
  } else if ((a.fl & AF_VEC) && a.sc == 1) {
    // dword-aligned chunks: 128-bit accesses for every chunk inside the
    // whole-chunk columns (the others are masked); a row-end chunk they do not
    // cover is completed element by element
    const int lim = chunk_cols(a, tl, ES, any_row ? (T_LANES >> G.lg) : tl.tre);
    const int nv = nv_pass(G);
    if (nv >= NVK) load_chunks<DT, CP, true>(d, rs, roff, rok, lim, nv, G, L);
    else load_chunks<DT, CP, false>(d, rs, roff, rok, lim, nv, G, L);
    if (lim < tl.tce) load_tail<DT>(d, rs, roff, G, tl, L, rok);
  } else {
    // element path: unaligned or strided operands
#pragma unroll
    for (int j = 0; j < NVK; ++j) {
      const int ct = (j * G.g + L.lane) * VEC;
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const int c = ct + i;
        const int off = lane_off(rok & (c < tl.tce), (roff + c * a.sc) * ES);
        float v;
        if constexpr (DT == DT_F32) v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
        else if constexpr (DT == DT_BF16) v = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
        else v = (float)__builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0);
        d.c[j][i] = v;
      }
    }
  }
}

template <int CP>
__device__ __forceinline__ void load_any_cp(Ch& d, const ArgD& a, const Geo& G, const Tile& tl, const Lane& L,
                                            bool any_row) {
  if (a.dt == DT_BF16) load_dir<DT_BF16, CP>(d, a, G, tl, L, any_row);
  else if (a.dt == DT_F32) load_dir<DT_F32, CP>(d, a, G, tl, L, any_row);
  else load_dir<DT_U8, CP>(d, a, G, tl, L, any_row);
}

__device__ __forceinline__ void load_any(Ch& d, const ArgD& a, const Geo& G, const Tile& tl, const Lane& L,
                                         bool stream, bool any_row = false) {
  if (stream) load_any_cp<CP_STREAM>(d, a, G, tl, L, any_row);
  else load_any_cp<0>(d, a, G, tl, L, any_row);
}

// The 128-bit chunk stores of store_dir: all chunks (ALL) or the first nv.
// The register comes by value: taken by reference from two instances, its
// chunks were kept in private memory instead of registers.
template <uint32_t DT, int CP, bool ALL>
__device__ __forceinline__ void store_chunks(const Ch s, const Rsrc& rs, int roff, int nv, const Geo& G,
                                             const Tile& tl, const Lane& L) {
  constexpr int ES = esize_c<DT>();
#pragma unroll
  for (int j = 0; j < NVK; ++j) {
    if (!ALL && j >= nv) continue;
    const int ct = (j * G.g + L.lane) * VEC;
    const int off = lane_off(L.rok & (ct + VEC <= tl.tce), (roff + ct) * ES);
    const V8 x = s.c[j];
    if constexpr (DT == DT_F32) {
      u4 v0, v1;
      v0.x = __float_as_uint(x[0]); v0.y = __float_as_uint(x[1]); v0.z = __float_as_uint(x[2]); v0.w = __float_as_uint(x[3]);
      v1.x = __float_as_uint(x[4]); v1.y = __float_as_uint(x[5]); v1.z = __float_as_uint(x[6]); v1.w = __float_as_uint(x[7]);
      __builtin_amdgcn_raw_buffer_store_b128(v0, rs, off, 0, CP);
      __builtin_amdgcn_raw_buffer_store_b128(v1, rs, off == OOB ? OOB : off + 16, 0, CP);
    } else if constexpr (DT == DT_BF16) {
      u4 v;
      v.x = f2bf_pack(x[0], x[1]);
      v.y = f2bf_pack(x[2], x[3]);
      v.z = f2bf_pack(x[4], x[5]);
      v.w = f2bf_pack(x[6], x[7]);
      __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, CP);
    } else {
      u2 v = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v.x |= ((uint32_t)x[i] & 0xffu) << (8 * i);
        v.y |= ((uint32_t)x[4 + i] & 0xffu) << (8 * i);
      }
      __builtin_amdgcn_raw_buffer_store_b64(v, rs, off, 0, CP);
    }
  }
}

template <uint32_t DT, int CP>
__device__ __forceinline__ void store_dir_cp(const Ch& s, const ArgD& a, const Geo& G, const Tile& tl,
                                             const Lane& L) {
  constexpr int ES = esize_c<DT>();
  const Rsrc rs = tile_rsrc(a, tl, ES);
  const int roff = L.row * (int)a.sr;
  if ((a.fl & AF_VEC) && a.sc == 1) {
    const int nv = nv_pass(G);
    if (nv >= NVK) store_chunks<DT, CP, true>(s, rs, roff, nv, G, tl, L);
    else store_chunks<DT, CP, false>(s, rs, roff, nv, G, tl, L);
    store_tail<DT>(s, rs, roff, G, tl, L);
  } else {
#pragma unroll
    for (int j = 0; j < NVK; ++j) {
      const int ct = (j * G.g + L.lane) * VEC;
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const int c = ct + i;
        const int off = lane_off(L.rok & (c < tl.tce), (roff + c * a.sc) * ES);
        const float v = s.c[j][i];
        if constexpr (DT == DT_F32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, off, 0, 0);
        else if constexpr (DT == DT_BF16)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(f2bf_pack(v, 0.f) & 0xffffu), rs, off, 0, 0);
        else __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, rs, off, 0, 0);
      }
    }
  }
}

template <uint32_t DT>
__device__ __forceinline__ void store_dir(const Ch& s, const ArgD& a, const Geo& G, const Tile& tl, const Lane& L,
                                          bool stream) {
  if (stream) store_dir_cp<DT, CP_STREAM>(s, a, G, tl, L);
  else store_dir_cp<DT, 0>(s, a, G, tl, L);
}

__device__ __forceinline__ void store_any(const Ch& v, const ArgD& a, const Geo& G, const Tile& tl, const Lane& L,
                                          bool stream) {
  if (a.dt == DT_BF16) store_dir<DT_BF16>(v, a, G, tl, L, stream);
  else if (a.dt == DT_F32) store_dir<DT_F32>(v, a, G, tl, L, stream);
  else store_dir<DT_U8>(v, a, G, tl, L, stream);
}

// ---------------------------------------------------------------------------
// LDS staging: next-tile prefetch (direct-to-LDS buffer loads) and
// LDS-resident tile-invariant operands.  A lane reads back only bytes that
// its own loads or stores put in LDS (or, for a shared invariant row, bytes
// that every lane of its column position wrote with the same values), so no
// barrier is needed, only waits on the lane's own outstanding operations.
// ---------------------------------------------------------------------------
// Issue the loads of tile nt of operand a into a prefetch slot (nv chunks).
// The direct-to-LDS loads are issued from inline assembly, so the compiler
// does not track them: it would otherwise make every later LDS read, and every
// instruction after a merge of paths, wait for all outstanding vector memory
// (the prefetch included).  Their completion is awaited explicitly, with the
// counted wait before the slot is read; waits the compiler places for its own
// loads stay correct (extra outstanding operations only make them stricter).
template <uint32_t DT, bool ALL>
__device__ __forceinline__ void pf_issue_n(char* slot, const ArgD& a, const Geo& G, const Tile& nt, const Lane& L,
                                           bool keep, int nv) {
  constexpr int ES = esize_c<DT>();
  constexpr int HV = DT == DT_F32 ? 2 : 1;
  const u4 rs = tile_rsrc_words(a, nt, ES);
  const bool rok = L.row < nt.tre;
  const int roff = L.row * (int)a.sr;
  const int wave = L.tid >> 6;
  const uint32_t base = (uint32_t)(uintptr_t)(lds_void*)slot;
  const int lim = chunk_cols(a, nt, ES, nt.tre);
#pragma unroll
  for (int j = 0; j < NVK; ++j) {
    if (ALL || j < nv) {
      // the tile's nv chunks; lanes past the tile's columns are masked (their
      // LDS bytes get zeros)
      const int ct = (j * G.g + L.lane) * VEC;
      const int off = lane_off(rok & (ct + VEC <= lim), (roff + ct) * ES);  // whole chunks only
#pragma unroll
      for (int h = 0; h < HV; ++h) {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(base + (uint32_t)(((j * HV + h) * T_LANES + wave * 64) * 16));
        const int o = off == OOB ? OOB : off + 16 * h;
        if (keep)
          asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                       :
                       : "s"(dst), "v"(o), "s"(rs)
                       : "memory", "m0");
        else
          asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                       :
                       : "s"(dst), "v"(o), "s"(rs)
                       : "memory", "m0");
      }
    }
  }
}

template <uint32_t DT>
__device__ __forceinline__ void pf_issue(char* slot, const ArgD& a, const Geo& G, const Tile& nt, const Lane& L,
                                         bool keep) {
  const int nv = nv_pass(G);
  if (nv >= NVK) pf_issue_n<DT, true>(slot, a, G, nt, L, keep, nv);
  else pf_issue_n<DT, false>(slot, a, G, nt, L, keep, nv);
}

template <uint32_t DT, bool ALL>
__device__ __forceinline__ void pf_read_n(Ch& d, const char* slot, int tid, int nv) {
  constexpr int HV = DT == DT_F32 ? 2 : 1;
#pragma unroll
  for (int j = 0; j < NVK; ++j) {
    // the slot's first nv chunks (the refill fills only those)
    if (!ALL && j >= nv) {
      d.c[j] = skipped_chunk();
      continue;
    }
    const int jj = j;
    const u4 v = *(const u4*)(slot + ((jj * HV) * T_LANES + tid) * 16);
    if constexpr (DT == DT_F32) {
      const u4 w = *(const u4*)(slot + ((jj * HV + 1) * T_LANES + tid) * 16);
      d.c[j] = unpack_f32(v, w);
    } else {
      d.c[j] = unpack_bf16(v);
    }
  }
}

template <uint32_t DT>
__device__ __forceinline__ void pf_read(Ch& d, const char* slot, const Geo& G, int tid) {
  const int nv = nv_pass(G);
  if (nv >= NVK) pf_read_n<DT, true>(d, slot, tid, nv);
  else pf_read_n<DT, false>(d, slot, tid, nv);
}

// Invariant slot addressing: a shared slot is indexed by the lane's position
// in its row (stride g), a lane-private one by the lane (stride T).  The slot
// holds 2 NVK planes of stride x 16 bytes: plane 2j + h carries elements
// 4h..4h+3 of every index's chunk j, so the 64 lanes of a wave touch 64
// consecutive 16-byte cells (no bank conflicts, and a direct-to-LDS load of
// one wave fills exactly the cells its lanes read back).
__device__ __forceinline__ int inv_base(KW* W, uint32_t k, const Geo& G, const Lane& L, int* stride) {
  const bool shared = W[H_INV_SHARED0 + k] != 0;
  *stride = shared ? G.g : T_LANES;
  return shared ? L.lane : L.tid;
}

__device__ __forceinline__ int inv_cell(int j, int h, int stride, int idx) { return ((2 * j + h) * stride + idx) * 16; }

__device__ __forceinline__ void inv_write(const Ch& c, char* slot, const Geo& G, int idx, int stride) {
#pragma unroll
  for (int j = 0; j < NVK; ++j) {
    {
      const V8 x = c.c[j];
      const f4 a = {x[0], x[1], x[2], x[3]};
      const f4 b = {x[4], x[5], x[6], x[7]};
      *(f4*)(slot + inv_cell(j, 0, stride, idx)) = a;
      *(f4*)(slot + inv_cell(j, 1, stride, idx)) = b;
    }
  }
}

// Stages an fp32 invariant operand whose columns are contiguous and whole
// chunks straight into its slot with direct-to-LDS loads (no registers, no
// wait here: the prologue ends with one wait for every load it issued).
// Needs each wave's indices to be 64 consecutive values: a lane-private slot,
// or a shared one whose rows span whole waves (g a multiple of 64).
__device__ __forceinline__ bool inv_direct_ok(const ArgD& a, const Geo& G, const Tile& tl, int stride) {
  return a.dt == DT_F32 && (a.fl & AF_VEC) && a.sc == 1 && (tl.tce & (VEC - 1)) == 0 &&
         (stride == T_LANES || (G.g & 63) == 0);
}

__device__ __forceinline__ void inv_issue(char* slot, const ArgD& a, const Geo& G, const Tile& tl, const Lane& L,
                                          int idx, int stride, bool any_row) {
  const u4 rs = tile_rsrc_words(a, tl, 4);
  const bool rok = any_row | L.rok;
  const int roff = L.row * (int)a.sr;
  // the wave's first index (its lanes hold it and the 63 after it)
  const int idx0 = __builtin_amdgcn_readfirstlane(idx);
  const uint32_t base = (uint32_t)(uintptr_t)(lds_void*)slot;
#pragma unroll
  for (int j = 0; j < NVK; ++j) {
    const int ct = (j * G.g + L.lane) * VEC;
    const int off = lane_off(rok & (ct + VEC <= tl.tce), (roff + ct) * 4);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t dst = __builtin_amdgcn_readfirstlane(base + (uint32_t)inv_cell(j, h, stride, idx0));
      const int o = off == OOB ? OOB : off + 16 * h;
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :
                   : "s"(dst), "v"(o), "s"(rs)
                   : "memory", "m0");
    }
  }
}

__device__ __forceinline__ void inv_read(Ch& c, const char* slot, const Geo& G, int idx, int stride) {
#pragma unroll
  for (int j = 0; j < NVK; ++j) {
    const int jj = j;
    const f4 a = *(const f4*)(slot + inv_cell(jj, 0, stride, idx));
    const f4 b = *(const f4*)(slot + inv_cell(jj, 1, stride, idx));
    V8 r;
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
    c.c[j] = r;
  }
}

// s_waitcnt vmcnt(n) for a wave-uniform n (0..63): the count is an immediate
// of the instruction, so a switch selects it.
#define DVM_VMC_CASE(n) case n: asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory"); break;
__device__ __forceinline__ void wait_vm(uint32_t n) {
  switch (n) {
    DVM_VMC_CASE(0) DVM_VMC_CASE(1) DVM_VMC_CASE(2) DVM_VMC_CASE(3) DVM_VMC_CASE(4) DVM_VMC_CASE(5)
    DVM_VMC_CASE(6) DVM_VMC_CASE(7) DVM_VMC_CASE(8) DVM_VMC_CASE(9) DVM_VMC_CASE(10) DVM_VMC_CASE(11)
    DVM_VMC_CASE(12) DVM_VMC_CASE(13) DVM_VMC_CASE(14) DVM_VMC_CASE(15) DVM_VMC_CASE(16) DVM_VMC_CASE(17)
    DVM_VMC_CASE(18) DVM_VMC_CASE(19) DVM_VMC_CASE(20) DVM_VMC_CASE(21) DVM_VMC_CASE(22) DVM_VMC_CASE(23)
    DVM_VMC_CASE(24) DVM_VMC_CASE(25) DVM_VMC_CASE(26) DVM_VMC_CASE(27) DVM_VMC_CASE(28) DVM_VMC_CASE(29)
    DVM_VMC_CASE(30) DVM_VMC_CASE(31) DVM_VMC_CASE(32) DVM_VMC_CASE(33) DVM_VMC_CASE(34) DVM_VMC_CASE(35)
    DVM_VMC_CASE(36) DVM_VMC_CASE(37) DVM_VMC_CASE(38) DVM_VMC_CASE(39) DVM_VMC_CASE(40) DVM_VMC_CASE(41)
    DVM_VMC_CASE(42) DVM_VMC_CASE(43) DVM_VMC_CASE(44) DVM_VMC_CASE(45) DVM_VMC_CASE(46) DVM_VMC_CASE(47)
    DVM_VMC_CASE(48) DVM_VMC_CASE(49) DVM_VMC_CASE(50) DVM_VMC_CASE(51) DVM_VMC_CASE(52) DVM_VMC_CASE(53)
    DVM_VMC_CASE(54) DVM_VMC_CASE(55) DVM_VMC_CASE(56) DVM_VMC_CASE(57) DVM_VMC_CASE(58) DVM_VMC_CASE(59)
    DVM_VMC_CASE(60) DVM_VMC_CASE(61) DVM_VMC_CASE(62)
    default: asm volatile("s_waitcnt vmcnt(63)" ::: "memory"); break;
  }
}
#undef DVM_VMC_CASE

// Per-workgroup context shared by the routines; slot addresses are
// re-derived from the header at each use (scalar loads) instead of being kept
// live across the interpreter loop.
struct Ctx {
  KW* W;
  char* lds;
  uint32_t tile, t_step, t_end;
  uint32_t alt;  // reduction buffer toggle: tile parity under HF_RED_ALT, else 0
  __device__ __forceinline__ char* pf(uint32_t k) const { return lds + W[H_PF_OFF0 + k]; }
  __device__ __forceinline__ char* inv(uint32_t k) const { return lds + W[H_INV_OFF0 + k]; }
};

// Read from prefetch slot `slot` (the tile was fetched while the previous one
// ran), then refill the slot with this workgroup's next tile (t_step on).
template <uint32_t DT>
__device__ __forceinline__ void read_pf(Ch& d, uint32_t w0, uint32_t vmc, const ArgD& a, const Geo& G,
                                        const Tile& tl, const Lane& L, const Ctx& S) {
  const uint32_t slot = f_b(w0) & 1u;
  // The count is a lower bound of the instructions issued after the
  // prefetch (ragged tiles issue more), so the wait covers the prefetch.
  wait_vm(vmc);
  pf_read<DT>(d, S.pf(slot), G, L.tid);
  // the prefetch moved whole chunks only: complete a row-end chunk they did
  // not cover
  if (chunk_cols(a, tl, esize_c<DT>(), tl.tre) < tl.tce)
    load_tail<DT>(d, tile_rsrc(a, tl, esize_c<DT>()), L.row * (int)a.sr, G, tl, L, L.rok);
  if ((f_flags(w0) & FL_ISSUE) && S.tile + S.t_step < S.t_end) {
    const Tile nt = make_tile(G, S.tile + S.t_step);
    // this lane's reads of the slot have completed before the refill starts
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    pf_issue<DT>(S.pf(slot), a, G, nt, L, !streaming(S.W));
  }
}

__device__ __forceinline__ void read_inv(Ch& d, uint32_t w0, const Geo& G, const Lane& L, const Ctx& S) {
  const uint32_t k = f_b(w0) & 1u;
  int stride;
  const int idx = inv_base(S.W, k, G, L, &stride);
  inv_read(d, S.inv(k), G, idx, stride);
}

// Memory operand of a compute instruction: invariant slot, prefetch slot or
// memory, in the operand's dtype.
__device__ __forceinline__ void read_mem(Ch& d, uint32_t w0, uint32_t vmc, const ArgD& a, const Geo& G,
                                         const Tile& tl, const Lane& L, const Ctx& S) {
  const uint32_t fl = f_flags(w0);
  if (fl & FL_INV) read_inv(d, w0, G, L, S);
  else if (fl & FL_PF) {
    if (a.dt == DT_F32) read_pf<DT_F32>(d, w0, vmc, a, G, tl, L, S);
    else read_pf<DT_BF16>(d, w0, vmc, a, G, tl, L, S);
  } else {
    load_any(d, a, G, tl, L, streaming(S.W));
  }
}

// ---------------------------------------------------------------------------
// Compute routines on tile registers
// ---------------------------------------------------------------------------
template <uint32_t OPK, bool REV>
__device__ __forceinline__ void bin_cc(Ch& acc, const Ch& b) {
#pragma unroll
  for (int j = 0; j < NVK; ++j)
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const float x = acc.c[j][i], y = b.c[j][i];
      acc.c[j][i] = REV ? alu<OPK>(y, x) : alu<OPK>(x, y);
    }
}

template <uint32_t OPK, bool REV>
__device__ __forceinline__ void bin_cs(Ch& acc, float s) {
#pragma unroll
  for (int j = 0; j < NVK; ++j)
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const float x = acc.c[j][i];
      acc.c[j][i] = REV ? alu<OPK>(s, x) : alu<OPK>(x, s);
    }
}

template <uint32_t F>
__device__ __forceinline__ void un_c(Ch& acc) {
#pragma unroll
  for (int j = 0; j < NVK; ++j)
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc.c[j][i] = una<F>(acc.c[j][i]);
}

// The same over the tile's first nv chunks only (nv wave-uniform: one scalar
// branch per chunk).  For the costly routines (transcendentals, divisions):
// chunks at or past nv hold columns past every row end, which reductions
// mask by column and stores skip, so they need no values.
template <uint32_t F>
__device__ __forceinline__ void un_cn(Ch& acc, int nv) {
#pragma unroll
  for (int j = 0; j < NVK; ++j) {
    if (j < nv) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc.c[j][i] = una<F>(acc.c[j][i]);
    }
  }
}

template <uint32_t OPK, bool REV>
__device__ __forceinline__ void bin_csn(Ch& acc, float s, int nv) {
#pragma unroll
  for (int j = 0; j < NVK; ++j) {
    if (j < nv) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const float x = acc.c[j][i];
        acc.c[j][i] = REV ? alu<OPK>(s, x) : alu<OPK>(x, s);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Cross-lane reductions: DPP and permlane swaps inside a wave, LDS across
// waves.
// ---------------------------------------------------------------------------
template <uint32_t KIND>
__device__ __forceinline__ float comb(float a, float b) {
  if constexpr (KIND == RK_SUM || KIND == RK_SUMSQ) return a + b;
  else return __builtin_elementwise_maximum(a, b);  // NaN-propagating
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Symmetric all-reduce over aligned groups of gs lanes (gs a power of two <=
// 64): DPP quad permutes and row mirrors inside 16 lanes, then the gfx950
// permlane16/permlane32 swaps across rows and wave halves.  Each step pairs
// every lane with one lane of the other half of its group.
template <uint32_t KIND>
__device__ __forceinline__ float group_reduce(float acc, int gs) {
  if (gs > 1) acc = comb<KIND>(acc, dpp<0xB1>(acc));   // quad_perm [1,0,3,2]
  if (gs > 2) acc = comb<KIND>(acc, dpp<0x4E>(acc));   // quad_perm [2,3,0,1]
  if (gs > 4) acc = comb<KIND>(acc, dpp<0x141>(acc));  // row_half_mirror
  if (gs > 8) acc = comb<KIND>(acc, dpp<0x140>(acc));  // row_mirror
  if (gs > 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(acc), __float_as_int(acc), false, false);
    acc = comb<KIND>(__int_as_float(p[0]), __int_as_float(p[1]));
  }
  if (gs > 32) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(acc), __float_as_int(acc), false, false);
    acc = comb<KIND>(__int_as_float(p[0]), __int_as_float(p[1]));
  }
  return acc;
}

// The reduce-all scalar from its n_part workgroup partials, computed by one
// wave in a fixed order: virtual lane t (of T_LANES) folds partials t,
// t + T_LANES, t + 2 T_LANES, ... in increasing order; each virtual wave of 64
// such lanes is combined by group_reduce; then the virtual waves in order.
// The combine launch and a branch program that folds the partials itself both
// take the scalar from here, so they agree bit for bit.  Every lane returns
// the result; all 64 lanes must be active.
// ONE: n_part <= 2 T_LANES, so the loop body runs once (straight-line code).
template <bool ONE = false>
__device__ __forceinline__ float fold_partials(const float* part, uint32_t n_part, uint32_t kind) {
  constexpr int VW = T_LANES / 64;
  const int lane = (int)(threadIdx.x & 63u);
  const Rsrc rp = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(part), 0, (int)(n_part * 4u), RSRC_W3);
  const float id = kind == RK_SUM ? 0.f : -__builtin_huge_valf();
  float acc[VW];
#pragma unroll
  for (int w = 0; w < VW; ++w) acc[w] = id;
  for (uint32_t i0 = 0; ONE ? i0 == 0 : i0 < n_part; i0 += 2u * T_LANES) {
    float v[2][VW];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int w = 0; w < VW; ++w) {
        const uint32_t i = i0 + (uint32_t)(j * T_LANES + 64 * w + lane);
        v[j][w] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, lane_off(i < n_part, (int)(i * 4u)), 0, 0));
      }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int w = 0; w < VW; ++w) {
        const bool ok = i0 + (uint32_t)(j * T_LANES + 64 * w + lane) < n_part;
        const float c = kind == RK_SUM ? acc[w] + v[j][w] : comb<RK_MAX>(acc[w], v[j][w]);
        acc[w] = ok ? c : acc[w];
      }
  }
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < VW; ++w) {
    const float rw = kind == RK_SUM ? group_reduce<RK_SUM>(acc[w], 64) : group_reduce<RK_MAX>(acc[w], 64);
    r = w == 0 ? rw : kind == RK_SUM ? r + rw : comb<RK_MAX>(r, rw);
  }
  return r;
}

// Partial over this lane's valid elements, combined as a balanced pairwise
// tree (a fixed order, so results are deterministic; short dependency
// chains).  Full tiles mask whole chunks; only ragged tiles mask element by
// element.
template <uint32_t KIND>
__device__ __forceinline__ float tree8(V8 v) {
  const float a = comb<KIND>(v[0], v[1]), b = comb<KIND>(v[2], v[3]);
  const float c = comb<KIND>(v[4], v[5]), d = comb<KIND>(v[6], v[7]);
  return comb<KIND>(comb<KIND>(a, b), comb<KIND>(c, d));
}

template <uint32_t KIND>
__device__ __forceinline__ V8 lane_terms(const V8& v) {
  if constexpr (KIND == RK_SUMSQ) return v * v;
  else return v;
}

template <uint32_t KIND>
__device__ __forceinline__ float lane_partial(const Ch& c, const Geo& G, const Tile& tl, const Lane& L) {
  const float id = KIND == RK_MAX ? -__builtin_huge_valf() : 0.f;
  float p[NVK];
  const int nv = nv_pass(G);
  if (tile_full(tl) && nv >= NVK) {
#pragma unroll
    for (int j = 0; j < NVK; ++j) {
      const int ct = (j * G.g + L.lane) * VEC;
      p[j] = lane_sel(L.rok & (ct < tl.tce), tree8<KIND>(lane_terms<KIND>(c.c[j])), id);
    }
  } else if (tile_full(tl)) {
#pragma unroll
    for (int j = 0; j < NVK; ++j) {
      const int ct = (j * G.g + L.lane) * VEC;
      p[j] = id;
      if (j < nv) p[j] = lane_sel(L.rok & (ct < tl.tce), tree8<KIND>(lane_terms<KIND>(c.c[j])), id);
    }
  } else {
    // only the row-end slot (wave-uniform) needs a mask per element
    const int jt = tail_of(G, tl).slot;
#pragma unroll
    for (int j = 0; j < NVK; ++j) {
      const int ct = (j * G.g + L.lane) * VEC;
      const V8 t = lane_terms<KIND>(c.c[j]);
      if (j == jt) {
        V8 m;
#pragma unroll
        for (int i = 0; i < VEC; ++i) m[i] = lane_sel(L.rok & (ct + i < tl.tce), t[i], id);
        p[j] = tree8<KIND>(m);
      } else {
        p[j] = lane_sel(L.rok & (ct < tl.tce), tree8<KIND>(t), id);
      }
    }
  }
  // balanced pairwise combine in a fixed order
#pragma unroll
  for (int w = 1; w < NVK; w *= 2)
#pragma unroll
    for (int j = 0; j + w < NVK; j += 2 * w) p[j] = comb<KIND>(p[j], p[j + w]);
  return p[0];
}

// ACC <- ACC pow B (B pow ACC if rev), one chunk at a time: the chunk in
// position 0 is computed and both registers rotate by one chunk, NVK times,
// so the long pow expansion appears once per routine instead of once per
// element.
__device__ __forceinline__ void pow_rot(Ch& acc, Ch& b, bool rev) {
#pragma nounroll
  for (int k = 0; k < NVK; ++k) {
    const V8 x = acc.c[0], y = b.c[0];
    V8 r;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const float u = rev ? y[i] : x[i], v = rev ? x[i] : y[i];
      r[i] = powf(u, v);
    }
#pragma unroll
    for (int j = 0; j < NVK - 1; ++j) {
      acc.c[j] = acc.c[j + 1];
      b.c[j] = b.c[j + 1];
    }
    acc.c[NVK - 1] = r;
    b.c[NVK - 1] = y;
  }
}

// One row-register instruction (RBIN / RUN).
__device__ __forceinline__ void row_op(RowRegs& rw, uint32_t w0, uint32_t w1) {
  if (f_op(w0) == HD_RBIN) {
    const float x = rget(rw, f_a(w0));
    const float y = f_bk(w0) == BK_RREG ? rget(rw, f_b(w0)) : __uint_as_float(w1);
    const bool rev = (f_flags(w0) & FL_REV) != 0;
    rset(rw, f_dst(w0), rev ? alu_rt(f_sub(w0), y, x) : alu_rt(f_sub(w0), x, y));
  } else {
    rset(rw, f_dst(w0), una_rt(f_sub(w0), rget(rw, f_a(w0))));
  }
}

// ---------------------------------------------------------------------------
// Register file of one lane: three tile registers and four row registers.
// ---------------------------------------------------------------------------
struct Regs {
  Ch t[TREGS];
  RowRegs rw;
};

// Tile register K (the wide build has only the accumulator: its encoder
// never names another register, and those handlers act on the accumulator)
template <int K>
__device__ __forceinline__ Ch& treg(Regs& r) {
  return r.t[K < TREGS ? K : 0];
}

}  // namespace

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
// The interpreter.  PROF = true builds the profiling twin: it reads the
// cycle counter around every dispatch and splits the workgroup's time into
// decode (instruction fetch, field decode and the dispatch to the handler),
// execute (the handler, row-register runs inside it included) and tile
// changes, written per workgroup at the end.  The product kernel is the
// PROF = false instance, with no counter reads.
// The program this workgroup runs and its place in that program's tiles:
// the first tile b and the stride grid (tiles b, b + grid, ... below
// block_dim).  The whole kernel argument, or in a spatially stacked launch the
// segment whose workgroup range holds blockIdx.x, with b and grid relative
// to that range (wave-uniform: every value comes from scalar loads).
struct Seg {
  KW* W;
  uint32_t b, grid;
};

// Temporally stacked launch: the segments' tiles form one space, numbered in
// segment order from the directory's tile bases; workgroup b runs the tiles
// b, b + G, b + 2G, ... of that space (G = gridDim.x), i.e. in segment s the
// local tiles congruent to b - base_s modulo G, segment after segment.
__device__ __forceinline__ Seg temporal_segment(KW* K, uint32_t s) {
  const uint32_t G = gridDim.x;
  const uint32_t base = K[S_DIR + 2 * s + 1] % G;
  return Seg{K + K[S_DIR + 2 * s], (blockIdx.x + G - base) % G, G};
}

__device__ __forceinline__ Seg segment_of() {
  KW* K = (KW*)__builtin_amdgcn_kernarg_segment_ptr();
  Seg g{K, blockIdx.x, gridDim.x};
  if (K[0] == STACK_MAGIC) {
    const uint32_t n = K[S_NSEG];
    uint32_t s = 0;
    for (uint32_t k = 1; k < n; ++k)
      if (blockIdx.x >= K[S_DIR + 2 * k + 1]) s = k;
    const uint32_t b0 = K[S_DIR + 2 * s + 1];
    const uint32_t b1 = s + 1 < n ? K[S_DIR + 2 * s + 3] : gridDim.x;
    g.W = K + K[S_DIR + 2 * s];
    g.b = blockIdx.x - b0;
    g.grid = b1 - b0;
  }
  return g;
}

template <bool PROF>
__device__ __forceinline__ void vm_main(const Seg& sg, float (*s_red)[T_LANES / 64], char* dlds) {
  KW* W = sg.W;
  uint64_t p_start = 0, p_top = 0, p_ent = 0, p_dec = 0, p_exe = 0, p_tile = 0, p_n = 0;
  if constexpr (PROF) p_start = __builtin_amdgcn_s_memtime();
#define PROF_ENTER() \
  if constexpr (PROF) p_ent = __builtin_amdgcn_s_memtime();
  const uint32_t block_dim = W[H_BLOCK_DIM];

  Geo G;
  G.g = (int)W[H_G];
  G.nv = (int)W[H_NV];
  G.tr = (int)W[H_TR];
  G.tc = (int)W[H_TC];
  G.nc = (int)W[H_NC];
  G.lg = 31 - __builtin_clz((uint32_t)G.g);
  G.R = (int64_t)w64(W, H_R_LO);
  G.C = (int64_t)w64(W, H_C_LO);
  const int tid = (int)threadIdx.x;
  const int gs = G.g < 64 ? G.g : 64;
  const int wave = tid >> 6;

  // Workgroup b runs tiles b, b + grid, b + 2 grid, ... (at most body_tile of
  // them): at any moment the resident workgroups work on neighbouring tiles,
  // so the streams they read and write advance together through memory.
  const uint32_t t_begin = sg.b;
  const uint32_t t_step = sg.grid;
  const uint32_t t_end = block_dim;

  Regs R;
#pragma unroll
  for (int k = 0; k < TREGS; ++k) fill(R.t[k], 0.f);
  R.rw = {0.f, 0.f, 0.f, 0.f};

  Ctx S;
  S.W = W;
  S.lds = dlds;
  S.t_step = t_step;
  S.t_end = t_end;
  S.alt = 0;
  const uint32_t alt_on = (W[H_FLAGS] & HF_RED_ALT) ? 2u : 0u;
  // reduce-all: each lane's running partial over the workgroup's tiles
  float all_acc = W[H_ALL_KIND] == RK_MAX ? -__builtin_huge_valf() : 0.f;

  // The body every tile runs.  A branch program reads its condition (a 0-d
  // fp32 operand written by an earlier launch on the stream) once, with a
  // wave-uniform load, and runs its else-body unless condition > threshold.
  // With HF_COND_FOLD the condition is a reduce-all whose combine this
  // program takes over: every wave folds the partials (operand
  // H_ALL_SCRATCH) itself, and workgroup 0 writes the scalar to the
  // condition operand, which no tile of this program reads.
  uint32_t body_begin = W[H_BODY_BEGIN], body_end = W[H_BODY_END];
  if (W[H_FLAGS] & HF_BRANCH) {
    const ArgD c = read_arg(W, W[H_COND_ARG]);
    const Rsrc rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(c.p), 0, 4, RSRC_W3);
    float v;
    if (W[H_FLAGS] & HF_COND_FOLD) {
      const ArgD pa = read_arg(W, W[H_ALL_SCRATCH]);
      // (readfirstlane moves 32-bit integers: the value crosses as its bits)
      v = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(
          fold_partials<true>(reinterpret_cast<const float*>(pa.p), (uint32_t)(pa.extent / 4u), W[H_ALL_KIND]))));
      // lane 0 of workgroup 0 stores (branch-free: the other lanes' offsets
      // are out of range, so their stores are dropped)
      if (sg.b == 0) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rc, lane_off(tid == 0, 0), 0, 0);
    } else {
      v = __uint_as_float(__builtin_amdgcn_readfirstlane(__builtin_amdgcn_raw_buffer_load_b32(rc, 0, 0, 0)));
    }
    if (!(v > __uint_as_float(W[H_COND_THR]))) {
      body_begin = W[H_ALT_BEGIN];
      body_end = W[H_ALT_END];
    }
  }

  Tile tl;
  uint32_t tile = t_begin;
  uint32_t pc = W[H_PRO_BEGIN], pc_end = W[H_PRO_END];
  bool in_pro = true;
  if (t_begin < t_end) {
    tl = make_tile(G, t_begin);
  } else {
    pc = pc_end = 0;
    in_pro = false;
    tile = t_end;
    tl = make_tile(G, 0);
  }
  // the next instruction's words, fetched one dispatch ahead (the encoder
  // leaves spare words after the body, so this never reads past the program)
  uint32_t nw0, nw1;
  fetch2(W, pc, nw0, nw1);

  // race-stress (profiling twin only): a seeded, wave-uniform delay per dispatch
  uint32_t stress = 0;
  if constexpr (PROF) {
    if (W[H_FLAGS] & HF_STRESS)
      stress = ((W[H_FLAGS] >> 8) * 0x9e3779b1u) ^ (sg.b * 0x85ebca6bu) ^
               (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 0xc2b2ae35u | 1u;
  }

  while (true) {
    if constexpr (PROF) {
      p_top = __builtin_amdgcn_s_memtime();
      if (stress) {
        stress ^= stress << 13;
        stress ^= stress >> 17;
        stress ^= stress << 5;
        for (uint32_t k = (stress >> 7) & 7u; k > 0; --k) __builtin_amdgcn_s_sleep(2);
      }
    }
    if (pc >= pc_end) {
      if (in_pro) {
        // the prologue's loads (direct-to-LDS invariant staging and the first
        // tile's prefetch) were issued back to back; one wait covers them all
        // before any body instruction reads a slot
        in_pro = false;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else {
        tile += t_step;
        S.alt ^= alt_on;  // this workgroup's next tile: the other reduction buffers
      }
      if (tile >= t_end) break;
      tl = make_tile(G, tile);
      pc = body_begin;
      pc_end = body_end;
      fetch2(W, pc, nw0, nw1);
      if constexpr (PROF) p_tile += __builtin_amdgcn_s_memtime() - p_top;
      continue;
    }
    const uint32_t w0 = nw0, w1 = nw1;
    pc += 2;
    // Fetch the next instruction only once this one's words have arrived:
    // scalar loads return out of order, so a wait for the current words
    // issued after the next fetch would also wait for that fetch.  The opaque
    // copy of pc makes the fetch address depend on the current words.
    uint32_t pcn = pc;
    asm volatile("" : "+s"(pcn) : "s"(w0), "s"(w1));
    fetch2(W, pcn, nw0, nw1);
    // Lane coordinates are recomputed per instruction (a few ALU ops) rather
    // than kept live across the whole interpreter loop.
    int tidv = tid;
    asm volatile("" : "+v"(tidv));
    Lane L;
    L.tid = tidv;
    L.row = tidv >> G.lg;
    L.lane = tidv & (G.g - 1);
    L.rok = L.row < tl.tre;
    S.tile = tile;

#define ARG read_arg(W, w1)
// Row-register instructions that follow run here, without going back
// through the dispatch.
#define ROW_RUN_TAIL()                                              \
  while (pc < pc_end && (f_op(nw0) == HD_RBIN || f_op(nw0) == HD_RUN)) { \
    const uint32_t a0 = nw0, a1 = nw1;                              \
    pc += 2;                                                        \
    uint32_t pcr = pc;                                              \
    asm volatile("" : "+s"(pcr) : "s"(a0), "s"(a1));                \
    fetch2(W, pcr, nw0, nw1);                                       \
    row_op(R.rw, a0, a1);                                           \
  }
#define CASE_LD(d)                                                                                          \
  case HD_LD_PF16 + d: PROF_ENTER() read_pf<DT_BF16>(treg<d>(R), w0, vmc_load(w0), ARG, G, tl, L, S); settle(treg<d>(R)); break; \
  case HD_LD_PF32 + d: PROF_ENTER() read_pf<DT_F32>(treg<d>(R), w0, vmc_load(w0), ARG, G, tl, L, S); settle(treg<d>(R)); break;  \
  case HD_LD_INV + d: PROF_ENTER() read_inv(treg<d>(R), w0, G, L, S); settle(treg<d>(R)); break;                          \
  case HD_BCAST + d: PROF_ENTER() fill(treg<d>(R), rget(R.rw, f_a(w0))); break;
#define CASE_COPY(d, a) \
  case HD_COPY + 3 * d + a: PROF_ENTER() treg<d>(R) = treg<a>(R); break;
#define SCALAR_B (f_bk(w0) == BK_IMM ? __uint_as_float(w1) : rget(R.rw, f_b(w0)))
#define CASE_BIN_DIR(k, rev)                                                                               \
  case HD_BIN + 10 * k + 5 * rev + BF_T0: PROF_ENTER() bin_cc<k, rev>(treg<0>(R), treg<0>(R)); break;                              \
  case HD_BIN + 10 * k + 5 * rev + BF_T1: PROF_ENTER() bin_cc<k, rev>(treg<0>(R), treg<1>(R)); break;                              \
  case HD_BIN + 10 * k + 5 * rev + BF_T2: PROF_ENTER() bin_cc<k, rev>(treg<0>(R), treg<2>(R)); break;                              \
  case HD_BIN + 10 * k + 5 * rev + BF_SCALAR: PROF_ENTER() bin_cs<k, rev>(treg<0>(R), SCALAR_B); break;
#define CASE_BIN_COMM(k) CASE_BIN_DIR(k, false)
#define CASE_BIN_NC(k) CASE_BIN_DIR(k, false) CASE_BIN_DIR(k, true)
#define CASE_ALL(kind, a)                                                                  \
  case HD_ALL + 3 * kind + a: PROF_ENTER()                                                  \
    /* reduce-all: the lane's running partial over this workgroup's tiles */                \
    all_acc = comb<kind>(all_acc, lane_partial<kind>(treg<a>(R), G, tl, L));               \
    break;
#define CASE_RED(kind, a) CASE_ALL(kind, a) CASE_RED_ROW(kind, a)
#define CASE_RED_ROW(kind, a)                                                              \
  case HD_RED + 3 * kind + a: PROF_ENTER()                                                              \
  case HD_REDX + 3 * kind + a: PROF_ENTER() {                                                           \
    const uint32_t h = f_op(w0);                                                           \
    float acc = lane_partial<kind>(treg<a>(R), G, tl, L);                                  \
    if (h == HD_RED + 3 * kind + a) {                                                      \
      /* rows inside one wave: the group all-reduce leaves the row's value */              \
      rset(R.rw, f_dst(w0), group_reduce<kind>(acc, gs));                                  \
      ROW_RUN_TAIL();                                                                      \
    } else {                                                                               \
      /* rows across waves: per-wave partial into LDS (after the 64-lane */                \
      /* all-reduce every lane holds it, so every lane stores it: no */                    \
      /* lane-dependent branch), barrier, then combine the row's partials */               \
      acc = group_reduce<kind>(acc, 64);                                                   \
      float* buf = s_red[f_b(w0) ^ S.alt];                                                 \
      buf[wave] = acc;                                                                     \
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");                                   \
      __builtin_amdgcn_s_barrier();                                                        \
      asm volatile("" ::: "memory");                                                       \
      const int nw = G.g >> 6;                                                             \
      const float* rb = buf + L.row * nw;                                                  \
      float r = rb[0];                                                                     \
      for (int k = 1; k < nw; ++k) r = comb<kind>(r, rb[k]);                               \
      rset(R.rw, f_dst(w0), r);                                                            \
      ROW_RUN_TAIL();                                                                      \
    }                                                                                      \
    break;                                                                                 \
  }

    switch (f_op(w0)) {
      CASE_LD(0) CASE_LD(1) CASE_LD(2)
      case HD_LD_DIR + 0: PROF_ENTER()
      case HD_LD_DIR + 1: PROF_ENTER()
      case HD_LD_DIR + 2: PROF_ENTER() {
        Ch m;
        load_any(m, ARG, G, tl, L, streaming(W));
        settle(m);
        if (f_dst(w0) == 0) treg<0>(R) = m;
        else if (f_dst(w0) == 1) treg<1>(R) = m;
        else treg<2>(R) = m;
        break;
      }
      case HD_ST_BF16: PROF_ENTER() store_dir<DT_BF16>(treg<0>(R), ARG, G, tl, L, streaming(W)); break;
      case HD_ST_F32: PROF_ENTER() store_dir<DT_F32>(treg<0>(R), ARG, G, tl, L, streaming(W)); break;
      case HD_ST_DIR + 0: PROF_ENTER() store_any(treg<0>(R), ARG, G, tl, L, streaming(W)); break;
      case HD_ST_DIR + 1: PROF_ENTER()
      case HD_ST_DIR + 2: PROF_ENTER() {
        Ch m;
        if (f_a(w0) == 1) m = treg<1>(R);
        else m = treg<2>(R);
        store_any(m, ARG, G, tl, L, streaming(W));
        break;
      }
      CASE_COPY(0, 1) CASE_COPY(0, 2) CASE_COPY(1, 0) CASE_COPY(1, 2) CASE_COPY(2, 0) CASE_COPY(2, 1)
      case HD_UN + UN_SQRT: PROF_ENTER() un_cn<UN_SQRT>(treg<0>(R), nv_pass(G)); break;
      case HD_UN + UN_ABS: PROF_ENTER() un_c<UN_ABS>(treg<0>(R)); break;
      case HD_UN + UN_LOG: PROF_ENTER() un_cn<UN_LOG>(treg<0>(R), nv_pass(G)); break;
      case HD_UN + UN_EXP: PROF_ENTER() un_cn<UN_EXP>(treg<0>(R), nv_pass(G)); break;
      case HD_UN + UN_ROUND: PROF_ENTER() un_c<UN_ROUND>(treg<0>(R)); break;
      case HD_UN + UN_FLOOR: PROF_ENTER() un_c<UN_FLOOR>(treg<0>(R)); break;
      case HD_UN + UN_ISFINITE: PROF_ENTER() un_c<UN_ISFINITE>(treg<0>(R)); break;
      case HD_UN + UN_NEG: PROF_ENTER() un_c<UN_NEG>(treg<0>(R)); break;
      case HD_UN + UN_RECIP: PROF_ENTER() un_cn<UN_RECIP>(treg<0>(R), nv_pass(G)); break;
      case HD_UN + UN_TOBF16: PROF_ENTER() un_c<UN_TOBF16>(treg<0>(R)); break;
      case HD_SILU: PROF_ENTER() un_cn<UN_SILU>(treg<0>(R), nv_pass(G)); break;
      case HD_SOFTMAX: PROF_ENTER() {
        // ACC <- softmax over its row (UN_SOFTMAX).  Rows inside a wave: the
        // chain's own steps (row max, subtract, exp, row sum, reciprocal,
        // multiply), bit for bit as the unfused program.  Rows across waves:
        // each wave's max m_w and sum s_w of exp(z - m_w) cross in one
        // exchange through buffers b and b + 1, then M = max m_k,
        // S = sum_k s_k exp(m_k - M) in wave order, and the wave scales its
        // exp(z - m_w) by exp(m_w - M) / S.  A wave whose elements are all
        // -inf subtracts 0 instead: its sum is 0 and exp(-inf - M) = 0 drops
        // it from S; a row with no finite maximum makes exp(-inf - (-inf))
        // NaN everywhere, as the chain does.  The row index and width are
        // made opaque so their products are formed here, not kept live
        // across the interpreter loop.
        const float ninf = -__builtin_huge_valf();
        const float mw = group_reduce<RK_MAX>(lane_partial<RK_MAX>(treg<0>(R), G, tl, L), gs);
        const bool across = G.g > 64;
        bin_csn<ALU_SUB, false>(treg<0>(R), across && mw == ninf ? 0.f : mw, nv_pass(G));
        un_cn<UN_EXP>(treg<0>(R), nv_pass(G));
        const float sw = group_reduce<RK_SUM>(lane_partial<RK_SUM>(treg<0>(R), G, tl, L), gs);
        float scale;
        if (!across) {
          scale = 1.f / sw;
        } else {
          float* bm = s_red[f_b(w0) ^ S.alt];
          float* bs = s_red[(f_b(w0) + 1) ^ S.alt];
          bm[wave] = mw;
          bs[wave] = sw;
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          int nw = G.g >> 6, rowv = L.row;
          asm volatile("" : "+v"(rowv), "+s"(nw));
          const float* rm = bm + rowv * nw;
          const float* rs = bs + rowv * nw;
          float M = rm[0];
          for (int k = 1; k < nw; ++k) M = comb<RK_MAX>(M, rm[k]);
          float S_row = 0.f;
          for (int k = 0; k < nw; ++k) S_row += rs[k] * __expf(rm[k] - M);
          scale = __expf(mw - M) / S_row;
        }
        bin_csn<ALU_MUL, false>(treg<0>(R), scale, nv_pass(G));
        // a store of the result that follows runs here, without going back
        // through the dispatch (the softmax body is read, softmax, store)
        if (f_op(nw0) == HD_ST_BF16 || f_op(nw0) == HD_ST_F32) {
          const uint32_t s0 = nw0, s1 = nw1;
          pc += 2;
          uint32_t pcs = pc;
          asm volatile("" : "+s"(pcs) : "s"(s0), "s"(s1));
          fetch2(W, pcs, nw0, nw1);
          if (f_op(s0) == HD_ST_BF16) store_dir<DT_BF16>(treg<0>(R), read_arg(W, s1), G, tl, L, streaming(W));
          else store_dir<DT_F32>(treg<0>(R), read_arg(W, s1), G, tl, L, streaming(W));
        }
        break;
      }
      CASE_BIN_COMM(ALU_ADD) CASE_BIN_NC(ALU_SUB) CASE_BIN_COMM(ALU_MUL)
      case HD_BIN + 10 * ALU_DIV + BF_SCALAR: PROF_ENTER() bin_cs<ALU_DIV, false>(treg<0>(R), SCALAR_B); break;
      case HD_BIN + 10 * ALU_DIV + BF_REV + BF_SCALAR: PROF_ENTER() bin_cs<ALU_DIV, true>(treg<0>(R), SCALAR_B); break;
      case HD_DIV_T: PROF_ENTER() {
        Ch b;
        if (f_b(w0) == 0) b = treg<0>(R);
        else if (f_b(w0) == 1) b = treg<1>(R);
        else b = treg<2>(R);
        if (f_flags(w0) & FL_REV) bin_cc<ALU_DIV, true>(treg<0>(R), b);
        else bin_cc<ALU_DIV, false>(treg<0>(R), b);
        break;
      }
      CASE_BIN_COMM(ALU_MAX) CASE_BIN_COMM(ALU_MIN)
      case HD_BIN_POW: PROF_ENTER() {
        Ch b;
        if (f_bk(w0) != BK_TREG) fill(b, SCALAR_B);
        else if (f_b(w0) == 0) b = treg<0>(R);
        else if (f_b(w0) == 1) b = treg<1>(R);
        else b = treg<2>(R);
        pow_rot(treg<0>(R), b, (f_flags(w0) & FL_REV) != 0);
        break;
      }
      case HD_FMA_INV: PROF_ENTER() {
        // (ACC * r) * inv[b] + inv[a], the last two in one rounding
        const float r = f_bk(w0) == BK_RREG ? rget(R.rw, f_dst(w0)) : 1.f;
        // chunk by chunk: the two invariant operands are read from LDS eight
        // values at a time (no tile-sized temporaries)
        int s1, s2;
        const uint32_t k1 = f_b(w0) & 1u, k2 = f_a(w0) & 1u;
        const int i1 = inv_base(W, k1, G, L, &s1), i2 = inv_base(W, k2, G, L, &s2);
        const char* b1 = S.inv(k1);
        const char* b2 = S.inv(k2);
#pragma unroll
        for (int j = 0; j < NVK; ++j) {
          const int jj = j;
          const f4 a0 = *(const f4*)(b1 + inv_cell(jj, 0, s1, i1)), a1 = *(const f4*)(b1 + inv_cell(jj, 1, s1, i1));
          const f4 c0 = *(const f4*)(b2 + inv_cell(jj, 0, s2, i2)), c1 = *(const f4*)(b2 + inv_cell(jj, 1, s2, i2));
          const float sc[VEC] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
          const float sh[VEC] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
          for (int i = 0; i < VEC; ++i) treg<0>(R).c[j][i] = __builtin_fmaf(treg<0>(R).c[j][i] * r, sc[i], sh[i]);
        }
        // a bf16 store of the result that follows runs here, without going
        // back through the dispatch (LayerNorm's body ends scale-and-shift,
        // store)
        if (f_op(nw0) == HD_ST_BF16) {
          const uint32_t s1 = nw1;
          pc += 2;
          uint32_t pcs = pc;
          asm volatile("" : "+s"(pcs) : "s"(s1));
          fetch2(W, pcs, nw0, nw1);
          store_dir<DT_BF16>(treg<0>(R), read_arg(W, s1), G, tl, L, streaming(W));
        }
        break;
      }
      case HD_BIN_MEM: PROF_ENTER() {
        Ch m;
        read_mem(m, w0, vmc_bin(w0), ARG, G, tl, L, S);
        const bool rev = (f_flags(w0) & FL_REV) != 0;
        switch (f_sub(w0)) {
          case ALU_ADD: bin_cc<ALU_ADD, false>(treg<0>(R), m); break;
          case ALU_SUB: if (rev) bin_cc<ALU_SUB, true>(treg<0>(R), m); else bin_cc<ALU_SUB, false>(treg<0>(R), m); break;
          case ALU_MUL: bin_cc<ALU_MUL, false>(treg<0>(R), m); break;
          case ALU_DIV: if (rev) bin_cc<ALU_DIV, true>(treg<0>(R), m); else bin_cc<ALU_DIV, false>(treg<0>(R), m); break;
          case ALU_MAX: bin_cc<ALU_MAX, false>(treg<0>(R), m); break;
          case ALU_MIN: bin_cc<ALU_MIN, false>(treg<0>(R), m); break;
          default: pow_rot(treg<0>(R), m, rev); break;
        }
        break;
      }
      CASE_RED(RK_SUM, 0) CASE_RED(RK_SUM, 1) CASE_RED(RK_SUM, 2)
      CASE_RED(RK_MAX, 0) CASE_RED(RK_MAX, 1) CASE_RED(RK_MAX, 2)
      CASE_RED_ROW(RK_SUMSQ, 0) CASE_RED_ROW(RK_SUMSQ, 1) CASE_RED_ROW(RK_SUMSQ, 2)
      case HD_SYNC: PROF_ENTER()
        // LDS exchange only: wait for this wave's LDS operations, then meet
        // the other waves (no wait on outstanding global loads, so prefetches
        // stay in flight across the barrier)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        break;
      case HD_RBIN: PROF_ENTER()
      case HD_RUN: PROF_ENTER()
        // a run of row-register instructions executes here
        row_op(R.rw, w0, w1);
        ROW_RUN_TAIL();
        break;
      case HD_LD_ROW: PROF_ENTER() {
        const ArgD a = ARG;
        const int es = esize(a.dt);
        const Rsrc rs = tile_rsrc(a, tl, es);
        const int off = lane_off(L.rok, L.row * (int)a.sr * es);
        float v;
        if (a.dt == DT_BF16) v = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
        else if (a.dt == DT_F32) v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
        else v = (float)__builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0);
        asm volatile("" : "+v"(v));  // settled before the routine returns
        rset(R.rw, f_dst(w0), v);
        break;
      }
      case HD_ST_ROW: PROF_ENTER() {
        const ArgD a = ARG;
        const int es = esize(a.dt);
        const Rsrc rs = tile_rsrc(a, tl, es);
        const int off = lane_off(L.rok & (L.lane == 0), L.row * (int)a.sr * es);
        const float v = rget(R.rw, f_a(w0));
        if (a.dt == DT_BF16) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(f2bf_pack(v, 0.f) & 0xffffu), rs, off, 0, 0);
        else if (a.dt == DT_F32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, off, 0, 0);
        else __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, rs, off, 0, 0);
        break;
      }
      case HD_DBG: PROF_ENTER() {
        const float v = f_sub(w0) == 0 ? (float)tl.id : (float)sg.b;
        if (f_dst(w0) == 0) fill(treg<0>(R), v);
        else if (f_dst(w0) == 1) fill(treg<1>(R), v);
        else fill(treg<2>(R), v);
        break;
      }
      case HD_LDS_INV: PROF_ENTER() {
        // prologue: the invariant operand's tile view, as fp32, into its slot
        const uint32_t k = f_dst(w0) & 1u;
        int stride;
        const int idx = inv_base(W, k, G, L, &stride);
        const ArgD a = ARG;
        if (inv_direct_ok(a, G, tl, stride)) {
          inv_issue(S.inv(k), a, G, tl, L, idx, stride, stride != T_LANES);
          break;
        }
        Ch tmp;
        load_any(tmp, a, G, tl, L, false, stride != T_LANES);  // reused by every tile: default policy
        // every chunk's load has returned before the handler ends, the ones
        // past nv (not written to LDS) included: a load left in flight would
        // make later writes of its registers wait on the vector-memory
        // counter, which also counts the prefetches
        settle(tmp);
        inv_write(tmp, S.inv(k), G, idx, stride);
        break;
      }
      case HD_PF: PROF_ENTER() {
        // prologue: fetch the workgroup's first tile into the prefetch slot
        const ArgD a = ARG;
        const bool keep = !streaming(W);
        if (a.dt == DT_F32) pf_issue<DT_F32>(S.pf(f_b(w0) & 1u), a, G, tl, L, keep);
        else pf_issue<DT_BF16>(S.pf(f_b(w0) & 1u), a, G, tl, L, keep);
        break;
      }
      default:
        PROF_ENTER()
        break;
    }
    if constexpr (PROF) {
      const uint64_t t = __builtin_amdgcn_s_memtime();
      p_dec += p_ent - p_top;
      p_exe += t - p_ent;
      ++p_n;
    }
#undef ARG
#undef CASE_LD
#undef CASE_COPY
#undef SCALAR_B
#undef CASE_BIN_DIR
#undef CASE_BIN_COMM
#undef CASE_BIN_NC
#undef CASE_RED
  }

  // Reduce-all epilogue: each workgroup stores one partial (its lanes'
  // running partials, each over the workgroup's tiles in order, combined
  // across the wave, then the waves in order).  The combine of the partials
  // is a second launch on the same stream (dvm_allreduce_combine), so no
  // workgroup waits for or publishes to another inside this one.
  if (W[H_TEMPLATE] == TM_ALLREDUCE) {
    const uint32_t kind = W[H_ALL_KIND];
    const ArgD sa = read_arg(W, W[H_ALL_SCRATCH]);
    float* part = reinterpret_cast<float*>(const_cast<char*>(sa.p) + 256);
    {
      const float wv = kind == RK_SUM ? group_reduce<RK_SUM>(all_acc, 64) : group_reduce<RK_MAX>(all_acc, 64);
      if ((tid & 63) == 0) s_red[0][wave] = wv;
    }
    __syncthreads();
    if (tid == 0) {
      float r = s_red[0][0];
      for (int k = 1; k < T_LANES / 64; ++k) r = kind == RK_SUM ? r + s_red[0][k] : comb<RK_MAX>(r, s_red[0][k]);
      // partials never go past the area the launch supplied
      const Rsrc rw = __builtin_amdgcn_make_buffer_rsrc(part, 0, (int)part_bytes(sa.extent, sg.grid), RSRC_W3);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(r), rw, (int)(sg.b * 4u), 0, 0);
    }
  }
  if constexpr (PROF) {
    // five counters per workgroup: total, decode, execute, tile-change
    // cycles, dispatches (wave 0's view; the waves run in lockstep per tile)
    const uint64_t total = __builtin_amdgcn_s_memtime() - p_start;
    if (tid == 0) {
      uint64_t* c = reinterpret_cast<uint64_t*>(w64(W, H_PROF_LO)) + (size_t)blockIdx.x * 5;
      c[0] = total;
      c[1] = p_dec;
      c[2] = p_exe;
      c[3] = p_tile;
      c[4] = p_n;
    }
  }
#undef PROF_ENTER
}

// Cross-wave reduction buffers and the reduce-all flag: a reserved part of
// each program's dynamic area (its offset is a header word, so it is looked up
// per segment), present only in programs whose reductions cross waves.
#define DVM_LDS_DECL extern __shared__ __attribute__((aligned(16))) char dlds[];
#define DVM_RED_PTRS(W)                                                                                \
  const uint32_t red_off = (W)[H_RED_OFF];                                                             \
  float(*s_red)[T_LANES / 64] = reinterpret_cast<float(*)[T_LANES / 64]>(dlds + red_off);
constexpr uint32_t LDS_CAP = LDS_BUDGET;

// One workgroup's run: its program (or its segment of a spatial stack), or
// every segment of a temporal stack in order, with a workgroup barrier
// between segments (the next segment's prologue rewrites LDS slots that waves
// still on the previous one may be reading).  One call site of the
// interpreter, so its code appears once per kernel.
template <bool PROF>
__device__ __forceinline__ void vm_kernel() {
  KW* K = (KW*)__builtin_amdgcn_kernarg_segment_ptr();
  DVM_LDS_DECL
  const bool temporal = K[0] == TSTACK_MAGIC;
  const uint32_t n = temporal ? K[S_NSEG] : 1u;
  for (uint32_t s = 0; s < n; ++s) {
    const Seg sg = temporal ? temporal_segment(K, s) : segment_of();
    DVM_RED_PTRS(sg.W)
    vm_main<PROF>(sg, s_red, dlds);
    if (temporal) __syncthreads();
  }
}

extern "C" __global__ void __launch_bounds__(T_LANES) __attribute__((amdgpu_waves_per_eu(2, 2)))
DVM_SYM(dvm_vm_vector)(const Program prog) {
  (void)prog;
  vm_kernel<false>();
}

// Profiling twin of dvm_vm_vector: same program, same results, plus the
// per-workgroup cycle split at the address in header words H_PROF_LO/HI.
extern "C" __global__ void __launch_bounds__(T_LANES) __attribute__((amdgpu_waves_per_eu(2, 2)))
DVM_SYM(dvm_vm_vector_prof)(const Program prog) {
  (void)prog;
  vm_kernel<true>();
}

#ifndef DVM_WIDE
// Reduce-all combine: the second launch of a reduce-all program, after the VM
// kernel on the same stream (the stream orders the workgroups' partials
// before it).  One wave folds the n_part partials in fold_partials' fixed
// order, so the result is the same in every run, and writes the scalar
// output.
extern "C" __global__ void __launch_bounds__(64)
dvm_allreduce_combine(const float* part, uint32_t n_part, uint32_t kind, void* out, uint32_t out_dt) {
  const float r = fold_partials(part, n_part, kind);
  if (threadIdx.x == 0) {
    if (out_dt == DT_BF16) *static_cast<uint16_t*>(out) = (uint16_t)(f2bf_pack(r, 0.f) & 0xffffu);
    else *static_cast<float*>(out) = r;
  }
}

extern "C" hipError_t dvm_launch_allreduce_combine(const float* part, uint32_t n_part, uint32_t kind, void* out,
                                                   uint32_t out_dt, hipStream_t s) {
  hipLaunchKernelGGL(dvm_allreduce_combine, dim3(1), dim3(64), 0, s, part, n_part, kind, out, out_dt);
  return hipGetLastError();
}
#endif

// Host-side launch of the VECTOR VM kernel with one program as its argument.
extern "C" hipError_t DVM_SYM(dvm_launch_vector_kernel)(const Program* p, unsigned grid, unsigned lds, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)DVM_SYM(dvm_vm_vector), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)LDS_CAP);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(DVM_SYM(dvm_vm_vector), dim3(grid), dim3(T_LANES), lds, s, *p);
  return hipGetLastError();
}

extern "C" hipError_t DVM_SYM(dvm_launch_vector_prof_kernel)(const Program* p, unsigned grid, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)DVM_SYM(dvm_vm_vector_prof),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_CAP);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(DVM_SYM(dvm_vm_vector_prof), dim3(grid), dim3(T_LANES), p->w[H_LDS_BYTES], s, *p);
  return hipGetLastError();
}
