// The resident VM kernel for MIX programs (the MATMUL template) on gfx950.
//
// A MIX program is a matmul A[M, K] x B[K, N] (bf16 inputs, fp32
// accumulation) followed by elementwise instructions on its [M, N] output,
// the cube-vector fusion of the DVM paper review page (section 5.1: the
// matmul result stays in local memory and the vector instructions consume it
// there).  Each workgroup computes its range of output tiles (the header's
// block_dim / body_tile, section 4.4); per tile it runs the whole K loop on
// the matrix cores and then interprets the program body on the accumulator.
//
// Tile: 128 x 128 outputs per 256-lane workgroup (the body is templated on
// the wave tile); the four waves own 64 x 64 quadrants, each as 2 x 2 blocks
// of v_mfma_f32_32x32x16_bf16.  Lane layout of
// that instruction (checked on the device): lane l supplies A[l % 32][8 (l /
// 32) + j] and B[8 (l / 32) + j][l % 32] for j < 8, and holds
// D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32] in accumulator register i.
//
// K runs in stages of MM_KT through a ring of LDS stages filled by
// direct-to-LDS buffer loads (no register staging), each slot refilled as
// soon as every wave is done with it; A is stored row-major and read with
// one 128-bit LDS load per lane and block, B is stored row-major too and read
// with transposing LDS loads, which give each lane its eight consecutive K
// values of one column.
//
// The epilogue (the program body) runs on the output tile staged in LDS as
// fp32, one row-major chunk of 8 columns per lane at a time, with three
// 8-value tile registers (register 0 starts as the chunk of the matmul
// result); memory operands and stores address element (m, n) of the [M, N]
// space through buffer resources, out-of-range offsets masking the edges.
//
// Tile order: a workgroup takes every grid-th tile of a grouped order (eight
// row tiles, walked column by column), starting from an XCD-aware slot, so
// the tiles in flight on one XCD at a time form an 8 x 8 block and share
// their A and B panels through that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bytecode.h"

using namespace dvmbc;

namespace {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef const __attribute__((address_space(4))) uint32_t KW;

constexpr int OOB = 0x7fffffff;
constexpr int RSRC_W3 = 0x00020000;

struct ArgD {
  const char* p;
  uint32_t dt, fl;
  int64_t sr;
  int32_t sc;
  uint64_t extent;
};

__device__ __forceinline__ uint64_t w64(KW* w, int lo) { return ((uint64_t)w[lo + 1] << 32) | (uint64_t)w[lo]; }

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

__device__ __forceinline__ int esize(uint32_t dt) { return dt == DT_F32 ? 4 : dt == DT_BF16 ? 2 : 1; }

// Descriptor from byte offset ob of the operand to its end (capped).
__device__ __forceinline__ Rsrc rsrc_at(const ArgD& a, int64_t ob) {
  const int64_t left = (int64_t)a.extent - ob;
  const int n = left <= 0 ? 0 : (left >= (int64_t)EXTENT_CAP ? (int)(EXTENT_CAP - 1) : (int)left);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a.p + ob), 0, n, RSRC_W3);
}

__device__ __forceinline__ int lane_off(bool ok, int off) { return ok ? off : OOB; }

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ uint32_t f2bf_pack(float lo, float hi) {
  f2 v = {lo, hi};
  bf2 b = __builtin_convertvector(v, bf2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, b);
}
__device__ __forceinline__ float round_bf16(float x) { return bf2f(f2bf_pack(x, 0.f) & 0xffffu); }

// Division in MIX epilogues: x times the hardware reciprocal of y (v_rcp_f32,
// within 1 ulp), within 2 fp32 ulp of the correctly rounded quotient, two
// instructions instead of about ten.  MatMul graphs are held to 1e-2 relative
// error, far above this.
__device__ __forceinline__ float div_mix(float x, float y) { return x * __builtin_amdgcn_rcpf(y); }

__device__ __forceinline__ float alu_rt(uint32_t k, float x, float y) {
  switch (k) {
    case ALU_ADD: return x + y;
    case ALU_SUB: return x - y;
    case ALU_MUL: return x * y;
    case ALU_DIV: return div_mix(x, y);
    case ALU_MAX: return __builtin_elementwise_maximum(x, y);  // NaN-propagating
    case ALU_MIN: return __builtin_elementwise_minimum(x, y);
    default: return powf(x, y);
  }
}

__device__ __forceinline__ float una_rt(uint32_t f, float x) {
  switch (f) {
    case UN_SQRT: return sqrtf(x);
    case UN_ABS: return fabsf(x);
    case UN_LOG: return logf(x);
    case UN_EXP: return __expf(x);  // v_exp_f32 of x log2(e)
    case UN_ROUND: return rintf(x);
    case UN_FLOOR: return floorf(x);
    case UN_ISFINITE: return isfinite(x) ? 1.f : 0.f;
    case UN_NEG: return -x;
    case UN_RECIP: return 1.f / x;
    case UN_TOBF16: return round_bf16(x);
    case UN_SILU: return div_mix(x, __expf(-x) + 1.f);  // a fused SiLU chain: its own operations, in order
    default: return x;
  }
}

// ---------------------------------------------------------------------------
// Variants
// ---------------------------------------------------------------------------
// WM x WN waves, each owning BM x BN blocks of 32 x 32 outputs; a ring of NS
// stages of KT values of K; the output tile staged for the epilogue in NSL slabs; U chunks of 8
// columns per lane and epilogue round.
template <int WM_, int WN_, int BM_, int BN_, int KT_, int NS_, int NSL_, int U_>
struct Cfg {
  static constexpr int WM = WM_, WN = WN_, BM = BM_, BN = BN_, KT = KT_, NS = NS_, NSL = NSL_, U = U_;
  static constexpr int SPS = KT / 16;                            // 16-deep steps per stage
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int TM = 32 * BM * WM, TN = 32 * BN * WN;     // workgroup tile
  static constexpr int UA = KT / 8, UB = TN / 8;                // 16-byte units per A row, per B row
  static constexpr int A_BYTES = TM * KT * 2, B_BYTES = KT * TN * 2, STAGE = A_BYTES + B_BYTES;
  static constexpr int QA = A_BYTES / (NT * 16), QB = B_BYTES / (NT * 16), Q = QA + QB;  // loads per lane
  static constexpr int IB = BM / NSL;    // block rows per wave in one slab
  static constexpr int PR = TM / NSL;    // rows per slab
  static constexpr int OSTR = TN + MM_OPAD;
  static constexpr int RING = NS * STAGE, SLAB = PR * OSTR * 4;
  static constexpr int LDS = RING > SLAB ? RING : SLAB;
  static constexpr int LPR = TN / 8;     // epilogue lanes per row
  static constexpr int RPP = NT / LPR;   // rows per chunk pass
  static constexpr int SP = PR / RPP;    // chunk passes per slab
  static_assert(A_BYTES % (NT * 16) == 0 && B_BYTES % (NT * 16) == 0, "whole loads per lane");
  static_assert(UB >= 16, "B swizzle needs 16 units per row");
  static_assert(BM % NSL == 0 && SP % U == 0 && SP >= 1, "slab geometry");
  static_assert(KT % 32 == 0 && NS >= 2, "an even number of steps per stage, two stages at least");
};

// ---------------------------------------------------------------------------
// K loop
// ---------------------------------------------------------------------------
// LDS ring of NS stages of KT values of K.  A stage holds
//  * A as TM rows of KT bf16 (KT / 8 16-byte units per row), unit kc of row r
//    stored at position kc ^ a_swz(r): the 16 rows read together by a quarter
//    wave (same kc) then cover all 64 banks;
//  * B row-major as KT rows of TN bf16 (TN / 8 units per row), unit cc of row
//    k stored at position cc ^ 4 (k & 3): the four rows read together by a
//    16-lane group of a transposing read land on disjoint banks.
// Both are written by direct-to-LDS buffer loads (lane i of a wave writes the
// 16 bytes at M0 + 16 i), so the swizzle is applied by choosing which global
// unit each lane fetches.  Out-of-range units (rows past M, columns past N,
// K past its end) read as zeros.
//
// Fragments: A as one 128-bit read per block (row l % 32, K unit 2 kk + l /
// 32); B with two transposing reads (ds_read_b64_tr_b16).  Within each group
// of 16 lanes such a read hands lane 4a + b the element b of the 8-byte words
// read by lanes a, a + 4, a + 8 and a + 12 (checked on the device), so lanes
// a + 4c reading row k0 + c at columns 4a .. 4a + 3 give lane 4a + b column
// 4a + b at K = k0 .. k0 + 3, the B operand layout of the matrix instruction.
typedef short s4 __attribute__((ext_vector_type(4)));
typedef short s8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s4 lds_s4;
typedef __attribute__((address_space(3))) void lds_void;

// A: the rows sharing a 256-byte bank line differ in the swizzle
template <int UA>
__device__ __forceinline__ int a_swz(int r) { return (r / (16 / UA)) & (UA - 1); }

__device__ __forceinline__ void dma16(uint32_t lds_dst, int voff, const u4& rs) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_dst), "v"(voff), "s"(rs)
               : "memory", "m0");
}

// Waits until at most N of this lane's direct-to-LDS loads are in flight.
template <int N>
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

__device__ __forceinline__ u4 rsrc_words(const ArgD& a, int64_t ob) {
  const int64_t left = (int64_t)a.extent - ob;
  const int n = left <= 0 ? 0 : (left >= (int64_t)EXTENT_CAP ? (int)(EXTENT_CAP - 1) : (int)left);
  const uint64_t base = (uint64_t)(uintptr_t)(a.p + ob);
  u4 r;
  r.x = (uint32_t)base;
  r.y = (uint32_t)(base >> 32) & 0xffffu;  // stride 0
  r.z = (uint32_t)n;
  r.w = (uint32_t)RSRC_W3;
  return r;
}

struct Panels {
  u4 ra, rb;          // A from row m0, B from column n0
  int64_t m0, n0;
};

// Issue the direct-to-LDS loads of stage s (K from s KT) into ring slot `slot`.
template <class CF>
__device__ __forceinline__ void issue_stage(uint32_t ring, int slot, int s, const Panels& P, const ArgD& A,
                                            const ArgD& B, int64_t M, int64_t N, int K, int wave, int lane) {
  const uint32_t base = ring + (uint32_t)(slot * CF::STAGE);
  const int k0 = s * CF::KT;
#pragma unroll
  for (int q = 0; q < CF::QA; ++q) {
    const int u = (q * CF::NW + wave) * 64 + lane;    // unit written by this lane
    const int r = u / CF::UA, pos = u % CF::UA;
    const int kc = pos ^ a_swz<CF::UA>(r);
    const bool ok = (P.m0 + r < M) & (k0 + kc * 8 < K);
    dma16(__builtin_amdgcn_readfirstlane(base + (uint32_t)((q * CF::NW + wave) * 64 * 16)),
          lane_off(ok, (r * (int)A.sr + k0 + kc * 8) * 2), P.ra);
  }
#pragma unroll
  for (int q = 0; q < CF::QB; ++q) {
    const int u = (q * CF::NW + wave) * 64 + lane;
    const int k = u / CF::UB, pos = u % CF::UB;
    const int cc = pos ^ ((k & 3) << 2);
    const bool ok = (k0 + k < K) & (P.n0 + cc * 8 < N);
    dma16(__builtin_amdgcn_readfirstlane(base + (uint32_t)(CF::A_BYTES + (q * CF::NW + wave) * 64 * 16)),
          lane_off(ok, ((k0 + k) * (int)B.sr + cc * 8) * 2), P.rb);
  }
}

// Fragments of one 16-deep step of K for this wave's BM x BN blocks.
template <class CF>
struct Frag {
  bf8 a[CF::BM], b[CF::BN];
};

// LDS reads of step kk of the stage at bytes `st`.
template <class CF>
__device__ __forceinline__ void load_frag(Frag<CF>& f, const char* st, int kk, int wm, int wn, int lane) {
  const char* abuf = st;
  const char* bbuf = st + CF::A_BYTES;
  const int g = lane >> 4, p = lane & 15;
#pragma unroll
  for (int i = 0; i < CF::BM; ++i) {
    const int r = wm * 32 * CF::BM + i * 32 + (lane & 31);
    const int kc = kk * 2 + (lane >> 5);
    f.a[i] = *(const bf8*)(abuf + (r * CF::UA + (kc ^ a_swz<CF::UA>(r))) * 16);
  }
#pragma unroll
  for (int j = 0; j < CF::BN; ++j) {
    const int k = kk * 16 + 8 * (g >> 1) + (p >> 2);
    const int n = wn * 32 * CF::BN + j * 32 + 16 * (g & 1) + 4 * (p & 3);
    const int off = (k * CF::UB + ((n >> 3) ^ ((k & 3) << 2))) * 16 + ((n >> 2) & 1) * 8;
    const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(lds_void*)(bbuf + off));
    const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(lds_void*)(bbuf + off + 4 * CF::UB * 16));
    const s8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    f.b[j] = __builtin_bit_cast(bf8, v);
  }
}

template <class CF>
__device__ __forceinline__ void mma(f16v (&c)[CF::BM][CF::BN], const Frag<CF>& f) {
#pragma unroll
  for (int i = 0; i < CF::BM; ++i)
#pragma unroll
    for (int j = 0; j < CF::BN; ++j)
      c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], c[i][j], 0, 0, 0);
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Epilogue: the program body on the tile, staged in LDS
// ---------------------------------------------------------------------------
// After the K loop the accumulators go to LDS as fp32, one slab of TM / NSL
// rows at a time (slab s holds block rows s IB .. s IB + IB - 1 of every
// wave, so each slab frees accumulator registers); slab rows are padded by
// MM_OPAD floats so the two half-waves of a write hit disjoint banks.  The
// body then runs on row-major chunks of 8 columns, U chunks per lane at a
// time: 128-bit LDS reads, and 128-bit global accesses for operands whose
// chunks are contiguous and dword aligned.  N is a multiple of 8, so a chunk
// is wholly inside or wholly outside the output.  Memory operands that do not
// vary along M (row stride 0, such as a bias row) are loaded once per tile
// into registers, before the K loop, for up to two such operands.
template <int U>
struct TV {
  float v[8 * U];
};

template <int U>
struct Round {
  int64_t m0, n0;  // tile origin in [M, N]
  uint32_t tile;   // row-major tile id (row tile * column tiles + column tile)
  int r[U];        // chunk rows inside the tile
  int c8;          // first column of this lane's chunks inside the tile
  bool ok[U];      // chunk inside [M, N]
};

struct Inv {
  int arg0, arg1;  // operands held in registers (-1: none)
  float v0[8], v1[8];
};

__device__ __forceinline__ u4 ld128(const Rsrc& rs, int off) { return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0); }

// 8 values from dword-aligned contiguous bytes at `off` (dtype dt).
__device__ __forceinline__ void vec_load8(float* d, const Rsrc& rs, uint32_t dt, bool ok, int off) {
  if (dt == DT_F32) {
    const u4 x = ld128(rs, lane_off(ok, off)), y = ld128(rs, lane_off(ok, off + 16));
    d[0] = __uint_as_float(x.x); d[1] = __uint_as_float(x.y); d[2] = __uint_as_float(x.z); d[3] = __uint_as_float(x.w);
    d[4] = __uint_as_float(y.x); d[5] = __uint_as_float(y.y); d[6] = __uint_as_float(y.z); d[7] = __uint_as_float(y.w);
  } else if (dt == DT_BF16) {
    const u4 x = ld128(rs, lane_off(ok, off));
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      d[2 * j] = bf2f(w[j] & 0xffffu);
      d[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  } else {
    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b32(rs, lane_off(ok, off), 0, 0);
    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b32(rs, lane_off(ok, off + 4), 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      d[j] = (float)((lo >> (8 * j)) & 0xffu);
      d[4 + j] = (float)((hi >> (8 * j)) & 0xffu);
    }
  }
}

// 8 values at element stride sc from `off`.
__device__ __forceinline__ void elem_load8(float* d, const Rsrc& rs, uint32_t dt, bool ok, int off, int step) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int o = lane_off(ok, off + j * step);
    if (dt == DT_BF16) d[j] = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rs, o, 0, 0));
    else if (dt == DT_F32) d[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, o, 0, 0));
    else d[j] = (float)__builtin_amdgcn_raw_buffer_load_b8(rs, o, 0, 0);
  }
}

// The 8 values of operand a at row r (inside the tile), this lane's columns.
__device__ __forceinline__ void chunk_load(float* d, const ArgD& a, int64_t m0, int64_t n0, int r, int c8, bool ok) {
  const int es = esize(a.dt);
  const Rsrc rs = rsrc_at(a, (m0 * a.sr + n0 * (int64_t)a.sc) * es);
  const int base = (r * (int)a.sr + c8 * a.sc) * es;
  if ((a.fl & AF_VEC) && a.sc == 1) vec_load8(d, rs, a.dt, ok, base);
  else elem_load8(d, rs, a.dt, ok, base, a.sc * es);
}

template <int U>
__device__ __forceinline__ void epi_load(TV<U>& d, uint32_t ai, KW* W, const Round<U>& C, const Inv& I) {
  if ((int)ai == I.arg0 || (int)ai == I.arg1) {
    const bool first = (int)ai == I.arg0;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) d.v[8 * u + e] = first ? I.v0[e] : I.v1[e];
    return;
  }
  const ArgD a = read_arg(W, ai);
#pragma unroll
  for (int u = 0; u < U; ++u) chunk_load(d.v + 8 * u, a, C.m0, C.n0, C.r[u], C.c8, C.ok[u]);
}

// Output stores take the cache policy CP: non-temporal (2) for programs
// flagged HF_STREAM, whose output no cache level keeps for a later launch
// and would otherwise push out the A and B panels the tiles share.
template <int U, int CP>
__device__ __forceinline__ void epi_store(const TV<U>& s, const ArgD& a, const Round<U>& C) {
  const int es = esize(a.dt);
  const Rsrc rs = rsrc_at(a, (C.m0 * a.sr + C.n0 * (int64_t)a.sc) * es);
  const bool vec = (a.fl & AF_VEC) && a.sc == 1;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float* x = s.v + 8 * u;
    const int base = (C.r[u] * (int)a.sr + C.c8 * a.sc) * es;
    const bool ok = C.ok[u];
    if (vec) {
      if (a.dt == DT_F32) {
        const u4 p = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
        const u4 q = {__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])};
        __builtin_amdgcn_raw_buffer_store_b128(p, rs, lane_off(ok, base), 0, CP);
        __builtin_amdgcn_raw_buffer_store_b128(q, rs, lane_off(ok, base + 16), 0, CP);
      } else if (a.dt == DT_BF16) {
        const u4 p = {f2bf_pack(x[0], x[1]), f2bf_pack(x[2], x[3]), f2bf_pack(x[4], x[5]), f2bf_pack(x[6], x[7])};
        __builtin_amdgcn_raw_buffer_store_b128(p, rs, lane_off(ok, base), 0, CP);
      } else {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lo |= (uint32_t)(uint8_t)x[j] << (8 * j);
          hi |= (uint32_t)(uint8_t)x[4 + j] << (8 * j);
        }
        __builtin_amdgcn_raw_buffer_store_b32(lo, rs, lane_off(ok, base), 0, CP);
        __builtin_amdgcn_raw_buffer_store_b32(hi, rs, lane_off(ok, base + 4), 0, CP);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int off = lane_off(ok, base + j * a.sc * es);
        if (a.dt == DT_BF16)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(f2bf_pack(x[j], 0.f) & 0xffffu), rs, off, 0, 0);
        else if (a.dt == DT_F32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x[j]), rs, off, 0, 0);
        else __builtin_amdgcn_raw_buffer_store_b8((uint8_t)x[j], rs, off, 0, 0);
      }
    }
  }
}

// Register k (wave-uniform) selected element by element, which keeps the
// three registers in VGPRs (a whole-struct copy under a dynamic k becomes
// an indexed stack array).
template <int U>
__device__ __forceinline__ void pick(TV<U>& d, uint32_t k, const TV<U>& t0, const TV<U>& t1, const TV<U>& t2) {
#pragma unroll
  for (int i = 0; i < 8 * U; ++i) d.v[i] = k == 0 ? t0.v[i] : k == 1 ? t1.v[i] : t2.v[i];
}

template <int U>
__device__ __forceinline__ void put(uint32_t k, const TV<U>& s, TV<U>& t0, TV<U>& t1, TV<U>& t2) {
#pragma unroll
  for (int i = 0; i < 8 * U; ++i) {
    t0.v[i] = k == 0 ? s.v[i] : t0.v[i];
    t1.v[i] = k == 1 ? s.v[i] : t1.v[i];
    t2.v[i] = k == 2 ? s.v[i] : t2.v[i];
  }
}

template <uint32_t OPK, int U>
__device__ __forceinline__ void bin(TV<U>& acc, const TV<U>& b, bool rev) {
#pragma unroll
  for (int i = 0; i < 8 * U; ++i) {
    const float x = acc.v[i], y = b.v[i];
    acc.v[i] = rev ? alu_rt(OPK, y, x) : alu_rt(OPK, x, y);
  }
}

template <int U>
__device__ __forceinline__ void run_epilogue(KW* W, TV<U>& t0, const Round<U>& C, const Inv& I) {
  TV<U> t1, t2;
#pragma unroll
  for (int i = 0; i < 8 * U; ++i) {
    t1.v[i] = 0.f;
    t2.v[i] = 0.f;
  }
  const uint32_t pc_end = W[H_BODY_END];
  for (uint32_t pc = W[H_BODY_BEGIN]; pc < pc_end; pc += 2) {
    const uint32_t w0 = W[pc], w1 = W[pc + 1];
    switch (f_op(w0)) {
      case OP_LOAD: {
        TV<U> m;
        epi_load(m, w1, W, C, I);
        put(f_dst(w0), m, t0, t1, t2);
        break;
      }
      case OP_STORE: {
        TV<U> m;
        pick(m, f_a(w0), t0, t1, t2);
        if (W[H_FLAGS] & HF_STREAM) epi_store<U, 2>(m, read_arg(W, w1), C);
        else epi_store<U, 0>(m, read_arg(W, w1), C);
        break;
      }
      case OP_COPY: {
        TV<U> m;
        pick(m, f_a(w0), t0, t1, t2);
        put(f_dst(w0), m, t0, t1, t2);
        break;
      }
      case OP_BIN: {
        TV<U> b;
        const uint32_t bk = f_bk(w0);
        if (bk == BK_MEM) epi_load(b, w1, W, C, I);
        else if (bk == BK_TREG) pick(b, f_b(w0), t0, t1, t2);
        else {
#pragma unroll
          for (int i = 0; i < 8 * U; ++i) b.v[i] = __uint_as_float(w1);
        }
        const bool rev = (f_flags(w0) & FL_REV) != 0;
        switch (f_sub(w0)) {
          case ALU_ADD: bin<ALU_ADD>(t0, b, rev); break;
          case ALU_SUB: bin<ALU_SUB>(t0, b, rev); break;
          case ALU_MUL: bin<ALU_MUL>(t0, b, rev); break;
          case ALU_DIV: bin<ALU_DIV>(t0, b, rev); break;
          case ALU_MAX: bin<ALU_MAX>(t0, b, rev); break;
          case ALU_MIN: bin<ALU_MIN>(t0, b, rev); break;
          default: bin<ALU_POW>(t0, b, rev); break;
        }
        break;
      }
      case OP_UN: {
        const uint32_t f = f_sub(w0);
#pragma unroll
        for (int i = 0; i < 8 * U; ++i) t0.v[i] = una_rt(f, t0.v[i]);
        break;
      }
      case OP_DBG: {
        // debug tile maps: the tile's row-major id (sub 0) or the workgroup (sub 1)
        TV<U> m;
        const float v = f_sub(w0) == 0 ? (float)C.tile : (float)blockIdx.x;
#pragma unroll
        for (int i = 0; i < 8 * U; ++i) m.v[i] = v;
        put(f_dst(w0), m, t0, t1, t2);
        break;
      }
      default:
        break;
    }
  }
}

// Row of accumulator register i of this lane inside its 32 x 32 block.
__device__ __forceinline__ int dm_of(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// Tile row of slab row rho in slab s.
template <class CF>
__device__ __forceinline__ int slab_row(int s, int rho) {
  const int wm = rho / (32 * CF::IB), il = (rho / 32) % CF::IB;
  return wm * 32 * CF::BM + (s * CF::IB + il) * 32 + (rho & 31);
}

// The up-to-two operands of the body that do not vary along M.
__device__ __forceinline__ void find_invariants(KW* W, Inv& I) {
  I.arg0 = I.arg1 = -1;
  const uint32_t pc_end = W[H_BODY_END];
  for (uint32_t pc = W[H_BODY_BEGIN]; pc < pc_end; pc += 2) {
    const uint32_t w0 = W[pc], w1 = W[pc + 1];
    const bool mem = f_op(w0) == OP_LOAD || (f_op(w0) == OP_BIN && f_bk(w0) == BK_MEM);
    if (!mem || (int)w1 == I.arg0 || (int)w1 == I.arg1) continue;
    if (read_arg(W, w1).sr != 0) continue;
    if (I.arg0 < 0) I.arg0 = (int)w1;
    else if (I.arg1 < 0) I.arg1 = (int)w1;
  }
}

template <class CF>
__device__ __forceinline__ void load_invariants(KW* W, Inv& I, int64_t n0, int64_t N, int tid) {
  const int c8 = (tid % CF::LPR) * 8;
  const bool ok = n0 + c8 < N;
  if (I.arg0 >= 0) chunk_load(I.v0, read_arg(W, (uint32_t)I.arg0), 0, n0, 0, c8, ok);
  if (I.arg1 >= 0) chunk_load(I.v1, read_arg(W, (uint32_t)I.arg1), 0, n0, 0, c8, ok);
}

// Stage slab s of the accumulators and run the body on it.
template <class CF, int S>
__device__ __forceinline__ void epilogue_slab(KW* W, const f16v (&c)[CF::BM][CF::BN], char* lds, int64_t m0,
                                              int64_t n0, int64_t M, int64_t N, int wm, int wn, int tid,
                                              const Inv& I, uint32_t tile) {
  constexpr int U = CF::U;
  const int lane = tid & 63;
  float* ot = (float*)lds;
#pragma unroll
  for (int il = 0; il < CF::IB; ++il)
#pragma unroll
    for (int j = 0; j < CF::BN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int rho = wm * 32 * CF::IB + il * 32 + dm_of(q, lane);
        const int col = wn * 32 * CF::BN + j * 32 + (lane & 31);
        ot[rho * CF::OSTR + col] = c[S * CF::IB + il][j][q];
      }
  lds_barrier();
  Round<U> C;
  C.m0 = m0;
  C.n0 = n0;
  C.tile = tile;
  C.c8 = (tid % CF::LPR) * 8;
#pragma nounroll
  for (int p = 0; p < CF::SP; p += U) {
    TV<U> t0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rho = (p + u) * CF::RPP + tid / CF::LPR;
      C.r[u] = slab_row<CF>(S, rho);
      C.ok[u] = (m0 + C.r[u] < M) & (n0 + C.c8 < N);
      const float* src = ot + rho * CF::OSTR + C.c8;
      const float4 x = *(const float4*)src, y = *(const float4*)(src + 4);
      float* d = t0.v + 8 * u;
      d[0] = x.x; d[1] = x.y; d[2] = x.z; d[3] = x.w;
      d[4] = y.x; d[5] = y.y; d[6] = y.z; d[7] = y.w;
    }
    run_epilogue<U>(W, t0, C, I);
  }
  lds_barrier();
}

template <class CF, int S>
__device__ __forceinline__ void epilogue_slabs(KW* W, const f16v (&c)[CF::BM][CF::BN], char* lds, int64_t m0,
                                               int64_t n0, int64_t M, int64_t N, int wm, int wn, int tid,
                                               const Inv& I, uint32_t tile) {
  epilogue_slab<CF, S>(W, c, lds, m0, n0, M, N, wm, wn, tid, I, tile);
  if constexpr (S + 1 < CF::NSL) epilogue_slabs<CF, S + 1>(W, c, lds, m0, n0, M, N, wm, wn, tid, I, tile);
}

// ---------------------------------------------------------------------------
// Tile order and the kernel body
// ---------------------------------------------------------------------------
// Linear tile v -> (row tile, column tile): groups of GM row tiles, walked
// column by column inside a group, so that consecutive tiles share A panels
// and B panels.
constexpr uint32_t GM = 8;

__device__ __forceinline__ void tile_rc(uint32_t v, uint32_t nrt, uint32_t nct, uint32_t& ir, uint32_t& ic) {
  const uint32_t per = GM * nct;
  const uint32_t g = v / per, w = v - g * per;
  const uint32_t r0 = g * GM;
  const uint32_t gm = nrt - r0 < GM ? nrt - r0 : GM;
  ir = r0 + w % gm;
  ic = w / gm;
}

// Workgroups are dealt round-robin over the eight XCDs (each with its own
// L2).  Slot of workgroup b: the workgroups of one XCD get consecutive
// slots, so the tiles that run together on an XCD are consecutive in the
// grouped order; the tail beyond a multiple of eight keeps its index.
__device__ __forceinline__ uint32_t xcd_slot(uint32_t b, uint32_t G) {
  const uint32_t G8 = G & ~7u;
  return b < G8 ? (b & 7u) * (G8 >> 3) + (b >> 3) : b;
}

template <class CF>
__device__ __forceinline__ void mix_body(char* lds) {
  KW* W = (KW*)__builtin_amdgcn_kernarg_segment_ptr();
  const uint32_t block_dim = W[H_BLOCK_DIM];
  const uint32_t nct = W[H_NC];
  const uint32_t nrt = block_dim / nct;
  const int64_t M = (int64_t)w64(W, H_R_LO);
  const int64_t N = (int64_t)w64(W, H_C_LO);
  const int K = (int)W[H_MM_K];
  const ArgD A = read_arg(W, W[H_MM_A]);
  const ArgD Bm = read_arg(W, W[H_MM_B]);
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave / CF::WN, wn = wave % CF::WN;
  const int n_stage = (K + CF::KT - 1) / CF::KT;
  const uint32_t ring = (uint32_t)(uintptr_t)(lds_void*)lds;
  const uint32_t G = gridDim.x;
  Inv I;
  find_invariants(W, I);

  for (uint32_t v = xcd_slot(blockIdx.x, G); v < block_dim; v += G) {
    uint32_t ir, ic;
    tile_rc(v, nrt, nct, ir, ic);
    Panels P;
    P.m0 = (int64_t)ir * CF::TM;
    P.n0 = (int64_t)ic * CF::TN;
    P.ra = rsrc_words(A, P.m0 * A.sr * 2);
    P.rb = rsrc_words(Bm, P.n0 * 2);
    load_invariants<CF>(W, I, P.n0, N, tid);  // lands during the K loop
    f16v c[CF::BM][CF::BN];
#pragma unroll
    for (int i = 0; i < CF::BM; ++i)
#pragma unroll
      for (int j = 0; j < CF::BN; ++j) c[i][j] = (f16v)0.f;

    // Software pipeline over 16-deep steps of K.  The barrier of stage s
    // sits after the reads of its last step were issued: past it every wave
    // is done with slot s, which is refilled at once with stage s + NS, and
    // stage s + 1 has landed, so its first step is read while the last step
    // of stage s is multiplied.
#pragma unroll
    for (int s = 0; s < CF::NS; ++s)
      if (s < n_stage) issue_stage<CF>(ring, s, s, P, A, Bm, M, N, K, wave, lane);
    if (n_stage >= CF::NS) wait_dma<(CF::NS - 1) * CF::Q>();
    else wait_dma<0>();
    lds_barrier();
    Frag<CF> f[2];
    load_frag<CF>(f[0], lds, 0, wm, wn, lane);
    for (int s = 0; s < n_stage; ++s) {
      const char* st = lds + (s % CF::NS) * CF::STAGE;
      // the two workgroups of a compute unit share its SIMDs: a wave in the
      // middle of its matrix work issues ahead of one waiting at a stage edge
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk + 1 < CF::SPS; ++kk) {
        load_frag<CF>(f[(kk + 1) & 1], st, kk + 1, wm, wn, lane);
        mma<CF>(c, f[kk & 1]);
      }
      __builtin_amdgcn_s_setprio(0);
      if (s + 1 < n_stage) {
        if (s + CF::NS <= n_stage) wait_dma<(CF::NS - 2) * CF::Q>();
        else wait_dma<0>();
        lds_barrier();
        if (s + CF::NS < n_stage) issue_stage<CF>(ring, s % CF::NS, s + CF::NS, P, A, Bm, M, N, K, wave, lane);
        load_frag<CF>(f[0], lds + ((s + 1) % CF::NS) * CF::STAGE, 0, wm, wn, lane);
      }
      mma<CF>(c, f[1]);
    }
    lds_barrier();
    epilogue_slabs<CF, 0>(W, c, lds, P.m0, P.n0, M, N, wm, wn, tid, I, ir * nct + ic);
  }
}

}  // namespace

// 128 x 128 tiles, 4 waves of 64 x 64, two workgroups per compute unit.
// (Measured on the MatMul+bias+SiLU call list: 256 x 128 tiles at two
// workgroups per compute unit and 256 x 256 tiles at one, with 8 or 4 waves,
// were no faster over the mix of M: the larger tiles run out of registers to
// read ahead, or leave the epilogue exposed.)
using Mix128 = Cfg<2, 2, 2, 2, MM_KT, MM_STAGES, 1, 4>;
static_assert(Mix128::LDS == mm_lds_bytes(Mix128::TM, Mix128::TN), "LDS size agrees with the header's");

extern "C" __global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
dvm_vm_mix_128(const Program prog) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  (void)prog;
  mix_body<Mix128>(lds);
}

// Host-side launch of the MIX VM kernel matching the program's tile.
extern "C" hipError_t dvm_launch_mix_kernel(const Program* p, unsigned grid, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)dvm_vm_mix_128, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       Mix128::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  if (p->w[H_TR] != (uint32_t)Mix128::TM || p->w[H_TC] != (uint32_t)Mix128::TN) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dvm_vm_mix_128, dim3(grid), dim3(Mix128::NT), Mix128::LDS, s, *p);
  return hipGetLastError();
}
