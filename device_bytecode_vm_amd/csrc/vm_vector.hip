// The resident VM kernel for VECTOR programs (elementwise, row-reduce and
// reduce-all templates) on gfx950.
//
// It follows the VM algorithm of the DVM paper review page (section 4.4):
// each workgroup computes its tile count and its tile range from the code
// header, and for every tile decodes the body instruction by instruction and
// calls the matching virtual-instruction function.  Decoding is wave-uniform:
// the program sits in the kernarg segment and every word is read with a scalar
// load, so the opcode switch is a chain of scalar compares and branches (the
// counterpart of the page's decode on the Scalar unit), and the instruction
// bodies run on the vector ALUs, the LDS and the vector memory pipeline.
//
// Tiles are staged in registers, not in LDS: each lane owns up to NV_MAX
// chunks of VEC consecutive columns of its row, so elementwise chains never
// leave the VGPR file (the page's "intermediate results stay in local memory"
// of section 5.1, with the CU's register file as that local memory).  LDS
// carries only what crosses lanes: the per-wave partials of a reduction whose
// row spans several waves, and the reduce-all partials.  Every register index
// is a compile-time constant: compute instructions have the two-address form
// treg[0] <- treg[0] (op) B, and each instruction body is instantiated for
// every register it can name.
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

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

constexpr int OOB = 0x7fffffff;                 // lane offset beyond any descriptor size
constexpr int RSRC_W3 = 0x00020000;             // raw buffer, 32-bit data format

struct ArgD {
  const char* p;
  uint32_t dt, fl;
  int64_t sr;
  int32_t sc;
  uint32_t extent;
};

struct Geo {
  int g, nv, tr, tc, nc, lg;  // lg = log2(g)
  int64_t R, C;
};

struct Tile {
  int64_t r0;   // first row of the tile
  int64_t c0;   // first column of the tile
  int tce;      // valid columns in this tile
  int tre;      // valid rows in this tile
  uint32_t id;
};

__device__ __forceinline__ uint64_t w64(const uint32_t* w, int lo) {
  return ((uint64_t)w[lo + 1] << 32) | (uint64_t)w[lo];
}

__device__ __forceinline__ ArgD read_arg(const uint32_t* W, uint32_t i) {
  const uint32_t* a = W + ARG_BASE + i * ARG_WORDS;
  ArgD d;
  d.p = reinterpret_cast<const char*>(w64(a, A_PTR_LO));
  d.dt = a[A_DTYPE];
  d.fl = a[A_FLAGS];
  d.sr = (int64_t)w64(a, A_SR_LO);
  d.sc = (int32_t)a[A_SC];
  d.extent = a[A_EXTENT];
  return d;
}

__device__ __forceinline__ int esize(uint32_t dt) { return dt == DT_F32 ? 4 : dt == DT_BF16 ? 2 : 1; }

// Descriptor over the operand's part of the tile: base at the tile's first
// element, size = bytes left in the tensor (capped).
__device__ __forceinline__ Rsrc tile_rsrc(const ArgD& a, const Tile& tl) {
  const int64_t es = esize(a.dt);
  const int64_t ob = (tl.r0 * a.sr + tl.c0 * (int64_t)a.sc) * es;
  const int64_t left = (int64_t)a.extent - ob;
  const int n = left <= 0 ? 0 : (left >= (int64_t)EXTENT_CAP ? (int)(EXTENT_CAP - 1) : (int)left);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a.p + ob), 0, n, RSRC_W3);
}

// ---------------------------------------------------------------------------
// element conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f2bf_pack(float lo, float hi) {
  f2 v = {lo, hi};
  bf2 b = __builtin_convertvector(v, bf2);  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float round_bf16(float x) { return bf2f(f2bf_pack(x, 0.f) & 0xffffu); }

// ---------------------------------------------------------------------------
// ALU
// ---------------------------------------------------------------------------
template <uint32_t OPK>
__device__ __forceinline__ float alu(float x, float y) {
  if constexpr (OPK == ALU_ADD) return x + y;
  else if constexpr (OPK == ALU_SUB) return x - y;
  else if constexpr (OPK == ALU_MUL) return x * y;
  else if constexpr (OPK == ALU_DIV) return x / y;
  else if constexpr (OPK == ALU_MAX) return (x != x || y != y) ? x + y : fmaxf(x, y);
  else if constexpr (OPK == ALU_MIN) return (x != x || y != y) ? x + y : fminf(x, y);
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
  else if constexpr (F == UN_EXP) return expf(x);
  else if constexpr (F == UN_ROUND) return rintf(x);
  else if constexpr (F == UN_FLOOR) return floorf(x);
  else if constexpr (F == UN_ISFINITE) return isfinite(x) ? 1.f : 0.f;
  else if constexpr (F == UN_NEG) return -x;
  else if constexpr (F == UN_RECIP) return 1.f / x;
  else if constexpr (F == UN_TOBF16) return round_bf16(x);
  else return x;
}

__device__ __forceinline__ float una_rt(uint32_t f, float x) {
  switch (f) {
    case UN_SQRT: return sqrtf(x);
    case UN_ABS: return fabsf(x);
    case UN_LOG: return logf(x);
    case UN_EXP: return expf(x);
    case UN_ROUND: return rintf(x);
    case UN_FLOOR: return floorf(x);
    case UN_ISFINITE: return isfinite(x) ? 1.f : 0.f;
    case UN_NEG: return -x;
    case UN_RECIP: return 1.f / x;
    case UN_TOBF16: return round_bf16(x);
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

typedef float Chunks __attribute__((ext_vector_type(E_MAX)));
typedef Chunks TReg[N_TREG];

// Lane coordinates inside the tile.
struct Lane {
  int row;   // row inside the tile
  int lane;  // lane inside the row group
  bool rok;  // row exists
};

// Lane masks are applied with selects over values computed on every lane:
// the arguments are evaluated before the call, so no lane-dependent branch
// (and no divergent join inside the interpreter loop) is formed.
__device__ __forceinline__ int lane_off(bool ok, int off) { return ok ? off : OOB; }
__device__ __forceinline__ float lane_sel(bool ok, float v, float other) { return ok ? v : other; }

// ---------------------------------------------------------------------------
// Load / Store (Table 1: Load/ViewLoad/Store/ViewStore)
// ---------------------------------------------------------------------------
// Fill dst (one tile register's worth) from operand a for this tile.
template <uint32_t DT>
__device__ __forceinline__ void load_chunks(Chunks& dst, const ArgD& a, const Geo& G, const Tile& tl,
                                            const Lane& L) {
  constexpr int ES = DT == DT_F32 ? 4 : DT == DT_BF16 ? 2 : 1;
  const Rsrc rs = tile_rsrc(a, tl);
  const int roff = L.row * (int)a.sr;  // tile spans < 2^31 bytes (host checked)
  if (a.sc == 0) {
    // broadcast along the row: one element per row
    const int off = lane_off(L.rok, roff * ES);
    float v;
    if constexpr (DT == DT_F32) v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
    else if constexpr (DT == DT_BF16) v = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
    else v = (float)__builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0);
#pragma unroll
    for (int e = 0; e < E_MAX; ++e) dst[e] = v;
  } else if ((a.fl & AF_VEC) && a.sc == 1 && (tl.tce & (VEC - 1)) == 0) {
    // full chunks, 16-byte aligned: 128-bit accesses; a chunk is wholly in or out
#pragma unroll
    for (int j = 0; j < NV_MAX; ++j) {
      {  // chunks past the row's last one fall out of range and are masked
        const int ct = (j * G.g + L.lane) * VEC;
        const int off = lane_off(L.rok & (ct < tl.tce), (roff + ct) * ES);
        if constexpr (DT == DT_F32) {
          const u4 v0 = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
          const u4 v1 = __builtin_amdgcn_raw_buffer_load_b128(rs, off == OOB ? OOB : off + 16, 0, 0);
          dst[j * VEC + 0] = __uint_as_float(v0.x); dst[j * VEC + 1] = __uint_as_float(v0.y);
          dst[j * VEC + 2] = __uint_as_float(v0.z); dst[j * VEC + 3] = __uint_as_float(v0.w);
          dst[j * VEC + 4] = __uint_as_float(v1.x); dst[j * VEC + 5] = __uint_as_float(v1.y);
          dst[j * VEC + 6] = __uint_as_float(v1.z); dst[j * VEC + 7] = __uint_as_float(v1.w);
        } else if constexpr (DT == DT_BF16) {
          const u4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
          dst[j * VEC + 0] = bf2f(v.x & 0xffffu); dst[j * VEC + 1] = __uint_as_float(v.x & 0xffff0000u);
          dst[j * VEC + 2] = bf2f(v.y & 0xffffu); dst[j * VEC + 3] = __uint_as_float(v.y & 0xffff0000u);
          dst[j * VEC + 4] = bf2f(v.z & 0xffffu); dst[j * VEC + 5] = __uint_as_float(v.z & 0xffff0000u);
          dst[j * VEC + 6] = bf2f(v.w & 0xffffu); dst[j * VEC + 7] = __uint_as_float(v.w & 0xffff0000u);
        } else {
          const u2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dst[j * VEC + i] = (float)((v.x >> (8 * i)) & 0xffu);
            dst[j * VEC + 4 + i] = (float)((v.y >> (8 * i)) & 0xffu);
          }
        }
      }
    }
  } else {
    // element path: ragged tiles, unaligned or strided operands
#pragma unroll
    for (int j = 0; j < NV_MAX; ++j) {
      {
        const int ct = (j * G.g + L.lane) * VEC;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const int c = ct + i;
          const int off = lane_off(L.rok & (c < tl.tce), (roff + c * a.sc) * ES);
          float v;
          if constexpr (DT == DT_F32) v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
          else if constexpr (DT == DT_BF16) v = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
          else v = (float)__builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0);
          dst[j * VEC + i] = v;
        }
      }
    }
  }
}

template <uint32_t DT>
__device__ __forceinline__ void store_chunks(const Chunks& src, const ArgD& a, const Geo& G, const Tile& tl,
                                             const Lane& L) {
  constexpr int ES = DT == DT_F32 ? 4 : DT == DT_BF16 ? 2 : 1;
  const Rsrc rs = tile_rsrc(a, tl);
  const int roff = L.row * (int)a.sr;
  if ((a.fl & AF_VEC) && a.sc == 1 && (tl.tce & (VEC - 1)) == 0) {
#pragma unroll
    for (int j = 0; j < NV_MAX; ++j) {
      {  // chunks past the row's last one fall out of range and are masked
        const int ct = (j * G.g + L.lane) * VEC;
        const int off = lane_off(L.rok & (ct < tl.tce), (roff + ct) * ES);
        if constexpr (DT == DT_F32) {
          u4 v0, v1;
          v0.x = __float_as_uint(src[j * VEC + 0]); v0.y = __float_as_uint(src[j * VEC + 1]);
          v0.z = __float_as_uint(src[j * VEC + 2]); v0.w = __float_as_uint(src[j * VEC + 3]);
          v1.x = __float_as_uint(src[j * VEC + 4]); v1.y = __float_as_uint(src[j * VEC + 5]);
          v1.z = __float_as_uint(src[j * VEC + 6]); v1.w = __float_as_uint(src[j * VEC + 7]);
          __builtin_amdgcn_raw_buffer_store_b128(v0, rs, off, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b128(v1, rs, off == OOB ? OOB : off + 16, 0, 0);
        } else if constexpr (DT == DT_BF16) {
          u4 v;
          v.x = f2bf_pack(src[j * VEC + 0], src[j * VEC + 1]);
          v.y = f2bf_pack(src[j * VEC + 2], src[j * VEC + 3]);
          v.z = f2bf_pack(src[j * VEC + 4], src[j * VEC + 5]);
          v.w = f2bf_pack(src[j * VEC + 6], src[j * VEC + 7]);
          __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 0);
        } else {
          u2 v = {0u, 0u};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v.x |= ((uint32_t)src[j * VEC + i] & 0xffu) << (8 * i);
            v.y |= ((uint32_t)src[j * VEC + 4 + i] & 0xffu) << (8 * i);
          }
          __builtin_amdgcn_raw_buffer_store_b64(v, rs, off, 0, 0);
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NV_MAX; ++j) {
      {
        const int ct = (j * G.g + L.lane) * VEC;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const int c = ct + i;
          const int off = lane_off(L.rok & (c < tl.tce), (roff + c * a.sc) * ES);
          const float v = src[j * VEC + i];
          if constexpr (DT == DT_F32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, off, 0, 0);
          else if constexpr (DT == DT_BF16)
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(f2bf_pack(v, 0.f) & 0xffffu), rs, off, 0, 0);
          else __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, rs, off, 0, 0);
        }
      }
    }
  }
}

__device__ __forceinline__ void load_any(Chunks& dst, const ArgD& a, const Geo& G, const Tile& tl, const Lane& L) {
  if (a.dt == DT_BF16) load_chunks<DT_BF16>(dst, a, G, tl, L);
  else if (a.dt == DT_F32) load_chunks<DT_F32>(dst, a, G, tl, L);
  else load_chunks<DT_U8>(dst, a, G, tl, L);
}

__device__ __forceinline__ void store_any(const Chunks& src, const ArgD& a, const Geo& G, const Tile& tl,
                                          const Lane& L) {
  if (a.dt == DT_BF16) store_chunks<DT_BF16>(src, a, G, tl, L);
  else if (a.dt == DT_F32) store_chunks<DT_F32>(src, a, G, tl, L);
  else store_chunks<DT_U8>(src, a, G, tl, L);
}

// ---------------------------------------------------------------------------
// Compute instructions on tile registers
// ---------------------------------------------------------------------------
__device__ __forceinline__ void copy_c(Chunks& d, const Chunks& s, int nv) {
#pragma unroll
  for (int j = 0; j < NV_MAX; ++j)
#pragma unroll
      for (int i = 0; i < VEC; ++i) d[j * VEC + i] = s[j * VEC + i];
}

// acc <- acc (op) b, or b (op) acc
template <uint32_t OPK, bool REV>
__device__ __forceinline__ void bin_cc(Chunks& acc, const Chunks& b, int nv) {
#pragma unroll
  for (int j = 0; j < NV_MAX; ++j)
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const float x = acc[j * VEC + i], y = b[j * VEC + i];
        acc[j * VEC + i] = REV ? alu<OPK>(y, x) : alu<OPK>(x, y);
      }
}

template <uint32_t OPK, bool REV>
__device__ __forceinline__ void bin_cs(Chunks& acc, float s, int nv) {
#pragma unroll
  for (int j = 0; j < NV_MAX; ++j)
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const float x = acc[j * VEC + i];
        acc[j * VEC + i] = REV ? alu<OPK>(s, x) : alu<OPK>(x, s);
      }
}

template <uint32_t F>
__device__ __forceinline__ void un_c(Chunks& acc, int nv) {
#pragma unroll
  for (int j = 0; j < NV_MAX; ++j)
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[j * VEC + i] = una<F>(acc[j * VEC + i]);
}

template <uint32_t OPK>
__device__ __forceinline__ void bin_op(TReg& t, uint32_t w0, uint32_t w1, float rowv, const Chunks& memv,
                                       const Geo& G) {
  const uint32_t bk = f_bk(w0), b = f_b(w0);
  const bool rev = (f_flags(w0) & FL_REV) != 0;
  const int nv = G.nv;
  if (bk == BK_TREG) {
    switch (b * 2 + (rev ? 1 : 0)) {
      case 0: bin_cc<OPK, false>(t[0], t[0], nv); break;
      case 1: bin_cc<OPK, true>(t[0], t[0], nv); break;
      case 2: bin_cc<OPK, false>(t[0], t[1], nv); break;
      case 3: bin_cc<OPK, true>(t[0], t[1], nv); break;
      case 4: bin_cc<OPK, false>(t[0], t[2], nv); break;
      default: bin_cc<OPK, true>(t[0], t[2], nv); break;
    }
  } else if (bk == BK_MEM) {
    if (rev) bin_cc<OPK, true>(t[0], memv, nv);
    else bin_cc<OPK, false>(t[0], memv, nv);
  } else {
    const float s = bk == BK_RREG ? rowv : __uint_as_float(w1);
    if (rev) bin_cs<OPK, true>(t[0], s, nv);
    else bin_cs<OPK, false>(t[0], s, nv);
  }
}

// ---------------------------------------------------------------------------
// Cross-lane reductions: DPP and permlane swaps inside a wave, LDS across
// waves.
// ---------------------------------------------------------------------------
template <uint32_t KIND>
__device__ __forceinline__ float comb(float a, float b) {
  if constexpr (KIND == RK_SUM) return a + b;
  else return (a != a || b != b) ? a + b : fmaxf(a, b);
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

// Partial over this lane's valid elements.  Full tiles mask whole chunks; only
// ragged tiles mask element by element.
template <uint32_t KIND>
__device__ __forceinline__ float lane_partial(const Chunks& c, const Geo& G, const Tile& tl, const Lane& L) {
  const float id = KIND == RK_SUM ? 0.f : -__builtin_huge_valf();
  float acc = id;
  if ((tl.tce & (VEC - 1)) == 0) {
#pragma unroll
    for (int j = 0; j < NV_MAX; ++j) {
        float s = c[j * VEC];
#pragma unroll
        for (int i = 1; i < VEC; ++i) s = comb<KIND>(s, c[j * VEC + i]);
        const int ct = (j * G.g + L.lane) * VEC;
        acc = comb<KIND>(acc, lane_sel(L.rok & (ct < tl.tce), s, id));
      }
  } else {
#pragma unroll
    for (int j = 0; j < NV_MAX; ++j) {
        const int ct = (j * G.g + L.lane) * VEC;
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc = comb<KIND>(acc, lane_sel(L.rok & (ct + i < tl.tce), c[j * VEC + i], id));
      }
  }
  return acc;
}

__device__ __forceinline__ float lane_partial_k(const Chunks& c, const Geo& G, const Tile& tl, const Lane& L,
                                                uint32_t kind) {
  return kind == RK_SUM ? lane_partial<RK_SUM>(c, G, tl, L) : lane_partial<RK_MAX>(c, G, tl, L);
}

__device__ __forceinline__ float lane_partial_any(const TReg& t, uint32_t k, const Geo& G, const Tile& tl,
                                                  const Lane& L, uint32_t kind) {
  switch (k) {
    case 0: return lane_partial_k(t[0], G, tl, L, kind);
    case 1: return lane_partial_k(t[1], G, tl, L, kind);
    default: return lane_partial_k(t[2], G, tl, L, kind);
  }
}

__device__ __forceinline__ float group_reduce_k(float acc, int gs, uint32_t kind) {
  return kind == RK_SUM ? group_reduce<RK_SUM>(acc, gs) : group_reduce<RK_MAX>(acc, gs);
}

__device__ __forceinline__ float comb_k(float a, float b, uint32_t kind) {
  return kind == RK_SUM ? a + b : comb<RK_MAX>(a, b);
}

__device__ __forceinline__ void fill_c(Chunks& c, float v) {
#pragma unroll
  for (int e = 0; e < E_MAX; ++e) c[e] = v;
}

// ---------------------------------------------------------------------------
// LDS staging: next-tile prefetch (direct-to-LDS buffer loads, two buffers
// by tile parity) and LDS-resident tile-invariant operands.  Every lane reads
// back exactly the bytes its own loads or stores put in LDS, so no barrier is
// needed, only the wait for its own outstanding loads.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

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

// a tile whose columns end on a chunk boundary is staged whole
__device__ __forceinline__ bool tile_full(const Tile& tl) { return (tl.tce & (VEC - 1)) == 0; }

__device__ __forceinline__ uint32_t pf_buf_bytes(const Geo& G, uint32_t dt) {
  return (uint32_t)G.nv * T_LANES * 16u * (dt == DT_F32 ? 2u : 1u);
}

__device__ __forceinline__ void pf_issue(char* slot, const ArgD& a, const Geo& G, const Tile& tl, int tid) {
  const int es = esize(a.dt);
  const int halves = a.dt == DT_F32 ? 2 : 1;
  char* base = slot + (tl.id & 1u) * pf_buf_bytes(G, a.dt);
  const Rsrc rs = tile_rsrc(a, tl);
  const int row = tid >> G.lg, lane = tid & (G.g - 1);
  const bool rok = row < tl.tre;
  const int roff = row * (int)a.sr;
  const int wave = tid >> 6;
#pragma unroll
  for (int j = 0; j < NV_MAX; ++j) {
    if (j < G.nv) {
      const int ct = (j * G.g + lane) * VEC;
      const int off = lane_off(rok & (ct < tl.tce), (roff + ct) * es);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h < halves) {
          lds_void* dst = (lds_void*)(base + ((j * halves + h) * T_LANES + wave * 64) * 16);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, off == OOB ? OOB : off + 16 * h, 0, 0, 0);
        }
      }
    }
  }
}

template <uint32_t DT>
__device__ __forceinline__ void pf_read(Chunks& dst, const char* slot, const Geo& G, const Tile& tl, int tid) {
  constexpr int HV = DT == DT_F32 ? 2 : 1;
  const char* base = slot + (tl.id & 1u) * pf_buf_bytes(G, DT);
#pragma unroll
  for (int j = 0; j < NV_MAX; ++j) {
    {  // a chunk past nv re-reads chunk 0 (its values are masked downstream)
      const int jj = j < G.nv ? j : 0;
      const u4 v = *(const u4*)(base + ((jj * HV) * T_LANES + tid) * 16);
      if constexpr (DT == DT_F32) {
        const u4 w = *(const u4*)(base + ((jj * HV + 1) * T_LANES + tid) * 16);
        dst[j * VEC + 0] = __uint_as_float(v.x); dst[j * VEC + 1] = __uint_as_float(v.y);
        dst[j * VEC + 2] = __uint_as_float(v.z); dst[j * VEC + 3] = __uint_as_float(v.w);
        dst[j * VEC + 4] = __uint_as_float(w.x); dst[j * VEC + 5] = __uint_as_float(w.y);
        dst[j * VEC + 6] = __uint_as_float(w.z); dst[j * VEC + 7] = __uint_as_float(w.w);
      } else {
        dst[j * VEC + 0] = bf2f(v.x & 0xffffu); dst[j * VEC + 1] = __uint_as_float(v.x & 0xffff0000u);
        dst[j * VEC + 2] = bf2f(v.y & 0xffffu); dst[j * VEC + 3] = __uint_as_float(v.y & 0xffff0000u);
        dst[j * VEC + 4] = bf2f(v.z & 0xffffu); dst[j * VEC + 5] = __uint_as_float(v.z & 0xffff0000u);
        dst[j * VEC + 6] = bf2f(v.w & 0xffffu); dst[j * VEC + 7] = __uint_as_float(v.w & 0xffff0000u);
      }
    }
  }
}

__device__ __forceinline__ void inv_write(const Chunks& c, char* slot, const Geo& G, int tid) {
#pragma unroll
  for (int j = 0; j < NV_MAX; ++j) {
    if (j < G.nv) {
      f4 a = {c[j * VEC + 0], c[j * VEC + 1], c[j * VEC + 2], c[j * VEC + 3]};
      f4 b = {c[j * VEC + 4], c[j * VEC + 5], c[j * VEC + 6], c[j * VEC + 7]};
      *(f4*)(slot + (j * T_LANES + tid) * 32) = a;
      *(f4*)(slot + (j * T_LANES + tid) * 32 + 16) = b;
    }
  }
}

__device__ __forceinline__ void inv_read(Chunks& c, const char* slot, const Geo& G, int tid) {
#pragma unroll
  for (int j = 0; j < NV_MAX; ++j) {
    {
      const int jj = j < G.nv ? j : 0;
      const f4 a = *(const f4*)(slot + (jj * T_LANES + tid) * 32);
      const f4 b = *(const f4*)(slot + (jj * T_LANES + tid) * 32 + 16);
      c[j * VEC + 0] = a.x; c[j * VEC + 1] = a.y; c[j * VEC + 2] = a.z; c[j * VEC + 3] = a.w;
      c[j * VEC + 4] = b.x; c[j * VEC + 5] = b.y; c[j * VEC + 6] = b.z; c[j * VEC + 7] = b.w;
    }
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

// Staging context shared by the operand readers; slot addresses are
// re-derived from the header at each use (scalar loads) instead of being kept
// live across the interpreter loop.
struct Stage {
  const uint32_t* W;
  char* lds;
  uint32_t tile, t_end;
  int tid;
  __device__ __forceinline__ char* pf(uint32_t k) const { return lds + W[H_PF_OFF0 + k]; }
  __device__ __forceinline__ char* inv(uint32_t k) const { return lds + W[H_INV_OFF0 + k]; }
};

// Operand read for LOAD and memory operands: from an invariant slot, from the
// prefetch slot (then prefetch the next tile), or straight from memory.
__device__ __forceinline__ void read_operand(Chunks& dst, uint32_t w0, uint32_t vmc, const ArgD& a, const Geo& G,
                                             const Tile& tl, const Lane& L, const Stage& S) {
  const uint32_t fl = f_flags(w0), slot = f_b(w0) & 1u;
  if (fl & FL_INV) {
    inv_read(dst, S.inv(slot), G, S.tid);
    return;
  }
  if (fl & FL_PF) {
    if (tile_full(tl)) {
      // the previous tile may have been ragged (more instructions issued after
      // the prefetch): the count stays a lower bound, so the wait stays exact
      wait_vm(vmc);
      if (a.dt == DT_F32) pf_read<DT_F32>(dst, S.pf(slot), G, tl, S.tid);
      else pf_read<DT_BF16>(dst, S.pf(slot), G, tl, S.tid);
    } else {
      load_any(dst, a, G, tl, L);
    }
    if ((fl & FL_ISSUE) && S.tile + 1 < S.t_end) {
      const Tile nt = make_tile(G, S.tile + 1);
      if (tile_full(nt)) pf_issue(S.pf(slot), a, G, nt, S.tid);
    }
    return;
  }
  load_any(dst, a, G, tl, L);
}

}  // namespace

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
extern "C" __global__ void __launch_bounds__(T_LANES) __attribute__((amdgpu_waves_per_eu(2, 2)))
dvm_vm_vector(const Program prog) {
  __shared__ float s_red[N_LDSBUF][T_LANES / 64];
  __shared__ int s_last;
  extern __shared__ __attribute__((aligned(16))) char dlds[];

  const uint32_t* W = prog.w;
  const uint32_t block_dim = W[H_BLOCK_DIM];
  const uint32_t body_tile = W[H_BODY_TILE];

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

  const uint32_t t_begin = blockIdx.x * body_tile;
  uint32_t t_end = t_begin + body_tile;
  if (t_end > block_dim) t_end = block_dim;

  TReg t;
#pragma unroll
  for (int k = 0; k < N_TREG; ++k) fill_c(t[k], 0.f);
  RowRegs rw = {0.f, 0.f, 0.f, 0.f};

  Tile tl;
  auto set_tile = [&](uint32_t id) {
    const uint32_t ir = id / (uint32_t)G.nc;
    const uint32_t ic = id - ir * (uint32_t)G.nc;
    tl.id = id;
    tl.r0 = (int64_t)ir * G.tr;
    tl.c0 = (int64_t)ic * G.tc;
    const int64_t remc = G.C - tl.c0;
    tl.tce = remc < G.tc ? (int)remc : G.tc;
    const int64_t remr = G.R - tl.r0;
    tl.tre = remr < G.tr ? (int)remr : G.tr;
  };

  Stage S;
  S.W = W;
  S.lds = dlds;
  S.t_end = t_end;
  S.tid = tid;

  uint32_t tile = t_begin;
  uint32_t pc = W[H_PRO_BEGIN], pc_end = W[H_PRO_END];
  bool in_pro = true;
  if (t_begin < t_end) {
    set_tile(t_begin);
  } else {
    pc = pc_end = 0;
    in_pro = false;
    tile = t_end;
  }

  while (true) {
    if (pc >= pc_end) {
      if (in_pro) in_pro = false;
      else ++tile;
      if (tile >= t_end) break;
      set_tile(tile);
      pc = W[H_BODY_BEGIN];
      pc_end = W[H_BODY_END];
      continue;
    }
    const uint32_t w0 = W[pc];
    const uint32_t w1 = W[pc + 1];
    pc += 2;
    // Lane coordinates are recomputed per instruction (a few ALU ops) rather
    // than kept live across the whole interpreter loop.
    int tidv = tid;
    asm volatile("" : "+v"(tidv));
    Lane L;
    L.row = tidv >> G.lg;
    L.lane = tidv & (G.g - 1);
    L.rok = L.row < tl.tre;
    S.tile = tile;
    S.tid = tidv;

    switch (f_op(w0)) {
      case OP_LOAD: {
        Chunks tmp;
        read_operand(tmp, w0, vmc_load(w0), read_arg(W, w1), G, tl, L, S);
        switch (f_dst(w0)) {
          case 0: copy_c(t[0], tmp, NV_MAX); break;
          case 1: copy_c(t[1], tmp, NV_MAX); break;
          default: copy_c(t[2], tmp, NV_MAX); break;
        }
        break;
      }
      case OP_PF: {
        const ArgD a = read_arg(W, w1);
        if (tile_full(tl)) pf_issue(S.pf(f_b(w0) & 1u), a, G, tl, tidv);
        break;
      }
      case OP_LDS_INV: {
        const ArgD a = read_arg(W, w1);
        Chunks tmp;
        load_any(tmp, a, G, tl, L);
        inv_write(tmp, S.inv(f_dst(w0) & 1u), G, tidv);
        break;
      }
      case OP_STORE: {
        const ArgD a = read_arg(W, w1);
        switch (f_a(w0)) {
          case 0: store_any(t[0], a, G, tl, L); break;
          case 1: store_any(t[1], a, G, tl, L); break;
          default: store_any(t[2], a, G, tl, L); break;
        }
        break;
      }
      case OP_LOAD_ROW: {
        const ArgD a = read_arg(W, w1);
        const Rsrc rs = tile_rsrc(a, tl);
        const int es = esize(a.dt);
        const int off = lane_off(L.rok, L.row * (int)a.sr * es);
        float v;
        if (a.dt == DT_BF16) v = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
        else if (a.dt == DT_F32) v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
        else v = (float)__builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0);
        rset(rw, f_dst(w0), v);
        break;
      }
      case OP_STORE_ROW: {
        const ArgD a = read_arg(W, w1);
        const Rsrc rs = tile_rsrc(a, tl);
        const int es = esize(a.dt);
        const int off = lane_off(L.rok & (L.lane == 0), L.row * (int)a.sr * es);
        const float v = rget(rw, f_a(w0));
        if (a.dt == DT_BF16) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(f2bf_pack(v, 0.f) & 0xffffu), rs, off, 0, 0);
        else if (a.dt == DT_F32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, off, 0, 0);
        else __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, rs, off, 0, 0);
        break;
      }
      case OP_COPY: {
        switch (f_dst(w0) * 4 + f_a(w0)) {
          case 1: copy_c(t[0], t[1], G.nv); break;
          case 2: copy_c(t[0], t[2], G.nv); break;
          case 4: copy_c(t[1], t[0], G.nv); break;
          case 6: copy_c(t[1], t[2], G.nv); break;
          case 8: copy_c(t[2], t[0], G.nv); break;
          case 9: copy_c(t[2], t[1], G.nv); break;
          default: break;
        }
        break;
      }
      case OP_BIN: {
        const float rowv = f_bk(w0) == BK_RREG ? rget(rw, f_b(w0)) : 0.f;
        Chunks tmp;
        if (f_bk(w0) == BK_MEM) read_operand(tmp, w0, vmc_bin(w0), read_arg(W, w1), G, tl, L, S);
        switch (f_sub(w0)) {
          case ALU_ADD: bin_op<ALU_ADD>(t, w0, w1, rowv, tmp, G); break;
          case ALU_SUB: bin_op<ALU_SUB>(t, w0, w1, rowv, tmp, G); break;
          case ALU_MUL: bin_op<ALU_MUL>(t, w0, w1, rowv, tmp, G); break;
          case ALU_DIV: bin_op<ALU_DIV>(t, w0, w1, rowv, tmp, G); break;
          case ALU_MAX: bin_op<ALU_MAX>(t, w0, w1, rowv, tmp, G); break;
          case ALU_MIN: bin_op<ALU_MIN>(t, w0, w1, rowv, tmp, G); break;
          default: bin_op<ALU_POW>(t, w0, w1, rowv, tmp, G); break;
        }
        break;
      }
      case OP_UN: {
        switch (f_sub(w0)) {
          case UN_SQRT: un_c<UN_SQRT>(t[0], G.nv); break;
          case UN_ABS: un_c<UN_ABS>(t[0], G.nv); break;
          case UN_LOG: un_c<UN_LOG>(t[0], G.nv); break;
          case UN_EXP: un_c<UN_EXP>(t[0], G.nv); break;
          case UN_ROUND: un_c<UN_ROUND>(t[0], G.nv); break;
          case UN_FLOOR: un_c<UN_FLOOR>(t[0], G.nv); break;
          case UN_ISFINITE: un_c<UN_ISFINITE>(t[0], G.nv); break;
          case UN_NEG: un_c<UN_NEG>(t[0], G.nv); break;
          case UN_RECIP: un_c<UN_RECIP>(t[0], G.nv); break;
          case UN_TOBF16: un_c<UN_TOBF16>(t[0], G.nv); break;
          default: break;
        }
        break;
      }
      case OP_RBIN: {
        const float x = rget(rw, f_a(w0));
        const float y = f_bk(w0) == BK_RREG ? rget(rw, f_b(w0)) : __uint_as_float(w1);
        const bool rev = (f_flags(w0) & FL_REV) != 0;
        rset(rw, f_dst(w0), rev ? alu_rt(f_sub(w0), y, x) : alu_rt(f_sub(w0), x, y));
        break;
      }
      case OP_RUN:
        rset(rw, f_dst(w0), una_rt(f_sub(w0), rget(rw, f_a(w0))));
        break;
      case OP_BCAST: {
        const float v = rget(rw, f_a(w0));
        switch (f_dst(w0)) {
          case 0: fill_c(t[0], v); break;
          case 1: fill_c(t[1], v); break;
          default: fill_c(t[2], v); break;
        }
        break;
      }
      case OP_RED: {
        const uint32_t kind = f_sub(w0);
        float acc = lane_partial_any(t, f_a(w0), G, tl, L, kind);
        acc = group_reduce_k(acc, gs, kind);
        // after the 64-lane all-reduce every lane of a wave holds the same
        // value, so every lane stores it (no lane-dependent branch in the loop)
        if (G.g <= 64) rset(rw, f_dst(w0), acc);
        else s_red[f_b(w0)][wave] = acc;
        break;
      }
      case OP_RED_FIN: {
        const uint32_t kind = f_sub(w0);
        const int nw = G.g >> 6;
        const int base = L.row * nw;
        const float* buf = s_red[f_b(w0)];
        float acc = buf[base];
        for (int k = 1; k < nw; ++k) acc = comb_k(acc, buf[base + k], kind);
        rset(rw, f_dst(w0), acc);
        break;
      }
      case OP_SYNC:
        __syncthreads();
        break;
      case OP_ALL: {
        const uint32_t kind = f_sub(w0);
        float acc = lane_partial_any(t, f_a(w0), G, tl, L, kind);
        acc = group_reduce_k(acc, 64, kind);
        s_red[f_b(w0)][wave] = acc;
        break;
      }
      case OP_ALL_FIN: {
        // every lane combines the per-wave partials (LDS broadcast reads);
        // lane 0 alone stores the tile's partial, the others are masked by
        // an out-of-range offset
        const uint32_t kind = f_sub(w0);
        const float* buf = s_red[f_b(w0)];
        float acc = buf[0];
        for (int k = 1; k < T_LANES / 64; ++k) acc = comb_k(acc, buf[k], kind);
        const ArgD a = read_arg(W, W[H_ALL_SCRATCH]);
        const Rsrc rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a.p) + 256, 0, (int)(block_dim * 4u),
                                                          RSRC_W3);
        const int off = tidv == 0 ? (int)(tl.id * 4u) : OOB;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc), rs, off, 0, 0);
        break;
      }
      case OP_DBG: {
        const float v = f_sub(w0) == 0 ? (float)tl.id : (float)blockIdx.x;
        switch (f_dst(w0)) {
          case 0: fill_c(t[0], v); break;
          case 1: fill_c(t[1], v); break;
          default: fill_c(t[2], v); break;
        }
        break;
      }
      default:
        break;
    }
  }

  // Reduce-all epilogue: the last workgroup to finish combines the per-tile
  // partials in tile order (deterministic) and writes the scalar result.
  if (W[H_TEMPLATE] == TM_ALLREDUCE) {
    const uint32_t kind = W[H_ALL_KIND];
    const ArgD sa = read_arg(W, W[H_ALL_SCRATCH]);
    uint32_t* counter = reinterpret_cast<uint32_t*>(const_cast<char*>(sa.p));
    float* part = reinterpret_cast<float*>(const_cast<char*>(sa.p) + 256);
    __syncthreads();
    if (tid == 0) {
      __atomic_thread_fence(__ATOMIC_RELEASE);
      const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == gridDim.x - 1;
    }
    __syncthreads();
    if (s_last) {
      __atomic_thread_fence(__ATOMIC_ACQUIRE);
      float acc = kind == RK_SUM ? 0.f : -__builtin_huge_valf();
      for (uint32_t i = (uint32_t)tid; i < block_dim; i += T_LANES)
        acc = comb_k(acc, __hip_atomic_load(part + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), kind);
      acc = group_reduce_k(acc, 64, kind);
      if ((tid & 63) == 0) s_red[0][wave] = acc;
      __syncthreads();
      if (tid == 0) {
        float r = s_red[0][0];
        for (int k = 1; k < T_LANES / 64; ++k) r = comb_k(r, s_red[0][k], kind);
        const ArgD oa = read_arg(W, W[H_ALL_OUT]);
        if (oa.dt == DT_BF16)
          *reinterpret_cast<uint16_t*>(const_cast<char*>(oa.p)) = (uint16_t)(f2bf_pack(r, 0.f) & 0xffffu);
        else
          *reinterpret_cast<float*>(const_cast<char*>(oa.p)) = r;
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// Host-side launch of the VECTOR VM kernel with one program as its argument.
extern "C" hipError_t dvm_launch_vector_kernel(const Program* p, unsigned grid, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)dvm_vm_vector, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)LDS_BUDGET);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(dvm_vm_vector, dim3(grid), dim3(T_LANES), p->w[H_LDS_BYTES], s, *p);
  return hipGetLastError();
}
