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
// K runs in stages of 64 through two LDS buffers: while stage s is multiplied,
// the global loads of stage s + 1 are in flight (128-bit loads into registers,
// written to the other buffer after the stage).  A is stored row-major, B is
// stored transposed (one row per output column), so both operands are read
// with one 128-bit LDS load per lane; the 16-byte chunks of every row are
// XOR-swizzled so that the eight lanes of a read phase hit distinct banks.
//
// The epilogue (the program body) runs per 32 x 32 accumulator block with
// three 16-value tile registers (register 0 starts as the block of the matmul
// result); memory operands and stores address element (m, n) of the [M, N]
// space through buffer resources, out-of-range offsets masking the edges.
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
constexpr int KT = MM_KT;
constexpr int ROW_BYTES = KT * 2;     // one LDS row: 64 bf16 = 8 chunks of 16 bytes

struct ArgD {
  const char* p;
  uint32_t dt, fl;
  int64_t sr;
  int32_t sc;
  uint32_t extent;
};

__device__ __forceinline__ uint64_t w64(KW* w, int lo) { return ((uint64_t)w[lo + 1] << 32) | (uint64_t)w[lo]; }

__device__ __forceinline__ ArgD read_arg(KW* W, uint32_t i) {
  KW* a = W + ARG_BASE + i * ARG_WORDS;
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

__device__ __forceinline__ float alu_rt(uint32_t k, float x, float y) {
  switch (k) {
    case ALU_ADD: return x + y;
    case ALU_SUB: return x - y;
    case ALU_MUL: return x * y;
    case ALU_DIV: return x / y;
    case ALU_MAX: return (x != x || y != y) ? x + y : fmaxf(x, y);
    case ALU_MIN: return (x != x || y != y) ? x + y : fminf(x, y);
    default: return powf(x, y);
  }
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

// ---------------------------------------------------------------------------
// K loop (templated on the wave tile: BM x BN blocks of 32 x 32 per wave,
// four waves in a 2 x 2 arrangement)
// ---------------------------------------------------------------------------
// Byte offset of chunk kc (8 bf16 along K) of LDS row r, swizzled by s.
__device__ __forceinline__ int chunk_at(int r, int kc, int s) { return r * ROW_BYTES + ((kc ^ (s & 7)) << 4); }
__device__ __forceinline__ int a_swz(int row) { return row; }
__device__ __forceinline__ int b_swz(int n) { return n ^ (n >> 3); }

template <int BM, int BN>
struct Cfg {
  static constexpr int TM = 64 * BM, TN = 64 * BN;       // workgroup tile
  static constexpr int QA = TM * (KT / 8) / 256;         // A chunks per lane per stage
  static constexpr int QB = TN * (KT / 8) / 256;         // B chunks per lane per stage
  static constexpr int NCH = TN / 8;                     // B chunks per K row
  static constexpr int A_BYTES = TM * ROW_BYTES;         // one A stage
  static constexpr int B_BYTES = TN * ROW_BYTES;         // one B stage
  static constexpr int LDS = 2 * (A_BYTES + B_BYTES);
};

// A chunk c of a stage: row c / 8, K chunk c % 8 (eight lanes read one row's
// 128 contiguous bytes).  B chunk c: eight K rows by eight column chunks per
// wave (each column chunk's 128-byte line is still read whole by one wave),
// so the transposed 16-bit LDS writes of a wave spread over all banks.
__device__ __forceinline__ void a_chunk(int c, int& row, int& kc) {
  row = c >> 3;
  kc = c & 7;
}
template <int NCH>
__device__ __forceinline__ void b_chunk(int c, int& kr, int& nc) {
  const int rest = c >> 6;
  kr = ((rest & 7) << 3) | (c & 7);
  nc = ((rest >> 3) << 3) | ((c >> 3) & 7);
}

template <class CF>
struct Stage {
  u4 a[CF::QA], b[CF::QB];  // this lane's 16-byte chunks of the next A and B stages
};

// Global loads of the stage at k0; masked chunks read as zeros.
template <class CF>
__device__ __forceinline__ void load_stage(Stage<CF>& st, const Rsrc& ra, const Rsrc& rb, const ArgD& A,
                                           const ArgD& B, int64_t m0, int64_t n0, int k0, int64_t M, int64_t N,
                                           int K, int tid) {
#pragma unroll
  for (int q = 0; q < CF::QA; ++q) {
    int row, kc;
    a_chunk(tid + 256 * q, row, kc);
    const bool ok = (m0 + row < M) & (k0 + kc * 8 < K);
    st.a[q] = __builtin_amdgcn_raw_buffer_load_b128(ra, lane_off(ok, (row * (int)A.sr + k0 + kc * 8) * 2), 0, 0);
  }
#pragma unroll
  for (int q = 0; q < CF::QB; ++q) {
    int kr, nc;
    b_chunk<CF::NCH>(tid + 256 * q, kr, nc);
    const bool ok = (k0 + kr < K) & (n0 + nc * 8 < N);
    st.b[q] = __builtin_amdgcn_raw_buffer_load_b128(rb, lane_off(ok, ((k0 + kr) * (int)B.sr + nc * 8) * 2), 0, 0);
  }
}

// Writes of the loaded stage to LDS buffers (A row-major, B transposed).
template <class CF>
__device__ __forceinline__ void write_stage(const Stage<CF>& st, char* abuf, char* bbuf, int tid) {
#pragma unroll
  for (int q = 0; q < CF::QA; ++q) {
    int row, kc;
    a_chunk(tid + 256 * q, row, kc);
    *(u4*)(abuf + chunk_at(row, kc, a_swz(row))) = st.a[q];
  }
#pragma unroll
  for (int q = 0; q < CF::QB; ++q) {
    int kr, nc;
    b_chunk<CF::NCH>(tid + 256 * q, kr, nc);
    const u4 v = st.b[q];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = nc * 8 + j;
      const uint32_t w = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
      const uint16_t h = (uint16_t)((j & 1) ? (w >> 16) : (w & 0xffffu));
      *(uint16_t*)(bbuf + chunk_at(n, kr >> 3, b_swz(n)) + (kr & 7) * 2) = h;
    }
  }
}

__device__ __forceinline__ bf8 read_frag(const char* buf, int r, int kc, int s) {
  return *(const bf8*)(buf + chunk_at(r, kc, s));
}

// One stage of KT values of K on this wave's BM x BN blocks.
template <int BM, int BN>
__device__ __forceinline__ void mma_stage(f16v (&c)[BM][BN], const char* abuf, const char* bbuf, int wm, int wn,
                                          int lane) {
#pragma unroll
  for (int kk = 0; kk < KT / 16; ++kk) {
    const int kc = kk * 2 + (lane >> 5);
    bf8 a[BM], b[BN];
#pragma unroll
    for (int i = 0; i < BM; ++i) {
      const int r = wm * 32 * BM + i * 32 + (lane & 31);
      a[i] = read_frag(abuf, r, kc, a_swz(r));
    }
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      const int n = wn * 32 * BN + j * 32 + (lane & 31);
      b[j] = read_frag(bbuf, n, kc, b_swz(n));
    }
#pragma unroll
    for (int i = 0; i < BM; ++i)
#pragma unroll
      for (int j = 0; j < BN; ++j) c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], c[i][j], 0, 0, 0);
  }
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Epilogue: the program body on one 32 x 32 block
// ---------------------------------------------------------------------------
struct T16 {
  float v[16];
};

struct Blk {
  int64_t mb, nb;  // block origin in [M, N]
  int64_t M, N;
  int lane;
};

// row of accumulator register i for this lane, relative to the block
__device__ __forceinline__ int dm_of(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

__device__ __forceinline__ void epi_load(T16& d, const ArgD& a, const Blk& B) {
  const int es = esize(a.dt);
  const Rsrc rs = rsrc_at(a, (B.mb * a.sr + B.nb * (int64_t)a.sc) * es);
  const int dn = B.lane & 31;
  const bool nok = B.nb + dn < B.N;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int dm = dm_of(i, B.lane);
    const int off = lane_off(nok & (B.mb + dm < B.M), (dm * (int)a.sr + dn * a.sc) * es);
    float x;
    if (a.dt == DT_BF16) x = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
    else if (a.dt == DT_F32) x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
    else x = (float)__builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0);
    d.v[i] = x;
  }
}

__device__ __forceinline__ void epi_store(const T16& s, const ArgD& a, const Blk& B) {
  const int es = esize(a.dt);
  const Rsrc rs = rsrc_at(a, (B.mb * a.sr + B.nb * (int64_t)a.sc) * es);
  const int dn = B.lane & 31;
  const bool nok = B.nb + dn < B.N;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int dm = dm_of(i, B.lane);
    const int off = lane_off(nok & (B.mb + dm < B.M), (dm * (int)a.sr + dn * a.sc) * es);
    const float x = s.v[i];
    if (a.dt == DT_BF16) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(f2bf_pack(x, 0.f) & 0xffffu), rs, off, 0, 0);
    else if (a.dt == DT_F32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs, off, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b8((uint8_t)x, rs, off, 0, 0);
  }
}

__device__ __forceinline__ void pick(T16& d, uint32_t k, const T16& t0, const T16& t1, const T16& t2) {
  if (k == 0) d = t0;
  else if (k == 1) d = t1;
  else d = t2;
}

__device__ __forceinline__ void put(uint32_t k, const T16& s, T16& t0, T16& t1, T16& t2) {
  if (k == 0) t0 = s;
  else if (k == 1) t1 = s;
  else t2 = s;
}

template <uint32_t OPK>
__device__ __forceinline__ void bin16(T16& acc, const T16& b, bool rev) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float x = acc.v[i], y = b.v[i];
    acc.v[i] = rev ? alu_rt(OPK, y, x) : alu_rt(OPK, x, y);
  }
}

__device__ __forceinline__ void run_epilogue(KW* W, T16& t0, const Blk& B) {
  T16 t1, t2;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    t1.v[i] = 0.f;
    t2.v[i] = 0.f;
  }
  const uint32_t pc_end = W[H_BODY_END];
  for (uint32_t pc = W[H_BODY_BEGIN]; pc < pc_end; pc += 2) {
    const uint32_t w0 = W[pc], w1 = W[pc + 1];
    switch (f_op(w0)) {
      case OP_LOAD: {
        T16 m;
        epi_load(m, read_arg(W, w1), B);
        put(f_dst(w0), m, t0, t1, t2);
        break;
      }
      case OP_STORE: {
        T16 m;
        pick(m, f_a(w0), t0, t1, t2);
        epi_store(m, read_arg(W, w1), B);
        break;
      }
      case OP_COPY: {
        T16 m;
        pick(m, f_a(w0), t0, t1, t2);
        put(f_dst(w0), m, t0, t1, t2);
        break;
      }
      case OP_BIN: {
        T16 b;
        const uint32_t bk = f_bk(w0);
        if (bk == BK_MEM) epi_load(b, read_arg(W, w1), B);
        else if (bk == BK_TREG) pick(b, f_b(w0), t0, t1, t2);
        else {
#pragma unroll
          for (int i = 0; i < 16; ++i) b.v[i] = __uint_as_float(w1);
        }
        const bool rev = (f_flags(w0) & FL_REV) != 0;
        switch (f_sub(w0)) {
          case ALU_ADD: bin16<ALU_ADD>(t0, b, rev); break;
          case ALU_SUB: bin16<ALU_SUB>(t0, b, rev); break;
          case ALU_MUL: bin16<ALU_MUL>(t0, b, rev); break;
          case ALU_DIV: bin16<ALU_DIV>(t0, b, rev); break;
          case ALU_MAX: bin16<ALU_MAX>(t0, b, rev); break;
          case ALU_MIN: bin16<ALU_MIN>(t0, b, rev); break;
          default: bin16<ALU_POW>(t0, b, rev); break;
        }
        break;
      }
      case OP_UN: {
        const uint32_t f = f_sub(w0);
#pragma unroll
        for (int i = 0; i < 16; ++i) t0.v[i] = una_rt(f, t0.v[i]);
        break;
      }
      default:
        break;
    }
  }
}

__device__ __forceinline__ void to16(T16& d, const f16v& c) {
#pragma unroll
  for (int i = 0; i < 16; ++i) d.v[i] = c[i];
}

template <int BM, int BN>
__device__ __forceinline__ void mix_body(char* lds) {
  using CF = Cfg<BM, BN>;
  KW* W = (KW*)__builtin_amdgcn_kernarg_segment_ptr();
  const uint32_t block_dim = W[H_BLOCK_DIM];
  const uint32_t body_tile = W[H_BODY_TILE];
  const uint32_t nct = W[H_NC];
  const int64_t M = (int64_t)w64(W, H_R_LO);
  const int64_t N = (int64_t)w64(W, H_C_LO);
  const int K = (int)W[H_MM_K];
  const ArgD A = read_arg(W, W[H_MM_A]);
  const ArgD Bm = read_arg(W, W[H_MM_B]);
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1, wn = wave & 1;
  const int n_stage = (K + KT - 1) / KT;
  char* const abuf0 = lds;
  char* const bbuf0 = lds + 2 * CF::A_BYTES;

  const uint32_t t_begin = blockIdx.x * body_tile;
  uint32_t t_end = t_begin + body_tile;
  if (t_end > block_dim) t_end = block_dim;

  for (uint32_t tile = t_begin; tile < t_end; ++tile) {
    const uint32_t ir = tile / nct, ic = tile - ir * nct;
    const int64_t m0 = (int64_t)ir * CF::TM, n0 = (int64_t)ic * CF::TN;
    const Rsrc ra = rsrc_at(A, m0 * A.sr * 2);
    const Rsrc rb = rsrc_at(Bm, n0 * 2);
    f16v c[BM][BN];
#pragma unroll
    for (int i = 0; i < BM; ++i)
#pragma unroll
      for (int j = 0; j < BN; ++j) c[i][j] = (f16v)0.f;

    Stage<CF> st;
    load_stage<CF>(st, ra, rb, A, Bm, m0, n0, 0, M, N, K, tid);
    write_stage<CF>(st, abuf0, bbuf0, tid);
    lds_barrier();
    for (int s = 0; s < n_stage; ++s) {
      const int cur = s & 1;
      const bool more = s + 1 < n_stage;
      if (more) load_stage<CF>(st, ra, rb, A, Bm, m0, n0, (s + 1) * KT, M, N, K, tid);
      mma_stage<BM, BN>(c, abuf0 + cur * CF::A_BYTES, bbuf0 + cur * CF::B_BYTES, wm, wn, lane);
      if (more) write_stage<CF>(st, abuf0 + (cur ^ 1) * CF::A_BYTES, bbuf0 + (cur ^ 1) * CF::B_BYTES, tid);
      lds_barrier();
    }

    // epilogue per 32 x 32 block
    Blk B;
    B.M = M;
    B.N = N;
    B.lane = lane;
#pragma nounroll
    for (int blk = 0; blk < BM * BN; ++blk) {
      const int bi = blk / BN, bj = blk % BN;
      B.mb = m0 + wm * 32 * BM + bi * 32;
      B.nb = n0 + wn * 32 * BN + bj * 32;
      T16 t0;
#pragma unroll
      for (int q = 0; q < BM * BN; ++q)
        if (q == blk) to16(t0, c[q / BN][q % BN]);
      run_epilogue(W, t0, B);
    }
  }
}

}  // namespace

// 128 x 128 tiles, two workgroups per compute unit.
extern "C" __global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
dvm_vm_mix_128(const Program prog) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  (void)prog;
  mix_body<2, 2>(lds);
}

// Host-side launch of the MIX VM kernel matching the program's tile.
extern "C" hipError_t dvm_launch_mix_kernel(const Program* p, unsigned grid, hipStream_t s) {
  using Small = Cfg<2, 2>;
  constexpr int lds_small = Small::LDS;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)dvm_vm_mix_128, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       lds_small);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  if (p->w[H_TR] != (uint32_t)Small::TM || p->w[H_TC] != (uint32_t)Small::TN) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dvm_vm_mix_128, dim3(grid), dim3(256), lds_small, s, *p);
  return hipGetLastError();
}
