// Host side of the DVM hot path: streaming fuser, shape tiling, bytecode
// encoder and the C ABI declared in include/dvm.h.
//
// Sources: the DVM paper review page (section 4.2 shape tiling, 4.3 bytecode
// format, 4.4 VM execution, 5.1 pattern fusion, 5.2 dynamic-graph streaming
// fusion) and the MindSpore DVM summary page (sections 3.2-3.3: runtime
// capture, flush at unsupported ops / fusion boundaries / sync interfaces).
// The readings taken where the pages are silent are stated next to the code.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <array>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <deque>
#include <mutex>
#include <string>
#include <vector>

#include "bytecode.h"
#include "dvm.h"

using namespace dvmbc;

namespace dvmbc {
bool verify_words(const uint32_t* W, uint32_t n_words, std::string* err);  // verify.cpp
}

extern "C" hipError_t dvm_launch_vector_kernel(const Program* p, unsigned grid, unsigned lds, hipStream_t s);
extern "C" hipError_t dvm_launch_mix_kernel(const Program* p, unsigned grid, hipStream_t s);
extern "C" hipError_t dvm_launch_vector_prof_kernel(const Program* p, unsigned grid, hipStream_t s);
extern "C" hipError_t dvm_launch_vector_kernel_wide(const Program* p, unsigned grid, unsigned lds, hipStream_t s);
extern "C" hipError_t dvm_launch_vector_prof_kernel_wide(const Program* p, unsigned grid, hipStream_t s);
extern "C" hipError_t dvm_static_scratch_init(int device, void** ptr, size_t* bytes);
extern "C" hipError_t dvm_launch_allreduce_combine(const float* part, uint32_t n_part, uint32_t kind, void* out,
                                                   uint32_t out_dt, hipStream_t s);

namespace {

thread_local std::string g_err;

dvm_status fail(dvm_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

int esize(int32_t dt) { return dt == DVM_F32 ? 4 : dt == DVM_BF16 ? 2 : 1; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ===========================================================================
// Shapes
// ===========================================================================
static int64_t numel_of(const dvm_tensor& t) {
  int64_t n = 1;
  for (int i = 0; i < t.ndim; ++i) n *= t.shape[i];
  return n;
}

struct Shape {
  int nd = 0;
  int64_t d[4] = {0, 0, 0, 0};
  int64_t numel() const {
    int64_t n = 1;
    for (int i = 0; i < nd; ++i) n *= d[i];
    return n;
  }
  bool operator==(const Shape& o) const {
    if (nd != o.nd) return false;
    for (int i = 0; i < nd; ++i)
      if (d[i] != o.d[i]) return false;
    return true;
  }
  bool operator!=(const Shape& o) const { return !(*this == o); }
};

Shape shape_of(const dvm_tensor& t) {
  Shape s;
  s.nd = t.ndim;
  for (int i = 0; i < t.ndim; ++i) s.d[i] = t.shape[i];
  return s;
}

Shape row_shape(const Shape& s) {
  Shape r = s;
  if (r.nd) r.d[r.nd - 1] = 1;
  return r;
}

bool broadcast(const Shape& a, const Shape& b, Shape* out) {
  Shape o;
  o.nd = std::max(a.nd, b.nd);
  for (int i = 0; i < o.nd; ++i) {
    const int ia = a.nd - o.nd + i, ib = b.nd - o.nd + i;
    const int64_t da = ia >= 0 ? a.d[ia] : 1, db = ib >= 0 ? b.d[ib] : 1;
    if (da != db && da != 1 && db != 1) return false;
    o.d[i] = da == 1 ? db : da;
  }
  *out = o;
  return true;
}

// strides of a tensor broadcast (numpy rules) to target
void bcast_strides(const dvm_tensor& t, const Shape& target, int64_t* out) {
  const int off = target.nd - t.ndim;
  for (int j = 0; j < target.nd; ++j) out[j] = 0;
  for (int i = 0; i < t.ndim; ++i) {
    const int j = off + i;
    out[j] = (t.shape[i] == 1 && target.d[j] != 1) ? 0 : t.stride[i];
  }
}

// Bytes spanned by a tensor (one past its last element).
int64_t extent_bytes(const dvm_tensor& t) {
  int64_t n = 1, last = 0;
  for (int i = 0; i < t.ndim; ++i) {
    n *= t.shape[i];
    last += (t.shape[i] - 1) * t.stride[i];
  }
  if (n == 0) return 0;
  return (last + 1) * esize(t.dtype);
}

// ===========================================================================
// Shape tiling (DVM review page, section 4.2)
//
// Readings taken (the page gives the steps, not the constants):
//  * the dominant shape is collapsed to [R, C] (C innermost); elementwise
//    graphs whose operands are all contiguous collapse to [1, numel];
//  * a tile is tr x tc; its rows go to P = next_pow2(tr) lane groups of
//    g = T / P lanes; each lane holds NV = ceil((tc + pad) / (g V)) chunks of
//    V elements and the tile is feasible iff P <= T and NV <= NV_MAX (the
//    per-core resource limit: the lane's share of a tile register);
//  * pad = V - 1 if some unit-stride operand's rows are not 16-byte aligned;
//  * hardware_align_div(n, k, W) = W ceil(ceil(n / k) / W), W = 64 V, is the
//    width one wave moves with 16-byte accesses of the narrowest type;
//  * the shrink path goes outer -> inner (rows first, then columns) by
//    doubling the split count k;
//  * cost in integer ticks (1/15625 us): G = 512 resident workgroups (two
//    per CU), A = 78125 ticks (5 us) per round of tiles, 1 tick per byte
//    per workgroup (8 TB/s shared by G workgroups).  A is the measured
//    marginal cost of one more round on latency-bound calls (LayerNorm over
//    1385 rows of 5120: 3 rounds 21.8 us, 2 rounds 15.4 us, of which the
//    bytes account for about 1.3 us);
//    cost = ceil(n_tiles / G) (A + var_bytes) + inv_bytes; least cost wins,
//    earlier (larger) candidates win ties.
// ===========================================================================
namespace tiling {
constexpr int64_t T = T_LANES, V = VEC, W = 64 * VEC, G = 512, A = 78125, A_MM = 7812, BT = 1;
// A wide-build program with more than WIDE_WG_TILES tiles per workgroup
// runs as min(WIDE_GRID_MAX, block_dim / WIDE_WG_TILES) workgroups, more than
// are resident: the two workgroups sharing a compute unit stream at unequal
// rates, and the dispatcher then hands the next workgroup to the slot that
// frees first (measured on MI355X; standard-build programs keep G).
constexpr int64_t WIDE_WG_TILES = 8, WIDE_GRID_MAX = 8192;

struct Operand {
  int64_t esize, sr, sc, base_mod16;
};

struct Plan {
  int tmpl = 0;
  int64_t R = 0, C = 0, pad = 0;
  int64_t tr = 0, tc = 0, g = 0, nv = 0, P = 0, n_r = 0, n_c = 0, block_dim = 0, body_tile = 0, grid = 0;
};

int64_t next_pow2(int64_t x) {
  int64_t p = 1;
  while (p < x) p *= 2;
  return p;
}
int64_t had(int64_t n, int64_t k, int64_t w) { return w * cdiv(cdiv(n, k), w); }

// Collapse the dominant shape to [R, C].  strides: per operand, strides over
// shape.  Returns false if some operand's outer dims cannot merge.
bool collapse(int tmpl, const Shape& shape, const std::vector<std::array<int64_t, 4>>& strides, int64_t* R,
              int64_t* C, std::vector<std::pair<int64_t, int64_t>>* out) {
  out->clear();
  const int64_t numel = shape.numel();
  if (numel == 0) {
    *R = 0;
    *C = 0;
    for (size_t i = 0; i < strides.size(); ++i) out->push_back({0, 0});
    return true;
  }
  // drop unit dims
  int keep[4], nk = 0;
  for (int i = 0; i < shape.nd; ++i)
    if (shape.d[i] != 1) keep[nk++] = i;
  if (nk == 0) {
    *R = 1;
    *C = 1;
    for (size_t i = 0; i < strides.size(); ++i) out->push_back({0, 0});
    return true;
  }
  auto mergeable = [&](const std::array<int64_t, 4>& s, int lo, int hi) {
    for (int i = lo; i < hi - 1; ++i)
      if (s[keep[i]] != s[keep[i + 1]] * shape.d[keep[i + 1]]) return false;
    return true;
  };
  if (tmpl == TM_ELEMWISE || tmpl == TM_ALLREDUCE) {
    bool all = true;
    for (auto& s : strides) all = all && mergeable(s, 0, nk);
    if (all) {
      *R = 1;
      *C = numel;
      for (auto& s : strides) out->push_back({0, s[keep[nk - 1]]});
      return true;
    }
  }
  const int64_t Cd = shape.nd ? shape.d[shape.nd - 1] : 1;
  const int no = Cd == 1 ? nk : nk - 1;  // outer (kept) dims
  int64_t Rr = 1;
  for (int i = 0; i < no; ++i) Rr *= shape.d[keep[i]];
  for (auto& s : strides) {
    if (!mergeable(s, 0, no)) return false;
    const int64_t sr = no ? s[keep[no - 1]] : 0;
    const int64_t sc = Cd != 1 ? s[shape.nd - 1] : 0;
    out->push_back({sr, sc});
  }
  *R = Rr;
  *C = Cd;
  return true;
}

int64_t alignment_pad(int64_t R, const std::vector<Operand>& ops) {
  for (auto& o : ops) {
    if (o.sc != 1) continue;
    if (o.base_mod16 % 16 != 0) return V - 1;
    if (R > 1 && ((o.sr * o.esize) % 16 + 16) % 16 != 0) return V - 1;
  }
  return 0;
}

bool geometry(int64_t tr, int64_t tc, int64_t pad, int64_t nvm, int64_t* P, int64_t* g, int64_t* nv) {
  *P = next_pow2(tr);
  if (*P > T) return false;
  *g = T / *P;
  *nv = cdiv(tc + pad, *g * V);
  return *nv <= nvm;
}

void shrink_path(int tmpl, int64_t R, int64_t C, std::vector<std::pair<int64_t, int64_t>>* path) {
  path->clear();
  auto push = [&](int64_t a, int64_t b) {
    if (path->empty() || path->back() != std::make_pair(a, b)) path->push_back({a, b});
  };
  // each row count is followed by its power-of-two floor, the largest tile
  // whose rows fill their lane groups (tr = 3 leaves one of 4 idle)
  auto push_rows = [&](int64_t tr, int64_t tc) {
    push(tr, tc);
    int64_t f = 1;
    while (f * 2 <= tr) f *= 2;
    push(f, tc);
  };
  if (tmpl == TM_ROWREDUCE) {
    for (int64_t k = 1;; k *= 2) {
      const int64_t tr = cdiv(R, k);
      push_rows(tr, C);
      if (tr <= 1) break;
    }
    return;
  }
  const int64_t tc0 = std::min(C, had(C, 1, W));
  for (int64_t k = 1;; k *= 2) {
    const int64_t tr = cdiv(R, k);
    push_rows(tr, tc0);
    if (tr <= 1) break;
  }
  int64_t prev = tc0;
  for (int64_t k = 2; prev > W; k *= 2) {
    const int64_t tc = std::min(C, had(C, k, W));
    if (tc == prev) break;
    push(1, tc);
    prev = tc;
  }
}

int64_t cost(int64_t R, int64_t C, int64_t tr, int64_t tc, const std::vector<Operand>& ops) {
  const int64_t n_r = cdiv(R, tr), n_c = cdiv(C, tc), n_tiles = n_r * n_c;
  int64_t var_b = 0, inv_b = 0;
  for (auto& o : ops) {
    const int64_t touched = (o.sr != 0 ? tr : 1) * (o.sc != 0 ? tc : 1) * o.esize;
    const bool invariant = (o.sr == 0 || n_r == 1) && (o.sc == 0 || n_c == 1);
    (invariant ? inv_b : var_b) += touched;
  }
  return cdiv(n_tiles, G) * (A + BT * var_b) + BT * inv_b;
}

void header(int64_t block_dim, int64_t* body_tile, int64_t* grid, int64_t g_res = G) {
  if (block_dim == 0) {
    *body_tile = 0;
    *grid = 0;
    return;
  }
  const int64_t gp = std::min(g_res, block_dim);
  *body_tile = cdiv(block_dim, gp);
  *grid = cdiv(block_dim, *body_tile);
}

// MATMUL graphs: K pinned; output tiles from the MIX kernel's variants (tm,
// tn, resident workgroups G_e), largest first.  With G_e workgroups sharing
// 8 TB/s and 2.5 PFLOP/s, a byte costs G_e / 512 ticks and a flop G_e / 160000:
// cost = ceil(n_tiles / G_e) (A_MM + ceil(var_bytes G_e / 512) + ceil(2 tm tn K G_e / 160000))
//        + ceil(inv_bytes G_e / 512), A_MM = 7812 ticks (0.5 us: a MIX tile's fixed
// work is small next to its K loop); least cost wins, ties to the earlier entry.
struct MmTile {
  int64_t tm, tn, g;
};
constexpr MmTile MM_TILES[] = {{128, 128, 512}};

bool plan_matmul(int64_t M, int64_t N, int64_t K, int64_t a_es, int64_t b_es, const std::vector<Operand>& ops,
                 Plan* p) {
  *p = Plan();
  p->tmpl = TM_MATMUL;
  p->R = M;
  p->C = N;
  if (M == 0 || N == 0) return true;
  bool found = false;
  int64_t best = 0, best_g = G;
  for (const MmTile& t : MM_TILES) {
    const int64_t n_r = cdiv(M, t.tm), n_c = cdiv(N, t.tn);
    int64_t var_b = t.tm * K * a_es + K * t.tn * b_es, inv_b = 0;
    for (auto& o : ops) {
      const int64_t touched = (o.sr != 0 ? t.tm : 1) * (o.sc != 0 ? t.tn : 1) * o.esize;
      const bool invariant = (o.sr == 0 || n_r == 1) && (o.sc == 0 || n_c == 1);
      (invariant ? inv_b : var_b) += touched;
    }
    const int64_t per_tile = A_MM + cdiv(var_b * t.g, 512) + cdiv(2 * t.tm * t.tn * K * t.g, 160000);
    const int64_t c = cdiv(n_r * n_c, t.g) * per_tile + cdiv(inv_b * t.g, 512);
    if (!found || c < best) {
      found = true;
      best = c;
      best_g = t.g;
      p->tr = t.tm;
      p->tc = t.tn;
    }
  }
  p->n_r = cdiv(M, p->tr);
  p->n_c = cdiv(N, p->tc);
  p->block_dim = p->n_r * p->n_c;
  header(p->block_dim, &p->body_tile, &p->grid, best_g);
  return true;
}

// nvm: chunks per lane of the VM variant (NV_MAX standard, NV_WIDE wide)
bool plan(int tmpl, int64_t R, int64_t C, const std::vector<Operand>& ops, Plan* p, int64_t nvm = NV_MAX) {
  *p = Plan();
  p->tmpl = tmpl;
  p->R = R;
  p->C = C;
  p->pad = alignment_pad(R, ops);
  if (R == 0 || C == 0) return true;
  std::vector<std::pair<int64_t, int64_t>> path;
  shrink_path(tmpl, R, C, &path);
  bool found = false;
  int64_t best = 0;
  for (auto& [tr, tc] : path) {
    int64_t P, g, nv;
    if (!geometry(tr, tc, p->pad, nvm, &P, &g, &nv)) continue;
    const int64_t c = cost(R, C, tr, tc, ops);
    if (!found || c < best) {
      found = true;
      best = c;
      p->tr = tr;
      p->tc = tc;
      p->P = P;
      p->g = g;
      p->nv = nv;
    }
  }
  if (!found) return false;
  p->n_r = cdiv(R, p->tr);
  p->n_c = cdiv(C, p->tc);
  p->block_dim = p->n_r * p->n_c;
  header(p->block_dim, &p->body_tile, &p->grid);
  if (nvm == NV_WIDE && p->body_tile > WIDE_WG_TILES)
    header(p->block_dim, &p->body_tile, &p->grid, std::min(WIDE_GRID_MAX, p->block_dim / WIDE_WG_TILES));
  return true;
}
}  // namespace tiling

// ===========================================================================
// Graph state
// ===========================================================================
enum ValKind : int { VK_INPUT = 0, VK_OP = 1 };

struct Val {
  uint32_t gen = 0;
  bool alive = false;  // slot in use
  int kind = VK_INPUT;
  dvm_tensor t{};       // inputs: the tensor; op outputs: dtype, shape, storage (data may be NULL)
  Shape shape;
  bool live = false;      // DVM_OUT_LIVE
  bool released = false;
  bool pending = false;   // produced by an op in the buffered graph or the open group
  bool stored = false;    // materialised in its storage by a flushed graph
  bool lost = false;      // its graph was flushed without storing it
  int uses = 0;           // inputs of ops still in the buffer or the open group
};

struct OpRec {
  int32_t op = 0;
  int n_in = 0;
  int64_t in[2] = {-1, -1};
  int scalar_pos = -1;
  float scalar = 0.f;
  int axis = -1;
  int64_t out = -1;  // value slot index
};

// Internal op of fused graphs (never added through the ABI): z / (exp(-z) + 1),
// a SiLU chain the encoder fused (fuse_silu).
constexpr int32_t OP_SILU = DVM_OP_COUNT;

bool is_reduce(int op) { return op == DVM_OP_REDUCE_SUM || op == DVM_OP_REDUCE_MAX; }
bool is_reduce_all(const OpRec& o) { return is_reduce(o.op) && o.axis == DVM_AXIS_ALL; }
bool is_binary(int op) { return op <= DVM_OP_POW; }

enum FlushReason { FR_EXPLICIT = 0, FR_SYNC = 1, FR_REDUCE_ALL = 2, FR_SHAPE = 3, FR_PATTERN = 4, FR_DEPENDENCE = 5,
                   FR_RESOURCE = 6, FR_BRANCH = 7 };

}  // namespace

// Reduce-all scratch: a counter (4 bytes) and the per-tile partials from byte
// 256.  One area per stream, allocated at the first reduce-all launched on
// that stream: launches on one stream run one after another, and launches on
// different streams never share the counter or the partials.
constexpr size_t SCRATCH_BYTES = 4u << 20;
constexpr size_t SCRATCH_PART_OFF = 256;

// A reduce-all's combine held back on its stream: the branch program opened
// on the reduce-all's scalar folds the partials itself (HF_COND_FOLD).
struct HeldCombine {
  hipStream_t s;
  const float* part;
  uint32_t n_part, kind;
  void* out;
  uint32_t out_dt;
};

struct dvm_context {
  int device = -1;
  std::mutex mu;  // guards scratch and held (graphs of one context may run on separate threads)
  std::vector<std::pair<hipStream_t, void*>> scratch;
  // combines held back (at most one per stream), and the stream whose next
  // reduce-all launch holds its combine back (set while a branch opens)
  std::vector<HeldCombine> held;
  hipStream_t hold_stream = nullptr;
  bool hold = false;
  // the device's static scratch array (dvm_launch_noalloc), looked up at creation
  void* static_scratch = nullptr;
  size_t static_bytes = 0;
  hipError_t static_err = hipSuccess;
};

using Range = std::pair<uintptr_t, uint64_t>;  // (address, bytes spanned)

struct dvm_program {
  Program prog;
  uint64_t bytes = 0;         // physical bytes: every operand read once, every stored output written once
  uint32_t n_words = 0;
  uint32_t n_instr = 0;
  int64_t R = 0, C = 0;
  uint32_t pad = 0;
  uint32_t grid_launch = 0;   // workgroups actually launched (reduce-all always launches >= 1)
  uint32_t segments = 1;      // > 1: a stacked program (a directory, then the segments)
  uint32_t lds = 0;           // dynamic LDS of the launch (bytes)
  std::vector<Range> reads, writes;  // memory the program reads and writes (stacking independence)
};

struct dvm_graph {
  dvm_context* ctx = nullptr;
  hipStream_t stream = nullptr;
  std::vector<Val> vals;
  std::vector<int64_t> free_slots;
  std::vector<OpRec> buf;   // buffered (fused) graph
  std::vector<OpRec> grp;   // open group
  bool in_group = false;
  dvm_stats stats{};
  struct LogEntry {
    int32_t ops, reason;
    float encode_us;
    uint64_t bytes;
  };
  std::vector<LogEntry> flush_log;  // per flushed graph
  // encode-only contexts cannot launch: programs of implicit flushes wait
  // here for dvm_graph_take_program (oldest first, at most MAX_HELD)
  std::deque<dvm_program*> held;
  std::vector<int32_t> remap;  // slot -> local index while a local view is built (-1 otherwise)
  // stacking: up to stack_max independent programs wait here and launch as one
  int stack_max = 1;
  bool stack_temporal = false;  // launch the stack temporally (segments in sequence per workgroup)
  std::vector<dvm_program*> stack;
  // a branch being captured: 1 then-ops, 2 else-ops (0 none)
  int branch = 0;
  int64_t branch_cond = -1;
  float branch_thr = 0.f;
  std::vector<OpRec> br[2];
  ~dvm_graph();
};
constexpr size_t MAX_HELD = 4096;

dvm_graph::~dvm_graph() {
  for (dvm_program* p : held) delete p;
  for (dvm_program* p : stack) delete p;
}

namespace {

// value handle = slot | gen << 32
dvm_value handle(const dvm_graph* g, int64_t slot) { return (dvm_value)(slot | ((int64_t)g->vals[slot].gen << 32)); }

bool resolve(const dvm_graph* g, dvm_value h, int64_t* slot) {
  const int64_t s = h & 0xffffffffLL;
  const uint32_t gen = (uint32_t)((uint64_t)h >> 32);
  if (s < 0 || s >= (int64_t)g->vals.size()) return false;
  const Val& v = g->vals[s];
  if (!v.alive || v.gen != gen) return false;
  *slot = s;
  return true;
}

int64_t new_slot(dvm_graph* g) {
  int64_t s;
  if (!g->free_slots.empty()) {
    s = g->free_slots.back();
    g->free_slots.pop_back();
  } else {
    s = (int64_t)g->vals.size();
    g->vals.emplace_back();
  }
  Val& v = g->vals[s];
  const uint32_t gen = v.gen + 1;
  v = Val();
  v.gen = gen;
  v.alive = true;
  return s;
}

void recycle(dvm_graph* g, int64_t s) {
  Val& v = g->vals[s];
  v.alive = false;
  g->free_slots.push_back(s);
}

// A released value's slot is reused only once no buffered op refers to it.
void maybe_recycle(dvm_graph* g, int64_t s) {
  Val& v = g->vals[s];
  if (v.alive && v.released && !v.pending && v.uses == 0) recycle(g, s);
}

// The ops leave the buffer (flushed or rejected): drop their input references.
void drop_uses(dvm_graph* g, const std::vector<OpRec>& ops) {
  for (auto& o : ops)
    for (int k = 0; k < o.n_in; ++k) g->vals[o.in[k]].uses--;
  for (auto& o : ops) {
    for (int k = 0; k < o.n_in; ++k) maybe_recycle(g, o.in[k]);
    maybe_recycle(g, o.out);
  }
}

// A fused graph over dense local value indices: copies of the values its ops
// use, numbered in order of first appearance.  The checker and the encoder
// run on it, so their per-value tables are sized by the graph (a few dozen
// values), not by every value the stream has created so far.
struct LocalView {
  dvm_graph lg;                  // only ctx and vals are set
  std::vector<OpRec> ops;
};

void make_local(dvm_graph* g, const std::vector<OpRec>& ops, LocalView* L) {
  std::vector<int32_t>& rm = g->remap;
  if (rm.size() < g->vals.size()) rm.resize(g->vals.size(), -1);
  L->lg.ctx = g->ctx;
  L->lg.stream = g->stream;
  L->lg.vals.clear();
  L->ops = ops;
  std::vector<int64_t> used;
  used.reserve(3 * ops.size());
  auto loc = [&](int64_t s) -> int64_t {
    if (rm[s] < 0) {
      rm[s] = (int32_t)L->lg.vals.size();
      L->lg.vals.push_back(g->vals[s]);
      used.push_back(s);
    }
    return rm[s];
  };
  for (OpRec& o : L->ops) {
    for (int k = 0; k < o.n_in; ++k) o.in[k] = loc(o.in[k]);
    o.out = loc(o.out);
  }
  for (int64_t s : used) rm[s] = -1;
}

// ===========================================================================
// Fusion rules (DVM review page, section 5.2; MindSpore summary, 3.2-3.3).
//
// Readings taken:
//  * the unit of decision is a group (one op, or a composite the caller
//    brackets); the group joins the buffered graph or the graph is flushed;
//  * iteration shape: elementwise op = its output shape, reduce = its input
//    shape, matmul = its [M, N] output; the dominant shape S_d is the
//    iteration shape of largest rank, then numel, then the earliest;
//  * pattern: reduces iterate over S_d, every other op over S_d or row(S_d);
//    matmul only as the first op and with no reduce; a reduce-all is the last
//    op (the graph closes) and does not mix with row reduces;
//  * dependence through memory: no WAR, RAW or WAW between the new group and
//    the buffered graph except through values;
//  * resources: <= 64 ops, <= 24 external tensors, <= 3 tile values and <= 4
//    row values in flight at every op, and a feasible tiling.
// ===========================================================================
constexpr int MAX_OPS = 64, MAX_EXT = 24, MAX_TILE_VALUES = 3, MAX_ROW_VALUES = 4;

struct Checker {
  dvm_graph* g;
  const std::vector<OpRec>& ops;
  std::vector<char> produced;  // per slot: produced inside ops

  Checker(dvm_graph* gr, const std::vector<OpRec>& o) : g(gr), ops(o) {
    produced.assign(g->vals.size(), 0);
    for (auto& r : ops) produced[r.out] = 1;
  }
  bool external(int64_t s) const { return !produced[s]; }
  const Shape& shp(int64_t s) const { return g->vals[s].shape; }

  Shape iter_shape(const OpRec& o) const { return is_reduce(o.op) ? shp(o.in[0]) : shp(o.out); }

  Shape dominant() const {
    Shape best;
    int64_t kr = -1, kn = -1;
    for (auto& o : ops) {
      const Shape s = iter_shape(o);
      const int64_t n = s.numel();
      if (s.nd > kr || (s.nd == kr && n > kn)) {
        best = s;
        kr = s.nd;
        kn = n;
      }
    }
    return best;
  }

  int tmpl() const {
    if (ops[0].op == DVM_OP_MATMUL) return TM_MATMUL;
    bool all = false, row = false;
    for (auto& o : ops) {
      if (is_reduce(o.op)) (o.axis == DVM_AXIS_ALL ? all : row) = true;
    }
    return all ? TM_ALLREDUCE : row ? TM_ROWREDUCE : TM_ELEMWISE;
  }

  // external operands read by non-matmul ops, first-use order
  std::vector<int64_t> ext_operands() const {
    std::vector<int64_t> out;
    for (auto& o : ops) {
      if (o.op == DVM_OP_MATMUL) continue;
      for (int k = 0; k < o.n_in; ++k) {
        const int64_t s = o.in[k];
        if (external(s) && std::find(out.begin(), out.end(), s) == out.end()) out.push_back(s);
      }
    }
    return out;
  }

  // outputs that may be stored (have storage), in op order
  std::vector<int64_t> storable_outputs() const {
    std::vector<int64_t> out;
    for (auto& o : ops) {
      if (o.op == DVM_OP_MATMUL || is_reduce_all(o)) continue;
      if (g->vals[o.out].t.data) out.push_back(o.out);
    }
    return out;
  }

  bool collapse(const Shape& sd, const std::vector<int64_t>& operands, int64_t* R, int64_t* C,
                std::vector<std::pair<int64_t, int64_t>>* st) const {
    std::vector<std::array<int64_t, 4>> strides;
    for (int64_t s : operands) {
      const dvm_tensor& t = g->vals[s].t;
      if (t.ndim > sd.nd) return false;
      Shape b;
      if (!broadcast(shp(s), sd, &b) || b != sd) return false;
      std::array<int64_t, 4> a{};
      bcast_strides(t, sd, a.data());
      strides.push_back(a);
    }
    return tiling::collapse(tmpl(), sd, strides, R, C, st);
  }

  int check_pattern() const {
    const Shape sd = dominant();
    const Shape rs = row_shape(sd);
    int n_all = 0, n_row = 0;
    for (size_t i = 0; i < ops.size(); ++i) {
      const OpRec& o = ops[i];
      if (o.op == DVM_OP_MATMUL) {
        if (i != 0) return FR_PATTERN;
        continue;
      }
      if (is_reduce(o.op)) {
        if (iter_shape(o) != sd) return FR_SHAPE;
        if (o.axis == DVM_AXIS_ALL) {
          ++n_all;
          if (i != ops.size() - 1) return FR_PATTERN;
        } else {
          ++n_row;
        }
        continue;
      }
      const Shape s = shp(o.out);
      if (s != sd && s != rs) return FR_SHAPE;
    }
    if (ops[0].op == DVM_OP_MATMUL && (n_all || n_row)) return FR_PATTERN;
    if (n_all && n_row) return FR_PATTERN;
    if (n_all > 1) return FR_PATTERN;
    if (tmpl() == TM_MATMUL) return -1;  // matmul graphs: epilogue operands checked at encode
    std::vector<int64_t> operands = ext_operands();
    for (int64_t s : storable_outputs()) operands.push_back(s);
    int64_t R, C;
    std::vector<std::pair<int64_t, int64_t>> st;
    if (!collapse(sd, operands, &R, &C, &st)) return FR_SHAPE;
    return -1;
  }

  // tile / row class of every value used or produced (mirrors the spec)
  void classes(std::vector<char>* cls) const {  // 0 none, 1 tile, 2 row
    const Shape sd = dominant(), rs = row_shape(sd);
    const int tm = tmpl();
    cls->assign(g->vals.size(), -1);
    for (auto& o : ops) {
      char oc;
      if (tm == TM_ROWREDUCE && (is_reduce(o.op) || (shp(o.out) == rs && rs != sd))) oc = 2;
      else if (is_reduce_all(o)) oc = 0;
      else oc = 1;
      (*cls)[o.out] = oc;
      for (int k = 0; k < o.n_in; ++k) {
        const int64_t s = o.in[k];
        if (external(s) && (*cls)[s] == -1) {
          if (o.op == DVM_OP_MATMUL) (*cls)[s] = 0;
          else if (oc == 2 && !is_reduce(o.op)) (*cls)[s] = 2;
          else (*cls)[s] = 1;
        }
      }
    }
  }

  void demand(int* tile_peak, int* row_peak) const {
    std::vector<char> cls;
    classes(&cls);
    const size_t n = g->vals.size();
    std::vector<int> first(n, -1), last(n, -1), def(n, -1);
    for (size_t i = 0; i < ops.size(); ++i) {
      def[ops[i].out] = (int)i;
      for (int k = 0; k < ops[i].n_in; ++k) {
        const int64_t s = ops[i].in[k];
        if (first[s] < 0) first[s] = (int)i;
        last[s] = (int)i;
      }
    }
    std::vector<int64_t> used;
    for (size_t s = 0; s < n; ++s)
      if (last[s] >= 0) used.push_back((int64_t)s);
    *tile_peak = 0;
    *row_peak = 0;
    for (size_t i = 0; i < ops.size(); ++i) {
      int nt = 0, nr = 0;
      for (int64_t s : used) {
        const int start = external(s) ? first[s] : def[s] + 1;
        if (start <= (int)i && (int)i <= last[s]) {
          if (cls[s] == 1) ++nt;
          else if (cls[s] == 2) ++nr;
        }
      }
      const char oc = cls[ops[i].out];
      if (oc == 1) ++nt;
      else if (oc == 2) ++nr;
      *tile_peak = std::max(*tile_peak, nt);
      *row_peak = std::max(*row_peak, nr);
    }
  }

  static bool overlap(const std::pair<uintptr_t, int64_t>& a, const std::pair<uintptr_t, int64_t>& b) {
    return a.first < b.first + (uintptr_t)b.second && b.first < a.first + (uintptr_t)a.second;
  }

  int check_dependence(size_t n_old) const {
    if (n_old == 0) return -1;
    auto range = [&](int64_t s) { return std::make_pair((uintptr_t)g->vals[s].t.data, extent_bytes(g->vals[s].t)); };
    std::vector<std::pair<uintptr_t, int64_t>> old_reads, old_writes, new_reads, new_writes;
    std::vector<char> prod_old(g->vals.size(), 0);
    for (size_t i = 0; i < n_old; ++i) prod_old[ops[i].out] = 1;
    for (size_t i = 0; i < n_old; ++i)
      for (int k = 0; k < ops[i].n_in; ++k) {
        const int64_t s = ops[i].in[k];
        if (!prod_old[s] && g->vals[s].t.data && extent_bytes(g->vals[s].t)) old_reads.push_back(range(s));
      }
    for (size_t i = 0; i < n_old; ++i) {
      const Val& v = g->vals[ops[i].out];
      if (v.t.data && (v.live || !v.released)) old_writes.push_back(range(ops[i].out));
    }
    for (size_t i = n_old; i < ops.size(); ++i) {
      for (int k = 0; k < ops[i].n_in; ++k) {
        const int64_t s = ops[i].in[k];
        if (external(s) && g->vals[s].t.data && extent_bytes(g->vals[s].t)) new_reads.push_back(range(s));
      }
      if (g->vals[ops[i].out].t.data) new_writes.push_back(range(ops[i].out));
    }
    for (auto& w : new_writes) {
      for (auto& r : old_reads)
        if (overlap(w, r)) return FR_DEPENDENCE;
      for (auto& r : old_writes)
        if (overlap(w, r)) return FR_DEPENDENCE;
    }
    for (auto& r : new_reads)
      for (auto& w : old_writes)
        if (overlap(r, w)) return FR_DEPENDENCE;
    return -1;
  }

  bool tile_operands(const Shape& sd, const std::vector<int64_t>& operands, int64_t* R, int64_t* C,
                     std::vector<tiling::Operand>* out, std::vector<std::pair<int64_t, int64_t>>* st) const {
    if (!collapse(sd, operands, R, C, st)) return false;
    out->clear();
    for (size_t i = 0; i < operands.size(); ++i) {
      const dvm_tensor& t = g->vals[operands[i]].t;
      out->push_back({esize(t.dtype), (*st)[i].first, (*st)[i].second, (int64_t)((uintptr_t)t.data % 16)});
    }
    return true;
  }

  int check_resources() const {
    if (ops.size() > (size_t)MAX_OPS) return FR_RESOURCE;
    std::vector<int64_t> exts;
    for (auto& o : ops)
      for (int k = 0; k < o.n_in; ++k)
        if (external(o.in[k]) && std::find(exts.begin(), exts.end(), o.in[k]) == exts.end()) exts.push_back(o.in[k]);
    if (exts.size() > (size_t)MAX_EXT) return FR_RESOURCE;
    int tp, rp;
    demand(&tp, &rp);
    if (tp > MAX_TILE_VALUES || rp > MAX_ROW_VALUES) return FR_RESOURCE;
    if (tmpl() == TM_MATMUL) return -1;
    const Shape sd = dominant();
    std::vector<int64_t> operands = ext_operands();
    for (int64_t s : storable_outputs()) operands.push_back(s);
    int64_t R, C;
    std::vector<tiling::Operand> tops;
    std::vector<std::pair<int64_t, int64_t>> st;
    if (!tile_operands(sd, operands, &R, &C, &tops, &st)) return FR_SHAPE;
    tiling::Plan p;
    if (!tiling::plan(tmpl(), R, C, tops, &p) && !tiling::plan(tmpl(), R, C, tops, &p, NV_WIDE)) return FR_RESOURCE;
    return -1;
  }

  int check(size_t n_old) const {
    int r = check_pattern();
    if (r >= 0) return r;
    r = check_dependence(n_old);
    if (r >= 0) return r;
    return check_resources();
  }
};

// ===========================================================================
// Encoder: lowers a fused graph to a tile-level bytecode program
// (DVM review page, section 4.3: code header + per-op bytecode + the syncs the
// encoder inserts).
// ===========================================================================
struct Encoder {
  dvm_graph* g;
  const std::vector<OpRec>& ops;
  Checker ck;
  dvm_program* prog;
  uint32_t* W;
  std::vector<uint32_t> body;
  int n_args = 0;
  std::vector<int> arg_of;        // slot -> arg index
  std::vector<int> last_use, n_uses;
  std::vector<char> cls;
  int treg[N_TREG];               // value slot held by each tile register (-1 none)
  int rreg[N_RREG];
  std::vector<int> tloc, rloc;    // slot -> register (-1 none)
  std::vector<char> store_it;
  tiling::Plan plan;
  int n_red = 0;
  bool cross_wave = false;
  bool red_alt = false;  // cross-wave buffers alternate with the tile parity (HF_RED_ALT)
  std::vector<int> pf_slot, inv_slot;   // slot -> LDS staging slot (-1 none)
  struct Consume {
    size_t pos;      // word index of the instruction in body
    uint32_t slot;
    bool is_bin;
  };
  std::vector<Consume> consumes;
  long issue_pos[2] = {-1, -1};
  std::vector<uint32_t> pro;            // prologue (once per workgroup)
  // VM variant the program is encoded for: the standard one (N_TREG tile
  // registers of NV_MAX chunks) or the wide one (the accumulator alone, of
  // NV_WIDE chunks)
  int64_t nvm = NV_MAX;
  int n_treg = N_TREG;
  uint32_t ktype = KT_VECTOR;
  int treg_hi = 0;          // highest tile register the program names
  bool plan_failed = false; // no tile of this variant fits the shape
  int staged_pf = 0, staged_inv = 0;
  void wide() {
    nvm = NV_WIDE;
    n_treg = 1;
    ktype = KT_VECTOR_WIDE;
  }

  Encoder(dvm_graph* gr, const std::vector<OpRec>& o, dvm_program* p) : g(gr), ops(o), ck(gr, o), prog(p), W(p->prog.w) {}

  void emit(uint32_t w0, uint32_t w1) {
    body.push_back(w0);
    body.push_back(w1);
  }

  int add_arg(int64_t slot, int64_t sr, int64_t sc) {
    const dvm_tensor& t = g->vals[slot].t;
    const int i = n_args++;
    uint32_t* a = W + ARG_BASE + i * ARG_WORDS;
    const uint64_t p = (uint64_t)(uintptr_t)t.data;
    a[A_PTR_LO] = (uint32_t)p;
    a[A_PTR_HI] = (uint32_t)(p >> 32);
    a[A_DTYPE] = (uint32_t)t.dtype;
    // vector accesses (8-element chunks with 64- and 128-bit buffer accesses)
    // need the base, every row start and every tile start aligned: to the
    // element for bf16 (buffer accesses run in the unaligned access mode, so
    // a bf16 row of odd length still moves whole chunks), to the dword for
    // fp32 and u8
    const int64_t es = esize(t.dtype);
    const int64_t al = es == 2 ? 2 : 4;
    bool vec = sc == 1 && (int64_t)(p % al) == 0 && (plan.R <= 1 || ((sr * es) % al + al) % al == 0) &&
               (plan.n_c <= 1 || (plan.tc * es) % al == 0);
    const int64_t ext = extent_bytes(t);
    a[A_FLAGS] = arg_flags_word(vec ? AF_VEC : 0u, (uint64_t)ext);
    a[A_SR_LO] = (uint32_t)(uint64_t)sr;
    a[A_SR_HI] = (uint32_t)((uint64_t)sr >> 32);
    a[A_SC] = (uint32_t)(int32_t)sc;
    a[A_EXTENT] = (uint32_t)(uint64_t)ext;
    arg_of[slot] = i;
    return i;
  }

  bool live_after(int64_t s, int i) const { return last_use[s] > i; }

  // Bytes of the tensors themselves (their own shapes: a broadcast operand
  // counts once): what the program reads or writes at the least.
  uint64_t tensor_bytes(const std::vector<int64_t>& slots) const {
    uint64_t b = 0;
    for (int64_t s : slots) b += (uint64_t)numel_of(g->vals[s].t) * (uint64_t)esize(g->vals[s].t.dtype);
    return b;
  }

  Range range_of(int64_t s) const {
    return {(uintptr_t)g->vals[s].t.data, (uint64_t)extent_bytes(g->vals[s].t)};
  }

  // Every external operand the program reads must have storage: a value with
  // elements but no address (never stored, or from a graph that failed) would
  // make the VM read address 0.
  dvm_status check_storage(const std::vector<int64_t>& exts) const {
    for (int64_t s : exts) {
      const Val& v = g->vals[s];
      if (!v.t.data && numel_of(v.t) > 0) return fail(DVM_ERR_INVALID_ARG, "an operand the graph reads has no storage");
    }
    return DVM_OK;
  }

  int free_treg(int avoid0 = 1) const {
    for (int k = avoid0; k < n_treg; ++k)
      if (treg[k] < 0) return k;
    return -1;
  }

  void bind_t(int k, int64_t s) {
    if (s >= 0) treg_hi = std::max(treg_hi, k);
    if (treg[k] >= 0) tloc[treg[k]] = -1;
    treg[k] = (int)s;
    if (s >= 0) tloc[s] = k;
  }
  void unbind_t(int k) {
    if (treg[k] >= 0) tloc[treg[k]] = -1;
    treg[k] = -1;
  }

  // Make room in register k: move or drop what it holds if still needed.
  dvm_status evict(int k, int i, int64_t keep_a) {
    const int64_t v = treg[k];
    if (v < 0 || v == keep_a) return DVM_OK;
    bool needed = live_after(v, i);
    const OpRec& o = ops[i];
    for (int q = 0; q < o.n_in; ++q) needed = needed || o.in[q] == v;
    if (!needed) {
      unbind_t(k);
      return DVM_OK;
    }
    const int f = free_treg();
    if (f >= 0) {
      emit(enc0(OP_COPY, f, k, 0, 0, 0, 0), 0);
      bind_t(f, v);
      treg[k] = -1;
      return DVM_OK;
    }
    if (ck.external(v)) {  // an external value can always be reloaded
      unbind_t(k);
      return DVM_OK;
    }
    return fail(DVM_ERR_RESOURCE, "tile registers exhausted at op %d", i);
  }

  // Bring tile value s into the accumulator, preserving it elsewhere if it is
  // still needed after op i.
  dvm_status to_acc(int64_t s, int i) {
    dvm_status st = evict(0, i, s);
    if (st != DVM_OK) return st;
    const int k = tloc[s];
    if (k == 0) {
      if (live_after(s, i)) {
        const int f = free_treg();
        if (f >= 0) {
          emit(enc0(OP_COPY, f, 0, 0, 0, 0, 0), 0);
          treg[f] = (int)s;
          tloc[s] = f;
          treg[0] = -1;
          treg_hi = std::max(treg_hi, f);
        } else if (ck.external(s)) {
          unbind_t(0);
        } else {
          return fail(DVM_ERR_RESOURCE, "tile registers exhausted at op %d", i);
        }
      } else {
        unbind_t(0);
      }
      return DVM_OK;
    }
    if (k > 0) {
      emit(enc0(OP_COPY, 0, k, 0, 0, 0, 0), 0);
      if (!live_after(s, i)) {
        bool again = false;
        for (int q = 0; q < ops[i].n_in; ++q) again = again || (ops[i].in[q] == s && q > 0);
        if (!again) unbind_t(k);
      }
      return DVM_OK;
    }
    // external, not in a register
    emit_load(0, s);
    return DVM_OK;
  }

  int free_rreg() const {
    for (int k = 0; k < N_RREG; ++k)
      if (rreg[k] < 0) return k;
    return -1;
  }

  // Row register holding row value s (loading an external row operand).
  int row_of(int64_t s) {
    if (rloc[s] >= 0) return rloc[s];
    const int f = free_rreg();
    if (f < 0) return -1;
    emit(enc0(OP_LOAD_ROW, f, 0, 0, 0, 0, 0), (uint32_t)arg_of[s]);
    rreg[f] = (int)s;
    rloc[s] = f;
    return f;
  }

  void free_dead(int i) {
    const OpRec& o = ops[i];
    for (int q = 0; q < o.n_in; ++q) {
      const int64_t s = o.in[q];
      if (last_use[s] > i) continue;
      if (tloc[s] >= 0 && treg[tloc[s]] == s) unbind_t(tloc[s]);
      if (rloc[s] >= 0) {
        rreg[rloc[s]] = -1;
        rloc[s] = -1;
      }
    }
  }

  uint32_t alu_of(int op) const {
    switch (op) {
      case DVM_OP_ADD: return ALU_ADD;
      case DVM_OP_SUB: return ALU_SUB;
      case DVM_OP_MUL: return ALU_MUL;
      case DVM_OP_DIV: return ALU_DIV;
      case DVM_OP_MAX: return ALU_MAX;
      case DVM_OP_MIN: return ALU_MIN;
      default: return ALU_POW;
    }
  }
  uint32_t un_of(const OpRec& o) const {
    switch (o.op) {
      case DVM_OP_SQRT: return UN_SQRT;
      case DVM_OP_ABS: return UN_ABS;
      case DVM_OP_LOG: return UN_LOG;
      case DVM_OP_EXP: return UN_EXP;
      case DVM_OP_ROUND: return UN_ROUND;
      case DVM_OP_FLOOR: return UN_FLOOR;
      case DVM_OP_ISFINITE: return UN_ISFINITE;
      case DVM_OP_NEG: return UN_NEG;
      case DVM_OP_RECIP: return UN_RECIP;
      case OP_SILU: return UN_SILU;
      default: return UN_IDENT;  // cast / copy: the dtype rounding follows
    }
  }

  // Rounding to the op's output dtype when later ops read the value.
  void round_out(int64_t s, int i, bool in_acc, int rr) {
    if (g->vals[s].t.dtype != DVM_BF16 || !live_after(s, i)) return;
    if (in_acc) emit(enc0(OP_UN, 0, 0, 0, UN_TOBF16, 0, 0), 0);
    else emit(enc0(OP_RUN, rr, rr, 0, UN_TOBF16, 0, 0), 0);
  }

  dvm_status tile_op(int i) {
    const OpRec& o = ops[i];
    // operands: tile values / external tiles, row values, scalar
    int64_t in[2] = {o.in[0], o.n_in > 1 ? o.in[1] : -1};
    const bool binary = is_binary(o.op);
    int64_t a = -1, b = -1;
    bool rev = false;
    if (!binary) {
      a = in[0];
    } else if (o.n_in == 1) {  // scalar operand
      a = in[0];
      rev = o.scalar_pos == 0;
    } else {
      const bool t0 = cls[in[0]] == 1, t1 = cls[in[1]] == 1;
      if (t0 && t1) {
        // prefer a value already in the accumulator, then one that dies here
        int pick = 0;
        auto score = [&](int q) {
          const int64_t s = in[q];
          int sc = 0;
          if (tloc[s] == 0) sc += 4;
          if (!live_after(s, i)) sc += 2;
          if (tloc[s] >= 0) sc += 1;
          return sc;
        };
        if (in[0] != in[1] && score(1) > score(0)) pick = 1;
        a = in[pick];
        b = in[1 - pick];
        rev = pick == 1;
      } else if (t0) {
        a = in[0];
        b = in[1];
      } else {
        a = in[1];
        b = in[0];
        rev = true;
      }
    }
    dvm_status st = to_acc(a, i);
    if (st != DVM_OK) return st;
    if (!binary) {
      const uint32_t f = un_of(o);
      if (f != UN_IDENT) emit(enc0(OP_UN, 0, 0, 0, f, 0, 0), 0);
    } else {
      uint32_t bk, bi = 0, w1 = 0, mflags = 0, alu = alu_of(o.op);
      if (o.n_in == 1) {
        bk = BK_IMM;
        float s = o.scalar;
        std::memcpy(&w1, &s, 4);
      } else if (b == a) {
        bk = BK_TREG;
        bi = 0;
      } else if (cls[b] == 2) {
        const int r = row_of(b);
        if (r < 0) return fail(DVM_ERR_RESOURCE, "row registers exhausted at op %d", i);
        bk = BK_RREG;
        bi = (uint32_t)r;
        // tile / row value: one reciprocal per row, then a multiply per element
        // (in place when the row value dies here, else in a spare register)
        if (o.op == DVM_OP_DIV && !rev) {
          const int rr = live_after(b, i) ? free_rreg() : r;
          if (rr >= 0) {
            emit(enc0(OP_RUN, rr, r, 0, UN_RECIP, 0, 0), 0);
            bi = (uint32_t)rr;
            alu = ALU_MUL;
          }
        }
      } else if (tloc[b] >= 0) {
        bk = BK_TREG;
        bi = (uint32_t)tloc[b];
      } else {
        // external tile operand: keep it in a free register if it is read again
        const int f = free_treg();
        if (n_uses[b] > 1 && live_after(b, i) && f >= 0) {
          emit_load(f, b);
          bind_t(f, b);
          bk = BK_TREG;
          bi = (uint32_t)f;
        } else {
          bk = BK_MEM;
          w1 = (uint32_t)arg_of[b];
          mflags = src_flags(b, &bi);
        }
      }
      emit(enc0(OP_BIN, 0, 0, bi, alu, bk, (rev ? FL_REV : 0) | mflags), w1);
      if (bk == BK_MEM) note_consume(mflags, bi, true);
    }
    free_dead(i);
    if (treg[0] >= 0 && treg[0] != o.out) unbind_t(0);
    bind_t(0, o.out);
    round_out(o.out, i, true, 0);
    if (store_it[o.out]) emit(enc0(OP_STORE, 0, 0, 0, 0, 0, 0), (uint32_t)arg_of[o.out]);
    if (last_use[o.out] <= i) unbind_t(0);
    return DVM_OK;
  }

  dvm_status row_op(int i) {
    const OpRec& o = ops[i];
    const bool binary = is_binary(o.op);
    int ra = -1, rb = -1;
    bool imm = false, rev = false;
    uint32_t w1 = 0;
    if (binary && o.n_in == 1) {
      ra = row_of(o.in[0]);
      imm = true;
      rev = o.scalar_pos == 0;
      float s = o.scalar;
      std::memcpy(&w1, &s, 4);
    } else {
      ra = row_of(o.in[0]);
      if (binary) rb = row_of(o.in[1]);
    }
    if (ra < 0 || (binary && !imm && rb < 0)) return fail(DVM_ERR_RESOURCE, "row registers exhausted at op %d", i);
    // destination: an input register that dies here, else a free one
    int dst = -1;
    if (!live_after(o.in[0], i) && rloc[o.in[0]] == ra) dst = ra;
    else if (binary && !imm && !live_after(o.in[1], i) && rloc[o.in[1]] == rb) dst = rb;
    else dst = free_rreg();
    if (dst < 0) return fail(DVM_ERR_RESOURCE, "row registers exhausted at op %d", i);
    if (binary) {
      emit(enc0(OP_RBIN, dst, ra, imm ? 0 : rb, alu_of(o.op), imm ? BK_IMM : BK_RREG, rev ? FL_REV : 0), w1);
    } else {
      emit(enc0(OP_RUN, dst, ra, 0, un_of(o), 0, 0), 0);
    }
    free_dead(i);
    if (rreg[dst] >= 0 && rreg[dst] != o.out) rloc[rreg[dst]] = -1;
    rreg[dst] = (int)o.out;
    rloc[o.out] = dst;
    round_out(o.out, i, false, dst);
    if (store_it[o.out]) emit(enc0(OP_STORE_ROW, 0, dst, 0, 0, 0, 0), (uint32_t)arg_of[o.out]);
    if (last_use[o.out] <= i) {
      rreg[dst] = -1;
      rloc[o.out] = -1;
    }
    return DVM_OK;
  }

  // tile register holding tile value s (loading an external one)
  dvm_status tile_src(int64_t s, int i, int* k) {
    if (tloc[s] >= 0) {
      *k = tloc[s];
      return DVM_OK;
    }
    int f = free_treg(0);
    if (f < 0) {
      dvm_status st = evict(0, i, -1);
      if (st != DVM_OK) return st;
      f = 0;
    }
    emit_load(f, s);
    bind_t(f, s);
    *k = f;
    return DVM_OK;
  }

  // A reduce_sum at op i whose input is mul(a, a) at op i - 1, an f32 tile
  // value read by nothing else: one sum-of-squares reduce of a.
  bool sumsq_pair(size_t i) const {
    if (i + 1 >= ops.size()) return false;
    const OpRec& m = ops[i];
    const OpRec& r = ops[i + 1];
    return m.op == DVM_OP_MUL && m.n_in == 2 && m.in[0] == m.in[1] && cls[m.out] == 1 && cls[m.in[0]] == 1 &&
           g->vals[m.out].t.dtype == DVM_F32 && !store_it[m.out] && n_uses[m.out] == 1 &&
           r.op == DVM_OP_REDUCE_SUM && r.axis != DVM_AXIS_ALL && r.n_in == 1 && r.in[0] == m.out;
  }

  // Row reduce (or reduce-all) of op i.  With src >= 0: a sum-of-squares
  // reduce of tile value src, fusing the square at op i_sq.
  dvm_status reduce_op(int i, int64_t src = -1, int i_sq = -1) {
    const OpRec& o = ops[i];
    const uint32_t kind = src >= 0 ? RK_SUMSQ : o.op == DVM_OP_REDUCE_SUM ? RK_SUM : RK_MAX;
    int k;
    dvm_status st = tile_src(src >= 0 ? src : o.in[0], i, &k);
    if (st != DVM_OK) return st;
    if (i_sq >= 0) free_dead(i_sq);
    if (o.axis == DVM_AXIS_ALL) {
      // each lane folds the tile into its running partial; the workgroup's
      // partial and the combine of the workgroups' partials follow the body
      // (the VM's reduce-all epilogue)
      emit(enc0(OP_ALL, 0, k, 0, kind, 0, 0), 0);
      W[H_ALL_KIND] = kind;
      free_dead(i);
      return DVM_OK;
    }
    int dst = free_rreg();
    if (dst < 0) return fail(DVM_ERR_RESOURCE, "row registers exhausted at op %d", i);
    if (plan.g > 64) {
      const uint32_t buf = (uint32_t)(n_red++ % N_LDSBUF);
      emit(enc0(OP_REDX, dst, k, buf, kind, 0, 0), 0);
      cross_wave = true;
    } else {
      emit(enc0(OP_RED, dst, k, 0, kind, 0, 0), 0);
    }
    free_dead(i);
    rreg[dst] = (int)o.out;
    rloc[o.out] = dst;
    round_out(o.out, i, false, dst);
    if (store_it[o.out]) emit(enc0(OP_STORE_ROW, 0, dst, 0, 0, 0, 0), (uint32_t)arg_of[o.out]);
    if (last_use[o.out] <= i) {
      rreg[dst] = -1;
      rloc[o.out] = -1;
    }
    return DVM_OK;
  }

  // Flags and staging slot for a read of external operand s.
  uint32_t src_flags(int64_t s, uint32_t* slot) {
    *slot = 0;
    if (inv_slot[s] >= 0) {
      *slot = (uint32_t)inv_slot[s];
      return FL_INV;
    }
    if (pf_slot[s] >= 0) {
      *slot = (uint32_t)pf_slot[s];
      return FL_PF;  // the refill goes on the slot's last read (place_refills)
    }
    return 0;
  }

  // Each prefetch slot is refilled with the next tile's data by its last read
  // in the body: every read of the slot then sees this tile's data (a refill
  // at an earlier read would hand the later reads the next tile's values).
  void place_refills() {
    long last[2] = {-1, -1};
    for (const Consume& c : consumes) last[c.slot] = std::max(last[c.slot], (long)c.pos);
    for (int k = 0; k < 2; ++k) {
      issue_pos[k] = last[k];
      if (last[k] >= 0) body[(size_t)last[k]] |= (uint32_t)FL_ISSUE << 28;
    }
  }

  void note_consume(uint32_t f, uint32_t slot, bool is_bin) {
    if (!(f & FL_PF)) return;
    consumes.push_back({body.size() - 2, slot, is_bin});
  }

  void emit_load(int k, int64_t s) {
    uint32_t slot;
    const uint32_t f = src_flags(s, &slot);
    emit(enc0(OP_LOAD, k, 0, slot, 0, 0, f), (uint32_t)arg_of[s]);
    note_consume(f, slot, false);
  }

  // Vector-memory instructions one wave issues for an instruction in a full
  // tile (a lower bound: ragged tiles take the element paths and issue
  // more).  Vector (128-bit chunk) loads, stores and prefetch refills issue
  // the tile's nv chunks; element loads and stores run all chunks of the
  // build (out-of-range ones masked).
  uint32_t halves(uint32_t arg) const { return W[ARG_BASE + arg * ARG_WORDS + A_DTYPE] == DT_F32 ? 2u : 1u; }
  uint32_t load_ops(uint32_t arg) const {
    const uint32_t* a = W + ARG_BASE + arg * ARG_WORDS;
    const int32_t sc = (int32_t)a[A_SC];
    if (sc == 0) return 1u;
    if ((a[A_FLAGS] & AF_VEC) && sc == 1) return (uint32_t)plan.nv * halves(arg);
    return 8u * (uint32_t)nvm;
  }
  uint32_t store_ops(uint32_t arg) const {
    const uint32_t* a = W + ARG_BASE + arg * ARG_WORDS;
    if ((a[A_FLAGS] & AF_VEC) && (int32_t)a[A_SC] == 1) return (uint32_t)plan.nv * halves(arg);
    return 8u * (uint32_t)nvm;
  }
  uint32_t src_ops(uint32_t w0, uint32_t w1) const {
    const uint32_t f = f_flags(w0);
    if (f & FL_INV) return 0;
    if (f & FL_PF) return (f & FL_ISSUE) ? (uint32_t)plan.nv * halves(w1) : 0u;
    return load_ops(w1);
  }
  uint32_t vm_ops(uint32_t w0, uint32_t w1) const {
    switch (f_op(w0)) {
      case OP_LOAD: return src_ops(w0, w1);
      case OP_BIN: return f_bk(w0) == BK_MEM ? src_ops(w0, w1) : 0u;
      case OP_STORE: return store_ops(w1);
      case OP_LOAD_ROW:
      case OP_STORE_ROW: return 1u;
      case OP_PF: return (uint32_t)plan.nv * halves(w1);
      case OP_LDS_INV: return load_ops(w1);
      default: return 0u;
    }
  }

  // Wait counts of prefetch reads: instructions issued after the prefetch of
  // the tile being read, counted over the end of the previous tile's body
  // plus this body up to the read.  A workgroup's first tile needs no count:
  // the VM waits for every prologue load (its prefetch included) before the
  // body starts, so the count only has to hold from the second tile on, and
  // the previous tile's stores stay in flight while the next tile starts.
  void patch_waits() {
    auto sum = [&](const std::vector<uint32_t>& v, size_t lo, size_t hi) {
      uint32_t n = 0;
      for (size_t q = lo; q < hi; q += 2) n += vm_ops(v[q], v[q + 1]);
      return n;
    };
    for (const Consume& c : consumes) {
      const size_t ip = (size_t)issue_pos[c.slot];
      const uint32_t after_issue = sum(body, ip + 2, body.size());
      uint32_t n = after_issue + sum(body, 0, c.pos);
      n = std::min<uint32_t>(n, VMC_MAX);
      uint32_t& w = body[c.pos];
      if (c.is_bin) w = (w & ~0xff00u) | ((n & 0xfu) << 8) | (((n >> 4) & 0xfu) << 12);
      else w = (w & ~0x00f0f000u) | ((n & 0xfu) << 12) | (((n >> 4) & 0xfu) << 20);
    }
  }

  // LDS staging (worth it when a workgroup runs several tiles): tile-invariant
  // operands are held in LDS once per workgroup; tile-varying streamed
  // operands are prefetched one tile ahead into LDS by direct-to-LDS loads.
  void decide_lds(const std::vector<int64_t>& exts, const std::vector<std::pair<int64_t, int64_t>>& st) {
    uint32_t off = 0;
    int n_pf = 0, n_inv = 0;
    // the cross-wave reduction buffers live in this area too: reserved when a
    // reduction may cross waves (rows wider than a wave, or a reduce-all)
    bool has_red = false;
    for (const OpRec& o : ops) has_red = has_red || is_reduce(o.op);
    const bool need_red = has_red && (plan.g > 64 || ck.tmpl() == TM_ALLREDUCE);
    const uint32_t budget = LDS_BUDGET - (need_red ? RED_LDS_BYTES : 0u);
    if (plan.body_tile >= 2) {
      for (size_t q = 0; q < exts.size(); ++q) {
        const int64_t s = exts[q];
        if (cls[s] != 1) continue;
        const int64_t sr = st[q].first, sc = st[q].second;
        const int es = esize(g->vals[s].t.dtype);
        const bool invariant = (sr == 0 || plan.n_r == 1) && (sc == 0 || plan.n_c == 1);
        const uint32_t* a = W + ARG_BASE + arg_of[s] * ARG_WORDS;
        if (invariant && n_inv < 2) {
          // an operand that does not vary along rows is held once (one row),
          // shared by the lane groups of all rows
          const bool shared = sr == 0;
          const uint32_t sz = (uint32_t)nvm * (uint32_t)(shared ? plan.g : T_LANES) * 32u;
          if (off + sz > budget) continue;
          inv_slot[s] = n_inv;
          W[H_INV_OFF0 + n_inv] = off;
          W[H_INV_SHARED0 + n_inv] = shared ? 1u : 0u;
          off += sz;
          pro.push_back(enc0(OP_LDS_INV, n_inv, 0, 0, 0, 0, 0));
          pro.push_back((uint32_t)arg_of[s]);
          ++n_inv;
        } else if (!invariant && n_pf < 2 && (a[A_FLAGS] & AF_VEC) && sc == 1 && (es == 2 || es == 4)) {
          // the tile's nv chunks (the VM fills and reads no others)
          const uint32_t sz = (uint32_t)plan.nv * T_LANES * 16u * (uint32_t)(es / 2);
          if (off + sz > budget) continue;
          pf_slot[s] = n_pf;
          W[H_PF_OFF0 + n_pf] = off;
          off += sz;
          pro.insert(pro.begin(), (uint32_t)arg_of[s]);
          pro.insert(pro.begin(), enc0(OP_PF, 0, 0, n_pf, 0, 0, 0));
          ++n_pf;
        }
      }
    }
    if (need_red) {
      off = (off + 15u) & ~15u;
      W[H_RED_OFF] = off;
      off += RED_LDS_BYTES;
    }
    W[H_LDS_BYTES] = off;
    staged_pf = n_pf;
    staged_inv = n_inv;
  }

  // Handler id of one instruction (generic opcode and fields -> the VM's
  // specialised routine).  Commutative ALU ops ignore the reversed flag.
  uint32_t handler_of(uint32_t w0, uint32_t w1) const {
    auto dt = [&](uint32_t arg) { return W[ARG_BASE + arg * ARG_WORDS + A_DTYPE]; };
    const uint32_t d = f_dst(w0), a = f_a(w0), sub = f_sub(w0), fl = f_flags(w0);
    switch (f_op(w0)) {
      case OP_LOAD:
        if (fl & FL_INV) return HD_LD_INV + d;
        if (fl & FL_PF) return (dt(w1) == DT_F32 ? HD_LD_PF32 : HD_LD_PF16) + d;
        return HD_LD_DIR + d;
      case OP_STORE:
        if (a == 0 && dt(w1) == DT_BF16) return HD_ST_BF16;
        if (a == 0 && dt(w1) == DT_F32) return HD_ST_F32;
        return HD_ST_DIR + a;
      case OP_COPY: return HD_COPY + 3 * d + a;
      case OP_UN: return sub == UN_SILU ? (uint32_t)HD_SILU : sub == UN_SOFTMAX ? (uint32_t)HD_SOFTMAX : HD_UN + sub;
      case OP_BIN: {
        const uint32_t bk = f_bk(w0);
        if (bk == BK_MEM) return HD_BIN_MEM;
        if (sub == ALU_POW) return HD_BIN_POW;
        if (sub == ALU_DIV && bk == BK_TREG) return HD_DIV_T;
        const uint32_t form = bk == BK_TREG ? f_b(w0) : (uint32_t)BF_SCALAR;
        const bool comm = sub == ALU_ADD || sub == ALU_MUL || sub == ALU_MAX || sub == ALU_MIN;
        const bool rev = !comm && (fl & FL_REV);
        return HD_BIN + 10 * sub + form + (rev ? (uint32_t)BF_REV : 0u);
      }
      case OP_RED: return HD_RED + 3 * sub + a;
      case OP_REDX: return HD_REDX + 3 * sub + a;
      case OP_ALL: return HD_ALL + 3 * sub + a;
      case OP_BCAST: return HD_BCAST + d;
      case OP_RBIN: return HD_RBIN;
      case OP_RUN: return HD_RUN;
      case OP_SYNC: return HD_SYNC;
      case OP_LOAD_ROW: return HD_LD_ROW;
      case OP_STORE_ROW: return HD_ST_ROW;
      case OP_DBG: return HD_DBG;
      case OP_LDS_INV: return HD_LDS_INV;
      case OP_PF: return HD_PF;
      case OP_FMA_INV: return HD_FMA_INV;
      default: return HD_END;
    }
  }
  // A softmax chain on the accumulator (row max into a row register, subtract
  // it, exp, row sum, its reciprocal, multiply) whose row registers no later
  // instruction reads -> one OP_UN UN_SOFTMAX.  Rows inside a wave (RED) run
  // the same steps in the same order; rows across waves (REDX, the two
  // reductions in consecutive buffers b, b + 1) exchange each wave's max and
  // sum once, behind one barrier instead of two.  None of the six issues
  // vector-memory instructions, so the patched waits stay valid.
  static void fuse_softmax(std::vector<uint32_t>& v) {
    auto rreg_reads = [](uint32_t w) -> uint32_t {
      const uint32_t op = f_op(w);
      if (op == OP_BIN && f_bk(w) == BK_RREG) return 1u << f_b(w);
      if (op == OP_RBIN) return (1u << f_a(w)) | (f_bk(w) == BK_RREG ? 1u << f_b(w) : 0u);
      if (op == OP_RUN || op == OP_BCAST || op == OP_STORE_ROW) return 1u << f_a(w);
      if (op == OP_FMA_INV && f_bk(w) == BK_RREG) return 1u << f_dst(w);
      return 0u;
    };
    auto rreg_writes = [](uint32_t w) -> uint32_t {
      const uint32_t op = f_op(w);
      if (op == OP_RED || op == OP_REDX || op == OP_RBIN || op == OP_RUN || op == OP_LOAD_ROW) return 1u << f_dst(w);
      return 0u;
    };
    std::vector<uint32_t> out;
    out.reserve(v.size());
    for (size_t q = 0; q < v.size(); q += 2) {
      if (q + 12 <= v.size()) {
        const uint32_t m = v[q], d = v[q + 2], e = v[q + 4], r = v[q + 6], c = v[q + 8], y = v[q + 10];
        const uint32_t red = f_op(m);
        const bool ok =
            (red == OP_RED || red == OP_REDX) && f_a(m) == 0 && f_sub(m) == RK_MAX &&
            f_op(d) == OP_BIN && f_sub(d) == ALU_SUB && f_bk(d) == BK_RREG && f_b(d) == f_dst(m) &&
            !(f_flags(d) & FL_REV) && f_op(e) == OP_UN && f_sub(e) == UN_EXP && f_op(r) == red && f_a(r) == 0 &&
            f_sub(r) == RK_SUM && (red == OP_RED || f_b(r) == f_b(m) + 1) && f_op(c) == OP_RUN &&
            f_sub(c) == UN_RECIP && f_a(c) == f_dst(r) && f_op(y) == OP_BIN && f_sub(y) == ALU_MUL &&
            f_bk(y) == BK_RREG && f_b(y) == f_dst(c) && !(f_flags(y) & FL_REV);
        if (ok) {
          // the chain's row registers until each is written again (row
          // registers do not outlive the tile)
          uint32_t watch = (1u << f_dst(m)) | (1u << f_dst(r)) | (1u << f_dst(c));
          bool read_later = false;
          for (size_t t = q + 12; t < v.size() && watch && !read_later; t += 2) {
            read_later = (rreg_reads(v[t]) & watch) != 0;
            watch &= ~rreg_writes(v[t]);
          }
          if (!read_later) {
            out.push_back(enc0(OP_UN, 0, 0, red == OP_REDX ? f_b(m) : 0u, UN_SOFTMAX, 0, 0));
            out.push_back(0);
            q += 10;
            continue;
          }
        }
      }
      out.push_back(v[q]);
      out.push_back(v[q + 1]);
    }
    v.swap(out);
  }

  // LDS reduction buffers a body instruction writes (and reads) across waves.
  uint32_t red_bufs(uint32_t w) const {
    const uint32_t op = f_op(w);
    if (op == OP_REDX) return 1u << f_b(w);
    if (op == OP_UN && f_sub(w) == UN_SOFTMAX && plan.g > 64) return 3u << f_b(w);
    return 0u;
  }

  // ACC * inv[s1] followed by ACC + inv[s2] (both tile-invariant operands in
  // LDS, an f32 product: no rounding step between them) -> one OP_FMA_INV,
  // with a preceding ACC * row register folded in as its row scale.
  // Invariant reads issue no vector-memory instructions, so the waits patched
  // into the body stay valid.
  static void fuse_scale_shift(std::vector<uint32_t>& v) {
    std::vector<uint32_t> out;
    out.reserve(v.size());
    for (size_t q = 0; q < v.size(); q += 2) {
      const uint32_t a0 = v[q];
      if (q + 2 < v.size()) {
        const uint32_t b0 = v[q + 2];
        auto inv_bin = [](uint32_t w, uint32_t alu) {
          return f_op(w) == OP_BIN && f_bk(w) == BK_MEM && (f_flags(w) & FL_INV) && f_sub(w) == alu;
        };
        if (inv_bin(a0, ALU_MUL) && inv_bin(b0, ALU_ADD)) {
          // a multiply by a row register just before folds in as well
          uint32_t rscale = 0, bk = 0;
          const size_t n = out.size();
          if (n >= 2 && f_op(out[n - 2]) == OP_BIN && f_bk(out[n - 2]) == BK_RREG && f_sub(out[n - 2]) == ALU_MUL) {
            rscale = f_b(out[n - 2]);
            bk = BK_RREG;
            out.resize(n - 2);
          }
          out.push_back(enc0(OP_FMA_INV, rscale, f_b(b0), f_b(a0), 0, bk, 0));
          out.push_back(0);
          q += 2;
          continue;
        }
      }
      out.push_back(a0);
      out.push_back(v[q + 1]);
    }
    v.swap(out);
  }

  void to_handlers(std::vector<uint32_t>& v) const {
    for (size_t q = 0; q < v.size(); q += 2) v[q] = (v[q] & ~0xffu) | handler_of(v[q], v[q + 1]);
  }

  // MATMUL template: the matmul's A and B are args 0 and 1; the body is the
  // epilogue on the [M, N] result, which starts in the accumulator.
  dvm_status run_matmul() {
    const OpRec& mm = ops[0];
    const dvm_tensor& A = g->vals[mm.in[0]].t;
    const dvm_tensor& B = g->vals[mm.in[1]].t;
    const int64_t M = A.shape[0], K = A.shape[1], N = B.shape[1];
    std::vector<int64_t> stored;
    for (auto& o : ops) {
      const Val& v = g->vals[o.out];
      if (v.live || !v.released) {
        // (an empty value needs no storage: nothing is stored)
        if (!v.t.data && numel_of(v.t) > 0) return fail(DVM_ERR_INVALID_ARG, "a value without storage escapes its graph");
        stored.push_back(o.out);
        store_it[o.out] = 1;
      }
    }
    const Shape sd = ck.dominant();
    std::vector<int64_t> operands = ck.ext_operands();
    {
      std::vector<int64_t> ab = operands;
      if (M > 0 && N > 0 && K > 0) {
        ab.push_back(mm.in[0]);
        ab.push_back(mm.in[1]);
      }
      dvm_status sv = check_storage(ab);
      if (sv != DVM_OK) return sv;
    }
    for (int64_t s : stored) operands.push_back(s);
    int64_t R, C;
    std::vector<tiling::Operand> tops;
    std::vector<std::pair<int64_t, int64_t>> st;
    if (!ck.tile_operands(sd, operands, &R, &C, &tops, &st))
      return fail(DVM_ERR_SHAPE, "epilogue operands do not collapse to [M, N]");
    if (!tiling::plan_matmul(M, N, K, 2, 2, tops, &plan)) return fail(DVM_ERR_RESOURCE, "no feasible tile");
    // 32-bit lane offsets inside a tile and inside the A and B panels
    for (size_t q = 0; q < operands.size(); ++q) {
      const int64_t span = ((plan.tr - 1) * std::llabs(st[q].first) + plan.tc * std::llabs(st[q].second) + 1) *
                           tops[q].esize;
      if (span >= (int64_t)EXTENT_CAP) return fail(DVM_ERR_RESOURCE, "tile spans >= 2^31 bytes");
    }
    if ((plan.tr * A.stride[0] + K) * 2 >= (int64_t)EXTENT_CAP || (K * B.stride[0] + plan.tc) * 2 >= (int64_t)EXTENT_CAP)
      return fail(DVM_ERR_RESOURCE, "matmul panel spans >= 2^31 bytes");
    if (operands.size() + 2 > (size_t)MAX_ARGS) return fail(DVM_ERR_RESOURCE, "too many operands");
    for (int k = 0; k < 2; ++k) {
      const dvm_tensor& t = k == 0 ? A : B;
      uint32_t* a = W + ARG_BASE + k * ARG_WORDS;
      const uint64_t p = (uint64_t)(uintptr_t)t.data;
      a[A_PTR_LO] = (uint32_t)p;
      a[A_PTR_HI] = (uint32_t)(p >> 32);
      a[A_DTYPE] = (uint32_t)t.dtype;
      a[A_FLAGS] = arg_flags_word(AF_VEC, (uint64_t)extent_bytes(t));
      a[A_SR_LO] = (uint32_t)(uint64_t)t.stride[0];
      a[A_SR_HI] = (uint32_t)((uint64_t)t.stride[0] >> 32);
      a[A_SC] = (uint32_t)t.stride[1];
      a[A_EXTENT] = (uint32_t)(uint64_t)extent_bytes(t);
    }
    n_args = 2;
    for (size_t q = 0; q < operands.size(); ++q) add_arg(operands[q], st[q].first, st[q].second);
    prog->bytes = tensor_bytes(operands) + tensor_bytes({mm.in[0], mm.in[1]});
    prog->reads = {range_of(mm.in[0]), range_of(mm.in[1])};
    for (int64_t q : ck.ext_operands()) prog->reads.push_back(range_of(q));
    for (int64_t q : stored) prog->writes.push_back(range_of(q));
    cls.clear();
    ck.classes(&cls);
    cls[mm.out] = 1;
    bind_t(0, mm.out);
    if (store_it[mm.out]) emit(enc0(OP_STORE, 0, 0, 0, 0, 0, 0), (uint32_t)arg_of[mm.out]);
    if (last_use[mm.out] <= 0) unbind_t(0);
    for (size_t i = 1; i < ops.size(); ++i) {
      if (cls[ops[i].out] != 1) return fail(DVM_ERR_UNSUPPORTED, "matmul epilogue op %zu is not elementwise", i);
      dvm_status e = tile_op((int)i);
      if (e != DVM_OK) return e;
    }
    const uint32_t instr_base = ARG_BASE + (uint32_t)n_args * ARG_WORDS;
    if (instr_base + body.size() + PAD_WORDS > (size_t)MAX_WORDS) return fail(DVM_ERR_RESOURCE, "program too large");
    std::copy(body.begin(), body.end(), W + instr_base);
    W[H_MAGIC] = MAGIC;
    W[H_VERSION] = VERSION;
    W[H_KTYPE] = KT_MIX;
    W[H_TEMPLATE] = TM_MATMUL;
    {
      uint64_t touched = 0;
      for (int q = 0; q < n_args; ++q) {
        const uint32_t* a = W + ARG_BASE + q * ARG_WORDS;
        touched += arg_extent(a[A_FLAGS], a[A_EXTENT]);
      }
      W[H_FLAGS] = touched >= STREAM_BYTES ? HF_STREAM : 0u;  // epilogue stores only
    }
    W[H_BLOCK_DIM] = (uint32_t)plan.block_dim;
    W[H_BODY_TILE] = (uint32_t)plan.body_tile;
    W[H_GRID] = (uint32_t)plan.grid;
    W[H_TR] = (uint32_t)plan.tr;
    W[H_TC] = (uint32_t)plan.tc;
    W[H_G] = 1;
    W[H_NC] = (uint32_t)(plan.n_c ? plan.n_c : 1);
    W[H_NARGS] = (uint32_t)n_args;
    W[H_PRO_BEGIN] = W[H_PRO_END] = W[H_BODY_BEGIN] = instr_base;
    W[H_BODY_END] = instr_base + (uint32_t)body.size();
    W[H_R_LO] = (uint32_t)(uint64_t)M;
    W[H_R_HI] = (uint32_t)((uint64_t)M >> 32);
    W[H_C_LO] = (uint32_t)(uint64_t)N;
    W[H_C_HI] = (uint32_t)((uint64_t)N >> 32);
    W[H_MM_K] = (uint32_t)K;
    W[H_MM_A] = 0;
    W[H_MM_B] = 1;
    W[H_LDS_BYTES] = (uint32_t)mm_lds_bytes((int)plan.tr, (int)plan.tc);
    W[H_N_INSTR] = (uint32_t)(body.size() / 2);
    prog->n_words = instr_base + (uint32_t)body.size();
    prog->n_instr = (uint32_t)(body.size() / 2);
    prog->R = M;
    prog->C = N;
    prog->pad = 0;
    prog->grid_launch = (uint32_t)plan.grid;
    prog->lds = W[H_LDS_BYTES];
    return DVM_OK;
  }

  dvm_status run() {
    std::memset(W, 0, sizeof(uint32_t) * HDR_WORDS);
    const size_t n = g->vals.size();
    arg_of.assign(n, -1);
    last_use.assign(n, -1);
    n_uses.assign(n, 0);
    tloc.assign(n, -1);
    rloc.assign(n, -1);
    store_it.assign(n, 0);
    pf_slot.assign(n, -1);
    inv_slot.assign(n, -1);
    for (int k = 0; k < N_TREG; ++k) treg[k] = -1;
    for (int k = 0; k < N_RREG; ++k) rreg[k] = -1;
    for (size_t i = 0; i < ops.size(); ++i)
      for (int q = 0; q < ops[i].n_in; ++q) {
        last_use[ops[i].in[q]] = (int)i;
        n_uses[ops[i].in[q]]++;
      }
    const int tm = ck.tmpl();
    if (tm == TM_MATMUL) return run_matmul();
    // stored outputs: live, or not released by flush time
    std::vector<int64_t> stored;
    for (auto& o : ops) {
      const Val& v = g->vals[o.out];
      if (v.live || !v.released) {
        // (an empty value needs no storage: nothing is stored)
        if (!v.t.data && numel_of(v.t) > 0) return fail(DVM_ERR_INVALID_ARG, "a value without storage escapes its graph");
        if (!is_reduce_all(o)) stored.push_back(o.out);
        store_it[o.out] = 1;
      }
    }
    const Shape sd = ck.dominant();
    std::vector<int64_t> operands = ck.ext_operands();
    const size_t n_ext = operands.size();
    dvm_status sv = check_storage(operands);
    if (sv != DVM_OK) return sv;
    for (int64_t s : stored) operands.push_back(s);
    int64_t R, C;
    std::vector<tiling::Operand> tops;
    std::vector<std::pair<int64_t, int64_t>> st;
    if (!ck.tile_operands(sd, operands, &R, &C, &tops, &st))
      return fail(DVM_ERR_SHAPE, "operands do not collapse to two dims");
    if (!tiling::plan(tm, R, C, tops, &plan, nvm)) {
      plan_failed = true;
      return fail(DVM_ERR_RESOURCE, "no feasible tile");
    }
    // 32-bit lane offsets: a tile must span < 2^31 bytes in every operand
    for (size_t q = 0; q < operands.size(); ++q) {
      const int64_t span = ((plan.tr - 1) * std::llabs(st[q].first) + plan.tc * std::llabs(st[q].second) + 1) *
                           tops[q].esize;
      if (span >= (int64_t)EXTENT_CAP) return fail(DVM_ERR_RESOURCE, "tile spans >= 2^31 bytes");
    }
    if (operands.size() + 2 > (size_t)MAX_ARGS) return fail(DVM_ERR_RESOURCE, "too many operands");
    for (size_t q = 0; q < operands.size(); ++q) add_arg(operands[q], st[q].first, st[q].second);
    prog->bytes = tensor_bytes(operands);
    if (tm == TM_ALLREDUCE) prog->bytes += (uint64_t)esize(g->vals[ops.back().out].t.dtype);
    for (size_t q = 0; q < operands.size(); ++q) (q < n_ext ? prog->reads : prog->writes).push_back(range_of(operands[q]));
    if (tm == TM_ALLREDUCE) prog->writes.push_back(range_of(ops.back().out));
    cls.clear();
    ck.classes(&cls);
    {
      std::vector<int64_t> exts(operands.begin(), operands.begin() + n_ext);
      std::vector<std::pair<int64_t, int64_t>> est(st.begin(), st.begin() + n_ext);
      decide_lds(exts, est);
    }
    // reduce-all output and scratch
    if (tm == TM_ALLREDUCE) {
      const OpRec& last = ops.back();
      const int ai = n_args++;
      uint32_t* a = W + ARG_BASE + ai * ARG_WORDS;
      const uint64_t p = (uint64_t)(uintptr_t)g->vals[last.out].t.data;
      a[A_PTR_LO] = (uint32_t)p;
      a[A_PTR_HI] = (uint32_t)(p >> 32);
      a[A_DTYPE] = (uint32_t)g->vals[last.out].t.dtype;
      a[A_EXTENT] = 4;
      W[H_ALL_OUT] = (uint32_t)ai;
      // the scratch operand: its address is supplied by the launch (the
      // stream's scratch area); the program records the bytes it needs
      const int si = n_args++;
      uint32_t* b = W + ARG_BASE + si * ARG_WORDS;
      // one partial per workgroup (an empty space still runs one)
      const uint64_t need = SCRATCH_PART_OFF + 4u * (uint64_t)std::max<int64_t>(plan.grid, 1);
      b[A_DTYPE] = DT_F32;
      b[A_FLAGS] = arg_flags_word(0, need);
      b[A_EXTENT] = (uint32_t)need;
      W[H_ALL_SCRATCH] = (uint32_t)si;
      if (need > SCRATCH_BYTES)
        return fail(DVM_ERR_RESOURCE, "reduce-all needs %lld partials", (long long)plan.grid);
    }
    for (size_t i = 0; i < ops.size(); ++i) {
      const OpRec& o = ops[i];
      dvm_status s;
      if (sumsq_pair(i)) {
        s = reduce_op((int)i + 1, o.in[0], (int)i);
        ++i;
      } else if (is_reduce(o.op)) {
        s = reduce_op((int)i);
      } else if (cls[o.out] == 2) {
        s = row_op((int)i);
      } else {
        s = tile_op((int)i);
      }
      if (s != DVM_OK) return s;
    }
    place_refills();
    patch_waits();
    fuse_scale_shift(body);
    fuse_softmax(body);
    // The next tile's first cross-wave reduction could overwrite an LDS
    // buffer some wave is still reading.  The reductions of a tile take
    // buffers in order (k % N_LDSBUF; a fused softmax a pair), and every one
    // after the k-th contains a barrier, so the reads of reduction k are
    // fenced unless k is the tile's last.  The next tile's first reduction
    // writes its buffers again: it races the last one's reads exactly when the
    // two share a buffer (one reduction per tile; or 9, 17, ... of them).
    // When the tile's reductions stay in buffers 0 and 1 the buffers
    // alternate with 2 and 3 by tile parity instead (HF_RED_ALT: no barrier);
    // otherwise the body ends with a sync.
    uint32_t first_bufs = 0, last_bufs = 0, all_bufs = 0;
    for (size_t q = 0; q < body.size(); q += 2) {
      const uint32_t m = red_bufs(body[q]);
      if (!m) continue;
      if (!first_bufs) first_bufs = m;
      last_bufs = m;
      all_bufs |= m;
    }
    if (first_bufs & last_bufs) {
      if (!(all_bufs & ~3u)) red_alt = true;
      else emit(enc0(OP_SYNC, 0, 0, 0, 0, 0, 0), 0);
    }
    // header
    const uint32_t instr_base = ARG_BASE + (uint32_t)n_args * ARG_WORDS;
    const uint32_t body_base = instr_base + (uint32_t)pro.size();
    if (body_base + body.size() + PAD_WORDS > (size_t)MAX_WORDS) return fail(DVM_ERR_RESOURCE, "program too large");
    to_handlers(pro);
    to_handlers(body);
    std::copy(pro.begin(), pro.end(), W + instr_base);
    std::copy(body.begin(), body.end(), W + body_base);
    W[H_MAGIC] = MAGIC;
    W[H_VERSION] = VERSION;
    W[H_KTYPE] = ktype;
    W[H_TEMPLATE] = (uint32_t)tm;
    uint64_t touched = 0;
    for (int q = 0; q < n_args; ++q) {
      const uint32_t* a = W + ARG_BASE + q * ARG_WORDS;
      touched += arg_extent(a[A_FLAGS], a[A_EXTENT]);
    }
    W[H_FLAGS] = (tm != TM_ALLREDUCE && touched >= STREAM_BYTES ? HF_STREAM : 0u) | (red_alt ? HF_RED_ALT : 0u);
    W[H_BLOCK_DIM] = (uint32_t)plan.block_dim;
    W[H_BODY_TILE] = (uint32_t)plan.body_tile;
    W[H_GRID] = (uint32_t)plan.grid;
    W[H_TR] = (uint32_t)plan.tr;
    W[H_TC] = (uint32_t)plan.tc;
    W[H_G] = (uint32_t)(plan.g ? plan.g : 1);
    W[H_NV] = (uint32_t)plan.nv;
    W[H_P] = (uint32_t)plan.P;
    W[H_NC] = (uint32_t)(plan.n_c ? plan.n_c : 1);
    W[H_NARGS] = (uint32_t)n_args;
    W[H_PRO_BEGIN] = instr_base;
    W[H_PRO_END] = body_base;
    W[H_BODY_BEGIN] = body_base;
    W[H_BODY_END] = body_base + (uint32_t)body.size();
    W[H_R_LO] = (uint32_t)(uint64_t)R;
    W[H_R_HI] = (uint32_t)((uint64_t)R >> 32);
    W[H_C_LO] = (uint32_t)(uint64_t)C;
    W[H_C_HI] = (uint32_t)((uint64_t)C >> 32);
    W[H_N_INSTR] = (uint32_t)((pro.size() + body.size()) / 2);
    prog->n_words = body_base + (uint32_t)body.size();
    prog->n_instr = (uint32_t)((pro.size() + body.size()) / 2);
    prog->R = R;
    prog->C = C;
    prog->pad = (uint32_t)plan.pad;
    prog->grid_launch = (uint32_t)plan.grid;
    if (tm == TM_ALLREDUCE && prog->grid_launch == 0) prog->grid_launch = 1;
    prog->lds = W[H_LDS_BYTES];
    return DVM_OK;
  }
};

// ===========================================================================
// Bytecode clean-up before tiling: constant propagation and dead-instruction
// elimination (named as encoder work on the DVM paper review page, section
// 5.2), restricted to rewrites that leave every stored value bit-identical.
//  - x * 1, 1 * x, x / 1, x - (+0), x + (-0) and (-0) + x equal x exactly in
//    IEEE arithmetic (signed zeros, infinities and NaNs included): the op
//    becomes a cast of x to its output dtype.  (x + (+0) turns -0 into +0 and
//    stays.)
//  - A cast to the input's own dtype whose result is not stored is an alias:
//    later readers read the input itself.
//  - An op whose result is neither stored (live, or not released by flush
//    time) nor read by a kept op is dropped; so is, in turn, its producer.
// Matmul graphs are left as they are.
// ===========================================================================
void simplify_ops(const dvm_graph* g, const std::vector<OpRec>& in, std::vector<OpRec>* out) {
  out->clear();
  for (const OpRec& o : in)
    if (o.op == DVM_OP_MATMUL) {
      *out = in;
      return;
    }
  auto stored = [&](int64_t s) { return g->vals[s].live || !g->vals[s].released; };
  // graphs hold a few dozen ops: small lists instead of per-slot tables
  std::vector<std::pair<int64_t, int64_t>> alias;  // (slot, the slot it reads as)
  std::vector<OpRec> fw;
  fw.reserve(in.size());
  for (OpRec o : in) {
    for (int k = 0; k < o.n_in; ++k)
      for (const auto& a : alias)
        if (a.first == o.in[k]) o.in[k] = a.second;
    if (o.n_in == 1 && (o.scalar_pos == 0 || o.scalar_pos == 1)) {
      const float c = o.scalar;
      const bool on_right = o.scalar_pos == 1;
      const bool pos0 = c == 0.f && !std::signbit(c), neg0 = c == 0.f && std::signbit(c);
      if ((o.op == DVM_OP_MUL && c == 1.f) || (o.op == DVM_OP_DIV && on_right && c == 1.f) ||
          (o.op == DVM_OP_SUB && on_right && pos0) || (o.op == DVM_OP_ADD && neg0)) {
        o.op = DVM_OP_CAST;
        o.scalar_pos = -1;
        o.scalar = 0.f;
      }
    }
    if (o.op == DVM_OP_CAST && g->vals[o.in[0]].t.dtype == g->vals[o.out].t.dtype && !stored(o.out)) {
      alias.emplace_back(o.out, o.in[0]);
      continue;
    }
    fw.push_back(o);
  }
  std::vector<int64_t> need;
  std::vector<char> keep(fw.size(), 0);
  size_t n_keep = 0;
  for (size_t i = fw.size(); i-- > 0;) {
    const OpRec& o = fw[i];
    if (!stored(o.out) && std::find(need.begin(), need.end(), o.out) == need.end()) continue;
    keep[i] = 1;
    ++n_keep;
    for (int k = 0; k < o.n_in; ++k) need.push_back(o.in[k]);
  }
  if (n_keep == fw.size() && alias.empty() && fw.size() == in.size()) {
    *out = std::move(fw);
    return;
  }
  for (size_t i = 0; i < fw.size(); ++i)
    if (keep[i]) out->push_back(fw[i]);
}

// SiLU chains (the composite x / (1 + e^-x) written as n = -z, e = exp(n),
// d = e + 1, s = z / d, with n, e and d fp32 values nobody else reads and
// nobody stores) become one op on z.  The VM computes the same four
// operations in registers, so every stored value is bit-identical; it saves
// three dispatches and the copy that keeps z alive across the chain.
void fuse_silu(const dvm_graph* g, std::vector<OpRec>& ops) {
  if (ops.size() < 4) return;
  std::vector<int> uses(g->vals.size(), 0);
  for (const OpRec& o : ops)
    for (int k = 0; k < o.n_in; ++k) uses[o.in[k]]++;
  auto temp = [&](int64_t s) {
    const Val& v = g->vals[s];
    return v.t.dtype == DVM_F32 && !(v.live || !v.released) && uses[s] == 1;
  };
  auto scalar_op = [](const OpRec& o, int op, float c) {
    return o.op == op && o.n_in == 1 && (o.scalar_pos == 0 || o.scalar_pos == 1) && o.scalar == c;
  };
  std::vector<OpRec> out;
  out.reserve(ops.size());
  for (size_t i = 0; i < ops.size(); ++i) {
    if (i + 3 < ops.size()) {
      const OpRec &a = ops[i], &b = ops[i + 1], &c = ops[i + 2], &d = ops[i + 3];
      const bool neg = (a.op == DVM_OP_NEG && a.n_in == 1) || scalar_op(a, DVM_OP_MUL, -1.f);
      if (neg && b.op == DVM_OP_EXP && b.in[0] == a.out && scalar_op(c, DVM_OP_ADD, 1.f) && c.in[0] == b.out &&
          d.op == DVM_OP_DIV && d.n_in == 2 && d.in[0] == a.in[0] && d.in[1] == c.out && temp(a.out) &&
          temp(b.out) && temp(c.out)) {
        OpRec f = d;
        f.op = OP_SILU;
        f.n_in = 1;
        f.in[1] = -1;
        f.scalar_pos = -1;
        out.push_back(f);
        i += 3;
        continue;
      }
    }
    out.push_back(ops[i]);
  }
  ops.swap(out);
}

// ===========================================================================
// Flushing
// ===========================================================================
// DVM_VERIFY set in the environment (to anything but 0): every program the
// library encodes, merges or stacks is verified before it is handed out or
// launched; a violation fails the flush with DVM_ERR_INTERNAL.
bool verify_on() {
  static const bool on = [] {
    const char* v = std::getenv("DVM_VERIFY");
    return v && *v && std::strcmp(v, "0") != 0;
  }();
  return on;
}

dvm_status checked(dvm_program* p) {
  if (!p || !verify_on()) return DVM_OK;
  std::string e;
  if (!verify_words(p->prog.w, p->n_words, &e)) return fail(DVM_ERR_INTERNAL, "bytecode verifier: %s", e.c_str());
  return DVM_OK;
}

// Encodes one fused op list (after the bytecode clean-up); *out = NULL when no
// op has an effect.  allow_wide: the wide VM build may be chosen.
dvm_status encode_list(dvm_graph* g, const std::vector<OpRec>& list, bool allow_wide, dvm_program** out) {
  *out = nullptr;
  std::vector<OpRec> ops;
  LocalView L;
  make_local(g, list, &L);
  simplify_ops(&L.lg, L.ops, &ops);
  if (ops.empty()) return DVM_OK;  // every op was dead: nothing to run, nothing stored
  fuse_silu(&L.lg, ops);
  dvm_program* p = new (std::nothrow) dvm_program();
  if (!p) return fail(DVM_ERR_INTERNAL, "out of host memory");
  Encoder enc(&L.lg, ops, p);
  dvm_status st = enc.run();
  // The wide VM for row-reduction programs that keep every tile value in the
  // accumulator, when the wide plan puts more rows in a tile and either keeps
  // the LDS staging or runs one tile per workgroup (half the interpreter work
  // per byte, and rows of up to 2560 columns keep their reductions inside a
  // wave: measured 5-25% faster for softmax, RMSNorm and LayerNorm bodies at
  // 5120 columns), and wherever no standard tile fits the rows.  Elementwise
  // programs stay standard.
  const bool acc_only = st == DVM_OK && p->prog.w[H_KTYPE] == KT_VECTOR && enc.treg_hi == 0 &&
                        enc.plan.n_c == 1 && enc.plan.block_dim > 0 && enc.plan.tmpl == TM_ROWREDUCE;
  if (allow_wide && (acc_only || (st != DVM_OK && enc.plan_failed))) {
    const std::string err = g_err;
    dvm_program* q = new (std::nothrow) dvm_program();
    if (q) {
      Encoder w(&L.lg, ops, q);
      w.wide();
      const dvm_status sw = w.run();
      // (staging matters only where a workgroup runs more than one tile)
      const bool take = sw == DVM_OK &&
                        (st != DVM_OK || (w.plan.tr > enc.plan.tr &&
                                          (w.plan.body_tile == 1 ||
                                           (w.staged_pf >= enc.staged_pf && w.staged_inv >= enc.staged_inv))));
      if (take) {
        delete p;
        p = q;
        st = DVM_OK;
      } else {
        delete q;
        g_err = err;
      }
    }
  }
  if (st == DVM_OK) st = checked(p);
  if (st != DVM_OK) {
    delete p;
    return st;
  }
  *out = p;
  return DVM_OK;
}

// The ops leave the buffer: their values are stored (ran = a program that
// computes them was produced) or lost; their input references are dropped.
void retire(dvm_graph* g, std::vector<OpRec>& list, bool ran) {
  for (auto& o : list) {
    Val& v = g->vals[o.out];
    v.pending = false;
    const bool stored = ran && (v.live || !v.released) && v.t.data;
    v.stored = stored;
    v.lost = !stored;
  }
  drop_uses(g, list);
}

void note_encode(dvm_graph* g, std::chrono::steady_clock::time_point t0, const dvm_program* p) {
  const double us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
  g->stats.graphs++;
  g->stats.encode_us_total += us;
  g->stats.encode_us_max = std::max(g->stats.encode_us_max, us);
  if (!g->flush_log.empty()) g->flush_log.back().encode_us = (float)us;
  if (p) {
    g->stats.bytes += p->bytes;
    if (!g->flush_log.empty()) g->flush_log.back().bytes = p->bytes;
  }
}

dvm_status encode_buffer(dvm_graph* g, dvm_program** out) {
  *out = nullptr;
  if (g->buf.empty()) return DVM_OK;
  const auto t0 = std::chrono::steady_clock::now();
  dvm_program* p = nullptr;
  const dvm_status st = encode_list(g, g->buf, true, &p);
  // the buffered values leave the buffer whatever the outcome
  std::vector<OpRec> done;
  done.swap(g->buf);
  retire(g, done, st == DVM_OK && p);
  note_encode(g, t0, p);
  if (st != DVM_OK) return st;
  *out = p;
  return DVM_OK;
}

// Branch program from the programs of the two bodies (DVM's dynamic control
// flow, resolved on the device: the condition is read by the VM, not by the
// host).  Both must share one tiling, operand table and prologue; the merged
// program appends the condition operand to the table and the else-body after
// the then-body.
// fold: the combine held back for the condition (its partials are folded
// by the branch program, HF_COND_FOLD), or null.
dvm_status merge_branch(const dvm_program* pt, const dvm_program* pe, const dvm_tensor& cond, float thr,
                        const HeldCombine* fold, dvm_program** out) {
  const uint32_t* A = pt->prog.w;
  const uint32_t* B = pe->prog.w;
  static const int same[] = {H_KTYPE, H_TEMPLATE, H_BLOCK_DIM, H_BODY_TILE, H_GRID, H_TR, H_TC, H_G, H_NV, H_P,
                             H_NC, H_NARGS, H_R_LO, H_R_HI, H_C_LO, H_C_HI, H_FLAGS, H_LDS_BYTES, H_PF_OFF0,
                             H_PF_OFF1, H_INV_OFF0, H_INV_OFF1, H_INV_SHARED0, H_INV_SHARED1, H_RED_OFF};
  for (int h : same)
    if (A[h] != B[h]) return fail(DVM_ERR_UNSUPPORTED, "branch bodies differ in their tiling (header word %d)", h);
  if (A[H_KTYPE] == KT_MIX || A[H_TEMPLATE] == TM_ALLREDUCE)
    return fail(DVM_ERR_UNSUPPORTED, "branch bodies must be elementwise or row-reduce graphs");
  const uint32_t n_args = A[H_NARGS];
  for (uint32_t q = ARG_BASE; q < ARG_BASE + n_args * ARG_WORDS; ++q)
    if (A[q] != B[q]) return fail(DVM_ERR_UNSUPPORTED, "branch bodies read or write different operands");
  const uint32_t pro_n = A[H_PRO_END] - A[H_PRO_BEGIN];
  if (pro_n != B[H_PRO_END] - B[H_PRO_BEGIN] ||
      !std::equal(A + A[H_PRO_BEGIN], A + A[H_PRO_END], B + B[H_PRO_BEGIN]))
    return fail(DVM_ERR_UNSUPPORTED, "branch bodies stage different operands");
  const uint32_t n_extra = fold ? 2u : 1u;  // the condition, and the partials it is folded from
  if (n_args + n_extra > (uint32_t)MAX_ARGS) return fail(DVM_ERR_RESOURCE, "too many operands");
  const uint32_t then_n = A[H_BODY_END] - A[H_BODY_BEGIN], else_n = B[H_BODY_END] - B[H_BODY_BEGIN];
  const uint32_t base = ARG_BASE + (n_args + n_extra) * ARG_WORDS;
  if (base + pro_n + then_n + else_n + PAD_WORDS > (uint32_t)MAX_WORDS) return fail(DVM_ERR_RESOURCE, "program too large");
  dvm_program* q = new (std::nothrow) dvm_program();
  if (!q) return fail(DVM_ERR_INTERNAL, "out of host memory");
  uint32_t* W = q->prog.w;
  std::copy(A, A + ARG_BASE + n_args * ARG_WORDS, W);
  uint32_t* c = W + ARG_BASE + n_args * ARG_WORDS;
  const uint64_t cp = (uint64_t)(uintptr_t)cond.data;
  c[A_PTR_LO] = (uint32_t)cp;
  c[A_PTR_HI] = (uint32_t)(cp >> 32);
  c[A_DTYPE] = DT_F32;
  c[A_FLAGS] = arg_flags_word(0, 4);
  c[A_EXTENT] = 4;
  if (fold) {
    uint32_t* f = c + ARG_WORDS;
    const uint64_t fp = (uint64_t)(uintptr_t)fold->part;
    f[A_PTR_LO] = (uint32_t)fp;
    f[A_PTR_HI] = (uint32_t)(fp >> 32);
    f[A_DTYPE] = DT_F32;
    f[A_FLAGS] = arg_flags_word(0, 4ull * fold->n_part);
    f[A_EXTENT] = 4u * fold->n_part;
  }
  std::copy(A + A[H_PRO_BEGIN], A + A[H_PRO_END], W + base);
  std::copy(A + A[H_BODY_BEGIN], A + A[H_BODY_END], W + base + pro_n);
  std::copy(B + B[H_BODY_BEGIN], B + B[H_BODY_END], W + base + pro_n + then_n);
  W[H_NARGS] = n_args + n_extra;
  W[H_PRO_BEGIN] = base;
  W[H_PRO_END] = W[H_BODY_BEGIN] = base + pro_n;
  W[H_BODY_END] = W[H_ALT_BEGIN] = base + pro_n + then_n;
  W[H_ALT_END] = base + pro_n + then_n + else_n;
  W[H_FLAGS] |= HF_BRANCH;
  W[H_COND_ARG] = n_args;
  std::memcpy(&W[H_COND_THR], &thr, 4);
  if (fold) {
    W[H_FLAGS] |= HF_COND_FOLD;
    W[H_ALL_SCRATCH] = n_args + 1;
    W[H_ALL_KIND] = fold->kind;
  }
  W[H_N_INSTR] = (pro_n + then_n + else_n) / 2;
  q->n_words = W[H_ALT_END];
  q->n_instr = W[H_N_INSTR];
  q->R = pt->R;
  q->C = pt->C;
  q->pad = pt->pad;
  q->grid_launch = pt->grid_launch;
  q->bytes = std::max(pt->bytes, pe->bytes) + 4 + (fold ? 4ull * fold->n_part : 0);
  q->lds = pt->lds;
  q->reads = pt->reads;
  q->reads.insert(q->reads.end(), pe->reads.begin(), pe->reads.end());
  q->reads.push_back({(uintptr_t)cond.data, 4});
  q->writes = pt->writes;
  q->writes.insert(q->writes.end(), pe->writes.begin(), pe->writes.end());
  if (fold) {
    q->reads.push_back({(uintptr_t)fold->part, 4ull * fold->n_part});
    q->writes.push_back({(uintptr_t)cond.data, 4});
  }
  const dvm_status v = checked(q);
  if (v != DVM_OK) {
    delete q;
    return v;
  }
  *out = q;
  return DVM_OK;
}

// The reduce-all scratch area of stream s (allocated and zeroed on first use).
dvm_status stream_scratch(dvm_context* ctx, hipStream_t s, void** out) {
  std::lock_guard<std::mutex> lk(ctx->mu);
  for (auto& e : ctx->scratch)
    if (e.first == s) {
      *out = e.second;
      return DVM_OK;
    }
  void* p = nullptr;
  hipError_t e = hipMalloc(&p, SCRATCH_BYTES);
  if (e != hipSuccess) return fail(DVM_ERR_DEVICE, "scratch allocation failed: %s", hipGetErrorString(e));
  e = hipMemset(p, 0, SCRATCH_BYTES);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipFree(p);
    return fail(DVM_ERR_DEVICE, "scratch init failed: %s", hipGetErrorString(e));
  }
  ctx->scratch.push_back({s, p});
  *out = p;
  return DVM_OK;
}

bool needs_scratch(const dvm_program* p) {
  return p->segments == 1 && p->prog.w[H_KTYPE] != KT_MIX && p->prog.w[H_TEMPLATE] == TM_ALLREDUCE;
}

// Points the program's reduce-all scratch operand at `area` of `bytes`.
void set_scratch(Program* q, void* area, uint64_t bytes) {
  uint32_t* b = q->w + ARG_BASE + q->w[H_ALL_SCRATCH] * ARG_WORDS;
  const uint64_t a = (uint64_t)(uintptr_t)area;
  b[A_PTR_LO] = (uint32_t)a;
  b[A_PTR_HI] = (uint32_t)(a >> 32);
  b[A_FLAGS] = arg_flags_word(0, bytes);
  b[A_EXTENT] = (uint32_t)bytes;
}

hipError_t launch_words(const Program* q, uint32_t kt, uint32_t grid, uint32_t lds, hipStream_t s) {
  return kt == KT_MIX           ? dvm_launch_mix_kernel(q, grid, s)
         : kt == KT_VECTOR_WIDE ? dvm_launch_vector_kernel_wide(q, grid, lds, s)
                                : dvm_launch_vector_kernel(q, grid, lds, s);
}

// Kernel type of a program (a stacked program: that of its segments).
uint32_t ktype_of(const dvm_program* p) {
  const uint32_t* W = p->prog.w;
  return p->segments > 1 ? W[W[S_DIR] + H_KTYPE] : W[H_KTYPE];
}

hipError_t launch_kernel(const dvm_program* p, const Program* q, hipStream_t s) {
  return launch_words(q, ktype_of(p), p->grid_launch, p->lds, s);
}

// The second launch of a reduce-all program (q: its words with the scratch
// area set): folds the workgroups' partials, which the stream orders before
// it, into the scalar output.
HeldCombine combine_of(const dvm_program* p, const Program* q, hipStream_t s) {
  const uint32_t* W = q->w;
  const uint32_t* sa = W + ARG_BASE + W[H_ALL_SCRATCH] * ARG_WORDS;
  const uint32_t* oa = W + ARG_BASE + W[H_ALL_OUT] * ARG_WORDS;
  const uint64_t area = ((uint64_t)sa[A_PTR_HI] << 32) | sa[A_PTR_LO];
  const uint64_t out = ((uint64_t)oa[A_PTR_HI] << 32) | oa[A_PTR_LO];
  // one partial per launched workgroup, never past the area
  const uint64_t slots = sa[A_EXTENT] > SCRATCH_PART_OFF ? (sa[A_EXTENT] - SCRATCH_PART_OFF) / 4u : 0u;
  HeldCombine c;
  c.s = s;
  c.part = reinterpret_cast<const float*>((uintptr_t)(area + SCRATCH_PART_OFF));
  c.n_part = (uint32_t)std::min<uint64_t>(p->grid_launch, slots);
  c.kind = W[H_ALL_KIND];
  c.out = reinterpret_cast<void*>((uintptr_t)out);
  c.out_dt = oa[A_DTYPE];
  return c;
}

hipError_t launch_held(const HeldCombine& c) {
  return dvm_launch_allreduce_combine(c.part, c.n_part, c.kind, c.out, c.out_dt, c.s);
}

hipError_t launch_combine(const dvm_program* p, const Program* q, hipStream_t s) {
  return launch_held(combine_of(p, q, s));
}

// Launches the combine held back on stream s, if any.  Every launch and sync
// on a stream runs this first, so the scalar is written before anything
// after it on the stream can read it, and before the next reduce-all on the
// stream rewrites the partials.
hipError_t settle(dvm_context* ctx, hipStream_t s) {
  HeldCombine c;
  {
    std::lock_guard<std::mutex> lk(ctx->mu);
    auto it = std::find_if(ctx->held.begin(), ctx->held.end(), [&](const HeldCombine& h) { return h.s == s; });
    if (it == ctx->held.end()) return hipSuccess;
    c = *it;
    ctx->held.erase(it);
  }
  return launch_held(c);
}

// Takes the combine held back on stream s if it writes the fp32 scalar at
// `out` (the branch program then folds the partials instead; the VM folds at
// most 2 T_LANES partials, one per workgroup of a reduce-all's launch).
bool take_held(dvm_context* ctx, hipStream_t s, const void* out, HeldCombine* c) {
  std::lock_guard<std::mutex> lk(ctx->mu);
  auto it = std::find_if(ctx->held.begin(), ctx->held.end(), [&](const HeldCombine& h) { return h.s == s; });
  if (it == ctx->held.end() || it->out != out || it->out_dt != DT_F32 || it->n_part == 0 ||
      it->n_part > 2u * T_LANES)
    return false;
  *c = *it;
  ctx->held.erase(it);
  return true;
}

dvm_status launch(dvm_context* ctx, const dvm_program* p, hipStream_t s) {
  if (!ctx || ctx->device < 0) return fail(DVM_ERR_DEVICE, "encode-only context cannot launch");
  hipError_t e = settle(ctx, s);
  if (e != hipSuccess) return fail(DVM_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
  if (p->grid_launch == 0) return DVM_OK;
  if (needs_scratch(p)) {
    void* area;
    dvm_status st = stream_scratch(ctx, s, &area);
    if (st != DVM_OK) return st;
    Program q = p->prog;  // the launch copies its argument: a stack copy is enough
    set_scratch(&q, area, SCRATCH_BYTES);
    e = launch_kernel(p, &q, s);
    if (e == hipSuccess) {
      const HeldCombine c = combine_of(p, &q, s);
      std::unique_lock<std::mutex> lk(ctx->mu);
      if (ctx->hold && ctx->hold_stream == s) {
        ctx->held.push_back(c);  // settle() above left none on s
      } else {
        lk.unlock();
        e = launch_held(c);
      }
    }
  } else {
    e = launch_kernel(p, &p->prog, s);
  }
  if (e != hipSuccess) return fail(DVM_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
  return DVM_OK;
}

// Runs a program: launches it on the graph's stream, or, in an encode-only
// context, holds it for dvm_graph_take_program.  Takes ownership of p.
dvm_status run_program(dvm_graph* g, dvm_program* p, int32_t* launched) {
  if (g->ctx->device < 0) {
    if (g->held.size() >= MAX_HELD) {
      delete g->held.front();
      g->held.pop_front();
    }
    g->held.push_back(p);
    return DVM_OK;
  }
  const auto t0 = std::chrono::steady_clock::now();
  const dvm_status st = launch(g->ctx, p, g->stream);
  g->stats.launch_us_total += std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
  if (st == DVM_OK) {
    g->stats.launches++;
    if (launched) *launched = 1;
  }
  delete p;
  return st;
}

// Stacking (DVM review page, section 5.1, stacking-based fusion): a program
// may join the graph's stack if it runs on the same VM build as the stack,
// is no reduce-all or branch program (those need the stream's scratch or a
// condition written before them), fits the kernel argument beside the stack,
// and is independent of every stacked program: it writes nothing they read
// or write, and reads nothing they write.  Stacked programs run side by side
// on disjoint workgroups, in one launch.
bool stackable(const dvm_program* p) {
  const uint32_t* W = p->prog.w;
  return p->segments == 1 && p->grid_launch > 0 && (W[H_KTYPE] == KT_VECTOR || W[H_KTYPE] == KT_VECTOR_WIDE) &&
         W[H_TEMPLATE] != TM_ALLREDUCE && !(W[H_FLAGS] & HF_BRANCH);
}

bool overlaps(const std::vector<Range>& a, const std::vector<Range>& b) {
  for (const Range& x : a)
    for (const Range& y : b)
      if (x.second && y.second && x.first < y.first + y.second && y.first < x.first + x.second) return true;
  return false;
}

uint32_t stack_words(const std::vector<dvm_program*>& ps) {
  uint32_t n = STACK_DIR_WORDS;
  for (const dvm_program* p : ps) n += p->n_words + PAD_WORDS;
  return n;
}

bool fits_stack(const dvm_graph* g, const dvm_program* p) {
  const std::vector<dvm_program*>& st = g->stack;
  if (st.size() >= (size_t)MAX_SEGS || st[0]->prog.w[H_KTYPE] != p->prog.w[H_KTYPE]) return false;
  if (stack_words(st) + p->n_words + PAD_WORDS > (uint32_t)MAX_WORDS) return false;
  for (const dvm_program* q : st)
    if (overlaps(p->writes, q->reads) || overlaps(p->writes, q->writes) || overlaps(p->reads, q->writes)) return false;
  return true;
}

// One program from 2..MAX_SEGS programs of one VECTOR build: the directory,
// then each program's words.  Spatial: each segment keeps its workgroups, in
// launch order.  Temporal: one tile space over the segments in order, run by
// min(G, total tiles) workgroups (tile u on workgroup u mod grid), each
// walking the segments in sequence.
dvm_status build_stack(const dvm_program* const* ps, size_t n, bool temporal, dvm_program** out) {
  *out = nullptr;
  if (n < 2 || n > (size_t)MAX_SEGS) return fail(DVM_ERR_INVALID_ARG, "a stack holds 2 to %d programs", MAX_SEGS);
  const uint32_t kt = ps[0]->prog.w[H_KTYPE];
  uint32_t words = STACK_DIR_WORDS;
  for (size_t i = 0; i < n; ++i) {
    const dvm_program* p = ps[i];
    if (!p) return fail(DVM_ERR_INVALID_ARG, "null program");
    if (p->segments != 1 || (kt != KT_VECTOR && kt != KT_VECTOR_WIDE) || p->prog.w[H_KTYPE] != kt)
      return fail(DVM_ERR_UNSUPPORTED, "stacked programs share one VECTOR build");
    if (p->prog.w[H_TEMPLATE] == TM_ALLREDUCE) return fail(DVM_ERR_UNSUPPORTED, "reduce-all programs do not stack");
    words += p->n_words + PAD_WORDS;
  }
  if (words > (uint32_t)MAX_WORDS) return fail(DVM_ERR_RESOURCE, "stacked programs exceed %d words", MAX_WORDS);
  dvm_program* q = new (std::nothrow) dvm_program();
  if (!q) return fail(DVM_ERR_INTERNAL, "out of host memory");
  uint32_t* W = q->prog.w;
  W[0] = temporal ? TSTACK_MAGIC : STACK_MAGIC;
  W[S_NSEG] = (uint32_t)n;
  uint32_t off = STACK_DIR_WORDS, wg = 0, tiles = 0;
  for (size_t i = 0; i < n; ++i) {
    const dvm_program* p = ps[i];
    W[S_DIR + 2 * i] = off;
    W[S_DIR + 2 * i + 1] = temporal ? tiles : wg;
    std::copy(p->prog.w, p->prog.w + p->n_words, W + off);
    off += p->n_words + PAD_WORDS;
    wg += p->grid_launch;
    tiles += p->prog.w[H_BLOCK_DIM];
    q->lds = std::max(q->lds, p->lds);
    q->bytes += p->bytes;
    q->n_instr += p->n_instr;
    q->reads.insert(q->reads.end(), p->reads.begin(), p->reads.end());
    q->writes.insert(q->writes.end(), p->writes.begin(), p->writes.end());
  }
  q->segments = (uint32_t)n;
  q->n_words = off;
  q->grid_launch = temporal ? (uint32_t)std::min<int64_t>(tiling::G, tiles) : wg;
  q->R = ps[0]->R;
  q->C = ps[0]->C;
  const dvm_status v = checked(q);
  if (v != DVM_OK) {
    delete q;
    return v;
  }
  *out = q;
  return DVM_OK;
}

// Launches (or holds) what the graph's stack holds, as one program.
dvm_status launch_stack(dvm_graph* g, int32_t* launched) {
  std::vector<dvm_program*> st;
  st.swap(g->stack);
  if (st.empty()) return DVM_OK;
  if (st.size() == 1) return run_program(g, st[0], launched);
  // Spatial stacks put the segments with the most work per workgroup first:
  // the dispatcher hands out workgroups in segment order, so the launch ends
  // on the shortest ones (the stacked programs are independent, so the order
  // does not change any result).
  if (!g->stack_temporal)
    std::stable_sort(st.begin(), st.end(), [](const dvm_program* a, const dvm_program* b) {
      auto work = [](const dvm_program* p) {
        const uint32_t* W = p->prog.w;
        return W[H_BLOCK_DIM] ? (double)p->bytes * W[H_BODY_TILE] / W[H_BLOCK_DIM] : 0.0;
      };
      return work(a) > work(b);
    });
  dvm_program* q = nullptr;
  dvm_status e = build_stack(st.data(), st.size(), g->stack_temporal, &q);
  for (dvm_program* p : st) delete p;
  if (e != DVM_OK) return e;
  g->stats.stacked += st.size();
  return run_program(g, q, launched);
}

// A newly encoded program: joins the stack, or runs after what the stack held.
dvm_status submit(dvm_graph* g, dvm_program* p, int32_t* launched) {
  if (g->stack_max > 1 && stackable(p)) {
    if (!g->stack.empty() && !fits_stack(g, p)) {
      const dvm_status e = launch_stack(g, launched);
      if (e != DVM_OK) {
        delete p;
        return e;
      }
    }
    g->stack.push_back(p);
    if (g->stack.size() >= (size_t)g->stack_max) return launch_stack(g, launched);
    return DVM_OK;
  }
  const dvm_status e = launch_stack(g, launched);
  if (e != DVM_OK) {
    delete p;
    return e;
  }
  return run_program(g, p, launched);
}

dvm_status flush_launch(dvm_graph* g, int reason, int32_t* launched) {
  if (launched) *launched = 0;
  if (g->buf.empty()) return DVM_OK;
  g->stats.flush_reason[reason]++;
  g->flush_log.push_back({(int32_t)g->buf.size(), (int32_t)reason, 0.f, 0});
  dvm_program* p = nullptr;
  dvm_status st = encode_buffer(g, &p);
  if (st != DVM_OK || !p) return st;
  return submit(g, p, launched);
}

// Host time of one fuser call (capture and fusion decisions), without the
// encodes and launches of the flushes it triggers.
struct FuseTimer {
  dvm_graph* g;
  std::chrono::steady_clock::time_point t0;
  double enc0, lau0;
  explicit FuseTimer(dvm_graph* gr)
      : g(gr), t0(std::chrono::steady_clock::now()), enc0(gr ? gr->stats.encode_us_total : 0.0),
        lau0(gr ? gr->stats.launch_us_total : 0.0) {}
  ~FuseTimer() {
    if (!g) return;
    const double us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count() -
                      (g->stats.encode_us_total - enc0) - (g->stats.launch_us_total - lau0);
    g->stats.fuse_us_total += std::max(us, 0.0);
  }
};

bool infer(const dvm_graph* g, int32_t op, const int64_t* in, int n_in, const dvm_attrs* at, Shape* out) {
  if (op < 0 || op >= DVM_OP_COUNT) return false;
  auto sh = [&](int k) { return g->vals[in[k]].shape; };
  if (op == DVM_OP_MATMUL) {
    if (n_in != 2) return false;
    const Shape a = sh(0), b = sh(1);
    if (a.nd != 2 || b.nd != 2 || a.d[1] != b.d[0]) return false;
    out->nd = 2;
    out->d[0] = a.d[0];
    out->d[1] = b.d[1];
    return true;
  }
  if (is_reduce(op)) {
    if (n_in != 1) return false;
    const Shape a = sh(0);
    if (at && at->axis == DVM_AXIS_ALL) {
      out->nd = 0;
      return true;
    }
    if (a.nd == 0) return false;
    *out = row_shape(a);
    return true;
  }
  if (is_binary(op)) {
    if (n_in == 2) return broadcast(sh(0), sh(1), out);
    if (n_in == 1 && at && (at->scalar_pos == 0 || at->scalar_pos == 1)) {
      *out = sh(0);
      return true;
    }
    return false;
  }
  if (n_in != 1) return false;
  *out = sh(0);
  return true;
}

dvm_status check_tensor(const dvm_tensor* t) {
  if (!t) return fail(DVM_ERR_INVALID_ARG, "null tensor");
  if (t->ndim < 0 || t->ndim > 4) return fail(DVM_ERR_INVALID_ARG, "ndim %d out of range", t->ndim);
  if (t->dtype < 0 || t->dtype > DVM_U8) return fail(DVM_ERR_INVALID_ARG, "bad dtype %d", t->dtype);
  for (int i = 0; i < t->ndim; ++i) {
    if (t->shape[i] < 0) return fail(DVM_ERR_INVALID_ARG, "negative dim");
    if (t->stride[i] < 0) return fail(DVM_ERR_INVALID_ARG, "negative stride");
  }
  return DVM_OK;
}

dvm_status end_group_impl(dvm_graph* g, int32_t* flushed) {
  if (flushed) *flushed = 0;
  g->in_group = false;
  if (g->grp.empty()) return DVM_OK;
  g->stats.groups++;
  std::vector<OpRec> grp;
  grp.swap(g->grp);
  if (!g->buf.empty()) {
    std::vector<OpRec> cand = g->buf;
    cand.insert(cand.end(), grp.begin(), grp.end());
    LocalView L;
    make_local(g, cand, &L);
    Checker ck(&L.lg, L.ops);
    const int why = ck.check(g->buf.size());
    if (why < 0) {
      g->buf.swap(cand);
      g->stats.ops += grp.size();
      if (is_reduce_all(g->buf.back())) return flush_launch(g, FR_REDUCE_ALL, flushed);
      return DVM_OK;
    }
    dvm_status st = flush_launch(g, why, flushed);
    if (flushed) *flushed = 1;
    if (st != DVM_OK) {
      // the buffered graph was not run: the new group, which may read its
      // values, is dropped too; its results are lost, never pending
      for (auto& o : grp) {
        Val& v = g->vals[o.out];
        v.pending = false;
        v.lost = true;
      }
      drop_uses(g, grp);
      return st;
    }
  }
  LocalView L;
  make_local(g, grp, &L);
  Checker ck(&L.lg, L.ops);
  const int why = ck.check(0);
  if (why >= 0) {
    g->stats.unsupported++;
    for (auto& o : grp) {
      Val& v = g->vals[o.out];
      v.pending = false;
      v.lost = true;
    }
    drop_uses(g, grp);
    return fail(DVM_ERR_UNSUPPORTED, "group cannot run on the VM (rule %d)", why);
  }
  g->buf = std::move(grp);
  g->stats.ops += g->buf.size();
  if (is_reduce_all(g->buf.back())) return flush_launch(g, FR_REDUCE_ALL, flushed);
  return DVM_OK;
}

// ===========================================================================
// Static-graph symbolic fusion (DVM review page, section 5.2, static-graph
// fusion; section 7's table lists it beside the dynamic, streaming kind).
//
// A template is an op graph recorded once with symbolic dims.  finalize()
// decides its fusion partition once, by running the streaming fuser's rules
// on representative shapes: each symbol stands for one size shared by all its
// occurrences and distinct from every other symbol and every concrete dim of
// the template, so every shape equality and broadcast the rules test comes
// out as it would for any binding.  Tensors get distinct, non-overlapping
// stand-in addresses (a binding must not alias them: run() checks).  run()
// binds concrete tensors and only tiles and encodes the precomputed graphs --
// no per-op fusion decision.  Readings: symbols are >= 2 (a symbol is never a
// broadcast dim); a tiling that exists for the representative shape may not
// exist for a binding (run() then fails with DVM_ERR_RESOURCE); a value that
// one graph produces and a later graph reads must be a template output (it
// needs storage the caller owns).
// ===========================================================================
struct TmplVal {
  int32_t dtype = 0;
  int nd = 0;
  int64_t dim[4] = {0, 0, 0, 0};  // >= 0 concrete, < 0 symbol -(k + 1)
  int op = -1;                    // producing op (-1: an input)
  int io = -1;                    // input or output index (-1: internal)
};

struct TmplOp {
  int32_t op = 0;
  int n_in = 0;
  int64_t in[2] = {-1, -1};
  dvm_attrs at{-1, -1, 0.f};
  int64_t out = -1;
  int group = 0;
};

}  // namespace

struct dvm_template {
  dvm_context* ctx = nullptr;
  std::vector<TmplVal> vals;
  std::vector<TmplOp> ops;
  std::vector<int64_t> inputs, outputs;  // value ids in binding order
  int n_groups = 0;
  bool in_group = false;
  bool finalized = false;
  std::vector<int32_t> graph_of_op;
  int32_t n_graphs = 0;
  double finalize_us = 0.0;
  dvm_graph* rg = nullptr;  // the graph runs encode and launch through
};

namespace {

int64_t sym_dim(const dvm_template* t, int64_t d, const std::vector<int64_t>& rep) {
  return d >= 0 ? d : rep[(size_t)(-d - 1)];
}

// One size per symbol: multiples of 8 (matmul operand forms), at least 1032,
// distinct from one another and from every concrete dim of the template.
std::vector<int64_t> representatives(const dvm_template* t) {
  std::vector<int64_t> concrete;
  int64_t n_sym = 0;
  for (const TmplVal& v : t->vals)
    for (int i = 0; i < v.nd; ++i) {
      if (v.dim[i] >= 0) concrete.push_back(v.dim[i]);
      else n_sym = std::max(n_sym, -v.dim[i]);
    }
  std::vector<int64_t> rep;
  for (int64_t cand = 1032; (int64_t)rep.size() < n_sym; cand += 8)
    if (std::find(concrete.begin(), concrete.end(), cand) == concrete.end()) rep.push_back(cand);
  return rep;
}

dvm_tensor stand_in(const TmplVal& v, int64_t id, const std::vector<int64_t>& rep, const dvm_template* t) {
  dvm_tensor x{};
  x.data = (void*)(uintptr_t)(((uint64_t)id + 1) << 40);
  x.dtype = v.dtype;
  x.ndim = v.nd;
  int64_t acc = 1;
  for (int i = v.nd - 1; i >= 0; --i) {
    x.shape[i] = sym_dim(t, v.dim[i], rep);
    x.stride[i] = acc;
    acc *= x.shape[i];
  }
  return x;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* dvm_last_error(void) { return g_err.c_str(); }

dvm_status dvm_context_create(int device, dvm_context** out) {
  if (!out) return fail(DVM_ERR_INVALID_ARG, "null out");
  *out = nullptr;
  dvm_context* c = new (std::nothrow) dvm_context();
  if (!c) return fail(DVM_ERR_INTERNAL, "out of host memory");
  c->device = device;
  if (device >= 0) {
    hipError_t e = hipSetDevice(device);
    if (e != hipSuccess) {
      delete c;
      return fail(DVM_ERR_DEVICE, "hipSetDevice(%d) failed: %s", device, hipGetErrorString(e));
    }
    // with the device current: the address of its copy of the static scratch
    c->static_err = dvm_static_scratch_init(device, &c->static_scratch, &c->static_bytes);
  }
  *out = c;
  return DVM_OK;
}

void dvm_context_destroy(dvm_context* ctx) {
  if (!ctx) return;
  if (!ctx->scratch.empty()) {
    (void)hipDeviceSynchronize();
    for (auto& e : ctx->scratch) (void)hipFree(e.second);
  }
  delete ctx;
}

dvm_status dvm_graph_create(dvm_context* ctx, void* stream, dvm_graph** out) {
  if (!ctx || !out) return fail(DVM_ERR_INVALID_ARG, "null argument");
  dvm_graph* g = new (std::nothrow) dvm_graph();
  if (!g) return fail(DVM_ERR_INTERNAL, "out of host memory");
  g->ctx = ctx;
  g->stream = (hipStream_t)stream;
  *out = g;
  return DVM_OK;
}

void dvm_graph_destroy(dvm_graph* g) {
  // a branch left open may hold back the combine that writes its condition
  if (g && g->branch && g->ctx->device >= 0) (void)settle(g->ctx, g->stream);
  delete g;
}

dvm_status dvm_graph_take_program(dvm_graph* g, dvm_program** out) {
  if (!g || !out) return fail(DVM_ERR_INVALID_ARG, "null argument");
  *out = nullptr;
  if (!g->held.empty()) {
    *out = g->held.front();
    g->held.pop_front();
  }
  return DVM_OK;
}

dvm_status dvm_graph_input(dvm_graph* g, const dvm_tensor* t, dvm_value* out) {
  FuseTimer ft(g);
  if (!g || !out) return fail(DVM_ERR_INVALID_ARG, "null argument");
  dvm_status st = check_tensor(t);
  if (st != DVM_OK) return st;
  const int64_t s = new_slot(g);
  Val& v = g->vals[s];
  v.kind = VK_INPUT;
  v.t = *t;
  v.shape = shape_of(*t);
  v.stored = true;
  *out = handle(g, s);
  return DVM_OK;
}

dvm_status dvm_graph_begin_group(dvm_graph* g) {
  if (!g) return fail(DVM_ERR_INVALID_ARG, "null graph");
  if (g->in_group) return fail(DVM_ERR_INVALID_ARG, "group already open");
  if (g->branch) return fail(DVM_ERR_INVALID_ARG, "groups cannot open inside a branch");
  g->in_group = true;
  return DVM_OK;
}

dvm_status dvm_graph_end_group(dvm_graph* g, int32_t* flushed) {
  FuseTimer ft(g);
  if (!g) return fail(DVM_ERR_INVALID_ARG, "null graph");
  if (!g->in_group) return fail(DVM_ERR_INVALID_ARG, "no open group");
  return end_group_impl(g, flushed);
}

dvm_status dvm_graph_infer_shape(dvm_graph* g, int32_t op, const dvm_value* in, int32_t n_in,
                                 const dvm_attrs* attrs, dvm_tensor* out_shape) {
  if (!g || !out_shape || n_in < 0 || n_in > 2) return fail(DVM_ERR_INVALID_ARG, "bad argument");
  int64_t slots[2];
  for (int k = 0; k < n_in; ++k)
    if (!resolve(g, in[k], &slots[k])) return fail(DVM_ERR_INVALID_ARG, "unknown value");
  Shape s;
  if (!infer(g, op, slots, n_in, attrs, &s)) return fail(DVM_ERR_SHAPE, "shapes do not fit op %d", op);
  out_shape->ndim = s.nd;
  for (int i = 0; i < s.nd; ++i) out_shape->shape[i] = s.d[i];
  return DVM_OK;
}

dvm_status dvm_graph_add_op(dvm_graph* g, int32_t op, const dvm_value* in, int32_t n_in, const dvm_attrs* attrs,
                            const dvm_tensor* out, uint32_t flags, dvm_value* out_value) {
  FuseTimer ft(g);
  if (!g || !out || !out_value || (n_in > 0 && !in)) return fail(DVM_ERR_INVALID_ARG, "null argument");
  if (n_in < 1 || n_in > 2) return fail(DVM_ERR_INVALID_ARG, "n_in %d", n_in);
  dvm_status st = check_tensor(out);
  if (st != DVM_OK) return st;
  OpRec r;
  r.op = op;
  r.n_in = n_in;
  for (int k = 0; k < n_in; ++k) {
    if (!resolve(g, in[k], &r.in[k])) return fail(DVM_ERR_INVALID_ARG, "unknown or released value");
    const Val& v = g->vals[r.in[k]];
    if (v.released) return fail(DVM_ERR_INVALID_ARG, "input was released");
    if (v.lost) return fail(DVM_ERR_INVALID_ARG, "input's graph was flushed without storing it");
  }
  if (attrs) {
    r.axis = attrs->axis;
    r.scalar_pos = attrs->scalar_pos;
    r.scalar = attrs->scalar;
  }
  if (is_binary(op) && n_in == 1 && !(attrs && (attrs->scalar_pos == 0 || attrs->scalar_pos == 1)))
    return fail(DVM_ERR_INVALID_ARG, "binary op needs two inputs or a scalar operand");
  if (is_reduce(op) && r.axis != -1 && r.axis != DVM_AXIS_ALL) return fail(DVM_ERR_UNSUPPORTED, "reduce axis");
  Shape s;
  if (!infer(g, op, r.in, n_in, attrs, &s)) return fail(DVM_ERR_SHAPE, "shapes do not fit op %d", op);
  if (shape_of(*out) != s) return fail(DVM_ERR_SHAPE, "out shape differs from the inferred shape");
  // F1: the op set and dtypes the VM runs
  if (op == DVM_OP_ISFINITE && out->dtype != DVM_U8) return fail(DVM_ERR_UNSUPPORTED, "isfinite writes u8");
  if (op != DVM_OP_ISFINITE && out->dtype == DVM_U8) return fail(DVM_ERR_UNSUPPORTED, "u8 output");
  if (op == DVM_OP_MATMUL) {
    // the MIX kernel's operand forms: bf16 A [M, K] and B [K, N], unit stride
    // along K (A) and N (B), 16-byte aligned rows, K and N multiples of 8
    const dvm_tensor& A = g->vals[r.in[0]].t;
    const dvm_tensor& B = g->vals[r.in[1]].t;
    // (with K = 0 nothing of A or B is read: their layout does not matter)
    const bool k0 = A.shape[1] == 0;
    const bool ok = A.dtype == DVM_BF16 && B.dtype == DVM_BF16 && B.shape[1] % 8 == 0 &&
                    (k0 || (A.stride[1] == 1 && B.stride[1] == 1 && A.shape[1] % 8 == 0 && A.stride[0] % 8 == 0 &&
                            B.stride[0] % 8 == 0 && (uintptr_t)A.data % 16 == 0 && (uintptr_t)B.data % 16 == 0)) &&
                    (out->dtype == DVM_F32 || out->dtype == DVM_BF16);
    if (!ok) return fail(DVM_ERR_UNSUPPORTED, "matmul operands outside the MIX kernel's forms");
  }
  const int64_t slot = new_slot(g);
  Val& v = g->vals[slot];
  v.kind = VK_OP;
  v.t = *out;
  v.shape = s;
  v.live = (flags & DVM_OUT_LIVE) != 0;
  v.pending = true;
  r.out = slot;
  *out_value = handle(g, slot);
  for (int k = 0; k < n_in; ++k) g->vals[r.in[k]].uses++;
  if (g->branch) {
    g->br[g->branch - 1].push_back(r);
    g->stats.ops++;
    return DVM_OK;
  }
  g->grp.push_back(r);
  if (!g->in_group) {
    int32_t fl;
    return end_group_impl(g, &fl);
  }
  return DVM_OK;
}

dvm_status dvm_graph_release(dvm_graph* g, dvm_value h) {
  FuseTimer ft(g);
  int64_t s;
  if (!g || !resolve(g, h, &s)) return fail(DVM_ERR_INVALID_ARG, "unknown value");
  Val& v = g->vals[s];
  v.released = true;
  maybe_recycle(g, s);
  return DVM_OK;
}

dvm_status dvm_flush(dvm_graph* g, dvm_program** out) {
  if (!g || !out) return fail(DVM_ERR_INVALID_ARG, "null argument");
  if (g->branch) return fail(DVM_ERR_INVALID_ARG, "branch still open");
  // what the stack holds runs first, so the returned program, launched on the
  // graph's stream, runs after it
  dvm_status sl = launch_stack(g, nullptr);
  if (sl != DVM_OK) return sl;
  if (!g->buf.empty()) {
    g->stats.flush_reason[FR_EXPLICIT]++;
    g->flush_log.push_back({(int32_t)g->buf.size(), (int32_t)FR_EXPLICIT, 0.f, 0});
  }
  return encode_buffer(g, out);
}

dvm_status dvm_launch(dvm_context* ctx, const dvm_program* p, void* stream) {
  if (!ctx || !p) return fail(DVM_ERR_INVALID_ARG, "null argument");
  return launch(ctx, p, (hipStream_t)stream);
}

dvm_status dvm_launch_noalloc(dvm_context* ctx, const dvm_program* p, void* stream) {
  if (!ctx || !p) return fail(DVM_ERR_INVALID_ARG, "null argument");
  if (ctx->device < 0) return fail(DVM_ERR_DEVICE, "encode-only context cannot launch");
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = settle(ctx, s);
  if (e != hipSuccess) return fail(DVM_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
  if (p->grid_launch == 0) return DVM_OK;
  if (needs_scratch(p)) {
    if (!ctx->static_scratch)
      return fail(DVM_ERR_DEVICE, "static scratch unavailable: %s", hipGetErrorString(ctx->static_err));
    // one partial per launched workgroup
    const uint64_t need = SCRATCH_PART_OFF + 4u * (uint64_t)p->grid_launch;
    if (need > ctx->static_bytes)
      return fail(DVM_ERR_RESOURCE, "reduce-all over %u workgroups: the static scratch holds %zu partials",
                  p->grid_launch, (ctx->static_bytes - SCRATCH_PART_OFF) / 4);
    Program q = p->prog;
    set_scratch(&q, ctx->static_scratch, ctx->static_bytes);
    e = launch_kernel(p, &q, s);
    if (e == hipSuccess) e = launch_combine(p, &q, s);
  } else {
    e = launch_kernel(p, &p->prog, s);
  }
  if (e != hipSuccess) return fail(DVM_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
  return DVM_OK;
}

dvm_status launch_twin(dvm_context* ctx, const dvm_program* p, void* stream, uint64_t* counters, size_t n_counters,
                       uint32_t flags_or);

dvm_status dvm_launch_profiled(dvm_context* ctx, const dvm_program* p, void* stream, uint64_t* counters,
                               size_t n_counters) {
  return launch_twin(ctx, p, stream, counters, n_counters, 0u);
}

dvm_status dvm_launch_stress(dvm_context* ctx, const dvm_program* p, void* stream, uint32_t seed, uint64_t* counters,
                             size_t n_counters) {
  return launch_twin(ctx, p, stream, counters, n_counters, HF_STRESS | ((seed & 0xffffffu) << 8));
}

dvm_status launch_twin(dvm_context* ctx, const dvm_program* p, void* stream, uint64_t* counters, size_t n_counters,
                       uint32_t flags_or) {
  if (!ctx || !p) return fail(DVM_ERR_INVALID_ARG, "null argument");
  if (ctx->device < 0) return fail(DVM_ERR_DEVICE, "encode-only context cannot launch");
  const uint32_t kt = p->prog.w[H_KTYPE];
  if (p->segments != 1 || (kt != KT_VECTOR && kt != KT_VECTOR_WIDE))
    return fail(DVM_ERR_UNSUPPORTED, "profiling covers single VECTOR programs");
  if (p->grid_launch == 0) return DVM_OK;
  if (!counters) return fail(DVM_ERR_INVALID_ARG, "null counter buffer");
  {
    const hipError_t e0 = settle(ctx, (hipStream_t)stream);
    if (e0 != hipSuccess) return fail(DVM_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e0));
  }
  const size_t need = (size_t)DVM_PROF_COUNTERS * p->grid_launch;
  if (n_counters < need) return fail(DVM_ERR_INVALID_ARG, "counter buffer holds %zu values, needs %zu", n_counters, need);
  Program q = p->prog;  // the launch copies its argument: a stack copy is enough
  if (needs_scratch(p)) {
    void* area;
    dvm_status st = stream_scratch(ctx, (hipStream_t)stream, &area);
    if (st != DVM_OK) return st;
    set_scratch(&q, area, SCRATCH_BYTES);
  }
  q.w[H_FLAGS] |= flags_or;
  const uint64_t a = (uint64_t)(uintptr_t)counters;
  q.w[H_PROF_LO] = (uint32_t)a;
  q.w[H_PROF_HI] = (uint32_t)(a >> 32);
  hipError_t e = kt == KT_VECTOR_WIDE ? dvm_launch_vector_prof_kernel_wide(&q, p->grid_launch, (hipStream_t)stream)
                                      : dvm_launch_vector_prof_kernel(&q, p->grid_launch, (hipStream_t)stream);
  if (e == hipSuccess && needs_scratch(p)) e = launch_combine(p, &q, (hipStream_t)stream);
  if (e != hipSuccess) return fail(DVM_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
  return DVM_OK;
}

dvm_status dvm_graph_begin_branch(dvm_graph* g, dvm_value cond, float threshold) {
  if (!g) return fail(DVM_ERR_INVALID_ARG, "null graph");
  FuseTimer ft(g);
  if (g->in_group || g->branch) return fail(DVM_ERR_INVALID_ARG, "a group or a branch is open");
  int64_t cs;
  if (!resolve(g, cond, &cs)) return fail(DVM_ERR_INVALID_ARG, "unknown condition value");
  {
    const Val& v = g->vals[cs];
    if (v.t.dtype != DVM_F32 || v.shape.numel() != 1)
      return fail(DVM_ERR_INVALID_ARG, "the condition is one fp32 value");
  }
  // a branch is a fusion boundary: the buffered graph (which may compute the
  // condition) runs first.  If its last launch is a reduce-all writing the
  // condition, that launch's combine is held back for the branch program.
  dvm_context* ctx = g->ctx;
  if (ctx->device >= 0) {
    std::lock_guard<std::mutex> lk(ctx->mu);
    ctx->hold = true;
    ctx->hold_stream = g->stream;
  }
  dvm_status st = flush_launch(g, FR_BRANCH, nullptr);
  if (ctx->device >= 0) {
    std::lock_guard<std::mutex> lk(ctx->mu);
    ctx->hold = false;
    ctx->hold_stream = nullptr;
  }
  const Val& v = g->vals[cs];
  const bool stored = !v.lost && !v.released && v.t.data;
  if (ctx->device >= 0) {
    // keep a held combine only for a condition it writes
    bool keep = false;
    if (st == DVM_OK && stored) {
      std::lock_guard<std::mutex> lk(ctx->mu);
      for (const HeldCombine& h : ctx->held)
        if (h.s == g->stream) keep = h.out == v.t.data;
    }
    if (!keep) {
      const hipError_t e = settle(ctx, g->stream);
      if (e != hipSuccess && st == DVM_OK) st = fail(DVM_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
    }
  }
  if (st != DVM_OK) return st;
  if (!stored) return fail(DVM_ERR_INVALID_ARG, "the condition has no stored value");
  g->vals[cs].uses++;
  g->branch = 1;
  g->branch_cond = cs;
  g->branch_thr = threshold;
  return DVM_OK;
}

dvm_status dvm_graph_begin_branch_reduce(dvm_graph* g, dvm_value x, int32_t op, const dvm_tensor* out,
                                         float threshold, dvm_value* cond) {
  if (!g || !out || !cond) return fail(DVM_ERR_INVALID_ARG, "null argument");
  if (op != DVM_OP_REDUCE_SUM && op != DVM_OP_REDUCE_MAX) return fail(DVM_ERR_INVALID_ARG, "op %d is no reduction", op);
  if (out->dtype != DVM_F32 || out->ndim != 0) return fail(DVM_ERR_INVALID_ARG, "the condition is one fp32 value");
  if (g->in_group || g->branch) return fail(DVM_ERR_INVALID_ARG, "a group or a branch is open");
  // what is buffered runs first; then the reduce-all, which closes its own
  // graph and launches at once, with its combine held back on the stream
  dvm_status st = flush_launch(g, FR_BRANCH, nullptr);
  if (st != DVM_OK) return st;
  dvm_context* ctx = g->ctx;
  if (ctx->device >= 0) {
    std::lock_guard<std::mutex> lk(ctx->mu);
    ctx->hold = true;
    ctx->hold_stream = g->stream;
  }
  dvm_attrs at{};
  at.axis = DVM_AXIS_ALL;
  at.scalar_pos = -1;
  st = dvm_graph_add_op(g, op, &x, 1, &at, out, DVM_OUT_LIVE, cond);
  if (st == DVM_OK) st = flush_launch(g, FR_REDUCE_ALL, nullptr);  // (nothing, if the op flushed itself)
  if (ctx->device >= 0) {
    std::lock_guard<std::mutex> lk(ctx->mu);
    ctx->hold = false;
    ctx->hold_stream = nullptr;
  }
  if (st == DVM_OK) st = dvm_graph_begin_branch(g, *cond, threshold);
  if (st != DVM_OK && ctx->device >= 0) (void)settle(ctx, g->stream);
  return st;
}

dvm_status dvm_graph_else_branch(dvm_graph* g) {
  if (!g) return fail(DVM_ERR_INVALID_ARG, "null graph");
  if (g->branch != 1) return fail(DVM_ERR_INVALID_ARG, "no then-branch open");
  g->branch = 2;
  return DVM_OK;
}

dvm_status dvm_graph_end_branch(dvm_graph* g, int32_t* launched) {
  if (launched) *launched = 0;
  if (!g) return fail(DVM_ERR_INVALID_ARG, "null graph");
  if (!g->branch) return fail(DVM_ERR_INVALID_ARG, "no branch open");
  FuseTimer ft(g);
  std::vector<OpRec> bt, be;
  bt.swap(g->br[0]);
  be.swap(g->br[1]);
  const int64_t cs = g->branch_cond;
  const float thr = g->branch_thr;
  g->branch = 0;
  g->branch_cond = -1;
  dvm_status st = DVM_OK;
  if (bt.empty() || be.empty()) st = fail(DVM_ERR_UNSUPPORTED, "both branch bodies must hold ops");
  for (const std::vector<OpRec>* list : {&bt, &be}) {
    if (st != DVM_OK) break;
    LocalView L;
    make_local(g, *list, &L);
    Checker ck(&L.lg, L.ops);
    if (ck.check(0) >= 0) st = fail(DVM_ERR_UNSUPPORTED, "a branch body is not one fusible graph");
  }
  g->stats.flush_reason[FR_BRANCH]++;
  g->flush_log.push_back({(int32_t)(bt.size() + be.size()), (int32_t)FR_BRANCH, 0.f, 0});
  const auto t0 = std::chrono::steady_clock::now();
  dvm_program *pt = nullptr, *pe = nullptr, *pb = nullptr;
  if (st == DVM_OK) st = encode_list(g, bt, false, &pt);
  if (st == DVM_OK) st = encode_list(g, be, false, &pe);
  if (st == DVM_OK && (!pt || !pe)) st = fail(DVM_ERR_UNSUPPORTED, "both branch bodies must store a result");
  // The combine of the reduce-all that wrote the condition, if it was held
  // back, is folded into the branch program when the branch program is the
  // next launch on the stream (nothing stacked before it) and its bodies do
  // not read the condition (workgroup 0 writes it while other workgroups run).
  HeldCombine fold;
  bool folding = false;
  if (st == DVM_OK && g->ctx->device >= 0 && g->stack.empty()) {
    const uintptr_t cp = (uintptr_t)g->vals[cs].t.data;
    bool reads_cond = false;
    for (const dvm_program* b : {pt, pe})
      for (const Range& r : b->reads) reads_cond = reads_cond || (r.first < cp + 4 && cp < r.first + r.second);
    if (!reads_cond) folding = take_held(g->ctx, g->stream, g->vals[cs].t.data, &fold);
  }
  if (st == DVM_OK) st = merge_branch(pt, pe, g->vals[cs].t, thr, folding ? &fold : nullptr, &pb);
  if (folding && st != DVM_OK) (void)launch_held(fold);
  delete pt;
  delete pe;
  retire(g, bt, st == DVM_OK);
  retire(g, be, st == DVM_OK);
  g->vals[cs].uses--;
  maybe_recycle(g, cs);
  note_encode(g, t0, pb);
  if (st != DVM_OK) return st;
  return submit(g, pb, launched);  // after whatever the stack holds
}

dvm_status dvm_graph_flush_launch(dvm_graph* g, int32_t* launched) {
  if (!g) return fail(DVM_ERR_INVALID_ARG, "null graph");
  if (g->in_group) return fail(DVM_ERR_INVALID_ARG, "group still open");
  if (g->branch) return fail(DVM_ERR_INVALID_ARG, "branch still open");
  if (launched) *launched = 0;
  int32_t l1 = 0, l2 = 0;
  dvm_status st = flush_launch(g, FR_EXPLICIT, &l1);
  if (st == DVM_OK) st = launch_stack(g, &l2);
  if (launched) *launched = l1 | l2;
  return st;
}

dvm_status dvm_graph_set_stacking(dvm_graph* g, int32_t max_segments) {
  if (!g) return fail(DVM_ERR_INVALID_ARG, "null graph");
  if (max_segments < 1 || max_segments > MAX_SEGS)
    return fail(DVM_ERR_INVALID_ARG, "max_segments %d outside 1..%d", max_segments, MAX_SEGS);
  dvm_status st = launch_stack(g, nullptr);
  g->stack_max = max_segments;
  return st;
}

dvm_status dvm_graph_set_stack_order(dvm_graph* g, int32_t temporal) {
  if (!g) return fail(DVM_ERR_INVALID_ARG, "null graph");
  if (temporal != 0 && temporal != 1) return fail(DVM_ERR_INVALID_ARG, "stack order %d is neither 0 nor 1", temporal);
  dvm_status st = launch_stack(g, nullptr);
  g->stack_temporal = temporal != 0;
  return st;
}

dvm_status dvm_program_stack(const dvm_program* const* programs, size_t n, dvm_program** out) {
  if (!programs || !out) return fail(DVM_ERR_INVALID_ARG, "null argument");
  return build_stack(programs, n, false, out);
}

dvm_status dvm_program_stack_temporal(const dvm_program* const* programs, size_t n, dvm_program** out) {
  if (!programs || !out) return fail(DVM_ERR_INVALID_ARG, "null argument");
  return build_stack(programs, n, true, out);
}

dvm_status dvm_sync(dvm_graph* g) {
  if (!g) return fail(DVM_ERR_INVALID_ARG, "null graph");
  if (g->in_group) return fail(DVM_ERR_INVALID_ARG, "group still open");
  if (g->branch) return fail(DVM_ERR_INVALID_ARG, "branch still open");
  dvm_status st = flush_launch(g, FR_SYNC, nullptr);
  if (st == DVM_OK) st = launch_stack(g, nullptr);
  if (st != DVM_OK) return st;
  if (g->ctx->device >= 0) {
    hipError_t e = settle(g->ctx, g->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(g->stream);
    if (e != hipSuccess) return fail(DVM_ERR_DEVICE, "stream sync: %s", hipGetErrorString(e));
  }
  return DVM_OK;
}

dvm_status dvm_program_header(const dvm_program* p, dvm_header* out) {
  if (!p || !out) return fail(DVM_ERR_INVALID_ARG, "null argument");
  // a stacked program reports its first segment's header
  const uint32_t* W = p->segments > 1 ? p->prog.w + p->prog.w[S_DIR] : p->prog.w;
  out->kernel_type = W[H_KTYPE];
  out->tmpl = W[H_TEMPLATE];
  out->block_dim = W[H_BLOCK_DIM];
  out->body_tile = W[H_BODY_TILE];
  out->grid = W[H_GRID];
  out->tr = W[H_TR];
  out->tc = W[H_TC];
  out->g = W[H_G];
  out->nv = W[H_NV];
  out->p = W[H_P];
  out->R = p->R;
  out->C = p->C;
  out->n_instr = p->n_instr;
  out->n_args = W[H_NARGS];
  out->pad = p->pad;
  out->n_words = p->n_words;
  out->bytes = p->bytes;
  out->segments = p->segments;
  if (p->segments > 1) out->grid = p->grid_launch;
  return DVM_OK;
}

dvm_status dvm_program_words(const dvm_program* p, uint32_t* buf, size_t* n_words) {
  if (!p || !n_words) return fail(DVM_ERR_INVALID_ARG, "null argument");
  const size_t cap = *n_words;
  *n_words = p->n_words;
  if (buf) std::memcpy(buf, p->prog.w, sizeof(uint32_t) * std::min<size_t>(cap, p->n_words));
  return DVM_OK;
}

void dvm_program_free(dvm_program* p) { delete p; }

dvm_status dvm_program_verify(const dvm_program* p, char* msg, size_t len) {
  if (!p) return fail(DVM_ERR_INVALID_ARG, "null program");
  std::string e;
  const bool ok = verify_words(p->prog.w, p->n_words, &e);
  if (msg && len) {
    std::snprintf(msg, len, "%s", ok ? "" : e.c_str());
  }
  if (!ok) return fail(DVM_ERR_INTERNAL, "bytecode verifier: %s", e.c_str());
  return DVM_OK;
}

dvm_status dvm_program_from_words(const uint32_t* words, size_t n_words, dvm_program** out) {
  if (!words || !out) return fail(DVM_ERR_INVALID_ARG, "null argument");
  *out = nullptr;
  if (n_words < (size_t)HDR_WORDS || n_words > (size_t)MAX_WORDS) return fail(DVM_ERR_INVALID_ARG, "%zu words", n_words);
  dvm_program* q = new (std::nothrow) dvm_program();
  if (!q) return fail(DVM_ERR_INTERNAL, "out of host memory");
  std::copy(words, words + n_words, q->prog.w);
  q->n_words = (uint32_t)n_words;
  *out = q;
  return DVM_OK;
}

dvm_status dvm_program_debug_tilemap(const dvm_program* p, const dvm_tensor* tile_out, const dvm_tensor* wg_out,
                                     dvm_program** out) {
  if (!p || !tile_out || !wg_out || !out) return fail(DVM_ERR_INVALID_ARG, "null argument");
  const uint32_t kt = p->prog.w[H_KTYPE];
  if (p->segments != 1) return fail(DVM_ERR_UNSUPPORTED, "tile maps of single programs only");
  if (kt != KT_VECTOR && kt != KT_VECTOR_WIDE && kt != KT_MIX) return fail(DVM_ERR_UNSUPPORTED, "unknown kernel type");
  for (const dvm_tensor* t : {tile_out, wg_out}) {
    if (t->dtype != DVM_F32 || t->ndim != 2 || t->shape[0] != p->R || t->shape[1] != p->C || t->stride[1] != 1 ||
        t->stride[0] != p->C || (!t->data && p->R * p->C > 0))
      return fail(DVM_ERR_SHAPE, "tilemap outputs must be dense fp32 [R, C]");
  }
  dvm_program* q = new (std::nothrow) dvm_program(*p);
  if (!q) return fail(DVM_ERR_INTERNAL, "out of host memory");
  uint32_t* W = q->prog.w;
  // MIX programs keep A and B (args 0 and 1: the K loop still runs, its
  // result unused) and write the maps from the epilogue
  const bool mix = kt == KT_MIX;
  const uint32_t a0 = mix ? 2u : 0u;
  const uint32_t n_args = a0 + 2;
  W[H_NARGS] = n_args;
  if (!mix) {
    W[H_TEMPLATE] = TM_ELEMWISE;  // same tiling; no reduce-all epilogue
    W[H_LDS_BYTES] = 0;
  }
  uint32_t k = a0;
  for (const dvm_tensor* t : {tile_out, wg_out}) {
    uint32_t* a = W + ARG_BASE + k * ARG_WORDS;
    const uint64_t ptr = (uint64_t)(uintptr_t)t->data;
    a[A_PTR_LO] = (uint32_t)ptr;
    a[A_PTR_HI] = (uint32_t)(ptr >> 32);
    a[A_DTYPE] = DT_F32;
    a[A_FLAGS] = arg_flags_word(mix && ptr % 16 == 0 && p->C % 4 == 0 ? AF_VEC : 0u, (uint64_t)extent_bytes(*t));
    const int64_t sr = p->R > 1 || mix ? p->C : 0;
    a[A_SR_LO] = (uint32_t)(uint64_t)sr;
    a[A_SR_HI] = (uint32_t)((uint64_t)sr >> 32);
    a[A_SC] = 1;
    a[A_EXTENT] = (uint32_t)(uint64_t)extent_bytes(*t);
    ++k;
  }
  const uint32_t base = ARG_BASE + n_args * ARG_WORDS;
  // vector programs take handler ids, MIX epilogues the generic opcodes
  const uint32_t dbg = mix ? (uint32_t)OP_DBG : (uint32_t)HD_DBG;
  const uint32_t st = mix ? (uint32_t)OP_STORE : (uint32_t)HD_ST_F32;
  const uint32_t code[] = {enc0(dbg, 0, 0, 0, 0, 0, 0), a0, enc0(st, 0, 0, 0, 0, 0, 0), a0,
                           enc0(dbg, 0, 0, 0, 1, 0, 0), 0, enc0(st, 0, 0, 0, 0, 0, 0), a0 + 1};
  std::memcpy(W + base, code, sizeof code);
  W[H_PRO_BEGIN] = W[H_PRO_END] = W[H_BODY_BEGIN] = base;
  W[H_BODY_END] = base + 8;
  W[H_N_INSTR] = 4;
  q->n_words = base + 8;
  q->n_instr = 4;
  q->grid_launch = W[H_GRID];
  *out = q;
  return DVM_OK;
}

dvm_status dvm_graph_flush_log(const dvm_graph* g, int32_t* n_ops, int32_t* reasons, float* encode_us,
                               uint64_t* bytes, size_t* n) {
  if (!g || !n) return fail(DVM_ERR_INVALID_ARG, "null argument");
  const size_t cap = *n;
  *n = g->flush_log.size();
  for (size_t i = 0; i < std::min(cap, g->flush_log.size()); ++i) {
    const dvm_graph::LogEntry& e = g->flush_log[i];
    if (n_ops) n_ops[i] = e.ops;
    if (reasons) reasons[i] = e.reason;
    if (encode_us) encode_us[i] = e.encode_us;
    if (bytes) bytes[i] = e.bytes;
  }
  return DVM_OK;
}

// ---------------------------------------------------------------------------
// Templates (static-graph symbolic fusion)
// ---------------------------------------------------------------------------
dvm_status dvm_template_create(dvm_context* ctx, void* stream, dvm_template** out) {
  if (!ctx || !out) return fail(DVM_ERR_INVALID_ARG, "null argument");
  dvm_template* t = new (std::nothrow) dvm_template();
  if (!t) return fail(DVM_ERR_INTERNAL, "out of host memory");
  t->ctx = ctx;
  dvm_status st = dvm_graph_create(ctx, stream, &t->rg);
  if (st != DVM_OK) {
    delete t;
    return st;
  }
  *out = t;
  return DVM_OK;
}

void dvm_template_destroy(dvm_template* t) {
  if (!t) return;
  dvm_graph_destroy(t->rg);
  delete t;
}

dvm_status dvm_template_graph(dvm_template* t, dvm_graph** out) {
  if (!t || !out) return fail(DVM_ERR_INVALID_ARG, "null argument");
  *out = t->rg;
  return DVM_OK;
}

dvm_status dvm_template_input(dvm_template* t, int32_t dtype, int32_t ndim, const int64_t* dims, dvm_value* out) {
  if (!t || !out || (ndim > 0 && !dims)) return fail(DVM_ERR_INVALID_ARG, "null argument");
  if (t->finalized) return fail(DVM_ERR_INVALID_ARG, "template already finalized");
  if (ndim < 0 || ndim > 4 || dtype < 0 || dtype > DVM_U8) return fail(DVM_ERR_INVALID_ARG, "bad dtype or ndim");
  TmplVal v;
  v.dtype = dtype;
  v.nd = ndim;
  for (int i = 0; i < ndim; ++i) v.dim[i] = dims[i];
  v.io = (int)t->inputs.size();
  t->inputs.push_back((int64_t)t->vals.size());
  *out = (dvm_value)t->vals.size();
  t->vals.push_back(v);
  return DVM_OK;
}

dvm_status dvm_template_begin_group(dvm_template* t) {
  if (!t || t->in_group || t->finalized) return fail(DVM_ERR_INVALID_ARG, "bad template state");
  t->in_group = true;
  return DVM_OK;
}

dvm_status dvm_template_end_group(dvm_template* t) {
  if (!t || !t->in_group) return fail(DVM_ERR_INVALID_ARG, "no open group");
  t->in_group = false;
  ++t->n_groups;
  return DVM_OK;
}

dvm_status dvm_template_add_op(dvm_template* t, int32_t op, const dvm_value* in, int32_t n_in, const dvm_attrs* attrs,
                               int32_t out_dtype, uint32_t flags, dvm_value* out) {
  if (!t || !out || (n_in > 0 && !in)) return fail(DVM_ERR_INVALID_ARG, "null argument");
  if (t->finalized) return fail(DVM_ERR_INVALID_ARG, "template already finalized");
  if (op < 0 || op >= DVM_OP_COUNT || n_in < 1 || n_in > 2) return fail(DVM_ERR_INVALID_ARG, "bad op");
  if (out_dtype < 0 || out_dtype > DVM_U8) return fail(DVM_ERR_INVALID_ARG, "bad dtype");
  TmplOp o;
  o.op = op;
  o.n_in = n_in;
  if (attrs) o.at = *attrs;
  for (int k = 0; k < n_in; ++k) {
    if (in[k] < 0 || in[k] >= (int64_t)t->vals.size()) return fail(DVM_ERR_INVALID_ARG, "unknown value");
    o.in[k] = in[k];
  }
  // symbolic shape inference: numpy broadcasting where equal symbols match
  // and a symbol meets only itself or a 1
  TmplVal v;
  v.dtype = out_dtype;
  const TmplVal& a = t->vals[(size_t)o.in[0]];
  if (op == DVM_OP_MATMUL) {
    const TmplVal& b = t->vals[(size_t)o.in[1]];
    if (n_in != 2 || a.nd != 2 || b.nd != 2 || a.dim[1] != b.dim[0]) return fail(DVM_ERR_SHAPE, "matmul shapes");
    v.nd = 2;
    v.dim[0] = a.dim[0];
    v.dim[1] = b.dim[1];
  } else if (is_reduce(op)) {
    if (o.at.axis == DVM_AXIS_ALL) {
      v.nd = 0;
    } else {
      if (a.nd == 0) return fail(DVM_ERR_SHAPE, "row reduce of a scalar");
      v = a;
      v.dim[v.nd - 1] = 1;
      v.dtype = out_dtype;
    }
  } else if (is_binary(op) && n_in == 2) {
    const TmplVal& b = t->vals[(size_t)o.in[1]];
    v.nd = std::max(a.nd, b.nd);
    for (int i = 0; i < v.nd; ++i) {
      const int ia = a.nd - v.nd + i, ib = b.nd - v.nd + i;
      const int64_t da = ia >= 0 ? a.dim[ia] : 1, db = ib >= 0 ? b.dim[ib] : 1;
      if (da != db && da != 1 && db != 1) return fail(DVM_ERR_SHAPE, "shapes do not broadcast");
      v.dim[i] = da == 1 ? db : da;
    }
  } else {
    v.nd = a.nd;
    for (int i = 0; i < a.nd; ++i) v.dim[i] = a.dim[i];
  }
  v.op = (int)t->ops.size();
  if (flags & DVM_OUT_LIVE) {
    v.io = (int)t->outputs.size();
    t->outputs.push_back((int64_t)t->vals.size());
  }
  o.out = (int64_t)t->vals.size();
  o.group = t->in_group ? t->n_groups : t->n_groups++;
  t->ops.push_back(o);
  *out = (dvm_value)t->vals.size();
  t->vals.push_back(v);
  return DVM_OK;
}

dvm_status dvm_template_finalize(dvm_template* t, int32_t* n_graphs) {
  if (!t) return fail(DVM_ERR_INVALID_ARG, "null template");
  if (t->in_group) return fail(DVM_ERR_INVALID_ARG, "group still open");
  if (t->finalized) return fail(DVM_ERR_INVALID_ARG, "template already finalized");
  const auto t0 = std::chrono::steady_clock::now();
  const std::vector<int64_t> rep = representatives(t);
  // replay the groups through the streaming fuser of an encode-only graph on
  // stand-in tensors; its flush log is the partition
  dvm_context* ec = nullptr;
  dvm_status st = dvm_context_create(-1, &ec);
  if (st != DVM_OK) return st;
  dvm_graph* fg = nullptr;
  st = dvm_graph_create(ec, nullptr, &fg);
  std::vector<dvm_value> h(t->vals.size(), -1);
  std::vector<int> last_group(t->vals.size(), -1);
  for (const TmplOp& o : t->ops)
    for (int k = 0; k < o.n_in; ++k) last_group[(size_t)o.in[k]] = o.group;
  for (size_t i = 0; st == DVM_OK && i < t->vals.size(); ++i)
    if (t->vals[i].op < 0) {
      const dvm_tensor x = stand_in(t->vals[i], (int64_t)i, rep, t);
      st = dvm_graph_input(fg, &x, &h[i]);
    }
  for (size_t i = 0; st == DVM_OK && i < t->ops.size();) {
    const int grp = t->ops[i].group;
    st = dvm_graph_begin_group(fg);
    for (; st == DVM_OK && i < t->ops.size() && t->ops[i].group == grp; ++i) {
      const TmplOp& o = t->ops[i];
      const dvm_tensor x = stand_in(t->vals[(size_t)o.out], o.out, rep, t);
      dvm_value in[2] = {h[(size_t)o.in[0]], o.n_in > 1 ? h[(size_t)o.in[1]] : 0};
      st = dvm_graph_add_op(fg, o.op, in, o.n_in, &o.at, &x, t->vals[(size_t)o.out].io >= 0 ? DVM_OUT_LIVE : 0u,
                            &h[(size_t)o.out]);
    }
    if (st != DVM_OK) break;
    int32_t fl = 0;
    st = dvm_graph_end_group(fg, &fl);
    // internal values are released after the group that reads them last
    for (size_t v = 0; st == DVM_OK && v < t->vals.size(); ++v)
      if (t->vals[v].op >= 0 && t->vals[v].io < 0 && h[v] >= 0 &&
          (last_group[v] == grp || (last_group[v] < 0 && t->ops[(size_t)t->vals[v].op].group == grp)))
        st = dvm_graph_release(fg, h[v]);
  }
  if (st == DVM_OK) st = dvm_graph_flush_launch(fg, nullptr);
  if (st == DVM_OK) {
    // the partition: graphs are runs of whole groups, in order
    t->graph_of_op.assign(t->ops.size(), -1);
    size_t i = 0;
    int32_t gi = 0;
    for (const dvm_graph::LogEntry& e : fg->flush_log) {
      for (int32_t k = 0; k < e.ops && i < t->ops.size(); ++k) t->graph_of_op[i++] = gi;
      ++gi;
    }
    if (i != t->ops.size()) st = fail(DVM_ERR_INTERNAL, "partition covers %zu of %zu ops", i, t->ops.size());
    t->n_graphs = gi;
    // a value read by a later graph than the one computing it needs storage
    for (size_t k = 0; st == DVM_OK && k < t->ops.size(); ++k)
      for (int q = 0; q < t->ops[k].n_in; ++q) {
        const TmplVal& v = t->vals[(size_t)t->ops[k].in[q]];
        if (v.op >= 0 && v.io < 0 && t->graph_of_op[(size_t)v.op] != t->graph_of_op[k])
          st = fail(DVM_ERR_RESOURCE, "value %lld crosses fused graphs: make it a template output",
                    (long long)t->ops[k].in[q]);
      }
  }
  dvm_graph_destroy(fg);
  dvm_context_destroy(ec);
  if (st != DVM_OK) return st;
  t->finalized = true;
  t->finalize_us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
  if (n_graphs) *n_graphs = t->n_graphs;
  return DVM_OK;
}

dvm_status dvm_template_partition(const dvm_template* t, int32_t* graph_of_op, size_t* n_ops, double* finalize_us) {
  if (!t || !n_ops) return fail(DVM_ERR_INVALID_ARG, "null argument");
  if (!t->finalized) return fail(DVM_ERR_INVALID_ARG, "template not finalized");
  const size_t cap = *n_ops;
  *n_ops = t->ops.size();
  if (graph_of_op) std::copy(t->graph_of_op.begin(), t->graph_of_op.begin() + std::min(cap, t->ops.size()), graph_of_op);
  if (finalize_us) *finalize_us = t->finalize_us;
  return DVM_OK;
}

dvm_status dvm_template_run(dvm_template* t, const dvm_tensor* inputs, int32_t n_inputs, const dvm_tensor* outputs,
                            int32_t n_outputs, int32_t* launched) {
  if (launched) *launched = 0;
  if (!t || (n_inputs && !inputs) || (n_outputs && !outputs)) return fail(DVM_ERR_INVALID_ARG, "null argument");
  if (!t->finalized) return fail(DVM_ERR_INVALID_ARG, "template not finalized");
  if (n_inputs != (int32_t)t->inputs.size() || n_outputs != (int32_t)t->outputs.size())
    return fail(DVM_ERR_INVALID_ARG, "template takes %zu inputs and %zu outputs", t->inputs.size(), t->outputs.size());
  dvm_graph* g = t->rg;
  if (g->in_group || g->branch || !g->buf.empty()) return fail(DVM_ERR_INVALID_ARG, "the run graph is busy");
  FuseTimer ft(g);
  // bind the symbols and check every bound tensor against its symbolic shape
  std::vector<int64_t> sym;
  auto bind = [&](const TmplVal& v, const dvm_tensor& x) -> dvm_status {
    dvm_status c = check_tensor(&x);
    if (c != DVM_OK) return c;
    if (x.dtype != v.dtype || x.ndim != v.nd) return fail(DVM_ERR_SHAPE, "bound tensor: dtype or rank");
    for (int i = 0; i < v.nd; ++i) {
      const int64_t d = v.dim[i];
      if (d >= 0) {
        if (x.shape[i] != d) return fail(DVM_ERR_SHAPE, "bound tensor: dim %d is %lld, not %lld", i, (long long)x.shape[i], (long long)d);
        continue;
      }
      const size_t k = (size_t)(-d - 1);
      if (sym.size() <= k) sym.resize(k + 1, -1);
      if (sym[k] < 0) sym[k] = x.shape[i];
      else if (sym[k] != x.shape[i]) return fail(DVM_ERR_SHAPE, "symbol %zu bound to %lld and %lld", k, (long long)sym[k], (long long)x.shape[i]);
    }
    return DVM_OK;
  };
  for (int32_t i = 0; i < n_inputs; ++i) {
    dvm_status c = bind(t->vals[(size_t)t->inputs[(size_t)i]], inputs[i]);
    if (c != DVM_OK) return c;
  }
  for (int32_t i = 0; i < n_outputs; ++i) {
    dvm_status c = bind(t->vals[(size_t)t->outputs[(size_t)i]], outputs[i]);
    if (c != DVM_OK) return c;
    if (!outputs[i].data && numel_of(outputs[i]) > 0) return fail(DVM_ERR_INVALID_ARG, "output %d has no storage", i);
  }
  // the partition assumed no aliasing: no output overlaps an input or another output
  auto rng = [](const dvm_tensor& x) { return Range{(uintptr_t)x.data, (uint64_t)extent_bytes(x)}; };
  for (int32_t i = 0; i < n_outputs; ++i) {
    std::vector<Range> o{rng(outputs[i])}, others;
    for (int32_t j = 0; j < n_inputs; ++j) others.push_back(rng(inputs[j]));
    for (int32_t j = 0; j < n_outputs; ++j)
      if (j != i) others.push_back(rng(outputs[j]));
    if (overlaps(o, others)) return fail(DVM_ERR_INVALID_ARG, "output %d aliases another bound tensor", i);
  }
  // values of this run in the run graph
  std::vector<int64_t> slot(t->vals.size(), -1);
  for (size_t i = 0; i < t->vals.size(); ++i) {
    const TmplVal& tv = t->vals[i];
    const int64_t s = new_slot(g);
    slot[i] = s;
    Val& v = g->vals[(size_t)s];
    if (tv.op < 0) {
      v.kind = VK_INPUT;
      v.t = inputs[tv.io];
      v.stored = true;
    } else {
      v.kind = VK_OP;
      const TmplOp& o = t->ops[(size_t)tv.op];
      int64_t ins[2] = {slot[(size_t)o.in[0]], o.n_in > 1 ? slot[(size_t)o.in[1]] : -1};
      Shape sh;
      if (!infer(g, o.op, ins, o.n_in, &o.at, &sh)) return fail(DVM_ERR_SHAPE, "op %d: shapes", tv.op);
      if (tv.io >= 0) {
        v.t = outputs[tv.io];
        v.live = true;
      } else {
        v.t = dvm_tensor{};
        v.t.dtype = tv.dtype;
        v.t.ndim = sh.nd;
        for (int d = 0; d < sh.nd; ++d) v.t.shape[d] = sh.d[d];
        v.released = true;  // internal: never stored (it stays inside its graph)
      }
    }
    g->vals[(size_t)s].shape = shape_of(g->vals[(size_t)s].t);
  }
  // the precomputed graphs, in order: tiling and encoding only
  dvm_status st = DVM_OK;
  int32_t any = 0;
  for (int32_t gi = 0; st == DVM_OK && gi < t->n_graphs; ++gi) {
    for (size_t k = 0; k < t->ops.size(); ++k) {
      if (t->graph_of_op[k] != gi) continue;
      const TmplOp& o = t->ops[k];
      OpRec r;
      r.op = o.op;
      r.n_in = o.n_in;
      for (int q = 0; q < o.n_in; ++q) {
        r.in[q] = slot[(size_t)o.in[q]];
        g->vals[(size_t)r.in[q]].uses++;
      }
      r.axis = o.at.axis;
      r.scalar_pos = o.at.scalar_pos;
      r.scalar = o.at.scalar;
      r.out = slot[(size_t)o.out];
      g->vals[(size_t)r.out].pending = true;
      g->buf.push_back(r);
      g->stats.ops++;
    }
    int32_t l = 0;
    st = flush_launch(g, FR_EXPLICIT, &l);
    any |= l;
  }
  if (st == DVM_OK) {
    int32_t l = 0;
    st = launch_stack(g, &l);
    any |= l;
  } else {
    std::vector<OpRec> left;
    left.swap(g->buf);
    retire(g, left, false);
  }
  for (int64_t s : slot) {
    Val& v = g->vals[(size_t)s];
    v.released = true;
    v.pending = false;
    maybe_recycle(g, s);
  }
  if (launched) *launched = any;
  return st;
}

dvm_status dvm_graph_stats(const dvm_graph* g, dvm_stats* out) {
  if (!g || !out) return fail(DVM_ERR_INVALID_ARG, "null argument");
  *out = g->stats;
  return DVM_OK;
}

}  // extern "C"
