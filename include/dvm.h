/*
 * dvm.h -- C ABI of the MI355X DVM hot path: a streaming fuser, a tile-level
 * bytecode encoder and a resident bytecode-interpreting VM kernel.
 *
 * The flow follows the DVM pages: ops are captured in order into a fusion
 * buffer and fused while the fusion conditions hold; the buffer is flushed when
 * an op cannot join, at a fusion boundary or at a synchronisation point
 * (MindSpore DVM summary page, sections 3.2-3.3; DVM paper review page,
 * section 5.2); a flushed graph is shape-tiled and encoded into a tile-level
 * bytecode program on the host (review page, sections 4.2-4.3) and run by a
 * resident VM kernel that interprets it tile by tile (review page, section
 * 4.4).  No machine code is generated at run time: a new shape only needs a new
 * program.
 *
 * Conventions
 * - All functions return a dvm_status; on failure dvm_last_error() returns a
 *   thread-local message.  No C++ exception crosses this boundary.
 * - Device memory is always the caller's.  Pointers inside dvm_tensor are
 *   borrowed: they must stay valid until the launch that reads or writes them
 *   has completed on the stream it was issued on.
 * - Contexts, graphs and programs are library-owned opaque handles.  A graph
 *   is not thread-safe; separate graphs may be used from separate threads.
 * - Strides are in elements; shapes have at most 4 dims.
 */
#ifndef DVM_H
#define DVM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DVM_OK = 0,
  DVM_ERR_INVALID_ARG = 1,  /* malformed call, unknown value, missing storage */
  DVM_ERR_UNSUPPORTED = 2,  /* the op (group) cannot run on the VM; run it elsewhere */
  DVM_ERR_SHAPE = 3,        /* shapes do not broadcast / do not match */
  DVM_ERR_RESOURCE = 4,     /* no feasible tiling / program too large */
  DVM_ERR_DEVICE = 5,       /* HIP error (launch, sync, allocation) or no device */
  DVM_ERR_INTERNAL = 6
} dvm_status;

typedef enum { DVM_F32 = 0, DVM_BF16 = 1, DVM_U8 = 2 } dvm_dtype;

/* Primitive ops.  Elementwise ops broadcast their inputs numpy-style; every op
 * computes in fp32 on the device and rounds its result to the output dtype
 * (bf16: round to nearest even).  Table 1 of the DVM review page lists
 * Sqrt/Abs/Log/Exp/Pow/Round/Floor/IsFinite and Copy/Broadcast; the binary
 * ops, reductions, cast and matmul are the ones its fusion patterns use
 * (section 5.1: c = a + b then sqrt; cube-vector fusion). */
typedef enum {
  DVM_OP_ADD = 0, DVM_OP_SUB, DVM_OP_MUL, DVM_OP_DIV, DVM_OP_MAX, DVM_OP_MIN, DVM_OP_POW,
  DVM_OP_SQRT, DVM_OP_ABS, DVM_OP_LOG, DVM_OP_EXP, DVM_OP_ROUND, DVM_OP_FLOOR,
  DVM_OP_ISFINITE,   /* output dtype u8 (0/1) */
  DVM_OP_NEG, DVM_OP_RECIP,
  DVM_OP_CAST,       /* to the output dtype */
  DVM_OP_COPY,
  DVM_OP_REDUCE_SUM, /* attrs.axis: -1 = innermost axis (keepdim), DVM_AXIS_ALL = all axes */
  DVM_OP_REDUCE_MAX,
  DVM_OP_MATMUL,     /* [M, K] x [K, N] -> [M, N], fp32 accumulate */
  DVM_OP_COUNT
} dvm_op;

#define DVM_AXIS_ALL 0x7fffffff

typedef struct {
  void* data;        /* device pointer; may be NULL for an output that never needs storage */
  int32_t dtype;     /* dvm_dtype */
  int32_t ndim;      /* 0..4 */
  int64_t shape[4];
  int64_t stride[4]; /* elements */
} dvm_tensor;

typedef int64_t dvm_value;   /* graph-scoped value handle */

typedef struct {
  int32_t axis;        /* reductions: -1 or DVM_AXIS_ALL */
  int32_t scalar_pos;  /* binary ops with a scalar operand: -1 none, 0 scalar is the left input, 1 the right */
  float scalar;
} dvm_attrs;

/* add_op flags */
#define DVM_OUT_LIVE 1u   /* store the output when its graph is flushed, even if released */

typedef struct dvm_context dvm_context;
typedef struct dvm_graph dvm_graph;
typedef struct dvm_program dvm_program;

/* Code header of an encoded program (DVM review page, section 4.3: tile
 * count block_dim, tiles per core body_tile, kernel type) plus the tiling. */
typedef struct {
  uint32_t kernel_type;  /* 0 VECTOR, 1 MIX (matmul), 2 VECTOR wide (one tile register of 10 chunks) */
  uint32_t tmpl;         /* 0 elementwise, 1 row reduce, 2 reduce-all, 3 matmul */
  uint32_t block_dim;    /* number of tiles */
  uint32_t body_tile;    /* tiles per workgroup */
  uint32_t grid;         /* workgroups launched */
  uint32_t tr, tc;       /* tile rows / columns in the collapsed [R, C] space */
  uint32_t g, nv, p;     /* lanes per tile row, chunks per lane, row groups */
  int64_t R, C;          /* collapsed iteration space */
  uint32_t n_instr;      /* instructions (prologue + body) */
  uint32_t n_args;       /* global operands */
  uint32_t pad;          /* alignment slack used by the tiling */
  uint32_t n_words;      /* program size in 32-bit words */
  uint64_t bytes;        /* physical bytes of the graph: each operand tensor read once and each
                            stored output written once (the least HBM traffic of a launch) */
  uint32_t segments;     /* 1, or the programs a stacked program holds (the fields above are
                            its first segment's, except grid and bytes: the whole launch's) */
} dvm_header;

typedef struct {
  uint64_t graphs;            /* programs encoded */
  uint64_t launches;          /* programs launched */
  uint64_t ops;               /* ops accepted */
  uint64_t groups;
  uint64_t unsupported;       /* groups rejected (caller ran them elsewhere) */
  uint64_t flush_reason[8];   /* 0 explicit, 1 sync, 2 reduce_all, 3 shape, 4 pattern, 5 dependence, 6 resource,
                                 7 branch (a begin_branch flush or an encoded branch program) */
  double encode_us_total;     /* host time of encoding (tiling + bytecode), all graphs */
  double encode_us_max;
  uint64_t bytes;             /* physical bytes of the encoded graphs (dvm_header.bytes summed) */
  double fuse_us_total;       /* host time of capture and fusion decisions (input, add_op, end_group,
                                 release), without the encodes and launches they trigger */
  double launch_us_total;     /* host time of the launches of implicit and explicit flushes */
  uint64_t stacked;           /* programs launched as segments of stacked launches */
} dvm_stats;

/* Contexts (the VM's code is loaded once and stays resident: MindSpore DVM
 * summary page, section 3.2).  device >= 0: the HIP device whose resident VM
 * kernels run the programs.  Reduce-all programs need a scratch area on the device (one
 * partial per workgroup): each stream gets its own 4 MiB area, allocated and
 * zeroed at the first reduce-all launched on it and freed with the context,
 * so launches on different streams never share it.
 * device < 0: an encode-only context (tiling and bytecode, no launches). */
dvm_status dvm_context_create(int device, dvm_context** out);
void dvm_context_destroy(dvm_context* ctx);

/* A graph is a streaming fusion buffer (the dynamic-graph streaming fusion of
 * the DVM review page, section 5.2; ops are captured in execution order,
 * MindSpore summary page, section 3.2) bound to a HIP stream (hipStream_t,
 * NULL = default stream); implicit flushes launch on that stream.  Errors:
 * DVM_ERR_INVALID_ARG for a null context or out. */
dvm_status dvm_graph_create(dvm_context* ctx, void* stream, dvm_graph** out);
void dvm_graph_destroy(dvm_graph* g);

/* A graph of an encode-only context cannot launch what it flushes implicitly
 * (flushes at fusion boundaries and sync points: MindSpore summary page,
 * section 3.2)
 * -- at a fusion boundary, or when a reduce-all closes its graph: those
 * programs wait in the graph, at most 4096 of them (older ones are freed).
 * This hands out the oldest one, or *out = NULL if none waits; the caller
 * frees it with dvm_program_free.  It may be launched on a device context if
 * its tensors' addresses are that device's. */
dvm_status dvm_graph_take_program(dvm_graph* g, dvm_program** out);

/* Registers an external tensor (a graph input: the tensors a Load reads,
 * DVM review page, section 4.1, Table 1) as a value; read by ops, never
 * written through this handle.  The tensor struct is copied; its memory is
 * borrowed.  DVM_ERR_INVALID_ARG for a malformed tensor (ndim > 4, negative
 * dims or strides, unknown dtype). */
dvm_status dvm_graph_input(dvm_graph* g, const dvm_tensor* t, dvm_value* out);

/* Groups: ops added between begin and end are decided together (a composite
 * such as LayerNorm; the fusion decision of the DVM review page, section 5.2:
 * shape compatibility and dependence, flush when they fail).  An op added outside a group is a group of its own.
 * end_group fuses the group into the buffered graph or, when the fusion
 * conditions fail, flushes the buffered graph (encode + launch on the graph's
 * stream) and starts a new graph with the group (*flushed = 1).  A group the
 * VM cannot run at all returns DVM_ERR_UNSUPPORTED after flushing; its
 * values are then invalid and the caller computes them elsewhere. */
dvm_status dvm_graph_begin_group(dvm_graph* g);
dvm_status dvm_graph_end_group(dvm_graph* g, int32_t* flushed);

/* Appends one op (a primitive of the DVM review page's instruction set,
 * section 4.1, Table 1, and the binary ops, reductions and matmul its fusion
 * patterns use, section 5.1).  in[] are value handles; n_in counts tensor inputs (1 for a
 * binary op with a scalar operand, see dvm_attrs).  out gives the output's
 * dtype and storage (shape must equal the inferred shape; data may be NULL if
 * the value is released before its graph is flushed).  Writes the new value's
 * handle to *out_value.  Errors: DVM_ERR_SHAPE (inputs do not broadcast, or
 * out's shape differs from the inferred one), DVM_ERR_UNSUPPORTED (dtype or
 * operand form the VM does not run), DVM_ERR_INVALID_ARG (unknown, released or
 * lost input); outside a group, also the errors of dvm_graph_end_group. */
dvm_status dvm_graph_add_op(dvm_graph* g, int32_t op, const dvm_value* in, int32_t n_in,
                            const dvm_attrs* attrs, const dvm_tensor* out, uint32_t flags,
                            dvm_value* out_value);

/* The caller will not use the value again (neither as an input nor by reading
 * its storage): what the fuser needs to keep intermediate values on chip (DVM
 * review page, section 5.1: intermediate results stay in local memory).  A released value whose graph has not been flushed yet is
 * never stored unless DVM_OUT_LIVE was given. */
dvm_status dvm_graph_release(dvm_graph* g, dvm_value v);

/* Output shape of an op (for allocating out; the shape inference the
 * streaming fuser runs per op, DVM review page, section 5.2).  DVM_ERR_SHAPE
 * if the inputs do not fit the op. */
dvm_status dvm_graph_infer_shape(dvm_graph* g, int32_t op, const dvm_value* in, int32_t n_in,
                                 const dvm_attrs* attrs, dvm_tensor* out_shape);

/* Encodes the buffered graph into a program (shape tiling, DVM review page,
 * section 4.2; code header and body, section 4.3) and empties the buffer; *out = NULL when the buffer is empty or no buffered op
 * has an effect (every result is released unread: such ops are dropped, as
 * are x*1, x/1, x-(+0), x+(-0) and same-dtype casts nobody stores, which the
 * encoder folds into their operand; results are bit-identical either way).
 * The program is immutable and never cached; free it with dvm_program_free. */
dvm_status dvm_flush(dvm_graph* g, dvm_program** out);

/* Launches a program on the resident VM kernel of its kernel type, on
 * stream (hipStream_t): each workgroup finds its tiles from the header and
 * interprets the body tile by tile (DVM review page, section 4.4).  The
 * program is copied into the launch.  A reduce-all is two launches on the
 * stream: the VM kernel (one partial per workgroup) and a one-workgroup
 * combine of the partials into the scalar output.  Asynchronous;
 * DVM_ERR_DEVICE for an encode-only context or a failed launch. */
dvm_status dvm_launch(dvm_context* ctx, const dvm_program* p, void* stream);

/* dvm_launch for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops, harnesses that forbid hipMalloc): it calls no
 * hipMalloc, hipFree or allocating library routine.  Programs other than
 * reduce-alls launch exactly as with dvm_launch.  A reduce-all runs on the
 * library's static scratch array instead of the stream's allocated area: one
 * array per GPU, held until the process ends, of 256 + 4 * 65536 bytes (at
 * most 65536 partials, one per workgroup; the tiling runs at most 4096
 * workgroups); a program launching more workgroups returns DVM_ERR_RESOURCE
 * without launching.  Nothing in it needs to start at zero: every partial is
 * written before the combine reads it.  Every call
 * on a GPU shares that GPU's array and it keeps the last call's contents:
 * calls whose launches overlap on one GPU (different streams, or graph
 * replays running concurrently) race on it; callers serialise them.
 * Asynchronous. */
dvm_status dvm_launch_noalloc(dvm_context* ctx, const dvm_program* p, void* stream);

/* Profiling launch of a VECTOR program (the decode-overhead measurement: the
 * paper review page's section 4.4 has the Scalar unit decode the bytecode
 * while the vector units execute, and claims the decode is cheap next to the
 * execution).  Runs the profiling twin of the VM kernel, which computes the
 * same results as dvm_launch and also reads the cycle counter around every
 * dispatch.  For each workgroup b it writes DVM_PROF_COUNTERS uint64 values to
 * counters[DVM_PROF_COUNTERS * b + k] (device memory, owned by the caller, at
 * least DVM_PROF_COUNTERS * grid values, grid = dvm_header.grid):
 *   k = 0 total cycles of the workgroup, 1 decode cycles (instruction fetch,
 *   field decode and the dispatch to the handler), 2 execute cycles (the
 *   handlers, row-register runs inside them included), 3 tile-change cycles,
 *   4 dispatches.  Counts are wave 0's and approximate: the counter reads
 *   themselves perturb the schedule.  DVM_ERR_UNSUPPORTED for MIX programs,
 *   DVM_ERR_INVALID_ARG for a short or null buffer.  Asynchronous. */
#define DVM_PROF_COUNTERS 5
dvm_status dvm_launch_profiled(dvm_context* ctx, const dvm_program* p, void* stream, uint64_t* counters,
                               size_t n_counters);

/* Stacking (the stacking-based fusion of the DVM review page, section 5.1,
 * Figure 9: independent graphs packed into one launch).  With max_segments > 1
 * a graph keeps up to that many encoded programs (at most 7) before launching
 * them as one: each keeps its own header, tiling and workgroups, and they run
 * side by side.  A program joins only if it runs on the same VECTOR build,
 * is no reduce-all or branch program, fits the kernel argument (1000 words)
 * and is independent of the stacked ones: it writes no memory they read or
 * write and reads none they write.  Otherwise the stack launches first and
 * the program starts a new one (or runs at once).  dvm_graph_flush_launch,
 * dvm_sync and dvm_flush launch what the stack holds first; a graph destroyed
 * with programs in its stack discards them.  Default 1 (every program
 * launches when flushed).  Launches what the stack holds when called. */
dvm_status dvm_graph_set_stacking(dvm_graph* g, int32_t max_segments);

/* One stacked program from n (2..7) programs of one VECTOR build, none a
 * reduce-all; the caller guarantees they are independent (see above).  The
 * inputs stay the caller's.  DVM_ERR_UNSUPPORTED for other kernel types,
 * DVM_ERR_RESOURCE when the words exceed the kernel argument. */
dvm_status dvm_program_stack(const dvm_program* const* programs, size_t n, dvm_program** out);

/* Temporal stacking (DVM review page, section 5.1, Figure 9: tiles of
 * different graphs run on the same core in sequence).  With temporal = 1 the
 * graph launches its stack temporally: the segments' tiles form one tile
 * space in segment order, a launch of min(512, total tiles) workgroups runs
 * tile u on workgroup u mod grid, and each workgroup walks the segments in
 * order with a barrier between them (no launch, workgroup start or kernel
 * entry between segments).  The same segments join as under spatial
 * stacking (dvm_graph_set_stacking gives their number).  0 (default): spatial.
 * Launches what the stack holds when called.  DVM_ERR_INVALID_ARG for other
 * values. */
dvm_status dvm_graph_set_stack_order(dvm_graph* g, int32_t temporal);

/* dvm_program_stack, temporal: one program whose launch runs the n (2..7)
 * programs' tiles as one tile space (see dvm_graph_set_stack_order).  Same
 * requirements and errors as dvm_program_stack. */
dvm_status dvm_program_stack_temporal(const dvm_program* const* programs, size_t n, dvm_program** out);

/* Static-graph symbolic fusion (DVM review page, section 5.2, static-graph
 * fusion): a template is an op graph recorded once over symbolic dims;
 * dvm_template_finalize decides its fusion partition once (the streaming
 * fuser's rules, applied to shapes in which each symbol is one size shared by
 * all its occurrences and distinct from every other dim), and every
 * dvm_template_run binds concrete tensors and only tiles, encodes and
 * launches the precomputed graphs, with no per-op fusion decision.
 *
 * dims: >= 0 a concrete size, < 0 the symbol -(dims[i] + 1).  Symbols stand
 * for sizes >= 2.  Values are template-scoped handles.  Ops are added as with
 * dvm_graph_add_op but name their output dtype; DVM_OUT_LIVE makes the value a
 * template output (bound at run, in the order the outputs were added);
 * every other op value is internal and never stored, so a value one fused
 * graph computes and a later one reads must be an output (finalize fails with
 * DVM_ERR_RESOURCE otherwise).  Groups as for graphs.
 *
 * dvm_template_run: inputs[] and outputs[] in the order added; their dims
 * must match the template's (concrete dims exactly, each symbol one size);
 * outputs must not overlap inputs or each other (DVM_ERR_INVALID_ARG).  The
 * programs launch on the template's graph (dvm_template_graph: its stream,
 * stats, flush log, stacking; on an encode-only context its programs wait
 * for dvm_graph_take_program); DVM_ERR_RESOURCE when a bound shape has no
 * feasible tiling.  dvm_template_partition: the graph index of every op and
 * the host time finalize took. */
typedef struct dvm_template dvm_template;
dvm_status dvm_template_create(dvm_context* ctx, void* stream, dvm_template** out);
void dvm_template_destroy(dvm_template* t);
dvm_status dvm_template_graph(dvm_template* t, dvm_graph** out);
dvm_status dvm_template_input(dvm_template* t, int32_t dtype, int32_t ndim, const int64_t* dims, dvm_value* out);
dvm_status dvm_template_begin_group(dvm_template* t);
dvm_status dvm_template_end_group(dvm_template* t);
dvm_status dvm_template_add_op(dvm_template* t, int32_t op, const dvm_value* in, int32_t n_in, const dvm_attrs* attrs,
                               int32_t out_dtype, uint32_t flags, dvm_value* out);
dvm_status dvm_template_finalize(dvm_template* t, int32_t* n_graphs);
dvm_status dvm_template_partition(const dvm_template* t, int32_t* graph_of_op, size_t* n_ops, double* finalize_us);
dvm_status dvm_template_run(dvm_template* t, const dvm_tensor* inputs, int32_t n_inputs, const dvm_tensor* outputs,
                            int32_t n_outputs, int32_t* launched);

/* Device-side control flow (the if-else of the DVM review page's dynamic
 * control-flow workload, section 6.2; the MindSpore summary page, section 3.2,
 * flushes at such points): ops added between begin_branch and else_branch
 * form the then-body, ops between else_branch and end_branch the else-body.
 * begin_branch flushes the buffered graph first (the condition may be its
 * result); cond is one fp32 value with storage.  end_branch encodes one branch
 * program holding both bodies and launches it on the graph's stream
 * (*launched = 1); the VM reads cond when the program runs and every tile runs
 * the then-body iff cond > threshold (strictly: a NaN or equal value runs the
 * else-body), so no value travels to the host.  Each body must be one fusible
 * graph, and the two must share one tiling, operand table and staging (the
 * same operands in the same order, as in out = x + y versus out = x - y);
 * otherwise DVM_ERR_UNSUPPORTED and the values of both bodies are lost.
 * Groups cannot open inside a branch; flush, flush_launch and sync refuse
 * while a branch is open. */
dvm_status dvm_graph_begin_branch(dvm_graph* g, dvm_value cond, float threshold);

/* begin_branch on a reduce-all that this call adds: op (DVM_OP_REDUCE_SUM or
 * DVM_OP_REDUCE_MAX) over every element of x into the 0-d fp32 tensor out
 * (a live value, returned in *cond), then a branch on it, as in the
 * if-else-add workload (DVM review page, section 6.2: a sum, then a branch on
 * its sign).  The reduce-all launches at once, like any reduce-all; its
 * scalar is then folded from the workgroups' partials by the branch program
 * itself (each of its workgroups folds them in the reduce-all's fixed order
 * and workgroup 0 writes out), which saves the reduce-all's own combine
 * launch.  out holds its value on the stream once the branch program has run.
 * If the branch program does not take the fold (a body reads out, the
 * branch fails, the graph is destroyed with the branch open) or anything else
 * launches or syncs on the stream first, the combine launches before it, so
 * the value is the same either way.  Errors: those of dvm_graph_add_op and
 * dvm_graph_begin_branch; after an error no branch is open. */
dvm_status dvm_graph_begin_branch_reduce(dvm_graph* g, dvm_value x, int32_t op, const dvm_tensor* out,
                                         float threshold, dvm_value* cond);
dvm_status dvm_graph_else_branch(dvm_graph* g);
dvm_status dvm_graph_end_branch(dvm_graph* g, int32_t* launched);

/* Race-stress launch of a single VECTOR program: the profiling twin (same
 * results, same counters as dvm_launch_profiled) with a delay before every
 * dispatch, a seeded pseudo-random number of sleep intervals that is uniform
 * within a wave and differs between waves, so the waves of a workgroup drift
 * apart.  Every synchronisation a program needs comes from the barriers the
 * encoder inserted (DVM review page, section 4.3), so a correct program
 * stores bit-identical results under any seed.  Arguments and errors as for
 * dvm_launch_profiled.  Asynchronous. */
dvm_status dvm_launch_stress(dvm_context* ctx, const dvm_program* p, void* stream, uint32_t seed, uint64_t* counters,
                             size_t n_counters);

/* dvm_flush + dvm_launch on the graph's stream (an explicit flush, MindSpore
 * summary page, section 3.2; no-op when nothing is encoded; *launched = 0
 * then). */
dvm_status dvm_graph_flush_launch(dvm_graph* g, int32_t* launched);

/* Synchronisation point (flush at the sync interface, MindSpore summary page,
 * section 3.2): flush + launch, then wait for the graph's stream.
 * Asynchronous device errors surface here as DVM_ERR_DEVICE. */
dvm_status dvm_sync(dvm_graph* g);

/* The code header of a program (DVM review page, section 4.3). */
dvm_status dvm_program_header(const dvm_program* p, dvm_header* out);
/* Copies the program words (header, operand table, body: the bytecode of the
 * DVM review page, section 4.3); *n_words in: capacity, out: size.  buf may be
 * NULL to query the size. */
dvm_status dvm_program_words(const dvm_program* p, uint32_t* buf, size_t* n_words);
void dvm_program_free(dvm_program* p);

/* The bytecode verifier (the syncs and staging the encoder inserts, DVM review
 * page, section 4.3, are what the VM relies on; this re-derives them from the
 * words): layout and version, the tile's fit to its VM build and the header
 * counts it implies, operand indices and access forms, registers read only
 * after being written in the same tile, prefetch and invariant slots filled
 * before they are read and refilled once per tile, and no cross-wave
 * reduction buffer written before a barrier fences the previous reads of it
 * (over consecutive tiles).  Stacked programs: the directory and each
 * segment.  DVM_OK, or DVM_ERR_INTERNAL with the first violation (also copied
 * into msg, at most len bytes, if msg is not NULL).  With DVM_VERIFY set in
 * the environment (not "0"), the library verifies every program it encodes,
 * merges or stacks and fails that flush with DVM_ERR_INTERNAL on a
 * violation. */
dvm_status dvm_program_verify(const dvm_program* p, char* msg, size_t len);

/* A program from raw words (tests of the verifier; a program so made is never
 * launched by the library unless the caller launches it). */
dvm_status dvm_program_from_words(const uint32_t* words, size_t n_words, dvm_program** out);

/* Debug program for tiling parity (the tile range and element-to-tile rules
 * of the DVM review page, sections 4.2 and 4.4): same header and tiling as p,
 * whose body writes, for every element of the collapsed [R, C] space (a MIX
 * program: its [M, N] output), the row-major id of the tile that holds it into
 * tile_out and the workgroup that ran that tile into wg_out (both dense fp32
 * [R, C], caller-owned device memory).  A MIX debug program still reads the
 * matmul operands of p (its K loop runs; the result is unused).
 * DVM_ERR_SHAPE for outputs of another shape, layout or dtype. */
dvm_status dvm_program_debug_tilemap(const dvm_program* p, const dvm_tensor* tile_out,
                                     const dvm_tensor* wg_out, dvm_program** out);

/* Counters of the graph's fuser and encoder (the compile-time and fusion
 * measurements of the DVM review page, section 6). */
dvm_status dvm_graph_stats(const dvm_graph* g, dvm_stats* out);

/* Partition record of the graphs flushed so far, oldest first: graph i held
 * n_ops[i] ops, was flushed for reason reasons[i] (the dvm_stats flush_reason
 * index), took encode_us[i] microseconds of host time to encode and moves
 * bytes[i] physical bytes (dvm_header.bytes; 0 if its encode failed or it had
 * no effect).  Any output array may be NULL.  *n in: capacity, out: number of
 * graphs recorded. */
dvm_status dvm_graph_flush_log(const dvm_graph* g, int32_t* n_ops, int32_t* reasons, float* encode_us,
                               uint64_t* bytes, size_t* n);
/* Thread-local message of the last failed call on this thread. */
const char* dvm_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DVM_H */
