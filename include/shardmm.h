/*
 * shardmm.h -- C ABI of libshardmm, the sharded-matmul hot path on one
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is A[I,J] . B[J,K] -> C[I,K] with J contracted, laid out on
 * a mesh of named axes ("logical ranks"). Every logical rank's shards stay
 * resident on the one GPU; the library computes each rank's local product
 * and finishes what the collectives of a multi-device run would finish:
 * the sum of unreduced partials (all-reduce or reduce-scatter semantics)
 * and the assembly of finished blocks (all-gather).
 *
 * Sources: lingze.zone "Cheetsheet for the four cases of sharded matmul"
 * (sections Notation, Case 1-4, Summary); learntpu.dev ch05 "Sharded
 * matmuls and collectives on a torus" (Notation table, the four cases, the
 * sharding sandbox, the table of the four collectives); semiaifoundry.com
 * "Sharded matrix multiplication and result ownership" (The mechanism,
 * Engineering example, Interfaces); mbrenndoerfer.com "Row Parallelism"
 * (Y = X A = sum_i X_i A_i).
 *
 * Conventions for every call
 *  - Return value: an sm_status (0 = SM_OK). Nothing is thrown across the
 *    ABI. sm_last_error() gives a thread-local text for the last failure.
 *  - All argument checks run on the host before anything is enqueued, so a
 *    non-OK status other than SM_ERR_HIP leaves every output untouched.
 *  - Memory: every device buffer is allocated and freed by the caller. The
 *    library allocates no device memory and starts no threads; its only
 *    device state is the static scratch of sm_local_gemm_reduce_noalloc.
 *    Plans are caller-owned plain structs that need no freeing.
 *  - Streams: device calls enqueue on the given stream (a hipStream_t
 *    passed as void*; NULL = the null stream) and return without
 *    synchronising. Calls that overlap in time on different streams and
 *    touch the same output race.
 *  - Matrices are row-major. An sm_buf describes one buffer: base pointer,
 *    leading dimension ld (elements between consecutive rows), block_stride
 *    (elements between consecutive blocks of a stacked layout, or 0 for the
 *    global layout), elems (number of elements the buffer holds; every
 *    access is checked against it on the host) and dtype (SM_BF16 or
 *    SM_F32, the type of those elements). A call that reads or writes a
 *    buffer as another element type than its dtype fails with SM_ERR_DTYPE,
 *    so element counts are never applied to the wrong element size.
 *  - Alignment: base pointers 16-byte aligned; ld and block_stride multiples
 *    of 8 elements for bfloat16 and of 4 for float32 (SM_ERR_ALIGN).
 *  - Memory: every buffer must be addressable by the GPU (device, managed,
 *    or HIP-allocated / registered host memory). Pageable host memory is
 *    refused with SM_ERR_ARG as the last check before a launch. Outputs
 *    must not overlap inputs.
 */
#ifndef SHARDMM_H
#define SHARDMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SM_ABI_VERSION 2
#define SM_MAX_AXES 4
#define SM_NAME_LEN 8

typedef enum {
  SM_OK = 0,
  SM_ERR_ARG = 1,          /* null pointer, bad enum, index or range */
  SM_ERR_MESH = 2,         /* 0 or > SM_MAX_AXES axes, size < 1, duplicate/empty name */
  SM_ERR_SPEC = 3,         /* unparsable spec text, unknown axis, > 2 dims */
  SM_ERR_AXIS_REUSED = 4,  /* one mesh axis shards two dims of one array */
  SM_ERR_SHAPE = 5,        /* I, J or K < 1; a view larger than its buffer; ld too small */
  SM_ERR_INDIVISIBLE = 6,  /* a sharded dim does not split evenly; RS rows % N != 0 */
  SM_ERR_J_MISMATCH = 7,   /* A and B shard J over different axis lists */
  SM_ERR_NEEDS_GATHER = 8, /* local product asked of a case-2 or case-4 plan */
  SM_ERR_UNREDUCED = 9,    /* unreduced partials treated as finished blocks */
  SM_ERR_CASE = 10,        /* operation does not fit the plan's case */
  SM_ERR_DTYPE = 11,       /* unsupported element type for this operation */
  SM_ERR_ALIGN = 12,       /* pointer / ld / block_stride alignment */
  SM_ERR_HIP = 13          /* the HIP runtime reported an error */
} sm_status;

typedef enum { SM_CASE1 = 1, SM_CASE2 = 2, SM_CASE3 = 3, SM_CASE4 = 4 } sm_case;
typedef enum { SM_BF16 = 0, SM_F32 = 1 } sm_dtype;
typedef enum { SM_ALLREDUCE = 0, SM_REDUCESCATTER = 1 } sm_reduce_mode;

/* Epilogue applied to each fp32 accumulator of the local product before it
 * is stored in the plan's out_dtype (bfloat16 stores round to nearest even).
 * GeLU is the tanh form 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))),
 * applied elementwise to column blocks (ana-alekseeva.com, "MLP block"). */
typedef enum { SM_EPI_STORE = 0, SM_EPI_GELU_TANH = 1 } sm_epilogue;

/* What sm_gather_shards assembles. */
typedef enum {
  SM_WHAT_A = 0,           /* operand A blocks (stacked by A block id) */
  SM_WHAT_B = 1,           /* operand B blocks (stacked by B block id) */
  SM_WHAT_C_BLOCKS = 2,    /* finished output blocks, one per group */
  SM_WHAT_C_SCATTERED = 3, /* reduce-scatter output, one per (group, y) */
  SM_WHAT_C_PARTIAL = 4    /* unreduced partials: always SM_ERR_UNREDUCED */
} sm_what;

/* A mesh of named axes, e.g. {X:4, Y:2} = 8 logical ranks. Ranks are
 * numbered row-major over the axes in declared order. */
typedef struct {
  int32_t n_axes;
  char names[SM_MAX_AXES][SM_NAME_LEN];
  int32_t sizes[SM_MAX_AXES];
} sm_mesh;

/* Sharding of a 2-D array: per dimension, the ordered list of mesh axis
 * indices that split it (first listed = major when flattened). */
typedef struct {
  int32_t n[2];
  int32_t axes[2][SM_MAX_AXES];
} sm_spec;

/* A plan: caller-owned, immutable once filled by sm_plan.
 * A "unit" is one distinct local product: unit = g * n_partials + y, with g
 * the output block (group) index = i_block * c_grid[1] + k_block and y the
 * index of the rank's J slice (0 unless case 3). Ranks on axes used by
 * neither operand compute identical units (c_copies of each). */
typedef struct {
  uint32_t magic;          /* set by sm_plan; calls reject other values */
  int32_t kase;            /* sm_case */
  int32_t n_ranks;
  int32_t in_dtype;        /* sm_dtype of A and B (bfloat16) */
  int32_t out_dtype;       /* sm_dtype of the local products */
  int32_t n_partials;      /* N: partials per output block (1 unless case 3) */
  int32_t n_groups;        /* G: distinct output blocks */
  int32_t n_units;         /* G * N */
  int64_t I, J, K;
  int64_t a_local[2], b_local[2], c_local[2];
  int32_t a_grid[2], b_grid[2], c_grid[2];
  int32_t a_copies, b_copies, c_copies;
  uint32_t reduce_axes;    /* case 3: bit i set = axis i still to be summed ({U_...}) */
  int32_t gather_operand;  /* case 2/4: 0 = A, 1 = B; -1 otherwise */
  uint32_t gather_axes;    /* case 2/4: axes to all-gather that operand over */
  sm_mesh mesh;
  sm_spec a, b;
  sm_spec c;               /* output spec of the local products */
  sm_spec c_rs;            /* case 3: output spec after reduce-scatter */
} sm_plan_t;

/* One rank's place in a plan (block indices and global coordinates). */
typedef struct {
  int32_t coords[SM_MAX_AXES];
  int32_t unit, group, partial;   /* -1 when the plan has no local product */
  int32_t a_block[2], b_block[2], c_block[2];
  int64_t a_row0, a_col0, b_row0, b_col0, c_row0, c_col0;
  int64_t rs_row0, rs_rows;       /* case 3: global rows owned after reduce-scatter */
} sm_rank_info_t;

typedef struct {
  void* ptr;
  int64_t ld;
  int64_t block_stride;
  int64_t elems;
  int32_t dtype;     /* sm_dtype of the elements */
  int32_t reserved;  /* set to 0 */
} sm_buf;

/* ABI version and the size of sm_plan_t, for bindings to check layouts. */
int32_t sm_abi_version(void);
size_t sm_plan_size(void);

/* sha256 (64 hex digits) of the sources this library was built from, for
 * bindings to refuse a build older than its sources ("unknown" when the
 * build did not stamp one). */
const char* sm_build_digest(void);

/* Human-readable name of a status; thread-local detail of the last error. */
const char* sm_status_str(int32_t status);
const char* sm_last_error(void);

/* Fill a mesh from axis names (each 1..SM_NAME_LEN-1 chars) and sizes. */
int32_t sm_mesh_init(sm_mesh* mesh, int32_t n_axes, const char* const* names,
                     const int32_t* sizes);

/* Parse a partition spec for a 2-D array (learntpu.dev ch05, Notation
 * table and the sandbox's accepted forms): "P('X','Y')",
 * "P(('X','Y'), None)", "P(None, None)", "P()", "('X','Y'), None", or the
 * subscript notation "A[I_X, J_Y]", "I_XY, J" (single-letter axes). */
int32_t sm_parse_spec(const sm_mesh* mesh, const char* text, sm_spec* out);

/* Classify A[I,J].B[J,K] on the mesh into the four cases and fill *out
 * (lingze.zone Case 1-4 and Summary; learntpu.dev ch05 "The four cases").
 * Checks, in order: mesh, specs (SM_ERR_SPEC, SM_ERR_AXIS_REUSED), shape
 * (SM_ERR_SHAPE), divisibility (SM_ERR_INDIVISIBLE); then case 4 (A's I
 * and B's K share an axis) before the J cases; J sharded by both on
 * different axis lists is SM_ERR_J_MISMATCH. in_dtype must be SM_BF16;
 * out_dtype SM_F32, or SM_BF16 when no partial sums arise (not case 3). */
int32_t sm_plan(const sm_mesh* mesh, const sm_spec* a, const sm_spec* b,
                int64_t I, int64_t J, int64_t K, int32_t in_dtype,
                int32_t out_dtype, sm_plan_t* out);

/* Where rank `rank` sits in the plan: its mesh coordinates, the unit it
 * computes (group g and partial index y), the blocks of A, B and C it holds
 * with their global coordinates, and, for case 3, the rows it owns after a
 * reduce-scatter. This is the per-rank side of the output interface:
 * finished values are handed over together with each rank's coordinates
 * (semiaifoundry.com "Sharded matrix multiplication and result ownership",
 * section "Specifications and interfaces", Interfaces table), and every
 * block of an operand names the devices that hold it (learntpu.dev ch05,
 * sharding sandbox). Errors: SM_ERR_ARG for a rank outside [0, n_ranks). */
int32_t sm_rank_info(const sm_plan_t* plan, int32_t rank, sm_rank_info_t* out);

/* Cases 2 and 4 by composition (lingze.zone "Case 2" and "Case 4": all-gather
 * the offending operand, then multiply locally; learntpu.dev ch05, the four
 * cases). Given a case-2 or case-4 plan, fill *out with the plan that holds
 * after plan->gather_operand has been all-gathered over plan->gather_axes
 * (those axes removed from that operand's spec): case 1 or 3, or case 2
 * when a case-4 fix leaves the other operand sharded on J (call again).
 * The gather itself is sm_gather_shards with
 * SM_WHAT_A / SM_WHAT_B into the global layout, whose views serve any
 * partial gather. Errors: SM_ERR_CASE for case-1/3 plans;
 * SM_ERR_J_MISMATCH when, after a case-4 fix, A and B shard J over
 * different axis lists (a reshard of J is needed first). */
int32_t sm_plan_gathered(const sm_plan_t* plan, sm_plan_t* out);

/* Local products C_u = A_u . B_u for units [unit_begin, unit_begin+count):
 * bfloat16 inputs, fp32 accumulation, epilogue, store in plan->out_dtype
 * (learntpu.dev ch05 sandbox "Local matmul"; lingze.zone Case 1 and 3).
 *  A, B: global layout (block_stride 0: the unit's view is taken at its
 *        block coordinates in the whole [I,J] / [J,K] array) or stacked
 *        (block_stride > 0: block id = row_block * grid[1] + col_block).
 *  C:    case 1: global layout (the [I,K] array) or stacked; case 3:
 *        stacked only (partials overlap in output coordinates, so a global
 *        layout is SM_ERR_UNREDUCED). Stacked output blocks are indexed
 *        relative to unit_begin.
 * Rows of at most 64 (a skinny batch) use a split-J streaming kernel; other
 * shapes use the LDS-tiled MFMA kernel. Errors: SM_ERR_NEEDS_GATHER for
 * case 2/4, SM_ERR_CASE for a GeLU epilogue on case 3. */
int32_t sm_local_gemm(const sm_plan_t* plan, const sm_buf* A, const sm_buf* B,
                      const sm_buf* C, int32_t epilogue, int32_t unit_begin,
                      int32_t unit_count, void* stream);

/* Sum the N partials of each group g in [group_begin, group_begin+count)
 * in rank order in fp32: S_g = (((P_{g,0} + P_{g,1}) + ...) + P_{g,N-1})
 * (semiaifoundry.com "The mechanism" step 4; learntpu.dev ch05 table of
 * the four collectives).
 *  partials: stacked fp32, block index = unit - group_begin * N.
 *  SM_ALLREDUCE: out receives S_g, one copy per group (every rank of the
 *    group shares it): global [I,K] layout (block_stride 0) or stacked by
 *    g - group_begin.
 *  SM_REDUCESCATTER: reduce coordinate y keeps rows [y m/N, (y+1) m/N) of
 *    S_g: global layout (rows at the plan's c_rs coordinates) or stacked by
 *    (g - group_begin) * N + y, each block [m/N, n].
 * Errors: SM_ERR_CASE unless case 3; SM_ERR_INDIVISIBLE if RS and m % N. */
int32_t sm_reduce_partials(const sm_plan_t* plan, const sm_buf* partials,
                           const sm_buf* out, int32_t mode, int32_t group_begin,
                           int32_t group_count, void* stream);

/* Local products and their reduction in one kernel, with no partial buffers
 * (the one-GPU counterpart of overlapping the reduce with the matmul,
 * learntpu.dev ch05 "Overlapping communication with compute: collective
 * matmul"). For each group g in [group_begin, group_begin+count) of a
 * case-3 plan, the N units' products accumulate into one fp32 accumulator
 * in rank order y = 0..N-1 -- the N slices of J are contiguous in the
 * global layout, so this is one product over the whole of J -- and the
 * finished block S_g is written:
 *  SM_ALLREDUCE: out global [I,K] at the group's block, or stacked by
 *    g - group_begin ([m, n] blocks);
 *  SM_REDUCESCATTER: out global (the same rows, at the plan's c_rs
 *    coordinates), or stacked by (g - group_begin) * N + y ([m/N, n]).
 * A and B must use the global layout (block_stride 0). The result equals
 * sm_local_gemm + sm_reduce_partials up to fp32 summation order (bit for
 * bit on integer-valued inputs). Local products of at most 64 rows are
 * refused with SM_ERR_SHAPE: their split-J kernel needs a workspace
 * (sm_local_gemm_reduce_ws). A launch with few output tiles (fewer than
 * 256, e.g. a 128-row batch) leaves most compute units idle for the whole
 * of J; sm_local_gemm_reduce_ws with a workspace runs such products in
 * parallel instead (about 4x faster on a 128-row batch split 8 ways). */
int32_t sm_local_gemm_reduce(const sm_plan_t* plan, const sm_buf* A, const sm_buf* B,
                             const sm_buf* out, int32_t mode, int32_t group_begin,
                             int32_t group_count, void* stream);

/* Bytes of device workspace sm_local_gemm_reduce_ws uses for group_count
 * groups of a case-3 plan: for local products of at most 64 rows the
 * arrival counters followed by the N partials of each group (required);
 * for taller products whose single launch would have fewer than 256 output
 * tiles, the N partials of each group (optional, see below); else 0.
 * Errors: SM_ERR_CASE unless case 3, SM_ERR_ARG for a group_count outside
 * [1, n_groups]. */
int32_t sm_gemm_reduce_workspace(const sm_plan_t* plan, int32_t group_count, int64_t* bytes);

/* sm_local_gemm_reduce for every local-product height, with a
 * caller-provided workspace (mbrenndoerfer.com "Row Parallelism": each rank
 * forms Z_i = X_i A_i and the output is their sum Y = sum_i X_i A_i;
 * semiaifoundry.com "The mechanism", step 4). Local products of more than
 * 64 rows run as in sm_local_gemm_reduce (one launch over the group's whole
 * J), unless that launch would have fewer than 256 output tiles and the
 * workspace holds the N partials of each group: then the N units' products
 * run in parallel into the workspace and a second launch sums them in rank
 * order (exactly sm_local_gemm + sm_reduce_partials; on floats this differs
 * from the single launch by fp32 rounding only). The workspace may be NULL
 * or smaller for these plans. Local products of at most 64 rows (a skinny
 * batch) run the split-J streaming kernel with the reduction fused into it,
 * in one launch per 64 units:
 *  - every workgroup (one unit y of group g, one block of 256 output
 *    columns) writes its partial P_{g,y} into the workspace and counts
 *    itself in at the counter of its (group, column block);
 *  - the workgroup that arrives last sums that block's N partials in rank
 *    order, S_g = ((P_{g,0} + P_{g,1}) + ...) + P_{g,N-1}, writes the rows
 *    to `out` as sm_local_gemm_reduce does (AR or RS, global or stacked),
 *    and returns the counter to zero. No workgroup waits for another.
 * Workspace (device memory, 256-byte aligned, workspace_bytes >=
 * sm_gemm_reduce_workspace(plan, group_count)), owned by the caller:
 *  - bytes [0, C): 32-bit arrival counters, C = 4 * group_count *
 *    ceil(n / 256) rounded up to 256. They must be zero before the first
 *    call (a zero-filled allocation); every call leaves them zero.
 *  - bytes [C, ...): the partials, float32, stacked by (g - group_begin)
 *    * N + y, each [m, ld] with ld = n rounded up to 4. After the call they
 *    hold every unit's partial (bit for bit what sm_local_gemm stores).
 * Calls that share a workspace must not overlap in time (same stream, or
 * synchronised). Errors as sm_local_gemm_reduce; SM_ERR_SHAPE for a
 * workspace too small or more than 64 partials per group; SM_ERR_ALIGN for
 * a misaligned workspace; SM_ERR_ARG for NULL or non-device workspace
 * memory when one is needed. */
int32_t sm_local_gemm_reduce_ws(const sm_plan_t* plan, const sm_buf* A, const sm_buf* B,
                                const sm_buf* out, int32_t mode, int32_t group_begin,
                                int32_t group_count, void* workspace, int64_t workspace_bytes,
                                void* stream);

/* sm_local_gemm_reduce_ws without a workspace argument, for callers that
 * cannot allocate device memory: code under stream capture, tight serving
 * loops, harnesses that forbid allocation. The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine). Skinny products keep
 * their counters and partials in the library's static device array
 * (64 KiB of counters + 32 MiB of partials, held by every GPU the library
 * runs on until the process ends); a call that needs more is refused with
 * SM_ERR_SHAPE before anything is launched (use sm_local_gemm_reduce_ws).
 * The first call on a device also enqueues, on `stream`, the clearing of
 * that device's counters; every completed call leaves them zero. All calls
 * on one GPU share the array: calls that overlap in time (other streams
 * without synchronisation, other threads) race. Products of more than 64
 * rows use the scratch as sm_local_gemm_reduce_ws uses its workspace when
 * their partials fit in it, else run as sm_local_gemm_reduce. Results are
 * bit for bit those of sm_local_gemm_reduce_ws with a workspace of the
 * same capacity. Errors as sm_local_gemm_reduce_ws. */
int32_t sm_local_gemm_reduce_noalloc(const sm_plan_t* plan, const sm_buf* A, const sm_buf* B,
                                     const sm_buf* out, int32_t mode, int32_t group_begin,
                                     int32_t group_count, void* stream);

/* Sequence-parallel tail (ana-alekseeva.com "Sequence parallelism": the
 * all-reduce of a tensor-parallel block becomes a reduce-scatter, layer norm
 * runs on each device's own token rows, and the rows are all-gathered before
 * the next block). For each group g, reduce the N partials in rank order
 * exactly as sm_reduce_partials(SM_REDUCESCATTER) and apply, to every owned
 * row x of length n:
 *   y = (x - mean(x)) / sqrt(var(x) + eps) * gamma + beta,
 * var the biased (1/n) variance, gamma/beta device float arrays of n
 * elements (NULL = 1 / 0). The plan's output must have whole rows
 * (c_grid[1] == 1, else SM_ERR_CASE); rows of at most 32768 elements, n a
 * multiple of 4 and 16-byte aligned rows (SM_ERR_SHAPE / SM_ERR_ALIGN).
 * out: global layout (then the all-gathered tensor is already in place) or
 * stacked by (g - group_begin) * N + y. */
int32_t sm_reduce_scatter_layernorm(const sm_plan_t* plan, const sm_buf* partials,
                                    const sm_buf* out, const float* gamma, const float* beta,
                                    float eps, int32_t group_begin, int32_t group_count,
                                    void* stream);

/* Reshard a 2-D array between two partition specs on one mesh: AllToAll
 * A[I, J_X] -> A[I_X, J] moves which dimension is sharded (learntpu.dev
 * ch05, table of the four collectives; lingze.zone "Communication
 * primitives"); a replicated target ("P()") is an all-gather. Every block
 * of `to` is assembled from the overlapping parts of the blocks of `from`.
 * src / dst: global layout (block_stride 0) or stacked by block id
 * (row_block * grid[1] + col_block), one copy per distinct block.
 * dtype: SM_BF16 or SM_F32. Errors: SM_ERR_SPEC, SM_ERR_AXIS_REUSED,
 * SM_ERR_INDIVISIBLE as for sm_plan; SM_ERR_ARG if both are global. */
int32_t sm_reshard(const sm_mesh* mesh, const sm_spec* from, const sm_spec* to,
                   int64_t rows, int64_t cols, int32_t dtype, const sm_buf* src,
                   const sm_buf* dst, void* stream);

/* All-gather on one GPU: copy each distinct finished block once from a
 * stacked layout into the global layout (lingze.zone Case 1, replication
 * as a separate AllGather; semiaifoundry.com step 5). what = SM_WHAT_A /
 * SM_WHAT_B (bfloat16 operand blocks), SM_WHAT_C_BLOCKS (one block per
 * group: case-1 outputs or all-reduced case-3 outputs), SM_WHAT_C_SCATTERED
 * (reduce-scatter outputs). SM_WHAT_C_PARTIAL is refused with
 * SM_ERR_UNREDUCED: concatenating partials does not add them. out must use
 * the global layout (block_stride 0). */
int32_t sm_gather_shards(const sm_plan_t* plan, int32_t what, const sm_buf* shards,
                         const sm_buf* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SHARDMM_H */
