/*
 * ja.h -- C ABI of libja, a one-GPU join-agg engine for AMD Instinct MI355X
 * (gfx950).
 *
 * Model ("Every Kernel Is a Join: Automatic Multi-GPU Parallelism for AI
 * Computations in Einsummable", paperpeel full text):
 *   - a tensor relation is a set of (key, sub-tensor) pairs (section 1,
 *     section 3.2); here the key of a block is its coordinate in a
 *     per-dimension interval grid and the block is the projection of the
 *     tensor onto that box;
 *   - an operator is executed as a join of input blocks into n-tuples, a
 *     per-tuple kernel f, an aggregation (the operator's sum-like operator,
 *     which need not be addition, section 5.2) of all partial results that
 *     share an output type, and a recompose of the aggregated blocks
 *     (section 3.2, Definition 3.7);
 *   - the join-agg spec for a request holds exactly one function spec per
 *     combination of intervals of the shardable indices (section 3.3);
 *   - between operators, data is re-blocked through the atoms of the overlay
 *     of producer and consumer blockings (section 5.3).
 *
 * On one GPU the pages' "one function spec per processor" becomes "one tuple
 * per unit of kernel work": tuples map to workgroups, and aggregation is fused
 * into the tuple kernel (eager aggregation) unless the unfused entry points
 * ja_kernel / ja_agg are used.
 *
 * Conventions for every entry point:
 *   - No exceptions cross the ABI.  Every function returns a ja_status; on
 *     failure ja_last_error() returns a thread-local message.
 *   - All validation of specs, decompositions and relation descriptors runs on
 *     the host before any HIP call, so every error except JA_ERR_HIP can be
 *     raised without a GPU.
 *   - The library never allocates device memory.  Device buffers (relations,
 *     plan tables, workspaces) are owned by the caller; their sizes come from
 *     the *_bytes queries.  Host handles (ja_spec, ja_decomp, ja_tuples,
 *     ja_plan, ja_repart) are owned by the library until the matching
 *     *_destroy call.
 *   - A `stream` argument is a hipStream_t passed as void* (NULL = the null
 *     stream).  Run calls are asynchronous on that stream and never
 *     synchronise the host; upload calls block until their copy is complete.
 *   - Device pointers must be 16-byte aligned.
 *
 * Relation storage layout (one contiguous device buffer per relation):
 * blocks are stored back to back in lexicographic order of their keys (first
 * dimension slowest); every block is dense row-major over its own box.  A
 * relation with one block per dimension is an ordinary dense row-major
 * tensor.
 */
#ifndef JA_H
#define JA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define JA_MAX_RANK 8
#define JA_ABI_VERSION 1

typedef int32_t ja_status;
#define JA_OK 0
#define JA_ERR_ARG (-1)         /* null pointer, bad enum or count */
#define JA_ERR_SPEC (-2)        /* malformed einsum string, op name or params */
#define JA_ERR_DECOMP (-3)      /* bad intervals: not a tiling, wrong count, or a letter that may not be split */
#define JA_ERR_SHAPE (-4)       /* relation shape or blocking does not match the spec / decomposition */
#define JA_ERR_DTYPE (-5)       /* unsupported or mismatched element type */
#define JA_ERR_WORKSPACE (-6)   /* a caller buffer is smaller than the size query returned */
#define JA_ERR_UNSUPPORTED (-7) /* valid request that the library has no kernel for */
#define JA_ERR_HIP (-8)         /* a HIP runtime call failed (message in ja_last_error) */
#define JA_ERR_STATE (-9)       /* plan used before ja_plan_upload / ja_repart_upload */

typedef enum { JA_F32 = 0, JA_BF16 = 1, JA_F16 = 2 } ja_dtype;

/* Aggregation operators for ja_agg (section 3.2 step 2; section 5.2: the
 * aggregation need not be addition).  JA_AGG_SOFTMAX folds attention's
 * per-tuple triples (m, l, acc) with m = max(m1, m2),
 * l = l1 e^(m1-m) + l2 e^(m2-m), acc = acc1 e^(m1-m) + acc2 e^(m2-m) and
 * writes acc / l. */
typedef enum { JA_AGG_SUM = 0, JA_AGG_MAX = 1, JA_AGG_SOFTMAX = 2 } ja_agg_op;

/* A blocked tensor relation.  For dimension d, the blocks' boundaries are
 * splits[d][0] = 0 < splits[d][1] < ... < splits[d][nblk[d]] = shape[d]
 * (half-open intervals).  splits[d] may be NULL: then dimension d is cut into
 * nblk[d] near-equal intervals, the first (shape[d] mod nblk[d]) of them one
 * element longer.  The descriptor and its split arrays are read only during
 * the call they are passed to. */
typedef struct ja_relation_desc {
    int32_t rank;                       /* 1 .. JA_MAX_RANK */
    int32_t dtype;                      /* ja_dtype */
    int64_t shape[JA_MAX_RANK];         /* logical extents, > 0 */
    int32_t nblk[JA_MAX_RANK];          /* blocks per dimension, 1 .. shape[d] */
    const int64_t* splits[JA_MAX_RANK]; /* nblk[d] + 1 points, or NULL */
} ja_relation_desc;

/* Logical re-indexing applied by a repartition: the source tensor is read
 * row-major as shape[0..rank), its axes are permuted (axis k of the result is
 * axis perm[k] of the view), and the result is read row-major as the
 * destination's shape.  Element counts must agree. */
typedef struct ja_view {
    int32_t rank;
    int64_t shape[JA_MAX_RANK];
    int32_t perm[JA_MAX_RANK];
} ja_view;

typedef struct ja_spec ja_spec;
typedef struct ja_decomp ja_decomp;
typedef struct ja_tuples ja_tuples;
typedef struct ja_plan ja_plan;
typedef struct ja_repart ja_repart;

/* ---- diagnostics ------------------------------------------------------ */

int32_t ja_abi_version(void);
/* Static string naming a status code. */
const char* ja_status_str(ja_status status);
/* Thread-local description of the last failure on this thread ("" if none). */
const char* ja_last_error(void);

/* ---- relations (section 3.1 tensor types and tilings; section 3.2) ----- */

/* Total bytes of the relation's buffer. */
ja_status ja_relation_bytes(const ja_relation_desc* rel, size_t* bytes);
/* Number of blocks (the product of nblk). */
ja_status ja_relation_nblocks(const ja_relation_desc* rel, int64_t* nblocks);
/* Box [lo, hi) of the block with key `key` (rank entries) and its byte
 * offset in the relation buffer. */
ja_status ja_relation_block(const ja_relation_desc* rel, const int64_t* key, int64_t* lo, int64_t* hi,
                            size_t* byte_off);

/* ---- operators and join-agg specs (section 3.2, section 3.3) ---------- */

/* An abstract operator over named indices, written as an einsum string whose
 * letters ('a'..'z') are the named indices; the letters' order of first
 * appearance is the "letter order" used by every per-letter array below.
 *
 *   op "contract":  "A,B->C", two operands (e.g. "ij,jk->ik").  f is the
 *                   block contraction; letters absent from the output are
 *                   aggregated with SUM (section 3.2, Examples 3.8, 3.9).
 *                   Every letter must appear in at least two of A, B, C.
 *   The next two fuse a 1:1 join (how section 1 models elementwise
 *   operators) into the contraction, applied to each aggregated block.
 *   op "contract_add": "A,B,C->C" (e.g. "tm,mn,tn->tn"): the contraction
 *                   with the residual relation R (third operand, the
 *                   output's letters and blocking) joined 1:1 on the output
 *                   key after the SUM: C = A B + R, rounded once.
 *   op "contract_swiglu": "A,B->C" where B's last letter (absent from A and
 *                   C, extent 2, one interval) indexes a (gate, up) pair
 *                   (e.g. "td,dfc->tf", B[d][f][0] the gate weights and
 *                   B[d][f][1] the up weights): the contraction's two
 *                   members g, u of each pair are joined 1:1 after the SUM,
 *                   C = g / (1 + exp(-g)) * u, rounded once.  Both fused
 *                   forms take and write bf16 or f16 (JA_ERR_DTYPE
 *                   otherwise) and have no unfused path (JA_ERR_UNSUPPORTED
 *                   from ja_plan_partial_bytes, ja_kernel and ja_agg).
 *   op "attention": "Q,K,V->O" with Q = O = [batch..., group..., s, d] and
 *                   K = V = [batch..., t, d] (e.g. "bhsd,bhtd,bhtd->bhsd").
 *                   The optional group letters, which must not index K and
 *                   V, number the query heads that share one key-value head
 *                   (grouped-query attention, section 3.3: with
 *                   "bgrsd,bgtd,bgtd->bgrsd", query head 4g + r of a
 *                   4-per-group layout reads key-value head g, and splitting
 *                   g splits the query heads with it).  The batch and group
 *                   letters may also follow the position letter, as in the
 *                   token-major relations a projection writes: Q = O =
 *                   [batch..., s, batch..., group..., d], K = V = [batch...,
 *                   t, batch..., d] with the same letters before s and t
 *                   (e.g. "bshd,bthd,bthd->bshd" or "bsgrd,btgd,btgd->bsgrd");
 *                   Q's second-to-last letter is read as s whenever it is
 *                   absent from K and t is K's second to last.
 *                   Scores Q K^T * scale joined on d; aggregation over t with
 *                   the online-softmax triple (max, sum of exponentials,
 *                   weighted sum of values); then O = weighted sum / sum.
 *                   params: "scale=<float>" (default 1/sqrt(|d|); must be
 *                   positive, JA_ERR_SPEC otherwise),
 *                   "causal=<s>,<t>" (key t visible to query s iff t <= s;
 *                   fully masked tuples are dropped at join),
 *                   "packed=<e1>,<e2>,...": independent sequences packed end
 *                   to end along s and t, ending at the ascending positions
 *                   e1 < e2 < ...; a key is visible to a query only inside
 *                   the query's sequence, the join drops (query block, key
 *                   block) pairs that share no sequence, and a decomposition
 *                   may split s and t only at sequence ends and must span
 *                   every sequence (section 3.3, Shardable Indices;
 *                   JA_ERR_DECOMP otherwise).
 *                   "packed=device": the sequences end exactly at the cuts
 *                   of s (and t, which must be cut alike, JA_ERR_DECOMP
 *                   otherwise), so the ends can be data computed on the GPU
 *                   and handed to the device-side join and planner
 *                   (ja_djoin_*, ja_dattn_*) as split points.
 *   op "rmsnorm":   "rd,d->rd": y = x / sqrt(mean_d x^2 + eps) * gain; the
 *                   per-row sum of squares is SUM-aggregated over d blocks,
 *                   then joined 1:1 with x and gain.  params "eps=<float>"
 *                   (default 1e-6).
 *   op "swiglu":    "rf,rf->rf": h = g / (1 + exp(-g)) * u, a 1:1 key join.
 *   op "add":       "rd,rd->rd": c = a + b, a 1:1 key join.
 */
ja_status ja_spec_create(const char* einsum, const char* op, const char* params, ja_spec** out);
void ja_spec_destroy(ja_spec* spec);
/* Letters in letter order, NUL-terminated, into buf (cap >= 27 suffices). */
ja_status ja_spec_letters(const ja_spec* spec, char* buf, size_t cap);

/* A decomposition: the intervals requested for every letter (section 3.3).
 * extents[i] is the extent of letter i (letter order).  For letter i either
 * splits[i] (intervals[i] + 1 points from 0 to extents[i]) is given, or
 * splits == NULL / splits[i] == NULL and the letter is cut into intervals[i]
 * near-equal intervals.  Letters an operator cannot split (attention: the
 * head dimension d) must have one interval (JA_ERR_DECOMP otherwise). */
ja_status ja_decomp_create(const ja_spec* spec, const int64_t* extents, const int32_t* intervals,
                           const int64_t* const* splits, ja_decomp** out);
void ja_decomp_destroy(ja_decomp* decomp);

/* ---- join: the tuple list (section 3.2 step 1) ------------------------- */

/* Enumerate the join-agg spec's function specs: one tuple per cell of the
 * interval grid (product of the interval counts), minus cells removed by
 * the operator's join predicate (causal attention drops a cell when its key
 * interval starts at or after the end of its query interval).  Tuples are
 * sorted by their group-by key (contract and attention: the output letters;
 * rmsnorm: the row letter; swiglu and add: all letters), then by the other
 * letters' interval indices in letter order.  Equal group-by keys form one
 * aggregation segment.  Host only, deterministic. */
ja_status ja_join(const ja_spec* spec, const ja_decomp* decomp, ja_tuples** out);
ja_status ja_tuples_count(const ja_tuples* tuples, int64_t* n_tuples, int64_t* n_segs, int32_t* n_letters);
/* rec: n_tuples * n_letters int32 (each record = the interval index of every
 * letter, letter order); seg_off: n_segs + 1 int64 CSR offsets. */
ja_status ja_tuples_export(const ja_tuples* tuples, int32_t* rec, int64_t rec_cap, int64_t* seg_off,
                           int64_t seg_cap);
void ja_tuples_destroy(ja_tuples* tuples);

/* ---- device-side join (section 3.2 step 1 on the GPU; section 3.3) ------ */

/* The same join as ja_join, run by kernels on a stream into caller-owned
 * device memory, with the split POSITIONS read from device memory at run
 * time: a decomposition whose cuts depend on device data (for example the
 * ends of packed sequences computed on the GPU, section 3.3) is joined with
 * no host round trip.  Only the extents and the interval COUNTS are fixed
 * when the join is created.  The result, for given split points, equals
 * ja_join's records and segment offsets for the decomposition with those
 * split points, bit for bit.
 *
 * ja_djoin_create: host only; extents[i] and intervals[i] per letter (letter
 * order).  JA_ERR_DECOMP for a count outside [1, extent], a split attention
 * head dimension, or (packed sequences) a sequence letter that does not span
 * every sequence or has more intervals than there are sequences;
 * JA_ERR_UNSUPPORTED beyond 2^28 grid cells.  The handle keeps no reference
 * to spec. */
typedef struct ja_djoin ja_djoin;
ja_status ja_djoin_create(const ja_spec* spec, const int64_t* extents, const int32_t* intervals, ja_djoin** out);
/* table_bytes: device table to upload once (the packed sequence ends);
 * workspace_bytes: device scratch of one run (256-byte aligned);
 * max_tuples / max_segs: capacities the outputs need (the full grid, the
 * number of group-by keys); n_splits: int64 entries of the split array. */
ja_status ja_djoin_device_bytes(const ja_djoin* join, size_t* table_bytes, size_t* workspace_bytes,
                                int64_t* max_tuples, int64_t* max_segs, int64_t* n_splits);
/* Copies the table into dev_buf (16-byte aligned, caller-owned, kept until
 * destroy) and waits for the copy. */
ja_status ja_djoin_upload(ja_djoin* join, void* dev_buf, size_t bytes, void* stream);
/* Enqueue the join on `stream` (asynchronous; no host synchronisation).
 *   splits_dev: device int64, n_splits entries: letter after letter (letter
 *               order), the intervals + 1 split points of the letter;
 *   rec:        device int32, max_tuples * n_letters: record i = the
 *               interval index of every letter (letter order), sorted as
 *               ja_join sorts; the first n_tuples records are written;
 *   seg_off:    device int64, max_segs + 1: CSR offsets, the first
 *               n_segs + 1 written;
 *   counts:     device int64[3]: n_tuples, n_segs, status.  status 0: valid;
 *               bit 0: some letter's split points do not start at 0, end at
 *               its extent and rise strictly; bit 1: a packed sequence
 *               letter is cut away from a sequence end; bit 2 (spec with
 *               "packed=device"): the two sequence letters are cut
 *               differently.  A nonzero status leaves n_tuples = n_segs = 0
 *               and seg_off[0] = 0.
 *   workspace:  device, workspace_bytes.
 * Host-side argument errors return before anything is enqueued; device
 * buffers too small for the stated sizes are undefined behaviour. */
ja_status ja_djoin_run(const ja_djoin* join, const int64_t* splits_dev, int32_t* rec, int64_t* seg_off,
                       int64_t* counts, void* workspace, void* stream);
void ja_djoin_destroy(ja_djoin* join);

/* ---- measurement aid ------------------------------------------------------ */

/* The matrix-core ceiling this GPU sustains: `workgroups` workgroups of 4
 * wavefronts, each wavefront issuing `iters` rounds of 4 independent bf16
 * 32x32x16 MFMAs with no memory traffic, LDS or barriers.  sink: device,
 * workgroups * 256 floats, written with the accumulators' sums.  *flops
 * (may be NULL) gets the flops enqueued; time the launch on `stream`. */
ja_status ja_calibrate_mfma(int32_t workgroups, int32_t iters, float* sink, double* flops, void* stream);
/* The HBM ceiling a plain streaming copy reaches: copy `bytes` bytes from
 * src to dst (device buffers, 16-byte aligned, bytes a multiple of 16, not
 * overlapping) with 16-byte vector loads and stores, four per thread in
 * flight.  Asynchronous on `stream`; time the launch there. */
ja_status ja_calibrate_copy(const void* src, void* dst, size_t bytes, void* stream);

/* ---- attention planned on the device (section 3.3; section 3.2 on the GPU) */

/* Packed sequences whose ends are device data: attention with
 * "packed=device" (the sequences end at the cuts of s and t), joined by the
 * device-side join, turned into the attention kernel's tables by kernels,
 * and computed, all enqueued on one stream with no host round trip.
 *
 * ja_dattn_create: host only.  extents / intervals per letter as for
 * ja_djoin_create; s and t have one interval per sequence (the same count),
 * the head dimension (128) one; every other letter is cut into near-equal
 * intervals.  dtype JA_BF16 or JA_F16 (Q, K, V, O alike).  JA_ERR_SPEC for
 * any other spec.
 *
 * Layouts (caller-owned, 16-byte aligned): Q and O are the relation
 * [batch..., group..., S, D] blocked by the intervals of its batch and group
 * letters only (s and d whole): blocks back to back in key order, each dense
 * row-major; K and V likewise over [batch..., S, D] with their batch
 * letters.  These layouts do not depend on where the sequences end. */
typedef struct ja_dattn ja_dattn;
ja_status ja_dattn_create(const ja_spec* spec, const int64_t* extents, const int32_t* intervals, int32_t dtype,
                          ja_dattn** out);
/* table_bytes: device table, uploaded once (256-byte aligned buffer);
 * workspace_bytes: scratch of one run (256-byte aligned); n_splits: int64
 * entries of the split array. */
ja_status ja_dattn_device_bytes(const ja_dattn* attn, size_t* table_bytes, size_t* workspace_bytes,
                                int64_t* n_splits);
ja_status ja_dattn_upload(ja_dattn* attn, void* dev_buf, size_t bytes, void* stream);
/* Enqueue join, table building and attention on `stream`.  splits_dev:
 * every letter's split points in letter order (device int64), those of s and
 * t being the sequence ends 0 < e1 < ... < S.  counts: device int64[3], the
 * join's tuple and segment counts and status (ja_djoin_run); with a nonzero
 * status nothing is computed and O is not written. */
ja_status ja_dattn_run(const ja_dattn* attn, const int64_t* splits_dev, const void* Q, const void* K, const void* V,
                       void* O, int64_t* counts, void* workspace, void* stream);
void ja_dattn_destroy(ja_dattn* attn);

/* ---- logical optimization (section 4) ------------------------------------ */

/* A computation graph of abstract operators (section 4.2: vertices are
 * operators, an edge runs from the producer of a tensor to each consumer)
 * and the choice of one join-agg spec per operator.
 *
 * Candidate specs of an operator cut its shardable indices (section 3.3:
 * every index of a contraction or an elementwise join; for attention the
 * key-value batch / head letters and both sequence letters, not the query
 * group letters nor the head dimension; for RMSNorm the row and the feature
 * letter) into near-equal intervals whose counts multiply to the processor
 * count p.  A tiling of a tensor is given by its interval count per
 * dimension.
 *
 * Cost proxy (section 4.3), in elements: repartition -- every element of an
 * operator-produced input whose tiling differs from the one the consumer's
 * spec asks for (computation inputs are materialised directly in the blocks
 * asked for: zero); join -- the elements of every input block of every
 * function specification the join keeps; aggregation -- (copies - 1) times
 * the elements of every distinct aggregated type (contraction and
 * attention: the output blocks; RMSNorm: the per-row sums of squares).
 *
 * Modes of ja_graph_plan:
 *   JA_PLAN_OPTIMAL: the dynamic program over output tilings (section 4.2):
 *       Opt(Op, T) = min over specs J with out(J) = T of join(J) + agg(J) +
 *       sum over inputs k of min over the producer's tilings T_k of
 *       [repartition(J, k, T_k) + Opt(producer_k, T_k)], then a trace back
 *       from the cheapest tiling of the output.  Graphs that are not trees
 *       are cut at every edge out of a tensor with several consumers and the
 *       pieces planned one at a time, larger first (section 4.5); an edge
 *       between pieces is charged when the second of its two pieces is
 *       planned.  Optimal within each piece.
 *   JA_PLAN_GREEDY: the same program with the repartition sub-cost removed,
 *       so each operator takes its cheapest join + aggregation (section 6,
 *       Experiment 3).
 *   JA_PLAN_RANDOM: one spec per operator, uniformly from `seed`.
 *   JA_PLAN_DEVICE: the same program and cuts with a compute-aware cost in
 *       place of the communication proxy (the computation awareness the
 *       pages leave as future work, section 8): a model, in microseconds, of
 *       this library's kernels on one MI355X -- a contraction as 256 x 256
 *       output tiles, each costing its segment's contracted extent at the
 *       measured per-CU rate of the fused bf16 contraction, placed longest
 *       first on the least loaded of 256 CUs; attention as 128-query-row
 *       tiles costed by the keys they see at the measured attention rate;
 *       RMSNorm, SwiGLU, add and every repartition as their bytes at the
 *       measured copy rate; 4 us per launch.  See ja_graph_device_time.
 * Ties go to the first candidate in lexicographic order of the interval
 * counts (letter order).  Host only. */
#define JA_PLAN_OPTIMAL 0
#define JA_PLAN_GREEDY 1
#define JA_PLAN_RANDOM 2
#define JA_PLAN_DEVICE 3
typedef struct ja_graph ja_graph;
ja_status ja_graph_create(ja_graph** out);
void ja_graph_destroy(ja_graph* graph);
/* A computation input of the given shape; writes its tensor id. */
ja_status ja_graph_add_input(ja_graph* graph, int32_t rank, const int64_t* shape, int32_t* tensor);
/* Operator `spec` (copied) on tensors inputs[0..n_inputs), whose dimensions
 * bind the spec's input letters in order; writes the output tensor's id.
 * JA_ERR_SHAPE when a letter gets two extents or a rank differs;
 * JA_ERR_UNSUPPORTED for packed-sequence attention and for the contractions
 * with an epilogue (contract_add, contract_swiglu). */
ja_status ja_graph_add_op(ja_graph* graph, const ja_spec* spec, const int32_t* inputs, int32_t n_inputs,
                          int32_t* tensor);
/* A view of `tensor` (a computation input or an operator output, not itself
 * a view): the tensor re-indexed by `view` (ja_repartition's reshape and
 * permutation) and read as shape[0..rank), with the same element count
 * (JA_ERR_SHAPE otherwise); writes its tensor id.  It is realised by a
 * repartition through the view into whatever blocking each consumer's spec
 * asks for, so it constrains neither its source's nor its consumers' tilings,
 * and every edge out of it is charged as one repartition: all its elements
 * in the proxy, one copy launch in the device model.  (A view is how
 * token-major projections feed head-major attention, and back.) */
ja_status ja_graph_add_view(ja_graph* graph, int32_t tensor, const ja_view* view, int32_t rank, const int64_t* shape,
                            int32_t* out);
ja_status ja_graph_count(const ja_graph* graph, int32_t* n_ops, int32_t* n_tensors);
/* Choose a spec for every operator (mode above); *cost (may be NULL) gets
 * the chosen plan's total proxy cost (JA_PLAN_DEVICE: its modelled time in
 * microseconds).  JA_ERR_UNSUPPORTED when an operator has no candidate with
 * p function specifications. */
ja_status ja_graph_plan(ja_graph* graph, int32_t p, int32_t mode, uint64_t seed, double* cost);
/* The chosen interval counts of operator `op` in its spec's letter order
 * (cap >= number of letters).  JA_ERR_STATE before ja_graph_plan. */
ja_status ja_graph_plan_intervals(const ja_graph* graph, int32_t op, int32_t* intervals, int32_t cap);
/* The proxy's three sub-costs for a full assignment: intervals[op] holds the
 * interval counts of operator op (letter order); intervals == NULL costs the
 * planned assignment. */
ja_status ja_graph_cost(const ja_graph* graph, const int32_t* const* intervals, double* repart, double* join,
                        double* agg);
/* The device-time model (JA_PLAN_DEVICE) of a full assignment, in
 * microseconds: every operator's modelled kernel time plus, on every edge
 * whose tilings differ, one repartition launch copying the tensor once
 * (computation inputs are free).  intervals as for ja_graph_cost. */
ja_status ja_graph_device_time(const ja_graph* graph, const int32_t* const* intervals, double* us);

/* ---- plans: join + fused kernel + aggregation + recompose -------------- */

/* Validate the relations against the spec and decomposition (each input and
 * the output must be blocked exactly as the decomposition cuts their letters;
 * dtypes: contract f32 x f32 -> f32, bf16 x bf16 -> bf16 / f32 or
 * f16 x f16 -> f16 / f32, accumulating in f32; attention, rmsnorm, swiglu,
 * add: every relation bf16, or every relation f16 -- JA_ERR_DTYPE
 * otherwise), run the join, and build the device tables.  16-bit outputs are
 * rounded to nearest even once from f32.  A 16-bit contraction needs block
 * extents along every contiguous axis that are multiples of 8 and operand
 * matrices (one batch entry of an operand block) of fewer than 2^30 elements,
 * which its kernel addresses with 32-bit byte offsets (JA_ERR_UNSUPPORTED
 * otherwise). */
ja_status ja_plan_create(const ja_spec* spec, const ja_decomp* decomp, const ja_relation_desc* const* in,
                         int32_t n_in, const ja_relation_desc* out, ja_plan** plan);
/* table_bytes: device buffer size for ja_plan_upload; workspace_bytes: the
 * workspace ja_plan_run needs (may be 0; bf16 attention: 16 bytes per query
 * tile of 128 rows). */
ja_status ja_plan_device_bytes(const ja_plan* plan, size_t* table_bytes, size_t* workspace_bytes);
/* Copy the plan's tables to dev_buf (at least table_bytes) on `stream` and
 * wait for the copy.  The buffer must stay alive while the plan is run. */
ja_status ja_plan_upload(ja_plan* plan, void* dev_buf, size_t bytes, void* stream);
/* Run the whole join-agg: every tuple's kernel with the aggregation fused
 * into it, writing each output block exactly once (recompose in place).
 * in_ptrs[i] / out_ptr: device buffers of the relations given at create;
 * workspace: workspace_bytes of device scratch, 16-byte aligned (NULL while
 * that is 0; JA_ERR_WORKSPACE when it is needed and NULL), overwritten by
 * the run, so two runs that share it must not overlap.
 * Attention rounds V to fp16 for its P V product; with bf16 relations a
 * query tile whose accumulators show V outside fp16's range (a value that is
 * not finite, or outputs averaging below 2^-12) is computed again, by a
 * second launch, with V multiplied by a power of two chosen from the largest
 * exponent among the V rows it reads and O divided by it, so every finite
 * bf16 V is in range. */
ja_status ja_plan_run(const ja_plan* plan, const void* const* in_ptrs, void* out_ptr, void* workspace,
                      void* stream);
/* Unfused path (section 3.2, Definition 3.7, with the join's per-tuple
 * results materialised): ja_kernel writes every tuple's partial result in
 * float32 to `partials` (ja_plan_partial_bytes bytes; tuple i's part starts
 * after the parts of tuples 0..i-1); ja_agg folds each segment's partials in
 * ascending tuple order with `op` and writes the output relation.
 *   contract (no epilogue): a tuple's part is its dense row-major partial
 *     output block; op JA_AGG_SUM (the contraction) or JA_AGG_MAX.
 *   attention (every batch and group letter before s; JA_ERR_UNSUPPORTED
 *     otherwise): a tuple's part holds, per query row of its query block (rows
 *     in the O block's order: batch-heads, then s), 132 floats [m, l, -, -,
 *     acc[128]]: over the keys of the tuple's key block the row may see,
 *     m = max of scale q.k (or a value below it: the triple is only defined
 *     up to the shift (m, l, acc) ~ (m', l e^(m-m'), acc e^(m-m'))),
 *     l = sum of exp(scale q.k - m), acc = sum of exp(scale q.k - m) v; a
 *     row that sees none of them gets (-inf, 0, 0).  op JA_AGG_SOFTMAX.
 *     With bf16 relations ja_plan_partial_bytes also counts 16 bytes per
 *     query tile of scratch after the parts (the range check of ja_plan_run).
 * Other operators and contractions with an epilogue: JA_ERR_UNSUPPORTED;
 * an op that does not match the operator: JA_ERR_UNSUPPORTED. */
ja_status ja_plan_partial_bytes(const ja_plan* plan, size_t* bytes);
ja_status ja_kernel(const ja_plan* plan, const void* const* in_ptrs, void* partials, void* stream);
ja_status ja_agg(const ja_plan* plan, ja_agg_op op, const void* partials, void* out_ptr, void* stream);
void ja_plan_destroy(ja_plan* plan);

/* One-shot convenience: create a plan, upload its tables into dev_ws, run,
 * and destroy the plan.  Blocks until the table upload is done; the run
 * itself stays asynchronous.  ws_bytes must be at least the value returned
 * by ja_einsum_workspace_bytes. */
ja_status ja_einsum_workspace_bytes(const ja_spec* spec, const ja_decomp* decomp, const ja_relation_desc* const* in,
                                    int32_t n_in, const ja_relation_desc* out, size_t* bytes);
ja_status ja_einsum(const ja_spec* spec, const ja_decomp* decomp, const ja_relation_desc* const* in,
                    const void* const* in_ptrs, int32_t n_in, const ja_relation_desc* out, void* out_ptr,
                    void* dev_ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under stream
 * loops, harnesses that forbid hipMalloc): ja_einsum
 * with the plan tables and the run's scratch in a static device array of
 * JA_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until the
 * process ends, instead of a caller workspace.  The caller passes inputs and
 * outputs only.  JA_ERR_WORKSPACE (before any HIP call) when the plan needs
 * more than the array holds -- ja_einsum_workspace_bytes gives the need --
 * otherwise the errors of ja_einsum.  Blocks until the table upload is done;
 * the run stays asynchronous on `stream` (the upload synchronises the stream, so a
 * call cannot be recorded into a stream capture).  No device memory is allocated or
 * freed.  Every call on a GPU shares that GPU's array: calls that overlap on
 * one GPU (other streams, other host threads) race; calls in order on one
 * stream do not. */
#define JA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
ja_status ja_einsum_noalloc(const ja_spec* spec, const ja_decomp* decomp, const ja_relation_desc* const* in,
                            const void* const* in_ptrs, int32_t n_in, const ja_relation_desc* out, void* out_ptr,
                            void* stream);

/* ---- repartition (section 4.3 repartition cost; section 5.3 atoms) ----- */

/* Plan the re-blocking of `src` into `dst`, optionally through `view` (NULL:
 * identity; then the shapes must be equal).  Both relations must have the
 * same dtype.  The plan's atoms are the cells of the overlay of both
 * blockings, refined so that every atom is a box in both; every destination
 * element is written exactly once, by a copy of its source bytes.  The
 * reshapes of the view must factor into common sub-dimensions
 * (JA_ERR_UNSUPPORTED otherwise). */
ja_status ja_repart_create(const ja_relation_desc* src, const ja_relation_desc* dst, const ja_view* view,
                           ja_repart** out);
/* n_atoms: overlay cells; n_tasks: device copy tasks (atoms, possibly cut
 * into chunks). */
ja_status ja_repart_count(const ja_repart* rp, int64_t* n_atoms, int64_t* n_tasks);
ja_status ja_repart_device_bytes(const ja_repart* rp, size_t* table_bytes);
ja_status ja_repart_upload(ja_repart* rp, void* dev_buf, size_t bytes, void* stream);
ja_status ja_repart_run(const ja_repart* rp, const void* src_ptr, void* dst_ptr, void* stream);
void ja_repart_destroy(ja_repart* rp);
/* One-shot convenience (create, upload into dev_ws, run, destroy). */
ja_status ja_repartition_workspace_bytes(const ja_relation_desc* src, const ja_relation_desc* dst,
                                         const ja_view* view, size_t* bytes);
ja_status ja_repartition(const ja_relation_desc* src, const void* src_ptr, const ja_relation_desc* dst,
                         void* dst_ptr, const ja_view* view, void* dev_ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* JA_H */
