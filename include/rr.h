/*
 * rr.h -- collective reductions over p virtual ranks resident in one GPU's HBM.
 *
 * C ABI of librr.so (AMD Instinct MI355X, gfx950).  A "virtual rank" r is a
 * device buffer; one call performs the whole collective for all p ranks, so
 * each entry point takes arrays of p rank buffers where a per-process API
 * (torch.distributed, MPI) takes one.
 *
 * Sources (web pages, cited by title and section):
 *   [SEM]  page "分布式训练/推理" (llm-from-scratch, chapter 7), section
 *          "通信原语：rank、world size 和 collective operations": the semantics
 *          table of the primitives, y = sum_{r=0}^{p-1} x_r, the worked example
 *          x_r = [0,1,2,3] + r (p = 4), all_reduce = reduce_scatter + all_gather;
 *          section "PyTorch distributed": all-reduce works in place,
 *          reduce-scatter writes a separate, p times smaller output.
 *   [RING] page "LLM Parallelism 基础", section "Ring AllReduce": N chunks,
 *          reduce-scatter phase then all-gather phase, 2(N-1) steps, each
 *          rank passes one chunk per step to the next rank on the ring; the
 *          receiver accumulates (phase 1) or overwrites (phase 2); rank c ends
 *          phase 1 holding the reduced chunk c.  Section "MPI Collective
 *          Operations": reduce, broadcast; all-reduce has the effect of a
 *          reduce followed by a broadcast.
 *   [HIER] page "大模型并行的最小闭环：集合通信、TP、FSDP/ZeRO-3 到权重分片",
 *          section "Source Log: 2026-05-05" (hierarchical AllReduce + SHARP,
 *          steps 1-6 and the traffic comparison).
 *   [DP]   page "分布式训练/推理", data-parallel section: the gradient is
 *          averaged over the p ranks, g = (1/p) sum_r grad L_r, by an
 *          all-reduce with the AVG op (or SUM followed by a division by the
 *          world size); the gradients are synchronised in flattened buckets.
 *   [TP]   page "分布式训练/推理", tensor-parallel section: column-parallel
 *          outputs [B, d/p] are all-gathered and concatenated along dim 1;
 *          in the scatter strategy each rank's partial [B, D] output is
 *          summed over ranks and cut into feature slices (psum_scatter).
 *   [MPI]  page "LLM Parallelism 基础", table of MPI collectives: scatter
 *          (the root cuts its array into p pieces, one per process) and
 *          gather (every process's piece collected at the root).
 *
 * Conventions common to every entry point
 * ----------------------------------------
 *  - p: number of virtual ranks, 1 <= p <= RR_MAX_RANKS.
 *  - n: ALWAYS the full per-rank vector length in elements (for
 *    reduce-scatter and all-gather the shard length is n / p).
 *  - Buffers are device pointers owned by the caller; rank arrays
 *    (sendbufs, recvbufs) are host arrays of p device pointers, read only
 *    during the call and passed to the kernels by value (no device-side
 *    table, no host-to-device copy, no device allocation on these paths).
 *  - Every pointer must be aligned to its element size.  16-byte alignment of
 *    every buffer selects the 128-bit vector path; otherwise a scalar path
 *    with the same arithmetic order runs, so results are identical.
 *  - Arithmetic: int32 sums wrap modulo 2^32; float32 sums are IEEE-754
 *    round-to-nearest-even additions; bfloat16 and float16 (IEEE binary16)
 *    inputs are widened exactly to float32, folded in float32 and rounded
 *    once to their type (nearest even; float16 results below 2^-14 become
 *    binary16 subnormals and magnitudes that round to 2^16 or more become
 *    +-inf; a NaN stays NaN, sign kept, made quiet); denormals are kept (no
 *    flush).  RR_AVG [DP] folds like RR_SUM, in the same order, then divides
 *    the float32 accumulator by p (one IEEE division, nearest even) before
 *    the one conversion; it is defined for the float dtypes only (int32 ->
 *    RR_ERROR_UNSUPPORTED).
 *    max/min are compare-and-select with the running value first: it is
 *    replaced only by a strictly greater (max) / strictly smaller (min)
 *    value, so ties (+0 vs -0) keep the earlier operand, a NaN running value
 *    stays and a NaN new value is skipped.
 *  - Fold orders (they decide float results bit for bit):
 *      ring all-reduce and reduce-scatter: element i of chunk c is folded as
 *        x_{c+1}, x_{c+2}, ..., x_{c+p-1}, x_c (indices mod p) -- the order in
 *        which the ring's reduce-scatter phase accumulates chunk c when every
 *        rank sends to rank r+1 [RING];
 *      reduce: x_0, x_1, ..., x_{p-1} (the order of the sum in [SEM]);
 *      hierarchical: ascending inside each group, then ascending over groups.
 *    Chunk c of a rank's vector is [floor(c*n/p), floor((c+1)*n/p)).
 *  - Asynchrony: every call validates on the host, enqueues its kernels on
 *    `stream` (NULL = the null stream of the current device) and returns.
 *    The library never synchronizes.  Completion is observed through the
 *    stream.  Buffers must stay valid until the work completes.
 *  - Graph capture: every call may be captured into a HIP graph (no
 *    allocation, no memset, no synchronization on the call path; call once
 *    before capturing, so that per-kernel set-up stays out of the graph).  A
 *    graph replays its launch arguments unchanged, so launches that keep
 *    per-launch state in device memory (the soft barrier of the multi-round
 *    fused fold, the step flags of RR_ALGO_RING_PERSISTENT) detect capture,
 *    take a fixed tag, and capture a reset of that state just before
 *    themselves.  The executor's flags order data, so each captured
 *    executor launch owns a slot of flags (see RR_ALGO_RING_PERSISTENT); the
 *    barrier's counters order nothing and are kept per capturing stream
 *    (sharing them only costs time).
 *  - Errors: return codes only.  All validation happens before the first
 *    launch, so a call that returns RR_ERROR_INVALID_ARGUMENT or
 *    RR_ERROR_UNSUPPORTED has written nothing.  A launch failure returns
 *    RR_ERROR_HIP; asynchronous faults surface on the stream's next sync.
 *    rr_last_error() gives a message for the calling thread's last failure.
 *  - n == 0 is a valid no-op (RR_SUCCESS, nothing launched) once p, dtype,
 *    op and the rank arrays are valid.
 *  - Aliasing: output buffers must not overlap each other or any input,
 *    except the exact in-place forms named per entry point.  Input buffers
 *    may alias each other (they are only read).
 *  - Calls on different streams that write the same buffers race; calls on
 *    one stream are ordered.
 */
#ifndef RR_H
#define RR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RR_MAX_RANKS 64

/* Opaque HIP stream handle (the same type as hipStream_t). */
typedef struct ihipStream_t* rr_stream_t;

typedef enum { RR_INT32 = 0, RR_FLOAT32 = 1, RR_BFLOAT16 = 2, RR_FLOAT16 = 3 } rr_dtype_t;

typedef enum { RR_SUM = 0, RR_MAX = 1, RR_MIN = 2, RR_AVG = 3 } rr_op_t;

typedef enum {
  RR_SUCCESS = 0,
  RR_ERROR_INVALID_ARGUMENT = 1,
  RR_ERROR_UNSUPPORTED = 2,
  RR_ERROR_HIP = 3
} rr_status_t;

typedef enum {
  RR_ALGO_RING_FUSED = 0,  /* one pass: ring-order fold of each chunk, all p outputs written */
  RR_ALGO_RING_STAGED = 1, /* the ring schedule executed step by step: 2(p-1) launches */
  RR_ALGO_HIER_FUSED = 2,  /* one pass: group folds, cross-group fold, all p outputs written */
  RR_ALGO_HIER_STAGED = 3, /* group reduce to the representative, cross-group reduce, broadcast */
  RR_ALGO_RING_PERSISTENT = 4 /* the ring schedule in one persistent kernel with per-step flags */
} rr_algo_t;

typedef enum {
  RR_COLL_ALL_REDUCE = 0,
  RR_COLL_REDUCE_SCATTER = 1,
  RR_COLL_ALL_GATHER = 2,
  RR_COLL_REDUCE = 3,
  RR_COLL_BROADCAST = 4,
  RR_COLL_SCATTER = 5,
  RR_COLL_GATHER = 6
} rr_coll_t;

/*
 * All-reduce [SEM] [RING]: every rank receives y = x_0 (+) x_1 (+) ... (+) x_{p-1}.
 *   sendbufs[r]: rank r's input, n elements.   recvbufs[r]: rank r's output, n
 *   elements.  In place allowed: recvbufs[r] == sendbufs[r] (for every r or
 *   for some r).  Fold order: ring order per chunk (see above); equivalent to
 *   the ring's reduce-scatter followed by its all-gather, fused into one pass
 *   that reads every input once and writes every output once.
 *   Any n is accepted (chunk bounds floor(c*n/p)).
 *   Returns RR_ERROR_INVALID_ARGUMENT for: p out of range, NULL arrays or
 *   buffers, misaligned buffers, overlapping outputs; RR_ERROR_UNSUPPORTED for
 *   an unknown dtype or op.
 */
rr_status_t rr_all_reduce(const void* const* sendbufs, void* const* recvbufs, int p, size_t n,
                          rr_dtype_t dtype, rr_op_t op, rr_stream_t stream);

/*
 * All-reduce with an explicit algorithm.
 *   algo = RR_ALGO_RING_FUSED: same as rr_all_reduce (group_size and workspace ignored).
 *   algo = RR_ALGO_RING_STAGED: the ring schedule of [RING] run literally, one
 *     launch per step (2(p-1) steps): reduce-scatter step s moves chunk
 *     (r-1-s) mod p from rank r to rank r+1 and the receiver stores
 *     message (+) local; all-gather step s moves chunk (r-s) mod p and the
 *     receiver overwrites.  Any n (the chunk bounds above).  For bfloat16 and
 *     float16 the partial sums live in a float32 workspace of
 *     rr_workspace_size() bytes, filled from the inputs first (one rounding
 *     at the end); int32/float32 work in recvbufs, need no workspace and read
 *     each not yet written value from sendbufs (no copy of the inputs into
 *     recvbufs first; recvbufs are written before they are read).  RR_AVG:
 *     the owner of each reduced chunk divides it by p before the all-gather
 *     phase.  Bitwise equal to RR_ALGO_RING_FUSED.
 *   algo = RR_ALGO_HIER_FUSED [HIER]: ranks form p/group_size contiguous groups
 *     [j*G, (j+1)*G) whose representative is rank j*G.  Each group's inputs are
 *     folded ascending in the accumulator type, the group partials are folded
 *     ascending over groups (no rounding in between), converted once, and
 *     written to every rank.  One pass; no workspace.
 *   algo = RR_ALGO_HIER_STAGED: the same arithmetic in the steps of [HIER]:
 *     (1) each group reduces into an accumulator-type workspace slot of its
 *     representative, (2-5) the representatives' partials are folded across
 *     groups and the result written to every representative's recvbuf,
 *     (6) each representative's result is broadcast inside its group.  Needs
 *     rr_workspace_size() bytes of workspace.  Bitwise equal to HIER_FUSED.
 *   algo = RR_ALGO_RING_PERSISTENT [RING]: the same schedule and arithmetic
 *     as RR_ALGO_RING_STAGED in ONE launch: every chunk is cut into slices
 *     and a workgroup per (slice, rank) performs that rank's side of every
 *     step for its slice, waiting on device-side completion flags of its
 *     ring neighbours (bounded waits) instead of on launch boundaries.
 *     Workspace as RR_ALGO_RING_STAGED.  Bitwise equal to RR_ALGO_RING_FUSED.
 *     If a wait runs out (the workgroups were not all resident, e.g. other
 *     kernels filled the GPU), the launch stops and its outputs are
 *     incomplete; rr_ring_exec_failures() counts such launches.  Its step
 *     flags come in slots.  An eager launch uses its stream's slot, one of
 *     16 per device: a stream keeps its slot while it has one, and every
 *     call that is not being captured frees the slots whose last launch has
 *     completed.  A launch captured into a graph takes a slot of its own,
 *     one of 48 more per device, and keeps it for the rest of the process,
 *     so that two captured launches never share flags (graphs captured on
 *     one stream may be replayed concurrently on different streams); one
 *     graph must not be replayed while an earlier replay of the same graph is
 *     still running.  A call that finds no free slot returns RR_ERROR_HIP.
 *   group_size: 1 <= group_size <= p and group_size | p (HIER algos only).
 *   workspace: device memory of at least rr_workspace_size(algo, ...) bytes,
 *     16-byte aligned, owned by the caller, not aliasing any buffer; may be
 *     NULL when that size is 0.
 *   Returns RR_ERROR_INVALID_ARGUMENT additionally for an unknown algo, a bad
 *   group_size, or a missing, short, misaligned or overlapping workspace.
 */
rr_status_t rr_all_reduce_ex(const void* const* sendbufs, void* const* recvbufs, int p, size_t n,
                             rr_dtype_t dtype, rr_op_t op, rr_algo_t algo, int group_size,
                             void* workspace, size_t workspace_bytes, rr_stream_t stream);

/* Bytes of the library's fixed device scratch used by rr_all_reduce_ex_noalloc. */
#define RR_NOALLOC_SCRATCH_BYTES (64ull << 20)

/*
 * rr_all_reduce_ex without a caller workspace, allocating nothing: for
 * callers that cannot allocate device memory at the call (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, results and errors as rr_all_reduce_ex, except that the
 * workspace of the staged algorithms is a fixed array of
 * RR_NOALLOC_SCRATCH_BYTES in the library's device memory, which each GPU the
 * library runs on holds until the process ends.  The call makes no
 * allocation of any kind (no hipMalloc, no allocating library routine).
 *   algo: RR_ALGO_RING_FUSED and RR_ALGO_HIER_FUSED need no workspace and
 *     behave exactly as in rr_all_reduce_ex; RR_ALGO_RING_STAGED and
 *     RR_ALGO_HIER_STAGED use the scratch for what rr_workspace_size()
 *     reports; RR_ALGO_RING_PERSISTENT -> RR_ERROR_UNSUPPORTED (its first
 *     launch on a stream creates a completion event).
 *   Returns RR_ERROR_INVALID_ARGUMENT, writing nothing, when
 *   rr_workspace_size(algo, p, group_size, n, dtype) exceeds
 *   RR_NOALLOC_SCRATCH_BYTES.
 *   Every call on a GPU shares that GPU's scratch, which keeps the last
 *   call's contents (the staged algorithms write every workspace element
 *   before reading it, so nothing needs clearing).  Calls that overlap in
 *   time on one GPU -- on different streams, or from different host threads
 *   without ordering -- race on the scratch and give undefined results;
 *   calls on one stream are ordered and safe.
 */
rr_status_t rr_all_reduce_ex_noalloc(const void* const* sendbufs, void* const* recvbufs, int p, size_t n,
                                     rr_dtype_t dtype, rr_op_t op, rr_algo_t algo, int group_size,
                                     rr_stream_t stream);

/* Variant bits of rr_all_reduce_hier [HIER]. */
#define RR_HIER_INTRA_RING 1 /* step 1 as a ring all-reduce inside each group */
#define RR_HIER_WIRE_ROUND 2 /* group partials rounded to the storage type before crossing groups */
#define RR_HIER_STAGED 4     /* run the steps of [HIER] one by one (workspace needed) */

/*
 * Hierarchical all-reduce with the variants of [HIER] (groups of group_size
 * consecutive ranks, representative = the group's first rank).
 *   flags = 0: as rr_all_reduce_ex with RR_ALGO_HIER_FUSED (ascending fold
 *     inside each group, ascending over groups, float32 partials, one
 *     rounding).
 *   RR_HIER_INTRA_RING: step 1 as the page words it, an all-reduce inside
 *     each group run as a ring of its G members: group-chunk k of the n
 *     elements, [floor(k*n/G), floor((k+1)*n/G)), is folded over the members
 *     in the order (k+1) mod G, ..., k mod G; the group partials are then
 *     folded ascending over groups.  Not available with RR_HIER_STAGED
 *     (RR_ERROR_UNSUPPORTED).
 *   RR_HIER_WIRE_ROUND: each group's partial is rounded to the storage type
 *     (nearest even) and widened again before the cross-group fold -- what
 *     the representative ships across groups.  Changes results for bfloat16
 *     and float16 only.
 *   RR_HIER_STAGED: the steps of [HIER] one launch at a time through a
 *     caller workspace of rr_hier_workspace_size() bytes (as
 *     RR_ALGO_HIER_STAGED; with RR_HIER_WIRE_ROUND the partials are stored
 *     in the storage type).
 *   RR_AVG divides by p after the cross-group fold.  Other rules (aliasing,
 *   in place, errors) as rr_all_reduce_ex; unknown flag bits ->
 *   RR_ERROR_INVALID_ARGUMENT.
 */
rr_status_t rr_all_reduce_hier(const void* const* sendbufs, void* const* recvbufs, int p, size_t n,
                               rr_dtype_t dtype, rr_op_t op, int group_size, int flags, void* workspace,
                               size_t workspace_bytes, rr_stream_t stream);

/* Workspace bytes of rr_all_reduce_hier: 0 without RR_HIER_STAGED; else
 * (p/group_size) group partials of n*4 bytes, or n*s with
 * RR_HIER_WIRE_ROUND on a 16-bit dtype, each rounded up to a multiple of 16
 * bytes (every partial starts 16-byte aligned).  0 for invalid arguments. */
size_t rr_hier_workspace_size(int p, int group_size, size_t n, rr_dtype_t dtype, int flags);

/*
 * Reduce-scatter [SEM] [RING]: rank c receives chunk c of y.
 *   sendbufs[r]: rank r's input, n elements.  recvbufs[c]: n/p elements.
 *   Requires p | n.  Fold order: ring order (bitwise equal to chunk c of
 *   rr_all_reduce).  In place allowed: recvbufs[c] == sendbufs[c] + c*(n/p)
 *   elements (the slot of the rank's own chunk).
 */
rr_status_t rr_reduce_scatter(const void* const* sendbufs, void* const* recvbufs, int p, size_t n,
                              rr_dtype_t dtype, rr_op_t op, rr_stream_t stream);

/*
 * All-gather [SEM] [RING]: every rank receives the concatenation of the p
 * shards: recvbufs[r][c*(n/p) + j] = sendbufs[c][j].
 *   sendbufs[c]: n/p elements.  recvbufs[r]: n elements.  Requires p | n.
 *   In place allowed: sendbufs[c] == recvbufs[c] + c*(n/p) elements.
 *   A bit copy: the dtype only sets the element size.
 */
rr_status_t rr_all_gather(const void* const* sendbufs, void* const* recvbufs, int p, size_t n,
                          rr_dtype_t dtype, rr_stream_t stream);

/*
 * Reduce [SEM] [RING]: the root receives y, folded x_0, x_1, ..., x_{p-1}.
 *   sendbufs[r]: n elements.  recvbuf: the root's output, n elements.
 *   root: 0 <= root < p; in place allowed: recvbuf == sendbufs[root].
 */
rr_status_t rr_reduce(const void* const* sendbufs, void* recvbuf, int root, int p, size_t n,
                      rr_dtype_t dtype, rr_op_t op, rr_stream_t stream);

/*
 * Broadcast [SEM] [RING]: every rank receives a copy of the root's buffer.
 *   sendbuf: the root's input, n elements.  recvbufs[r]: n elements.
 *   root: 0 <= root < p; in place allowed: recvbufs[root] == sendbuf (that
 *   copy is skipped).  A bit copy: the dtype only sets the element size.
 */
rr_status_t rr_broadcast(const void* sendbuf, void* const* recvbufs, int root, int p, size_t n,
                         rr_dtype_t dtype, rr_stream_t stream);

/*
 * Scatter [MPI] [SEM]: rank c receives slice c of the root's buffer:
 * recvbufs[c][j] = sendbuf[c*(n/p) + j].
 *   sendbuf: the root's input, n elements.  recvbufs[c]: n/p elements.
 *   Requires p | n.  root: 0 <= root < p; in place allowed:
 *   recvbufs[root] == sendbuf + root*(n/p) elements (that copy is skipped).
 *   A bit copy: the dtype only sets the element size.
 */
rr_status_t rr_scatter(const void* sendbuf, void* const* recvbufs, int root, int p, size_t n,
                       rr_dtype_t dtype, rr_stream_t stream);

/*
 * Gather [MPI] [SEM]: the root receives the p slices in rank order:
 * recvbuf[c*(n/p) + j] = sendbufs[c][j].
 *   sendbufs[c]: n/p elements.  recvbuf: the root's output, n elements.
 *   Requires p | n.  root: 0 <= root < p; in place allowed:
 *   sendbufs[root] == recvbuf + root*(n/p) elements (that copy is skipped).
 */
rr_status_t rr_gather(const void* const* sendbufs, void* recvbuf, int root, int p, size_t n,
                      rr_dtype_t dtype, rr_stream_t stream);

/*
 * Bucketed all-reduce [DP]: one call all-reduces a bucket of ntensors tensors
 * per rank as if they were laid end to end in one buffer, without copying
 * them into one.
 *   sendbufs[t*p + r]: tensor t of rank r, counts[t] elements.
 *   recvbufs[t*p + r]: its output, counts[t] elements.  In place allowed:
 *   recvbufs[i] == sendbufs[i] (for any i).
 *   The bucket of rank r is the concatenation of its tensors 0..ntensors-1
 *   (N = sum of counts elements); its chunk c is [floor(c*N/p),
 *   floor((c+1)*N/p)) and every element is folded in the ring order of its
 *   bucket chunk, so the result is bitwise that of rr_all_reduce on the
 *   concatenated bucket.  Tensors with counts[t] == 0 are skipped (their
 *   pointers are not read).  Tensors whose 2p pointers are all 16-byte
 *   aligned take the 128-bit path inside each chunk; the rest move element
 *   by element (same results).  The host tables are read during the call
 *   only.  One launch serves up to 96 runs of up to 192/(2p) tensors; longer
 *   lists take more launches, all on `stream`.
 *   Returns RR_ERROR_INVALID_ARGUMENT for a negative ntensors, NULL tables,
 *   NULL or misaligned buffers of non-empty tensors, overlapping outputs or
 *   an output overlapping any input other than its own exact in-place form,
 *   a bucket over 2^56 elements; RR_ERROR_UNSUPPORTED for an unknown dtype or
 *   op and for RR_AVG on int32.
 */
rr_status_t rr_all_reduce_bucket(const void* const* sendbufs, void* const* recvbufs, const size_t* counts,
                                 int ntensors, int p, rr_dtype_t dtype, rr_op_t op, rr_stream_t stream);

/*
 * All-gather along dim 1 [TP]: every rank receives the row-major
 * [rows, cols] matrix whose column block c (columns [c*w, (c+1)*w),
 * w = cols/p) is rank c's row-major [rows, w] matrix:
 * recvbufs[r][b*cols + c*w + j] = sendbufs[c][b*w + j].
 *   Requires p | cols.  No in-place form (outputs must not overlap inputs).
 *   A bit copy: the dtype only sets the element size; 16-byte units when
 *   every address and w*s allow, else 4-, 2- or 1-byte units.
 */
rr_status_t rr_all_gather_dim1(const void* const* sendbufs, void* const* recvbufs, int p, size_t rows,
                               size_t cols, rr_dtype_t dtype, rr_stream_t stream);

/*
 * Reduce-scatter along dim 1 [TP] (psum_scatter of partial outputs): rank c
 * receives the row-major [rows, w] feature slice c (w = cols/p) of the
 * reduction of the p row-major [rows, cols] inputs:
 * recvbufs[c][b*w + j] = x_{c+1} (+) x_{c+2} (+) ... (+) x_c at
 * [b, c*w + j] (ring order of chunk c of the feature dimension; AVG divides
 * by p after the fold).
 *   Requires p | cols.  No in-place form.  The 128-bit path needs every
 *   buffer 16-byte aligned and w*s a multiple of 16 bytes; otherwise the
 *   element path runs with the same results.
 */
rr_status_t rr_reduce_scatter_dim1(const void* const* sendbufs, void* const* recvbufs, int p, size_t rows,
                                   size_t cols, rr_dtype_t dtype, rr_op_t op, rr_stream_t stream);

/*
 * Workspace bytes that rr_all_reduce_ex needs for (algo, p, group_size, n,
 * dtype): 0 for the fused algorithms and for the staged ring on int32/float32;
 * p*n*4 for the staged ring on bfloat16 and float16; (p/group_size) times
 * n*4 rounded up to a multiple of 16 for the staged hierarchy.  Returns 0 for
 * invalid arguments as well (rr_all_reduce_ex then reports them).
 */
size_t rr_workspace_size(rr_algo_t algo, int p, int group_size, size_t n, rr_dtype_t dtype);

/*
 * The ring schedule of [RING] as a transfer list (host only; no GPU needed).
 * Writes at most `cap` transfers, in execution order, into the caller's
 * arrays: phase (0 = reduce-scatter: the receiver accumulates, 1 = all-gather:
 * the receiver overwrites), step within the phase, source rank, destination
 * rank (= source + 1 mod p) and chunk index.  Returns the total number of
 * transfers, 2(p-1)p, or -1 for p out of range.  Any array may be NULL when
 * cap is 0 (query the count).
 */
int rr_ring_schedule(int p, int* phase, int* step, int* src, int* dst, int* chunk, int cap);

/* Chunk bounds (host only): bounds[c] = floor(c*n/p) for c = 0..p (p+1 values). */
rr_status_t rr_chunk_bounds(int p, size_t n, size_t* bounds);

/*
 * Algorithmic HBM bytes of one call (host only): each input element read once
 * and each output element written once.  all-reduce 2pns; reduce-scatter,
 * all-gather and reduce (p+1)ns; broadcast ns + p*ns, or ns + (p-1)ns when the
 * root's copy is in place (in_place != 0).  s = element size.
 */
rr_status_t rr_algorithmic_bytes(rr_coll_t coll, int p, size_t n, rr_dtype_t dtype, int in_place,
                                 uint64_t* bytes);

/*
 * Bytes moved by the ring schedule per rank (host only), from the transfer
 * list: sent_rs and sent_ag are the bytes one rank sends in each phase (each
 * (p-1)/p of the rank's n*s bytes when p | n, the ring cost model of page
 * "分布式训练/推理", section "Ring all-reduce 的带宽账").  max over ranks.
 */
rr_status_t rr_ring_bytes_per_rank(int p, size_t n, rr_dtype_t dtype, uint64_t* sent_rs,
                                   uint64_t* sent_ag);

/*
 * Per-level traffic of a hierarchical all-reduce of `bytes_per_rank` bytes
 * over p ranks in groups of group_size (host only), counting what [HIER]
 * counts: intra_per_group = bytes the group's own all-reduce moves in step 1
 * (group_size * bytes_per_rank); cross_per_group_flat = bytes a group sends
 * across groups when every member ships its own buffer (group_size *
 * bytes_per_rank); cross_per_group_hier = bytes a group sends across groups
 * when only its representative ships the group's result (bytes_per_rank).
 */
rr_status_t rr_hier_traffic(int p, int group_size, uint64_t bytes_per_rank, uint64_t* intra_per_group,
                            uint64_t* cross_per_group_flat, uint64_t* cross_per_group_hier);

/*
 * Alpha-beta cost model (host only) [COST]: page "分布式训练/推理", section
 * "从单卡到多卡" -- one message costs its fixed latency plus its bytes over
 * the link bandwidth, T = alpha + bytes/bandwidth; section "Ring all-reduce
 * 的带宽账" -- a ring all-reduce is 2(N-1) rounds in which every device sends
 * S/N bytes; page "大模型并行的最小闭环：集合通信、TP、FSDP/ZeRO-3 到权重分片",
 * section "总体时间模型" -- without the hierarchy a node ships B*N bytes over
 * the slow links, T = T_slow(B*N); with it T = T_fast(B*N) + T_slow(B).
 */
typedef struct {
  double alpha_s;     /* fixed cost of one message, seconds */
  double bytes_per_s; /* link bandwidth, bytes per second (> 0) */
} rr_link_t;

/* Ring all-reduce of `bytes` per rank over p ranks on one link class:
 * 2(p-1) * (alpha + bytes/(p*bandwidth)) seconds (0 for p = 1). */
rr_status_t rr_cost_ring_all_reduce(int p, double bytes, rr_link_t link, double* seconds);

/* The hierarchy's time model for groups (nodes) of group_size ranks holding
 * `bytes` each: *t_flat = T_slow(group_size*bytes), *t_hier =
 * T_fast(group_size*bytes) + T_slow(bytes), T_x(m) = alpha_x + m/bandwidth_x;
 * *use_hier = 1 when t_hier < t_flat.  Any output pointer may be NULL. */
rr_status_t rr_cost_hier_all_reduce(int group_size, double bytes, rr_link_t fast, rr_link_t slow, double* t_flat,
                                    double* t_hier, int* use_hier);

/*
 * Diagnostics (needs a GPU; synchronizes the device): the number of times,
 * since the library was loaded, that a workgroup of a fused fold on `device`
 * stopped waiting at the soft barrier between the read phase and the write
 * phase of a round because its bounded wait ran out.  That barrier only
 * shapes the HBM traffic (no result depends on it), so a nonzero count means
 * lost throughput, never wrong results; it grows when the grid's workgroups
 * are not all resident at once (other kernels occupying the GPU).
 * Returns RR_ERROR_INVALID_ARGUMENT for a NULL count or a bad device.
 */
rr_status_t rr_barrier_timeouts(int device, uint64_t* count);

/*
 * Diagnostics (needs a GPU; synchronizes the device): the number of
 * RR_ALGO_RING_PERSISTENT launches on `device` that stopped because a wait
 * on a neighbour's step flag ran out (their outputs are incomplete) since the
 * library was loaded.  Returns RR_ERROR_INVALID_ARGUMENT for a NULL count or
 * a bad device.
 */
rr_status_t rr_ring_exec_failures(int device, uint64_t* count);

/*
 * Tuning knobs (RR_* environment variables: tile depths, workgroups per
 * compute unit, barrier and wait bounds, store policies, launch logging) are
 * read from the environment once per process, at the first call of any entry
 * point, never on the call path.  rr_reload_tuning() reads them again; calls
 * that start after it returns use the new values (calls already in progress
 * on other threads finish with the old ones).  No result depends on a knob:
 * they select among schedules that compute the same bits.
 */
void rr_reload_tuning(void);

/* Static description of a status code. */
const char* rr_status_string(rr_status_t status);

/* Message describing the calling thread's most recent failed call ("" if none). */
const char* rr_last_error(void);

/* Library version string. */
const char* rr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RR_H */
