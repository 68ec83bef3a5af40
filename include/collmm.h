/*
 * libcollmm -- tensor-parallel AllGather->GEMM and GEMM->ReduceScatter,
 * decomposed into per-shard partial GEMMs that overlap with ring hops,
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (cited by page title and section):
 *   - "Hiding Tensor-Parallel Collectives: AG/RS Overlap in Megatron",
 *     sections 3 (P2P AllGather overlap), 5 (P2P ReduceScatter overlap),
 *     6 (pipeline-chunk ReduceScatter), 8 (dependency classes) and 9 (what a
 *     trace should show).
 *   - "Overlap Communication with Dependent Computation via Decomposition in
 *     Large Deep Learning Models", sections "The idea" (AllGather->Einsum with
 *     a slice-update of each partial result; Einsum->ReduceScatter with a
 *     circulating accumulator; asynchronous transfer start/done pairs;
 *     bidirectional rings; a cost model that can decline) and "What it costs"
 *     (the pre-shift and realigning addition of bidirectional rings).
 *
 * Emulation model.  An N-rank tensor-parallel group is emulated on ONE GPU:
 * every virtual rank's shards, weights, receive slots and buckets are
 * regions of buffers in that GPU's memory.  A ring hop ("send to one
 * neighbour, receive from the other") is an asynchronous device-to-device
 * copy on a communication stream, executed by the SDMA copy engines
 * (hipMemcpyDeviceToDeviceNoCU), ordered against the compute stream with
 * events.  The partial GEMMs of all N ranks for one step are one kernel
 * launch on the compute stream.
 *
 * Layouts (all row-major, C order; "bf16" = IEEE binary32 upper half):
 *   AllGather->GEMM  (column-parallel linear; T = N*m tokens)
 *     x  [N][m][k]     bf16   rank r's sequence shard X_r
 *     w  [N][n][k]     bf16   W_r, one output feature per row (k contiguous)
 *     y  [N][T][n]     out    Y_r = concat_r(X_r) . W_r^T
 *   GEMM->ReduceScatter  (row-parallel linear)
 *     x  [N][T][k]     bf16   H_r, rank r's activation for all T tokens
 *     w  [N][n][k]     bf16   W_r, one output feature per row
 *     y  [N][m][n]     out    Out_q = sum_r (H_r . W_r^T)[q*m:(q+1)*m, :]
 *   out dtype: CM_F32 or CM_BF16 (round to nearest even, once, at the end).
 *   Accumulation is fp32 (MFMA); RS buckets travel in fp32.
 *
 * Ownership and ordering.  The caller allocates every device buffer (the
 * library never allocates or frees device memory; its only resources are
 * per-thread HIP events).  Calls are asynchronous: they enqueue work on the
 * compute stream and the comm streams and return.  At entry every comm
 * stream waits for the work already enqueued on the compute stream; at exit
 * the compute stream waits for every comm stream, so the caller needs to
 * synchronise only the compute stream.  Inputs must stay alive and
 * unmodified, and outputs and the workspace untouched, until the compute
 * stream passes the operation.  Two calls that share a workspace or streams
 * must not be issued from different host threads at the same time.
 *
 * Errors.  Every entry point returns a cm_status; nothing throws across the
 * ABI.  Arguments are validated before any HIP call, so an invalid call
 * enqueues nothing.  CM_ERR_HIP carries the HIP error text in
 * cm_last_error().  Faults inside kernels surface at the caller's stream
 * synchronisation, like any other HIP kernel fault.
 */
#ifndef COLLMM_H
#define COLLMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CM_OK = 0,
  CM_ERR_INVALID_ARG = 1, /* null pointer, N < 1, stream count wrong, bad enum */
  CM_ERR_SHAPE = 2,       /* divisibility or size limits violated */
  CM_ERR_ALIGN = 3,       /* a device pointer is not 16-byte aligned */
  CM_ERR_WORKSPACE = 4,   /* ws_bytes smaller than the plan needs */
  CM_ERR_UNSUPPORTED = 5, /* dtype or device not supported (gfx950 only) */
  CM_ERR_HIP = 6,         /* a HIP call failed; see cm_last_error() */
  CM_ERR_CAPACITY = 7     /* a caller-provided output array is too small */
} cm_status;

typedef enum {
  CM_OP_AG_GEMM = 0,      /* AllGather -> GEMM */
  CM_OP_GEMM_RS = 1,      /* GEMM -> ReduceScatter, circulating bucket */
  CM_OP_GEMM_RS_PIPE = 2, /* GEMM -> ReduceScatter, pipeline chunks */
  CM_OP_ALLGATHER = 3     /* the AllGather alone (cm_allgather): k = row length in
                             bf16 elements (a multiple of 8), n = 0; dir, sched,
                             chunks, act, hop_add, bucket_bf16 and tile at their
                             defaults */
} cm_op;

/*
 * CM_RING_DIRECT: no forwarding.  AllGather: at step s rank r fetches shard
 * (r - s - 1) straight from its owner's input for step s + 1 (the shard
 * order of the one-way ring, but every transfer is owner -> consumer).
 * ReduceScatter: at step s rank r sends its partial product for bucket
 * (r - s - 1) straight to the bucket's owner, which adds the arrivals in the
 * ring's order into a home accumulator (with the library's add kernel on a
 * comm stream) and adds its own partial last in its final GEMM.  On a fully
 * connected fabric each transfer has a link of its own; on one GPU it moves
 * the same bytes as the ring.  Results equal the one-way ring's bitwise.
 */
typedef enum { CM_RING_UNI = 0, CM_RING_BI = 1, CM_RING_DIRECT = 2 } cm_ring_dir;

typedef enum {
  CM_SCHED_DECOMPOSED = 0, /* partial GEMMs overlapped with ring hops */
  CM_SCHED_NAIVE = 1,      /* the blocking baseline: the whole collective, then the whole GEMM
                              (AG), or the whole GEMM, then the whole collective (RS) */
  CM_SCHED_AUTO = 2        /* the cost model decides per op ("Knowing when to decline"):
                              decomposed with the best chunking if it predicts a win over the
                              naive schedule, else naive; plan.desc.sched holds the result and
                              plan.declined is 1 when the rewrite was declined */
} cm_sched;

typedef enum { CM_BF16 = 0, CM_F32 = 1 } cm_dtype;

/* Epilogue activation: none, or GELU in its erf form, x * Phi(x) =
 * 0.5 * x * (1 + erf(x / sqrt(2))), evaluated in fp32 before the rounding to
 * the output type. */
typedef enum { CM_ACT_NONE = 0, CM_ACT_GELU = 1 } cm_act;

/*
 * CM_EXEC_GRAPH: the first call with a given plan, set of buffers and trace
 * builds the program as a HIP graph (kernel and memcpy nodes whose edges
 * are the program's stream order and event waits); that call and every later
 * identical call launch the graph on the compute stream with one host call.
 * The comm streams are then not used (the graph's copy nodes run on the
 * engine that copy_engine names).  CM_EXEC_EAGER: every call enqueues the program op
 * by op on the compute and comm streams.  Both run the same operations with
 * the same ordering; the graph form avoids the host-side cost of enqueueing
 * SDMA copies behind cross-stream waits.  Up to 256 graphs are cached per
 * process (shared by its host threads, least recently used dropped first,
 * a quarter at a time, after a device-wide wait).
 */
typedef enum { CM_EXEC_GRAPH = 0, CM_EXEC_EAGER = 1 } cm_exec_mode;

/*
 * Which engine moves a ring hop.  CM_COPY_SDMA (the default): the system DMA
 * copy engines (hipMemcpyDeviceToDeviceNoCU), which use no compute units.
 * CM_COPY_CU: the runtime's copy kernel (hipMemcpyDeviceToDevice), which
 * runs on compute units beside the GEMMs.  The two give identical results.
 * CM_COPY_AUTO (a request only): the planner plans the op with each engine
 * and keeps the one its cost model predicts faster, charging each for what
 * its hops take from the GEMMs (HBM bandwidth for SDMA; HBM bandwidth and
 * compute units for the copy kernel); a near tie keeps SDMA.  The returned
 * plan's desc.copy_engine holds the engine chosen, so re-planning it gives
 * the same plan.
 */
typedef enum { CM_COPY_SDMA = 0, CM_COPY_CU = 1, CM_COPY_AUTO = 2 } cm_copy_engine;

/*
 * Measurement modes: what a trace of the parts alone needs in order to set the
 * decomposed time against them ("Hiding Tensor-Parallel Collectives", section 9:
 * a step is judged against its compute and its communication, each timed on
 * its own).  The program is unchanged -- the same launches, copies and
 * ordering edges -- but one class of its operations is replaced by an empty
 * operation:
 *   CM_SKIP_HOPS   every hop is skipped (copies, and the add launches that run
 *                  on comm streams): the op's GEMM time alone, "G";
 *   CM_SKIP_GEMMS  every launch on the compute stream is skipped (the partial
 *                  GEMMs and split-K reduces): the op's hop time alone, "C".
 * The outputs of a call in either mode are meaningless (not computed); the
 * mode is for timing only.  CM_SKIP_NONE runs the operation.
 */
typedef enum { CM_SKIP_NONE = 0, CM_SKIP_HOPS = 1, CM_SKIP_GEMMS = 2 } cm_skip;

#define CM_MAX_RANKS 64
#define CM_MAX_CHUNKS 16
#define CM_MAX_COMM 32

/* What the caller asks for. */
typedef struct {
  int op;        /* cm_op */
  int n_ranks;   /* N, 1..CM_MAX_RANKS */
  int m;         /* rows per sequence shard; T = N*m */
  int k;         /* contraction length per rank (AG: d; RS: f/N) */
  int n;         /* output columns per rank (AG: f/N; RS: d) */
  int dir;       /* cm_ring_dir */
  int chunks;    /* c: AG row chunks per shard, RS column chunks per bucket,
                    PIPE output column chunks; 0 = choose with the cost model */
  int sched;     /* cm_sched */
  int in_dtype;  /* CM_BF16 */
  int out_dtype; /* CM_F32 or CM_BF16 */
  int n_comm;    /* number of comm streams the calls will pass, 1..CM_MAX_COMM;
                    a program puts hops on at most three of them (with the
                    compute stream, the four hardware queues a process has by
                    default) */
  int tile_m;    /* GEMM block tile: 0 x 0 = choose per launch, else one of */
  int tile_n;    /* 256x256, 256x192, 256x128, 128x256, 128x128, 64x256 */
  int exec_mode; /* cm_exec_mode: how the calls enqueue the program */
  int copy_engine; /* cm_copy_engine: what moves the ring hops */
  int bucket_bf16; /* GEMM-RS (decomposed) only: 0 = the circulating bucket is
                      fp32; 1 = it is stored and sent in bf16 (half the hop
                      bytes), rounded to nearest-even after every addition,
                      which adds up to half a bf16 spacing of error per hop
                      (outside the fp32-bucket error bound) */
  int hop_add;     /* GEMM-RS on a uni or bi ring with an fp32 bucket only.
                      Decomposed CM_OP_GEMM_RS: 0 = each step's GEMM adds the
                      arrived bucket in its epilogue (read-add-write) and the
                      hop is a copy, so a step's GEMM waits for the previous
                      hop; 1 = each step's GEMM stores its partial product and
                      the hop is an add-and-forward launch on compute units (on
                      the first comm stream) that writes partial + arrived
                      bucket into the next rank's receive slot, so a step's
                      GEMM waits for nothing but a free partial slot; the
                      owner's last GEMM still adds in its epilogue.
                      CM_OP_GEMM_RS_PIPE and the naive GEMM-RS: 0 = each ring
                      hop is a copy followed by an add launch; 1 = the chunk's
                      GEMM starts every bucket by storing into the next rank's
                      slot and each further hop is one add-and-forward launch
                      (ring slots per chunk, so a chunk's GEMM never waits for
                      an earlier chunk's ring).  Bitwise the same result. */
  /* Cost-model inputs (0 = built-in defaults for MI355X). */
  double copy_gbps;      /* sustained hop bandwidth of ONE comm stream, GB/s */
  double mfma_tflops;    /* sustained bf16 GEMM rate, TFLOP/s */
  double launch_us;      /* fixed cost per step launch / hop, microseconds */
  int act;               /* AllGather->GEMM only: cm_act applied to every output
                            element before it is stored (the MLP activation fused
                            into the slice update); CM_ACT_NONE for the other ops */
  int share;             /* 0 = every virtual rank's work (the N-rank group on one
                            GPU); 1 = one rank's share: only virtual rank 0's
                            steps, at their real shapes, as one GPU of the group
                            would run them (see "One rank's share" below) */
  int split_k;           /* share = 1 only: number of K slices each step's GEMM is
                            split into (0 = choose: enough slices for the step's
                            tiles to fill the chip, at least 8 slabs of 64 each);
                            must divide k/64, at most 16 */
  int skip;              /* cm_skip: a measurement mode (0 = normal) */
  int stress;            /* 0 = off.  Otherwise a test mode of the eager executor
                            (exec_mode must be CM_EXEC_EAGER), seeded by this
                            value: before some operations (chosen by a hash of the
                            seed and the operation's index) a kernel that sleeps
                            up to ~60 us is enqueued on that operation's stream,
                            and every copy or launch that writes a workspace
                            region is preceded, on its stream, by a fill of that
                            region with 0xFF bytes (NaN in fp32 and bf16).  With
                            the program's ordering right, the results equal those
                            of a run without stress bit for bit; a missing wait
                            shows up as changed or NaN outputs. */
  int group;             /* steps per GEMM launch, for the decomposed AllGather->GEMM
                            and the add-and-forward GEMM->ReduceScatter (hop_add = 1)
                            on a uni- or bidirectional ring with one chunk: 0 = the
                            cost model picks how consecutive steps are grouped (at
                            most 3 per launch for the AllGather, 4 for the
                            ReduceScatter), 1 = one step per launch, g >= 2 = at
                            most g.  A launch multiplies every rank's shards (or
                            bucket rows) of its steps, so each rank's weights are
                            streamed once per launch instead of once per step; a
                            step still uses only shards that have arrived.  A
                            grouped ReduceScatter computes the owner's own partial
                            like any other step's and writes Out with a final add
                            (arrived bucket(s) + own partial, in the fp32 order of
                            the owner's epilogue) on the first comm stream.  Other
                            ops and chunkings use one step per launch. */
} cm_plan_desc;

/* The resolved schedule.  Plain data: no heap, nothing to destroy. */
typedef struct {
  cm_plan_desc desc;   /* copy of the request with defaults filled in */
  int chunks;          /* chosen c */
  int n_steps;         /* compute steps per chunk (AG uni: N; bi: 1 + ceil((N-1)/2)) */
  int arc_cw;          /* ring hops clockwise  (uni: N-1; bi: ceil((N-1)/2)) */
  int arc_ccw;         /* ring hops counter-clockwise (uni: 0; bi: floor((N-1)/2)) */
  int tile_m, tile_n;  /* GEMM block tile */
  int declined;        /* 1 if the cost model found no chunking that hides the hops */
  int n_ops;           /* length of the program cm_plan_program() emits */
  int n_jobs;          /* total GEMM / reduce jobs in that program */
  int n_events;        /* events the program uses */
  size_t ws_bytes;     /* workspace bytes the calls need */
  double est_gemm_us;  /* cost model: one step's GEMM time (all ranks, one chunk) */
  double est_hop_us;   /* cost model: one step's hop time (all ranks, one chunk) */
  double est_total_us; /* cost model: the whole op */
  int split;           /* share = 1: the K slices per step GEMM (S); else 0 */
  int n_launches;      /* decomposed ring ops: GEMM launches per chunk (n_steps when
                          every launch is one step); else 0 */
  int group_len[CM_MAX_RANKS]; /* steps of each of those launches, in order */
  int slots;           /* receive slots per rank and direction (AllGather) or
                          partial-product slots (add-and-forward ReduceScatter):
                          2, alternating by step, or one per step when steps are
                          grouped (no slot is then written twice) */
} cm_plan;

/*
 * One rank's share (cm_plan_desc.share = 1; AllGather->GEMM and the
 * decomposed GEMM->ReduceScatter on a one-way ring, one chunk, fp32 bucket,
 * copy hops).  On a real group each GPU runs only its own rank's steps; this
 * program runs virtual rank 0's, at the real per-rank shapes, and brings in
 * what its ring neighbour would send from buffers that stand for that
 * neighbour.  One step's GEMM of one rank has too few output tiles to fill
 * the chip (the GPT-3 fc1 step: 32 tiles of 256x192 for 256 compute units),
 * so it is split along K into S slices (cm_plan.split) that write fp32
 * partial products to the workspace, and one reduce launch adds the S
 * partials in slice order (and, for the ReduceScatter, the arrived bucket)
 * and stores the step's result.  Per step the GPU moves what rank 0's HBM
 * would: the step GEMM's operands, the partials, and one hop copy of the
 * shard (or bucket) that arrives.
 *
 *   AllGather->GEMM: x = [N][m][k] (the N shards; the ones of ranks 1..N-1
 *   stand for the peers'), w = rank 0's weights [n][k] (the first block of a
 *   [N][n][k] array is what is read), y = rank 0's output [N*m][n]:
 *   y[c*m .. c*m+m) = act(X_c . W_0^T) for every shard c.  Step s multiplies
 *   shard (N - s) mod N; hop s copies shard (N - s - 1) mod N from x into the
 *   receive slot of step s + 1.
 *   Workspace: receive slots [2][m][k] bf16, then partials [S][m][n] fp32.
 *
 *   GEMM->ReduceScatter: h = rank 0's activations [N*m][k], w = rank 0's
 *   weights [n][k] (first block), out = rank 0's result [m][n].  Step s adds
 *   rank 0's contribution H_0[b*m .. b*m+m) . W_0^T for bucket
 *   b = (N - 1 - s) mod N to the bucket that arrived (none at s = 0) and
 *   sends it on; at s = N - 1 (b = 0, the home bucket) the sum is rank 0's
 *   output.  The arriving buckets are the caller's: the workspace starts
 *   with peer[N-1][m][n] fp32, peer[s - 1] being the bucket the neighbour
 *   sends for step s; hop s - 1 copies it into a receive slot.  The buckets
 *   rank 0 sends are stored in sent[N-1][m][n] fp32 (sent[s] = step s's sum,
 *   s < N - 1).  Workspace: peer, receive slots [2][m][n], sent, partials
 *   [S][m][n], all fp32, in that order.
 */

/*
 * Build a plan: the ring schedule of one decomposed collective matmul, i.e.
 * which shard (AllGather) or bucket (ReduceScatter) every virtual rank
 * multiplies at every step, which hop moves it next, the chunk count and the
 * GEMM tile.  Defined by the per-step order of "The idea" on the
 * decomposition page (each partial uses only shards that have arrived; the
 * accumulator circulates and reaches its home last), the ring hops of
 * sections 3 and 5 of the Megatron page, the chunk count as a tuning knob
 * (section 6 there) and the peak-rate cost model that may decline to
 * decompose ("Knowing when to decline").
 * Fails with CM_ERR_SHAPE unless: N*m <= 2^24 rows; k and n
 * are multiples of 64; one virtual rank's operands stay under 4 GiB
 * (N*m*k*2 and n*k*2 bytes); AG: c divides m; RS: c divides n and n/c is a
 * multiple of 64; PIPE: same as RS.  Host only: makes no HIP call.
 */
cm_status cm_ring_plan(const cm_plan_desc *desc, cm_plan *out);

/* Workspace bytes a plan needs (same as plan->ws_bytes). */
cm_status cm_workspace_size(const cm_plan *plan, size_t *bytes);

/*
 * Pick one of two collectives to decompose ("Knowing when to decline" on the
 * decomposition page: when an einsum could overlap either of two collectives,
 * the cost model chooses between them).  An einsum whose
 * input is all-gathered and whose output is reduce-scattered can overlap only
 * one of them with its partial products.  `ag` describes the AllGather-side
 * candidate (op CM_OP_AG_GEMM) and `rs` the ReduceScatter-side candidate (op
 * CM_OP_GEMM_RS or CM_OP_GEMM_RS_PIPE), each with the shapes the einsum would
 * have in that form.  The cost model predicts each candidate's decomposed
 * time (best chunking) and naive time; *choice receives 0 (decompose the
 * AllGather), 1 (decompose the ReduceScatter) or -1 (neither is predicted to
 * win), and saving_us[2] (may be NULL) the predicted savings, naive minus
 * decomposed, of the two.  Host only.  Errors: CM_ERR_INVALID_ARG for null
 * pointers or wrong ops, and every error of cm_ring_plan for either request.
 */
cm_status cm_pick_overlap(const cm_plan_desc *ag, const cm_plan_desc *rs, int *choice, double *saving_us);

/*
 * The plan as a program: the exact sequence of operations the executor
 * enqueues, in order, for inspection and CPU simulation.  Buffers are named
 * symbolically and addressed by byte offsets.  Host only.
 */
typedef enum { CM_BUF_X = 0, CM_BUF_W = 1, CM_BUF_Y = 2, CM_BUF_WS = 3 } cm_buf;

typedef enum {
  CM_OPK_GEMM = 0,   /* one launch of partial GEMMs: jobs [first_job, first_job+n_jobs) */
  CM_OPK_COPY = 1,   /* one hop copy of `bytes` from (src_buf, src_off) to (dst_buf, dst_off) */
  CM_OPK_RECORD = 2, /* record event `event` on `stream` */
  CM_OPK_WAIT = 3,   /* `stream` waits for the last record of `event` */
  CM_OPK_REDUCE = 4  /* one launch of elementwise adds: jobs [first_job, ...) */
} cm_op_kind;

typedef struct {
  int kind;      /* cm_op_kind */
  int stream;    /* 0 = compute stream, 1..n_comm = comm stream (stream-1) */
  int event;     /* RECORD / WAIT */
  int step;      /* schedule step this op belongs to (-1 = entry/exit) */
  int chunk;     /* chunk index */
  int first_job; /* GEMM / REDUCE */
  int n_jobs;
  int rows, cols, depth; /* GEMM: M, N, K of every job; REDUCE: rows, cols and
                            the number S of fp32 blocks summed from in0 (0 = 1) */
  int tile_m, tile_n;    /* GEMM: block tile the launch uses */
  int src_buf, dst_buf;  /* COPY */
  size_t src_off, dst_off, bytes;
  int act;               /* GEMM: cm_act of the epilogue (launches without addends
                            only); REDUCE: cm_act applied to the sum */
  int b_share;           /* GEMM: jobs come in runs of b_share consecutive jobs that
                            read the same B (one rank's grouped steps); the kernel
                            runs a run's tiles of one B column together.  n_jobs is
                            a multiple of it; 1 = no sharing */
} cm_op_rec;

/*
 * One job of a GEMM op:  C[i][j] = sum_kk A[i][kk] * B[j][kk] + in0[i][j] + in1[i][j]
 * for i < rows, j < cols, kk < depth.  A, B bf16; in0/in1 fp32, each optional
 * (buf -1 = absent; in0 may alias C: read-add-write); C in c_dtype.
 * lda/ldb/ldc/ld_in are row strides in elements.  For a REDUCE op with
 * S = max(1, depth): C = act(B_0 + B_1 + ... + B_{S-1} (+ in1)), added in that
 * order, where B_s is the fp32 block of rows x ld_in elements at in0 +
 * s * rows * ld_in (in0 present, in1 optional, both fp32).  `rank`, `dir` and `index` (the
 * shard or bucket the job works on) label the job for tests; the executor
 * does not use them.
 */
typedef struct {
  int rank, dir, index;
  int a_buf, b_buf, c_buf, in0_buf, in1_buf;
  size_t a_off, b_off, c_off, in0_off, in1_off;
  int lda, ldb, ldc, ld_in;
  int c_dtype;
  int add_dtype; /* element type of in0/in1: CM_F32, or CM_BF16 for bf16 buckets */
} cm_job_rec;

/*
 * Emit the plan's program.  ops (capacity op_cap) and jobs (capacity
 * job_cap) are caller-owned host arrays; pass NULL with zero capacity to
 * query the sizes (also in plan->n_ops / n_jobs).  CM_ERR_CAPACITY if an
 * array is too small.
 */
cm_status cm_plan_program(const cm_plan *plan, cm_op_rec *ops, int op_cap, int *n_ops,
                          cm_job_rec *jobs, int job_cap, int *n_jobs);

/*
 * Optional timing trace.  When a non-NULL trace is passed to a call, the
 * executor records a timing event on the issuing stream before and after
 * every GEMM launch, every hop group and every reduce launch (the work is
 * the same as without a trace).  After the compute stream has completed,
 * cm_trace_read() converts the events into microseconds since the call's
 * entry event.  The trace owns its events: create once, reuse, destroy.
 */
typedef struct cm_trace cm_trace;

typedef struct {
  int kind;      /* CM_OPK_GEMM, CM_OPK_COPY (one per hop group per stream) or CM_OPK_REDUCE */
  int stream;    /* as in cm_op_rec */
  int step, chunk;
  double start_us, end_us;
} cm_span;

cm_status cm_trace_create(int capacity, cm_trace **out);
cm_status cm_trace_destroy(cm_trace *trace);
/* Spans of the last call that used `trace`; *n_spans receives the count. */
cm_status cm_trace_read(cm_trace *trace, cm_span *spans, int cap, int *n_spans, double *total_us);

/*
 * AllGather -> GEMM (see "Layouts").  Decomposed schedule: at step s rank r
 * multiplies the shard it holds into rows of Y_r belonging to that shard
 * (the slice update), while the same shard is copied to the next rank.
 * Defined by section 3 of the Megatron page (P2P AllGather overlap) and the
 * AllGather->Einsum loop of "The idea" on the decomposition page (a partial
 * einsum per arrived shard, written into its slice of the result).
 *   plan     from cm_ring_plan with op CM_OP_AG_GEMM
 *   x, w, y  device pointers, 16-byte aligned
 *   ws       device workspace of ws_bytes >= plan->ws_bytes (receive slots)
 *   compute  the compute stream (hipStream_t passed as void*; NULL = default)
 *   comm     array of plan->desc.n_comm comm streams (distinct, non-NULL)
 *   trace    optional (NULL)
 */
cm_status cm_ag_gemm(const cm_plan *plan, const void *x, const void *w, void *y, void *ws,
                     size_t ws_bytes, void *compute, void *const *comm, int n_comm,
                     cm_trace *trace);

/*
 * GEMM -> ReduceScatter (see "Layouts").  CM_OP_GEMM_RS: at step s rank r
 * adds its partial product for the bucket it holds into that bucket (fp32),
 * then the bucket moves to the next rank; the owner adds its share last and
 * writes Out_q.  CM_OP_GEMM_RS_PIPE: the output columns are split into c
 * chunks; each chunk's full partial products are computed in one launch and
 * reduce-scattered around the ring (copy + add) while the next chunk
 * computes.  Defined by section 5 of the Megatron page (P2P ReduceScatter
 * overlap) with the Einsum->ReduceScatter loop of "The idea" on the
 * decomposition page (the circulating accumulator), and by section 6 of the
 * Megatron page for the pipeline-chunk variant.  Arguments as for
 * cm_ag_gemm; x holds H.
 */
cm_status cm_gemm_rs(const cm_plan *plan, const void *x, const void *w, void *y, void *ws,
                     size_t ws_bytes, void *compute, void *const *comm, int n_comm,
                     cm_trace *trace);

/* ------------------------------------------------------------------------
 * The sequence-parallel transformer layer around the two collective matmuls.
 *
 * The Megatron page's sequence parallelism keeps per-token work (LayerNorm,
 * dropout) on the sequence-sharded activation between the ReduceScatter that
 * ends one tensor-parallel block and the AllGather that starts the next;
 * "Tensor Parallelism > Communication Patterns" places LayerNorm in the same
 * gap between the two halves of an all-reduce.  The pages give no formulas
 * for the layer's other stages; these entry points compute the textbook
 * definitions.
 * ------------------------------------------------------------------------ */

/*
 * Causal (or full) scaled dot-product attention of every head of every
 * virtual rank, softmax(Q K^T / sqrt(D)) V, bf16 in and out, fp32 scores,
 * probabilities rounded to bf16 for the value product and the normaliser.
 *   qkv  [n_ranks][T][3*heads*head_dim] bf16: columns h*D.. hold head h's
 *        query, heads*D + h*D.. its key, 2*heads*D + h*D.. its value (the
 *        QKV projection's output in this library's layout)
 *   o    [n_ranks][T][heads*head_dim] bf16: head h in columns h*D..
 *   causal 1: query t attends to keys 0..t; 0: to every key
 *   stream the stream to enqueue on (hipStream_t as void*; NULL = default)
 * head_dim must be 128 (CM_ERR_UNSUPPORTED otherwise).  Asynchronous.
 * Errors: CM_ERR_INVALID_ARG (null pointer, bad count), CM_ERR_ALIGN
 * (pointers not 16-byte aligned), CM_ERR_SHAPE (too large), CM_ERR_HIP.
 */
cm_status cm_attention(const void *qkv, void *o, int n_ranks, int T, int heads, int head_dim, int causal,
                       void *stream);

/*
 * LayerNorm of every row: y = (x - mean) / sqrt(var + eps) * gamma + beta,
 * with the population variance; x fp32 [rows][cols], y bf16 [rows][cols]
 * (nearest-even), gamma and beta fp32 [cols] or NULL (1 and 0).  cols must be
 * a multiple of 4 in 4..16384.  Asynchronous on `stream`.  Errors:
 * CM_ERR_SHAPE, CM_ERR_INVALID_ARG (null x or y, eps < 0 or not finite),
 * CM_ERR_ALIGN, CM_ERR_HIP.
 */
cm_status cm_layernorm(const void *x, void *y, int rows, int cols, float eps, const void *gamma, const void *beta,
                       void *stream);

/* One sequence-parallel transformer layer (forward), N virtual ranks. */
typedef struct {
  int n_ranks;     /* N */
  int m;           /* tokens per sequence shard; T = N*m */
  int d;           /* hidden size */
  int heads;       /* attention heads per rank (the layer has N*heads) */
  int head_dim;    /* 128 */
  int ffn;         /* MLP width per rank (f/N) */
  int dir;         /* cm_ring_dir of the QKV, fc1 and fc2 collective matmuls (the
                      output projection's pipeline-chunk ReduceScatter is a one-way ring) */
  int n_comm;      /* comm streams the call passes */
  int copy_engine; /* cm_copy_engine of every stage's hops; CM_COPY_AUTO lets the
                      planner choose per stage (the stage plans name the engine chosen) */
  int exec_mode;   /* cm_exec_mode */
  int ag_chunks;   /* chunks of both AllGather->GEMMs (0 = cost model) */
  int rs_chunks;   /* chunks of the fc2 ReduceScatter (0 = cost model) */
  int proj_chunks; /* pipeline chunks of the output projection's ReduceScatter (0 = 4) */
  int out_dtype;   /* CM_BF16 or CM_F32: the layer output */
  float ln_eps;    /* LayerNorm epsilon (0 = 1e-5) */
} cm_layer_desc;

/* The resolved layer: plain data, nothing to destroy. */
typedef struct {
  cm_layer_desc desc; /* the request with defaults filled in */
  cm_plan qkv;        /* AllGather -> QKV projection (k = d, n = 3*heads*D), bf16 out */
  cm_plan proj;       /* output projection -> pipeline-chunk ReduceScatter (k = heads*D, n = d), fp32 out,
                         add-and-forward hops */
  cm_plan fc1;        /* AllGather -> fc1 (k = d, n = ffn) with GELU, bf16 out */
  cm_plan fc2;        /* fc2 -> ReduceScatter (k = ffn, n = d), add-and-forward hops on a ring */
  size_t off_qkv, off_attn, off_proj, off_ln, off_fc1, off_ops; /* workspace regions (bytes) */
  size_t ws_bytes;    /* workspace the call needs */
} cm_layer_plan;

/*
 * Plan a layer.  Host only.  Errors: those of cm_ring_plan for any of the four
 * collective matmuls, of cm_attention (head_dim) and of cm_layernorm (d).
 */
cm_status cm_plan_layer(const cm_layer_desc *desc, cm_layer_plan *out);

/*
 * The layer forward (all inputs bf16, row-major, rank r = block r):
 *   x    [N][m][d]             the sequence shards entering the layer
 *   wqkv [N][3*heads*D][d]     rank r's query, key and value projections (its
 *                              heads r*heads..), one output feature per row
 *   wo   [N][d][heads*D]       rank r's slice of the output projection
 *   w1   [N][ffn][d]           rank r's fc1 columns
 *   w2   [N][d][ffn]           rank r's fc2 rows
 *   out  [N][m][d]             the shards leaving the layer (desc.out_dtype)
 *   ws   workspace of ws_bytes >= plan->ws_bytes; after the call it holds the
 *        intermediates at the plan's offsets: QKV [N][T][3*heads*D] bf16,
 *        attention [N][T][heads*D] bf16, projection [N][m][d] fp32, LayerNorm
 *        [N][m][d] bf16, fc1 (after GELU) [N][T][ffn] bf16
 * Chain: x -> AG->QKV -> attention (causal) -> out-proj->RS (pipeline chunks)
 * -> LayerNorm (gamma 1, beta 0) -> AG->fc1 (+GELU) -> fc2->RS.  No residual
 * connections.  Streams, ordering and errors as for cm_ag_gemm; asynchronous.
 */
cm_status cm_layer_forward(const cm_layer_plan *plan, const void *x, const void *wqkv, const void *wo,
                           const void *w1, const void *w2, void *out, void *ws, size_t ws_bytes, void *compute,
                           void *const *comm, int n_comm);

/* ------------------------------------------------------------------------
 * The backward pass of the two collective matmuls, with bulk overlap.
 *
 * "Tensor Parallelism > Communication Patterns": the backward communication
 * pattern is the dual of the forward one.  Megatron page, section 7 ("Bulk
 * Overlap"): an AllGather that only the weight gradient needs can run on a
 * communication stream while the input-gradient GEMM runs on the compute
 * stream, into buffers the compute stream leaves alone until an event.
 * ------------------------------------------------------------------------ */

/*
 * AllGather alone: y[r] = concat_q x[q] for every virtual rank r, by N - 1
 * ring hops of copies (the plan's copy engine).  plan from cm_ring_plan with op
 * CM_OP_ALLGATHER; x [N][m][k] bf16, y [N][N*m][k] bf16 (16-byte aligned).
 * Streams, ordering and errors as for cm_ag_gemm (no workspace).
 */
cm_status cm_allgather(const cm_plan *plan, const void *x, void *y, void *compute, void *const *comm, int n_comm,
                       cm_trace *trace);

/*
 * Batched bf16 transpose: dst[b][c][r] = src[b][r][c] (r < rows, c < cols) and
 * dst[b][c][r] = 0 for rows <= r < ld_dst, b < batch; src [batch][rows][cols],
 * dst [batch][cols][ld_dst].  Asynchronous on `stream`.  Errors: CM_ERR_SHAPE
 * (batch outside 1..65535, rows or cols < 1, ld_dst < rows), CM_ERR_INVALID_ARG,
 * CM_ERR_ALIGN (odd addresses), CM_ERR_HIP.
 */
cm_status cm_transpose(const void *src, void *dst, int batch, int rows, int cols, int ld_dst, void *stream);

/*
 * Batched GEMM on the library's MFMA kernel: for b < batch,
 *   C_b[i][j] = sum_kk A_b[i][kk] * B_b[j][kk]   (i < M, j < N, kk < K)
 * A_b = a + b * stride_a (bf16, row stride lda), B_b = b + b * stride_b (bf16,
 * row stride ldb), C_b = c + b * stride_c (out_dtype, row stride ldc); strides
 * in elements.  fp32 accumulation; bf16 outputs rounded to nearest even.  K a
 * multiple of 64; lda, ldb, stride_a and stride_b multiples of 8; stride_c a
 * multiple of 4 (fp32) or 8 (bf16); 16-byte aligned pointers.
 * Asynchronous.  Errors: CM_ERR_SHAPE, CM_ERR_INVALID_ARG, CM_ERR_ALIGN,
 * CM_ERR_UNSUPPORTED, CM_ERR_HIP.
 */
cm_status cm_gemm(int batch, int M, int N, int K, const void *a, int lda, long long stride_a, const void *b, int ldb,
                  long long stride_b, void *c, int ldc, long long stride_c, int out_dtype, void *stream);

typedef enum {
  CM_BWD_COL = 0, /* the forward was AllGather -> GEMM (column-parallel):
                     dX = ReduceScatter_r(dY_r . W_r), dW_r = dY_r^T . Xfull */
  CM_BWD_ROW = 1  /* the forward was GEMM -> ReduceScatter (row-parallel):
                     dH_r = AllGather(dOut) . W_r, dW_r = AllGather(dOut)^T . H_r */
} cm_bwd_kind;

typedef struct {
  int kind;         /* cm_bwd_kind */
  int n_ranks, m, k, n; /* the forward's shapes: W_r [n][k]; T = N*m tokens */
  int dir;          /* cm_ring_dir of the input gradient's collective matmul */
  int chunks;       /* its chunks (0 = cost model) */
  int n_comm;       /* its comm streams */
  int bulk;         /* 1: the weight gradient's AllGather (and transposes) run on
                       the bulk stream beside the input gradient; 0: in the
                       compute stream's order, before it */
  int dx_dtype;     /* CM_F32 or CM_BF16: the input gradient */
  int dw_dtype;     /* CM_F32 or CM_BF16: the weight gradient */
  int exec_mode;    /* cm_exec_mode */
  int copy_engine;  /* cm_copy_engine of the input gradient's ring hops (CM_COPY_AUTO:
                       the planner's choice); the weight gradient's AllGather always
                       uses CM_COPY_CU */
} cm_bwd_desc;

typedef struct {
  cm_bwd_desc desc;
  cm_plan dgrad;    /* COL: GEMM -> ReduceScatter (k' = n, n' = k, add-and-forward
                       hops on a ring); ROW: AllGather -> GEMM (k' = n, n' = k) */
  cm_plan gather;   /* the bulk AllGather (COL: of x, rows of k; ROW: of dOut, rows of n) */
  size_t off_wt;    /* workspace: W_r^T [N][k][n] (made unless the caller passes it) */
  size_t off_g;     /* the gathered operand [N][T][k or n] */
  size_t off_gt;    /* its transpose [N][k or n][Tp], Tp = T rounded up to 64 (zero padded) */
  size_t off_ot;    /* COL: dY_r^T [N][n][Tp]; ROW: H_r^T [N][k][Tp] */
  size_t off_ops;   /* the input gradient's workspace */
  size_t ws_bytes;
} cm_bwd_plan;

/* Plan a backward.  Host only.  Errors: those of cm_ring_plan for the input
 * gradient's collective matmul and for the AllGather, CM_ERR_INVALID_ARG,
 * CM_ERR_UNSUPPORTED (gradient dtypes), CM_ERR_SHAPE. */
cm_status cm_plan_backward(const cm_bwd_desc *desc, cm_bwd_plan *out);

/*
 * The backward (all inputs bf16, rank r = block r):
 *   COL: act = x [N][m][k], grad = dY [N][T][n] -> dact = dX [N][m][k]
 *   ROW: act = H [N][T][k], grad = dOut [N][m][n] -> dact = dH [N][T][k]
 *   w [N][n][k] the forward weights; wt [N][k][n] their transpose or NULL (then
 *   the call transposes w into the workspace); dw [N][n][k] (desc.dw_dtype).
 * comm: the plan's n_comm streams for the input gradient's hops, then the bulk
 * stream, then the bulk AllGather's copy lane (n_comm + 2 distinct streams).
 * The call orders everything against `compute`: the bulk stream starts after
 * the work already on `compute`, and the weight gradient waits for the bulk
 * stream.  Asynchronous; errors as for cm_ag_gemm.
 */
cm_status cm_linear_backward(const cm_bwd_plan *plan, const void *act, const void *w, const void *wt,
                             const void *grad, void *dact, void *dw, void *ws, size_t ws_bytes, void *compute,
                             void *const *comm, int n_comm);

/*
 * For callers that cannot allocate device memory (code a caller captures into
 * a graph, tight serving loops, harnesses that forbid hipMalloc): cm_gemm_rs
 * with its workspace taken from a static array the library holds on each GPU
 * (CM_NOALLOC_WS_BYTES bytes, allocated when the library's code object is
 * loaded on that GPU and held until the process ends), instead of the
 * caller's `ws`.  Arguments, layouts, ordering and results are those of
 * cm_gemm_rs; the program is always enqueued op by op (exec_mode is taken as
 * CM_EXEC_EAGER, since instantiating a graph may allocate) and no trace is
 * recorded.  Nothing in the array has to start at zero: every program writes
 * each bucket and partial slot before it reads it.  The call allocates no
 * memory (no hipMalloc, no hipFree).  All calls on one GPU share that GPU's
 * array: two calls whose work overlaps in time on one GPU (on different
 * streams, or from different threads) race on it.
 * Errors: those of cm_gemm_rs; CM_ERR_WORKSPACE if plan->ws_bytes exceeds
 * CM_NOALLOC_WS_BYTES.
 */
#define CM_NOALLOC_WS_BYTES ((size_t)256 << 20)
cm_status cm_gemm_rs_noalloc(const cm_plan *plan, const void *x, const void *w, void *y, void *compute,
                             void *const *comm, int n_comm);

const char *cm_status_string(cm_status s);
/* Detail of the last failing call on this thread ("" if none). */
const char *cm_last_error(void);
/* Library version, "major.minor.patch". */
const char *cm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* COLLMM_H */
