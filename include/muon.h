/*
 * muon.h: C ABI of the whole-tensor Muon optimizer step on one gfx950 GPU.
 *
 * The operation. A data-parallel rank updates the whole matrices it owns with
 * no communication. This is the "optimizer step (local)" phase of the Canzona
 * analysis page (paper-graph-ui), section 3.4, DP per-iteration execution. The
 * step also equals ΔW = Muon_step(G, States_local) followed by P <- P + ΔW,
 * from the micro-group lifecycle in the same section (steps 2 and 4). The
 * update has the form W_{t+1} = W_t - eta * MatrixOp(W_t, grad W_t) (same page,
 * section 2). Muon's MatrixOp orthogonalises the whole gradient with
 * Newton-Schulz iterations, and the momentum buffer is state that stays on the
 * owning rank (section 3.4, "Task abstraction").
 *
 * For every matrix (rows r, cols c) one step computes:
 *   M' = beta*M + G                          momentum, updated in place
 *   U  = G + beta*M'   (nesterov; else M')
 *   X0 = U (or U^T if r > c, so X is m x n with m <= n) / (||U||_F + eps)
 *   T times: A = X X^T;  B = b*A + c*A*A;  X = a*X + B X
 *   O  = X (or X^T if r > c)
 *   W' = W - lr * sqrt(max(1, r/c)) * O      weights, updated in place
 *
 * Conventions for every function:
 * - It returns muon_status (0 = MUON_OK) and never throws or aborts across the
 *   ABI. On error, muon_last_error() gives this thread's message.
 * - Pointers named w, g, m and delta are device pointers. They address
 *   row-major, contiguous matrices of the plan's dtype (MUON_BF16_F32_MASTER:
 *   fp32 w, m and delta with a bf16 g).
 * - Every other pointer is a host pointer.
 */
#ifndef MUON_H_
#define MUON_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARG = -1, /* null/negative/non-finite argument, bad shape   */
  MUON_ERR_ALIAS = -2,       /* two device ranges of the batch overlap         */
  MUON_ERR_ALIGN = -3,       /* a device pointer is not 16-byte aligned        */
  MUON_ERR_UNSUPPORTED = -4, /* dtype or option not supported                  */
  MUON_ERR_HIP = -5,         /* a HIP runtime call failed (message has it)     */
  MUON_ERR_OOM = -6          /* workspace allocation failed                    */
} muon_status;

typedef enum {
  MUON_F32 = 0,  /* W, G, M fp32; all arithmetic fp32 (fp32 MFMA)          */
  MUON_BF16 = 1, /* W, G, M bf16; bf16 MFMA with fp32 accumulation,         */
                 /* intermediates stored bf16 (round to nearest even)      */
  MUON_BF16_F32_MASTER = 2
                 /* fp32 master weights and momentum with bf16 gradients,  */
                 /* the training setup of the pages (Canzona analysis page, */
                 /* section 3.4, the Atomicity Constraint): W, M and delta  */
                 /* fp32, G bf16; X, A and B bf16 as for MUON_BF16, and     */
                 /* W' = W - lr*s*O formed in fp32 and stored fp32         */
} muon_dtype;

/* One matrix of the batch: rows x cols, row-major, contiguous.
 * w     weights, updated in place. May be NULL when delta is set.
 * g     gradient, read only.
 * m     momentum buffer, updated in place.
 * delta optional (NULL = none). When set, it receives
 *       Delta W = -lr*sqrt(max(1,r/c))*O, the update that the host rank
 *       returns in the micro-group lifecycle (Canzona analysis page, section
 *       3.4, step 2).
 * All four ranges must be 16-byte aligned and must not overlap any other
 * range of the batch. */
typedef struct {
  void* w;
  const void* g;
  void* m;
  void* delta;
  int64_t rows;
  int64_t cols;
} muon_matrix;

/* Hyperparameters. muon_hparams_default() fills in:
 * lr = 0.02, beta = 0.95, eps = 1e-7, (a,b,c) = (3.4445, -4.7750, 2.0315),
 * ns_steps = 5, nesterov = 1, dtype = MUON_BF16. */
typedef struct {
  float lr;
  float beta;     /* momentum, 0 <= beta < 1                               */
  float eps;      /* added to the Frobenius norm, eps >= 0                 */
  float a, b, c;  /* Newton-Schulz polynomial a*x + b*x^3 + c*x^5          */
  int32_t ns_steps; /* >= 0; 0 applies the normalised direction itself    */
  int32_t nesterov; /* 0 or 1                                              */
  int32_t dtype;    /* muon_dtype                                          */
} muon_hparams;

typedef struct muon_plan_s* muon_plan_t;

/* Fills *hp with the defaults listed above. Returns INVALID_ARG if hp is NULL. */
muon_status muon_hparams_default(muon_hparams* hp);

/* Builds a static plan for a batch of n matrices. The plan is computed once
 * and reused every step; the pages' planners likewise run once at
 * initialisation (Canzona analysis page, section 3.3 "Output and offline
 * nature").
 * mats  host array of n descriptors. The plan keeps the device pointers, so
 *       the tensors must stay allocated and unmoved until muon_plan_destroy.
 * hp    host pointer to the hyperparameters (copied).
 * out   receives the plan handle (NULL on error).
 * Every argument is validated before any HIP call. Errors: INVALID_ARG (n < 1,
 * null pointers, rows or cols < 1 or > 2^24 (> 2^23 for MUON_F32),
 * non-finite lr/beta/eps/a/b/c, beta outside [0,1), eps < 0, ns_steps < 0),
 * ALIAS, ALIGN, UNSUPPORTED (dtype). Then the
 * plan allocates and zeroes its device workspace on the current device: HIP
 * or OOM on failure. The call synchronises the device once, at its end. */
muon_status muon_plan(const muon_matrix* mats, int32_t n, const muon_hparams* hp,
                      muon_plan_t* out);

/* Device workspace bytes held by the plan (written to *bytes). */
muon_status muon_plan_workspace_bytes(muon_plan_t plan, size_t* bytes);

/* Enqueues one step over the whole batch on `stream` (a hipStream_t; NULL is
 * the null stream). It is asynchronous: no host synchronisation and no
 * allocation. Launch errors return HIP; faults surface at the caller's next
 * synchronisation. A plan must not be stepped concurrently on two streams,
 * because its work-queue counters live in its workspace. Matrices are
 * independent, and the result does not depend on descriptor order. For a
 * fixed plan the result is bitwise deterministic.
 * A step only launches kernels and records and waits on events (no memset,
 * copy or host synchronisation; the work-queue counters are cleared by the
 * step's own kernels), so it may be captured in a HIP graph on `stream` and
 * the graph replayed; a replay equals an eager step bit for bit. Kernel
 * timing (muon_plan_set_timing) must be off during capture. */
muon_status muon_step(muon_plan_t plan, void* stream);

/* Frees the plan and its workspace. NULL is a no-op. Synchronises the device. */
muon_status muon_plan_destroy(muon_plan_t plan);

/* Bytes of the static device scratch that muon_step_noalloc works in. */
#define MUON_NOALLOC_SCRATCH_BYTES (64u << 20)

/* One step that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. It computes what muon_plan, one muon_step and
 * muon_plan_destroy compute, bit for bit, but keeps its workspace (the
 * Newton-Schulz buffers, norm partials, work-queue counters and tile tables)
 * in a static device array of MUON_NOALLOC_SCRATCH_BYTES (64 MiB), one per
 * GPU, which the library holds from its first use on that GPU until the
 * process ends. It calls no hipMalloc or hipFree and creates no stream or
 * event: everything is enqueued on `stream` (a hipStream_t; NULL is the null
 * stream) as one chain of launches: a fill kernel clears the workspace,
 * small kernels copy the tables in (their bytes travel as kernel arguments),
 * then the step's kernels run. Host-side bookkeeping (building the tables) uses
 * ordinary host memory.
 * mats, n, hp: as for muon_plan (the same validation and errors), device
 * pointers on the current device. The tensors must stay valid until the step
 * has run on the stream.
 * Errors: those of muon_plan's validation; INVALID_ARG if the batch's
 * workspace exceeds the scratch (the message gives both sizes); HIP.
 * Every call on a GPU works in that GPU's one array, which keeps the last
 * call's contents: calls that overlap on one GPU (on two streams without an
 * ordering between them, or from two threads) race and give wrong results.
 * Calls issued one after another on one stream are safe. */
muon_status muon_step_noalloc(const muon_matrix* mats, int32_t n, const muon_hparams* hp, void* stream);

/* This thread's last error message ("" if none). Valid until this thread's
 * next call into the library. */
const char* muon_last_error(void);

/* Kernel kinds, for the timing counters below. */
typedef enum {
  MUON_K_MOMENTUM = 0, /* fused momentum + Nesterov + sum-of-squares partials */
  MUON_K_NORM = 1,     /* fixed-order norm reduction to 1/(||U||+eps)        */
  MUON_K_GRAM = 2,     /* symmetric A = X X^T (upper tiles, mirrored)        */
  MUON_K_SQUARE = 3,   /* B = b*A + c*A*A (upper tiles, mirrored)            */
  MUON_K_UPDATE = 4,   /* X = a*X + B X; on the last step, the weight apply  */
  MUON_K_APPLY = 5,    /* weight apply when ns_steps == 0                    */
  MUON_K_GRAM_REDUCE = 6, /* sum of split-K Gram pieces, then A's epilogue   */
  MUON_K_COUNT = 7
} muon_kernel_kind;

/* enable != 0: every later muon_step records a HIP event pair on its stream
 * around each kernel launch. Timing is off by default. */
muon_status muon_plan_set_timing(muon_plan_t plan, int32_t enable);

/* Waits for the recorded events and adds their durations to per-kind totals.
 * Then writes, for kind k in [0, MUON_K_COUNT):
 *   total_ms[k] = summed launch durations;
 *   launches[k] = number of launches.
 * Either array may be NULL. Totals accumulate until muon_plan_reset_timing. */
muon_status muon_plan_kernel_times(muon_plan_t plan, double* total_ms, int64_t* launches);
muon_status muon_plan_reset_timing(muon_plan_t plan);

/* Plan facts, for logs and benchmarks (host pointers; any may be NULL):
 * n_tiles[k] = tiles per launch of kind k (K1 tiles for MOMENTUM);
 * grid[k]    = workgroups launched per launch of kind k. */
muon_status muon_plan_info(muon_plan_t plan, int64_t* n_tiles, int64_t* grid);

/* ---------------------------------------------------------------------------
 * Tensor-parallel local update.
 *
 * Under tensor parallelism a rank holds shards of each weight matrix: a
 * column-parallel layer splits the output dimension (a block of rows of the
 * rows x cols W), a row-parallel layer the input dimension (a block of
 * columns) (Canzona analysis page, section 2, "The Core Problem"). The host
 * rank of a tensor runs muon_step on the whole matrix with delta set (and w
 * NULL); the update is then cut into the TP partition's slices, and every rank
 * adds its slices to its parameter shards, P_local <- P_local + Delta W_local,
 * element by element and with no communication (section 3.4, "The TP Task
 * Abstraction", micro-group lifecycle, steps 3 and 4).
 *
 * One shard: p and d are device pointers of the plan's dtype.
 * p     the local parameter shard, rows x cols, row stride ldp elements,
 *       updated in place;
 * d     its update slice, rows x cols, row stride ldd elements, read only
 *       (a view into a delta matrix, or a buffer the shard arrived in).
 * A column block of a row-major matrix is such a view: its first element and
 * the matrix's row stride. */
typedef struct {
  void* p;
  const void* d;
  int64_t rows;
  int64_t cols;
  int64_t ldp;
  int64_t ldd;
} muon_shard;

typedef struct muon_apply_plan_s* muon_apply_plan_t;

/* Builds a static plan over n shards; the TP layout is fixed at
 * initialisation, as the pages' assignment of tensors is. shards is a host
 * array; the plan keeps the device pointers. Every argument is validated
 * before any HIP call. Errors: INVALID_ARG (n < 1, null pointers, rows or
 * cols < 1 or > 2^24, ldp or ldd < cols, more than 2^31 - 1 tiles of 16 rows
 * x 1 KB),
 * ALIGN (p or d not aligned to the element size), ALIAS (an element of a p
 * view is also in another p view or in a d view; d views may share elements),
 * UNSUPPORTED (dtype). Two views with the same row stride are checked element
 * by element (column blocks of one matrix are disjoint); views with different
 * strides whose address ranges overlap are rejected. Then the plan copies its
 * shard table to the current device: HIP or OOM on failure. The call
 * synchronises the device once, at its end. */
muon_status muon_apply_plan(const muon_shard* shards, int32_t n, int32_t dtype,
                            muon_apply_plan_t* out);

/* Enqueues P_local <- P_local + Delta W_local for every shard of the plan on
 * `stream` (a hipStream_t; NULL is the null stream): one kernel, no
 * allocation, no host synchronisation. Each sum is formed in fp32 and stored
 * once (bf16: round to nearest even), which for two values of the storage type
 * is their exactly rounded sum. Shards are independent and the result does not
 * depend on their order. The call may be captured in a HIP graph on `stream`. */
muon_status muon_apply(muon_apply_plan_t plan, void* stream);

/* Frees the plan. NULL is a no-op. Synchronises the device. */
muon_status muon_apply_plan_destroy(muon_apply_plan_t plan);

/* ---------------------------------------------------------------------------
 * MFMA throughput probe (measurement, not part of the step). Enqueues one
 * kernel of `blocks` workgroups of 4 waves on `stream`; every wave issues
 * iters * 8 bf16 MFMAs of 32 x 32 x 16 (32768 flops each) back to back on
 * random register data and stores one sum per lane into out (a device buffer
 * of blocks * 256 floats). Timed by the caller, it gives the bf16 MFMA rate
 * the chip sustains on random data under its power limit, against which the
 * step's rate can be read. It is a measurement aid, not an operation of the
 * pages' method. Errors:
 * INVALID_ARG (out NULL, blocks outside [1, 2^20], iters < 1), HIP. */
muon_status muon_mfma_probe(float* out, int32_t blocks, int32_t iters, void* stream);

/* ---------------------------------------------------------------------------
 * Data-parallel static partition: which whole parameters each DP rank owns
 * (host only, no GPU). A rank's share is the batch it passes to muon_plan.
 *
 * The parameter buffer is a list of n_buckets buckets; bucket i is an ordered
 * run of bucket_len[i] atomic parameters. sizes[] holds the element count of
 * every parameter, bucket after bucket; loads[] (NULL: the sizes) holds its
 * load W(p). On return, cuts[i*(ranks+1) + r] .. cuts[i*(ranks+1) + r+1] - 1
 * are the parameters of bucket i that rank r owns (cuts are parameter indices
 * within the bucket: 0 first, bucket_len[i] last, non-decreasing), and
 * rank_loads[r] (if not NULL) is rank r's total load. Errors: INVALID_ARG
 * (null sizes, bucket_len or cuts; n_buckets < 1; ranks outside [1, 2^20];
 * an empty bucket; a size outside [1, 2^40]; a negative or non-finite load;
 * alpha outside [0, 1]). */

/* The Start_Index rule without load balancing (Canzona analysis page,
 * section 3.4, "Paradigm 3: Static Partitioning"): with S = |B_i| / R, a
 * parameter whose first element lies in [r S, (r+1) S) of its bucket belongs
 * to rank r (evaluated exactly, in integers). */
muon_status muon_dp_partition_static(const int64_t* sizes, const double* loads, const int32_t* bucket_len,
                                     int32_t n_buckets, int32_t ranks, int32_t* cuts, double* rank_loads);

/* The alpha-Balanced Greedy LPT algorithm (same section, "Algorithm 1"):
 * buckets in descending load order (equal loads keep their order); per bucket,
 * deficits d_r = max(0, mu - L_r) against the mean load mu, the target share
 * v_r = (1 - alpha)/R + alpha d_r / sum(d) (1/R when every deficit is 0), and
 * the cut of rank r < R-1 at the parameter boundary whose cumulative load is
 * closest to the cumulative target (the earlier one on a tie, never before
 * rank r-1's cut); the last rank takes the rest. O(N log N + N R log P) for N
 * buckets of at most P parameters. */
muon_status muon_dp_partition(const int64_t* sizes, const double* loads, const int32_t* bucket_len,
                              int32_t n_buckets, int32_t ranks, double alpha, int32_t* cuts, double* rank_loads);

/* TP micro groups (host only; Canzona analysis page, section 3.4, "The TP
 * Hierarchical Partitioning and Scheduling", the LPT with greedy rollback and
 * its min-heap solver). n tensors with costs cost[i] (their ID is i) are
 * sorted by (cost, ID) descending and packed, in that order, into groups: a
 * tensor joins the current group if the min-heap LPT assignment of the group
 * (by cost descending, each tensor to the least-loaded of `ranks` host ranks,
 * the lower rank on a tie) keeps every rank's load within c_max; otherwise the
 * group closes and the tensor starts the next one (a tensor heavier than
 * c_max alone forms its own group). On return order[] holds the IDs in
 * schedule order (every group a consecutive run), group_of[i] and host_of[i]
 * the group and host rank of tensor i, and *n_groups the number of groups.
 * Every tentative group is solved again, as the pages do: O(n K log K) for
 * groups of up to K tensors (milliseconds for thousands of tensors in groups
 * of tens). Errors: INVALID_ARG (null pointers, n < 1, ranks outside [1, 2^20], c_max
 * not finite and > 0, a negative or non-finite cost). */
muon_status muon_tp_micro_groups(const double* cost, int32_t n, int32_t ranks, double c_max, int32_t* order,
                                 int32_t* group_of, int32_t* host_of, int32_t* n_groups);

#ifdef __cplusplus
}
#endif

#endif /* MUON_H_ */
