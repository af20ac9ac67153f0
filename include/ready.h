/*
 * ready.h -- C ABI of the ReaDy state-reader library for AMD Instinct MI355X
 * (gfx950).
 *
 * The state reader conditions a block of n draft representations h_j on the
 * committed Gated DeltaNet states of a hybrid-linear-attention target
 * (ReaDy arXiv text, section 3.1 "State-Conditioned Block Drafting"; rainbus
 * summary, 方法步骤详情; onedev summary, 어떻게 동작하나).  One call runs, for
 * B independent sequences:
 *
 *   1. gather     G[b][m] = states[b][accept_idx[b]][layer_ids[l]][a],
 *                 m = l*H + a, written to a caller-preallocated buffer
 *                 (arXiv text, section 3.2 "Avoiding redundant data movement";
 *                 section 3.1 "Drafting, verification, and commitment").
 *   2. prepare    rms = sqrt(mean(G^2) + state_eps), S_bar = G / rms,
 *                 ell = ln(rms)  (section 3.1 "Position-conditioned reading",
 *                 "Fusion and residual injection").
 *   3. project    T = V^T S_bar, r x d_k, once per state (section 3.1;
 *                 section 3.2 "State-access footprint").
 *   4. query      h_hat = gamma * h_j / sqrt(mean(h_j^2) + h_eps),
 *                 z = W_q h_hat, q = U^T z, u = T q / sqrt(d_k)
 *                 (section 3.1, Eq. (3), written out in the rainbus summary,
 *                 方法步骤详情 step (2)).
 *   5. fuse       f_j = [u^0, ell_0, u^1, ell_1, ...] (M (r+1) values),
 *                 Delta h = W2 act(W1 f + b1) + b2, out = h + Delta h
 *                 (section 3.1 "Fusion and residual injection", Eq. (4)).
 *
 * Conventions for every function:
 *   - All functions are extern "C", never throw, and return a readyStatus.
 *   - Argument errors are detected on the host before anything is launched;
 *     on error nothing is launched and no output is touched.
 *   - Device pointers are caller-owned memory on the current HIP device.  The
 *     library never allocates, frees or copies device memory and never
 *     synchronises the stream on the call path.
 *   - "elements" counts values of the array's own dtype.
 */
#ifndef READY_H
#define READY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define READY_VERSION 100 /* 1.0.0 */

typedef enum readyStatus {
  READY_OK = 0,
  READY_ERR_NULL_POINTER = 1,       /* a required pointer is NULL */
  READY_ERR_BAD_SHAPE = 2,          /* a size is out of the supported range */
  READY_ERR_UNSUPPORTED_DTYPE = 3,  /* a dtype / activation code is unknown */
  READY_ERR_MISALIGNED = 4,         /* a pointer or outer stride is not 16-byte aligned */
  READY_ERR_WORKSPACE_TOO_SMALL = 5,
  READY_ERR_ALIASING = 6,           /* outputs overlap inputs in a forbidden way */
  READY_ERR_LAYER_ID_RANGE = 7,     /* a layer id is outside [0, L_tot) */
  READY_ERR_HIP = 8,                /* the HIP runtime reported an error at launch */
  READY_ERR_ACCEPT_IDX = 9,         /* device-side only: accept_idx[b] outside [0, P) */
  READY_ERR_OUT_OF_HOST_MEMORY = 10,
  READY_ERR_SYNC_TIMEOUT = 11,      /* device-side only: a wait between work items of one launch
                                       gave up (should never happen; outputs are then invalid) */
  READY_ERR_WORKSPACE_UNINIT = 12,  /* device-side only: the workspace was not prepared by
                                       readyWorkspaceInit for this plan; nothing was computed */
  READY_ERR_UNSUPPORTED = 13,       /* the operation is not available for this plan's dtypes and rank
                                       (readyPrepSize, readyStatePrepare, readyStateApply), or
                                       readyStateReaderStatic's first call on a device was made
                                       while its stream was capturing */
  READY_ERR_STATIC_SCRATCH_TOO_SMALL = 14, /* readyStateReaderStatic: the plan needs more scratch than
                                       the library's static per-device array holds */
  /* range markers, not status codes: they make every int32_t a value of the
     type, so that readyStatusString may be passed any code a C caller holds */
  READY_STATUS_RANGE_MIN = -2147483647 - 1,
  READY_STATUS_RANGE_MAX = 2147483647
} readyStatus;

typedef enum readyDtype { READY_F32 = 0, READY_BF16 = 1 } readyDtype;

/*
 * Kernel path.  READY_PATH_FUSED runs the whole call as one persistent kernel
 * where it can (bf16 states, activations and weights, r <= 32) and as four
 * launches otherwise.  READY_PATH_UNFUSED always runs the four launches
 * (query sums; gather, RMS, log-RMS, projection and readout; first MLP layer;
 * second MLP layer and residual): a comparator and a debugging aid with the
 * same outputs and tolerance.
 */
typedef enum readyPath { READY_PATH_FUSED = 0, READY_PATH_UNFUSED = 1 } readyPath;

/* Activation of the bottleneck MLP (the pages do not name it; SiLU default). */
typedef enum readyAct { READY_ACT_SILU = 0, READY_ACT_GELU_TANH = 1, READY_ACT_RELU = 2 } readyAct;

/*
 * Problem shape.  Supported ranges (READY_ERR_BAD_SHAPE otherwise):
 *   B >= 0 (B = 0 is a valid no-op), B * n <= 1 << 20
 *   1 <= P <= 64 positions per verify buffer (root + drafts; the pages use 8)
 *   1 <= n <= 16 draft positions per block (the pages use 7)
 *   1 <= L_sel <= 64 selected layers, 1 <= L_tot, 1 <= H, M = L_sel * H <= 4096
 *   d_k = d_v = 128 (the pages' per-head state size)
 *   r in {8, 16, 24, ..., 128} (multiple of 8; the pages use 8 and 128)
 *   d >= 8 and a multiple of 8; 1 <= Hm <= 4096
 * Dtypes: state_dtype (states, gathered), act_dtype (h, out), weight_dtype
 * (W_q, U, V, gamma, W1, b1, W2, b2), each READY_F32 or READY_BF16.
 * Arithmetic is fp32 throughout; bf16 values are widened exactly.
 */
typedef struct readyShape {
  int32_t B, P, n;
  int32_t L_tot, L_sel, H;
  int32_t d_k, d_v, r, d, Hm;
  int32_t state_dtype, act_dtype, weight_dtype;
  int32_t act;             /* readyAct */
  int32_t shared_params;   /* 0: W_q, U, V stacked per pair; 1: one set for all pairs */
  float state_eps;         /* added to mean(S^2); the pages are silent, 1e-6 suggested */
  float h_eps;             /* added to mean(h^2) in RMSNorm(h); 1e-6 suggested */
  int32_t path;            /* readyPath: READY_PATH_FUSED (0, default) or READY_PATH_UNFUSED */
} readyShape;

/*
 * Verify-step per-position state buffer (read only).  Element
 * [b][p][slot][a][v][k] is at base + b*stride_b + p*stride_p + slot*stride_l
 * + a*stride_h + v*128 + k: each 128 x 128 tile is contiguous, value-by-key
 * (row v = value index, column k = key index; arXiv text, section 3.1
 * "State interface").  Strides are in elements and must keep every tile
 * 16-byte aligned.
 */
typedef struct readyStates {
  const void* base;
  int64_t stride_b, stride_p, stride_l, stride_h;
} readyStates;

/*
 * Reader weights, all in weight_dtype, row-major, device memory (wq, u, v,
 * h_gamma, w1, w2 and b2 16-byte aligned):
 *   wq [M][r][d] (or [r][d] when shared_params)  -- z = W_q h_hat
 *   u  [M][r][d_k] (or [r][d_k])                  -- q = U^T z
 *   v  [M][d_v][r] (or [d_v][r])                  -- T = V^T S_bar
 *   h_gamma [d] or NULL (gain of RMSNorm(h), ones when NULL)
 *   w1 [Hm][F], F = M (r + 1); b1 [Hm] or NULL
 *   w2 [d][Hm]; b2 [d] or NULL
 */
typedef struct readyWeights {
  const void* wq;
  const void* u;
  const void* v;
  const void* h_gamma;
  const void* w1;
  const void* b1;
  const void* w2;
  const void* b2;
} readyWeights;

/*
 * Outputs (device memory, caller-owned):
 *   gathered  [B][M][d_v][d_k] in state_dtype (required).  Must not overlap
 *             the states' address range.
 *   out       [B][n][d] in act_dtype (required): h + Delta h, rounded to
 *             nearest even for bf16.  May be exactly h (in place); any other
 *             overlap with an input is READY_ERR_ALIASING.
 *   logrms    [B][M] fp32 ell = ln rms (optional, NULL to skip)
 *   delta     [B][n][d] fp32 Delta h before the residual (optional,
 *             16-byte aligned)
 *   feat      [B][n][F] fp32 packed features f_j (optional, 16-byte aligned)
 *   dev_status  one int32 (optional).  When accept_idx[b] is outside [0, P)
 *             the kernels store READY_ERR_ACCEPT_IDX there and leave that
 *             sequence's gathered, logrms, out and delta unwritten (its feat
 *             row is zero).  The library never clears it; the caller does.
 */
typedef struct readyOutputs {
  void* gathered;
  void* out;
  float* logrms;
  float* delta;
  float* feat;
  int32_t* dev_status;
} readyOutputs;

typedef struct readyPlan readyPlan;

/*
 * Validate a shape and the selected layer slots, and build a plan.
 * layer_ids: host array of L_sel slots on the buffer's layer axis (each in
 * [0, L_tot); repeats allowed).  The plan copies what it needs; it is
 * immutable afterwards and may be used from several host threads.  This is the
 * only function that allocates (host memory, for the plan).
 */
readyStatus readyPlanCreate(const readyShape* shape, const int32_t* layer_ids, readyPlan** plan);

/* Release a plan (NULL is accepted). */
readyStatus readyPlanDestroy(readyPlan* plan);

/* Bytes of device workspace readyStateReader needs for this plan. */
readyStatus readyWorkspaceSize(const readyPlan* plan, size_t* bytes);

/*
 * Kernel launches one readyStateReader call makes with this plan, into
 * *launches: 1 where the whole reader runs as one persistent kernel (bf16
 * states, activations and weights with r <= 32; fp32 throughout with at most
 * 16 rows B n and r <= 16, the serving shapes), 4 or 5 on the general path
 * (query GEMM, per-state kernel, MLP layer 1, whose K-split form adds a
 * reduction, MLP layer 2 with the residual).  Host only.  Returns
 * READY_ERR_NULL_POINTER for a null argument.
 */
readyStatus readyPlanLaunches(const readyPlan* plan, int32_t* launches);

/*
 * Prepare a workspace for use with `plan`: enqueue on `stream` a small kernel
 * that clears the synchronisation counters the state reader keeps in the
 * workspace and stamps it for this plan.  Call it once after allocating the
 * workspace (and again before using the workspace with a different plan);
 * every readyStateReader call leaves the counters cleared for the next call.
 * A call on an unprepared workspace computes nothing and stores
 * READY_ERR_WORKSPACE_UNINIT in the caller's device status word.  The
 * function allocates nothing and does not synchronise.  Returns
 * READY_ERR_NULL_POINTER, READY_ERR_MISALIGNED (workspace not 256-byte
 * aligned), READY_ERR_WORKSPACE_TOO_SMALL or READY_ERR_HIP.
 */
readyStatus readyWorkspaceInit(const readyPlan* plan, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Run steps 1-5 for every sequence, asynchronously on `stream` (a
 * hipStream_t; NULL = the default stream).  accept_idx: device int32 [B].
 * h: device [B][n][d] in act_dtype.  workspace: device memory of at least
 * readyWorkspaceSize() bytes, 256-byte aligned, prepared once by
 * readyWorkspaceInit, used as scratch by this call only (concurrent calls
 * need separate workspaces).  The enqueued work
 * allocates nothing and synchronises nothing, so it may be captured into a
 * HIP graph.  Returns READY_ERR_HIP if a launch fails.
 * Calls on different streams (each with its own workspace) may run at the
 * same time as each other and as other kernels: the single-kernel path
 * claims all of its work items from counters in the workspace and never
 * needs its whole grid resident at once, so a launch completes whatever part
 * of the GPU it gets.  Its waits between work items are bounded all the same:
 * should one last about half a second (never expected), the call stops
 * waiting, its outputs are invalid and READY_ERR_SYNC_TIMEOUT is stored in
 * outputs->dev_status -- the only place this failure shows, so callers that
 * need to detect it pass a status word.
 */
readyStatus readyStateReader(const readyPlan* plan, const readyStates* states,
                             const int32_t* accept_idx, const void* h,
                             const readyWeights* weights, const readyOutputs* outputs,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Same computation as readyStateReader, with kernel timestamps: events[2 i]
 * and events[2 i + 1] (hipEvent_t, or NULL to skip) are recorded at the
 * start and at the end of the kernel of launch stage i itself (the launch
 * records them; no marker packet is inserted between stages).  On the bf16
 * path (bf16 states, activations and weights, r <= 32) the whole call is one
 * kernel: stage 1 carries its start and end, and the events of stages 0, 2
 * and 3 are recorded right after it.  On the general path the stages are
 * 0 query GEMM, 1 per-state kernel (gather, RMS, log-RMS, projection,
 * readout, packing), 2 first MLP layer, 3 second MLP layer and residual.
 * The events must have been created by the caller on the device of `stream`
 * with timing enabled; the library only records them.
 */
#define READY_STAGES 4
readyStatus readyStateReaderProfiled(const readyPlan* plan, const readyStates* states,
                                     const int32_t* accept_idx, const void* h,
                                     const readyWeights* weights, const readyOutputs* outputs,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     void* const* events);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the same
 * computation as readyStateReader (same kernels, bitwise the same outputs),
 * with no workspace argument.  Its scratch is a static device array of
 * READY_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends: the first READY_STATIC_COUNTER_BYTES hold the
 * synchronisation counters, the rest the arrays readyWorkspaceSize counts.
 *   Arguments, layouts, ownership and device-side errors as for
 *   readyStateReader.
 *   READY_ERR_STATIC_SCRATCH_TOO_SMALL: the plan's arrays need more than
 *   READY_STATIC_SCRATCH_BYTES - READY_STATIC_COUNTER_BYTES bytes, or its
 *   counters more than READY_STATIC_COUNTER_BYTES (readyWorkspaceSize gives
 *   their sum; every plan whose workspace is at most 15 MiB fits).  Nothing
 *   is launched.
 *   The first call on a device looks up the array's address on that device
 *   (READY_ERR_HIP on failure) and enqueues, on `stream` before the reader,
 *   a small kernel that clears the counters.  That first call must not be
 *   made while `stream` is capturing a graph (READY_ERR_UNSUPPORTED); later
 *   calls may be captured.
 *   Every call on one device shares that device's array, which keeps the
 *   last call's contents; each call leaves the counters cleared, so calls
 *   one after another (one stream, or streams ordered by events) may use any
 *   plans.  Calls that overlap in time on one device race on the array and
 *   give wrong results.
 * Allocates nothing (no hipMalloc, hipFree or allocating library call) and
 * never synchronises.
 */
#define READY_STATIC_SCRATCH_BYTES (16u << 20)
#define READY_STATIC_COUNTER_BYTES (64u << 10)
readyStatus readyStateReaderStatic(const readyPlan* plan, const readyStates* states,
                                   const int32_t* accept_idx, const void* h,
                                   const readyWeights* weights, const readyOutputs* outputs, void* stream);

/*
 * Step 1 alone: gathered[b][m] = states[b][accept_idx[b]][layer_ids[l]][a]
 * (m = l H + a) for every sequence and selected layer-head pair, a bit copy
 * into the caller's preallocated buffer (arXiv text, section 3.2 "Avoiding
 * redundant data movement"; section 3.1 "Drafting, verification, and
 * commitment").  readyStateReader does the same copy fused with the later
 * steps; this entry point is for callers that want only the committed states.
 *   states, accept_idx  as for readyStateReader (plan's B, P, L_tot, H,
 *                       layer slots and state_dtype).
 *   gathered   [B][M][d_v][d_k] in state_dtype, 16-byte aligned; must not
 *              overlap the states, accept_idx or dev_status.
 *   dev_status one int32 or NULL: an accept index outside [0, P) stores
 *              READY_ERR_ACCEPT_IDX there and leaves that sequence's tiles.
 * Asynchronous on `stream`; allocates and synchronises nothing.  Returns
 * READY_ERR_NULL_POINTER, READY_ERR_BAD_SHAPE (negative stride),
 * READY_ERR_MISALIGNED, READY_ERR_ALIASING or READY_ERR_HIP.
 */
readyStatus readyGather(const readyPlan* plan, const readyStates* states, const int32_t* accept_idx, void* gathered,
                        int32_t* dev_status, void* stream);

/*
 * Several readers sharing one gather.  The pages compare drafters with one
 * reader (final draft layer) and with readers injected into draft layers
 * (0, 2, 4) or all five, each reader with its own parameters (arXiv text,
 * section 4 "Number of injections", Table 5).  Every reader of a block reads
 * the same committed states, and the h of a later draft layer exists only
 * after the earlier layers have run, so the work splits in two:
 *
 *   readyStatePrepare  steps 1-3 once for every reader: each committed tile
 *                      is read once, gathered, and its ell = ln rms and, for
 *                      every reader i, P_i = V_i^T S_bar U_i^T / sqrt(d_k)
 *                      (r x r; u = P_i z_j is T_i q_j / sqrt(d_k) with
 *                      T_i = V_i^T S_bar and q_j = U_i^T z_j, reassociated)
 *                      are left in a caller buffer `prep`.
 *   readyStateApply    steps 4-5 of reader i for its own h: z = W_q,i
 *                      RMSNorm(h), u = P_i z, f, MLP and residual.  It reads
 *                      no state.
 * readyStateApply(i) gives the outputs readyStateReader gives with reader i's
 * weights and the same states (the same arithmetic in the same order).
 * Available when readyStateReader runs as one kernel: bf16 states,
 * activations and weights, r <= 32 (READY_ERR_UNSUPPORTED otherwise).
 *
 * Bytes of the prepared-state buffer for n_inj readers (1 <= n_inj <= 8):
 * 4 (n_inj B M r^2 + B M + B) rounded up per section to 256.
 */
readyStatus readyPrepSize(const readyPlan* plan, int32_t n_inj, size_t* bytes);

/*
 * Steps 1-3 for n_inj readers, asynchronously on `stream`.
 *   states, accept_idx  as for readyStateReader.
 *   inj_weights  host array of n_inj readyWeights; only u and v are read
 *                (device, 16-byte aligned, layouts as in readyWeights).
 *   gathered     [B][M][d_v][d_k] bf16 (required); logrms [B][M] fp32 and
 *                dev_status one int32 (optional), as in readyOutputs.
 *   prep         device, 256-byte aligned, at least readyPrepSize(n_inj)
 *                bytes; written.  Its contents are meaningful only to
 *                readyStateApply with the same plan and n_inj.
 *   workspace    as for readyStateReader (prepared by readyWorkspaceInit).
 * An accept index outside [0, P) stores READY_ERR_ACCEPT_IDX in dev_status,
 * leaves that sequence's gathered and logrms unwritten and marks the sequence
 * in prep, so that readyStateApply leaves its out and delta unwritten.
 * Returns READY_ERR_NULL_POINTER, READY_ERR_UNSUPPORTED, READY_ERR_BAD_SHAPE
 * (n_inj), READY_ERR_WORKSPACE_TOO_SMALL (workspace or prep),
 * READY_ERR_MISALIGNED, READY_ERR_ALIASING (outputs overlapping inputs or
 * each other) or READY_ERR_HIP.  Allocates and synchronises nothing.
 */
readyStatus readyStatePrepare(const readyPlan* plan, const readyStates* states, const int32_t* accept_idx,
                              int32_t n_inj, const readyWeights* inj_weights, void* gathered, float* logrms,
                              int32_t* dev_status, void* prep, size_t prep_bytes, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * Steps 4-5 of reader `inj` (0 <= inj < n_inj, n_inj as given to
 * readyStatePrepare), asynchronously on `stream`, after the prepare call on
 * the same stream (or ordered after it).  prep (prep_bytes, at least
 * readyPrepSize(n_inj)) is read only.
 *   h        device [B][n][d] bf16: the draft representations at this
 *            reader's injection site.
 *   weights  reader inj's wq, h_gamma, w1, b1, w2, b2 (u and v are not
 *            read: they are folded into P).
 *   outputs  out (required; may be exactly h), delta, feat and dev_status
 *            (optional) as in readyOutputs; gathered and logrms are ignored.
 *   workspace  as for readyStateReader.  Calls that share a workspace must
 *            run one after another (the same stream does that).
 * Returns READY_ERR_NULL_POINTER, READY_ERR_UNSUPPORTED, READY_ERR_BAD_SHAPE
 * (n_inj or inj), READY_ERR_WORKSPACE_TOO_SMALL (workspace or prep), READY_ERR_MISALIGNED,
 * READY_ERR_ALIASING or READY_ERR_HIP.  Allocates and synchronises nothing.
 */
readyStatus readyStateApply(const readyPlan* plan, const void* prep, size_t prep_bytes, int32_t n_inj, int32_t inj,
                            const void* h, const readyWeights* weights, const readyOutputs* outputs,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Verify buffer written by readyVerifyStates: element [b][p][l][a][v][k] at
 * base + b*stride_b + p*stride_p + l*stride_l + a*stride_h + v*128 + k, the
 * same layout readyStates describes for reading.
 */
typedef struct readyVerifyBuffer {
  void* base;
  int64_t stride_b, stride_p, stride_l, stride_h;
} readyVerifyBuffer;

/*
 * Verify-state producer, the step just upstream of the gather: for every
 * sequence b and layer-head pair m = l*H + a, write the P per-position states
 * of the verify block into layers 0 .. L-1 of the verify buffer:
 *   S_{t+0} = S_t                                           (a bit copy)
 *   S_{t+p} = alpha_p S_{t+p-1} + beta_p (v_p - alpha_p S_{t+p-1} k_p) k_p^T,
 *             p = 1 .. P-1
 * i.e. S_{t+p-1} A_p + B_p with A_p = alpha_p (I - beta_p k_p k_p^T),
 * B_p = beta_p v_p k_p^T: the gated delta rule (arXiv text, Appendix D.1),
 * applied to the positions of one verify step (section 3.1 "Drafting,
 * verification, and commitment"); Proposition 2 (Appendix A.2) writes the
 * same states as S_t P_j + W_j.
 *   B >= 0 (0 is a no-op), 1 <= P <= 64, L >= 1, H >= 1, L * H <= 4096.
 *   state_dtype (S_t and the buffer) and kv_dtype (k, v): READY_F32 or
 *   READY_BF16.  Arithmetic is fp32: the chain continues in fp32 and each
 *   state is rounded to state_dtype (nearest even) only when stored.
 *   state_t  device [B][L*H][128][128], value-by-key, 16-byte aligned.
 *   k, v     device [B][P-1][L*H][128]; entry [b][p-1] drives step p.  May be
 *            NULL when P = 1.  16-byte aligned.
 *   alpha, beta  device fp32 [B][P-1][L*H] (decay gate and write strength);
 *            may be NULL when P = 1.
 *   out      the verify buffer (its base and outer strides keep every tile
 *            16-byte aligned); written, must not overlap any input.
 * Asynchronous on `stream`; allocates and synchronises nothing.  Returns
 * READY_ERR_NULL_POINTER, READY_ERR_BAD_SHAPE, READY_ERR_UNSUPPORTED_DTYPE,
 * READY_ERR_MISALIGNED, READY_ERR_ALIASING or READY_ERR_HIP.
 */
readyStatus readyVerifyStates(int32_t B, int32_t P, int32_t L, int32_t H, int32_t state_dtype, int32_t kv_dtype,
                              const void* state_t, const void* k, const void* v, const float* alpha,
                              const float* beta, const readyVerifyBuffer* out, void* stream);

/* Static, human-readable name of a status code. */
const char* readyStatusString(readyStatus status);

/* READY_VERSION of the built library. */
int32_t readyVersion(void);

#ifdef __cplusplus
}
#endif

#endif /* READY_H */
