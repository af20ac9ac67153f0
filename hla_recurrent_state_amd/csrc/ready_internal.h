// Internal interface between the host plan/dispatch code and the gfx950
// kernels of the state reader.  Not installed; the public ABI is ready.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ready.h"

#define READY_MAX_LSEL 64
#define READY_TILE 128            // d_k = d_v
#define READY_TILE_ELEMS (READY_TILE * READY_TILE)
#define READY_HIDDEN __attribute__((visibility("hidden")))

// Arguments of the per-state kernels (one (sequence, pair) tile per
// workgroup).
struct StateArgs {
  const void* states;
  int64_t sb, sp, sl, sh;          // element strides of the verify buffer
  const int32_t* accept_idx;       // [B]
  int32_t slot[READY_MAX_LSEL];    // buffer layer slot of each selected layer
  int B, P, n, M, H, r, d, F;
  int shared;                      // reader parameters shared by all pairs
  float state_eps, h_eps;
  const void* u;                   // [M][r][128] weight dtype
  const void* v;                   // [M][128][r] weight dtype
  void* gathered;                  // [B][M][128][128] state dtype
  float* logrms;                   // [B][M] or null
  int32_t* dev_status;             // or null
  int32_t* seq_invalid;            // [B] workspace
  // readout from q = U^T z, packing into f
  const float* zpart;              // [ksz][B*n][nz] raw partial sums of W_q (gamma*h)
  const float* hss;                // [ksz][B*n] partial sums of h^2
  int ksz, nz;
  float* f;                        // [B*n][F] workspace
  float* feat;                     // [B*n][F] or null
};

#define READY_MODE_FULL 0
#define READY_MODE_PREPARE 1
#define READY_MODE_APPLY 2
#define READY_MAX_INJ 8            // injections one prepare launch serves

// Fast path (bf16 states, activations and weights; r <= 32): one persistent
// launch, k_reader, whose workgroups run four kinds of work items:
//   Z  query sums z = W_q (gamma h) per 64 x 64 tile and K chunk, and the
//      sums of squares of h
//   S  per (sequence, pair) tile: gather, RMS, log-RMS and
//      P = V^T S_bar U^T / sqrt(d_k)
//   A  per 16 rows and 64 columns of a: f and a = act(W1 f + b1)
//   O  per output tile: out = h + W2 a + b2
struct FastArgs {
  const uint16_t* states;
  int64_t sb, sp, sl, sh;          // element strides of the verify buffer
  const int32_t* accept_idx;       // [B]
  int32_t slot[READY_MAX_LSEL];
  const uint16_t* h;               // [R][d]
  const uint16_t* wq;              // [Nz][d]  (Nz = Mz r)
  const uint16_t* u;               // [Mz][r][128]
  const uint16_t* v;               // [Mz][128][r]
  const uint16_t* gamma;           // [d] or null
  const uint16_t* w1;              // [Hm][F]
  const uint16_t* b1;              // [Hm] or null
  const uint16_t* w2;              // [d][Hm]
  const uint16_t* b2;              // [d] or null
  uint16_t* gathered;              // [B][M][128][128]
  uint16_t* out;                   // [R][d]
  float* logrms;                   // [B][M] or null
  float* delta;                    // [R][d] or null
  float* feat;                     // [R][F] or null
  int32_t* dev_status;             // or null
  float* zpart;                    // [ksplit][R][Nz]
  float* hss;                      // [ksplit][R]
  float* rsv;                       // [R]: 1 / rms(h) per row (from the items completing z column block 0)
  float* zfin;                     // [R][Nz]: z summed over the K chunks (before 1 / rms(h))
  float* fu;                       // [R][Fp]: f rows formed by the state tiles (Fp = F rounded up to 32)
  float* pmat;                     // [B M][r][r]
  float* ell;                      // [B M]
  uint16_t* abuf;                  // [R][Hm] bf16
  uint32_t* seq_invalid;           // [B]
  // Counters, READY_CTR_STRIDE words apart: [0] the workspace magic,
  // [1] abort flag, [2 .. 2 + READY_DONE_GROUPS] workgroups finished per
  // group and overall, then the Z items done per tile of z, the finished
  // tiles of z per row block, the S items done per 16 rows, the A items done
  // per row tile of out, the state-tile tickets, the Z-, A- and O-item
  // claim counters, the arrival flags per XCD.
  // The last workgroup to finish clears all of them except the magic.
  uint32_t* counters;
  int n_counters;                  // words
  uint32_t magic;
  uint32_t* abort_flag;
  uint32_t* done;                  // [READY_DONE_GROUPS + 1]
  uint32_t* zcnt;                  // [cdiv(R, BMZ) * cdiv(Nz, 64)]: Z items done per tile of z
  uint32_t* zdone;                 // [cdiv(R, BMZ)]: tiles of zfin complete per row block
  uint32_t* sdone;                 // [cdiv(R, 16)]
  uint32_t* adone;                 // [cdiv(R, BMO)]
  uint32_t* tk;                    // [READY_TICKET_GROUPS]: positions claimed in the queue of XCD x: its Z
                                   // items first, then the tickets of state-tile group x (tiles t with
                                   // t % READY_TICKET_GROUPS == x)
  uint32_t* arr_x;                 // [8]: a workgroup of the launch has run on XCD x
  uint32_t* aq;                    // [8]: A items claimed per XCD queue
  uint32_t* oq;                    // [8]: O items claimed per XCD queue
  int n_z, n_s, n_a, n_o;          // work items per kind
  int B, P, n, M, H, r, d, F, Hm, R, Nz, shared, ksplit, kchunk, act;
  float state_eps, h_eps;
  // Several readers sharing one gather.  READY_MODE_FULL runs every item
  // kind.  READY_MODE_PREPARE runs only the state tiles and forms one P per
  // injection i, from u_inj[i] and v_inj[i], stored at pmat + i p_inj_stride
  // (u_inj[0] = u, v_inj[0] = v).  READY_MODE_APPLY runs every kind but the
  // state tiles: its A and O items read the P, ell and invalid-sequence flags
  // a prepare launch left (pmat, ell and seq_invalid point there).
  int mode;
  int n_inj;                       // 1 outside READY_MODE_PREPARE
  int64_t p_inj_stride;            // floats
  const uint16_t* u_inj[READY_MAX_INJ];
  const uint16_t* v_inj[READY_MAX_INJ];
};

// fp32 single-launch path (fp32 states, activations and weights; at most 16
// rows, r <= 16): one persistent launch, k_reader_f32, whose workgroups claim
// S, Z, A and O items (see ready_f32.hip) from one counter
struct F32Args {
  const float* states;
  int64_t sb, sp, sl, sh;          // element strides of the verify buffer
  const int32_t* accept_idx;       // [B], B <= 16
  int32_t slot[READY_MAX_LSEL];
  const float* h;                  // [R][d]
  const float* wq;                 // [Nz][d]
  const float* u;                  // [Mz][r][128]
  const float* v;                  // [Mz][128][r]
  const float* gamma;              // [d] or null
  const float* w1;                 // [Hm][F]
  const float* b1;                 // [Hm] or null
  const float* w2;                 // [d][Hm]
  const float* b2;                 // [d] or null
  float* gathered;                 // [B][M][128][128]
  float* out;                      // [R][d] (may be h)
  float* logrms;                   // [B][M] or null
  float* delta;                    // [R][d] or null
  float* feat;                     // [R][F] or null
  int32_t* dev_status;             // or null
  float* zpart;                    // [nks][R][Nz]: partial sums of W_q (gamma h) per K chunk
  float* hss;                      // [ncz][nks][R]: partial sums of h^2 (one copy per column block of z)
  float* fbuf;                     // [R][Fp]: f rows (Fp = F rounded up to 64), formed with z's sums
  float* pmat;                     // [B M][r][r]
  float* ell;                      // [B M]
  float* abuf;                     // [R][Hm]
  uint32_t* seq_invalid;           // [B]
  // Counters, READY_CTR_STRIDE words apart: [0] the workspace magic, [1]
  // abort flag, [2 .. 2 + READY_DONE_GROUPS] workgroups finished per group
  // and overall, then per queue the claim counters of the S and Z items, of
  // the A items and of the O items and the arrival flags, then the finished
  // column blocks of z, the S items done, the A items done and the Z items
  // done per column block.  The last workgroup to finish clears all of them
  // but the magic.
  uint32_t* counters;
  int n_counters;                  // words
  uint32_t magic;
  uint32_t* abort_flag;
  uint32_t* done;
  uint32_t* lq;                    // [READY_F32_QUEUES]: S and Z items claimed per queue
  uint32_t* aq;                    // [READY_F32_QUEUES]: A items claimed per queue
  uint32_t* oq;                    // [READY_F32_QUEUES]: O items claimed per queue
  uint32_t* arr_x;                 // [READY_F32_QUEUES]: a workgroup of the launch has taken from queue x
  uint32_t* zdone;
  uint32_t* sdone;
  uint32_t* adone;
  uint32_t* zcnt;                  // [ncz]
  int n_s, n_z, n_a, n_o;          // work items per kind
  int nks, ncz;                    // K chunks and column blocks of z
  int zsum_a;                      // the A items sum z's K chunks and form f (no summing Z item); zdone
                                   // then counts Z items, else the column blocks of z summed and f formed
  int B, P, n, M, H, r, d, F, Hm, R, Nz, shared, act;
  float state_eps, h_eps;
};
#define READY_F32_QUEUES 64        // claim queues of each item kind (8 per XCD)
#define READY_F32_KC 256           // K chunk of a query item (4 waves x 64)
#define READY_F32_ZC 64            // columns of z per query item (one per lane)
#define READY_F32_AC 16            // columns of a per A item (4 waves x 4)
#define READY_F32_OC 32            // columns of out per O item (2 passes of 4 waves x 4)
#define READY_F32_MAX_F 1024       // W1 row values a lane holds: 16 x 4
#define READY_F32_MAX_HM 512       // W2 row values a lane holds per pass: 8 x 4
#define READY_F32_MAX_RNZ 8192     // query sums of all rows staged in LDS
#define READY_F32_MAX_UNITS 1024   // rows of P (B M r) one A item reads, 4 per thread
#define READY_F32_MAX_LDS (64 * 1024)
// the A items sum z's K chunks themselves when z has at most 256 chunks of
// 16 bytes and every thread sums at most READY_F32_ZSUM_LOADS of them
#define READY_F32_ZSUM_LOADS 8
// dynamic LDS bytes of a k_reader_f32 launch: the largest of its item kinds'
// areas (rows R, rows rounded up to the 8 or 16 the kernel is built for)
inline size_t ready_f32_lds(int r, int R, int Nz, int F, int Hm) {
  const size_t RB = R <= 8 ? 8 : 16;
  const size_t s_f = (size_t)r * (READY_TILE + 4) + (size_t)READY_TILE * r + 4 * 8 * (READY_TILE + 4) + 4;
  const size_t z_f = RB * READY_F32_KC + 4 * RB * 64;
  const size_t fa = RB * (((size_t)F + 63) & ~(size_t)63);
  const size_t a_f = (((size_t)R * Nz + 3) & ~(size_t)3) + (fa > 1040 ? fa : 1040);
  const size_t o_f = RB * (((size_t)Hm + 63) & ~(size_t)63) + 16;
  size_t m = s_f;
  if (z_f > m) m = z_f;
  if (a_f > m) m = a_f;
  if (o_f > m) m = o_f;
  return 4 * m;
}

#define READY_FAST_MAX_F 1536      // f rows of 16 positions staged in LDS
#define READY_FAST_MAX_NZ 1024     // query sums of 16 positions staged in LDS
#define READY_CTR_STRIDE 32        // counters sit 128 bytes apart
#define READY_DONE_GROUPS 16
#define READY_WS_MAGIC 0x52454459u // "READY"
// k_reader tiles: z in BMZ x 64 tiles over K chunks of READY_ZCHUNK_* (a
// multiple of 128), out in BMO x READY_OCOLS tiles; BMZ = BMO = 16 for at
// most 16 rows, else READY_BMZ_LARGE and READY_BMO_LARGE.  Apply launches
// use READY_BMZ_APPLY and READY_BMO_APPLY: with no state stream beside them,
// more query items spread the query sums over more workgroups, and fewer,
// larger output items cost less than shorter ones would save
#define READY_BMZ_LARGE 64
#define READY_BMZ_APPLY 32
#define READY_BMO_LARGE 32
#define READY_BMO_APPLY 64
#define READY_ZCHUNK_SMALL 384
#define READY_ZCHUNK_LARGE 640
#define READY_OCOLS 128
// columns of out per O item at most 16 rows (more, shorter items where the
// O items follow a short chain)
#ifndef READY_OCOLS_SMALL
#define READY_OCOLS_SMALL 64
#endif
#define READY_ABM 8                // rows of an A item (and of a state-tile count)
#ifndef READY_UPATH_MIN_R
#define READY_UPATH_MIN_R 24        // the state tiles form f themselves from this rank on
#endif
#define READY_TICKET_GROUPS 8     // state-tile ticket counters, one per XCD
#define READY_ACC_LDS 1024        // accept indices staged in LDS

// Step 1 alone: one workgroup per (sequence, pair) tile
struct GatherArgs {
  const void* states;
  int64_t sb, sp, sl, sh;          // element strides of the verify buffer
  const int32_t* accept_idx;       // [B]
  int32_t slot[READY_MAX_LSEL];
  int B, P, M, H;
  int esize;                       // bytes per state element (2 or 4)
  void* gathered;                  // [B][M][128][128]
  int32_t* dev_status;             // or null
};
READY_HIDDEN hipError_t ready_launch_gather(const GatherArgs& a, hipStream_t s);

// Verify-state producer: one workgroup per (sequence, pair)
struct VerifyArgs {
  const void* state_t;             // [B][M][128][128] state dtype
  const void* k;                   // [B][P-1][M][128] kv dtype
  const void* v;                   // [B][P-1][M][128] kv dtype
  const float* alpha;              // [B][P-1][M]
  const float* beta;               // [B][P-1][M]
  void* out;                       // verify buffer, state dtype
  int64_t sb, sp, sl, sh;          // its element strides
  int B, P, M, H;
};
READY_HIDDEN hipError_t ready_launch_verify(const VerifyArgs& a, int state_dt, int kv_dt, hipStream_t s);
READY_HIDDEN size_t ready_verify_lds(int P);

enum { EPI_PARTIAL = 0, EPI_BIAS_ACT = 1, EPI_RESID = 2 };

// Y[rho][c] = sum_k X[rho][k] W[c][k] over rows rho < R, columns c < N,
// with the K range split over blockIdx.y in chunks of kchunk.
struct GemmArgs {
  const void* X;
  int64_t ldx;
  const void* W;
  int64_t ldw;
  int R, N, K;
  int kchunk;
  int vec_ok;                      // W rows and chunks are 16-byte aligned
  // query GEMM only: RMSNorm gain and partial sums of squares of the raw rows
  const void* gamma;               // [K] weight dtype or null
  float* hss;                      // [ksplit][R] (written by column block 0)
  // EPI_PARTIAL
  float* ypart;                    // [ksplit][R][N]
  // EPI_BIAS_ACT
  const void* bias;                // [N] weight dtype or null
  int act;
  float* yout;                     // [R][N]
  // EPI_RESID (bias in `bias`)
  const void* h;                   // [R][N] act dtype
  void* out;                       // [R][N] act dtype (may equal h)
  float* delta;                    // [R][N] or null
  const int32_t* seq_invalid;      // [R / n]
  int n;
  int epi_vec;                     // k_gemm_mm residual: N % 8 == 0 and h, out, delta 16-byte aligned
  int tiles_c, tiles_r;            // k_gemm_mm: column and row tiles (set by its launcher)
  int wave_k;                      // k_gemm: 4 columns per workgroup, K split over its waves
};

// VALU skinny GEMM tiling
#define READY_GEMM_RB 8           // rows of X per workgroup
#define READY_GEMM_KSTAGE 1024    // K elements staged in LDS per pass
#define READY_GEMM_COLS 16        // output columns per workgroup
// MFMA GEMM tiling
#define READY_MFMA_BN 64
#define READY_MFMA_BK 64

// Every launcher takes a pair of caller events (or nulls): when either is
// set, the kernel is launched with hipExtLaunchKernelGGL, which records the
// start and stop of that kernel itself, with no marker packet in between.
struct StageEvents {
  hipEvent_t start, stop;
};

READY_HIDDEN hipError_t ready_launch_state(const StateArgs& a, int state_dt, int weight_dt, hipStream_t s,
                                           StageEvents ev);
// bf16 states and weights: matrix-core per-state kernel, `grid` persistent
// workgroups (at most one per CU)
READY_HIDDEN hipError_t ready_launch_state_mm(const StateArgs& a, int grid, hipStream_t s, StageEvents ev);
READY_HIDDEN hipError_t ready_launch_gemm(const GemmArgs& g, int x_dt, int w_dt, int out_dt, int epi,
                                          dim3 grid, size_t lds_bytes, hipStream_t s, StageEvents ev);
// 128 x 128 tiles for large row counts; weights must be bf16
READY_HIDDEN hipError_t ready_launch_gemm_mm(const GemmArgs& g, int x_dt, int out_dt, int epi, int ksplit,
                                             hipStream_t s, StageEvents ev);
// yout = act(sum of ksplit partial sums in ypart + bias)
READY_HIDDEN hipError_t ready_launch_reduce_bias_act(const GemmArgs& g, int ksplit, hipStream_t s, StageEvents ev);
#define READY_GM_TILE 128         // k_gemm_mm tile rows and columns
#define READY_GM_BK 64            // k_gemm_mm K step
// bm: rows per workgroup tile (16 or 64); weights must be bf16
READY_HIDDEN hipError_t ready_launch_gemm_mfma(const GemmArgs& g, int x_dt, int out_dt, int epi, int bm,
                                               dim3 grid, hipStream_t s, StageEvents ev);
// fast path; small: at most 16 rows (16-row tiles), else the large tiles
READY_HIDDEN hipError_t ready_launch_reader(const FastArgs& a, int small, int grid, hipStream_t s, StageEvents ev);
// fp32 single-launch path: `grid` workgroups (two per CU at most)
READY_HIDDEN hipError_t ready_launch_reader_f32(const F32Args& a, int grid, size_t lds, hipStream_t s,
                                                StageEvents ev);
READY_HIDDEN hipError_t ready_launch_ws_init(uint32_t* counters, int n_counters, uint32_t magic, hipStream_t s);

// Where a call's scratch lives: `data` holds every scratch array at the plan's
// offsets (data_bytes of them), `ctr` the synchronisation counters (ctr_bytes),
// whose first word must equal `magic`.  For a caller's workspace both sit in
// it (the counters at the end, the magic tied to the plan); the no-allocation
// entry point places them in the library's static per-device array.
struct WsView {
  char* data;
  uint32_t* ctr;
  uint32_t magic;
  size_t data_bytes, ctr_bytes;
};

// Called once the arguments of a call have passed validation and before
// anything is enqueued: fills in the final scratch view (for the static array:
// its device address on the current device, cleared counters on first use).
typedef readyStatus (*WsResolve)(WsView* view, hipStream_t stream);

extern "C" {
// readyStateReader with the scratch given by `sv` (sv == nullptr: the caller's
// workspace, validated as readyStateReader documents).  With `resolve`, the
// aliasing checks use sv's ranges as given and `resolve` then supplies the
// view the launches use.
READY_HIDDEN readyStatus ready_run_reader(const readyPlan* plan, const readyStates* states,
                                          const int32_t* accept_idx, const void* h, const readyWeights* w,
                                          const readyOutputs* o, void* workspace, size_t workspace_bytes,
                                          void* stream, void* const* events, const WsView* sv,
                                          WsResolve resolve);
// Scratch bytes a plan's calls use: the arrays, then the counters
READY_HIDDEN void ready_plan_scratch_needs(const readyPlan* plan, size_t* data_bytes, size_t* ctr_bytes);
}
// dynamic LDS bytes of a k_reader launch: the largest of its item kinds' areas
inline size_t ready_reader_lds(int r, int F, int Nz, int small) {
  // the O item's area is sized for the larger of the two large-row forms
  const int BMZ = small ? 16 : (READY_BMZ_APPLY > READY_BMZ_LARGE ? READY_BMZ_APPLY : READY_BMZ_LARGE);
  const int BMO = small ? 16 : (READY_BMO_APPLY > READY_BMO_LARGE ? READY_BMO_APPLY : READY_BMO_LARGE);
  const int NB = (r + 15) / 16;
  const size_t z_bytes = (size_t)(BMZ + 64) * 256 + 16;
  const size_t s_bytes = (size_t)READY_TILE_ELEMS * 2 + (size_t)r * (READY_TILE + 8) * 2 + (size_t)READY_TILE * r * 2 +
                         4 * (4 * NB * r * 16 + 4) + 4 * ((size_t)r * r + 16 * (size_t)r + 16 + 4);
  const int Fs = ((F + 31) & ~31) + 8;
  const size_t a_bytes = (size_t)READY_ABM * Nz * 4 + (size_t)16 * Fs * 2 + 4 * 16 + 16;
  const size_t sa = (size_t)BMO * (256 + 8) * 2, so = (size_t)BMO * (READY_OCOLS + 4) * 4;
  const size_t o_bytes = (sa > so ? sa : so) + 16;
  size_t m = z_bytes;
  if (s_bytes > m) m = s_bytes;
  if (a_bytes > m) m = a_bytes;
  if (o_bytes > m) m = o_bytes;
  return (m + 15) & ~(size_t)15;
}
READY_HIDDEN int ready_reader_per_cu(int r, int small, size_t lds, int mode);
