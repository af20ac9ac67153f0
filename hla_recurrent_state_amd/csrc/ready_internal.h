// Internal interface between the host plan/dispatch code and the gfx950
// kernels of the state reader.  Not installed; the public ABI is ready.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ready.h"

#define READY_MAX_LSEL 64
#define READY_TILE 128            // d_k = d_v
#define READY_TILE_ELEMS (READY_TILE * READY_TILE)

// Arguments of the per-state kernel (steps 1-4 and packing for one
// (sequence, pair) tile per workgroup).
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
  const float* zpart;              // [ksz][B*n][nz] raw partial sums of W_q (gamma*h)
  const float* hss;                // [ksz][B*n] partial sums of h^2
  int ksz, nz;
  void* gathered;                  // [B][M][128][128] state dtype
  float* logrms;                   // [B][M] or null
  float* f;                        // [B*n][F] workspace
  float* feat;                     // [B*n][F] or null
  int32_t* dev_status;             // or null
  int32_t* seq_invalid;            // [B] workspace
};

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
};

#define READY_HIDDEN __attribute__((visibility("hidden")))

READY_HIDDEN hipError_t ready_launch_state(const StateArgs& a, int state_dt, int weight_dt, hipStream_t s);
READY_HIDDEN hipError_t ready_launch_gemm(const GemmArgs& g, int x_dt, int w_dt, int out_dt, int epi,
                             dim3 grid, size_t lds_bytes, hipStream_t s);

// Rows of X staged in LDS per workgroup, and K elements staged per pass.
#define READY_GEMM_RB 8
#define READY_GEMM_KSTAGE 1024
#define READY_GEMM_COLS 16
