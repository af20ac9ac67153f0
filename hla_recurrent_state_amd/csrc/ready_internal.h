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
  // coupled form (k_state): readout from q = U^T z, packing into f
  const float* zpart;              // [ksz][B*n][nz] raw partial sums of W_q (gamma*h)
  const float* hss;                // [ksz][B*n] partial sums of h^2
  int ksz, nz;
  float* f;                        // [B*n][F] workspace
  float* feat;                     // [B*n][F] or null
  // decoupled form (k_state_p): P = V^T S_bar U^T / sqrt(d_k) and ell per tile
  float* pmat;                     // [B*M][r][r]
  float* ell;                      // [B*M]
};

// Packing of f_j from P, the raw query sums and ell (decoupled form).
struct FeatArgs {
  const float* pmat;               // [B*M][r][r]
  const float* ell;                // [B*M]
  const float* zpart;              // [ksz][R][nz]
  const float* hss;                // [ksz][R]
  int ksz, nz, R, n, M, r, F, d, shared;
  float h_eps;
  float* f;                        // [R][F]
  float* feat;                     // [R][F] or null
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

// VALU skinny GEMM tiling
#define READY_GEMM_RB 8           // rows of X per workgroup
#define READY_GEMM_KSTAGE 1024    // K elements staged in LDS per pass
#define READY_GEMM_COLS 16        // output columns per workgroup
// MFMA GEMM tiling
#define READY_MFMA_BN 64
#define READY_MFMA_BK 64

READY_HIDDEN hipError_t ready_launch_state(const StateArgs& a, int state_dt, int weight_dt, hipStream_t s);
READY_HIDDEN hipError_t ready_launch_state_p(const StateArgs& a, hipStream_t s);
READY_HIDDEN hipError_t ready_launch_feat(const FeatArgs& a, hipStream_t s);
READY_HIDDEN hipError_t ready_launch_gemm(const GemmArgs& g, int x_dt, int w_dt, int out_dt, int epi,
                                          dim3 grid, size_t lds_bytes, hipStream_t s);
// bm: rows per workgroup tile (16 or 64); weights must be bf16
READY_HIDDEN hipError_t ready_launch_gemm_mfma(const GemmArgs& g, int x_dt, int out_dt, int epi, int bm,
                                               dim3 grid, hipStream_t s);
