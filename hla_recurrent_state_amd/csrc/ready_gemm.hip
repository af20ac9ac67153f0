// GEMM kernels of the ReaDy state reader for gfx950: Y = X W^T over rows of
// X (draft positions) and rows of W (output features), used for
//   z   = W_q (gamma * h)        (query bottleneck; split-K partial sums, with
//                                 the sums of squares of h for RMSNorm),
//   a   = act(W1 f + b1)         (first layer of the bottleneck MLP),
//   out = h + W2 a + b2          (second layer and the residual).
// ReaDy arXiv text, section 3.1 "Position-conditioned reading" and "Fusion and
// residual injection" (Eqs. (3)-(4); rainbus summary, 方法步骤详情 (2)-(3)).
//
//   k_gemm       VALU: each workgroup owns 16 columns and 8 rows, stages X in
//                LDS in fp32 and streams W with 16-byte loads (any dtypes).
//   k_gemm_mfma  matrix cores: bf16 operands (X narrowed to bf16 when it is
//                fp32), fp32 accumulation, 64-column tiles of 16 or 64 rows.
#include <algorithm>

#include "ready_common.h"

// ---------------------------------------------------------------- k_gemm

// Each workgroup owns 16 output columns (4 waves x 4 groups of LPC = 16
// lanes), READY_GEMM_RB rows and one K split.  X rows are staged in LDS in fp32
// by passes of READY_GEMM_KSTAGE; each lane group streams its column of W
// with 16-byte loads and keeps RB accumulators.  With g.wave_k (grids too
// small to fill the GPU) a workgroup owns 4 columns instead and its four
// waves split each column's K range, summed through LDS in wave order.
template <typename TX, typename TW, typename TO, int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g) {
  constexpr int RB = READY_GEMM_RB;
  constexpr int LPC = 16;
  constexpr int VW = Elem<TW>::VW;
  extern __shared__ float xs[];  // [RB][klen]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane / LPC, lic = lane - grp * LPC;
  const int nw = g.wave_k ? 4 : 1;                   // waves sharing a column
  const int c = g.wave_k ? blockIdx.x * 4 + grp : blockIdx.x * READY_GEMM_COLS + wave * 4 + grp;
  const int wk = g.wave_k ? wave : 0;                // this wave's share of K
  const int ks = blockIdx.y;
  const int row0 = blockIdx.z * RB;
  const int nrows = min(RB, g.R - row0);
  const int kbeg = ks * g.kchunk;
  const int kend = min(g.K, kbeg + g.kchunk);
  const bool want_hss = (EPI == EPI_PARTIAL) && g.hss != nullptr && blockIdx.x == 0;

  float acc[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) acc[i] = 0.0f;
  float hsq0 = 0.0f, hsq1 = 0.0f;  // rows `wave` and `wave + 4`

  for (int k0 = kbeg; k0 < kend; k0 += READY_GEMM_KSTAGE) {
    const int klen = min(READY_GEMM_KSTAGE, kend - k0);
    __syncthreads();
    // batches of 8 loads in flight (issued unconditionally: element 0 stands
    // in for one out of range), then their stores
    for (int e0 = tid; e0 < RB * klen; e0 += 8 * 256) {
      float xv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + 256 * u;
        const int rr = e / klen, kk = e - rr * klen;
        const bool ok = e < RB * klen && rr < nrows;
        const float x = Elem<TX>::ld(g.X, ok ? (int64_t)(row0 + rr) * g.ldx + k0 + kk : 0);
        xv[u] = ok ? x : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (e0 + 256 * u < RB * klen) xs[e0 + 256 * u] = xv[u];
    }
    __syncthreads();
    if (want_hss) {
      for (int kk = lane; kk < klen; kk += 64) {
        const float x0 = xs[wave * klen + kk], x1 = xs[(wave + 4) * klen + kk];
        hsq0 += x0 * x0;
        hsq1 += x1 * x1;
      }
    }
    if (EPI == EPI_PARTIAL && g.gamma != nullptr) {
      __syncthreads();
      for (int e = tid; e < RB * klen; e += 256) {
        const int kk = e % klen;
        xs[e] *= Elem<TW>::ld(g.gamma, k0 + kk);
      }
      __syncthreads();
    }
    if (c < g.N) {
      const TW* wrow = (const TW*)g.W + (int64_t)c * g.ldw + k0;
      if (g.vec_ok) {
        // batches of 4 row chunks in flight (a clamped address stands in for
        // a chunk past the end; it is not used)
        const int step = LPC * VW * nw;
        for (int kk0 = (wk * LPC + lic) * VW; kk0 < klen; kk0 += 4 * step) {
          u32x4 wv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) wv[u] = *(const u32x4*)(wrow + min(kk0 + u * step, klen - VW));
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int kk = kk0 + u * step;
            if (kk < klen) {
              float w[VW];
              Elem<TW>::unpack(wv[u], w);
#pragma unroll
              for (int rr = 0; rr < RB; ++rr)
#pragma unroll
                for (int e = 0; e < VW; ++e) acc[rr] += w[e] * xs[rr * klen + kk + e];
            }
          }
        }
      } else {
        for (int kk = wk * LPC + lic; kk < klen; kk += LPC * nw) {
          const float w = Elem<TW>::ld(wrow, kk);
#pragma unroll
          for (int rr = 0; rr < RB; ++rr) acc[rr] += w * xs[rr * klen + kk];
        }
      }
    }
  }

#pragma unroll
  for (int rr = 0; rr < RB; ++rr)
#pragma unroll
    for (int off = LPC / 2; off > 0; off >>= 1) acc[rr] += __shfl_xor(acc[rr], off, 64);
  if (g.wave_k) {
    __shared__ float s_wk[4][4][RB];  // [wave][group][row]
    if (lic == 0)
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) s_wk[wave][grp][rr] = acc[rr];
    __syncthreads();
    if (wave == 0 && lic == 0)
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) acc[rr] = (s_wk[0][grp][rr] + s_wk[1][grp][rr]) + (s_wk[2][grp][rr] + s_wk[3][grp][rr]);
  }

  if (want_hss) {
    hsq0 = wave_sum(hsq0);
    hsq1 = wave_sum(hsq1);
    if (lane == 0) {
      if (wave < nrows) g.hss[(int64_t)ks * g.R + row0 + wave] = hsq0;
      if (wave + 4 < nrows) g.hss[(int64_t)ks * g.R + row0 + wave + 4] = hsq1;
    }
  }

  if (lic != 0 || c >= g.N || (g.wave_k && wave != 0)) return;
  for (int rr = 0; rr < nrows; ++rr) {
    const int64_t rho = row0 + rr;
    if (EPI == EPI_PARTIAL) {
      g.ypart[((int64_t)ks * g.R + rho) * g.N + c] = acc[rr];
    } else if (EPI == EPI_BIAS_ACT) {
      const float pre = acc[rr] + (g.bias ? Elem<TW>::ld(g.bias, c) : 0.0f);
      g.yout[rho * g.N + c] = activation(pre, g.act);
    } else {
      if (g.seq_invalid[rho / g.n]) continue;
      const float dh = acc[rr] + (g.bias ? Elem<TW>::ld(g.bias, c) : 0.0f);
      const float hv = Elem<TO>::ld(g.h, rho * g.N + c);
      Elem<TO>::st(g.out, rho * g.N + c, hv + dh);
      if (g.delta) g.delta[rho * g.N + c] = dh;
    }
  }
}


// ---------------------------------------------------------------- k_gemm_mfma

// Tile BM x 64 outputs, K in steps of 64 staged in LDS as bf16 (rows padded to
// 72 elements).  Wave w owns output columns [16 w, 16 w + 16) and every 16-row
// block of the tile; per K step it issues 2 x (BM / 16) 16 x 16 x 32 matrix
// instructions.  Requires K, ldx and ldw to keep 16-byte row chunks aligned.
template <typename TX, typename TO, int EPI, int BM>
__global__ __launch_bounds__(256) void k_gemm_mfma(GemmArgs g) {
  constexpr int BN = READY_MFMA_BN, BK = READY_MFMA_BK, LDK = BK + 8;
  constexpr int WM = BM / 16;
  constexpr bool XBF = sizeof(TX) == 2;
  constexpr int XCH = XBF ? BM * 8 : BM * 16;          // 16-byte X chunks per K step
  constexpr int NIT = (XCH + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint16_t sX[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sW[BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col0 = blockIdx.x * BN, ks = blockIdx.y, row0 = blockIdx.z * BM;
  const int kbeg = ks * g.kchunk;
  const int kend = min(g.K, kbeg + g.kchunk);
  const bool want_hss = (EPI == EPI_PARTIAL) && XBF && g.hss != nullptr && blockIdx.x == 0;
  const uint16_t* W = (const uint16_t*)g.W;

  f32x4 acc[WM];
#pragma unroll
  for (int rb = 0; rb < WM; ++rb) acc[rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float hsq[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) hsq[it] = 0.0f;

  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    // W tile: 64 rows x 64 k = 512 chunks of 8 bf16
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = tid + 256 * it;
      const int nn = c >> 3, kc = (c & 7) * 8;
      const int gn = col0 + nn, gk = k0 + kc;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (gn < g.N && gk < kend) v = *(const u32x4*)(W + (int64_t)gn * g.ldw + gk);
      *(u32x4*)&sW[nn * LDK + kc] = v;
    }
    // X tile: BM rows x 64 k, narrowed to bf16
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int c = tid + 256 * it;
      if (c < XCH) {
        if (XBF) {
          const int rr = c >> 3, kc = (c & 7) * 8;
          const int gr = row0 + rr, gk = k0 + kc;
          u32x4 v = u32x4{0u, 0u, 0u, 0u};
          if (gr < g.R && gk < kend) v = *(const u32x4*)((const uint16_t*)g.X + (int64_t)gr * g.ldx + gk);
          if (want_hss || g.gamma != nullptr) {
            float x[8];
            Elem<uint16_t>::unpack(v, x);
            if (want_hss) {
              float sq = 0.0f;
#pragma unroll
              for (int e = 0; e < 8; ++e) sq += x[e] * x[e];
              // the 8 chunks of one row sit in 8 consecutive lanes
              sq += __shfl_xor(sq, 1, 64);
              sq += __shfl_xor(sq, 2, 64);
              sq += __shfl_xor(sq, 4, 64);
              hsq[it] += sq;
            }
            if (g.gamma != nullptr && gk < kend) {
              uint32_t w4[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float a0 = x[2 * e] * Elem<uint16_t>::ld(g.gamma, gk + 2 * e);
                const float a1 = x[2 * e + 1] * Elem<uint16_t>::ld(g.gamma, gk + 2 * e + 1);
                w4[e] = (uint32_t)f32_to_bf16_rne(a0) | ((uint32_t)f32_to_bf16_rne(a1) << 16);
              }
              v = u32x4{w4[0], w4[1], w4[2], w4[3]};
            }
          }
          *(u32x4*)&sX[rr * LDK + kc] = v;
        } else {
          const int rr = c >> 4, kc = (c & 15) * 4;
          const int gr = row0 + rr, gk = k0 + kc;
          u32x4 v = u32x4{0u, 0u, 0u, 0u};
          if (gr < g.R && gk < kend) v = *(const u32x4*)((const float*)g.X + (int64_t)gr * g.ldx + gk);
          const uint32_t lo = (uint32_t)f32_to_bf16_rne(__uint_as_float(v.x)) |
                              ((uint32_t)f32_to_bf16_rne(__uint_as_float(v.y)) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16_rne(__uint_as_float(v.z)) |
                              ((uint32_t)f32_to_bf16_rne(__uint_as_float(v.w)) << 16);
          *(uint2*)&sX[rr * LDK + kc] = make_uint2(lo, hi);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4 bop = *(const u32x4*)&sW[(16 * wave + (lane & 15)) * LDK + 32 * kk + 8 * (lane >> 4)];
#pragma unroll
      for (int rb = 0; rb < WM; ++rb) {
        const u32x4 aop = *(const u32x4*)&sX[(16 * rb + (lane & 15)) * LDK + 32 * kk + 8 * (lane >> 4)];
        acc[rb] = mfma16x16x32(aop, bop, acc[rb]);
      }
    }
    __syncthreads();
  }

  if (want_hss) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int c = tid + 256 * it;
      const int gr = row0 + (c >> 3);
      if (c < XCH && (c & 7) == 0 && gr < g.R) g.hss[(int64_t)ks * g.R + gr] = hsq[it];
    }
  }

  const int col = col0 + 16 * wave + (lane & 15);
  if (col >= g.N) return;
  float bias = 0.0f;
  if (EPI != EPI_PARTIAL && g.bias != nullptr) bias = Elem<uint16_t>::ld(g.bias, col);
#pragma unroll
  for (int rb = 0; rb < WM; ++rb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t rho = row0 + 16 * rb + 4 * (lane >> 4) + e;
      if (rho >= g.R) continue;
      const float y = acc[rb][e];
      if (EPI == EPI_PARTIAL) {
        g.ypart[((int64_t)ks * g.R + rho) * g.N + col] = y;
      } else if (EPI == EPI_BIAS_ACT) {
        g.yout[rho * g.N + col] = activation(y + bias, g.act);
      } else {
        if (g.seq_invalid[rho / g.n]) continue;
        const float dh = y + bias;
        const float hv = Elem<TO>::ld(g.h, rho * g.N + col);
        Elem<TO>::st(g.out, rho * g.N + col, hv + dh);
        if (g.delta) g.delta[rho * g.N + col] = dh;
      }
    }
}

// ---------------------------------------------------------------- k_gemm_mm

// Large-row form of k_gemm_mfma: 128 x 128 output tiles.  Four waves in a
// 2 x 2 arrangement each own a 64 x 64 block (4 x 4 blocks of 16 x 16), so
// every operand fragment read from LDS feeds four matrix instructions.  The
// next K step's global loads are held in registers while the current step's
// matrix instructions run from LDS; then the registers go to LDS between two
// barriers.  One LDS buffer keeps three workgroups on a CU.  Requires K, ldx
// and ldw to keep 16-byte row chunks aligned.
constexpr int GM_BM = READY_GM_TILE, GM_BN = READY_GM_TILE;

// Residual epilogue staging: per wave, 16 rows x 64 columns of fp32 dh
constexpr int GM_ELD = 68;
template <typename TX, typename TO, int EPI, int GM_BK>
__device__ __forceinline__ void gemm_mm_body(const GemmArgs& g, uint16_t* sX, uint16_t* sW, float* sE) {
  constexpr int GM_LD = GM_BK + 8;                 // padded LDS row
  constexpr bool XBF = sizeof(TX) == 2;
  constexpr int CPR = GM_BK / 8;                   // 16-byte bf16 chunks per row and step
  constexpr int XN = GM_BM * GM_BK * sizeof(TX) / 16 / 256;  // 16-byte X chunks per thread per step
  constexpr int WN = GM_BN * GM_BK * 2 / 16 / 256;           // 16-byte W chunks per thread per step

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int wr = wave >> 1, wc = wave & 1;
  // blockIdx.x runs over the output tiles, padded to a multiple of 8: the
  // tiles are numbered column-major (row tiles inner) and each XCD takes a
  // contiguous run of them, so the workgroups on one XCD share a few column
  // panels of W and the row panels of X in its L2.  With at most four column
  // tiles (a narrow output, X the larger operand) they are numbered row-major
  // instead, so the column tiles of one X row panel run on one XCD and the
  // panel is read from HBM once.
  const int q = xcd_remap(blockIdx.x, gridDim.x, g.tiles_c * g.tiles_r);
  if (q < 0) return;
  const bool rmaj = g.tiles_c <= 4;
  const int tc = rmaj ? q % g.tiles_c : q / g.tiles_r;
  const int tr = rmaj ? q / g.tiles_c : q - tc * g.tiles_r;
  const int col0 = tc * GM_BN, ks = blockIdx.y, row0 = tr * GM_BM;
  const int kbeg = ks * g.kchunk;
  const int kend = min(g.K, kbeg + g.kchunk);
  const int nsteps = kend > kbeg ? (kend - kbeg + GM_BK - 1) / GM_BK : 0;
  const bool want_hss = (EPI == EPI_PARTIAL) && XBF && g.hss != nullptr && tc == 0;
  const uint16_t* W = (const uint16_t*)g.W;

  u32x4 xq[XN], wq[WN];
  float hsq[XN];
#pragma unroll
  for (int it = 0; it < XN; ++it) hsq[it] = 0.0f;

  auto load = [&](int k0) {
#pragma unroll
    for (int it = 0; it < WN; ++it) {
      const int c = tid + 256 * it;
      const int gn = col0 + c / CPR, gk = k0 + (c % CPR) * 8;
      wq[it] = u32x4{0u, 0u, 0u, 0u};
      if (gn < g.N && gk < kend) wq[it] = *(const u32x4*)(W + (int64_t)gn * g.ldw + gk);
    }
#pragma unroll
    for (int it = 0; it < XN; ++it) {
      const int c = tid + 256 * it;
      xq[it] = u32x4{0u, 0u, 0u, 0u};
      if (XBF) {
        const int gr = row0 + c / CPR, gk = k0 + (c % CPR) * 8;
        if (gr < g.R && gk < kend) xq[it] = *(const u32x4*)((const uint16_t*)g.X + (int64_t)gr * g.ldx + gk);
      } else {
        const int gr = row0 + c / (2 * CPR), gk = k0 + (c % (2 * CPR)) * 4;
        if (gr < g.R && gk < kend) xq[it] = *(const u32x4*)((const float*)g.X + (int64_t)gr * g.ldx + gk);
      }
    }
  };
  auto store = [&](int k0) {
#pragma unroll
    for (int it = 0; it < WN; ++it) {
      const int c = tid + 256 * it;
      *(u32x4*)&sW[(c / CPR) * GM_LD + (c % CPR) * 8] = wq[it];
    }
#pragma unroll
    for (int it = 0; it < XN; ++it) {
      const int c = tid + 256 * it;
      if (XBF) {
        u32x4 v = xq[it];
        if (want_hss || g.gamma != nullptr) {
          float x[8];
          Elem<uint16_t>::unpack(v, x);
          if (want_hss) {
            float sq = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) sq += x[e] * x[e];
            // the CPR chunks of one row sit in CPR consecutive lanes
#pragma unroll
            for (int o = 1; o < CPR; o <<= 1) sq += __shfl_xor(sq, o, 64);
            hsq[it] += sq;
          }
          const int gk = k0 + (c % CPR) * 8;
          if (g.gamma != nullptr && gk < kend) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= Elem<uint16_t>::ld(g.gamma, gk + e);
            v = pack_bf16x8(x);
          }
        }
        *(u32x4*)&sX[(c / CPR) * GM_LD + (c % CPR) * 8] = v;
      } else {
        const u32x4 v = xq[it];
        const uint32_t lo = (uint32_t)f32_to_bf16_rne(__uint_as_float(v.x)) |
                            ((uint32_t)f32_to_bf16_rne(__uint_as_float(v.y)) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_rne(__uint_as_float(v.z)) |
                            ((uint32_t)f32_to_bf16_rne(__uint_as_float(v.w)) << 16);
        *(uint2*)&sX[(c / (2 * CPR)) * GM_LD + (c % (2 * CPR)) * 4] = make_uint2(lo, hi);
      }
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  if (nsteps > 0) {
    load(kbeg);
    store(kbeg);
  }
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int knext = kbeg + (s + 1) * GM_BK;
    if (s + 1 < nsteps) load(knext);
#pragma unroll
    for (int kk = 0; kk < GM_BK / 32; ++kk) {
      u32x4 bop[4], aop[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bop[j] = *(const u32x4*)&sW[(64 * wc + 16 * j + lr) * GM_LD + 32 * kk + 8 * lg];
#pragma unroll
      for (int i = 0; i < 4; ++i) aop[i] = *(const u32x4*)&sX[(64 * wr + 16 * i + lr) * GM_LD + 32 * kk + 8 * lg];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(aop[i], bop[j], acc[i][j]);
    }
    if (s + 1 < nsteps) {
      __syncthreads();  // every wave is done reading this step's tiles
      store(knext);
    }
    __syncthreads();
  }

  if (want_hss) {
#pragma unroll
    for (int it = 0; it < XN; ++it) {
      const int c = tid + 256 * it;
      const int gr = row0 + c / CPR;
      if (c % CPR == 0 && gr < g.R) g.hss[(int64_t)ks * g.R + gr] = hsq[it];
    }
  }

  // epilogue: rows outer (16 per lane), so the per-row work -- the validity of
  // the row's sequence -- is done once per row, not once per value
  float bias[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = col0 + 64 * wc + 16 * j + lr;
    bias[j] = (EPI != EPI_PARTIAL && g.bias != nullptr && col < g.N) ? Elem<uint16_t>::ld(g.bias, col) : 0.0f;
  }
  if constexpr (EPI == EPI_RESID) {
    if (g.epi_vec) {
      // out = h + dh in 16-byte pieces: each 16-row block of the wave's
      // 64 x 64 goes through LDS (fp32), then a lane takes 8 consecutive
      // columns of a row at a time (two pieces per lane and block), so h
      // and out move in whole 16-byte chunks.  Same arithmetic as below.
      float* E = sE + wave * 16 * GM_ELD;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) E[(4 * lg + e) * GM_ELD + 16 * j + lr] = acc[i][j][e] + bias[j];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int c = lane + 64 * q;
          const int rr = c >> 3, c8 = (c & 7) * 8;
          const int64_t rho = row0 + 64 * wr + 16 * i + rr;
          const int col = col0 + 64 * wc + c8;
          if (rho < g.R && col < g.N && !g.seq_invalid[rho / g.n]) {
            float dh[8];
            *(float4*)&dh[0] = *(const float4*)&E[rr * GM_ELD + c8];
            *(float4*)&dh[4] = *(const float4*)&E[rr * GM_ELD + c8 + 4];
            const int64_t o = rho * g.N + col;
            float hv[8];
            if constexpr (sizeof(TO) == 2) {
              Elem<uint16_t>::unpack(*(const u32x4*)((const uint16_t*)g.h + o), hv);
            } else {
              *(float4*)&hv[0] = *(const float4*)((const float*)g.h + o);
              *(float4*)&hv[4] = *(const float4*)((const float*)g.h + o + 4);
            }
            float ov[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) ov[e] = hv[e] + dh[e];
            if constexpr (sizeof(TO) == 2) {
              *(u32x4*)((uint16_t*)g.out + o) = pack_bf16x8(ov);
            } else {
              *(float4*)((float*)g.out + o) = *(const float4*)&ov[0];
              *(float4*)((float*)g.out + o + 4) = *(const float4*)&ov[4];
            }
            if (g.delta) {
              *(float4*)(g.delta + o) = *(const float4*)&dh[0];
              *(float4*)(g.delta + o + 4) = *(const float4*)&dh[4];
            }
          }
        }
        __syncthreads();
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t rho = row0 + 64 * wr + 16 * i + 4 * lg + e;
      if (rho >= g.R) continue;
      if (EPI == EPI_RESID && g.seq_invalid[rho / g.n]) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = col0 + 64 * wc + 16 * j + lr;
        if (col >= g.N) continue;
        const float y = acc[i][j][e];
        if (EPI == EPI_PARTIAL) {
          g.ypart[((int64_t)ks * g.R + rho) * g.N + col] = y;
        } else if (EPI == EPI_BIAS_ACT) {
          g.yout[rho * g.N + col] = activation(y + bias[j], g.act);
        } else {
          const float dh = y + bias[j];
          const float hv = Elem<TO>::ld(g.h, rho * g.N + col);
          Elem<TO>::st(g.out, rho * g.N + col, hv + dh);
          if (g.delta) g.delta[rho * g.N + col] = dh;
        }
      }
    }
}

// bf16 X: K steps of 64, three workgroups on a CU.  fp32 X (twice the
// staging registers per K): steps of 64 as well where the launch has few
// workgroups (the first MLP layer's K split: about one per CU, so the fewer,
// longer steps matter more than a third workgroup); the residual form, with
// a workgroup per output tile, keeps steps of 32 and three on a CU.
template <typename TO, int EPI>
__global__ __launch_bounds__(256, 3) void k_gemm_mm_bx(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t sX[GM_BM * (64 + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sW[GM_BN * (64 + 8)];
  __shared__ __attribute__((aligned(16))) float sE[EPI == EPI_RESID ? 4 * 16 * GM_ELD : 4];
  gemm_mm_body<uint16_t, TO, EPI, 64>(g, sX, sW, sE);
}
template <typename TO, int EPI>
__global__ __launch_bounds__(256, EPI == EPI_RESID ? 3 : 2) void k_gemm_mm_fx(GemmArgs g) {
  constexpr int BK = EPI == EPI_RESID ? 32 : 64;
  __shared__ __attribute__((aligned(16))) uint16_t sX[GM_BM * (BK + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sW[GM_BN * (BK + 8)];
  __shared__ __attribute__((aligned(16))) float sE[EPI == EPI_RESID ? 4 * 16 * GM_ELD : 4];
  gemm_mm_body<float, TO, EPI, BK>(g, sX, sW, sE);
}

// a = act(sum over K splits of the partial sums + bias), one thread per value
__global__ __launch_bounds__(256) void k_reduce_bias_act(GemmArgs g, int ksplit) {
  const int64_t total = (int64_t)g.R * g.N;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    float s = 0.0f;
    for (int ks = 0; ks < ksplit; ++ks) s += g.ypart[(int64_t)ks * total + e];
    const int col = (int)(e % g.N);
    const float bias = g.bias != nullptr ? Elem<uint16_t>::ld(g.bias, col) : 0.0f;
    g.yout[e] = activation(s + bias, g.act);
  }
}

// ---------------------------------------------------------------- launchers
template <int EPI>
static void launch_gemm_epi(const GemmArgs& g, int x_dt, int w_dt, int out_dt, dim3 grid,
                            size_t lds, hipStream_t s, StageEvents ev) {
  const dim3 block(256);
#define READY_GEMM_CASE(TX, TW, TO) READY_LAUNCH((k_gemm<TX, TW, TO, EPI>), grid, block, lds, s, ev, g)
  if (EPI == EPI_PARTIAL) {
    if (x_dt == READY_BF16 && w_dt == READY_BF16) READY_GEMM_CASE(uint16_t, uint16_t, float);
    else if (x_dt == READY_BF16) READY_GEMM_CASE(uint16_t, float, float);
    else if (w_dt == READY_BF16) READY_GEMM_CASE(float, uint16_t, float);
    else READY_GEMM_CASE(float, float, float);
  } else if (EPI == EPI_BIAS_ACT) {
    if (w_dt == READY_BF16) READY_GEMM_CASE(float, uint16_t, float);
    else READY_GEMM_CASE(float, float, float);
  } else {
    if (w_dt == READY_BF16 && out_dt == READY_BF16) READY_GEMM_CASE(float, uint16_t, uint16_t);
    else if (w_dt == READY_BF16) READY_GEMM_CASE(float, uint16_t, float);
    else if (out_dt == READY_BF16) READY_GEMM_CASE(float, float, uint16_t);
    else READY_GEMM_CASE(float, float, float);
  }
#undef READY_GEMM_CASE
  (void)x_dt;
}

hipError_t ready_launch_gemm(const GemmArgs& g, int x_dt, int w_dt, int out_dt, int epi,
                             dim3 grid, size_t lds_bytes, hipStream_t s, StageEvents ev) {
  if (epi == EPI_PARTIAL) launch_gemm_epi<EPI_PARTIAL>(g, x_dt, w_dt, out_dt, grid, lds_bytes, s, ev);
  else if (epi == EPI_BIAS_ACT) launch_gemm_epi<EPI_BIAS_ACT>(g, x_dt, w_dt, out_dt, grid, lds_bytes, s, ev);
  else launch_gemm_epi<EPI_RESID>(g, x_dt, w_dt, out_dt, grid, lds_bytes, s, ev);
  return hipGetLastError();
}

template <int BM>
static void launch_mfma_bm(const GemmArgs& g, int x_dt, int out_dt, int epi, dim3 grid, hipStream_t s,
                           StageEvents ev) {
  const dim3 block(256);
  if (epi == EPI_PARTIAL) {
    if (x_dt == READY_BF16) READY_LAUNCH((k_gemm_mfma<uint16_t, float, EPI_PARTIAL, BM>), grid, block, 0, s, ev, g);
    else READY_LAUNCH((k_gemm_mfma<float, float, EPI_PARTIAL, BM>), grid, block, 0, s, ev, g);
  } else if (epi == EPI_BIAS_ACT) {
    READY_LAUNCH((k_gemm_mfma<float, float, EPI_BIAS_ACT, BM>), grid, block, 0, s, ev, g);
  } else {
    if (out_dt == READY_BF16) READY_LAUNCH((k_gemm_mfma<float, uint16_t, EPI_RESID, BM>), grid, block, 0, s, ev, g);
    else READY_LAUNCH((k_gemm_mfma<float, float, EPI_RESID, BM>), grid, block, 0, s, ev, g);
  }
}

hipError_t ready_launch_gemm_mfma(const GemmArgs& g, int x_dt, int out_dt, int epi, int bm, dim3 grid,
                                  hipStream_t s, StageEvents ev) {
  if (bm == 16) launch_mfma_bm<16>(g, x_dt, out_dt, epi, grid, s, ev);
  else launch_mfma_bm<64>(g, x_dt, out_dt, epi, grid, s, ev);
  return hipGetLastError();
}

hipError_t ready_launch_gemm_mm(const GemmArgs& g0, int x_dt, int out_dt, int epi, int ksplit, hipStream_t s,
                                StageEvents ev) {
  const dim3 block(256);
  GemmArgs g = g0;
  g.tiles_c = (g.N + GM_BN - 1) / GM_BN;
  g.tiles_r = (g.R + GM_BM - 1) / GM_BM;
  const dim3 grid((unsigned)((g.tiles_c * g.tiles_r + 7) / 8 * 8), (unsigned)ksplit);
  if (epi == EPI_PARTIAL) {
    if (x_dt == READY_BF16) READY_LAUNCH((k_gemm_mm_bx<float, EPI_PARTIAL>), grid, block, 0, s, ev, g);
    else READY_LAUNCH((k_gemm_mm_fx<float, EPI_PARTIAL>), grid, block, 0, s, ev, g);
  } else if (epi == EPI_BIAS_ACT) {
    READY_LAUNCH((k_gemm_mm_fx<float, EPI_BIAS_ACT>), grid, block, 0, s, ev, g);
  } else {
    if (out_dt == READY_BF16) READY_LAUNCH((k_gemm_mm_fx<uint16_t, EPI_RESID>), grid, block, 0, s, ev, g);
    else READY_LAUNCH((k_gemm_mm_fx<float, EPI_RESID>), grid, block, 0, s, ev, g);
  }
  return hipGetLastError();
}

hipError_t ready_launch_reduce_bias_act(const GemmArgs& g, int ksplit, hipStream_t s, StageEvents ev) {
  const int64_t total = (int64_t)g.R * g.N;
  const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 4096);
  READY_LAUNCH(k_reduce_bias_act, dim3(blocks), dim3(256), 0, s, ev, g, ksplit);
  return hipGetLastError();
}
