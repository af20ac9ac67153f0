// gfx950 kernels of the ReaDy state reader.
//
// Two kernel families:
//   k_state  one workgroup per (sequence, layer-head pair) state tile: the
//            fused gather at the accept index (step 1), the mean square and
//            log-RMS (step 2), T = V^T S_bar by chunks of 8 ranks (step 3),
//            the per-position readout u_j = T q_j / sqrt(d_k) (step 4) and the
//            packing of [u, ell] into f_j (step 5, first half).
//   k_gemm   a split-K skinny GEMM Y = X W^T streaming W once per row block,
//            used for z = W_q (gamma * h) (with the RMSNorm sums of squares of
//            h as a by-product), a = act(W1 f + b1) and
//            out = h + W2 a + b2.
// Formulas: ReaDy arXiv text, section 3.1 "Position-conditioned reading" and
// "Fusion and residual injection" (Eqs. (3)-(4), written out in the rainbus
// summary, 方法步骤详情 steps (1)-(3)); section 3.2 "Avoiding redundant data
// movement" for the fused gather into a preallocated buffer.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ready_internal.h"

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- numerics

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int VW = 4;  // elements per 16-byte vector
  __device__ static __forceinline__ float ld(const void* p, int64_t i) { return ((const float*)p)[i]; }
  __device__ static __forceinline__ void st(void* p, int64_t i, float v) { ((float*)p)[i] = v; }
  __device__ static __forceinline__ void unpack(const u32x4& v, float* o) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
};
template <> struct Elem<uint16_t> {
  static constexpr int VW = 8;
  __device__ static __forceinline__ float ld(const void* p, int64_t i) {
    return bf16_bits_to_f32(((const uint16_t*)p)[i]);
  }
  __device__ static __forceinline__ void st(void* p, int64_t i, float v) { ((uint16_t*)p)[i] = f32_to_bf16_rne(v); }
  __device__ static __forceinline__ void unpack(const u32x4& v, float* o) {
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    o[4] = __uint_as_float(v.z << 16); o[5] = __uint_as_float(v.z & 0xffff0000u);
    o[6] = __uint_as_float(v.w << 16); o[7] = __uint_as_float(v.w & 0xffff0000u);
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float activation(float x, int act) {
  if (act == READY_ACT_SILU) return x / (1.0f + expf(-x));
  if (act == READY_ACT_GELU_TANH) {
    const float c = 0.7978845608028654f;  // sqrt(2 / pi)
    return 0.5f * x * (1.0f + tanhf(c * (x + 0.044715f * x * x * x)));
  }
  return fmaxf(x, 0.0f);
}

// ---------------------------------------------------------------- k_state

// Lanes of one wave hold 16-byte vectors of consecutive columns of a tile row:
// CG vectors span a row, so a wave covers 64/CG rows per pass and the 256
// threads cover RPP rows per pass.  Each thread keeps its NP vectors of the
// tile in registers for all of steps 1-3.
template <typename TS, typename TW>
__global__ __launch_bounds__(256) void k_state(StateArgs a) {
  constexpr int VW = Elem<TS>::VW;
  constexpr int CG = READY_TILE / VW;   // vectors per row: 16 (bf16) or 32 (fp32)
  constexpr int RPP = 256 / CG;         // rows per pass
  constexpr int NP = READY_TILE / RPP;  // passes
  constexpr int RC = 8;                 // ranks per chunk of T

  __shared__ float s_red[4][RC * READY_TILE];   // per-wave partial T chunk
  __shared__ float s_T[RC][READY_TILE];
  __shared__ float s_q[16][READY_TILE];         // q_j, j < n <= 16
  __shared__ float s_z[16 * 128];               // z_j, n x r
  __shared__ float s_rs[16];                    // 1 / rms(h_j)
  __shared__ float s_wsum[4];

  const int tile = blockIdx.x;
  const int b = tile / a.M;
  const int m = tile - b * a.M;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.n, r = a.r, F = a.F;
  const int rows = a.B * n;
  const int mz = a.shared ? 0 : m;
  const int64_t frow = (int64_t)(b * n) * F + (int64_t)m * (r + 1);

  const int p_acc = a.accept_idx[b];
  if (p_acc < 0 || p_acc >= a.P) {
    // Out-of-range accept index: flag it, leave this sequence's outputs alone.
    if (tid == 0) {
      if (a.dev_status) a.dev_status[0] = READY_ERR_ACCEPT_IDX;
      if (m == 0) a.seq_invalid[b] = 1;
    }
    for (int e = tid; e < n * (r + 1); e += 256) {
      const int j = e / (r + 1), i = e - j * (r + 1);
      a.f[frow + (int64_t)j * F + i] = 0.0f;
      if (a.feat) a.feat[frow + (int64_t)j * F + i] = 0.0f;
    }
    return;
  }
  if (m == 0 && tid == 0) a.seq_invalid[b] = 0;

  // ---- step 1: fused gather straight into the caller's buffer ----
  const int l = m / a.H, hh = m - (m / a.H) * a.H;
  const TS* src = (const TS*)a.states + (int64_t)b * a.sb + (int64_t)p_acc * a.sp +
                  (int64_t)a.slot[l] * a.sl + (int64_t)hh * a.sh;
  TS* dst = (TS*)a.gathered + (int64_t)tile * READY_TILE_ELEMS;
  const int cg = tid % CG, r0 = tid / CG;
  u32x4 data[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p)
    data[p] = __builtin_nontemporal_load((const u32x4*)(src + (r0 + p * RPP) * READY_TILE + cg * VW));
#pragma unroll
  for (int p = 0; p < NP; ++p)
    __builtin_nontemporal_store(data[p], (u32x4*)(dst + (r0 + p * RPP) * READY_TILE + cg * VW));

  // ---- step 2: mean square of the tile ----
  float ss = 0.0f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    float x[VW];
    Elem<TS>::unpack(data[p], x);
#pragma unroll
    for (int e = 0; e < VW; ++e) ss += x[e] * x[e];
  }
  ss = wave_sum(ss);
  if (lane == 0) s_wsum[wave] = ss;

  // ---- step 4 (query side): z_j and q_j of this pair ----
  if (tid < n) {
    const int rho = b * n + tid;
    float hs = 0.0f;
    for (int ks = 0; ks < a.ksz; ++ks) hs += a.hss[(int64_t)ks * rows + rho];
    s_rs[tid] = 1.0f / sqrtf(hs / (float)a.d + a.h_eps);
  }
  __syncthreads();
  const float ms = ((s_wsum[0] + s_wsum[1]) + (s_wsum[2] + s_wsum[3])) * (1.0f / READY_TILE_ELEMS);
  const float rms = sqrtf(ms + a.state_eps);
  const float inv_rms = 1.0f / rms;
  for (int e = tid; e < n * r; e += 256) {
    const int j = e / r, i = e - j * r;
    const int64_t rho = b * n + j;
    float s = 0.0f;
    for (int ks = 0; ks < a.ksz; ++ks) s += a.zpart[((int64_t)ks * rows + rho) * a.nz + mz * r + i];
    s_z[e] = s * s_rs[j];
  }
  __syncthreads();
  const void* U = (const char*)a.u + (int64_t)mz * r * READY_TILE * sizeof(TW);
  for (int e = tid; e < n * READY_TILE; e += 256) {
    const int j = e >> 7, k = e & 127;
    float s = 0.0f;
    for (int i = 0; i < r; ++i) s += Elem<TW>::ld(U, (int64_t)i * READY_TILE + k) * s_z[j * r + i];
    s_q[j][k] = s;
  }

  // ---- step 3 by chunks of RC ranks, each followed by its readouts ----
  const void* V = (const char*)a.v + (int64_t)mz * READY_TILE * r * sizeof(TW);
  const float qscale = 0.08838834764831845f;  // 1 / sqrt(d_k), d_k = 128
  for (int rc = 0; rc < r; rc += RC) {
    float acc[RC][VW];
#pragma unroll
    for (int i = 0; i < RC; ++i)
#pragma unroll
      for (int e = 0; e < VW; ++e) acc[i][e] = 0.0f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int v = r0 + p * RPP;
      float vv[RC];
#pragma unroll
      for (int i = 0; i < RC; ++i) vv[i] = Elem<TW>::ld(V, (int64_t)v * r + rc + i);
      float x[VW];
      Elem<TS>::unpack(data[p], x);
#pragma unroll
      for (int i = 0; i < RC; ++i)
#pragma unroll
        for (int e = 0; e < VW; ++e) acc[i][e] += vv[i] * x[e];
    }
    // lanes with equal lane % CG hold the same columns: fold them together
#pragma unroll
    for (int off = CG; off < 64; off <<= 1)
#pragma unroll
      for (int i = 0; i < RC; ++i)
#pragma unroll
        for (int e = 0; e < VW; ++e) acc[i][e] += __shfl_xor(acc[i][e], off, 64);
    if (lane < CG) {
#pragma unroll
      for (int i = 0; i < RC; ++i)
#pragma unroll
        for (int e = 0; e < VW; ++e) s_red[wave][(i * VW + e) * CG + cg] = acc[i][e];
    }
    __syncthreads();
    for (int e = tid; e < RC * READY_TILE; e += 256) {
      const int i = e >> 7, k = e & 127;
      const int idx = (i * VW + (k % VW)) * CG + k / VW;
      s_T[i][k] = ((s_red[0][idx] + s_red[1][idx]) + (s_red[2][idx] + s_red[3][idx])) * inv_rms;
    }
    __syncthreads();
    for (int o = wave; o < n * RC; o += 4) {
      const int j = o / RC, i = o - j * RC;
      float s = s_T[i][lane] * s_q[j][lane] + s_T[i][lane + 64] * s_q[j][lane + 64];
      s = wave_sum(s);
      if (lane == 0 && rc + i < r) {
        const float uv = s * qscale;
        a.f[frow + (int64_t)j * F + rc + i] = uv;
        if (a.feat) a.feat[frow + (int64_t)j * F + rc + i] = uv;
      }
    }
    __syncthreads();
  }

  // ---- log-RMS scale, packed after the pair's readouts ----
  const float ell = logf(rms);
  if (tid < n) {
    a.f[frow + (int64_t)tid * F + r] = ell;
    if (a.feat) a.feat[frow + (int64_t)tid * F + r] = ell;
  }
  if (tid == 0 && a.logrms) a.logrms[tile] = ell;
}

// ---------------------------------------------------------------- k_gemm

// Each workgroup owns 16 output columns (4 waves x 4 groups of LPC = 16
// lanes), READY_GEMM_RB rows and one K split.  X rows are staged in LDS in fp32
// by passes of READY_GEMM_KSTAGE; each lane group streams its column of W
// with 16-byte loads and keeps RB accumulators.
template <typename TX, typename TW, typename TO, int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g) {
  constexpr int RB = READY_GEMM_RB;
  constexpr int LPC = 16;
  constexpr int VW = Elem<TW>::VW;
  extern __shared__ float xs[];  // [RB][klen]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane / LPC, lic = lane - grp * LPC;
  const int c = blockIdx.x * READY_GEMM_COLS + wave * 4 + grp;
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
    for (int e = tid; e < RB * klen; e += 256) {
      const int rr = e / klen, kk = e - rr * klen;
      float x = 0.0f;
      if (rr < nrows) x = Elem<TX>::ld(g.X, (int64_t)(row0 + rr) * g.ldx + k0 + kk);
      xs[e] = x;
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
        for (int kk = lic * VW; kk < klen; kk += LPC * VW) {
          float w[VW];
          Elem<TW>::unpack(*(const u32x4*)(wrow + kk), w);
#pragma unroll
          for (int rr = 0; rr < RB; ++rr)
#pragma unroll
            for (int e = 0; e < VW; ++e) acc[rr] += w[e] * xs[rr * klen + kk + e];
        }
      } else {
        for (int kk = lic; kk < klen; kk += LPC) {
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

  if (want_hss) {
    hsq0 = wave_sum(hsq0);
    hsq1 = wave_sum(hsq1);
    if (lane == 0) {
      if (wave < nrows) g.hss[(int64_t)ks * g.R + row0 + wave] = hsq0;
      if (wave + 4 < nrows) g.hss[(int64_t)ks * g.R + row0 + wave + 4] = hsq1;
    }
  }

  if (lic != 0 || c >= g.N) return;
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

// ---------------------------------------------------------------- launchers

hipError_t ready_launch_state(const StateArgs& a, int state_dt, int weight_dt, hipStream_t s) {
  const dim3 grid((unsigned)(a.B * a.M)), block(256);
  if (state_dt == READY_BF16 && weight_dt == READY_BF16)
    hipLaunchKernelGGL((k_state<uint16_t, uint16_t>), grid, block, 0, s, a);
  else if (state_dt == READY_BF16)
    hipLaunchKernelGGL((k_state<uint16_t, float>), grid, block, 0, s, a);
  else if (weight_dt == READY_BF16)
    hipLaunchKernelGGL((k_state<float, uint16_t>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((k_state<float, float>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int EPI>
static void launch_gemm_epi(const GemmArgs& g, int x_dt, int w_dt, int out_dt, dim3 grid,
                            size_t lds, hipStream_t s) {
  const dim3 block(256);
#define READY_GEMM_CASE(TX, TW, TO) hipLaunchKernelGGL((k_gemm<TX, TW, TO, EPI>), grid, block, lds, s, g)
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
                             dim3 grid, size_t lds_bytes, hipStream_t s) {
  if (epi == EPI_PARTIAL) launch_gemm_epi<EPI_PARTIAL>(g, x_dt, w_dt, out_dt, grid, lds_bytes, s);
  else if (epi == EPI_BIAS_ACT) launch_gemm_epi<EPI_BIAS_ACT>(g, x_dt, w_dt, out_dt, grid, lds_bytes, s);
  else launch_gemm_epi<EPI_RESID>(g, x_dt, w_dt, out_dt, grid, lds_bytes, s);
  return hipGetLastError();
}
