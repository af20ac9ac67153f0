// Per-state kernel of the ReaDy state reader for gfx950, general form (any
// dtype mix and any rank up to 128; the bf16 fast path of rank <= 32 is in
// ready_fast.hip).
//
//   k_state    one workgroup per (sequence, layer-head pair) tile does the
//              fused gather at the accept index (step 1), the mean square and
//              log-RMS (step 2), T = V^T S_bar by chunks of 8 ranks on the
//              VALU (step 3), the readout u_j = T q_j / sqrt(d_k) with
//              q_j = U^T z_j (step 4) and the packing of [u, ell] (step 5,
//              first half).  Needs the query sums z first.
// Formulas: ReaDy arXiv text, section 3.1 "Position-conditioned reading" and
// "Fusion and residual injection" (Eq. (3), written out in the rainbus summary,
// 方法步骤详情 steps (1)-(3)); section 3.2 "Avoiding redundant data movement"
// for the fused gather into a preallocated buffer, and "State-access
// footprint" for sharing the projected state across the block.
#include "ready_common.h"

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


// ---------------------------------------------------------------- launchers

hipError_t ready_launch_state(const StateArgs& a, int state_dt, int weight_dt, hipStream_t s,
                              StageEvents ev) {
  const dim3 grid((unsigned)(a.B * a.M)), block(256);
  if (state_dt == READY_BF16 && weight_dt == READY_BF16)
    READY_LAUNCH((k_state<uint16_t, uint16_t>), grid, block, 0, s, ev, a);
  else if (state_dt == READY_BF16)
    READY_LAUNCH((k_state<uint16_t, float>), grid, block, 0, s, ev, a);
  else if (weight_dt == READY_BF16)
    READY_LAUNCH((k_state<float, uint16_t>), grid, block, 0, s, ev, a);
  else
    READY_LAUNCH((k_state<float, float>), grid, block, 0, s, ev, a);
  return hipGetLastError();
}

