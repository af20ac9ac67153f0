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
  // The K-split partial sums are spread over several lanes per value, so
  // that few loads per lane stand between the query launch and this one:
  // 32 lanes per row for the sums of squares of h, 4 per value of z; the
  // lanes of one value are consecutive and meet through shuffles (a fixed
  // order, so the result does not depend on timing).
  for (int t32 = tid; t32 < 32 * n; t32 += 256) {  // whole groups of 32 lanes
    const int j = t32 >> 5, part = t32 & 31;
    const int rho = b * n + j;
    float hs = 0.0f;
#pragma unroll 4
    for (int ks = part; ks < a.ksz; ks += 32) hs += a.hss[(int64_t)ks * rows + rho];
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) hs += __shfl_xor(hs, o, 64);
    if (part == 0) s_rs[j] = 1.0f / sqrtf(hs / (float)a.d + a.h_eps);
  }
  __syncthreads();
  const float ms = ((s_wsum[0] + s_wsum[1]) + (s_wsum[2] + s_wsum[3])) * (1.0f / READY_TILE_ELEMS);
  const float rms = sqrtf(ms + a.state_eps);
  const float inv_rms = 1.0f / rms;
  for (int e4 = tid; e4 < 4 * n * r; e4 += 256) {  // 4 n r is a multiple of 4: whole groups of 4 lanes
    const int e = e4 >> 2, part = e4 & 3;
    const int j = e / r, i = e - j * r;
    const int64_t rho = b * n + j;
    float s = 0.0f;
#pragma unroll 4
    for (int ks = part; ks < a.ksz; ks += 4) s += a.zpart[((int64_t)ks * rows + rho) * a.nz + mz * r + i];
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    if (part == 0) s_z[e] = s * s_rs[j];
  }
  __syncthreads();
  const void* U = (const char*)a.u + (int64_t)mz * r * READY_TILE * sizeof(TW);
  for (int e = tid; e < n * READY_TILE; e += 256) {
    const int j = e >> 7, k = e & 127;
    float s = 0.0f;
    for (int i0 = 0; i0 < r; i0 += 8) {  // r is a multiple of 8: 8 loads in flight
      float uv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) uv[u] = Elem<TW>::ld(U, (int64_t)(i0 + u) * READY_TILE + k);
#pragma unroll
      for (int u = 0; u < 8; ++u) s += uv[u] * s_z[j * r + i0 + u];
    }
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


// ---------------------------------------------------------------- k_state_mm

// Matrix-core form of the per-state work for bf16 states and weights with
// r <= 128 (a multiple of 8) and n <= 16.  The readout is taken in the order
// u_j = V^T (S_bar q_j) / sqrt(d_k): the same value as T q_j / sqrt(d_k) with
// T = V^T S_bar, at 2 n (2 r + d_k) d_k operations per tile instead of
// 2 r d_k (d_k + n) -- the cheaper order once r exceeds n.  All three
// contractions run on 16 x 16 x 32 bf16 matrix instructions:
//   q^T = z^T U      (j x c, over i)
//   Y   = S q        (v x j, over c)
//   u^T = Y^T V      (j x i, over v)
// z, q and Y are fp32 values carried as two bf16 terms (hi + lo), so each
// product is accurate to about 2^-16 of the fp32 operand; U, V and S are bf16
// already.  U and V contract over their slow index, so each workgroup stages
// U^T and V^T of its layer-head pair in LDS and walks the tiles in pair-major
// order, restaging only when the pair changes.  Persistent: one workgroup of
// 8 waves per CU; the state tiles of the next three items are loaded into
// registers while the current one is worked on, so every CU keeps up to
// three tiles of loads in flight.

namespace {

constexpr int MM_THREADS = 512;
constexpr int MM_LD = READY_TILE + 8;   // padded LDS row of 128 bf16 (272 bytes)
constexpr int MM_CH = READY_TILE_ELEMS * 2 / 16 / MM_THREADS;  // 16-byte state chunks per thread: 4
constexpr int MM_S = 0;                                   // state tile, rows of 16 swizzled chunks
constexpr int MM_UT = MM_S + READY_TILE_ELEMS * 2;        // U^T [c][i]
constexpr int MM_VT = MM_UT + READY_TILE * MM_LD * 2;     // V^T [i][v]
constexpr int MM_ZS = MM_VT + READY_TILE * MM_LD * 2;     // z [hi, lo][j][i]
constexpr int MM_QS = MM_ZS + 2 * 16 * MM_LD * 2;         // q^T [hi, lo][j][c]
constexpr int MM_YT = MM_QS + 2 * 16 * MM_LD * 2;         // Y^T [hi, lo][j][v]
constexpr int MM_SS = MM_YT + 2 * 16 * MM_LD * 2;         // per-wave sums of squares
constexpr int MM_ACC = MM_SS + 64;                        // accept indices of the first READY_ACC_LDS sequences
constexpr int MM_BYTES = MM_ACC + 4 * READY_ACC_LDS;

__device__ __forceinline__ uint32_t bf16_pair(float x0, float x1) {
  return (uint32_t)f32_to_bf16_rne(x0) | ((uint32_t)f32_to_bf16_rne(x1) << 16);
}

// x as hi + lo with hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16_rne(x);
  lo = f32_to_bf16_rne(x - bf16_bits_to_f32(hi));
}

// Loads of one tile (item t of the pair-major order) into registers; pa is
// its accept index (or -1 past the end).
// Loads of one tile (item t of the pair-major order) into registers; pa is
// its accept index, or -1 past the end.  Every load is issued whatever the
// item (an address clamped into range stands in for a missing or invalid
// one), so the number of loads in flight after it is the same on every path
// and the waits for it do not drain the loads of the items behind it.
// ACC_LDS: the accept indices are staged in LDS (B <= READY_ACC_LDS); a load
// from global memory here would be waited for at once, together with every
// load and store still in flight.
template <bool ACC_LDS>
__device__ __forceinline__ void mm_fetch(const StateArgs& a, int t, int T, u32x4 (&P)[MM_CH], int& pa,
                                         const int* s_acc) {
  const int tc = min(t, T - 1);
  const int m = tc / a.B, b = tc - m * a.B;
  const int p = ACC_LDS ? s_acc[b] : a.accept_idx[b];
  pa = t < T ? p : -1;
  const int pc = min(max(p, 0), a.P - 1);
  const int l = m / a.H, hh = m - l * a.H;
  const uint16_t* src = (const uint16_t*)a.states + (int64_t)b * a.sb + (int64_t)pc * a.sp +
                        (int64_t)a.slot[l] * a.sl + (int64_t)hh * a.sh;
#pragma unroll
  for (int p2 = 0; p2 < MM_CH; ++p2) {
    const int e = threadIdx.x + MM_THREADS * p2;
    P[p2] = __builtin_nontemporal_load((const u32x4*)(src + (e >> 4) * READY_TILE + (e & 15) * 8));
  }
}

// First K-split partial sums of z and of the squares of h for item t: the
// four elements (zj, zi .. zi + 3) of this thread, one 16-byte load, and the
// sum of squares of row zj (clamped into range like the tile loads; values
// outside j < n, i < r are not used).  r is a multiple of 8, so the four
// elements lie in one row and one aligned 16-byte chunk.
__device__ __forceinline__ void mm_zfetch(const StateArgs& a, int t, int T, int zj, int zi, float (&zr)[4],
                                          float& hr) {
  const int tc = min(t, T - 1);
  const int m = tc / a.B, b = tc - m * a.B;
  const int mz = a.shared ? 0 : m;
  const int64_t row = (int64_t)b * a.n + min(zj, a.n - 1);
  const float4 v = *(const float4*)(a.zpart + row * a.nz + mz * a.r + min(zi, a.r - 4));
  zr[0] = v.x; zr[1] = v.y; zr[2] = v.z; zr[3] = v.w;
  hr = a.hss[row];
}

// U^T and V^T of reader pair mz into LDS, zero past rank r up to rp.
__device__ __forceinline__ void mm_stage_uv(const StateArgs& a, int mz, int rp, unsigned char* smem) {
  uint16_t* ut = (uint16_t*)(smem + MM_UT);
  uint16_t* vt = (uint16_t*)(smem + MM_VT);
  const int r = a.r;
  const uint16_t* U = (const uint16_t*)a.u + (int64_t)mz * r * READY_TILE;
  const uint16_t* V = (const uint16_t*)a.v + (int64_t)mz * READY_TILE * r;
  // U [i][c]: chunk (i, 8 columns) -> U^T[c .. c + 7][i]
  for (int e = threadIdx.x; e < rp * 16; e += MM_THREADS) {
    const int i = e >> 4, c0 = (e & 15) * 8;
    u32x4 w = u32x4{0u, 0u, 0u, 0u};
    if (i < r) w = *(const u32x4*)(U + (int64_t)i * READY_TILE + c0);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ut[(c0 + 2 * k) * MM_LD + i] = (uint16_t)(ww[k] & 0xffffu);
      ut[(c0 + 2 * k + 1) * MM_LD + i] = (uint16_t)(ww[k] >> 16);
    }
  }
  // V [v][i]: chunk (v, 8 ranks) -> V^T[i .. i + 7][v]
  const int vch = rp / 8;
  for (int e = threadIdx.x; e < READY_TILE * vch; e += MM_THREADS) {
    const int v = e / vch, i0 = (e - v * vch) * 8;
    u32x4 w = u32x4{0u, 0u, 0u, 0u};
    if (i0 < r) w = *(const u32x4*)(V + (int64_t)v * r + i0);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      vt[(i0 + 2 * k) * MM_LD + v] = (uint16_t)(ww[k] & 0xffffu);
      vt[(i0 + 2 * k + 1) * MM_LD + v] = (uint16_t)(ww[k] >> 16);
    }
  }
}

// One tile: item t with its loaded chunks P and accept index pa.
__device__ __forceinline__ void mm_tile(const StateArgs& a, int t, const u32x4 (&P)[MM_CH], int pa, int rp,
                                        int zj, int zi, const float (&zr)[4], float hr, unsigned char* smem,
                                        int& cur_mz) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int m = t / a.B, b = t - m * a.B;
  const int mz = a.shared ? 0 : m;
  const int n = a.n, r = a.r, F = a.F;
  const int64_t frow = (int64_t)(b * n) * F + (int64_t)m * (r + 1);
  const int tile = b * a.M + m;
  const bool valid = pa >= 0 && pa < a.P;

  if (mz != cur_mz) {
    __syncthreads();  // the previous tile's readout is done with V^T
    mm_stage_uv(a, mz, rp, smem);
    cur_mz = mz;
  }

  // ---- steps 1-2: gathered copy, sum of squares, tile into LDS ----
  float ss = 0.0f;
  if (valid) {
    uint16_t* dst = (uint16_t*)a.gathered + (int64_t)tile * READY_TILE_ELEMS;
#pragma unroll
    for (int p = 0; p < MM_CH; ++p) {
      const int e = tid + MM_THREADS * p;
      const int v = e >> 4, ch = e & 15;
      __builtin_nontemporal_store(P[p], (u32x4*)(dst + v * READY_TILE + ch * 8));
      ss += sumsq_bf16x8(P[p]);
      *(u32x4*)(smem + MM_S + v * 256 + ((ch ^ (v & 15)) << 4)) = P[p];
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) ((float*)(smem + MM_SS))[wave] = ss;

  // ---- z_j of this pair (zero outside j < n, i < r) as hi + lo ----
  uint16_t* zs = (uint16_t*)(smem + MM_ZS);
  if (zj < 16 && zi < rp) {
    float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (zj < n && zi < r) {
      const int64_t row = (int64_t)b * n + zj;
      float zz[4] = {zr[0], zr[1], zr[2], zr[3]};
      float hs = hr;
      for (int ks = 1; ks < a.ksz; ++ks) {
        const float4 v = *(const float4*)(a.zpart + ((int64_t)ks * a.B * n + row) * a.nz + mz * r + zi);
        zz[0] += v.x; zz[1] += v.y; zz[2] += v.z; zz[3] += v.w;
        hs += a.hss[(int64_t)ks * a.B * n + row];
      }
      const float rs = 1.0f / sqrtf(hs / (float)a.d + a.h_eps);
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = zz[e] * rs;
    }
    uint16_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split_bf16(z[e], hi[e], lo[e]);
    *(uint2*)(zs + zj * MM_LD + zi) = make_uint2((uint32_t)hi[0] | ((uint32_t)hi[1] << 16),
                                                 (uint32_t)hi[2] | ((uint32_t)hi[3] << 16));
    *(uint2*)(zs + (16 + zj) * MM_LD + zi) = make_uint2((uint32_t)lo[0] | ((uint32_t)lo[1] << 16),
                                                        (uint32_t)lo[2] | ((uint32_t)lo[3] << 16));
  }
  __syncthreads();
  const float* wss = (const float*)(smem + MM_SS);
  const float ms = (((wss[0] + wss[1]) + (wss[2] + wss[3])) + ((wss[4] + wss[5]) + (wss[6] + wss[7]))) *
                   (1.0f / READY_TILE_ELEMS);
  const float rms = sqrtf(ms + a.state_eps);

  // ---- q^T = z^T U: wave w owns columns c in [16 w, 16 w + 16) ----
  {
    f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const uint16_t* ut = (const uint16_t*)(smem + MM_UT);
    for (int ks = 0; ks < rp / 32; ++ks) {
      const int k0 = 32 * ks + 8 * lg;
      const u32x4 bop = *(const u32x4*)(ut + (16 * wave + lr) * MM_LD + k0);
      const u32x4 ahi = *(const u32x4*)(zs + lr * MM_LD + k0);
      const u32x4 alo = *(const u32x4*)(zs + (16 + lr) * MM_LD + k0);
      acc = mfma16x16x32(ahi, bop, acc);
      acc = mfma16x16x32(alo, bop, acc);
    }
    uint16_t* qs = (uint16_t*)(smem + MM_QS);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint16_t hi, lo;
      split_bf16(acc[e], hi, lo);
      qs[(4 * lg + e) * MM_LD + 16 * wave + lr] = hi;
      qs[(16 + 4 * lg + e) * MM_LD + 16 * wave + lr] = lo;
    }
  }
  __syncthreads();

  // ---- Y = S q: wave w owns rows v in [16 w, 16 w + 16) ----
  {
    f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const uint16_t* qs = (const uint16_t*)(smem + MM_QS);
    const int v = 16 * wave + lr;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = 4 * ks + lg;
      const u32x4 aop = *(const u32x4*)(smem + MM_S + v * 256 + ((ch ^ (v & 15)) << 4));
      const u32x4 bhi = *(const u32x4*)(qs + lr * MM_LD + 8 * ch);
      const u32x4 blo = *(const u32x4*)(qs + (16 + lr) * MM_LD + 8 * ch);
      acc = mfma16x16x32(aop, bhi, acc);
      acc = mfma16x16x32(aop, blo, acc);
    }
    // lane holds Y[16 w + 4 lg + e][lr]: four neighbouring v of row lr of Y^T
    uint16_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split_bf16(acc[e], hi[e], lo[e]);
    uint16_t* yt = (uint16_t*)(smem + MM_YT);
    const int v0 = 16 * wave + 4 * lg;
    *(uint2*)(yt + lr * MM_LD + v0) = make_uint2((uint32_t)hi[0] | ((uint32_t)hi[1] << 16),
                                                 (uint32_t)hi[2] | ((uint32_t)hi[3] << 16));
    *(uint2*)(yt + (16 + lr) * MM_LD + v0) = make_uint2((uint32_t)lo[0] | ((uint32_t)lo[1] << 16),
                                                        (uint32_t)lo[2] | ((uint32_t)lo[3] << 16));
  }
  __syncthreads();

  // ---- u^T = Y^T V / (rms sqrt(d_k)): wave w owns ranks i in [16 w, 16 w + 16) ----
  const float scale = 0.08838834764831845f / rms;  // 1 / (sqrt(d_k) rms), d_k = 128
  if (16 * wave < rp) {
    f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const uint16_t* yt = (const uint16_t*)(smem + MM_YT);
    const uint16_t* vt = (const uint16_t*)(smem + MM_VT);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k0 = 32 * ks + 8 * lg;
      const u32x4 bop = *(const u32x4*)(vt + (16 * wave + lr) * MM_LD + k0);
      const u32x4 ahi = *(const u32x4*)(yt + lr * MM_LD + k0);
      const u32x4 alo = *(const u32x4*)(yt + (16 + lr) * MM_LD + k0);
      acc = mfma16x16x32(ahi, bop, acc);
      acc = mfma16x16x32(alo, bop, acc);
    }
    const int i = 16 * wave + lr;
    if (i < r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * lg + e;
        if (j < n) {
          const float uv = valid ? acc[e] * scale : 0.0f;
          a.f[frow + (int64_t)j * F + i] = uv;
          if (a.feat) a.feat[frow + (int64_t)j * F + i] = uv;
        }
      }
    }
  }

  // ---- log-RMS scale after the pair's readouts; validity flags ----
  const float ell = valid ? logf(rms) : 0.0f;
  if (tid < n) {
    a.f[frow + (int64_t)tid * F + r] = ell;
    if (a.feat) a.feat[frow + (int64_t)tid * F + r] = ell;
  }
  if (tid == 0) {
    if (valid) {
      if (a.logrms) a.logrms[tile] = ell;
      if (m == 0) a.seq_invalid[b] = 0;
    } else {
      if (a.dev_status) a.dev_status[0] = READY_ERR_ACCEPT_IDX;
      if (m == 0) a.seq_invalid[b] = 1;
    }
  }
}

}  // namespace

template <bool ACC_LDS>
__global__ __launch_bounds__(MM_THREADS, 1) void k_state_mm(StateArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int T = a.B * a.M;
  const int G = gridDim.x, g = blockIdx.x;
  const int t0 = (int)((int64_t)g * T / G), t1 = (int)((int64_t)(g + 1) * T / G);
  const int rp = (a.r + 31) & ~31;
  // this thread's elements of z: row zj, ranks zi .. zi + 3 (rp / 4 threads
  // per row; 16 rows need at most 512 threads since rp <= 128)
  const int zj = threadIdx.x / (rp / 4), zi = 4 * (threadIdx.x - zj * (rp / 4));
  int* s_acc = (int*)(smem + MM_ACC);
  if (ACC_LDS)
    for (int i = threadIdx.x; i < a.B; i += MM_THREADS) s_acc[i] = a.accept_idx[i];
  __syncthreads();
  // three sets of prefetched registers, for items t, t + 1 and t + 2 modulo
  // 3 (a register copy of a value still being loaded would wait for every
  // load in flight)
  float z0[4], z1[4], z2[4], h0, h1, h2;
  u32x4 P0[MM_CH], P1[MM_CH], P2[MM_CH];
  int pa0, pa1, pa2;
  mm_fetch<ACC_LDS>(a, t0, t1, P0, pa0, s_acc);
  mm_zfetch(a, t0, t1, zj, zi, z0, h0);
  mm_fetch<ACC_LDS>(a, t0 + 1, t1, P1, pa1, s_acc);
  mm_zfetch(a, t0 + 1, t1, zj, zi, z1, h1);
  mm_fetch<ACC_LDS>(a, t0 + 2, t1, P2, pa2, s_acc);
  mm_zfetch(a, t0 + 2, t1, zj, zi, z2, h2);
  int cur_mz = -1;
  for (int t = t0; t < t1; t += 3) {
    mm_tile(a, t, P0, pa0, rp, zj, zi, z0, h0, smem, cur_mz);
    mm_fetch<ACC_LDS>(a, t + 3, t1, P0, pa0, s_acc);
    mm_zfetch(a, t + 3, t1, zj, zi, z0, h0);
    if (t + 1 < t1) mm_tile(a, t + 1, P1, pa1, rp, zj, zi, z1, h1, smem, cur_mz);
    mm_fetch<ACC_LDS>(a, t + 4, t1, P1, pa1, s_acc);
    mm_zfetch(a, t + 4, t1, zj, zi, z1, h1);
    if (t + 2 < t1) mm_tile(a, t + 2, P2, pa2, rp, zj, zi, z2, h2, smem, cur_mz);
    mm_fetch<ACC_LDS>(a, t + 5, t1, P2, pa2, s_acc);
    mm_zfetch(a, t + 5, t1, zj, zi, z2, h2);
  }
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

hipError_t ready_launch_state_mm(const StateArgs& a, int grid, hipStream_t s, StageEvents ev) {
  if (a.B <= READY_ACC_LDS)
    READY_LAUNCH(k_state_mm<true>, dim3((unsigned)grid), dim3(MM_THREADS), MM_BYTES, s, ev, a);
  else
    READY_LAUNCH(k_state_mm<false>, dim3((unsigned)grid), dim3(MM_THREADS), MM_BYTES, s, ev, a);
  return hipGetLastError();
}
