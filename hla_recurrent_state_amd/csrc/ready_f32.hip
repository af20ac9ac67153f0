// Single-launch form of the ReaDy state reader for fp32 states, activations
// and weights at serving sizes (at most 16 rows B n, rank r <= 16), for
// gfx950: k_reader_f32.  Arithmetic is fp32 FMA throughout (VALU); nothing
// is narrowed.
//
// The workgroups run four kinds of work item:
//   S  per (sequence, pair) tile: fused gather at the accept index into the
//      caller's buffer, mean square, log-RMS and P = V^T S_bar U^T / sqrt(d_k),
//      an r x r matrix (steps 1-3; u_j = T q_j / sqrt(d_k) with T = V^T S_bar
//      and q_j = U^T z_j is P z_j)
//   Z  per 64 columns of z and K chunk of 256: the partial sums of
//      z = W_q (gamma h) and of the squares of h (step 4).  The item that
//      completes a column block's last chunk sums the chunks in chunk order
//      and divides by rms(h_j); where the chunks are few (zsum_a), the A
//      items sum them instead.
//   A  per 16 columns of a: f_j = [P z_j / rms(h_j), ell] per pair, then
//      a = act(W1 f + b1) (step 4 readout, step 5)
//   O  per 32 columns of out: out = h + W2 a + b2 (step 5)
// S and Z items never wait; an A item waits for every S item and every
// column block of z; an O item waits for every A item.  Each kind sits in
// 64 queues, 8 per XCD (S items first, then Z items, in one queue set; item
// i in queue i % 64), so that few workgroups share a claim counter.  A
// workgroup claims from one queue of each kind on the XCD it runs on: all
// its S and Z items, then A items, then O items, claiming the next item of a
// queue while it works on the current one (the claim's round trip hides
// behind the item).  Before its first A item it reads the queues' arrival
// flags: a queue that no workgroup of the launch has taken from yet (other
// kernels hold its XCD, say, or the grid is smaller) is an orphan, and the
// workgroup drains the orphan's S and Z queue, then after its own A queue
// the orphan's A queue, and likewise for O.  So every item waits only for items that
// running workgroups hold or take before they wait themselves, and the
// launch completes whatever part of its grid is resident.  A and O items
// request their weights before they wait.
//
// Cross-workgroup data (z partial sums, P, ell, the invalid-sequence flags,
// a) goes through device-coherent stores and loads, announced by relaxed
// counters (ready_sync.h).  Waits are bounded; the last workgroup to finish
// clears the counters for the next call.
//
// Formulas: ReaDy arXiv text, section 3.1 "Position-conditioned reading" and
// "Fusion and residual injection" (the Eq. (3) and Eq. (4) displays are lost
// in extraction; the rainbus summary, 方法步骤详情 steps (1)-(3), writes the
// reader out); section 3.2 "Avoiding redundant data movement" for the fused
// gather and "State-access footprint" for the projected state shared by
// every position of the block.
#include "ready_common.h"
#include "ready_sync.h"

namespace {

__device__ __forceinline__ float4 as_f4(const u32x4& v) {
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
__device__ __forceinline__ float dot4(float acc, const float4& p, const float4& q) {
  acc = fmaf(p.x, q.x, acc);
  acc = fmaf(p.y, q.y, acc);
  acc = fmaf(p.z, q.z, acc);
  return fmaf(p.w, q.w, acc);
}

// Sum over each row of 16 lanes, left in every lane of the row: four DPP
// steps (lanes i ^ 1, i ^ 2, then the mirror within 8 and within 16 lanes),
// no trip through LDS.  Every lane adds the same pairs, so all get the same
// bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xb1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4e>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  return v;
}
// LDS reads above this point are issued before any use below it: the
// compiler would otherwise place each read just before its first use and
// wait for it there, one read at a time.
__device__ __forceinline__ void issue_point() { asm volatile("" ::: "memory"); }

// Thread 0 waits until *c1 >= w1 and *c2 >= w2; the workgroup learns the
// outcome (false: the wait gave up, see wait_count).
__device__ bool f32_wait(const F32Args& a, const uint32_t* c1, uint32_t w1, const uint32_t* c2, uint32_t w2,
                         int* s_flag) {
  if (threadIdx.x == 0) {
    uint32_t last;
    *s_flag = wait_count2<true>(c1, w1, c2, 0xffffffffu, w2, &last, a.abort_flag, a.dev_status) ? 1 : 0;
  }
  __syncthreads();
  const bool ok = *s_flag != 0;
  __syncthreads();
  return ok;
}

// ---------------------------------------------------------------- S items

// Tile t = b M + m.  Thread i holds columns 4 (i % 32) .. + 3 of rows
// i / 32 + 8 k (k < 16), and stores them into the gathered buffer once P
// and ell are out and counted.  T = V^T S is formed 8 ranks at a time: each
// thread sums its 16 rows, lanes i and i + 32 of a wave fold together, and
// the four waves' partial rows meet in LDS, where P's rows of the chunk are
// formed against U (TP threads per element of P).
template <int RR>
__device__ void f32_s_item(const F32Args& a, int t, const int* s_acc, float* smem) {
  constexpr int LU = READY_TILE + 4;        // padded row of U and of T (floats)
  constexpr int NUV = RR * 32 * 2 / 256;    // 16-byte chunks of U and V per thread
  constexpr int TP = 32 / RR;               // threads per element of P
  float* sU = smem;                         // [RR][LU]
  float* sV = sU + RR * LU;                 // [128][RR]
  float* sT = sV + READY_TILE * RR;         // [4 waves][8][LU]: partial rows of T
  float* s_ws = sT + 4 * 8 * LU;            // [4]
  const int tid = item_tid(), lane = tid & 63, wave = tid >> 6;
  const int b = t / a.M, m = t - (t / a.M) * a.M;
  const int p = s_acc[b];
  const bool valid = p >= 0 && p < a.P;
  const int mz = a.shared ? 0 : m;
  const int cc = tid & 31, v0 = tid >> 5;

  const u32x4* Ug = (const u32x4*)(a.u + (int64_t)mz * RR * READY_TILE);
  const u32x4* Vg = (const u32x4*)(a.v + (int64_t)mz * READY_TILE * RR);
  u32x4 uv[NUV];
#pragma unroll
  for (int k = 0; k < NUV; ++k) {
    const int c = tid + 256 * k;
    uv[k] = c < RR * 32 ? Ug[c] : Vg[c - RR * 32];
  }
  u32x4 x[16];
  if (valid) {
    const int l = m / a.H, hh = m - (m / a.H) * a.H;
    const u32x4* src = (const u32x4*)(a.states + (int64_t)b * a.sb + (int64_t)p * a.sp + (int64_t)a.slot[l] * a.sl +
                                      (int64_t)hh * a.sh);
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = __builtin_nontemporal_load(src + (v0 + 8 * i) * 32 + cc);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = u32x4{0u, 0u, 0u, 0u};
  }
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 f = as_f4(x[i]);
    ss = fmaf(f.x, f.x, ss);
    ss = fmaf(f.y, f.y, ss);
    ss = fmaf(f.z, f.z, ss);
    ss = fmaf(f.w, f.w, ss);
  }
#pragma unroll
  for (int k = 0; k < NUV; ++k) {
    const int c = tid + 256 * k;
    if (c < RR * 32) *(u32x4*)&sU[(c >> 5) * LU + 4 * (c & 31)] = uv[k];
    else *(u32x4*)&sV[4 * (c - RR * 32)] = uv[k];
  }
  ss = wave_sum(ss);
  if (lane == 0) s_ws[wave] = ss;
  __syncthreads();

  if (!valid) {
    // out-of-range accept index: flag it; the A items give the sequence's
    // rows zero features and the O items leave its out and delta alone
    if (tid == 0) {
      if (a.dev_status) st_coh_u32(a.dev_status, (uint32_t)READY_ERR_ACCEPT_IDX);
      if (m == 0) st_coh_u32(a.seq_invalid + b, 1u);
    }
    wait_mem();
    __syncthreads();
    if (tid == 0) count_up(a.sdone);
    return;
  }

  const float ms = ((s_ws[0] + s_ws[1]) + (s_ws[2] + s_ws[3])) * (1.0f / READY_TILE_ELEMS);
  const float rms = sqrtf(ms + a.state_eps);
  const float scale = 0.08838834764831845f / rms;  // 1 / (rms sqrt(d_k)), d_k = 128
  float* P = a.pmat + (int64_t)t * RR * RR;
#pragma unroll 1
  for (int rc = 0; rc < RR; rc += 8) {
    float acc[8][4];
#pragma unroll
    for (int ii = 0; ii < 8; ++ii)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[ii][e] = 0.0f;
#pragma unroll
    for (int i0 = 0; i0 < 16; i0 += 8) {
      float4 vr[8][2];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int v = v0 + 8 * (i0 + i);
        vr[i][0] = *(const float4*)&sV[v * RR + rc];
        vr[i][1] = *(const float4*)&sV[v * RR + rc + 4];
      }
      issue_point();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float vv[8] = {vr[i][0].x, vr[i][0].y, vr[i][0].z, vr[i][0].w,
                             vr[i][1].x, vr[i][1].y, vr[i][1].z, vr[i][1].w};
        const float4 f = as_f4(x[i0 + i]);
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          acc[ii][0] = fmaf(vv[ii], f.x, acc[ii][0]);
          acc[ii][1] = fmaf(vv[ii], f.y, acc[ii][1]);
          acc[ii][2] = fmaf(vv[ii], f.z, acc[ii][2]);
          acc[ii][3] = fmaf(vv[ii], f.w, acc[ii][3]);
        }
      }
    }
#pragma unroll
    for (int ii = 0; ii < 8; ++ii)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[ii][e] += __shfl_xor(acc[ii][e], 32, 64);
    if (lane < 32) {
#pragma unroll
      for (int ii = 0; ii < 8; ++ii)
        *(float4*)&sT[(wave * 8 + ii) * LU + 4 * lane] = make_float4(acc[ii][0], acc[ii][1], acc[ii][2], acc[ii][3]);
    }
    __syncthreads();
    {
      // element (rc + ii, ip) of P: TP threads, each over the columns
      // 4 part + 4 TP q of T's row and U's row
      const int o = tid / TP, part = tid - (tid / TP) * TP;
      const int ii = o / RR, ip = o - (o / RR) * RR;
      float s = 0.0f;
      constexpr int NQ = 32 / TP, QB = 4;  // columns in NQ steps, QB steps per batch of reads
#pragma unroll
      for (int q0 = 0; q0 < NQ; q0 += QB) {
        float4 tv[QB][5];
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          const int k = 4 * part + 4 * TP * (q0 + q);
#pragma unroll
          for (int w = 0; w < 4; ++w) tv[q][w] = *(const float4*)&sT[(w * 8 + ii) * LU + k];
          tv[q][4] = *(const float4*)&sU[ip * LU + k];
        }
        issue_point();
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          const float4 tr = make_float4((tv[q][0].x + tv[q][1].x) + (tv[q][2].x + tv[q][3].x),
                                        (tv[q][0].y + tv[q][1].y) + (tv[q][2].y + tv[q][3].y),
                                        (tv[q][0].z + tv[q][1].z) + (tv[q][2].z + tv[q][3].z),
                                        (tv[q][0].w + tv[q][1].w) + (tv[q][2].w + tv[q][3].w));
          s = dot4(s, tr, tv[q][4]);
        }
      }
#pragma unroll
      for (int off = 1; off < TP; off <<= 1) s += __shfl_xor(s, off, 64);
      if (part == 0) st_coh_f32(P + (rc + ii) * RR + ip, s * scale);
    }
    __syncthreads();  // sT is rewritten by the next chunk
  }
  if (tid == 0) {
    const float ell = logf(rms);
    st_coh_f32(a.ell + t, ell);
    if (a.logrms) a.logrms[t] = ell;
    if (m == 0) st_coh_u32(a.seq_invalid + b, 0u);
  }
  wait_mem();
  __syncthreads();
  if (tid == 0) count_up(a.sdone);
  // the gathered tile last: nothing in the launch reads it, so the count
  // above does not wait for these stores
  u32x4* dst = (u32x4*)(a.gathered + (int64_t)t * READY_TILE_ELEMS);
#pragma unroll
  for (int i = 0; i < 16; ++i) __builtin_nontemporal_store(x[i], dst + (v0 + 8 * i) * 32 + cc);
}

// ---------------------------------------------------------------- Z items

// Columns [64 cb, 64 cb + 64) of z (one per lane) over K chunk ks: wave w
// takes the chunk's values [64 w, 64 w + 64), its W_q row pieces straight
// into registers, gamma h of every row staged in LDS (read by all lanes at
// once).  The four waves' sums meet in LDS and are stored in zpart; the
// sums of squares of h of the chunk go to hss (every column block keeps its
// own copy, so that the item completing a column block finds all it needs).
template <int RR, int RB>
__device__ void f32_z_item(const F32Args& a, int cb, int ks, float* smem, int* s_flag) {
  constexpr int KC = READY_F32_KC;
  constexpr int HQ = RB * 64 / 256;          // 16-byte chunks of h per thread
  float* s_h = smem;                         // [RB][KC]: gamma h
  float* s_red = s_h + RB * KC;              // [4][RB][64]
  const int tid = item_tid(), lane = tid & 63, wave = tid >> 6;
  const int R = a.R, d = a.d;
  const int k0 = ks * KC, kn = min(KC, d - k0);
  const int c = READY_F32_ZC * cb + lane;
  const bool cval = c < a.Nz;
  const int kw = 64 * wave;
  u32x4 w[16];
#pragma unroll
  for (int s = 0; s < 16; ++s)
    w[s] = ld_ro16_at(cval && kw + 4 * s < kn, a.wq, 4u * (uint32_t)(c * d + k0 + kw + 4 * s));
  u32x4 hv[HQ];
#pragma unroll
  for (int q = 0; q < HQ; ++q) {
    const int j = wave + 4 * q;
    hv[q] = ld_ro16_at(j < R && 4 * lane < kn, a.h, 4u * (uint32_t)(j * d + k0 + 4 * lane));
  }
  const u32x4 gv = ld_ro16_at(a.gamma != nullptr && 4 * lane < kn, a.gamma ? a.gamma : a.h, 4u * (uint32_t)(k0 + 4 * lane));
  const float4 g = a.gamma ? as_f4(gv) : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
#pragma unroll
  for (int q = 0; q < HQ; ++q) {
    const int j = wave + 4 * q;
    const float4 f = as_f4(hv[q]);
    float sq = fmaf(f.x, f.x, fmaf(f.y, f.y, fmaf(f.z, f.z, f.w * f.w)));
    sq = wave_sum(sq);
    if (lane == 0 && j < R) st_coh_f32(a.hss + ((int64_t)(cb * a.nks + ks) * R + j), sq);
    *(float4*)&s_h[j * KC + 4 * lane] = make_float4(g.x * f.x, g.y * f.y, g.z * f.z, g.w * f.w);
  }
  __syncthreads();
  float acc[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j) acc[j] = 0.0f;
  // gamma h of step s + 1 is requested before step s is summed
  float4 hb[2][RB];
#pragma unroll
  for (int j = 0; j < RB; ++j) hb[0][j] = *(const float4*)&s_h[j * KC + kw];
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    if (s + 1 < 16) {
#pragma unroll
      for (int j = 0; j < RB; ++j) hb[(s + 1) & 1][j] = *(const float4*)&s_h[j * KC + kw + 4 * (s + 1)];
    }
    issue_point();
    const float4 wf = as_f4(w[s]);
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[j] = dot4(acc[j], wf, hb[s & 1][j]);
  }
#pragma unroll
  for (int j = 0; j < RB; ++j) s_red[(wave * RB + j) * 64 + lane] = acc[j];
  __syncthreads();
  for (int e = tid; e < RB * 64; e += 256) {
    const int j = e >> 6, cl = e & 63, col = READY_F32_ZC * cb + cl;
    if (j < R && col < a.Nz)
      st_coh_f32(a.zpart + ((int64_t)ks * R + j) * a.Nz + col,
                 ((s_red[j * 64 + cl] + s_red[(RB + j) * 64 + cl]) + s_red[(2 * RB + j) * 64 + cl]) +
                     s_red[(3 * RB + j) * 64 + cl]);
  }
  wait_mem();
  __syncthreads();
  if (a.zsum_a) {
    // the A items sum the chunks themselves: count this one
    if (tid == 0) count_up(a.zdone);
    return;
  }
  if (tid == 0) *s_flag = count_up(ctr(a.zcnt, cb)) == (uint32_t)(a.nks - 1) ? 1 : 0;
  __syncthreads();
  if (*s_flag == 0) return;

  // the column block's last chunk: z = (sum of the chunks in chunk order) /
  // rms(h_j), rows j = w + 4 q of wave w, in trips of up to KB chunks;
  // the squares of h of row j come one chunk per lane and meet in a wave sum
  // (the same order in every column block, so every block divides by the
  // same rms(h_j))
  constexpr int KB = 64 / HQ;
  float zs[HQ], hs[HQ];
#pragma unroll
  for (int q = 0; q < HQ; ++q) zs[q] = hs[q] = 0.0f;
  for (int kb = 0; kb < a.nks; kb += KB) {
    float zv[HQ][KB], hl[HQ];
#pragma unroll
    for (int q = 0; q < HQ; ++q) {
      const int j = wave + 4 * q;
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int kk = kb + u;
        zv[q][u] = ld_coh4_at(kk < a.nks && j < R && cval, a.zpart, 4u * (uint32_t)((kk * R + j) * a.Nz + c));
      }
      hl[q] = ld_coh4_at(lane < KB && kb + lane < a.nks && j < R, a.hss,
                         4u * (uint32_t)((cb * a.nks + kb + lane) * R + j));
    }
#pragma unroll
    for (int q = 0; q < HQ; ++q) {
#pragma unroll
      for (int u = 0; u < KB; ++u)
        if (kb + u < a.nks) zs[q] += zv[q][u];
      hs[q] += wave_sum(hl[q]);
    }
  }
  // z of the block's 64 columns into LDS (rows past R hold zeros)
  float* s_zb = s_h;  // [RB][64]
#pragma unroll
  for (int q = 0; q < HQ; ++q) {
    const int j = wave + 4 * q;
    s_zb[j * 64 + lane] = zs[q] * (1.0f / sqrtf(hs[q] / (float)d + a.h_eps));
  }
  // then f of the pairs whose z columns lie in this block (every pair when
  // the reader's parameters are shared), once every S item is done: a unit
  // is row i of one tile's P, giving u_j[i] for the n rows of the tile's
  // sequence, stored with ell into f (rows Fp apart)
  if (!f32_wait(a, a.sdone, (uint32_t)a.n_s, a.sdone, (uint32_t)a.n_s, s_flag)) return;
  constexpr int UM = READY_F32_MAX_UNITS / 256;
  constexpr int PC = RR / 4;
  const int m0 = a.shared ? 0 : (READY_F32_ZC * cb) / RR;
  const int npm = a.shared ? a.M : min(a.M - m0, READY_F32_ZC / RR);
  const int nu = a.B * npm * RR, n = a.n, Fp = (a.F + 63) & ~63;
  u32x4 pr[UM][PC];
  float el[UM];
  uint32_t inv[UM];
#pragma unroll
  for (int k = 0; k < UM; ++k) {
    const int u = tid + 256 * k;
    const bool live = u < nu;
    const int i = u % RR, rest = u / RR, b = live ? rest / npm : 0, t = b * a.M + m0 + (live ? rest - (rest / npm) * npm : 0);
#pragma unroll
    for (int cq = 0; cq < PC; ++cq) pr[k][cq] = ld_coh16_at(live, a.pmat, 16u * (uint32_t)((t * RR + i) * PC + cq));
    el[k] = ld_coh4_at(live, a.ell, 4u * (uint32_t)t);
    inv[k] = __float_as_uint(ld_coh4_at(live, (const float*)a.seq_invalid, 4u * (uint32_t)b));
  }
#pragma unroll
  for (int k = 0; k < UM; ++k) {
    const int u = tid + 256 * k;
    if (u < nu) {
      const int i = u % RR, rest = u / RR, b = rest / npm, m = m0 + rest - (rest / npm) * npm;
      const int zoff = a.shared ? 0 : m * RR - READY_F32_ZC * cb;
      float4 zv[RB][PC];
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const float* zr = &s_zb[min(b * n + j, R - 1) * 64 + zoff];
#pragma unroll
        for (int cq = 0; cq < PC; ++cq) zv[j][cq] = *(const float4*)&zr[4 * cq];
      }
      issue_point();
      const bool ok = inv[k] == 0u;
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        float f = 0.0f;
#pragma unroll
        for (int cq = 0; cq < PC; ++cq) f = dot4(f, as_f4(pr[k][cq]), zv[j][cq]);
        if (j < n) {
          float* fr = a.fbuf + (int64_t)(b * n + j) * Fp + m * (RR + 1);
          st_coh_f32(fr + i, ok ? f : 0.0f);
          if (i == 0) st_coh_f32(fr + RR, ok ? el[k] : 0.0f);
        }
      }
    }
  }
  wait_mem();
  __syncthreads();
  if (tid == 0) count_up(a.zdone);
}

// ---------------------------------------------------------------- A items

// Columns [16 ca, 16 ca + 16) of a: column 16 ca + 4 w + l / 16 for lane l
// of wave w, whose 16 lanes split f's values 4 (l % 16) + 64 s .. + 3; after
// the sums meet, lane l % 16 = j writes row j.  Once every S item and the
// query sums are done, one trip brings z of every row (into LDS), and the
// rows of P, ell and the invalid flags of this thread's units: a unit is one
// row i of one tile's P, giving u_j[i] for the n rows j of the tile's
// sequence.  Where the query sums have few K chunks (zsum_a), the Z items
// leave them unsummed and this trip brings the chunks instead: thread t sums
// chunks g, g + G, ... of 16 bytes t % nq of z (g = t / nq, G = 256 / nq),
// the G slices meet in LDS in slice order, and the scale 1 / rms(h_j) comes
// from the chunks' sums of squares of h.
template <int RR, int RB>
__device__ void f32_a_item(const F32Args& a, int ca, float* smem, int* s_flag) {
  constexpr int FS = READY_F32_MAX_F / 64;
  constexpr int ZQ = READY_F32_MAX_RNZ / 4 / 256;
  static_assert(ZQ >= READY_F32_ZSUM_LOADS, "the chunk loads of zsum_a use the same registers");
  constexpr int UM = READY_F32_MAX_UNITS / 256;
  constexpr int PC = RR / 4;                 // 16-byte chunks of a row of P
  constexpr int HR = RB / 4;                 // rows of h's sums of squares per wave
  const int tid = item_tid(), lane = tid & 63, wave = tid >> 6, part = lane & 15;
  const int R = a.R, F = a.F, Nz = a.Nz, n = a.n;
  const int Fp = (F + 63) & ~63, ns = Fp >> 6;
  float* s_z = smem;                               // [R][Nz]
  float* s_f = s_z + ((R * Nz + 3) & ~3);          // [RB][Fp]
  float* s_zp = s_f;                               // zsum_a: [G][nq] 16-byte slices (before s_f is written)
  float* s_rs = s_f + 1024;                        // zsum_a: [16] 1 / rms(h_j)
  const int col = READY_F32_AC * ca + 4 * wave + (lane >> 4);
  const bool cval = col < a.Hm;
  // W1 row `col` and b1, requested before the wait
  float w1v[FS][4];
#pragma unroll
  for (int s = 0; s < FS; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = 4 * part + 64 * s + e;
      w1v[s][e] = ld_ro4_at(cval && k < F, a.w1, 4u * (uint32_t)(col * F + k));
    }
  const float bias = ld_ro4_at(a.b1 != nullptr && cval, a.b1 ? a.b1 : a.w1, 4u * (uint32_t)col);

  const bool zs_a = a.zsum_a != 0;
  if (!f32_wait(a, a.zdone, zs_a ? (uint32_t)a.n_z : (uint32_t)a.ncz, a.sdone, (uint32_t)a.n_s, s_flag)) return;

  if (!zs_a) {
    // f of every row, formed by the items that summed z (rows Fp apart)
    constexpr int FQ = 16 * READY_F32_MAX_F / 4 / 256;
    const int nf = (R * Fp) >> 2;
    u32x4 fq[FQ];
#pragma unroll
    for (int q = 0; q < FQ; ++q) fq[q] = ld_coh16_at(tid + 256 * q < nf, a.fbuf, 16u * (uint32_t)(tid + 256 * q));
#pragma unroll
    for (int q = 0; q < FQ; ++q)
      if (tid + 256 * q < nf) *(u32x4*)&s_f[4 * (tid + 256 * q)] = fq[q];
    __syncthreads();
  } else {
    const int nq = (R * Nz) >> 2;              // 16-byte chunks of z
    const int G = 256 / nq, g = tid / nq, e4 = tid - g * nq;
    u32x4 zq[ZQ];
    float hl[HR];
#pragma unroll
    for (int q = 0; q < ZQ; ++q) {
      const int kk = g + G * q;
      zq[q] = ld_coh16_at(g < G && kk < a.nks, a.zpart, 16u * (uint32_t)(kk * nq + e4));
    }
#pragma unroll
    for (int i = 0; i < HR; ++i) {
      const int j = wave + 4 * i;  // column block 0's copy of the sums of squares
      hl[i] = ld_coh4_at(lane < a.nks && j < R, a.hss, 4u * (uint32_t)(lane * R + j));
    }
    const int nu = a.n_s * RR;
    u32x4 pr[UM][PC];
    float el[UM];
    uint32_t inv[UM];
#pragma unroll
    for (int k = 0; k < UM; ++k) {
      const int u = tid + 256 * k;
      const bool live = u < nu;
      const int t = live ? u / RR : 0, b = t / a.M;
#pragma unroll
      for (int c = 0; c < PC; ++c) pr[k][c] = ld_coh16_at(live, a.pmat, 16u * (uint32_t)(u * PC + c));
      el[k] = ld_coh4_at(live, a.ell, 4u * (uint32_t)t);
      inv[k] = __float_as_uint(ld_coh4_at(live, (const float*)a.seq_invalid, 4u * (uint32_t)b));
    }
    {
      float4 zsum = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
      for (int q = 0; q < ZQ; ++q) {
        if (g + G * q < a.nks) {
          const float4 v = as_f4(zq[q]);
          zsum.x += v.x; zsum.y += v.y; zsum.z += v.z; zsum.w += v.w;
        }
      }
      if (g < G) *(float4*)&s_zp[4 * (g * nq + e4)] = zsum;
#pragma unroll
      for (int i = 0; i < HR; ++i) {
        const int j = wave + 4 * i;
        const float hs = wave_sum(hl[i]);
        if (lane == 0 && j < R) s_rs[j] = 1.0f / sqrtf(hs / (float)a.d + a.h_eps);
      }
      __syncthreads();
      if (tid < nq) {
        float4 z = *(const float4*)&s_zp[4 * tid];
        for (int gg = 1; gg < G; ++gg) {
          const float4 v = *(const float4*)&s_zp[4 * (gg * nq + tid)];
          z.x += v.x; z.y += v.y; z.z += v.z; z.w += v.w;
        }
        const float rs = s_rs[(4 * tid) / Nz];
        *(float4*)&s_z[4 * tid] = make_float4(z.x * rs, z.y * rs, z.z * rs, z.w * rs);
      }
      __syncthreads();  // s_f reuses the slices' area
    }
#pragma unroll
    for (int k = 0; k < UM; ++k) {
      const int u = tid + 256 * k;
      if (u < nu) {
        const int t = u / RR, i = u - (u / RR) * RR, b = t / a.M, m = t - (t / a.M) * a.M;
        const int mz = a.shared ? 0 : m;
        // u_j[i] for the RB rows from the sequence's first (rows past the
        // last one read row R - 1 and are dropped): every read issued before
        // any sum needs one
        float4 zv[RB][PC];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          const float* zr = &s_z[min(b * n + j, R - 1) * Nz + mz * RR];
#pragma unroll
          for (int c = 0; c < PC; ++c) zv[j][c] = *(const float4*)&zr[4 * c];
        }
        issue_point();
        float f[RB];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          f[j] = 0.0f;
#pragma unroll
          for (int c = 0; c < PC; ++c) f[j] = dot4(f[j], as_f4(pr[k][c]), zv[j][c]);
        }
        const bool ok = inv[k] == 0u;
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          if (j < n) {
            float* fr = &s_f[(b * n + j) * Fp + m * (RR + 1)];
            fr[i] = ok ? f[j] : 0.0f;
            if (i == 0) fr[RR] = ok ? el[k] : 0.0f;
          }
        }
      }
    }
  }
  // f's padding columns [F, Fp) are zero in LDS
  if (tid < Fp - F) {
    for (int j = 0; j < R; ++j) s_f[j * Fp + F + tid] = 0.0f;
  }
  __syncthreads();
  if (ca == 0 && a.feat) {
    for (int j = 0; j < R; ++j)
      for (int k = tid; k < F; k += 256) a.feat[(int64_t)j * F + k] = s_f[j * Fp + k];
  }
  float acc[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j) acc[j] = 0.0f;
  // rows j >= R of s_f hold no data; their sums are dropped
#pragma unroll
  for (int s = 0; s < FS; ++s) {
    if (s < ns) {
      const float4 wf = make_float4(w1v[s][0], w1v[s][1], w1v[s][2], w1v[s][3]);
      float4 fv[RB];
#pragma unroll
      for (int j = 0; j < RB; ++j) fv[j] = *(const float4*)&s_f[j * Fp + 4 * part + 64 * s];
      issue_point();
#pragma unroll
      for (int j = 0; j < RB; ++j) acc[j] = dot4(acc[j], wf, fv[j]);
    }
  }
  float v = 0.0f;
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const float sj = row16_sum(acc[j]);
    v = part == j ? sj : v;
  }
  if (part < R && cval) st_coh_f32(a.abuf + (int64_t)part * a.Hm + col, activation(v + bias, a.act));
  wait_mem();
  __syncthreads();
  if (tid == 0) count_up(a.adone);
}

// ---------------------------------------------------------------- O items

// Columns [32 co, 32 co + 32) of out in two passes of 16: column
// 32 co + 16 pass + 4 w + l / 16 for lane l of wave w, whose 16 lanes split
// a's values 4 (l % 16) + 64 s .. + 3; after the sums meet, lane l % 16 = j
// writes row j.  W2 rows, b2 and h are requested before the wait for the A
// items; a of every row comes into LDS after it.
template <int RB>
__device__ void f32_o_item(const F32Args& a, int co, float* smem, int* s_flag) {
  constexpr int HS = READY_F32_MAX_HM / 64;
  constexpr int NP = READY_F32_OC / 16;
  const int tid = item_tid(), lane = tid & 63, wave = tid >> 6, part = lane & 15;
  const int R = a.R, Hm = a.Hm, d = a.d;
  const int Hp = (Hm + 63) & ~63, hn = Hp >> 6, h4 = Hm >> 2;
  float* s_a = smem;                         // [RB][Hp]
  const bool rowl = part < R;                // this lane writes row `part`
  u32x4 wv[NP][HS];
  float hv[NP], bv[NP];
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int col = READY_F32_OC * co + 16 * pp + 4 * wave + (lane >> 4);
    const bool cval = col < d;
#pragma unroll
    for (int s = 0; s < HS; ++s)
      wv[pp][s] = ld_ro16_at(cval && 4 * part + 64 * s < Hm, a.w2, 4u * (uint32_t)(col * Hm + 4 * part + 64 * s));
    hv[pp] = ld_ro4_at(rowl && cval, a.h, 4u * (uint32_t)(part * d + col));
    bv[pp] = ld_ro4_at(a.b2 != nullptr && cval, a.b2 ? a.b2 : a.w2, 4u * (uint32_t)col);
  }

  if (!f32_wait(a, a.adone, (uint32_t)a.n_a, a.adone, (uint32_t)a.n_a, s_flag)) return;

  // a of every row (Hm / 4 <= 128 chunks of 16 bytes a row), and the flag of
  // the sequence of this lane's row
  u32x4 aq[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j) aq[j] = ld_coh16_at(j < R && tid < h4, a.abuf, 16u * (uint32_t)(j * h4 + tid));
  const uint32_t inv = __float_as_uint(ld_coh4_at(rowl, (const float*)a.seq_invalid, 4u * (uint32_t)(part / a.n)));
#pragma unroll
  for (int j = 0; j < RB; ++j)
    if (j < R && tid < h4) *(u32x4*)&s_a[j * Hp + 4 * tid] = aq[j];
  if (tid < (Hp - Hm) >> 2) {
    for (int j = 0; j < R; ++j) *(float4*)&s_a[j * Hp + Hm + 4 * tid] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  __syncthreads();
  const bool wr = rowl && inv == 0u;
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int col = READY_F32_OC * co + 16 * pp + 4 * wave + (lane >> 4);
    float acc[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[j] = 0.0f;
    // rows j >= R of s_a hold no data; their sums are dropped
#pragma unroll
    for (int s = 0; s < HS; ++s) {
      if (s < hn) {
        const float4 wf = as_f4(wv[pp][s]);
        float4 av[RB];
#pragma unroll
        for (int j = 0; j < RB; ++j) av[j] = *(const float4*)&s_a[j * Hp + 4 * part + 64 * s];
        issue_point();
#pragma unroll
        for (int j = 0; j < RB; ++j) acc[j] = dot4(acc[j], wf, av[j]);
      }
    }
    float v = 0.0f;
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const float sj = row16_sum(acc[j]);
      v = part == j ? sj : v;
    }
    if (wr && col < d) {
      const float dh = v + bv[pp];
      a.out[(int64_t)part * d + col] = hv[pp] + dh;
      if (a.delta) a.delta[(int64_t)part * d + col] = dh;
    }
  }
}

}  // namespace

// ---------------------------------------------------------------- k_reader_f32

// RR: the rank (8 or 16); RB: the rows the item loops are built for (8 or
// 16, at least R).
// The items of queue x of one kind, from position k on: thread 0 claims the
// next position as an item starts; run(i) runs item i = x + NQ k.
template <typename Run>
__device__ __forceinline__ void drain(uint32_t* qctr, int x, uint32_t size, uint32_t k, uint32_t* s_bc, Run run) {
  while (k < size) {
    uint32_t nxt = NO_ITEM;
    if (threadIdx.x == 0) nxt = count_up(ctr(qctr, x));
    run(x + READY_F32_QUEUES * (int)k);
    __syncthreads();  // the LDS area is reused by the next item
    if (threadIdx.x == 0) *s_bc = nxt;
    __syncthreads();
    k = *s_bc;
    __syncthreads();
  }
}

template <int RR, int RB>
__global__ __launch_bounds__(256, 2) void k_reader_f32(F32Args a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int s_acc[16];
  __shared__ uint32_t s_bc[3];
  __shared__ int s_flag;
  __shared__ int s_last;
  const int tid = item_tid();
  const int g = blockIdx.x, G = gridDim.x;
  // this workgroup's queues: 8 per XCD, so that few workgroups share a
  // claim counter
  const int xq = hw_xcc() + 8 * ((g >> 3) & 7);
  uint32_t first = NO_ITEM;
  if (tid == 0) {
    first = count_up(ctr(a.lq, xq));
    st_coh_u32(ctr(a.arr_x, xq), 1u);
  }
  const int accv = tid < a.B ? a.accept_idx[tid] : 0;
  if (a.counters[0] != a.magic) {
    // the workspace was not prepared for this plan: touch nothing else (the
    // claim and the mark above changed counter words of the workspace only)
    if (g == 0 && tid == 0 && a.dev_status) *a.dev_status = READY_ERR_WORKSPACE_UNINIT;
    return;
  }
  if (tid < 16) s_acc[tid] = accv;
  if (tid == 0) s_bc[0] = first;
  __syncthreads();
  const uint32_t k0 = s_bc[0];
  __syncthreads();

  const int nl = a.n_s + a.n_z;
  auto qsize = [](int total, int x) { return (uint32_t)((total - x + READY_F32_QUEUES - 1) / READY_F32_QUEUES); };
  auto run_l = [&](int i) {
    if (i < a.n_s) {
      f32_s_item<RR>(a, i, s_acc, smem);
    } else {
      const int k = i - a.n_s, cb = k / a.nks;
      f32_z_item<RR, RB>(a, cb, k - cb * a.nks, smem, &s_flag);
    }
  };
  auto run_a = [&](int i) { f32_a_item<RR, RB>(a, i, smem, &s_flag); };
  auto run_o = [&](int i) { f32_o_item<RB>(a, i, smem, &s_flag); };

  // S and Z items of this workgroup's queue
  drain(a.lq, xq, qsize(nl, xq), k0, s_bc, run_l);
  // the arrival flags, read in the trip of the first A claim; then the S and
  // Z items of orphan queues
  auto flag = [&](int l) { return ctr(a.arr_x, l); };
  uint32_t ka;
  const uint64_t orph = arrival_check(ctr(a.aq, xq), READY_F32_QUEUES, flag, &ka, s_bc);
  for (uint64_t m = orph; m != 0; m &= m - 1) {
    const int y = __ffsll((unsigned long long)m) - 1;
    drain(a.lq, y, qsize(nl, y), claim_one(a.lq, y, qsize(nl, y), s_bc), s_bc, run_l);
  }
  // A items: this workgroup's queue, then the orphans'
  drain(a.aq, xq, qsize(a.n_a, xq), ka, s_bc, run_a);
  for (uint64_t m = orph; m != 0; m &= m - 1) {
    const int y = __ffsll((unsigned long long)m) - 1;
    drain(a.aq, y, qsize(a.n_a, y), claim_one(a.aq, y, qsize(a.n_a, y), s_bc), s_bc, run_a);
  }
  // O items likewise
  drain(a.oq, xq, qsize(a.n_o, xq), claim_one(a.oq, xq, qsize(a.n_o, xq), s_bc), s_bc, run_o);
  for (uint64_t m = orph; m != 0; m &= m - 1) {
    const int y = __ffsll((unsigned long long)m) - 1;
    drain(a.oq, y, qsize(a.n_o, y), claim_one(a.oq, y, qsize(a.n_o, y), s_bc), s_bc, run_o);
  }

  // the last workgroup to finish clears the counters (two-level count)
  __syncthreads();
  if (tid == 0) {
    int last = 0;
    const int grp = g % READY_DONE_GROUPS;
    const int in_grp = (G - grp + READY_DONE_GROUPS - 1) / READY_DONE_GROUPS;
    if (count_up(ctr(a.done, grp)) == (uint32_t)(in_grp - 1))
      last = count_up(ctr(a.done, READY_DONE_GROUPS)) == (uint32_t)(min(G, READY_DONE_GROUPS) - 1);
    s_last = last;
  }
  __syncthreads();
  if (s_last) {
    for (int i = READY_CTR_STRIDE + tid; i < a.n_counters; i += 256) a.counters[i] = 0u;
  }
}

hipError_t ready_launch_reader_f32(const F32Args& a, int grid, size_t lds, hipStream_t s, StageEvents ev) {
  if (a.R < 1 || a.R > 16 || a.B > 16 || (a.r != 8 && a.r != 16)) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), block(256);
  if (a.r == 8) {
    if (a.R <= 8) READY_LAUNCH((k_reader_f32<8, 8>), g, block, lds, s, ev, a);
    else READY_LAUNCH((k_reader_f32<8, 16>), g, block, lds, s, ev, a);
  } else {
    if (a.R <= 8) READY_LAUNCH((k_reader_f32<16, 8>), g, block, lds, s, ev, a);
    else READY_LAUNCH((k_reader_f32<16, 16>), g, block, lds, s, ev, a);
  }
  return hipGetLastError();
}
