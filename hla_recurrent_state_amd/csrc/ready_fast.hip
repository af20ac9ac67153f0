// Fast path of the ReaDy state reader for gfx950: bf16 states, activations
// and weights, rank r <= 32.  Two launches on the caller's stream:
//
//   k_zgemm   z = W_q (gamma h) as split-K partial sums, plus the partial
//             sums of squares of h for RMSNorm(h_j)            (step 4, query);
//             it also clears the counters of k_fused.
//   k_fused   one kernel for everything else.  Each workgroup takes a ticket
//             from an atomic counter and runs the work item with that number:
//     S items (sequence b, pair m): fused gather at the accept index into the
//             caller's buffer, mean square, log-RMS and
//             P = V^T S_bar U^T / sqrt(d_k), an r x r matrix  (steps 1-3)
//     A items (16 rows, 64 columns of a): f_j = [P z_j / rms(h_j), ell] per
//             pair (u_j = T q_j / sqrt(d_k) with T = V^T S_bar and
//             q_j = U^T z_j, reassociated through P), a = act(W1 f + b1)
//                                                    (step 4 readout, step 5)
//     O items (BM rows, 64 columns of out): out = h + W2 a + b2   (step 5)
//   Tickets are handed out in the order S, A, O and an item waits only for
//   items with smaller tickets (A for the S items of its sequences, O for the
//   A items of its rows), which were claimed by workgroups that are already
//   running; so every wait ends.  While the last state tiles stream in, the
//   workgroups that took early A and O tickets already run the MLP of the
//   sequences whose states are complete.
//
// Cross-workgroup data (P, ell, the invalid-sequence flags, a) is written
// with device-coherent stores (sc1), made complete with a wait on the memory
// counter, and announced by a relaxed device-scope atomic increment; readers
// poll the counter and load the data with device-coherent loads (sc1).  No
// release or acquire fence is used: on this GPU an agent-scope release writes
// back the whole L2 of the XCD and made the state stream five times slower.
// Every wait is bounded; when a bound is hit the kernel sets an abort flag,
// stores READY_ERR_SYNC_TIMEOUT in the caller's status word and finishes
// without waiting further.
//
// Formulas: ReaDy arXiv text, section 3.1 "Position-conditioned reading" and
// "Fusion and residual injection" (the Eq. (3) and Eq. (4) displays are lost
// in extraction; the rainbus summary, 方法步骤详情 steps (1)-(3), writes the
// reader out); section 3.2 "Avoiding redundant data movement" for the fused
// gather into a preallocated buffer and "State-access footprint" for the
// projected state shared by every position of the block.
//
// Matrix-core operand layout (v_mfma_f32_16x16x32_bf16): lane l holds
// A[l % 16][8 (l / 16) .. + 7], B[8 (l / 16) .. + 7][l % 16] and
// D[4 (l / 16) .. + 3][l % 16].  For Y = X W^T both operands are 16-byte
// chunks of rows (X rows for A, W rows for B), so they load straight from
// memory into registers.
#include "ready_common.h"

namespace {

__host__ __device__ __forceinline__ int cdiv_d(int a, int b) { return (a + b - 1) / b; }

// ---- device-coherent accesses (sc1) for data shared between workgroups of
// one launch, and the counters that announce it

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
constexpr int SC1 = 16;  // cache-policy operand of the buffer intrinsics: sc1

// `base` must be the same for every lane (a kernel argument): a per-lane base
// would make the compiler loop over the lanes to build the descriptor.
__device__ __forceinline__ u32x4 ld_coh16(const void* base, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), byte_off, 0, SC1);
}
__device__ __forceinline__ float ld_coh_f32(const float* p) {
  return __uint_as_float(__hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_coh_f32(float* p, float v) {
  __hip_atomic_store((uint32_t*)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh_u32(void* p, uint32_t v) {
  __hip_atomic_store((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coh_u32(const void* p) {
  return __hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// All memory operations of this thread issued so far are complete.
__device__ __forceinline__ void wait_mem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void count_up(uint32_t* c) {
  __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll *c until it reaches `want`, backing off from about 100 ns to about
// 1.7 us between polls so that waiting workgroups do not flood the memory
// channel that holds the counter while the state tiles stream.  Bounded:
// after about a second, or as soon as another workgroup has given up, it
// raises the abort flag, reports READY_ERR_SYNC_TIMEOUT and returns false.
constexpr int SPIN_LIMIT = 1 << 19;
__device__ bool wait_count(const uint32_t* c, uint32_t want, uint32_t* abort_flag, int32_t* dev_status) {
  int nap = 0;
  for (int it = 0;; ++it) {
    if (ld_coh_u32(c) >= want) return true;
    if ((it & 15) == 15 && ld_coh_u32(abort_flag) != 0) return false;
    if (it >= SPIN_LIMIT) {
      st_coh_u32(abort_flag, 1u);
      if (dev_status) st_coh_u32(dev_status, (uint32_t)READY_ERR_SYNC_TIMEOUT);
      return false;
    }
    switch (nap) {  // s_sleep takes an immediate operand
      case 0: __builtin_amdgcn_s_sleep(4); break;
      case 1: __builtin_amdgcn_s_sleep(8); break;
      case 2: __builtin_amdgcn_s_sleep(16); break;
      case 3: __builtin_amdgcn_s_sleep(32); break;
      default: __builtin_amdgcn_s_sleep(64); break;
    }
    if (nap < 4) ++nap;
  }
}

}  // namespace

// ---------------------------------------------------------------- k_zgemm

// Work item q = (ks * ncb + cb) * nrb + rb: a BM x 64 tile of z over K chunk
// ks; with 8 K chunks the items of one chunk (which share its h and W_q
// columns) all land on one XCD.  The four waves take consecutive quarters of
// the chunk and load their whole quarter (up to KS k-steps of 32) before the
// matrix instructions; the quarters are summed through LDS in a fixed order
// and the tile is written with 16-byte stores.  Column block 0 also sums the
// squares of the h values it loads (before the gain).  Block 0 clears the
// counters of k_fused.
template <int BM, int KS>
__global__ __launch_bounds__(256) void k_zgemm(FastArgs a) {
  constexpr int RB = BM / 16;
  constexpr int LD = 68;
  __shared__ __attribute__((aligned(16))) float red[3][BM * LD];
  __shared__ float hred[4][BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (blockIdx.x == 0) {
    for (int i = tid; i < a.n_counters; i += 256) a.counters[i] = 0u;
  }
  const int nrb = cdiv_d(a.R, BM), ncb = cdiv_d(a.Nz, 64);
  const int q = xcd_remap(blockIdx.x, gridDim.x, nrb * ncb * a.ksplit);
  if (q < 0) return;
  const int rb = q % nrb;
  const int cb = (q / nrb) % ncb;
  const int ks = q / (nrb * ncb);
  const int lr = lane & 15, lg = lane >> 4;
  const int kbeg = ks * a.kchunk;
  const int kend = min(a.d, kbeg + a.kchunk);
  const int kq = a.kchunk >> 2;  // multiple of 32, at most 32 KS
  const int wk0 = kbeg + wave * kq;
  const int wk1 = min(kend, wk0 + kq);
  const bool want_hss = (cb == 0);
  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};

  f32x4 acc[RB][4];
  float hsq[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    hsq[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  {
    u32x4 A[KS][RB], Bw[KS][4];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int kk = wk0 + 32 * s + 8 * lg;
      const bool kv = kk < wk1;
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int row = rb * BM + 16 * i + lr;
        A[s][i] = (kv && row < a.R) ? *(const u32x4*)(a.h + (int64_t)row * a.d + kk) : zero;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = cb * 64 + 16 * j + lr;
        Bw[s][j] = (kv && col < a.Nz) ? *(const u32x4*)(a.wq + (int64_t)col * a.d + kk) : zero;
      }
    }
    if (a.gamma != nullptr) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int kk = wk0 + 32 * s + 8 * lg;
        if (kk < wk1) {
          float g[8];
          Elem<uint16_t>::unpack(*(const u32x4*)(a.gamma + kk), g);
#pragma unroll
          for (int i = 0; i < RB; ++i) {
            float x[8];
            Elem<uint16_t>::unpack(A[s][i], x);
            if (want_hss) {
#pragma unroll
              for (int e = 0; e < 8; ++e) hsq[i] += x[e] * x[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= g[e];
            A[s][i] = pack_bf16x8(x);
          }
        }
      }
    } else if (want_hss) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int i = 0; i < RB; ++i) hsq[i] += sumsq_bf16x8(A[s][i]);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(A[s][i], Bw[s][j], acc[i][j]);
  }

  // the four K quarters: waves 1-3 park theirs in LDS, wave 0 adds them in
  // order and parks the sum, then all threads write the tile
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave - 1][(16 * i + 4 * lg + e) * LD + 16 * j + lr] = acc[i][j][e];
  }
  if (want_hss) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      float v = hsq[i];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (lg == 0) hred[wave][16 * i + lr] = v;
    }
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int o = (16 * i + 4 * lg + e) * LD + 16 * j + lr;
          red[0][o] = ((acc[i][j][e] + red[0][o]) + red[1][o]) + red[2][o];
        }
  }
  __syncthreads();
  for (int c = tid; c < BM * 16; c += 256) {
    const int rr = c >> 4, c4 = (c & 15) * 4;
    const int row = rb * BM + rr, col = cb * 64 + c4;
    if (row < a.R && col < a.Nz)
      *(float4*)(a.zpart + ((int64_t)ks * a.R + row) * a.Nz + col) = *(const float4*)&red[0][rr * LD + c4];
  }
  if (want_hss) {
    for (int rr = tid; rr < BM; rr += 256) {
      const int row = rb * BM + rr;
      if (row < a.R) a.hss[(int64_t)ks * a.R + row] = ((hred[0][rr] + hred[1][rr]) + hred[2][rr]) + hred[3][rr];
    }
  }
}

// ---------------------------------------------------------------- S items

// One workgroup per (sequence b, pair m) tile.  Wave w owns tile rows
// [32 w, 32 w + 32) as two 16-row blocks; lane l holds, for block mb and key
// step ks, the 16-byte chunk S[32 w + 16 mb + l % 16][32 ks + 8 (l / 16) .. + 7],
// which is exactly the A operand of S U^T (the contraction runs along the
// contiguous key axis).  The pair's U and V (2 r 256 bytes) are loaded first
// and parked in LDS while the tile is in flight, so the work after the tile
// arrives needs no further memory round trip and the registers hold little
// beyond the tile itself.
template <int RR>
__device__ __forceinline__ void state_item(const FastArgs& a, int tile, unsigned char* smem) {
  constexpr int NB = (RR + 15) / 16;  // 16-column blocks of U^T
  constexpr int VC = RR / 8;          // 16-byte chunks per V row
  constexpr int LU = READY_TILE + 8;  // padded U row in LDS (bf16)
  constexpr int WCH = RR * 16;        // 16-byte chunks of U, and of V
  constexpr int NW = 2 * WCH / 256;   // weight chunks per thread
  constexpr int WS = NB * RR * 16;    // per-wave partials of P
  uint16_t* sU = (uint16_t*)smem;                       // [RR][LU]
  uint16_t* sV = sU + RR * LU;                          // [128][RR]
  float* s_red = (float*)(sV + READY_TILE * RR);        // [4][WS]
  float* s_wsum = s_red + 4 * WS;                       // [4]

  const int b = tile / a.M;
  const int m = tile - b * a.M;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mz = a.shared ? 0 : m;
  float* P = a.pmat + (int64_t)tile * RR * RR;

  const int p_acc = a.accept_idx[b];
  if (p_acc < 0 || p_acc >= a.P) {
    // out-of-range accept index: flag it and leave this sequence's outputs
    for (int e = tid; e < RR * RR; e += 256) st_coh_f32(P + e, 0.0f);
    if (tid == 0) {
      if (a.dev_status) st_coh_u32(a.dev_status, (uint32_t)READY_ERR_ACCEPT_IDX);
      if (m == 0) st_coh_u32(a.seq_invalid + b, 1u);
      st_coh_f32(a.ell + tile, 0.0f);
    }
    wait_mem();
    __syncthreads();
    if (tid == 0) count_up(a.seqdone + READY_CTR_STRIDE * b);
    return;
  }

  // the pair's weights first: they return ahead of the tile
  const u32x4* Ug = (const u32x4*)(a.u + (int64_t)mz * RR * READY_TILE);
  const u32x4* Vg = (const u32x4*)(a.v + (int64_t)mz * READY_TILE * RR);
  u32x4 wtmp[NW];
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    const int c = tid + 256 * k;
    wtmp[k] = c < WCH ? Ug[c] : Vg[c - WCH];
  }

  // ---- step 1: the committed tile, 16-byte nontemporal loads ----
  const int l = m / a.H, hh = m - (m / a.H) * a.H;
  const uint16_t* src = a.states + (int64_t)b * a.sb + (int64_t)p_acc * a.sp + (int64_t)a.slot[l] * a.sl +
                        (int64_t)hh * a.sh;
  uint16_t* dst = a.gathered + (int64_t)tile * READY_TILE_ELEMS;
  const int lrow = lane & 15, lk = (lane >> 4) * 8;
  u32x4 data[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      data[mb][ks] = __builtin_nontemporal_load(
          (const u32x4*)(src + (32 * wave + 16 * mb + lrow) * READY_TILE + 32 * ks + lk));

#pragma unroll
  for (int k = 0; k < NW; ++k) {
    const int c = tid + 256 * k;
    if (c < WCH) *(u32x4*)&sU[(c >> 4) * LU + 8 * (c & 15)] = wtmp[k];
    else *(u32x4*)&sV[8 * (c - WCH)] = wtmp[k];
  }
  __syncthreads();

#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      __builtin_nontemporal_store(data[mb][ks],
                                  (u32x4*)(dst + (32 * wave + 16 * mb + lrow) * READY_TILE + 32 * ks + lk));

  // ---- step 2: mean square ----
  float ss = 0.0f;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ss += sumsq_bf16x8(data[mb][ks]);
  ss = wave_sum(ss);
  if (lane == 0) s_wsum[wave] = ss;

  // ---- S U^T on the matrix cores ----
  f32x4 acc[2][NB];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int i = 16 * nb + lrow;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 ub = (i < RR) ? *(const u32x4*)&sU[i * LU + 32 * ks + lk] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) acc[mb][nb] = mfma16x16x32(data[mb][ks], ub, acc[mb][nb]);
    }
  }

  // ---- P = V^T (S U^T): each lane sums over its eight rows ----
  // acc[mb][nb][e] = (S U^T)[v = 32 w + 16 mb + 4 (l / 16) + e][i' = 16 nb + l % 16]
  float part[NB][RR];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < RR; ++i) part[nb][i] = 0.0f;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = 32 * wave + 16 * mb + 4 * (lane >> 4) + e;
      float vrow[RR];
#pragma unroll
      for (int c = 0; c < VC; ++c) Elem<uint16_t>::unpack(*(const u32x4*)&sV[v * RR + 8 * c], vrow + 8 * c);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < RR; ++i) part[nb][i] += vrow[i] * acc[mb][nb][e];
    }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < RR; ++i) {
      part[nb][i] += __shfl_xor(part[nb][i], 16, 64);
      part[nb][i] += __shfl_xor(part[nb][i], 32, 64);
    }
  if (lane < 16) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < RR; ++i) s_red[wave * WS + (nb * RR + i) * 16 + lane] = part[nb][i];
  }
  __syncthreads();

  const float ms = ((s_wsum[0] + s_wsum[1]) + (s_wsum[2] + s_wsum[3])) * (1.0f / READY_TILE_ELEMS);
  const float rms = sqrtf(ms + a.state_eps);
  const float scale = 0.08838834764831845f / rms;  // 1 / (rms sqrt(d_k)), d_k = 128
  for (int e = tid; e < RR * RR; e += 256) {
    const int i = e / RR, ip = e - (e / RR) * RR;
    const int idx = ((ip >> 4) * RR + i) * 16 + (ip & 15);
    st_coh_f32(P + e, ((s_red[idx] + s_red[WS + idx]) + (s_red[2 * WS + idx] + s_red[3 * WS + idx])) * scale);
  }
  if (tid == 0) {
    const float ell = logf(rms);
    st_coh_f32(a.ell + tile, ell);
    if (m == 0) st_coh_u32(a.seq_invalid + b, 0u);
    if (a.logrms) a.logrms[tile] = ell;
  }
  wait_mem();
  __syncthreads();
  if (tid == 0) count_up(a.seqdone + READY_CTR_STRIDE * b);
}

// ---------------------------------------------------------------- A items

// Rows [16 rb, 16 rb + 16) of f and a, columns [64 cb, 64 cb + 64) of a.
// After the S items of the rows' sequences are counted, each thread builds f
// for one (row, pair) at a time: z from the K partial sums, times
// 1 / rms(h), u = P z, then [u, ell] goes to LDS in bf16 (and to `feat` in
// fp32).  Wave w computes a's columns 64 cb + 16 w .. + 15 on the matrix
// cores, W1 rows streaming straight from memory.
template <int RR>
__device__ __forceinline__ void mlp1_item(const FastArgs& a, int item, unsigned char* smem) {
  const int ncb = cdiv_d(a.Hm, 64);
  const int rb = item / ncb, cb = item - (item / ncb) * ncb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int row0 = rb * 16;
  const int F = a.F;
  const int Fp = (F + 31) & ~31;
  const int Fs = Fp + 8;
  uint16_t* fsh = (uint16_t*)smem;                 // [16][Fs]
  float* s_rs = (float*)(fsh + 16 * Fs);           // [16]
  int* s_ok = (int*)(s_rs + 16);

  // wait for the state tiles of the sequences these rows belong to
  const int b0 = row0 / a.n, b1 = (min(a.R, row0 + 16) - 1) / a.n;
  if (tid == 0) *s_ok = 1;
  __syncthreads();
  if (tid == 0) {
    for (int bb = b0; bb <= b1; ++bb)
      if (!wait_count(a.seqdone + READY_CTR_STRIDE * bb, (uint32_t)a.M, a.abort_flag, a.dev_status)) {
        *s_ok = 0;
        break;
      }
  }
  __syncthreads();
  const bool ok = *s_ok != 0;

  if (tid < 16) {
    const int rho = row0 + tid;
    float rs = 0.0f;
    if (rho < a.R) {
      float hs = 0.0f;
      for (int ks = 0; ks < a.ksplit; ++ks) hs += a.hss[(int64_t)ks * a.R + rho];
      rs = 1.0f / sqrtf(hs / (float)a.d + a.h_eps);
    }
    s_rs[tid] = rs;
  }
  const int padw = Fs - F;
  for (int e = tid; e < 16 * padw; e += 256) {
    const int rr = e / padw;
    fsh[rr * Fs + F + (e - rr * padw)] = 0;
  }
  __syncthreads();

  for (int e = tid; e < 16 * a.M; e += 256) {
    const int rr = e / a.M, m = e - (e / a.M) * a.M;
    const int rho = row0 + rr;
    float u[RR + 1];
#pragma unroll
    for (int i = 0; i <= RR; ++i) u[i] = 0.0f;
    if (rho < a.R && ok) {
      const int b = rho / a.n;
      const int mz = a.shared ? 0 : m;
      float z[RR];
#pragma unroll
      for (int i = 0; i < RR; ++i) z[i] = 0.0f;
      for (int ks = 0; ks < a.ksplit; ++ks) {
        const float4* zp = (const float4*)(a.zpart + ((int64_t)ks * a.R + rho) * a.Nz + mz * RR);
#pragma unroll
        for (int c = 0; c < RR / 4; ++c) {
          const float4 v = zp[c];
          z[4 * c] += v.x; z[4 * c + 1] += v.y; z[4 * c + 2] += v.z; z[4 * c + 3] += v.w;
        }
      }
      const float rs = s_rs[rr];
#pragma unroll
      for (int i = 0; i < RR; ++i) z[i] *= rs;
      const uint32_t pofs = (uint32_t)(((b * a.M + m) * RR * RR) * 4);
#pragma unroll
      for (int i = 0; i < RR; ++i) {
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < RR / 4; ++c) {
          const u32x4 p = ld_coh16(a.pmat, pofs + (uint32_t)(16 * (i * (RR / 4) + c)));
          s += __uint_as_float(p.x) * z[4 * c] + __uint_as_float(p.y) * z[4 * c + 1] +
               __uint_as_float(p.z) * z[4 * c + 2] + __uint_as_float(p.w) * z[4 * c + 3];
        }
        u[i] = s;
      }
      u[RR] = ld_coh_f32(a.ell + b * a.M + m);
      if (a.feat && cb == 0) {
        float* fr = a.feat + (int64_t)rho * F + m * (RR + 1);
#pragma unroll
        for (int i = 0; i <= RR; ++i) fr[i] = u[i];
      }
    }
    uint16_t* fr = fsh + rr * Fs + m * (RR + 1);
#pragma unroll
    for (int i = 0; i <= RR; ++i) fr[i] = f32_to_bf16_rne(u[i]);
  }
  __syncthreads();

  const int col = cb * 64 + 16 * wave + lr;
  const bool cv = col < a.Hm;
  const uint16_t* wrow = a.w1 + (int64_t)col * F;
  f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = 0; k0 < Fp; k0 += 256) {
    u32x4 bq[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int kk = k0 + 32 * s + 8 * lg;
      bq[s] = (cv && kk < F) ? *(const u32x4*)(wrow + kk) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int kb = k0 + 32 * s;
      if (kb < Fp) {
        const u32x4 aop = *(const u32x4*)&fsh[lr * Fs + kb + 8 * lg];
        acc = mfma16x16x32(aop, bq[s], acc);
      }
    }
  }
  // a in bf16: lanes l and l + 1 hold neighbouring columns; the even lane
  // stores the pair as one 32-bit word
  const float bias = (cv && a.b1) ? Elem<uint16_t>::ld(a.b1, col) : 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t mine = f32_to_bf16_rne(activation(acc[e] + bias, a.act));
    const uint32_t next = __shfl_down(mine, 1, 64);
    const int rho = row0 + 4 * lg + e;
    if ((lr & 1) == 0 && cv && rho < a.R) st_coh_u32(a.abuf + (int64_t)rho * a.Hm + col, mine | (next << 16));
  }
  wait_mem();
  __syncthreads();
  if (tid == 0) count_up(a.adone + READY_CTR_STRIDE * rb);
}

// ---------------------------------------------------------------- O items

// Item q = cb * nrb + rb: a BM x 64 tile of out.  After the A items of its
// rows are counted, the a rows of the tile are staged in LDS by passes of
// 128 values of K (device-coherent loads); wave w streams the W2 rows of its
// 16 columns straight into registers.  The epilogue goes through LDS so that
// h, out and delta move in 16-byte row chunks.
template <int BM>
__device__ __forceinline__ void mlp2_item(const FastArgs& a, int item, unsigned char* smem) {
  constexpr int KT = 128, LA = KT + 8, LO = 68;
  constexpr int SA = BM * LA * 2, SO = BM * LO * 4;
  uint16_t* sA = (uint16_t*)smem;   // [BM][LA]
  float* sO = (float*)smem;         // [BM][LO], after the K passes
  int* s_ok = (int*)(smem + (SA > SO ? SA : SO));

  const int nrb = cdiv_d(a.R, BM);
  const int rb = item % nrb, cb = item / nrb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int row0 = rb * BM, col0 = cb * 64;
  const int col = col0 + 16 * wave + lr;
  const bool cv = col < a.d;
  const uint16_t* wrow = a.w2 + (int64_t)col * a.Hm;

  // wait for the A items of these rows
  const int a0 = row0 / 16, a1 = (min(a.R, row0 + BM) - 1) / 16;
  const uint32_t want = (uint32_t)cdiv_d(a.Hm, 64);
  if (tid == 0) *s_ok = 1;
  __syncthreads();
  if (tid == 0) {
    for (int aa = a0; aa <= a1; ++aa)
      if (!wait_count(a.adone + READY_CTR_STRIDE * aa, want, a.abort_flag, a.dev_status)) {
        *s_ok = 0;
        break;
      }
  }
  __syncthreads();
  if (*s_ok == 0) return;

  f32x4 acc[BM / 16];
#pragma unroll
  for (int i = 0; i < BM / 16; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int kb = 0; kb < a.Hm; kb += KT) {
    const int klen = min(KT, a.Hm - kb);
    u32x4 bq[KT / 32];
#pragma unroll
    for (int s = 0; s < KT / 32; ++s) {
      const int kk = 32 * s + 8 * lg;
      bq[s] = (cv && kk < klen) ? *(const u32x4*)(wrow + kb + kk) : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    for (int c = tid; c < BM * (KT / 8); c += 256) {
      const int rr = c / (KT / 8), kc = (c - rr * (KT / 8)) * 8;
      const int row = row0 + rr;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (row < a.R && kc < klen) v = ld_coh16(a.abuf, (uint32_t)(2 * (row * a.Hm + kb + kc)));
      *(u32x4*)&sA[rr * LA + kc] = v;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < KT / 32; ++s) {
      if (32 * s < klen) {
#pragma unroll
        for (int i = 0; i < BM / 16; ++i) {
          const u32x4 aop = *(const u32x4*)&sA[(16 * i + lr) * LA + 32 * s + 8 * lg];
          acc[i] = mfma16x16x32(aop, bq[s], acc[i]);
        }
      }
    }
  }

  __syncthreads();
#pragma unroll
  for (int i = 0; i < BM / 16; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) sO[(16 * i + 4 * lg + e) * LO + 16 * wave + lr] = acc[i][e];
  __syncthreads();
  for (int c = tid; c < BM * 8; c += 256) {
    const int rr = c >> 3, c8 = (c & 7) * 8;
    const int row = row0 + rr, gc = col0 + c8;
    if (row >= a.R || gc >= a.d) continue;
    if (ld_coh_u32(a.seq_invalid + row / a.n)) continue;
    float dv[8];
    const float4 d0 = *(const float4*)&sO[rr * LO + c8];
    const float4 d1 = *(const float4*)&sO[rr * LO + c8 + 4];
    dv[0] = d0.x; dv[1] = d0.y; dv[2] = d0.z; dv[3] = d0.w;
    dv[4] = d1.x; dv[5] = d1.y; dv[6] = d1.z; dv[7] = d1.w;
    if (a.b2) {
      float bb[8];
      Elem<uint16_t>::unpack(*(const u32x4*)(a.b2 + gc), bb);
#pragma unroll
      for (int e = 0; e < 8; ++e) dv[e] += bb[e];
    }
    const int64_t off = (int64_t)row * a.d + gc;
    float hv[8];
    Elem<uint16_t>::unpack(*(const u32x4*)(a.h + off), hv);
#pragma unroll
    for (int e = 0; e < 8; ++e) hv[e] += dv[e];
    *(u32x4*)(a.out + off) = pack_bf16x8(hv);
    if (a.delta) {
      *(float4*)(a.delta + off) = make_float4(dv[0], dv[1], dv[2], dv[3]);
      *(float4*)(a.delta + off + 4) = make_float4(dv[4], dv[5], dv[6], dv[7]);
    }
  }
}

// ---------------------------------------------------------------- k_fused

template <int RR, int OBM>
__global__ __launch_bounds__(256) void k_fused(FastArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_ticket;
  if (threadIdx.x == 0)
    s_ticket = (int)__hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int t = s_ticket;
  if (t < a.n_s) state_item<RR>(a, t, smem);
  else if (t < a.n_s + a.n_a) mlp1_item<RR>(a, t - a.n_s, smem);
  else if (t < a.n_s + a.n_a + a.n_o) mlp2_item<OBM>(a, t - a.n_s - a.n_a, smem);
}

// ---------------------------------------------------------------- launchers

size_t ready_fused_lds(int r, int F, int obm) {
  const int NB = (r + 15) / 16;
  const size_t s_bytes = (size_t)r * (READY_TILE + 8) * 2 + (size_t)READY_TILE * r * 2 + 4 * (4 * NB * r * 16 + 4);
  const int Fs = ((F + 31) & ~31) + 8;
  const size_t a_bytes = (size_t)16 * Fs * 2 + 4 * 16 + 16;
  const size_t sa = (size_t)obm * (128 + 8) * 2, so = (size_t)obm * 68 * 4;
  const size_t o_bytes = (sa > so ? sa : so) + 16;
  size_t m = s_bytes > a_bytes ? s_bytes : a_bytes;
  return m > o_bytes ? m : o_bytes;
}

hipError_t ready_launch_zgemm(const FastArgs& a, int bm, hipStream_t s, StageEvents ev) {
  const int ncb = cdiv_d(a.Nz, 64);
  const int nrb = cdiv_d(a.R, bm);
  const int total = nrb * ncb * a.ksplit;
  const dim3 grid((unsigned)(8 * cdiv_d(total, 8))), block(256);
  const int ks = (a.kchunk / 4) / 32;  // k-steps per wave
  if (bm == 16) {
    if (ks <= 1) READY_LAUNCH((k_zgemm<16, 1>), grid, block, 0, s, ev, a);
    else if (ks <= 2) READY_LAUNCH((k_zgemm<16, 2>), grid, block, 0, s, ev, a);
    else if (ks <= 3) READY_LAUNCH((k_zgemm<16, 3>), grid, block, 0, s, ev, a);
    else if (ks <= 4) READY_LAUNCH((k_zgemm<16, 4>), grid, block, 0, s, ev, a);
    else READY_LAUNCH((k_zgemm<16, 5>), grid, block, 0, s, ev, a);
  } else {
    if (ks <= 1) READY_LAUNCH((k_zgemm<64, 1>), grid, block, 0, s, ev, a);
    else if (ks <= 2) READY_LAUNCH((k_zgemm<64, 2>), grid, block, 0, s, ev, a);
    else if (ks <= 3) READY_LAUNCH((k_zgemm<64, 3>), grid, block, 0, s, ev, a);
    else if (ks <= 4) READY_LAUNCH((k_zgemm<64, 4>), grid, block, 0, s, ev, a);
    else READY_LAUNCH((k_zgemm<64, 5>), grid, block, 0, s, ev, a);
  }
  return hipGetLastError();
}

hipError_t ready_launch_fused(const FastArgs& a, int obm, hipStream_t s, StageEvents ev) {
  const dim3 grid((unsigned)(a.n_s + a.n_a + a.n_o)), block(256);
  const size_t lds = ready_fused_lds(a.r, a.F, obm);
#define READY_FUSED_CASE(RRV)                                                       \
  do {                                                                              \
    if (obm == 16) READY_LAUNCH((k_fused<RRV, 16>), grid, block, lds, s, ev, a);    \
    else READY_LAUNCH((k_fused<RRV, 64>), grid, block, lds, s, ev, a);              \
  } while (0)
  switch (a.r) {
    case 8: READY_FUSED_CASE(8); break;
    case 16: READY_FUSED_CASE(16); break;
    case 24: READY_FUSED_CASE(24); break;
    default: READY_FUSED_CASE(32); break;
  }
#undef READY_FUSED_CASE
  return hipGetLastError();
}
