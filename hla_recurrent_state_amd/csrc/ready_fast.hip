// Fast path of the ReaDy state reader for gfx950: bf16 states, activations
// and weights, rank r <= 32.  One persistent launch, k_reader.
//
// Its grid is two workgroups per CU, which the register and LDS budget of
// the kernel lets the GPU hold at the same time.  Work is assigned
// statically; each workgroup runs, in this order:
//   Z  at most one (or a few) query item: a BM x 64 tile of the partial sums
//      z = W_q (gamma h) over one K chunk, plus the sums of squares of h for
//      RMSNorm(h_j)                                        (step 4, query)
//   S  (workgroups [0, g_s)) the state tiles t = rank, rank + g_s, ...: fused
//      gather at the accept index into the caller's buffer, mean square,
//      log-RMS and P = V^T S_bar U^T / sqrt(d_k), an r x r matrix; the next
//      tile's loads are issued before the current tile is processed
//                                                          (steps 1-3)
//   A  (workgroups [g_s, G)) items of 16 rows and 64 columns of a, in row
//      order: f_j = [P z_j / rms(h_j), ell] per pair (u_j = T q_j / sqrt(d_k)
//      with T = V^T S_bar and q_j = U^T z_j, reassociated through P), then
//      a = act(W1 f + b1)                        (step 4 readout, step 5)
//   O  items o = g, g + G, ...: a BM x 64 tile of out = h + W2 a + b2 (step 5)
// An A item waits for the Z items of its rows and the S items of its
// sequences; an O item waits for the A items of its rows.  Z and S items
// never wait and A items wait only for Z and S items, so with every
// workgroup resident at once each wait ends; while the state tiles stream,
// the A workgroups already run the MLP of the sequences whose states are
// complete.
//
// Cross-workgroup data (z partial sums, P, ell, the invalid-sequence flags,
// a) is written with device-coherent stores (sc1), made complete with a wait
// on the memory counter, and announced by a relaxed device-scope atomic
// increment; readers poll the counter and load the data with device-coherent
// loads (sc1).  No release or acquire fence is used: on this GPU an
// agent-scope release writes back the whole L2 of the XCD and made the state
// stream five times slower.  Every wait is bounded; when a bound is hit the
// kernel sets an abort flag, stores READY_ERR_SYNC_TIMEOUT in the caller's
// status word and finishes without waiting further.  The last workgroup to
// finish clears the counters, so the next call starts from zero; the first
// call needs a workspace prepared by readyWorkspaceInit (checked through a
// magic word).
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
__device__ __forceinline__ void st_coh16(void* base, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(base), byte_off, 0, SC1);
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
__device__ __forceinline__ uint32_t count_up(uint32_t* c) {
  return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t* ctr(uint32_t* base, int i) { return base + READY_CTR_STRIDE * i; }

// Poll *c until it reaches `want`, backing off from about 100 ns to about
// 0.9 us between polls so that waiting workgroups do not flood the memory
// channel that holds the counter while the state tiles stream.  Bounded:
// after about a second, or as soon as another workgroup has given up, it
// raises the abort flag, reports READY_ERR_SYNC_TIMEOUT and returns false.
constexpr int SPIN_LIMIT = 1 << 20;
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
      case 3: __builtin_amdgcn_s_sleep(24); break;
      default: __builtin_amdgcn_s_sleep(32); break;
    }
    if (nap < 4) ++nap;
  }
}

// Thread 0 waits for *c >= want; the whole workgroup learns the outcome.
__device__ bool wg_wait(const uint32_t* c, uint32_t want, const FastArgs& a, int* s_flag) {
  if (threadIdx.x == 0) *s_flag = wait_count(c, want, a.abort_flag, a.dev_status) ? 1 : 0;
  __syncthreads();
  const bool ok = *s_flag != 0;
  __syncthreads();
  return ok;
}

}  // namespace

// ---------------------------------------------------------------- Z items

// Item q = (ks * ncb + cb) * nrb + rb: a BM x 64 tile of z over K chunk ks
// of 128 KS values.  The four waves take consecutive quarters of the chunk
// (KS k-steps of 32 each) and load them straight into registers before the
// matrix instructions; the quarters are summed through LDS in a fixed order
// and the tile is stored with 16-byte device-coherent stores.  Column block
// 0 also sums the squares of the h values it loads (before the gain).
template <int BM, int KS>
__device__ void z_item(const FastArgs& a, int q, unsigned char* smem) {
  constexpr int RB = BM / 16;
  constexpr int ZCH = 128 * KS;  // K chunk
  constexpr int LD = 68;
  float* red = (float*)smem;              // [3][BM][LD]
  float* hred = red + 3 * BM * LD;        // [4][BM]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nrb = cdiv_d(a.R, BM), ncb = cdiv_d(a.Nz, 64);
  const int rb = q % nrb;
  const int cb = (q / nrb) % ncb;
  const int ks = q / (nrb * ncb);
  const int lr = lane & 15, lg = lane >> 4;
  const int kbeg = ks * ZCH;
  const int kend = min(a.d, kbeg + ZCH);
  const int wk0 = kbeg + wave * (ZCH / 4);
  const int wk1 = min(kend, wk0 + ZCH / 4);
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

  __syncthreads();  // the LDS area may still be in use by the previous item
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(wave - 1) * BM * LD + (16 * i + 4 * lg + e) * LD + 16 * j + lr] = acc[i][j][e];
  }
  if (want_hss) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      float v = hsq[i];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (lg == 0) hred[wave * BM + 16 * i + lr] = v;
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
          red[o] = ((acc[i][j][e] + red[o]) + red[BM * LD + o]) + red[2 * BM * LD + o];
        }
  }
  __syncthreads();
  for (int c = tid; c < BM * 16; c += 256) {
    const int rr = c >> 4, c4 = (c & 15) * 4;
    const int row = rb * BM + rr, col = cb * 64 + c4;
    if (row < a.R && col < a.Nz)
      st_coh16(a.zpart, (uint32_t)(4 * ((ks * a.R + row) * a.Nz + col)), *(const u32x4*)&red[rr * LD + c4]);
  }
  if (want_hss) {
    for (int rr = tid; rr < BM; rr += 256) {
      const int row = rb * BM + rr;
      if (row < a.R)
        st_coh_f32(a.hss + ks * a.R + row,
                   ((hred[rr] + hred[BM + rr]) + hred[2 * BM + rr]) + hred[3 * BM + rr]);
    }
  }
  wait_mem();
  __syncthreads();
  if (tid == 0) count_up(ctr(a.zdone, rb));
}

// ---------------------------------------------------------------- S items

// Tile t = (sequence b, pair m).  Wave w owns tile rows [32 w, 32 w + 32) as
// two 16-row blocks; lane l holds, for block mb and key step ks, the 16-byte
// chunk S[32 w + 16 mb + l % 16][32 ks + 8 (l / 16) .. + 7], which is exactly
// the A operand of S U^T (the contraction runs along the contiguous key
// axis).  Each thread also carries NW 16-byte chunks of the pair's U and V,
// parked in LDS when the tile is processed.
template <int RR>
struct TileRegs {
  static constexpr int NW = 2 * RR * 16 / 256;  // weight chunks per thread
  u32x4 data[2][4];
  u32x4 w[NW];
  int p;  // accept index of the tile's sequence
};

template <int RR>
__device__ __forceinline__ void tile_issue(const FastArgs& a, int t, TileRegs<RR>& R) {
  constexpr int WCH = RR * 16;
  const int b = t / a.M, m = t - (t / a.M) * a.M;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mz = a.shared ? 0 : m;
  R.p = a.accept_idx[b];
  const u32x4* Ug = (const u32x4*)(a.u + (int64_t)mz * RR * READY_TILE);
  const u32x4* Vg = (const u32x4*)(a.v + (int64_t)mz * READY_TILE * RR);
#pragma unroll
  for (int k = 0; k < TileRegs<RR>::NW; ++k) {
    const int c = tid + 256 * k;
    R.w[k] = c < WCH ? Ug[c] : Vg[c - WCH];
  }
  if (R.p < 0 || R.p >= a.P) return;
  const int l = m / a.H, hh = m - (m / a.H) * a.H;
  const uint16_t* src = a.states + (int64_t)b * a.sb + (int64_t)R.p * a.sp + (int64_t)a.slot[l] * a.sl +
                        (int64_t)hh * a.sh;
  const int lrow = lane & 15, lk = (lane >> 4) * 8;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      R.data[mb][ks] = __builtin_nontemporal_load(
          (const u32x4*)(src + (32 * wave + 16 * mb + lrow) * READY_TILE + 32 * ks + lk));
}

// Process tile t whose loads have arrived: copy to `gathered`, sum of
// squares, S U^T, P, ell.  Its stores are complete (and the tile can be
// announced) after the caller's next wait_mem().
template <int RR>
__device__ __forceinline__ void tile_process(const FastArgs& a, int t, const TileRegs<RR>& R, unsigned char* smem,
                                             int announce);
__device__ __forceinline__ void tile_count(const FastArgs& a, int t) {
  const int b = t / a.M;
  const int r0 = b * a.n, r1 = b * a.n + a.n - 1;
  for (int q = r0 / 16; q <= r1 / 16; ++q) count_up(ctr(a.sdone, q));
}

template <int RR>
__device__ __forceinline__ void tile_process(const FastArgs& a, int t, const TileRegs<RR>& R, unsigned char* smem,
                                             int announce) {
  constexpr int NB = (RR + 15) / 16;  // 16-column blocks of U^T
  constexpr int VC = RR / 8;          // 16-byte chunks per V row
  constexpr int LU = READY_TILE + 8;  // padded U row in LDS (bf16)
  constexpr int WCH = RR * 16;
  constexpr int WS = NB * RR * 16;    // per-wave partials of P
  uint16_t* sU = (uint16_t*)smem;                       // [RR][LU]
  uint16_t* sV = sU + RR * LU;                          // [128][RR]
  float* s_red = (float*)(sV + READY_TILE * RR);        // [4][WS]
  float* s_wsum = s_red + 4 * WS;                       // [4]

  const int b = t / a.M, m = t - (t / a.M) * a.M;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* P = a.pmat + (int64_t)t * RR * RR;

  if (R.p < 0 || R.p >= a.P) {
    // out-of-range accept index: flag it and leave this sequence's outputs.
    // No tile loads were issued, so wait explicitly before announcing.
    for (int e = tid; e < RR * RR; e += 256) st_coh_f32(P + e, 0.0f);
    if (tid == 0) {
      if (a.dev_status) st_coh_u32(a.dev_status, (uint32_t)READY_ERR_ACCEPT_IDX);
      if (m == 0) st_coh_u32(a.seq_invalid + b, 1u);
      st_coh_f32(a.ell + t, 0.0f);
    }
    wait_mem();
    __syncthreads();
    if (tid == 0 && announce >= 0) tile_count(a, announce);
    return;
  }

  const int lrow = lane & 15, lk = (lane >> 4) * 8;
  uint16_t* dst = a.gathered + (int64_t)t * READY_TILE_ELEMS;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      __builtin_nontemporal_store(R.data[mb][ks],
                                  (u32x4*)(dst + (32 * wave + 16 * mb + lrow) * READY_TILE + 32 * ks + lk));

  // The stores above waited for this tile's loads, issued after the stores
  // of tile `announce` (two turns back): with in-order completion of the
  // memory counter those are complete on every thread after this barrier.
  __syncthreads();  // (also: the previous tile is done with the LDS area)
  if (tid == 0 && announce >= 0) tile_count(a, announce);
#pragma unroll
  for (int k = 0; k < TileRegs<RR>::NW; ++k) {
    const int c = tid + 256 * k;
    if (c < WCH) *(u32x4*)&sU[(c >> 4) * LU + 8 * (c & 15)] = R.w[k];
    else *(u32x4*)&sV[8 * (c - WCH)] = R.w[k];
  }

  // ---- step 2: mean square ----
  float ss = 0.0f;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ss += sumsq_bf16x8(R.data[mb][ks]);
  ss = wave_sum(ss);
  if (lane == 0) s_wsum[wave] = ss;
  __syncthreads();

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
      for (int mb = 0; mb < 2; ++mb) acc[mb][nb] = mfma16x16x32(R.data[mb][ks], ub, acc[mb][nb]);
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
    st_coh_f32(a.ell + t, ell);
    if (m == 0) st_coh_u32(a.seq_invalid + b, 0u);
    if (a.logrms) a.logrms[t] = ell;
  }
}

// The S items of one workgroup: tiles t = rank, rank + g_s, ...  Two tiles
// are in flight while one is processed: the loads of tile t + 2 g_s are
// issued right after tile t's P is stored.  Tile t is announced while tile
// t + 2 g_s is processed (see tile_process); the last two at the end.
template <int RR>
__device__ void s_phase(const FastArgs& a, int rank, TileRegs<RR>& r0, TileRegs<RR>& r1, unsigned char* smem) {
  const int gs = a.g_s;
  int t = rank;
  for (; t < a.n_s; t += gs) {
    const int tb = t - 2 * gs;
    tile_process<RR>(a, t, r0, smem, tb >= rank ? tb : -1);
    r0 = r1;
    if (t + 2 * gs < a.n_s) tile_issue<RR>(a, t + 2 * gs, r1);
  }
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k <= 2; ++k) {
      const int tb = t - k * gs;
      if (tb >= rank) tile_count(a, tb);
    }
  }
}

// ---------------------------------------------------------------- A items

// Rows [16 rb, 16 rb + 16) of f and a, columns [64 cb, 64 cb + 64) of a.
// After the Z items of the rows' tile are counted, the z partial sums are
// reduced into LDS; after the S items of the rows' sequences are counted,
// each thread builds f for one (row, pair) at a time (u = P z / rms(h), then
// ell) into LDS in bf16 (and into `feat` in fp32).  Wave w computes a's
// columns 64 cb + 16 w .. + 15 on the matrix cores, W1 rows streaming
// straight from memory.
template <int RR, int BMZ, int OBM>
__device__ void mlp1_item(const FastArgs& a, int item, unsigned char* smem) {
  const int ncb = cdiv_d(a.Hm, 64);
  const int rb = item / ncb, cb = item - (item / ncb) * ncb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int row0 = rb * 16;
  const int rows = min(16, a.R - row0);
  const int F = a.F, Nz = a.Nz;
  const int Fp = (F + 31) & ~31;
  const int Fs = Fp + 8;
  float* z_s = (float*)smem;                       // [16][Nz]
  uint16_t* fsh = (uint16_t*)(z_s + 16 * Nz);      // [16][Fs]
  float* s_rs = (float*)(fsh + 16 * Fs);           // [16]
  int* s_flag = (int*)(s_rs + 16);

  // W1 rows of this lane's column: independent of every other item
  const int col = cb * 64 + 16 * wave + lr;
  const bool cv = col < a.Hm;
  const uint16_t* wrow = a.w1 + (int64_t)col * F;
  u32x4 bq[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int kk = 32 * s + 8 * lg;
    bq[s] = (cv && kk < F) ? *(const u32x4*)(wrow + kk) : u32x4{0u, 0u, 0u, 0u};
  }

  bool ok = wg_wait(ctr(a.zdone, row0 / BMZ), (uint32_t)(cdiv_d(Nz, 64) * a.ksplit), a, s_flag);

  // z of the 16 rows from the K partial sums (up to 16 loads in flight per
  // thread), and 1 / rms(h)
  const int nc4 = Nz / 4;
  for (int c0 = tid; c0 < 16 * nc4; c0 += 256 * 4) {
    float4 s4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) s4[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = 0; k0 < a.ksplit; k0 += 4) {
      u32x4 v[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = c0 + 256 * j;
        const int rr = c / nc4, c4 = c - (c / nc4) * nc4;
        const bool live = c < 16 * nc4 && rr < rows && ok;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          v[j][k] = (live && k0 + k < a.ksplit)
                        ? ld_coh16(a.zpart, (uint32_t)(4 * (((k0 + k) * a.R + row0 + rr) * Nz + 4 * c4)))
                        : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          s4[j].x += __uint_as_float(v[j][k].x); s4[j].y += __uint_as_float(v[j][k].y);
          s4[j].z += __uint_as_float(v[j][k].z); s4[j].w += __uint_as_float(v[j][k].w);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + 256 * j;
      if (c < 16 * nc4) {
        const int rr = c / nc4, c4 = c - (c / nc4) * nc4;
        *(float4*)&z_s[rr * Nz + 4 * c4] = s4[j];
      }
    }
  }
  if (tid < 16) {
    float rs = 0.0f;
    if (tid < rows && ok) {
      float hv[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) hv[k] = k < a.ksplit ? ld_coh_f32(a.hss + k * a.R + row0 + tid) : 0.0f;
      float hs = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) hs += hv[k];
      for (int k = 16; k < a.ksplit; ++k) hs += ld_coh_f32(a.hss + k * a.R + row0 + tid);
      rs = 1.0f / sqrtf(hs / (float)a.d + a.h_eps);
    }
    s_rs[tid] = rs;
  }
  const int padw = Fs - F;
  for (int e = tid; e < 16 * padw; e += 256) {
    const int rr = e / padw;
    fsh[rr * Fs + F + (e - rr * padw)] = 0;
  }

  // the state tiles of the sequences these rows belong to
  const int b0 = row0 / a.n, b1 = (row0 + rows - 1) / a.n;
  if (!wg_wait(ctr(a.sdone, rb), (uint32_t)(a.M * (b1 - b0 + 1)), a, s_flag)) ok = false;

  // f for one (row, pair) at a time; at r = 8 a thread's two items load
  // their P matrices in one round
  constexpr int PCH = RR * RR / 4;             // 16-byte chunks of P
  constexpr int IPR = PCH <= 16 ? 2 : 1;       // items per round
  constexpr int PG = PCH < 32 ? PCH : 32;      // chunks per load group
  for (int e0 = tid; e0 < 16 * a.M; e0 += 256 * IPR) {
    u32x4 pv[IPR][PG];
    float ellv[IPR];
    int rrv[IPR], mv[IPR];
    bool live[IPR];
#pragma unroll
    for (int it = 0; it < IPR; ++it) {
      const int e = e0 + 256 * it;
      rrv[it] = e / a.M;
      mv[it] = e - (e / a.M) * a.M;
      live[it] = e < 16 * a.M && rrv[it] < rows && ok;
      const int b = (row0 + rrv[it]) / a.n;
      const uint32_t pofs = (uint32_t)(((b * a.M + mv[it]) * RR * RR) * 4);
#pragma unroll
      for (int c = 0; c < PG; ++c) pv[it][c] = live[it] ? ld_coh16(a.pmat, pofs + 16 * c) : u32x4{0u, 0u, 0u, 0u};
      ellv[it] = live[it] ? ld_coh_f32(a.ell + b * a.M + mv[it]) : 0.0f;
    }
#pragma unroll
    for (int it = 0; it < IPR; ++it) {
      const int e = e0 + 256 * it;
      if (e >= 16 * a.M) break;
      const int rr = rrv[it], m = mv[it];
      float u[RR + 1];
#pragma unroll
      for (int i = 0; i <= RR; ++i) u[i] = 0.0f;
      if (live[it]) {
        const int b = (row0 + rr) / a.n;
        const int mz = a.shared ? 0 : m;
        const float rs = s_rs[rr];
        float z[RR];
#pragma unroll
        for (int c = 0; c < RR / 4; ++c) {
          const float4 v = *(const float4*)&z_s[rr * Nz + mz * RR + 4 * c];
          z[4 * c] = v.x * rs; z[4 * c + 1] = v.y * rs; z[4 * c + 2] = v.z * rs; z[4 * c + 3] = v.w * rs;
        }
        const uint32_t pofs = (uint32_t)(((b * a.M + m) * RR * RR) * 4);
#pragma unroll
        for (int g0 = 0; g0 < PCH; g0 += PG) {
          u32x4 pq[PG];
#pragma unroll
          for (int c = 0; c < PG; ++c) pq[c] = g0 == 0 ? pv[it][c] : ld_coh16(a.pmat, pofs + 16 * (g0 + c));
#pragma unroll
          for (int c = 0; c < PG; ++c) {
            const int i = (g0 + c) / (RR / 4), c4 = (g0 + c) % (RR / 4);
            u[i] += __uint_as_float(pq[c].x) * z[4 * c4] + __uint_as_float(pq[c].y) * z[4 * c4 + 1] +
                    __uint_as_float(pq[c].z) * z[4 * c4 + 2] + __uint_as_float(pq[c].w) * z[4 * c4 + 3];
          }
        }
        u[RR] = ellv[it];
        if (a.feat && cb == 0) {
          float* fr = a.feat + (int64_t)(row0 + rr) * F + m * (RR + 1);
#pragma unroll
          for (int i = 0; i <= RR; ++i) fr[i] = u[i];
        }
      }
      uint16_t* fr = fsh + rr * Fs + m * (RR + 1);
#pragma unroll
      for (int i = 0; i <= RR; ++i) fr[i] = f32_to_bf16_rne(u[i]);
    }
  }
  __syncthreads();

  f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = 0; k0 < Fp; k0 += 256) {
    if (k0 > 0) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int kk = k0 + 32 * s + 8 * lg;
        bq[s] = (cv && kk < F) ? *(const u32x4*)(wrow + kk) : u32x4{0u, 0u, 0u, 0u};
      }
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
    const int rr = 4 * lg + e;
    if ((lr & 1) == 0 && cv && rr < rows) st_coh_u32(a.abuf + (int64_t)(row0 + rr) * a.Hm + col, mine | (next << 16));
  }
  wait_mem();
  __syncthreads();
  if (tid == 0) count_up(ctr(a.adone, row0 / OBM));
  __syncthreads();  // the LDS area is reused by the next item
}

// ---------------------------------------------------------------- O items

// Item q = cb * nrb + rb: a BM x 64 tile of out.  The W2 rows of the lane's
// column are loaded before waiting; after the A items of the tile's rows are
// counted, the a rows are staged in LDS by passes of 256 values of K
// (device-coherent loads) for the matrix instructions.  The epilogue goes
// through LDS so that h, out and delta move in 16-byte row chunks.
template <int BM>
__device__ void mlp2_item(const FastArgs& a, int item, unsigned char* smem) {
  constexpr int KT = 256, LA = KT + 8, LO = 68;
  constexpr int SA = BM * LA * 2, SO = BM * LO * 4;
  uint16_t* sA = (uint16_t*)smem;   // [BM][LA]
  float* sO = (float*)smem;         // [BM][LO], after the K passes
  int* s_flag = (int*)(smem + (SA > SO ? SA : SO));

  const int nrb = cdiv_d(a.R, BM);
  const int rb = item % nrb, cb = item / nrb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int row0 = rb * BM, col0 = cb * 64;
  const int rows = min(BM, a.R - row0);
  const int col = col0 + 16 * wave + lr;
  const bool cv = col < a.d;
  const uint16_t* wrow = a.w2 + (int64_t)col * a.Hm;

  u32x4 bq[KT / 32];
#pragma unroll
  for (int s = 0; s < KT / 32; ++s) {
    const int kk = 32 * s + 8 * lg;
    bq[s] = (cv && kk < a.Hm) ? *(const u32x4*)(wrow + kk) : u32x4{0u, 0u, 0u, 0u};
  }

  // the epilogue's h chunks (BM rows x 8 chunks of 8 values: up to 2 per thread)
  constexpr int EPT = (BM * 8 + 255) / 256;
  u32x4 hq[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int c = tid + 256 * k;
    const int rr = c >> 3, gc = col0 + (c & 7) * 8;
    hq[k] = (c < BM * 8 && rr < rows && gc < a.d) ? *(const u32x4*)(a.h + (int64_t)(row0 + rr) * a.d + gc)
                                                 : u32x4{0u, 0u, 0u, 0u};
  }

  const uint32_t want = (uint32_t)(cdiv_d(rows, 16) * cdiv_d(a.Hm, 64));
  if (!wg_wait(ctr(a.adone, rb), want, a, s_flag)) return;

  f32x4 acc[BM / 16];
#pragma unroll
  for (int i = 0; i < BM / 16; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int kb = 0; kb < a.Hm; kb += KT) {
    const int klen = min(KT, a.Hm - kb);
    if (kb > 0) {
#pragma unroll
      for (int s = 0; s < KT / 32; ++s) {
        const int kk = 32 * s + 8 * lg;
        bq[s] = (cv && kk < klen) ? *(const u32x4*)(wrow + kb + kk) : u32x4{0u, 0u, 0u, 0u};
      }
    }
    __syncthreads();
    for (int c = tid; c < BM * (KT / 8); c += 256) {
      const int rr = c / (KT / 8), kc = (c - rr * (KT / 8)) * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (rr < rows && kc < klen) v = ld_coh16(a.abuf, (uint32_t)(2 * ((row0 + rr) * a.Hm + kb + kc)));
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
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int c = tid + 256 * k;
    const int rr = c >> 3, c8 = (c & 7) * 8;
    const int row = row0 + rr, gc = col0 + c8;
    if (c >= BM * 8 || rr >= rows || gc >= a.d) continue;
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
    Elem<uint16_t>::unpack(hq[k], hv);
#pragma unroll
    for (int e = 0; e < 8; ++e) hv[e] += dv[e];
    *(u32x4*)(a.out + off) = pack_bf16x8(hv);
    if (a.delta) {
      *(float4*)(a.delta + off) = make_float4(dv[0], dv[1], dv[2], dv[3]);
      *(float4*)(a.delta + off + 4) = make_float4(dv[4], dv[5], dv[6], dv[7]);
    }
  }
  __syncthreads();  // the LDS area is reused by the next item
}

// ---------------------------------------------------------------- k_reader

// Two workgroups of four waves per CU: at most 256 registers per lane.
// Z item of workgroup g's j-th turn, or -1.  The hardware hands workgroup g
// to XCD g % 8; K chunk ks goes to XCD ks % 8, so the items that share a
// chunk's h and W_q columns meet in one L2.
__device__ __forceinline__ int z_of(const FastArgs& a, int g, int G, int j) {
  const int tiles = cdiv_d(a.R, a.R <= 16 ? 16 : 64) * cdiv_d(a.Nz, 64);
  if ((G & 7) != 0) {
    const int q = g + j * G;
    return q < a.n_z ? q : -1;
  }
  const int x = g & 7;
  const int i = (g >> 3) + j * (G >> 3);  // item within the XCD
  const int ks = x + 8 * (i / tiles);
  if (ks >= a.ksplit) return -1;
  return ks * tiles + i % tiles;
}

template <int RR, int BM>
__global__ __launch_bounds__(256, 2) void k_reader(FastArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_last;
  const int g = blockIdx.x, G = gridDim.x;
  if (a.counters[0] != a.magic) {
    // the workspace was not prepared for this plan: touch nothing else
    if (g == 0 && threadIdx.x == 0 && a.dev_status) *a.dev_status = READY_ERR_WORKSPACE_UNINIT;
    return;
  }
  // the first state tile is issued before the Z items, so the state stream
  // starts at once
  TileRegs<RR> r0, r1;
  const int rank = g;
  if (g < a.g_s && rank < a.n_s) tile_issue<RR>(a, rank, r0);
  for (int j = 0;; ++j) {
    const int q = z_of(a, g, G, j);
    if (q < 0) break;
    z_item<BM, BM == 16 ? 5 : 3>(a, q, smem);
  }
  if (g < a.g_s) {
    if (rank + a.g_s < a.n_s) tile_issue<RR>(a, rank + a.g_s, r1);
    s_phase<RR>(a, rank, r0, r1, smem);
  } else {
    for (int j = g - a.g_s; j < a.n_a; j += a.g_t) mlp1_item<RR, BM, BM>(a, j, smem);
  }
  for (int o = g; o < a.n_o; o += G) mlp2_item<BM>(a, o, smem);

  // the last workgroup to finish clears the counters (two-level count)
  __syncthreads();
  if (threadIdx.x == 0) {
    int last = 0;
    const int grp = g % READY_DONE_GROUPS;
    const int in_grp = (G - grp + READY_DONE_GROUPS - 1) / READY_DONE_GROUPS;
    if (count_up(ctr(a.done, grp)) == (uint32_t)(in_grp - 1))
      last = count_up(ctr(a.done, READY_DONE_GROUPS)) == (uint32_t)(min(G, READY_DONE_GROUPS) - 1);
    s_last = last;
  }
  __syncthreads();
  if (s_last) {
    for (int i = READY_CTR_STRIDE + threadIdx.x; i < a.n_counters; i += 256) a.counters[i] = 0u;
  }
}

__global__ void k_ws_init(uint32_t* counters, int n, uint32_t magic) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    counters[i] = (i == 0) ? magic : 0u;
}

// ---------------------------------------------------------------- launchers

size_t ready_reader_lds(int r, int F, int Nz, int small) {
  const int BM = small ? 16 : 64;
  const int NB = (r + 15) / 16;
  const size_t z_bytes = (size_t)3 * BM * 68 * 4 + (size_t)4 * BM * 4;
  const size_t s_bytes = (size_t)r * (READY_TILE + 8) * 2 + (size_t)READY_TILE * r * 2 + 4 * (4 * NB * r * 16 + 4);
  const int Fs = ((F + 31) & ~31) + 8;
  const size_t a_bytes = (size_t)16 * Nz * 4 + (size_t)16 * Fs * 2 + 4 * 16 + 16;
  const size_t sa = (size_t)BM * (256 + 8) * 2, so = (size_t)BM * 68 * 4;
  const size_t o_bytes = (sa > so ? sa : so) + 16;
  size_t m = z_bytes;
  if (s_bytes > m) m = s_bytes;
  if (a_bytes > m) m = a_bytes;
  if (o_bytes > m) m = o_bytes;
  return (m + 15) & ~(size_t)15;
}

hipError_t ready_launch_reader(const FastArgs& a, int small, int grid, hipStream_t s, StageEvents ev) {
  const dim3 g((unsigned)grid), block(256);
  const size_t lds = ready_reader_lds(a.r, a.F, a.Nz, small);
#define READY_READER_CASE(RRV)                                                   \
  do {                                                                           \
    if (small) READY_LAUNCH((k_reader<RRV, 16>), g, block, lds, s, ev, a);       \
    else READY_LAUNCH((k_reader<RRV, 64>), g, block, lds, s, ev, a);             \
  } while (0)
  switch (a.r) {
    case 8: READY_READER_CASE(8); break;
    case 16: READY_READER_CASE(16); break;
    case 24: READY_READER_CASE(24); break;
    default: READY_READER_CASE(32); break;
  }
#undef READY_READER_CASE
  return hipGetLastError();
}

// Workgroups of k_reader that one CU holds at once (0 on error).
int ready_reader_per_cu(int r, int small, size_t lds) {
  int nb = 0;
  hipError_t e = hipSuccess;
#define READY_OCC_CASE(RRV)                                                                              \
  do {                                                                                                   \
    if (small) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_reader<RRV, 16>, 256, lds);      \
    else e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_reader<RRV, 64>, 256, lds);            \
  } while (0)
  switch (r) {
    case 8: READY_OCC_CASE(8); break;
    case 16: READY_OCC_CASE(16); break;
    case 24: READY_OCC_CASE(24); break;
    default: READY_OCC_CASE(32); break;
  }
#undef READY_OCC_CASE
  return e == hipSuccess ? nb : 0;
}

hipError_t ready_launch_ws_init(uint32_t* counters, int n_counters, uint32_t magic, hipStream_t s) {
  hipLaunchKernelGGL(k_ws_init, dim3((unsigned)((n_counters + 255) / 256)), dim3(256), 0, s, counters, n_counters,
                     magic);
  return hipGetLastError();
}
