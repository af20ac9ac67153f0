// Fast path of the ReaDy state reader for gfx950: bf16 states, activations
// and weights, rank r <= 32.  One persistent launch, k_reader.
//
// Its grid is two workgroups per CU.  Workgroups run four kinds of work
// item, in this order:
//   Z  the query sums: a BM x 64 tile of the partial sums z = W_q (gamma h)
//      over one K chunk, plus the sums of squares of h for RMSNorm(h_j)
//      (step 4); the item that completes a tile's last chunk sums the chunks
//      in chunk order.
//   S  the state tiles, drawn through ticket positions in sequence order:
//      fused gather at the accept index into the caller's buffer, mean
//      square, log-RMS and P = V^T S_bar U^T / sqrt(d_k), an r x r matrix
//      (steps 1-3; u_j = T q_j / sqrt(d_k) with T = V^T S_bar and
//      q_j = U^T z_j is P z_j).  One tile per workgroup is in flight
//      at a time.
//   A  8 rows x 64 columns of a: f_j = [P z_j / rms(h_j), ell] per pair,
//      a = act(W1 f + b1) (step 4 readout, step 5), in row order.
//   O  a BM x 128 tile of out = h + W2 a + b2 (step 5), in row order.
// Every item is claimed from a counter (see "claiming work items"): no item
// belongs to a workgroup by its index, and the launch completes whatever
// part of its grid is resident at a time.  Z and S items never wait; A items
// wait for the Z and S items of their rows; O items wait for the A items of
// their rows; a workgroup waits only for items that running workgroups hold
// or will take before they wait themselves.
//
// Several readers sharing one gather use two more forms of the same kernel
// (the MODE template parameter): a prepare launch runs only the S items and
// forms one P per reader from the same tile in LDS; an apply launch runs
// only the Z, A and O items of one reader, reading the P, ell and
// invalid-sequence flags a prepare launch left.
//
// The K chunks of the Z items, and the column blocks of the O items, sit in
// per-XCD queues that the workgroups running on that XCD (hardware XCC id)
// draw from, so the h and W_q columns of a chunk, and the W2 rows of a
// column block, are read from HBM once and then served by that XCD's L2.
// The Z items and the state tiles share one queue per XCD, Z items first:
// a workgroup's first claim, made in the launch's first trip to memory,
// hands it either Z items or its first tiles, so no workgroup spends a trip
// on a claim that finds its kind of item gone.
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
#include <type_traits>

#include "ready_common.h"
#include "ready_sync.h"

namespace {
// Thread 0 waits for *c >= want; the whole workgroup learns the outcome.
__device__ bool wg_wait(const uint32_t* c, uint32_t want, const FastArgs& a, int* s_flag) {
  if (threadIdx.x == 0) *s_flag = wait_count(c, want, a.abort_flag, a.dev_status) ? 1 : 0;
  __syncthreads();
  const bool ok = *s_flag != 0;
  __syncthreads();
  return ok;
}

// Thread 0 of a state tile (u path): have the query items of sequence b's
// rows been counted done?  `known` is the count read when the tile's loads
// were issued.  Polls at most Z_WAIT_POLLS times (about 100 us): the query
// items are taken before any tile (they come first in every queue) and never
// wait, so in a launch whose grid is resident they finish well within it;
// when some XCD's workgroups have not run (other kernels hold it), the tile
// gives up and takes the P path, so no tile ever waits on such an XCD.
constexpr int Z_WAIT_POLLS = 256;
__device__ bool rows_query_done(const FastArgs& a, int b, int bmz, uint32_t known) {
  const uint32_t want = (uint32_t)((a.Nz + 63) / 64);
  if (known >= want) return true;
  const int r0 = b * a.n, r1 = b * a.n + a.n - 1;
  const uint32_t* c0 = ctr(a.zdone, r0 / bmz);
  const uint32_t* c1 = ctr(a.zdone, r1 / bmz);
  int nap = 0;
  for (int it = 0; it < Z_WAIT_POLLS; ++it) {
    if (min(ld_coh_u32(c0), ld_coh_u32(c1)) >= want) return true;
    if ((it & 15) == 15 && ld_coh_u32(a.abort_flag) != 0) return false;
    switch (nap) {
      case 0: __builtin_amdgcn_s_sleep(4); break;
      case 1: __builtin_amdgcn_s_sleep(8); break;
      default: __builtin_amdgcn_s_sleep(16); break;
    }
    if (nap < 2) ++nap;
  }
  return false;
}

// ---- claiming work items
//
// Items sit in queue sets with one queue per XCD: the Z items (K chunks ks
// with ks % 8 == x), the state tiles (t % 8 == x, through a ticket counter),
// the A items (j % 8 == x) and the O items (column blocks cb % 8 == x).  A
// workgroup marks its arrival on its XCD (the hardware XCC id; flag arr_x)
// at start and claims from its XCD's queue of each kind until that queue is
// exhausted; it takes every item of its XCD's Z queue and ticket group
// before any item that waits.  An XCD whose flag is still clear when a
// workgroup is about to take its first A item is an orphan: no workgroup of
// this launch has run there yet (other kernels hold it, say, so the grid is
// only partly resident).  That workgroup then claims and runs the orphan's Z
// items and tiles itself, and drains the orphan's A and O queues after its
// own.  So every wait is for items that running workgroups hold or will take
// before they wait themselves, and every item runs.  In a launch whose grid
// is all resident every flag is set by then, and the check costs the flag
// loads that travel with the first A claim.  (Each XCD has as many Z items as
// the others, so the tiles, shared by all the workgroups of an XCD, are
// balanced too.)


}  // namespace

// ---------------------------------------------------------------- Z items

// 16-byte slot of chunk c (of 16) in row v of a 256-byte-per-row LDS tile:
// rotated by v % 16 so that both row-wise writes and matrix-operand reads
// (16 rows at one chunk) hit distinct banks.
__device__ __forceinline__ int tile_slot(int v, int c) { return v * 16 + (c ^ (v & 15)); }

// Rows [BMZ rb, BMZ rb + BMZ) and columns [64 cb, 64 cb + 64) of the partial
// sums of z = W_q (gamma h) over K chunk ks.  The chunk is walked in stages
// of 128 values of K: the workgroup loads a stage of h and W_q rows with
// row-contiguous 16-byte loads (a wave instruction moves whole 256-byte row
// pieces; three stages are in flight at a time), applies the gain and parks
// one stage at a time in LDS for the matrix instructions; each wave owns a
// (16 WR) x (16 WC) block of the tile.  Column block 0 also stores the sums
// of squares of the h values (before the gain), for RMSNorm(h_j).  The item
// that completes the last chunk of a tile (counted per tile) sums the chunks
// in chunk order into zfin, so the result does not depend on which item came
// last.
template <int BMZ>
struct ZStage {
  static constexpr int HC = BMZ / 16;  // h chunks per thread
  u32x4 h[HC];
  u32x4 w[4];                          // W_q chunks per thread
  u32x4 g;                             // gain chunk
};

template <int BMZ>
__device__ __forceinline__ void z_stage_load(const FastArgs& a, int rb, int cb, int k0, int kend, ZStage<BMZ>& S) {
  const int tid = item_tid();
  const int kk = k0 + 8 * (tid & 15);
  const bool kv = kk < kend;
  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < ZStage<BMZ>::HC; ++q) {
    const int row = rb * BMZ + (tid >> 4) + 16 * q;
    S.h[q] = (kv && row < a.R) ? *(const u32x4*)(a.h + (int64_t)row * a.d + kk) : zero;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int col = cb * 64 + (tid >> 4) + 16 * q;
    S.w[q] = (kv && col < a.Nz) ? *(const u32x4*)(a.wq + (int64_t)col * a.d + kk) : zero;
  }
  S.g = (kv && a.gamma != nullptr) ? *(const u32x4*)(a.gamma + kk) : zero;
}

template <int BMZ, int NST, bool RSV>
__device__ __forceinline__ void z_item(const FastArgs& a, int ks, int cb, int rb, unsigned char* smem) {
  constexpr int RBT = BMZ / 16;                  // 16-row blocks of the tile
  constexpr int WR = RBT >= 4 ? 2 : 1;           // row blocks per wave
  constexpr int WC = (RBT * 4) / (4 * WR);       // column blocks per wave
  constexpr int HC = ZStage<BMZ>::HC;
  constexpr int LD = 68;
  u32x4* sH = (u32x4*)smem;                      // [BMZ][16 slots]
  u32x4* sW = sH + BMZ * 16;                     // [64][16 slots]
  float* red = (float*)smem;                     // [BMZ][LD], after the stages
  int* s_flag = (int*)(smem + (BMZ + 64) * 256);

  const int tid = item_tid(), lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int rbw = (wave % (RBT / WR)) * WR, cbw = (wave / (RBT / WR)) * WC;
  const int kbeg = ks * a.kchunk;
  const int kend = min(a.d, kbeg + a.kchunk);
  const bool want_hss = (cb == 0);

  f32x4 acc[WR][WC];
#pragma unroll
  for (int i = 0; i < WR; ++i)
#pragma unroll
    for (int j = 0; j < WC; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float hsq[HC];
#pragma unroll
  for (int q = 0; q < HC; ++q) hsq[q] = 0.0f;

  // a ring of ZR stages in registers: the first ZR are requested at once,
  // and each later one as soon as a slot has been written to LDS
  constexpr int ZR = NST < 3 ? NST : 3;
  ZStage<BMZ> S[ZR];
#pragma unroll
  for (int st = 0; st < ZR; ++st) z_stage_load<BMZ>(a, rb, cb, kbeg + 128 * st, kend, S[st]);
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    ZStage<BMZ>& Sc = S[st % ZR];
    // the gain and the sums of squares, on the way into LDS
    if (a.gamma != nullptr || want_hss) {
      float g[8];
      Elem<uint16_t>::unpack(Sc.g, g);
#pragma unroll
      for (int q = 0; q < HC; ++q) {
        float x[8];
        Elem<uint16_t>::unpack(Sc.h[q], x);
        if (want_hss) {
#pragma unroll
          for (int e = 0; e < 8; ++e) hsq[q] += x[e] * x[e];
        }
        if (a.gamma != nullptr) {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= g[e];
          Sc.h[q] = pack_bf16x8(x);
        }
      }
    }
    __syncthreads();  // the previous stage (or item) is done with the LDS area
#pragma unroll
    for (int q = 0; q < HC; ++q) sH[tile_slot((tid >> 4) + 16 * q, tid & 15)] = Sc.h[q];
#pragma unroll
    for (int q = 0; q < 4; ++q) sW[tile_slot((tid >> 4) + 16 * q, tid & 15)] = Sc.w[q];
    if (st + ZR < NST) z_stage_load<BMZ>(a, rb, cb, kbeg + 128 * (st + ZR), kend, Sc);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 av[WR], bv[WC];
#pragma unroll
      for (int i = 0; i < WR; ++i) av[i] = sH[tile_slot(16 * (rbw + i) + lr, 4 * s + lg)];
#pragma unroll
      for (int j = 0; j < WC; ++j) bv[j] = sW[tile_slot(16 * (cbw + j) + lr, 4 * s + lg)];
#pragma unroll
      for (int i = 0; i < WR; ++i)
#pragma unroll
        for (int j = 0; j < WC; ++j) acc[i][j] = mfma16x16x32(av[i], bv[j], acc[i][j]);
    }
  }

  __syncthreads();  // the stages are done with the LDS area
#pragma unroll
  for (int i = 0; i < WR; ++i)
#pragma unroll
    for (int j = 0; j < WC; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[(16 * (rbw + i) + 4 * lg + e) * LD + 16 * (cbw + j) + lr] = acc[i][j][e];
  __syncthreads();
  for (int c = tid; c < BMZ * 16; c += 256) {
    const int rr = c >> 4, c4 = (c & 15) * 4;
    const int row = rb * BMZ + rr, col = cb * 64 + c4;
    if (row < a.R && col < a.Nz)
      st_coh16(a.zpart, (uint32_t)(4 * ((ks * a.R + row) * a.Nz + col)), *(const u32x4*)&red[rr * LD + c4]);
  }
  if (want_hss) {
    // lanes 16 k .. 16 k + 15 hold the pieces of rows (tid >> 4) + 16 q
#pragma unroll
    for (int q = 0; q < HC; ++q) {
      float v = hsq[q];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      v += __shfl_xor(v, 8, 64);
      const int row = rb * BMZ + (tid >> 4) + 16 * q;
      if ((tid & 15) == 0 && row < a.R) st_coh_f32(a.hss + ks * a.R + row, v);
    }
  }
  wait_mem();
  __syncthreads();
  const int ncbz = cdiv_d(a.Nz, 64);
  if (tid == 0) *s_flag = count_up(ctr(a.zcnt, rb * ncbz + cb)) == (uint32_t)(a.ksplit - 1) ? 1 : 0;
  __syncthreads();
  if (*s_flag) {
    // every chunk of the tile is stored (each item waited for its stores
    // before counting): sum them in chunk order.  The loads of all of this
    // thread's RBT chunks, KG K chunks at a time, are issued before any is
    // summed, so a group costs one trip to memory (KG * RBT = 32 or 16 loads)
    constexpr int KG = RBT == 1 ? 16 : 8;
    float4 sum[RBT];
    bool live[RBT];
    uint32_t off[RBT];
#pragma unroll
    for (int q = 0; q < RBT; ++q) {
      const int c = tid + 256 * q;
      const int rr = c >> 4, c4 = (c & 15) * 4;
      const int row = rb * BMZ + rr, col = cb * 64 + c4;
      live[q] = row < a.R && col < a.Nz;
      off[q] = live[q] ? (uint32_t)(row * a.Nz + col) : 0u;
      sum[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // (column block 0) the K chunks' sums of squares of the rows' h, for
    // 1 / rms(h), travel with the first group
    const bool hrow = RSV && cb == 0 && tid < BMZ && rb * BMZ + tid < a.R;
    float hv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      hv[k] = ld_coh4_at(hrow && k < a.ksplit, a.hss, (uint32_t)(4 * (k * a.R + rb * BMZ + tid)));
    for (int k0 = 0; k0 < a.ksplit; k0 += KG) {
      u32x4 v[RBT][KG];
#pragma unroll
      for (int q = 0; q < RBT; ++q)
#pragma unroll
        for (int k = 0; k < KG; ++k)
          v[q][k] = (live[q] && k0 + k < a.ksplit)
                        ? ld_coh16(a.zpart, (uint32_t)(4 * ((k0 + k) * a.R * a.Nz + off[q])))
                        : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int q = 0; q < RBT; ++q)
#pragma unroll
        for (int k = 0; k < KG; ++k) {
          sum[q].x += __uint_as_float(v[q][k].x); sum[q].y += __uint_as_float(v[q][k].y);
          sum[q].z += __uint_as_float(v[q][k].z); sum[q].w += __uint_as_float(v[q][k].w);
        }
    }
#pragma unroll
    for (int q = 0; q < RBT; ++q)
      if (live[q])
        st_coh16(a.zfin, 4 * off[q], u32x4{__float_as_uint(sum[q].x), __float_as_uint(sum[q].y),
                                           __float_as_uint(sum[q].z), __float_as_uint(sum[q].w)});
    if (RSV && hrow) {
      // 1 / rms(h) of the rows (RMSNorm of the pages' h), from the K chunks'
      // sums of squares that this column block's items stored, in chunk order
      const int row = rb * BMZ + tid;
      float hs = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) hs += k < a.ksplit ? hv[k] : 0.0f;
      for (int k = 16; k < a.ksplit; ++k) hs += ld_coh4(a.hss, (uint32_t)(4 * (k * a.R + row)));
      st_coh_f32(a.rsv + row, 1.0f / sqrtf(hs / (float)a.d + a.h_eps));
    }
    wait_mem();
    __syncthreads();
    if (tid == 0) count_up(ctr(a.zdone, rb));
  }
  __syncthreads();  // s_flag and the LDS area are reused by the next item
}

// acc + p . z over four values, rounded step by step in a fixed order: the
// state tiles and the A items form u = P z / rms(h) with it, so f is the same
// bit for bit whichever of them forms it.
__device__ __forceinline__ float dot4_acc(float acc, float4 p, float4 z) {
  float t = __fmul_rn(p.x, z.x);
  t = __fmaf_rn(p.y, z.y, t);
  t = __fmaf_rn(p.z, z.z, t);
  t = __fmaf_rn(p.w, z.w, t);
  return __fadd_rn(acc, t);
}

// ---------------------------------------------------------------- S items

// Tile t = (sequence b, pair m).  Thread i loads and stores the 16-byte
// chunks i + 256 j, j < 8, of the tile (rows 16 j + i / 16, column chunk
// i % 16): each wave instruction moves four whole rows, 1 KB in a row of
// addresses, which is what lets the gather run at copy speed.  The S U^T
// operand is read back from an LDS copy of the tile in which chunk c of row
// v sits at slot c ^ (v % 16) of the row, so that both the row-wise writes
// and the matrix-operand reads (16 rows at one column chunk) hit distinct
// banks.  Each thread also carries RR / 8 chunks of the pair's U and V,
// parked in LDS when the tile is processed.
template <int RR>
struct TileRegs {
  static constexpr int NW = 2 * RR * 16 / 256;  // weight chunks per thread
  u32x4 data[8];
  u32x4 w[NW];
  int p;        // accept index of the tile's sequence
  uint32_t zc;  // query items counted done for the tile's rows (the smaller of its row blocks' counts)
};

// UP: the counts of the query items of the sequence's rows are read in the
// same trip (see tile_process).
template <int RR, bool UP, int BMZ>
__device__ __forceinline__ void tile_issue(const FastArgs& a, int t, TileRegs<RR>& R, const int* s_acc) {
  constexpr int WCH = RR * 16;
  const int b = t / a.M, m = t - (t / a.M) * a.M;
  const int tid = item_tid();
  const int mz = a.shared ? 0 : m;
  R.p = b < READY_ACC_LDS ? s_acc[b] : a.accept_idx[b];
  if constexpr (UP) {
    const int r0 = b * a.n, r1 = b * a.n + a.n - 1;
    const uint32_t c0 = ld_coh_u32(ctr(a.zdone, r0 / BMZ)), c1 = ld_coh_u32(ctr(a.zdone, r1 / BMZ));
    R.zc = min(c0, c1);
  }
  const u32x4* Ug = (const u32x4*)(a.u + (int64_t)mz * RR * READY_TILE);
  const u32x4* Vg = (const u32x4*)(a.v + (int64_t)mz * READY_TILE * RR);
#pragma unroll
  for (int k = 0; k < TileRegs<RR>::NW; ++k) {
    const int c = tid + 256 * k;
    R.w[k] = c < WCH ? Ug[c] : Vg[c - WCH];
  }
  if (R.p < 0 || R.p >= a.P) return;
  const int l = m / a.H, hh = m - (m / a.H) * a.H;
  const u32x4* src = (const u32x4*)(a.states + (int64_t)b * a.sb + (int64_t)R.p * a.sp + (int64_t)a.slot[l] * a.sl +
                                    (int64_t)hh * a.sh);
#pragma unroll
  for (int j = 0; j < 8; ++j) R.data[j] = __builtin_nontemporal_load(src + tid + 256 * j);
}

// A tile counts itself in the state-tile counters of the 8-row blocks its
// sequence touches: 1 in the low half, and 1 in the high half too when it
// wrote its columns of f itself (u_path).
__device__ __forceinline__ void tile_count(const FastArgs& a, int t, bool u_path) {
  const int b = t / a.M;
  const int r0 = b * a.n, r1 = b * a.n + a.n - 1;
  for (int q = r0 / READY_ABM; q <= r1 / READY_ABM; ++q)
    __hip_atomic_fetch_add(ctr(a.sdone, q), u_path ? 0x10001u : 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// P = V^T (S U^T) * scale for the tile in LDS (sS) and the U, V of one
// reader in LDS (sU, sV): S U^T on the matrix cores, wave w taking rows
// [32 w, 32 w + 32); then V^T (S U^T) over those rows on the matrix cores
// too (S U^T enters as bf16), and the four waves' partials meet in s_red.
// P is stored device-coherently.
template <int RR>
__device__ __forceinline__ void tile_project(const u32x4* sS, const uint16_t* sU, const uint16_t* sV, float* s_red,
                                             float scale, float* P, float* sP = nullptr) {
  constexpr int NB = (RR + 15) / 16;  // 16-column blocks of U^T
  constexpr int LU = READY_TILE + 8;  // padded U row in LDS (bf16)
  constexpr int WS = NB * RR * 16;    // per-wave partials of P
  const int tid = item_tid(), lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lq = lane >> 4;
  f32x4 acc[2][NB];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 sa[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) sa[mb] = sS[tile_slot(32 * wave + 16 * mb + lrow, 4 * ks + lq)];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int i = 16 * nb + lrow;
      const u32x4 ub = (i < RR) ? *(const u32x4*)&sU[i * LU + 32 * ks + 8 * lq] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) acc[mb][nb] = mfma16x16x32(sa[mb], ub, acc[mb][nb]);
    }
  }

  // acc[mb][nb][e] = (S U^T)[v = 32 w + 16 mb + 4 (l / 16) + e][i' = 16 nb + l % 16]
  // P_w = V_w^T (S U^T)_w on the matrix cores (k = the wave's 32 rows v):
  // with k taken in the order (mb, e), each lane's accumulators are
  // already its B operand (rounded to bf16), and its A operand is
  // V[v][16 mi + l % 16] at its 8 rows v.  The waves' partials, P rows i
  // and columns i', go to s_red[w][i][i'] (16 NB columns a row).
  f32x4 pacc[NB][NB];
  u32x4 bop[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float w8[8] = {acc[0][nb][0], acc[0][nb][1], acc[0][nb][2], acc[0][nb][3],
                         acc[1][nb][0], acc[1][nb][1], acc[1][nb][2], acc[1][nb][3]};
    bop[nb] = pack_bf16x8(w8);
  }
#pragma unroll
  for (int mi = 0; mi < NB; ++mi) {
    const int i = 16 * mi + lrow;
    uint32_t av[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int v = 32 * wave + 16 * (j >> 2) + 4 * lq + (j & 3);
      av[j] = i < RR ? (uint32_t)sV[v * RR + i] : 0u;
    }
    const u32x4 aop = {av[0] | (av[1] << 16), av[2] | (av[3] << 16), av[4] | (av[5] << 16), av[6] | (av[7] << 16)};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) pacc[mi][nb] = mfma16x16x32(aop, bop[nb], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
  }
#pragma unroll
  for (int mi = 0; mi < NB; ++mi)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * mi + 4 * lq + e;
        if (i < RR) s_red[wave * WS + i * 16 * NB + 16 * nb + lrow] = pacc[mi][nb][e];
      }
  __syncthreads();
  for (int e = tid; e < RR * RR; e += 256) {
    const int i = e / RR, ip = e - (e / RR) * RR;
    const int idx = i * 16 * NB + ip;
    const float pv = ((s_red[idx] + s_red[WS + idx]) + (s_red[2 * WS + idx] + s_red[3 * WS + idx])) * scale;
    st_coh_f32(P + e, pv);
    if (sP) sP[e] = pv;
  }
}

// Process tile t whose loads were issued into R: copy to `gathered`, sum of
// squares, S U^T, P, ell.  Once R's data is in LDS, the loads of the tile at
// position `raw` of queue q (published in *s_pub, NO_ITEM when that is past
// the queue's zs Z items and nt tickets) go out into R, after thread 0's claim
// of the position after it (returned; tk == nullptr: no claim).  So the next
// tile's loads overlap this tile's projection and stores, and the claim has a
// whole turn to return.  At the end every wave waits for its stores, and the
// tile is counted done.
//
// UP (one-reader launches at r >= 16, where forming f from P in the A items
// means moving r^2 floats per (sequence, pair) again): once the query items of
// the tile's rows are counted done (rows_query_done), the tile also forms its
// pair's columns of f for its sequence's rows, u = P z / rms(h) and ell, into
// fu, and counts itself with the u mark (tile_count): A items whose rows'
// tiles all did so load f instead of forming it from P.
template <int RR, bool MULTI, bool UP, int BMZ>
__device__ __forceinline__ uint32_t tile_process(const FastArgs& a, int t, TileRegs<RR>& R, unsigned char* smem,
                                                 uint32_t* s_pub, uint32_t raw, int q, uint32_t zs, uint32_t nt,
                                                 uint32_t* tk, const int* s_acc) {
  auto pub_of = [&]() {
    return (raw != NO_ITEM && raw >= zs && raw - zs < nt) ? (uint32_t)(q + READY_TICKET_GROUPS * (int)(raw - zs))
                                                          : NO_ITEM;
  };
  constexpr int NB = (RR + 15) / 16;  // 16-column blocks of U^T
  constexpr int LU = READY_TILE + 8;  // padded U row in LDS (bf16)
  constexpr int WCH = RR * 16;
  constexpr int WS = NB * RR * 16;    // per-wave partials of P
  u32x4* sS = (u32x4*)smem;                              // [128 rows][16 slots]
  uint16_t* sU = (uint16_t*)(sS + READY_TILE * 16);      // [RR][LU]
  uint16_t* sV = sU + RR * LU;                           // [128][RR]
  float* s_red = (float*)(sV + READY_TILE * RR);         // [4][WS]
  float* s_wsum = s_red + 4 * WS;                        // [4]
  float* s_P = s_wsum + 4;                               // [RR][RR]: P (u path)
  float* s_zu = s_P + RR * RR;                           // [16][RR]: z of the sequence's rows (u path)
  float* s_ru = s_zu + 16 * RR;                          // [16]: their 1 / rms(h)
  float* s_el = s_ru + 16;                               // ell

  const int b = t / a.M, m = t - (t / a.M) * a.M;
  const int tid = item_tid(), lane = tid & 63, wave = tid >> 6;
  float* P = a.pmat + (int64_t)t * RR * RR;

  const bool valid = R.p >= 0 && R.p < a.P;
  u32x4* dst = (u32x4*)(a.gathered + (int64_t)t * READY_TILE_ELEMS);
  // the u path is taken on thread 0's reading of the query counts (waves may
  // have read different counts), published with the first barrier
  if constexpr (UP) {
    if (tid == 0) s_pub[2] = (valid && rows_query_done(a, b, BMZ, R.zc)) ? 1u : 0u;
  }
  __syncthreads();  // the previous tile is done with the LDS area and *s_pub
  if (tid == 0) *s_pub = pub_of();
  const bool up = UP && s_pub[2] != 0u;
  // u path: z of the sequence's rows for this pair, and their 1 / rms(h)
  constexpr int RC = RR / 4;
  const int mz = a.shared ? 0 : m;
  const int zj = tid / RC, zk = tid - (tid / RC) * RC;
  const u32x4 zq = ld_coh16_at(up && tid < a.n * RC, a.zfin, (uint32_t)(4 * ((b * a.n + zj) * a.Nz + mz * RR + 4 * zk)));
  const float rq = ld_coh4_at(up && tid < a.n, a.rsv, (uint32_t)(4 * (b * a.n + tid)));
  float ss = 0.0f;
  if (valid) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = tid + 256 * j;
      __builtin_nontemporal_store(R.data[j], dst + c);
      sS[tile_slot(c >> 4, c & 15)] = R.data[j];
      ss += sumsq_bf16x8(R.data[j]);
    }
#pragma unroll
    for (int k = 0; k < TileRegs<RR>::NW; ++k) {
      const int c = tid + 256 * k;
      if (c < WCH) *(u32x4*)&sU[(c >> 4) * LU + 8 * (c & 15)] = R.w[k];
      else *(u32x4*)&sV[8 * (c - WCH)] = R.w[k];
    }
  }
  // ---- step 2: mean square ----
  ss = wave_sum(ss);
  if (lane == 0) s_wsum[wave] = ss;
  __syncthreads();
  // R is free: claim the position after the next tile, then issue its loads
  const int tn = (int)*s_pub;
  uint32_t claim = NO_ITEM;
  if (tid == 0 && tn >= 0 && tk != nullptr) claim = count_up(tk);
  if (tn >= 0) tile_issue<RR, UP, BMZ>(a, tn, R, s_acc);

  if (!valid) {
    // out-of-range accept index: flag it and leave this sequence's outputs
    for (int inj = 0; inj < (MULTI ? a.n_inj : 1); ++inj)
      for (int e = tid; e < RR * RR; e += 256) st_coh_f32(P + (int64_t)inj * a.p_inj_stride + e, 0.0f);
    if (tid == 0) {
      if (a.dev_status) st_coh_u32(a.dev_status, (uint32_t)READY_ERR_ACCEPT_IDX);
      if (m == 0) st_coh_u32(a.seq_invalid + b, 1u);
      st_coh_f32(a.ell + t, 0.0f);
    }
    wait_mem();
    __syncthreads();
    if (tid == 0) tile_count(a, t, false);
    return claim;
  }

  const float ms = ((s_wsum[0] + s_wsum[1]) + (s_wsum[2] + s_wsum[3])) * (1.0f / READY_TILE_ELEMS);
  const float rms = sqrtf(ms + a.state_eps);
  const float scale = 0.08838834764831845f / rms;  // 1 / (rms sqrt(d_k)), d_k = 128
  tile_project<RR>(sS, sU, sV, s_red, scale, P, up ? s_P : nullptr);
  if (tid == 0) {
    const float ell = logf(rms);
    st_coh_f32(a.ell + t, ell);
    if (m == 0) st_coh_u32(a.seq_invalid + b, 0u);
    if (a.logrms) a.logrms[t] = ell;
    s_el[0] = ell;
  }
  if (up) {
    // f of the sequence's rows for this pair: u_j = P z_j / rms(h_j), ell
    if (tid < a.n * RC) *(u32x4*)&s_zu[zj * RR + 4 * zk] = zq;
    if (tid < a.n) s_ru[tid] = rq;
    __syncthreads();
    const int Fp = (a.F + 31) & ~31;
    for (int e = tid; e < a.n * (RR + 1); e += 256) {
      const int j = e / (RR + 1), i = e - (e / (RR + 1)) * (RR + 1);
      float v = s_el[0];
      if (i < RR) {
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < RC; ++c)
          acc = dot4_acc(acc, *(const float4*)&s_P[i * RR + 4 * c], *(const float4*)&s_zu[j * RR + 4 * c]);
        v = __fmul_rn(acc, s_ru[j]);
      }
      st_coh_f32(a.fu + (int64_t)(b * a.n + j) * Fp + m * (RR + 1) + i, v);
    }
  }
  // further readers of the same state (prepare launches only): the tile
  // stays in LDS, their U and V replace the first reader's.  The next
  // reader's U and V are requested while the current one is projected.
  if (MULTI && a.n_inj > 1) {
    const int mz = a.shared ? 0 : m;
    u32x4 wn[TileRegs<RR>::NW];
    auto fetch = [&](int inj) {
      const u32x4* Ug = (const u32x4*)(a.u_inj[inj] + (int64_t)mz * RR * READY_TILE);
      const u32x4* Vg = (const u32x4*)(a.v_inj[inj] + (int64_t)mz * READY_TILE * RR);
#pragma unroll
      for (int k = 0; k < TileRegs<RR>::NW; ++k) {
        const int c = tid + 256 * k;
        wn[k] = c < WCH ? Ug[c] : Vg[c - WCH];
      }
    };
    fetch(1);
    for (int inj = 1; inj < a.n_inj; ++inj) {
      __syncthreads();  // every wave is done with the previous reader's U, V and partials
#pragma unroll
      for (int k = 0; k < TileRegs<RR>::NW; ++k) {
        const int c = tid + 256 * k;
        if (c < WCH) *(u32x4*)&sU[(c >> 4) * LU + 8 * (c & 15)] = wn[k];
        else *(u32x4*)&sV[8 * (c - WCH)] = wn[k];
      }
      __syncthreads();
      if (inj + 1 < a.n_inj) fetch(inj + 1);
      tile_project<RR>(sS, sU, sV, s_red, scale, P + (int64_t)inj * a.p_inj_stride);
    }
  }
  wait_mem();
  __syncthreads();
  if (tid == 0) tile_count(a, t, up);
  return claim;
}

// Ticket i of group q is tile q + G i (G = READY_TICKET_GROUPS); group q
// holds group_tiles(q) tickets.
__device__ __forceinline__ uint32_t group_tiles(const FastArgs& a, int q) {
  return (uint32_t)((a.n_s - q + READY_TICKET_GROUPS - 1) / READY_TICKET_GROUPS);
}

// The S items of one workgroup: the tiles at the positions it claims in
// queue q after the queue's zs Z items (ticket i of group q is position
// zs + i), starting with position p0 (NO_ITEM for none).  One tile is in
// flight at a time: the next tile's loads are issued once the current one's
// data is in LDS (see tile_process), and each position is claimed a turn
// before its loads, so that waiting for a claim never waits for tile data.
// (More tiles in flight per workgroup only lengthen the memory queues once
// the whole grid streams: the launch is then bound by bandwidth, and the
// deeper queues delay the last tiles.)
template <int RR, bool MULTI, bool UP, int BMZ>
__device__ __forceinline__ void s_phase(const FastArgs& a, int q, uint32_t zs, uint32_t p0, unsigned char* smem,
                                        const int* s_acc, uint32_t* s_tk) {
  constexpr int NQ = READY_TICKET_GROUPS;
  const int tid = item_tid();
  const uint32_t nt = group_tiles(a, q);
  uint32_t* tk = ctr(a.tk, q);
  int t0 = (p0 != NO_ITEM && p0 >= zs && p0 - zs < nt) ? q + NQ * (int)(p0 - zs) : -1;
  uint32_t raw = NO_ITEM;  // thread 0: the position after t0
  if (tid == 0 && t0 >= 0) raw = count_up(tk);
  TileRegs<RR> r0;
  if (t0 >= 0) tile_issue<RR, UP, BMZ>(a, t0, r0, s_acc);
  while (t0 >= 0) {
    raw = tile_process<RR, MULTI, UP, BMZ>(a, t0, r0, smem, s_tk, raw, q, zs, nt, tk, s_acc);
    t0 = (int)*s_tk;
  }
  __syncthreads();  // the LDS area is reused by the next item
}

// ---------------------------------------------------------------- A items

// Rows [8 rb, 8 rb + 8) of f and a (READY_ABM = 8; the matrix instructions
// take 16-row tiles, whose upper half is zero), columns [64 cb, 64 cb + 64).
// After the tiles of zfin of these rows and the S items of their sequences
// are counted, one trip to memory brings z (into LDS), the sums of squares of
// h, and the P rows and log-RMS this thread applies: f = [u = P z / rms(h),
// ell] per (row, pair), into LDS in bf16 and into `feat` in fp32.
// Wave w computes a's columns 64 cb + 16 w .. + 15 on the matrix cores, W1
// rows streaming straight from memory.
template <int RR, int BMZ, int BMO, bool UP>
__device__ __forceinline__ void mlp1_item(const FastArgs& a, int item, unsigned char* smem) {
  const int ncb = cdiv_d(a.Hm, 64);
  const int rb = item / ncb, cb = item - (item / ncb) * ncb;
  const int tid = item_tid(), lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int row0 = rb * READY_ABM;
  const int rows = min(READY_ABM, a.R - row0);
  const int F = a.F, Nz = a.Nz;
  const int Fp = (F + 31) & ~31;
  const int Fs = Fp + 8;
  float* z_s = (float*)smem;                       // [READY_ABM][Nz]
  uint16_t* fsh = (uint16_t*)(z_s + READY_ABM * Nz);  // [16][Fs]: rows past READY_ABM stay zero
  float* s_rs = (float*)(fsh + 16 * Fs);           // [16]
  int* s_flag = (int*)(s_rs + 16);

  // W1 rows of this lane's column: independent of every other item
  const int col = cb * 64 + 16 * wave + lr;
  const bool cv = col < a.Hm;
  const uint16_t* wrow = a.w1 + (int64_t)col * F;
  constexpr int W1S = 12;  // steps of 32 values of K per pass (F <= 384: one pass)
  u32x4 bq[W1S];
#pragma unroll
  for (int s = 0; s < W1S; ++s) {
    const int kk = 32 * s + 8 * lg;
    bq[s] = (cv && kk < F) ? *(const u32x4*)(wrow + kk) : u32x4{0u, 0u, 0u, 0u};
  }
  // the bias of this lane's column, with the W1 rows (before the wait)
  const float bias = (cv && a.b1) ? Elem<uint16_t>::ld(a.b1, col) : 0.0f;

  const int b0 = row0 / a.n, b1 = (row0 + rows - 1) / a.n;
  // the state-tile count of these rows: tiles in the low half, tiles that
  // formed their columns of f themselves in the high half (tile_count)
  const uint32_t want_s = a.n_s > 0 ? (uint32_t)(a.M * (b1 - b0 + 1)) : 0u;
  if (threadIdx.x == 0) {
    uint32_t last = 0u;
    const bool okw = wait_count2(ctr(a.zdone, row0 / BMZ), (uint32_t)cdiv_d(Nz, 64), ctr(a.sdone, rb), 0xffffu,
                                 want_s, &last, a.abort_flag, a.dev_status);
    *s_flag = !okw ? 0 : ((UP && want_s > 0u && (last >> 16) >= want_s) ? 2 : 1);
  }
  __syncthreads();
  const bool ok = *s_flag != 0;
  const bool f_ready = UP && *s_flag == 2;  // every tile of these rows formed its columns of f
  const bool want_feat = a.feat != nullptr && cb == 0;
  float* feat0 = a.feat + (int64_t)row0 * F;

  if (f_ready) {
    // ---- one trip to memory: the f rows (fp32, rows Fp apart), placed in
    // LDS in bf16 (and into `feat` in fp32)
    constexpr int FC = 8;
    const int cpr = Fp / 4;  // 16-byte chunks per row
    const int nfc = rows * cpr;
    u32x4 fv[FC];
#pragma unroll
    for (int j = 0; j < FC; ++j) {
      const int c = tid + 256 * j;
      fv[j] = ld_coh16_at(c < nfc, a.fu, (uint32_t)(4 * ((row0 + c / cpr) * Fp + 4 * (c - (c / cpr) * cpr))));
    }
    // f starts at zero (rows past the end, padding columns); Fs is a multiple of 8
    for (int e = tid; e < 2 * Fs; e += 256) ((u32x4*)fsh)[e] = u32x4{0u, 0u, 0u, 0u};
    wait_mem();
#pragma unroll
    for (int j = 0; j < FC; ++j) pin(fv[j]);
    __syncthreads();
    auto put = [&](int c, u32x4 v) {
      const int rr = c / cpr, c0 = 4 * (c - (c / cpr) * cpr);
      const float x[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (c0 + e < F) {
          fsh[rr * Fs + c0 + e] = f32_to_bf16_rne(x[e]);
          if (want_feat) feat0[rr * F + c0 + e] = x[e];
        }
      }
    };
#pragma unroll
    for (int j = 0; j < FC; ++j) {
      const int c = tid + 256 * j;
      if (c < nfc) put(c, fv[j]);
    }
    for (int c = tid + 256 * FC; c < nfc; c += 256)
      put(c, ld_coh16(a.fu, (uint32_t)(4 * ((row0 + c / cpr) * Fp + 4 * (c - (c / cpr) * cpr)))));
    __syncthreads();
  } else {

  // ---- one trip to memory: z of the rows, the sums of squares of h,
  // the P rows of this thread's first f item and the log-RMS entries it
  // places.  An f item is (pair m, output i): it holds row i of P[b][m] for
  // the sequences b of this block (up to PS at a time) and applies it to
  // each of their rows here.
  constexpr int CR4 = RR / 4;   // 16-byte chunks of a row of P
  constexpr int PS = RR <= 16 ? 4 : 2;  // sequences per load group
  constexpr int RU = RR <= 8 ? 4 : (RR <= 16 ? 2 : 1);  // rows per step of the f loop
  const int nseq = b1 - b0 + 1;
  const int nmi = a.M * RR;
  // at r <= 8 the P rows of a thread's second f item (e = tid + 256) come
  // in the same trip as its first, into a second register set
  constexpr bool PRE2 = RR <= 8;
  u32x4 pv[PS][CR4], pv2[PRE2 ? PS : 1][PRE2 ? CR4 : 1];
  auto load_p_into = [&](int e, int s0, auto& dst) {
    const int m = e / RR, i = e - (e / RR) * RR;
#pragma unroll
    for (int s = 0; s < PS; ++s) {
      const int b = b0 + s0 + s;
      const bool live = e < nmi && s0 + s < nseq && ok;
      const uint32_t pofs = (uint32_t)((((b * a.M + m) * RR + i) * RR) * 4);
#pragma unroll
      for (int c = 0; c < CR4; ++c) dst[s][c] = ld_coh16_at(live, a.pmat, pofs + 16 * c);
    }
  };
  auto load_p = [&](int e, int s0) { load_p_into(e, s0, pv); };
  // the ell columns of f: (row, pair) entries e = tid + 256 j of the 16 x M
  // of them, EL per thread in the trip, the rest after it
  constexpr int EL = 2;
  const int nel = READY_ABM * a.M;
  auto ell_of = [&](int e, bool& live, int& fofs) {
    const int rr = e / a.M, m = e - (e / a.M) * a.M;
    live = e < nel && rr < rows && ok;
    fofs = rr * Fs + m * (RR + 1) + RR;
    return (uint32_t)(4 * (((row0 + rr) / a.n) * a.M + m));
  };
  float ev[EL];
#pragma unroll
  for (int j = 0; j < EL; ++j) {
    bool live;
    int fofs;
    const uint32_t off = ell_of(tid + 256 * j, live, fofs);
    ev[j] = ld_coh4_at(live, a.ell, off);
  }
  // z of the rows: READY_ABM Nz / 4 chunks of 16 bytes, ZC per thread in the
  // trip (all of them for Nz <= 256), the rest after it
  constexpr int ZC = 4;
  const int nzc = rows * (Nz / 4), nzall = READY_ABM * (Nz / 4);
  u32x4 zv[ZC];
#pragma unroll
  for (int j = 0; j < ZC; ++j) {
    const int c = tid + 256 * j;
    zv[j] = ld_coh16_at(c < nzc && ok, a.zfin, (uint32_t)(4 * (row0 * Nz + 4 * c)));
  }
  load_p(tid, 0);
  if constexpr (PRE2) load_p_into(tid + 256, 0, pv2);
  // 1 / rms(h) of the rows (threads below `rows`, one row each) travels with
  // the other loads: at the ranks where the tiles form f, as the value the
  // query items left in rsv; below, as the K chunks' sums of squares
  constexpr bool RSV = RR >= READY_UPATH_MIN_R;
  const bool hrow = tid < rows && ok;
  float rsl = 0.0f, hv[RSV ? 1 : 16];
  if constexpr (RSV) {
    rsl = ld_coh4_at(hrow, a.rsv, (uint32_t)(4 * (row0 + tid)));
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k)
      hv[k] = ld_coh4_at(hrow && k < a.ksplit, a.hss, (uint32_t)(4 * (k * a.R + row0 + tid)));
  }
  // every load of the trip is in flight before this wait; the pins keep the
  // compiler from sinking any of them into a later trip
  wait_mem();
#pragma unroll
  for (int j = 0; j < ZC; ++j) pin(zv[j]);
#pragma unroll
  for (int s = 0; s < PS; ++s) {
#pragma unroll
    for (int c = 0; c < CR4; ++c) {
      pin(pv[s][c]);
      if constexpr (PRE2) pin(pv2[s][c]);
    }
  }
#pragma unroll
  for (int j = 0; j < EL; ++j) pin(ev[j]);
  if constexpr (RSV) {
    pin(rsl);
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) pin(hv[k]);
  }
#pragma unroll
  for (int j = 0; j < ZC; ++j) {
    const int c = tid + 256 * j;
    if (c < nzall) *(u32x4*)&z_s[4 * c] = zv[j];
  }
  for (int c = tid + 256 * ZC; c < nzall; c += 256)
    *(u32x4*)&z_s[4 * c] = (c < nzc && ok) ? ld_coh16(a.zfin, (uint32_t)(4 * (row0 * Nz + 4 * c))) : u32x4{0u, 0u, 0u, 0u};
  if constexpr (!RSV) {
    if (hrow) {
      float hs = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) hs += k < a.ksplit ? hv[k] : 0.0f;
      for (int k = 16; k < a.ksplit; ++k) hs += ld_coh4(a.hss, (uint32_t)(4 * (k * a.R + row0 + tid)));
      rsl = 1.0f / sqrtf(hs / (float)a.d + a.h_eps);
    }
  }
  if (tid < 16) s_rs[tid] = hrow ? rsl : 0.0f;
  // f starts at zero (rows past the end, padding columns); Fs is a multiple of 8
  for (int e = tid; e < 2 * Fs; e += 256) ((u32x4*)fsh)[e] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  // the ell columns
#pragma unroll
  for (int j = 0; j < EL; ++j) {
    bool live;
    int fofs;
    ell_of(tid + 256 * j, live, fofs);
    if (live) {
      fsh[fofs] = f32_to_bf16_rne(ev[j]);
      if (want_feat) feat0[fofs - (fofs / Fs) * (Fs - F)] = ev[j];
    }
  }
  for (int e = tid + 256 * EL; e < nel; e += 256) {
    bool live;
    int fofs;
    const uint32_t off = ell_of(e, live, fofs);
    if (live) {
      const float v = ld_coh4(a.ell, off);
      fsh[fofs] = f32_to_bf16_rne(v);
      if (want_feat) feat0[fofs - (fofs / Fs) * (Fs - F)] = v;
    }
  }
  // the u columns.  Each step computes RU rows of one sequence's range; a
  // step's rows past the range are rewritten later by the sequence they
  // belong to (or are zero rows past the block), so they need no test.
  auto f_loop = [&](auto feat_tag) {
    constexpr bool FEAT = decltype(feat_tag)::value;
    for (int e0 = tid; e0 < nmi; e0 += 256) {
      const int m = e0 / RR, i = e0 - (e0 / RR) * RR;
      const int mz = a.shared ? 0 : m;
      const int fcol = m * (RR + 1) + i;
      for (int s0 = 0; s0 < nseq; s0 += PS) {
        if constexpr (PRE2) {
          if (e0 == tid + 256 && s0 == 0) {
#pragma unroll
            for (int s = 0; s < PS; ++s) {
#pragma unroll
              for (int c = 0; c < CR4; ++c) pv[s][c] = pv2[s][c];
            }
          } else if (e0 != tid || s0 != 0) {
            load_p(e0, s0);
          }
        } else if (e0 != tid || s0 != 0) {
          load_p(e0, s0);
        }
#pragma unroll
        for (int s = 0; s < PS; ++s) {
          const int b = b0 + s0 + s;
          // rows of sequence b in this block (none when b is past the last)
          const int ra = max(row0, b * a.n) - row0;
          const int rz = s0 + s < nseq ? min(row0 + rows, (b + 1) * a.n) - row0 : ra;
          for (int r0 = ra; r0 < rz; r0 += RU) {
#pragma unroll
            for (int q = 0; q < RU; ++q) {
              const int rr = min(r0 + q, READY_ABM - 1);
              float acc = 0.0f;
#pragma unroll
              for (int c = 0; c < CR4; ++c) {
                const float4 pq = make_float4(__uint_as_float(pv[s][c].x), __uint_as_float(pv[s][c].y),
                                              __uint_as_float(pv[s][c].z), __uint_as_float(pv[s][c].w));
                const float4 zq = *(const float4*)&z_s[rr * Nz + mz * RR + 4 * c];
                if constexpr (RR >= READY_UPATH_MIN_R) {
                  // the same rounding as the tiles' u path (at these ranks
                  // one-reader launches take it, and every launch of the
                  // rank must give the same f)
                  acc = dot4_acc(acc, pq, zq);
                } else {
                  acc += pq.x * zq.x + pq.y * zq.y + pq.z * zq.z + pq.w * zq.w;
                }
              }
              const float u = __fmul_rn(acc, s_rs[rr]);
              fsh[rr * Fs + fcol] = f32_to_bf16_rne(u);
              if constexpr (FEAT) {
                if (r0 + q < rz) feat0[rr * F + fcol] = u;
              }
            }
          }
        }
      }
    }
  };
  // The same sums when the block's rows belong to at most PS sequences (one
  // P load group): every row of the block in one pass, z of RG rows read
  // from LDS first, then the rows' dot products, then their stores, so a
  // thread waits for LDS once per RG rows rather than once per row.  Row rr
  // takes the P rows of its sequence (index s within the block) by selects
  // over the NS candidates.
  auto f_rows = [&](auto feat_tag, auto ns_tag) {
    constexpr bool FEAT = decltype(feat_tag)::value;
    constexpr int NS = decltype(ns_tag)::value;
    constexpr int RG = RR <= 8 ? 4 : (RR <= 16 ? 2 : 1);
    for (int e0 = tid; e0 < nmi; e0 += 256) {
      const int m = e0 / RR, i = e0 - (e0 / RR) * RR;
      const int mz = a.shared ? 0 : m;
      const int fcol = m * (RR + 1) + i;
      if constexpr (PRE2) {
        if (e0 == tid + 256) {
#pragma unroll
          for (int s = 0; s < PS; ++s) {
#pragma unroll
            for (int c = 0; c < CR4; ++c) pv[s][c] = pv2[s][c];
          }
        } else if (e0 != tid) {
          load_p(e0, 0);
        }
      } else if (e0 != tid) {
        load_p(e0, 0);
      }
      // sequence index of the current row, and the first row of the next
      int sq = 0, bnd = (b0 + 1) * a.n - row0;
#pragma unroll
      for (int g0 = 0; g0 < READY_ABM; g0 += RG) {
        float4 zr[RG][CR4];
        float rs[RG], u[RG];
#pragma unroll
        for (int q = 0; q < RG; ++q) {
#pragma unroll
          for (int c = 0; c < CR4; ++c) zr[q][c] = *(const float4*)&z_s[(g0 + q) * Nz + mz * RR + 4 * c];
          rs[q] = s_rs[g0 + q];
        }
#pragma unroll
        for (int q = 0; q < RG; ++q) {
          const bool next = g0 + q >= bnd;
          sq += next ? 1 : 0;
          bnd += next ? a.n : 0;
          float acc = 0.0f;
#pragma unroll
          for (int c = 0; c < CR4; ++c) {
            u32x4 pw = pv[0][c];
#pragma unroll
            for (int k = 1; k < NS; ++k) pw = sq == k ? pv[k][c] : pw;
            const float4 pq = make_float4(__uint_as_float(pw.x), __uint_as_float(pw.y), __uint_as_float(pw.z),
                                          __uint_as_float(pw.w));
            const float4 zq = zr[q][c];
            if constexpr (RR >= READY_UPATH_MIN_R) {
              acc = dot4_acc(acc, pq, zq);
            } else {
              acc += pq.x * zq.x + pq.y * zq.y + pq.z * zq.z + pq.w * zq.w;
            }
          }
          u[q] = __fmul_rn(acc, rs[q]);
        }
#pragma unroll
        for (int q = 0; q < RG; ++q) {
          if (g0 + q < rows) {
            fsh[(g0 + q) * Fs + fcol] = f32_to_bf16_rne(u[q]);
            if constexpr (FEAT) feat0[(g0 + q) * F + fcol] = u[q];
          }
        }
      }
    }
  };
  using two = std::integral_constant<int, 2>;
  using all = std::integral_constant<int, PS>;
  if (nseq <= 2) {
    if (want_feat) f_rows(std::true_type{}, two{});
    else f_rows(std::false_type{}, two{});
  } else if (nseq <= PS) {
    if (want_feat) f_rows(std::true_type{}, all{});
    else f_rows(std::false_type{}, all{});
  } else {
    if (want_feat) f_loop(std::true_type{});
    else f_loop(std::false_type{});
  }
  __syncthreads();
  }

  // a = act(W1 f + b1) for this wave's 16 columns.  The A operands of a
  // pass are read from LDS first (steps past F read the last step's
  // columns: their W1 chunks are zero), then the matrix instructions run
  // back to back, alternating between two accumulators.
  f32x4 acc0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, acc1 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = 0; k0 < Fp; k0 += 32 * W1S) {
    if (k0 > 0) {
#pragma unroll
      for (int s = 0; s < W1S; ++s) {
        const int kk = k0 + 32 * s + 8 * lg;
        bq[s] = (cv && kk < F) ? *(const u32x4*)(wrow + kk) : u32x4{0u, 0u, 0u, 0u};
      }
    }
    u32x4 aop[W1S];
#pragma unroll
    for (int s = 0; s < W1S; ++s) {
      const int kb = min(k0 + 32 * s, Fp - 32);
      aop[s] = *(const u32x4*)&fsh[lr * Fs + kb + 8 * lg];
    }
#pragma unroll
    for (int s = 0; s < W1S; s += 2) {
      acc0 = mfma16x16x32(aop[s], bq[s], acc0);
      if (s + 1 < W1S) acc1 = mfma16x16x32(aop[s + 1], bq[s + 1], acc1);
    }
  }
  const f32x4 acc = acc0 + acc1;
  // a in bf16: lanes l and l + 1 hold neighbouring columns; the even lane
  // stores the pair as one 32-bit word
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t mine = f32_to_bf16_rne(activation(acc[e] + bias, a.act));
    const uint32_t next = __shfl_down(mine, 1, 64);
    const int rr = 4 * lg + e;
    if ((lr & 1) == 0 && cv && rr < rows) st_coh_u32(a.abuf + (int64_t)(row0 + rr) * a.Hm + col, mine | (next << 16));
  }
  wait_mem();
  __syncthreads();
  if (tid == 0) count_up(ctr(a.adone, row0 / BMO));
  __syncthreads();  // the LDS area is reused by the next item
}

// ---------------------------------------------------------------- O items

// Rows [BM rb, BM rb + BM) and columns [OC cb, OC cb + OC) of out (OC =
// READY_OCOLS, READY_OCOLS_SMALL at most 16 rows); wave w computes columns
// OC cb + (OC / 4) w .. + OC / 4 - 1,
// 16 at a time.  The W2 rows of the lane's columns, the tile's h values and
// the b2 chunk are loaded before waiting; after the A items of the rows are
// counted, the a rows are staged in LDS by passes of 256 values of K
// (device-coherent loads) for the matrix instructions.  The epilogue goes
// through LDS so that h, out and delta move in 16-byte row chunks.
template <int BM, int OC>
__device__ __forceinline__ void mlp2_item(const FastArgs& a, int rb, int cb, unsigned char* smem) {
  static_assert(OC <= READY_OCOLS, "the LDS area is sized for READY_OCOLS columns");
  constexpr int KT = 256, LA = KT + 8, LO = OC + 4;
  constexpr int WCOL = OC / 4, H2 = WCOL / 16;  // columns per wave, 16-column blocks per wave
  static_assert(WCOL % 16 == 0, "whole 16-column blocks per wave");
  constexpr int SA = BM * LA * 2, SO = BM * LO * 4;
  uint16_t* sA = (uint16_t*)smem;   // [BM][LA]
  float* sO = (float*)smem;         // [BM][LO], after the K passes
  int* s_flag = (int*)(smem + (SA > SO ? SA : SO));

  const int tid = item_tid(), lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int row0 = rb * BM, col0 = cb * OC;
  const int rows = min(BM, a.R - row0);
  int colv[H2];
  bool cv[H2];
#pragma unroll
  for (int h2 = 0; h2 < H2; ++h2) {
    colv[h2] = col0 + WCOL * wave + 16 * h2 + lr;
    cv[h2] = colv[h2] < a.d;
  }

  u32x4 bq[H2][KT / 32];
#pragma unroll
  for (int h2 = 0; h2 < H2; ++h2)
#pragma unroll
    for (int s = 0; s < KT / 32; ++s) {
      const int kk = 32 * s + 8 * lg;
      bq[h2][s] = (cv[h2] && kk < a.Hm) ? *(const u32x4*)(a.w2 + (int64_t)colv[h2] * a.Hm + kk) : u32x4{0u, 0u, 0u, 0u};
    }

  // the epilogue's h chunks (BM rows x CPR chunks of 8 values), and the b2
  // chunk of this thread's columns (the same for each of its chunks, since
  // 256 is a multiple of CPR)
  constexpr int CPR = OC / 8;
  constexpr int EPT = (BM * CPR + 255) / 256;
  static_assert(256 % CPR == 0, "one column chunk per thread");
  const int gcb = col0 + (tid % CPR) * 8;
  const u32x4 b2q = (a.b2 != nullptr && gcb < a.d) ? *(const u32x4*)(a.b2 + gcb) : u32x4{0u, 0u, 0u, 0u};
  u32x4 hq[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int c = tid + 256 * k;
    const int rr = c / CPR, gc = col0 + (c % CPR) * 8;
    hq[k] = (c < BM * CPR && rr < rows && gc < a.d) ? *(const u32x4*)(a.h + (int64_t)(row0 + rr) * a.d + gc)
                                                   : u32x4{0u, 0u, 0u, 0u};
  }

  const uint32_t want = (uint32_t)(cdiv_d(rows, READY_ABM) * cdiv_d(a.Hm, 64));
  if (!wg_wait(ctr(a.adone, rb), want, a, s_flag)) return;
  // the invalid-sequence flags of the epilogue's rows, with the a loads
  uint32_t inv[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int c = tid + 256 * k;
    const int rr = c / CPR;
    inv[k] = (c < BM * CPR && rr < rows) ? __float_as_uint(ld_coh4(a.seq_invalid, (uint32_t)(4 * ((row0 + rr) / a.n))))
                                         : 1u;
  }

  f32x4 acc[BM / 16][H2];
#pragma unroll
  for (int i = 0; i < BM / 16; ++i)
#pragma unroll
    for (int h2 = 0; h2 < H2; ++h2) acc[i][h2] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int kb = 0; kb < a.Hm; kb += KT) {
    const int klen = min(KT, a.Hm - kb);
    if (kb > 0) {
#pragma unroll
      for (int h2 = 0; h2 < H2; ++h2)
#pragma unroll
        for (int s = 0; s < KT / 32; ++s) {
          const int kk = 32 * s + 8 * lg;
          bq[h2][s] = (cv[h2] && kk < klen) ? *(const u32x4*)(a.w2 + (int64_t)colv[h2] * a.Hm + kb + kk)
                                            : u32x4{0u, 0u, 0u, 0u};
        }
    }
    // the pass's a chunks are all requested before the first is parked in
    // LDS: one trip to memory per pass instead of one per chunk
    constexpr int ACH = BM * (KT / 8) / 256;  // 16-byte chunks per thread
    static_assert(BM * (KT / 8) % 256 == 0, "whole chunks per thread");
    u32x4 av[ACH];
#pragma unroll
    for (int j = 0; j < ACH; ++j) {
      const int c = tid + 256 * j;
      const int rr = c / (KT / 8), kc = (c - rr * (KT / 8)) * 8;
      av[j] = (rr < rows && kc < klen) ? ld_coh16(a.abuf, (uint32_t)(2 * ((row0 + rr) * a.Hm + kb + kc)))
                                       : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ACH; ++j) {
      const int c = tid + 256 * j;
      const int rr = c / (KT / 8), kc = (c - rr * (KT / 8)) * 8;
      *(u32x4*)&sA[rr * LA + kc] = av[j];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < KT / 32; ++s) {
      if (32 * s < klen) {
#pragma unroll
        for (int i = 0; i < BM / 16; ++i) {
          const u32x4 aop = *(const u32x4*)&sA[(16 * i + lr) * LA + 32 * s + 8 * lg];
#pragma unroll
          for (int h2 = 0; h2 < H2; ++h2) acc[i][h2] = mfma16x16x32(aop, bq[h2][s], acc[i][h2]);
        }
      }
    }
  }

  __syncthreads();
#pragma unroll
  for (int i = 0; i < BM / 16; ++i)
#pragma unroll
    for (int h2 = 0; h2 < H2; ++h2)
#pragma unroll
      for (int e = 0; e < 4; ++e) sO[(16 * i + 4 * lg + e) * LO + WCOL * wave + 16 * h2 + lr] = acc[i][h2][e];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int c = tid + 256 * k;
    const int rr = c / CPR, c8 = (c % CPR) * 8;
    const int row = row0 + rr, gc = col0 + c8;
    if (c >= BM * CPR || rr >= rows || gc >= a.d || inv[k]) continue;
    float dv[8];
    const float4 d0 = *(const float4*)&sO[rr * LO + c8];
    const float4 d1 = *(const float4*)&sO[rr * LO + c8 + 4];
    dv[0] = d0.x; dv[1] = d0.y; dv[2] = d0.z; dv[3] = d0.w;
    dv[4] = d1.x; dv[5] = d1.y; dv[6] = d1.z; dv[7] = d1.w;
    if (a.b2) {
      float bb[8];
      Elem<uint16_t>::unpack(b2q, bb);
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

// Item k of Z queue x.  Queue x holds the K chunks ks = x, x + 8, ... of every
// (row block, column block) tile, row blocks outermost: the first rows' z is
// complete (every column block, every K chunk) before any later row block's
// item is taken, so the state tiles of the first sequences, which wait for
// their rows' z, can start while the Z phase is still running.
template <int BMZ, int NST, bool RSV>
__device__ __forceinline__ void z_run(const FastArgs& a, int x, uint32_t k, unsigned char* smem) {
  const int ncbz = cdiv_d(a.Nz, 64), nk = (a.ksplit - x + 7) >> 3;
  const int per_rb = nk * ncbz;
  const int rb = (int)k / per_rb, rem = (int)k - rb * per_rb;
  const int kk = rem / ncbz, cb = rem - kk * ncbz;
  z_item<BMZ, NST, RSV>(a, x + 8 * kk, cb, rb, smem);
}

// Tile t alone (an orphan group's): gather, statistics and projection, then
// counted.
template <int RR, bool MULTI>
__device__ __forceinline__ void s_single(const FastArgs& a, int t, unsigned char* smem, const int* s_acc,
                                         uint32_t* s_tk) {
  TileRegs<RR> r;
  tile_issue<RR, false, 16>(a, t, r, s_acc);
  tile_process<RR, MULTI, false, 16>(a, t, r, smem, s_tk, NO_ITEM, 0, 0u, 0u, nullptr, s_acc);
  __syncthreads();
}

// Two workgroups of four waves per CU: at most 256 registers per lane.  A
// workgroup takes positions of its XCD's queue (Z items, then the tickets of
// tile group x) until the queue is exhausted, then A items, then O items,
// each kind until its home queue is exhausted (items of queue x share
// operands: K chunks ks % 8 == x, A items j % 8 == x, column blocks
// cb % 8 == x), with the orphan checks described with claim_one before its
// first A item, its first O item and its end.  The first claim and the
// arrival marks ride on the launch's first trip to memory.
template <int RR, int SMALL, int MODE>
__global__ __launch_bounds__(256, (MODE == READY_MODE_PREPARE && RR <= 16) ? 3 : 2) void k_reader(FastArgs a) {
  constexpr int BMZ = SMALL ? 16 : (MODE == READY_MODE_APPLY ? READY_BMZ_APPLY : READY_BMZ_LARGE);
  constexpr int BMO = SMALL ? 16 : (MODE == READY_MODE_APPLY ? READY_BMO_APPLY : READY_BMO_LARGE);
  constexpr int NST = (SMALL ? READY_ZCHUNK_SMALL : READY_ZCHUNK_LARGE) / 128;
  // a prepare launch (several readers sharing one gather) has no Z, A or O
  // items; an apply launch has no state tiles (n_s = 0)
  constexpr bool zao = MODE != READY_MODE_PREPARE;
  constexpr bool has_s = MODE != READY_MODE_APPLY;
  constexpr bool multi = MODE == READY_MODE_PREPARE;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_last;
  __shared__ int s_acc[READY_ACC_LDS];
  __shared__ uint32_t s_tk[3];
  const int tid = item_tid();
  const int g = blockIdx.x, G = gridDim.x;
  const int xcc = hw_xcc();  // the queue of XCD x holds its Z items, then tile group x
  uint32_t first = NO_ITEM;
  if (tid == 0) {
    first = count_up(ctr(a.tk, xcc));
    st_coh_u32(ctr(a.arr_x, xcc), 1u);
  }
  // the accept indices are requested with the magic word, and staged in LDS
  // before the state tiles
  constexpr int APT = READY_ACC_LDS / 256;
  int accv[APT];
#pragma unroll
  for (int k = 0; k < APT; ++k) {
    const int b = tid + 256 * k;
    accv[k] = (MODE != READY_MODE_APPLY && b < a.B) ? a.accept_idx[b] : 0;  // apply launches have none
  }
  if (a.counters[0] != a.magic) {
    // the workspace was not prepared for this plan: touch nothing else (the
    // claim and marks above changed counter words of the workspace only)
    if (g == 0 && tid == 0 && a.dev_status) *a.dev_status = READY_ERR_WORKSPACE_UNINIT;
    return;
  }

  // queue sizes
  const int ztiles = cdiv_d(a.R, BMZ) * cdiv_d(a.Nz, 64);
  constexpr int OCK = SMALL ? READY_OCOLS_SMALL : READY_OCOLS;
  const int ncb = cdiv_d(a.d, OCK), nrbo = cdiv_d(a.R, BMO);
  auto z_size = [&](int x) { return zao ? (uint32_t)(((a.ksplit - x + 7) >> 3) * ztiles) : 0u; };
  auto a_size = [&](int x) { return (uint32_t)((a.n_a - x + 7) >> 3); };
  auto o_size = [&](int x) { return (uint32_t)(nrbo * ((ncb - x + 7) >> 3)); };

  // position p of the home queue is this workgroup's: Z items are run
  // (claiming the next position after each), the first tile position goes
  // to the S phase
  if (tid == 0) s_tk[0] = first;
  __syncthreads();
  uint32_t p = s_tk[0];
  __syncthreads();
  const uint32_t zs = z_size(xcc);
  if constexpr (zao) {
    while (p < zs) {
      z_run<BMZ, NST, RR >= READY_UPATH_MIN_R>(a, xcc, p, smem);
      if (tid == 0) s_tk[0] = count_up(ctr(a.tk, xcc));
      __syncthreads();
      p = s_tk[0];
      __syncthreads();
    }
  }
#pragma unroll
  for (int k = 0; k < APT; ++k) s_acc[tid + 256 * k] = accv[k];
  __syncthreads();
  if constexpr (has_s) s_phase<RR, multi, MODE == READY_MODE_FULL && RR >= READY_UPATH_MIN_R, BMZ>(a, xcc, zs, p, smem, s_acc, s_tk);

  if constexpr (zao) {
    // before the first A item: the arrival flags of the XCDs, read in the
    // trip of the first A claim
    auto flag = [&](int l) { return ctr(a.arr_x, l); };
    uint32_t first;
    const uint32_t orph_x = (uint32_t)arrival_check(ctr(a.aq, xcc), 8, flag, &first, s_tk);
    // orphan XCDs (a partly resident grid only): their Z items and tiles
    for (uint32_t m = orph_x; m != 0; m &= m - 1) {
      const int x = __ffs(m) - 1;
      const uint32_t zsx = z_size(x), qx = zsx + (has_s ? group_tiles(a, x) : 0u);
      for (uint32_t i; (i = claim_one(a.tk, x, qx, s_tk)) != NO_ITEM;) {
        if (i < zsx) {
          z_run<BMZ, NST, RR >= READY_UPATH_MIN_R>(a, x, i, smem);
        } else if constexpr (has_s) {
          s_single<RR, multi>(a, x + READY_TICKET_GROUPS * (int)(i - zsx), smem, s_acc, s_tk);
        }
      }
    }
    // A items in row order from the home queue, then from orphan XCDs' (A
    // item j in queue j % 8); an item is claimed only when the previous one
    // is done, so that no workgroup holds an item it cannot start yet
    for (uint32_t qs = orph_x | (1u << xcc), x = (uint32_t)xcc, i = first; qs != 0;) {
      const uint32_t na = a_size((int)x);
      if (i >= na) {
        qs &= ~(1u << x);
        if (qs == 0) break;
        x = (uint32_t)(__ffs(qs) - 1);
        i = claim_one(a.aq, (int)x, a_size((int)x), s_tk);
        continue;
      }
      mlp1_item<RR, BMZ, BMO, MODE == READY_MODE_FULL && RR >= READY_UPATH_MIN_R>(a, (int)x + 8 * (int)i, smem);
      i = claim_one(a.aq, (int)x, na, s_tk);
    }
    // O items likewise (O item (rb, cb) in queue cb % 8)
    for (uint32_t qs = orph_x | (1u << xcc), x = (uint32_t)xcc, i = claim_one(a.oq, xcc, o_size(xcc), s_tk);
         qs != 0;) {
      const uint32_t no = o_size((int)x);
      if (i >= no) {
        qs &= ~(1u << x);
        if (qs == 0) break;
        x = (uint32_t)(__ffs(qs) - 1);
        i = claim_one(a.oq, (int)x, o_size((int)x), s_tk);
        continue;
      }
      const int ncx = (ncb - (int)x + 7) >> 3;  // column blocks of queue x
      mlp2_item<BMO, OCK>(a, (int)i / ncx, (int)x + 8 * ((int)i % ncx), smem);
      i = claim_one(a.oq, (int)x, no, s_tk);
    }
  } else {
    // a prepare launch, before finishing: tiles of ticket groups no
    // workgroup has arrived in
    auto flag = [&](int l) { return ctr(a.arr_x, l); };
    uint32_t none;
    const uint64_t orph = arrival_check(nullptr, READY_TICKET_GROUPS, flag, &none, s_tk);
    for (uint64_t m = orph; m != 0; m &= m - 1) {
      const int q = __ffsll((unsigned long long)m) - 1;
      for (uint32_t i; (i = claim_one(a.tk, q, group_tiles(a, q), s_tk)) != NO_ITEM;)
        s_single<RR, multi>(a, q + READY_TICKET_GROUPS * (int)i, smem, s_acc, s_tk);
    }
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

__global__ void k_ws_init(uint32_t* counters, int n, uint32_t magic) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    counters[i] = (i == 0) ? magic : 0u;
}

// ---------------------------------------------------------------- launchers

hipError_t ready_launch_reader(const FastArgs& a, int small, int grid, hipStream_t s, StageEvents ev) {
  // the query items walk their K chunk in the stages the variant is built for
  if (a.kchunk != (small ? READY_ZCHUNK_SMALL : READY_ZCHUNK_LARGE)) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), block(256);
  const size_t lds = ready_reader_lds(a.r, a.F, a.Nz, small);
#define READY_READER_MODE(RRV, SM)                                                          \
  do {                                                                                      \
    if (a.mode == READY_MODE_PREPARE)                                                       \
      READY_LAUNCH((k_reader<RRV, SM, READY_MODE_PREPARE>), g, block, lds, s, ev, a);       \
    else if (a.mode == READY_MODE_APPLY)                                                    \
      READY_LAUNCH((k_reader<RRV, SM, READY_MODE_APPLY>), g, block, lds, s, ev, a);         \
    else                                                                                    \
      READY_LAUNCH((k_reader<RRV, SM, READY_MODE_FULL>), g, block, lds, s, ev, a);          \
  } while (0)
#define READY_READER_CASE(RRV)             \
  do {                                     \
    if (small) READY_READER_MODE(RRV, 1);  \
    else READY_READER_MODE(RRV, 0);        \
  } while (0)
  switch (a.r) {
    case 8: READY_READER_CASE(8); break;
    case 16: READY_READER_CASE(16); break;
    case 24: READY_READER_CASE(24); break;
    default: READY_READER_CASE(32); break;
  }
#undef READY_READER_CASE
#undef READY_READER_MODE
  return hipGetLastError();
}

// Workgroups of k_reader in launch mode `mode` that one CU holds at once (0 on
// error).
int ready_reader_per_cu(int r, int small, size_t lds, int mode) {
  int nb = 1 << 20;
  hipError_t e = hipSuccess;
#define READY_OCC_ONE(KERNEL)                                                     \
  do {                                                                            \
    int n1 = 0;                                                                   \
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n1, KERNEL, 256, lds); \
    nb = n1 < nb ? n1 : nb;                                                       \
  } while (0)
#define READY_OCC_SM(RRV, SM)                                                               \
  do {                                                                                      \
    if (mode == READY_MODE_PREPARE) READY_OCC_ONE((k_reader<RRV, SM, READY_MODE_PREPARE>)); \
    else if (mode == READY_MODE_APPLY) READY_OCC_ONE((k_reader<RRV, SM, READY_MODE_APPLY>)); \
    else READY_OCC_ONE((k_reader<RRV, SM, READY_MODE_FULL>));                               \
  } while (0)
#define READY_OCC_CASE(RRV)            \
  do {                                 \
    if (small) READY_OCC_SM(RRV, 1);   \
    else READY_OCC_SM(RRV, 0);         \
  } while (0)
  switch (r) {
    case 8: READY_OCC_CASE(8); break;
    case 16: READY_OCC_CASE(16); break;
    case 24: READY_OCC_CASE(24); break;
    default: READY_OCC_CASE(32); break;
  }
#undef READY_OCC_CASE
#undef READY_OCC_SM
#undef READY_OCC_ONE
  return e == hipSuccess ? nb : 0;
}

hipError_t ready_launch_ws_init(uint32_t* counters, int n_counters, uint32_t magic, hipStream_t s) {
  hipLaunchKernelGGL(k_ws_init, dim3((unsigned)((n_counters + 255) / 256)), dim3(256), 0, s, counters, n_counters,
                     magic);
  return hipGetLastError();
}
