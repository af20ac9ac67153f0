// Host side of the ready.h C ABI: argument validation, the plan (kernel
// choices and workspace layout) and the launch sequence.
//
// Two launch sequences, both on the caller's stream:
//
// fast (bf16 states, activations and weights, r <= 32, F and Hm multiples of
// 8): one persistent launch, k_reader (query sums, state tiles, f and the
// first MLP layer, the second MLP layer and the residual as work items of one
// grid that the GPU holds at once)
// general (any other dtype mix or rank):
//   0. query GEMM (split-K partial sums of z and of the squares of h)
//   1. k_state    gather, RMS, log-RMS, T = V^T S_bar, q = U^T z,
//                 u = T q / sqrt(d_k), packing into f (VALU); for bf16
//                 states and weights k_state_mm, the same on the matrix
//                 cores in the order u = V^T (S_bar q) / sqrt(d_k)
//   2. MLP layer 1
//   3. MLP layer 2 and residual
//   Each GEMM runs on the matrix cores when the weights are bf16 and the rows
//   are 16-byte aligned, on the VALU otherwise.
//
// Validation never touches the HIP runtime, so every argument error can be
// exercised on a machine without a GPU.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <new>

#include "ready_internal.h"

struct GemmPlan {
  int mfma;      // matrix-core kernel
  int big;       // matrix-core kernel with 128 x 128 tiles (k_gemm_mm)
  int bm;        // rows per tile (matrix-core kernel)
  int ksplit;    // K splits (query GEMM only)
  int kchunk;
};

struct readyPlan {
  readyShape s;
  int32_t slot[READY_MAX_LSEL];
  int M, F, R, Mz, Nz;
  int fast;
  int f32;       // fp32 single-launch path (k_reader_f32)
  int small;     // fast path: at most 16 rows (16-row tiles; 64 otherwise)
  int n_z, n_s, n_a, n_o, n_counters;
  int c_zcnt, c_zdone, c_sdone, c_adone, c_tk, c_aq, c_oq, c_arx;  // first counter slot of each group
  size_t lds;
  GemmPlan gz, g1, g2;
  size_t off_zpart, off_hss, off_rsv, off_f, off_fu, off_a, off_g1p, off_flags, off_pmat, off_ell, off_ctr, ws_bytes;
};

namespace {

size_t dsize(int dt) { return dt == READY_BF16 ? 2 : 4; }
bool dtype_ok(int dt) { return dt == READY_F32 || dt == READY_BF16; }
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
  bool empty() const { return hi <= lo; }
};
Range range_of(const void* p, size_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(const Range& a, const Range& b) {
  return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

readyStatus validate_shape(const readyShape& s, const int32_t* layer_ids) {
  if (!dtype_ok(s.state_dtype) || !dtype_ok(s.act_dtype) || !dtype_ok(s.weight_dtype))
    return READY_ERR_UNSUPPORTED_DTYPE;
  if (s.act != READY_ACT_SILU && s.act != READY_ACT_GELU_TANH && s.act != READY_ACT_RELU)
    return READY_ERR_UNSUPPORTED_DTYPE;
  if (s.B < 0 || s.P < 1 || s.P > 64 || s.n < 1 || s.n > 16) return READY_ERR_BAD_SHAPE;
  if ((int64_t)s.B * s.n > (1 << 20)) return READY_ERR_BAD_SHAPE;
  if (s.L_sel < 1 || s.L_sel > READY_MAX_LSEL || s.L_tot < 1 || s.H < 1) return READY_ERR_BAD_SHAPE;
  if ((int64_t)s.L_sel * s.H > 4096) return READY_ERR_BAD_SHAPE;
  if (s.d_k != READY_TILE || s.d_v != READY_TILE) return READY_ERR_BAD_SHAPE;
  if (s.r < 8 || s.r > 128 || s.r % 8 != 0) return READY_ERR_BAD_SHAPE;
  if (s.d < 8 || s.d % 8 != 0 || s.Hm < 1 || s.Hm > 4096) return READY_ERR_BAD_SHAPE;
  if (s.shared_params != 0 && s.shared_params != 1) return READY_ERR_BAD_SHAPE;
  if (s.path != READY_PATH_FUSED && s.path != READY_PATH_UNFUSED) return READY_ERR_BAD_SHAPE;
  if (!(s.state_eps >= 0.0f) || !(s.h_eps >= 0.0f)) return READY_ERR_BAD_SHAPE;
  for (int l = 0; l < s.L_sel; ++l)
    if (layer_ids[l] < 0 || layer_ids[l] >= s.L_tot) return READY_ERR_LAYER_ID_RANGE;
  return READY_OK;
}

}  // namespace

extern "C" {

int32_t readyVersion(void) { return READY_VERSION; }

const char* readyStatusString(readyStatus st) {
  switch (static_cast<int>(st)) {
    case READY_OK: return "READY_OK";
    case READY_ERR_NULL_POINTER: return "READY_ERR_NULL_POINTER";
    case READY_ERR_BAD_SHAPE: return "READY_ERR_BAD_SHAPE";
    case READY_ERR_UNSUPPORTED_DTYPE: return "READY_ERR_UNSUPPORTED_DTYPE";
    case READY_ERR_MISALIGNED: return "READY_ERR_MISALIGNED";
    case READY_ERR_WORKSPACE_TOO_SMALL: return "READY_ERR_WORKSPACE_TOO_SMALL";
    case READY_ERR_ALIASING: return "READY_ERR_ALIASING";
    case READY_ERR_LAYER_ID_RANGE: return "READY_ERR_LAYER_ID_RANGE";
    case READY_ERR_HIP: return "READY_ERR_HIP";
    case READY_ERR_ACCEPT_IDX: return "READY_ERR_ACCEPT_IDX";
    case READY_ERR_OUT_OF_HOST_MEMORY: return "READY_ERR_OUT_OF_HOST_MEMORY";
    case READY_ERR_SYNC_TIMEOUT: return "READY_ERR_SYNC_TIMEOUT";
    case READY_ERR_WORKSPACE_UNINIT: return "READY_ERR_WORKSPACE_UNINIT";
    case READY_ERR_UNSUPPORTED: return "READY_ERR_UNSUPPORTED";
    case READY_ERR_STATIC_SCRATCH_TOO_SMALL: return "READY_ERR_STATIC_SCRATCH_TOO_SMALL";
  }
  return "READY_ERR_UNKNOWN";
}

readyStatus readyPlanCreate(const readyShape* shape, const int32_t* layer_ids, readyPlan** plan) {
  if (!shape || !layer_ids || !plan) return READY_ERR_NULL_POINTER;
  *plan = nullptr;
  const readyShape& s = *shape;
  if (s.L_sel < 1 || s.L_sel > READY_MAX_LSEL) return READY_ERR_BAD_SHAPE;
  readyStatus st = validate_shape(s, layer_ids);
  if (st != READY_OK) return st;
  readyPlan* p = new (std::nothrow) readyPlan;
  if (!p) return READY_ERR_OUT_OF_HOST_MEMORY;
  memset(p, 0, sizeof(*p));
  p->s = s;
  for (int l = 0; l < s.L_sel; ++l) p->slot[l] = layer_ids[l];
  p->M = s.L_sel * s.H;
  p->F = p->M * (s.r + 1);
  p->R = s.B * s.n;
  p->Mz = s.shared_params ? 1 : p->M;
  p->Nz = p->Mz * s.r;

  const bool wbf = s.weight_dtype == READY_BF16;
  const bool allbf = wbf && s.state_dtype == READY_BF16 && s.act_dtype == READY_BF16;
  // (the fast path addresses z partial sums, P and a with 32-bit byte offsets)
  const int64_t zchunk = p->R <= 16 ? READY_ZCHUNK_SMALL : READY_ZCHUNK_LARGE;
  const int64_t fks = cdiv(s.d, zchunk);
  const bool small_ws = (int64_t)s.B * p->M * s.r * s.r * 4 < (1LL << 31) &&
                        (int64_t)p->R * s.Hm * 2 < (1LL << 31) &&
                        fks * p->R * p->Nz * 4 < (1LL << 31) &&
                        (int64_t)p->R * ((p->F + 31) & ~31) * 4 < (1LL << 31);
  p->small = p->R <= 16 ? 1 : 0;
  bool fits = allbf && s.r <= 32 && p->F % 8 == 0 && p->F <= READY_FAST_MAX_F && s.Hm % 8 == 0 &&
                    p->Nz <= READY_FAST_MAX_NZ && small_ws;
  {
    // per-XCD queue lengths: Z items and state tiles (one queue), O items
    // (the A items are fewer)
    const int64_t bmz = p->small ? 16 : std::min(READY_BMZ_LARGE, READY_BMZ_APPLY);
    const int64_t bmo = p->small ? 16 : std::min(READY_BMO_LARGE, READY_BMO_APPLY);
    const int64_t rows = std::max(p->R, 1);
    const int64_t zq = cdiv(fks, 8) * cdiv(rows, bmz) * cdiv(p->Nz, 64) + cdiv((int64_t)s.B * p->M, 8);
    const int64_t oq = cdiv(rows, bmo) * cdiv(cdiv(s.d, p->small ? READY_OCOLS_SMALL : READY_OCOLS), 8);
    if (zq >= (1 << 24) || oq >= (1 << 24)) fits = false;
  }
  p->lds = fits ? ready_reader_lds(s.r, p->F, p->Nz, p->small) : 0;
  p->fast = (fits && p->lds <= 80 * 1024 && s.path == READY_PATH_FUSED) ? 1 : 0;  // two workgroups per CU
  {
    // fp32 states, activations and weights at serving sizes: k_reader_f32
    // (its byte offsets into W_q, W1, W2, h and the partial sums of z are
    // 32-bit)
    const bool allf = s.state_dtype == READY_F32 && s.act_dtype == READY_F32 && s.weight_dtype == READY_F32;
    const int64_t R = p->R, nks = cdiv(s.d, READY_F32_KC);
    const bool ok = allf && s.path == READY_PATH_FUSED && R >= 1 && R <= 16 && (s.r == 8 || s.r == 16) &&
                    s.Hm % 4 == 0 && s.Hm <= READY_F32_MAX_HM && p->F <= READY_F32_MAX_F &&
                    R * p->Nz <= READY_F32_MAX_RNZ && (int64_t)s.B * p->M * s.r <= READY_F32_MAX_UNITS &&
                    (int64_t)p->Nz * s.d * 4 < (1LL << 31) && nks * R * p->Nz * 4 < (1LL << 31) &&
                    (int64_t)s.d * s.Hm * 4 < (1LL << 31) && (int64_t)s.Hm * p->F * 4 < (1LL << 31) &&
                    R * s.d * 4 < (1LL << 31) && ready_f32_lds(s.r, p->R, p->Nz, p->F, s.Hm) <= READY_F32_MAX_LDS;
    p->f32 = ok ? 1 : 0;
  }

  if (p->fast) {
    // work items of k_reader
    // the counters per row block of z and of out are sized for the finer of
    // the two large-row forms (apply launches use READY_BMZ_APPLY and
    // READY_BMO_APPLY)
    const int bmz = p->small ? 16 : std::min(READY_BMZ_LARGE, READY_BMZ_APPLY);
    const int bmo = p->small ? 16 : std::min(READY_BMO_LARGE, READY_BMO_APPLY);
    const int64_t rows = std::max(p->R, 1);
    const int64_t nrbz = cdiv(rows, bmz), ncbz = cdiv(p->Nz, 64), nrba = cdiv(rows, READY_ABM), nrbo = cdiv(rows, bmo);
    p->gz.ksplit = (int)fks;
    p->gz.kchunk = (int)zchunk;
    p->n_z = (int)(nrbz * ncbz * fks);
    // each per-XCD queue holds fewer than 2^24 items (checked above)
    p->n_s = s.B * p->M;
    p->n_a = (int)(nrba * cdiv(s.Hm, 64));
    p->n_o = (int)(nrbo * cdiv(s.d, p->small ? READY_OCOLS_SMALL : READY_OCOLS));
    // counter slots: magic, abort, READY_DONE_GROUPS + 1 done counts, then
    // per tile of z, per row block of z, per 16 rows, per row block of out
    p->c_zcnt = 2 + READY_DONE_GROUPS + 1;
    p->c_zdone = (int)(p->c_zcnt + nrbz * ncbz);
    p->c_sdone = (int)(p->c_zdone + nrbz);
    p->c_adone = (int)(p->c_sdone + nrba);
    p->c_tk = (int)(p->c_adone + nrbo);
    p->c_aq = p->c_tk + READY_TICKET_GROUPS;
    p->c_oq = p->c_aq + 8;
    p->c_arx = p->c_oq + 8;
    p->n_counters = (int)(READY_CTR_STRIDE * (p->c_arx + 8));
  } else if (p->f32) {
    // work items of k_reader_f32, and its counters: magic, abort,
    // READY_DONE_GROUPS + 1 done counts, READY_F32_QUEUES claim counters each
    // of the S and Z items, of the A items and of the O items and as many
    // arrival flags, the column
    // blocks of z done, the S items done, the A items done, the Z items done
    // per column block
    const int64_t nks = cdiv(s.d, READY_F32_KC), ncz = cdiv(p->Nz, READY_F32_ZC);
    p->gz.ksplit = (int)nks;
    p->gz.kchunk = READY_F32_KC;
    p->n_s = s.B * p->M;
    p->n_z = (int)(ncz * nks);
    p->n_a = (int)cdiv(s.Hm, READY_F32_AC);
    p->n_o = (int)cdiv(s.d, READY_F32_OC);
    p->lds = ready_f32_lds(s.r, p->R, p->Nz, p->F, s.Hm);
    p->c_tk = 2 + READY_DONE_GROUPS + 1;
    p->c_aq = p->c_tk + READY_F32_QUEUES;
    p->c_oq = p->c_aq + READY_F32_QUEUES;
    p->c_arx = p->c_oq + READY_F32_QUEUES;
    p->c_zdone = p->c_arx + READY_F32_QUEUES;
    p->c_sdone = p->c_zdone + 1;
    p->c_adone = p->c_sdone + 1;
    p->c_zcnt = p->c_adone + 1;
    p->n_counters = (int)(READY_CTR_STRIDE * (p->c_zcnt + ncz));
  } else {
    // query GEMM: matrix cores for bf16 h and weights; K split so that about
    // 256 (matrix cores) or 512 (VALU) workgroups run
    p->gz.mfma = (wbf && s.act_dtype == READY_BF16) ? 1 : 0;
    p->gz.big = (p->gz.mfma && p->R >= 2 * READY_GM_TILE) ? 1 : 0;
    if (p->gz.big) {
      const int64_t tiles = cdiv(p->Nz, READY_GM_TILE) * cdiv(p->R, READY_GM_TILE);
      int64_t ks = std::max<int64_t>(1, cdiv(256, tiles));
      ks = std::min<int64_t>(ks, cdiv(s.d, 8 * READY_GM_BK));
      const int64_t kchunk = align_up((size_t)cdiv(s.d, ks), READY_GM_BK);
      p->gz.kchunk = (int)kchunk;
      p->gz.ksplit = (int)cdiv(s.d, kchunk);
    } else if (p->gz.mfma) {
      p->gz.bm = p->R <= 16 ? 16 : 64;
      const int64_t tiles = cdiv(p->Nz, READY_MFMA_BN) * cdiv(std::max(p->R, 1), p->gz.bm);
      int64_t ks = std::max<int64_t>(1, cdiv(256, tiles));
      ks = std::min<int64_t>(ks, cdiv(s.d, READY_MFMA_BK));
      const int64_t kchunk = align_up((size_t)cdiv(s.d, ks), READY_MFMA_BK);
      p->gz.kchunk = (int)kchunk;
      p->gz.ksplit = (int)cdiv(s.d, kchunk);
    } else {
      const int64_t tiles = cdiv(p->Nz, READY_GEMM_COLS) * cdiv(std::max(p->R, 1), READY_GEMM_RB);
      int64_t ks = std::max<int64_t>(1, cdiv(512, tiles));
      ks = std::min<int64_t>(ks, cdiv(s.d, 128));
      const int64_t kchunk = align_up((size_t)cdiv(s.d, ks), 128);
      p->gz.kchunk = (int)kchunk;
      p->gz.ksplit = (int)cdiv(s.d, kchunk);
    }
    // MLP layers: f and a are fp32 rows of F and Hm values
    p->g1.mfma = (wbf && p->F % 8 == 0) ? 1 : 0;
    p->g1.bm = p->R <= 16 ? 16 : 64;
    p->g1.ksplit = 1;
    p->g1.kchunk = p->F;
    p->g1.big = (p->g1.mfma && p->R >= 2 * READY_GM_TILE) ? 1 : 0;
    if (p->g1.big) {
      // few output tiles (Hm columns): split K, then sum, bias and activation
      const int64_t tiles = cdiv(s.Hm, READY_GM_TILE) * cdiv(p->R, READY_GM_TILE);
      int64_t ks = std::max<int64_t>(1, cdiv(256, tiles));
      ks = std::min<int64_t>(ks, cdiv(p->F, 8 * READY_GM_BK));
      const int64_t kchunk = align_up((size_t)cdiv(p->F, ks), READY_GM_BK);
      p->g1.kchunk = (int)kchunk;
      p->g1.ksplit = (int)cdiv(p->F, kchunk);
    }
    p->g2.mfma = (wbf && s.Hm % 8 == 0) ? 1 : 0;
    // 128 x 128 tiles only when there is at least one per CU (no K split
    // here); else the 64-row kernel gives more workgroups
    p->g2.big = (p->g2.mfma && p->R >= 2 * READY_GM_TILE &&
                 cdiv(s.d, READY_GM_TILE) * cdiv(p->R, READY_GM_TILE) >= 256) ? 1 : 0;
    p->g2.bm = p->R <= 16 ? 16 : 64;
    p->g2.ksplit = 1;
    p->g2.kchunk = s.Hm;
  }

  const size_t R = (size_t)p->R;
  const size_t BM = (size_t)s.B * p->M;
  const size_t ks = (size_t)p->gz.ksplit;
  size_t off = 0;
  p->off_zpart = off; off = align_up(off + 4 * ks * R * p->Nz, 256);
  p->off_hss = off;   off = align_up(off + 4 * ks * R * (p->f32 ? (size_t)cdiv(p->Nz, READY_F32_ZC) : 1), 256);
  p->off_rsv = off;   off = align_up(off + (p->fast ? 4 * R : 0), 256);
  // f on the general path, z summed over the K chunks on the fast path
  p->off_f = off;     off = align_up(off + (p->f32 ? 0 : 4 * R * (p->fast ? p->Nz : p->F)), 256);
  p->off_fu = off;
  off = align_up(off + (p->fast ? 4 * R * (size_t)((p->F + 31) & ~31) : p->f32 ? 4 * R * (size_t)((p->F + 63) & ~63) : 0),
                 256);
  // a: bf16 on the fast path, fp32 otherwise
  p->off_a = off;     off = align_up(off + (p->fast ? 2 : 4) * R * s.Hm, 256);
  // K-split partial sums of the first MLP layer (k_gemm_mm with ksplit > 1)
  p->off_g1p = off;   off = align_up(off + (p->g1.ksplit > 1 ? 4 * (size_t)p->g1.ksplit * R * s.Hm : 0), 256);
  p->off_flags = off; off = align_up(off + 4 * (size_t)std::max(s.B, 1), 256);
  p->off_pmat = off;  off = align_up(off + (p->fast || p->f32 ? 4 * BM * s.r * s.r : 0), 256);
  p->off_ell = off;   off = align_up(off + (p->fast || p->f32 ? 4 * BM : 0), 256);
  p->off_ctr = off;   off = align_up(off + 4 * (size_t)p->n_counters, 256);
  p->ws_bytes = off;
  *plan = p;
  return READY_OK;
}

readyStatus readyPlanDestroy(readyPlan* plan) {
  delete plan;
  return READY_OK;
}

readyStatus readyWorkspaceSize(const readyPlan* plan, size_t* bytes) {
  if (!plan || !bytes) return READY_ERR_NULL_POINTER;
  *bytes = plan->ws_bytes;
  return READY_OK;
}

readyStatus readyPlanLaunches(const readyPlan* plan, int32_t* launches) {
  if (!plan || !launches) return READY_ERR_NULL_POINTER;
  if (plan->fast || plan->f32) *launches = 1;
  else *launches = (plan->g1.big && plan->g1.ksplit > 1) ? 5 : 4;
  return READY_OK;
}

namespace {

StageEvents stage_events(void* const* events, int i) {
  StageEvents ev{nullptr, nullptr};
  if (events) {
    ev.start = (hipEvent_t)events[2 * i];
    ev.stop = (hipEvent_t)events[2 * i + 1];
  }
  return ev;
}

// The scratch of a call held in a caller's workspace: the arrays at the
// plan's offsets, the counters at off_ctr, stamped with the plan's magic word.
WsView workspace_view(const readyPlan* plan, void* workspace) {
  WsView v;
  v.data = (char*)workspace;
  v.ctr = (uint32_t*)((char*)workspace + plan->off_ctr);
  v.magic = READY_WS_MAGIC ^ (uint32_t)plan->n_counters;
  v.data_bytes = plan->off_ctr;
  v.ctr_bytes = plan->ws_bytes - plan->off_ctr;
  return v;
}

// FastArgs fields that depend only on the plan and the scratch: sizes,
// work-item counts, scratch arrays and counters.  One reader (n_inj = 1),
// every item kind (READY_MODE_FULL).
void fast_common(const readyPlan* plan, const WsView& view, FastArgs& a) {
  char* wsb = view.data;
  const readyShape& s = plan->s;
  memset(&a, 0, sizeof(a));
  for (int l = 0; l < s.L_sel; ++l) a.slot[l] = plan->slot[l];
  a.zpart = (float*)(wsb + plan->off_zpart);
  a.hss = (float*)(wsb + plan->off_hss);
  a.rsv = (float*)(wsb + plan->off_rsv);
  a.zfin = (float*)(wsb + plan->off_f);
  a.fu = (float*)(wsb + plan->off_fu);
  a.pmat = (float*)(wsb + plan->off_pmat);
  a.ell = (float*)(wsb + plan->off_ell);
  a.abuf = (uint16_t*)(wsb + plan->off_a);
  a.seq_invalid = (uint32_t*)(wsb + plan->off_flags);
  uint32_t* ctr = view.ctr;
  a.counters = ctr; a.n_counters = plan->n_counters;
  a.magic = view.magic;
  a.abort_flag = ctr + READY_CTR_STRIDE;
  a.done = ctr + 2 * READY_CTR_STRIDE;
  a.zcnt = ctr + READY_CTR_STRIDE * plan->c_zcnt;
  a.zdone = ctr + READY_CTR_STRIDE * plan->c_zdone;
  a.sdone = ctr + READY_CTR_STRIDE * plan->c_sdone;
  a.adone = ctr + READY_CTR_STRIDE * plan->c_adone;
  a.tk = ctr + READY_CTR_STRIDE * plan->c_tk;
  a.arr_x = ctr + READY_CTR_STRIDE * plan->c_arx;
  a.aq = ctr + READY_CTR_STRIDE * plan->c_aq;
  a.oq = ctr + READY_CTR_STRIDE * plan->c_oq;
  a.n_z = plan->n_z; a.n_s = plan->n_s; a.n_a = plan->n_a; a.n_o = plan->n_o;
  a.B = s.B; a.P = s.P; a.n = s.n; a.M = plan->M; a.H = s.H; a.r = s.r; a.d = s.d; a.F = plan->F;
  a.Hm = s.Hm; a.R = plan->R; a.Nz = plan->Nz; a.shared = s.shared_params;
  a.ksplit = plan->gz.ksplit; a.kchunk = plan->gz.kchunk; a.act = s.act;
  a.state_eps = s.state_eps; a.h_eps = s.h_eps;
  a.mode = READY_MODE_FULL;
  a.n_inj = 1;
}

// Launch k_reader with the grid the GPU holds at once (every wait in the
// kernel is for a workgroup that is already running).
readyStatus launch_fast(const readyPlan* plan, FastArgs& a, hipStream_t strm, void* const* events) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return READY_ERR_HIP;
  // prepare launches (state tiles only, no waits between workgroups) take a
  // third workgroup per CU for more tiles in flight where registers allow
  // (r <= 16)
  const int cap = (a.mode == READY_MODE_PREPARE && plan->s.r <= 16) ? 3 : 2;
  const int per_cu = std::min(cap, ready_reader_per_cu(plan->s.r, plan->small, plan->lds, a.mode));
  if (per_cu < 1 || cus < 1) return READY_ERR_HIP;
  // a one-reader launch of at most 16 rows has few items (the paper shape:
  // 56 query items and 32 tiles): one workgroup per CU, or one per query
  // item and tile where there are more, so that fewer idle workgroups
  // contend for the claim counters (B = 1: 23.0 -> 21.6 us cold; 128 or
  // 192 workgroups gave the same)
  int grid = per_cu * cus;
  if (plan->small && a.mode == READY_MODE_FULL)
    grid = std::min(grid, std::max(cus, plan->n_z + plan->n_s));
  if (ready_launch_reader(a, plan->small, grid, strm, stage_events(events, 1)) != hipSuccess)
    return READY_ERR_HIP;
  // the other stages run inside the same kernel: their marks (if any) are
  // recorded together after it
  for (int i = 0; events && i < 2 * READY_STAGES; ++i)
    if ((i < 2 || i > 3) && events[i] && hipEventRecord((hipEvent_t)events[i], strm) != hipSuccess)
      return READY_ERR_HIP;
  return READY_OK;
}

// Layout of the prepared-state buffer of several readers: P of every reader
// [n_inj][B M][r][r] fp32, then ell [B M] fp32, then the invalid-sequence
// flags [B] uint32, each section 256-byte aligned.
struct PrepLayout {
  size_t off_p, off_ell, off_flags, bytes;
  int64_t p_stride;  // floats per reader
};
PrepLayout prep_layout(const readyPlan* plan, int n_inj) {
  PrepLayout L;
  const size_t BM = (size_t)plan->s.B * plan->M;
  L.p_stride = (int64_t)BM * plan->s.r * plan->s.r;
  L.off_p = 0;
  L.off_ell = align_up(4 * (size_t)n_inj * (size_t)L.p_stride, 256);
  L.off_flags = align_up(L.off_ell + 4 * BM, 256);
  L.bytes = align_up(L.off_flags + 4 * (size_t)std::max(plan->s.B, 1), 256);
  return L;
}

}  // namespace

// `sv` is the scratch when the library supplies it (the static per-device
// array); with sv == nullptr the caller's workspace is checked and used.
readyStatus ready_run_reader(const readyPlan* plan, const readyStates* states, const int32_t* accept_idx,
                             const void* h, const readyWeights* w, const readyOutputs* o, void* workspace,
                             size_t workspace_bytes, void* stream, void* const* events, const WsView* sv,
                             WsResolve resolve) {
  if (!plan || !states || !w || !o) return READY_ERR_NULL_POINTER;
  const readyShape& s = plan->s;
  if (!states->base || !accept_idx || !h || !w->wq || !w->u || !w->v || !w->w1 || !w->w2 ||
      !o->gathered || !o->out || (!sv && !workspace))
    return READY_ERR_NULL_POINTER;
  if (!sv && workspace_bytes < plan->ws_bytes) return READY_ERR_WORKSPACE_TOO_SMALL;
  WsView view = sv ? *sv : workspace_view(plan, workspace);

  const size_t ss = dsize(s.state_dtype), as = dsize(s.act_dtype), ws = dsize(s.weight_dtype);
  // alignment: 16 bytes for everything read or written with vector accesses
  const void* vec_ptrs[] = {states->base, h, w->wq, w->u, w->v, w->h_gamma, w->w1, w->w2, w->b2,
                            o->gathered, o->out, o->delta, o->feat};
  for (const void* ptr : vec_ptrs)
    if (ptr && !aligned16(ptr)) return READY_ERR_MISALIGNED;
  if (!sv && ((uintptr_t)workspace & 255u) != 0) return READY_ERR_MISALIGNED;
  const int64_t strides[4] = {states->stride_b, states->stride_p, states->stride_l, states->stride_h};
  for (int64_t st : strides) {
    if (st < 0) return READY_ERR_BAD_SHAPE;
    if ((st * (int64_t)ss) % 16 != 0) return READY_ERR_MISALIGNED;
  }

  // address ranges for the aliasing rules
  const size_t M = plan->M, R = plan->R, F = plan->F, Hm = s.Hm, d = s.d;
  const int64_t span = s.B == 0 ? 0 :
                       (int64_t)(s.B - 1) * states->stride_b + (int64_t)(s.P - 1) * states->stride_p +
                       (int64_t)(s.L_tot - 1) * states->stride_l + (int64_t)(s.H - 1) * states->stride_h +
                       READY_TILE_ELEMS;
  const Range r_states = range_of(states->base, (size_t)span * ss);
  const Range r_gath = range_of(o->gathered, (size_t)s.B * M * READY_TILE_ELEMS * ss);
  const Range r_h = range_of(h, R * d * as);
  const Range r_out = range_of(o->out, R * d * as);
  const Range r_ws = range_of(view.data, view.data_bytes);
  const Range r_ctr = range_of(view.ctr, view.ctr_bytes);
  const Range r_acc = range_of(accept_idx, (size_t)s.B * 4);
  const size_t mz = s.shared_params ? 1 : M;
  const Range inputs[] = {
      r_states, r_acc,
      range_of(w->wq, mz * s.r * d * ws), range_of(w->u, mz * s.r * READY_TILE * ws),
      range_of(w->v, mz * READY_TILE * s.r * ws), range_of(w->h_gamma, w->h_gamma ? d * ws : 0),
      range_of(w->w1, Hm * F * ws), range_of(w->b1, w->b1 ? Hm * ws : 0),
      range_of(w->w2, d * Hm * ws), range_of(w->b2, w->b2 ? d * ws : 0)};
  const Range outputs[] = {r_gath, r_out, range_of(o->logrms, o->logrms ? (size_t)s.B * M * 4 : 0),
                           range_of(o->delta, o->delta ? R * d * 4 : 0),
                           range_of(o->feat, o->feat ? R * F * 4 : 0),
                           range_of(o->dev_status, o->dev_status ? 4 : 0), r_ws, r_ctr};
  const int n_out = (int)(sizeof(outputs) / sizeof(outputs[0]));
  for (int i = 0; i < n_out; ++i) {
    for (const Range& in : inputs)
      if (overlap(outputs[i], in)) return READY_ERR_ALIASING;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outputs[i], outputs[j])) return READY_ERR_ALIASING;
  }
  // out may be h itself (in place); any other overlap with h is an error
  if (o->out != h && overlap(r_out, r_h)) return READY_ERR_ALIASING;
  for (int i = 0; i < n_out; ++i)
    if (i != 1 && overlap(outputs[i], r_h)) return READY_ERR_ALIASING;

  if (s.B == 0) return READY_OK;

  hipStream_t strm = (hipStream_t)stream;
  if (resolve) {
    const readyStatus rs = resolve(&view, strm);
    if (rs != READY_OK) return rs;
  }
  char* wsb = view.data;
  float* zpart = (float*)(wsb + plan->off_zpart);
  float* hss = (float*)(wsb + plan->off_hss);
  float* fbuf = (float*)(wsb + plan->off_f);
  float* abuf = (float*)(wsb + plan->off_a);
  int32_t* flags = (int32_t*)(wsb + plan->off_flags);

  if (plan->fast) {
    FastArgs a;
    fast_common(plan, view, a);
    a.states = (const uint16_t*)states->base;
    a.sb = states->stride_b; a.sp = states->stride_p; a.sl = states->stride_l; a.sh = states->stride_h;
    a.accept_idx = accept_idx;
    a.h = (const uint16_t*)h;
    a.wq = (const uint16_t*)w->wq; a.u = (const uint16_t*)w->u; a.v = (const uint16_t*)w->v;
    a.gamma = (const uint16_t*)w->h_gamma;
    a.w1 = (const uint16_t*)w->w1; a.b1 = (const uint16_t*)w->b1;
    a.w2 = (const uint16_t*)w->w2; a.b2 = (const uint16_t*)w->b2;
    a.gathered = (uint16_t*)o->gathered; a.out = (uint16_t*)o->out;
    a.logrms = o->logrms; a.delta = o->delta; a.feat = o->feat; a.dev_status = o->dev_status;
    a.u_inj[0] = a.u; a.v_inj[0] = a.v;
    return launch_fast(plan, a, strm, events);
  }

  if (plan->f32) {
    F32Args a;
    memset(&a, 0, sizeof(a));
    a.states = (const float*)states->base;
    a.sb = states->stride_b; a.sp = states->stride_p; a.sl = states->stride_l; a.sh = states->stride_h;
    a.accept_idx = accept_idx;
    for (int l = 0; l < s.L_sel; ++l) a.slot[l] = plan->slot[l];
    a.h = (const float*)h;
    a.wq = (const float*)w->wq; a.u = (const float*)w->u; a.v = (const float*)w->v;
    a.gamma = (const float*)w->h_gamma;
    a.w1 = (const float*)w->w1; a.b1 = (const float*)w->b1;
    a.w2 = (const float*)w->w2; a.b2 = (const float*)w->b2;
    a.gathered = (float*)o->gathered; a.out = (float*)o->out;
    a.logrms = o->logrms; a.delta = o->delta; a.feat = o->feat; a.dev_status = o->dev_status;
    a.zpart = zpart; a.hss = hss;
    a.fbuf = (float*)(wsb + plan->off_fu);
    a.pmat = (float*)(wsb + plan->off_pmat);
    a.ell = (float*)(wsb + plan->off_ell);
    a.abuf = abuf;
    a.seq_invalid = (uint32_t*)flags;
    uint32_t* ctr = view.ctr;
    a.counters = ctr; a.n_counters = plan->n_counters; a.magic = view.magic;
    a.abort_flag = ctr + READY_CTR_STRIDE;
    a.done = ctr + 2 * READY_CTR_STRIDE;
    a.lq = ctr + READY_CTR_STRIDE * plan->c_tk;
    a.aq = ctr + READY_CTR_STRIDE * plan->c_aq;
    a.oq = ctr + READY_CTR_STRIDE * plan->c_oq;
    a.arr_x = ctr + READY_CTR_STRIDE * plan->c_arx;
    a.zdone = ctr + READY_CTR_STRIDE * plan->c_zdone;
    a.sdone = ctr + READY_CTR_STRIDE * plan->c_sdone;
    a.adone = ctr + READY_CTR_STRIDE * plan->c_adone;
    a.zcnt = ctr + READY_CTR_STRIDE * plan->c_zcnt;
    a.n_s = plan->n_s; a.n_z = plan->n_z; a.n_a = plan->n_a; a.n_o = plan->n_o;
    a.nks = plan->gz.ksplit; a.ncz = (int)cdiv(plan->Nz, READY_F32_ZC);
    {
      // z of all rows in at most 256 chunks of 16 bytes, each summed by
      // 256 / nq threads over at most READY_F32_ZSUM_LOADS K chunks apiece
      const int nq = plan->R * plan->Nz / 4;
      a.zsum_a = (nq <= 256 && a.nks <= 64 && a.nks <= READY_F32_ZSUM_LOADS * (256 / nq)) ? 1 : 0;
    }
    a.B = s.B; a.P = s.P; a.n = s.n; a.M = plan->M; a.H = s.H; a.r = s.r; a.d = s.d; a.F = plan->F;
    a.Hm = s.Hm; a.R = plan->R; a.Nz = plan->Nz; a.shared = s.shared_params; a.act = s.act;
    a.state_eps = s.state_eps; a.h_eps = s.h_eps;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return READY_ERR_HIP;
    // one and a half workgroups per CU whatever the item count: at the
    // serving sizes every S and Z item then finds a workgroup that has not
    // run another first, and the spare ones find their queues empty and
    // finish (wide: 46.6 -> 45.9 us cold against two per CU, 51.0 at one,
    // 48.9 at five quarters; tiny the same at 384 and 512)
    const int grid = (int)(3 * (int64_t)cus / 2);
    if (ready_launch_reader_f32(a, grid, plan->lds, strm, stage_events(events, 1)) != hipSuccess) return READY_ERR_HIP;
    // the other stages run inside the same kernel: their marks (if any) are
    // recorded together after it
    for (int i = 0; events && i < 2 * READY_STAGES; ++i)
      if ((i < 2 || i > 3) && events[i] && hipEventRecord((hipEvent_t)events[i], strm) != hipSuccess)
        return READY_ERR_HIP;
    return READY_OK;
  }

  const int wvw = (int)(16 / ws);
  // 0. z partials and sums of squares of h
  {
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.X = h; g.ldx = d; g.W = w->wq; g.ldw = d;
    g.R = (int)R; g.N = plan->Nz; g.K = (int)d; g.kchunk = plan->gz.kchunk;
    g.vec_ok = (d % wvw == 0) && (plan->gz.kchunk % wvw == 0);
    g.gamma = w->h_gamma; g.hss = hss; g.ypart = zpart;
    hipError_t e;
    const StageEvents ev = stage_events(events, 0);
    if (plan->gz.big) {
      e = ready_launch_gemm_mm(g, s.act_dtype, s.act_dtype, EPI_PARTIAL, plan->gz.ksplit, strm, ev);
    } else if (plan->gz.mfma) {
      const dim3 grid((unsigned)cdiv(plan->Nz, READY_MFMA_BN), (unsigned)plan->gz.ksplit,
                      (unsigned)cdiv(R, plan->gz.bm));
      e = ready_launch_gemm_mfma(g, s.act_dtype, s.act_dtype, EPI_PARTIAL, plan->gz.bm, grid, strm, ev);
    } else {
      const dim3 grid((unsigned)cdiv(plan->Nz, READY_GEMM_COLS), (unsigned)plan->gz.ksplit,
                      (unsigned)cdiv(R, READY_GEMM_RB));
      const size_t lds = 4 * READY_GEMM_RB * (size_t)std::min(plan->gz.kchunk, READY_GEMM_KSTAGE);
      e = ready_launch_gemm(g, s.act_dtype, s.weight_dtype, s.act_dtype, EPI_PARTIAL, grid, lds, strm, ev);
    }
    if (e != hipSuccess) return READY_ERR_HIP;
  }
  // 1. per-state work
  {
    StateArgs a;
    memset(&a, 0, sizeof(a));
    a.states = states->base;
    a.sb = states->stride_b; a.sp = states->stride_p; a.sl = states->stride_l; a.sh = states->stride_h;
    a.accept_idx = accept_idx;
    for (int l = 0; l < s.L_sel; ++l) a.slot[l] = plan->slot[l];
    a.B = s.B; a.P = s.P; a.n = s.n; a.M = (int)M; a.H = s.H; a.r = s.r; a.d = (int)d; a.F = (int)F;
    a.shared = s.shared_params; a.state_eps = s.state_eps; a.h_eps = s.h_eps;
    a.u = w->u; a.v = w->v;
    a.gathered = o->gathered; a.logrms = o->logrms;
    a.dev_status = o->dev_status; a.seq_invalid = flags;
    a.zpart = zpart; a.hss = hss; a.ksz = plan->gz.ksplit; a.nz = plan->Nz;
    a.f = fbuf; a.feat = o->feat;
    if (s.state_dtype == READY_BF16 && s.weight_dtype == READY_BF16) {
      // matrix-core form: one persistent workgroup per CU walking the tiles
      int dev = 0, cus = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return READY_ERR_HIP;
      const int grid = (int)std::min<int64_t>((int64_t)s.B * M, cus);
      if (ready_launch_state_mm(a, grid, strm, stage_events(events, 1)) != hipSuccess) return READY_ERR_HIP;
    } else if (ready_launch_state(a, s.state_dtype, s.weight_dtype, strm, stage_events(events, 1)) != hipSuccess) {
      return READY_ERR_HIP;
    }
  }
  // 2. a = act(W1 f + b1)
  {
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.X = fbuf; g.ldx = F; g.W = w->w1; g.ldw = F;
    g.R = (int)R; g.N = (int)Hm; g.K = (int)F; g.kchunk = (int)F;
    g.vec_ok = (F % wvw == 0);
    g.bias = w->b1; g.act = s.act; g.yout = abuf;
    hipError_t e;
    const StageEvents ev = stage_events(events, 2);
    if (plan->g1.big && plan->g1.ksplit > 1) {
      g.kchunk = plan->g1.kchunk;
      g.ypart = (float*)(wsb + plan->off_g1p);
      e = ready_launch_gemm_mm(g, READY_F32, s.act_dtype, EPI_PARTIAL, plan->g1.ksplit, strm,
                               StageEvents{ev.start, nullptr});
      if (e == hipSuccess) e = ready_launch_reduce_bias_act(g, plan->g1.ksplit, strm, StageEvents{nullptr, ev.stop});
    } else if (plan->g1.big) {
      e = ready_launch_gemm_mm(g, READY_F32, s.act_dtype, EPI_BIAS_ACT, 1, strm, ev);
    } else if (plan->g1.mfma) {
      const dim3 grid((unsigned)cdiv(Hm, READY_MFMA_BN), 1u, (unsigned)cdiv(R, plan->g1.bm));
      e = ready_launch_gemm_mfma(g, READY_F32, s.act_dtype, EPI_BIAS_ACT, plan->g1.bm, grid, strm, ev);
    } else {
      // too few workgroups for the GPU: four columns per workgroup, K split over its waves
      g.wave_k = cdiv(Hm, READY_GEMM_COLS) * cdiv(R, READY_GEMM_RB) < 128 ? 1 : 0;
      const dim3 grid((unsigned)cdiv(Hm, g.wave_k ? 4 : READY_GEMM_COLS), 1u, (unsigned)cdiv(R, READY_GEMM_RB));
      const size_t lds = 4 * READY_GEMM_RB * (size_t)std::min((int)F, READY_GEMM_KSTAGE);
      e = ready_launch_gemm(g, READY_F32, s.weight_dtype, s.act_dtype, EPI_BIAS_ACT, grid, lds, strm, ev);
    }
    if (e != hipSuccess) return READY_ERR_HIP;
  }
  // 3. out = h + W2 a + b2
  {
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.X = abuf; g.ldx = Hm; g.W = w->w2; g.ldw = Hm;
    g.R = (int)R; g.N = (int)d; g.K = (int)Hm; g.kchunk = (int)Hm;
    g.vec_ok = (Hm % wvw == 0);
    g.bias = w->b2; g.h = h; g.out = o->out; g.delta = o->delta; g.seq_invalid = flags; g.n = s.n;
    auto a16 = [](const void* q) { return ((uintptr_t)q & 15u) == 0u; };
    g.epi_vec = (d % 8 == 0 && a16(h) && a16(o->out) && a16(o->delta)) ? 1 : 0;
    hipError_t e;
    const StageEvents ev = stage_events(events, 3);
    if (plan->g2.big) {
      e = ready_launch_gemm_mm(g, READY_F32, s.act_dtype, EPI_RESID, 1, strm, ev);
    } else if (plan->g2.mfma) {
      const dim3 grid((unsigned)cdiv(d, READY_MFMA_BN), 1u, (unsigned)cdiv(R, plan->g2.bm));
      e = ready_launch_gemm_mfma(g, READY_F32, s.act_dtype, EPI_RESID, plan->g2.bm, grid, strm, ev);
    } else {
      g.wave_k = cdiv(d, READY_GEMM_COLS) * cdiv(R, READY_GEMM_RB) < 128 ? 1 : 0;
      const dim3 grid((unsigned)cdiv(d, g.wave_k ? 4 : READY_GEMM_COLS), 1u, (unsigned)cdiv(R, READY_GEMM_RB));
      const size_t lds = 4 * READY_GEMM_RB * (size_t)std::min((int)Hm, READY_GEMM_KSTAGE);
      e = ready_launch_gemm(g, READY_F32, s.weight_dtype, s.act_dtype, EPI_RESID, grid, lds, strm, ev);
    }
    if (e != hipSuccess) return READY_ERR_HIP;
  }
  return READY_OK;
}

void ready_plan_scratch_needs(const readyPlan* plan, size_t* data_bytes, size_t* ctr_bytes) {
  *data_bytes = plan->off_ctr;
  *ctr_bytes = plan->ws_bytes - plan->off_ctr;
}

readyStatus readyVerifyStates(int32_t B, int32_t P, int32_t L, int32_t H, int32_t state_dtype, int32_t kv_dtype,
                              const void* state_t, const void* k, const void* v, const float* alpha,
                              const float* beta, const readyVerifyBuffer* out, void* stream) {
  if (!out) return READY_ERR_NULL_POINTER;
  if (B < 0 || P < 1 || P > 64 || L < 1 || H < 1 || (int64_t)L * H > 4096) return READY_ERR_BAD_SHAPE;
  if (!dtype_ok(state_dtype) || !dtype_ok(kv_dtype)) return READY_ERR_UNSUPPORTED_DTYPE;
  if (B == 0) return READY_OK;
  if (!state_t || !out->base) return READY_ERR_NULL_POINTER;
  if (P > 1 && (!k || !v || !alpha || !beta)) return READY_ERR_NULL_POINTER;
  const void* vec_ptrs[] = {state_t, out->base, P > 1 ? k : nullptr, P > 1 ? v : nullptr};
  for (const void* ptr : vec_ptrs)
    if (ptr && !aligned16(ptr)) return READY_ERR_MISALIGNED;
  const size_t ss = dsize(state_dtype), ks = dsize(kv_dtype);
  const int64_t strides[4] = {out->stride_b, out->stride_p, out->stride_l, out->stride_h};
  for (int64_t st : strides) {
    if (st < 0) return READY_ERR_BAD_SHAPE;
    if ((st * (int64_t)ss) % 16 != 0) return READY_ERR_MISALIGNED;
  }
  const int64_t M = (int64_t)L * H, steps = P - 1;
  const int64_t span = (int64_t)(B - 1) * out->stride_b + (int64_t)(P - 1) * out->stride_p +
                       (int64_t)(L - 1) * out->stride_l + (int64_t)(H - 1) * out->stride_h + READY_TILE_ELEMS;
  const Range r_out = range_of(out->base, (size_t)span * ss);
  const Range inputs[] = {range_of(state_t, (size_t)B * M * READY_TILE_ELEMS * ss),
                          range_of(k, steps ? (size_t)B * steps * M * READY_TILE * ks : 0),
                          range_of(v, steps ? (size_t)B * steps * M * READY_TILE * ks : 0),
                          range_of(alpha, steps ? (size_t)B * steps * M * 4 : 0),
                          range_of(beta, steps ? (size_t)B * steps * M * 4 : 0)};
  for (const Range& in : inputs)
    if (overlap(r_out, in)) return READY_ERR_ALIASING;
  if ((int64_t)B * M > 0x7fffffff) return READY_ERR_BAD_SHAPE;

  VerifyArgs a;
  memset(&a, 0, sizeof(a));
  a.state_t = state_t; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.out = out->base;
  a.sb = out->stride_b; a.sp = out->stride_p; a.sl = out->stride_l; a.sh = out->stride_h;
  a.B = B; a.P = P; a.M = (int)M; a.H = H;
  return ready_launch_verify(a, state_dtype, kv_dtype, (hipStream_t)stream) == hipSuccess ? READY_OK : READY_ERR_HIP;
}

readyStatus readyWorkspaceInit(const readyPlan* plan, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan || !workspace) return READY_ERR_NULL_POINTER;
  if (((uintptr_t)workspace & 255u) != 0) return READY_ERR_MISALIGNED;
  if (workspace_bytes < plan->ws_bytes) return READY_ERR_WORKSPACE_TOO_SMALL;
  if ((!plan->fast && !plan->f32) || plan->n_counters == 0) return READY_OK;  // the general path keeps no counters
  uint32_t* ctr = (uint32_t*)((char*)workspace + plan->off_ctr);
  if (ready_launch_ws_init(ctr, plan->n_counters, READY_WS_MAGIC ^ (uint32_t)plan->n_counters,
                           (hipStream_t)stream) != hipSuccess)
    return READY_ERR_HIP;
  return READY_OK;
}

readyStatus readyStateReader(const readyPlan* plan, const readyStates* states,
                             const int32_t* accept_idx, const void* h,
                             const readyWeights* w, const readyOutputs* o,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return ready_run_reader(plan, states, accept_idx, h, w, o, workspace, workspace_bytes, stream, nullptr, nullptr, nullptr);
}

readyStatus readyStateReaderProfiled(const readyPlan* plan, const readyStates* states,
                                     const int32_t* accept_idx, const void* h,
                                     const readyWeights* w, const readyOutputs* o,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     void* const* events) {
  return ready_run_reader(plan, states, accept_idx, h, w, o, workspace, workspace_bytes, stream, events, nullptr, nullptr);
}

// ---------------------------------------------------------------- step 1 alone

readyStatus readyGather(const readyPlan* plan, const readyStates* states, const int32_t* accept_idx, void* gathered,
                        int32_t* dev_status, void* stream) {
  if (!plan || !states) return READY_ERR_NULL_POINTER;
  const readyShape& s = plan->s;
  if (s.B == 0) return READY_OK;
  if (!states->base || !accept_idx || !gathered) return READY_ERR_NULL_POINTER;
  const size_t ss = dsize(s.state_dtype);
  if (!aligned16(states->base) || !aligned16(gathered)) return READY_ERR_MISALIGNED;
  const int64_t strides[4] = {states->stride_b, states->stride_p, states->stride_l, states->stride_h};
  for (int64_t st : strides) {
    if (st < 0) return READY_ERR_BAD_SHAPE;
    if ((st * (int64_t)ss) % 16 != 0) return READY_ERR_MISALIGNED;
  }
  const size_t M = plan->M;
  const int64_t span = (int64_t)(s.B - 1) * states->stride_b + (int64_t)(s.P - 1) * states->stride_p +
                       (int64_t)(s.L_tot - 1) * states->stride_l + (int64_t)(s.H - 1) * states->stride_h +
                       READY_TILE_ELEMS;
  const Range r_states = range_of(states->base, (size_t)span * ss);
  const Range r_acc = range_of(accept_idx, (size_t)s.B * 4);
  const Range r_gath = range_of(gathered, (size_t)s.B * M * READY_TILE_ELEMS * ss);
  const Range r_st = range_of(dev_status, dev_status ? 4 : 0);
  if (overlap(r_gath, r_states) || overlap(r_gath, r_acc) || overlap(r_gath, r_st) || overlap(r_st, r_states) ||
      overlap(r_st, r_acc))
    return READY_ERR_ALIASING;
  GatherArgs a;
  memset(&a, 0, sizeof(a));
  a.states = states->base;
  a.sb = states->stride_b; a.sp = states->stride_p; a.sl = states->stride_l; a.sh = states->stride_h;
  a.accept_idx = accept_idx;
  for (int l = 0; l < s.L_sel; ++l) a.slot[l] = plan->slot[l];
  a.B = s.B; a.P = s.P; a.M = (int)M; a.H = s.H; a.esize = (int)ss;
  a.gathered = gathered; a.dev_status = dev_status;
  return ready_launch_gather(a, (hipStream_t)stream) == hipSuccess ? READY_OK : READY_ERR_HIP;
}

// ---------------------------------------------------------------- several readers sharing one gather

readyStatus readyPrepSize(const readyPlan* plan, int32_t n_inj, size_t* bytes) {
  if (!plan || !bytes) return READY_ERR_NULL_POINTER;
  if (!plan->fast) return READY_ERR_UNSUPPORTED;
  if (n_inj < 1 || n_inj > READY_MAX_INJ) return READY_ERR_BAD_SHAPE;
  *bytes = prep_layout(plan, n_inj).bytes;
  return READY_OK;
}

readyStatus readyStatePrepare(const readyPlan* plan, const readyStates* states, const int32_t* accept_idx,
                              int32_t n_inj, const readyWeights* inj_weights, void* gathered, float* logrms,
                              int32_t* dev_status, void* prep, size_t prep_bytes, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!plan || !states || !inj_weights) return READY_ERR_NULL_POINTER;
  if (!plan->fast) return READY_ERR_UNSUPPORTED;
  if (n_inj < 1 || n_inj > READY_MAX_INJ) return READY_ERR_BAD_SHAPE;
  const readyShape& s = plan->s;
  if (!states->base || !accept_idx || !gathered || !prep || !workspace) return READY_ERR_NULL_POINTER;
  for (int i = 0; i < n_inj; ++i)
    if (!inj_weights[i].u || !inj_weights[i].v) return READY_ERR_NULL_POINTER;
  const PrepLayout L = prep_layout(plan, n_inj);
  if (workspace_bytes < plan->ws_bytes || prep_bytes < L.bytes) return READY_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(states->base) || !aligned16(gathered)) return READY_ERR_MISALIGNED;
  for (int i = 0; i < n_inj; ++i)
    if (!aligned16(inj_weights[i].u) || !aligned16(inj_weights[i].v)) return READY_ERR_MISALIGNED;
  if (((uintptr_t)workspace & 255u) != 0 || ((uintptr_t)prep & 255u) != 0) return READY_ERR_MISALIGNED;
  const int64_t strides[4] = {states->stride_b, states->stride_p, states->stride_l, states->stride_h};
  for (int64_t st : strides) {
    if (st < 0) return READY_ERR_BAD_SHAPE;
    if ((st * 2) % 16 != 0) return READY_ERR_MISALIGNED;
  }
  const size_t M = plan->M, mz = s.shared_params ? 1 : M;
  const int64_t span = s.B == 0 ? 0 :
                       (int64_t)(s.B - 1) * states->stride_b + (int64_t)(s.P - 1) * states->stride_p +
                       (int64_t)(s.L_tot - 1) * states->stride_l + (int64_t)(s.H - 1) * states->stride_h +
                       READY_TILE_ELEMS;
  Range inputs[2 + 2 * READY_MAX_INJ];  // (no host allocation on the call path)
  int n_in = 0;
  inputs[n_in++] = range_of(states->base, (size_t)span * 2);
  inputs[n_in++] = range_of(accept_idx, (size_t)s.B * 4);
  for (int i = 0; i < n_inj; ++i) {
    inputs[n_in++] = range_of(inj_weights[i].u, mz * s.r * READY_TILE * 2);
    inputs[n_in++] = range_of(inj_weights[i].v, mz * READY_TILE * s.r * 2);
  }
  const Range outputs[] = {range_of(gathered, (size_t)s.B * M * READY_TILE_ELEMS * 2),
                           range_of(logrms, logrms ? (size_t)s.B * M * 4 : 0),
                           range_of(dev_status, dev_status ? 4 : 0), range_of(prep, L.bytes),
                           range_of(workspace, plan->ws_bytes)};
  const int n_out = (int)(sizeof(outputs) / sizeof(outputs[0]));
  for (int i = 0; i < n_out; ++i) {
    for (int k = 0; k < n_in; ++k)
      if (overlap(outputs[i], inputs[k])) return READY_ERR_ALIASING;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outputs[i], outputs[j])) return READY_ERR_ALIASING;
  }
  if (s.B == 0) return READY_OK;

  char* pb = (char*)prep;
  FastArgs a;
  fast_common(plan, workspace_view(plan, workspace), a);
  a.mode = READY_MODE_PREPARE;
  a.n_inj = n_inj;
  a.states = (const uint16_t*)states->base;
  a.sb = states->stride_b; a.sp = states->stride_p; a.sl = states->stride_l; a.sh = states->stride_h;
  a.accept_idx = accept_idx;
  for (int i = 0; i < n_inj; ++i) {
    a.u_inj[i] = (const uint16_t*)inj_weights[i].u;
    a.v_inj[i] = (const uint16_t*)inj_weights[i].v;
  }
  a.u = a.u_inj[0]; a.v = a.v_inj[0];
  a.gathered = (uint16_t*)gathered; a.logrms = logrms; a.dev_status = dev_status;
  a.pmat = (float*)(pb + L.off_p); a.p_inj_stride = L.p_stride;
  a.ell = (float*)(pb + L.off_ell);
  a.seq_invalid = (uint32_t*)(pb + L.off_flags);
  return launch_fast(plan, a, (hipStream_t)stream, nullptr);
}

readyStatus readyStateApply(const readyPlan* plan, const void* prep, size_t prep_bytes, int32_t n_inj, int32_t inj,
                            const void* h, const readyWeights* w, const readyOutputs* o, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!plan || !w || !o) return READY_ERR_NULL_POINTER;
  if (!plan->fast) return READY_ERR_UNSUPPORTED;
  if (n_inj < 1 || n_inj > READY_MAX_INJ || inj < 0 || inj >= n_inj) return READY_ERR_BAD_SHAPE;
  const readyShape& s = plan->s;
  if (!prep || !h || !w->wq || !w->w1 || !w->w2 || !o->out || !workspace) return READY_ERR_NULL_POINTER;
  const PrepLayout L = prep_layout(plan, n_inj);
  if (workspace_bytes < plan->ws_bytes || prep_bytes < L.bytes) return READY_ERR_WORKSPACE_TOO_SMALL;
  const void* vec_ptrs[] = {h, w->wq, w->h_gamma, w->w1, w->w2, w->b2, o->out, o->delta, o->feat};
  for (const void* ptr : vec_ptrs)
    if (ptr && !aligned16(ptr)) return READY_ERR_MISALIGNED;
  if (((uintptr_t)workspace & 255u) != 0 || ((uintptr_t)prep & 255u) != 0) return READY_ERR_MISALIGNED;
  const size_t M = plan->M, R = plan->R, F = plan->F, Hm = s.Hm, d = s.d, mz = s.shared_params ? 1 : M;
  const Range r_h = range_of(h, R * d * 2), r_out = range_of(o->out, R * d * 2);
  const Range inputs[] = {range_of(prep, L.bytes), range_of(w->wq, mz * s.r * d * 2),
                          range_of(w->h_gamma, w->h_gamma ? d * 2 : 0), range_of(w->w1, Hm * F * 2),
                          range_of(w->b1, w->b1 ? Hm * 2 : 0), range_of(w->w2, d * Hm * 2),
                          range_of(w->b2, w->b2 ? d * 2 : 0)};
  const Range outputs[] = {r_out, range_of(o->delta, o->delta ? R * d * 4 : 0),
                           range_of(o->feat, o->feat ? R * F * 4 : 0),
                           range_of(o->dev_status, o->dev_status ? 4 : 0), range_of(workspace, plan->ws_bytes)};
  const int n_out = (int)(sizeof(outputs) / sizeof(outputs[0]));
  for (int i = 0; i < n_out; ++i) {
    for (const Range& in : inputs)
      if (overlap(outputs[i], in)) return READY_ERR_ALIASING;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outputs[i], outputs[j])) return READY_ERR_ALIASING;
    if (i != 0 && overlap(outputs[i], r_h)) return READY_ERR_ALIASING;
  }
  // out may be h itself (in place); any other overlap with h is an error
  if (o->out != h && overlap(r_out, r_h)) return READY_ERR_ALIASING;
  if (s.B == 0) return READY_OK;

  const char* pb = (const char*)prep;
  FastArgs a;
  fast_common(plan, workspace_view(plan, workspace), a);
  a.mode = READY_MODE_APPLY;
  a.n_s = 0;  // no state tiles: P, ell and the flags come from the prepare launch
  a.h = (const uint16_t*)h;
  a.wq = (const uint16_t*)w->wq; a.gamma = (const uint16_t*)w->h_gamma;
  a.w1 = (const uint16_t*)w->w1; a.b1 = (const uint16_t*)w->b1;
  a.w2 = (const uint16_t*)w->w2; a.b2 = (const uint16_t*)w->b2;
  a.out = (uint16_t*)o->out; a.delta = o->delta; a.feat = o->feat; a.dev_status = o->dev_status;
  a.pmat = (float*)(pb + L.off_p) + (int64_t)inj * L.p_stride;
  a.ell = (float*)(pb + L.off_ell);
  a.seq_invalid = (uint32_t*)(pb + L.off_flags);
  return launch_fast(plan, a, (hipStream_t)stream, nullptr);
}

}  // extern "C"
