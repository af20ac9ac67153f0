// Step 1 on its own for gfx950: the fused gather of each sequence's committed
// state at its accept index into a caller-preallocated buffer (ReaDy arXiv
// text, section 3.2 "Avoiding redundant data movement": selected committed
// states are written straight into a preallocated execution buffer, with no
// intermediate tensor; section 3.1 "Drafting, verification, and commitment":
// only the states of committed tokens are kept).  The state reader runs the
// same copy fused with the later steps; this form serves callers that want
// the committed states alone, and times the pages' gather operator.
//
//   k_gather  one workgroup per (sequence, pair) tile.  Thread i moves the
//             16-byte chunks i + 256 j of the tile, so every wave
//             instruction reads and writes four (bf16) or two (fp32) whole
//             rows; all of a thread's loads are issued before its stores.
//             An accept index outside [0, P) stores READY_ERR_ACCEPT_IDX in
//             the status word and leaves the tile unwritten.
#include "ready_common.h"

template <int CPT>  // 16-byte chunks per thread: 8 (bf16 tile) or 16 (fp32 tile)
__global__ __launch_bounds__(256) void k_gather(GatherArgs a) {
  const int t = blockIdx.x;
  const int b = t / a.M, m = t - (t / a.M) * a.M;
  const int p = a.accept_idx[b];
  if (p < 0 || p >= a.P) {
    if (threadIdx.x == 0 && a.dev_status) *a.dev_status = READY_ERR_ACCEPT_IDX;
    return;
  }
  const int l = m / a.H, hh = m - (m / a.H) * a.H;
  const int64_t elem = b * a.sb + p * a.sp + a.slot[l] * a.sl + hh * a.sh;
  const u32x4* src = (const u32x4*)((const char*)a.states + elem * a.esize);
  u32x4* dst = (u32x4*)((char*)a.gathered + (int64_t)t * (CPT * 256 * 16));
  u32x4 v[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) v[j] = __builtin_nontemporal_load(src + threadIdx.x + 256 * j);
#pragma unroll
  for (int j = 0; j < CPT; ++j) __builtin_nontemporal_store(v[j], dst + threadIdx.x + 256 * j);
}

hipError_t ready_launch_gather(const GatherArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.B * a.M)), block(256);
  if (a.esize == 2)
    hipLaunchKernelGGL(k_gather<8>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(k_gather<16>, grid, block, 0, s, a);
  return hipGetLastError();
}
