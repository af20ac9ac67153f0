// Verify-state producer for gfx950: the per-position Gated DeltaNet states of
// one verify block, written into the verify buffer the state reader gathers
// from.  For each sequence b and layer-head pair m:
//   S_{t+0} = S_t
//   S_{t+p} = alpha_p S_{t+p-1} + beta_p (v_p - alpha_p S_{t+p-1} k_p) k_p^T
// which is S_{t+p-1} A_p + B_p with A_p = alpha_p (I - beta_p k_p k_p^T) and
// B_p = beta_p v_p k_p^T (ReaDy arXiv text, Appendix D.1, the gated delta
// rule; section 3.1 "Drafting, verification, and commitment" for the
// per-position states of the verify step; Proposition 2 in Appendix A.2
// writes the same states as S_t P_j + W_j).
//
//   k_verify_states  one workgroup per (sequence, pair).  Thread t keeps rows
//                    t / 16 + 16 i (i < 8) and key columns 8 (t % 16) .. + 7
//                    of the fp32 state in registers, so every load and store
//                    moves whole 256-byte rows (16 lanes per row).  S k is a
//                    partial dot product per thread and a reduction over the
//                    16 lanes of a row; the rank-one update needs no exchange.
//                    The block's k, v, alpha and beta are staged in LDS once.
//                    The chain runs in fp32; each state is rounded to the
//                    state dtype (nearest even for bf16) only when stored, and
//                    position 0 is a bit copy of S_t.
#include "ready_common.h"

namespace {

// 8 consecutive values of a row as fp32, from a bf16 or fp32 array
__device__ __forceinline__ void load_row8(const uint16_t* p, float* x, u32x4 (&raw)[2]) {
  raw[0] = __builtin_nontemporal_load((const u32x4*)p);
  Elem<uint16_t>::unpack(raw[0], x);
}
__device__ __forceinline__ void load_row8(const float* p, float* x, u32x4 (&raw)[2]) {
  raw[0] = __builtin_nontemporal_load((const u32x4*)p);
  raw[1] = __builtin_nontemporal_load((const u32x4*)p + 1);
  Elem<float>::unpack(raw[0], x);
  Elem<float>::unpack(raw[1], x + 4);
}
__device__ __forceinline__ void store_raw8(uint16_t* p, const u32x4 (&raw)[2]) {
  __builtin_nontemporal_store(raw[0], (u32x4*)p);
}
__device__ __forceinline__ void store_raw8(float* p, const u32x4 (&raw)[2]) {
  __builtin_nontemporal_store(raw[0], (u32x4*)p);
  __builtin_nontemporal_store(raw[1], (u32x4*)p + 1);
}
__device__ __forceinline__ void store_row8(uint16_t* p, const float* x) {
  __builtin_nontemporal_store(pack_bf16x8(x), (u32x4*)p);
}
__device__ __forceinline__ void store_row8(float* p, const float* x) {
  __builtin_nontemporal_store(u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                                    __float_as_uint(x[3])},
                              (u32x4*)p);
  __builtin_nontemporal_store(u32x4{__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]),
                                    __float_as_uint(x[7])},
                              (u32x4*)p + 1);
}

}  // namespace

template <typename TS, typename TKV>
__global__ __launch_bounds__(256) void k_verify_states(VerifyArgs a) {
  extern __shared__ float sv[];  // k [P-1][128], v [P-1][128], alpha [P-1], beta [P-1]
  const int tile = blockIdx.x;
  const int b = tile / a.M, m = tile - (tile / a.M) * a.M;
  const int l = m / a.H, hh = m - (m / a.H) * a.H;
  const int tid = threadIdx.x;
  const int c8 = tid & 15, rg = tid >> 4;
  const int steps = a.P - 1;
  float* sk = sv;
  float* svv = sv + steps * READY_TILE;
  float* sa = sv + 2 * steps * READY_TILE;
  float* sb = sa + steps;

  // the block's inputs: step p uses k[b][p-1][m], v[b][p-1][m], alpha, beta
  // (in batches of 8 loads in flight; a clamped index stands in past the end)
  const int nkv = 2 * steps * READY_TILE;
  for (int e0 = tid; e0 < nkv; e0 += 8 * 256) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = min(e0 + 256 * u, nkv - 1);
      const int which = e / (steps * READY_TILE), rest = e - which * steps * READY_TILE;
      const int p = rest >> 7, c = rest & 127;
      const int64_t off = (((int64_t)b * steps + p) * a.M + m) * READY_TILE + c;
      x[u] = Elem<TKV>::ld(which == 0 ? a.k : a.v, off);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (e0 + 256 * u < nkv) sv[e0 + 256 * u] = x[u];
  }
  for (int e = tid; e < 2 * steps; e += 256) {
    const int p = e < steps ? e : e - steps;
    const int64_t off = ((int64_t)b * steps + p) * a.M + m;
    sa[e] = e < steps ? a.alpha[off] : a.beta[off];
  }

  // S_t into registers; position 0 is its bit copy
  const TS* src = (const TS*)a.state_t + (int64_t)tile * READY_TILE_ELEMS;
  TS* dst0 = (TS*)a.out + (int64_t)b * a.sb + (int64_t)l * a.sl + (int64_t)hh * a.sh;
  float s[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int v = rg + 16 * i;
    u32x4 raw[2];
    load_row8(src + v * READY_TILE + 8 * c8, s[i], raw);
    store_raw8(dst0 + v * READY_TILE + 8 * c8, raw);
  }
  __syncthreads();

  for (int p = 1; p <= steps; ++p) {
    const float* kp = sk + (p - 1) * READY_TILE;
    const float* vp = svv + (p - 1) * READY_TILE;
    const float alpha = sa[p - 1], beta = sb[p - 1];
    float kv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) kv[e] = kp[8 * c8 + e];
    // (S k)_v over this thread's 8 columns, then over the 16 lanes of the row
    float dot[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += s[i][e] * kv[e];
      dot[i] = acc;
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int i = 0; i < 8; ++i) dot[i] += __shfl_xor(dot[i], off, 64);
    TS* dst = dst0 + (int64_t)p * a.sp;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int v = rg + 16 * i;
      // S <- alpha S + beta (v - alpha S k) k^T
      const float w = beta * (vp[v] - alpha * dot[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[i][e] = alpha * s[i][e] + w * kv[e];
      store_row8(dst + v * READY_TILE + 8 * c8, s[i]);
    }
  }
}

size_t ready_verify_lds(int P) { return (size_t)(P - 1) * (2 * READY_TILE + 2) * sizeof(float); }

hipError_t ready_launch_verify(const VerifyArgs& a, int state_dt, int kv_dt, hipStream_t s) {
  const dim3 grid((unsigned)(a.B * a.M)), block(256);
  const size_t lds = ready_verify_lds(a.P);
  const StageEvents ev{nullptr, nullptr};
  if (state_dt == READY_BF16 && kv_dt == READY_BF16)
    READY_LAUNCH((k_verify_states<uint16_t, uint16_t>), grid, block, lds, s, ev, a);
  else if (state_dt == READY_BF16)
    READY_LAUNCH((k_verify_states<uint16_t, float>), grid, block, lds, s, ev, a);
  else if (kv_dt == READY_BF16)
    READY_LAUNCH((k_verify_states<float, uint16_t>), grid, block, lds, s, ev, a);
  else
    READY_LAUNCH((k_verify_states<float, float>), grid, block, lds, s, ev, a);
  return hipGetLastError();
}
