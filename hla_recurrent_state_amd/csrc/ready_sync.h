// Device helpers for work items that hand data to one another inside one
// launch: device-coherent loads and stores (sc1), the counters that announce
// the data, bounded waits on them, and the XCD of the running wave.
//
// Data a workgroup hands to another is written with device-coherent stores,
// made complete with a wait on the memory counter (wait_mem), and announced
// by a relaxed device-scope atomic increment; the reader polls the counter
// and loads the data with device-coherent loads.  (No release or acquire
// fence: on this GPU an agent-scope release writes back the whole L2 of the
// XCD.)
#pragma once

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
__device__ __forceinline__ float ld_coh4(const void* base, uint32_t byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(base), byte_off, 0, SC1));
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
// The value is in registers here: a load producing it may not be sunk past
// this point (into a later trip).
__device__ __forceinline__ void pin(u32x4& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }
// Loads for a trip of many: always issued; when `live` is false the offset
// lies past the descriptor's record count, so the load returns zero and
// moves no data.  A branch around a load, or a use of the value right after
// it, makes the compiler wait for the load there and splits the trip.
constexpr uint32_t DEAD_OFF = 0x80000000u;  // past 0x7fffffff records, with room for an immediate offset
__device__ __forceinline__ u32x4 ld_coh16_at(bool live, const void* base, uint32_t byte_off) {
  return ld_coh16(base, live ? byte_off : DEAD_OFF);
}
__device__ __forceinline__ float ld_coh4_at(bool live, const void* base, uint32_t byte_off) {
  return ld_coh4(base, live ? byte_off : DEAD_OFF);
}
// The thread index, as a value the compiler cannot match with other reads
// of it: the work items derive their lane offsets from their own copy, so
// those are recomputed per item instead of held (and spilled) across the
// whole kernel.
__device__ __forceinline__ int item_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}
__device__ __forceinline__ uint32_t count_up(uint32_t* c) {
  return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t* ctr(uint32_t* base, int i) { return base + READY_CTR_STRIDE * i; }

// Poll *c until it reaches `want`, backing off from about 100 ns to about
// 0.2 us between polls so that waiting workgroups do not flood the memory
// channel that holds the counter.  Bounded:
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
      default: __builtin_amdgcn_s_sleep(8); break;
    }
    if (nap < 2) ++nap;
  }
}

// Poll two counters at once until *c1 >= w1 and (*c2 & m2) >= w2 (same
// bounds and failure reporting as wait_count); *last2 gets *c2's last value.
// SHORT: a constant nap of about 50 ns instead of the backoff, for launches
// with few waiting workgroups (the fp32 single launch: tiny 25.0 -> 24.3 us
// cold; the bf16 launches gained nothing from it).
template <bool SHORT = false>
__device__ bool wait_count2(const uint32_t* c1, uint32_t w1, const uint32_t* c2, uint32_t m2, uint32_t w2,
                            uint32_t* last2, uint32_t* abort_flag, int32_t* dev_status) {
  int nap = 0;
  for (int it = 0;; ++it) {
    const uint32_t v1 = ld_coh_u32(c1), v2 = ld_coh_u32(c2);
    *last2 = v2;
    if (v1 >= w1 && (v2 & m2) >= w2) return true;
    if ((it & 15) == 15 && ld_coh_u32(abort_flag) != 0) return false;
    if (it >= SPIN_LIMIT) {
      st_coh_u32(abort_flag, 1u);
      if (dev_status) st_coh_u32(dev_status, (uint32_t)READY_ERR_SYNC_TIMEOUT);
      return false;
    }
    if constexpr (SHORT) {
      __builtin_amdgcn_s_sleep(2);
    } else {
      switch (nap) {
        case 0: __builtin_amdgcn_s_sleep(4); break;
        case 1: __builtin_amdgcn_s_sleep(8); break;
        default: __builtin_amdgcn_s_sleep(8); break;
      }
      if (nap < 2) ++nap;
    }
  }
}

// A read-only input loaded in a trip of many (see ld_coh16_at): always
// issued; with `live` false it moves no data and returns zero.
__device__ __forceinline__ u32x4 ld_ro16_at(bool live, const void* base, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), live ? byte_off : DEAD_OFF, 0, 0);
}
__device__ __forceinline__ float ld_ro4_at(bool live, const void* base, uint32_t byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(base), live ? byte_off : DEAD_OFF, 0, 0));
}

constexpr uint32_t NO_ITEM = 0xffffffffu;

// XCD (0..7) of the running wave
__device__ __forceinline__ int hw_xcc() {
  uint32_t x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return (int)(x & 7u);
}


// Thread 0 claims an item of queue x for the workgroup; every thread gets
// its index, or NO_ITEM when the queue is exhausted.
__device__ __forceinline__ uint32_t claim_one(uint32_t* qctr, int x, uint32_t size, uint32_t* s_bc) {
  if (threadIdx.x == 0) {
    const uint32_t i = count_up(ctr(qctr, x));
    *s_bc = i < size ? i : NO_ITEM;
  }
  __syncthreads();
  const uint32_t r = *s_bc;
  __syncthreads();
  return r;
}

// One trip of wave 0: lane 0 claims from `claim` (count_up) unless it is
// null; lanes l < n
// read the arrival flag flag(l).  Every thread gets the claim's raw result
// (in *claimed) and the mask of clear flags.  s_bc: 3 words of LDS.
template <typename Flag>
__device__ __forceinline__ uint64_t arrival_check(uint32_t* claim, int n, Flag flag, uint32_t* claimed,
                                                  uint32_t* s_bc) {
  const int tid = item_tid();
  if (tid < 64) {
    uint32_t i = NO_ITEM;
    if (tid == 0 && claim != nullptr) i = count_up(claim);
    const bool clear = tid < n && ld_coh_u32(flag(tid)) == 0u;
    const uint64_t m = __ballot(clear);
    if (tid == 0) {
      s_bc[0] = i;
      s_bc[1] = (uint32_t)m;
      s_bc[2] = (uint32_t)(m >> 32);
    }
  }
  __syncthreads();
  *claimed = s_bc[0];
  const uint64_t m = (uint64_t)s_bc[1] | ((uint64_t)s_bc[2] << 32);
  __syncthreads();
  return m;
}

}  // namespace
