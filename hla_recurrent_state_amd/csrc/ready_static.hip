// readyStateReaderStatic: the state reader for callers that cannot allocate.
// Its scratch is the static device array below instead of a caller's
// workspace; the kernels and their arithmetic are those of readyStateReader.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// array's address on a device comes from hipGetSymbolAddress (one lookup per
// device, kept in g_scratch) and only that address is ever handed to a kernel.
#include <mutex>

#include "ready_internal.h"

static_assert(READY_STATIC_COUNTER_BYTES % 256 == 0 && READY_STATIC_COUNTER_BYTES < READY_STATIC_SCRATCH_BYTES,
              "counters first, arrays after them");

// Counters in the first READY_STATIC_COUNTER_BYTES, arrays after them.  Each
// GPU the library runs on holds its own copy from module load to process end.
static __device__ __align__(256) unsigned char scratch[READY_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
constexpr uint32_t kStaticMagic = READY_WS_MAGIC ^ 0x5a5a5a5au;

std::mutex g_mu;
char* g_scratch[kMaxDevices];  // device address of `scratch` per device (null until looked up)

// Device address of the array on the current device; on first use, look it
// up and clear its counters on `stream` (the fill kernel, never a memset, so
// that nothing of the kind lands in a graph).
readyStatus resolve_static(WsView* view, hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return READY_ERR_HIP;
  if (dev >= kMaxDevices) return READY_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return READY_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone) return READY_ERR_UNSUPPORTED;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return READY_ERR_HIP;
    if (ready_launch_ws_init((uint32_t*)ptr, (int)(READY_STATIC_COUNTER_BYTES / 4), kStaticMagic, stream) !=
        hipSuccess)
      return READY_ERR_HIP;
    g_scratch[dev] = (char*)ptr;
  }
  char* base = g_scratch[dev];
  view->ctr = (uint32_t*)base;
  view->data = base + READY_STATIC_COUNTER_BYTES;
  view->magic = kStaticMagic;
  return READY_OK;
}

}  // namespace

extern "C" readyStatus readyStateReaderStatic(const readyPlan* plan, const readyStates* states,
                                              const int32_t* accept_idx, const void* h, const readyWeights* w,
                                              const readyOutputs* o, void* stream) {
  if (!plan) return READY_ERR_NULL_POINTER;
  size_t data_bytes = 0, ctr_bytes = 0;
  ready_plan_scratch_needs(plan, &data_bytes, &ctr_bytes);
  if (ctr_bytes > READY_STATIC_COUNTER_BYTES || data_bytes > READY_STATIC_SCRATCH_BYTES - READY_STATIC_COUNTER_BYTES)
    return READY_ERR_STATIC_SCRATCH_TOO_SMALL;
  // The array is its own allocation, so it cannot overlap the caller's
  // buffers: the aliasing checks run with empty scratch ranges, and the
  // device address is looked up only once the arguments have passed them.
  WsView v;
  v.data = nullptr;
  v.ctr = nullptr;
  v.magic = kStaticMagic;
  v.data_bytes = 0;
  v.ctr_bytes = 0;
  return ready_run_reader(plan, states, accept_idx, h, w, o, nullptr, 0, stream, nullptr, &v, resolve_static);
}
