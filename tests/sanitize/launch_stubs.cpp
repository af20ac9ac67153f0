// Kernel launchers for the sanitizer build of the host code: every launcher
// reports that no device is present.  The CPU tests run against this build
// only on paths that end before a launch (argument validation, plans,
// workspace sizes, error strings); the real launchers live in the .hip
// sources, whose host parts are thin wrappers around hipLaunchKernelGGL.
#include "../../hla_recurrent_state_amd/csrc/ready_internal.h"

hipError_t ready_launch_gather(const GatherArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t ready_launch_verify(const VerifyArgs&, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t ready_launch_state(const StateArgs&, int, int, hipStream_t, StageEvents) { return hipErrorNoDevice; }
hipError_t ready_launch_state_mm(const StateArgs&, int, hipStream_t, StageEvents) { return hipErrorNoDevice; }
hipError_t ready_launch_gemm(const GemmArgs&, int, int, int, int, dim3, size_t, hipStream_t, StageEvents) {
  return hipErrorNoDevice;
}
hipError_t ready_launch_gemm_mm(const GemmArgs&, int, int, int, int, hipStream_t, StageEvents) {
  return hipErrorNoDevice;
}
hipError_t ready_launch_reduce_bias_act(const GemmArgs&, int, hipStream_t, StageEvents) { return hipErrorNoDevice; }
hipError_t ready_launch_gemm_mfma(const GemmArgs&, int, int, int, int, dim3, hipStream_t, StageEvents) {
  return hipErrorNoDevice;
}
hipError_t ready_launch_reader(const FastArgs&, int, int, hipStream_t, StageEvents) { return hipErrorNoDevice; }
hipError_t ready_launch_reader_f32(const F32Args&, int, size_t, hipStream_t, StageEvents) { return hipErrorNoDevice; }
hipError_t ready_launch_ws_init(uint32_t*, int, uint32_t, hipStream_t) { return hipErrorNoDevice; }
int ready_reader_per_cu(int, int, size_t, int) { return 0; }
