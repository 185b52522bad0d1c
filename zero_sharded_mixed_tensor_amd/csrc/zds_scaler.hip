// Row a3: the dynamic loss-scale state machine on the device.
//
// Lower the scale when the grads overflowed, raise it after a stable stretch
// (devpress.csdn.net DeepSpeed tutorial §2.2; its §3.2 fp16 block names the
// window, initial power, hysteresis and floor; aidhplus.com "DeepSpeed" lists
// dynamic loss scaling among the features). One thread reads the step's
// overflow flag and applies scaler_transition(), the same function the host
// twin runs; on a clean step it also commits the Adam step count and the
// beta powers the update kernel used.
#include "zds_internal.h"

namespace zds {

__global__ void __launch_bounds__(64) scaler_kernel(zds_step_state *state, const zds_step_scalars *sc,
                                                    float beta1, float beta2) {
  if (threadIdx.x != 0) return;
  zds_step_state s = *state;
  scaler_transition(s, sc->overflow, beta1, beta2);
  *state = s;
}

__global__ void __launch_bounds__(64) state_init_kernel(zds_step_state *state, zds_step_state init) {
  if (threadIdx.x == 0) *state = init;
}

zds_status launch_scaler(zds_step_state *state, const zds_step_scalars *scalars, float beta1,
                         float beta2, hipStream_t stream) {
  hipLaunchKernelGGL(scaler_kernel, dim3(1), dim3(64), 0, stream, state, scalars, beta1, beta2);
  return check_launch("loss_scaler_update kernel");
}

zds_status launch_state_init(zds_step_state *state, const zds_step_state &init, hipStream_t stream) {
  hipLaunchKernelGGL(state_init_kernel, dim3(1), dim3(64), 0, stream, state, init);
  return check_launch("step_state_init kernel");
}

}  // namespace zds
