// Instance reset: every cache of the named requests (all layers) back to
// empty, the initial state the swap-in calls start from (an empty cache per
// request and layer; sglang PR #20343 summary, "Implementation breakdown").
#include "internal.h"

namespace hisparse {

namespace {

__global__ __launch_bounds__(256) void reset_instances(ResetArgs a) {
  const int r = a.reqs ? a.reqs[blockIdx.x] : static_cast<int>(blockIdx.x);
  const int layer = blockIdx.y;
  if (r < 0 || r >= a.R) {
    if (threadIdx.x == 0 && layer == 0) raise_error(a.err, HISPARSE_ERR_BAD_ROW);
    return;
  }
  const size_t q = static_cast<size_t>(layer) * a.R + r;
  for (int s = threadIdx.x; s < a.H; s += blockDim.x) {
    a.slot_key[q * a.H + s] = kEmpty;
    if (a.ts) a.ts[q * a.H + s] = -1;
    if (a.order) a.order[q * a.H + s] = static_cast<int16_t>(s);
  }
  if (a.refbits)
    for (int w = threadIdx.x; w < a.Hw; w += blockDim.x) a.refbits[q * a.Hw + w] = 0u;
  if (threadIdx.x == 0) {
    a.ctrl[2 * q] = 0;
    a.ctrl[2 * q + 1] = 0;
  }
}

}  // namespace

hipError_t launch_reset(const ResetArgs& a, int n, int layers, hipStream_t s) {
  hipLaunchKernelGGL(reset_instances, dim3(n, layers), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hisparse
