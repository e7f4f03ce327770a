// Combine step of the gated MLP projection when the two projections ran as
// separate qmm launches (mlxcel issue "perf(metal): close native NVFP4
// prefill gap", "Activation-path follow-up": the GeGLU activation of the
// scaled MLP): out = act(gate) * up, in float32, rounded once to the output
// type.  `out` holds the up projection on entry.
#include "glu_act.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4_internal.hpp"

using namespace nvfp4dev;

namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ float to_f32(T v) { return (float)v; }

template <typename T>
__global__ __launch_bounds__(kThreads) void glu_combine_kernel(const T* __restrict__ gate, T* __restrict__ out,
                                                               int64_t n, int act) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
    out[i] = (T)(glu_act(to_f32(gate[i]), act) * to_f32(out[i]));
}

template <typename T>
void combine_typed(const T* gate, T* out, int64_t n, int act, hipStream_t s) {
  int64_t grid = (n + kThreads - 1) / kThreads;
  if (grid > 16384) grid = 16384;
  if (grid < 1) grid = 1;
  glu_combine_kernel<T><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(gate, out, n, act);
}

}  // namespace

namespace nvfp4host {

void launch_glu_combine(const void* gate, void* out, int64_t n, nvfp4_dtype_t dt, int act, hipStream_t s) {
  if (n <= 0) return;
  switch (dt) {
    case NVFP4_F32:
      combine_typed(static_cast<const float*>(gate), static_cast<float*>(out), n, act, s);
      break;
    case NVFP4_BF16:
      combine_typed(static_cast<const __bf16*>(gate), static_cast<__bf16*>(out), n, act, s);
      break;
    case NVFP4_F16:
      combine_typed(static_cast<const _Float16*>(gate), static_cast<_Float16*>(out), n, act, s);
      break;
  }
}

}  // namespace nvfp4host
