// Measurement aid, built into its own library (libnvfp4_measure.so) and
// used only by the benchmark: a plain streaming read, which measures the rate
// a kernel can reach on this device for a given byte count (the context for
// the decode kernel's HBM roofline).  It reads every 16-byte chunk once in a
// grid-stride loop and folds the data into one word per lane; a word is
// stored only if the fold hits a sentinel, so the loads cannot be elided and
// nothing is written in practice.
//
//   int nvfp4_stream_read(const void* p, int64_t bytes, int64_t blocks,
//                         uint32_t* sink, hipStream_t stream);
//
// p: device pointer, 16-byte aligned; bytes: a multiple of 16; blocks >= 1
// workgroups of 256 threads; sink: device uint32, 4-byte aligned.  Returns 0,
// or the libnvfp4 status codes -1 (NULL pointer), -2 (bad size), -7 (launch
// error), -8 (misaligned pointer); on an error nothing is launched.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

extern "C" int nvfp4_stream_read(const void* p, int64_t bytes, int64_t blocks, uint32_t* sink,
                                 hipStream_t stream) {
  if (bytes < 0 || bytes % 16 != 0 || blocks < 1 || blocks > 2147483647LL) return -2;
  if (bytes == 0) return 0;
  if (!p || !sink) return -1;
  if ((reinterpret_cast<uintptr_t>(p) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3) != 0) return -8;
  stream_read_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(static_cast<const uint4*>(p),
                                                                          bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}
