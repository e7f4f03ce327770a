// Load-time kernels: ModelOpt triplet transcode and exact plane dequantize.
//
// Transcode (mlxcel issue "perf(nvfp4): direct-transcode ModelOpt triplets to
// MLX native", "Technical notes" and "Implementation plan" step 3): four
// source bytes form one little-endian word, so on a little-endian device the
// packed plane is a byte move of the source and never passes through dense
// values; the E4M3 block scales are kept as bytes; weight_scale_2 becomes the
// float32 sidecar gs = ws2 * 2688 (so that gs / (448 * 6) is ws2).
//
// Dequantize (mlxcel PR "native NVFP4 for ROCm QuantizedMatmul/GatherQMM",
// "Summary"): expands a plane exactly; the grid covers the weight words
// ("Changes during review": sized from the weight, not from the scales).
#include "nvfp4_device.hpp"
#include "nvfp4_internal.hpp"

using namespace nvfp4dev;

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void copy_bytes_kernel(const uint8_t* __restrict__ src,
                                                              uint8_t* __restrict__ dst, int64_t n,
                                                              int vec16) {
  const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t done = 0;
  if (vec16) {
    const int64_t n16 = n / 16;
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    for (int64_t i = tid; i < n16; i += stride) d4[i] = s4[i];
    done = n16 * 16;
  }
  for (int64_t i = done + tid; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(uint8_t* __restrict__ dst, int64_t n) {
  const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t n16 = n / 16;
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  for (int64_t i = tid; i < n16; i += stride) d4[i] = make_uint4(0, 0, 0, 0);
  for (int64_t i = n16 * 16 + tid; i < n; i += stride) dst[i] = 0;
}

__global__ void sidecar_kernel(const float* __restrict__ ws2, float* __restrict__ gs, int64_t batch) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < batch) gs[i] = ws2[i] * kGlobalDivisor;
}

template <typename TO>
__device__ __forceinline__ void store8(TO* p, const float (&v)[8]);

template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&v)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

template <>
__device__ __forceinline__ void store8<__bf16>(__bf16* p, const float (&v)[8]) {
  __bf16 h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (__bf16)v[i];
  *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, h);
}

template <>
__device__ __forceinline__ void store8<_Float16>(_Float16* p, const float (&v)[8]) {
  _Float16 h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (_Float16)v[i];
  *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, h);
}

// One thread per packed word: 8 output elements.
template <typename TO>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint32_t* __restrict__ w,
                                                           const uint8_t* __restrict__ sc,
                                                           const float* __restrict__ gs,
                                                           int64_t nwords, int64_t kw,
                                                           int64_t words_per_mat,
                                                           TO* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < nwords; idx += stride) {
    const int64_t row = idx / kw;
    const int64_t wi = idx - row * kw;
    const float s = e4m3<0>(sc[row * (kw >> 1) + (wi >> 1)]);
    float v[8];
    decode_word_f32(w[idx], s, v);
    if (gs) {
      const float g = gs[idx / words_per_mat] / kGlobalDivisor;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] *= g;
    }
    store8<TO>(out + idx * 8, v);
  }
}

int64_t grid_for(int64_t work, int64_t per_block, int64_t cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return g > cap ? cap : g;
}

}  // namespace

namespace nvfp4host {

void launch_copy_bytes(const uint8_t* src, uint8_t* dst, int64_t n, hipStream_t s) {
  if (n == 0 || src == dst) return;
  const int vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
  const int64_t units = vec ? n / 16 + 1 : n;
  const int64_t grid = grid_for(units, kThreads, 1 << 16);
  copy_bytes_kernel<<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(src, dst, n, vec);
}

void launch_fill_zero(void* dst, int64_t n, hipStream_t s) {
  if (n == 0) return;
  const int64_t grid = grid_for(n / 16 + 1, kThreads, 1 << 16);
  fill_zero_kernel<<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(static_cast<uint8_t*>(dst), n);
}

void launch_sidecar(const float* ws2, float* gs_out, int64_t batch, hipStream_t s) {
  if (batch == 0) return;
  const int64_t grid = grid_for(batch, kThreads, 1 << 16);
  sidecar_kernel<<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(ws2, gs_out, batch);
}

void launch_dequantize(const uint32_t* w, const uint8_t* sc, const float* gs, int64_t batch,
                       int64_t rows, int64_t cols, nvfp4_dtype_t dt, void* out, hipStream_t s) {
  const int64_t kw = cols / 8;
  const int64_t nwords = batch * rows * kw;
  if (nwords == 0) return;
  const int64_t grid = grid_for(nwords, kThreads, 1 << 20);
  const int64_t wpm = rows * kw;
  switch (dt) {
    case NVFP4_F32:
      dequant_kernel<float><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(w, sc, gs, nwords, kw, wpm,
                                                                          static_cast<float*>(out));
      break;
    case NVFP4_BF16:
      dequant_kernel<__bf16><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(w, sc, gs, nwords, kw, wpm,
                                                                           static_cast<__bf16*>(out));
      break;
    case NVFP4_F16:
      dequant_kernel<_Float16><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(w, sc, gs, nwords, kw, wpm,
                                                                             static_cast<_Float16*>(out));
      break;
  }
}

}  // namespace nvfp4host
