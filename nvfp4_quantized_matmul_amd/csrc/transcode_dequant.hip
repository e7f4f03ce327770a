// Load-time kernels: ModelOpt triplet transcode, exact plane dequantize and
// quantize from dense weights.
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

// ----------------------------------------------------------------------------
// Quantize: dense matrices -> packed words, E4M3 block scales, global scale
// (mlxcel PR "native NVFP4 for ROCm QuantizedMatmul/GatherQMM", "Summary":
// block scales are encoded as scale * 448 * 6 / global_scale, and dequantize
// multiplies by global_scale / (448 * 6)).  Every step is one float32
// operation in a fixed order, so codes and nibbles are reproducible:
//   gs    = largest |w| of the matrix (unless given)
//   code  = E4M3 nearest, ties to even, of fl32(amax * fl32(448 / gs)),
//           saturating at 448; 0 when amax or gs is 0
//   d     = fl32(e4m3(code) * fl32(gs / 2688))
//   nibble= E2M1 nearest, ties to even, of fl32(w / d), saturating at 6,
//           with w's sign bit; only the sign when d is 0 or NaN.
// ----------------------------------------------------------------------------

template <typename TI> __device__ __forceinline__ float widen(TI v) { return (float)v; }

// |v| as unsigned bits: an unsigned max over these is the float max of the
// magnitudes with NaN above every number (as a float max that propagates NaN).
__device__ __forceinline__ uint32_t abs_bits(float v) { return __builtin_bit_cast(uint32_t, v) & 0x7FFFFFFFu; }

// Largest |w| of each matrix into gs_bits[b] (zeroed beforehand), as bits.
template <typename TI>
__global__ __launch_bounds__(kThreads) void amax_kernel(const TI* __restrict__ w, int64_t per_mat,
                                                       int64_t batch, uint32_t* __restrict__ gs_bits) {
  __shared__ uint32_t part[kThreads / 64];
  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    const TI* m = w + b * per_mat;
    uint32_t mx = 0;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < per_mat; i += (int64_t)gridDim.x * kThreads)
      mx = max(mx, abs_bits(widen(m[i])));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t t = part[0];
#pragma unroll
      for (int i = 1; i < kThreads / 64; ++i) t = max(t, part[i]);
      atomicMax(gs_bits + b, t);
    }
    __syncthreads();
  }
}

// E4M3 code of a non-negative float: nearest value, ties to the even code;
// 448 and above saturate to 448 (0x7E); NaN gives 0x7F.
__device__ __forceinline__ uint32_t e4m3_nearest(float x) {
  if (!(x == x)) return 0x7Fu;
  if (x >= 448.0f) return 0x7Eu;
  if (x < 0.015625f) return (uint32_t)__builtin_rintf(x * 512.0f);   // subnormals m * 2^-9; 8 is 2^-6
  int e;
  const float frac = __builtin_frexpf(x, &e);                         // x = frac * 2^e, frac in [0.5, 1)
  uint32_t mant = (uint32_t)__builtin_rintf((frac * 2.0f - 1.0f) * 8.0f);
  int ex = e - 1;                                                      // x = (1 + f) * 2^ex, ex in [-6, 8]
  if (mant == 8u) {
    mant = 0u;
    ++ex;
  }
  const uint32_t code = ((uint32_t)(ex + 7) << 3) | mant;
  return code > 0x7Eu ? 0x7Eu : code;
}

// E2M1 magnitude index (0, 0.5, 1, 1.5, 2, 3, 4, 6) nearest to a >= 0, ties
// to the even index, saturating at 6: one step per midpoint crossed, a tie
// at a midpoint counting toward the even side.
__device__ __forceinline__ uint32_t e2m1_nearest(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
         (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
}

// One thread per 16-element block.
template <typename TI>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const TI* __restrict__ w, int64_t nblocks,
                                                           int64_t blocks_per_mat, const float* __restrict__ gs,
                                                           uint32_t* __restrict__ w_out,
                                                           uint8_t* __restrict__ sc_out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblocks; blk += stride) {
    float v[16];
    if constexpr (sizeof(TI) == 4) {
      const float4* p = reinterpret_cast<const float4*>(w + blk * 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 t = p[q];
        v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
      }
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(w + blk * 16);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 t = p[q];
        const TI* h = reinterpret_cast<const TI*>(&t);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[8 * q + j] = widen(h[j]);
      }
    }
    uint32_t am = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) am = max(am, abs_bits(v[j]));
    const float amax = __builtin_bit_cast(float, am);
    const float gsb = gs[blk / blocks_per_mat];
    uint32_t code = 0;
    if (amax != 0.0f && gsb != 0.0f) code = e4m3_nearest(amax * (448.0f / gsb));
    const float d = e4m3<0>(code) * (gsb / kGlobalDivisor);
    const bool no_scale = !(d != 0.0f && d == d);
    uint32_t word[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t sign = (__builtin_bit_cast(uint32_t, v[j]) >> 31) << 3;
      const uint32_t mag = no_scale ? 0u : e2m1_nearest(__builtin_fabsf(v[j] / d));
      word[j >> 3] |= (sign | mag) << (4 * (j & 7));
    }
    *reinterpret_cast<uint2*>(w_out + blk * 2) = make_uint2(word[0], word[1]);
    sc_out[blk] = (uint8_t)code;
  }
}

__global__ void copy_floats_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
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

template <typename TI>
static void quantize_typed(const TI* w, int64_t batch, int64_t rows, int64_t cols, const float* gs_in,
                           uint32_t* w_out, uint8_t* sc_out, float* gs_out, hipStream_t s) {
  const int64_t per_mat = rows * cols;
  const float* gs = gs_in;
  if (!gs_in) {
    launch_fill_zero(gs_out, batch * 4, s);
    if (per_mat > 0) {
      const int64_t gx = grid_for(per_mat, kThreads * 8, 1024);
      const int64_t gy = batch < 65535 ? batch : 65535;
      amax_kernel<TI><<<dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0, s>>>(
          w, per_mat, batch, reinterpret_cast<uint32_t*>(gs_out));
    }
    gs = gs_out;
  } else if (gs_out && gs_out != gs_in) {
    copy_floats_kernel<<<dim3((unsigned)grid_for(batch, kThreads, 1 << 16)), dim3(kThreads), 0, s>>>(gs_in, gs_out,
                                                                                                      batch);
  }
  const int64_t nblocks = batch * per_mat / 16;
  if (nblocks == 0) return;
  quantize_kernel<TI><<<dim3((unsigned)grid_for(nblocks, kThreads, 1 << 20)), dim3(kThreads), 0, s>>>(
      w, nblocks, per_mat / 16, gs, w_out, sc_out);
}

void launch_quantize(const void* w, nvfp4_dtype_t dt, int64_t batch, int64_t rows, int64_t cols,
                     const float* gs_in, uint32_t* w_out, uint8_t* sc_out, float* gs_out, hipStream_t s) {
  switch (dt) {
    case NVFP4_F32:
      quantize_typed(static_cast<const float*>(w), batch, rows, cols, gs_in, w_out, sc_out, gs_out, s);
      break;
    case NVFP4_BF16:
      quantize_typed(static_cast<const __bf16*>(w), batch, rows, cols, gs_in, w_out, sc_out, gs_out, s);
      break;
    case NVFP4_F16:
      quantize_typed(static_cast<const _Float16*>(w), batch, rows, cols, gs_in, w_out, sc_out, gs_out, s);
      break;
  }
}

}  // namespace nvfp4host
