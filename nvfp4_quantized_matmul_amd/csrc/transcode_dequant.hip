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

// Eight outputs as non-temporal 16-byte stores (the expanded plane is
// written once and not read back by this call).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <typename TO>
__device__ __forceinline__ void store8_nt(TO* p, const float (&v)[8]) {
  if constexpr (sizeof(TO) == 4) {
    const float a[4] = {v[0], v[1], v[2], v[3]}, b[4] = {v[4], v[5], v[6], v[7]};
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, a), reinterpret_cast<u32x4_t*>(p));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, b), reinterpret_cast<u32x4_t*>(p) + 1);
  } else {
    TO h[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) h[k] = (TO)v[k];
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, h), reinterpret_cast<u32x4_t*>(p));
  }
}

// Dequantize, one thread per packed word (8 outputs), with no index
// division: block row y takes matrices y, y + gridDim.y, ..., and over a
// matrix's words taken as one flat array, word i uses scale byte i / 2
// (every row holds an even number of words).  Lane l of a wavefront writes
// the 8 outputs of word base + l, so each store instruction covers one
// contiguous run.  The word loads and output stores are non-temporal (each
// byte is touched once): measured 9% faster (54.8 vs 60.0 us for bf16 at
// 21504 x 5376).  Earlier a separate kernel with a division per word served
// batches beyond the grid's y limit; the matrix loop replaces it.
template <typename TO>
__global__ __launch_bounds__(kThreads) void dequant_flat_kernel(const uint32_t* __restrict__ w,
                                                                const uint8_t* __restrict__ sc,
                                                                const float* __restrict__ gs, int64_t wpm,
                                                                int64_t batch, TO* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t mat = blockIdx.y; mat < batch; mat += gridDim.y) {
    const uint32_t* wm = w + mat * wpm;
    const uint8_t* sm = sc + mat * (wpm >> 1);
    TO* om = out + mat * wpm * 8;
    const float g = gs ? gs[mat] / kGlobalDivisor : 1.0f;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < wpm; i += stride) {
      float v[8];
      decode_word_f32(__builtin_nontemporal_load(wm + i), e4m3<0>(sm[i >> 1]), v);
      if (gs) {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] *= g;
      }
      store8_nt<TO>(om + i * 8, v);
    }
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

// The 16 bytes at p as float values (8 bf16/f16 or 4 f32).
template <typename TI>
__device__ __forceinline__ void unpack16(const uint4& raw, float (&v)[16 / sizeof(TI)]) {
  const TI* h = reinterpret_cast<const TI*>(&raw);
#pragma unroll
  for (int j = 0; j < (int)(16 / sizeof(TI)); ++j) v[j] = widen(h[j]);
}

template <typename TI>
__device__ __forceinline__ uint32_t chunk_amax_bits(const uint4& raw) {
  float v[16 / sizeof(TI)];
  unpack16<TI>(raw, v);
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < (int)(16 / sizeof(TI)); ++j) m = max(m, abs_bits(v[j]));
  return m;
}

// Largest |w| of each matrix into gs_bits[b] (zeroed beforehand), as bits:
// for non-negative floats the unsigned order of the bit patterns is the
// numeric order, and a NaN pattern sits above +inf, so NaN propagates.  Each
// matrix is a whole number of 16-byte chunks (its length is a multiple of 16
// elements) and starts 16-byte aligned; a lane keeps four chunk loads in
// flight.
template <typename TI>
__global__ __launch_bounds__(kThreads) void amax_kernel(const TI* __restrict__ w, int64_t chunks_per_mat,
                                                       int64_t batch, uint32_t* __restrict__ gs_bits) {
  __shared__ uint32_t part[kThreads / 64];
  const int64_t st = (int64_t)gridDim.x * kThreads;
  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    const uint4* m = reinterpret_cast<const uint4*>(w) + b * chunks_per_mat;
    uint32_t mx = 0;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + 3 * st < chunks_per_mat; i += 4 * st) {
      const uint4 r0 = m[i];
      const uint4 r1 = m[i + st];
      const uint4 r2 = m[i + 2 * st];
      const uint4 r3 = m[i + 3 * st];
      mx = max(max(mx, chunk_amax_bits<TI>(r0)), chunk_amax_bits<TI>(r1));
      mx = max(max(mx, chunk_amax_bits<TI>(r2)), chunk_amax_bits<TI>(r3));
    }
    for (; i < chunks_per_mat; i += st) mx = max(mx, chunk_amax_bits<TI>(m[i]));
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
  int e;
  const float frac = __builtin_frexpf(x, &e);                         // x = frac * 2^e, frac in [0.5, 1)
  const uint32_t mant = (uint32_t)__builtin_rintf((frac * 2.0f - 1.0f) * 8.0f);   // 0..8; 8 carries
  const uint32_t normal = ((uint32_t)(e - 1 + 7) << 3) + mant;        // x = (1 + f) * 2^(e-1), e-1 in [-6, 8]
  const uint32_t sub = (uint32_t)__builtin_rintf(x * 512.0f);         // subnormals m * 2^-9; 8 is 2^-6
  uint32_t code = x < 0.015625f ? sub : normal;
  code = code > 0x7Eu ? 0x7Eu : code;
  code = x >= 448.0f ? 0x7Eu : code;
  return x == x ? code : 0x7Fu;
}

// One lane per 16-byte chunk of the input, so sizeof(TI) consecutive lanes
// hold one 16-element block: 16/sizeof(TI) elements each.  The lanes of a
// block share its largest magnitude through a cross-lane exchange, each
// encodes its own elements into 4*16/sizeof(TI) bits of the block's two
// little-endian words (element j at bits 4j of the 64), and the first lane
// writes the scale byte.  A workgroup takes kQuantUnroll * kThreads chunks
// and issues all their loads before any arithmetic, which keeps enough bytes
// in flight per CU to cover memory latency.  Tiles go in reverse order of
// address: the matrix-maximum pass that precedes this one sweeps forwards, so
// the part of the input still held by the last-level cache is read first.
constexpr int kQuantUnroll = 4;

template <typename TI>
__device__ __forceinline__ void quantize_chunk(const uint4& raw, int64_t c, float gsb,
                                               uint32_t* __restrict__ w_out, uint8_t* __restrict__ sc_out) {
  constexpr int L = (int)sizeof(TI);   // lanes per block
  constexpr int E = 16 / L;            // elements per lane
  float v[E];
  unpack16<TI>(raw, v);
  uint32_t am = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) am = max(am, abs_bits(v[j]));
#pragma unroll
  for (int off = 1; off < L; off <<= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off, 64));
  const int64_t blk = c / L;
  const float amax = __builtin_bit_cast(float, am);
  const uint32_t code = (amax != 0.0f && gsb != 0.0f) ? e4m3_nearest(amax * (448.0f / gsb)) : 0u;
  const float d = e4m3<0>(code) * (gsb / kGlobalDivisor);
  const bool no_scale = !(d != 0.0f && d == d);
  uint32_t bits = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) bits |= (__builtin_bit_cast(uint32_t, v[j]) >> 31) << (4 * j + 3);
  if (!no_scale) {
    // |v| / d rounded once in float32 (correctly rounded division), then to
    // the nearest E2M1 magnitude by the hardware converter: ties to even,
    // saturating at 6 (the clamp keeps infinities in its finite range).
    float q[E];
#pragma unroll
    for (int j = 0; j < E; ++j) q[j] = __builtin_fminf(__builtin_fabsf(v[j]) / d, 8.0f);
    uint32_t mags = 0;
    mags = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(mags, q[0], q[1], 1.0f, 0);
    mags = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(mags, q[2], q[3], 1.0f, 1);
    if constexpr (E == 8) {
      mags = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(mags, q[4], q[5], 1.0f, 2);
      mags = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(mags, q[6], q[7], 1.0f, 3);
    }
    bits |= mags;
  }
  if constexpr (L == 2)
    w_out[c] = bits;
  else
    reinterpret_cast<uint16_t*>(w_out)[c] = (uint16_t)bits;
  if (c % L == 0) sc_out[blk] = (uint8_t)code;
}

// Grid: x over tiles of one matrix, y over matrices, so each workgroup's
// global scale is one uniform value.
template <typename TI>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const TI* __restrict__ w, int64_t chunks_per_mat,
                                                           int64_t batch, const float* __restrict__ gs,
                                                           uint32_t* __restrict__ w_out,
                                                           uint8_t* __restrict__ sc_out) {
  constexpr int64_t kTile = (int64_t)kThreads * kQuantUnroll;
  const int64_t tiles = (chunks_per_mat + kTile - 1) / kTile;
  for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
    const float gsb = gs[b];
    const int64_t mat0 = b * chunks_per_mat;
    const uint4* src = reinterpret_cast<const uint4*>(w) + mat0;
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
      const int64_t base = (tiles - 1 - t) * kTile + threadIdx.x;
      uint4 raw[kQuantUnroll];
#pragma unroll
      for (int u = 0; u < kQuantUnroll; ++u) {
        const int64_t c = base + u * kThreads;
        raw[u] = c < chunks_per_mat ? src[c] : make_uint4(0u, 0u, 0u, 0u);
      }
      // chunks_per_mat is a multiple of sizeof(TI) and so is every chunk
      // index's lane offset: the lanes of one block are all in or all out.
#pragma unroll
      for (int u = 0; u < kQuantUnroll; ++u) {
        const int64_t c = base + u * kThreads;
        if (c < chunks_per_mat) quantize_chunk<TI>(raw[u], mat0 + c, gsb, w_out, sc_out);
      }
    }
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
  const int64_t wpm = rows * kw;
  const dim3 gridf((unsigned)grid_for(wpm, kThreads, 1 << 16), (unsigned)(batch < kMaxGridY ? batch : kMaxGridY));
  switch (dt) {
    case NVFP4_F32:
      dequant_flat_kernel<float><<<gridf, dim3(kThreads), 0, s>>>(w, sc, gs, wpm, batch, static_cast<float*>(out));
      break;
    case NVFP4_BF16:
      dequant_flat_kernel<__bf16><<<gridf, dim3(kThreads), 0, s>>>(w, sc, gs, wpm, batch, static_cast<__bf16*>(out));
      break;
    case NVFP4_F16:
      dequant_flat_kernel<_Float16><<<gridf, dim3(kThreads), 0, s>>>(w, sc, gs, wpm, batch,
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
      const int64_t chunks = per_mat * (int64_t)sizeof(TI) / 16;
      const int64_t gx = grid_for(chunks, kThreads * 16, 2048);
      const int64_t gy = batch < 65535 ? batch : 65535;
      amax_kernel<TI><<<dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0, s>>>(
          w, chunks, batch, reinterpret_cast<uint32_t*>(gs_out));
    }
    gs = gs_out;
  } else if (gs_out && gs_out != gs_in) {
    copy_floats_kernel<<<dim3((unsigned)grid_for(batch, kThreads, 1 << 16)), dim3(kThreads), 0, s>>>(gs_in, gs_out,
                                                                                                      batch);
  }
  const int64_t chunks = per_mat * (int64_t)sizeof(TI) / 16;
  if (chunks == 0) return;
  const int64_t gx = grid_for(chunks, kThreads * kQuantUnroll, 1 << 16);
  const int64_t gy = batch < 65535 ? batch : 65535;
  quantize_kernel<TI><<<dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0, s>>>(w, chunks, batch, gs, w_out,
                                                                                  sc_out);
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
