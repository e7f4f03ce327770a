// Device helpers for NVFP4 on gfx950 (CDNA4).
//
// Format (mlxcel issue "perf(nvfp4): direct-transcode ModelOpt triplets to MLX
// native", "Technical notes"): eight E2M1 nibbles per little-endian uint32,
// element j at bits [4j, 4j+4); one OCP E4M3FN scale byte per 16 elements.
//
// Decoding uses the gfx950 hardware converters:
//  * v_cvt_f32_fp8 decodes one OCP E4M3FN byte exactly (NaN codes give NaN);
//  * v_cvt_scalef32_pk_{f32,bf16}_fp4 decodes the two nibbles of one byte
//    exactly when the scale operand is 1.0.  Its scale operand only applies
//    the power-of-two exponent of the float, so the E4M3 block scale (which
//    has three mantissa bits) is applied by an ordinary multiply instead.
// Every product e2m1 * e4m3 has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in float32 and in bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4dev {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// Per-matrix strides of a batch of weight matrices launched together (grid
// dimension y is the matrix): elements of x and out, words of the weight
// plane, bytes of the scale plane; the global scale advances by one float.
// All zero for a single matrix.
struct MatrixStrides {
  int64_t x, w, s, o;
};

// The divisor of the global scale: 448 (largest E4M3) * 6 (largest E2M1)
// (mlxcel PR "native NVFP4 for ROCm QuantizedMatmul/GatherQMM", "Summary").
constexpr float kGlobalDivisor = 2688.0f;

// One E4M3 byte (byte SEL of v) to float, exact.
template <int SEL>
__device__ __forceinline__ float e4m3(uint32_t v) {
  return __builtin_amdgcn_cvt_f32_fp8((int)v, SEL);
}

// The two E2M1 nibbles of byte SEL of w as floats: .x = low nibble
// (even element), .y = high nibble.
template <int SEL>
__device__ __forceinline__ f32x2_t e2m1x2_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Same, as a packed bf16 pair (low half = even element).
template <int SEL>
__device__ __forceinline__ bf16x2_t e2m1x2_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}

__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Pack two floats whose values are exact in bf16 into one bf16 pair by
// keeping their upper halves (lo -> bits 0..15, hi -> bits 16..31).
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(fbits(hi), fbits(lo), 0x07060302u);
}

// Eight elements of one word times the block scale s, as exact bf16 (the
// MFMA operand for eight consecutive k).
__device__ __forceinline__ bf16x8_t decode_word_bf16(uint32_t w, float s) {
  f32x2_t p0 = e2m1x2_f32<0>(w), p1 = e2m1x2_f32<1>(w), p2 = e2m1x2_f32<2>(w), p3 = e2m1x2_f32<3>(w);
  uint32_t d[4];
  d[0] = pack_bf16_exact(p0.x * s, p0.y * s);
  d[1] = pack_bf16_exact(p1.x * s, p1.y * s);
  d[2] = pack_bf16_exact(p2.x * s, p2.y * s);
  d[3] = pack_bf16_exact(p3.x * s, p3.y * s);
  return __builtin_bit_cast(bf16x8_t, d);
}

// Eight elements of one word times the block scale s as exact f16 (every
// product e2m1 * e4m3 lies in [2^-10, 2688] with at most 6 significant
// bits, and every E4M3 value is an f16).  One FP4 convert and one packed
// f16 multiply per pair.
__device__ __forceinline__ f16x8_t decode_word_f16(uint32_t w, float s) {
  const _Float16 h = (_Float16)s;
  const f16x2_t ss = {h, h};
  const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
  const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
  const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
  const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
  const uint32_t d[4] = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                         __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
  return __builtin_bit_cast(f16x8_t, d);
}

// A float32 split exactly into three bf16 values whose sum is the input
// (bit patterns, low halves zero): hi keeps the top 8 significand bits
// (truncation), mid the next 8 of the remainder, lo the rest (at most 8
// bits, so exact).  The products of an exact bf16 weight with each part are
// exact in an MFMA, so three MFMAs accumulate float32-level products.
// Infinities and NaNs go whole into hi (a NaN keeps a mantissa bit), with mid
// and lo zero.
__device__ __forceinline__ void split3_bits(uint32_t u, uint32_t& h, uint32_t& m, uint32_t& l) {
  const bool fin = (u & 0x7f800000u) != 0x7f800000u;
  h = (u & 0xffff0000u) | ((!fin && (u & 0x007fffffu)) ? 0x00400000u : 0u);
  const float r1 = fin ? __builtin_bit_cast(float, u) - __builtin_bit_cast(float, h) : 0.0f;
  m = __builtin_bit_cast(uint32_t, r1) & 0xffff0000u;
  const float r2 = r1 - __builtin_bit_cast(float, m);
  l = __builtin_bit_cast(uint32_t, r2);
}

// Eight elements of one word times s, as floats (exact).
__device__ __forceinline__ void decode_word_f32(uint32_t w, float s, float (&v)[8]) {
  f32x2_t p0 = e2m1x2_f32<0>(w), p1 = e2m1x2_f32<1>(w), p2 = e2m1x2_f32<2>(w), p3 = e2m1x2_f32<3>(w);
  v[0] = p0.x * s; v[1] = p0.y * s; v[2] = p1.x * s; v[3] = p1.y * s;
  v[4] = p2.x * s; v[5] = p2.y * s; v[6] = p3.x * s; v[7] = p3.y * s;
}

// Sum of x[i] * e2m1(word element i) over the eight elements of one word,
// x given as four packed bf16 pairs; float32 accumulation starting at acc.
__device__ __forceinline__ float dot_word_bf16(uint32_t w, const uint32_t* xp, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<0>(w), __builtin_bit_cast(bf16x2_t, xp[0]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<1>(w), __builtin_bit_cast(bf16x2_t, xp[1]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<2>(w), __builtin_bit_cast(bf16x2_t, xp[2]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<3>(w), __builtin_bit_cast(bf16x2_t, xp[3]), acc, false);
  return acc;
}

// Same with float32 activations (eight floats), FMA accumulation.
__device__ __forceinline__ float dot_word_f32(uint32_t w, const float* xv, float acc) {
  f32x2_t p0 = e2m1x2_f32<0>(w), p1 = e2m1x2_f32<1>(w), p2 = e2m1x2_f32<2>(w), p3 = e2m1x2_f32<3>(w);
  acc = __builtin_fmaf(xv[0], p0.x, acc); acc = __builtin_fmaf(xv[1], p0.y, acc);
  acc = __builtin_fmaf(xv[2], p1.x, acc); acc = __builtin_fmaf(xv[3], p1.y, acc);
  acc = __builtin_fmaf(xv[4], p2.x, acc); acc = __builtin_fmaf(xv[5], p2.y, acc);
  acc = __builtin_fmaf(xv[6], p3.x, acc); acc = __builtin_fmaf(xv[7], p3.y, acc);
  return acc;
}

// g = fl32(gs / 2688), the once-per-output global factor; 1 when absent
// (multiplying by 1 is exact, so the absent case is unchanged).
__device__ __forceinline__ float global_factor(const float* gs, int64_t i) {
  return gs ? gs[i] / kGlobalDivisor : 1.0f;
}

// Sum over the 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum over the 64 lanes of a fully active wavefront with DPP: pairs, quads,
// half-rows and rows of 16 lanes inside the VALU, then the four row sums
// through scalar registers.  The result is wave-uniform.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<0xb1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4e>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Output element stores (round to nearest even).
__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(__bf16* p, float v) { *p = (__bf16)v; }
__device__ __forceinline__ void store_out(_Float16* p, float v) { *p = (_Float16)v; }

__device__ __forceinline__ float load_x(const float* p) { return *p; }
__device__ __forceinline__ float load_x(const __bf16* p) { return (float)*p; }
__device__ __forceinline__ float load_x(const _Float16* p) { return (float)*p; }

}  // namespace nvfp4dev
