// NVFP4 GEMM kernels for the large-M ("prefill") route.
//
// The pages' ROCm design (mlxcel PR "native NVFP4 for ROCm QuantizedMatmul/
// GatherQMM", "Summary") dequantizes the whole plane and then calls a vendor
// GEMM, applying the global scale after the matmul.  Here, for transposed
// planes, the dequantize is fused into the GEMM instead, so no dense plane is
// written to HBM:
//
//  * gemm_mfma_v3_kernel (transposed plane, K % 64 == 0): the main kernel,
//    operands streamed global -> LDS, each packed word decoded once per block
//    into exact bf16 (or f16) MFMA operands; float32 activations run it over
//    their exact three-part bf16 split (split_f32_kernel); forms for the K
//    split of few tiles and for the gated MLP projection.  Described below.
//  * gemm_mfma_v3p_kernel: the plain v3 tile as a persistent launch (one
//    block per compute unit walking its tiles, each tile's first slabs queued
//    during the previous tile's last steps, each step's first operands read
//    during the previous step's last multiplies) when there are more tiles
//    than compute units and K is a multiple of 384; the same for the gated
//    MLP projection's whole rounds of tiles.
//  * gemm_mfma_kernel (bf16 activations, transposed plane, K % 32 == 0):
//    each wavefront decodes its weight rows straight from the packed words
//    into bf16 MFMA operands (one 32-bit word = the eight k-values one lane
//    feeds to a 32x32x16 MFMA), while the activation tile is staged in LDS
//    (double buffered) and shared by the four wavefronts.  Products
//    e2m1 * e4m3 are exact in bf16, the MFMA accumulates in float32, and
//    g = gs / 2688 multiplies each output once at the end.
//  * dequant_nt_kernel + gemm_mfma_dense_kernel (non-transposed planes,
//    K % 64 == 0): the pages' order, an exact dense transposed copy of the
//    plane in the caller's workspace, then a matrix-core GEMM on it.
//  * gemm_generic_kernel: a float32 FMA tiled GEMM for the rest (K not a
//    multiple of 64, or a form that needs a workspace called without one),
//    with both tiles decoded to float32 in LDS.
#include <atomic>

#include "glu_act.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4_internal.hpp"

using namespace nvfp4dev;

namespace {

// ----------------------------------------------------------------------------
// MFMA kernel
// ----------------------------------------------------------------------------

constexpr int kBN = 256;       // weight rows (output columns) per block
constexpr int kBM = 256;       // activation rows per block
constexpr int kBK = 64;        // k per pipeline stage
constexpr int kLdsK = kBK + 8; // padded LDS row (bf16 elements)
constexpr int kMfmaThreads = 256;

__global__ __launch_bounds__(kMfmaThreads, 1) void gemm_mfma_kernel(
    const __bf16* __restrict__ x, const uint32_t* __restrict__ w, const uint8_t* __restrict__ sc,
    const float* __restrict__ gs, __bf16* __restrict__ out, int64_t M, int64_t K, int64_t N,
    int64_t tiles_m, int64_t tiles_total) {
  __shared__ __attribute__((aligned(16))) __bf16 xs[2][kBM][kLdsK];

  // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs,
  // so give each XCD a contiguous run of logical tiles (activation tiles
  // fastest) and the tiles that share weight rows share that XCD's L2.
  const int64_t per_xcd = (int64_t)gridDim.x / 8;
  const int64_t logical = ((int64_t)blockIdx.x % 8) * per_xcd + (int64_t)blockIdx.x / 8;
  if (logical >= tiles_total) return;  // whole block, before any barrier
  const int64_t m_blk = (logical % tiles_m) * kBM;
  const int64_t n_blk = (logical / tiles_m) * kBN;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t kw = K / 8, ks = K / 16;
  const int64_t nslabs = (K + kBK - 1) / kBK;

  // Weight rows fed by this lane, one per 32-row fragment.
  int64_t wrow[4];
  bool wok[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t n = n_blk + wn * 128 + a * 32 + l32;
    wok[a] = n < N;
    wrow[a] = wok[a] ? n : 0;
  }

  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  uint4 xreg[8];
  uint4 wcur[4], wnext[4];
  uint32_t scur[4], snext[4];

  // Activation slab [kBM][kBK] -> registers (zeros outside M or K).
  auto load_x = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int lin = i * kMfmaThreads + t;
      const int row = lin >> 3, col = (lin & 7) * 8;
      const int64_t m = m_blk + row, k = k0 + col;
      xreg[i] = (m < M && k < K) ? *reinterpret_cast<const uint4*>(x + m * K + k) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int lin = i * kMfmaThreads + t;
      const int row = lin >> 3, col = (lin & 7) * 8;
      *reinterpret_cast<uint4*>(&xs[buf][row][col]) = xreg[i];
    }
  };
  // Weights: lane (row, h) takes words [4h, 4h+4) of the 8-word slab and
  // the two scale bytes of those words (K % 32 == 0, so a lane's four words
  // are all inside K or all outside).
  auto load_w = [&](int64_t k0, uint4 (&wr)[4], uint32_t (&sr)[4]) {
    const int64_t word0 = k0 / 8 + 4 * h;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if (wok[a] && word0 < kw) {
        wr[a] = *reinterpret_cast<const uint4*>(w + wrow[a] * kw + word0);
        sr[a] = *reinterpret_cast<const uint16_t*>(sc + wrow[a] * ks + word0 / 2);
      } else {
        wr[a] = make_uint4(0, 0, 0, 0);
        sr[a] = 0;
      }
    }
  };

  load_x(0);
  load_w(0, wcur, scur);
  store_x(0);
  __syncthreads();

  for (int64_t s = 0; s < nslabs; ++s) {
    const int buf = (int)(s & 1);
    const bool more = s + 1 < nslabs;
    if (more) {
      load_x((s + 1) * kBK);
      load_w((s + 1) * kBK, wnext, snext);
    }
    float slo[4], shi[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      slo[a] = e4m3<0>(scur[a]);
      shi[a] = e4m3<1>(scur[a]);
    }
    // MFMA step j: lane half h supplies word 4h+j, i.e. physical k in
    // [8(4h+j), 8(4h+j)+8) of the slab; the activation operand reads the
    // same k range, so the contraction covers every k exactly once.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8_t A[4], B[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const uint32_t word = j == 0 ? wcur[a].x : j == 1 ? wcur[a].y : j == 2 ? wcur[a].z : wcur[a].w;
        A[a] = decode_word_bf16(word, j < 2 ? slo[a] : shi[a]);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int row = wm * 128 + b * 32 + l32;
        B[b] = *reinterpret_cast<const bf16x8_t*>(&xs[buf][row][8 * (4 * h + j)]);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[a], B[b], acc[a][b], 0, 0, 0);
    }
    if (more) {
      store_x(buf ^ 1);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        wcur[a] = wnext[a];
        scur[a] = snext[a];
      }
    }
    __syncthreads();
  }

  // Epilogue: C[n][m] fragment, lane holds n = 8*jj + 4h + i, m = l32.
  const float g = global_factor(gs, 0);
  const bool vec_ok = (N % 4) == 0;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t m = m_blk + wm * 128 + b * 32 + l32;
      if (m >= M) continue;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int64_t n = n_blk + wn * 128 + a * 32 + jj * 8 + h * 4;
        __bf16 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (__bf16)(acc[a][b][jj * 4 + i] * g);
        __bf16* p = out + m * N + n;
        if (vec_ok && n + 3 < N) {
          *reinterpret_cast<uint2*>(p) = __builtin_bit_cast(uint2, v);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (n + i < N) p[i] = v[i];
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// MFMA kernel, K % 64 == 0: weight rows split across the wavefronts, all
// operands streamed global -> LDS by the gfx950 load-to-LDS path.
//
// Block tile: 256 weight rows x 256 activation rows, k in slabs of 64.
// Wavefront w owns weight rows [64w, 64w+64) of the tile and all 256
// activation rows, so every packed weight word is decoded exactly once per
// block (into the A operand of two 32x32x16 MFMAs) and feeds 8 activation
// fragments.  Per slab, each wavefront issues 11 direct-to-LDS loads (8 of
// activations, 2 of packed weights, 1 of scale bytes) and nothing passes
// through registers on the way.  The activations move through three LDS
// stages (two slabs in flight while a third is multiplied) and the small
// weight and scale parts through six, queued three slabs ahead: loads
// complete in issue order, so a weight load queued before a slab's
// activations must land by the time those are waited for, and queuing it a
// step earlier gives the weights (streamed from HBM, where the activations
// mostly hit L2) three slab times instead of two.  A stage is released by an
// explicit wait on the vector-memory counter followed by a plain barrier (a
// fenced __syncthreads would drain the prefetches).  The activation and weight
// tiles keep their 16-byte chunks XOR-swizzled by row, which keeps the
// fragment reads free of bank conflicts without padding.
// ----------------------------------------------------------------------------

constexpr int kV3BN = 256;
constexpr int kV3BM = 256;
constexpr int kV3BK = 64;
// Direct-to-LDS loads per wavefront and step: 8 of activations, then 2 of
// packed weights and 1 of scale bytes.  When a step starts, the loads queued
// after that slab's activations are the weights of the same step (3) and the
// whole next step (11): 14 may still be in flight.
constexpr int kV3WaitLoads = 14;

// One pipeline stage in LDS: the activation tile (256 rows x 8 swizzled
// 16-byte chunks, 32 KiB), the packed words (256 rows x 32 bytes, 8 KiB)
// and the scale bytes (256 rows x 4 bytes, 1 KiB) of one slab; a step reads
// the activation part of one activation stage and the weight and scale parts
// of one weight stage.  Each part is its own __shared__ array so the compiler
// can tell a stage being read from the stages being filled and does not wait
// for those loads.
struct V3Stage {
  uint4* x;
  uint4* w;
  uint32_t* s;
};

#define NVFP4_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Bank-conflict-free placement of 16-byte chunks: the 16 lanes served in
// one LDS cycle (consecutive rows, same chunk) land in 16 distinct 16-byte
// bank groups of 256 bytes, and any 8 consecutive rows in 8 distinct groups
// of 128 bytes.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int xslot(int row, int chunk) { return row * 8 + (chunk ^ swz(row)); }
__device__ __forceinline__ int wslot(int row, int half) { return row * 2 + (half ^ ((row >> 3) & 1)); }

// vmcnt(n) with the other counters left unconstrained (gfx9 encoding).
__device__ __forceinline__ void wait_vmem(bool keep_in_flight) {
  if (keep_in_flight)
    __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4) | kV3WaitLoads);
  else
    __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4) | 0);
}

struct V3Src {
  const uint16_t* x[8];      // activation chunk per x load, slab 0 (2-byte elements)
  const uint32_t* w[2];      // packed-word chunk per weight load, slab 0
  const uint8_t* s;          // scale bytes, slab 0
};

// Queues slab `slab` of the activations and slab `wslab` of the weights and
// scales (the same slab, except for the float32 form, whose activation rows
// are three bf16 parts laid end to end against one weight row).
__device__ __forceinline__ void v3_issue_x(const V3Stage& st, const V3Src& src, int64_t slab, int wave) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_global_load_lds(src.x[i] + slab * kV3BK, NVFP4_LDS(&st.x[(i * 4 + wave) * 64]), 16, 0, 0);
}
__device__ __forceinline__ void v3_issue_w(const V3Stage& st, const V3Src& src, int64_t wslab, int wave) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
    __builtin_amdgcn_global_load_lds(src.w[i] + wslab * 8, NVFP4_LDS(&st.w[(i * 4 + wave) * 64]), 16, 0, 0);
  __builtin_amdgcn_global_load_lds(src.s + wslab * 4, NVFP4_LDS(&st.s[wave * 64]), 4, 0, 0);
}

// 2-byte activation types of the MFMA GEMM: bf16 runs the bf16 MFMA on exact
// bf16 weight products, f16 the f16 MFMA on exact f16 products.
template <typename TA> struct V3Ops;
template <> struct V3Ops<__bf16> {
  typedef bf16x8_t vec;
  static __device__ __forceinline__ vec decode(uint32_t w, float s) { return decode_word_bf16(w, s); }
  // Pair P of decode(w, s): elements 2P and 2P + 1 as one dword.
  template <int P>
  static __device__ __forceinline__ uint32_t pair(uint32_t w, float s) {
    const f32x2_t v = e2m1x2_f32<P>(w);
    return pack_bf16_exact(v.x * s, v.y * s);
  }
  static __device__ __forceinline__ f32x16_t mfma(vec a, vec b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct V3Ops<_Float16> {
  typedef f16x8_t vec;
  static __device__ __forceinline__ vec decode(uint32_t w, float s) { return decode_word_f16(w, s); }
  template <int P>
  static __device__ __forceinline__ uint32_t pair(uint32_t w, float s) {
    const _Float16 hs = (_Float16)s;
    const f16x2_t ss = {hs, hs};
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, P) * ss);
  }
  static __device__ __forceinline__ f32x16_t mfma(vec a, vec b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Four 32x32x16 steps over one slab: lane half h supplies word 4h+j (k in
// [8(4h+j), 8(4h+j)+8)) and the activation fragment reads the same chunk.
template <typename TA>
__device__ __forceinline__ void v3_compute(f32x16_t (&acc)[2][8], const V3Stage& st, int wave,
                                           int l32, int h) {
  typedef typename V3Ops<TA>::vec vec;
  uint4 wr[2];
  float slo[2], shi[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int row = wave * 64 + a * 32 + l32;
    wr[a] = st.w[wslot(row, h)];
    const uint32_t sv = st.s[row] >> (16 * h);
    slo[a] = e4m3<0>(sv);
    shi[a] = e4m3<1>(sv);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // All eight activation fragments of this step first, into their own
    // registers, then the multiplies: each read's LDS latency hides behind
    // the reads after it (with one register reused per fragment, every
    // read's latency sits before its two multiplies).  The scheduler would
    // sink each read back to its multiplies, so the order is pinned.
    // (Reading the next step's fragments during this step's multiplies
    // measured slower: the extra 32 registers cost more than they hide.)
    vec B[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) B[b] = __builtin_bit_cast(vec, st.x[xslot(b * 32 + l32, 4 * h + j)]);
    vec A[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const uint32_t word = j == 0 ? wr[a].x : j == 1 ? wr[a].y : j == 2 ? wr[a].z : wr[a].w;
      A[a] = V3Ops<TA>::decode(word, j < 2 ? slo[a] : shi[a]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      acc[0][b] = V3Ops<TA>::mfma(A[0], B[b], acc[0][b]);
      acc[1][b] = V3Ops<TA>::mfma(A[1], B[b], acc[1][b]);
    }
  }
}

// Zeroes the accumulators, then streams `nslabs` slabs through the LDS
// stages (X: activations, three; W: weights and scales, six) and multiplies
// them.  One step: wait for slab s, release the stages read in earlier
// steps, queue the activations of slab s + 2 and the weights of slab s + 3
// (the last slab again near the end, so the issue is unconditional and the
// compiler keeps exact track of what is in flight), multiply slab s.  The load counter is
// drained before returning, so no load-to-LDS lands after the caller moves
// on.  Weight rows hold wslabs slabs; activation slab s meets weight slab
// s mod wslabs (the same slab unless the activation rows are longer).
template <typename TA>
__device__ __forceinline__ void v3_mainloop(f32x16_t (&acc)[2][8], const V3Stage (&X)[3], const V3Stage (&W)[6],
                                            const V3Src& src, int64_t nslabs, int64_t wslabs,
                                            int wave, int l32, int h) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  auto wsl = [&](int64_t q) { return q < wslabs ? q : q % wslabs; };
  auto cl = [&](int64_t q) { return q < nslabs ? q : nslabs - 1; };
  v3_issue_w(W[0], src, 0, wave);
  v3_issue_x(X[0], src, 0, wave);
  v3_issue_w(W[1], src, wsl(cl(1)), wave);
  v3_issue_x(X[1], src, cl(1), wave);
  v3_issue_w(W[2], src, wsl(cl(2)), wave);

#define NVFP4_V3_STEP(S, XI, WI)                                                     \
  do {                                                                               \
    wait_vmem(true);                                                                 \
    __builtin_amdgcn_s_barrier();                                                    \
    v3_issue_x(X[((XI) + 2) % 3], src, cl((S) + 2), wave);                           \
    v3_issue_w(W[((WI) + 3) % 6], src, wsl(cl((S) + 3)), wave);                      \
    const V3Stage cur{X[XI].x, W[WI].w, W[WI].s};                                    \
    v3_compute<TA>(acc, cur, wave, l32, h);                                          \
  } while (0)

  int64_t s = 0;
  for (; s + 6 <= nslabs; s += 6) {
    NVFP4_V3_STEP(s, 0, 0);
    NVFP4_V3_STEP(s + 1, 1, 1);
    NVFP4_V3_STEP(s + 2, 2, 2);
    NVFP4_V3_STEP(s + 3, 0, 3);
    NVFP4_V3_STEP(s + 4, 1, 4);
    NVFP4_V3_STEP(s + 5, 2, 5);
  }
  if (s < nslabs) NVFP4_V3_STEP(s, 0, 0);
  if (s + 1 < nslabs) NVFP4_V3_STEP(s + 1, 1, 1);
  if (s + 2 < nslabs) NVFP4_V3_STEP(s + 2, 2, 2);
  if (s + 3 < nslabs) NVFP4_V3_STEP(s + 3, 0, 3);
  if (s + 4 < nslabs) NVFP4_V3_STEP(s + 4, 1, 4);
  wait_vmem(false);   // no load-to-LDS may land after this point
#undef NVFP4_V3_STEP
}

// Epilogue of a plain tile: fragment (a, b) holds C[n][m] with n = 8*jj +
// 4h + i, m = l32.  A swap between the lane halves gives lane h the eight
// consecutive n 16p + 8h .. 16p + 8h + 7 of jj pair p, stored as one 16-byte
// write.
template <typename TO>
__device__ __forceinline__ void v3_store_tile(const f32x16_t (&acc)[2][8], TO* __restrict__ out, int64_t M,
                                              int64_t N, int64_t m_blk, int64_t n_blk, float g, int wave,
                                              int l32, int h) {
  if constexpr (sizeof(TO) == 4) {
    // float32 output: lane h holds n = 8 jj + 4h .. 8 jj + 4h + 3 of each
    // jj, one 16-byte store each.
    const bool vec4 = (N % 4) == 0;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int64_t m = m_blk + b * 32 + l32;
        if (m >= M) continue;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int64_t n = n_blk + wave * 64 + a * 32 + jj * 8 + h * 4;
          const float v[4] = {acc[a][b][jj * 4] * g, acc[a][b][jj * 4 + 1] * g, acc[a][b][jj * 4 + 2] * g,
                              acc[a][b][jj * 4 + 3] * g};
          TO* q = out + m * N + n;
          if (vec4 && n + 3 < N) {
            *reinterpret_cast<float4*>(q) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (n + i < N) q[i] = v[i];
          }
        }
      }
  } else {
    const bool vec_ok = (N % 8) == 0;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int64_t m = m_blk + b * 32 + l32;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          uint32_t r0[2], r1[2];
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const TO lo0 = (TO)(acc[a][b][(2 * p) * 4 + 2 * d] * g);
            const TO hi0 = (TO)(acc[a][b][(2 * p) * 4 + 2 * d + 1] * g);
            const TO lo1 = (TO)(acc[a][b][(2 * p + 1) * 4 + 2 * d] * g);
            const TO hi1 = (TO)(acc[a][b][(2 * p + 1) * 4 + 2 * d + 1] * g);
            r0[d] = (uint32_t)__builtin_bit_cast(uint16_t, lo0) | ((uint32_t)__builtin_bit_cast(uint16_t, hi0) << 16);
            r1[d] = (uint32_t)__builtin_bit_cast(uint16_t, lo1) | ((uint32_t)__builtin_bit_cast(uint16_t, hi1) << 16);
          }
          const auto s0 = __builtin_amdgcn_permlane32_swap(r0[0], r1[0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(r0[1], r1[1], false, false);
          const uint4 v = make_uint4(s0[0], s1[0], s0[1], s1[1]);
          const int64_t n = n_blk + wave * 64 + a * 32 + 16 * p + 8 * h;
          if (m >= M) continue;
          TO* q = out + m * N + n;
          if (vec_ok && n + 7 < N) {
            *reinterpret_cast<uint4*>(q) = v;
          } else {
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
              if (n + i < N) q[i] = __builtin_bit_cast(TO, (uint16_t)(wv[i / 2] >> (16 * (i % 2))));
          }
        }
      }
    }
  }
}

// Epilogue of a gated tile: fragment (0, b) holds the gate sums and (1, b)
// the up sums of the same (feature, row) pairs (feature n_blk + 32 wave +
// 8 jj + 4 h + i, row m_blk + 32 b + l32); out = act(g_gate gate) (g_up up),
// rounded once, as one 16-byte store of eight features per row.
template <int kAct>
__device__ __forceinline__ void v3_store_glu(const f32x16_t (&acc)[2][8], __bf16* __restrict__ out, int64_t M,
                                             int64_t N, int64_t m_blk, int64_t n_blk, float gg, float gu, int wave,
                                             int l32, int h) {
  const bool vec_ok = (N % 8) == 0;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int64_t m = m_blk + b * 32 + l32;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      uint32_t r0[2], r1[2];
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        float v[4];
        const int idx[4] = {(2 * p) * 4 + 2 * d, (2 * p) * 4 + 2 * d + 1, (2 * p + 1) * 4 + 2 * d,
                            (2 * p + 1) * 4 + 2 * d + 1};
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = glu_act_t<kAct>(acc[0][b][idx[e]] * gg) * (acc[1][b][idx[e]] * gu);
        r0[d] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[0]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[1]) << 16);
        r1[d] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[3]) << 16);
      }
      const auto s0 = __builtin_amdgcn_permlane32_swap(r0[0], r1[0], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(r0[1], r1[1], false, false);
      const uint4 v = make_uint4(s0[0], s1[0], s0[1], s1[1]);
      const int64_t f = n_blk + wave * 32 + 16 * p + 8 * h;
      if (m >= M) continue;
      __bf16* q = out + m * N + f;
      if (vec_ok && f + 7 < N) {
        *reinterpret_cast<uint4*>(q) = v;
      } else {
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (f + i < N) q[i] = __builtin_bit_cast(__bf16, (uint16_t)(wv[i / 2] >> (16 * (i % 2))));
      }
    }
  }
}

// 32-bit byte offsets of a plain tile's slab-0 loads from the operand bases
// (as in gemm_mfma_v3_kernel).  The loads are buffer loads to LDS: a buffer
// resource per operand, the fixed lane offset in a register and the slab's
// offset in a scalar, so there is no address arithmetic per load and no load
// waits for an earlier one to release a shared address register (with
// 64-bit addresses built per load in one register pair, issuing a slab's 11
// loads took ~580 cycles).
struct V3Off {
  uint32_t x[8];
  uint32_t w[2];
  uint32_t s;
};

typedef __amdgpu_buffer_rsrc_t v3_rsrc_t;

__device__ __forceinline__ v3_rsrc_t v3_buffer(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

struct V3Base {
  v3_rsrc_t x, w, s;
};

// The next slabs' 11 loads of a step (8 activation, 2 weight, 1 scale
// copies), issued one at a time between the step's multiplies.  kLaneScale:
// the scale copy is a global load from a per-lane address (the gated form,
// whose scale lanes read two planes), the others buffer loads.
template <bool kLaneScale = false>
struct V3pIssueT {
  const V3Stage* xs;
  const V3Stage* ws;
  const V3Off* xo;
  const V3Off* wo;
  uint32_t xslab, wslab;
  int wave;
  const V3Base* b;
  const uint8_t* lane_s;   // kLaneScale: this lane's scale row at slab 0
  __device__ __forceinline__ void operator()(int k) const {
    if (k < 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b->x, NVFP4_LDS(&xs->x[(k * 4 + wave) * 64]), 16, xo->x[k],
                                               xslab * (kV3BK * 2), 0, 0);
    else if (k < 10)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b->w, NVFP4_LDS(&ws->w[((k - 8) * 4 + wave) * 64]), 16, wo->w[k - 8],
                                               wslab * 32, 0, 0);
    else if constexpr (kLaneScale)
      __builtin_amdgcn_global_load_lds(lane_s + (size_t)wslab * 4, NVFP4_LDS(&ws->s[wave * 64]), 4, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b->s, NVFP4_LDS(&ws->s[wave * 64]), 4, wo->s, wslab * 4, 0, 0);
  }
};
typedef V3pIssueT<false> V3pIssue;

// v3_compute with the step's loads spread over its multiplies, in issue
// order: load k goes out after multiply kV3pLoadAfter[k] of the step's 64
// (-1: before the first fragment reads), so no multiply waits for the whole
// step's loads to enter the memory pipeline, and the loads still leave early
// in the step.
constexpr int kV3pLoadAfter[11] = {1, 3, 5, 7, 9, 11, 13, 15, 17, 19, 21};
template <typename TA, typename Issue>
__device__ __forceinline__ void v3p_compute(f32x16_t (&acc)[2][8], const V3Stage& st, int wave, int l32, int h,
                                            const Issue& iss) {
  typedef typename V3Ops<TA>::vec vec;
  uint4 wr[2];
  float slo[2], shi[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int row = wave * 64 + a * 32 + l32;
    wr[a] = st.w[wslot(row, h)];
    const uint32_t sv = st.s[row] >> (16 * h);
    slo[a] = e4m3<0>(sv);
    shi[a] = e4m3<1>(sv);
  }
#pragma unroll
  for (int k = 0; k < 11; ++k)
    if (kV3pLoadAfter[k] < 0) iss(k);
  // Each sub-step multiplies by A operand (weight rows 0-31 against the
  // eight fragments, then rows 32-63), so with no extra registers: the
  // second A is decoded one dword (pair) after each of the first four
  // multiplies, and during the second half each fragment register is
  // refilled with the next sub-step's fragment once its last multiply is
  // issued and the next sub-step's first A is decoded one pair at a time
  // (no more than four VALU instructions between two multiplies; a whole
  // word is sixteen).  Each accumulator still takes one multiply per
  // sub-step in k order, so the sums are those of v3_compute.
  auto word = [&](int j, int a) { return j == 0 ? wr[a].x : j == 1 ? wr[a].y : j == 2 ? wr[a].z : wr[a].w; };
  auto rdB = [&](int j, int b) { return __builtin_bit_cast(vec, st.x[xslot(b * 32 + l32, 4 * h + j)]); };
  auto pair = [&](uint32_t (&A)[4], int j, int a, int p) {
    const uint32_t w = word(j, a);
    const float sc = j < 2 ? slo[a] : shi[a];
    switch (p) {
      case 0: A[0] = V3Ops<TA>::template pair<0>(w, sc); break;
      case 1: A[1] = V3Ops<TA>::template pair<1>(w, sc); break;
      case 2: A[2] = V3Ops<TA>::template pair<2>(w, sc); break;
      default: A[3] = V3Ops<TA>::template pair<3>(w, sc); break;
    }
  };
  vec B[8];
  uint32_t A0[4], A1[4];
#pragma unroll
  for (int b = 0; b < 8; ++b) B[b] = rdB(0, b);
#pragma unroll
  for (int p = 0; p < 4; ++p) pair(A0, 0, 0, p);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        acc[a][b] = V3Ops<TA>::mfma(__builtin_bit_cast(vec, a == 0 ? A0 : A1), B[b], acc[a][b]);
#pragma unroll
        for (int k = 0; k < 11; ++k)
          if (kV3pLoadAfter[k] == 16 * j + 8 * a + b) {
            __builtin_amdgcn_sched_barrier(0);
            iss(k);
            __builtin_amdgcn_sched_barrier(0);
          }
        if (a == 0 && b < 4) {
          __builtin_amdgcn_sched_barrier(0);
          pair(A1, j, 1, b);
          __builtin_amdgcn_sched_barrier(0);
        } else if (a == 1 && j < 3) {
          __builtin_amdgcn_sched_barrier(0);
          B[b] = rdB(j + 1, b);
          if (b < 4) pair(A0, j + 1, 0, b);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
}

// v3_mainloop with buffer loads spread between the multiplies, as in the
// persistent launch (same stages, waits and issue order, so the same sums).
// Activation slab s meets weight slab s mod wslabs; the loads past the last
// slab queue it again.  `lane_s`: the gated form's per-lane scale rows.
template <typename TA, bool kLaneScale>
__device__ __forceinline__ void v3b_mainloop(f32x16_t (&acc)[2][8], const V3Stage (&X)[3], const V3Stage (&W)[6],
                                             const V3Base& b, const V3Off& o, const uint8_t* lane_s,
                                             int64_t nslabs, int64_t wslabs, int wave, int l32, int h) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][c][i] = 0.0f;
  auto wsl = [&](int64_t q) { return (uint32_t)(q < wslabs ? q : q % wslabs); };
  auto cl = [&](int64_t q) { return q < nslabs ? q : nslabs - 1; };
  typedef V3pIssueT<kLaneScale> Issue;
  {
    const Issue p0{&X[0], &W[0], &o, &o, 0u, 0u, wave, &b, lane_s};
    const Issue p1{&X[1], &W[1], &o, &o, (uint32_t)cl(1), wsl(cl(1)), wave, &b, lane_s};
    const Issue p2{&X[2], &W[2], &o, &o, (uint32_t)cl(2), wsl(cl(2)), wave, &b, lane_s};
#pragma unroll
    for (int k = 8; k < 11; ++k) p0(k);
#pragma unroll
    for (int k = 0; k < 8; ++k) p0(k);
#pragma unroll
    for (int k = 8; k < 11; ++k) p1(k);
#pragma unroll
    for (int k = 0; k < 8; ++k) p1(k);
#pragma unroll
    for (int k = 8; k < 11; ++k) p2(k);
  }
#define NVFP4_V3B_STEP(S, XI, WI)                                                    \
  do {                                                                               \
    wait_vmem(true);                                                                 \
    __builtin_amdgcn_s_barrier();                                                    \
    const Issue iss{&X[((XI) + 2) % 3], &W[((WI) + 3) % 6], &o, &o, (uint32_t)cl((S) + 2), \
                    wsl(cl((S) + 3)), wave, &b, lane_s};                             \
    const V3Stage cur{X[XI].x, W[WI].w, W[WI].s};                                    \
    v3p_compute<TA>(acc, cur, wave, l32, h, iss);                                    \
  } while (0)
  int64_t s = 0;
  for (; s + 6 <= nslabs; s += 6) {
    NVFP4_V3B_STEP(s, 0, 0);
    NVFP4_V3B_STEP(s + 1, 1, 1);
    NVFP4_V3B_STEP(s + 2, 2, 2);
    NVFP4_V3B_STEP(s + 3, 0, 3);
    NVFP4_V3B_STEP(s + 4, 1, 4);
    NVFP4_V3B_STEP(s + 5, 2, 5);
  }
  if (s < nslabs) NVFP4_V3B_STEP(s, 0, 0);
  if (s + 1 < nslabs) NVFP4_V3B_STEP(s + 1, 1, 1);
  if (s + 2 < nslabs) NVFP4_V3B_STEP(s + 2, 2, 2);
  if (s + 3 < nslabs) NVFP4_V3B_STEP(s + 3, 0, 3);
  if (s + 4 < nslabs) NVFP4_V3B_STEP(s + 4, 1, 4);
  wait_vmem(false);   // no load-to-LDS may land after this point
#undef NVFP4_V3B_STEP
}

// What one block computes.
//   kV3Plain: out tile = round(g * x W^T) over 256 weight rows.
//   kV3Split: the block multiplies slabs [split * per_split, ...) of its tile
//             only and writes the unscaled float32 partial to ws[split][M][N];
//             a second kernel adds the partials in split order, applies g and
//             rounds.
//   kV3Glu:   the gated MLP projection.  N is the feature count F and a tile
//             covers 128 features: the first 32-row MFMA tile of wavefront w
//             holds gate rows f0 + 32w .. f0 + 32w + 31 (plane w, sc, gs) and
//             the second the up rows of the same features (wu, scu, gsu), so
//             each lane ends with the gate and up sums of the same outputs and
//             the epilogue forms act(g_gate * gate) * (g_up * up) in float32,
//             act being the template argument kAct.
//   kV3GluSplit: tiles tile0 .. tile0 + tiles_total - 1 of the gated
//             projection, each shared by `splits` blocks along K as in
//             kV3Split; block (split, t) writes its unscaled float32 gate and
//             up sums to ws[split][t][256 rows][256 tile rows], and
//             glu_tail_reduce_kernel finishes them.
constexpr int kV3Plain = 0, kV3Split = 1, kV3Glu = 2, kV3GluSplit = 3;

//
// TA is the 2-byte activation type (bf16 or f16, the MFMA operand type) and
// TO the output type.  K is the activation row length and wslabs the number
// of 64-element slabs of a weight row; activation slab s meets weight slab
// s mod wslabs.  They are equal (K = 64 wslabs) except in the float32 form,
// whose activation rows are three bf16 parts laid end to end (K = 192
// wslabs): one plane multiplies each part and the three sums accumulate
// together.
// kBuf: every operand below 2^31 bytes, so the loads are buffer loads from
// 32-bit offsets, spread between the multiplies (v3b_mainloop); otherwise
// global loads from 64-bit addresses, all issued after each step's barrier.
template <int kMode, int kAct = 0, typename TA = __bf16, typename TO = __bf16, bool kBuf = false>
__global__ __launch_bounds__(kMfmaThreads, 1) void gemm_mfma_v3_kernel(
    const TA* __restrict__ x, const uint32_t* __restrict__ w, const uint8_t* __restrict__ sc,
    const float* __restrict__ gs, TO* __restrict__ out, int64_t M, int64_t K, int64_t N,
    int64_t tiles_m, int64_t tiles_total, int64_t per_split, float* __restrict__ ws,
    const uint32_t* __restrict__ wu, const uint8_t* __restrict__ scu, const float* __restrict__ gsu,
    int64_t tile0, int64_t wslabs) {
  constexpr bool kSplit = kMode == kV3Split || kMode == kV3GluSplit;
  constexpr bool kGlu = kMode == kV3Glu || kMode == kV3GluSplit;
  __shared__ uint4 x0[kV3BM * 8], x1[kV3BM * 8], x2[kV3BM * 8];
  __shared__ uint4 w0[kV3BN * 2], w1[kV3BN * 2], w2[kV3BN * 2], w3[kV3BN * 2], w4[kV3BN * 2], w5[kV3BN * 2];
  __shared__ uint32_t s0[kV3BN], s1[kV3BN], s2[kV3BN], s3[kV3BN], s4[kV3BN], s5[kV3BN];
  const V3Stage st0{x0, w0, s0}, st1{x1, w1, s1}, st2{x2, w2, s2};
  const V3Stage XS[3] = {st0, st1, st2};   // only .x is read
  const V3Stage WS[6] = {st0, st1, st2, {x0, w3, s3}, {x0, w4, s4}, {x0, w5, s5}};   // only .w and .s

  // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs;
  // each XCD gets a contiguous run of logical tiles (activation tiles
  // fastest), so the tiles sharing weight rows share that XCD's L2.
  // With a split, logical = split * tiles_total + tile: an XCD's run holds
  // neighbouring tiles of one split.
  const int64_t per_xcd = (int64_t)gridDim.x / 8;
  const int64_t logical = ((int64_t)blockIdx.x % 8) * per_xcd + (int64_t)blockIdx.x / 8;
  const int64_t all_slabs = K / kV3BK;
  const int64_t split = kSplit ? logical / tiles_total : 0;
  const int64_t tloc = kSplit ? logical - split * tiles_total : logical;
  const int64_t first_slab = split * per_split;
  if (tloc >= tiles_total || first_slab >= all_slabs) return;  // whole block, before any barrier
  const int64_t tile = tile0 + tloc;
  const int64_t m_blk = (tile % tiles_m) * kV3BM;
  const int64_t n_blk = (tile / tiles_m) * (kGlu ? kV3BN / 2 : kV3BN);

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t kw = wslabs * (kV3BK / 8), ks = wslabs * (kV3BK / 16);   // weight and scale row lengths
  const int64_t nslabs = kSplit ? (all_slabs - first_slab < per_split ? all_slabs - first_slab : per_split)
                                : all_slabs;

  f32x16_t acc[2][8];
  if constexpr (kBuf) {
    // Byte offsets of this lane's loads for slab 0 (rows past M or N re-read
    // the last row; their results are never stored).
    V3Off o;
    const uint8_t* lane_s = nullptr;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int slot = (i * 4 + wave) * 64 + lane;
      const int r = slot >> 3, c = (slot & 7) ^ swz(r);
      int64_t m = m_blk + r;
      if (m >= M) m = M - 1;
      o.x[i] = (uint32_t)((m * K + c * 8 + first_slab * kV3BK) * 2);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = (i * 4 + wave) * 64 + lane;
      const int r = q >> 1, half = (q & 1) ^ ((r >> 3) & 1);
      int64_t n = kGlu ? n_blk + (r >> 6) * 32 + (r & 31) : n_blk + r;   // gated: plane (r >> 5) & 1 = wave & 1
      if (n >= N) n = N - 1;
      o.w[i] = (uint32_t)((n * kw + 4 * half + first_slab * 8) * 4);
    }
    if constexpr (kGlu) {
      int64_t f = n_blk + wave * 32 + (lane & 31);
      if (f >= N) f = N - 1;
      lane_s = ((lane >> 5) ? scu : sc) + f * ks + first_slab * 4;
      o.s = 0;
    } else {
      int64_t n = n_blk + wave * 64 + lane;
      if (n >= N) n = N - 1;
      o.s = (uint32_t)(n * ks + first_slab * 4);
    }
    const V3Base b{v3_buffer(x, M * K * 2), v3_buffer((kGlu && (wave & 1)) ? wu : w, N * kw * 4),
                   v3_buffer(sc, N * ks)};
    v3b_mainloop<TA, kGlu>(acc, XS, WS, b, o, lane_s, nslabs, wslabs, wave, l32, h);
  } else {
    // Source addresses of this lane's loads for slab 0.  Rows past M or N
    // re-read the last row (their results are never stored).
    V3Src src;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int slot = (i * 4 + wave) * 64 + lane;
      const int r = slot >> 3, c = (slot & 7) ^ swz(r);
      int64_t m = m_blk + r;
      if (m >= M) m = M - 1;
      src.x[i] = reinterpret_cast<const uint16_t*>(x) + m * K + c * 8;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = (i * 4 + wave) * 64 + lane;
      const int r = q >> 1, half = (q & 1) ^ ((r >> 3) & 1);   // inverse of wslot
      if constexpr (kGlu) {
        // Tile row r = 64 w' + 32 a + l: feature n_blk + 32 w' + l of the gate
        // (a = 0) or up (a = 1) plane.
        int64_t f = n_blk + (r >> 6) * 32 + (r & 31);
        if (f >= N) f = N - 1;
        src.w[i] = (((r >> 5) & 1) ? wu : w) + f * kw + 4 * half;
      } else {
        int64_t n = n_blk + r;
        if (n >= N) n = N - 1;
        src.w[i] = w + n * kw + 4 * half;
      }
    }
    if constexpr (kGlu) {
      int64_t f = n_blk + wave * 32 + (lane & 31);
      if (f >= N) f = N - 1;
      src.s = ((lane >> 5) ? scu : sc) + f * ks;
    } else {
      int64_t n = n_blk + wave * 64 + lane;
      if (n >= N) n = N - 1;
      src.s = sc + n * ks;
    }
    if (kSplit) {
#pragma unroll
      for (int i = 0; i < 8; ++i) src.x[i] += first_slab * kV3BK;
#pragma unroll
      for (int i = 0; i < 2; ++i) src.w[i] += first_slab * 8;
      src.s += first_slab * 4;
    }

    v3_mainloop<TA>(acc, XS, WS, src, nslabs, wslabs, wave, l32, h);
  }

  if constexpr (kMode == kV3GluSplit) {
    // Tile-local partial: fragment (a, b) holds C[n][m] with tile row
    // n = 64 wave + 32a + 8jj + 4h + i and row m = 32b + l32; every row of the
    // 256 x 256 slice is written (the reduction skips rows past M or F).
    float* wsp = ws + ((split * tiles_total + tloc) << 16);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 8; ++b)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *reinterpret_cast<float4*>(wsp + (b * 32 + l32) * 256 + wave * 64 + a * 32 + jj * 8 + h * 4) =
              make_float4(acc[a][b][jj * 4], acc[a][b][jj * 4 + 1], acc[a][b][jj * 4 + 2], acc[a][b][jj * 4 + 3]);
    return;
  }
  if constexpr (kSplit) {
    // Partial: fragment (a, b) holds C[n][m] with n = 8*jj + 4h + i, m =
    // l32; four consecutive n per jj go out as one 16-byte store.
    float* wsp = ws + split * M * N;
    const bool vec4 = (N % 4) == 0;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int64_t m = m_blk + b * 32 + l32;
        if (m >= M) continue;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int64_t n = n_blk + wave * 64 + a * 32 + jj * 8 + h * 4;
          float* p = wsp + m * N + n;
          if (vec4 && n + 3 < N) {
            *reinterpret_cast<float4*>(p) =
                make_float4(acc[a][b][jj * 4], acc[a][b][jj * 4 + 1], acc[a][b][jj * 4 + 2], acc[a][b][jj * 4 + 3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (n + i < N) p[i] = acc[a][b][jj * 4 + i];
          }
        }
      }
    }
    return;
  }
  if constexpr (kGlu) {
    v3_store_glu<kAct>(acc, out, M, N, m_blk, n_blk, global_factor(gs, 0), global_factor(gsu, 0), wave, l32, h);
    return;
  }
  v3_store_tile<TO>(acc, out, M, N, m_blk, n_blk, global_factor(gs, 0), wave, l32, h);
}

// ----------------------------------------------------------------------------
// Persistent form of the plain tile (2-byte activations, K a multiple of 384
// with at least 12 slabs).  The plain launch starts every tile of a round on
// every compute unit at once, and the first slabs' loads then queue behind
// each other before any multiply can start.  Here one block per compute unit
// walks its tiles, and the last three steps of a tile queue the next tile's
// first two activation slabs and three weight slabs into exactly the stages
// its first steps read (slab counts are multiples of the stage rings), so
// the next tile's start-up overlaps this tile's last multiplies and its
// epilogue.  Each XCD owns a contiguous run of tiles (activation tiles
// fastest), its blocks taking them round-robin, as in the plain launch.
// ----------------------------------------------------------------------------

// kGlu: the gated tile (128 features from n_blk; wavefront w's rows come
// from the gate plane for even w and the up plane for odd w, feature
// n_blk + 32 (r / 64) + r % 32 for tile row r), and `ls` the lane's scale row
// at slab 0 (the gate plane's for lanes 0-31, the up plane's for 32-63).
// K is the activation row length, Kw the weight row length (K except for
// float32 activations, whose rows are three bf16 parts: K = 3 Kw).
template <bool kGlu = false>
__device__ __forceinline__ void v3p_offsets(V3Off& o, int64_t M, int64_t K, int64_t N, int64_t m_blk,
                                            int64_t n_blk, int wave, int lane, const uint8_t* sc = nullptr,
                                            const uint8_t* scu = nullptr, const uint8_t** ls = nullptr,
                                            int64_t Kw = 0) {
  if (Kw == 0) Kw = K;
  const int64_t kw = Kw / 8, ks = Kw / 16;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int slot = (i * 4 + wave) * 64 + lane;
    const int r = slot >> 3, c = (slot & 7) ^ swz(r);
    int64_t m = m_blk + r;
    if (m >= M) m = M - 1;
    o.x[i] = (uint32_t)((m * K + c * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = (i * 4 + wave) * 64 + lane;
    const int r = q >> 1, half = (q & 1) ^ ((r >> 3) & 1);
    int64_t n = kGlu ? n_blk + (r >> 6) * 32 + (r & 31) : n_blk + r;
    if (n >= N) n = N - 1;
    o.w[i] = (uint32_t)((n * kw + 4 * half) * 4);
  }
  if constexpr (kGlu) {
    int64_t f = n_blk + wave * 32 + (lane & 31);
    if (f >= N) f = N - 1;
    *ls = ((lane >> 5) ? scu : sc) + f * ks;
    o.s = 0;
  } else {
    int64_t n = n_blk + wave * 64 + lane;
    if (n >= N) n = N - 1;
    o.s = (uint32_t)(n * ks);
  }
}

// Fragment registers of the persistent launch, carried from one step to the
// next: two sets of eight activation fragments and two decoded A operands
// (set j & 1 feeds sub-step j), and the weight words and block scales of the
// step being decoded.
template <typename TA>
struct V3Frags {
  typename V3Ops<TA>::vec B[2][8];
  uint32_t A[2][2][4];
  uint4 wr[2];
  uint32_t sr[2];
  float slo[2], shi[2];
};

// The step's words and scale words from LDS (v3q_words), then the two block
// scales of each row decoded (v3q_scales), kept apart so that the LDS reads
// can be in flight during multiplies before anything waits for them.
template <typename TA>
__device__ __forceinline__ void v3q_words(V3Frags<TA>& f, const V3Stage& st, int wave, int l32, int h) {
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int row = wave * 64 + a * 32 + l32;
    f.wr[a] = st.w[wslot(row, h)];
    f.sr[a] = st.s[row];
  }
}
template <typename TA>
__device__ __forceinline__ void v3q_scales(V3Frags<TA>& f, int h) {
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const uint32_t sv = f.sr[a] >> (16 * h);
    f.slo[a] = e4m3<0>(sv);
    f.shi[a] = e4m3<1>(sv);
  }
}
// Pair P of sub-step j's A operand for weight rows a (the word's elements
// 2P, 2P + 1), into set n: four VALU instructions, so that one pair fits in
// the shadow of one multiply (a whole word's sixteen in one place would
// hold the next multiply back).
template <typename TA, int P>
__device__ __forceinline__ void v3q_pair(V3Frags<TA>& f, int n, int j, int a) {
  const uint32_t word = j == 0 ? f.wr[a].x : j == 1 ? f.wr[a].y : j == 2 ? f.wr[a].z : f.wr[a].w;
  f.A[n][a][P] = V3Ops<TA>::template pair<P>(word, j < 2 ? f.slo[a] : f.shi[a]);
}
template <typename TA>
__device__ __forceinline__ void v3q_pair_any(V3Frags<TA>& f, int n, int j, int a, int p) {
  switch (p) {
    case 0: v3q_pair<TA, 0>(f, n, j, a); break;
    case 1: v3q_pair<TA, 1>(f, n, j, a); break;
    case 2: v3q_pair<TA, 2>(f, n, j, a); break;
    default: v3q_pair<TA, 3>(f, n, j, a); break;
  }
}
template <typename TA>
__device__ __forceinline__ typename V3Ops<TA>::vec v3q_A(const V3Frags<TA>& f, int c, int a) {
  return __builtin_bit_cast(typename V3Ops<TA>::vec, f.A[c][a]);
}
template <typename TA>
__device__ __forceinline__ typename V3Ops<TA>::vec v3q_rdB(const V3Stage& st, int j, int b, int l32, int h) {
  return __builtin_bit_cast(typename V3Ops<TA>::vec, st.x[xslot(b * 32 + l32, 4 * h + j)]);
}

// A step's first operands: words, scales, sub-step 0's A operands and
// fragments of stage `st` into set 0.
template <typename TA>
__device__ __forceinline__ void v3q_first(V3Frags<TA>& f, const V3Stage& st, int wave, int l32, int h) {
  v3q_words<TA>(f, st, wave, l32, h);
#pragma unroll
  for (int b = 0; b < 8; ++b) f.B[0][b] = v3q_rdB<TA>(st, 0, b, l32, h);
  v3q_scales<TA>(f, h);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int p = 0; p < 4; ++p) v3q_pair_any<TA>(f, 0, 0, a, p);
}

// One step of the persistent launch, entered with sub-step 0's operands of
// stage `st` in set 0.  Sub-step j + 1's fragments are read and its words
// decoded into the other set between sub-step j's multiplies, and the
// step's loads go out between its multiplies as in v3p_compute.  With
// kNext, the wait and barrier that make the next slab readable come after
// the first multiply pair of sub-step 3 (every fragment of this step is in
// registers by then), and the rest of sub-step 3 reads the next step's
// words, scales and sub-step 0 operands from stage `nx` into set 0, so the
// next step starts with its multiplies.  The next step's loads overwrite
// only stages that every wavefront has finished reading at that barrier.
template <typename TA, bool kNext, typename Issue>
__device__ __forceinline__ void v3q_step(f32x16_t (&acc)[2][8], V3Frags<TA>& f, const V3Stage& st,
                                         const V3Stage& nx, int wave, int l32, int h, const Issue& iss) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = j & 1, n = c ^ 1;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        acc[a][b] = V3Ops<TA>::mfma(v3q_A<TA>(f, c, a), f.B[c][b], acc[a][b]);
        const int m = 2 * b + a;   // multiplies issued in this sub-step, minus one
#pragma unroll
        for (int k = 0; k < 11; ++k)
          if (kV3pLoadAfter[k] == 16 * j + m) {
            __builtin_amdgcn_sched_barrier(0);
            iss(k);
            __builtin_amdgcn_sched_barrier(0);
          }
        if (j < 3) {
          // sub-step j + 1: fragment b after the first multiply of pair b,
          // the A operands one dword (pair) after each odd multiply
          if (a == 0) {
            __builtin_amdgcn_sched_barrier(0);
            f.B[n][b] = v3q_rdB<TA>(st, j + 1, b, l32, h);
            __builtin_amdgcn_sched_barrier(0);
          } else {
            __builtin_amdgcn_sched_barrier(0);
            v3q_pair_any<TA>(f, n, j + 1, b >> 2, b & 3);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else if constexpr (kNext) {
          if (m == 1) {
            // every LDS read of this step has returned (lgkmcnt 0) and
            // this wavefront's part of the next slab has landed (vmcnt 14:
            // the step's 11 loads went out in sub-steps 0 and 1); then the
            // block meets
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt((0x7 << 4) | kV3WaitLoads);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            v3q_words<TA>(f, nx, wave, l32, h);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (m == 5) {
            __builtin_amdgcn_sched_barrier(0);
            v3q_scales<TA>(f, h);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (b >= 1 && a == 0) {
            __builtin_amdgcn_sched_barrier(0);
            f.B[n][b - 1] = v3q_rdB<TA>(nx, 0, b - 1, l32, h);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (m >= 7 && m <= 14) {
            // the next step's sub-step 0 A operands, one dword per multiply
            __builtin_amdgcn_sched_barrier(0);
            v3q_pair_any<TA>(f, n, 0, (m - 7) >> 2, (m - 7) & 3);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
  }
  if constexpr (kNext) f.B[0][7] = v3q_rdB<TA>(nx, 0, 7, l32, h);
}

// One tile's slabs (nslabs % 6 == 0, nslabs >= 12).  `issued`: the first
// slabs were queued by the previous tile.  With has_next, the last three
// steps queue the next tile's slabs 0-1 (activations) and 0-2 (weights) from
// the offsets `no`, and the loads stay in flight when this returns;
// otherwise they queue this tile's last slab again and the load counter is
// drained.
// kWrap: activation slab s meets weight slab s mod wslabs (float32
// activations: three bf16 parts per row against one plane row).
template <typename TA, bool kGlu = false, bool kWrap = false>
__device__ __forceinline__ void v3p_mainloop(f32x16_t (&acc)[2][8], const V3Stage (&X)[3], const V3Stage (&W)[6],
                                             const V3Base& b, const V3Off& o, const V3Off& no, bool has_next,
                                             bool issued, uint32_t nslabs, int wave, int l32, int h,
                                             const uint8_t* ls = nullptr, const uint8_t* nls = nullptr,
                                             uint32_t wslabs = 0) {
  typedef V3pIssueT<kGlu> Issue;
  auto wsl = [&](uint32_t q) -> uint32_t {
    if constexpr (kWrap) return q < wslabs ? q : q % wslabs;
    return q;
  };
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][c][i] = 0.0f;
  if (!issued) {
    // weights of slab 0, activations of slab 0, weights of slab 1, ...
    const Issue p0{&X[0], &W[0], &o, &o, 0u, 0u, wave, &b, ls};
    const Issue p1{&X[1], &W[1], &o, &o, 1u, 1u, wave, &b, ls};
    const Issue p2{&X[2], &W[2], &o, &o, 2u, 2u, wave, &b, ls};
#pragma unroll
    for (int k = 8; k < 11; ++k) p0(k);
#pragma unroll
    for (int k = 0; k < 8; ++k) p0(k);
#pragma unroll
    for (int k = 8; k < 11; ++k) p1(k);
#pragma unroll
    for (int k = 0; k < 8; ++k) p1(k);
#pragma unroll
    for (int k = 8; k < 11; ++k) p2(k);
  }
  // slab 0 readable, its operands into set 0; every later step is made
  // readable inside the step before it
  wait_vmem(true);
  __builtin_amdgcn_s_barrier();
  V3Frags<TA> f;
  {
    const V3Stage first{X[0].x, W[0].w, W[0].s};
    v3q_first<TA>(f, first, wave, l32, h);
  }
#define NVFP4_V3P_STEP(XI, WI, XO, XSLAB, WO, WSLAB, WLS, NEXT)                      \
  do {                                                                               \
    const Issue iss{&X[((XI) + 2) % 3], &W[((WI) + 3) % 6], &(XO), &(WO), (XSLAB), wsl(WSLAB), wave, &b, (WLS)}; \
    const V3Stage cur{X[XI].x, W[WI].w, W[WI].s};                                    \
    const V3Stage nxt{X[((XI) + 1) % 3].x, W[((WI) + 1) % 6].w, W[((WI) + 1) % 6].s}; \
    v3q_step<TA, NEXT>(acc, f, cur, nxt, wave, l32, h, iss);                         \
  } while (0)
  uint32_t s = 0;
  for (; s + 6 < nslabs; s += 6) {
    NVFP4_V3P_STEP(0, 0, o, s + 2, o, s + 3, ls, true);
    NVFP4_V3P_STEP(1, 1, o, s + 3, o, s + 4, ls, true);
    NVFP4_V3P_STEP(2, 2, o, s + 4, o, s + 5, ls, true);
    NVFP4_V3P_STEP(0, 3, o, s + 5, o, s + 6, ls, true);
    NVFP4_V3P_STEP(1, 4, o, s + 6, o, s + 7, ls, true);
    NVFP4_V3P_STEP(2, 5, o, s + 7, o, s + 8, ls, true);
  }
  NVFP4_V3P_STEP(0, 0, o, s + 2, o, s + 3, ls, true);
  NVFP4_V3P_STEP(1, 1, o, s + 3, o, s + 4, ls, true);
  NVFP4_V3P_STEP(2, 2, o, s + 4, o, s + 5, ls, true);
  // without a next tile, `no` holds this tile's offsets and the tail
  // queues its last slab again
  const uint32_t last = nslabs - 1;
  const uint32_t q0 = has_next ? 0u : last, q1 = has_next ? 1u : last, q2 = has_next ? 2u : last;
  NVFP4_V3P_STEP(0, 3, o, last, no, q0, nls, true);
  NVFP4_V3P_STEP(1, 4, no, q0, no, q1, nls, true);
  NVFP4_V3P_STEP(2, 5, no, q1, no, q2, nls, false);
  if (!has_next) wait_vmem(false);   // no load-to-LDS may land after the last tile
#undef NVFP4_V3P_STEP
}

// kGlu: the gated MLP projection's tiles (N is the feature count; the
// second plane wu, scu, gsu holds the up rows) with the gated epilogue for
// activation kAct, bf16 only.
// TO float: float32 activations as rows of three bf16 parts (K = 3 Kw,
// Kw = 64 wslabs the plane's row length), float32 output.
template <typename TA, bool kGlu = false, int kAct = 0, typename TO = TA>
__global__ __launch_bounds__(kMfmaThreads, 1) void gemm_mfma_v3p_kernel(
    const TA* __restrict__ x, const uint32_t* __restrict__ w, const uint8_t* __restrict__ sc,
    const float* __restrict__ gs, TO* __restrict__ out, int64_t M, int64_t K, int64_t N, int64_t tiles_m,
    int64_t tiles_total, int64_t per_xcd, const uint32_t* __restrict__ wu = nullptr,
    const uint8_t* __restrict__ scu = nullptr, const float* __restrict__ gsu = nullptr, int64_t wslabs = 0) {
  constexpr bool kWrap = sizeof(TO) == 4;
  static_assert(!kGlu || __is_same(TA, __bf16), "the gated form is bf16");
  constexpr int64_t kTileN = kGlu ? kV3BN / 2 : kV3BN;   // output columns per tile
  __shared__ uint4 x0[kV3BM * 8], x1[kV3BM * 8], x2[kV3BM * 8];
  __shared__ uint4 w0[kV3BN * 2], w1[kV3BN * 2], w2[kV3BN * 2], w3[kV3BN * 2], w4[kV3BN * 2], w5[kV3BN * 2];
  __shared__ uint32_t s0[kV3BN], s1[kV3BN], s2[kV3BN], s3[kV3BN], s4[kV3BN], s5[kV3BN];
  const V3Stage st0{x0, w0, s0}, st1{x1, w1, s1}, st2{x2, w2, s2};
  const V3Stage XS[3] = {st0, st1, st2};
  const V3Stage WS[6] = {st0, st1, st2, {x0, w3, s3}, {x0, w4, s4}, {x0, w5, s5}};

  // XCD x (blocks b with b % 8 == x) owns logical tiles [x per_xcd, (x + 1)
  // per_xcd); its bpx blocks take them round-robin.
  const int64_t bpx = (int64_t)gridDim.x / 8;
  const int64_t t_begin = ((int64_t)blockIdx.x % 8) * per_xcd;
  const int64_t t_end = t_begin + per_xcd < tiles_total ? t_begin + per_xcd : tiles_total;
  int64_t tile = t_begin + (int64_t)blockIdx.x / 8;
  if (tile >= t_end) return;   // whole block, before any barrier

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const uint32_t nslabs = (uint32_t)(K / kV3BK);
  const float g = global_factor(gs, 0);
  const float gu = kGlu ? global_factor(gsu, 0) : 0.0f;
  const int64_t Kw = kWrap ? wslabs * kV3BK : K;
  const V3Base base{v3_buffer(x, M * K * 2), v3_buffer((kGlu && (wave & 1)) ? wu : w, N * (Kw / 2)),
                    v3_buffer(sc, N * (Kw / 16))};
  V3Off o, no;
  const uint8_t *ls = nullptr, *nls = nullptr;
  v3p_offsets<kGlu>(o, M, K, N, (tile % tiles_m) * kV3BM, (tile / tiles_m) * kTileN, wave, lane, sc, scu, &ls, Kw);
  bool issued = false;
  for (;;) {
    // The lane index passes through an empty asm each tile, so values
    // derived from it are computed per tile instead of being hoisted out of
    // the tile loop and held in registers across it.
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    const int lx = ln & 31, hx = ln >> 5;
    const int64_t next = tile + bpx;
    const bool has_next = next < t_end;
    v3p_offsets<kGlu>(no, M, K, N, ((has_next ? next : tile) % tiles_m) * kV3BM,
                      ((has_next ? next : tile) / tiles_m) * kTileN, wave, ln, sc, scu, &nls, Kw);
    f32x16_t acc[2][8];
    v3p_mainloop<TA, kGlu, kWrap>(acc, XS, WS, base, o, no, has_next, issued, nslabs, wave, lx, hx, ls, nls,
                                  (uint32_t)(Kw / kV3BK));
    if constexpr (kGlu)
      v3_store_glu<kAct>(acc, out, M, N, (tile % tiles_m) * kV3BM, (tile / tiles_m) * kTileN, g, gu, wave, lx, hx);
    else
      v3_store_tile<TO>(acc, out, M, N, (tile % tiles_m) * kV3BM, (tile / tiles_m) * kTileN, g, wave, lx, hx);
    if (!has_next) break;
    tile = next;
    o = no;
    ls = nls;
    issued = true;
  }
}

// ----------------------------------------------------------------------------
// Non-transposed planes (w [K, N/8], quantized along N): dequantize, then a
// matrix-core GEMM on the dense copy, the order of the pages' own GEMM route.
// ----------------------------------------------------------------------------

// Dense copy of a non-transposed plane, transposed: wt[n][k] =
// e2m1(w[k][n]) * e4m3(scale[k][n / 16]) as bf16 or f16 bits (exact in both:
// at most 6 significant bits, magnitudes in [2^-10, 2688]); the global factor
// is left to the GEMM's epilogue.  Block (kb, nb) covers k in [64 kb, 64 kb
// + 64) and n in [64 nb, 64 nb + 64): thread t decodes words 2 (t & 3) and
// 2 (t & 3) + 1 of row k = 64 kb + (t >> 2) (sixteen n, one scale block) into
// an LDS tile that is written back along k, 16 bytes per store.
constexpr int kNtTile = 64;
template <typename TW>
__global__ __launch_bounds__(256) void dequant_nt_kernel(const uint32_t* __restrict__ w, const uint8_t* __restrict__ sc,
                                                         int64_t K, int64_t N, uint16_t* __restrict__ wt) {
  __shared__ __align__(16) uint16_t tile[kNtTile][kNtTile + 8];   // [n][k], rows padded by 16 bytes
  const int t = threadIdx.x;
  const int64_t k0 = (int64_t)blockIdx.x * kNtTile, n0 = (int64_t)blockIdx.y * kNtTile;
  {
    const int kl = t >> 2, g = t & 3;
    const int64_t k = k0 + kl, n = n0 + 16 * g;     // N % 16 == 0: a group is wholly in or out
    if (k < K && n < N) {
      const uint2 wv = *reinterpret_cast<const uint2*>(w + k * (N / 8) + n / 8);
      const float s = e4m3<0>(sc[k * (N / 16) + n / 16]);
      const uint4 ua = __builtin_bit_cast(uint4, V3Ops<TW>::decode(wv.x, s));
      const uint4 ub = __builtin_bit_cast(uint4, V3Ops<TW>::decode(wv.y, s));
      const uint32_t d[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        tile[16 * g + 2 * i][kl] = (uint16_t)d[i];
        tile[16 * g + 2 * i + 1][kl] = (uint16_t)(d[i] >> 16);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int idx = r * 256 + t, nl = idx >> 3, c = idx & 7;
    const int64_t n = n0 + nl, k = k0 + 8 * c;
    if (n < N && k < K)
      *reinterpret_cast<uint4*>(wt + n * K + k) = *reinterpret_cast<const uint4*>(&tile[nl][8 * c]);
  }
}

// GEMM of 2-byte activations x [M, K] against a dense 2-byte weight copy
// wt [N, wk] (rows of K elements when wk == K; the float32 form runs over
// activation rows of three bf16 parts, K = 3 wk, and activation slab s meets
// weight slab s mod (wk / 64)).  The tile and fragments are those of the
// NVFP4 GEMM above (256 weight rows x 256 activation rows, wavefront w owning
// weight rows [64w, 64w + 64)), with the weight fragments read from LDS like
// the activation fragments.  Both operands move global -> LDS through two
// stages of 32 KiB each: slab s + 1 is queued after the barrier that ends
// slab s - 1, so it streams while slab s is multiplied.
template <typename TA, typename TO>
__global__ __launch_bounds__(kMfmaThreads, 1) void gemm_mfma_dense_kernel(
    const TA* __restrict__ x, const uint16_t* __restrict__ wt, const float* __restrict__ gs, TO* __restrict__ out,
    int64_t M, int64_t K, int64_t N, int64_t tiles_m, int64_t tiles_total, int64_t wk) {
  typedef typename V3Ops<TA>::vec vec;
  __shared__ uint4 xa[kV3BM * 8], xb[kV3BM * 8], wa[kV3BN * 8], wb[kV3BN * 8];

  const int64_t per_xcd = (int64_t)gridDim.x / 8;
  const int64_t tile = ((int64_t)blockIdx.x % 8) * per_xcd + (int64_t)blockIdx.x / 8;
  if (tile >= tiles_total) return;   // whole block, before any barrier
  const int64_t m_blk = (tile % tiles_m) * kV3BM;
  const int64_t n_blk = (tile / tiles_m) * kV3BN;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t nslabs = K / kV3BK, wslabs = wk / kV3BK;

  // Per load i: 16-byte chunk `slot` of the tile, the same placement for
  // both operands; rows past M or N re-read the last row (never stored).
  const uint16_t* xs[8];
  const uint16_t* ws[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int slot = (i * 4 + wave) * 64 + lane;
    const int r = slot >> 3, c = (slot & 7) ^ swz(r);
    const int64_t m = m_blk + r < M ? m_blk + r : M - 1;
    const int64_t n = n_blk + r < N ? n_blk + r : N - 1;
    xs[i] = reinterpret_cast<const uint16_t*>(x) + m * K + c * 8;
    ws[i] = wt + n * wk + c * 8;
  }
  auto issue = [&](uint4* xd, uint4* wd, int64_t slab) {
    const int64_t wsl = slab < wslabs ? slab : slab % wslabs;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds(xs[i] + slab * kV3BK, NVFP4_LDS(&xd[(i * 4 + wave) * 64]), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds(ws[i] + wsl * kV3BK, NVFP4_LDS(&wd[(i * 4 + wave) * 64]), 16, 0, 0);
  };
  auto compute = [&](f32x16_t (&acc)[2][8], const uint4* xd, const uint4* wd) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vec B[8], A[2];
#pragma unroll
      for (int b = 0; b < 8; ++b) B[b] = __builtin_bit_cast(vec, xd[xslot(b * 32 + l32, 4 * h + j)]);
#pragma unroll
      for (int a = 0; a < 2; ++a) A[a] = __builtin_bit_cast(vec, wd[xslot(wave * 64 + a * 32 + l32, 4 * h + j)]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        acc[0][b] = V3Ops<TA>::mfma(A[0], B[b], acc[0][b]);
        acc[1][b] = V3Ops<TA>::mfma(A[1], B[b], acc[1][b]);
      }
    }
  };

  f32x16_t acc[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
  issue(xa, wa, 0);
  int64_t s = 0;
  for (; s + 2 <= nslabs; s += 2) {
    wait_vmem(false);
    __builtin_amdgcn_s_barrier();
    issue(xb, wb, s + 1);
    compute(acc, xa, wa);
    wait_vmem(false);
    __builtin_amdgcn_s_barrier();
    if (s + 2 < nslabs) issue(xa, wa, s + 2);
    compute(acc, xb, wb);
  }
  if (s < nslabs) {
    wait_vmem(false);
    __builtin_amdgcn_s_barrier();
    compute(acc, xa, wa);
  }
  wait_vmem(false);   // nothing is in flight here; kept so no load-to-LDS can outlive the loop
  v3_store_tile<TO>(acc, out, M, N, m_blk, n_blk, global_factor(gs, 0), wave, l32, h);
}

// out = round(g * sum over splits of ws[split]), splits added in order.
template <typename TO>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ ws, int64_t splits,
                                                           int64_t MN, const float* __restrict__ gs,
                                                           TO* __restrict__ out) {
  static_assert(sizeof(TO) == 2, "partials are reduced into 2-byte outputs");
  const float g = global_factor(gs, 0);
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; e < MN; e += stride * 4) {
    if (e + 3 < MN) {
      float4 v = *reinterpret_cast<const float4*>(ws + e);
      for (int64_t sp = 1; sp < splits; ++sp) {
        const float4 u = *reinterpret_cast<const float4*>(ws + sp * MN + e);
        v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
      }
      const TO o[4] = {(TO)(v.x * g), (TO)(v.y * g), (TO)(v.z * g), (TO)(v.w * g)};
      *reinterpret_cast<uint2*>(out + e) = __builtin_bit_cast(uint2, o);
    } else {
      for (int64_t i = e; i < MN; ++i) {
        float v = ws[i];
        for (int64_t sp = 1; sp < splits; ++sp) v += ws[sp * MN + i];
        out[i] = (TO)(v * g);
      }
    }
  }
}

// float32 activations for the MFMA GEMM: row m of x [M, K] becomes row m of
// xs [M, 3K], its exact three-part bf16 split (split3_bits) laid end to end:
// hi in [0, K), mid in [K, 2K), lo in [2K, 3K).  One thread per eight
// consecutive elements (K % 64 == 0, so a group never crosses a row).
__global__ __launch_bounds__(256) void split_f32_kernel(const float* __restrict__ x, int64_t M, int64_t K,
                                                        uint16_t* __restrict__ xs) {
  const int64_t groups = M * K / 8;
  for (int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x; gi < groups; gi += (int64_t)gridDim.x * 256) {
    const int64_t m = gi / (K / 8), k = (gi - m * (K / 8)) * 8;
    const uint4 a = reinterpret_cast<const uint4*>(x + m * K + k)[0];
    const uint4 b = reinterpret_cast<const uint4*>(x + m * K + k)[1];
    const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t hv[8], mv[8], lv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split3_bits(u[e], hv[e], mv[e], lv[e]);
    uint32_t ph[4], pm[4], pl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ph[j] = __builtin_amdgcn_perm(hv[2 * j + 1], hv[2 * j], 0x07060302u);
      pm[j] = __builtin_amdgcn_perm(mv[2 * j + 1], mv[2 * j], 0x07060302u);
      pl[j] = __builtin_amdgcn_perm(lv[2 * j + 1], lv[2 * j], 0x07060302u);
    }
    uint16_t* row = xs + m * 3 * K + k;
    *reinterpret_cast<uint4*>(row) = make_uint4(ph[0], ph[1], ph[2], ph[3]);
    *reinterpret_cast<uint4*>(row + K) = make_uint4(pm[0], pm[1], pm[2], pm[3]);
    *reinterpret_cast<uint4*>(row + 2 * K) = make_uint4(pl[0], pl[1], pl[2], pl[3]);
  }
}

// ----------------------------------------------------------------------------
// Generic float32 kernel
// ----------------------------------------------------------------------------

constexpr int kGT = 64;   // output tile edge
constexpr int kGK = 16;   // k per stage (one scale block)

// Finishes the K-split tail tiles of the gated projection: for each output
// of tile tile0 + t, the gate and up sums are the partials of every split
// added in split order; out = bf16(act(g_gate * gate) * (g_up * up)).  One
// thread per four consecutive features (tile rows 64 w' + i and
// 64 w' + 32 + i hold feature 32 w' + i of the gate and of the up plane).
__global__ __launch_bounds__(256) void glu_tail_reduce_kernel(const float* __restrict__ ws, int64_t splits,
                                                              int64_t ntiles, int64_t tile0, int64_t tiles_m,
                                                              int64_t M, int64_t F, const float* __restrict__ gs,
                                                              const float* __restrict__ gsu, int act,
                                                              __bf16* __restrict__ out) {
  const int64_t total = ntiles * 256 * 32;
  const float gg = global_factor(gs, 0), gu = global_factor(gsu, 0);
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t t = idx / (256 * 32);
    const int ml = (int)((idx / 32) % 256), f4 = (int)(idx % 32);
    const int64_t tile = tile0 + t;
    const int64_t m = (tile % tiles_m) * 256 + ml;
    const int64_t f = (tile / tiles_m) * 128 + 4 * f4;
    if (m >= M || f >= F) continue;
    const int nl = 64 * (f4 >> 3) + 4 * (f4 & 7);
    float4 ga = make_float4(0.0f, 0.0f, 0.0f, 0.0f), ua = ga;
    for (int64_t sp = 0; sp < splits; ++sp) {
      const float* base = ws + ((sp * ntiles + t) << 16) + ml * 256;
      const float4 a = *reinterpret_cast<const float4*>(base + nl);
      const float4 b = *reinterpret_cast<const float4*>(base + nl + 32);
      ga.x += a.x; ga.y += a.y; ga.z += a.z; ga.w += a.w;
      ua.x += b.x; ua.y += b.y; ua.z += b.z; ua.w += b.w;
    }
    const float gv[4] = {ga.x, ga.y, ga.z, ga.w}, uv[4] = {ua.x, ua.y, ua.z, ua.w};
    __bf16* q = out + m * F + f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (f + i < F) q[i] = (__bf16)(glu_act(gv[i] * gg, act) * (uv[i] * gu));
  }
}

template <typename TX, bool TRANS>
__global__ __launch_bounds__(256) void gemm_generic_kernel(const TX* __restrict__ x,
                                                           const uint32_t* __restrict__ w,
                                                           const uint8_t* __restrict__ sc,
                                                           const float* __restrict__ gs,
                                                           TX* __restrict__ out, int64_t M,
                                                           int64_t K, int64_t N) {
  __shared__ float xs[kGK][kGT + 4];
  __shared__ float ws[kGK][kGT + 4];
  const int t = threadIdx.x;
  const int tm = t >> 4, tn = t & 15;
  const int64_t n0 = (int64_t)blockIdx.x * kGT;
  const float g = global_factor(gs, 0);

  for (int64_t m0 = (int64_t)blockIdx.y * kGT; m0 < M; m0 += (int64_t)gridDim.y * kGT) {
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

    for (int64_t k0 = 0; k0 < K; k0 += kGK) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = i * 256 + t;
        const int mm = e >> 4, kk = e & 15;
        const int64_t m = m0 + mm, k = k0 + kk;
        xs[kk][mm] = (m < M && k < K) ? load_x(x + m * K + k) : 0.0f;
      }
      if (t < 128) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
        if constexpr (TRANS) {
          // plane [N, K/8]: row n, words k0/8 and k0/8 + 1 (K % 16 == 0)
          const int nn = t >> 1, wi = t & 1;
          const int64_t n = n0 + nn;
          if (n < N) {
            const float s = e4m3<0>(sc[n * (K / 16) + k0 / 16]);
            decode_word_f32(w[n * (K / 8) + k0 / 8 + wi], s, v);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) ws[wi * 8 + i][nn] = v[i];
        } else {
          // plane [K, N/8]: row k, words n0/8 .. n0/8 + 7 (N % 16 == 0)
          const int kk = t >> 3, wi = t & 7;
          const int64_t k = k0 + kk;
          if (k < K && n0 + wi * 8 < N) {
            const float s = e4m3<0>(sc[k * (N / 16) + n0 / 16 + wi / 2]);
            decode_word_f32(w[k * (N / 8) + n0 / 8 + wi], s, v);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) ws[kk][wi * 8 + i] = v[i];
        }
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kGK; ++kk) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] = xs[kk][tm * 4 + i];
          b[i] = ws[kk][tn * 4 + i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + tm * 4 + i;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + tn * 4 + j;
        if (n < N) store_out(out + m * N + n, acc[i][j] * g);
      }
    }
  }
}

template <typename TX>
void generic_dispatch(const TX* x, int64_t M, int64_t K, int64_t N, const uint32_t* w,
                      const uint8_t* sc, const float* gs, int transpose, TX* out, hipStream_t s) {
  const int64_t gx = (N + kGT - 1) / kGT;
  int64_t gy = (M + kGT - 1) / kGT;
  if (gy > nvfp4host::kMaxGridY) gy = nvfp4host::kMaxGridY;
  if (transpose)
    gemm_generic_kernel<TX, true><<<dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s>>>(x, w, sc, gs, out, M, K, N);
  else
    gemm_generic_kernel<TX, false><<<dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s>>>(x, w, sc, gs, out, M, K, N);
}

// Compute units of the current device (cached per device; 256 if the
// runtime cannot say).
int64_t device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

namespace nvfp4host {

// Slabs per piece when `nslabs` slabs are shared by `sp` blocks.
static int64_t v3_piece(int64_t nslabs, int64_t sp) { return (nslabs + sp - 1) / sp; }

// Splits of K for the MFMA GEMM: with few tiles most compute units would
// idle, so the slabs of each tile are shared among `splits` blocks and their
// float32 partials added afterwards.  Model: rounds of blocks times the
// per-block time (slab time plus a fixed start-up and epilogue cost), plus
// the partials' traffic; returns 1 when splitting does not pay.
int64_t gemm_splits(int64_t M, int64_t K, int64_t N) {
  if (K % kV3BK != 0) return 1;
  const int64_t tiles = ((M + kV3BM - 1) / kV3BM) * ((N + kV3BN - 1) / kV3BN);
  const int64_t nslabs = K / kV3BK;
  const int64_t cus = device_cu_count();
  const double slab_us = 1.4, block_us = 20.0, bytes_per_us = 4.0e6;
  int64_t best = 1;
  double best_t = 0.0;
  for (int64_t sp = 1; sp <= 8 && sp <= nslabs / 4; ++sp) {
    const int64_t per = v3_piece(nslabs, sp);
    if ((sp - 1) * per >= nslabs) continue;   // the last split would be empty
    const double rounds = (double)((tiles * sp + cus - 1) / cus);
    double t = rounds * (per * slab_us + block_us);
    if (sp > 1) t += (double)(sp * 4 + 2) * (double)M * (double)N / bytes_per_us;
    if (sp == 1 || t < best_t) {
      best = sp;
      best_t = t;
    }
  }
  return best;
}

// The v3 kernel's buffer-load form applies when every operand stays below
// 2^31 bytes (buffer resources hold 31-bit sizes): activation rows of Kx
// 2-byte elements, planes of N rows of K / 2 bytes.
static bool v3_buffers_fit(int64_t M, int64_t Kx, int64_t N, int64_t K) {
  const int64_t lim = (int64_t)1 << 31;
  return M * Kx * 2 < lim && N * (K / 2) < lim && N * (K / 16) < lim;
}

// The two-byte MFMA GEMM (bf16 or f16 activations and output) with an
// optional K split through the workspace.
template <typename T>
static void launch_v3(const T* x, int64_t M, int64_t K, int64_t N, const uint32_t* w, const uint8_t* sc,
                      const float* gs, T* out, hipStream_t s, void* ws, int64_t ws_bytes) {
  const int64_t tiles_m = (M + kV3BM - 1) / kV3BM;
  const int64_t tiles = tiles_m * ((N + kV3BN - 1) / kV3BN);
  const int64_t sp = ws ? gemm_splits(M, K, N) : 1;
  if (sp > 1 && ws_bytes >= sp * M * N * 4 && (reinterpret_cast<uintptr_t>(ws) & 15) == 0) {
    const int64_t per = v3_piece(K / kV3BK, sp);
    const int64_t grid = (tiles * sp + 7) / 8 * 8;
    auto kern = v3_buffers_fit(M, K, N, K) ? gemm_mfma_v3_kernel<kV3Split, 0, T, T, true>
                                           : gemm_mfma_v3_kernel<kV3Split, 0, T, T, false>;
    kern<<<dim3((unsigned)grid), dim3(kMfmaThreads), 0, s>>>(x, w, sc, gs, out, M, K, N, tiles_m, tiles, per,
                                                            static_cast<float*>(ws), nullptr, nullptr, nullptr, 0,
                                                            K / kV3BK);
    const int64_t MN = M * N;
    int64_t rgrid = (MN / 4 + 255) / 256;
    if (rgrid > 4096) rgrid = 4096;
    if (rgrid < 1) rgrid = 1;
    split_reduce_kernel<T><<<dim3((unsigned)rgrid), dim3(256), 0, s>>>(static_cast<const float*>(ws), sp, MN, gs, out);
    return;
  }
  const int64_t nslabs = K / kV3BK;
  const int64_t cus = device_cu_count();
  // (buffer resources hold at most 2^31 - 1 bytes: activations M K 2 and
  // plane N K / 2 bytes below 2^31)
  if (nslabs % 6 == 0 && nslabs >= 12 && tiles > cus && cus % 8 == 0 && M * K < ((int64_t)1 << 30) &&
      N * (K / 8) < ((int64_t)1 << 29)) {
    // persistent: one block per compute unit, each XCD a contiguous run of tiles
    const int64_t per_xcd = (tiles + 7) / 8;
    const int64_t bpx = per_xcd < cus / 8 ? per_xcd : cus / 8;
    gemm_mfma_v3p_kernel<T><<<dim3((unsigned)(8 * bpx)), dim3(kMfmaThreads), 0, s>>>(x, w, sc, gs, out, M, K, N,
                                                                                    tiles_m, tiles, per_xcd);
    return;
  }
  const int64_t grid = (tiles + 7) / 8 * 8;
  auto kern = v3_buffers_fit(M, K, N, K) ? gemm_mfma_v3_kernel<kV3Plain, 0, T, T, true>
                                         : gemm_mfma_v3_kernel<kV3Plain, 0, T, T, false>;
  kern<<<dim3((unsigned)grid), dim3(kMfmaThreads), 0, s>>>(x, w, sc, gs, out, M, K, N, tiles_m, tiles, 0, nullptr,
                                                          nullptr, nullptr, nullptr, 0, K / kV3BK);
}

// Workspace of the float32 form: the [M, 3K] bf16 split of the activations.
static int64_t f32_split_bytes(int64_t M, int64_t K) { return (M * 3 * K * 2 + 255) / 256 * 256; }

// Non-transposed planes take the dense route whenever K % 64 == 0: the
// generic kernel is latency-bound on them at every M (at K = N = 4096 it
// took 515-575 us for M = 1..64, the dense route 118-121 us).
static bool nt_applies(int64_t K, int64_t N) {
  return K % kV3BK == 0 && (N + kNtTile - 1) / kNtTile <= 65535;
}

static int64_t nt_dense_bytes(int64_t K, int64_t N) { return (N * K * 2 + 255) / 256 * 256; }

// Non-transposed plane: its dense transposed copy (and, for float32
// activations, their three-part copy after it) in the workspace, then the
// dense matrix-core GEMM.  False (nothing launched) when the route does not
// apply or the workspace is short.
static bool launch_gemm_mfma_nt(const void* x, nvfp4_dtype_t dt, int64_t M, int64_t K, int64_t N, const uint32_t* w,
                                const uint8_t* sc, const float* gs, void* out, hipStream_t s, void* ws,
                                int64_t ws_bytes) {
  if (!nt_applies(K, N) || !ws || (reinterpret_cast<uintptr_t>(ws) & 15) != 0) return false;
  const int64_t dense = nt_dense_bytes(K, N);
  if (ws_bytes < dense + (dt == NVFP4_F32 ? f32_split_bytes(M, K) : 0)) return false;
  uint16_t* wt = static_cast<uint16_t*>(ws);
  const dim3 dgrid((unsigned)(K / kNtTile), (unsigned)((N + kNtTile - 1) / kNtTile));
  if (dt == NVFP4_F16)
    dequant_nt_kernel<_Float16><<<dgrid, dim3(256), 0, s>>>(w, sc, K, N, wt);
  else
    dequant_nt_kernel<__bf16><<<dgrid, dim3(256), 0, s>>>(w, sc, K, N, wt);
  const int64_t tiles_m = (M + kV3BM - 1) / kV3BM;
  const int64_t tiles = tiles_m * ((N + kV3BN - 1) / kV3BN);
  const dim3 grid((unsigned)((tiles + 7) / 8 * 8));
  switch (dt) {
    case NVFP4_BF16:
      gemm_mfma_dense_kernel<__bf16, __bf16><<<grid, dim3(kMfmaThreads), 0, s>>>(
          static_cast<const __bf16*>(x), wt, gs, static_cast<__bf16*>(out), M, K, N, tiles_m, tiles, K);
      break;
    case NVFP4_F16:
      gemm_mfma_dense_kernel<_Float16, _Float16><<<grid, dim3(kMfmaThreads), 0, s>>>(
          static_cast<const _Float16*>(x), wt, gs, static_cast<_Float16*>(out), M, K, N, tiles_m, tiles, K);
      break;
    case NVFP4_F32: {
      uint16_t* xs = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + dense);
      int64_t sgrid = (M * K / 8 + 255) / 256;
      if (sgrid > 8192) sgrid = 8192;
      split_f32_kernel<<<dim3((unsigned)sgrid), dim3(256), 0, s>>>(static_cast<const float*>(x), M, K, xs);
      gemm_mfma_dense_kernel<__bf16, float><<<grid, dim3(kMfmaThreads), 0, s>>>(
          reinterpret_cast<const __bf16*>(xs), wt, gs, static_cast<float*>(out), M, 3 * K, N, tiles_m, tiles, K);
      break;
    }
  }
  return true;
}

bool launch_gemm_mfma(const void* x, nvfp4_dtype_t dt, int64_t M, int64_t K, int64_t N, const uint32_t* w,
                      const uint8_t* sc, const float* gs, int transpose, void* out, hipStream_t s, void* ws,
                      int64_t ws_bytes) {
  if (!transpose) return launch_gemm_mfma_nt(x, dt, M, K, N, w, sc, gs, out, s, ws, ws_bytes);
  const bool v3 = K % kV3BK == 0 && (reinterpret_cast<uintptr_t>(sc) & 3) == 0;
  switch (dt) {
    case NVFP4_BF16:
      if (v3) {
        launch_v3(static_cast<const __bf16*>(x), M, K, N, w, sc, gs, static_cast<__bf16*>(out), s, ws, ws_bytes);
        return true;
      }
      if (K % 32 == 0) {
        const int64_t tiles_m = (M + kBM - 1) / kBM;
        const int64_t tiles = tiles_m * ((N + kBN - 1) / kBN);
        const int64_t grid = (tiles + 7) / 8 * 8;
        gemm_mfma_kernel<<<dim3((unsigned)grid), dim3(kMfmaThreads), 0, s>>>(
            static_cast<const __bf16*>(x), w, sc, gs, static_cast<__bf16*>(out), M, K, N, tiles_m, tiles);
        return true;
      }
      return false;
    case NVFP4_F16:
      if (!v3) return false;
      launch_v3(static_cast<const _Float16*>(x), M, K, N, w, sc, gs, static_cast<_Float16*>(out), s, ws, ws_bytes);
      return true;
    case NVFP4_F32: {
      // The exact three-part bf16 split of the activations goes to the
      // workspace; the bf16 kernel then runs over rows of 3K against the one
      // plane (weight slab s mod K/64), so the three partial products sum in
      // its float32 accumulators, and stores float32.
      if (!v3 || !ws || ws_bytes < f32_split_bytes(M, K) || (reinterpret_cast<uintptr_t>(ws) & 15) != 0) return false;
      uint16_t* xs = static_cast<uint16_t*>(ws);
      int64_t sgrid = (M * K / 8 + 255) / 256;
      if (sgrid > 8192) sgrid = 8192;
      split_f32_kernel<<<dim3((unsigned)sgrid), dim3(256), 0, s>>>(static_cast<const float*>(x), M, K, xs);
      const int64_t tiles_m = (M + kV3BM - 1) / kV3BM;
      const int64_t tiles = tiles_m * ((N + kV3BN - 1) / kV3BN);
      const int64_t cus = device_cu_count();
      if ((3 * K / kV3BK) % 6 == 0 && K / kV3BK >= 4 && tiles > cus && cus % 8 == 0 &&
          M * 3 * K < ((int64_t)1 << 30) && N * (K / 8) < ((int64_t)1 << 29)) {
        // persistent, as the bf16 prefill: one block per compute unit
        const int64_t per_xcd = (tiles + 7) / 8;
        const int64_t bpx = per_xcd < cus / 8 ? per_xcd : cus / 8;
        gemm_mfma_v3p_kernel<__bf16, false, 0, float><<<dim3((unsigned)(8 * bpx)), dim3(kMfmaThreads), 0, s>>>(
            reinterpret_cast<const __bf16*>(xs), w, sc, gs, static_cast<float*>(out), M, 3 * K, N, tiles_m, tiles,
            per_xcd, nullptr, nullptr, nullptr, K / kV3BK);
        return true;
      }
      const int64_t grid = (tiles + 7) / 8 * 8;
      auto kern = v3_buffers_fit(M, 3 * K, N, K) ? gemm_mfma_v3_kernel<kV3Plain, 0, __bf16, float, true>
                                                 : gemm_mfma_v3_kernel<kV3Plain, 0, __bf16, float, false>;
      kern<<<dim3((unsigned)grid), dim3(kMfmaThreads), 0, s>>>(reinterpret_cast<const __bf16*>(xs), w, sc, gs,
                                                              static_cast<float*>(out), M, 3 * K, N, tiles_m, tiles,
                                                              0, nullptr, nullptr, nullptr, nullptr, 0, K / kV3BK);
      return true;
    }
  }
  return false;
}

// K-split of the gated projection's last, partial round of tiles: with
// `rem` tiles left over after whole rounds on the device's compute units,
// each is shared by floor(cus / rem) blocks (at most 8, each at least 4 slabs
// of K), so the last round takes a fraction of a tile's time; the float32
// partials go through a workspace and a reduction.  0 splits: no split.
void glu_tail_split(int64_t M, int64_t K, int64_t F, int64_t* tail_tiles, int64_t* splits) {
  *tail_tiles = 0;
  *splits = 0;
  if (K % kV3BK != 0) return;
  const int64_t tiles = gemm_glu_tiles(M, F);
  const int64_t cus = device_cu_count();
  const int64_t rem = tiles % cus;
  if (rem == 0) return;
  int64_t sp = cus / rem;
  if (sp > 8) sp = 8;
  const int64_t nslabs = K / kV3BK;
  while (sp > 1 && nslabs / sp < 4) --sp;
  // Pieces of ceil(nslabs / sp) slabs; recount the splits from the piece
  // length so that none is empty (42 slabs over 8 splits would give pieces
  // of 6 and an eighth split starting past the end).
  if (sp > 1) sp = (nslabs + v3_piece(nslabs, sp) - 1) / v3_piece(nslabs, sp);
  if (sp < 2) return;
  *tail_tiles = rem;
  *splits = sp;
}

int64_t gemm_glu_workspace_bytes(int64_t M, int64_t K, int64_t F) {
  int64_t tail, sp;
  glu_tail_split(M, K, F, &tail, &sp);
  return sp > 1 ? tail * sp * 65536 * 4 : 0;
}

void launch_gemm_glu(const void* x, int64_t M, int64_t K, int64_t F, const uint32_t* w_gate,
                     const uint8_t* s_gate, const float* gs_gate, const uint32_t* w_up, const uint8_t* s_up,
                     const float* gs_up, int act, void* out, hipStream_t s, void* ws, int64_t ws_bytes) {
  const int64_t tiles_m = (M + kV3BM - 1) / kV3BM;
  const int64_t tiles = gemm_glu_tiles(M, F);
  int64_t tail = 0, sp = 0;
  if (ws && (reinterpret_cast<uintptr_t>(ws) & 15) == 0) glu_tail_split(M, K, F, &tail, &sp);
  if (sp < 2 || ws_bytes < tail * sp * 65536 * 4) tail = 0;
  const int64_t dp = tiles - tail;
  const int64_t nslabs = K / kV3BK;
  const int64_t cus = device_cu_count();
  if (dp > cus && nslabs % 6 == 0 && nslabs >= 12 && cus % 8 == 0 && M * K < ((int64_t)1 << 30) &&
      F * (K / 8) < ((int64_t)1 << 29)) {
    // whole rounds as a persistent launch (as the plain GEMM's), one block
    // per compute unit, each XCD a contiguous run of tiles
    const int64_t per_xcd = (dp + 7) / 8;
    const int64_t bpx = per_xcd < cus / 8 ? per_xcd : cus / 8;
    auto glu = gemm_mfma_v3p_kernel<__bf16, true, NVFP4_ACT_SILU>;
    if (act == NVFP4_ACT_GELU_TANH) glu = gemm_mfma_v3p_kernel<__bf16, true, NVFP4_ACT_GELU_TANH>;
    if (act == NVFP4_ACT_GELU) glu = gemm_mfma_v3p_kernel<__bf16, true, NVFP4_ACT_GELU>;
    glu<<<dim3((unsigned)(8 * bpx)), dim3(kMfmaThreads), 0, s>>>(static_cast<const __bf16*>(x), w_gate, s_gate,
                                                               gs_gate, static_cast<__bf16*>(out), M, K, F, tiles_m,
                                                               dp, per_xcd, w_up, s_up, gs_up, 0);
  } else if (dp > 0) {
    const int64_t grid = (dp + 7) / 8 * 8;
    const bool buf = v3_buffers_fit(M, K, F, K);
    auto glu = buf ? gemm_mfma_v3_kernel<kV3Glu, NVFP4_ACT_SILU, __bf16, __bf16, true>
                   : gemm_mfma_v3_kernel<kV3Glu, NVFP4_ACT_SILU, __bf16, __bf16, false>;
    if (act == NVFP4_ACT_GELU_TANH)
      glu = buf ? gemm_mfma_v3_kernel<kV3Glu, NVFP4_ACT_GELU_TANH, __bf16, __bf16, true>
                : gemm_mfma_v3_kernel<kV3Glu, NVFP4_ACT_GELU_TANH, __bf16, __bf16, false>;
    if (act == NVFP4_ACT_GELU)
      glu = buf ? gemm_mfma_v3_kernel<kV3Glu, NVFP4_ACT_GELU, __bf16, __bf16, true>
                : gemm_mfma_v3_kernel<kV3Glu, NVFP4_ACT_GELU, __bf16, __bf16, false>;
    glu<<<dim3((unsigned)grid), dim3(kMfmaThreads), 0, s>>>(static_cast<const __bf16*>(x), w_gate, s_gate, gs_gate,
                                                          static_cast<__bf16*>(out), M, K, F, tiles_m, dp, 0, nullptr,
                                                          w_up, s_up, gs_up, 0, K / kV3BK);
  }
  if (tail == 0) return;
  const int64_t per = v3_piece(K / kV3BK, sp);
  const int64_t grid = (tail * sp + 7) / 8 * 8;
  auto split = v3_buffers_fit(M, K, F, K) ? gemm_mfma_v3_kernel<kV3GluSplit, 0, __bf16, __bf16, true>
                                          : gemm_mfma_v3_kernel<kV3GluSplit, 0, __bf16, __bf16, false>;
  split<<<dim3((unsigned)grid), dim3(kMfmaThreads), 0, s>>>(
      static_cast<const __bf16*>(x), w_gate, s_gate, gs_gate, static_cast<__bf16*>(out), M, K, F, tiles_m, tail, per,
      static_cast<float*>(ws), w_up, s_up, gs_up, dp, K / kV3BK);
  int64_t rgrid = (tail * 256 * 32 + 255) / 256;
  if (rgrid > 4096) rgrid = 4096;
  glu_tail_reduce_kernel<<<dim3((unsigned)rgrid), dim3(256), 0, s>>>(static_cast<const float*>(ws), sp, tail, dp,
                                                                    tiles_m, M, F, gs_gate, gs_up, act,
                                                                    static_cast<__bf16*>(out));
}

int64_t gemm_glu_tiles(int64_t M, int64_t F) {
  return ((M + kV3BM - 1) / kV3BM) * ((F + kV3BN / 2 - 1) / (kV3BN / 2));
}

int64_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t N, nvfp4_dtype_t dt, int transpose) {
  if (!transpose)
    return nt_applies(K, N) ? nt_dense_bytes(K, N) + (dt == NVFP4_F32 ? f32_split_bytes(M, K) : 0) : 0;
  if (dt == NVFP4_F32) return K % kV3BK == 0 ? f32_split_bytes(M, K) : 0;
  const int64_t sp = gemm_splits(M, K, N);
  return sp > 1 ? sp * M * N * 4 : 0;
}

void launch_gemm_generic(const void* x, nvfp4_dtype_t dt, int64_t M, int64_t K, int64_t N,
                         const uint32_t* w, const uint8_t* sc, const float* gs, int transpose,
                         void* out, hipStream_t s) {
  switch (dt) {
    case NVFP4_F32:
      generic_dispatch<float>((const float*)x, M, K, N, w, sc, gs, transpose, (float*)out, s);
      break;
    case NVFP4_BF16:
      generic_dispatch<__bf16>((const __bf16*)x, M, K, N, w, sc, gs, transpose, (__bf16*)out, s);
      break;
    case NVFP4_F16:
      generic_dispatch<_Float16>((const _Float16*)x, M, K, N, w, sc, gs, transpose, (_Float16*)out, s);
      break;
  }
}

}  // namespace nvfp4host
