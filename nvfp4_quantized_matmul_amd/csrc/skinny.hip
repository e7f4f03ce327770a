// MFMA kernel for small M ("multi-row qmv", speculative-decode verify widths):
// out[M, N] = x[M, K] @ W[N, K]^T * g with bf16 activations, 2 <= M <= 64.
//
// The pages run these widths through their qmv kernel, eight activation
// rows per block (mlxcel PR "native NVFP4 for ROCm QuantizedMatmul/
// GatherQMM", "Summary" and the multi-row rows of "Numerical results").
// On gfx950 a dot-product loop costs one VALU operation per weight element
// per activation row; here each packed weight word is decoded once (exact
// bf16 products e2m1 * e4m3) into the A operand of a 16x16x32 bf16 MFMA and
// multiplied against every 16-row activation fragment, so the VALU cost no
// longer grows with M.
//
// Block: 4 wavefronts, 64 weight rows (16 per wavefront), all activation
// rows (MF fragments of 16).  k advances in groups of 128 (16 words per
// row).  Activation tile, packed words and scale bytes of a group stream
// global -> LDS by the load-to-LDS path into one of four statically named
// stages; three groups are in flight while one is multiplied.  A stage
// is released by an explicit vector-memory-counter wait plus a plain barrier,
// and loads are issued unconditionally (the last group is re-read near the
// end) so the compiler keeps exact track of what is in flight.
#include "nvfp4_device.hpp"
#include "nvfp4_internal.hpp"

using namespace nvfp4dev;

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;       // weight rows per block
constexpr int kKG = 128;        // k per group (one pipeline stage)

#define NVFP4_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Activation tile row r holds 16 chunks of 8 k; chunk c sits at slot
// r * 16 + (c ^ (r & 15)) so the 16 rows read in one LDS cycle hit 16
// distinct 16-byte bank groups.
__device__ __forceinline__ int xslot(int row, int chunk) { return row * 16 + (chunk ^ (row & 15)); }

template <int MF>
struct Stage {
  uint4* x;       // [MF * 16 rows][16 chunks]
  uint4* w;       // [64 rows][4 x 16 bytes]: words 4q..4q+3 of the group in part q
  uint32_t* s;    // [64 rows][2 dwords]: the group's 8 scale bytes of each row,
                  // then a second copy written by wavefronts 2 and 3 (unread)
};

template <int MF>
struct Src {
  const __bf16* x[MF];
  const uint32_t* w;
  const uint8_t* s;
};

// Per wavefront and group: MF activation loads, one word load, one scale
// load.  (Load-to-LDS writes 4 bytes per lane for its 1-, 2- and 4-byte
// forms, so the scales move as dwords; wavefronts 2 and 3 repeat the rows of
// 0 and 1 into the unread half so that every wavefront issues the same
// number of loads and one counter value fits all of them.)
template <int MF>
__device__ __forceinline__ void issue(const Stage<MF>& st, const Src<MF>& src, int64_t kg, int wave) {
#pragma unroll
  for (int i = 0; i < MF; ++i)
    __builtin_amdgcn_global_load_lds(src.x[i] + kg * kKG, NVFP4_LDS(&st.x[(i * 4 + wave) * 64]), 16, 0, 0);
  __builtin_amdgcn_global_load_lds(src.w + kg * 16, NVFP4_LDS(&st.w[wave * 64]), 16, 0, 0);
  __builtin_amdgcn_global_load_lds(src.s + kg * 8, NVFP4_LDS(&st.s[wave * 64]), 4, 0, 0);
}

// Wait until this wavefront's loads of the oldest group in flight have
// landed: at most two more groups (MF + 2 loads each) may be outstanding.
template <int MF>
__device__ __forceinline__ void wait_oldest_group() {
  constexpr int n = 2 * (MF + 2);
  static_assert(n < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4) | n);
}

// Four 16x16x32 steps over one group: lane (row, q) supplies word 4q+j of
// its weight row (k in [8(4q+j), 8(4q+j)+8) of the group) and the
// activation fragment reads the same chunk.
template <int MF>
__device__ __forceinline__ void compute(f32x4_t (&acc)[MF], const Stage<MF>& st, int wave, int lane) {
  const int r16 = lane & 15, q = lane >> 4;
  const int row = wave * 16 + r16;
  const uint4 wr = st.w[row * 4 + q];
  const uint32_t sv = st.s[row * 2 + (q >> 1)] >> (16 * (q & 1));
  const float s0 = e4m3<0>(sv), s1 = e4m3<1>(sv);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t word = j == 0 ? wr.x : j == 1 ? wr.y : j == 2 ? wr.z : wr.w;
    const bf16x8_t A = decode_word_bf16(word, j < 2 ? s0 : s1);
#pragma unroll
    for (int f = 0; f < MF; ++f) {
      const bf16x8_t B = __builtin_bit_cast(bf16x8_t, st.x[xslot(f * 16 + r16, 4 * q + j)]);
      acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[f], 0, 0, 0);
    }
  }
}

template <int MF>
__global__ __launch_bounds__(kThreads) void skinny_kernel(const __bf16* __restrict__ x,
                                                          const uint32_t* __restrict__ w,
                                                          const uint8_t* __restrict__ sc,
                                                          const float* __restrict__ gs,
                                                          __bf16* __restrict__ out, int64_t M,
                                                          int64_t K, int64_t N) {
  __shared__ uint4 x0[MF * 256], x1[MF * 256], x2[MF * 256], x3[MF * 256];
  __shared__ uint4 w0[256], w1[256], w2[256], w3[256];
  __shared__ uint32_t s0[256], s1[256], s2[256], s3[256];
  const Stage<MF> st0{x0, w0, s0}, st1{x1, w1, s1}, st2{x2, w2, s2}, st3{x3, w3, s3};

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int64_t kw = K / 8, ks = K / 16, nkg = K / kKG;

  // Source addresses for group 0.  Rows past M or N re-read the last row;
  // their results are never stored.
  Src<MF> src;
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const int slot = (i * 4 + wave) * 64 + lane;
    const int r = slot >> 4, c = (slot & 15) ^ (r & 15);
    const int64_t m = r < M ? r : M - 1;
    src.x[i] = x + m * K + c * 8;
  }
  {
    const int qd = wave * 64 + lane;            // words: [row][part of 16 bytes]
    int64_t n = n0 + (qd >> 2);
    if (n >= N) n = N - 1;
    src.w = w + n * kw + (qd & 3) * 4;
    const int qs = qd & 127;                    // scales: [row][dword]
    int64_t ns = n0 + (qs >> 1);
    if (ns >= N) ns = N - 1;
    src.s = sc + ns * ks + (qs & 1) * 4;
  }

  f32x4_t acc[MF];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[f][i] = 0.0f;

  issue(st0, src, 0, wave);
  issue(st1, src, nkg > 1 ? 1 : 0, wave);
  issue(st2, src, nkg > 2 ? 2 : nkg - 1, wave);

#define NVFP4_SK_STEP(S, CUR, FREE)                                            \
  do {                                                                         \
    wait_oldest_group<MF>();                                                   \
    __builtin_amdgcn_s_barrier();                                              \
    issue(FREE, src, ((S) + 3 < nkg) ? (S) + 3 : nkg - 1, wave);              \
    compute(acc, CUR, wave, lane);                                             \
  } while (0)

  int64_t s = 0;
  for (; s + 4 <= nkg; s += 4) {
    NVFP4_SK_STEP(s, st0, st3);
    NVFP4_SK_STEP(s + 1, st1, st0);
    NVFP4_SK_STEP(s + 2, st2, st1);
    NVFP4_SK_STEP(s + 3, st3, st2);
  }
  if (s < nkg) NVFP4_SK_STEP(s, st0, st3);
  if (s + 1 < nkg) NVFP4_SK_STEP(s + 1, st1, st0);
  if (s + 2 < nkg) NVFP4_SK_STEP(s + 2, st2, st1);
#undef NVFP4_SK_STEP
  __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4) | 0);  // no load may land after exit

  // C[n][m]: lane holds n = 4q + i (i = 0..3) of this wavefront's 16 rows,
  // m = lane % 16 of fragment f.
  const float g = global_factor(gs, 0);
  const bool vec_ok = (N % 4) == 0;
  const int q = lane >> 4;
#pragma unroll
  for (int f = 0; f < MF; ++f) {
    const int64_t m = f * 16 + (lane & 15);
    if (m >= M) continue;
    const int64_t n = n0 + wave * 16 + 4 * q;
    __bf16 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (__bf16)(acc[f][i] * g);
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

}  // namespace

namespace nvfp4host {

bool launch_skinny(const void* x, int64_t M, int64_t K, int64_t N, const uint32_t* w,
                   const uint8_t* sc, const float* gs, void* out, hipStream_t s) {
  if (M < 2 || M > 64 || K % kKG != 0 || (reinterpret_cast<uintptr_t>(sc) & 3) != 0) return false;
  const int64_t blocks = (N + kRows - 1) / kRows;
  const __bf16* xb = static_cast<const __bf16*>(x);
  __bf16* ob = static_cast<__bf16*>(out);
  const int mf = (int)((M + 15) / 16);
  switch (mf) {
    case 1: skinny_kernel<1><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(xb, w, sc, gs, ob, M, K, N); break;
    case 2: skinny_kernel<2><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(xb, w, sc, gs, ob, M, K, N); break;
    case 3: skinny_kernel<3><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(xb, w, sc, gs, ob, M, K, N); break;
    default: skinny_kernel<4><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(xb, w, sc, gs, ob, M, K, N); break;
  }
  return true;
}

}  // namespace nvfp4host
