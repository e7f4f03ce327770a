// MFMA kernel for small M ("multi-row qmv", speculative-decode verify widths):
// out[M, N] = x[M, K] @ W[N, K]^T * g with bf16 activations, 2 <= M <= 64.
//
// The pages run these widths through their qmv kernel, eight activation
// rows per block (mlxcel PR "native NVFP4 for ROCm QuantizedMatmul/
// GatherQMM", "Summary" and the multi-row rows of "Numerical results").
// On gfx950 a dot-product loop costs one VALU operation per weight element
// per activation row; here each packed word is decoded once (exact bf16
// products e2m1 * e4m3) into the A operand of a 16x16x32 bf16 MFMA and
// multiplied against every 16-row activation fragment, so the VALU cost no
// longer grows with M.
//
// The work is bound by streaming the weight plane, and what streams it
// fastest on this part is many wavefronts each holding all of their loads
// in flight in registers (measured: a barrier-paced global->LDS pipeline of
// the same plane reached 50-75% of that rate).  A load instruction costs
// about one cache-line lookup per line it touches, whatever it takes from
// the line, so the k order inside the MFMA is chosen to make every load
// read 64 contiguous bytes per row:
//  * a block owns 64 weight rows (four 16-row MFMA tiles, so one activation
//    load feeds four tiles) and up to 16 wavefronts;
//  * k runs in "pair-groups" of 256 (two chunks of 16 words per row); wave
//    w takes pair-groups w, w + W, ... of the W wavefronts -- for K up to
//    4096 that is one pair-group each, with every load of the block in
//    flight at once (a software pipeline inside a wavefront is what the
//    compiler reorders into load-wait-compute, so parallelism comes from
//    the wavefronts instead);
//  * lane (r, q) (r = lane % 16, q = lane / 16) loads words 4q..4q+3 of
//    each chunk of its weight row (16 bytes; the four q lanes cover 64
//    contiguous bytes), then a 4x4 transpose across the q lanes (two
//    v_permlane32_swap and two v_permlane16_swap per four words) leaves it
//    words q, 4+q, 8+q, 12+q;
//  * MFMA step (c, i) of chunk c takes word 4i+q of that chunk from lane q,
//    so the activations it multiplies -- 8 bf16 per lane, one 16-byte load
//    -- are again 64 contiguous bytes across the q lanes;
//  * the 16 scale bytes of a row's pair-group come in one 16-byte load;
//    word 4i+q uses byte 2i + q/2 of its chunk's eight;
//  * the four wavefronts' partial sums meet in LDS at the end, are added in
//    a fixed order and scaled by g once.
#include "nvfp4_device.hpp"
#include "nvfp4_internal.hpp"

using namespace nvfp4dev;

namespace {

constexpr int kTiles = 4;       // 16-row MFMA tiles per block
constexpr int kRows = 16 * kTiles;
constexpr int kPG = 256;        // k per pair-group

// One pair-group's operands for one lane.
template <int MF>
struct PairGroup {
  uint4 w[kTiles][2]; // [tile][chunk]: words 4q..4q+3 of the chunk
  uint4 s[kTiles];    // [tile]: the row's 16 scale bytes of the pair-group
  uint4 x[MF][8];     // [fragment][step 4c+i]: activations of word 16c+4i+q
};

template <int MF>
struct Sources {
  const uint4* w[kTiles]; // weight row base + 4q words
  const uint4* s[kTiles]; // scale row base
  const uint4* x[MF];     // activation row base + 8q elements
};

// Loads are issued in the order compute_pg consumes them (chunk 0: its
// activations, then scales and words tile by tile; chunk 1: activations,
// words), so the in-order load counter lets chunk 0 be multiplied while
// chunk 1 is still arriving.
template <int MF>
__device__ __forceinline__ void load_pg(PairGroup<MF>& p, const Sources<MF>& src, int64_t pg) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i)         // element offset 128c + 32i = 16-byte unit 16c + 4i
        p.x[f][4 * c + i] = src.x[f][pg * 32 + c * 16 + i * 4];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      if (c == 0) p.s[t] = src.s[t][pg];  // 16 scale bytes per pair-group
      p.w[t][c] = src.w[t][pg * 8 + c * 4];  // 32 words per pair-group; chunk 1 is 16 words on
    }
  }
}

// 4x4 transpose across the four 16-lane rows: on entry lane row q holds
// words 4q..4q+3 (v.x..v.w); on return element i holds word 4i+q.
__device__ __forceinline__ void transpose_q(const uint4 v, uint32_t (&o)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  o[0] = c[0];
  o[1] = c[1];
  o[2] = d[0];
  o[3] = d[1];
}

template <int MF>
__device__ __forceinline__ void compute_pg(f32x4_t (&acc)[kTiles][MF], const PairGroup<MF>& p, int half) {
  // word 4i+q of chunk c uses scale byte 8c + 2i + q/2: dword 2c + i/2,
  // byte 2(i%2) + q/2
  const uint32_t sh = 8u * (uint32_t)half;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const uint32_t d0 = (c == 0 ? p.s[t].x : p.s[t].z) >> sh;
      const uint32_t d1 = (c == 0 ? p.s[t].y : p.s[t].w) >> sh;
      uint32_t wd[4];
      transpose_q(p.w[t][c], wd);
      const float sc[4] = {e4m3<0>(d0), e4m3<2>(d0), e4m3<0>(d1), e4m3<2>(d1)};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8_t A = decode_word_bf16(wd[i], sc[i]);
#pragma unroll
        for (int f = 0; f < MF; ++f)
          acc[t][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              A, __builtin_bit_cast(bf16x8_t, p.x[f][4 * c + i]), acc[t][f], 0, 0, 0);
      }
    }
  }
}

template <int MF, int MAXW>
__global__ __launch_bounds__(64 * MAXW) void skinny_kernel(const __bf16* __restrict__ x,
                                                          const uint32_t* __restrict__ w,
                                                          const uint8_t* __restrict__ sc,
                                                          const float* __restrict__ gs,
                                                          __bf16* __restrict__ out, int64_t M,
                                                          int64_t K, int64_t N) {
  __shared__ f32x4_t red[MAXW][kTiles * MF][64];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nw = (int)(blockDim.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int64_t npg = K / kPG;

  // Rows past N or M re-read the last row; their results are never stored.
  Sources<MF> src;
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    int64_t n = n0 + 16 * t + r16;
    if (n >= N) n = N - 1;
    src.w[t] = reinterpret_cast<const uint4*>(w + n * (K / 8) + 4 * q);
    src.s[t] = reinterpret_cast<const uint4*>(sc + n * (K / 16));
  }
#pragma unroll
  for (int f = 0; f < MF; ++f) {
    int64_t m = 16 * f + r16;
    if (m >= M) m = M - 1;
    src.x[f] = reinterpret_cast<const uint4*>(x + m * K + 8 * q);
  }

  f32x4_t acc[kTiles][MF];
#pragma unroll
  for (int t = 0; t < kTiles; ++t)
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][f][i] = 0.0f;

  PairGroup<MF> p;
  for (int64_t pg = wid; pg < npg; pg += nw) {
    load_pg(p, src, pg);
    // keep every load ahead of the multiply: the scheduler would otherwise
    // sink each load to its use and expose its latency one by one
    __builtin_amdgcn_sched_barrier(0);
    compute_pg(acc, p, q >> 1);
  }

  // Partial sums of the wavefronts, added in wavefront order.
#pragma unroll
  for (int t = 0; t < kTiles; ++t)
#pragma unroll
    for (int f = 0; f < MF; ++f) red[wid][t * MF + f][lane] = acc[t][f];
  __syncthreads();

  const float g = global_factor(gs, 0);
  const bool vec_ok = (N % 4) == 0;
  for (int idx = threadIdx.x; idx < kTiles * MF * 64; idx += blockDim.x) {
    const int tf = idx >> 6, l = idx & 63;
    const int t = tf / MF, f = tf % MF;
    f32x4_t v = red[0][tf][l];
    for (int k = 1; k < nw; ++k) {
      const f32x4_t pk = red[k][tf][l];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += pk[i];
    }
    // C[n][m]: element i is weight row 16t + 4(l/16) + i, activation row 16f + l%16.
    const int64_t m = 16 * f + (l & 15);
    if (m >= M) continue;
    const int64_t n = n0 + 16 * t + 4 * (l >> 4);
    __bf16 o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (__bf16)(v[i] * g);
    __bf16* po = out + m * N + n;
    if (vec_ok && n + 3 < N) {
      *reinterpret_cast<uint2*>(po) = __builtin_bit_cast(uint2, o);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n + i < N) po[i] = o[i];
    }
  }
}

// One wavefront per pair-group up to MAXW wavefronts.
template <int MF, int MAXW>
void launch_mf(const __bf16* x, int64_t M, int64_t K, int64_t N, const uint32_t* w, const uint8_t* sc,
               const float* gs, __bf16* out, hipStream_t s) {
  const int64_t blocks = (N + kRows - 1) / kRows;
  const int64_t npg = K / kPG;
  const int waves = (int)(npg < MAXW ? npg : MAXW);
  skinny_kernel<MF, MAXW><<<dim3((unsigned)blocks), dim3(64 * waves), 0, s>>>(x, w, sc, gs, out, M, K, N);
}

}  // namespace

namespace nvfp4host {

bool launch_skinny(const void* x, int64_t M, int64_t K, int64_t N, const uint32_t* w,
                   const uint8_t* sc, const float* gs, void* out, hipStream_t s) {
  // 16-byte activation, word and scale loads.
  const bool aligned =
      ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(sc)) & 15) == 0;
  if (M < 2 || M > 64 || K % kPG != 0 || !aligned) return false;
  const __bf16* xb = static_cast<const __bf16*>(x);
  __bf16* ob = static_cast<__bf16*>(out);
  switch ((M + 15) / 16) {
    case 1: launch_mf<1, 16>(xb, M, K, N, w, sc, gs, ob, s); break;
    case 2: launch_mf<2, 8>(xb, M, K, N, w, sc, gs, ob, s); break;
    case 3: launch_mf<3, 4>(xb, M, K, N, w, sc, gs, ob, s); break;
    default: launch_mf<4, 4>(xb, M, K, N, w, sc, gs, ob, s); break;
  }
  return true;
}

}  // namespace nvfp4host
