// Decode kernel: out[1, N] = x[1, K] @ W[N, K]^T * g for one activation row
// (mlxcel PR "native NVFP4 for ROCm QuantizedMatmul/GatherQMM", "Summary":
// the qmv kernel the pages run for decode; g = global_scale / (448 * 6)
// applied once per output).
#include "glu_act.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4_internal.hpp"

using namespace nvfp4dev;

namespace {

// Wavefronts per block: eight for the one-row and gather forms, four for the
// gated form (two rows per wavefront).  Same-process A/B on the decode,
// gated decode and MoE decode shapes: eight measured 1-3% faster than four
// for the one-row and gather forms and about 1% slower for the gated form;
// two and sixteen were slower for all three.
template <bool GLU> constexpr int qmv1_waves() { return GLU ? 4 : 8; }
constexpr int kGatherWaves = 8;

// ----------------------------------------------------------------------------
// Decode kernel for M = 1.
//
// Each wavefront owns R consecutive weight rows (R = 1 measured best) and
// issues every load of its rows (16-byte word chunks and their scale bytes)
// right after its share of the activation row, which goes to LDS once per
// block; it then waits for the activation pieces only and decodes each chunk
// as it lands.  Lane l owns chunk positions l, l+64, ... (CPL of them) of
// each row, so a wave load is 1 KiB of one row.  Waves are short-lived and
// the grid has N / (8R) blocks of eight wavefronts (the gated form: four);
// with ~50 VGPRs eight waves fit per SIMD, so
// several blocks' loads overlap each other's decode.  Measured against a
// plain streaming read of the same bytes, this beats a persistent
// row-streaming kernel whose prefetch depth could not cover HBM latency,
// and two or more rows per wavefront.
// ----------------------------------------------------------------------------

// LDS placement of the staged activation row.  A weight chunk (32
// elements) meets PPC 16-byte activation pieces (4 for 2-byte types, 8 for
// float32), and lane l reads the pieces of chunk l, so the 16 lanes served
// together read 16 consecutive chunks.  Stored in order, every fourth (2-byte
// types) or second (float32) chunk would start in the same bank; instead the
// pieces of chunk c are rotated by its position within the 256-byte bank
// row, piece q at slot c * PPC + (q + c / CPR) mod PPC with CPR = 256 / (16
// PPC) chunks per row, which spreads the 16 lanes over all 64 banks.
template <int PPC>
__device__ __forceinline__ int x_slot(int c, int q) {
  constexpr int kCpr = 16 / PPC;
  return c * PPC + ((q + c / kCpr) & (PPC - 1));
}

// The global piece stored at LDS slot s (the inverse of x_slot).
template <int PPC>
__device__ __forceinline__ int64_t x_piece(int64_t s) {
  constexpr int kCpr = 16 / PPC;
  const int64_t c = s / PPC;
  const int64_t rot = (c / kCpr) & (PPC - 1);
  return c * PPC + ((s - c * PPC - rot) & (PPC - 1));
}

// One 16-byte chunk (two scale blocks) against 32 activations.
__device__ __forceinline__ float chunk_dot_lds(const uint4& w, uint32_t s, const uint4* xl, int c, __bf16*) {
  uint32_t xp[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = xl[x_slot<4>(c, q)];
    xp[4 * q] = v.x; xp[4 * q + 1] = v.y; xp[4 * q + 2] = v.z; xp[4 * q + 3] = v.w;
  }
  float p0 = dot_word_bf16(w.x, xp + 0, 0.0f);
  p0 = dot_word_bf16(w.y, xp + 4, p0);
  float p1 = dot_word_bf16(w.z, xp + 8, 0.0f);
  p1 = dot_word_bf16(w.w, xp + 12, p1);
  return __builtin_fmaf(p1, e4m3<1>(s), p0 * e4m3<0>(s));
}

// float32 activations.
__device__ __forceinline__ float chunk_dot_lds(const uint4& w, uint32_t s, const uint4* xl, int c, float*) {
  float xv[32];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint4 v = xl[x_slot<8>(c, q)];
    xv[4 * q] = __builtin_bit_cast(float, v.x); xv[4 * q + 1] = __builtin_bit_cast(float, v.y);
    xv[4 * q + 2] = __builtin_bit_cast(float, v.z); xv[4 * q + 3] = __builtin_bit_cast(float, v.w);
  }
  float p0 = dot_word_f32(w.x, xv + 0, 0.0f);
  p0 = dot_word_f32(w.y, xv + 8, p0);
  float p1 = dot_word_f32(w.z, xv + 16, 0.0f);
  p1 = dot_word_f32(w.w, xv + 24, p1);
  return __builtin_fmaf(p1, e4m3<1>(s), p0 * e4m3<0>(s));
}

// f16 activations, widened to float32 after the LDS read.
__device__ __forceinline__ float chunk_dot_lds(const uint4& w, uint32_t s, const uint4* xl, int c, _Float16*) {
  float xv[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = xl[x_slot<4>(c, q)];
    const _Float16* h = reinterpret_cast<const _Float16*>(&v);
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[8 * q + j] = (float)h[j];
  }
  float p0 = dot_word_f32(w.x, xv + 0, 0.0f);
  p0 = dot_word_f32(w.y, xv + 8, p0);
  float p1 = dot_word_f32(w.z, xv + 16, 0.0f);
  p1 = dot_word_f32(w.w, xv + 24, p1);
  return __builtin_fmaf(p1, e4m3<1>(s), p0 * e4m3<0>(s));
}

// The activation row is copied to LDS by the load-to-LDS path (no
// registers involved), 1 KiB per wavefront instruction; lane l of piece p
// fills slot 64 p + l with the global piece x_piece(64 p + l).  The last
// piece may run past the row: those lanes re-read the row's last 16 bytes
// into LDS padding that is never read.
#define NVFP4_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// W = wavefronts per block: wavefront `wave` copies pieces wave, wave + W, ...
template <int W, typename TX>
__device__ __forceinline__ int stage_x_lds(uint4* xl, const TX* x, int64_t K, int lane, int wave) {
  const int64_t n16 = K * (int64_t)sizeof(TX) / 16;
  const int64_t pieces = (n16 + 63) / 64;
  int issued = 0;
  constexpr int kPpc = 32 * (int)sizeof(TX) / 16;   // pieces per 32-element chunk
  for (int64_t p = wave; p < pieces; p += W) {
    int64_t q = x_piece<kPpc>(p * 64 + lane);
    q = q < n16 ? q : n16 - 1;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(x) + q, NVFP4_LDS(xl + p * 64), 16, 0, 0);
    ++issued;
  }
  return issued;
}

// Bytes of LDS the staged row occupies (whole 1 KiB pieces).
template <typename TX>
size_t staged_x_bytes(int64_t K) {
  const int64_t n16 = K * (int64_t)sizeof(TX) / 16;
  return (size_t)((n16 + 63) / 64) * 1024;
}

// Element type of the staged activations (the activation type itself).
template <typename TX> struct LdsElem { typedef TX type; };

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw byte-buffer descriptor: loads at offsets >= bytes return 0 without
// touching memory.
__device__ __forceinline__ rsrc_t byte_buffer(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// An offset no plane reaches (planes stay below 2^31 bytes).
constexpr uint32_t kOutOfRange = 0x80000000u;

// Cache policy of the weight and scale plane loads.  The one-row kernel
// reads each plane byte once per call, so its loads are non-temporal (the
// `nt` bit): measured 2% faster on the decode workload and 9% on the gated
// decode form (`sc1` was slower).  In the gather form, pairs that share an
// expert re-read its plane, which the default policy leaves in the caches:
// `nt` there measured 3-9% slower.
constexpr int kPlaneLoad = 2;
constexpr int kGatherPlaneLoad = 0;

// GLU: the gated projection of an MLP at M = 1 (mlxcel issue "perf(metal):
// close native NVFP4 prefill gap", "Activation-path follow-up").  The
// wavefront's two rows are feature f of the gate plane (w, sc, gs) and of the
// up plane (wu, scu, gsu), and lane 0 stores act(g * gate) * (g_u * up).
// BAT: batched weights, blockIdx.y selects the matrix (strides bst); a
// separate instantiation so the single-matrix kernel reads no strides.
template <typename TX, int CPL, int R, bool GLU = false, bool BAT = false>
__global__ __launch_bounds__(64 * qmv1_waves<GLU>()) void qmv1_kernel(const TX* __restrict__ x,
                                                        const uint32_t* w,
                                                        const uint8_t* sc,
                                                        const float* __restrict__ gs,
                                                        TX* __restrict__ out, int64_t K, int64_t N,
                                                        const uint32_t* wu = nullptr,
                                                        const uint8_t* scu = nullptr,
                                                        const float* __restrict__ gsu = nullptr, int act = 0,
                                                        MatrixStrides bst = {}) {
  static_assert(!GLU || R == 2, "the gated form streams one gate row and one up row");
  extern __shared__ uint4 xl[];
  if constexpr (BAT) {
    const int64_t bm = blockIdx.y;
    x += bm * bst.x;
    w += bm * bst.w;
    sc += bm * bst.s;
    out += bm * bst.o;
    if (gs) gs += bm;
  }
  const int lane = threadIdx.x & 63;
  constexpr int kW = qmv1_waves<GLU>();
  const int64_t n0 = ((int64_t)blockIdx.x * kW + (threadIdx.x >> 6)) * (GLU ? 1 : R);
  const int64_t kw = K / 8, ks = K / 16, nchunks = kw / 4;
  const int nch = (int)nchunks;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // 0. The activation row goes straight to LDS (no registers, so nothing
  //    below has to wait for it to land before issuing).  These are this
  //    wave's first vector-memory operations.
  stage_x_lds<kW>(xl, x, K, lane, wave);
  __builtin_amdgcn_sched_barrier(0);
  // 1. All weight and scale loads of this wave's rows, back to back, as
  //    buffer loads: chunks past the row end and rows past N get an
  //    out-of-range offset and read 0 without a memory access (their
  //    results are never used), so every lane issues every load and no
  //    result has to be merged with a default value.
  const rsrc_t wb = byte_buffer(w, N * kw * 4);
  const rsrc_t sb = byte_buffer(sc, N * ks);
  const rsrc_t wb2 = GLU ? byte_buffer(wu, N * kw * 4) : wb;
  const rsrc_t sb2 = GLU ? byte_buffer(scu, N * ks) : sb;
  uint4 wv[R][CPL];
  uint32_t sv[R][CPL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t n = GLU ? n0 : n0 + r;
    const rsrc_t& wr = (GLU && r == 1) ? wb2 : wb;
    const rsrc_t& sr = (GLU && r == 1) ? sb2 : sb;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      const bool ok = n < N && c < nch;
      const uint32_t wo = ok ? (uint32_t)(n * kw * 4 + c * 16) : kOutOfRange;
      const uint32_t so = ok ? (uint32_t)(n * ks + c * 2) : kOutOfRange;
      wv[r][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, wo, 0, kPlaneLoad));
      sv[r][i] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(sr, so, 0, kPlaneLoad);
    }
  }
  // 2. Wait only for the activation pieces (issued before the 2 R CPL loads
  //    above; loads complete in order), then the block barrier makes every
  //    wave's pieces visible.  The weights are consumed as they arrive.
  constexpr int kLoads = 2 * R * CPL;   // vmcnt: 6 bits, low 4 at [3:0], high 2 at [15:14]
  static_assert(kLoads < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4) | (kLoads & 0xF) | ((kLoads >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  // 3. Decode and reduce.
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        acc[r] += chunk_dot_lds(wv[r][i], sv[r][i], xl, c, (typename LdsElem<TX>::type*)nullptr);
    }
  }
  const float g = global_factor(gs, 0);
  if constexpr (GLU) {
    const float gate = wave_sum_dpp(acc[0]), up = wave_sum_dpp(acc[1]);
    if (lane == 0 && n0 < N) store_out(out + n0, glu_act(gate * g, act) * (up * global_factor(gsu, 0)));
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = wave_sum_dpp(acc[r]);
      if (lane == 0 && n0 + r < N) store_out(out + n0 + r, v * g);
    }
  }
}

// Gather form of the one-row kernel, for GatherQMM with one activation row
// per pair (mlxcel PR "native NVFP4 for ROCm QuantizedMatmul/GatherQMM",
// "Summary" and "Changes during review": pair r multiplies activation row
// lhs[r] by expert rhs[r]'s planes, scaled by that expert's global factor;
// an out-of-range expert or activation row gives exact zeros).  Block (b, r)
// computes outputs 8b .. 8b+7 of pair r exactly as the one-row kernel does
// for that expert's plane, so a gathered row equals the plain decode of the
// same expert bit for bit.
template <typename TX, int CPL>
__global__ __launch_bounds__(64 * kGatherWaves) void qmv1_gather_kernel(const TX* __restrict__ x, int64_t X, int64_t K,
                                                               const int32_t* __restrict__ lhs,
                                                               const int32_t* __restrict__ rhs, const uint32_t* w,
                                                               const uint8_t* sc, const float* __restrict__ gs,
                                                               int64_t E, int64_t N, TX* __restrict__ out) {
  extern __shared__ uint4 xl[];
  const int64_t r = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t n = (int64_t)blockIdx.x * kGatherWaves + wave;
  const int64_t e = rhs[r];
  const int64_t src = lhs ? (int64_t)lhs[r] : r;
  TX* o = out + r * N;
  if (e < 0 || e >= E || src < 0 || src >= X) {   // uniform over the block, before any barrier
    if (lane == 0 && n < N) store_out(o + n, 0.0f);
    return;
  }
  const int64_t kw = K / 8, ks = K / 16;
  const int nch = (int)(kw / 4);
  stage_x_lds<kGatherWaves>(xl, x + src * K, K, lane, wave);
  __builtin_amdgcn_sched_barrier(0);
  const rsrc_t wb = byte_buffer(w + e * N * kw, N * kw * 4);
  const rsrc_t sb = byte_buffer(sc + e * N * ks, N * ks);
  uint4 wv[CPL];
  uint32_t sv[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    const bool ok = n < N && c < nch;
    const uint32_t wo = ok ? (uint32_t)(n * kw * 4 + c * 16) : kOutOfRange;
    const uint32_t so = ok ? (uint32_t)(n * ks + c * 2) : kOutOfRange;
    wv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wb, wo, 0, kGatherPlaneLoad));
    sv[i] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(sb, so, 0, kGatherPlaneLoad);
  }
  constexpr int kLoads = 2 * CPL;
  __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4) | (kLoads & 0xF) | ((kLoads >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) acc += chunk_dot_lds(wv[i], sv[i], xl, c, (typename LdsElem<TX>::type*)nullptr);
  }
  const float v = wave_sum_dpp(acc);
  if (lane == 0 && n < N) store_out(o + n, v * global_factor(gs, e));
}

template <typename TX, int CPL>
void qmv1_gather_launch(const TX* x, int64_t X, int64_t K, const int32_t* lhs, const int32_t* rhs, int64_t R,
                        const uint32_t* w, const uint8_t* sc, const float* gs, int64_t E, int64_t N, TX* out,
                        hipStream_t s) {
  const int64_t blocks = (N + kGatherWaves - 1) / kGatherWaves;
  qmv1_gather_kernel<TX, CPL><<<dim3((unsigned)blocks, (unsigned)R), dim3(64 * kGatherWaves), staged_x_bytes<TX>(K), s>>>(
      x, X, K, lhs, rhs, w, sc, gs, E, N, out);
}

// True when the gather form handles this case (and launches it): as for
// try_qmv1 with each expert's plane below 2^31 bytes, and at most one grid
// row per pair.
template <typename TX>
bool try_qmv1_gather(const TX* x, int64_t X, int64_t K, const int32_t* lhs, const int32_t* rhs, int64_t R,
                     const uint32_t* w, const uint8_t* sc, const float* gs, int64_t E, int64_t N, TX* out,
                     hipStream_t s) {
  if (K % 32 != 0 || N * (K / 2) >= ((int64_t)1 << 31) || R > nvfp4host::kMaxGridY) return false;
  switch ((K / 32 + 63) / 64) {
    case 1: qmv1_gather_launch<TX, 1>(x, X, K, lhs, rhs, R, w, sc, gs, E, N, out, s); return true;
    case 2: qmv1_gather_launch<TX, 2>(x, X, K, lhs, rhs, R, w, sc, gs, E, N, out, s); return true;
    case 3: qmv1_gather_launch<TX, 3>(x, X, K, lhs, rhs, R, w, sc, gs, E, N, out, s); return true;
    case 4: qmv1_gather_launch<TX, 4>(x, X, K, lhs, rhs, R, w, sc, gs, E, N, out, s); return true;
    default: return false;
  }
}

constexpr int kQmv1Rows = 1;

// B matrices (B <= 65535) with strides bst, one per grid row.
template <typename TX, int CPL>
void qmv1_launch(const TX* x, int64_t K, int64_t N, const uint32_t* w, const uint8_t* sc,
                 const float* gs, TX* out, hipStream_t s, int64_t B, MatrixStrides bst) {
  constexpr int kW = qmv1_waves<false>();
  const int64_t blocks = (N + kW * kQmv1Rows - 1) / (kW * kQmv1Rows);
  const size_t lds = staged_x_bytes<TX>(K);
  if (B > 1)
    qmv1_kernel<TX, CPL, kQmv1Rows, false, true><<<dim3((unsigned)blocks, (unsigned)B), dim3(64 * kW), lds, s>>>(
        x, w, sc, gs, out, K, N, nullptr, nullptr, nullptr, 0, bst);
  else
    qmv1_kernel<TX, CPL, kQmv1Rows><<<dim3((unsigned)blocks), dim3(64 * kW), lds, s>>>(x, w, sc, gs, out, K, N);
}

template <typename TX, int CPL>
void qmv1_glu_launch(const TX* x, int64_t K, int64_t F, const uint32_t* w, const uint8_t* sc, const float* gs,
                     const uint32_t* wu, const uint8_t* scu, const float* gsu, int act, TX* out, hipStream_t s) {
  constexpr int kW = qmv1_waves<true>();
  const int64_t blocks = (F + kW - 1) / kW;
  const size_t lds = staged_x_bytes<TX>(K);
  qmv1_kernel<TX, CPL, 2, true><<<dim3((unsigned)blocks), dim3(64 * kW), lds, s>>>(x, w, sc, gs, out, K, F, wu, scu,
                                                                                   gsu, act);
}

// True when the decode kernel's gated form handles this K (and launches it):
// as for try_qmv1, with both planes below 2^31 bytes.
template <typename TX>
bool try_qmv1_glu(const TX* x, int64_t K, int64_t F, const uint32_t* w, const uint8_t* sc, const float* gs,
                  const uint32_t* wu, const uint8_t* scu, const float* gsu, int act, TX* out, hipStream_t s) {
  if (K % 32 != 0 || F * (K / 2) >= ((int64_t)1 << 31)) return false;
  switch ((K / 32 + 63) / 64) {
    case 1: qmv1_glu_launch<TX, 1>(x, K, F, w, sc, gs, wu, scu, gsu, act, out, s); return true;
    case 2: qmv1_glu_launch<TX, 2>(x, K, F, w, sc, gs, wu, scu, gsu, act, out, s); return true;
    case 3: qmv1_glu_launch<TX, 3>(x, K, F, w, sc, gs, wu, scu, gsu, act, out, s); return true;
    case 4: qmv1_glu_launch<TX, 4>(x, K, F, w, sc, gs, wu, scu, gsu, act, out, s); return true;
    default: return false;
  }
}

// True when the M = 1 decode kernel handles this K (and launches it):
// K % 32 == 0, at most 4 chunks per lane (K <= 8192, LDS <= 32 KiB) and a
// weight plane below 2^31 bytes (32-bit buffer offsets).  B matrices with
// strides bst (1 and zeros for one matrix), B <= 65535.
template <typename TX>
bool try_qmv1(const TX* x, int64_t K, int64_t N, const uint32_t* w, const uint8_t* sc,
              const float* gs, TX* out, hipStream_t s, int64_t B = 1, MatrixStrides bst = {}) {
  if (K % 32 != 0 || N * (K / 2) >= ((int64_t)1 << 31)) return false;
  const int64_t cpl = (K / 32 + 63) / 64;
  switch (cpl) {
    case 1: qmv1_launch<TX, 1>(x, K, N, w, sc, gs, out, s, B, bst); return true;
    case 2: qmv1_launch<TX, 2>(x, K, N, w, sc, gs, out, s, B, bst); return true;
    case 3: qmv1_launch<TX, 3>(x, K, N, w, sc, gs, out, s, B, bst); return true;
    case 4: qmv1_launch<TX, 4>(x, K, N, w, sc, gs, out, s, B, bst); return true;
    default: return false;
  }
}


}  // namespace

namespace nvfp4host {

bool launch_decode(const void* x, nvfp4_dtype_t dt, int64_t K, int64_t N, const uint32_t* w,
                   const uint8_t* sc, const float* gs, void* out, hipStream_t s, int64_t B, int64_t x_stride) {
  const MatrixStrides bst{x_stride, N * (K / 8), N * (K / 16), N};
  switch (dt) {
    case NVFP4_BF16:
      return try_qmv1<__bf16>(static_cast<const __bf16*>(x), K, N, w, sc, gs, static_cast<__bf16*>(out), s, B, bst);
    case NVFP4_F32:
      return try_qmv1<float>(static_cast<const float*>(x), K, N, w, sc, gs, static_cast<float*>(out), s, B, bst);
    case NVFP4_F16:
      return try_qmv1<_Float16>(static_cast<const _Float16*>(x), K, N, w, sc, gs, static_cast<_Float16*>(out), s,
                                B, bst);
  }
  return false;
}

bool launch_decode_gather(const void* x, nvfp4_dtype_t dt, int64_t X, int64_t K, const int32_t* lhs,
                          const int32_t* rhs, int64_t R, const uint32_t* w, const uint8_t* sc, const float* gs,
                          int64_t E, int64_t N, void* out, hipStream_t s) {
  switch (dt) {
    case NVFP4_BF16:
      return try_qmv1_gather<__bf16>(static_cast<const __bf16*>(x), X, K, lhs, rhs, R, w, sc, gs, E, N,
                                     static_cast<__bf16*>(out), s);
    case NVFP4_F32:
      return try_qmv1_gather<float>(static_cast<const float*>(x), X, K, lhs, rhs, R, w, sc, gs, E, N,
                                    static_cast<float*>(out), s);
    case NVFP4_F16:
      return try_qmv1_gather<_Float16>(static_cast<const _Float16*>(x), X, K, lhs, rhs, R, w, sc, gs, E, N,
                                       static_cast<_Float16*>(out), s);
  }
  return false;
}

bool decode_glu_applies(int64_t K, int64_t F) {
  return K > 0 && K % 32 == 0 && (K / 32 + 63) / 64 <= 4 && F * (K / 2) < ((int64_t)1 << 31);
}

bool launch_decode_glu(const void* x, nvfp4_dtype_t dt, int64_t K, int64_t F, const uint32_t* w,
                       const uint8_t* sc, const float* gs, const uint32_t* wu, const uint8_t* scu,
                       const float* gsu, int act, void* out, hipStream_t s) {
  switch (dt) {
    case NVFP4_BF16:
      return try_qmv1_glu<__bf16>(static_cast<const __bf16*>(x), K, F, w, sc, gs, wu, scu, gsu, act,
                                  static_cast<__bf16*>(out), s);
    case NVFP4_F32:
      return try_qmv1_glu<float>(static_cast<const float*>(x), K, F, w, sc, gs, wu, scu, gsu, act,
                                 static_cast<float*>(out), s);
    case NVFP4_F16:
      return try_qmv1_glu<_Float16>(static_cast<const _Float16*>(x), K, F, w, sc, gs, wu, scu, gsu, act,
                                    static_cast<_Float16*>(out), s);
  }
  return false;
}

}  // namespace nvfp4host
