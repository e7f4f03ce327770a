// Internal host-side launchers shared between the C-ABI layer and the kernel
// translation units.  Every launcher assumes its arguments were validated by
// the C-ABI layer (shapes, alignment, grid limits) and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4.h"

namespace nvfp4host {

// Byte copy dst <- src of n bytes (dst == src is a no-op).
void launch_copy_bytes(const uint8_t* src, uint8_t* dst, int64_t n, hipStream_t s);
// Zero n bytes at dst (16-byte aligned), with a kernel rather than a memset
// so the call is safe inside captured graphs.
void launch_fill_zero(void* dst, int64_t n, hipStream_t s);
// gs_out[b] = fl32(ws2[b] * 2688).
void launch_sidecar(const float* ws2, float* gs_out, int64_t batch, hipStream_t s);
// Dequantize [batch*rows, cols/8] words into out of dtype.
void launch_dequantize(const uint32_t* w, const uint8_t* sc, const float* gs, int64_t batch,
                       int64_t rows, int64_t cols, nvfp4_dtype_t dt, void* out, hipStream_t s);
// Quantize [batch, rows, cols] dense values (cols % 16 == 0) into words,
// scale codes and (when gs_in is NULL) per-matrix global scales in gs_out;
// with gs_in, gs_out (if not NULL) receives a copy of it.
void launch_quantize(const void* w, nvfp4_dtype_t dt, int64_t batch, int64_t rows, int64_t cols,
                     const float* gs_in, uint32_t* w_out, uint8_t* sc_out, float* gs_out, hipStream_t s);
// Gated projection at M = 1 in one launch of the decode kernel (two rows
// per wavefront: a feature's gate row and up row).  decode_glu_applies says
// whether launch_decode_glu takes these sizes (it returns false otherwise).
bool decode_glu_applies(int64_t K, int64_t F);
bool launch_decode_glu(const void* x, nvfp4_dtype_t dt, int64_t K, int64_t F, const uint32_t* w,
                       const uint8_t* sc, const float* gs, const uint32_t* wu, const uint8_t* scu,
                       const float* gsu, int act, void* out, hipStream_t s);
// Gated projection for 2 <= M <= 64 through the multi-row MFMA kernel (a
// block holds 32 features' gate and up rows).  skinny_glu_applies checks the
// sizes; launch_skinny_glu also needs 16-byte aligned x, planes and scales
// and returns false otherwise.
bool skinny_glu_applies(int64_t M, int64_t K, int64_t F);
bool launch_skinny_glu(const void* x, nvfp4_dtype_t dt, int64_t M, int64_t K, int64_t F, const uint32_t* w,
                       const uint8_t* sc, const float* gs, const uint32_t* wu, const uint8_t* scu,
                       const float* gsu, int act, void* out, hipStream_t s);
// GatherQMM with one activation row per pair through the decode kernel's
// gather form; false when that form does not apply (nothing launched).
bool launch_decode_gather(const void* x, nvfp4_dtype_t dt, int64_t X, int64_t K, const int32_t* lhs,
                          const int32_t* rhs, int64_t R, const uint32_t* w, const uint8_t* sc, const float* gs,
                          int64_t E, int64_t N, void* out, hipStream_t s);

// Decode kernel (M = 1): returns false, launching nothing, when K is not
// a multiple of 32, K > 8192 or the weight plane reaches 2^31 bytes.
// With B > 1 (B <= 65535), one launch serves B matrices: matrix b reads
// x + b * x_stride (elements), plane b, scales b and gs[b] (when gs is not
// NULL) and writes out + b * N.
bool launch_decode(const void* x, nvfp4_dtype_t dt, int64_t K, int64_t N, const uint32_t* w,
                   const uint8_t* sc, const float* gs, void* out, hipStream_t s, int64_t B = 1,
                   int64_t x_stride = 0);
// Dense qmv: out[M,N] = x[M,K] @ W[N,K]^T (transposed plane).
void launch_qmv(const void* x, nvfp4_dtype_t dt, int64_t M, int64_t K, int64_t N,
                const uint32_t* w, const uint8_t* sc, const float* gs, void* out, hipStream_t s);
// MFMA kernel for 2 <= M <= 64 (bf16, f16, or f32 activations split into
// three bf16 parts), transposed plane, K % 256 == 0, 16-byte aligned x, w
// and scales; returns false (launching nothing) otherwise.  With B > 1 (B <=
// 65535) one launch serves B matrices as launch_decode's batched form does
// (x + b * x_stride elements, plane, scales and gs[b] of matrix b; out + b *
// M * N).
bool launch_skinny(const void* x, nvfp4_dtype_t dt, int64_t M, int64_t K, int64_t N, const uint32_t* w,
                   const uint8_t* sc, const float* gs, void* out, hipStream_t s, int64_t B = 1,
                   int64_t x_stride = 0);
// launch_qmv over B weight matrices in one launch per 65535 of them, when the
// kernel launch_qmv would pick for one matrix (decode at M = 1, multi-row
// for 2 <= M <= 64) has a batched form and applies; returns false, launching
// nothing, otherwise.  Matrix b: x + b * x_stride elements, w + b * N * K/8,
// sc + b * N * K/16, gs + b (gs may be NULL), out + b * M * N.
bool launch_qmv_batched(const void* x, nvfp4_dtype_t dt, int64_t B, int64_t x_stride, int64_t M, int64_t K,
                        int64_t N, const uint32_t* w, const uint8_t* sc, const float* gs, void* out,
                        hipStream_t s);
// GatherQMM through the MFMA kernel (bf16 and f16 activations directly,
// f32 as three bf16 parts): each expert's pairs are gathered and multiplied
// together.  Needs K % 256 == 0, E >= 1, X >= 1, 16-byte aligned x, w and
// scales; returns false (launching nothing) otherwise.
bool launch_gather_mfma(const void* x, nvfp4_dtype_t dt, int64_t X, int64_t M, int64_t K, const int32_t* lhs,
                        const int32_t* rhs, int64_t R, const uint32_t* w, const uint8_t* sc,
                        const float* gs, int64_t E, int64_t N, void* out, hipStream_t s);
// MFMA GEMM.  Transposed plane: bf16 through the LDS-pipelined kernel (K %
// 64 == 0, 4-byte aligned scales) or the older one (K % 32 == 0); f16
// through the pipelined kernel on the f16 MFMA; float32 as the activations'
// exact three-part bf16 split in the workspace, then the bf16 kernel over
// rows of 3K (K % 64 == 0).  With a workspace of at least
// gemm_workspace_bytes bytes (16-byte aligned) the 2-byte forms split the
// slabs of K among several blocks per tile when that pays (few tiles) and add
// the float32 partials in a second kernel.  Non-transposed plane (K % 64 ==
// 0, a workspace of gemm_workspace_bytes): its exact dense copy,
// transposed, in the workspace, then a matrix-core GEMM on the dense copy.
// Returns false, launching nothing, when no MFMA form applies.
bool launch_gemm_mfma(const void* x, nvfp4_dtype_t dt, int64_t M, int64_t K, int64_t N, const uint32_t* w,
                      const uint8_t* sc, const float* gs, int transpose, void* out, hipStream_t s,
                      void* ws = nullptr, int64_t ws_bytes = 0);
// Workspace the MFMA GEMM wants for this shape on the current device (0:
// none): the K split's partials (2-byte types, few tiles), the float32
// form's split activations, or a non-transposed plane's dense copy.
int64_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t N, nvfp4_dtype_t dt, int transpose);
// Gated MLP projection as one MFMA GEMM: bf16 activations, transposed gate
// and up planes [F, K/8] with K % 64 == 0 and 4-byte aligned scale planes;
// a tile holds 128 features of both planes.  With a 16-byte aligned
// workspace of at least gemm_glu_workspace_bytes(M, K, F) bytes, the last,
// partial round of tiles is split along K (two more launches: the split
// tiles and their reduction); otherwise one launch.
void launch_gemm_glu(const void* x, int64_t M, int64_t K, int64_t F, const uint32_t* w_gate,
                     const uint8_t* s_gate, const float* gs_gate, const uint32_t* w_up, const uint8_t* s_up,
                     const float* gs_up, int act, void* out, hipStream_t s, void* ws = nullptr,
                     int64_t ws_bytes = 0);
// Workspace the gated projection's tail split wants on the current device
// (0: no split).
int64_t gemm_glu_workspace_bytes(int64_t M, int64_t K, int64_t F);
// Blocks launch_gemm_glu runs for these sizes (before rounding to XCDs).
int64_t gemm_glu_tiles(int64_t M, int64_t F);
// out[i] = act(gate[i]) * out[i] over n elements of dtype dt.
void launch_glu_combine(const void* gate, void* out, int64_t n, nvfp4_dtype_t dt, int act, hipStream_t s);
// Generic float32-accumulating GEMM for any dtype and either plane layout.
void launch_gemm_generic(const void* x, nvfp4_dtype_t dt, int64_t M, int64_t K, int64_t N,
                         const uint32_t* w, const uint8_t* sc, const float* gs, int transpose,
                         void* out, hipStream_t s);
// GatherQMM over experts.
void launch_gather(const void* x, nvfp4_dtype_t dt, int64_t X, int64_t M, int64_t K,
                   const int32_t* lhs, const int32_t* rhs, int64_t R, const uint32_t* w,
                   const uint8_t* sc, const float* gs, int64_t E, int64_t N, int sorted,
                   void* out, hipStream_t s);

// Grid limits used by the launchers (HIP: gridDim.x < 2^31, y/z < 2^16).
constexpr int64_t kMaxGridX = 2147483647LL;
constexpr int64_t kMaxGridY = 65535;

}  // namespace nvfp4host
