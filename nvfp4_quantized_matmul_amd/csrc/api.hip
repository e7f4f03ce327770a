// C ABI of libnvfp4: argument validation, route selection and launches.
//
// Every check runs on the host before anything is enqueued, mirroring the
// plane checks of mlxcel PR "native NVFP4 for ROCm QuantizedMatmul/
// GatherQMM" ("Changes during review" and "Security and performance
// review"): the scale plane is derived from the weight plane so the two
// cannot disagree, the quantized axis must be a multiple of 16, grids are
// bounded, and an empty output launches nothing.
#include <climits>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "nvfp4_internal.hpp"

namespace {

// Crossover between the weight-streaming qmv kernels and the GEMM kernels
// (the pages test qmv up to M = 33 and the GEMM route from M = 64).  With
// K % 256 == 0 the qmv route goes up to M = 64: there the MFMA qmv kernel
// decodes each weight once for all rows and is several times faster than a
// GEMM tile that is mostly padding.
constexpr int64_t kQmvMaxRows = 33;
constexpr int64_t kQmvMaxRowsMfma = 64;

bool mul_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_mul_overflow(a, b, r) && *r >= 0; }

bool size3(int64_t a, int64_t b, int64_t c, int64_t* r) {
  int64_t t;
  return mul_ok(a, b, &t) && mul_ok(t, c, r);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool valid_dtype(int dt) { return dt == NVFP4_F32 || dt == NVFP4_BF16 || dt == NVFP4_F16; }

int64_t dtype_size(nvfp4_dtype_t dt) { return dt == NVFP4_F32 ? 4 : 2; }

int launched() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

// What one qmm call launches, decided on the host with every check done.
struct QmmPlan {
  enum Kind { kNothing, kZeroFill, kQmv, kGemmMfma } kind;
};

// All host checks of one nvfp4_qmm call (no launch).
int qmm_plan(const void* x, nvfp4_dtype_t dtype, int64_t M, int64_t K, int64_t N, const uint32_t* w,
             const uint8_t* scales, const float* gs, int transpose, nvfp4_route_t route, const void* out,
             QmmPlan* plan) {
  plan->kind = QmmPlan::kNothing;
  const int auto_route = nvfp4_select_route(M, K, N, transpose, dtype);
  if (auto_route < 0) return auto_route;
  if (route != NVFP4_ROUTE_AUTO && route != NVFP4_ROUTE_QMV && route != NVFP4_ROUTE_GEMM) return NVFP4_ERR_ROUTE;
  if (route == NVFP4_ROUTE_QMV && !transpose) return NVFP4_ERR_ROUTE;
  int64_t t;
  if (!mul_ok(M, K, &t) || !mul_ok(M, N, &t) || !mul_ok(K, N, &t)) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!out) return NVFP4_ERR_NULLPTR;
  if (!aligned(out, 16)) return NVFP4_ERR_ALIGN;
  if (K == 0) {
    plan->kind = QmmPlan::kZeroFill;
    return NVFP4_OK;
  }
  if (!x || !w || !scales) return NVFP4_ERR_NULLPTR;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(scales, 2) || (gs && !aligned(gs, 4))) return NVFP4_ERR_ALIGN;
  const int r = route == NVFP4_ROUTE_AUTO ? auto_route : (int)route;
  if (r == NVFP4_ROUTE_QMV) {
    if ((N + 15) / 16 > nvfp4host::kMaxGridX) return NVFP4_ERR_GRID;
    plan->kind = QmmPlan::kQmv;
  } else {
    // the MFMA GEMM where one of its forms applies, else the generic kernel
    const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
    if (tiles + 8 > nvfp4host::kMaxGridX || (N + 63) / 64 > nvfp4host::kMaxGridX) return NVFP4_ERR_GRID;
    plan->kind = QmmPlan::kGemmMfma;
  }
  return NVFP4_OK;
}

// Enqueues what qmm_plan decided (arguments already checked).
void qmm_launch(const QmmPlan& plan, const void* x, nvfp4_dtype_t dtype, int64_t M, int64_t K, int64_t N,
                const uint32_t* w, const uint8_t* scales, const float* gs, int transpose, void* out,
                hipStream_t stream, void* ws = nullptr, int64_t ws_bytes = 0) {
  switch (plan.kind) {
    case QmmPlan::kNothing: break;
    case QmmPlan::kZeroFill: nvfp4host::launch_fill_zero(out, M * N * dtype_size(dtype), stream); break;
    case QmmPlan::kQmv: nvfp4host::launch_qmv(x, dtype, M, K, N, w, scales, gs, out, stream); break;
    case QmmPlan::kGemmMfma:
      if (!nvfp4host::launch_gemm_mfma(x, dtype, M, K, N, w, scales, gs, transpose, out, stream, ws, ws_bytes))
        nvfp4host::launch_gemm_generic(x, dtype, M, K, N, w, scales, gs, transpose, out, stream);
      break;
  }
}

// True when nvfp4_qmm_glu runs the fused gate/up kernel for these sizes:
// bf16 activations, K % 64 == 0, and sizes where qmm takes the GEMM route.
bool glu_fused(int64_t M, int64_t K, int64_t F, nvfp4_dtype_t dtype) {
  return dtype == NVFP4_BF16 && K > 0 && K % 64 == 0 && M > 0 && F > 0 &&
         nvfp4_select_route(M, K, F, 1, dtype) == NVFP4_ROUTE_GEMM;
}

bool valid_act(int act) { return act == NVFP4_ACT_GELU_TANH || act == NVFP4_ACT_GELU || act == NVFP4_ACT_SILU; }

// nvfp4_qmm_batched and nvfp4_qmm_batched_ws: the workspace (work,
// work_bytes, both checked by the caller) serves the GEMM route of every
// matrix in turn; the launches are ordered on the stream, so one workspace
// is enough.
int qmm_batched_impl(const void* x, nvfp4_dtype_t dtype, int64_t XB, int64_t B, int64_t M, int64_t K, int64_t N,
                     const uint32_t* w, const uint8_t* scales, const float* gs, int transpose,
                     nvfp4_route_t route, void* work, int64_t work_bytes, void* out, hipStream_t stream) {
  if (B < 0 || XB < 0 || M < 0 || K < 0 || N < 0) return NVFP4_ERR_SHAPE;
  if (B == 0) return (XB == 0 || XB == 1) ? NVFP4_OK : NVFP4_ERR_SHAPE;
  if (XB != 1 && XB != B) return NVFP4_ERR_SHAPE;
  if (!valid_dtype(dtype)) return NVFP4_ERR_DTYPE;
  if (transpose != 0 && transpose != 1) return NVFP4_ERR_SHAPE;
  if (transpose ? (K % 16) != 0 : (N % 16) != 0) return NVFP4_ERR_SHAPE;
  // Per-matrix strides (elements of x and out, words of w, bytes of scales);
  // every total must fit in int64.
  const int64_t ds = dtype_size(dtype);
  int64_t xs, ws, ss, os, t;
  if (!mul_ok(M, K, &xs) || !mul_ok(M, N, &os) || !mul_ok(N, K, &t)) return NVFP4_ERR_SHAPE;
  ws = t / 8;
  ss = t / 16;
  if (!size3(XB, xs, ds, &t) || !size3(B, os, ds, &t) || !size3(B, ws, 4, &t) || !mul_ok(B, ss, &t))
    return NVFP4_ERR_SHAPE;
  if (XB == 1) xs = 0;
  const char* xb = static_cast<const char*>(x);
  char* ob = static_cast<char*>(out);
  // Every slice is checked before anything is enqueued.
  QmmPlan plan{};
  for (int64_t b = 0; b < B; ++b) {
    const int st = qmm_plan(xb ? xb + b * xs * ds : nullptr, dtype, M, K, N, w ? w + b * ws : nullptr,
                            scales ? scales + b * ss : nullptr, gs ? gs + b : nullptr, transpose, route,
                            ob ? ob + b * os * ds : nullptr, &plan);
    if (st != NVFP4_OK) return st;
  }
  if (plan.kind == QmmPlan::kNothing) return NVFP4_OK;
  if (work && plan.kind == QmmPlan::kGemmMfma &&
      (overlaps(work, work_bytes, out, B * os * ds) || overlaps(work, work_bytes, x, (XB == 1 ? 1 : B) * M * K * ds)))
    return NVFP4_ERR_SHAPE;
  // The decode and multi-row kernels take the whole batch in one launch
  // (the same kernel and arithmetic as one call per matrix); other routes
  // launch per matrix.
  if (plan.kind == QmmPlan::kQmv && transpose &&
      nvfp4host::launch_qmv_batched(x, dtype, B, xs, M, K, N, w, scales, gs, out, stream))
    return launched();
  for (int64_t b = 0; b < B; ++b)
    qmm_launch(plan, xb ? xb + b * xs * ds : nullptr, dtype, M, K, N, w ? w + b * ws : nullptr,
               scales ? scales + b * ss : nullptr, gs ? gs + b : nullptr, transpose, ob + b * os * ds,
               stream, work, work_bytes);
  return launched();
}

}  // namespace

extern "C" {

int nvfp4_version(void) { return (1 << 16) | 0; }

int64_t nvfp4_qmv_max_rows(void) { return kQmvMaxRows; }

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULLPTR: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid shape (negative size, quantized axis not a multiple of 16, overflow or inconsistent optional arguments)";
    case NVFP4_ERR_DTYPE: return "unknown or unsupported dtype";
    case NVFP4_ERR_GRID: return "launch would exceed a HIP grid limit";
    case NVFP4_ERR_ROUTE: return "the qmv route needs a transposed weight plane";
    case NVFP4_ERR_UNSUPPORTED: return "request not implemented";
    case NVFP4_ERR_HIP: return "HIP runtime error at launch";
    case NVFP4_ERR_ALIGN: return "pointer not aligned as required";
    case NVFP4_ERR_SCRATCH: return "the call needs more scratch than the library's static array holds";
    default: return "unknown status";
  }
}

int nvfp4_select_route(int64_t M, int64_t K, int64_t N, int transpose, nvfp4_dtype_t dtype) {
  if (M < 0 || K < 0 || N < 0) return NVFP4_ERR_SHAPE;
  if (transpose != 0 && transpose != 1) return NVFP4_ERR_SHAPE;
  if (!valid_dtype(dtype)) return NVFP4_ERR_DTYPE;
  if (transpose ? (K % 16) != 0 : (N % 16) != 0) return NVFP4_ERR_SHAPE;
  if (!transpose) return NVFP4_ROUTE_GEMM;
  if (M <= kQmvMaxRows) return NVFP4_ROUTE_QMV;
  if (M <= kQmvMaxRowsMfma && K % 256 == 0) return NVFP4_ROUTE_QMV;
  return NVFP4_ROUTE_GEMM;
}

int nvfp4_transcode(const uint8_t* weight, const uint8_t* weight_scale, const float* weight_scale_2,
                    int64_t batch, int64_t rows, int64_t cols, uint32_t* w_out, uint8_t* scales_out,
                    float* gs_out, hipStream_t stream) {
  if (batch < 0 || rows < 0 || cols < 0 || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if ((weight_scale_2 == nullptr) != (gs_out == nullptr)) return NVFP4_ERR_SHAPE;
  int64_t elems;
  if (!size3(batch, rows, cols, &elems)) return NVFP4_ERR_SHAPE;
  if (batch == 0) return NVFP4_OK;
  if (weight_scale_2 && (!aligned(weight_scale_2, 4) || !aligned(gs_out, 4))) return NVFP4_ERR_ALIGN;
  const int64_t wbytes = elems / 2, sbytes = elems / 16;
  if (elems > 0) {
    if (!weight || !weight_scale || !w_out || !scales_out) return NVFP4_ERR_NULLPTR;
    if (!aligned(w_out, 4)) return NVFP4_ERR_ALIGN;
    const void* wo = static_cast<const void*>(w_out);
    if (wo != static_cast<const void*>(weight) && overlaps(wo, wbytes, weight, wbytes)) return NVFP4_ERR_SHAPE;
    if (scales_out != weight_scale && overlaps(scales_out, sbytes, weight_scale, sbytes)) return NVFP4_ERR_SHAPE;
  }
  if (weight_scale_2 && overlaps(gs_out, batch * 4, weight_scale_2, batch * 4) &&
      static_cast<const void*>(gs_out) != static_cast<const void*>(weight_scale_2))
    return NVFP4_ERR_SHAPE;
  nvfp4host::launch_copy_bytes(weight, reinterpret_cast<uint8_t*>(w_out), wbytes, stream);
  nvfp4host::launch_copy_bytes(weight_scale, scales_out, sbytes, stream);
  if (weight_scale_2) nvfp4host::launch_sidecar(weight_scale_2, gs_out, batch, stream);
  return launched();
}

int nvfp4_dequantize(const uint32_t* w, const uint8_t* scales, const float* gs, int64_t batch,
                     int64_t rows, int64_t cols, nvfp4_dtype_t out_dtype, void* out,
                     hipStream_t stream) {
  if (batch < 0 || rows < 0 || cols < 0 || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!valid_dtype(out_dtype)) return NVFP4_ERR_DTYPE;
  int64_t elems, bytes;
  if (!size3(batch, rows, cols, &elems) || !mul_ok(elems, dtype_size(out_dtype), &bytes)) return NVFP4_ERR_SHAPE;
  if (elems == 0) return NVFP4_OK;
  if (!w || !scales || !out) return NVFP4_ERR_NULLPTR;
  if (!aligned(w, 4) || !aligned(out, 16) || (gs && !aligned(gs, 4))) return NVFP4_ERR_ALIGN;
  nvfp4host::launch_dequantize(w, scales, gs, batch, rows, cols, out_dtype, out, stream);
  return launched();
}

int nvfp4_quantize(const void* w, nvfp4_dtype_t dtype, int64_t batch, int64_t rows, int64_t cols,
                   const float* gs_in, uint32_t* w_out, uint8_t* scales_out, float* gs_out, hipStream_t stream) {
  if (batch < 0 || rows < 0 || cols < 0 || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!valid_dtype(dtype)) return NVFP4_ERR_DTYPE;
  int64_t elems, bytes;
  if (!size3(batch, rows, cols, &elems) || !mul_ok(elems, dtype_size(dtype), &bytes)) return NVFP4_ERR_SHAPE;
  if (batch == 0) return NVFP4_OK;
  if (!gs_in && !gs_out) return NVFP4_ERR_NULLPTR;
  if ((gs_in && !aligned(gs_in, 4)) || (gs_out && !aligned(gs_out, 4))) return NVFP4_ERR_ALIGN;
  if (elems > 0) {
    if (!w || !w_out || !scales_out) return NVFP4_ERR_NULLPTR;
    if (!aligned(w, 16) || !aligned(w_out, 8)) return NVFP4_ERR_ALIGN;
    if (overlaps(w, bytes, w_out, elems / 2) || overlaps(w, bytes, scales_out, elems / 16) ||
        overlaps(w_out, elems / 2, scales_out, elems / 16))
      return NVFP4_ERR_SHAPE;
    if (gs_out && (overlaps(gs_out, batch * 4, w, bytes) || overlaps(gs_out, batch * 4, w_out, elems / 2) ||
                   overlaps(gs_out, batch * 4, scales_out, elems / 16)))
      return NVFP4_ERR_SHAPE;
  }
  if (gs_in && gs_out && gs_in != gs_out && overlaps(gs_in, batch * 4, gs_out, batch * 4)) return NVFP4_ERR_SHAPE;
  nvfp4host::launch_quantize(w, dtype, batch, rows, cols, gs_in, w_out, scales_out, gs_out, stream);
  return launched();
}

int nvfp4_qmm(const void* x, nvfp4_dtype_t dtype, int64_t M, int64_t K, int64_t N,
              const uint32_t* w, const uint8_t* scales, const float* gs, int transpose,
              nvfp4_route_t route, void* out, hipStream_t stream) {
  QmmPlan plan;
  const int st = qmm_plan(x, dtype, M, K, N, w, scales, gs, transpose, route, out, &plan);
  if (st != NVFP4_OK) return st;
  if (plan.kind == QmmPlan::kNothing) return NVFP4_OK;
  qmm_launch(plan, x, dtype, M, K, N, w, scales, gs, transpose, out, stream);
  return launched();
}

int64_t nvfp4_qmm_workspace_size(int64_t M, int64_t K, int64_t N, int transpose, nvfp4_dtype_t dtype,
                                 nvfp4_route_t route) {
  const int auto_route = nvfp4_select_route(M, K, N, transpose, dtype);
  if (auto_route < 0) return auto_route;
  if (route != NVFP4_ROUTE_AUTO && route != NVFP4_ROUTE_QMV && route != NVFP4_ROUTE_GEMM) return NVFP4_ERR_ROUTE;
  int64_t t;
  if (!mul_ok(M, K, &t) || !mul_ok(M, N, &t) || !mul_ok(K, N, &t)) return NVFP4_ERR_SHAPE;
  const int r = route == NVFP4_ROUTE_AUTO ? auto_route : (int)route;
  if (r != NVFP4_ROUTE_GEMM || M == 0 || N == 0 || K == 0) return 0;
  return nvfp4host::gemm_workspace_bytes(M, K, N, dtype, transpose);
}

int nvfp4_qmm_ws(const void* x, nvfp4_dtype_t dtype, int64_t M, int64_t K, int64_t N, const uint32_t* w,
                 const uint8_t* scales, const float* gs, int transpose, nvfp4_route_t route, void* workspace,
                 int64_t workspace_bytes, void* out, hipStream_t stream) {
  if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace)) return NVFP4_ERR_SHAPE;
  if (workspace && !aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
  QmmPlan plan;
  const int st = qmm_plan(x, dtype, M, K, N, w, scales, gs, transpose, route, out, &plan);
  if (st != NVFP4_OK) return st;
  if (plan.kind == QmmPlan::kNothing) return NVFP4_OK;
  if (workspace && plan.kind == QmmPlan::kGemmMfma) {
    int64_t mn;
    const int64_t osz = dtype_size(dtype);
    if (mul_ok(M, N, &mn) && (overlaps(workspace, workspace_bytes, out, mn * osz) ||
                              overlaps(workspace, workspace_bytes, x, M * K * osz)))
      return NVFP4_ERR_SHAPE;
  }
  qmm_launch(plan, x, dtype, M, K, N, w, scales, gs, transpose, out, stream, workspace, workspace_bytes);
  return launched();
}

}  // extern "C"

namespace {

// Scratch of nvfp4_qmm_noalloc: a file-scope device array, one copy per GPU,
// held until the process ends.  Host code never passes the array's name to
// a kernel (on the host it only stands for the symbol); it uses the device
// address that hipGetSymbolAddress returns for the current device.
constexpr int64_t kStaticScratchBytes = NVFP4_STATIC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device with
// that device current; nullptr when the runtime cannot give it.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();   // leave no sticky error for the caller's next call
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int nvfp4_qmm_noalloc(const void* x, nvfp4_dtype_t dtype, int64_t M, int64_t K, int64_t N, const uint32_t* w,
                      const uint8_t* scales, const float* gs, int transpose, nvfp4_route_t route, void* out,
                      hipStream_t stream) {
  QmmPlan plan;
  const int st = qmm_plan(x, dtype, M, K, N, w, scales, gs, transpose, route, out, &plan);
  if (st != NVFP4_OK) return st;
  if (plan.kind == QmmPlan::kNothing) return NVFP4_OK;
  int64_t need = nvfp4_qmm_workspace_size(M, K, N, transpose, dtype, route);
  if (need < 0) return (int)need;
  if (need > kStaticScratchBytes) {
    // a float32 copy or a non-transposed plane's dense copy that does not
    // fit leaves the generic kernel, which needs no scratch; a K split that
    // does not fit is refused
    if (dtype != NVFP4_F32 && transpose) return NVFP4_ERR_SCRATCH;
    need = 0;
  }
  void* ws = nullptr;
  if (need > 0 && plan.kind == QmmPlan::kGemmMfma) {
    ws = scratch_address();
    if (!ws) return NVFP4_ERR_HIP;
  }
  qmm_launch(plan, x, dtype, M, K, N, w, scales, gs, transpose, out, stream, ws, ws ? need : 0);
  return launched();
}

int64_t nvfp4_static_scratch_bytes(void) { return kStaticScratchBytes; }

int64_t nvfp4_qmm_glu_workspace_size(int64_t M, int64_t K, int64_t F, nvfp4_dtype_t dtype) {
  if (M < 0 || K < 0 || F < 0 || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!valid_dtype(dtype)) return NVFP4_ERR_DTYPE;
  int64_t t, mf;
  if (!mul_ok(M, K, &t) || !mul_ok(K, F, &t) || !mul_ok(M, F, &mf) || !mul_ok(mf, dtype_size(dtype), &t) ||
      t > INT64_MAX - 256)
    return NVFP4_ERR_SHAPE;
  if (M == 0 || F == 0 || K == 0) return 0;
  if (glu_fused(M, K, F, dtype)) return nvfp4host::gemm_glu_workspace_bytes(M, K, F);
  if (M == 1 && nvfp4host::decode_glu_applies(K, F)) return 0;   // the decode kernel's gated form
  if (nvfp4host::skinny_glu_applies(M, K, F)) return 0;           // the multi-row kernel's gated form
  return (t + 255) / 256 * 256;
}

int nvfp4_qmm_glu(const void* x, nvfp4_dtype_t dtype, int64_t M, int64_t K, int64_t F, const uint32_t* w_gate,
                  const uint8_t* s_gate, const float* gs_gate, const uint32_t* w_up, const uint8_t* s_up,
                  const float* gs_up, nvfp4_act_t act, void* workspace, int64_t workspace_bytes, void* out,
                  hipStream_t stream) {
  const int64_t need = nvfp4_qmm_glu_workspace_size(M, K, F, dtype);
  if (need < 0) return (int)need;
  if (!valid_act((int)act)) return NVFP4_ERR_SHAPE;
  if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace)) return NVFP4_ERR_SHAPE;
  // Both projections get qmm's full checks (pointers, alignment, grid).
  QmmPlan pg, pu;
  int st = qmm_plan(x, dtype, M, K, F, w_gate, s_gate, gs_gate, 1, NVFP4_ROUTE_AUTO, out, &pg);
  if (st != NVFP4_OK) return st;
  st = qmm_plan(x, dtype, M, K, F, w_up, s_up, gs_up, 1, NVFP4_ROUTE_AUTO, out, &pu);
  if (st != NVFP4_OK) return st;
  if (pg.kind == QmmPlan::kNothing) return NVFP4_OK;
  if (pg.kind == QmmPlan::kZeroFill) {   // K == 0: act(0) * 0 = 0 for every activation
    nvfp4host::launch_fill_zero(out, M * F * dtype_size(dtype), stream);
    return launched();
  }
  const int64_t ds = dtype_size(dtype);
  const int64_t wbytes = F * (K / 2), sbytes = F * (K / 16);
  const bool ws_overlaps =
      workspace && (overlaps(workspace, workspace_bytes, out, M * F * ds) ||
                    overlaps(workspace, workspace_bytes, x, M * K * ds) ||
                    overlaps(workspace, workspace_bytes, w_gate, wbytes) ||
                    overlaps(workspace, workspace_bytes, w_up, wbytes) ||
                    overlaps(workspace, workspace_bytes, s_gate, sbytes) ||
                    overlaps(workspace, workspace_bytes, s_up, sbytes) ||
                    (gs_gate && overlaps(workspace, workspace_bytes, gs_gate, 4)) ||
                    (gs_up && overlaps(workspace, workspace_bytes, gs_up, 4)));
  if (glu_fused(M, K, F, dtype)) {
    // The fused kernel; a workspace is optional (it splits the last,
    // partial round of tiles along K when large enough).
    if (!aligned(s_gate, 4) || !aligned(s_up, 4)) return NVFP4_ERR_ALIGN;
    if (workspace && !aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
    if (ws_overlaps) return NVFP4_ERR_SHAPE;
    if (nvfp4host::gemm_glu_tiles(M, F) * 9 + 8 > nvfp4host::kMaxGridX) return NVFP4_ERR_GRID;
    nvfp4host::launch_gemm_glu(x, M, K, F, w_gate, s_gate, gs_gate, w_up, s_up, gs_up, (int)act, out, stream,
                               workspace, workspace_bytes);
    return launched();
  }
  if (M == 1 && nvfp4host::decode_glu_applies(K, F)) {
    // one launch of the decode kernel, a feature's gate and up rows per
    // wavefront; no workspace
    if (!nvfp4host::launch_decode_glu(x, dtype, K, F, w_gate, s_gate, gs_gate, w_up, s_up, gs_up, (int)act, out,
                                      stream))
      return NVFP4_ERR_UNSUPPORTED;
    return launched();
  }
  if (nvfp4host::skinny_glu_applies(M, K, F)) {
    // one launch of the multi-row MFMA kernel, 32 features' gate and up rows
    // per block; its 16-byte loads need 16-byte aligned operands
    if (!aligned(x, 16) || !aligned(w_gate, 16) || !aligned(s_gate, 16) || !aligned(w_up, 16) ||
        !aligned(s_up, 16))
      return NVFP4_ERR_ALIGN;
    if (!nvfp4host::launch_skinny_glu(x, dtype, M, K, F, w_gate, s_gate, gs_gate, w_up, s_up, gs_up, (int)act, out,
                                      stream))
      return NVFP4_ERR_UNSUPPORTED;
    return launched();
  }
  if (workspace_bytes < need) return NVFP4_ERR_SHAPE;
  if (!aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
  if (ws_overlaps) return NVFP4_ERR_SHAPE;
  qmm_launch(pg, x, dtype, M, K, F, w_gate, s_gate, gs_gate, 1, workspace, stream);
  qmm_launch(pu, x, dtype, M, K, F, w_up, s_up, gs_up, 1, out, stream);
  nvfp4host::launch_glu_combine(workspace, out, M * F, dtype, (int)act, stream);
  return launched();
}

int nvfp4_qmm_batched(const void* x, nvfp4_dtype_t dtype, int64_t XB, int64_t B, int64_t M, int64_t K,
                      int64_t N, const uint32_t* w, const uint8_t* scales, const float* gs,
                      int transpose, nvfp4_route_t route, void* out, hipStream_t stream) {
  return qmm_batched_impl(x, dtype, XB, B, M, K, N, w, scales, gs, transpose, route, nullptr, 0, out, stream);
}

int nvfp4_qmm_batched_ws(const void* x, nvfp4_dtype_t dtype, int64_t XB, int64_t B, int64_t M, int64_t K,
                         int64_t N, const uint32_t* w, const uint8_t* scales, const float* gs, int transpose,
                         nvfp4_route_t route, void* workspace, int64_t workspace_bytes, void* out,
                         hipStream_t stream) {
  if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace)) return NVFP4_ERR_SHAPE;
  if (workspace && !aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
  return qmm_batched_impl(x, dtype, XB, B, M, K, N, w, scales, gs, transpose, route, workspace, workspace_bytes,
                          out, stream);
}

int nvfp4_gather_qmm(const void* x, nvfp4_dtype_t dtype, int64_t X, int64_t M, int64_t K,
                     const int32_t* lhs, const int32_t* rhs, int64_t R, const uint32_t* w,
                     const uint8_t* scales, const float* gs, int64_t E, int64_t N,
                     int sorted_indices, void* out, hipStream_t stream) {
  if (X < 0 || M < 0 || K < 0 || R < 0 || E < 0 || N < 0 || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!valid_dtype(dtype)) return NVFP4_ERR_DTYPE;
  int64_t t;
  if (!size3(X, M, K, &t) || !size3(R, M, N, &t) || !size3(E, N, K, &t)) return NVFP4_ERR_SHAPE;
  if (R == 0 || M == 0 || N == 0) return NVFP4_OK;
  if (!rhs || !out) return NVFP4_ERR_NULLPTR;
  if (!aligned(out, 16) || !aligned(rhs, 4) || (lhs && !aligned(lhs, 4))) return NVFP4_ERR_ALIGN;
  if (K == 0) {
    nvfp4host::launch_fill_zero(out, R * M * N * dtype_size(dtype), stream);
    return launched();
  }
  if (!x && X > 0) return NVFP4_ERR_NULLPTR;
  if ((!w || !scales) && E > 0) return NVFP4_ERR_NULLPTR;
  if ((x && !aligned(x, 16)) || (w && !aligned(w, 16)) || (scales && !aligned(scales, 2)) ||
      (gs && !aligned(gs, 4)))
    return NVFP4_ERR_ALIGN;
  if ((N + 15) / 16 > nvfp4host::kMaxGridX) return NVFP4_ERR_GRID;
  nvfp4host::launch_gather(x, dtype, X, M, K, lhs, rhs, R, w, scales, gs, E, N, sorted_indices ? 1 : 0,
                           out, stream);
  return launched();
}

}  // extern "C"
