"""NVFP4 quantized matmul for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libnvfp4.so``: it checks shapes, dtypes,
devices and contiguity, allocates outputs with PyTorch, and passes raw device
pointers and the current HIP stream to the C ABI declared in
``include/nvfp4.h``.  Every step of the computation runs in the library's
HIP kernels; there is no Python or CPU fallback, and every entry point raises
if the library has not been built.

Format (mlxcel issue "perf(nvfp4): direct-transcode ModelOpt triplets to MLX
native", "Technical notes"): uint32 words with eight E2M1 nibbles, one E4M3
scale byte per 16 elements, and an optional float32 global scale applied as
global_scale / (448 * 6).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "NVFP4Error", "library_path", "load_library", "transcode", "dequantize", "quantize", "qmm",
    "qmm_batched", "qmm_glu", "gather_qmm", "select_route", "qmv_max_rows", "status_string",
    "ROUTE_AUTO", "ROUTE_QMV", "ROUTE_GEMM", "GLU_ACTIVATIONS",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libnvfp4.so"

ROUTE_AUTO, ROUTE_QMV, ROUTE_GEMM = 0, 1, 2
_ROUTES = {"auto": ROUTE_AUTO, "qmv": ROUTE_QMV, "gemm": ROUTE_GEMM}
_DTYPES = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
# Gate activations of qmm_glu, by the names the C header's nvfp4_act_t stands for.
_ACTS = {"gelu_tanh": 0, "gelu": 1, "silu": 2}
GLU_ACTIVATIONS = tuple(_ACTS)
_WORD_DTYPES = (torch.int32, torch.uint32)

_lib = None


class NVFP4Error(RuntimeError):
    """A negative status returned by libnvfp4."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


def library_path() -> str:
    return os.path.join(_PKG_DIR, _LIB_NAME)


def load_library() -> ctypes.CDLL:
    """Load libnvfp4.so from the package directory (built in-tree)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m nvfp4_quantized_matmul_amd.build` "
            "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(path)
    i64, vp, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    sig = {
        "nvfp4_transcode": [vp, vp, vp, i64, i64, i64, vp, vp, vp, vp],
        "nvfp4_dequantize": [vp, vp, vp, i64, i64, i64, c_int, vp, vp],
        "nvfp4_quantize": [vp, c_int, i64, i64, i64, vp, vp, vp, vp, vp],
        "nvfp4_qmm": [vp, c_int, i64, i64, i64, vp, vp, vp, c_int, c_int, vp, vp],
        "nvfp4_qmm_batched": [vp, c_int, i64, i64, i64, i64, i64, vp, vp, vp, c_int, c_int, vp, vp],
        "nvfp4_qmm_batched_ws": [vp, c_int, i64, i64, i64, i64, i64, vp, vp, vp, c_int, c_int, vp, i64, vp, vp],
        "nvfp4_qmm_ws": [vp, c_int, i64, i64, i64, vp, vp, vp, c_int, c_int, vp, i64, vp, vp],
        "nvfp4_qmm_noalloc": [vp, c_int, i64, i64, i64, vp, vp, vp, c_int, c_int, vp, vp],
        "nvfp4_static_scratch_bytes": [],
        "nvfp4_qmm_workspace_size": [i64, i64, i64, c_int, c_int, c_int],
        "nvfp4_qmm_glu": [vp, c_int, i64, i64, i64, vp, vp, vp, vp, vp, vp, c_int, vp, i64, vp, vp],
        "nvfp4_qmm_glu_workspace_size": [i64, i64, i64, c_int],
        "nvfp4_gather_qmm": [vp, c_int, i64, i64, i64, vp, vp, i64, vp, vp, vp, i64, i64, c_int, vp, vp],
        "nvfp4_select_route": [i64, i64, i64, c_int, c_int],
        "nvfp4_qmv_max_rows": [],
        "nvfp4_status_string": [c_int],
        "nvfp4_version": [],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = c_int
    lib.nvfp4_qmv_max_rows.restype = i64
    lib.nvfp4_qmm_workspace_size.restype = i64
    lib.nvfp4_qmm_glu_workspace_size.restype = i64
    lib.nvfp4_static_scratch_bytes.restype = i64
    lib.nvfp4_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().nvfp4_status_string(int(status)).decode()


def select_route(M: int, K: int, N: int, transpose: bool = True, dtype=torch.bfloat16) -> str:
    """Route nvfp4_qmm takes for AUTO ("qmv" or "gemm"); host only."""
    r = load_library().nvfp4_select_route(M, K, N, int(bool(transpose)), _dtype_code(dtype))
    if r < 0:
        raise NVFP4Error("nvfp4_select_route", r)
    return "qmv" if r == ROUTE_QMV else "gemm"


def qmv_max_rows() -> int:
    return int(load_library().nvfp4_qmv_max_rows())


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------

def _dtype_code(dtype) -> int:
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}; expected float32, bfloat16 or float16")
    return _DTYPES[dtype]


def _ptr(t: Optional[torch.Tensor]):
    # a plain int: every library function declares c_void_p arguments, so
    # ctypes converts it without a wrapper object per call
    return None if t is None else t.data_ptr()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise NVFP4Error(fn, status)


# The current stream's handle as an int.  torch's raw accessor skips building
# a Stream object per call (the per-token path goes through here); the public
# API serves where it is absent.
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device):
    if _RAW_STREAM is not None:
        return _RAW_STREAM(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _require_gpu(*tensors: Optional[torch.Tensor]) -> torch.device:
    first, index = None, -1
    for t in tensors:
        if t is None:
            continue
        d = t.get_device()            # -1 on the CPU
        if d < 0:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if first is None:
            first, index = t, d
        elif d != index:
            raise ValueError("all tensors must be on the same device")
    return None if first is None else first.device


# nvfp4_qmm_workspace_size answers, per device and call shape: a per-token
# decode call then costs a dictionary lookup instead of a library round trip.
_QMM_WS_CACHE: dict = {}


def _qmm_workspace_bytes(lib, dev: torch.device, M: int, K: int, N: int, tr: int, code: int, route: int) -> int:
    key = (dev.index, M, K, N, tr, code, route)
    ws_bytes = _QMM_WS_CACHE.get(key)
    if ws_bytes is None:
        ws_bytes = int(lib.nvfp4_qmm_workspace_size(M, K, N, tr, code, route))
        if ws_bytes < 0:
            raise NVFP4Error("nvfp4_qmm_workspace_size", ws_bytes)
        if len(_QMM_WS_CACHE) < 4096:
            _QMM_WS_CACHE[key] = ws_bytes
    return ws_bytes


def check_planes(w: torch.Tensor, scales: torch.Tensor) -> None:
    """The scale plane must be w.shape[:-1] + [w.shape[-1] / 2] with one byte
    per scale (mlxcel PR "native NVFP4 for ROCm QuantizedMatmul/GatherQMM",
    "Changes during review")."""
    if w.dtype not in _WORD_DTYPES:
        raise TypeError(f"weight plane must be int32/uint32 words, got {w.dtype}")
    if scales.dtype != torch.uint8:
        raise TypeError(f"scale plane must be uint8, got {scales.dtype}")
    if w.dim() < 1 or w.shape[-1] % 2 != 0:
        raise ValueError(f"weight plane {tuple(w.shape)} must have an even last axis")
    want = tuple(w.shape[:-1]) + (w.shape[-1] // 2,)
    if tuple(scales.shape) != want:
        raise ValueError(f"scale plane {tuple(scales.shape)} does not match weight plane "
                         f"{tuple(w.shape)} (expected {want})")


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------

def transcode(weight: torch.Tensor, weight_scale: torch.Tensor,
              weight_scale_2: Optional[torch.Tensor] = None, inplace: bool = False
              ) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """ModelOpt NVFP4 triplet -> (uint32 word plane, E4M3 scale plane, gs sidecar).

    weight uint8 [..., rows, cols/2]; weight_scale uint8 [..., rows, cols/16];
    weight_scale_2 float32 with one value per matrix (numel = prod of the
    leading dims) or None.  With ``inplace`` the returned planes alias the
    source storage.
    """
    if weight.dtype != torch.uint8 or weight_scale.dtype != torch.uint8:
        raise TypeError("weight and weight_scale must be uint8")
    if weight.dim() < 2 or weight.shape[-1] % 8 != 0:
        raise ValueError("weight must be [..., rows, cols/2] with cols a multiple of 16")
    lead = tuple(weight.shape[:-2])
    rows, cols = weight.shape[-2], weight.shape[-1] * 2
    if tuple(weight_scale.shape) != lead + (rows, cols // 16):
        raise ValueError(f"weight_scale {tuple(weight_scale.shape)} does not match weight "
                         f"{tuple(weight.shape)}")
    batch = 1
    for d in lead:
        batch *= d
    if weight_scale_2 is not None:
        if weight_scale_2.dtype != torch.float32 or weight_scale_2.numel() != batch:
            raise ValueError("weight_scale_2 must be float32 with one value per matrix")
    dev = _require_gpu(weight, weight_scale, weight_scale_2)
    lib = load_library()
    if inplace:
        w_out = weight.view(torch.int32).view(lead + (rows, cols // 8))
        s_out = weight_scale
    else:
        w_out = torch.empty(lead + (rows, cols // 8), dtype=torch.int32, device=dev)
        s_out = torch.empty_like(weight_scale)
    gs = None
    if weight_scale_2 is not None:
        gs = torch.empty(batch, dtype=torch.float32, device=dev)
    _check("nvfp4_transcode", lib.nvfp4_transcode(
        _ptr(weight), _ptr(weight_scale), _ptr(weight_scale_2), batch, rows, cols,
        _ptr(w_out), _ptr(s_out), _ptr(gs), _stream(dev)))
    return w_out, s_out, gs


def dequantize(w: torch.Tensor, scales: torch.Tensor, gs: Optional[torch.Tensor] = None,
               dtype=torch.float32) -> torch.Tensor:
    """Exact expansion of a plane: [..., rows, cols/8] words -> [..., rows, cols].
    gs (optional) holds one float32 global scale per matrix."""
    check_planes(w, scales)
    if w.dim() < 2:
        raise ValueError("weight plane must be at least 2-D")
    lead = tuple(w.shape[:-2])
    rows, cols = w.shape[-2], w.shape[-1] * 8
    batch = 1
    for d in lead:
        batch *= d
    if gs is not None and (gs.dtype != torch.float32 or gs.numel() != batch):
        raise ValueError("gs must be float32 with one value per matrix")
    code = _dtype_code(dtype)
    dev = _require_gpu(w, scales, gs)
    lib = load_library()
    out = torch.empty(lead + (rows, cols), dtype=dtype, device=dev)
    _check("nvfp4_dequantize", lib.nvfp4_dequantize(
        _ptr(w), _ptr(scales), _ptr(gs), batch, rows, cols, code, _ptr(out), _stream(dev)))
    return out


def quantize(w: torch.Tensor, gs: Optional[torch.Tensor] = None
             ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Dense [..., rows, cols] (float32, bfloat16 or float16; cols % 16 == 0)
    -> (int32 words [..., rows, cols/8], uint8 E4M3 scales [..., rows, cols/16],
    float32 global scales, one per matrix).  gs (float32, one per matrix) sets
    the global scales; by default each matrix's largest |w| is used."""
    if w.dim() < 2 or w.shape[-1] % 16 != 0:
        raise ValueError("w must be [..., rows, cols] with cols a multiple of 16")
    lead = tuple(w.shape[:-2])
    rows, cols = w.shape[-2], w.shape[-1]
    batch = 1
    for d in lead:
        batch *= d
    if gs is not None and (gs.dtype != torch.float32 or gs.numel() != batch):
        raise ValueError("gs must be float32 with one value per matrix")
    code = _dtype_code(w.dtype)
    dev = _require_gpu(w, gs)
    lib = load_library()
    w_out = torch.empty(lead + (rows, cols // 8), dtype=torch.int32, device=dev)
    s_out = torch.empty(lead + (rows, cols // 16), dtype=torch.uint8, device=dev)
    gs_out = torch.empty(batch, dtype=torch.float32, device=dev)
    _check("nvfp4_quantize", lib.nvfp4_quantize(
        _ptr(w), code, batch, rows, cols, _ptr(gs), _ptr(w_out), _ptr(s_out), _ptr(gs_out), _stream(dev)))
    return w_out, s_out, gs_out


def qmm(x: torch.Tensor, w: torch.Tensor, scales: torch.Tensor, gs: Optional[torch.Tensor] = None,
        transpose: bool = True, route: str = "auto", out: Optional[torch.Tensor] = None
        ) -> torch.Tensor:
    """out = x @ dequantize(w).T (transpose) or x @ dequantize(w).

    When the GEMM route wants a workspace (a K split for few output tiles, or
    the three-part bf16 copy of float32 activations) the call goes through
    nvfp4_qmm_ws with a workspace from torch's allocator.

    x [..., K] (float32, bfloat16 or float16); w [N, K/8] (transpose) or
    [K, N/8]; scales as for check_planes; gs float32 with one element or None.
    The output has x's dtype and shape [..., N].
    """
    check_planes(w, scales)
    if w.dim() != 2:
        raise ValueError("qmm takes a 2-D weight plane")
    if transpose:
        N, K = w.shape[0], w.shape[1] * 8
    else:
        K, N = w.shape[0], w.shape[1] * 8
    if x.shape[-1] != K:
        raise ValueError(f"x has K={x.shape[-1]}, weight plane implies K={K}")
    if gs is not None and (gs.dtype != torch.float32 or gs.numel() != 1):
        raise ValueError("gs must be a float32 tensor with one element")
    if route not in _ROUTES:
        raise ValueError(f"route must be one of {sorted(_ROUTES)}")
    code = _dtype_code(x.dtype)
    M = 1
    for d in x.shape[:-1]:
        M *= d
    dev = _require_gpu(x, w, scales, gs)
    lib = load_library()
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (N,), dtype=x.dtype, device=dev)
    elif out.dtype != x.dtype or tuple(out.shape) != tuple(x.shape[:-1]) + (N,):
        raise ValueError("out has the wrong dtype or shape")
    _require_gpu(out)
    tr = int(bool(transpose))
    ws_bytes = _qmm_workspace_bytes(lib, dev, M, K, N, tr, code, _ROUTES[route])
    if ws_bytes > 0:
        # K-split partials or the float32 split copy live in a workspace from
        # torch's allocator (the library itself never allocates)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        _check("nvfp4_qmm_ws", lib.nvfp4_qmm_ws(
            _ptr(x), code, M, K, N, _ptr(w), _ptr(scales), _ptr(gs), tr, _ROUTES[route],
            _ptr(ws), ws_bytes, _ptr(out), _stream(dev)))
        return out
    _check("nvfp4_qmm", lib.nvfp4_qmm(
        _ptr(x), code, M, K, N, _ptr(w), _ptr(scales), _ptr(gs), tr,
        _ROUTES[route], _ptr(out), _stream(dev)))
    return out


def qmm_glu(x: torch.Tensor, w_gate: torch.Tensor, s_gate: torch.Tensor, gs_gate: Optional[torch.Tensor],
            w_up: torch.Tensor, s_up: torch.Tensor, gs_up: Optional[torch.Tensor], act: str = "gelu_tanh",
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gated MLP projection: out = act(x @ dequantize(w_gate).T) * (x @ dequantize(w_up).T).

    x [..., K] (float32, bfloat16 or float16); w_gate and w_up transposed
    planes [F, K/8] of one shape with their scale planes; gs_gate and gs_up
    float32 with one element, or None; act one of GLU_ACTIVATIONS.  The output
    has x's dtype and shape [..., F].  Where the library runs the two
    projections separately it gets a workspace from torch's allocator.
    """
    check_planes(w_gate, s_gate)
    check_planes(w_up, s_up)
    if w_gate.dim() != 2 or tuple(w_gate.shape) != tuple(w_up.shape):
        raise ValueError("w_gate and w_up must be 2-D planes of one shape")
    F, K = w_gate.shape[0], w_gate.shape[1] * 8
    if x.shape[-1] != K:
        raise ValueError(f"x has K={x.shape[-1]}, weight planes imply K={K}")
    for g in (gs_gate, gs_up):
        if g is not None and (g.dtype != torch.float32 or g.numel() != 1):
            raise ValueError("global scales must be float32 tensors with one element")
    if act not in _ACTS:
        raise ValueError(f"act must be one of {GLU_ACTIVATIONS}")
    code = _dtype_code(x.dtype)
    M = 1
    for d in x.shape[:-1]:
        M *= d
    dev = _require_gpu(x, w_gate, s_gate, gs_gate, w_up, s_up, gs_up)
    lib = load_library()
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (F,), dtype=x.dtype, device=dev)
    elif out.dtype != x.dtype or tuple(out.shape) != tuple(x.shape[:-1]) + (F,):
        raise ValueError("out has the wrong dtype or shape")
    _require_gpu(out)
    ws_bytes = int(lib.nvfp4_qmm_glu_workspace_size(M, K, F, code))
    if ws_bytes < 0:
        raise NVFP4Error("nvfp4_qmm_glu_workspace_size", ws_bytes)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes > 0 else None
    _check("nvfp4_qmm_glu", lib.nvfp4_qmm_glu(
        _ptr(x), code, M, K, F, _ptr(w_gate), _ptr(s_gate), _ptr(gs_gate), _ptr(w_up), _ptr(s_up),
        _ptr(gs_up), _ACTS[act], _ptr(ws), ws_bytes, _ptr(out), _stream(dev)))
    return out


def qmm_batched(x: torch.Tensor, w: torch.Tensor, scales: torch.Tensor,
                gs: Optional[torch.Tensor] = None, transpose: bool = True, route: str = "auto",
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """qmm over a batch of weight matrices: out[b] = x[b or 0] @ dequantize(w[b]).T.

    x [XB, M, K] with XB = 1 (shared by every matrix) or XB = B; w [B, N, K/8]
    (transpose) or [B, K, N/8]; scales as for check_planes; gs float32 [B] or
    None.  Returns [B, M, N] in x's dtype.  Where the GEMM route wants a
    workspace (as for qmm), one from torch's allocator serves every matrix
    through nvfp4_qmm_batched_ws.
    """
    check_planes(w, scales)
    if w.dim() != 3 or x.dim() != 3:
        raise ValueError("qmm_batched takes x [XB, M, K] and a 3-D weight plane")
    B = w.shape[0]
    if transpose:
        N, K = w.shape[1], w.shape[2] * 8
    else:
        K, N = w.shape[1], w.shape[2] * 8
    XB, M = x.shape[0], x.shape[1]
    if x.shape[2] != K:
        raise ValueError(f"x has K={x.shape[2]}, weight plane implies K={K}")
    if XB not in (1, B):
        raise ValueError(f"x batch {XB} must be 1 or the weight batch {B}")
    if gs is not None and (gs.dtype != torch.float32 or gs.numel() != B):
        raise ValueError("gs must be float32 with one value per weight matrix")
    if route not in _ROUTES:
        raise ValueError(f"route must be one of {sorted(_ROUTES)}")
    code = _dtype_code(x.dtype)
    dev = _require_gpu(x, w, scales, gs)
    lib = load_library()
    if out is None:
        out = torch.empty((B, M, N), dtype=x.dtype, device=dev)
    elif out.dtype != x.dtype or tuple(out.shape) != (B, M, N):
        raise ValueError("out has the wrong dtype or shape")
    _require_gpu(out)
    tr = int(bool(transpose))
    ws_bytes = _qmm_workspace_bytes(lib, dev, M, K, N, tr, code, _ROUTES[route]) if B > 0 else 0
    if ws_bytes > 0:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        _check("nvfp4_qmm_batched_ws", lib.nvfp4_qmm_batched_ws(
            _ptr(x), code, XB, B, M, K, N, _ptr(w), _ptr(scales), _ptr(gs), tr, _ROUTES[route],
            _ptr(ws), ws_bytes, _ptr(out), _stream(dev)))
        return out
    _check("nvfp4_qmm_batched", lib.nvfp4_qmm_batched(
        _ptr(x), code, XB, B, M, K, N, _ptr(w), _ptr(scales), _ptr(gs), tr,
        _ROUTES[route], _ptr(out), _stream(dev)))
    return out


def gather_qmm(x: torch.Tensor, w: torch.Tensor, scales: torch.Tensor,
               rhs_indices: torch.Tensor, lhs_indices: Optional[torch.Tensor] = None,
               gs: Optional[torch.Tensor] = None, sorted_indices: bool = False,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GatherQMM over NVFP4 experts.

    x [X, M, K]; w [E, N, K/8]; scales [E, N, K/16]; rhs_indices int32 [R]
    (expert per pair); lhs_indices int32 [R] or None (pair r uses x[r]);
    gs float32 [E] or None.  Returns [R, M, N] in x's dtype; pairs whose
    expert or row index is out of range give +0.0.
    """
    check_planes(w, scales)
    if w.dim() != 3 or x.dim() != 3:
        raise ValueError("gather_qmm takes x [X, M, K] and w [E, N, K/8]")
    E, N, K = w.shape[0], w.shape[1], w.shape[2] * 8
    X, M = x.shape[0], x.shape[1]
    if x.shape[2] != K:
        raise ValueError(f"x has K={x.shape[2]}, weight plane implies K={K}")
    if rhs_indices.dtype != torch.int32 or rhs_indices.dim() != 1:
        raise ValueError("rhs_indices must be a 1-D int32 tensor")
    R = rhs_indices.shape[0]
    if lhs_indices is not None and (lhs_indices.dtype != torch.int32 or tuple(lhs_indices.shape) != (R,)):
        raise ValueError("lhs_indices must be int32 shaped like rhs_indices")
    if gs is not None and (gs.dtype != torch.float32 or gs.numel() != E):
        raise ValueError("gs must be float32 with one value per expert")
    code = _dtype_code(x.dtype)
    dev = _require_gpu(x, w, scales, rhs_indices, lhs_indices, gs)
    lib = load_library()
    if out is None:
        out = torch.empty((R, M, N), dtype=x.dtype, device=dev)
    elif out.dtype != x.dtype or tuple(out.shape) != (R, M, N):
        raise ValueError("out has the wrong dtype or shape")
    _require_gpu(out)
    _check("nvfp4_gather_qmm", lib.nvfp4_gather_qmm(
        _ptr(x), code, X, M, K, _ptr(lhs_indices), _ptr(rhs_indices), R, _ptr(w), _ptr(scales),
        _ptr(gs), E, N, int(bool(sorted_indices)), _ptr(out), _stream(dev)))
    return out
