"""nvfp4_qmm_noalloc: nvfp4_qmm for callers that cannot allocate, whose
K-split partials (or the three-part bf16 copy of float32 activations) live
in the library's static device scratch.  Checked through the C ABI against
nvfp4_qmm_ws with a caller workspace (the same kernels and split, so the
same bits) on two calls in a row, the second smaller, and against the
oracle."""

import ctypes

import numpy as np
import pytest
import torch

import nvfp4_quantized_matmul_amd as nv
import nvfp4_synth as synth
import oracle
from gpu_util import DEV, TOL, activations, f32, guarded, host, u8, words

pytestmark = pytest.mark.gpu

P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())


def _inputs(seed, M, K, N, dtype, tr=1):
    case = synth.dense_case(seed, M, K, N, with_gs=True, transpose=bool(tr))
    x_t, x_ref = activations(case.x, dtype)
    return case, x_t, x_ref, words(case.w), u8(case.scales), f32(case.gs)


def _noalloc(lib, code, x_t, w_t, s_t, gs_t, M, K, N, tr=1):
    out, check = guarded((M, N), x_t.dtype)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.nvfp4_qmm_noalloc(P(x_t), code, M, K, N, P(w_t), P(s_t), P(gs_t), tr, 0, P(out), st) == 0
    torch.cuda.synchronize()
    check()
    return out


def _with_workspace(lib, code, x_t, w_t, s_t, gs_t, M, K, N, tr=1):
    need = int(lib.nvfp4_qmm_workspace_size(M, K, N, tr, code, 0))
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    out = torch.empty((M, N), dtype=x_t.dtype, device=DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.nvfp4_qmm_ws(P(x_t), code, M, K, N, P(w_t), P(s_t), P(gs_t), tr, 0, P(ws), need, P(out), st) == 0
    torch.cuda.synchronize()
    return out, need


def test_noalloc_matches_workspace_call_twice_second_smaller():
    lib = nv.load_library()
    assert lib.nvfp4_static_scratch_bytes() == 64 << 20
    # a prefill chunk on the GEMM route that splits K three ways (the split's
    # partials fill 3 * 256 * 21504 floats, just under the 64 MiB), then a
    # smaller call that splits on a smaller slice of the same scratch
    for seed, (M, K, N) in ((9100, (256, 5376, 21504)), (9101, (96, 2048, 1024))):
        case, x_t, x_ref, w_t, s_t, gs_t = _inputs(seed, M, K, N, torch.bfloat16)
        want, need = _with_workspace(lib, 1, x_t, w_t, s_t, gs_t, M, K, N)
        assert 0 < need <= lib.nvfp4_static_scratch_bytes(), (M, K, N, need)
        got = _noalloc(lib, 1, x_t, w_t, s_t, gs_t, M, K, N)
        assert torch.equal(got, want), (M, K, N)
        rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 12)), [M - 1]]))
        ref = oracle.qmm(x_ref[rows], case.w, case.scales, case.gs[0])
        assert oracle.relative_error(host(got)[rows], ref) <= TOL[torch.bfloat16]


def test_noalloc_float32_copy_matches_workspace_call_twice_second_smaller():
    """Float32 activations on the matrix cores: the three-part copy lives in
    the scratch; the second, smaller call reuses its start."""
    lib = nv.load_library()
    for seed, (M, K, N) in ((9105, (300, 512, 272)), (9106, (70, 192, 96))):
        case, x_t, x_ref, w_t, s_t, gs_t = _inputs(seed, M, K, N, torch.float32)
        want, need = _with_workspace(lib, 0, x_t, w_t, s_t, gs_t, M, K, N)
        assert need == (M * 3 * K * 2 + 255) // 256 * 256, (M, K, N, need)
        got = _noalloc(lib, 0, x_t, w_t, s_t, gs_t, M, K, N)
        assert torch.equal(got, want), (M, K, N)
        ref = oracle.qmm(x_ref, case.w, case.scales, case.gs[0])
        assert oracle.relative_error(host(got), ref) <= TOL[torch.float32]


def test_noalloc_non_transposed_dense_copy_twice_second_smaller():
    """A non-transposed plane's dense copy (and, for float32, the activations'
    copy after it) lives in the scratch; the second, smaller call reuses its
    start."""
    lib = nv.load_library()
    for seed, (M, K, N), dt, code in ((9107, (300, 512, 272), torch.bfloat16, 1),
                                      (9108, (40, 256, 48), torch.float32, 0)):
        case, x_t, x_ref, w_t, s_t, gs_t = _inputs(seed, M, K, N, dt, tr=0)
        want, need = _with_workspace(lib, code, x_t, w_t, s_t, gs_t, M, K, N, tr=0)
        assert need >= N * K * 2, (M, K, N, need)
        got = _noalloc(lib, code, x_t, w_t, s_t, gs_t, M, K, N, tr=0)
        assert torch.equal(got, want), (M, K, N)
        ref = oracle.qmm(x_ref, case.w, case.scales, case.gs[0], transpose=False)
        assert oracle.relative_error(host(got), ref) <= TOL[dt]


def test_noalloc_without_scratch_is_nvfp4_qmm():
    """Shapes that need no scratch (decode qmv; float32 with K % 64 != 0) and
    float32 whose copy would not fit the scratch (M * 3K * 2 bytes above
    64 MiB: the float32 FMA kernel) give nvfp4_qmm's bits."""
    lib = nv.load_library()
    for seed, (M, K, N), dt, code in ((9110, (1, 4096, 1000), torch.bfloat16, 1),
                                      (9111, (300, 528, 272), torch.float32, 0),
                                      (9112, (2048, 5632, 128), torch.float32, 0)):
        case, x_t, x_ref, w_t, s_t, gs_t = _inputs(seed, M, K, N, dt)
        need = int(lib.nvfp4_qmm_workspace_size(M, K, N, 1, code, 0))
        assert need == 0 or need > lib.nvfp4_static_scratch_bytes(), (M, K, N, need)
        got = _noalloc(lib, code, x_t, w_t, s_t, gs_t, M, K, N)
        want = torch.empty((M, N), dtype=dt, device=DEV)
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert lib.nvfp4_qmm(P(x_t), code, M, K, N, P(w_t), P(s_t), P(gs_t), 1, 0, P(want), st) == 0
        torch.cuda.synchronize()
        assert torch.equal(got, want)
        ref = oracle.qmm(x_ref, case.w, case.scales, case.gs[0])
        assert oracle.relative_error(host(got), ref) <= TOL[dt]
