"""Host-side checks of libnvfp4 that need no GPU.

The library must load on a machine without a GPU, export every function
declared in include/nvfp4.h, and reject invalid requests on the host before
anything is launched.  No call here reaches a kernel launch.
"""

import ctypes
import os
import re

import pytest
import torch

import nvfp4_quantized_matmul_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

OK, NULLPTR, SHAPE, DTYPE, GRID, ROUTE, UNSUP, HIP, ALIGN, SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
F32, BF16, F16 = 0, 1, 2
P = ctypes.c_void_p
FAKE = P(0x100000)       # never dereferenced: every call below fails validation first
MISALIGNED = P(0x100004)


@pytest.fixture(scope="module")
def lib():
    return nv.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("nvfp4_transcode", "nvfp4_dequantize", "nvfp4_quantize", "nvfp4_qmm", "nvfp4_qmm_ws",
                 "nvfp4_qmm_noalloc", "nvfp4_static_scratch_bytes",
                 "nvfp4_qmm_workspace_size", "nvfp4_qmm_batched", "nvfp4_qmm_batched_ws", "nvfp4_gather_qmm",
                 "nvfp4_qmm_glu", "nvfp4_qmm_glu_workspace_size",
                 "nvfp4_select_route", "nvfp4_status_string", "nvfp4_version", "nvfp4_qmv_max_rows"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.nvfp4_version() >> 16 == 1
    for code in (OK, NULLPTR, SHAPE, DTYPE, GRID, ROUTE, UNSUP, HIP, ALIGN, SCRATCH):
        s = nv.status_string(code)
        assert s and s != "unknown status"
    assert nv.status_string(12345) == "unknown status"


def test_route_selection(lib):
    assert nv.qmv_max_rows() == 33
    assert nv.select_route(1, 5376, 21504) == "qmv"
    assert nv.select_route(33, 4096, 14336, dtype=torch.float32) == "qmv"
    assert nv.select_route(34, 4096, 14336, dtype=torch.float32) == "qmv"   # K % 256 == 0
    assert nv.select_route(64, 4096, 14336) == "qmv"
    assert nv.select_route(65, 4096, 14336) == "gemm"
    assert nv.select_route(34, 4112, 14336, dtype=torch.float32) == "gemm"  # K % 256 != 0
    assert nv.select_route(2048, 5376, 21504) == "gemm"
    # non-transposed planes always take the GEMM route, any K, N % 16 == 0
    assert nv.select_route(1, 17, 32, transpose=False) == "gemm"
    assert lib.nvfp4_select_route(1, 17, 32, 1, BF16) == SHAPE      # quantized axis K=17
    assert lib.nvfp4_select_route(1, 17, 24, 0, BF16) == SHAPE      # quantized axis N=24
    assert lib.nvfp4_select_route(-1, 16, 16, 1, BF16) == SHAPE
    assert lib.nvfp4_select_route(1, 16, 16, 2, BF16) == SHAPE
    assert lib.nvfp4_select_route(1, 16, 16, 1, 7) == DTYPE


def qmm(lib, x=FAKE, dt=BF16, M=4, K=64, N=32, w=FAKE, s=FAKE, gs=None, tr=1, route=0, out=FAKE):
    return lib.nvfp4_qmm(x, dt, M, K, N, w, s, gs, tr, route, out, None)


def test_qmm_validation(lib):
    assert qmm(lib, x=None) == NULLPTR
    assert qmm(lib, w=None) == NULLPTR
    assert qmm(lib, s=None) == NULLPTR
    assert qmm(lib, out=None) == NULLPTR
    assert qmm(lib, K=24) == SHAPE                      # quantized axis not a multiple of 16
    assert qmm(lib, M=-1) == SHAPE
    assert qmm(lib, dt=9) == DTYPE
    assert qmm(lib, tr=0, route=1, K=17) == ROUTE       # qmv needs a transposed plane
    assert qmm(lib, route=5) == ROUTE
    assert qmm(lib, x=MISALIGNED) == ALIGN
    assert qmm(lib, w=MISALIGNED) == ALIGN
    assert qmm(lib, out=MISALIGNED) == ALIGN
    assert qmm(lib, s=P(0x100001)) == ALIGN
    assert qmm(lib, gs=P(0x100002)) == ALIGN
    assert qmm(lib, M=1 << 40, K=1 << 40) == SHAPE      # size overflow
    # empty outputs launch nothing and succeed, even with NULL buffers
    assert qmm(lib, M=0, x=None, w=None, s=None, out=None) == OK
    assert qmm(lib, N=0, x=None, w=None, s=None, out=None) == OK


def test_qmm_workspace_size_and_validation(lib):
    ws = lib.nvfp4_qmm_workspace_size
    ws.restype = ctypes.c_int64
    # few output tiles on the GEMM route: a split workspace of splits * M * N floats
    small = ws(128, 5376, 21504, 1, BF16, 0)
    assert small > 0 and small % (128 * 21504 * 4) == 0
    assert ws(2048, 5376, 21504, 1, BF16, 0) == 0            # enough tiles: no split
    assert ws(16, 5376, 21504, 1, BF16, 0) == 0              # qmv route
    assert ws(128, 5376, 21504, 1, F16, 0) == small          # f16 splits like bf16
    # float32 on the matrix cores: the [M, 3K] bf16 copy, rounded up to 256
    assert ws(128, 5376, 21504, 1, F32, 0) == 128 * 3 * 5376 * 2
    assert ws(7, 64, 32, 1, F32, 2) == (7 * 3 * 64 * 2 + 255) // 256 * 256
    assert ws(2048, 5376, 21504, 1, F32, 0) == 2048 * 3 * 5376 * 2
    assert ws(128, 5392, 21504, 1, F32, 0) == 0              # K % 64 != 0: float32 FMA kernel
    # non-transposed plane with K % 64 == 0: its dense copy [N, K]
    # of 2-byte values (and the float32 copy of the activations after it)
    dense = (21504 * 5376 * 2 + 255) // 256 * 256
    assert ws(300, 5376, 21504, 0, BF16, 0) == dense
    assert ws(300, 5376, 21504, 0, F16, 2) == dense
    assert ws(300, 5376, 21504, 0, F32, 0) == dense + 300 * 3 * 5376 * 2
    assert ws(1, 5376, 21504, 0, BF16, 0) == dense           # any M
    assert ws(300, 5392, 21504, 0, BF16, 0) == 0             # K % 64 != 0: generic kernel
    assert ws(300, 17, 32, 0, BF16, 0) == 0
    assert ws(128, 5392, 21504, 1, BF16, 0) == 0             # K % 64 != 0: no split
    assert ws(128, 5376, 21504, 1, BF16, 1) == 0             # forced qmv
    assert ws(128, 24, 64, 1, BF16, 0) == SHAPE
    qws = lib.nvfp4_qmm_ws
    args = lambda **k: (k.get("x", FAKE), BF16, 4, 64, 32, FAKE, FAKE, None, 1, 0,
                        k.get("ws", FAKE), k.get("nb", 1024), k.get("out", FAKE), None)
    assert qws(*args(nb=-1)) == SHAPE
    assert qws(*args(ws=None, nb=16)) == SHAPE
    assert qws(*args(ws=MISALIGNED)) == ALIGN
    assert qws(*args(x=None)) == NULLPTR


def test_qmm_noalloc_validation(lib):
    """The no-allocation qmm checks like nvfp4_qmm and refuses, before any
    launch, a split whose partials exceed the static scratch."""
    na = lib.nvfp4_qmm_noalloc
    args = lambda **k: (k.get("x", FAKE), k.get("dt", BF16), k.get("M", 128), k.get("K", 5376),
                        k.get("N", 21504), FAKE, FAKE, None, 1, 0, k.get("out", FAKE), None)
    assert lib.nvfp4_static_scratch_bytes() == 64 << 20
    assert na(*args(x=None)) == NULLPTR
    assert na(*args(out=MISALIGNED)) == ALIGN
    assert na(*args(K=24)) == SHAPE
    assert na(*args(dt=7)) == DTYPE
    assert na(*args(M=0, x=None, out=None)) == OK
    # M = 256, K = 8192 on a 36864-row plane splits K three ways into
    # 3 * 256 * 36864 floats (113 MB): more than the 64 MiB scratch
    ws = lib.nvfp4_qmm_workspace_size
    ws.restype = ctypes.c_int64
    assert ws(256, 8192, 36864, 1, BF16, 0) == 3 * 256 * 36864 * 4
    assert na(*args(M=256, K=8192, N=36864)) == SCRATCH


def glu(lib, x=FAKE, dt=BF16, M=300, K=64, F=32, wg=FAKE, sg=FAKE, gg=None, wu=FAKE, su=FAKE, gu=None, act=0,
        ws=None, nb=0, out=FAKE):
    return lib.nvfp4_qmm_glu(x, dt, M, K, F, wg, sg, gg, wu, su, gu, act, ws, nb, out, None)


def test_qmm_glu_workspace_size_and_validation(lib):
    wsz = lib.nvfp4_qmm_glu_workspace_size
    # the fused kernel (bf16, K % 64 == 0, GEMM-route sizes) takes a workspace
    # only to split its last, partial round of tiles along K: 1344 tiles of
    # 128 features leave 64 after five rounds on 256 compute units (the host
    # reading without a GPU), each split 4 ways, 256 x 256 floats per piece
    assert wsz(2048, 5376, 21504, BF16) == 64 * 4 * 256 * 256 * 4
    assert wsz(300, 64, 32, BF16) == 0          # one slab of K: nothing to split
    # otherwise gate goes to a workspace of M * F elements, rounded up to 256 bytes
    assert wsz(1, 5376, 21504, BF16) == 0                          # M = 1: the decode kernel's gated form
    assert wsz(1, 5376, 21504, F32) == 0
    assert wsz(1, 8208, 64, BF16) == 64 * 2 + 128                  # K beyond the decode kernel (> 8192)
    assert wsz(3, 5392, 21504, BF16) == 3 * 21504 * 2              # K % 256 != 0: separate projections
    assert wsz(3, 4096, 14336, BF16) == 0                           # the multi-row kernel's gated form
    assert wsz(64, 4096, 14336, F32) == 0
    assert wsz(65, 4096, 14336, F32) == 65 * 14336 * 4             # beyond the multi-row widths
    assert wsz(300, 48, 40, BF16) == (300 * 40 * 2 + 255) // 256 * 256   # K % 64 != 0
    assert wsz(300, 64, 32, F32) == 300 * 32 * 4
    assert wsz(300, 64, 32, F16) == 300 * 32 * 2
    assert wsz(0, 64, 32, F32) == 0 and wsz(3, 0, 32, F32) == 0
    assert wsz(3, 24, 32, BF16) == SHAPE
    assert wsz(-1, 64, 32, BF16) == SHAPE
    assert wsz(3, 64, 32, 9) == DTYPE
    assert wsz(1 << 40, 64, 1 << 40, BF16) == SHAPE
    # validation before any launch
    assert glu(lib, x=None) == NULLPTR
    assert glu(lib, wg=None) == NULLPTR
    assert glu(lib, su=None) == NULLPTR
    assert glu(lib, out=None) == NULLPTR
    assert glu(lib, K=24) == SHAPE
    assert glu(lib, act=3) == SHAPE
    assert glu(lib, act=-1) == SHAPE
    assert glu(lib, dt=7) == DTYPE
    assert glu(lib, nb=-1) == SHAPE
    assert glu(lib, nb=64, ws=None) == SHAPE
    assert glu(lib, wu=MISALIGNED) == ALIGN
    assert glu(lib, gu=P(0x100002)) == ALIGN
    assert glu(lib, sg=P(0x100002)) == ALIGN         # the fused kernel reads scale words
    assert glu(lib, su=P(0x100002)) == ALIGN
    # the multi-row gated form (2 <= M <= 64, K % 256 == 0) reads 16-byte scale chunks
    assert glu(lib, M=16, K=256, sg=P(0x100004)) == ALIGN
    assert glu(lib, M=16, K=256, x=P(0x100010), wu=P(0x100008)) == ALIGN
    # the separate-projection case needs its workspace
    assert glu(lib, dt=F32) == SHAPE                 # no workspace given
    assert glu(lib, dt=F32, ws=P(0x200000), nb=300 * 32 * 4 - 1) == SHAPE
    assert glu(lib, dt=F32, ws=P(0x200004), nb=300 * 32 * 4) == ALIGN
    assert glu(lib, dt=F32, ws=P(0x100000), nb=300 * 32 * 4) == SHAPE   # overlaps the inputs
    # empty outputs succeed without launching
    assert glu(lib, M=0, x=None, wg=None, sg=None, wu=None, su=None, out=None) == OK
    assert glu(lib, F=0, x=None, wg=None, sg=None, wu=None, su=None, out=None) == OK


def test_split_counts_leave_no_split_empty(lib):
    """Both K splits of the bf16 GEMM (the split-K launch for few tiles and
    the gated projection's tail split) give each split ceil(slabs / splits)
    slabs; the split count must be recounted from that piece length so the
    last split still starts inside K (42 slabs over 8 splits would leave the
    eighth empty and its partial unwritten).  The host reading here assumes
    256 compute units, as without a GPU."""
    qws = lib.nvfp4_qmm_workspace_size
    qws.restype = ctypes.c_int64
    gws = lib.nvfp4_qmm_glu_workspace_size
    seen_glu = set()
    for K in range(64, 8192 + 1, 64):
        nslabs = K // 64
        # gated projection: one tile of 256 rows x 128 features, split up to 8 ways
        b = int(gws(256, K, 128, BF16))
        if b:
            assert b % (256 * 256 * 4) == 0
            sp = b // (256 * 256 * 4)
            per = -(-nslabs // sp)
            assert 2 <= sp <= 8 and (sp - 1) * per < nslabs, (K, sp, per)
            seen_glu.add(sp)
        # split-K qmm: M = 128 rows, a few tiles
        for N in (256, 4096):
            b = int(qws(128, K, N, 1, BF16, 0))
            if b:
                assert b % (128 * N * 4) == 0
                sp = b // (128 * N * 4)
                per = -(-nslabs // sp)
                assert 2 <= sp <= 8 and (sp - 1) * per < nslabs, (K, N, sp, per)
    # K = 2688 (42 slabs) and K = 2112 (33 slabs) split 7 ways, not 8;
    # K = 1600 (25 slabs) 5 ways, not 6
    assert gws(256, 2688, 128, BF16) == 7 * 256 * 256 * 4
    assert gws(256, 2112, 128, BF16) == 7 * 256 * 256 * 4
    assert gws(256, 1600, 128, BF16) == 5 * 256 * 256 * 4
    assert 8 in seen_glu


def measure_library():
    """The benchmark's streaming-read aid, a library of its own."""
    m = ctypes.CDLL(os.path.join(ROOT, "nvfp4_quantized_matmul_amd", "libnvfp4_measure.so"))
    m.nvfp4_stream_read.argtypes = [P, ctypes.c_int64, ctypes.c_int64, P, P]
    m.nvfp4_stream_read.restype = ctypes.c_int
    return m


def test_measurement_aid_is_not_in_the_library(lib):
    assert not hasattr(lib, "nvfp4_stream_read")
    assert "nvfp4_stream_read" not in declared_functions()


def test_stream_read_validation():
    sr = measure_library().nvfp4_stream_read
    assert sr(FAKE, 24, 64, FAKE, None) == SHAPE       # not a multiple of 16
    assert sr(FAKE, -16, 64, FAKE, None) == SHAPE
    assert sr(FAKE, 1024, 0, FAKE, None) == SHAPE
    assert sr(None, 1024, 64, FAKE, None) == NULLPTR
    assert sr(FAKE, 1024, 64, None, None) == NULLPTR
    assert sr(P(0x100008), 1024, 64, FAKE, None) == ALIGN
    assert sr(FAKE, 1024, 64, P(0x100002), None) == ALIGN
    assert sr(None, 0, 64, None, None) == OK


def test_binding_qmm_glu_checks_before_the_gpu():
    w = torch.zeros(32, 8, dtype=torch.int32)
    s = torch.zeros(32, 4, dtype=torch.uint8)
    x = torch.zeros(2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        nv.qmm_glu(x, w, s, None, w[:16], s[:16], None)
    with pytest.raises(ValueError):
        nv.qmm_glu(x[:, :32], w, s, None, w, s, None)
    with pytest.raises(ValueError):
        nv.qmm_glu(x, w, s, None, w, s, None, act="relu")
    with pytest.raises(ValueError):
        nv.qmm_glu(x, w, s, torch.ones(2), w, s, None)
    assert nv.GLU_ACTIVATIONS == ("gelu_tanh", "gelu", "silu")


def qmm_b(lib, x=FAKE, dt=BF16, XB=3, B=3, M=4, K=64, N=32, w=FAKE, s=FAKE, gs=None, tr=1, route=0,
          out=FAKE):
    return lib.nvfp4_qmm_batched(x, dt, XB, B, M, K, N, w, s, gs, tr, route, out, None)


def test_qmm_batched_validation(lib):
    assert qmm_b(lib, x=None) == NULLPTR
    assert qmm_b(lib, w=None) == NULLPTR
    assert qmm_b(lib, s=None) == NULLPTR
    assert qmm_b(lib, out=None) == NULLPTR
    assert qmm_b(lib, XB=2) == SHAPE                    # x batch must be 1 or B
    assert qmm_b(lib, B=-1) == SHAPE
    assert qmm_b(lib, K=24) == SHAPE
    assert qmm_b(lib, dt=9) == DTYPE
    assert qmm_b(lib, tr=0, route=1, K=17) == ROUTE
    assert qmm_b(lib, XB=1, B=1 << 40, M=1 << 20, K=1 << 20) == SHAPE   # total size overflow
    assert qmm_b(lib, gs=P(0x100002)) == ALIGN
    # every matrix's pointers are checked before any launch: with M=1, N=4
    # (bf16) the second output matrix starts 8 bytes in, not 16-aligned
    assert qmm_b(lib, M=1, N=4) == ALIGN
    assert qmm_b(lib, B=0, XB=1, x=None, w=None, s=None, out=None) == OK
    assert qmm_b(lib, B=0, XB=0, x=None, w=None, s=None, out=None) == OK
    assert qmm_b(lib, M=0, x=None, w=None, s=None, out=None) == OK


def test_qmm_batched_ws_validation(lib):
    """The workspace form checks its workspace like nvfp4_qmm_ws and the
    batch like nvfp4_qmm_batched, all before any launch (M = 300: the GEMM
    route, where the workspace is used)."""
    f = lib.nvfp4_qmm_batched_ws
    args = lambda **k: (k.get("x", FAKE), BF16, 3, 3, 300, 64, 32, FAKE, FAKE, None, 1, 0,
                        k.get("ws", P(0x40000000)), k.get("nb", 1024), k.get("out", FAKE), None)
    assert f(*args(nb=-1)) == SHAPE
    assert f(*args(ws=None, nb=16)) == SHAPE
    assert f(*args(ws=MISALIGNED)) == ALIGN
    assert f(*args(x=None)) == NULLPTR
    assert f(*args(ws=P(0x100000 + 3 * 300 * 32 * 2 - 512))) == SHAPE   # overlaps the last output matrix
    assert f(*args(ws=P(0x100000 + 300 * 64 * 2 - 512), out=P(0x20000000))) == SHAPE   # overlaps x


def gather(lib, x=FAKE, dt=BF16, X=2, M=1, K=64, lhs=None, rhs=FAKE, R=4, w=FAKE, s=FAKE,
           gs=None, E=3, N=32, out=FAKE):
    return lib.nvfp4_gather_qmm(x, dt, X, M, K, lhs, rhs, R, w, s, gs, E, N, 0, out, None)


def test_gather_validation(lib):
    assert gather(lib, rhs=None) == NULLPTR
    assert gather(lib, out=None) == NULLPTR
    assert gather(lib, x=None) == NULLPTR
    assert gather(lib, w=None) == NULLPTR
    assert gather(lib, K=40) == SHAPE
    assert gather(lib, E=-1) == SHAPE
    assert gather(lib, dt=5) == DTYPE
    assert gather(lib, rhs=P(0x100002)) == ALIGN
    assert gather(lib, lhs=P(0x100002)) == ALIGN
    assert gather(lib, x=MISALIGNED) == ALIGN
    assert gather(lib, R=0, x=None, rhs=None, w=None, s=None, out=None) == OK


def quant(lib, w=FAKE, dt=F32, batch=2, rows=4, cols=32, gs_in=None, w_out=P(0x200000), s_out=P(0x300000),
          gs_out=P(0x400000)):
    return lib.nvfp4_quantize(w, dt, batch, rows, cols, gs_in, w_out, s_out, gs_out, None)


def test_quantize_validation(lib):
    assert quant(lib, w=None) == NULLPTR
    assert quant(lib, w_out=None) == NULLPTR
    assert quant(lib, s_out=None) == NULLPTR
    assert quant(lib, gs_out=None) == NULLPTR            # no gs_in: gs_out is where gs goes
    assert quant(lib, cols=24) == SHAPE
    assert quant(lib, rows=-1) == SHAPE
    assert quant(lib, dt=7) == DTYPE
    assert quant(lib, w=MISALIGNED) == ALIGN
    assert quant(lib, w_out=P(0x200004)) == ALIGN
    assert quant(lib, gs_out=P(0x400002)) == ALIGN
    assert quant(lib, batch=1 << 40, rows=1 << 20, cols=1 << 20) == SHAPE
    assert quant(lib, w_out=FAKE) == SHAPE                # output overlapping the input
    assert quant(lib, batch=0, w=None, w_out=None, s_out=None, gs_out=None) == OK


def test_dequantize_and_transcode_validation(lib):
    d = lib.nvfp4_dequantize
    assert d(FAKE, FAKE, None, 1, 4, 24, F32, FAKE, None) == SHAPE
    assert d(FAKE, FAKE, None, 1, 4, 32, 9, FAKE, None) == DTYPE
    assert d(None, FAKE, None, 1, 4, 32, F32, FAKE, None) == NULLPTR
    assert d(FAKE, FAKE, None, 1, 4, 32, F32, MISALIGNED, None) == ALIGN
    assert d(None, None, None, 0, 4, 32, F32, None, None) == OK
    t = lib.nvfp4_transcode
    assert t(FAKE, FAKE, None, 1, 4, 24, FAKE, FAKE, None, None) == SHAPE
    # weight_scale_2 and gs_out must be given together
    assert t(FAKE, FAKE, FAKE, 1, 4, 32, P(0x200000), P(0x300000), None, None) == SHAPE
    assert t(None, FAKE, None, 1, 4, 32, FAKE, FAKE, None, None) == NULLPTR
    # a partially overlapping output is refused (exact aliasing is allowed)
    assert t(P(0x100000), FAKE, None, 1, 4, 32, P(0x100010), P(0x300000), None, None) == SHAPE
    assert t(None, None, None, 0, 4, 32, None, None, None, None) == OK


def test_binding_checks_planes_before_touching_the_gpu():
    w = torch.zeros((8, 4), dtype=torch.int32)
    with pytest.raises(ValueError):
        nv.qmm(torch.zeros((1, 32)), w, torch.zeros((8, 3), dtype=torch.uint8))
    with pytest.raises(ValueError):
        nv.gather_qmm(torch.zeros((1, 1, 32)), w.view(1, 8, 4), torch.zeros((1, 8, 3), dtype=torch.uint8),
                      torch.zeros(1, dtype=torch.int32))
    with pytest.raises(TypeError):
        nv.dequantize(w, torch.zeros((8, 2), dtype=torch.int32))
    with pytest.raises(ValueError):
        nv.qmm(torch.zeros((1, 32)), w, torch.zeros((8, 2), dtype=torch.uint8))   # CPU tensors
