"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars: transcode and dequantize bit-exact; qmm / gather with float32 output
max|err|/max|ref| <= 1e-5; bf16 (and f16) output <= 1e-2.  Inputs are the
seeded synthetic workloads of nvfp4_synth; full-size workloads are checked
on sampled outputs that the oracle computes directly.
"""

import ctypes

import numpy as np
import pytest
import torch

import nvfp4_quantized_matmul_amd as nv
import nvfp4_synth as synth
import oracle
from gpu_util import DEV, TOL, activations, f32, guarded, host, i32, u8, words

pytestmark = pytest.mark.gpu

INT32_MAX = 2 ** 31 - 1


def rel(out_t, ref):
    return oracle.relative_error(host(out_t), ref)


def bits32(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def same_f32(got, want):
    """Bit equality, treating any NaN as equal to any NaN."""
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn)
    assert np.array_equal(bits32(got[~gn]), bits32(want[~wn]))


# ----------------------------------------------------------------------------
# transcode
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("batch,rows,cols,with_ws2", [
    (None, 512, 1024, False),   # the tiny workload's U8 [512, 512] source
    (None, 512, 1024, True),
    (3, 40, 96, True),
    (2, 7, 16, True),
])
def test_transcode_bit_exact(batch, rows, cols, with_ws2):
    g = synth.rng(100 + rows + cols)
    wu8, ws, ws2 = synth.modelopt_triplet(g, batch or 1, rows, cols, with_ws2=with_ws2,
                                          code_range=synth.FINITE_POSITIVE_CODES)
    if batch is None:
        wu8, ws = wu8[0], ws[0]
    want_w, want_s, want_gs = oracle.transcode(wu8, ws, ws2)
    w, s, gs = nv.transcode(u8(wu8), u8(ws), None if ws2 is None else f32(ws2))
    torch.cuda.synchronize()
    assert np.array_equal(w.cpu().numpy().view(np.uint32), want_w)
    assert np.array_equal(s.cpu().numpy(), want_s)
    if with_ws2:
        assert np.array_equal(bits32(gs.cpu().numpy()), bits32(want_gs))
    else:
        assert gs is None


def test_direct_transcode_against_dense_requantization():
    """P1's acceptance fixture through the library: two ModelOpt triplets
    transcoded and dequantized (the direct path) against the dense path
    (float16 reconstruction by the library's dequantize, then its quantize
    and dequantize).  Every stage equals the oracle's bit for bit, and the
    dense result stays within the FP8 scale-rounding bound of the direct
    one."""
    from test_oracle_pins import dense_requantization, fp8_rounding_bound
    g = synth.rng(7150)
    weight, scale, ws2 = synth.modelopt_triplet(g, 2, 48, 256)
    tw, ts, tg = nv.transcode(torch.from_numpy(weight).to(DEV), torch.from_numpy(scale).to(DEV),
                              torch.from_numpy(ws2).to(DEV))
    direct = nv.dequantize(tw, ts, tg)
    w16 = nv.dequantize(tw, ts, tg, dtype=torch.float16)
    qw, qs, qg = nv.quantize(w16)
    dense = nv.dequantize(qw, qs, qg)
    torch.cuda.synchronize()
    for b in range(2):
        w, s, gs = oracle.transcode(weight[b], scale[b], ws2[b:b + 1])
        want_direct = oracle.dequantize(w, s, gs[0])
        r16, rqw, rqs, rqg, want_dense = dense_requantization(w, s, gs[0])
        assert np.array_equal(direct[b].cpu().numpy().view(np.uint32), want_direct.view(np.uint32))
        assert np.array_equal(w16[b].cpu().numpy().view(np.uint16), r16.view(np.uint16))
        assert np.array_equal(qw[b].cpu().numpy().view(np.uint32), rqw)
        assert np.array_equal(qs[b].cpu().numpy(), rqs)
        assert qg[b].cpu().numpy().view(np.uint32) == rqg.view(np.uint32)[0]
        assert np.array_equal(dense[b].cpu().numpy().view(np.uint32), want_dense.view(np.uint32))
        err = np.abs(host(dense[b]) - want_direct.astype(np.float64))
        assert np.all(err <= fp8_rounding_bound(r16, rqg[0]))


def test_transcode_in_place_and_guard_bands():
    g = synth.rng(120)
    wu8, ws, ws2 = synth.modelopt_triplet(g, 2, 33, 64)
    want_w, want_s, want_gs = oracle.transcode(wu8, ws, ws2)
    src_w, src_s = u8(wu8), u8(ws)
    w, s, gs = nv.transcode(src_w, src_s, f32(ws2), inplace=True)
    torch.cuda.synchronize()
    assert w.data_ptr() == src_w.data_ptr() and s.data_ptr() == src_s.data_ptr()
    assert np.array_equal(w.cpu().numpy().view(np.uint32), want_w)
    assert np.array_equal(s.cpu().numpy(), want_s)
    # out-of-place through the C ABI with guarded outputs
    lib = nv.load_library()
    w_out, chk_w = guarded((2, 33, 8), torch.int32, fill=0x5A5A5A5A)
    s_out, chk_s = guarded((2, 33, 4), torch.uint8)
    g_out, chk_g = guarded((2,), torch.float32)
    # keep the device inputs referenced until the kernel has run
    d_w, d_s, d_g = u8(wu8), u8(ws), f32(ws2)
    st = lib.nvfp4_transcode(ctypes.c_void_p(d_w.data_ptr()), ctypes.c_void_p(d_s.data_ptr()),
                             ctypes.c_void_p(d_g.data_ptr()), 2, 33, 64,
                             ctypes.c_void_p(w_out.data_ptr()), ctypes.c_void_p(s_out.data_ptr()),
                             ctypes.c_void_p(g_out.data_ptr()), None)
    assert st == 0
    chk_w(); chk_s(); chk_g()
    assert np.array_equal(w_out.cpu().numpy().view(np.uint32), want_w)
    assert np.array_equal(bits32(g_out.cpu().numpy()), bits32(want_gs))


# ----------------------------------------------------------------------------
# dequantize
# ----------------------------------------------------------------------------

def every_pair_plane():
    w = np.tile(np.array([0x76543210, 0xFEDCBA98], dtype=np.uint32), (256, 1))
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    return w, scales


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("gs", [None, 777.25, 0.5, 2688.0])
def test_dequantize_every_pair_bit_exact(dtype, gs):
    w, sc = every_pair_plane()
    want = oracle.dequantize(w, sc, None if gs is None else np.float32(gs))
    out = nv.dequantize(words(w), u8(sc), None if gs is None else f32([gs]), dtype=dtype)
    torch.cuda.synchronize()
    if dtype == torch.float32:
        same_f32(out.cpu().numpy(), want)
    elif dtype == torch.bfloat16:
        got = out.cpu().view(torch.int16).numpy().view(np.uint16)
        exp = oracle.f32_to_bf16_bits(want)
        nan = np.isnan(want)
        assert np.array_equal(got[~nan], exp[~nan])
        assert np.all(np.isnan(oracle.bf16_bits_to_f32(got[nan])))
    else:
        got = out.cpu().numpy()
        exp = want.astype(np.float16)
        nan = np.isnan(want)
        assert np.array_equal(got[~nan].view(np.uint16), exp[~nan].view(np.uint16))
        assert np.all(np.isnan(got[nan]))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize_batched_ragged_with_guard_bands(dtype):
    g = synth.rng(130)
    w = synth.packed_words(g, (3, 37, 6))
    sc = synth.scale_codes(g, (3, 37, 3), synth.FINITE_POSITIVE_CODES)
    gs = synth.global_scales(g, 3)
    want = np.stack([oracle.dequantize(w[b], sc[b], gs[b]) for b in range(3)])
    lib = nv.load_library()
    out, check = guarded((3, 37, 48), dtype)
    d_w, d_s, d_g = words(w), u8(sc), f32(gs)
    st = lib.nvfp4_dequantize(ctypes.c_void_p(d_w.data_ptr()), ctypes.c_void_p(d_s.data_ptr()),
                              ctypes.c_void_p(d_g.data_ptr()), 3, 37, 48,
                              0 if dtype == torch.float32 else 1, ctypes.c_void_p(out.data_ptr()), None)
    assert st == 0
    check()
    if dtype == torch.float32:
        same_f32(out.cpu().numpy(), want)
    else:
        assert np.array_equal(out.cpu().view(torch.int16).numpy().view(np.uint16),
                              oracle.f32_to_bf16_bits(want))


def test_dequantize_batch_beyond_grid_y_limit():
    """65,573 tiny matrices (one row of 16 elements each), more than the
    65,535 block rows of the grid's y axis: the kernel's matrix loop covers
    the rest.  Seven global scales in turn; bit-exact in bf16 against the
    oracle per group of matrices sharing a scale."""
    B = 65573
    g = synth.rng(132)
    w = synth.packed_words(g, (B, 1, 2))
    sc = synth.scale_codes(g, (B, 1, 1), synth.FINITE_POSITIVE_CODES)
    gs7 = synth.global_scales(g, 7)
    gs = gs7[np.arange(B) % 7]
    want = np.empty((B, 1, 16), dtype=np.float32)
    for k in range(7):
        want[k::7] = oracle.dequantize(w[k::7], sc[k::7], gs7[k])
    lib = nv.load_library()
    out, check = guarded((B, 1, 16), torch.bfloat16)
    d_w, d_s, d_g = words(w), u8(sc), f32(gs)
    st = lib.nvfp4_dequantize(ctypes.c_void_p(d_w.data_ptr()), ctypes.c_void_p(d_s.data_ptr()),
                              ctypes.c_void_p(d_g.data_ptr()), B, 1, 16, 1, ctypes.c_void_p(out.data_ptr()), None)
    assert st == 0
    check()
    assert np.array_equal(out.cpu().view(torch.int16).numpy().view(np.uint16), oracle.f32_to_bf16_bits(want))


def test_dequantize_decode_row_length_bit_exact():
    """Rows of the decode workload's length (K = 5376), 2048 of them."""
    g = synth.rng(131)
    w = synth.packed_words(g, (2048, 672))
    sc = synth.scale_codes(g, (2048, 336))
    gs = synth.global_scales(g, 1)
    want = oracle.dequantize(w, sc, gs[0])
    out = nv.dequantize(words(w), u8(sc), f32(gs))
    same_f32(out.cpu().numpy(), want)


# ----------------------------------------------------------------------------
# quantize
# ----------------------------------------------------------------------------

def dense_weights(seed, shape, lo=-20, hi=4):
    """N(0,1) rows scaled by 2^k, k uniform in [lo, hi], so block scales span
    zero, subnormal and large E4M3 codes within one matrix."""
    g = synth.rng(seed)
    base = synth.activations(g, shape)
    k = g.integers(lo, hi + 1, size=shape[:-1] + (1,))
    return (base * np.exp2(k)).astype(np.float32), g


def quantize_both(dense, dtype, gs=None):
    x_t, x_ref = activations(dense, dtype)
    lead = dense.shape[:-2]
    want_w, want_s, want_g = oracle.quantize(x_ref, gs)
    w, s, g = nv.quantize(x_t, None if gs is None else f32(np.asarray(gs, dtype=np.float32)))
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), want_s)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), want_w)
    same_f32(g.cpu().numpy(), want_g)
    return w, s, g


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("shape", [(1, 16), (37, 48), (3, 5, 256), (8, 5376)])
@pytest.mark.parametrize("given_gs", [False, True])
def test_quantize_bit_exact(dtype, shape, given_gs):
    """Codes, words and global scales equal the oracle's bit for bit, for
    float32, bf16 and f16 inputs, one or several matrices, computed or given
    global scales (given ones below the matrix maximum saturate at 448)."""
    dense, g = dense_weights(3800 + sum(shape), shape)
    batch = int(np.prod(shape[:-2])) if len(shape) > 2 else 1
    gs = synth.global_scales(g, batch, lo=0.5, hi=20.0) if given_gs else None
    quantize_both(dense, dtype, gs)


def test_quantize_special_values():
    """Zeros and -0, a NaN, an infinity, values at E2M1 and E4M3 ties."""
    dense = np.zeros((6, 32), dtype=np.float32)
    dense[0, 3] = -0.0
    dense[1, :16] = [6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, -5, -6, 0.3, 5.5, 0, -0.0]
    dense[2, 5] = np.nan
    dense[2, 20] = 1.5
    dense[3, 17] = np.inf
    dense[3, 18] = -2.0
    dense[4, :16] = np.float32(1.0625)
    dense[5, 16] = np.float32(0.0048828125)
    dense[5, 0] = np.float32(0.0009765625)
    quantize_both(dense, torch.float32, gs=[2688.0])
    quantize_both(dense[4:], torch.float32, gs=[448.0])
    quantize_both(dense, torch.float32)                 # gs = NaN (the matrix holds one)


def test_quantize_e2m1_thresholds():
    """Every E2M1 rounding midpoint (0.25 .. 5) and its two float32
    neighbours, as quotients of block scales that are not powers of two
    (normal and subnormal E4M3), with either sign; then saturation of
    quotients beyond 6 (and of an infinity) under a small global scale, and
    tiny or subnormal elements that keep only their sign."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rows = []
    for sc in [1.0, 1.125, 0.8125, 3.5, 0.01171875, 88.0]:
        d = np.float32(sc)
        vals = []
        for t in mids:
            c = np.float32(np.float32(t) * d)
            vals += [np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(np.inf))]
        vals += [np.float32(0.0)] * (30 - len(vals))
        for sign in (1.0, -1.0):
            row = np.zeros(32, dtype=np.float32)
            row[0] = row[16] = np.float32(6.0) * d
            row[1:16] = np.float32(sign) * np.asarray(vals[:15], dtype=np.float32)
            row[17:32] = np.float32(sign) * np.asarray(vals[15:30], dtype=np.float32)
            rows.append(row)
    quantize_both(np.stack(rows), torch.float32, gs=[2688.0])

    sat = np.zeros((2, 32), dtype=np.float32)
    sat[0, :16] = [100, 7.0, 6.5, -50, np.inf, 3, -np.inf, 1e30, 0.2, -0.2, 5, 6, 0, -0.0, 1, 2]
    sat[1, :16] = np.float32(6.0)
    sat[1, 1:5] = [1e-30, -1e-30, 1e-40, -1e-40]
    sat[1, 16:] = np.float32(-3.0)
    quantize_both(sat, torch.float32, gs=[1.0])
    quantize_both(sat[1:], torch.float32, gs=[2688.0])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_round_trip_through_the_library(dtype):
    """Planes whose blocks each hold a +-6 come back unchanged through the
    library's dequantize and quantize (with the same global scale)."""
    g = synth.rng(3900)
    nib = g.integers(0, 16, size=(64, 512)).astype(np.uint32)
    pos = g.integers(0, 16, size=(64, 32))
    for r in range(64):
        for b in range(32):
            c = 16 * b + pos[r, b]
            nib[r, c] = 0x7 | (nib[r, c] & 0x8)
    shifts = (np.arange(8, dtype=np.uint32) * 4)
    words_np = (nib.reshape(64, 64, 8) << shifts).sum(axis=-1, dtype=np.uint64).astype(np.uint32)
    sc = synth.scale_codes(g, (64, 32), synth.NORMAL_POSITIVE_CODES)
    gs = synth.global_scales(g, 1, lo=0.5, hi=20.0)
    dense = nv.dequantize(words(words_np), u8(sc), f32(gs), dtype=dtype)
    w2, s2, g2 = nv.quantize(dense, f32(gs))
    torch.cuda.synchronize()
    if dtype == torch.float32:
        assert np.array_equal(w2.cpu().numpy().view(np.uint32), words_np)
        assert np.array_equal(s2.cpu().numpy(), sc)
    else:
        # bf16 rounds the dequantized values; the library must still match the oracle
        want_w, want_s, _ = oracle.quantize(dense.float().cpu().numpy(), gs)
        assert np.array_equal(w2.cpu().numpy().view(np.uint32), want_w)
        assert np.array_equal(s2.cpu().numpy(), want_s)


# ----------------------------------------------------------------------------
# qmm
# ----------------------------------------------------------------------------

def run_qmm(case, dtype, route="auto", guard=False):
    x_t, x_ref = activations(case.x, dtype)
    gs = None if case.gs is None else case.gs[0]
    ref = oracle.qmm(x_ref, case.w, case.scales, gs, transpose=case.transpose)
    out = check = None
    if guard:
        out, check = guarded((case.M, case.N), dtype)
    out = nv.qmm(x_t, words(case.w), u8(case.scales), None if case.gs is None else f32(case.gs),
                 transpose=case.transpose, route=route, out=out)
    torch.cuda.synchronize()
    if check:
        check()
    return out, ref


@pytest.mark.parametrize("route", ["auto", "qmv", "gemm"])
def test_tiny_qmv_f32(route):
    """M=1, K=1024, N=512, float32, no global scale, every finite positive
    scale code (including subnormal scales)."""
    w = synth.WORKLOADS["tiny_qmv_m1_k1024_n512_f32"]
    case = synth.dense_case(w["seed"], 1, 1024, 512, with_gs=False, code_range=w["codes"])
    out, ref = run_qmm(case, torch.float32, route, guard=True)
    assert rel(out, ref) <= TOL[torch.float32]


@pytest.mark.parametrize("route", ["auto", "gemm"])
def test_decode_qmv_full_size(route):
    """M=1, K=5376, N=21504, bf16 activations and output, scalar global
    scale -- the decode workload in the launch configuration that is timed."""
    w = synth.WORKLOADS["decode_qmv_m1_k5376_n21504_bf16"]
    case = synth.dense_case(w["seed"], 1, 5376, 21504, with_gs=True)
    out, ref = run_qmm(case, torch.bfloat16, route)
    assert rel(out, ref) <= TOL[torch.bfloat16]


@pytest.fixture(scope="module")
def multirow_plane():
    w = synth.WORKLOADS["multirow_qmv_k4096_n14336"]
    case = synth.dense_case(w["seed"], 33, 4096, 14336, with_gs=True)
    W = oracle.dequantize(case.w, case.scales, case.gs[0]).astype(np.float64)
    return case, W


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M", [3, 6, 16, 33])
def test_multirow_qmv_full_size(multirow_plane, M, dtype):
    case, W = multirow_plane
    x_t, x_ref = activations(case.x[:M], dtype)
    ref = x_ref.astype(np.float64) @ W.T          # == oracle.qmm on the same planes
    out = nv.qmm(x_t, words(case.w), u8(case.scales), f32(case.gs))
    assert nv.select_route(M, 4096, 14336, dtype=dtype) == "qmv"
    assert rel(out, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M", [1, 3, 33, 64])
@pytest.mark.parametrize("route", ["qmv", "gemm"])
def test_partial_block_n272(M, dtype, route):
    case = synth.dense_case(3100 + M, M, 4096, 272, with_gs=True)
    out, ref = run_qmm(case, dtype, route, guard=True)
    assert rel(out, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M", [1, 3, 6, 16, 33])
@pytest.mark.parametrize("with_gs", [False, True])
def test_non_transposed_k17(M, dtype, with_gs):
    case = synth.dense_case(3200 + M, M, 17, 32, transpose=False, with_gs=with_gs)
    out, ref = run_qmm(case, dtype, "auto", guard=True)
    assert rel(out, ref) <= TOL[dtype]


@pytest.mark.parametrize("shape", [(300, 1056, 600), (64, 512, 272), (5, 48, 40), (7, 64, 263),
                                   (257, 96, 520), (1, 16, 16)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("route", ["qmv", "gemm"])
def test_ragged_shapes(shape, dtype, route):
    M, K, N = shape
    case = synth.dense_case(3300 + M + K + N, M, K, N, with_gs=True)
    out, ref = run_qmm(case, dtype, route, guard=True)
    assert rel(out, ref) <= TOL[dtype]


# ----------------------------------------------------------------------------
# qmm over a batch of weight matrices
# ----------------------------------------------------------------------------

def run_qmm_batched(c, dtype, route="auto", with_gs=True):
    x_t, x_ref = activations(c.x, dtype)
    gs = c.gs if with_gs else None
    ref = oracle.qmm_batched(x_ref, c.w, c.scales, gs, transpose=c.transpose)
    out, check = guarded((c.B, c.M, c.N), dtype)
    nv.qmm_batched(x_t, words(c.w), u8(c.scales), None if gs is None else f32(gs),
                   transpose=c.transpose, route=route, out=out)
    check()
    return out, ref


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("M,route", [(1, "auto"), (3, "auto"), (3, "qmv"), (3, "gemm"), (64, "auto"),
                                     (64, "gemm"), (300, "auto")])
@pytest.mark.parametrize("broadcast_x", [False, True])
def test_qmm_batched_transposed(dtype, M, route, broadcast_x):
    """Three weight matrices (N = 272, a partial 256-row tile), each with its
    own global scale, against their own or one shared activation matrix."""
    c = synth.batched_case(3400 + M, B=3, M=M, K=512, N=272, broadcast_x=broadcast_x)
    out, ref = run_qmm_batched(c, dtype, route)
    assert rel(out, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M", [3, 64])
@pytest.mark.parametrize("with_gs", [False, True])
def test_qmm_batched_non_transposed(dtype, M, with_gs):
    c = synth.batched_case(3500 + M, B=2, M=M, K=40, N=48, transpose=False)
    out, ref = run_qmm_batched(c, dtype, "auto", with_gs=with_gs)
    assert rel(out, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_qmm_batched_multirow_plane(dtype):
    """Two matrices of the multi-row workload's shape (K=4096, N=14336) at
    M=3 through the qmv route, as the pages test batched weights."""
    c = synth.batched_case(3600, B=2, M=3, K=4096, N=14336)
    out, ref = run_qmm_batched(c, dtype)
    assert rel(out, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("M", [1, 2, 16, 33, 64])
@pytest.mark.parametrize("broadcast_x", [False, True])
def test_qmm_batched_one_launch_equals_single_calls(dtype, M, broadcast_x):
    """On the qmv route the decode (M = 1) and multi-row (2 <= M <= 64)
    kernels take the whole batch in one launch: every matrix's result is
    within tolerance of the oracle and bit for bit what one qmm call on that
    matrix alone gives."""
    c = synth.batched_case(3800 + M, B=5, M=M, K=512, N=272, broadcast_x=broadcast_x)
    out, ref = run_qmm_batched(c, dtype)
    assert rel(out, ref) <= TOL[dtype]
    x_t, _ = activations(c.x, dtype)
    for b in range(c.B):
        single = nv.qmm(x_t[0 if broadcast_x else b], words(c.w[b]), u8(c.scales[b]), f32(c.gs[b:b + 1]))
        assert torch.equal(out[b], single), f"matrix {b}"


@pytest.mark.parametrize("M", [1, 16])
def test_qmm_batched_beyond_one_grid_row_limit(M):
    """65540 matrices (K = 256, N = 16), more than one launch's 65535 grid
    rows: the batch goes out in two launches; matrices on both sides of the
    split are checked against the oracle one by one."""
    B = 65540
    c = synth.batched_case(3900 + M, B=B, M=M, K=256, N=16, broadcast_x=True)
    x_t, x_ref = activations(c.x, torch.bfloat16)
    out = nv.qmm_batched(x_t, words(c.w), u8(c.scales), f32(c.gs))
    torch.cuda.synchronize()
    for b in (0, 1, 65533, 65534, 65535, 65536, B - 1):
        ref = oracle.qmm(x_ref[0], c.w[b], c.scales[b], c.gs[b])
        assert rel(out[b], ref) <= TOL[torch.bfloat16], f"matrix {b}"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("transpose", [True, False])
def test_qmm_batched_gemm_route_workspace(dtype, transpose):
    """GEMM-route batches with one workspace for every matrix (the K split of
    few tiles, the float32 three-part split, the non-transposed dense copy):
    within tolerance of the oracle and, matrix by matrix, bit for bit what
    qmm gives with its own workspace.  The same batch through the C ABI
    without a workspace (float32 and non-transposed then take the float32
    FMA kernel) stays within tolerance too."""
    c = synth.batched_case(3960 + int(transpose), B=3, M=200, K=2048, N=272, transpose=transpose)
    lib = nv.load_library()
    code = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}[dtype]
    assert lib.nvfp4_qmm_workspace_size(200, 2048, 272, int(transpose), code, 0) > 0
    out, ref = run_qmm_batched(c, dtype)
    assert rel(out, ref) <= TOL[dtype]
    x_t, _ = activations(c.x, dtype)
    for b in range(c.B):
        single = nv.qmm(x_t[b], words(c.w[b]), u8(c.scales[b]), f32(c.gs[b:b + 1]), transpose=transpose)
        assert torch.equal(out[b], single), f"matrix {b}"
    w_t, s_t, g_t = words(c.w), u8(c.scales), f32(c.gs)
    plain = torch.empty_like(out)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.nvfp4_qmm_batched(P(x_t), code, c.XB, c.B, c.M, c.K, c.N, P(w_t), P(s_t), P(g_t), int(transpose), 0,
                               P(plain), None)
    assert st == 0
    torch.cuda.synchronize()
    assert rel(plain, ref) <= TOL[dtype]


def test_qmm_batched_empty_and_misaligned():
    c = synth.batched_case(3700, B=2, M=1, K=32, N=4)
    x_t, _ = activations(c.x, torch.bfloat16)
    empty = nv.qmm_batched(x_t[:0], words(c.w[:0]), u8(c.scales[:0]), f32(c.gs[:0]))
    assert tuple(empty.shape) == (0, 1, 4)
    # the second output matrix would start 8 bytes in: refused before any launch
    with pytest.raises(nv.NVFP4Error):
        nv.qmm_batched(x_t, words(c.w), u8(c.scales), f32(c.gs))


# ----------------------------------------------------------------------------
# GEMM with K split among blocks (few output tiles)
# ----------------------------------------------------------------------------

def qmm_ws_raw(x_t, w_t, s_t, gs_t, M, K, N, ws_bytes, out):
    lib = nv.load_library()
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV) if ws_bytes else None
    st = lib.nvfp4_qmm_ws(ctypes.c_void_p(x_t.data_ptr()), 1, M, K, N, ctypes.c_void_p(w_t.data_ptr()),
                          ctypes.c_void_p(s_t.data_ptr()), None if gs_t is None else ctypes.c_void_p(gs_t.data_ptr()),
                          1, 0, None if ws is None else ctypes.c_void_p(ws.data_ptr()), ws_bytes,
                          ctypes.c_void_p(out.data_ptr()), None)
    assert st == 0
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("M,K,N", [(65, 2048, 1024), (200, 2048, 300), (256, 1024, 520), (96, 4352, 264)])
def test_gemm_split_k_small_shapes(M, K, N):
    """Few output tiles: the binding passes a workspace and K is split
    (up to 8 ways; K = 4352 leaves a shorter last split); full comparison."""
    case = synth.dense_case(3950 + M + K, M, K, N, with_gs=True)
    lib = nv.load_library()
    assert lib.nvfp4_qmm_workspace_size(M, K, N, 1, 1, 0) > 0
    out, ref = run_qmm(case, torch.bfloat16, "gemm", guard=True)
    assert rel(out, ref) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("M", [65, 128, 256])
def test_gemm_split_k_prefill_shape_sampled(M):
    """The prefill plane (K=5376, N=21504) at chunk sizes that split three
    ways: sampled rows against the oracle, all rows against the unsplit
    path (float32 summation order only)."""
    wl = synth.WORKLOADS["prefill_gemm_m2048_k5376_n21504_bf16"]
    case = synth.dense_case(wl["seed"] + M, M, 5376, 21504, with_gs=True)
    x_t, x_ref = activations(case.x, torch.bfloat16)
    w_t, s_t, gs_t = words(case.w), u8(case.scales), f32(case.gs)
    lib = nv.load_library()
    ws_bytes = int(lib.nvfp4_qmm_workspace_size(M, 5376, 21504, 1, 1, 0))
    assert ws_bytes == 3 * M * 21504 * 4
    split = qmm_ws_raw(x_t, w_t, s_t, gs_t, M, 5376, 21504, ws_bytes,
                       torch.empty((M, 21504), dtype=torch.bfloat16, device=DEV))
    whole = qmm_ws_raw(x_t, w_t, s_t, gs_t, M, 5376, 21504, 0,
                       torch.empty((M, 21504), dtype=torch.bfloat16, device=DEV))
    assert oracle.relative_error(host(split), host(whole)) <= TOL[torch.bfloat16]
    rows = sorted(set([0, M - 1] + list(np.linspace(0, M - 1, 12).astype(int))))
    W = oracle.dequantize(case.w, case.scales, case.gs[0]).astype(np.float64)
    ref = x_ref[rows].astype(np.float64) @ W.T
    assert oracle.relative_error(host(split)[rows], ref) <= TOL[torch.bfloat16]


def test_gemm_split_k_workspace_too_small_falls_back():
    M, K, N = 128, 2048, 1024
    case = synth.dense_case(3990, M, K, N, with_gs=True)
    x_t, x_ref = activations(case.x, torch.bfloat16)
    ref = oracle.qmm(x_ref, case.w, case.scales, case.gs[0])
    lib = nv.load_library()
    need = int(lib.nvfp4_qmm_workspace_size(M, K, N, 1, 1, 0))
    out = qmm_ws_raw(x_t, words(case.w), u8(case.scales), f32(case.gs), M, K, N, need // 2,
                     torch.empty((M, N), dtype=torch.bfloat16, device=DEV))
    assert rel(out, ref) <= TOL[torch.bfloat16]


def test_prefill_gemm_full_size_sampled():
    """M=2048, K=5376, N=21504 bf16 through the route that is timed; 48
    sampled activation rows (spread over all row tiles) against the oracle."""
    wl = synth.WORKLOADS["prefill_gemm_m2048_k5376_n21504_bf16"]
    case = synth.dense_case(wl["seed"], 2048, 5376, 21504, with_gs=True)
    assert nv.select_route(2048, 5376, 21504) == "gemm"
    x_t, x_ref = activations(case.x, torch.bfloat16)
    out = nv.qmm(x_t, words(case.w), u8(case.scales), f32(case.gs))
    rows = np.unique(np.concatenate([np.arange(0, 2048, 47), [1, 255, 256, 1023, 2047]]))
    ref = oracle.qmm(x_ref[rows], case.w, case.scales, case.gs[0])
    got = host(out)[rows]
    assert oracle.relative_error(got, ref) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("shape,dtype", [((1300, 768, 12000), torch.bfloat16),
                                         ((777, 1152, 30000), torch.float16),
                                         ((1300, 768, 12000), torch.float32)])
def test_prefill_persistent_route_ragged(shape, dtype):
    """More output tiles than compute units and K a multiple of 384: the
    persistent prefill kernel, whose blocks walk several tiles and queue each
    next tile's first slabs during the current tile's last steps (float32
    activations: their three-part bf16 rows of 3K, weight slab s mod K/64,
    with the binding's workspace).  Partial row and column tiles; sampled
    rows (every row tile) against the oracle, and a second call equal to the
    first bit for bit."""
    M, K, N = shape
    assert ((M + 255) // 256) * ((N + 255) // 256) > 256 and K % 384 == 0
    case = synth.dense_case(4300 + M + K, M, K, N, with_gs=True)
    x_t, x_ref = activations(case.x, dtype)
    out = nv.qmm(x_t, words(case.w), u8(case.scales), f32(case.gs), route="gemm")
    again = nv.qmm(x_t, words(case.w), u8(case.scales), f32(case.gs), route="gemm")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), again.view(torch.uint8))
    rows = np.unique(np.concatenate([np.arange(0, M, 61), [1, 255, 256, M - 2, M - 1]]))
    ref = oracle.qmm(x_ref[rows], case.w, case.scales, case.gs[0])
    assert oracle.relative_error(host(out)[rows], ref) <= TOL[dtype]


# ----------------------------------------------------------------------------
# f16 and float32 activations on the matrix cores
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(300, 576, 520), (513, 128, 264), (96, 4352, 264), (1, 64, 16)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_gemm_f16_f32_matrix_cores_ragged(shape, dtype):
    """K % 64 == 0 on the GEMM route: f16 runs the f16 matrix-core GEMM (with
    the K split for few tiles), float32 the three-part bf16 copy through the
    binding's workspace; partial row and column tiles; full comparison."""
    M, K, N = shape
    code = 0 if dtype == torch.float32 else 2
    need = int(nv.load_library().nvfp4_qmm_workspace_size(M, K, N, 1, code, 2))
    if dtype == torch.float32:
        assert need == (M * 3 * K * 2 + 255) // 256 * 256
    case = synth.dense_case(4100 + M + K + N, M, K, N, with_gs=True)
    out, ref = run_qmm(case, dtype, "gemm", guard=True)
    assert rel(out, ref) <= TOL[dtype]


def test_gemm_f32_matrix_cores_match_fma_kernel():
    """The three-part copy and the float32 FMA kernel (nvfp4_qmm without a
    workspace) compute the same products exactly; they differ only in float32
    summation order."""
    M, K, N = 300, 1024, 520
    case = synth.dense_case(4190, M, K, N, with_gs=True)
    x_t, x_ref = activations(case.x, torch.float32)
    w_t, s_t, gs_t = words(case.w), u8(case.scales), f32(case.gs)
    lib = nv.load_library()
    need = int(lib.nvfp4_qmm_workspace_size(M, K, N, 1, 0, 0))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    mfma = torch.empty((M, N), dtype=torch.float32, device=DEV)
    fma = torch.empty((M, N), dtype=torch.float32, device=DEV)
    assert lib.nvfp4_qmm_ws(P(x_t), 0, M, K, N, P(w_t), P(s_t), P(gs_t), 1, 0, P(ws), need, P(mfma), None) == 0
    assert lib.nvfp4_qmm(P(x_t), 0, M, K, N, P(w_t), P(s_t), P(gs_t), 1, 0, P(fma), None) == 0
    torch.cuda.synchronize()
    assert oracle.relative_error(host(mfma), host(fma)) <= TOL[torch.float32]
    ref = oracle.qmm(x_ref, case.w, case.scales, case.gs[0])
    assert rel(mfma, ref) <= TOL[torch.float32]


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_gemm_matrix_cores_nonfinite_activations(dtype):
    """An infinity or NaN among the activations reaches the outputs of its
    row as in IEEE arithmetic (inf * 0 is NaN, inf + -inf is NaN), the other
    rows stay finite; float32 infinities go whole into the copy's first part."""
    M, K, N = 70, 128, 96
    case = synth.dense_case(4195, M, K, N, with_gs=True)
    x = case.x.astype(np.float32).copy()
    x[0, 5] = np.inf
    x[1, 7] = -np.inf
    x[2, 9] = np.nan
    x[3, 11] = np.inf
    x[3, 12] = -np.inf
    x_t, x_ref = activations(x, dtype)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = oracle.qmm(x_ref, case.w, case.scales, case.gs[0])
    out = nv.qmm(x_t, words(case.w), u8(case.scales), f32(case.gs), route="gemm")
    got = host(out)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert np.array_equal(np.sign(got[np.isinf(ref)]), np.sign(ref[np.isinf(ref)]))
    assert np.isfinite(ref[4:]).all()
    assert oracle.relative_error(got[4:], ref[4:]) <= TOL[dtype]


@pytest.mark.parametrize("shape", [(300, 512, 272), (64, 128, 32), (257, 192, 528), (1030, 320, 4112),
                                   (1, 64, 16), (33, 256, 48)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("with_gs", [False, True])
def test_gemm_non_transposed_matrix_cores(shape, dtype, with_gs):
    """Non-transposed planes [K, N/8] with K % 64 == 0: the
    binding's workspace holds the plane's dense transposed copy (and the
    float32 activations' three-part copy), the matrix-core GEMM runs on it;
    partial row and column tiles (N = 272, 528, 4112), full comparison."""
    M, K, N = shape
    code = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}[dtype]
    need = int(nv.load_library().nvfp4_qmm_workspace_size(M, K, N, 0, code, 0))
    assert need >= N * K * 2
    case = synth.dense_case(4300 + M + K + N, M, K, N, transpose=False, with_gs=with_gs)
    out, ref = run_qmm(case, dtype, "auto", guard=True)
    assert rel(out, ref) <= TOL[dtype]


def test_gemm_non_transposed_matrix_cores_match_generic():
    """The dense route (nvfp4_qmm_ws) and the generic kernel (nvfp4_qmm, no
    workspace) on one non-transposed float32 call: the same exact products,
    float32 summation order only."""
    M, K, N = 300, 1024, 528
    case = synth.dense_case(4390, M, K, N, transpose=False, with_gs=True)
    x_t, x_ref = activations(case.x, torch.float32)
    w_t, s_t, gs_t = words(case.w), u8(case.scales), f32(case.gs)
    lib = nv.load_library()
    need = int(lib.nvfp4_qmm_workspace_size(M, K, N, 0, 0, 0))
    assert need == (N * K * 2 + 255) // 256 * 256 + M * 3 * K * 2
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    dense = torch.empty((M, N), dtype=torch.float32, device=DEV)
    generic = torch.empty((M, N), dtype=torch.float32, device=DEV)
    assert lib.nvfp4_qmm_ws(P(x_t), 0, M, K, N, P(w_t), P(s_t), P(gs_t), 0, 0, P(ws), need, P(dense), None) == 0
    assert lib.nvfp4_qmm(P(x_t), 0, M, K, N, P(w_t), P(s_t), P(gs_t), 0, 0, P(generic), None) == 0
    torch.cuda.synchronize()
    assert oracle.relative_error(host(dense), host(generic)) <= TOL[torch.float32]
    ref = oracle.qmm(x_ref, case.w, case.scales, case.gs[0], transpose=False)
    assert rel(dense, ref) <= TOL[torch.float32]


def test_prefill_plane_f16_and_f32_sampled():
    """The prefill plane (M=2048, K=5376, N=21504) with f16 activations and
    with float32 activations (the three-part copy, 66 MB, through the
    binding's workspace): 45 sampled rows of each against the oracle."""
    wl = synth.WORKLOADS["prefill_gemm_m2048_k5376_n21504_bf16"]
    case = synth.dense_case(wl["seed"] + 7, 2048, 5376, 21504, with_gs=True)
    w_t, s_t, gs_t = words(case.w), u8(case.scales), f32(case.gs)
    rows = np.unique(np.concatenate([np.arange(0, 2048, 53), [1, 255, 256, 1023, 2047]]))
    got, refs = [], []
    for dtype in (torch.float16, torch.float32):
        x_t, x_ref = activations(case.x, dtype)
        out = nv.qmm(x_t, w_t, s_t, gs_t)
        torch.cuda.synchronize()
        got.append(host(out)[rows])
        refs.append(x_ref[rows])
        del x_t, out
    ref = oracle.qmm(np.concatenate(refs), case.w, case.scales, case.gs[0])
    n = len(rows)
    assert oracle.relative_error(got[0], ref[:n]) <= TOL[torch.float16]
    assert oracle.relative_error(got[1], ref[n:]) <= TOL[torch.float32]


# ----------------------------------------------------------------------------
# gated MLP projection
# ----------------------------------------------------------------------------

GLU_CODES = (0x08, 0x28)   # block scales 2^-6 .. 2^-2: gate sums of unit size, where the activations bend


def glu_planes(seed, M, K, F, gs=(True, True)):
    g = synth.dense_case(seed, M, K, F, with_gs=gs[0], code_range=GLU_CODES)
    u = synth.dense_case(seed + 1, M, K, F, with_gs=gs[1], code_range=GLU_CODES)
    return g, u


def gs_arg(c):
    return None if c.gs is None else f32(c.gs)


def gs_ref(c):
    return None if c.gs is None else c.gs[0]


def run_glu(g, u, dtype, act, guard=True):
    x_t, x_ref = activations(g.x, dtype)
    ref = oracle.qmm_glu(x_ref, g.w, g.scales, gs_ref(g), u.w, u.scales, gs_ref(u), act)
    out = check = None
    if guard:
        out, check = guarded((g.M, g.N), dtype)
    out = nv.qmm_glu(x_t, words(g.w), u8(g.scales), gs_arg(g), words(u.w), u8(u.scales), gs_arg(u),
                     act=act, out=out)
    torch.cuda.synchronize()
    if check:
        check()
    return out, ref


def glu_workspace(M, K, F, dtype):
    code = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}[dtype]
    return int(nv.load_library().nvfp4_qmm_glu_workspace_size(M, K, F, code))


def glu_is_fused(M, K, F, dtype):
    return dtype == torch.bfloat16 and K > 0 and K % 64 == 0 and nv.select_route(M, K, F) == "gemm"


def glu_route(M, K, F, dtype):
    """Which form nvfp4_qmm_glu takes: the fused GEMM, the decode kernel's
    (M = 1), the multi-row kernel's (2 <= M <= 64, K % 256 == 0), or the two
    projections and a combine."""
    if glu_is_fused(M, K, F, dtype):
        return "gemm"
    if M == 1 and K % 32 == 0:
        return "decode"
    if 2 <= M <= 64 and K % 256 == 0:
        return "rows"
    return "separate"


ACT_CODES = {"gelu_tanh": 0, "gelu": 1, "silu": 2}


def run_glu_no_workspace(g, u, act):
    """The fused kernel through the C ABI with no workspace: one launch, no
    tail split."""
    x_t, x_ref = activations(g.x, torch.bfloat16)
    ref = oracle.qmm_glu(x_ref, g.w, g.scales, gs_ref(g), u.w, u.scales, gs_ref(u), act)
    out, check = guarded((g.M, g.N), torch.bfloat16)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    keep = [x_t, words(g.w), u8(g.scales), gs_arg(g), words(u.w), u8(u.scales), gs_arg(u)]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    status = nv.load_library().nvfp4_qmm_glu(P(keep[0]), 1, g.M, g.K, g.N, P(keep[1]), P(keep[2]), P(keep[3]),
                                             P(keep[4]), P(keep[5]), P(keep[6]), ACT_CODES[act], None, 0, P(out), st)
    assert status == 0
    torch.cuda.synchronize()
    check()
    return out, ref


@pytest.mark.parametrize("act", ["gelu_tanh", "gelu", "silu"])
@pytest.mark.parametrize("shape", [(300, 1024, 1000), (513, 320, 257), (65, 64, 128), (256, 4096, 384)])
@pytest.mark.parametrize("workspace", [True, False])
def test_qmm_glu_fused_kernel(shape, act, workspace):
    """bf16 with K % 64 == 0 at GEMM sizes runs the fused kernel: several row
    and feature tiles, a ragged feature count (257, and 1000 = 7 full tiles +
    104), one slab (K = 64), rows past a tile.  With the binding's workspace
    the tiles (fewer than the compute units here) are also split along K
    where each piece keeps at least four slabs; without one, one launch."""
    M, K, F = shape
    assert glu_is_fused(M, K, F, torch.bfloat16)
    g, u = glu_planes(6100 + M + K + F, M, K, F)
    out, ref = run_glu(g, u, torch.bfloat16, act) if workspace else run_glu_no_workspace(g, u, act)
    assert rel(out, ref) <= TOL[torch.bfloat16], (shape, act)


@pytest.mark.parametrize("gs", [(False, False), (True, False), (False, True)])
def test_qmm_glu_fused_global_scales(gs):
    """Each plane's global scale applies to its own projection only."""
    g, u = glu_planes(6200, 300, 512, 272, gs=gs)
    out, ref = run_glu(g, u, torch.bfloat16, "gelu_tanh")
    assert rel(out, ref) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("shape", [(1, 512, 300), (3, 256, 200), (40, 512, 96), (300, 48, 40), (70, 96, 64)])
@pytest.mark.parametrize("act", ["gelu_tanh", "silu"])
def test_qmm_glu_separate_projections(shape, dtype, act):
    """Every case the fused GEMM does not take: M = 1 is the decode kernel's
    gated form and M = 3 and 40 (K % 256 == 0) the multi-row kernel's (one
    launch each); the GEMM-size shapes with K = 48 (300 rows) and K = 96 (70
    rows) run both projections through qmm's routes into a workspace, then
    combine."""
    M, K, F = shape
    route = glu_route(M, K, F, dtype)
    if route in ("decode", "rows"):
        assert glu_workspace(M, K, F, dtype) == 0
    elif route == "separate":
        size = M * F * (4 if dtype == torch.float32 else 2)
        assert glu_workspace(M, K, F, dtype) == (size + 255) // 256 * 256
    g, u = glu_planes(6300 + M + K + F, M, K, F)
    out, ref = run_glu(g, u, dtype, act)
    assert rel(out, ref) <= TOL[dtype], (shape, dtype, act)


@pytest.mark.parametrize("K", [256, 4096, 5376, 8192])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("act", ["gelu_tanh", "gelu", "silu"])
def test_qmm_glu_decode_kernel(K, dtype, act):
    """M = 1 runs the decode kernel's gated form in one launch (no
    workspace): one to four chunks per lane (K = 8192 keeps 16 loads in
    flight per wavefront), a ragged feature count, each plane its own global
    scale."""
    assert glu_workspace(1, K, 333, dtype) == 0
    g, u = glu_planes(6700 + K, 1, K, 333)
    out, ref = run_glu(g, u, dtype, act)
    assert rel(out, ref) <= TOL[dtype], (K, dtype, act)


@pytest.mark.parametrize("M", [2, 16, 17, 33, 64])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
def test_qmm_glu_multirow_kernel(M, dtype):
    """2 <= M <= 64 with K % 256 == 0 runs the multi-row kernel's gated form
    in one launch (no workspace): one to four 16-row fragments, one and
    sixteen pair-groups, a ragged feature count (the last 32-feature block
    partial), each plane its own global scale."""
    for K, F, act in ((256, 100, "silu"), (4096, 333, "gelu_tanh")):
        assert glu_route(M, K, F, dtype) == "rows" and glu_workspace(M, K, F, dtype) == 0
        g, u = glu_planes(6900 + M + K, M, K, F)
        out, ref = run_glu(g, u, dtype, act)
        assert rel(out, ref) <= TOL[dtype], (M, K, dtype)


def test_qmm_glu_decode_mlp_shape():
    """The decode MLP's gate/up shape, M = 1, K = 5376, F = 21504, bf16, in
    full against the oracle."""
    g, u = glu_planes(6800, 1, 5376, 21504)
    out, ref = run_glu(g, u, torch.bfloat16, "gelu_tanh")
    assert rel(out, ref) <= TOL[torch.bfloat16]


def test_qmm_glu_zero_k_and_empty():
    g, u = glu_planes(6400, 5, 0, 32)
    out, ref = run_glu(g, u, torch.bfloat16, "gelu")
    assert np.all(host(out) == 0.0)
    x = torch.zeros(0, 64, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(32, 8, dtype=torch.int32, device=DEV)
    s = torch.zeros(32, 4, dtype=torch.uint8, device=DEV)
    assert nv.qmm_glu(x, w, s, None, w, s, None).shape == (0, 32)


def test_qmm_glu_fused_tail_split():
    """300 tiles of 128 features leave 44 after one round on 256 compute
    units; with the workspace they are split 5 ways along K (32 slabs) and
    reduced: sampled features of whole-round and split tiles against the
    oracle, and the whole output against the unsplit fused launch."""
    M, K, F = 256, 2048, 128 * 300
    lib = nv.load_library()
    ws_bytes = glu_workspace(M, K, F, torch.bfloat16)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip(f"split sizes are chosen for 256 compute units, this device has {cus}")
    assert ws_bytes == 44 * 5 * 256 * 256 * 4
    g, u = glu_planes(6600, M, K, F)
    x_t, x_ref = activations(g.x, torch.bfloat16)
    wg, sg, wu_, su_ = words(g.w), u8(g.scales), words(u.w), u8(u.scales)
    ggs, ugs = f32(g.gs), f32(u.gs)
    out = nv.qmm_glu(x_t, wg, sg, ggs, wu_, su_, ugs, act="silu")     # the binding passes the workspace
    plain, check = guarded((M, F), torch.bfloat16)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    assert lib.nvfp4_qmm_glu(P(x_t), 1, M, K, F, P(wg), P(sg), P(ggs), P(wu_), P(su_), P(ugs), 2, None, 0,
                             P(plain), st) == 0
    torch.cuda.synchronize()
    check()
    feats = np.unique(np.concatenate([np.arange(0, 256 * 128, 509), np.arange(256 * 128, F, 37), [F - 1]]))
    ref = oracle.qmm_glu(x_ref, g.w[feats], g.scales[feats], g.gs[0], u.w[feats], u.scales[feats], u.gs[0], "silu")
    assert oracle.relative_error(host(out)[:, feats], ref) <= TOL[torch.bfloat16]
    assert oracle.relative_error(host(out), host(plain)) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("shape,workspace", [((300, 768, 128 * 140 - 37), False),
                                             ((300, 768, 128 * 300 - 100), True),
                                             ((2048, 5376, 21504), True)])
def test_qmm_glu_persistent_route(shape, workspace):
    """More whole-round tiles of the fused gated kernel than compute units
    and K a multiple of 384: the persistent launch, whose blocks walk several
    tiles with the next tile's first slabs queued during the current tile's
    last steps.  280 tiles in one launch (no workspace); 600 tiles with the
    binding's workspace (512 persistent, the 88 left split along K) and the
    same call without one (600 persistent); and the MLP prefill shape.
    Ragged row and feature tiles; sampled features of every feature tile
    region against the oracle, a second call bit-equal to the first, and
    the workspace form against the one-launch form."""
    M, K, F = shape
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = ((M + 255) // 256) * ((F + 127) // 128)
    assert tiles > cus and K % 384 == 0 and glu_is_fused(M, K, F, torch.bfloat16)
    g, u = glu_planes(6900 + M + F, M, K, F)
    x_t, x_ref = activations(g.x, torch.bfloat16)
    wg, sg, wu_, su_ = words(g.w), u8(g.scales), words(u.w), u8(u.scales)
    ggs, ugs = f32(g.gs), f32(u.gs)
    lib = nv.load_library()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def one_launch():
        out, check = guarded((M, F), torch.bfloat16)
        assert lib.nvfp4_qmm_glu(P(x_t), 1, M, K, F, P(wg), P(sg), P(ggs), P(wu_), P(su_), P(ugs), 0, None, 0,
                                 P(out), st) == 0
        torch.cuda.synchronize()
        check()
        return out

    plain = one_launch()
    assert torch.equal(plain.view(torch.int16), one_launch().view(torch.int16))
    outs = [plain]
    if workspace:
        assert glu_workspace(M, K, F, torch.bfloat16) > 0
        outs.append(nv.qmm_glu(x_t, wg, sg, ggs, wu_, su_, ugs, act="gelu_tanh"))
        torch.cuda.synchronize()
        assert oracle.relative_error(host(outs[1]), host(plain)) <= TOL[torch.bfloat16]
    feats = np.unique(np.concatenate([np.arange(0, F, max(1, F // 97)), np.arange(F - 130, F), [127, 128]]))
    ref = oracle.qmm_glu(x_ref, g.w[feats], g.scales[feats], g.gs[0], u.w[feats], u.scales[feats], u.gs[0],
                         "gelu_tanh")
    for out in outs:
        assert oracle.relative_error(host(out)[:, feats], ref) <= TOL[torch.bfloat16], shape


@pytest.mark.parametrize("K,splits", [(2688, 7), (2112, 7), (1600, 5)])
def test_qmm_glu_tail_split_piece_lengths(K, splits):
    """One tile of 256 rows x 128 features shared by up to 8 blocks along K:
    at K = 2688 (42 slabs) pieces of 6 slabs need 7 splits, at 2112 (33
    slabs) pieces of 5 need 7, at 1600 (25 slabs, at most 6 splits of four or
    more) pieces of 5 need 5.  Every
    split must start inside K, or its partial would never be written and the
    reduction would add whatever the workspace held.  The binding's
    workspace is filled with NaN first, so an unwritten partial would show."""
    M, F = 256, 128
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip(f"split sizes are chosen for 256 compute units, this device has {cus}")
    ws_bytes = glu_workspace(M, K, F, torch.bfloat16)
    assert ws_bytes == splits * 256 * 256 * 4, ws_bytes
    g, u = glu_planes(6650 + K, M, K, F)
    x_t, x_ref = activations(g.x, torch.bfloat16)
    ref = oracle.qmm_glu(x_ref, g.w, g.scales, g.gs[0], u.w, u.scales, u.gs[0], "gelu_tanh")
    ws = torch.full((ws_bytes // 4,), float("nan"), dtype=torch.float32, device=DEV)
    out, check = guarded((M, F), torch.bfloat16)
    keep = [x_t, words(g.w), u8(g.scales), f32(g.gs), words(u.w), u8(u.scales), f32(u.gs)]
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert nv.load_library().nvfp4_qmm_glu(P(keep[0]), 1, M, K, F, *[P(t) for t in keep[1:]], 0, P(ws), ws_bytes,
                                           P(out), st) == 0
    torch.cuda.synchronize()
    check()
    assert np.all(np.isfinite(host(out)))
    assert rel(out, ref) <= TOL[torch.bfloat16], K


def test_qmm_glu_full_size_sampled():
    """The prefill MLP's gate/up shape, M=2048, K=5376, F=21504, bf16, through
    the fused kernel that is timed, with the binding's workspace (so the 64
    tiles past five whole rounds are split along K); sampled rows and
    features, among them the split tiles' (features 20480 on), against the
    oracle (features are independent rows of both planes)."""
    M, K, F = 2048, 5376, 21504
    assert glu_is_fused(M, K, F, torch.bfloat16)
    g, u = glu_planes(6500, M, K, F)
    x_t, x_ref = activations(g.x, torch.bfloat16)
    out = nv.qmm_glu(x_t, words(g.w), u8(g.scales), f32(g.gs), words(u.w), u8(u.scales), f32(u.gs))
    rows = np.unique(np.concatenate([np.arange(0, M, 97), [1, 255, 256, 2047]]))
    feats = np.unique(np.concatenate([np.arange(0, F, 61), np.arange(20480, F, 13), [127, 128, 21503]]))
    ref = oracle.qmm_glu(x_ref[rows], g.w[feats], g.scales[feats], g.gs[0], u.w[feats], u.scales[feats],
                         u.gs[0], "gelu_tanh")
    got = host(out)[np.ix_(rows, feats)]
    assert oracle.relative_error(got, ref) <= TOL[torch.bfloat16]


def test_global_scale_2688_is_identity():
    case = synth.dense_case(3400, 4, 256, 96, with_gs=False)
    x_t, _ = activations(case.x, torch.float32)
    for route in ("qmv", "gemm"):
        a = nv.qmm(x_t, words(case.w), u8(case.scales), None, route=route)
        b = nv.qmm(x_t, words(case.w), u8(case.scales), f32([2688.0]), route=route)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("route", ["qmv", "gemm"])
def test_nan_scale_propagates_to_its_output_only(route):
    case = synth.dense_case(3500, 2, 128, 64, with_gs=True)
    sc = case.scales.copy()
    sc[5, 3] = 0x7F
    x_t, x_ref = activations(case.x, torch.bfloat16)
    out = host(nv.qmm(x_t, words(case.w), u8(sc), f32(case.gs), route=route))
    assert np.all(np.isnan(out[:, 5]))
    assert not np.any(np.isnan(np.delete(out, 5, axis=1)))


def test_zero_k_gives_zeros():
    x = torch.zeros((3, 0), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((8, 0), dtype=torch.int32, device=DEV)
    s = torch.zeros((8, 0), dtype=torch.uint8, device=DEV)
    out = nv.qmm(x, w, s)
    assert torch.equal(out.float().cpu(), torch.zeros((3, 8)))


# ----------------------------------------------------------------------------
# gather
# ----------------------------------------------------------------------------

def run_gather(case, dtype, lhs=True, sorted_flag=None, guard=False):
    x_t, x_ref = activations(case.x, dtype)
    lhs_np = case.lhs if lhs else None
    ref = oracle.gather_qmm(x_ref, lhs_np, case.rhs, case.w, case.scales, case.gs)
    R = case.rhs.shape[0]
    out = check = None
    if guard:
        out, check = guarded((R, case.M, case.N), dtype)
    out = nv.gather_qmm(x_t, words(case.w), u8(case.scales), i32(case.rhs),
                        None if lhs_np is None else i32(lhs_np),
                        None if case.gs is None else f32(case.gs),
                        sorted_indices=case.sorted_indices if sorted_flag is None else sorted_flag,
                        out=out)
    torch.cuda.synchronize()
    if check:
        check()
    return out, ref


def assert_zero_rows(out_t, rhs, lhs, E, X):
    got = out_t.float().cpu().numpy()
    for r in range(len(rhs)):
        src = r if lhs is None else int(lhs[r])
        if not (0 <= int(rhs[r]) < E) or not (0 <= src < X):
            assert np.all(got[r] == 0.0) and not np.any(np.signbit(got[r])), r


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("sort", [False, True])
@pytest.mark.parametrize("M", [1, 3])
@pytest.mark.parametrize("with_gs", [False, True])
@pytest.mark.parametrize("K", [96, 48])
def test_gather_small_full(dtype, sort, M, with_gs, K):
    case = synth.gather_case(5100 + M + K, tokens=5, E=6, N=80, K=K, top_k=2, sort=sort,
                             with_gs=with_gs, M=M, out_of_range=(6, 7, INT32_MAX, -1))
    out, ref = run_gather(case, dtype, guard=True)
    assert oracle.relative_error(host(out), ref) <= TOL[dtype]
    assert_zero_rows(out, case.rhs, case.lhs, 6, 5)


def test_gather_lhs_out_of_range_and_identity_lhs():
    case = synth.gather_case(5200, tokens=4, E=5, N=48, K=64, top_k=1, sort=False, M=2)
    case.lhs = case.lhs.copy()
    case.lhs[1] = 4            # x has 4 rows: out of range
    case.lhs[2] = -3
    out, ref = run_gather(case, torch.float32, guard=True)
    assert oracle.relative_error(host(out), ref) <= 1e-5
    assert_zero_rows(out, case.rhs, case.lhs, 5, 4)
    out, ref = run_gather(case, torch.float32, lhs=False)
    assert oracle.relative_error(host(out), ref) <= 1e-5


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("K,N", [(2048, 1536), (96, 301), (5376, 64)])
def test_gather_one_row_pairs_equal_plain_decode(dtype, K, N):
    """Gather with one activation row per pair (below two rows per expert)
    runs the decode kernel's gather form: every valid pair's row equals the
    plain M = 1 qmm of its activation row against its expert's plane, bit for
    bit, pairs with an out-of-range expert or row give +0.0, and the sorted
    hint does not change a bit.  Against the oracle too."""
    # 12 pairs over 8 experts: below two rows per expert, so not the grouped path
    case = synth.gather_case(5400 + K + N, tokens=6, E=8, N=N, K=K, top_k=2, sort=False, M=1,
                             with_gs=True, out_of_range=(8, -1))
    case.lhs = case.lhs.copy()
    case.lhs[3] = 6            # x has 6 rows: out of range
    out, ref = run_gather(case, dtype, guard=True)
    assert oracle.relative_error(host(out), ref) <= TOL[dtype]
    assert_zero_rows(out, case.rhs, case.lhs, 8, 6)
    x_t, _ = activations(case.x, dtype)
    view = torch.int32 if dtype == torch.float32 else torch.int16
    checked = 0
    for r in range(case.rhs.shape[0]):
        e, src = int(case.rhs[r]), int(case.lhs[r])
        if not (0 <= e < 8 and 0 <= src < 6):
            continue
        plain = nv.qmm(x_t[src], words(case.w[e]), u8(case.scales[e]), f32(case.gs[e:e + 1]))
        assert torch.equal(out[r].view(view), plain.view(view)), r
        checked += 1
    assert checked >= 6
    hinted, _ = run_gather(case, dtype, sorted_flag=True)
    assert torch.equal(hinted.view(view), out.view(view))


def test_gather_sorted_hint_on_unsorted_indices():
    case = synth.gather_case(5300, tokens=9, E=4, N=64, K=128, top_k=3, sort=False, M=1)
    a, ref = run_gather(case, torch.bfloat16, sorted_flag=True)
    b, _ = run_gather(case, torch.bfloat16, sorted_flag=False)
    assert oracle.relative_error(host(a), ref) <= 1e-2
    assert oracle.relative_error(host(b), ref) <= 1e-2


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("K", [256, 2304])
@pytest.mark.parametrize("N", [64, 300])
@pytest.mark.parametrize("M", [1, 3])
@pytest.mark.parametrize("sort", [False, True])
def test_gather_mfma_grouped_experts(K, N, M, sort, dtype):
    """Gather at several rows per expert (the expert-grouped MFMA path,
    K % 256 == 0; f32 activations as three bf16 parts): ~14 pairs per expert
    times M rows needs one to three 16-row passes per expert; K = 2304 runs
    nine pair-groups over four wavefronts; N = 300 leaves a partial 64-row
    tile; out-of-range rhs and lhs give exact +0.0 rows; sorted and unsorted
    pairs agree."""
    case = synth.gather_case(5400 + K + N + M, tokens=24, E=5, N=N, K=K, top_k=3, sort=sort,
                             with_gs=(M == 3), M=M, out_of_range=(5, 6, INT32_MAX, -1))
    case.lhs = case.lhs.copy()
    case.lhs[3] = 24           # x has 24 rows: out of range
    case.lhs[10] = -1
    if dtype == torch.float16:  # keep the f16 outputs finite
        case.scales = np.minimum(case.scales, 0x50).astype(np.uint8)
    out, ref = run_gather(case, dtype, guard=True)
    assert oracle.relative_error(host(out), ref) <= TOL[dtype]
    assert_zero_rows(out, case.rhs, case.lhs, 5, 24)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("sort", [False, True])
def test_gather_mfma_many_scan_rounds(sort, dtype):
    """K = 256 runs the grouped kernel with one wavefront, so its scan of rhs
    takes 64 pairs per round: R = 400 pairs over 3 experts is seven rounds,
    with an expert's pairs split across rounds when unsorted."""
    case = synth.gather_case(5500 + int(sort), tokens=200, E=3, N=80, K=256, top_k=2, sort=sort,
                             with_gs=True, M=1, out_of_range=(3, INT32_MAX))
    if dtype == torch.float16:  # keep the f16 outputs finite
        case.scales = np.minimum(case.scales, 0x50).astype(np.uint8)
    out, ref = run_gather(case, dtype, guard=True)
    assert oracle.relative_error(host(out), ref) <= TOL[dtype]
    assert_zero_rows(out, case.rhs, case.lhs, 3, 200)


def moe_reference_sampled(case, x_ref, experts):
    """Rows of the given in-range experts, computed expert by expert with the
    oracle's qmm (gather semantics themselves are pinned on small cases)."""
    rows, refs = [], []
    for e in experts:
        rr = np.nonzero(case.rhs == e)[0]
        if len(rr) == 0:
            continue
        xs = x_ref[case.lhs[rr], 0, :]
        refs.append(oracle.qmm(xs, case.w[e], case.scales[e], case.gs[e]))
        rows.append(rr)
    return np.concatenate(rows), np.concatenate(refs)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_moe_sorted_prefill_full_size(dtype):
    wl = synth.WORKLOADS["moe_gather_e128_n1536_k2048_top8"]
    case = synth.gather_case(wl["seed"], tokens=128, E=128, N=1536, K=2048, top_k=8, sort=True,
                             with_gs=True, out_of_range=(128, 129, INT32_MAX))
    x_t, x_ref = activations(case.x, dtype)
    out = nv.gather_qmm(x_t, words(case.w), u8(case.scales), i32(case.rhs), i32(case.lhs),
                        f32(case.gs), sorted_indices=True)
    experts = np.unique(case.rhs[(case.rhs >= 0) & (case.rhs < 128)])
    pick = experts[np.linspace(0, len(experts) - 1, 10).astype(int)]
    rows, ref = moe_reference_sampled(case, x_ref, pick)
    got = host(out)[rows, 0, :]
    assert oracle.relative_error(got, ref) <= TOL[dtype]
    assert_zero_rows(out, case.rhs, case.lhs, 128, 128)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("sort", [True, False])
def test_moe_prefill_large_batch(dtype, sort):
    """512 tokens on the MoE shape: about 32 rows per expert, so each
    (tile, expert) block makes two or more 16-row passes over the expert's
    plane; sampled experts against the oracle."""
    wl = synth.WORKLOADS["moe_gather_e128_n1536_k2048_top8"]
    case = synth.gather_case(wl["seed"] + 3, tokens=512, E=128, N=1536, K=2048, top_k=8, sort=sort,
                             with_gs=True, out_of_range=(128, INT32_MAX))
    if dtype == torch.float16:  # keep the f16 outputs finite
        case.scales = np.minimum(case.scales, 0x50).astype(np.uint8)
    x_t, x_ref = activations(case.x, dtype)
    out = nv.gather_qmm(x_t, words(case.w), u8(case.scales), i32(case.rhs), i32(case.lhs),
                        f32(case.gs), sorted_indices=sort)
    experts = np.unique(case.rhs[(case.rhs >= 0) & (case.rhs < 128)])
    pick = experts[np.linspace(0, len(experts) - 1, 8).astype(int)]
    rows, ref = moe_reference_sampled(case, x_ref, pick)
    got = host(out)[rows, 0, :]
    assert oracle.relative_error(got, ref) <= TOL[dtype]
    assert_zero_rows(out, case.rhs, case.lhs, 128, 512)


@pytest.mark.parametrize("tokens", [1, 2, 4, 8])
def test_moe_unsorted_decode_full_size(tokens):
    wl = synth.WORKLOADS["moe_gather_e128_n1536_k2048_top8"]
    case = synth.gather_case(wl["seed"] + tokens, tokens=tokens, E=128, N=1536, K=2048, top_k=8,
                             sort=False, with_gs=True, out_of_range=(128, INT32_MAX) if tokens > 1 else ())
    x_t, x_ref = activations(case.x, torch.bfloat16)
    out = nv.gather_qmm(x_t, words(case.w), u8(case.scales), i32(case.rhs), i32(case.lhs),
                        f32(case.gs), sorted_indices=False)
    experts = np.unique(case.rhs[(case.rhs >= 0) & (case.rhs < 128)])
    rows, ref = moe_reference_sampled(case, x_ref, experts)
    got = host(out)[rows, 0, :]
    assert oracle.relative_error(got, ref) <= TOL[torch.bfloat16]
    assert_zero_rows(out, case.rhs, case.lhs, 128, tokens)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("K", [32, 2048, 6144, 8192, 8224])
@pytest.mark.parametrize("N", [1, 7, 300, 5000])
@pytest.mark.parametrize("with_gs", [False, True])
def test_decode_kernel_shapes(dtype, K, N, with_gs):
    """M = 1 over every activation-stationary variant (1..4 chunks per lane)
    and the general kernel beyond them (K = 8224), with row counts that leave
    partial runs of rows per wave."""
    # f16 outputs: scales up to 2^3 keep every dot product inside f16 range
    codes = (0x08, 0x50) if dtype == torch.float16 else synth.NORMAL_POSITIVE_CODES
    case = synth.dense_case(3600 + K + N, 1, K, N, with_gs=with_gs, code_range=codes)
    out, ref = run_qmm(case, dtype, "auto", guard=True)
    assert rel(out, ref) <= TOL[dtype]


@pytest.mark.parametrize("K", [64, 128, 192, 256, 320, 448])
@pytest.mark.parametrize("M", [1, 100, 300])
@pytest.mark.parametrize("N", [40, 300])
def test_gemm_slab_pipeline_shapes(K, M, N):
    """bf16 GEMM route with K a multiple of 64: 1..7 slabs of 64 exercise
    every tail of the three-stage pipeline; M and N leave partial tiles."""
    case = synth.dense_case(3700 + K + M + N, M, K, N, with_gs=True)
    out, ref = run_qmm(case, torch.bfloat16, "gemm", guard=True)
    assert rel(out, ref) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("K", [256, 512, 2304, 4352, 6144])
@pytest.mark.parametrize("M", [2, 15, 17, 33, 48, 64])
@pytest.mark.parametrize("N", [40, 300])
def test_multirow_mfma_pipeline_shapes(dtype, K, M, N):
    """qmv route for 2 <= M <= 64 with K a multiple of 256 (the MFMA
    kernel): 1, 2, 9, 17 and 24 pair-groups of 256 k over up to 16, 8 or 4
    wavefronts leave one to six pair-groups per wavefront; 1..4 activation
    fragments (bf16, f16) or 16-row launches (f32, split into three bf16
    parts); N leaves partial 64-row tiles.  f16 uses small scale codes so
    its outputs stay finite."""
    codes = (0x08, 0x50) if dtype == torch.float16 else synth.NORMAL_POSITIVE_CODES
    case = synth.dense_case(3800 + K + M + N, M, K, N, with_gs=True, code_range=codes)
    out, ref = run_qmm(case, dtype, "qmv", guard=True)
    assert rel(out, ref) <= TOL[dtype]


# ----------------------------------------------------------------------------
# Seeded random sweep over shapes, dtypes, routes and global scales
# ----------------------------------------------------------------------------

def _sweep_cases(n, seed):
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kmul = int(g.choice([16, 32, 64, 256]))
        K = kmul * int(g.integers(1, 4096 // kmul + 1))
        M = int(g.choice([1, 2, 3, int(g.integers(4, 34)), int(g.integers(34, 65)), int(g.integers(65, 400))]))
        N = int(g.integers(1, 700))
        dtype = [torch.float32, torch.bfloat16, torch.float16][int(g.integers(0, 3))]
        route = ["auto", "qmv", "gemm"][int(g.integers(0, 3))]
        cases.append((i, M, K, N, dtype, route, bool(g.integers(0, 2))))
    return cases


@pytest.mark.parametrize("i,M,K,N,dtype,route,with_gs", _sweep_cases(48, 2024))
def test_qmm_random_sweep(i, M, K, N, dtype, route, with_gs):
    case = synth.dense_case(7000 + i, M, K, N, with_gs=with_gs)
    if dtype == torch.float16:   # keep f16 outputs finite
        case.scales = np.minimum(case.scales, 0x48).astype(np.uint8)
    out, ref = run_qmm(case, dtype, route, guard=True)
    assert rel(out, ref) <= TOL[dtype], (M, K, N, dtype, route)


def _slice_sweep_cases(n, seed):
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        K = 256 * int(g.integers(16, 33))          # at least 16 pair-groups: full blocks for every width
        M = int(g.integers(2, 65))
        N = int(g.integers(1, 1200))
        dtype = [torch.bfloat16, torch.float32][int(g.integers(0, 2))]
        gated = dtype == torch.bfloat16 and M <= 16 and bool(g.integers(0, 2))
        cases.append((i, M, K, N, dtype, gated))
    return cases


@pytest.mark.parametrize("i,M,K,N,dtype,gated", _slice_sweep_cases(20, 2026))
def test_multirow_lds_slices_random_sweep(i, M, K, N, dtype, gated):
    """The multi-row kernel's forms whose weights go through per-wavefront
    LDS slices (bf16 with one, three or four fragments, the gated bf16 form
    with one, float32 with whole pair-groups per wavefront; bf16 with two
    fragments keeps registers), at random K >= 4096 (several pair-groups per
    wavefront for K > 4096), random M and ragged N, against the oracle."""
    if gated:
        g, u = glu_planes(7700 + i, M, K, N)
        out, ref = run_glu(g, u, dtype, "silu")
    else:
        case = synth.dense_case(7800 + i, M, K, N, with_gs=bool(i % 2))
        out, ref = run_qmm(case, dtype, "qmv", guard=True)
    assert rel(out, ref) <= TOL[dtype], (M, K, N, dtype, gated)


def _nt_sweep_cases(n, seed):
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        K = int(g.choice([64, 128, 192, 512, 1024, 17, 40, 96 + 16]))      # K % 64 == 0: the dense route
        if K % 64 == 0 and g.integers(0, 2):
            K = 64 * int(g.integers(1, 40))
        M = int(g.choice([1, 3, int(g.integers(4, 65)), int(g.integers(65, 600))]))
        N = 16 * int(g.integers(1, 60))
        dtype = [torch.float32, torch.bfloat16, torch.float16][int(g.integers(0, 3))]
        cases.append((i, M, K, N, dtype, bool(g.integers(0, 2))))
    return cases


@pytest.mark.parametrize("i,M,K,N,dtype,with_gs", _nt_sweep_cases(24, 2026))
def test_qmm_non_transposed_random_sweep(i, M, K, N, dtype, with_gs):
    """Non-transposed planes through the binding: the dense copy and the
    matrix-core GEMM where K % 64 == 0, the generic kernel otherwise."""
    case = synth.dense_case(7300 + i, M, K, N, transpose=False, with_gs=with_gs)
    if dtype == torch.float16:   # keep f16 outputs finite
        case.scales = np.minimum(case.scales, 0x48).astype(np.uint8)
    out, ref = run_qmm(case, dtype, "auto", guard=True)
    assert rel(out, ref) <= TOL[dtype], (M, K, N, dtype)


def _gather_sweep(n, seed):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        K = int(g.choice([32, 256, 512, 2048, 48]))
        out.append((i, int(g.integers(1, 40)), int(g.integers(1, 12)), int(g.integers(1, 300)), K,
                    int(g.integers(1, 4)), bool(g.integers(0, 2)), int(g.integers(1, 4)),
                    [torch.float32, torch.bfloat16, torch.float16][int(g.integers(0, 3))]))
    return out


@pytest.mark.parametrize("i,tokens,E,N,K,top_k,sort,M,dtype", _gather_sweep(24, 2025))
def test_gather_random_sweep(i, tokens, E, N, K, top_k, sort, M, dtype):
    top_k = min(top_k, E)
    case = synth.gather_case(7500 + i, tokens=tokens, E=E, N=N, K=K, top_k=top_k, sort=sort, with_gs=bool(i % 2),
                             M=M, out_of_range=(E, 2 ** 31 - 1) if i % 3 == 0 else ())
    if dtype == torch.float16:
        case.scales = np.minimum(case.scales, 0x48).astype(np.uint8)
    out, ref = run_gather(case, dtype, guard=True)
    assert oracle.relative_error(host(out), ref) <= TOL[dtype], (tokens, E, N, K, top_k, M, dtype)
    assert_zero_rows(out, case.rhs, case.lhs, E, tokens)


# ----------------------------------------------------------------------------
# measurement aid
# ----------------------------------------------------------------------------

def test_stream_read_reads_every_chunk_and_writes_only_on_the_sentinel():
    """The benchmark's streaming-read aid (its own library, not libnvfp4)."""
    import os
    lib = ctypes.CDLL(os.path.join(os.path.dirname(nv.library_path()), "libnvfp4_measure.so"))
    lib.nvfp4_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_void_p]
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    zeros = torch.zeros(1 << 20, dtype=torch.int32, device=DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.nvfp4_stream_read(ctypes.c_void_p(zeros.data_ptr()), zeros.numel() * 4, 2048,
                                 ctypes.c_void_p(sink.data_ptr()), st) == 0
    torch.cuda.synchronize()
    assert int(sink[0]) == 0
    # the last 16-byte chunk folds to the sentinel: its lane stores it
    last = torch.zeros(1 << 20, dtype=torch.int32, device=DEV)
    last[-4] = int(np.array(0x9E3779B9, dtype=np.uint32).view(np.int32))
    assert lib.nvfp4_stream_read(ctypes.c_void_p(last.data_ptr()), last.numel() * 4, 2048,
                                 ctypes.c_void_p(sink.data_ptr()), st) == 0
    torch.cuda.synchronize()
    assert np.uint32(int(sink[0]) & 0xFFFFFFFF) == np.uint32(0x9E3779B9)


# ----------------------------------------------------------------------------
# HIP graph capture
# ----------------------------------------------------------------------------

def test_graph_capture_replays_match_eager():
    """Every entry point's kernels captured in one HIP graph (decode qmv,
    multi-row MFMA qmv, GEMM, split-K GEMM with its workspace, sorted and
    unsorted gather, fused and separate-projection gated projection,
    quantize with its zero fill and atomic maximum) and replayed three times
    on new inputs, with eager work and synchronizations in between: each
    replay equals the eager result bit for bit (all reductions here run in a
    fixed order)."""
    g = synth.rng(8100)
    K, N = 512, 768
    w = words(synth.packed_words(g, (N, K // 8)))
    s = u8(synth.scale_codes(g, (N, K // 16), (0x08, 0x30)))
    gs = f32(synth.global_scales(g, 1))
    wu = words(synth.packed_words(g, (N, K // 8)))
    su = u8(synth.scale_codes(g, (N, K // 16), (0x08, 0x30)))
    Ks, Ns = 2048, 4096
    ws_ = words(synth.packed_words(g, (Ns, Ks // 8)))
    ss_ = u8(synth.scale_codes(g, (Ns, Ks // 16), (0x08, 0x30)))
    assert int(nv.load_library().nvfp4_qmm_workspace_size(96, Ks, Ns, 1, 1, 0)) > 0   # split-K applies
    ge = synth.gather_case(8101, tokens=24, E=6, N=256, K=512, top_k=2, sort=True, with_gs=True)
    gu = synth.gather_case(8102, tokens=5, E=6, N=256, K=512, top_k=2, sort=False, with_gs=True)
    gw, gsc, ggs = words(ge.w), u8(ge.scales), f32(ge.gs)
    rs, ls = i32(ge.rhs), i32(ge.lhs)
    ru, lu = i32(gu.rhs), i32(gu.lhs)
    bufs = {
        "x1": torch.empty(1, K, dtype=torch.bfloat16, device=DEV),
        "x16": torch.empty(16, K, dtype=torch.bfloat16, device=DEV),
        "x300": torch.empty(300, K, dtype=torch.bfloat16, device=DEV),
        "x3f": torch.empty(3, K, dtype=torch.float32, device=DEV),
        "xs": torch.empty(96, Ks, dtype=torch.bfloat16, device=DEV),
        "xg": torch.empty(24, 1, 512, dtype=torch.bfloat16, device=DEV),
        "xgu": torch.empty(5, 1, 512, dtype=torch.bfloat16, device=DEV),
        "dense": torch.empty(64, 256, dtype=torch.bfloat16, device=DEV),
    }

    def fill(seed):
        gg = synth.rng(seed)
        for name, t in bufs.items():
            t.copy_(torch.from_numpy(synth.activations(gg, tuple(t.shape))).to(t.dtype))

    def run():
        return [
            nv.qmm(bufs["x1"], w, s, gs),
            nv.qmm(bufs["x16"], w, s, gs),
            nv.qmm(bufs["x300"], w, s, gs),
            nv.qmm(bufs["xs"], ws_, ss_, gs),
            nv.gather_qmm(bufs["xg"], gw, gsc, rs, ls, ggs, sorted_indices=True),
            nv.gather_qmm(bufs["xgu"], gw, gsc, ru, lu, ggs),
            nv.qmm_glu(bufs["x300"], w, s, gs, wu, su, None, act="gelu_tanh"),
            nv.qmm_glu(bufs["x3f"], w, s, gs, wu, su, gs, act="silu"),
        ] + list(nv.quantize(bufs["dense"]))

    fill(1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = run()
    for rep in range(3):
        fill(100 + rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = run()
        torch.cuda.synchronize()
        for i, (c, e) in enumerate(zip(captured, eager)):
            assert torch.equal(c, e), (rep, i)


# ----------------------------------------------------------------------------
# planes beyond 2 GiB
# ----------------------------------------------------------------------------

def test_plane_beyond_2gib():
    """A 2,147,614,720-byte word plane (N = 262160, K = 16384): the decode,
    multi-row and grouped kernels address planes with 32-bit buffer offsets
    and hand such a plane to the generic qmv kernel, whose offsets are 64-bit;
    the GEMM route uses 64-bit pointers.  Sampled weight rows (features are
    independent rows) against the oracle at M = 1, 16 (qmv route) and 300
    (GEMM route), outputs inside guard bands."""
    N, K = 262160, 16384
    assert N * K // 2 > 2 ** 31
    g = synth.rng(8200)
    w_np = synth.packed_words(g, (N, K // 8))
    s_np = synth.scale_codes(g, (N, K // 16), (0x08, 0x30))
    gs_np = synth.global_scales(g, 1)
    x_np = synth.activations(g, (300, K))
    w_t, s_t, gs_t = words(w_np), u8(s_np), f32(gs_np)
    rows = np.unique(np.concatenate([np.arange(0, N, 4099), [1, 63, 64, 131071, 131072, N - 17, N - 1]]))
    for M in (1, 16, 300):
        x_t, x_ref = activations(x_np[:M], torch.bfloat16)
        out, check = guarded((M, N), torch.bfloat16)
        nv.qmm(x_t, w_t, s_t, gs_t, out=out)
        torch.cuda.synchronize()
        check()
        ref = oracle.qmm(x_ref, w_np[rows], s_np[rows], gs_np[0])
        assert oracle.relative_error(host(out)[:, rows], ref) <= TOL[torch.bfloat16], M
        del out
    torch.cuda.empty_cache()
