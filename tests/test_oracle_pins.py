"""Pins for the CPU oracle, independent of the oracle itself.

Each test checks the oracle against something other than its own code:
the E2M1 table the pages print, a library FP8 decoder, exact rational
arithmetic (fractions.Fraction) with an independently written float32
rounding, byte identities, and exact zeros.  The mutation tests at the end
plant plausible mistakes in the oracle (on the CPU) and check that these
pins catch every one of them.
"""

import functools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import nvfp4_oracle as orc
import nvfp4_synth as synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# Independent helpers
# ----------------------------------------------------------------------------

def load_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def golden_e2m1():
    return {int(k): float(v) for k, v in load_table("e2m1_lut.txt")}


def golden_constants():
    return {k: float(v) for k, v in load_table("global_scale.txt")}


@functools.lru_cache(maxsize=None)
def torch_e4m3(code: int) -> float:
    """Library decode of one FP8 E4M3FN byte."""
    t = torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn)
    return float(t.to(torch.float64)[0])


def round_to_f32(q: Fraction) -> Fraction:
    """Round an exact rational to the nearest float32 (ties to even),
    written from the IEEE 754 definition rather than by calling a float
    conversion."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum_exp = max(e, -126) - 23          # 24 significant bits, subnormals below 2^-126
    quantum = Fraction(2) ** quantum_exp
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * quantum
    assert v <= Fraction(2) ** 128, "overflow"
    return sign * v


def f32_bits(values) -> np.ndarray:
    return np.ascontiguousarray(values, dtype=np.float32).view(np.uint32)


def words_from_nibbles(nibbles):
    """Pack a flat list of nibbles, element j of each word at bits 4j."""
    out = []
    for i in range(0, len(nibbles), 8):
        w = 0
        for j, n in enumerate(nibbles[i:i + 8]):
            w |= (n & 0xF) << (4 * j)
        out.append(w)
    return np.array(out, dtype=np.uint32)


def brute_dequant(w, scales, gs=None):
    """Element-by-element exact dequantize with Fraction; returns Fractions
    (or None for NaN) in a nested list [rows][elements]."""
    e2m1 = golden_e2m1()
    divisor = Fraction(int(golden_constants()["divisor"]))
    g = None if gs is None else round_to_f32(Fraction(float(np.float32(gs))) / divisor)
    rows = []
    for r in range(w.shape[0]):
        row = []
        for k in range(w.shape[1] * 8):
            word = int(w[r, k // 8])
            nib = (word >> (4 * (k % 8))) & 0xF
            s = torch_e4m3(int(scales[r, k // 16]))
            if math.isnan(s):
                row.append(None)
                continue
            v = Fraction(e2m1[nib]) * Fraction(s)
            if g is not None:
                v = round_to_f32(v * g)
            row.append(v)
        rows.append(row)
    return rows


def brute_zero_sign(w, scales, r, k):
    """Sign of a zero element: the product of the nibble's and the scale's
    signs (IEEE multiply of signed values)."""
    nib = (int(w[r, k // 8]) >> (4 * (k % 8))) & 0xF
    neg = (math.copysign(1.0, golden_e2m1()[nib]) < 0) != (math.copysign(1.0, torch_e4m3(int(scales[r, k // 16]))) < 0)
    return -0.0 if neg else 0.0


# ----------------------------------------------------------------------------
# Element decoders
# ----------------------------------------------------------------------------

def test_e2m1_matches_page_table():
    table = golden_e2m1()
    for nib in range(16):
        got = orc.e2m1_value(nib)
        assert got == table[nib] and math.copysign(1, got) == math.copysign(1, table[nib]), nib


def test_e4m3_matches_library_decoder_all_codes():
    for code in range(256):
        want = torch_e4m3(code)
        got = orc.e4m3_value(code)
        if math.isnan(want):
            assert math.isnan(got), code
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), hex(code)


def test_e4m3_spot_values_and_max():
    for code_hex, value in load_table("e4m3_spot.txt"):
        got = orc.e4m3_value(int(code_hex, 16))
        want = float(value)
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code_hex
    finite = [orc.e4m3_value(c) for c in range(256) if not math.isnan(orc.e4m3_value(c))]
    assert max(finite) == golden_constants()["e4m3_max"]
    assert max(abs(orc.e2m1_value(n)) for n in range(16)) == golden_constants()["e2m1_max"]


def test_nibble_order_low_first():
    w = np.array([[0x76543210, 0xFEDCBA98]], dtype=np.uint32)
    assert orc.unpack_nibbles(w).tolist() == [list(range(16))]


# ----------------------------------------------------------------------------
# Dequantize
# ----------------------------------------------------------------------------

def every_pair_plane():
    """256 rows (one per scale code), 16 elements per row = nibbles 0..15."""
    w = np.tile(words_from_nibbles(list(range(16))), (256, 1))
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    return w, scales


@pytest.mark.parametrize("gs", [None, 1.0, 777.25, 2688.0 * 3.5, 0.5, 1999.0])
def test_dequantize_every_nibble_and_code_bruteforce(gs):
    w, scales = every_pair_plane()
    got = orc.dequantize(w, scales, None if gs is None else np.float32(gs))
    assert got.dtype == np.float32
    want = brute_dequant(w, scales, gs)
    for r in range(256):
        for k in range(16):
            if want[r][k] is None:
                assert np.isnan(got[r, k])
                continue
            wv = np.float32(float(want[r][k]))
            if want[r][k] == 0:
                wv = np.float32(brute_zero_sign(w, scales, r, k))
            assert float(wv) == want[r][k]
            assert f32_bits(got[r, k]) == f32_bits(wv), (r, k, got[r, k], float(want[r][k]))


def test_dequantize_random_plane_bruteforce():
    g = synth.rng(11)
    w = synth.packed_words(g, (5, 6))          # 48 elements per row, 3 blocks
    sc = synth.scale_codes(g, (5, 3), synth.FINITE_POSITIVE_CODES)
    gs = synth.global_scales(g, 1)[0]
    for gsv in (None, gs):
        got = orc.dequantize(w, sc, gsv)
        want = brute_dequant(w, sc, gsv)
        for r in range(5):
            for k in range(48):
                assert Fraction(float(got[r, k])) == want[r][k]


def test_global_scale_of_2688_is_identity():
    w, scales = every_pair_plane()
    a = orc.dequantize(w, scales, None)
    b = orc.dequantize(w, scales, np.float32(2688.0))
    assert np.array_equal(f32_bits(a), f32_bits(b))


def test_dequantize_bf16_matches_library_rounding():
    g = synth.rng(12)
    w = synth.packed_words(g, (64, 16))
    sc = synth.scale_codes(g, (64, 8))
    gs = synth.global_scales(g, 1)[0]
    f = orc.dequantize(w, sc, gs)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.dequantize_bf16_bits(w, sc, gs)
    assert np.array_equal(got, want)


def test_bf16_rounding_matches_library():
    g = synth.rng(13)
    vals = np.concatenate([
        g.standard_normal(4096).astype(np.float32) * np.float32(1e3),
        np.array([0.0, -0.0, np.inf, -np.inf, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                  3.4e38, 1e-40, -1e-40], dtype=np.float32),
    ])
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.f32_to_bf16_bits(vals)
    assert np.array_equal(got, want)
    nan = orc.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(orc.bf16_bits_to_f32(nan)[0])
    back = orc.bf16_bits_to_f32(got)
    assert np.array_equal(back, torch.from_numpy(vals).to(torch.bfloat16).float().numpy())


def test_scale_plane_shape_is_checked():
    w = np.zeros((4, 4), dtype=np.uint32)
    with pytest.raises(ValueError):
        orc.dequantize(w, np.zeros((4, 3), dtype=np.uint8))
    with pytest.raises(ValueError):
        orc.dequantize(w, np.zeros((4, 2, 1), dtype=np.uint8))


# ----------------------------------------------------------------------------
# Quantized matmul
# ----------------------------------------------------------------------------

class Exact:
    """An exact dot product and the sum of its terms' magnitudes."""
    def __init__(self, terms):
        self.value = sum(terms, Fraction(0))
        self.mag = sum((abs(t) for t in terms), Fraction(0))

    def close(self, got, rel=Fraction(1, 2 ** 50)):
        """float64 summation error is bounded by K * eps * sum|terms|."""
        return abs(Fraction(float(got)) - self.value) <= self.mag * rel


def brute_qmm(x, w, scales, gs, transpose):
    W = brute_dequant(w, scales, gs)            # rows of the plane
    M = x.shape[0]
    if transpose:
        N, K = len(W), len(W[0])
        return [[Exact([Fraction(float(x[m, k])) * W[n][k] for k in range(K)]) for n in range(N)] for m in range(M)]
    K, N = len(W), len(W[0])
    return [[Exact([Fraction(float(x[m, k])) * W[k][n] for k in range(K)]) for n in range(N)] for m in range(M)]


@pytest.mark.parametrize("with_gs", [False, True])
def test_qmm_transposed_bruteforce(with_gs):
    c = synth.dense_case(21, M=2, K=32, N=3, transpose=True, with_gs=with_gs,
                         code_range=synth.FINITE_POSITIVE_CODES)
    gs = None if c.gs is None else c.gs[0]
    got = orc.qmm(c.x, c.w, c.scales, gs, transpose=True)
    want = brute_qmm(c.x, c.w, c.scales, gs, True)
    assert got.shape == (2, 3)
    for m in range(2):
        for n in range(3):
            assert want[m][n].close(got[m, n]), (m, n)


@pytest.mark.parametrize("with_gs", [False, True])
def test_qmm_nontransposed_k17_bruteforce(with_gs):
    c = synth.dense_case(22, M=3, K=17, N=32, transpose=False, with_gs=with_gs)
    assert c.w.shape == (17, 4) and c.scales.shape == (17, 2)
    gs = None if c.gs is None else c.gs[0]
    got = orc.qmm(c.x, c.w, c.scales, gs, transpose=False)
    want = brute_qmm(c.x, c.w, c.scales, gs, False)
    assert got.shape == (3, 32)
    for m in range(3):
        for n in range(32):
            assert want[m][n].close(got[m, n]), (m, n)


def test_qmm_one_hot_picks_a_dequantized_element():
    c = synth.dense_case(23, M=1, K=64, N=5, with_gs=True)
    W = brute_dequant(c.w, c.scales, c.gs[0])
    for k in (0, 7, 8, 15, 16, 63):
        x = np.zeros((1, 64), dtype=np.float32)
        x[0, k] = 1.0
        got = orc.qmm(x, c.w, c.scales, c.gs[0])
        for n in range(5):
            assert Fraction(float(got[0, n])) == W[n][k]


@pytest.mark.parametrize("broadcast_x", [False, True])
@pytest.mark.parametrize("transpose", [True, False])
def test_qmm_batched_bruteforce(broadcast_x, transpose):
    """Each weight matrix with its own global scale, against x[b] (or the
    one shared x), by exact rational arithmetic."""
    K = 32 if transpose else 5
    c = synth.batched_case(24, B=3, M=2, K=K, N=16, broadcast_x=broadcast_x, transpose=transpose,
                           with_gs=True)
    got = orc.qmm_batched(c.x, c.w, c.scales, c.gs, transpose=transpose)
    assert got.shape == (3, 2, 16)
    for b in range(3):
        src = 0 if broadcast_x else b
        want = brute_qmm(c.x[src], c.w[b], c.scales[b], c.gs[b], transpose)
        for m in range(2):
            for n in range(16):
                assert want[m][n].close(got[b, m, n]), (b, m, n)


def test_qmm_batched_empty_batch():
    c = synth.batched_case(25, B=1, M=2, K=32, N=16)
    got = orc.qmm_batched(c.x, c.w[:0], c.scales[:0], c.gs[:0])
    assert got.shape == (0, 2, 16)


# ----------------------------------------------------------------------------
# Quantize
# ----------------------------------------------------------------------------

def read_quantize_fixture():
    cases = []
    for line in open(os.path.join(GOLDEN, "quantize_rounding.txt")).read().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        gs, vals, code, nibs = [p.strip() for p in line.split("|")]
        cases.append((np.float32(gs), np.array([float(v) for v in vals.split()], dtype=np.float32),
                      int(code, 16), [int(n, 16) for n in nibs.split()]))
    return cases


def block_nibbles(words_row):
    """The 16 nibbles of one block, element j from bits [4j, 4j+4) of word j // 8."""
    return [(int(words_row[j // 8]) >> (4 * (j % 8))) & 0xF for j in range(16)]


def test_quantize_rounding_fixture():
    cases = read_quantize_fixture()
    assert len(cases) == 6
    for gs, vals, code, nibs in cases:
        w, sc, g = orc.quantize(vals.reshape(1, 16), gs=[gs])
        assert int(sc[0, 0]) == code, (gs, vals, hex(int(sc[0, 0])))
        assert block_nibbles(w[0]) == nibs, (gs, vals, block_nibbles(w[0]))
        assert g[0] == gs


def test_quantize_dequantize_round_trip_is_exact():
    """Planes whose every block holds a +-6 (so the block maximum is 6 times
    its scale) come back unchanged, signed zeros included, through
    dequantize -> quantize with the same global scale."""
    g = synth.rng(26)
    w = synth.packed_words(g, (2, 5, 8))                 # 2 matrices, 5 rows, 64 columns
    nib = [[[(int(w[b, r, c // 8]) >> (4 * (c % 8))) & 0xF for c in range(64)] for r in range(5)]
           for b in range(2)]
    for b in range(2):
        for r in range(5):
            for blk in range(4):
                c = blk * 16 + int(g.integers(0, 16))
                six = 0x7 | (nib[b][r][c] & 0x8)      # +6 or -6 somewhere in each block
                word = int(w[b, r, c // 8]) & ~(0xF << (4 * (c % 8))) | (six << (4 * (c % 8)))
                w[b, r, c // 8] = np.uint32(word)
    sc = synth.scale_codes(g, (2, 5, 4), synth.FINITE_POSITIVE_CODES)
    gs = synth.global_scales(g, 2)
    dense = np.stack([orc.dequantize(w[b], sc[b], gs[b]) for b in range(2)])
    w2, sc2, gs2 = orc.quantize(dense, gs=gs)
    assert np.array_equal(sc2, sc)
    assert np.array_equal(w2, w)
    assert np.array_equal(gs2, gs)


def test_quantize_picks_the_nearest_value_for_its_scale():
    """Every element's dequantized value is the closest of the 16 signed E2M1
    multiples of its block's dequantized scale (brute force), and the default
    global scale is the matrix's largest magnitude, which lands on code 448."""
    g = synth.rng(27)
    dense = (synth.activations(g, (3, 64)) * np.float32(7.5)).astype(np.float32)
    w, sc, gs = orc.quantize(dense)
    assert gs[0] == np.abs(dense).max()
    assert int(sc.max()) == 0x7E
    back = orc.dequantize(w, sc, gs[0])
    gf = Fraction(float(orc.global_factor(gs[0])))
    for r in range(3):
        for c in range(64):
            d = Fraction(float(np.float32(Fraction(float(orc.e4m3_value(int(sc[r, c // 16])))) * gf)))
            x = Fraction(float(dense[r, c]))
            best = min(abs(x - sgn * Fraction(m) * d) for m in orc.E2M1_MAGNITUDES for sgn in (1, -1))
            got = abs(x - Fraction(float(back[r, c])))
            # the dequantized value rounds fl32(e2m1 * e4m3) * g once more: allow one f32 ulp of it
            assert got <= best + abs(Fraction(float(back[r, c]))) * Fraction(1, 2 ** 23), (r, c)


def test_quantize_all_zero_matrix():
    w, sc, gs = orc.quantize(np.zeros((2, 32), dtype=np.float32))
    assert gs[0] == 0 and not sc.any() and not w.any()
    w, sc, gs = orc.quantize(np.full((1, 16), -0.0, dtype=np.float32))
    assert w[0, 0] == 0x88888888 and w[0, 1] == 0x88888888 and sc[0, 0] == 0


# ----------------------------------------------------------------------------
# Gather
# ----------------------------------------------------------------------------

def test_gather_rows_and_out_of_range_zeros():
    c = synth.gather_case(31, tokens=3, E=4, N=5, K=32, top_k=2, sort=False,
                          with_gs=True, M=2, out_of_range=(4, 5, 2 ** 31 - 1, -1))
    lhs = c.lhs.copy()
    lhs[1] = 3                      # lhs outside [0, X) as well
    got = orc.gather_qmm(c.x, lhs, c.rhs, c.w, c.scales, c.gs)
    assert got.shape == (6, 2, 5)
    for r in range(6):
        e, src = int(c.rhs[r]), int(lhs[r])
        if not (0 <= e < 4) or not (0 <= src < 3):
            assert np.all(got[r] == 0.0) and not np.any(np.signbit(got[r])), r
            continue
        want = brute_qmm(c.x[src], c.w[e], c.scales[e], c.gs[e], True)
        for m in range(2):
            for n in range(5):
                assert want[m][n].close(got[r, m, n]), (r, m, n)
    zero_rows = [r for r in range(6) if not (0 <= int(c.rhs[r]) < 4) or not (0 <= int(lhs[r]) < 3)]
    assert len(zero_rows) >= 4


# ----------------------------------------------------------------------------
# Transcode
# ----------------------------------------------------------------------------

def test_transcode_is_a_byte_move():
    g = synth.rng(41)
    wu8, ws, ws2 = synth.modelopt_triplet(g, 2, 8, 64)
    words, scales, gs = orc.transcode(wu8, ws, ws2)
    assert words.shape == (2, 8, 8) and words.dtype == np.uint32
    # On a little-endian host the word plane viewed as bytes is the source.
    assert np.array_equal(words.astype("<u4").view(np.uint8).reshape(wu8.shape), wu8)
    assert np.array_equal(scales, ws)
    assert gs.dtype == np.float32 and gs.shape == (2,)


def test_transcode_reconstructs_source_weights():
    """Dequantizing the transcoded planes gives e2m1 * weight_scale *
    weight_scale_2 of the source within a few float32 roundings."""
    g = synth.rng(42)
    wu8, ws, ws2 = synth.modelopt_triplet(g, 3, 4, 32)
    words, scales, gs = orc.transcode(wu8, ws, ws2)
    e2m1 = golden_e2m1()
    for b in range(3):
        deq = orc.dequantize(words[b], scales[b], gs[b])
        for r in range(4):
            for k in range(32):
                byte = int(wu8[b, r, k // 2])
                nib = byte & 0xF if k % 2 == 0 else byte >> 4
                want = Fraction(e2m1[nib]) * Fraction(torch_e4m3(int(ws[b, r, k // 16]))) * Fraction(float(ws2[b]))
                got = Fraction(float(deq[r, k]))
                assert abs(got - want) <= abs(want) * Fraction(3, 2 ** 24), (b, r, k)


def test_transcode_without_second_scale():
    g = synth.rng(43)
    wu8, ws, _ = synth.modelopt_triplet(g, 1, 2, 16, with_ws2=False)
    words, scales, gs = orc.transcode(wu8, ws, None)
    assert gs is None and words.shape == (1, 2, 2)


# ----------------------------------------------------------------------------
# Direct transcode against the dense-f16 requantization path (P1 "Acceptance
# criteria", third bullet, and "Implementation plan" step 4)
# ----------------------------------------------------------------------------

def dense_requantization(w, scales, gs):
    """P1's conservative load path, restated with the oracle: reconstruct the
    dense weights in float16 (round to nearest even of the direct path's
    dequantized float32 values), quantize them again (the global scale is
    the matrix maximum) and dequantize the result."""
    w16 = orc.dequantize(w, scales, gs).astype(np.float16)
    qw, qs, qg = orc.quantize(w16.astype(np.float32))
    return w16, qw, qs, qg, orc.dequantize(qw, qs, qg[0])


def fp8_rounding_bound(w16, gs_new):
    """Largest |dense - direct| the requantization can cause, per element
    (the reading documented with the fixture): for a 16-block whose largest
    |value| is a, the requantized E4M3 block scale is within 1/16 of
    a * 448 / gs (or 2^-10 absolute where that is subnormal), so its step
    d = e4m3 * gs / 2688 is at most (17/16) a / 6 + 2^-10 g; each element
    moves by at most one such step (half the widest E2M1 gap, 4 to 6), or by
    a / 16 + 6 * 2^-10 g where it saturates, plus the float16 rounding of the
    reconstruction (2^-11 relative, 2^-25 absolute below 2^-14).  With
    g = gs / 2688: (17/96) a + 2^-7 g + 2^-10 a + 2^-24."""
    a = np.abs(w16.astype(np.float64)).reshape(w16.shape[:-1] + (-1, 16)).max(axis=-1)
    g = float(gs_new) / 2688.0
    per_block = (17.0 / 96.0) * a + 2.0 ** -7 * g + 2.0 ** -10 * a + 2.0 ** -24
    return np.repeat(per_block, 16, axis=-1)


def test_direct_transcode_equals_dense_path_when_scales_round_trip():
    """Every 16-block holds a +-6 nibble, the largest block code is 448 and the
    second-level scale is a power of two: then the float16 reconstruction is
    exact, its maximum is 6 * 448 * ws2, every requantized block scale lands
    on the source code and every element on the source nibble, so the dense
    path gives the direct planes and sidecar bit for bit (signed zeros
    included)."""
    g = synth.rng(7100)
    weight, scale, _ = synth.modelopt_triplet(g, 1, 24, 256)
    weight, scale = weight[0].copy(), scale[0].copy()
    nib = np.stack([weight & 0xF, weight >> 4], axis=-1).reshape(24, 256)
    blocks = nib.reshape(24, 16, 16)
    pos = g.integers(0, 16, size=(24, 16))
    sign = g.integers(0, 2, size=(24, 16)) * 8
    np.put_along_axis(blocks, pos[..., None], (7 | sign)[..., None], axis=-1)
    nib = blocks.reshape(24, 128, 2)
    weight = (nib[..., 0] | (nib[..., 1] << 4)).astype(np.uint8)
    scale[5, 3] = 0x7E
    ws2 = np.array([2.0 ** -10], dtype=np.float32)
    w, s, gs = orc.transcode(weight, scale, ws2)
    direct = orc.dequantize(w, s, gs[0])
    w16, qw, qs, qg, dense = dense_requantization(w, s, gs[0])
    assert np.array_equal(w16.astype(np.float32).view(np.uint32), direct.view(np.uint32))
    assert np.array_equal(qs, s) and np.array_equal(qw, w)
    assert qg.view(np.uint32)[0] == gs.view(np.uint32)[0]
    assert np.array_equal(dense.view(np.uint32), direct.view(np.uint32))


def test_direct_transcode_against_dense_path_within_fp8_rounding():
    """Random triplets (uniform nibbles, normal block codes, log-uniform
    second-level scale): the dense path differs from the direct transcode by
    no more than the FP8 scale-rounding bound, element by element, and the
    bound is not vacuous (a few blocks' scales do change)."""
    for seed in (7110, 7111, 7112):
        g = synth.rng(seed)
        weight, scale, ws2 = synth.modelopt_triplet(g, 1, 32, 256)
        w, s, gs = orc.transcode(weight[0], scale[0], ws2)
        direct = orc.dequantize(w, s, gs[0]).astype(np.float64)
        w16, qw, qs, qg, dense = dense_requantization(w, s, gs[0])
        err = np.abs(dense.astype(np.float64) - direct)
        assert np.all(err <= fp8_rounding_bound(w16, qg[0])), seed
        assert np.any(err > 0), seed
        # a plain error check that a dropped global scale would fail
        assert orc.relative_error(dense, direct) <= 0.2


# ----------------------------------------------------------------------------
# Gated MLP projection
# ----------------------------------------------------------------------------

# The standard normal distribution function at a few points, as printed in
# tables of Phi.
PHI_TABLE = {0.0: 0.5, 1.0: 0.8413447460685429, -1.0: 0.15865525393145707,
             2.0: 0.9772498680518208, -2.5: 0.006209665325776132, 3.0: 0.9986501019683699}


def test_gelu_is_z_times_the_normal_distribution_function():
    for z, phi in PHI_TABLE.items():
        got = float(orc.glu_activation(np.array([z]), "gelu")[0])
        assert abs(got - z * phi) <= 1e-15 * max(1.0, abs(z)), z
    from scipy.stats import norm
    zs = np.linspace(-12.0, 12.0, 481)
    assert np.allclose(orc.glu_activation(zs, "gelu"), zs * norm.cdf(zs), rtol=1e-13, atol=1e-300)


def library_activation(z, act):
    t = torch.as_tensor(np.asarray(z, dtype=np.float64))
    if act == "gelu":
        return torch.nn.functional.gelu(t, approximate="none").numpy()
    if act == "gelu_tanh":
        return torch.nn.functional.gelu(t, approximate="tanh").numpy()
    return torch.nn.functional.silu(t).numpy()


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh", "silu"])
def test_activations_match_library_routines(act):
    zs = np.concatenate([np.linspace(-30.0, 30.0, 2401), [-700.0, -88.0, 1e-300, -1e-300, 0.0, 88.0, 700.0]])
    got = orc.glu_activation(zs, act)
    want = library_activation(zs, act)
    # torch forms the erf GELU as 1 + erf(z / sqrt 2), which cancels to 0
    # below z ~ -8.3 (true values < 1e-16): an absolute floor covers that tail.
    assert np.allclose(got, want, rtol=1e-13, atol=1e-15), act


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh", "silu"])
def test_activation_odd_part_is_the_identity(act):
    """act(z) = z * c(z) with c(-z) = 1 - c(z) for all three, so
    act(z) - act(-z) = z."""
    zs = np.linspace(-9.0, 9.0, 361)
    d = orc.glu_activation(zs, act) - orc.glu_activation(-zs, act)
    assert np.allclose(d, zs, rtol=1e-14, atol=1e-14)


def test_gelu_forms_differ():
    """The tanh form is an approximation: close to the erf form, not equal."""
    zs = np.linspace(-5.0, 5.0, 201)
    d = np.abs(orc.glu_activation(zs, "gelu") - orc.glu_activation(zs, "gelu_tanh"))
    assert 1e-5 < d.max() < 1e-3


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh", "silu"])
def test_qmm_glu_bruteforce(act):
    """Gate and up planes with their own global scales: exact rational
    projections, the library activation on the gate, times the up."""
    g = synth.dense_case(25, M=2, K=32, N=3, with_gs=True, code_range=synth.FINITE_POSITIVE_CODES)
    u = synth.dense_case(26, M=2, K=32, N=3, with_gs=True, code_range=synth.FINITE_POSITIVE_CODES)
    got = orc.qmm_glu(g.x, g.w, g.scales, g.gs[0], u.w, u.scales, u.gs[0], act)
    gate = brute_qmm(g.x, g.w, g.scales, g.gs[0], True)
    up = brute_qmm(g.x, u.w, u.scales, u.gs[0], True)
    assert got.shape == (2, 3)
    want = np.zeros((2, 3))
    for m in range(2):
        for f in range(3):
            a = library_activation(np.array([float(gate[m][f].value)]), act)[0]
            want[m, f] = a * float(up[m][f].value)
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want)), (got, want)


def test_qmm_glu_without_global_scales_and_shape_check():
    g = synth.dense_case(27, M=1, K=16, N=2, with_gs=False)
    u = synth.dense_case(28, M=1, K=16, N=2, with_gs=False)
    got = orc.qmm_glu(g.x, g.w, g.scales, None, u.w, u.scales, None, "silu")
    gate = orc.qmm(g.x, g.w, g.scales)
    up = orc.qmm(g.x, u.w, u.scales)
    assert np.allclose(got, gate / (1.0 + np.exp(-gate)) * up, rtol=1e-15, atol=0)
    with pytest.raises(ValueError):
        orc.qmm_glu(g.x, g.w, g.scales, None, u.w[:1], u.scales[:1], None, "silu")


def test_relative_error_metric():
    ref = np.array([1.0, -4.0, 2.0])
    out = np.array([1.0, -4.5, 2.0])
    assert orc.relative_error(out, ref) == 0.125


# ----------------------------------------------------------------------------
# Mutation checks: plausible mistakes planted in the oracle must be caught.
# ----------------------------------------------------------------------------

PIN_TESTS = [
    test_e2m1_matches_page_table,
    test_e4m3_matches_library_decoder_all_codes,
    test_nibble_order_low_first,
    lambda: test_dequantize_every_nibble_and_code_bruteforce(777.25),
    test_dequantize_random_plane_bruteforce,
    lambda: test_qmm_transposed_bruteforce(True),
    lambda: test_qmm_nontransposed_k17_bruteforce(True),
    test_gather_rows_and_out_of_range_zeros,
    lambda: test_qmm_batched_bruteforce(False, True),
    lambda: test_qmm_batched_bruteforce(True, False),
    test_quantize_rounding_fixture,
    test_quantize_dequantize_round_trip_is_exact,
    test_transcode_reconstructs_source_weights,
    lambda: test_qmm_glu_bruteforce("gelu_tanh"),
    lambda: test_activations_match_library_routines("gelu_tanh"),
    lambda: test_activations_match_library_routines("gelu"),
    lambda: test_activations_match_library_routines("silu"),
]


def caught(monkeypatch_fn):
    """True when at least one pin fails with the mutation in place."""
    for t in PIN_TESTS:
        try:
            t()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


def _mut_e4m3_bias(code):
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return float("nan")
    return s * (m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 8))


def _mut_e4m3_nan(code):
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    return s * (m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))


def _mut_nibble_order(words):
    words = np.asarray(words, dtype=np.uint32)
    shifts = (7 - np.arange(8, dtype=np.uint32)) * np.uint32(4)
    nib = (words[..., None] >> shifts) & np.uint32(0xF)
    return nib.reshape(words.shape[:-1] + (words.shape[-1] * 8,)).astype(np.uint8)


def _mut_sign(n):
    mag = orc.E2M1_MAGNITUDES[n & 7]
    return mag


def _mut_qmm_transpose(x, w, scales, gs=None, transpose=True):
    W = orc.dequantize(w, scales, gs).astype(np.float64)
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    if transpose:
        return x64 @ W.T
    return (x64 @ W[::-1]) if W.shape[0] > 1 else x64 @ W


def _mut_gather_no_zero(x, lhs, rhs, w, scales, gs):
    R = rhs.shape[0]
    out = np.zeros((R, x.shape[1], w.shape[1]))
    for r in range(R):
        e = int(rhs[r]) % w.shape[0]
        src = (int(lhs[r]) if lhs is not None else r) % x.shape[0]
        out[r] = orc.qmm(x[src], w[e], scales[e], None if gs is None else gs[e])
    return out


def _mut_batched_x0(x, w, scales, gs=None, transpose=True):
    return np.stack([orc.qmm(x[0], w[b], scales[b], None if gs is None else gs[b], transpose=transpose)
                     for b in range(w.shape[0])])


def _mut_batched_gs0(x, w, scales, gs=None, transpose=True):
    return np.stack([orc.qmm(x[0] if x.shape[0] == 1 else x[b], w[b], scales[b],
                             None if gs is None else gs[0], transpose=transpose)
                     for b in range(w.shape[0])])


def _mut_e2m1_ties_away(value):
    v = float(value)
    sign = 8 if np.signbit(np.float32(v)) else 0
    a = abs(v)
    best, best_d = 0, None
    for i, c in enumerate(orc.E2M1_MAGNITUDES):
        d = abs(a - c)
        if best_d is None or d <= best_d:          # ties go up
            best, best_d = i, d
    return sign | best


def _mut_e4m3_truncate(value):
    v = float(value)
    if v != v:
        return 0x7F
    best = 0
    for c in range(0x7F):
        if orc.e4m3_value(c) <= v:
            best = c
    return best


def _mut_glu_act_on_up(x, w_gate, s_gate, gs_gate, w_up, s_up, gs_up, act):
    gate = orc.qmm(x, w_gate, s_gate, gs_gate)
    up = orc.qmm(x, w_up, s_up, gs_up)
    return gate * orc.glu_activation(up, act)


def _mut_glu_shared_gs(x, w_gate, s_gate, gs_gate, w_up, s_up, gs_up, act):
    gate = orc.qmm(x, w_gate, s_gate, gs_gate)
    up = orc.qmm(x, w_up, s_up, gs_gate)
    return orc.glu_activation(gate, act) * up


_glu_activation = orc.glu_activation


def _mut_gelu_tanh_no_cubic(z, act):
    if act == "gelu_tanh":
        z = np.asarray(z, dtype=np.float64)
        return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * z))
    return _glu_activation(z, act)


def _mut_silu_sigmoid_only(z, act):
    if act == "silu":
        return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))
    return _glu_activation(z, act)


def _mut_gelu_no_sqrt2(z, act):
    if act == "gelu":
        z = np.asarray(z, dtype=np.float64)
        return 0.5 * z * np.vectorize(math.erfc)(-z)
    return _glu_activation(z, act)


MUTATIONS = {
    "quantize E2M1 ties away from zero": ("e2m1_round", _mut_e2m1_ties_away),
    "quantize E4M3 scale truncated": ("e4m3_round", _mut_e4m3_truncate),
    "quantize scale range 6 instead of 448": ("E4M3_MAX", 6.0),
    "batched x always matrix 0": ("qmm_batched", _mut_batched_x0),
    "batched global scale of matrix 0": ("qmm_batched", _mut_batched_gs0),
    "e4m3 exponent bias 8": ("e4m3_value", _mut_e4m3_bias),
    "e4m3 no NaN code": ("e4m3_value", _mut_e4m3_nan),
    "nibble order high first": ("unpack_nibbles", _mut_nibble_order),
    "e2m1 sign dropped": ("e2m1_value", _mut_sign),
    "global divisor 448": ("GLOBAL_DIVISOR", 448.0),
    "global divisor 6": ("GLOBAL_DIVISOR", 6.0),
    "E2M1 table swapped": ("E2M1_MAGNITUDES", (0.0, 0.5, 1.0, 1.5, 2.0, 4.0, 3.0, 6.0)),
    "non-transposed operand reversed": ("qmm", _mut_qmm_transpose),
    "gather out-of-range wraps": ("gather_qmm", _mut_gather_no_zero),
    "glu activation on the up projection": ("qmm_glu", _mut_glu_act_on_up),
    "glu up projection with the gate's global scale": ("qmm_glu", _mut_glu_shared_gs),
    "gelu tanh form without the cubic term": ("glu_activation", _mut_gelu_tanh_no_cubic),
    "silu as the sigmoid alone": ("glu_activation", _mut_silu_sigmoid_only),
    "gelu erf argument not divided by sqrt 2": ("glu_activation", _mut_gelu_no_sqrt2),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, value = MUTATIONS[name]
    monkeypatch.setattr(orc, attr, value)
    assert caught(monkeypatch), f"no pin caught: {name}"
