"""Plain CPU oracle for NVFP4 quantized matmul.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
constants with the HIP library; it is written from the pages' description
of the format and is deliberately slow and literal.

Sources (pages as published on the web):

* P1 = mlxcel issue "perf(nvfp4): direct-transcode ModelOpt triplets to
  MLX native" -- sections "Technical notes" (packing, E2M1 table, E4M3 block
  scales of 16, little-endian words) and "Implementation plan" (four source
  bytes become one word; weight_scale kept as E4M3 bytes; weight_scale_2
  kept as a global-scale sidecar).
* P3 = mlxcel PR "native NVFP4 for ROCm QuantizedMatmul/GatherQMM" --
  "Summary" (global_scale[expert] / (448 * 6) applied once per output;
  GatherQMM over experts), "Numerical results" (the reference is
  ``x @ dequantize(w).T`` on the CPU, error = max abs error relative to
  max|reference|), "Changes during review" (quantized-axis rule, partial
  blocks, out-of-range experts give exact zeros, scale-plane shape) and
  "Implementation Review Summary / Verification" (fp_dequantize multiplies
  by global_scale / (448 * 6)).

Readings where the pages are silent (each listed in the design notes):

* element j of a packed word sits at bits [4j, 4j+4) (low nibble first);
* the E2M1 sign is nibble bit 3;
* "FP8 E4M3" is the OCP E4M3FN encoding (bias 7, subnormals, no infinity,
  NaN only at S.1111.111) -- 448, its largest finite value, is the constant
  the pages divide by;
* the sidecar written by transcode is gs = fl32(weight_scale_2 * 2688), so
  that gs / 2688 restores weight_scale_2 (to one f32 rounding);
* g = fl32(gs / 2688) is formed once in float32 and each dequantized value is
  fl32(e2m1 * e4m3 * g) -- float32 is the precision the pages fix for the
  global scale and for the dequantized reference;
* the contraction is carried out in float64 (stricter than the pages' f32
  reference) so the oracle's own rounding does not eat the error budget;
* gather rows whose expert or lhs index is out of range are +0.0;
* quantize takes each matrix's largest |w| as its global scale unless one is
  given, rounds the block scale amax * 448 / gs to E4M3 and each w / d to
  E2M1 by round-to-nearest-even in float32 (saturating at 448 and 6), and
  keeps the sign of values that round to zero;
* the gated MLP projection of P2 ("Hypothesis", "Activation-path
  follow-up": the scaled gate/up MLP of the Gemma and Llama 4 paths with its
  GeGLU activation) is act(x @ Wg.T) * (x @ Wu.T), each plane with its own
  global scale, the activation applied to the gate projection; the pages do
  not define the activation, so the oracle offers GELU in its erf form, the
  tanh approximation that Gemma's GeGLU uses, and SiLU (Llama's SwiGLU).

Every function below works on numpy arrays; bf16 tensors are represented as
their uint16 bit patterns.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np

# P1 "Technical notes": E2M1 magnitudes in LUT order, with a sign bit.
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)

# P3 "Summary" / "Verification": the global scale is divided by 448 * 6
# (448 = largest E4M3 value, 6 = largest E2M1 value).
GLOBAL_DIVISOR = 448.0 * 6.0

# P1 "Technical notes": one E4M3 scale per 16 elements, eight nibbles per word.
GROUP_SIZE = 16
NIBBLES_PER_WORD = 8


# ----------------------------------------------------------------------------
# Element decoders
# ----------------------------------------------------------------------------

def e2m1_value(nibble: int) -> float:
    """Value of one FP4 E2M1 nibble (P1 "Technical notes": LUT order 0, 0.5,
    1, 1.5, 2, 3, 4, 6 plus a sign bit; sign read as bit 3)."""
    magnitude = E2M1_MAGNITUDES[nibble & 7]
    return -magnitude if nibble & 8 else magnitude


def e4m3_value(code: int) -> float:
    """Value of one FP8 E4M3 byte (P1 "Technical notes": the block scales are
    "uint8 FP8 E4M3"), decoded as OCP E4M3FN: sign bit 7, exponent bits 6..3
    with bias 7, mantissa bits 2..0, subnormals at exponent 0, NaN at
    exponent 15 with mantissa 7, no infinities."""
    sign = -1.0 if code & 0x80 else 1.0
    exponent = (code >> 3) & 0xF
    mantissa = code & 0x7
    if exponent == 0xF and mantissa == 0x7:
        return float("nan")
    if exponent == 0:
        return sign * mantissa * 2.0 ** -9          # (m / 8) * 2^(1 - 7)
    return sign * (1.0 + mantissa / 8.0) * 2.0 ** (exponent - 7)


def decode_e2m1(nibbles: np.ndarray) -> np.ndarray:
    """Vectorised :func:`e2m1_value` over an integer array (float64 out)."""
    table = np.array([e2m1_value(n) for n in range(16)], dtype=np.float64)
    return table[np.asarray(nibbles, dtype=np.int64)]


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """Vectorised :func:`e4m3_value` over a uint8 array (float64 out)."""
    table = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.int64)]


def unpack_nibbles(words: np.ndarray) -> np.ndarray:
    """Split uint32 words into their eight nibbles along a new last axis,
    element j taken from bits [4j, 4j+4); the result's last axis is 8x the
    input's (P1 "Technical notes": eight nibbles per uint32 word)."""
    words = np.asarray(words, dtype=np.uint32)
    shifts = np.arange(NIBBLES_PER_WORD, dtype=np.uint32) * np.uint32(4)
    nibbles = (words[..., None] >> shifts) & np.uint32(0xF)
    return nibbles.reshape(words.shape[:-1] + (words.shape[-1] * NIBBLES_PER_WORD,)).astype(np.uint8)


# ----------------------------------------------------------------------------
# bf16 helpers (bit patterns in uint16)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(values: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and return
    the uint16 bit patterns.  NaN maps to a quiet NaN of the same sign."""
    f = np.ascontiguousarray(values, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    rounded = ((bits + np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    out[nan] = ((bits[nan] >> np.uint64(16)).astype(np.uint16) | np.uint16(0x0040))
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


# ----------------------------------------------------------------------------
# Global scale
# ----------------------------------------------------------------------------

def global_factor(gs) -> np.float32:
    """Per-output factor g = global_scale / (448 * 6), formed once in float32
    (P3 "Summary": applied once per output; "Verification": fp_dequantize
    multiplies by global_scale / (448 * 6))."""
    return np.float32(np.float32(gs) / np.float32(GLOBAL_DIVISOR))


# ----------------------------------------------------------------------------
# Dequantize
# ----------------------------------------------------------------------------

def check_planes(w: np.ndarray, scales: np.ndarray) -> None:
    """The scale plane must be shaped w.shape[:-1] + [w.shape[-1] / 2] with one
    byte per scale (P3 "Changes during review", scale-plane check)."""
    if w.dtype != np.uint32 or scales.dtype != np.uint8:
        raise ValueError("w must be uint32 and scales uint8")
    if w.shape[-1] % 2 != 0 or scales.shape != w.shape[:-1] + (w.shape[-1] // 2,):
        raise ValueError(f"scale plane {scales.shape} does not match weight plane {w.shape}")


def dequantize(w: np.ndarray, scales: np.ndarray, gs=None) -> np.ndarray:
    """Expand a packed plane along its last (quantized) axis to float32.

    value = e2m1(nibble) * e4m3(scale of its 16-block), which is exact in
    float32; with a global scale, value = fl32(value * g), g = fl32(gs/2688)
    (P1 "Technical notes"; P3 "Summary": the dequantize kernel expands a plane
    exactly; P3 "Verification": the global-scale multiply).
    """
    check_planes(w, scales)
    elements = decode_e2m1(unpack_nibbles(w))                      # [..., 8W]
    block = decode_e4m3(scales)                                    # [..., 8W/16]
    block = np.repeat(block, GROUP_SIZE, axis=-1)                  # one per element
    exact = (elements * block).astype(np.float32)                  # exact product
    if gs is None:
        return exact
    return (exact * global_factor(gs)).astype(np.float32)


def dequantize_bf16_bits(w: np.ndarray, scales: np.ndarray, gs=None) -> np.ndarray:
    """Dequantize, then round the float32 values to bf16 (uint16 bits)."""
    return f32_to_bf16_bits(dequantize(w, scales, gs))


# ----------------------------------------------------------------------------
# Quantize (dense -> planes + global scale)
# ----------------------------------------------------------------------------

# Largest finite E4M3 value: the block-scale range the global scale maps the
# matrix maximum onto (P3 "Summary": block scales are encoded as scale times
# 448 * 6 / global_scale).
E4M3_MAX = 448.0


def _nearest_code(value: float, candidates) -> int:
    """Index of the candidate nearest to value; on a tie the even index (the
    one whose lowest mantissa bit is 0): round to nearest, ties to even."""
    best, best_d = 0, None
    for i, c in enumerate(candidates):
        d = abs(value - c)
        if best_d is None or d < best_d or (d == best_d and i % 2 == 0):
            best, best_d = i, d
    return best


_E4M3_FINITE = [e4m3_value(c) for c in range(0x7F)]       # codes 0x00 .. 0x7E, increasing


def e4m3_round(value: float) -> int:
    """E4M3 code of a non-negative float32 value: the nearest finite E4M3
    value, ties to the even code, above 448 saturating to 448; NaN gives the
    NaN code 0x7F."""
    v = float(value)
    if v != v:
        return 0x7F
    if v >= E4M3_MAX:
        return 0x7E
    return _nearest_code(v, _E4M3_FINITE)


def e2m1_round(value: float) -> int:
    """E2M1 nibble of a float32 value: the nearest of 0, 0.5, 1, 1.5, 2, 3, 4,
    6 in magnitude, ties to the even index, above 6 saturating to 6; the sign
    bit (nibble bit 3) is the value's sign bit, so a negative value that
    rounds to zero gives -0."""
    v = float(value)
    sign = 8 if np.signbit(np.float32(v)) else 0
    a = abs(v)
    if a >= E2M1_MAGNITUDES[-1]:
        return sign | 7
    return sign | _nearest_code(a, E2M1_MAGNITUDES)


def quantize(w: np.ndarray, gs=None):
    """Dense float32 matrices -> (words, scale codes, global scales), quantized
    along the last axis in blocks of 16 (P1 "Technical notes": E2M1 values,
    one E4M3 scale per 16 elements, eight nibbles per little-endian word;
    P3 "Summary": the block scales are encoded as scale times 448 * 6 /
    global_scale, and dequantize multiplies by global_scale / (448 * 6)).

    w is [..., rows, cols] (cols % 16 == 0); gs is None (then gs of each
    matrix is its largest |w|) or one float32 per matrix.  In float32, per
    16-block with largest magnitude a:

    * code = E4M3 nearest (ties to even, saturating) of fl32(a * fl32(448 / gs)),
      0 when a or gs is 0;
    * d = fl32(e4m3(code) * fl32(gs / 2688)), the block's dequantized scale;
    * nibble = E2M1 nearest (ties to even, saturating, signed) of fl32(w / d),
      or just the sign of w when d is 0 or NaN.

    Returns uint32 [..., rows, cols/8], uint8 [..., rows, cols/16] and
    float32 [batch] (batch = product of the leading axes).
    """
    W = np.ascontiguousarray(w, dtype=np.float32)
    if W.ndim < 2 or W.shape[-1] % GROUP_SIZE != 0:
        raise ValueError("w must be [..., rows, cols] with cols a multiple of 16")
    lead = W.shape[:-2]
    rows, cols = W.shape[-2], W.shape[-1]
    mats = W.reshape((-1, rows, cols))
    batch = mats.shape[0]
    if gs is None:
        gsv = np.array([np.abs(m).max() if m.size else 0.0 for m in mats], dtype=np.float32)
    else:
        gsv = np.asarray(gs, dtype=np.float32).reshape(batch)
    words = np.zeros((batch, rows, cols // NIBBLES_PER_WORD), dtype=np.uint32)
    codes = np.zeros((batch, rows, cols // GROUP_SIZE), dtype=np.uint8)
    for b in range(batch):
        g_b = gsv[b]
        t = np.float32(np.float32(E4M3_MAX) / g_b) if g_b != 0 else np.float32(0)
        g = global_factor(g_b)
        for r in range(rows):
            for k in range(cols // GROUP_SIZE):
                block = mats[b, r, k * GROUP_SIZE:(k + 1) * GROUP_SIZE]
                a = np.float32(np.abs(block).max())
                if a == 0 or g_b == 0:
                    code = 0
                else:
                    code = e4m3_round(np.float32(a * t))
                codes[b, r, k] = code
                d = np.float32(np.float32(e4m3_value(code)) * g)
                for j, v in enumerate(block):
                    if d == 0 or d != d:
                        nib = 8 if np.signbit(v) else 0
                    else:
                        nib = e2m1_round(np.float32(v / d))
                    col = k * GROUP_SIZE + j
                    words[b, r, col // NIBBLES_PER_WORD] |= np.uint32(nib) << np.uint32(4 * (col % NIBBLES_PER_WORD))
    return (words.reshape(lead + (rows, cols // NIBBLES_PER_WORD)),
            codes.reshape(lead + (rows, cols // GROUP_SIZE)), gsv)


# ----------------------------------------------------------------------------
# Quantized matmul
# ----------------------------------------------------------------------------

def qmm(x: np.ndarray, w: np.ndarray, scales: np.ndarray, gs=None,
        transpose: bool = True) -> np.ndarray:
    """Reference quantized matmul (P3 "Numerical results": x @ dequantize(w).T
    on the CPU).

    transpose=True: w is [N, K/8] quantized along K, out = x @ W.T.
    transpose=False: w is [K, N/8] quantized along N, out = x @ W.
    x is float32 values (bf16 inputs widened exactly).  The result is float64:
    each product of two float32 values is exact in float64 and the sum is
    formed in float64.
    """
    W = dequantize(w, scales, gs).astype(np.float64)
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    if transpose:
        if W.shape[-1] != x64.shape[-1]:
            raise ValueError("K mismatch")
        return x64 @ W.T
    if W.shape[0] != x64.shape[-1]:
        raise ValueError("K mismatch")
    return x64 @ W


def qmm_batched(x: np.ndarray, w: np.ndarray, scales: np.ndarray, gs=None,
                transpose: bool = True) -> np.ndarray:
    """Reference qmm over a batch of weight matrices (P3 "Numerical results":
    qmm with batched weights, checked against x @ dequantize(w).T per matrix).

    x [XB, M, K] with XB = 1 (one activation matrix for every weight matrix)
    or XB = B; w [B, N, K/8] (transpose) or [B, K, N/8]; scales shaped from w;
    gs [B] or None, one global scale per weight matrix.
    out[b] = qmm(x[0 if XB == 1 else b], w[b], scales[b], gs[b]).  Returns
    float64 [B, M, N].
    """
    B = w.shape[0]
    XB = x.shape[0]
    if XB not in (1, B):
        raise ValueError("x batch must be 1 or match the weight batch")
    parts = []
    for b in range(B):
        src = x[0] if XB == 1 else x[b]
        parts.append(qmm(src, w[b], scales[b], None if gs is None else gs[b], transpose=transpose))
    if not parts:
        M = x.shape[1]
        N = w.shape[1] if transpose else w.shape[2] * NIBBLES_PER_WORD
        return np.zeros((0, M, N), dtype=np.float64)
    return np.stack(parts)


# ----------------------------------------------------------------------------
# Gated MLP projection
# ----------------------------------------------------------------------------

GLU_ACTIVATIONS = ("gelu_tanh", "gelu", "silu")


def glu_activation(z, act: str) -> np.ndarray:
    """Gate activation in float64.

    gelu:      z * Phi(z), Phi the standard normal distribution function
               (Hendrycks and Gimpel, "Gaussian Error Linear Units", the exact
               form), written as erfc(-z / sqrt 2) / 2, which keeps its
               relative accuracy where 1 + erf(z / sqrt 2) would cancel.
    gelu_tanh: the same paper's approximation
               z / 2 * (1 + tanh(sqrt(2 / pi) * (z + 0.044715 * z^3))).
    silu:      z * sigmoid(z) (the sigmoid-weighted linear unit, "Swish"
               with beta = 1).
    """
    z = np.asarray(z, dtype=np.float64)
    if act == "gelu":
        erfc = np.vectorize(math.erfc, otypes=[np.float64])
        return 0.5 * z * erfc(-z / math.sqrt(2.0))
    if act == "gelu_tanh":
        inner = math.sqrt(2.0 / math.pi) * (z + 0.044715 * z * z * z)
        return 0.5 * z * (1.0 + np.tanh(inner))
    if act == "silu":
        with np.errstate(over="ignore"):
            return z / (1.0 + np.exp(-z))
    raise ValueError(f"unknown activation {act!r}")


def qmm_glu(x: np.ndarray, w_gate: np.ndarray, s_gate: np.ndarray, gs_gate,
            w_up: np.ndarray, s_up: np.ndarray, gs_up, act: str) -> np.ndarray:
    """Gated projection of an MLP against two NVFP4 planes (P2 "Hypothesis"
    and "Activation-path follow-up": the gate/up projections of the scaled
    MLP, each with its global-scale sidecar, and the GeGLU activation):

        out = act(x @ dequantize(w_gate).T) * (x @ dequantize(w_up).T)

    w_gate and w_up are transposed planes [F, K/8] of the same shape.  Both
    projections are the float64 ``qmm`` above; the activation and the
    product are taken in float64.  Returns float64 [M, F].
    """
    if w_gate.shape != w_up.shape:
        raise ValueError("gate and up planes differ in shape")
    gate = qmm(x, w_gate, s_gate, gs_gate, transpose=True)
    up = qmm(x, w_up, s_up, gs_up, transpose=True)
    return glu_activation(gate, act) * up


def gather_qmm(x: np.ndarray, lhs: Optional[np.ndarray], rhs: np.ndarray,
               w: np.ndarray, scales: np.ndarray, gs: Optional[np.ndarray]) -> np.ndarray:
    """Reference GatherQMM over experts (P3 "Summary": GatherQMM with a
    per-expert global scale; "Changes during review": out-of-range expert
    indices produce exact zeros).

    x [X, M, K]; lhs [R] (None = identity, r -> r); rhs [R];
    w [E, N, K/8]; scales [E, N, K/16]; gs [E] or None.
    out[r] = x[lhs[r]] @ dequantize(w[rhs[r]]).T, or +0.0 when rhs[r] is not
    in [0, E) or lhs[r] is not in [0, X).  Returns float64 [R, M, N].
    """
    X, M, _ = x.shape
    E, N = w.shape[0], w.shape[1]
    R = rhs.shape[0]
    out = np.zeros((R, M, N), dtype=np.float64)
    for r in range(R):
        e = int(rhs[r])
        src = int(lhs[r]) if lhs is not None else r
        if not (0 <= e < E) or not (0 <= src < X):
            continue
        out[r] = qmm(x[src], w[e], scales[e], None if gs is None else gs[e], transpose=True)
    return out


# ----------------------------------------------------------------------------
# Transcode (ModelOpt triplet -> native planes + sidecar)
# ----------------------------------------------------------------------------

def transcode(weight_u8: np.ndarray, weight_scale: np.ndarray,
              weight_scale_2: Optional[np.ndarray]):
    """ModelOpt NVFP4 triplet to native planes, without dense values
    (P1 "Goal", "Technical notes" and "Implementation plan" step 3):

    * every four source bytes b0..b3 become one little-endian word
      b0 | b1 << 8 | b2 << 16 | b3 << 24;
    * the E4M3 block-scale bytes are kept as they are;
    * weight_scale_2 becomes the global-scale sidecar gs = fl32(ws2 * 2688),
      the value whose gs / (448 * 6) is the second-level scale.

    weight_u8 [..., rows, cols/2]; weight_scale [..., rows, cols/16];
    weight_scale_2 [batch] float32 or None.
    """
    src = np.asarray(weight_u8, dtype=np.uint8)
    if src.shape[-1] % 4 != 0:
        raise ValueError("source row length must be a multiple of four bytes")
    b = src.reshape(src.shape[:-1] + (src.shape[-1] // 4, 4)).astype(np.uint32)
    words = b[..., 0] | (b[..., 1] << np.uint32(8)) | (b[..., 2] << np.uint32(16)) | (b[..., 3] << np.uint32(24))
    words = words.astype(np.uint32)
    scales = np.array(weight_scale, dtype=np.uint8, copy=True)
    check_planes(words, scales)
    gs = None
    if weight_scale_2 is not None:
        gs = (np.asarray(weight_scale_2, dtype=np.float32) * np.float32(GLOBAL_DIVISOR)).astype(np.float32)
    return words, scales, gs


# ----------------------------------------------------------------------------
# Error metric
# ----------------------------------------------------------------------------

def relative_error(out: np.ndarray, ref: np.ndarray) -> float:
    """max |out - ref| / max |ref| (P3 "Numerical results")."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.max(np.abs(ref)) if ref.size else 0.0
    err = np.max(np.abs(out - ref)) if ref.size else 0.0
    if denom == 0.0:
        return float(err)
    return float(err / denom)
