"""CPU oracle for NVFP4 quantized matmul -- test infrastructure only.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package; the product path never does.
"""

from .nvfp4_oracle import (  # noqa: F401
    E2M1_MAGNITUDES,
    GLOBAL_DIVISOR,
    GROUP_SIZE,
    bf16_bits_to_f32,
    check_planes,
    decode_e2m1,
    decode_e4m3,
    dequantize,
    dequantize_bf16_bits,
    e2m1_value,
    e4m3_value,
    f32_to_bf16_bits,
    GLU_ACTIVATIONS,
    gather_qmm,
    glu_activation,
    global_factor,
    qmm,
    qmm_batched,
    qmm_glu,
    quantize,
    e2m1_round,
    e4m3_round,
    relative_error,
    transcode,
    unpack_nibbles,
)
