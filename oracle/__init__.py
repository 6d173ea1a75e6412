"""Plain float64 CPU oracle for the Matryoshka-nested integer matmul.

TEST INFRASTRUCTURE ONLY: imported by tests, by the smoke check and by the
CPU-baseline leg of the benchmark, never by the product path.  It shares no
code with the HIP library (nested_int_matmul_amd) and imports nothing from it.
Every function cites the passage of the pages it restates.
"""
from .matquant import (  # noqa: F401
    C_BITS,
    LAYER_LINEARS,
    bf16_bits_from_float,
    bf16_round,
    bitplane_bytes_read,
    dequant,
    dequant_extra_precision,
    dequant_rows,
    effective_bits,
    float_from_bf16_bits,
    linear,
    linear_extra_precision,
    MLP_ACTIVATIONS,
    mlp_activation,
    mlp_decode,
    mixnmatch_forward,
    mixnmatch_layer,
    overflow_lists,
    pack_bitplanes,
    pack_codes,
    pack_indices,
    quantize_minmax,
    rms_normalize,
    slice_index,
    slice_index_from_bitplanes,
    slice_value,
    slice_value_noclamp,
    unpack_bitplanes,
    unpack_indices,
)
