"""MI355X (gfx950) BitNet b1.58 BitLinear: ternary weights x int8 activations.

The projection runs in hand-written HIP kernels behind the C ABI declared in
include/bitlinear.h; this package is its Python binding.
"""
from .binding import (  # noqa: F401
    DTYPES,
    KERNELS,
    LIB_PATH,
    SIGNATURES,
    STATUS,
    MAX_GROUP,
    NOALLOC_SCRATCH_BYTES,
    BitLinearError,
    bitlinear_base3_to_blt2,
    bitlinear_forward,
    bitlinear_forward_base3,
    bitlinear_forward_f32,
    bitlinear_forward_f32_noalloc,
    bitlinear_forward_f32_grouped,
    bitlinear_forward_grouped,
    bitlinear_forward_rmsnorm,
    bitlinear_forward_rmsnorm_grouped,
    bitlinear_pack_weights,
    bitlinear_pack_weights_base3,
    bitlinear_quant_acts,
    bitlinear_rmsnorm_quant,
    forward_f32_grouped_workspace_bytes,
    forward_f32_workspace_bytes,
    forward_grouped_workspace_bytes,
    forward_kernel,
    forward_rmsnorm_grouped_workspace_bytes,
    forward_rmsnorm_workspace_bytes,
    forward_workspace_bytes,
    load,
    pack_workspace_bytes,
    packed3_bytes,
    packed_bytes,
)
