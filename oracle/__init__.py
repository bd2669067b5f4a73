"""CPU oracle for the W4A16 group-wise AWQ linear layer (test infrastructure).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
use this package.  The product path never imports it.
"""
from .awq_oracle import (  # noqa: F401
    PACK_ORDER,
    codes,
    dequant,
    dequant_packed,
    fake_quant,
    group_params,
    matmul_ref,
    matmul_ref_fsum,
    pack,
    pack_qweight,
    pack_qzeros,
    pack_scales,
    quantize,
    recon_loss,
    scale_candidates,
    scale_weights,
    search_scale,
    weight_scale,
    tolerance_ratio,
    unpack,
    unpack_qweight,
    unpack_qzeros,
    unpack_scales,
)
