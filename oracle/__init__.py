"""CPU oracle of the RT-Lynx sparse + LoRA linear layer (fp64, NumPy).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package entry point's
smoke check and by the benchmark's CPU-baseline leg, never by the HIP path.
"""
from .lynx_oracle import (  # noqa: F401
    SparsifyResult,
    decode_bf16,
    keep_mask,
    linear_dense,
    linear_from_packed,
    linear_sparse_lora,
    norm_scale,
    pack_meta,
    pack_values,
    select_top2_of_4,
    sparsify,
    unpack_dense,
    unpack_meta,
)
