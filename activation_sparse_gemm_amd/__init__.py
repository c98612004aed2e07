"""RT-Lynx sparse + LoRA linear layer on AMD MI355X (gfx950).

Python face of liblynx.so: `sparsify`, `linear_sparse_lora`,
`linear_sparse_lora_packed`, `linear_sparse_lora_noalloc` and `linear_dense` take torch device tensors and
call the library's HIP kernels on torch's current stream.
"""
from ._abi import (  # noqa: F401
    LIB_PATH,
    SCRATCH_BYTES,
    LynxError,
    lib,
    linear_dense,
    linear_sequence,
    sequence_workspace_bytes,
    linear_sparse_lora,
    linear_sparse_lora_noalloc,
    linear_sparse_lora_packed,
    sparsify,
    status_string,
    version,
    workspace_bytes,
)
