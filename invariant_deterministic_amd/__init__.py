"""Batch-invariant reduction kernels for MI355X (gfx950): RMSNorm, bf16 GEMM and
LoRA-shrink split-K with a fixed-order combine, behind the C ABI of libbi.so.

The ``bi_*`` functions come from :mod:`invariant_deterministic_amd.binding`,
loaded on first use; it raises if the HIP library has not been built.
"""
__all__ = [
    "bi_abi_version", "bi_status_str", "bi_rmsnorm", "bi_gemm", "bi_gemm_config_id",
    "bi_gemm_num_configs", "bi_gemm_with_config", "bi_lora_shrink_workspace_bytes",
    "bi_lora_shrink", "bi_lora_shrink_atomic", "bi_row_bitdiff", "BiError",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
