"""SageSLA forward (sparse-linear attention with INT8 SageAttention QK^T) for
MI355X (gfx950): hand-written HIP kernels behind a C ABI, with a thin ctypes
binding.  Importing this package loads nothing; ``sparse_bit_attention_amd.sla``
loads the HIP library and fails loudly when it is missing."""

__all__ = ["synth", "sla"]
