"""MI355X-native multi-LoRA adapter branch (gfx950 HIP kernels behind a C ABI).

Importing the package loads nothing native; ``heterogeneous_adapters_amd.lora``
loads ``liblora.so`` on first use and raises if it is missing.
"""
__all__ = ["lora", "traffic"]
