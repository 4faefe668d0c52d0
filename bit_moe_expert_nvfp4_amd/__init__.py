"""MI355X-native 2-bit + FP4-delta MoE expert layer (HIP kernels behind a C ABI).

Submodules (imported lazily so that nothing loads the HIP library on import):
  moet   - ctypes binding of libmoet (include/moet.h)
  synth  - seeded synthetic NVFP4 layers, activations and router logits
  build  - hipcc build of libmoet.so for gfx950
"""
__all__ = ["moet", "synth", "build"]
