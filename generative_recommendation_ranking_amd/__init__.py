"""MI355X-native forward pass of the MTGR HSTU encoder over packed jagged user batches.

Submodules:
  synth  -- seeded synthetic inputs and weights (no arithmetic of the method)
  mtgr   -- ctypes binding over the C-ABI library libmtgr.so (HIP kernels for gfx950)
  build  -- hipcc build of libmtgr.so

Nothing is imported eagerly, so that importing the generator never loads the HIP library.
"""
__all__ = ["synth", "mtgr", "build"]
