"""MI355X-native 3D Gaussian Splatting training step: HIP kernels for gfx950 behind a C-ABI
library (``libgsmi.so``) and a thin ctypes binding.

Submodules:
  ``gsmi``    -- the binding (argument marshalling over the C-ABI; loads the library lazily)
  ``inputs``  -- seeded synthetic scenes and orbit cameras (no method arithmetic)
"""
__all__ = ["gsmi", "inputs"]
