"""MI355X-native (gfx950) block-diffusion canvas denoising step behind a small C ABI.

libdg.so (built from ``csrc/`` by ``build.py``) holds the HIP kernels and the C ABI declared in
``include/dg.h``; ``_lib`` binds it with ctypes and ``driver`` wraps the calls around torch device
tensors.  ``synth`` makes the seeded synthetic inputs.
"""
