"""MI355X-native canvas denoising for DiffusionGemma-style discrete text diffusion.

The compute path is libdg.so (HIP kernels for gfx950, C ABI in include/dg.h);
``binding`` marshals torch tensors into it. Import ``binding`` explicitly: it
fails loudly when the library has not been built.
"""
import os

PACKAGE_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PACKAGE_DIR, "libdg.so")
