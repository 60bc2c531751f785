"""MI355X-native FLUX-class VAE decoder: hand-written HIP kernels for gfx950
behind the C ABI of ``libvae.so`` (include/vae.h), with a thin torch binding.

Importing the package does not load the library; the first call does, and it
raises if ``libvae.so`` has not been built (``python -m
diffusion_vae_decoder_amd.build``).  There is no CPU fallback.
"""
from ._lib import VaeError, load  # noqa: F401

__all__ = ["VaeError", "load", "api"]


def __getattr__(name):
    if name == "api":
        import importlib
        return importlib.import_module(__name__ + ".api")
    raise AttributeError(name)
