"""ctypes declarations of libvae.so (see include/vae.h).

The library is loaded from this package directory.  There is no fallback: if
``libvae.so`` is missing, :func:`load` raises, naming the build command.  The
environment variable VAE_LIBRARY may name the sanitizer build
``libvae_san.so`` of the same directory instead (it needs the ASan runtime
preloaded into the process).
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_void_p

_LIB_NAMES = ("libvae.so", "libvae_san.so")
_LIB_NAME = os.environ.get("VAE_LIBRARY", "libvae.so")
if _LIB_NAME not in _LIB_NAMES:
    raise ImportError(f"VAE_LIBRARY={_LIB_NAME!r}; expected one of {_LIB_NAMES}")
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), _LIB_NAME)

VAE_OK = 0
VAE_ERR_INVALID_ARG = -1
VAE_ERR_UNSUPPORTED = -2
VAE_ERR_WORKSPACE = -3
VAE_ERR_HIP = -4
ABI_VERSION = 11


class VaeConv(ctypes.Structure):
    _fields_ = [("weight", c_void_p), ("bias", c_void_p), ("out_channels", c_int32),
                ("in_channels", c_int32), ("kernel", c_int32)]


class VaeNorm(ctypes.Structure):
    _fields_ = [("gamma", c_void_p), ("beta", c_void_p), ("channels", c_int32)]


class VaeResnet(ctypes.Structure):
    _fields_ = [("norm1", VaeNorm), ("conv1", VaeConv), ("norm2", VaeNorm), ("conv2", VaeConv),
                ("shortcut", VaeConv)]


class VaeAttn(ctypes.Structure):
    _fields_ = [("norm", VaeNorm), ("q", VaeConv), ("k", VaeConv), ("v", VaeConv), ("out", VaeConv)]


class VaeUp(ctypes.Structure):
    _fields_ = [("n_resnets", c_int32), ("resnets", POINTER(VaeResnet)), ("upsample", VaeConv)]


class VaeWeights(ctypes.Structure):
    _fields_ = [("conv_in", VaeConv), ("mid_res0", VaeResnet), ("mid_attn", VaeAttn),
                ("mid_res1", VaeResnet), ("n_up", c_int32), ("ups", POINTER(VaeUp)),
                ("norm_out", VaeNorm), ("conv_out", VaeConv), ("scaling_factor", c_float),
                ("shift_factor", c_float)]


class VaeProfRecord(ctypes.Structure):
    _fields_ = [("kernel", c_char * 40), ("layer", c_char * 72), ("ms", c_float),
                ("flops", c_double), ("bytes", c_double)]


# name -> (restype, argtypes); every symbol include/vae.h declares.
SIGNATURES = {
    "vae_last_error": (c_char_p, []),
    "vae_abi_version": (c_int32, []),
    "vae_conv2d_workspace_bytes": (c_int32, [POINTER(VaeConv), c_int32, c_int32, c_int32, POINTER(c_size_t)]),
    "vae_conv2d": (c_int32, [c_void_p, c_int32, c_int32, c_int32, POINTER(VaeConv), c_int32, c_void_p,
                             c_void_p, c_void_p, c_size_t, c_void_p]),
    "vae_conv_in": (c_int32, [c_void_p, c_int32, c_int32, c_int32, POINTER(VaeConv), c_float, c_float,
                              c_void_p, c_void_p, c_size_t, c_void_p]),
    "vae_groupnorm_workspace_bytes": (c_int32, [c_int32, c_int64, POINTER(c_size_t)]),
    "vae_groupnorm_silu": (c_int32, [c_void_p, c_int32, c_int64, POINTER(VaeNorm), c_int32, c_void_p,
                                     c_void_p, c_void_p, c_size_t, c_void_p]),
    "vae_groupnorm_silu_noalloc": (c_int32, [c_void_p, c_int32, c_int64, POINTER(VaeNorm), c_int32, c_void_p,
                                             c_void_p, c_void_p]),
    "vae_conv2d_groupnorm_workspace_bytes": (c_int32, [POINTER(VaeConv), c_int32, c_int32, c_int32,
                                                       POINTER(c_size_t)]),
    "vae_conv2d_groupnorm_silu": (c_int32, [c_void_p, c_int32, c_int32, c_int32, POINTER(VaeConv), c_int32,
                                            c_void_p, POINTER(VaeNorm), c_int32, c_void_p, c_void_p, c_void_p,
                                            c_size_t, c_void_p]),
    "vae_upsample_nearest2x": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    "vae_attention_workspace_bytes": (c_int32, [c_int32, c_int32, c_int32, POINTER(c_size_t)]),
    "vae_attention": (c_int32, [c_void_p, c_int32, c_int32, c_int32, POINTER(VaeAttn), c_void_p,
                                c_void_p, c_size_t, c_void_p]),
    "vae_attention_streaming_workspace_bytes": (c_int32, [c_int32, c_int32, c_int32, POINTER(c_size_t)]),
    "vae_attention_streaming": (c_int32, [c_void_p, c_int32, c_int32, c_int32, POINTER(VaeAttn), c_void_p,
                                          c_void_p, c_size_t, c_void_p]),
    "vae_conv3d_causal_workspace_bytes": (c_int32, [POINTER(VaeConv), c_int32, c_int32, c_int32,
                                                    POINTER(c_size_t)]),
    "vae_conv3d_causal": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, POINTER(VaeConv),
                                    c_void_p, c_void_p, c_size_t, c_void_p]),
    "vae_conv3d_causal_groupnorm_workspace_bytes": (c_int32, [POINTER(VaeConv), c_int32, c_int32, c_int32,
                                                              POINTER(c_size_t)]),
    "vae_conv3d_causal_groupnorm_silu": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, POINTER(VaeConv),
                                                   POINTER(VaeNorm), c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                                   c_size_t, c_void_p]),
    "vae_decoder_pack_bytes": (c_int32, [POINTER(VaeWeights), POINTER(c_size_t)]),
    "vae_decoder_create": (c_int32, [POINTER(c_void_p), POINTER(VaeWeights), c_void_p, c_size_t, c_void_p]),
    "vae_decoder_workspace_bytes": (c_int32, [c_void_p, c_int32, c_int32, POINTER(c_size_t)]),
    "vae_decode": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "vae_decoder3d_pack_bytes": (c_int32, [POINTER(VaeWeights), POINTER(c_size_t)]),
    "vae_decoder3d_create": (c_int32, [POINTER(c_void_p), POINTER(VaeWeights), c_void_p, c_size_t, c_void_p]),
    "vae_decoder3d_workspace_bytes": (c_int32, [c_void_p, c_int32, c_int32, c_int32, POINTER(c_size_t)]),
    "vae_decode3d": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_size_t,
                               c_void_p]),
    "vae_decoder_tiled_workspace_bytes": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, POINTER(c_size_t)]),
    "vae_decode_tiled": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                   c_size_t, c_void_p]),
    "vae_probe_mfma_f32": (c_int32, [c_int32, c_int32, c_void_p, c_size_t, POINTER(c_double), c_void_p]),
    "vae_probe_hbm": (c_int32, [c_void_p, c_size_t, c_void_p, c_int32, c_void_p, c_size_t, c_void_p]),
    "vae_decoder_output_shape": (c_int32, [c_void_p, c_int32, c_int32, POINTER(c_int32), POINTER(c_int32),
                                           POINTER(c_int32)]),
    "vae_decoder_destroy": (None, [c_void_p]),
    "vae_decoder_set_groupnorm_fusion": (c_int32, [c_void_p, c_int32]),
    "vae_decoder_set_graph": (c_int32, [c_void_p, c_int32]),
    "vae_decoder_set_attention": (c_int32, [c_void_p, c_int32]),
    "vae_decoder_get_attention": (c_int32, [c_void_p]),
    "vae_set_conv3x3_algorithm": (c_int32, [c_int32]),
    "vae_get_conv3x3_algorithm": (c_int32, []),
    "vae_decoder_set_profiling": (c_int32, [c_void_p, c_int32]),
    "vae_decoder_profile": (c_int32, [c_void_p, POINTER(VaeProfRecord), c_int32, POINTER(c_int32)]),
}

_LIB = None


class VaeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"libvae error {code}: {message}")
        self.code = code


def load() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m diffusion_vae_decoder_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.vae_abi_version() != ABI_VERSION:
            raise ImportError("libvae.so ABI version mismatch; rebuild it")
        _LIB = lib
    return _LIB


def check(code: int) -> None:
    if code != VAE_OK:
        msg = load().vae_last_error()
        raise VaeError(code, msg.decode() if msg else "")
