"""Thin torch-facing binding of libvae.so.

Every function here only marshals arguments: it checks that tensors are
contiguous float32 tensors on the GPU, allocates outputs and workspaces with
torch (device memory), passes raw pointers and torch's current stream to the
C ABI, and turns error codes into :class:`VaeError`.  All computation happens
in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
from ctypes import byref, c_int32, c_size_t, c_void_p
from typing import Dict, List, Optional

import torch

from . import _lib
from ._lib import VaeAttn, VaeConv, VaeError, VaeNorm, VaeProfRecord, VaeResnet, VaeUp, VaeWeights, check

__all__ = [
    "VaeError", "conv2d", "conv_in", "groupnorm_silu", "groupnorm_silu_noalloc", "upsample_nearest2x", "attention",
    "attention_streaming", "ATTENTION_FORMS",
    "conv3d_causal", "conv3d_causal_groupnorm_silu", "probe_mfma_f32", "probe_hbm", "Decoder", "CONV3X3_ALGORITHMS", "set_conv3x3_algorithm", "get_conv3x3_algorithm",
]

# Forms of the 3x3 convolutions (vae_set_conv3x3_algorithm): Winograd
# F(2x2, 3x3), the implicit GEMM of the direct conv, Winograd F(4x4, 3x3).
CONV3X3_ALGORITHMS = {"winograd_2x2": 0, "implicit_gemm": 1, "winograd_4x4": 2}
# Forms of the decoder's mid-block attention (vae_decoder_set_attention).
ATTENTION_FORMS = {"split_softmax": 0, "streaming": 1}


def set_conv3x3_algorithm(name: str) -> None:
    """Process-wide form of the 3x3 convs for decoders created and per-layer
    calls made afterwards: one of CONV3X3_ALGORITHMS."""
    if name not in CONV3X3_ALGORITHMS:
        raise ValueError(f"unknown conv3x3 algorithm {name!r}; expected one of {sorted(CONV3X3_ALGORITHMS)}")
    check(_lib_().vae_set_conv3x3_algorithm(CONV3X3_ALGORITHMS[name]))


def get_conv3x3_algorithm() -> str:
    code = _lib_().vae_get_conv3x3_algorithm()
    return {v: k for k, v in CONV3X3_ALGORITHMS.items()}[code]


def _lib_():
    return _lib.load()


def _stream() -> c_void_p:
    return c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 GPU tensor")
    return t


def _out(out: Optional[torch.Tensor], shape, device) -> torch.Tensor:
    if out is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    _dev(out, "out")
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(shape)}")
    return out


def _ws(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _conv(weight: torch.Tensor, bias: torch.Tensor, name: str = "conv") -> VaeConv:
    _dev(weight, name + ".weight")
    _dev(bias, name + ".bias")
    if weight.dim() == 2:
        k = 1
    else:
        k = weight.shape[-1]
    return VaeConv(weight.data_ptr(), bias.data_ptr(), weight.shape[0], weight.shape[1], k)


def _norm(gamma: torch.Tensor, beta: torch.Tensor, name: str = "norm") -> VaeNorm:
    _dev(gamma, name + ".gamma")
    _dev(beta, name + ".beta")
    return VaeNorm(gamma.data_ptr(), beta.data_ptr(), gamma.numel())


# ---------------------------------------------------------------------------
# layers
# ---------------------------------------------------------------------------

def conv2d(x: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor, upsample2x: bool = False,
           residual: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Conv2d (stride 1, pad k/2) of x [cin, h, w], optionally of its nearest-x2
    upsample, plus an optional residual; returns [cout, H, W]."""
    lib = _lib_()
    _dev(x, "x")
    cin, h, w = x.shape
    conv = _conv(weight, bias)
    H, W = (2 * h, 2 * w) if upsample2x else (h, w)
    if residual is not None:
        _dev(residual, "residual")
    y = _out(out, (weight.shape[0], H, W), x.device)
    nb = c_size_t()
    check(lib.vae_conv2d_workspace_bytes(byref(conv), h, w, int(bool(upsample2x)), byref(nb)))
    ws = _ws(nb.value, x.device)
    check(lib.vae_conv2d(x.data_ptr(), cin, h, w, byref(conv), int(bool(upsample2x)), _ptr(residual),
                         y.data_ptr(), _ptr(ws), nb.value, _stream()))
    return y


def conv_in(z: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor, scaling_factor: float,
            shift_factor: float, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """conv_in applied to z / scaling_factor + shift_factor (padding stays zero)."""
    lib = _lib_()
    _dev(z, "z")
    cin, h, w = z.shape
    conv = _conv(weight, bias)
    y = _out(out, (weight.shape[0], h, w), z.device)
    nb = c_size_t()
    check(lib.vae_conv2d_workspace_bytes(byref(conv), h, w, 0, byref(nb)))
    ws = _ws(nb.value, z.device)
    check(lib.vae_conv_in(z.data_ptr(), cin, h, w, byref(conv), float(scaling_factor), float(shift_factor),
                          y.data_ptr(), _ptr(ws), nb.value, _stream()))
    return y


def groupnorm_silu(x: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, silu: bool = True,
                   residual: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GroupNorm(32, eps 1e-6) over x [c, ...], then SiLU, then + residual.
    ``out`` may be ``x`` itself (in place)."""
    lib = _lib_()
    _dev(x, "x")
    c = x.shape[0]
    spatial = x.numel() // c
    norm = _norm(gamma, beta)
    if residual is not None:
        _dev(residual, "residual")
    y = torch.empty_like(x) if out is None else _dev(out, "out")
    nb = c_size_t()
    check(lib.vae_groupnorm_workspace_bytes(c, spatial, byref(nb)))
    ws = _ws(nb.value, x.device)
    check(lib.vae_groupnorm_silu(x.data_ptr(), c, spatial, byref(norm), int(bool(silu)), _ptr(residual),
                                 y.data_ptr(), _ptr(ws), nb.value, _stream()))
    return y


def groupnorm_silu_noalloc(x: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, silu: bool = True,
                           residual: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """:func:`groupnorm_silu` through the entry point that allocates nothing
    (its partial sums in the library's static device buffer).  With ``out``
    given, this call allocates nothing either."""
    lib = _lib_()
    _dev(x, "x")
    c = x.shape[0]
    norm = _norm(gamma, beta)
    if residual is not None:
        _dev(residual, "residual")
    y = torch.empty_like(x) if out is None else _dev(out, "out")
    check(lib.vae_groupnorm_silu_noalloc(x.data_ptr(), c, x.numel() // c, byref(norm), int(bool(silu)),
                                         _ptr(residual), y.data_ptr(), _stream()))
    return y


def conv2d_groupnorm_silu(x: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor, gamma: torch.Tensor,
                          beta: torch.Tensor, silu: bool = True, upsample2x: bool = False,
                          residual: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                          out_norm: Optional[torch.Tensor] = None):
    """y = conv2d(x) (+ residual) as :func:`conv2d` (3x3), then
    z = SiLU(GroupNorm(y)) with the group statistics taken in the conv's
    epilogue.  Returns (y, z); ``out_norm`` may be ``out`` (z overwrites y)."""
    lib = _lib_()
    _dev(x, "x")
    cin, h, w = x.shape
    conv = _conv(weight, bias)
    norm = _norm(gamma, beta)
    H, W = (2 * h, 2 * w) if upsample2x else (h, w)
    if residual is not None:
        _dev(residual, "residual")
    y = _out(out, (weight.shape[0], H, W), x.device)
    z = _out(out_norm, (weight.shape[0], H, W), x.device)
    nb = c_size_t()
    check(lib.vae_conv2d_groupnorm_workspace_bytes(byref(conv), h, w, int(bool(upsample2x)), byref(nb)))
    ws = _ws(nb.value, x.device)
    check(lib.vae_conv2d_groupnorm_silu(x.data_ptr(), cin, h, w, byref(conv), int(bool(upsample2x)),
                                        _ptr(residual), byref(norm), int(bool(silu)), y.data_ptr(),
                                        z.data_ptr(), _ptr(ws), nb.value, _stream()))
    return y, z


def upsample_nearest2x(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    lib = _lib_()
    _dev(x, "x")
    c, h, w = x.shape
    y = _out(out, (c, 2 * h, 2 * w), x.device)
    check(lib.vae_upsample_nearest2x(x.data_ptr(), c, h, w, y.data_ptr(), _stream()))
    return y


def _attn(p: Dict[str, torch.Tensor], prefix: str) -> VaeAttn:
    return VaeAttn(_norm(p[prefix + ".group_norm.weight"], p[prefix + ".group_norm.bias"]),
                   _conv(p[prefix + ".to_q.weight"], p[prefix + ".to_q.bias"]),
                   _conv(p[prefix + ".to_k.weight"], p[prefix + ".to_k.bias"]),
                   _conv(p[prefix + ".to_v.weight"], p[prefix + ".to_v.bias"]),
                   _conv(p[prefix + ".to_out.0.weight"], p[prefix + ".to_out.0.bias"]))


def attention(x: torch.Tensor, p: Dict[str, torch.Tensor], prefix: str,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Mid-block attention; ``p`` holds diffusers-named tensors under ``prefix``
    (group_norm, to_q, to_k, to_v, to_out.0)."""
    lib = _lib_()
    _dev(x, "x")
    c, h, w = x.shape
    a = _attn(p, prefix)
    y = _out(out, (c, h, w), x.device)
    nb = c_size_t()
    check(lib.vae_attention_workspace_bytes(c, h, w, byref(nb)))
    ws = _ws(nb.value, x.device)
    check(lib.vae_attention(x.data_ptr(), c, h, w, byref(a), y.data_ptr(), _ptr(ws), nb.value, _stream()))
    return y


def attention_streaming(x: torch.Tensor, p: Dict[str, torch.Tensor], prefix: str,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """:func:`attention` with a streaming softmax (no score matrix in memory);
    128, 256 or 512 channels."""
    lib = _lib_()
    _dev(x, "x")
    c, h, w = x.shape
    a = _attn(p, prefix)
    y = _out(out, (c, h, w), x.device)
    nb = c_size_t()
    check(lib.vae_attention_streaming_workspace_bytes(c, h, w, byref(nb)))
    ws = _ws(nb.value, x.device)
    check(lib.vae_attention_streaming(x.data_ptr(), c, h, w, byref(a), y.data_ptr(), _ptr(ws), nb.value, _stream()))
    return y


def conv3d_causal(x: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal 3x3x3 conv of x [cin, t, h, w] (frame 0 replicated twice in front)."""
    lib = _lib_()
    _dev(x, "x")
    cin, t, h, w = x.shape
    conv = _conv(weight, bias)
    y = _out(out, (weight.shape[0], t, h, w), x.device)
    nb = c_size_t()
    check(lib.vae_conv3d_causal_workspace_bytes(byref(conv), t, h, w, byref(nb)))
    ws = _ws(nb.value, x.device)
    check(lib.vae_conv3d_causal(x.data_ptr(), cin, t, h, w, byref(conv), y.data_ptr(), _ptr(ws), nb.value,
                                _stream()))
    return y


def conv3d_causal_groupnorm_silu(x: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor, gamma: torch.Tensor,
                                 beta: torch.Tensor, silu: bool = True, residual: Optional[torch.Tensor] = None,
                                 out: Optional[torch.Tensor] = None, out_norm: Optional[torch.Tensor] = None):
    """y = conv3d_causal(x), then z = SiLU(GroupNorm(y)) (+ residual) with the
    group statistics from the conv's epilogue.  Returns (y, z); ``out_norm``
    may be ``out`` (z overwrites y)."""
    lib = _lib_()
    _dev(x, "x")
    cin, t, h, w = x.shape
    conv = _conv(weight, bias)
    norm = _norm(gamma, beta)
    if residual is not None:
        _dev(residual, "residual")
    y = _out(out, (weight.shape[0], t, h, w), x.device)
    z = _out(out_norm, (weight.shape[0], t, h, w), x.device)
    nb = c_size_t()
    check(lib.vae_conv3d_causal_groupnorm_workspace_bytes(byref(conv), t, h, w, byref(nb)))
    ws = _ws(nb.value, x.device)
    check(lib.vae_conv3d_causal_groupnorm_silu(x.data_ptr(), cin, t, h, w, byref(conv), byref(norm), int(bool(silu)),
                                               _ptr(residual), y.data_ptr(), z.data_ptr(), _ptr(ws), nb.value,
                                               _stream()))
    return y, z


def probe_mfma_f32(blocks: int, iters: int, out: Optional[torch.Tensor] = None):
    """Enqueues the FP32 MFMA probe (vae_probe_mfma_f32) on the current
    stream; returns (out [blocks * 256], FLOPs of the launch)."""
    lib = _lib_()
    o = _out(out, (blocks * 256,), torch.device("cuda", torch.cuda.current_device()))
    flops = ctypes.c_double()
    check(lib.vae_probe_mfma_f32(blocks, iters, o.data_ptr(), o.numel(), byref(flops), _stream()))
    return o, flops.value


def probe_hbm(x: torch.Tensor, y: Optional[torch.Tensor] = None, blocks: int = 2048,
              out: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    """Enqueues the HBM probe (vae_probe_hbm): a read of x (returns the
    per-thread sums [blocks * 256]) or, with y, a copy of x into y."""
    lib = _lib_()
    _dev(x, "x")
    if y is not None:
        _dev(y, "y")
        if y.numel() != x.numel():
            raise ValueError("probe_hbm: y must have as many elements as x")
        check(lib.vae_probe_hbm(x.data_ptr(), x.numel(), y.data_ptr(), blocks, None, 0, _stream()))
        return None
    o = _out(out, (blocks * 256,), x.device)
    check(lib.vae_probe_hbm(x.data_ptr(), x.numel(), None, blocks, o.data_ptr(), o.numel(), _stream()))
    return o


# ---------------------------------------------------------------------------
# the decoder
# ---------------------------------------------------------------------------

class Decoder:
    """The whole FLUX-class decoder behind ``vae_decode``.

    ``params`` maps diffusers tensor names (conv_in.*, mid_block.*,
    up_blocks.*, conv_norm_out.*, conv_out.*) to float32 GPU tensors.  The
    library copies them once into its own packed buffer.  With ``causal3d``
    the same chain decodes video latents ``[c, t, h, w]`` (``vae_decode3d``):
    the 3x3 conv weights are ``[cout, cin, 3, 3, 3]`` causal kernels.
    """

    def __init__(self, params: Dict[str, torch.Tensor], scaling_factor: float, shift_factor: float,
                 causal3d: bool = False):
        lib = _lib_()
        self._lib = lib
        p = params
        self._keep: List = []

        def conv(prefix):
            return _conv(p[prefix + ".weight"], p[prefix + ".bias"], prefix)

        def norm(prefix):
            return _norm(p[prefix + ".weight"], p[prefix + ".bias"], prefix)

        def resnet(prefix):
            sc = VaeConv(None, None, 0, 0, 0)
            if prefix + ".conv_shortcut.weight" in p:
                sc = conv(prefix + ".conv_shortcut")
            return VaeResnet(norm(prefix + ".norm1"), conv(prefix + ".conv1"), norm(prefix + ".norm2"),
                             conv(prefix + ".conv2"), sc)

        ups = []
        i = 0
        while f"up_blocks.{i}.resnets.0.conv1.weight" in p:
            j = 0
            rs = []
            while f"up_blocks.{i}.resnets.{j}.conv1.weight" in p:
                rs.append(resnet(f"up_blocks.{i}.resnets.{j}"))
                j += 1
            arr = (VaeResnet * len(rs))(*rs)
            self._keep.append(arr)
            upc = VaeConv(None, None, 0, 0, 0)
            if f"up_blocks.{i}.upsamplers.0.conv.weight" in p:
                upc = conv(f"up_blocks.{i}.upsamplers.0.conv")
            ups.append(VaeUp(len(rs), arr, upc))
            i += 1
        ups_arr = (VaeUp * len(ups))(*ups)
        self._keep.append(ups_arr)
        attn = VaeAttn(norm("mid_block.attentions.0.group_norm"), conv("mid_block.attentions.0.to_q"),
                       conv("mid_block.attentions.0.to_k"), conv("mid_block.attentions.0.to_v"),
                       conv("mid_block.attentions.0.to_out.0"))
        w = VaeWeights(conv("conv_in"), resnet("mid_block.resnets.0"), attn, resnet("mid_block.resnets.1"),
                       len(ups), ups_arr, norm("conv_norm_out"), conv("conv_out"), float(scaling_factor),
                       float(shift_factor))
        self.causal3d = bool(causal3d)
        nb = c_size_t()
        pack_bytes = lib.vae_decoder3d_pack_bytes if self.causal3d else lib.vae_decoder_pack_bytes
        create = lib.vae_decoder3d_create if self.causal3d else lib.vae_decoder_create
        check(pack_bytes(byref(w), byref(nb)))
        device = p["conv_in.weight"].device
        self.device = device
        self.pack = torch.empty(nb.value, dtype=torch.uint8, device=device)
        handle = c_void_p()
        check(create(byref(handle), byref(w), self.pack.data_ptr(), nb.value, _stream()))
        self._h = handle
        self.latent_channels = p["conv_in.weight"].shape[1]
        self._ws: Optional[torch.Tensor] = None

    def output_shape(self, h: int, w: int):
        c, ho, wo = c_int32(), c_int32(), c_int32()
        check(self._lib.vae_decoder_output_shape(self._h, h, w, byref(c), byref(ho), byref(wo)))
        return c.value, ho.value, wo.value

    def workspace_bytes(self, h: int, w: int, t: Optional[int] = None) -> int:
        nb = c_size_t()
        if self.causal3d:
            check(self._lib.vae_decoder3d_workspace_bytes(self._h, 1 if t is None else t, h, w, byref(nb)))
        else:
            check(self._lib.vae_decoder_workspace_bytes(self._h, h, w, byref(nb)))
        return nb.value

    def decode(self, latent: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """latent [c, h, w] -> rgb [3, 8h, 8w]; for a 3-D decoder [c, t, h, w] -> [3, t, 8h, 8w].

        The latent's rank, channel count (conv_in's inputs) and device are
        checked here: vae_decode takes no channel count, so a latent with
        fewer channels would be read past its end."""
        self._check_latent(latent)
        if self.causal3d:
            c, t, h, w = latent.shape
        else:
            c, h, w = latent.shape
            t = None
        nb = self.workspace_bytes(h, w, t)
        if self._ws is None or self._ws.numel() < nb:
            self._ws = torch.empty(nb, dtype=torch.uint8, device=latent.device)
        co, ho, wo = self.output_shape(h, w)
        shape = (co, ho, wo) if t is None else (co, t, ho, wo)
        rgb = _out(out, shape, latent.device)
        if self.causal3d:
            check(self._lib.vae_decode3d(self._h, latent.data_ptr(), t, h, w, rgb.data_ptr(), self._ws.data_ptr(),
                                         self._ws.numel(), _stream()))
        else:
            check(self._lib.vae_decode(self._h, latent.data_ptr(), h, w, rgb.data_ptr(), self._ws.data_ptr(),
                                       self._ws.numel(), _stream()))
        return rgb

    def tiled_workspace_bytes(self, h: int, w: int, tile: int = 256, overlap: int = 64) -> int:
        nb = c_size_t()
        check(self._lib.vae_decoder_tiled_workspace_bytes(self._h, h, w, tile, overlap, byref(nb)))
        return nb.value

    def decode_tiled(self, latent: torch.Tensor, tile: int = 256, overlap: int = 64,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """latent [c, h, w] -> rgb [3, 8h, 8w], decoded in tiles of `tile`
        output pixels overlapping by at least `overlap` (vae_decode_tiled)."""
        self._check_latent(latent)
        if self.causal3d:
            raise ValueError("decode_tiled: a 2-D decoder only")
        c, h, w = latent.shape
        nb = self.tiled_workspace_bytes(h, w, tile, overlap)
        ws = torch.empty(nb, dtype=torch.uint8, device=latent.device)
        co, ho, wo = self.output_shape(h, w)
        rgb = _out(out, (co, ho, wo), latent.device)
        check(self._lib.vae_decode_tiled(self._h, latent.data_ptr(), h, w, tile, overlap, rgb.data_ptr(),
                                         ws.data_ptr(), ws.numel(), _stream()))
        return rgb

    def _check_latent(self, latent) -> None:
        if not isinstance(latent, torch.Tensor):
            raise TypeError("latent must be a torch.Tensor")
        rank = 4 if self.causal3d else 3
        if latent.dim() != rank:
            raise ValueError(f"latent must have {rank} dimensions ({'[c, t, h, w]' if self.causal3d else '[c, h, w]'}), "
                             f"got shape {tuple(latent.shape)}")
        if latent.shape[0] != self.latent_channels:
            raise ValueError(f"latent has {latent.shape[0]} channels; the decoder's conv_in takes "
                             f"{self.latent_channels}")
        _dev(latent, "latent")
        if latent.device != self.device:
            raise ValueError(f"latent is on {latent.device}, the decoder's weights on {self.device}")

    def set_groupnorm_fusion(self, on: bool) -> None:
        """Apply GroupNorm + SiLU while each conv loads its input (off by default)."""
        check(self._lib.vae_decoder_set_groupnorm_fusion(self._h, int(bool(on))))

    def set_attention(self, form: str) -> None:
        """The mid-block attention's form: "split_softmax" (default) or "streaming"."""
        if form not in ATTENTION_FORMS:
            raise ValueError(f"unknown attention form {form!r}; expected one of {sorted(ATTENTION_FORMS)}")
        check(self._lib.vae_decoder_set_attention(self._h, ATTENTION_FORMS[form]))

    def get_attention(self) -> str:
        return {v: k for k, v in ATTENTION_FORMS.items()}[self._lib.vae_decoder_get_attention(self._h)]

    def set_graph(self, on: bool) -> None:
        """Replay decodes with the same buffers and sizes from a captured HIP graph."""
        check(self._lib.vae_decoder_set_graph(self._h, int(bool(on))))

    def set_profiling(self, on: bool) -> None:
        check(self._lib.vae_decoder_set_profiling(self._h, int(bool(on))))

    def profile(self) -> List[dict]:
        n = c_int32()
        check(self._lib.vae_decoder_profile(self._h, None, 0, byref(n)))
        recs = (VaeProfRecord * max(n.value, 1))()
        check(self._lib.vae_decoder_profile(self._h, recs, n.value, byref(n)))
        return [{"kernel": r.kernel.decode(), "layer": r.layer.decode(), "ms": float(r.ms),
                 "flops": float(r.flops), "bytes": float(r.bytes)} for r in recs[:n.value]]

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.vae_decoder_destroy(self._h)
            self._h = c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
