"""Seeded synthetic inputs for the FLUX-class VAE decoder.

This module is the only code that both the oracle-side tests and the GPU side
use.  It draws random numbers and lays them out under diffusers-style tensor
names; it holds none of the decoder's arithmetic.

Generator
---------
SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014), used counter-style: draw ``i`` (1-based) of a stream
with key ``s`` is ``mix(s + i * 0x9E3779B97F4A7C15)`` with the published
finaliser ``mix``.  Each tensor has its own stream; its key is
``mix(seed ^ fnv1a64(name))`` (FNV-1a, 64-bit), so adding or reordering
tensors never shifts the values of the others.

* uniform on [0,1): ``(bits >> 40) * 2**-24`` (exact in f32);
  ``U(lo, hi) = lo + (hi - lo) * u`` in f64, rounded once to f32.
* N(0,1): Box-Muller on consecutive pairs of draws,
  ``u1 = ((b1 >> 11) + 1) * 2**-53`` in (0,1], ``u2 = (b2 >> 11) * 2**-53``,
  giving ``r cos(2 pi u2)`` then ``r sin(2 pi u2)`` with ``r = sqrt(-2 ln u1)``;
  computed in f64 and rounded once to f32.

Initialisation recipe (the decoder workloads: FLUX-class AutoencoderKL with a
16-channel latent, decoder widths 512, 512, 256, 128, three resnets per up
block):

* conv weight ``U(+-1/sqrt(Cin*k*k))`` (``k*k*k`` for the 3-D conv), bias ``U(+-0.01)``
* GroupNorm ``gamma = 1 + U(+-0.1)``, ``beta = U(+-0.1)``
* attention q/k/v/out weight ``U(+-1/sqrt(c))``, bias ``U(+-0.01)``
* latents and layer inputs ``N(0,1)``
"""
from __future__ import annotations

import math

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1

# Decoder hyper-parameters of the FLUX-class AutoencoderKL.
LATENT_CHANNELS = 16
OUT_CHANNELS = 3
DECODER_WIDTHS = (512, 512, 256, 128)   # up block i produces DECODER_WIDTHS[i] channels
RESNETS_PER_UP_BLOCK = 3
SCALING_FACTOR = 0.3611
SHIFT_FACTOR = 0.1159


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _mix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def fnv1a64(text: str) -> int:
    h = 0xCBF29CE484222325
    for byte in text.encode("utf-8"):
        h ^= byte
        h = (h * 0x100000001B3) & _MASK64
    return h


def stream_key(seed: int, name: str) -> int:
    return _mix64_int((seed & _MASK64) ^ fnv1a64(name))


def raw_bits(seed: int, name: str, n: int) -> np.ndarray:
    """The first ``n`` 64-bit draws of the stream for tensor ``name``."""
    key = np.uint64(stream_key(seed, name))
    out = np.empty(n, dtype=np.uint64)
    step = 1 << 24
    with np.errstate(over="ignore"):
        for lo in range(0, n, step):
            hi = min(n, lo + step)
            i = np.arange(lo + 1, hi + 1, dtype=np.uint64)
            out[lo:hi] = _mix64(key + i * _GOLDEN)
    return out


def uniform(seed: int, name: str, shape, lo: float, hi: float) -> np.ndarray:
    n = int(np.prod(shape)) if len(shape) else 1
    u = (raw_bits(seed, name, n) >> np.uint64(40)).astype(np.float64) * (2.0 ** -24)
    return (lo + (hi - lo) * u).astype(np.float32).reshape(shape)


def normal(seed: int, name: str, shape) -> np.ndarray:
    n = int(np.prod(shape)) if len(shape) else 1
    pairs = (n + 1) // 2
    out = np.empty(2 * pairs, dtype=np.float32)
    step = 1 << 23
    bits_all = None
    if pairs <= step:
        bits_all = raw_bits(seed, name, 2 * pairs)
    key = np.uint64(stream_key(seed, name))
    for lo in range(0, pairs, step):
        hi = min(pairs, lo + step)
        if bits_all is not None:
            b = bits_all[2 * lo:2 * hi]
        else:
            with np.errstate(over="ignore"):
                i = np.arange(2 * lo + 1, 2 * hi + 1, dtype=np.uint64)
                b = _mix64(key + i * _GOLDEN)
        u1 = ((b[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
        u2 = (b[1::2] >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
        r = np.sqrt(-2.0 * np.log(u1))
        t = 2.0 * math.pi * u2
        out[2 * lo:2 * hi:2] = (r * np.cos(t)).astype(np.float32)
        out[2 * lo + 1:2 * hi:2] = (r * np.sin(t)).astype(np.float32)
    return out[:n].reshape(shape)


# ---------------------------------------------------------------------------
# parameter helpers
# ---------------------------------------------------------------------------

def conv_params(seed: int, prefix: str, cin: int, cout: int, k: int, dims: int = 2) -> dict:
    fan_in = cin * k ** dims
    a = 1.0 / math.sqrt(fan_in)
    shape = (cout, cin) + (k,) * dims
    return {
        prefix + ".weight": uniform(seed, prefix + ".weight", shape, -a, a),
        prefix + ".bias": uniform(seed, prefix + ".bias", (cout,), -0.01, 0.01),
    }


def norm_params(seed: int, prefix: str, c: int) -> dict:
    return {
        prefix + ".weight": uniform(seed, prefix + ".weight", (c,), 0.9, 1.1),
        prefix + ".bias": uniform(seed, prefix + ".bias", (c,), -0.1, 0.1),
    }


def linear_params(seed: int, prefix: str, cin: int, cout: int) -> dict:
    a = 1.0 / math.sqrt(cin)
    return {
        prefix + ".weight": uniform(seed, prefix + ".weight", (cout, cin), -a, a),
        prefix + ".bias": uniform(seed, prefix + ".bias", (cout,), -0.01, 0.01),
    }


def resnet_params(seed: int, prefix: str, cin: int, cout: int, dims: int = 2) -> dict:
    p = {}
    p.update(norm_params(seed, prefix + ".norm1", cin))
    p.update(conv_params(seed, prefix + ".conv1", cin, cout, 3, dims))
    p.update(norm_params(seed, prefix + ".norm2", cout))
    p.update(conv_params(seed, prefix + ".conv2", cout, cout, 3, dims))
    if cin != cout:
        p.update(conv_params(seed, prefix + ".conv_shortcut", cin, cout, 1, dims))
    return p


def attention_params(seed: int, prefix: str, c: int) -> dict:
    p = {}
    p.update(norm_params(seed, prefix + ".group_norm", c))
    for name in ("to_q", "to_k", "to_v", "to_out.0"):
        p.update(linear_params(seed, prefix + "." + name, c, c))
    return p


def decoder_params(seed: int = 0,
                   widths=DECODER_WIDTHS,
                   latent_channels: int = LATENT_CHANNELS,
                   out_channels: int = OUT_CHANNELS,
                   resnets_per_block: int = RESNETS_PER_UP_BLOCK, dims: int = 2) -> dict:
    """All decoder tensors, diffusers names, f32 numpy arrays.  ``dims=3``
    gives the causal 3-D decoder: every conv kernel gets a time axis
    (3x3x3, and 1x1x1 for the skips), fan-in counted over all its taps."""
    c0 = widths[0]
    p = {}
    p.update(conv_params(seed, "conv_in", latent_channels, c0, 3, dims))
    p.update(resnet_params(seed, "mid_block.resnets.0", c0, c0, dims))
    p.update(attention_params(seed, "mid_block.attentions.0", c0))
    p.update(resnet_params(seed, "mid_block.resnets.1", c0, c0, dims))
    prev = c0
    for i, c in enumerate(widths):
        for j in range(resnets_per_block):
            p.update(resnet_params(seed, f"up_blocks.{i}.resnets.{j}", prev if j == 0 else c, c, dims))
        prev = c
        if i + 1 < len(widths):
            p.update(conv_params(seed, f"up_blocks.{i}.upsamplers.0.conv", c, c, 3, dims))
    p.update(norm_params(seed, "conv_norm_out", prev))
    p.update(conv_params(seed, "conv_out", prev, out_channels, 3, dims))
    return p


def latent(seed: int, h: int, w: int, channels: int = LATENT_CHANNELS) -> np.ndarray:
    return normal(seed, "latent", (channels, h, w))


def latent3d(seed: int, t: int, h: int, w: int, channels: int = LATENT_CHANNELS) -> np.ndarray:
    """A video latent [channels, t, h, w] for the causal 3-D decoder."""
    return normal(seed, "latent3d", (channels, t, h, w))


def activation(seed: int, name: str, shape) -> np.ndarray:
    """An N(0,1) layer input, e.g. for the single-layer sweep."""
    return normal(seed, name, tuple(shape))


def causal_stack_params(seed: int = 0, c: int = 128, layers: int = 4) -> dict:
    """The 3-D causal conv stack: ``layers`` x (3x3x3 conv c->c, GroupNorm32)."""
    p = {}
    for i in range(layers):
        p.update(conv_params(seed, f"stack.{i}.conv", c, c, 3, dims=3))
        p.update(norm_params(seed, f"stack.{i}.norm", c))
    return p
