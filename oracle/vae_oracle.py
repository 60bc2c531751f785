"""Plain CPU float64 oracle of the FLUX-class VAE decoder.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP kernels and imports
nothing from the product package.

Every function is the plain definition of one step, computed in float64 from
whatever (float32) arrays it is handed.  The only library routine used as a
step is the matrix product (``@``, BLAS ``dgemm``).  Nothing is blocked, fused
or reordered beyond what the definition states.

Sources (web pages):
  [handoff]  "VAE decode -> GPU handoff (FLUX/LTX render services)"
  [vae-doc]  docs.rs, cortiq-engine 0.7.7, module ``vae`` (struct index)
  [vae3d]    docs.rs, cortiq-engine 0.8.78, source of ``vae3d.rs``

Readings taken where the pages are silent (each is listed in the design
document with its reason):
  * padding of every 2-D conv is zero, ``k//2`` per side ([vae-doc] Conv2d,
    VaeConvRef "stride 1, pad k/2"); cross-correlation, no kernel flip
    ([vae3d] EncConv::apply, whose panel columns follow the weight's own
    (channel, ky, kx) order);
  * GroupNorm statistics are the mean and the biased (divide-by-n) variance
    over a group's channels and all positions ([vae3d] GroupNorm::apply);
  * the decoder output is returned raw (no clamp, no rescale);
  * attention's GroupNorm is GroupNorm(32, eps 1e-6, affine) like every other
    norm of the decoder;
  * the causal 3-D stack pads time at the front with two copies of frame 0,
    GroupNorm statistics span (C/32 channels) x T x H x W, and the residual
    add follows the second layer's GroupNorm+SiLU;
  * the causal 3-D decoder is the decoder chain with every 3x3 conv a causal
    3x3x3 conv, attention over all positions of the clip and upsampling in
    height and width only (the pages name the 3-D causal conv and its time
    padding, nothing more);
  * the tiled decode is the tiling of [vae3d] (VideoVae's tile schedule,
    cross-fade and crop) applied unchanged to this decoder, with the 8 pixels
    of a latent cell as the schedule's step.
"""
from __future__ import annotations

import math

import numpy as np

GROUPS = 32
EPS = 1e-6


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# elementwise steps
# ---------------------------------------------------------------------------

def denormalize(z, scaling_factor: float, shift_factor: float) -> np.ndarray:
    """Latent de-normalisation ``z / scaling_factor + shift_factor``.

    [vae-doc] VaeDecoder: the diffusers latent de-normalisation.  Divide, then
    add, as written there.
    """
    return _f64(z) / float(scaling_factor) + float(shift_factor)


def silu(x) -> np.ndarray:
    """``v / (1 + exp(-v))`` ([vae3d] fn silu; [vae-doc] module doc)."""
    x = _f64(x)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def upsample_nearest2x(x) -> np.ndarray:
    """Nearest x2: ``u[c, y, x] = t[c, y // 2, x // 2]`` ([vae-doc] VaeUpRef)."""
    x = _f64(x)
    return x.repeat(2, axis=-2).repeat(2, axis=-1)


def softmax_rows(s) -> np.ndarray:
    """Row softmax: subtract the row max, exponentiate, divide by the row sum
    ([vae3d] fn softmax_inplace)."""
    s = _f64(s)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# GroupNorm
# ---------------------------------------------------------------------------

def group_norm(x, gamma, beta, groups: int = GROUPS, eps: float = EPS) -> np.ndarray:
    """GroupNorm over ``x[C, ...]``.

    Group ``g`` holds channels ``[g*C/groups, (g+1)*C/groups)`` over every
    position.  ``y = (x - mean_g) / sqrt(var_g + eps) * gamma[c] + beta[c]``
    with the mean and the biased variance of the group, computed in two passes
    ([vae3d] GroupNorm::apply; [vae-doc] GroupNorm / VaeNormRef: eps 1e-6,
    affine, 32 groups).
    """
    x = _f64(x)
    c = x.shape[0]
    if c % groups:
        raise ValueError("channels must be divisible by the group count")
    xg = x.reshape(groups, -1)
    n = xg.shape[1]
    mean = xg.sum(axis=1) / n
    var = ((xg - mean[:, None]) ** 2).sum(axis=1) / n
    inv = 1.0 / np.sqrt(var + eps)
    y = ((xg - mean[:, None]) * inv[:, None]).reshape(x.shape)
    bshape = (c,) + (1,) * (x.ndim - 1)
    return y * _f64(gamma).reshape(bshape) + _f64(beta).reshape(bshape)


def group_norm_silu(x, gamma, beta) -> np.ndarray:
    return silu(group_norm(x, gamma, beta))


# ---------------------------------------------------------------------------
# convolutions
# ---------------------------------------------------------------------------

def conv2d(x, w, b) -> np.ndarray:
    """2-D convolution, stride 1, zero padding ``k//2`` on each side.

    ``y[o, i, j] = b[o] + sum_{c, dy, dx} w[o, c, dy, dx] * xp[c, i + dy, j + dx]``
    where ``xp`` is ``x`` with ``k//2`` zeros around it
    ([vae-doc] Conv2d and VaeConvRef: weight ``[oc, ic, k, k]`` row-major,
    bias ``[oc]``, stride 1, pad k/2; [vae3d] EncConv::apply for the tap order).
    The sum over ``c`` for one tap is a matrix product.
    """
    x = _f64(x)
    w = _f64(w)
    oc, ic, k, k2 = w.shape
    if k != k2 or x.shape[0] != ic:
        raise ValueError("shape mismatch")
    p = k // 2
    _, h, wd = x.shape
    xp = np.zeros((ic, h + 2 * p, wd + 2 * p))
    xp[:, p:p + h, p:p + wd] = x
    y = np.empty((oc, h, wd))
    y[:] = _f64(b)[:, None, None]
    for dy in range(k):
        for dx in range(k):
            window = xp[:, dy:dy + h, dx:dx + wd].reshape(ic, h * wd)
            tap = np.ascontiguousarray(w[:, :, dy, dx])           # [oc, ic]
            y += (tap @ window).reshape(oc, h, wd)
    return y


def conv3d_causal(x, w, b) -> np.ndarray:
    """Causal 3-D convolution over ``x[C, T, H, W]`` with a ``3x3x3`` kernel.

    Time is padded at the front with two copies of frame 0 and not at the
    back; height and width are zero-padded by 1 ([handoff] "The CPU VAE code"
    and "GPU plan": 3-D causal conv with causal padding on the time axis).
    ``y[o, t, i, j] = b[o] + sum_{c, dt, dy, dx} w[o, c, dt, dy, dx] *
    xp[c, t + dt, i + dy, j + dx]``.
    """
    x = _f64(x)
    w = _f64(w)
    oc, ic, kt, kh, kw = w.shape
    if (kt, kh, kw) != (3, 3, 3) or x.shape[0] != ic:
        raise ValueError("shape mismatch")
    _, t, h, wd = x.shape
    xp = np.zeros((ic, t + 2, h + 2, wd + 2))
    xp[:, 2:, 1:h + 1, 1:wd + 1] = x
    xp[:, 0, 1:h + 1, 1:wd + 1] = x[:, 0]
    xp[:, 1, 1:h + 1, 1:wd + 1] = x[:, 0]
    y = np.empty((oc, t, h, wd))
    y[:] = _f64(b)[:, None, None, None]
    for dt in range(3):
        for dy in range(3):
            for dx in range(3):
                window = xp[:, dt:dt + t, dy:dy + h, dx:dx + wd].reshape(ic, t * h * wd)
                tap = np.ascontiguousarray(w[:, :, dt, dy, dx])   # [oc, ic]
                y += (tap @ window).reshape(oc, t, h, wd)
    return y


# ---------------------------------------------------------------------------
# decoder blocks
# ---------------------------------------------------------------------------

def resnet(x, p: dict, prefix: str) -> np.ndarray:
    """``skip(x) + conv2(silu(norm2(conv1(silu(norm1(x))))))``; the skip is a
    1x1 conv when the block changes the channel count, else the identity
    ([vae-doc] VaeResnetRef)."""
    x = _f64(x)
    h = group_norm_silu(x, p[prefix + ".norm1.weight"], p[prefix + ".norm1.bias"])
    h = conv2d(h, p[prefix + ".conv1.weight"], p[prefix + ".conv1.bias"])
    h = group_norm_silu(h, p[prefix + ".norm2.weight"], p[prefix + ".norm2.bias"])
    h = conv2d(h, p[prefix + ".conv2.weight"], p[prefix + ".conv2.bias"])
    if prefix + ".conv_shortcut.weight" in p:
        skip = conv2d(x, p[prefix + ".conv_shortcut.weight"], p[prefix + ".conv_shortcut.bias"])
    else:
        skip = x
    return skip + h


def attention(x, p: dict, prefix: str) -> np.ndarray:
    """Mid-block single-head spatial attention ([vae-doc] VaeAttnRef).

    ``xn = GroupNorm(x)``; per token ``t`` (row-major over h, w):
    ``q_t = Wq xn[:, t] + bq`` (likewise k, v; Linear weights ``[c, c]``
    row-major out x in); ``P = softmax_rows(q . k^T / sqrt(c))``;
    ``o_t = sum_u P[t, u] v_u``; ``y[:, t] = x[:, t] + Wo o_t + bo``.
    """
    x = _f64(x)
    c, h, w = x.shape
    n = h * w
    xn = group_norm(x, p[prefix + ".group_norm.weight"], p[prefix + ".group_norm.bias"])
    tokens = xn.reshape(c, n).T                                   # [n, c], token-major

    def linear(name, inp):
        return inp @ _f64(p[prefix + "." + name + ".weight"]).T + _f64(p[prefix + "." + name + ".bias"])

    q = linear("to_q", tokens)
    k = linear("to_k", tokens)
    v = linear("to_v", tokens)
    probs = softmax_rows((q @ k.T) / math.sqrt(c))               # [n, n]
    o = probs @ v                                                 # [n, c]
    out = linear("to_out.0", o)                                   # [n, c]
    return x + out.T.reshape(c, h, w)


def decode(z, p: dict, scaling_factor: float, shift_factor: float,
           resnets_per_block: int = 3, return_trace: bool = False):
    """The whole decoder, in the execution order of [vae-doc] VaeChainArgs:
    de-normalise -> conv_in -> mid (resnet, attention, resnet) -> up blocks
    (resnets, then nearest x2 + conv on all but the last) -> GroupNorm + SiLU
    -> conv_out.  ``[16, h, w] -> [3, 8h, 8w]`` for four up blocks
    ([vae-doc] module doc, VaeDecoder, VaeUpRef).

    With ``return_trace`` a dict of every block output (float64) is returned
    as well, keyed by the block's name.
    """
    trace = {}
    x = conv2d(denormalize(z, scaling_factor, shift_factor), p["conv_in.weight"], p["conv_in.bias"])
    trace["conv_in"] = x
    x = resnet(x, p, "mid_block.resnets.0")
    trace["mid_block.resnets.0"] = x
    x = attention(x, p, "mid_block.attentions.0")
    trace["mid_block.attentions.0"] = x
    x = resnet(x, p, "mid_block.resnets.1")
    trace["mid_block.resnets.1"] = x
    i = 0
    while f"up_blocks.{i}.resnets.0.conv1.weight" in p:
        for j in range(resnets_per_block):
            name = f"up_blocks.{i}.resnets.{j}"
            x = resnet(x, p, name)
            trace[name] = x
        up = f"up_blocks.{i}.upsamplers.0.conv"
        if up + ".weight" in p:
            x = conv2d(upsample_nearest2x(x), p[up + ".weight"], p[up + ".bias"])
            trace[up] = x
        i += 1
    x = group_norm_silu(x, p["conv_norm_out.weight"], p["conv_norm_out.bias"])
    trace["conv_norm_out"] = x
    x = conv2d(x, p["conv_out.weight"], p["conv_out.bias"])
    trace["conv_out"] = x
    return (x, trace) if return_trace else x


def causal_stack(x, p: dict, layers: int = 4) -> np.ndarray:
    """The 3-D causal conv stack: each layer is ``SiLU(GroupNorm32(conv3d(x)))``
    and every second layer's output is added to the input of the pair:
    ``x <- x + L2(L1(x))`` ([handoff] "The CPU VAE code": LTX's 3-D causal
    conv decoder)."""
    x = _f64(x)
    for i in range(0, layers, 2):
        h = x
        for j in (i, i + 1):
            h = conv3d_causal(h, p[f"stack.{j}.conv.weight"], p[f"stack.{j}.conv.bias"])
            h = group_norm_silu(h, p[f"stack.{j}.norm.weight"], p[f"stack.{j}.norm.bias"])
        x = x + h
    return x


# ---------------------------------------------------------------------------
# the causal 3-D decoder
# ---------------------------------------------------------------------------

def pointwise_conv(x, w, b) -> np.ndarray:
    """A 1x1 (or 1x1x1) convolution of ``x[C, ...]``:
    ``y[o, ...] = b[o] + sum_c w[o, c] x[c, ...]`` (the channel-changing skip
    of a resnet, [vae-doc] VaeResnetRef)."""
    x = _f64(x)
    c = x.shape[0]
    w2 = _f64(w).reshape(w.shape[0], c)
    y = (w2 @ x.reshape(c, -1)).reshape((w.shape[0],) + x.shape[1:])
    return y + _f64(b).reshape((-1,) + (1,) * (x.ndim - 1))


def resnet_causal3d(x, p: dict, prefix: str) -> np.ndarray:
    """The resnet of ``resnet`` on a video ``x[C, T, H, W]`` with causal 3-D
    convs ([handoff] "The CPU VAE code": LTX's decoder is a 3-D causal conv
    decode); GroupNorm statistics span (C/32) x T x H x W."""
    x = _f64(x)
    h = group_norm_silu(x, p[prefix + ".norm1.weight"], p[prefix + ".norm1.bias"])
    h = conv3d_causal(h, p[prefix + ".conv1.weight"], p[prefix + ".conv1.bias"])
    h = group_norm_silu(h, p[prefix + ".norm2.weight"], p[prefix + ".norm2.bias"])
    h = conv3d_causal(h, p[prefix + ".conv2.weight"], p[prefix + ".conv2.bias"])
    if prefix + ".conv_shortcut.weight" in p:
        skip = pointwise_conv(x, p[prefix + ".conv_shortcut.weight"], p[prefix + ".conv_shortcut.bias"])
    else:
        skip = x
    return skip + h


def decode_causal3d(z, p: dict, scaling_factor: float, shift_factor: float,
                    resnets_per_block: int = 3) -> np.ndarray:
    """The decoder chain of ``decode`` on a video latent ``z[16, T, h, w]``
    with every 3x3 conv a causal 3x3x3 conv (time front-padded with two copies
    of frame 0; [handoff] "The CPU VAE code", "GPU plan"): the mid attention
    runs over all T*h*w positions (row-major over t, y, x), upsampling is
    nearest x2 in height and width only, and the output is ``[3, T, 8h, 8w]``.
    """
    x = conv3d_causal(denormalize(z, scaling_factor, shift_factor), p["conv_in.weight"], p["conv_in.bias"])
    x = resnet_causal3d(x, p, "mid_block.resnets.0")
    c, t, h, w = x.shape
    x = attention(x.reshape(c, t * h, w), p, "mid_block.attentions.0").reshape(c, t, h, w)
    x = resnet_causal3d(x, p, "mid_block.resnets.1")
    i = 0
    while f"up_blocks.{i}.resnets.0.conv1.weight" in p:
        for j in range(resnets_per_block):
            x = resnet_causal3d(x, p, f"up_blocks.{i}.resnets.{j}")
        up = f"up_blocks.{i}.upsamplers.0.conv"
        if up + ".weight" in p:
            x = conv3d_causal(upsample_nearest2x(x), p[up + ".weight"], p[up + ".bias"])
        i += 1
    x = group_norm_silu(x, p["conv_norm_out.weight"], p["conv_norm_out.bias"])
    return conv3d_causal(x, p["conv_out.weight"], p["conv_out.bias"])


# ---------------------------------------------------------------------------
# single outputs, for spot checks of full-size layers
# ---------------------------------------------------------------------------

def conv2d_at(x, w, b, o: int, i: int, j: int, upsample2x: bool = False) -> float:
    """One output ``y[o, i, j]`` of :func:`conv2d` (of the nearest-x2
    upsampled input when ``upsample2x``), summed directly from the definition
    without forming the whole output."""
    w = _f64(w)
    _, ic, k, _ = w.shape
    p = k // 2
    h, wd = x.shape[1], x.shape[2]
    if upsample2x:
        h, wd = 2 * h, 2 * wd
    acc = float(_f64(b)[o])
    for dy in range(k):
        for dx in range(k):
            yy, xx = i + dy - p, j + dx - p
            if 0 <= yy < h and 0 <= xx < wd:
                sy, sx = (yy // 2, xx // 2) if upsample2x else (yy, xx)
                acc += float(w[o, :, dy, dx] @ _f64(x[:, sy, sx]))
    return acc


def conv3d_causal_at(x, w, b, o: int, t: int, i: int, j: int) -> float:
    """One output ``y[o, t, i, j]`` of :func:`conv3d_causal`."""
    w = _f64(w)
    _, _, h, wd = x.shape
    acc = float(_f64(b)[o])
    for dt in range(3):
        tt = max(t + dt - 2, 0)
        for dy in range(3):
            for dx in range(3):
                yy, xx = i + dy - 1, j + dx - 1
                if 0 <= yy < h and 0 <= xx < wd:
                    acc += float(w[o, :, dt, dy, dx] @ _f64(x[:, tt, yy, xx]))
    return acc


# --------------------------------------------------------------------------
# Tiled decode ([vae3d]: the constants TILE and TILE_OVERLAP_MIN, split_tiles,
# VideoVae::decode_clip and blend).

TILE = 256           # pixel edge of a tile
TILE_OVERLAP_MIN = 64


def split_tiles(length: int, ratio: int, tile: int = TILE, overlap_min: int = TILE_OVERLAP_MIN):
    """Tile schedule along one pixel axis ([vae3d] split_tiles): every tile is
    exactly ``tile`` long, or one tile covers an axis no longer than that.
    The tile count is the smallest for which tiles overlapping by
    ``overlap_min`` cover the axis; the length left over is then handed to the
    overlaps ``ratio`` pixels (one latent cell) at a time, cycling from the
    first overlap, so the count stays and the overlaps grow.  Tile ``k + 1``
    starts ``tile - overlaps[k]`` after tile ``k``.  Returns
    ``(starts, lengths, overlaps)``."""
    if tile >= length:
        return [0], [length], []
    if overlap_min >= tile:
        raise ValueError("the overlap must be shorter than a tile")
    n = -(-length // tile)
    while n * tile < (n - 1) * overlap_min + length:
        n += 1
    overlaps = [overlap_min] * (n - 1)
    for step in range((n * tile - (n - 1) * overlap_min - length) // ratio):
        overlaps[step % (n - 1)] += ratio
    starts = [0]
    for ov in overlaps:
        starts.append(starts[-1] + tile - ov)
    return starts, [tile] * n, overlaps


def decode_tiled(z, p: dict, scaling_factor: float, shift_factor: float, tile: int = TILE,
                 overlap_min: int = TILE_OVERLAP_MIN, scale: int = 8, decode_fn=None) -> np.ndarray:
    """The decoder run tile by tile ([vae3d] VideoVae::decode_clip, blend):
    the output plane ``[8h, 8w]`` is cut by :func:`split_tiles` along each
    axis (step ``scale``, the pixels per latent cell), each tile's latent
    block is decoded on its own, and the tiles are assembled in row-major
    order.  A tile's first ``e`` rows (``e`` = its overlap with the tile above)
    become ``(1 - k/e) * above + (k/e) * tile`` for row ``k``, ``above`` being
    the last ``e`` rows of the tile above as decoded (before its own blends);
    then its first ``e'`` columns likewise with the last ``e'`` columns of the
    decoded tile to its left.  Each tile then drops its trailing overlap rows
    and columns (not the last tile of a column or row) and the rest is placed
    at the tile's start, so each output pixel comes from one tile.
    ``decode_fn(latent_block)`` decodes one block (default: :func:`decode`
    with the given parameters)."""
    if decode_fn is None:
        def decode_fn(block):
            return decode(block, p, scaling_factor, shift_factor)
    z = _f64(z)
    h, w = z.shape[-2:]
    H, W = h * scale, w * scale
    ys, yl, yo = split_tiles(H, scale, tile, overlap_min)
    xs, xl, xo = split_tiles(W, scale, tile, overlap_min)
    raw = {}
    for i, (y0, th) in enumerate(zip(ys, yl)):
        for j, (x0, tw) in enumerate(zip(xs, xl)):
            raw[i, j] = _f64(decode_fn(z[..., y0 // scale:(y0 + th) // scale, x0 // scale:(x0 + tw) // scale]))
    out = np.zeros(raw[0, 0].shape[:-2] + (H, W))
    for i in range(len(ys)):
        for j in range(len(xs)):
            t = raw[i, j].copy()
            th, tw = yl[i], xl[j]
            if i > 0:
                e = yo[i - 1]
                k = np.arange(e) / e
                above = raw[i - 1, j][..., yl[i - 1] - e:, :]
                t[..., :e, :] = above * (1 - k)[:, None] + t[..., :e, :] * k[:, None]
            if j > 0:
                e = xo[j - 1]
                k = np.arange(e) / e
                left = raw[i, j - 1][..., :, xl[j - 1] - e:]
                t[..., :, :e] = left * (1 - k) + t[..., :, :e] * k
            kh = th - yo[i] if i + 1 < len(ys) else th
            kw = tw - xo[j] if j + 1 < len(xs) else tw
            out[..., ys[i]:ys[i] + kh, xs[j]:xs[j] + kw] = t[..., :kh, :kw]
    return out
