"""GPU parity: every entry point of libvae.so against the float64 oracle.

Inputs come from the seeded generator and are rounded to float32 once; both
sides see the same float32 values.  Outputs are pre-filled with NaN so that
an element the kernel never writes fails the comparison.

Bars (per layer): max|gpu - ref| / max|ref| <= 1e-4 over the layer output.
End to end (RGB): cosine >= 0.99999 and max|gpu - ref| <= 1e-3 * max|ref|.
Exact copies (upsample) must be bit-identical.
"""
import ctypes
import math
import os

import numpy as np
import pytest

import oracle
import vaegen

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_helpers import LAYER_TOL, conv_params, dev, host, nan_like, rel_err, rgb_metrics  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_vae_decoder_amd import api as a
    a._lib_()           # raises if libvae.so is missing: no fallback
    return a


FORMS = ["winograd_2x2", "implicit_gemm", "winograd_4x4"]


@pytest.fixture(params=FORMS)
def algo(api, request):
    """Runs the test with each form of the 3x3 convs, then restores the setting."""
    before = api.get_conv3x3_algorithm()
    api.set_conv3x3_algorithm(request.param)
    yield request.param
    api.set_conv3x3_algorithm(before)


def make_decoder(api, p, form, dims=2):
    """A decoder packed under `form` (the process-wide setting is restored)."""
    before = api.get_conv3x3_algorithm()
    api.set_conv3x3_algorithm(form)
    try:
        return api.Decoder({k: dev(v) for k, v in p.items()}, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR,
                           causal3d=dims == 3)
    finally:
        api.set_conv3x3_algorithm(before)


# ---------------------------------------------------------------------------
# 3x3 convolution (Winograd form and implicit GEMM, both on MFMA)
# ---------------------------------------------------------------------------

CONV_CASES = [
    # cin, cout, h, w
    (16, 128, 8, 8),        # conv_in width: TC=8 tiles
    (32, 64, 19, 37),       # ragged rows/cols, partial output block
    (24, 200, 13, 70),      # cin not a multiple of 8, cout not a multiple of 128
    (64, 64, 5, 5),         # image smaller than one tile
    (8, 128, 16, 16),       # TC=16 tiles
    (512, 512, 8, 8),       # long K (64 chunks)
    (128, 128, 64, 64),     # several full tiles
    (256, 128, 40, 33),     # the 256->128 shape, ragged
    (99, 96, 9, 11),        # K-split into 8/8/9 chunks, last channel chunk partial
]


@pytest.mark.parametrize("cin,cout,h,w", CONV_CASES)
def test_conv3x3(api, algo, cin, cout, h, w):
    x = vaegen.activation(1, f"x{cin}_{h}_{w}", (cin, h, w))
    wt, b = conv_params(1, f"c{cin}_{cout}", cin, cout, 3)
    y = api.conv2d(dev(x), dev(wt), dev(b), out=nan_like((cout, h, w)))
    assert rel_err(host(y), oracle.conv2d(x, wt, b)) <= LAYER_TOL


@pytest.mark.parametrize("cin,cout,h,w,res", [
    (32, 64, 9, 13, False),      # ragged source: partial output tiles
    (64, 128, 16, 16, False),
    (16, 32, 4, 4, False),
    (128, 128, 32, 32, False),
    (30, 40, 7, 5, False),       # last channel quad partial, cout not a multiple of 32
    (512, 64, 6, 10, False),     # long K on a small image: split along K
    (48, 96, 11, 9, True),       # residual added in the epilogue
])
def test_conv3x3_upsample_folded(api, algo, cin, cout, h, w, res):
    x = vaegen.activation(2, f"xu{cin}_{h}_{w}", (cin, h, w))
    wt, b = conv_params(2, f"cu{cin}_{cout}", cin, cout, 3)
    r = vaegen.activation(2, f"ru{cout}_{h}_{w}", (cout, 2 * h, 2 * w)) if res else None
    y = api.conv2d(dev(x), dev(wt), dev(b), upsample2x=True, residual=dev(r) if res else None,
                   out=nan_like((cout, 2 * h, 2 * w)))
    ref = oracle.conv2d(oracle.upsample_nearest2x(x), wt, b) + (r if res else 0.0)
    assert rel_err(host(y), ref) <= LAYER_TOL


@pytest.mark.parametrize("cin,cout,h,w", [(64, 64, 23, 17), (128, 128, 32, 32), (99, 96, 9, 11)])
def test_conv3x3_residual_epilogue(api, algo, cin, cout, h, w):
    x = vaegen.activation(3, "xr", (cin, h, w))
    r = vaegen.activation(3, "rr", (cout, h, w))
    wt, b = conv_params(3, "cr", cin, cout, 3)
    y = api.conv2d(dev(x), dev(wt), dev(b), residual=dev(r), out=nan_like((cout, h, w)))
    assert rel_err(host(y), oracle.conv2d(x, wt, b) + r) <= LAYER_TOL


@pytest.mark.parametrize("h,w", [(8, 8), (32, 32), (11, 7)])
def test_conv_in_with_denormalisation(api, h, w):
    z = vaegen.latent(4, h, w)
    wt, b = conv_params(4, "conv_in", 16, 512, 3)
    s, t = vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR
    y = api.conv_in(dev(z), dev(wt), dev(b), s, t, out=nan_like((512, h, w)))
    ref = oracle.conv2d(oracle.denormalize(z, s, t), wt, b)
    assert rel_err(host(y), ref) <= LAYER_TOL


# ---------------------------------------------------------------------------
# 1x1 conv (GEMM) and conv_out (direct)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cin,cout,h,w,res", [(256, 128, 32, 32, False), (512, 256, 16, 16, True),
                                               (37, 50, 11, 13, False), (64, 130, 9, 9, True)])
def test_conv1x1(api, cin, cout, h, w, res):
    x = vaegen.activation(5, "x1", (cin, h, w))
    wt, b = conv_params(5, "c1", cin, cout, 1)
    r = vaegen.activation(5, "r1", (cout, h, w)) if res else None
    y = api.conv2d(dev(x), dev(wt), dev(b), residual=dev(r) if res else None, out=nan_like((cout, h, w)))
    ref = oracle.conv2d(x, wt, b) + (r if res else 0.0)
    assert rel_err(host(y), ref) <= LAYER_TOL


@pytest.mark.parametrize("cin,cout,h,w", [(128, 3, 64, 64), (128, 3, 37, 45), (64, 1, 10, 130), (32, 4, 9, 9),
                                          (24, 2, 16, 16), (128, 3, 40, 256), (22, 3, 17, 131),
                                          (32, 3, 256, 2048)])
def test_conv_out_direct(api, cin, cout, h, w):
    # small images split the input channels across workgroups; the last case is big enough not to
    x = vaegen.activation(6, "xo", (cin, h, w))
    wt, b = conv_params(6, "co", cin, cout, 3)
    y = api.conv2d(dev(x), dev(wt), dev(b), out=nan_like((cout, h, w)))
    assert rel_err(host(y), oracle.conv2d(x, wt, b)) <= LAYER_TOL


def test_conv_out_direct_unaligned(api):
    # input and output views that start one float into their allocations
    cin, cout, h, w = 32, 3, 24, 256
    x = vaegen.activation(6, "xa", (cin, h, w))
    wt, b = conv_params(6, "ca", cin, cout, 3)
    xb = torch.empty(cin * h * w + 1, dtype=torch.float32, device="cuda")
    xb[1:].copy_(dev(x).flatten())
    yb = torch.full((cout * h * w + 1,), float("nan"), dtype=torch.float32, device="cuda")
    y = api.conv2d(xb[1:].view(cin, h, w), dev(wt), dev(b), out=yb[1:].view(cout, h, w))
    assert rel_err(host(y), oracle.conv2d(x, wt, b)) <= LAYER_TOL


# ---------------------------------------------------------------------------
# GroupNorm + SiLU, upsample
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape,silu,res", [((128, 32, 32), True, False), ((512, 16, 16), True, False),
                                            ((64, 7, 5), True, False), ((256, 9, 31), False, False),
                                            ((128, 3, 8, 8), True, True), ((32, 1, 1), True, False)])
def test_groupnorm_silu(api, shape, silu, res):
    x = vaegen.activation(7, "xg", shape) * 2.0 + 0.5
    n = vaegen.norm_params(7, "gn", shape[0])
    g, bt = n["gn.weight"], n["gn.bias"]
    r = vaegen.activation(7, "rg", shape) if res else None
    y = api.groupnorm_silu(dev(x), dev(g), dev(bt), silu=silu, residual=dev(r) if res else None,
                           out=nan_like(shape))
    ref = oracle.group_norm(x, g, bt)
    if silu:
        ref = oracle.silu(ref)
    if res:
        ref = ref + r
    assert rel_err(host(y), ref) <= LAYER_TOL


def test_groupnorm_in_place_and_large_mean(api):
    # a large common offset: the statistics must not cancel
    shape = (64, 40, 40)
    x = (vaegen.activation(8, "xm", shape) + 100.0).astype(np.float32)
    n = vaegen.norm_params(8, "gm", 64)
    t = dev(x)
    api.groupnorm_silu(t, dev(n["gm.weight"]), dev(n["gm.bias"]), out=t)
    ref = oracle.silu(oracle.group_norm(x, n["gm.weight"], n["gm.bias"]))
    assert rel_err(host(t), ref) <= LAYER_TOL


# conv -> GroupNorm(+SiLU) with the group statistics recorded by the conv:
# in the MFMA epilogue (whole 4-channel quads per group, not K-split), in the
# split-K reduction, or (fewer than 4 channels per group) by a separate pass.
CONV_GN_CASES = [
    # cin, cout, h, w, upsample, residual, silu
    (16, 128, 37, 45, False, False, True),    # epilogue records, TC=32, ragged rows and columns
    (16, 256, 40, 13, False, True, True),     # TC=16, 8 channels per group, residual
    (16, 512, 50, 7, False, False, False),    # TC=8, 16 channels per group, no SiLU
    (16, 128, 19, 21, True, True, True),      # folded upsample to 38x42 + residual
    (64, 128, 24, 20, False, False, True),    # K-split: records from the reduction (vector path)
    (64, 128, 23, 19, False, True, True),     # K-split, odd plane (scalar path), residual
    (16, 64, 21, 30, False, False, True),     # 2 channels per group: separate statistics pass
    (16, 128, 200, 330, False, False, True),  # 550 tiles: more records than the apply pass merges itself
]


@pytest.mark.parametrize("cin,cout,h,w,up,res,silu", CONV_GN_CASES)
def test_conv_groupnorm_silu(api, algo, cin, cout, h, w, up, res, silu):
    H, W = (2 * h, 2 * w) if up else (h, w)
    x = vaegen.activation(21, "xcg", (cin, h, w))
    wt, b = conv_params(21, f"ccg{cin}_{cout}", cin, cout, 3)
    n = vaegen.norm_params(21, "ncg", cout)
    g, bt = n["ncg.weight"], n["ncg.bias"]
    r = vaegen.activation(21, "rcg", (cout, H, W)) if res else None
    y, z = api.conv2d_groupnorm_silu(dev(x), dev(wt), dev(b), dev(g), dev(bt), silu=silu, upsample2x=up,
                                     residual=dev(r) if res else None, out=nan_like((cout, H, W)),
                                     out_norm=nan_like((cout, H, W)))
    yref = oracle.conv2d(oracle.upsample_nearest2x(x) if up else x, wt, b) + (r if res else 0.0)
    zref = oracle.group_norm(yref, g, bt)
    if silu:
        zref = oracle.silu(zref)
    assert rel_err(host(y), yref) <= LAYER_TOL
    assert rel_err(host(z), zref) <= LAYER_TOL


def test_conv_groupnorm_large_mean_in_place(api):
    # outputs with a common offset 50x their spread: per-tile centring keeps
    # the variance free of cancellation; z overwrites y
    cin, cout, h, w = 16, 128, 33, 70
    x = vaegen.activation(22, "xcm", (cin, h, w))
    wt, b = conv_params(22, "ccm", cin, cout, 3)
    b = (b + 50.0).astype(np.float32)
    n = vaegen.norm_params(22, "ncm", cout)
    t = nan_like((cout, h, w))
    y, z = api.conv2d_groupnorm_silu(dev(x), dev(wt), dev(b), dev(n["ncm.weight"]), dev(n["ncm.bias"]),
                                     out=t, out_norm=t)
    assert y.data_ptr() == z.data_ptr()
    zref = oracle.silu(oracle.group_norm(oracle.conv2d(x, wt, b), n["ncm.weight"], n["ncm.bias"]))
    assert rel_err(host(z), zref) <= LAYER_TOL


@pytest.mark.parametrize("c,h,w", [(128, 64, 64), (3, 5, 7), (16, 1, 1)])
def test_upsample_exact(api, c, h, w):
    x = vaegen.activation(9, "xu2", (c, h, w))
    y = api.upsample_nearest2x(dev(x), out=nan_like((c, 2 * h, 2 * w)))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), oracle.upsample_nearest2x(x).astype(np.float32))


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

# token counts: one partial key block (64, 63, 1), two blocks with a ragged
# tail (156), many full blocks (1024, 4096), many blocks with a ragged tail (1640)
@pytest.mark.parametrize("c,h,w", [(512, 8, 8), (64, 7, 9), (512, 32, 32), (128, 1, 1), (64, 12, 13),
                                   (512, 40, 41), (32, 64, 64)])
def test_attention(api, c, h, w):
    p = vaegen.attention_params(10, "a", c)
    x = vaegen.activation(10, "xa", (c, h, w))
    y = api.attention(dev(x), {k: dev(v) for k, v in p.items()}, "a", out=nan_like((c, h, w)))
    assert rel_err(host(y), oracle.attention(x, p, "a")) <= LAYER_TOL


def test_attention_peaked_softmax(api):
    # queries scaled up 40x: scores span hundreds, so each query's softmax is
    # dominated by a few keys spread over different key blocks
    c, h, w = 64, 20, 20
    p = vaegen.attention_params(13, "a", c)
    p["a.to_q.weight"] = (p["a.to_q.weight"] * 40.0).astype(np.float32)
    x = vaegen.activation(13, "xp", (c, h, w))
    y = api.attention(dev(x), {k: dev(v) for k, v in p.items()}, "a", out=nan_like((c, h, w)))
    assert rel_err(host(y), oracle.attention(x, p, "a")) <= LAYER_TOL


# streaming softmax: one query block with a partial key block (8x8, 7x9, 3x5),
# a single token, ragged tails over several key blocks (12x13, 40x41), key
# ranges split across workgroups and merged (32x32, 64x64: 16 query blocks or
# fewer), and every supported width
@pytest.mark.parametrize("c,h,w", [(128, 8, 8), (128, 7, 9), (512, 3, 5), (128, 1, 1), (256, 12, 13),
                                   (512, 40, 41), (512, 32, 32), (128, 64, 64), (256, 33, 1)])
def test_attention_streaming(api, c, h, w):
    p = vaegen.attention_params(14, "a", c)
    x = vaegen.activation(14, "xs", (c, h, w))
    y = api.attention_streaming(dev(x), {k: dev(v) for k, v in p.items()}, "a", out=nan_like((c, h, w)))
    assert rel_err(host(y), oracle.attention(x, p, "a")) <= LAYER_TOL


def test_attention_streaming_peaked_softmax(api):
    # queries scaled up 40x: each query's maximum moves between key blocks,
    # so the running maximum and the output are rescaled many times
    c, h, w = 128, 20, 20
    p = vaegen.attention_params(13, "a", c)
    p["a.to_q.weight"] = (p["a.to_q.weight"] * 40.0).astype(np.float32)
    x = vaegen.activation(13, "xp", (c, h, w))
    y = api.attention_streaming(dev(x), {k: dev(v) for k, v in p.items()}, "a", out=nan_like((c, h, w)))
    assert rel_err(host(y), oracle.attention(x, p, "a")) <= LAYER_TOL


def test_attention_streaming_key_bias_cancels(api):
    # a large key bias shifts every score of a query by q . b_k, which the
    # softmax removes; the streaming form never adds it
    c, h, w = 128, 9, 10
    p = vaegen.attention_params(15, "a", c)
    p["a.to_k.bias"] = (p["a.to_k.bias"] * 500.0 + 3.0).astype(np.float32)
    x = vaegen.activation(15, "xb", (c, h, w))
    y = api.attention_streaming(dev(x), {k: dev(v) for k, v in p.items()}, "a", out=nan_like((c, h, w)))
    assert rel_err(host(y), oracle.attention(x, p, "a")) <= LAYER_TOL


# ---------------------------------------------------------------------------
# causal 3-D conv
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cin,cout,t,h,w", [(16, 32, 5, 6, 10), (128, 128, 4, 16, 16), (24, 130, 3, 9, 35)])
def test_conv3d_causal(api, algo, cin, cout, t, h, w):
    x = vaegen.activation(11, "x3", (cin, t, h, w))
    wt, b = conv_params(11, "c3", cin, cout, 3, dims=3)
    y = api.conv3d_causal(dev(x), dev(wt), dev(b), out=nan_like((cout, t, h, w)))
    assert rel_err(host(y), oracle.conv3d_causal(x, wt, b)) <= LAYER_TOL


@pytest.mark.parametrize("cin,cout,t,h,w,res,silu", [(16, 128, 3, 9, 13, False, True),
                                                     (128, 128, 4, 16, 16, True, True),
                                                     (64, 256, 2, 7, 33, True, False)])
def test_conv3d_causal_groupnorm_silu(api, cin, cout, t, h, w, res, silu):
    # GroupNorm statistics from the causal conv's epilogue (or its K-split
    # reduction on these small shapes), residual added after the SiLU
    x = vaegen.activation(23, "x3g", (cin, t, h, w))
    wt, b = conv_params(23, "c3g", cin, cout, 3, dims=3)
    n = vaegen.norm_params(23, "n3g", cout)
    r = vaegen.activation(23, "r3g", (cout, t, h, w)) if res else None
    y, z = api.conv3d_causal_groupnorm_silu(dev(x), dev(wt), dev(b), dev(n["n3g.weight"]), dev(n["n3g.bias"]),
                                            silu=silu, residual=dev(r) if res else None,
                                            out=nan_like((cout, t, h, w)), out_norm=nan_like((cout, t, h, w)))
    yref = oracle.conv3d_causal(x, wt, b)
    zref = oracle.group_norm(yref, n["n3g.weight"], n["n3g.bias"])
    if silu:
        zref = oracle.silu(zref)
    if res:
        zref = zref + r
    assert rel_err(host(y), yref) <= LAYER_TOL
    assert rel_err(host(z), zref) <= LAYER_TOL


def test_causal_stack_small(api):
    c = 64
    p = vaegen.causal_stack_params(12, c=c)
    x = vaegen.activation(12, "xs", (c, 5, 12, 12))
    P = {k: dev(v) for k, v in p.items()}
    h = dev(x)
    for i in (0, 2):
        cur = h
        for j in (i, i + 1):
            cur = api.conv3d_causal(cur, P[f"stack.{j}.conv.weight"], P[f"stack.{j}.conv.bias"])
            cur = api.groupnorm_silu(cur, P[f"stack.{j}.norm.weight"], P[f"stack.{j}.norm.bias"],
                                     residual=h if j == i + 1 else None, out=cur)
        h = cur
    ref = oracle.causal_stack(x, p)
    assert rel_err(host(h), ref) <= LAYER_TOL
    # the same stack through the conv -> GroupNorm entry point, in place
    h2 = dev(x)
    for i in (0, 2):
        cur = h2
        for j in (i, i + 1):
            out = nan_like(cur.shape)
            _, cur = api.conv3d_causal_groupnorm_silu(cur, P[f"stack.{j}.conv.weight"], P[f"stack.{j}.conv.bias"],
                                                      P[f"stack.{j}.norm.weight"], P[f"stack.{j}.norm.bias"],
                                                      residual=h2 if j == i + 1 else None, out=out, out_norm=out)
        h2 = cur
    assert rel_err(host(h2), ref) <= LAYER_TOL


# ---------------------------------------------------------------------------
# whole decoder
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def params():
    return vaegen.decoder_params(0)


@pytest.fixture(scope="module")
def decoder(api, params):
    d = api.Decoder({k: dev(v) for k, v in params.items()}, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
    yield d
    d.close()


def test_decode_64(decoder, params):
    z = vaegen.latent(0, 8, 8)
    rgb = decoder.decode(dev(z), out=nan_like((3, 64, 64)))
    ref = oracle.decode(z, params, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
    cos, mx = rgb_metrics(host(rgb), ref)
    assert cos >= 0.99999 and mx <= 1e-3 * np.abs(ref).max(), (cos, mx)


def test_decode_ragged_latent(decoder, params):
    z = vaegen.latent(5, 5, 3)
    rgb = decoder.decode(dev(z), out=nan_like((3, 40, 24)))
    ref = oracle.decode(z, params, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
    cos, mx = rgb_metrics(host(rgb), ref)
    assert cos >= 0.99999 and mx <= 1e-3 * np.abs(ref).max(), (cos, mx)


@pytest.mark.parametrize("h,w", [(1, 1), (1, 7), (3, 1)])
def test_decode_degenerate_latent(decoder, params, h, w):
    # one token (the attention's softmax over a single key), one latent row,
    # one latent column: every layer smaller than a tile in at least one axis
    z = vaegen.latent(9, h, w)
    rgb = decoder.decode(dev(z), out=nan_like((3, 8 * h, 8 * w)))
    ref = oracle.decode(z, params, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
    cos, mx = rgb_metrics(host(rgb), ref)
    assert cos >= 0.99999 and mx <= 1e-3 * np.abs(ref).max(), (cos, mx)


def test_decode_1024_against_stored_oracle(decoder):
    # stored oracle values (tests/golden/make_golden.py): a lattice of rows and
    # columns covering every residue mod 4, the border rows and columns and
    # 16384 random pixels, plus the whole image's max|ref| and L2 norm
    path = os.path.join(GOLDEN, "decode_1024.npz")
    g = np.load(path)
    assert int(g["seed"]) == 0
    z = vaegen.latent(0, 128, 128)
    rgb = host(decoder.decode(dev(z), out=nan_like(tuple(g["shape"]))))
    rows, cols, pix = g["rows"], g["cols"], g["pixels"]
    assert {int(r) % 4 for r in rows} == {0, 1, 2, 3} and {int(c) % 4 for c in cols} == {0, 1, 2, 3}
    got = np.concatenate([rgb[:, rows][:, :, cols].ravel(), rgb[:, 0, :].ravel(), rgb[:, -1, :].ravel(),
                          rgb[:, :, 0].ravel(), rgb[:, :, -1].ravel(), rgb[pix[:, 0], pix[:, 1], pix[:, 2]]])
    ref = np.concatenate([g["lattice"].ravel(), g["first_row"].ravel(), g["last_row"].ravel(),
                          g["first_col"].ravel(), g["last_col"].ravel(), g["pixel_values"]])
    cos, mx = rgb_metrics(got, ref)
    assert cos >= 0.99999 and mx <= 1e-3 * float(g["max_abs"]), (cos, mx)
    # the whole image: finite, and its norm matches the oracle's
    assert np.isfinite(rgb).all()
    assert abs(math.sqrt((rgb * rgb).sum()) / float(g["l2"]) - 1.0) < 1e-4


@pytest.fixture(scope="module")
def decoder_2x2(api, params):
    """GroupNorm on load needs a form whose kernels normalise while loading."""
    d = make_decoder(api, params, "winograd_2x2")
    yield d
    d.close()


@pytest.mark.parametrize("h,w", [(8, 8), (5, 3), (32, 32)])
def test_decode_with_groupnorm_on_load(decoder_2x2, params, h, w):
    # the optional fused path: GroupNorm + SiLU applied while each conv loads
    z = vaegen.latent(6, h, w)
    decoder_2x2.set_groupnorm_fusion(True)
    try:
        rgb = decoder_2x2.decode(dev(z), out=nan_like((3, 8 * h, 8 * w)))
        got = host(rgb)
    finally:
        decoder_2x2.set_groupnorm_fusion(False)
    ref = oracle.decode(z, params, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
    cos, mx = rgb_metrics(got, ref)
    assert cos >= 0.99999 and mx <= 1e-3 * np.abs(ref).max(), (cos, mx)


@pytest.fixture(scope="module")
def decoder_streaming(api, params):
    d = api.Decoder({k: dev(v) for k, v in params.items()}, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
    d.set_attention("streaming")
    assert d.get_attention() == "streaming"
    yield d
    d.close()


@pytest.mark.parametrize("h,w", [(8, 8), (5, 3), (1, 1), (32, 32)])
def test_decode_with_streaming_attention(decoder_streaming, params, h, w):
    z = vaegen.latent(10, h, w)
    rgb = decoder_streaming.decode(dev(z), out=nan_like((3, 8 * h, 8 * w)))
    ref = oracle.decode(z, params, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
    cos, mx = rgb_metrics(host(rgb), ref)
    assert cos >= 0.99999 and mx <= 1e-3 * np.abs(ref).max(), (cos, mx)


def test_decode_streaming_graph_replay_matches_eager(decoder_streaming):
    z = dev(vaegen.latent(11, 12, 12))
    e = decoder_streaming.decode(z).cpu()
    out = torch.empty((3, 96, 96), dtype=torch.float32, device="cuda")
    decoder_streaming.set_graph(True)
    try:
        for _ in range(3):
            decoder_streaming.decode(z, out=out)
            assert torch.equal(out.cpu(), e)
            torch.cuda.synchronize()
            _ = (torch.randn(4096, device="cuda") * 2).sum().item()
    finally:
        decoder_streaming.set_graph(False)


def test_decode_is_deterministic(decoder):
    z = dev(vaegen.latent(1, 16, 16))
    a = decoder.decode(z).cpu()
    b = decoder.decode(z).cpu()
    assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# the causal 3-D decoder
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def params3d():
    return vaegen.decoder_params(0, dims=3)


@pytest.fixture(scope="module")
def decoder3d(api, params3d):
    d = api.Decoder({k: dev(v) for k, v in params3d.items()}, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR,
                    causal3d=True)
    yield d
    d.close()


# clips: one frame, three frames, a ragged spatial size over two frames
@pytest.mark.parametrize("t,h,w", [(1, 4, 4), (3, 4, 4), (2, 5, 3)])
def test_decode_causal3d(decoder3d, params3d, t, h, w):
    z = vaegen.latent3d(2, t, h, w)
    rgb = decoder3d.decode(dev(z), out=nan_like((3, t, 8 * h, 8 * w)))
    ref = oracle.decode_causal3d(z, params3d, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
    cos, mx = rgb_metrics(host(rgb), ref)
    assert cos >= 0.99999 and mx <= 1e-3 * np.abs(ref).max(), (cos, mx)


@pytest.mark.parametrize("form,dims,fused", [(f, d, g) for f in FORMS for d in (2, 3) for g in (False, True)
                                             if not (g and f == "winograd_4x4")])
def test_decode_form(api, params, params3d, form, dims, fused):
    # a decoder keeps the form it was created under (the setting is restored
    # before decoding), with and without GroupNorm on load
    p = params if dims == 2 else params3d
    d = make_decoder(api, p, form, dims)
    try:
        d.set_groupnorm_fusion(fused)
        if dims == 2:
            z = vaegen.latent(7, 5, 6)
            rgb = d.decode(dev(z), out=nan_like((3, 40, 48)))
            ref = oracle.decode(z, p, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
        else:
            z = vaegen.latent3d(7, 2, 4, 5)
            rgb = d.decode(dev(z), out=nan_like((3, 2, 32, 40)))
            ref = oracle.decode_causal3d(z, p, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
        got = host(rgb)
    finally:
        d.close()
    cos, mx = rgb_metrics(got, ref)
    assert cos >= 0.99999 and mx <= 1e-3 * np.abs(ref).max(), (cos, mx)


def test_groupnorm_on_load_needs_a_loading_form(api, params):
    # the F(4x4) Winograd kernel does not normalise on load: the switch is refused
    d = make_decoder(api, params, "winograd_4x4")
    try:
        with pytest.raises(api.VaeError, match="F\\(4x4\\)"):
            d.set_groupnorm_fusion(True)
        z = vaegen.latent(8, 4, 4)           # and the decoder still works
        got = host(d.decode(dev(z), out=nan_like((3, 32, 32))))
    finally:
        d.close()
    ref = oracle.decode(z, params, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
    cos, mx = rgb_metrics(got, ref)
    assert cos >= 0.99999 and mx <= 1e-3 * np.abs(ref).max(), (cos, mx)


@pytest.fixture(scope="module")
def decoder3d_2x2(api, params3d):
    d = make_decoder(api, params3d, "winograd_2x2", dims=3)
    yield d
    d.close()


def test_decode_causal3d_with_groupnorm_on_load(decoder3d_2x2, params3d):
    z = vaegen.latent3d(3, 2, 4, 4)
    decoder3d_2x2.set_groupnorm_fusion(True)
    try:
        got = host(decoder3d_2x2.decode(dev(z), out=nan_like((3, 2, 32, 32))))
    finally:
        decoder3d_2x2.set_groupnorm_fusion(False)
    ref = oracle.decode_causal3d(z, params3d, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
    cos, mx = rgb_metrics(got, ref)
    assert cos >= 0.99999 and mx <= 1e-3 * np.abs(ref).max(), (cos, mx)


def test_decode_causal3d_with_streaming_attention(decoder3d, params3d):
    # attention over all t*h*w positions of the clip
    z = vaegen.latent3d(4, 3, 4, 5)
    decoder3d.set_attention("streaming")
    try:
        got = host(decoder3d.decode(dev(z), out=nan_like((3, 3, 32, 40))))
    finally:
        decoder3d.set_attention("split_softmax")
    ref = oracle.decode_causal3d(z, params3d, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
    cos, mx = rgb_metrics(got, ref)
    assert cos >= 0.99999 and mx <= 1e-3 * np.abs(ref).max(), (cos, mx)


def test_decode_causal3d_rejects_2d_calls(api, decoder3d, decoder):
    lib = api._lib_()
    nb = ctypes.c_size_t()
    assert lib.vae_decoder_workspace_bytes(decoder3d._h, 4, 4, ctypes.byref(nb)) != 0
    assert lib.vae_decoder3d_workspace_bytes(decoder._h, 1, 4, 4, ctypes.byref(nb)) != 0
    assert "3-D" in lib.vae_last_error().decode()


def test_decode_graph_replay_matches_eager(decoder):
    # two latents through one input buffer: every replay is bit-identical to the
    # eager decode of the buffer's current contents, with eager work in between
    z1, z2 = dev(vaegen.latent(7, 16, 16)), dev(vaegen.latent(8, 16, 16))
    e1, e2 = decoder.decode(z1).cpu(), decoder.decode(z2).cpu()
    zin = torch.empty_like(z1)
    out = torch.empty((3, 128, 128), dtype=torch.float32, device="cuda")
    decoder.set_graph(True)
    try:
        for _ in range(3):
            zin.copy_(z1)
            decoder.decode(zin, out=out)
            assert torch.equal(out.cpu(), e1)
            torch.cuda.synchronize()
            _ = (torch.randn(4096, device="cuda") * 2).sum().item()
            zin.copy_(z2)
            decoder.decode(zin, out=out)
            assert torch.equal(out.cpu(), e2)
    finally:
        decoder.set_graph(False)


def test_decode3d_graph_replay_matches_eager(decoder3d):
    z = dev(vaegen.latent3d(9, 2, 4, 4))
    e = decoder3d.decode(z).cpu()
    out = torch.empty((3, 2, 32, 32), dtype=torch.float32, device="cuda")
    decoder3d.set_graph(True)
    try:
        for _ in range(3):
            decoder3d.decode(z, out=out)
            assert torch.equal(out.cpu(), e)
            torch.cuda.synchronize()
    finally:
        decoder3d.set_graph(False)
