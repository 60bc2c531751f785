"""GPU parity of the 256 x 256 decode (latent [16,32,32]) on every pixel, and
of each entry point fed with the oracle's own activations of that decode.

The oracle runs the whole decode once (float64, about half a minute of CPU
time) and keeps every block's output.  The RGB of the GPU decoder is compared
with it on every pixel.  Each per-layer case then takes the input a layer
sees inside the decode -- the oracle's activation, rounded to float32 once --
feeds it to the entry point, and compares the result with the oracle applied
to the same float32 input, so errors do not compound across layers.  Cases
cover every distinct layer shape of this decode: conv_in, the resnets at 32,
64, 128 and 256 (with and without the 1x1 shortcut), the mid attention (1024
tokens at c = 512), the three upsample convs, and norm_out + conv_out, under
each form of the 3x3 convs.

Bars: per layer max|gpu - ref| / max|ref| <= 1e-4; RGB cosine >= 0.99999 and
max|gpu - ref| <= 1e-3 max|ref|.
"""
import numpy as np
import pytest

import oracle
import vaegen

from gpu_helpers import LAYER_TOL, dev, host, nan_like, rel_err, rgb_metrics  # noqa: E402

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FORMS = ["winograd_4x4", "winograd_2x2", "implicit_gemm"]
S, T = vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_vae_decoder_amd import api as a
    a._lib_()
    return a


@pytest.fixture(scope="module")
def params():
    return vaegen.decoder_params(0)


@pytest.fixture(scope="module")
def trace(params):
    """The oracle's decode of latent [16,32,32], seed 0, with every block output."""
    z = vaegen.latent(0, 32, 32)
    rgb, tr = oracle.decode(z, params, S, T, return_trace=True)
    tr["latent"] = z
    tr["rgb"] = rgb
    return tr


@pytest.fixture(params=FORMS)
def form(api, request):
    before = api.get_conv3x3_algorithm()
    api.set_conv3x3_algorithm(request.param)
    yield request.param
    api.set_conv3x3_algorithm(before)


def f32(a):
    return np.asarray(a, dtype=np.float32)


def P(params, name):
    return dev(params[name])


def block_input(name):
    """The trace key of the activation a block reads."""
    order = ["conv_in", "mid_block.resnets.0", "mid_block.attentions.0", "mid_block.resnets.1"]
    for i in range(4):
        order += [f"up_blocks.{i}.resnets.{j}" for j in range(3)]
        if i < 3:
            order.append(f"up_blocks.{i}.upsamplers.0.conv")
    order.append("conv_norm_out")
    return order[order.index(name) - 1]


def test_decode_256_every_pixel(api, params, trace):
    d = api.Decoder({k: dev(v) for k, v in params.items()}, S, T)
    try:
        rgb = host(d.decode(dev(trace["latent"]), out=nan_like((3, 256, 256))))
    finally:
        d.close()
    ref = trace["rgb"]
    cos, mx = rgb_metrics(rgb, ref)
    assert cos >= 0.99999 and mx <= 1e-3 * np.abs(ref).max(), (cos, mx)


def test_conv_in_on_the_latent(api, params, trace):
    z = trace["latent"]
    y = api.conv_in(dev(z), P(params, "conv_in.weight"), P(params, "conv_in.bias"), S, T,
                    out=nan_like((512, 32, 32)))
    ref = oracle.conv2d(oracle.denormalize(z, S, T), params["conv_in.weight"], params["conv_in.bias"])
    assert rel_err(host(y), ref) <= LAYER_TOL


RESNETS = ["mid_block.resnets.0", "up_blocks.1.resnets.0", "up_blocks.2.resnets.0", "up_blocks.2.resnets.1",
           "up_blocks.3.resnets.0", "up_blocks.3.resnets.2"]


_refs = {}


def resnet_refs(params, trace, name):
    """The oracle's side of a resnet's layers on f32-rounded inputs (cached
    across the forms of the 3x3 convs)."""
    if name not in _refs:
        p = params
        x = f32(trace[block_input(name)])
        r = {"x": x}
        r["h1"] = oracle.group_norm_silu(x, p[name + ".norm1.weight"], p[name + ".norm1.bias"])
        r["c1"] = oracle.conv2d(f32(r["h1"]), p[name + ".conv1.weight"], p[name + ".conv1.bias"])
        h2 = f32(oracle.group_norm_silu(r["c1"], p[name + ".norm2.weight"], p[name + ".norm2.bias"]))
        r["h2"] = h2
        skip = x
        if name + ".conv_shortcut.weight" in p:
            r["s"] = oracle.conv2d(x, p[name + ".conv_shortcut.weight"], p[name + ".conv_shortcut.bias"])
            skip = f32(r["s"])
        r["skip"] = skip
        r["out"] = oracle.conv2d(h2, p[name + ".conv2.weight"], p[name + ".conv2.bias"]) + skip
        _refs[name] = r
    return _refs[name]


@pytest.mark.parametrize("name", RESNETS)
def test_resnet_layers_on_decode_activations(api, params, trace, form, name):
    # norm1 -> conv1 (+ the norm2 that follows, statistics from conv1's
    # epilogue) -> conv2 with the skip as its residual; the 1x1 shortcut where
    # the block changes width.  Every input is the oracle's, rounded to f32.
    p = params
    r = resnet_refs(params, trace, name)
    x = r["x"]
    c, h, w = x.shape
    g1 = api.groupnorm_silu(dev(x), P(p, name + ".norm1.weight"), P(p, name + ".norm1.bias"),
                            out=nan_like(x.shape))
    assert rel_err(host(g1), r["h1"]) <= LAYER_TOL

    co = p[name + ".conv1.weight"].shape[0]
    y1, z1 = api.conv2d_groupnorm_silu(dev(f32(r["h1"])), P(p, name + ".conv1.weight"), P(p, name + ".conv1.bias"),
                                       P(p, name + ".norm2.weight"), P(p, name + ".norm2.bias"),
                                       out=nan_like((co, h, w)), out_norm=nan_like((co, h, w)))
    g_y1 = host(y1)
    assert rel_err(g_y1, r["c1"]) <= LAYER_TOL
    # the normalisation of the conv's own output, statistics from its epilogue
    assert rel_err(host(z1), oracle.group_norm_silu(g_y1, p[name + ".norm2.weight"], p[name + ".norm2.bias"])) \
        <= LAYER_TOL

    if "s" in r:
        s = api.conv2d(dev(x), P(p, name + ".conv_shortcut.weight"), P(p, name + ".conv_shortcut.bias"),
                       out=nan_like((co, h, w)))
        assert rel_err(host(s), r["s"]) <= LAYER_TOL
    y2 = api.conv2d(dev(r["h2"]), P(p, name + ".conv2.weight"), P(p, name + ".conv2.bias"), residual=dev(r["skip"]),
                    out=nan_like((co, h, w)))
    assert rel_err(host(y2), r["out"]) <= LAYER_TOL


@pytest.mark.parametrize("streaming", [False, True])
def test_attention_on_decode_activations(api, params, trace, streaming):
    x = f32(trace["mid_block.resnets.0"])
    pre = "mid_block.attentions.0"
    pa = {k: v for k, v in params.items() if k.startswith(pre)}
    fn = api.attention_streaming if streaming else api.attention
    y = fn(dev(x), {k: dev(v) for k, v in pa.items()}, pre, out=nan_like(x.shape))
    if "attention" not in _refs:
        _refs["attention"] = oracle.attention(x, pa, pre)
    assert rel_err(host(y), _refs["attention"]) <= LAYER_TOL


@pytest.mark.parametrize("block", [0, 1, 2])
def test_upsample_conv_on_decode_activations(api, params, trace, form, block):
    name = f"up_blocks.{block}.upsamplers.0.conv"
    x = f32(trace[block_input(name)])
    c, h, w = x.shape
    y = api.conv2d(dev(x), P(params, name + ".weight"), P(params, name + ".bias"), upsample2x=True,
                   out=nan_like((c, 2 * h, 2 * w)))
    if name not in _refs:
        _refs[name] = oracle.conv2d(oracle.upsample_nearest2x(x), params[name + ".weight"], params[name + ".bias"])
    assert rel_err(host(y), _refs[name]) <= LAYER_TOL


def test_norm_out_and_conv_out_on_decode_activations(api, params, trace):
    x = f32(trace["up_blocks.3.resnets.2"])
    g = api.groupnorm_silu(dev(x), P(params, "conv_norm_out.weight"), P(params, "conv_norm_out.bias"),
                           out=nan_like(x.shape))
    n_ref = oracle.group_norm_silu(x, params["conv_norm_out.weight"], params["conv_norm_out.bias"])
    assert rel_err(host(g), n_ref) <= LAYER_TOL
    xn = f32(n_ref)
    y = api.conv2d(dev(xn), P(params, "conv_out.weight"), P(params, "conv_out.bias"), out=nan_like((3, 256, 256)))
    assert rel_err(host(y), oracle.conv2d(xn, params["conv_out.weight"], params["conv_out.bias"])) <= LAYER_TOL
