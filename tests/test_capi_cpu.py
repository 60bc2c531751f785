"""The C ABI without a GPU: the library loads, exports every function that
include/vae.h declares, and rejects bad arguments before any launch."""
import ctypes
import os
import re
from ctypes import byref, c_int32, c_size_t, c_void_p

import pytest

from diffusion_vae_decoder_amd import _lib
from diffusion_vae_decoder_amd._lib import (VAE_ERR_INVALID_ARG, VAE_ERR_UNSUPPORTED, VAE_ERR_WORKSPACE, VAE_OK,
                                            VaeAttn, VaeConv, VaeNorm, VaeResnet, VaeUp, VaeWeights)

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "vae.h")
FAKE = 0x7F0000000000          # a non-NULL "device" pointer; never dereferenced on these paths
NULL = None


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vae_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), set(names) ^ set(_lib.SIGNATURES)


def test_abi_version(lib):
    assert lib.vae_abi_version() == _lib.ABI_VERSION


def test_the_named_library_is_loaded(lib):
    # VAE_LIBRARY selects the sanitizer build; then ASan must be live in the process
    name = os.environ.get("VAE_LIBRARY", "libvae.so")
    assert os.path.basename(_lib.LIB_PATH) == name
    if name == "libvae_san.so":
        assert hasattr(ctypes.CDLL(None), "__asan_report_load4")


def conv(cout, cin, k, w=FAKE, b=FAKE):
    return VaeConv(w, b, cout, cin, k)


def err(lib):
    return lib.vae_last_error().decode()


def packed_bytes(cout, cin, kt=1):
    """Room the per-layer 3x3 entry points reserve for packed weights: the
    largest of the implicit GEMM's layout (128-channel output blocks x chunks
    of 4 input channels x 36 x 128 floats), the F(2x2) Winograd form's
    (32-channel output blocks x chunks of 4 input channels x 64 lanes x 32
    floats: 16 transform points per output and input channel) and the F(4x4)
    form's (32-channel output blocks x chunks of 4 input channels x 2 row
    blocks x 10 float4s x 64 lanes: 36 transform points, padded to 40, per
    output and input channel)."""
    direct = ((cout + 127) // 128) * kt * ((cin + 3) // 4) * 36 * 128 * 4
    wino = ((cout + 31) // 32) * kt * ((cin + 3) // 4) * 64 * 32 * 4
    wino4 = ((cout + 31) // 32) * kt * ((cin + 3) // 4) * 2 * 10 * 64 * 16
    return max(direct, wino, wino4)


def test_conv3x3_algorithm_setting(lib):
    assert lib.vae_get_conv3x3_algorithm() == 2            # Winograd F(4x4) by default
    assert lib.vae_set_conv3x3_algorithm(3) == VAE_ERR_INVALID_ARG and "algorithm" in err(lib)
    assert lib.vae_set_conv3x3_algorithm(-1) == VAE_ERR_INVALID_ARG
    assert lib.vae_get_conv3x3_algorithm() == 2
    try:
        assert lib.vae_set_conv3x3_algorithm(0) == VAE_OK   # Winograd F(2x2)
        assert lib.vae_get_conv3x3_algorithm() == 0
        w, keep = fake_weights()
        nb = c_size_t()
        assert lib.vae_decoder_pack_bytes(byref(w), byref(nb)) == VAE_OK
        assert 83_000_000 * 4 < nb.value < 84_000_000 * 4   # 16 transform points per weight (32 per 2 on x2 input)
        assert lib.vae_set_conv3x3_algorithm(1) == VAE_OK
        assert lib.vae_get_conv3x3_algorithm() == 1
        # the per-layer workspace covers either form, whichever is set
        ws = c_size_t()
        assert lib.vae_conv2d_workspace_bytes(byref(conv(64, 32, 3)), 8, 8, 0, byref(ws)) == VAE_OK
        assert ws.value >= packed_bytes(64, 32)
        # decoders pack for the form set when they are created
        w, keep = fake_weights()
        nb = c_size_t()
        assert lib.vae_decoder_pack_bytes(byref(w), byref(nb)) == VAE_OK
        assert 49_000_000 * 4 < nb.value < 52_000_000 * 4   # raw-sized implicit-GEMM packing
    finally:
        assert lib.vae_set_conv3x3_algorithm(2) == VAE_OK


def test_conv2d_validation(lib):
    c = conv(64, 32, 3)
    ws = c_size_t()
    assert lib.vae_conv2d_workspace_bytes(byref(c), 8, 8, 0, byref(ws)) == VAE_OK
    # the packed weights, then split-K partial sums (whole [64, 8, 8] slices)
    assert ws.value >= packed_bytes(64, 32) == 2 * 8 * 2 * 10 * 64 * 16    # the F(4x4) packing is the largest
    assert (ws.value - packed_bytes(64, 32)) % (64 * 8 * 8 * 4) == 0
    # a small shape: the 32x32 conv with 512 channels is K-split, so partial sums are added
    big = conv(512, 512, 3)
    w1, w2 = c_size_t(), c_size_t()
    assert lib.vae_conv2d_workspace_bytes(byref(big), 32, 32, 0, byref(w1)) == VAE_OK
    assert lib.vae_conv2d_workspace_bytes(byref(big), 256, 256, 0, byref(w2)) == VAE_OK
    packed = packed_bytes(512, 512)
    assert w2.value == packed and w1.value == packed + 16 * 512 * 32 * 32 * 4
    assert lib.vae_conv2d_workspace_bytes(byref(big), 0, 32, 0, byref(w1)) == VAE_ERR_INVALID_ARG
    args = lambda **k: dict(dict(x=FAKE, cin=32, h=8, w=8, conv=byref(c), up=0, res=NULL, y=FAKE + 4096,
                                 ws=FAKE + 8192, nb=ws.value, s=NULL), **k)

    def call(a):
        return lib.vae_conv2d(a["x"], a["cin"], a["h"], a["w"], a["conv"], a["up"], a["res"], a["y"], a["ws"],
                              a["nb"], a["s"])
    assert call(args(x=NULL)) == VAE_ERR_INVALID_ARG
    assert call(args(cin=31)) == VAE_ERR_INVALID_ARG and "input channels" in err(lib)
    assert call(args(h=0)) == VAE_ERR_INVALID_ARG
    assert call(args(w=-3)) == VAE_ERR_INVALID_ARG
    assert call(args(nb=ws.value - 1)) == VAE_ERR_WORKSPACE
    assert call(args(ws=NULL)) == VAE_ERR_WORKSPACE
    assert call(args(y=FAKE)) == VAE_ERR_INVALID_ARG and "alias" in err(lib)
    bad = conv(64, 32, 5)
    assert call(args(conv=byref(bad))) == VAE_ERR_UNSUPPORTED
    nob = conv(64, 32, 3, b=NULL)
    assert call(args(conv=byref(nob))) == VAE_ERR_INVALID_ARG
    one = conv(64, 32, 1)
    assert call(args(conv=byref(one), up=1)) == VAE_ERR_UNSUPPORTED
    assert call(args(h=1 << 16, w=1 << 16)) == VAE_ERR_UNSUPPORTED


def test_conv_in_and_3d_validation(lib):
    c = conv(512, 16, 3)
    nb = c_size_t()
    assert lib.vae_conv2d_workspace_bytes(byref(c), 8, 8, 0, byref(nb)) == VAE_OK
    assert lib.vae_conv_in(FAKE, 16, 8, 8, byref(c), 0.0, 0.1, FAKE + 64, FAKE + 128, nb.value, NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_conv_in(FAKE, 16, 8, 8, byref(conv(512, 16, 1)), 0.36, 0.1, FAKE + 64, FAKE, 0, NULL) == VAE_ERR_UNSUPPORTED
    c3 = conv(128, 128, 3)
    assert lib.vae_conv3d_causal_workspace_bytes(byref(c3), 3, 8, 8, byref(nb)) == VAE_OK
    packed = packed_bytes(128, 128, 3)
    assert nb.value >= packed and (nb.value - packed) % (128 * 3 * 64 * 4) == 0
    full = c_size_t()
    assert lib.vae_conv3d_causal_workspace_bytes(byref(c3), 17, 256, 256, byref(full)) == VAE_OK
    assert full.value == packed                          # big enough to fill the GPU: no split
    assert lib.vae_conv3d_causal(FAKE, 128, 0, 8, 8, byref(c3), FAKE + 64, FAKE, nb.value, NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_conv3d_causal(FAKE, 128, 3, 8, 8, byref(c3), FAKE + 64, FAKE, nb.value - 4, NULL) == VAE_ERR_WORKSPACE
    assert lib.vae_conv3d_causal(FAKE, 64, 3, 8, 8, byref(c3), FAKE + 64, FAKE, nb.value, NULL) == VAE_ERR_INVALID_ARG


def test_conv_groupnorm_validation(lib):
    c = conv(128, 16, 3)
    nb = c_size_t()
    assert lib.vae_conv2d_groupnorm_workspace_bytes(byref(c), 37, 45, 0, byref(nb)) == VAE_OK
    # packed weights, 32 groups x 16-byte records for the form writing the most
    # (the implicit GEMM's 2 x 10 blocks of 4 x 32 outputs; F(2x2): 2 x 5, F(4x4):
    # 1 x 3), GroupNorm partials (sums, shift) and per-group (mean, rstd)
    assert nb.value == packed_bytes(128, 16) + 20 * 32 * 16 + 32 * 16 + 32 * 8 + 32 * 8
    c64 = conv(64, 16, 3)                        # 2 channels per group: no records, a statistics pass
    n64 = c_size_t()
    assert lib.vae_conv2d_groupnorm_workspace_bytes(byref(c64), 37, 45, 0, byref(n64)) == VAE_OK
    assert n64.value == 256 * ((packed_bytes(64, 16) + 255) // 256) + 32 * 16 + 32 * 8 + 32 * 8
    assert lib.vae_conv2d_groupnorm_workspace_bytes(byref(conv(100, 16, 3)), 8, 8, 0, byref(nb)) == VAE_ERR_UNSUPPORTED
    assert lib.vae_conv2d_groupnorm_workspace_bytes(byref(conv(128, 16, 1)), 8, 8, 0, byref(nb)) == VAE_ERR_UNSUPPORTED
    n = VaeNorm(FAKE, FAKE, 128)
    ws = c_size_t()
    lib.vae_conv2d_groupnorm_workspace_bytes(byref(c), 8, 8, 0, byref(ws))

    def call(**k):
        a = dict(x=FAKE, cin=16, h=8, w=8, conv=byref(c), up=0, res=NULL, norm=byref(n), silu=1, y=FAKE + 4096,
                 z=FAKE + 8192, ws=FAKE + 16384, nb=ws.value)
        a.update(k)
        return lib.vae_conv2d_groupnorm_silu(a["x"], a["cin"], a["h"], a["w"], a["conv"], a["up"], a["res"],
                                             a["norm"], a["silu"], a["y"], a["z"], a["ws"], a["nb"], NULL)
    assert call(z=NULL) == VAE_ERR_INVALID_ARG
    assert call(norm=NULL) == VAE_ERR_INVALID_ARG
    assert call(norm=byref(VaeNorm(FAKE, FAKE, 64))) == VAE_ERR_INVALID_ARG and "norm" in err(lib)
    assert call(cin=15) == VAE_ERR_INVALID_ARG
    assert call(y=FAKE) == VAE_ERR_INVALID_ARG and "alias" in err(lib)
    assert call(nb=ws.value - 1) == VAE_ERR_WORKSPACE
    c100 = conv(100, 16, 3)
    assert call(conv=byref(c100), norm=byref(VaeNorm(FAKE, FAKE, 100))) == VAE_ERR_UNSUPPORTED


def test_groupnorm_validation(lib):
    nb = c_size_t()
    assert lib.vae_groupnorm_workspace_bytes(128, 512 * 512, byref(nb)) == VAE_OK
    assert nb.value > 0
    assert lib.vae_groupnorm_workspace_bytes(100, 64, byref(nb)) == VAE_ERR_UNSUPPORTED
    n = VaeNorm(FAKE, FAKE, 64)
    assert lib.vae_groupnorm_silu(FAKE, 64, 16, byref(n), 1, NULL, FAKE, FAKE, 0, NULL) == VAE_ERR_WORKSPACE
    assert lib.vae_groupnorm_silu(FAKE, 96, 16, byref(n), 1, NULL, FAKE, FAKE, 1 << 20, NULL) == VAE_ERR_INVALID_ARG
    n40 = VaeNorm(FAKE, FAKE, 40)
    assert lib.vae_groupnorm_silu(FAKE, 40, 16, byref(n40), 1, NULL, FAKE, FAKE, 1 << 20, NULL) == VAE_ERR_UNSUPPORTED
    nn = VaeNorm(NULL, FAKE, 64)
    assert lib.vae_groupnorm_silu(FAKE, 64, 16, byref(nn), 1, NULL, FAKE, FAKE, 1 << 20, NULL) == VAE_ERR_INVALID_ARG


def test_attention_and_upsample_validation(lib):
    nb = c_size_t()
    assert lib.vae_attention_workspace_bytes(512, 128, 128, byref(nb)) == VAE_OK
    n = 128 * 128
    assert nb.value >= 4 * (n * n + 5 * 512 * n)
    a = VaeAttn(VaeNorm(FAKE, FAKE, 64), conv(64, 64, 1), conv(64, 64, 1), conv(64, 64, 1), conv(64, 64, 1))
    assert lib.vae_attention(FAKE, 64, 4, 4, byref(a), FAKE + 64, FAKE, 16, NULL) == VAE_ERR_WORKSPACE
    a.k = conv(64, 32, 1)
    assert lib.vae_attention(FAKE, 64, 4, 4, byref(a), FAKE + 64, FAKE, 1 << 30, NULL) == VAE_ERR_INVALID_ARG
    a.k = conv(64, 64, 3)
    assert lib.vae_attention(FAKE, 64, 4, 4, byref(a), FAKE + 64, FAKE, 1 << 30, NULL) == VAE_ERR_UNSUPPORTED
    assert lib.vae_upsample_nearest2x(FAKE, 4, 3, 3, FAKE, NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_upsample_nearest2x(FAKE, 0, 3, 3, FAKE + 64, NULL) == VAE_ERR_INVALID_ARG


def fake_weights(widths=(512, 512, 256, 128), zc=16, oc=3):
    keep = []

    def resnet(cin, cout):
        sc = conv(cout, cin, 1) if cin != cout else VaeConv(None, None, 0, 0, 0)
        return VaeResnet(VaeNorm(FAKE, FAKE, cin), conv(cout, cin, 3), VaeNorm(FAKE, FAKE, cout),
                         conv(cout, cout, 3), sc)
    c0 = widths[0]
    ups = []
    prev = c0
    for i, c in enumerate(widths):
        rs = (VaeResnet * 3)(*[resnet(prev if j == 0 else c, c) for j in range(3)])
        keep.append(rs)
        prev = c
        up = conv(c, c, 3) if i + 1 < len(widths) else VaeConv(None, None, 0, 0, 0)
        ups.append(VaeUp(3, rs, up))
    ua = (VaeUp * len(ups))(*ups)
    keep.append(ua)
    attn = VaeAttn(VaeNorm(FAKE, FAKE, c0), *[conv(c0, c0, 1) for _ in range(4)])
    w = VaeWeights(conv(c0, zc, 3), resnet(c0, c0), attn, resnet(c0, c0), len(ups), ua,
                   VaeNorm(FAKE, FAKE, prev), conv(oc, prev, 3), 0.3611, 0.1159)
    return w, keep


def test_decoder_pack_and_validation(lib):
    w, keep = fake_weights()
    nb = c_size_t()
    assert lib.vae_decoder_pack_bytes(byref(w), byref(nb)) == VAE_OK, err(lib)
    # about 50M parameters, of which 48.3M in 3x3 convs; the F(4x4) Winograd
    # packing of the convs on a plain input (43M parameters) holds 40 floats
    # per (output, input channel) pair instead of 9 (36 transform points, padded
    # to whole float4s per half), that of the three convs on a nearest-x2 input
    # (5.3M parameters) 28 (25 distinct products, 13 + 12 per half, padded to
    # whole float4s): about 208.5M floats in all
    assert 208_000_000 * 4 < nb.value < 209_000_000 * 4
    h = c_void_p()
    assert lib.vae_decoder_create(byref(h), byref(w), FAKE, nb.value - 1, NULL) == VAE_ERR_WORKSPACE
    assert lib.vae_decoder_create(byref(h), byref(w), FAKE + 4, nb.value, NULL) == VAE_ERR_INVALID_ARG
    # broken chains
    w2, k2 = fake_weights()
    w2.mid_res1.conv1 = conv(512, 256, 3)
    assert lib.vae_decoder_pack_bytes(byref(w2), byref(nb)) == VAE_ERR_INVALID_ARG
    w3, k3 = fake_weights()
    w3.ups[2].resnets[0].shortcut = VaeConv(None, None, 0, 0, 0)
    assert lib.vae_decoder_pack_bytes(byref(w3), byref(nb)) == VAE_ERR_INVALID_ARG
    assert "shortcut" in err(lib)
    w4, k4 = fake_weights(widths=(512, 512, 256, 100))
    assert lib.vae_decoder_pack_bytes(byref(w4), byref(nb)) == VAE_ERR_UNSUPPORTED
    w5, k5 = fake_weights()
    w5.scaling_factor = 0.0
    assert lib.vae_decoder_pack_bytes(byref(w5), byref(nb)) == VAE_ERR_INVALID_ARG
    w6, k6 = fake_weights()
    w6.n_up = 0
    assert lib.vae_decoder_pack_bytes(byref(w6), byref(nb)) == VAE_ERR_INVALID_ARG
    assert lib.vae_decode(NULL, FAKE, 8, 8, FAKE, FAKE, 1, NULL) == VAE_ERR_INVALID_ARG
    nb0 = c_size_t()
    assert lib.vae_decoder_tiled_workspace_bytes(NULL, 8, 8, 256, 64, byref(nb0)) == VAE_ERR_INVALID_ARG
    assert lib.vae_decode_tiled(NULL, FAKE, 8, 8, 256, 64, FAKE, FAKE, 1, NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_decode_tiled(NULL, NULL, 8, 8, 256, 64, FAKE, FAKE, 1, NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_decoder_set_profiling(NULL, 1) == VAE_ERR_INVALID_ARG


def test_decoder3d_pack_and_validation(lib):
    w, keep = fake_weights()
    n2, n3 = c_size_t(), c_size_t()
    assert lib.vae_decoder_pack_bytes(byref(w), byref(n2)) == VAE_OK
    assert lib.vae_decoder3d_pack_bytes(byref(w), byref(n3)) == VAE_OK, err(lib)
    # three time taps per 3x3 conv: about three times the 3x3 weights (and conv_out packed too)
    assert 2.7 * n2.value < n3.value < 3.1 * n2.value
    h = c_void_p()
    assert lib.vae_decoder3d_create(byref(h), byref(w), FAKE, n3.value - 1, NULL) == VAE_ERR_WORKSPACE
    assert lib.vae_decode3d(NULL, FAKE, 2, 8, 8, FAKE, FAKE, 1, NULL) == VAE_ERR_INVALID_ARG
    nb = c_size_t()
    assert lib.vae_decoder3d_workspace_bytes(NULL, 2, 8, 8, byref(nb)) == VAE_ERR_INVALID_ARG


@pytest.mark.parametrize("causal3d, shape, match", [
    (False, (4, 8, 8), "4 channels"),          # a 4-channel latent for a 16-channel conv_in
    (False, (16, 8), "3 dimensions"),
    (False, (16, 2, 8, 8), "3 dimensions"),
    (True, (16, 8, 8), "4 dimensions"),
    (True, (8, 2, 8, 8), "8 channels"),
])
def test_decoder_rejects_a_mismatched_latent_before_any_launch(causal3d, shape, match):
    # the decoder object is built without the library (no GPU here): the
    # check runs before any call into it, so a wrong latent never reaches
    # vae_decode, which takes no channel count and would read past the tensor
    import torch
    from diffusion_vae_decoder_amd import api

    d = object.__new__(api.Decoder)
    d.causal3d = causal3d
    d.latent_channels = 16
    d.device = torch.device("cuda", 0)
    with pytest.raises(ValueError, match=match):
        d.decode(torch.zeros(shape))
    # the right shape on the wrong device is refused as well
    ok = (16, 2, 8, 8) if causal3d else (16, 8, 8)
    with pytest.raises(ValueError, match="GPU tensor"):
        d.decode(torch.zeros(ok))


def test_attention_streaming_validation(lib):
    # the workspace holds no score matrix: xn, q, v, k^T and the output (five
    # [c, n] tensors), GroupNorm partials and the concatenated q/k/v weights
    nb = c_size_t()
    c, n = 512, 128 * 128
    assert lib.vae_attention_streaming_workspace_bytes(c, 128, 128, byref(nb)) == VAE_OK
    assert 5 * 4 * c * n <= nb.value < 5 * 4 * c * n + 4 * (3 * c * c + 3 * c) + (1 << 20)
    split = c_size_t()
    assert lib.vae_attention_workspace_bytes(c, 128, 128, byref(split)) == VAE_OK
    assert nb.value < split.value - 4 * n * n + (1 << 20)
    # channel counts the streaming kernel has no form for
    assert lib.vae_attention_streaming_workspace_bytes(64, 8, 8, byref(nb)) == VAE_ERR_UNSUPPORTED
    a = VaeAttn(VaeNorm(FAKE, FAKE, 64), conv(64, 64, 1), conv(64, 64, 1), conv(64, 64, 1), conv(64, 64, 1))
    assert lib.vae_attention_streaming(FAKE, 64, 4, 4, byref(a), FAKE + 64, FAKE, 1 << 30, NULL) == VAE_ERR_UNSUPPORTED
    assert "128, 256 and 512" in err(lib)
    a = VaeAttn(VaeNorm(FAKE, FAKE, 128), *[conv(128, 128, 1) for _ in range(4)])
    assert lib.vae_attention_streaming(FAKE, 128, 4, 4, byref(a), FAKE + 64, FAKE, 16, NULL) == VAE_ERR_WORKSPACE
    assert lib.vae_attention_streaming(FAKE, 128, 4, 4, byref(a), FAKE, FAKE, 1 << 30, NULL) == VAE_ERR_INVALID_ARG
    a.v = conv(128, 64, 1)
    assert lib.vae_attention_streaming(FAKE, 128, 4, 4, byref(a), FAKE + 64, FAKE, 1 << 30, NULL) \
        == VAE_ERR_INVALID_ARG
    # the decoder's form switch rejects a NULL decoder and unknown forms
    assert lib.vae_decoder_set_attention(NULL, 1) == VAE_ERR_INVALID_ARG


def test_conv3d_groupnorm_validation(lib):
    c3 = conv(128, 128, 3)
    nb = c_size_t()
    assert lib.vae_conv3d_causal_groupnorm_workspace_bytes(byref(c3), 17, 256, 256, byref(nb)) == VAE_OK
    plain = c_size_t()
    assert lib.vae_conv3d_causal_workspace_bytes(byref(c3), 17, 256, 256, byref(plain)) == VAE_OK
    # the conv's workspace, then the records (32 groups x 16 bytes per tile) and GroupNorm partials
    assert plain.value < nb.value < plain.value + (1 << 24)
    assert lib.vae_conv3d_causal_groupnorm_workspace_bytes(byref(conv(100, 128, 3)), 2, 8, 8, byref(nb)) \
        == VAE_ERR_UNSUPPORTED
    n = VaeNorm(FAKE, FAKE, 128)
    ws = c_size_t()
    lib.vae_conv3d_causal_groupnorm_workspace_bytes(byref(c3), 3, 8, 8, byref(ws))

    def call(**k):
        a = dict(x=FAKE, cin=128, t=3, h=8, w=8, conv=byref(c3), norm=byref(n), silu=1, res=NULL, y=FAKE + 4096,
                 z=FAKE + 4096, ws=FAKE + 1 << 20, nb=ws.value)
        a.update(k)
        return lib.vae_conv3d_causal_groupnorm_silu(a["x"], a["cin"], a["t"], a["h"], a["w"], a["conv"], a["norm"],
                                                    a["silu"], a["res"], a["y"], a["z"], a["ws"], a["nb"], NULL)
    assert call(z=NULL) == VAE_ERR_INVALID_ARG
    assert call(t=0) == VAE_ERR_INVALID_ARG
    assert call(norm=byref(VaeNorm(FAKE, FAKE, 64))) == VAE_ERR_INVALID_ARG and "norm" in err(lib)
    assert call(y=FAKE) == VAE_ERR_INVALID_ARG and "alias" in err(lib)
    assert call(res=FAKE + 4096) == VAE_ERR_INVALID_ARG and "residual" in err(lib)
    assert call(nb=ws.value - 1) == VAE_ERR_WORKSPACE


def test_probe_validation(lib):
    # the measurement probes refuse bad arguments before any launch
    fl = ctypes.c_double()
    assert lib.vae_probe_mfma_f32(0, 16, FAKE, 1 << 20, byref(fl), NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_probe_mfma_f32(256, 0, FAKE, 1 << 20, byref(fl), NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_probe_mfma_f32(256, (1 << 20) + 1, FAKE, 1 << 20, byref(fl), NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_probe_mfma_f32(256, 16, NULL, 1 << 20, byref(fl), NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_probe_mfma_f32(256, 16, FAKE, 1 << 20, NULL, NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_probe_mfma_f32(256, 16, FAKE, 256 * 256 - 1, byref(fl), NULL) == VAE_ERR_INVALID_ARG
    assert "out holds" in err(lib)
    assert lib.vae_probe_hbm(NULL, 1024, NULL, 16, FAKE, 1 << 20, NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_probe_hbm(FAKE, 1024, NULL, 16, NULL, 1 << 20, NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_probe_hbm(FAKE, 1022, NULL, 16, FAKE, 1 << 20, NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_probe_hbm(FAKE, 0, NULL, 16, FAKE, 1 << 20, NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_probe_hbm(FAKE + 4, 1024, NULL, 16, FAKE, 1 << 20, NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_probe_hbm(FAKE, 1024, FAKE + 8, 16, NULL, 0, NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_probe_hbm(FAKE, 1024, NULL, 0, FAKE, 1 << 20, NULL) == VAE_ERR_INVALID_ARG
    assert lib.vae_probe_hbm(FAKE, 1024, NULL, 16, FAKE, 16 * 256 - 1, NULL) == VAE_ERR_INVALID_ARG
