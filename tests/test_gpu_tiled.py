"""GPU parity of the tiled decode (vae_decode_tiled) against the oracle's
decode_tiled: the tile schedule, per-tile decodes and the cross-fade assembly
of the pages' video VAE applied to the decoder.  Same bars as the whole
decode: cosine >= 0.99999 and max|gpu - ref| <= 1e-3 * max|ref|."""
import ctypes
import math
import os

import numpy as np
import pytest

import oracle
import vaegen

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_helpers import check_guards, dev, host, nan_like, rgb_metrics  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SF, SH = vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR


@pytest.fixture(scope="module")
def api():
    from diffusion_vae_decoder_amd import api as a
    return a


@pytest.fixture(scope="module")
def params():
    return vaegen.decoder_params(0)


@pytest.fixture(scope="module")
def decoder(api, params):
    d = api.Decoder({k: dev(v) for k, v in params.items()}, SF, SH)
    yield d
    d.close()


@pytest.mark.parametrize("h,w,tile,ov", [
    (12, 10, 64, 16),   # 96 x 80 px: 2 x 2 tiles of 64, overlaps 32 and 48
    (9, 5, 32, 8),      # 72 x 40 px: 3 x 2 tiles of 32, overlaps (16, 8) and 24
    (12, 10, 32, 0),    # 96 x 80 px, no minimum overlap: rows of tiles abut, columns overlap by 8
])
def test_tiled_decode_matches_oracle(decoder, params, h, w, tile, ov):
    z = vaegen.latent(11, h, w)
    print(f"tiled decode {h}x{w} tile {tile} overlap {ov}", flush=True)
    rgb = decoder.decode_tiled(dev(z), tile, ov, out=nan_like((3, 8 * h, 8 * w)))
    check_guards(rgb)
    ref = oracle.decode_tiled(z, params, SF, SH, tile=tile, overlap_min=ov)
    cos, mx = rgb_metrics(host(rgb), ref)
    assert cos >= 0.99999 and mx <= 1e-3 * np.abs(ref).max(), (cos, mx)


def test_one_tile_is_the_plain_decode(decoder):
    z = dev(vaegen.latent(12, 16, 12))
    plain = host(decoder.decode(z))
    tiled = host(decoder.decode_tiled(z, 256, 64, out=nan_like((3, 128, 96))))
    np.testing.assert_array_equal(tiled, plain)


def test_tiled_decode_in_graph_mode_matches_eager(decoder):
    # every tile replays the one graph captured for the tile shape
    z = dev(vaegen.latent(13, 12, 10))
    eager = host(decoder.decode_tiled(z, 64, 16))
    decoder.set_graph(True)
    try:
        for _ in range(2):
            out = host(decoder.decode_tiled(z, 64, 16))
            np.testing.assert_array_equal(out, eager)
    finally:
        decoder.set_graph(False)


def test_concurrent_tiles_equal_sequential_tiles(decoder):
    # 3 x 2 tiles: by default they decode on the handle's three streams; with
    # profiling on, one after another on the caller's stream.  Both run the
    # same kernels on the same blocks, so the results agree bit for bit, also
    # when the caller's stream is a side stream and when the call repeats.
    z = dev(vaegen.latent(15, 9, 5))
    conc = host(decoder.decode_tiled(z, 32, 8))
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for _ in range(2):
            out = decoder.decode_tiled(z, 32, 8)
    side.synchronize()
    np.testing.assert_array_equal(host(out), conc)
    decoder.set_profiling(True)
    try:
        seq = host(decoder.decode_tiled(z, 32, 8))
        assert len(decoder.profile()) > 0
    finally:
        decoder.set_profiling(False)
    np.testing.assert_array_equal(seq, conc)


@pytest.mark.parametrize("name,h", [
    # 3 x 3 tiles of 256 pixels overlapping by 128
    ("decode_tiled_512", 64),
    # the benchmarked configuration: 5 x 5 tiles overlapping by 64
    ("decode_tiled_1024", 128),
])
def test_tiled_decode_against_stored_oracle(decoder, name, h):
    # stored oracle values (tests/golden/make_golden.py): rows and columns at
    # and around every tile start and end, every 16th row and column, 16384
    # random pixels
    g = np.load(os.path.join(GOLDEN, name + ".npz"))
    assert int(g["seed"]) == 0
    z = vaegen.latent(0, h, h)
    print(f"{name}: tiled decode of latent [16,{h},{h}]", flush=True)
    rgb = decoder.decode_tiled(dev(z), int(g["tile"]), int(g["overlap"]), out=nan_like(tuple(g["shape"])))
    check_guards(rgb)
    rgb = host(rgb)
    rows, cols, pix = g["rows"], g["cols"], g["pixels"]
    got = np.concatenate([rgb[:, rows][:, :, cols].ravel(), rgb[pix[:, 0], pix[:, 1], pix[:, 2]]])
    ref = np.concatenate([g["lattice"].ravel(), g["pixel_values"]])
    cos, mx = rgb_metrics(got, ref)
    assert cos >= 0.99999 and mx <= 1e-3 * float(g["max_abs"]), (cos, mx)
    assert np.isfinite(rgb).all()
    assert abs(math.sqrt((rgb.astype(np.float64) ** 2).sum()) / float(g["l2"]) - 1.0) < 1e-4


def test_tiled_decode_4096_corner_tiles_against_oracle(decoder, params):
    """A 4096 x 4096 output (latent [16,512,512], 21 x 21 tiles), far beyond
    what the whole-image decode's workspace and score matrix allow: the first
    and the last tile keep, unblended, the part before (after) their
    neighbours' overlap, which must equal the oracle's decode of their latent
    blocks; everything is written and finite."""
    h = 512
    z = vaegen.latent(21, h, h)
    starts, lens, _ = oracle.split_tiles(8 * h, 8, 256, 64)
    assert len(starts) == 21 and lens == [256] * 21
    print("tiled decode of latent [16,512,512] in 21 x 21 tiles", flush=True)
    rgb = decoder.decode_tiled(dev(z), 256, 64, out=nan_like((3, 8 * h, 8 * h)))
    check_guards(rgb)
    rgb = host(rgb)
    assert np.isfinite(rgb).all()
    e0 = starts[1]                  # tile 0 alone before tile 1 begins
    e1 = starts[-2] + lens[-2]      # the last tile alone after tile n-2 ends
    b0, b1 = starts[-1] // 8, starts[-1] // 8 + 32
    for rows, cols, block, crop in [
        (slice(0, e0), slice(0, e0), z[:, :32, :32], (slice(0, e0), slice(0, e0))),
        (slice(e1, 8 * h), slice(e1, 8 * h), z[:, b0:b1, b0:b1],
         (slice(e1 - starts[-1], 256), slice(e1 - starts[-1], 256))),
    ]:
        ref = oracle.decode(block, params, SF, SH)[:, crop[0], crop[1]]
        cos, mx = rgb_metrics(rgb[:, rows, cols], ref)
        assert cos >= 0.99999 and mx <= 1e-3 * np.abs(ref).max(), (cos, mx)


def test_tiled_decode_rejects_bad_arguments(api, decoder):
    lib = decoder._lib
    nb = ctypes.c_size_t()
    for tile, ov in [(60, 16), (64, 12), (64, 64), (64, -8), (0, 0)]:
        assert lib.vae_decoder_tiled_workspace_bytes(decoder._h, 12, 10, tile, ov, ctypes.byref(nb)) == -1
    assert lib.vae_decoder_tiled_workspace_bytes(decoder._h, 12, 10, 64, 16, ctypes.byref(nb)) == 0
    z = dev(vaegen.latent(14, 12, 10))
    out = torch.empty((3, 96, 80), dtype=torch.float32, device="cuda")
    ws = torch.empty(nb.value, dtype=torch.uint8, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # a workspace one byte short is refused before anything runs
    assert lib.vae_decode_tiled(decoder._h, z.data_ptr(), 12, 10, 64, 16, out.data_ptr(), ws.data_ptr(),
                                nb.value - 1, s) == -3
    # more than 64 tiles along an axis
    assert lib.vae_decoder_tiled_workspace_bytes(decoder._h, 1024, 8, 16, 8, ctypes.byref(nb)) == -2
    with pytest.raises(api.VaeError):
        decoder.decode_tiled(z, 60, 16)
