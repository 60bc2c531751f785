"""Pins of the oracle's tiled decode (oracle.split_tiles, oracle.decode_tiled):
the tile schedule and the cross-fade of [vae3d] (VideoVae's split_tiles,
decode_clip and blend), checked against properties the pages' description
fixes, values worked by hand, and fake per-tile decoders whose exact output
is known."""
import numpy as np
import pytest

import oracle
import vaegen


def covers(starts, lens, L):
    return starts[0] == 0 and starts[-1] + lens[-1] >= L


@pytest.mark.parametrize("tile,ovmin,ratio", [(256, 64, 8), (64, 16, 8), (48, 8, 4), (256, 64, 1), (32, 0, 8)])
def test_split_tiles_schedule_properties(tile, ovmin, ratio):
    for L in range(1, 1400):
        starts, lens, ovs = oracle.split_tiles(L, ratio, tile, ovmin)
        if L <= tile:
            assert (starts, lens, ovs) == ([0], [L], [])
            continue
        n = len(starts)
        assert lens == [tile] * n and len(ovs) == n - 1
        # neighbours overlap by ovs[k]; every overlap at least the minimum,
        # grown in whole steps of `ratio`, the first ones first and evenly
        for k in range(n - 1):
            assert starts[k + 1] - starts[k] == tile - ovs[k]
        assert all(ov >= ovmin and (ov - ovmin) % ratio == 0 for ov in ovs)
        assert max(ovs) - min(ovs) <= ratio and ovs == sorted(ovs, reverse=True)
        # the tiles cover the axis, overshooting by less than one step
        assert covers(starts, lens, L) and starts[-1] + tile - L < ratio
        if L % ratio == 0 and tile % ratio == 0 and ovmin % ratio == 0:
            assert starts[-1] + tile == L
        # the fewest tiles that can cover it with the minimum overlap
        assert n * tile >= (n - 1) * ovmin + L
        assert n - 1 == 1 or (n - 1) * tile < (n - 2) * ovmin + L


def test_split_tiles_worked_values():
    # 1024 px: four 256-px tiles overlapping by 64 reach only 832 px, so five
    # are needed, and five with 64-px overlaps span exactly 1024 (no slack)
    assert oracle.split_tiles(1024, 8) == ([0, 192, 384, 576, 768], [256] * 5, [64] * 4)
    # 384 px: two tiles, 512 - 64 - 384 = 64 px of slack, 8 steps of 8 into
    # the one overlap: 128, so the second tile starts at 128
    assert oracle.split_tiles(384, 8) == ([0, 128], [256, 256], [128])
    # 300 px: slack 148, 18 whole steps of 8 (144): overlap 208, 4 px overhang
    assert oracle.split_tiles(300, 8) == ([0, 48], [256, 256], [208])
    # 1000 px, 5 tiles: slack 1280 - 256 - 1000 = 24, three steps of 8 go to
    # the first three overlaps
    assert oracle.split_tiles(1000, 8) == ([0, 184, 368, 552, 744], [256] * 5, [72, 72, 72, 64])
    assert oracle.split_tiles(256, 8) == ([0], [256], [])
    # no minimum overlap: tiles that divide the axis abut; 80 px in 32-px
    # tiles leave 16 px of slack, one step of 8 to each overlap
    assert oracle.split_tiles(96, 8, 32, 0) == ([0, 32, 64], [32] * 3, [0, 0])
    assert oracle.split_tiles(80, 8, 32, 0) == ([0, 24, 48], [32] * 3, [8, 8])
    with pytest.raises(ValueError):
        oracle.split_tiles(300, 8, 64, 64)


def coord_latent(h, w):
    """A 2-channel 'latent' whose cells carry their own row and column."""
    z = np.zeros((2, h, w))
    z[0] = np.arange(h)[:, None]
    z[1] = np.arange(w)[None, :]
    return z


@pytest.mark.parametrize("h,w,tile,ov", [(12, 10, 64, 16), (48, 40, 256, 64), (21, 9, 64, 8)])
def test_tiles_that_agree_reproduce_the_image(h, w, tile, ov):
    """Every tile a crop of one image: any cross-fade of equal values returns
    them, so the assembled output is that image."""
    rng = np.random.default_rng(1)
    img = rng.standard_normal((3, 8 * h, 8 * w))

    def crop(block):
        r0, c0 = int(block[0, 0, 0]), int(block[1, 0, 0])
        bh, bw = block.shape[-2:]
        return img[:, 8 * r0:8 * (r0 + bh), 8 * c0:8 * (c0 + bw)]

    out = oracle.decode_tiled(coord_latent(h, w), None, 1.0, 0.0, tile, ov, decode_fn=crop)
    np.testing.assert_allclose(out, img, rtol=0, atol=1e-13)


def test_cross_fade_ramp_and_corner():
    """Constant tiles (a value per tile): inside the overlaps the output is the
    stated ramp, in the corner the left fade applied over the top fade, with
    the left tile taken as decoded (not faded)."""
    h, w, tile, ov = 12, 10, 64, 16          # 96 x 80 px: rows [0,64) [32,96), cols [0,64) [16,80)
    ys, _, yo = oracle.split_tiles(96, 8, tile, ov)
    xs, _, xo = oracle.split_tiles(80, 8, tile, ov)
    assert (ys, yo, xs, xo) == ([0, 32], [32], [0, 16], [48])
    val = {}

    def const(block):
        r0, c0 = int(block[0, 0, 0]), int(block[1, 0, 0])
        i, j = ys.index(8 * r0), xs.index(8 * c0)
        val[i, j] = 10.0 * i + j + 1.0
        return np.full((3,) + tuple(8 * np.array(block.shape[-2:])), val[i, j])

    out = oracle.decode_tiled(coord_latent(h, w), None, 1.0, 0.0, tile, ov, decode_fn=const)[0]
    a, b, c, d = val[0, 0], val[0, 1], val[1, 0], val[1, 1]
    for y in range(96):
        for x in range(80):
            i = 1 if y >= 32 else 0
            j = 1 if x >= 16 else 0
            hh, ww = y - ys[i], x - xs[j]
            if i == 0 and j == 0:
                want = a
            elif i == 0:                           # left fade only, over 48 columns
                want = a * (1 - ww / 48) + b * (ww / 48) if ww < 48 else b
            elif j == 0:                           # top fade only, over 32 rows
                want = a * (1 - hh / 32) + c * (hh / 32) if hh < 32 else c
            else:
                top = b * (1 - hh / 32) + d * (hh / 32) if hh < 32 else d
                want = c * (1 - ww / 48) + top * (ww / 48) if ww < 48 else top
            assert out[y, x] == pytest.approx(want, abs=1e-12), (y, x)


def test_one_tile_is_the_plain_decode():
    h = w = 3
    seen = []

    def fake(block):
        seen.append(block.shape)
        return np.arange(3 * 64 * h * w, dtype=np.float64).reshape(3, 8 * h, 8 * w)

    out = oracle.decode_tiled(coord_latent(h, w), None, 1.0, 0.0, 256, 64, decode_fn=fake)
    assert seen == [(2, h, w)]
    np.testing.assert_array_equal(out, fake(coord_latent(h, w)))


def test_tiled_decode_of_the_real_decoder():
    """The real decoder on a 12 x 10 latent in 64-px tiles: where no fade
    reaches (the part of tile (0, 0) before the next tiles start) the output
    is the decode of that tile's latent block; the rest is its blend."""
    p = vaegen.decoder_params(0, widths=(64, 64, 32, 32))   # a narrow decoder: seconds on the CPU
    z = vaegen.latent(0, 12, 10)
    out = oracle.decode_tiled(z, p, 0.3611, 0.1159, tile=64, overlap_min=16)
    assert out.shape == (3, 96, 80)
    t00 = oracle.decode(z[:, :8, :8], p, 0.3611, 0.1159)
    np.testing.assert_allclose(out[:, :32, :16], t00[:, :32, :16], rtol=0, atol=1e-12)
