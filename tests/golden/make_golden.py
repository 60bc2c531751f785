"""Writes the stored expected values for the full-size parity tests.

Calls only the float64 oracle (oracle/) on inputs from the seeded generator
(vaegen/, seed 0); nothing here touches the GPU path.  Run from the repo root:

    python tests/golden/make_golden.py [decode1024] [stack3d] [tiled512] [tiled1024]

Outputs (numpy .npz, float64):
  decode_1024.npz  latent [16,128,128] -> RGB [3,1024,1024]: a lattice of
                   rows and columns that covers every residue mod 4 (the
                   first four rows and columns of every 32-row / 32-column
                   band, so each 4 x 4 output block position of the
                   Winograd tiling appears), the whole first and last rows
                   and columns, and 16384 pseudo-random pixels
  stack3d.npz      x [128,17,256,256] -> 4-layer causal stack, 4096 sampled elements
  decode_tiled_512.npz  latent [16,64,64] -> RGB [3,512,512] decoded in 256-pixel
                   tiles with overlaps of at least 64 (3 x 3 tiles, overlaps 128):
                   every row and column within 2 pixels of a tile start or
                   end, a lattice of every 16th row and column, and 16384
                   pseudo-random pixels
  decode_tiled_1024.npz  latent [16,128,128] -> RGB [3,1024,1024] in the same
                   tiles (5 x 5 tiles, overlaps 64), sampled the same way
Each file also holds max|ref| and the L2 norm of the whole reference output.
The 256 x 256 decode is compared on every pixel by running the oracle inside
the test, so it has no stored file.
"""
from __future__ import annotations

import ctypes
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import vaegen  # noqa: E402

SEED = 0


def keep_heap():
    try:
        libc = ctypes.CDLL("libc.so.6")
        libc.mallopt(-4, 0)
        libc.mallopt(-1, 1 << 30)
    except OSError:
        pass


def lattice(n: int) -> np.ndarray:
    """Indices 32 k + r, r = 0..3, plus the last index: every residue mod 4."""
    idx = sorted({b + r for b in range(0, n, 32) for r in range(4) if b + r < n} | {n - 1})
    return np.array(idx, dtype=np.int64)


def decode1024():
    h = 128
    p = vaegen.decoder_params(SEED)
    z = vaegen.latent(SEED, h, h)
    t = time.time()
    y = oracle.decode(z, p, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
    print(f"decode_1024: oracle decode {h}x{h} took {time.time() - t:.1f} s", flush=True)
    c, H, W = y.shape
    rows, cols = lattice(H), lattice(W)
    rng = np.random.default_rng(20241)
    pix = np.stack([rng.integers(0, c, 16384), rng.integers(0, H, 16384), rng.integers(0, W, 16384)], axis=1)
    np.savez_compressed(os.path.join(HERE, "decode_1024"), rows=rows, cols=cols,
                        lattice=y[:, rows][:, :, cols], first_row=y[:, 0, :], last_row=y[:, H - 1, :],
                        first_col=y[:, :, 0], last_col=y[:, :, W - 1], pixels=pix,
                        pixel_values=y[pix[:, 0], pix[:, 1], pix[:, 2]], shape=np.array(y.shape),
                        max_abs=np.abs(y).max(), l2=np.sqrt((y * y).sum()), seed=SEED)


def stack3d():
    p = vaegen.causal_stack_params(SEED, c=128)
    x = vaegen.activation(SEED, "stack.x", (128, 17, 256, 256))
    t = time.time()
    y = oracle.causal_stack(x, p)
    print(f"stack3d: oracle took {time.time() - t:.1f} s", flush=True)
    rng = np.random.default_rng(12345)
    idx = np.stack([rng.integers(0, n, 4096) for n in y.shape], axis=1)
    # always include the corners of the first and last frames
    corners = np.array([[c, t, i, j] for c in (0, 127) for t in (0, 16) for i in (0, 255) for j in (0, 255)])
    idx = np.concatenate([corners, idx])
    vals = y[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]]
    np.savez_compressed(os.path.join(HERE, "stack3d"), index=idx, sample=vals, shape=np.array(y.shape),
                        max_abs=np.abs(y).max(), l2=np.sqrt((y * y).sum()), seed=SEED)


def tiled(h: int, name: str):
    """The oracle's tiled decode (256-pixel tiles, overlaps of at least 64) of
    the seed's latent [16, h, h]: rows and columns at and around every tile
    start and end, every 16th, and 16384 random pixels."""
    p = vaegen.decoder_params(SEED)
    z = vaegen.latent(SEED, h, h)
    t = time.time()
    y = oracle.decode_tiled(z, p, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR, tile=256, overlap_min=64)
    print(f"{name}: oracle took {time.time() - t:.1f} s", flush=True)
    c, H, W = y.shape
    starts, lens, _ = oracle.split_tiles(H, 8, 256, 64)
    edges = sorted({e + d for s0, n in zip(starts, lens) for e in (s0, s0 + n) for d in (-2, -1, 0, 1)
                    if 0 <= e + d < H} | set(range(0, H, 16)) | {H - 1})
    idx = np.array(edges, dtype=np.int64)
    rng = np.random.default_rng(20251)
    pix = np.stack([rng.integers(0, c, 16384), rng.integers(0, H, 16384), rng.integers(0, W, 16384)], axis=1)
    np.savez_compressed(os.path.join(HERE, name), rows=idx, cols=idx, lattice=y[:, idx][:, :, idx],
                        pixels=pix, pixel_values=y[pix[:, 0], pix[:, 1], pix[:, 2]], shape=np.array(y.shape),
                        tile=256, overlap=64, max_abs=np.abs(y).max(), l2=np.sqrt((y * y).sum()), seed=SEED)


if __name__ == "__main__":
    keep_heap()
    which = sys.argv[1:] or ["decode1024", "stack3d", "tiled512", "tiled1024"]
    if "decode1024" in which:
        decode1024()
    if "stack3d" in which:
        stack3d()
    if "tiled512" in which:
        tiled(64, "decode_tiled_512")
    if "tiled1024" in which:
        tiled(128, "decode_tiled_1024")
