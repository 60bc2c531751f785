"""Writes the stored expected values for the full-size parity tests.

Calls only the float64 oracle (oracle/) on inputs from the seeded generator
(vaegen/, seed 0); nothing here touches the GPU path.  Run from the repo root:

    python tests/golden/make_golden.py [decode256] [decode1024] [stack3d]

Outputs (numpy .npz, float64):
  decode_256.npz   latent [16,32,32]  -> RGB [3,256,256], every 4th pixel per axis
  decode_1024.npz  latent [16,128,128] -> RGB [3,1024,1024], every 16th pixel per axis
  stack3d.npz      x [128,17,256,256] -> 4-layer causal stack, 4096 sampled elements
Each file also holds max|ref| and the L2 norm of the whole reference output.
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


def decode(h: int, stride: int, name: str):
    p = vaegen.decoder_params(SEED)
    z = vaegen.latent(SEED, h, h)
    t = time.time()
    y = oracle.decode(z, p, vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR)
    print(f"{name}: oracle decode {h}x{h} took {time.time() - t:.1f} s", flush=True)
    np.savez_compressed(os.path.join(HERE, name), sample=y[:, ::stride, ::stride], stride=stride,
                        shape=np.array(y.shape), max_abs=np.abs(y).max(), l2=np.sqrt((y * y).sum()),
                        seed=SEED)


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


if __name__ == "__main__":
    keep_heap()
    which = sys.argv[1:] or ["decode256", "decode1024", "stack3d"]
    if "decode256" in which:
        decode(32, 4, "decode_256")
    if "decode1024" in which:
        decode(128, 16, "decode_1024")
    if "stack3d" in which:
        stack3d()
