"""Helpers shared by the GPU parity tests (imported by them; no tests here).

Bars: per layer max|gpu - ref| / max|ref| <= LAYER_TOL over the layer output;
end to end (RGB) cosine >= 0.99999 and max|gpu - ref| <= 1e-3 * max|ref|.
"""
import math

import numpy as np
import torch

import vaegen

LAYER_TOL = 1e-4


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


# Output buffers sit inside a larger allocation whose head and tail hold a
# sentinel value (GUARD floats each side, a multiple of 64 so the view keeps
# the alignment a fresh allocation has); host() checks that neither was
# written.  The body starts as NaN, so an element the kernel never writes
# fails the comparison.
GUARD = 4096
SENTINEL = -1.2345678e33


def nan_like(shape):
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.float32, device="cuda")
    body = buf[GUARD:GUARD + n]
    body.fill_(float("nan"))
    view = body.view(tuple(shape))
    view._guard = (buf, n)   # the api returns the `out` tensor itself, attribute included
    return view


def check_guards(t):
    """The sentinel head and tail around an output from nan_like are intact."""
    entry = getattr(t, "_guard", None)
    if entry is None:
        return
    buf, n = entry
    torch.cuda.synchronize()
    head = buf[:GUARD].cpu().numpy()
    tail = buf[GUARD + n:].cpu().numpy()
    assert (head == np.float32(SENTINEL)).all(), "a kernel wrote before the start of its output"
    assert (tail == np.float32(SENTINEL)).all(), "a kernel wrote past the end of its output"


def host(t):
    torch.cuda.synchronize()
    check_guards(t)
    return t.cpu().numpy().astype(np.float64)


def rel_err(g, r):
    assert not np.isnan(g).any(), "output has unwritten (NaN) elements"
    return float(np.abs(g - r).max() / max(np.abs(r).max(), 1e-30))


def conv_params(seed, name, cin, cout, k, dims=2):
    p = vaegen.conv_params(seed, name, cin, cout, k, dims)
    return p[name + ".weight"], p[name + ".bias"]


def rgb_metrics(g, r):
    assert not np.isnan(g).any()
    cos = float((g * r).sum() / math.sqrt((g * g).sum() * (r * r).sum()))
    return cos, float(np.abs(g - r).max())
