"""Pins of the float64 oracle against things other than itself.

Each test ties one oracle function to a brute-force loop nest on tiny inputs,
a closed form, an invariant, or an independent library routine (torch CPU
float64), chosen so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import vaegen

RNG = np.random.default_rng(1234)


def rand(*shape):
    return RNG.standard_normal(shape)


def t64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


# ---------------------------------------------------------------------------
# conv2d
# ---------------------------------------------------------------------------

def brute_conv2d(x, w, b):
    oc, ic, k, _ = w.shape
    p = k // 2
    _, h, wd = x.shape
    y = [[[0.0] * wd for _ in range(h)] for _ in range(oc)]
    for o in range(oc):
        for i in range(h):
            for j in range(wd):
                acc = float(b[o])
                for c in range(ic):
                    for dy in range(k):
                        for dx in range(k):
                            yy, xx = i + dy - p, j + dx - p
                            if 0 <= yy < h and 0 <= xx < wd:
                                acc += float(w[o, c, dy, dx]) * float(x[c, yy, xx])
                y[o][i][j] = acc
    return np.array(y)


@pytest.mark.parametrize("k", [1, 3])
def test_conv2d_brute_force(k):
    x, w, b = rand(3, 5, 7), rand(4, 3, k, k), rand(4)
    assert np.allclose(oracle.conv2d(x, w, b), brute_conv2d(x, w, b), atol=1e-12, rtol=0)


def test_conv2d_identity_1x1_and_delta_3x3():
    x = rand(6, 9, 11)
    eye = np.eye(6).reshape(6, 6, 1, 1)
    assert np.array_equal(oracle.conv2d(x, eye, np.zeros(6)), x)
    delta = np.zeros((6, 6, 3, 3))
    delta[:, :, 1, 1] = np.eye(6)
    assert np.array_equal(oracle.conv2d(x, delta, np.zeros(6)), x)


def test_conv2d_shifted_delta_moves_the_image():
    # a single off-centre tap (dy=0, dx=2) reads x[c, i-1, j+1]: cross-correlation
    x = rand(2, 6, 8)
    w = np.zeros((2, 2, 3, 3))
    w[0, 1, 0, 2] = 1.0
    y = oracle.conv2d(x, w, np.zeros(2))
    expect = np.zeros((6, 8))
    expect[1:, :-1] = x[1, :-1, 1:]
    assert np.array_equal(y[0], expect)
    assert np.array_equal(y[1], np.zeros((6, 8)))


def test_conv2d_constant_input_closed_form():
    # x == 1 gives b[o] + the sum of the in-bounds taps at each position
    oc, ic, h, wd = 3, 4, 6, 5
    w, b = rand(oc, ic, 3, 3), rand(oc)
    y = oracle.conv2d(np.ones((ic, h, wd)), w, b)
    s = w.sum(axis=1)                          # [oc, 3, 3]
    for o in range(oc):
        assert math.isclose(y[o, 2, 2], b[o] + s[o].sum(), abs_tol=1e-12)          # interior
        assert math.isclose(y[o, 0, 0], b[o] + s[o, 1:, 1:].sum(), abs_tol=1e-12)  # corner
        assert math.isclose(y[o, 0, 2], b[o] + s[o, 1:, :].sum(), abs_tol=1e-12)   # top edge
        assert math.isclose(y[o, 3, wd - 1], b[o] + s[o, :, :2].sum(), abs_tol=1e-12)  # right edge


def test_conv2d_linearity():
    x1, x2, w, b = rand(3, 6, 6), rand(3, 6, 6), rand(5, 3, 3, 3), rand(5)
    z = np.zeros(5)
    lhs = oracle.conv2d(2.0 * x1 - 3.0 * x2, w, z)
    rhs = 2.0 * oracle.conv2d(x1, w, z) - 3.0 * oracle.conv2d(x2, w, z)
    assert np.allclose(lhs, rhs, atol=1e-12)
    w2 = rand(5, 3, 3, 3)
    assert np.allclose(oracle.conv2d(x1, w + w2, z), oracle.conv2d(x1, w, z) + oracle.conv2d(x1, w2, z), atol=1e-12)


@pytest.mark.parametrize("k,cin,cout,h,w", [(3, 16, 24, 19, 23), (1, 32, 8, 17, 9), (3, 64, 64, 32, 32)])
def test_conv2d_matches_torch(k, cin, cout, h, w):
    x, wt, b = rand(cin, h, w), rand(cout, cin, k, k), rand(cout)
    ref = F.conv2d(t64(x)[None], t64(wt), t64(b), padding=k // 2)[0].numpy()
    assert np.allclose(oracle.conv2d(x, wt, b), ref, atol=1e-10, rtol=0)


def test_conv2d_at_matches_full_conv():
    x, w, b = rand(5, 7, 6), rand(4, 5, 3, 3), rand(4)
    y = oracle.conv2d(x, w, b)
    yu = oracle.conv2d(oracle.upsample_nearest2x(x), w, b)
    for (o, i, j) in [(0, 0, 0), (3, 6, 5), (2, 3, 0), (1, 0, 5)]:
        assert math.isclose(oracle.conv2d_at(x, w, b, o, i, j), y[o, i, j], abs_tol=1e-12)
    for (o, i, j) in [(0, 0, 0), (3, 13, 11), (2, 7, 4), (1, 0, 11)]:
        assert math.isclose(oracle.conv2d_at(x, w, b, o, i, j, upsample2x=True), yu[o, i, j], abs_tol=1e-12)


# ---------------------------------------------------------------------------
# GroupNorm, SiLU, upsample, de-normalisation
# ---------------------------------------------------------------------------

def test_group_norm_normalises_each_group():
    x = rand(64, 5, 7) * 3.0 + 2.0
    y = oracle.group_norm(x, np.ones(64), np.zeros(64))
    g = y.reshape(32, -1)
    assert np.allclose(g.mean(axis=1), 0.0, atol=1e-12)
    # biased variance of the normalised group is var/(var+eps)
    xv = x.reshape(32, -1).var(axis=1)
    assert np.allclose(g.var(axis=1), xv / (xv + 1e-6), atol=1e-12)


def test_group_norm_groups_are_contiguous_channels():
    # changing channel 0 (group 0 = channels 0 and 1) leaves other groups unchanged
    x = rand(64, 4, 4)
    y0 = oracle.group_norm(x, np.ones(64), np.zeros(64))
    x2 = x.copy()
    x2[0] = x2[0] * 5.0 + 1.0
    y1 = oracle.group_norm(x2, np.ones(64), np.zeros(64))
    assert np.array_equal(y0[2:], y1[2:])
    assert not np.allclose(y0[:2], y1[:2])


def test_group_norm_constant_group_gives_beta():
    x = rand(32, 3, 3)
    x[5] = 7.25
    beta = rand(32)
    y = oracle.group_norm(x, rand(32), beta)
    assert np.array_equal(y[5], np.full((3, 3), beta[5]))


def test_group_norm_affine_and_torch():
    x, gmm, bta = rand(128, 9, 13), rand(128), rand(128)
    ref = F.group_norm(t64(x)[None], 32, t64(gmm), t64(bta), eps=1e-6)[0].numpy()
    assert np.allclose(oracle.group_norm(x, gmm, bta), ref, atol=1e-10, rtol=0)
    # 5-D input (the causal stack): statistics over channels x T x H x W
    x5 = rand(64, 3, 4, 5)
    g5, b5 = rand(64), rand(64)
    ref5 = F.group_norm(t64(x5)[None], 32, t64(g5), t64(b5), eps=1e-6)[0].numpy()
    assert np.allclose(oracle.group_norm(x5, g5, b5), ref5, atol=1e-10, rtol=0)


def test_silu_closed_forms():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    x = rand(1000) * 10
    s = oracle.silu(x)
    assert np.allclose(s - oracle.silu(-x), x, atol=1e-12)
    brute = np.array([v / (1.0 + math.exp(-v)) for v in x])
    assert np.allclose(s, brute, atol=1e-14, rtol=1e-14)
    assert np.allclose(s, F.silu(t64(x)).numpy(), atol=1e-14)
    # large negative: tends to -0 without NaN
    assert oracle.silu(np.array([-1e4]))[0] == 0.0


def test_upsample_exact_replication():
    x = rand(3, 4, 5)
    u = oracle.upsample_nearest2x(x)
    assert u.shape == (3, 8, 10)
    for c in range(3):
        for y in range(8):
            for xx in range(10):
                assert u[c, y, xx] == x[c, y // 2, xx // 2]
    ref = F.interpolate(t64(x)[None], scale_factor=2, mode="nearest")[0].numpy()
    assert np.array_equal(u, ref)


def test_denormalize():
    s, t = vaegen.SCALING_FACTOR, vaegen.SHIFT_FACTOR
    z = np.array([0.0, s, -2 * s], dtype=np.float64)
    assert np.allclose(oracle.denormalize(z, s, t), [t, 1 + t, -2 + t], atol=1e-15)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def attn_params(c, rng_scale=1.0):
    p = {"a.group_norm.weight": 1 + 0.1 * rand(c), "a.group_norm.bias": 0.1 * rand(c)}
    for n in ("to_q", "to_k", "to_v", "to_out.0"):
        p[f"a.{n}.weight"] = rng_scale * rand(c, c) / math.sqrt(c)
        p[f"a.{n}.bias"] = 0.01 * rand(c)
    return p


def test_softmax_rows_sum_to_one_and_shift_invariant():
    s = rand(7, 11) * 20
    pr = oracle.softmax_rows(s)
    assert np.allclose(pr.sum(axis=1), 1.0, atol=1e-12)
    assert np.allclose(oracle.softmax_rows(s + 123.0), pr, atol=1e-12)
    e = np.exp(s[0] - s[0].max())
    assert np.allclose(pr[0], e / e.sum(), atol=1e-15)


def test_softmax_rows_of_very_different_scale():
    # each row is shifted by its own max: a row far below another stays finite
    s = np.array([[1000.0, 999.0], [0.0, -1.0]])
    pr = oracle.softmax_rows(s)
    e = 1.0 / (1.0 + math.exp(-1.0))
    assert np.allclose(pr, [[e, 1 - e], [e, 1 - e]], atol=1e-15)


def test_attention_single_token_closed_form():
    c = 32
    p = attn_params(c)
    x = rand(c, 1, 1)
    xn = oracle.group_norm(x, p["a.group_norm.weight"], p["a.group_norm.bias"])[:, 0, 0]
    v = p["a.to_v.weight"] @ xn + p["a.to_v.bias"]
    expect = x[:, 0, 0] + p["a.to_out.0.weight"] @ v + p["a.to_out.0.bias"]
    assert np.allclose(oracle.attention(x, p, "a")[:, 0, 0], expect, atol=1e-12)


def test_attention_zero_query_gives_mean_of_values():
    c = 32
    p = attn_params(c)
    p["a.to_q.weight"][:] = 0.0
    p["a.to_q.bias"][:] = 0.0
    x = rand(c, 3, 5)
    xn = oracle.group_norm(x, p["a.group_norm.weight"], p["a.group_norm.bias"]).reshape(c, -1)
    v = p["a.to_v.weight"] @ xn + p["a.to_v.bias"][:, None]
    o = v.mean(axis=1)
    expect = x.reshape(c, -1) + (p["a.to_out.0.weight"] @ o + p["a.to_out.0.bias"])[:, None]
    assert np.allclose(oracle.attention(x, p, "a").reshape(c, -1), expect, atol=1e-12)


def test_attention_brute_force_tiny():
    c, h, w = 32, 2, 3
    n = h * w
    p = attn_params(c, rng_scale=3.0)
    x = rand(c, h, w)
    xn = oracle.group_norm(x, p["a.group_norm.weight"], p["a.group_norm.bias"]).reshape(c, n)

    def lin(name, vec):
        W, b = p[f"a.{name}.weight"], p[f"a.{name}.bias"]
        return [sum(W[r, s] * vec[s] for s in range(c)) + b[r] for r in range(c)]

    toks = [[xn[ch, t] for ch in range(c)] for t in range(n)]
    q = [lin("to_q", tk) for tk in toks]
    k = [lin("to_k", tk) for tk in toks]
    v = [lin("to_v", tk) for tk in toks]
    y = np.zeros((c, n))
    for t in range(n):
        sc = [sum(q[t][r] * k[u][r] for r in range(c)) / math.sqrt(c) for u in range(n)]
        m = max(sc)
        e = [math.exp(s - m) for s in sc]
        den = sum(e)
        o = [sum(e[u] / den * v[u][r] for u in range(n)) for r in range(c)]
        out = lin("to_out.0", o)
        for r in range(c):
            y[r, t] = x.reshape(c, n)[r, t] + out[r]
    assert np.allclose(oracle.attention(x, p, "a").reshape(c, n), y, atol=1e-12)


def test_attention_token_permutation_equivariance():
    c, h, w = 32, 4, 4
    p = attn_params(c, rng_scale=2.0)
    x = rand(c, h, w)
    perm = RNG.permutation(h * w)
    y = oracle.attention(x, p, "a").reshape(c, -1)
    yp = oracle.attention(x.reshape(c, -1)[:, perm].reshape(c, h, w), p, "a").reshape(c, -1)
    assert np.allclose(yp, y[:, perm], atol=1e-12)


def test_attention_matches_torch_sdpa():
    c, h, w = 64, 6, 5
    p = attn_params(c, rng_scale=2.0)
    x = rand(c, h, w)
    xt = t64(x)
    xn = F.group_norm(xt[None], 32, t64(p["a.group_norm.weight"]), t64(p["a.group_norm.bias"]), eps=1e-6)[0]
    tok = xn.reshape(c, -1).T
    q = F.linear(tok, t64(p["a.to_q.weight"]), t64(p["a.to_q.bias"]))
    k = F.linear(tok, t64(p["a.to_k.weight"]), t64(p["a.to_k.bias"]))
    v = F.linear(tok, t64(p["a.to_v.weight"]), t64(p["a.to_v.bias"]))
    o = F.scaled_dot_product_attention(q[None, None], k[None, None], v[None, None], scale=1 / math.sqrt(c))[0, 0]
    out = F.linear(o, t64(p["a.to_out.0.weight"]), t64(p["a.to_out.0.bias"]))
    ref = (xt.reshape(c, -1) + out.T).reshape(c, h, w).numpy()
    assert np.allclose(oracle.attention(x, p, "a"), ref, atol=1e-11, rtol=0)


# ---------------------------------------------------------------------------
# resnet and the decoder
# ---------------------------------------------------------------------------

def res_params(cin, cout):
    p = {
        "r.norm1.weight": 1 + 0.1 * rand(cin), "r.norm1.bias": 0.1 * rand(cin),
        "r.conv1.weight": rand(cout, cin, 3, 3) / math.sqrt(9 * cin), "r.conv1.bias": 0.01 * rand(cout),
        "r.norm2.weight": 1 + 0.1 * rand(cout), "r.norm2.bias": 0.1 * rand(cout),
        "r.conv2.weight": rand(cout, cout, 3, 3) / math.sqrt(9 * cout), "r.conv2.bias": 0.01 * rand(cout),
    }
    if cin != cout:
        p["r.conv_shortcut.weight"] = rand(cout, cin, 1, 1) / math.sqrt(cin)
        p["r.conv_shortcut.bias"] = 0.01 * rand(cout)
    return p


def test_resnet_zero_residual_branch_is_skip():
    x = rand(64, 5, 6)
    p = res_params(64, 64)
    p["r.conv2.weight"][:] = 0
    p["r.conv2.bias"][:] = 0
    assert np.array_equal(oracle.resnet(x, p, "r"), x)
    p2 = res_params(64, 32)
    p2["r.conv2.weight"][:] = 0
    p2["r.conv2.bias"][:] = 0
    sc = F.conv2d(t64(x)[None], t64(p2["r.conv_shortcut.weight"]), t64(p2["r.conv_shortcut.bias"]))[0].numpy()
    assert np.allclose(oracle.resnet(x, p2, "r"), sc, atol=1e-12)


@pytest.mark.parametrize("cin,cout", [(64, 64), (64, 32)])
def test_resnet_matches_torch_composition(cin, cout):
    x = rand(cin, 7, 9)
    p = res_params(cin, cout)
    T = {k: t64(v) for k, v in p.items()}
    xt = t64(x)[None]
    h = F.silu(F.group_norm(xt, 32, T["r.norm1.weight"], T["r.norm1.bias"], eps=1e-6))
    h = F.conv2d(h, T["r.conv1.weight"], T["r.conv1.bias"], padding=1)
    h = F.silu(F.group_norm(h, 32, T["r.norm2.weight"], T["r.norm2.bias"], eps=1e-6))
    h = F.conv2d(h, T["r.conv2.weight"], T["r.conv2.bias"], padding=1)
    skip = F.conv2d(xt, T["r.conv_shortcut.weight"], T["r.conv_shortcut.bias"]) if cin != cout else xt
    assert np.allclose(oracle.resnet(x, p, "r"), (skip + h)[0].numpy(), atol=1e-11, rtol=0)


def small_decoder(seed=0):
    # the decoder's structure at reduced widths so the whole chain runs in ms
    return vaegen.decoder_params(seed, widths=(128, 128, 64, 32), latent_channels=4)


def test_decode_shape_law_and_layer_counts(monkeypatch):
    counts = {"conv3": 0, "conv1": 0, "gn": 0, "attn": 0, "up": 0}
    real_conv, real_gn, real_up = oracle.vae_oracle.conv2d, oracle.vae_oracle.group_norm, oracle.vae_oracle.upsample_nearest2x
    real_attn = oracle.vae_oracle.attention

    def conv(x, w, b):
        counts["conv3" if w.shape[-1] == 3 else "conv1"] += 1
        return real_conv(x, w, b)

    def gn(*a, **k):
        counts["gn"] += 1
        return real_gn(*a, **k)

    def up(x):
        counts["up"] += 1
        return real_up(x)

    def at(*a, **k):
        counts["attn"] += 1
        return real_attn(*a, **k)

    monkeypatch.setattr(oracle.vae_oracle, "conv2d", conv)
    monkeypatch.setattr(oracle.vae_oracle, "group_norm", gn)
    monkeypatch.setattr(oracle.vae_oracle, "upsample_nearest2x", up)
    monkeypatch.setattr(oracle.vae_oracle, "attention", at)
    p = small_decoder()
    for h, w in [(2, 3), (4, 4)]:
        z = vaegen.normal(0, "z", (4, h, w))
        y = oracle.vae_oracle.decode(z, p, 0.5, 0.1)
        assert y.shape == (3, 8 * h, 8 * w)
    assert counts == {"conv3": 66, "conv1": 4, "gn": 60, "attn": 2, "up": 6}


def test_decode_matches_torch_composition():
    p = small_decoder(seed=3)
    z = vaegen.normal(3, "z", (4, 3, 2))
    T = {k: t64(v) for k, v in p.items()}

    def gn(x, pre):
        return F.group_norm(x, 32, T[pre + ".weight"], T[pre + ".bias"], eps=1e-6)

    def cv(x, pre):
        w = T[pre + ".weight"]
        return F.conv2d(x, w, T[pre + ".bias"], padding=w.shape[-1] // 2)

    def res(x, pre):
        h = cv(F.silu(gn(x, pre + ".norm1")), pre + ".conv1")
        h = cv(F.silu(gn(h, pre + ".norm2")), pre + ".conv2")
        s = cv(x, pre + ".conv_shortcut") if pre + ".conv_shortcut.weight" in T else x
        return s + h

    def attn(x, pre):
        c = x.shape[1]
        tok = gn(x, pre + ".group_norm")[0].reshape(c, -1).T
        q = F.linear(tok, T[pre + ".to_q.weight"], T[pre + ".to_q.bias"])
        k = F.linear(tok, T[pre + ".to_k.weight"], T[pre + ".to_k.bias"])
        v = F.linear(tok, T[pre + ".to_v.weight"], T[pre + ".to_v.bias"])
        o = F.scaled_dot_product_attention(q[None], k[None], v[None], scale=c ** -0.5)[0]
        o = F.linear(o, T[pre + ".to_out.0.weight"], T[pre + ".to_out.0.bias"])
        return x + o.T.reshape(x.shape)

    x = t64(z)[None] / 0.5 + 0.1
    x = cv(x, "conv_in")
    x = res(x, "mid_block.resnets.0")
    x = attn(x, "mid_block.attentions.0")
    x = res(x, "mid_block.resnets.1")
    for i in range(4):
        for j in range(3):
            x = res(x, f"up_blocks.{i}.resnets.{j}")
        if i < 3:
            x = cv(F.interpolate(x, scale_factor=2, mode="nearest"), f"up_blocks.{i}.upsamplers.0.conv")
    x = cv(F.silu(gn(x, "conv_norm_out")), "conv_out")[0].numpy()
    y = oracle.decode(z, p, 0.5, 0.1)
    assert np.allclose(y, x, atol=1e-10, rtol=0)


# ---------------------------------------------------------------------------
# causal 3-D conv and the stack
# ---------------------------------------------------------------------------

def brute_conv3d(x, w, b):
    oc, ic = w.shape[:2]
    _, t, h, wd = x.shape
    y = np.zeros((oc, t, h, wd))
    for o in range(oc):
        for tt in range(t):
            for i in range(h):
                for j in range(wd):
                    acc = float(b[o])
                    for c in range(ic):
                        for dt in range(3):
                            src_t = max(tt + dt - 2, 0)
                            for dy in range(3):
                                for dx in range(3):
                                    yy, xx = i + dy - 1, j + dx - 1
                                    if 0 <= yy < h and 0 <= xx < wd:
                                        acc += float(w[o, c, dt, dy, dx]) * float(x[c, src_t, yy, xx])
                    y[o, tt, i, j] = acc
    return y


def test_conv3d_brute_force():
    x, w, b = rand(2, 4, 3, 4), rand(3, 2, 3, 3, 3), rand(3)
    assert np.allclose(oracle.conv3d_causal(x, w, b), brute_conv3d(x, w, b), atol=1e-12)
    for (o, t, i, j) in [(0, 0, 0, 0), (2, 3, 2, 3), (1, 1, 1, 0)]:
        assert math.isclose(oracle.conv3d_causal_at(x, w, b, o, t, i, j),
                            brute_conv3d(x, w, b)[o, t, i, j], abs_tol=1e-12)


def test_conv3d_causality():
    x, w, b = rand(3, 6, 5, 5), rand(4, 3, 3, 3, 3), rand(4)
    y = oracle.conv3d_causal(x, w, b)
    for tau in range(5):
        x2 = x.copy()
        x2[:, tau + 1] += rand(3, 5, 5)
        y2 = oracle.conv3d_causal(x2, w, b)
        assert np.array_equal(y2[:, :tau + 1], y[:, :tau + 1])
        assert not np.allclose(y2[:, tau + 1], y[:, tau + 1])


def test_conv3d_reduces_to_2d_on_the_first_frames():
    x, w, b = rand(3, 3, 6, 7), rand(4, 3, 3, 3, 3), rand(4)
    y = oracle.conv3d_causal(x, w, b)
    # frame 0 sees frame 0 through all three time taps
    ref0 = F.conv2d(t64(x[:, 0])[None], t64(w.sum(axis=2)), t64(b), padding=1)[0].numpy()
    assert np.allclose(y[:, 0], ref0, atol=1e-12)
    # frame 1: taps 0 and 1 see frame 0, tap 2 sees frame 1
    ref1 = (F.conv2d(t64(x[:, 0])[None], t64(w[:, :, 0] + w[:, :, 1]), t64(b), padding=1)
            + F.conv2d(t64(x[:, 1])[None], t64(w[:, :, 2]), None, padding=1))[0].numpy()
    assert np.allclose(y[:, 1], ref1, atol=1e-12)


def test_conv3d_matches_torch_with_replicated_front():
    x, w, b = rand(8, 5, 9, 7), rand(6, 8, 3, 3, 3), rand(6)
    xt = t64(x)
    front = xt[:, :1].expand(-1, 2, -1, -1)
    xp = torch.cat([front, xt], dim=1)
    ref = F.conv3d(xp[None], t64(w), t64(b), padding=(0, 1, 1))[0].numpy()
    assert np.allclose(oracle.conv3d_causal(x, w, b), ref, atol=1e-11, rtol=0)


def test_causal_stack_residual_placement():
    c = 32
    p = {}
    for i in range(4):
        p[f"stack.{i}.conv.weight"] = np.zeros((c, c, 3, 3, 3))
        p[f"stack.{i}.conv.bias"] = np.zeros(c)
        p[f"stack.{i}.norm.weight"] = 1 + 0.1 * rand(c)
        p[f"stack.{i}.norm.bias"] = rand(c)
    x = rand(c, 3, 4, 4)
    y = oracle.causal_stack(x, p)
    # every conv outputs 0, so each layer emits silu(beta): only layers 1 and 3 reach x
    add = oracle.silu(p["stack.1.norm.bias"]) + oracle.silu(p["stack.3.norm.bias"])
    assert np.allclose(y, x + add[:, None, None, None], atol=1e-14)


def test_causal_stack_matches_torch():
    c = 32
    p = vaegen.causal_stack_params(0, c=c)
    x = vaegen.normal(0, "x3", (c, 3, 5, 4))
    T = {k: t64(v) for k, v in p.items()}
    h = t64(x)
    for i in (0, 2):
        cur = h
        for j in (i, i + 1):
            front = cur[:, :1].expand(-1, 2, -1, -1)
            cur = F.conv3d(torch.cat([front, cur], 1)[None], T[f"stack.{j}.conv.weight"],
                           T[f"stack.{j}.conv.bias"], padding=(0, 1, 1))
            cur = F.silu(F.group_norm(cur, 32, T[f"stack.{j}.norm.weight"], T[f"stack.{j}.norm.bias"], eps=1e-6))[0]
        h = h + cur
    assert np.allclose(oracle.causal_stack(x, p), h.numpy(), atol=1e-11, rtol=0)


# ---------------------------------------------------------------------------
# the causal 3-D decoder
# ---------------------------------------------------------------------------

def small_decoder3d(seed):
    return vaegen.decoder_params(seed, widths=(64, 64, 32, 32), latent_channels=4, dims=3)


def test_pointwise_conv_is_the_1x1_conv():
    x = rand(12, 5, 7)
    w, b = rand(9, 12, 1, 1), rand(9)
    assert np.allclose(oracle.pointwise_conv(x, w, b), oracle.conv2d(x, w, b), atol=1e-13)
    x4 = rand(12, 3, 5, 7)
    y4 = oracle.pointwise_conv(x4, w[..., None], b)
    for t in range(3):
        assert np.allclose(y4[:, t], oracle.conv2d(x4[:, t], w, b), atol=1e-13)


def test_decode_causal3d_single_frame_is_the_2d_decode():
    # one frame: the front padding repeats that frame, so every causal conv is a
    # 2-D conv with the time taps summed, and the 1x1x1 skips are 1x1 convs
    p3 = small_decoder3d(5)
    p2 = {}
    for k, v in p3.items():
        if v.ndim == 5:
            v = v.astype(np.float64).sum(axis=2) if v.shape[2] == 3 else v[:, :, 0]
        p2[k] = v
    z = vaegen.normal(5, "z3", (4, 1, 3, 2))
    y3 = oracle.decode_causal3d(z, p3, 0.5, 0.1)
    y2 = oracle.decode(z[:, 0], p2, 0.5, 0.1)
    assert y3.shape == (3, 1, 24, 16)
    assert np.allclose(y3[:, 0], y2, atol=1e-10, rtol=0)


def test_decode_causal3d_repeated_frame():
    # a clip that repeats one frame: every layer keeps the frames equal (the
    # causal window sees copies of frame 0, the GroupNorm statistics and the
    # attention's key set are those of one frame, duplicated)
    p3 = small_decoder3d(6)
    z1 = vaegen.normal(6, "z3", (4, 1, 2, 3))
    y1 = oracle.decode_causal3d(z1, p3, 0.5, 0.1)
    y3 = oracle.decode_causal3d(np.concatenate([z1] * 3, axis=1), p3, 0.5, 0.1)
    assert y3.shape == (3, 3, 16, 24)
    for t in range(3):
        assert np.allclose(y3[:, t], y1[:, 0], atol=1e-10, rtol=0)


def test_decode_causal3d_matches_torch_composition():
    p = small_decoder3d(7)
    z = vaegen.normal(7, "z3", (4, 3, 2, 3))
    T = {k: t64(v) for k, v in p.items()}

    def gn(x, pre):
        return F.group_norm(x, 32, T[pre + ".weight"], T[pre + ".bias"], eps=1e-6)

    def cv(x, pre):
        w = T[pre + ".weight"]
        if w.shape[2] == 1:
            return F.conv3d(x, w, T[pre + ".bias"])
        front = x[:, :, :1].expand(-1, -1, 2, -1, -1)
        return F.conv3d(torch.cat([front, x], 2), w, T[pre + ".bias"], padding=(0, 1, 1))

    def res(x, pre):
        h = cv(F.silu(gn(x, pre + ".norm1")), pre + ".conv1")
        h = cv(F.silu(gn(h, pre + ".norm2")), pre + ".conv2")
        s = cv(x, pre + ".conv_shortcut") if pre + ".conv_shortcut.weight" in T else x
        return s + h

    def attn(x, pre):
        c = x.shape[1]
        tok = gn(x, pre + ".group_norm")[0].reshape(c, -1).T
        q = F.linear(tok, T[pre + ".to_q.weight"], T[pre + ".to_q.bias"])
        k = F.linear(tok, T[pre + ".to_k.weight"], T[pre + ".to_k.bias"])
        v = F.linear(tok, T[pre + ".to_v.weight"], T[pre + ".to_v.bias"])
        o = F.scaled_dot_product_attention(q[None], k[None], v[None], scale=c ** -0.5)[0]
        o = F.linear(o, T[pre + ".to_out.0.weight"], T[pre + ".to_out.0.bias"])
        return x + o.T.reshape(x.shape)

    x = t64(z)[None] / 0.5 + 0.1
    x = cv(x, "conv_in")
    x = res(x, "mid_block.resnets.0")
    x = attn(x, "mid_block.attentions.0")
    x = res(x, "mid_block.resnets.1")
    for i in range(4):
        for j in range(3):
            x = res(x, f"up_blocks.{i}.resnets.{j}")
        if i < 3:
            x = cv(F.interpolate(x, scale_factor=(1, 2, 2), mode="nearest"), f"up_blocks.{i}.upsamplers.0.conv")
    x = cv(F.silu(gn(x, "conv_norm_out")), "conv_out")[0].numpy()
    y = oracle.decode_causal3d(z, p, 0.5, 0.1)
    assert y.shape == (3, 3, 16, 24)
    assert np.allclose(y, x, atol=1e-10, rtol=0)
