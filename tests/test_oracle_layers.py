"""Pins for the oracle's rotary positions, attention, convolutions, norms and block.

References used: page-printed facts (tests/golden/rope.json), closed forms of plane
rotations, brute-force loops in float64 on tiny shapes, numpy.correlate/convolve, and
degenerate parameter choices that reduce a module to a known function.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ RoPE tables

def test_rope_base_divergence_matches_page():
    g = _gold("rope.json")
    dk = g["d_model"] // g["n_heads"]
    L = int(g["clip_seconds_for_claim"] * 16000)
    U = oracle.encoder_frames(L)[2]
    c5, s5 = oracle.rope_tables(U, dk, g["base"])
    c10, s10 = oracle.rope_tables(U, dk, g["wrong_base"])
    lo, hi = g["table_divergence_bounds"]
    dc = np.abs(c5 - c10).max()
    ds = np.abs(s5 - s10).max()
    assert lo <= max(dc, ds) <= hi
    # at the longest positions of a 20 s clip the tables come apart by ~2
    c5, _ = oracle.rope_tables(500, dk, 5000.0)
    c10, _ = oracle.rope_tables(500, dk, 10000.0)
    assert np.abs(c5 - c10).max() > 1.99


def test_rope_closed_forms():
    dk = 48
    cos, sin = oracle.rope_tables(10, dk, 5000.0)
    np.testing.assert_array_equal(cos[0], 1.0)
    np.testing.assert_array_equal(sin[0], 0.0)
    # pair i uses frequency 5000^(-2i/dk); position 3, pair 5
    ang = 3 * 5000.0 ** (-10.0 / 48)
    assert abs(cos[3, 5] - np.cos(ang)) < 1e-15 and abs(cos[3, 5 + 24] - np.cos(ang)) < 1e-15
    assert abs(sin[3, 5] - np.sin(ang)) < 1e-15
    # pair 0 turns by exactly one radian per position
    np.testing.assert_allclose(cos[:, 0], np.cos(np.arange(10)), atol=1e-15)


def test_rope_is_rotation_and_relative():
    rng = np.random.default_rng(0)
    H, dk, T = 2, 8, 6
    y = rng.standard_normal((T, H * dk))
    r = oracle.apply_rope(y, H, 5000.0)
    # per-head norms preserved
    np.testing.assert_allclose(np.linalg.norm(r.reshape(T, H, dk), axis=2),
                               np.linalg.norm(y.reshape(T, H, dk), axis=2), rtol=1e-12)
    # <R_m a, R_n b> depends on m - n only
    a, b = rng.standard_normal(dk), rng.standard_normal(dk)

    def rot(v, t):
        z = np.zeros((t + 1, dk))
        z[t] = v
        return oracle.apply_rope(z, 1, 5000.0)[t]
    d1 = rot(a, 5) @ rot(b, 2)
    d2 = rot(a, 4) @ rot(b, 1)
    assert abs(d1 - d2) < 1e-12
    # the rotation pairs element i with i + dk/2 (rotate_half), as a 2x2 plane rotation
    v = np.zeros(dk)
    v[1] = 1.0
    out = rot(v, 1)
    th = 5000.0 ** (-2.0 / dk)
    expect = np.zeros(dk)
    expect[1], expect[1 + dk // 2] = np.cos(th), np.sin(th)
    np.testing.assert_allclose(out, expect, atol=1e-15)


def test_rotation_before_projection_hand_check():
    """q comes from the rotated input, v from the raw input (value not rotated);
    rotating after the projection gives a different q."""
    rng = np.random.default_rng(3)
    T, d, H = 3, 4, 1
    y = rng.standard_normal((T, d))
    P = {}
    for n in ("linear_q", "linear_k", "linear_v", "linear_out"):
        P["a." + n + ".weight"] = rng.standard_normal((d, d))
        P["a." + n + ".bias"] = np.zeros(d)
    P["a.linear_out.weight"] = np.eye(d)
    # hand-built rotation for d_k = 4: pairs (0,2), (1,3), frequencies 1 and 5000^-0.5
    def R(t):
        M = np.eye(4)
        for i, w in enumerate([1.0, 5000.0 ** -0.5]):
            c, s = np.cos(t * w), np.sin(t * w)
            M[i, i], M[i, i + 2], M[i + 2, i], M[i + 2, i + 2] = c, -s, s, c
        return M
    q_expect = np.stack([P["a.linear_q.weight"] @ (R(t) @ y[t]) for t in range(T)])
    k_expect = np.stack([P["a.linear_k.weight"] @ (R(t) @ y[t]) for t in range(T)])
    v_expect = y @ P["a.linear_v.weight"].T
    out = oracle.mhsa_rope(y, P, "a.", H, 5000.0)
    s = q_expect @ k_expect.T / 2.0
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    np.testing.assert_allclose(out, p @ v_expect, rtol=1e-10, atol=1e-12)
    # post-projection rotation differs
    q_post = np.stack([R(t) @ (P["a.linear_q.weight"] @ y[t]) for t in range(T)])
    assert np.abs(q_post - q_expect).max() > 1e-3


# ------------------------------------------------------------------ attention

def _attn_brute(q, k, v, H, valid):
    T, d = q.shape
    dk = d // H
    out = np.zeros((T, d))
    for h in range(H):
        for i in range(T):
            sc = [sum(q[i, h * dk + c] * k[j, h * dk + c] for c in range(dk)) / dk ** 0.5
                  for j in range(valid)]
            m = max(sc)
            e = [np.exp(s - m) for s in sc]
            z = sum(e)
            for c in range(dk):
                out[i, h * dk + c] = sum(e[j] / z * v[j, h * dk + c] for j in range(valid))
    return out


@pytest.mark.parametrize("T,H,dk", [(5, 2, 4), (9, 1, 48), (1, 3, 4)])
def test_attention_brute_force(T, H, dk):
    rng = np.random.default_rng(T * 7 + dk)
    q, k, v = (rng.standard_normal((T, H * dk)) for _ in range(3))
    np.testing.assert_allclose(oracle.attention(q, k, v, H), _attn_brute(q, k, v, H, T), rtol=1e-12, atol=1e-12)


def test_attention_key_padding_and_degenerate_cases():
    rng = np.random.default_rng(5)
    T, H, dk, valid = 7, 2, 4, 4
    q, k, v = (rng.standard_normal((T, H * dk)) for _ in range(3))
    ref = _attn_brute(q, k, v, H, valid)
    k2, v2 = k.copy(), v.copy()
    k2[valid:] = 1e3 * rng.standard_normal((T - valid, H * dk))
    v2[valid:] = np.nan
    out = oracle.attention(q, k2, v2, H, key_valid=valid)
    np.testing.assert_allclose(out, ref, rtol=1e-12)
    # identical keys -> output is the mean of the (valid) values
    keq = np.tile(k[:1], (T, 1))
    out = oracle.attention(q, keq, v, H)
    np.testing.assert_allclose(out, np.tile(v.mean(0), (T, 1)), rtol=1e-12)


# ------------------------------------------------------------------ convolutions

def test_conv1d_brute_force_and_correlate():
    rng = np.random.default_rng(7)
    T, Cin, Cout, K = 11, 3, 4, 5
    x = rng.standard_normal((T, Cin))
    w = rng.standard_normal((Cout, Cin, K))
    b = rng.standard_normal(Cout)
    for stride in (1, 2):
        out = oracle.conv1d(x, w, b, stride=stride, pad=2)
        S = (T + 4 - K) // stride + 1
        ref = np.zeros((S, Cout))
        for s in range(S):
            for o in range(Cout):
                acc = b[o]
                for c in range(Cin):
                    for j in range(K):
                        t = stride * s + j - 2
                        if 0 <= t < T:
                            acc += w[o, c, j] * x[t, c]
                ref[s, o] = acc
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # stride 1 equals numpy.correlate per (out, in) pair ('same' with pad 2, K 5)
    out1 = oracle.conv1d(x, w, None, stride=1, pad=2)
    ref = np.zeros_like(out1)
    for o in range(Cout):
        for c in range(Cin):
            ref[:, o] += np.correlate(np.pad(x[:, c], 2), w[o, c], mode="valid")
    np.testing.assert_allclose(out1, ref, rtol=1e-12, atol=1e-12)
    # stride 2 output is every other stride-1 output
    np.testing.assert_allclose(oracle.conv1d(x, w, None, 2, 2), out1[::2], rtol=1e-12, atol=1e-12)


def test_depthwise_impulse_and_convolve():
    rng = np.random.default_rng(8)
    C, K, T = 3, 31, 40
    w = rng.standard_normal((C, K))
    b = np.zeros(C)
    x = np.zeros((T, C))
    x[20] = 1.0
    out = oracle.depthwise_conv1d(x, w, b)
    # cross-correlation: an impulse at 20 shows the taps reversed around it
    for c in range(C):
        np.testing.assert_allclose(out[20 - 15:20 + 16, c], w[c, ::-1], rtol=1e-15)
    x = rng.standard_normal((T, C))
    out = oracle.depthwise_conv1d(x, w, b)
    for c in range(C):
        np.testing.assert_allclose(out[:, c], np.convolve(x[:, c], w[c, ::-1], mode="same"), rtol=1e-12, atol=1e-12)
    # zero halo: a clip of length 1 sees only the centre tap
    one = oracle.depthwise_conv1d(np.ones((1, C)), w, b)
    np.testing.assert_allclose(one[0], w[:, 15])


# ------------------------------------------------------------------ norms / activations

def test_layer_norm_statistics():
    rng = np.random.default_rng(9)
    x = 3 + 2 * rng.standard_normal((5, 768))
    y = oracle.layer_norm(x, np.ones(768), np.zeros(768), eps=0.0)
    np.testing.assert_allclose(y.mean(1), 0, atol=1e-12)
    np.testing.assert_allclose(y.var(1), 1, atol=1e-12)
    g, b = rng.standard_normal(768), rng.standard_normal(768)
    np.testing.assert_allclose(oracle.layer_norm(x, g, b, 0.0), y * g + b, rtol=1e-12)


def test_batch_norm_identity_and_affine():
    x = np.random.default_rng(10).standard_normal((4, 6))
    eps = 1e-5
    np.testing.assert_allclose(oracle.batch_norm_inference(x, 1, 0, 0, 1 - eps, eps), x, rtol=1e-12)
    # folding into alpha, beta gives the same result
    g, b, m, v = 1.3, -0.2, 0.4, 0.8
    a = g / np.sqrt(v + eps)
    np.testing.assert_allclose(oracle.batch_norm_inference(x, g, b, m, v, eps), a * x + (b - m * a), rtol=1e-12)


def test_activations_known_values():
    assert oracle.silu(np.array(0.0)) == 0.0
    assert abs(oracle.silu(np.array(1.0)) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16
    assert abs(oracle.silu(np.array(40.0)) - 40.0) < 1e-12
    x = np.array([[1.0, -2.0, 50.0, 50.0]])
    np.testing.assert_allclose(oracle.glu(x), [[1.0, -2.0]], rtol=1e-12)   # open gate
    x = np.array([[1.0, -2.0, -50.0, 0.0]])
    np.testing.assert_allclose(oracle.glu(x), [[0.0, -1.0]], atol=1e-20)


# ------------------------------------------------------------------ block composition

def _zero_block(d, f, k, i=0):
    P = {}
    p = f"layers.{i}."
    for ff in ("ff1.", "ff2."):
        P[p + ff + "norm.weight"], P[p + ff + "norm.bias"] = np.ones(d), np.zeros(d)
        P[p + ff + "linear1.weight"], P[p + ff + "linear1.bias"] = np.zeros((f, d)), np.zeros(f)
        P[p + ff + "linear2.weight"], P[p + ff + "linear2.bias"] = np.zeros((d, f)), np.zeros(d)
    P[p + "att.norm.weight"], P[p + "att.norm.bias"] = np.ones(d), np.zeros(d)
    for n in ("linear_q", "linear_k", "linear_v", "linear_out"):
        P[p + "att." + n + ".weight"], P[p + "att." + n + ".bias"] = np.zeros((d, d)), np.zeros(d)
    P[p + "conv.norm.weight"], P[p + "conv.norm.bias"] = np.ones(d), np.zeros(d)
    P[p + "conv.pointwise1.weight"], P[p + "conv.pointwise1.bias"] = np.zeros((2 * d, d)), np.zeros(2 * d)
    P[p + "conv.depthwise.weight"], P[p + "conv.depthwise.bias"] = np.zeros((d, k)), np.zeros(d)
    P[p + "conv.bn.weight"], P[p + "conv.bn.bias"] = np.ones(d), np.zeros(d)
    P[p + "conv.bn.running_mean"], P[p + "conv.bn.running_var"] = np.zeros(d), np.ones(d)
    P[p + "conv.pointwise2.weight"], P[p + "conv.pointwise2.bias"] = np.zeros((d, d)), np.zeros(d)
    P[p + "norm_out.weight"], P[p + "norm_out.bias"] = np.ones(d), np.zeros(d)
    return P


def test_block_order_and_half_steps():
    """With module outputs forced to constants through their last biases, the block
    output is LN(x + c1/2 + c_att + c_conv + c2/2): pins the macaron half steps, the
    residual adds and the final norm."""
    d, f, k = 8, 16, 5
    cfg = dict(n_heads=2, rope_base=5000.0, ln_eps=1e-5, bn_eps=1e-5)
    rng = np.random.default_rng(11)
    P = _zero_block(d, f, k)
    c = {n: rng.standard_normal(d) for n in ("ff1", "att", "conv", "ff2")}
    P["layers.0.ff1.linear2.bias"] = c["ff1"]
    P["layers.0.att.linear_out.bias"] = c["att"]
    P["layers.0.conv.pointwise2.bias"] = c["conv"]
    P["layers.0.ff2.linear2.bias"] = c["ff2"]
    x = rng.standard_normal((6, d))
    out = oracle.conformer_block(x, P, 0, cfg)
    pre = x + 0.5 * c["ff1"] + c["att"] + c["conv"] + 0.5 * c["ff2"]
    mu = pre.mean(1, keepdims=True)
    sd = np.sqrt(((pre - mu) ** 2).mean(1, keepdims=True) + 1e-5)
    np.testing.assert_allclose(out, (pre - mu) / sd, rtol=1e-12)


def test_conv_module_glu_dw_bn_silu_chain():
    """Conv module with identity-like pointwise weights: output = SiLU(BN(dw(GLU)))."""
    d, k, T = 4, 5, 9
    rng = np.random.default_rng(12)
    P = {"c.norm.weight": np.ones(d), "c.norm.bias": np.zeros(d)}
    W1 = np.zeros((2 * d, d))
    W1[:d] = np.eye(d)
    P["c.pointwise1.weight"], P["c.pointwise1.bias"] = W1, np.concatenate([np.zeros(d), 60 * np.ones(d)])
    P["c.depthwise.weight"], P["c.depthwise.bias"] = rng.standard_normal((d, k)), rng.standard_normal(d)
    g, b, m, v = rng.standard_normal(d), rng.standard_normal(d), rng.standard_normal(d), rng.uniform(0.5, 1.5, d)
    P["c.bn.weight"], P["c.bn.bias"], P["c.bn.running_mean"], P["c.bn.running_var"] = g, b, m, v
    P["c.pointwise2.weight"], P["c.pointwise2.bias"] = np.eye(d), np.zeros(d)
    x = rng.standard_normal((T, d))
    y = oracle.layer_norm(x, np.ones(d), np.zeros(d), 1e-5)
    gate = 1.0 / (1.0 + np.exp(-60.0))
    dw = np.zeros((T, d))
    for t in range(T):
        for c in range(d):
            dw[t, c] = P["c.depthwise.bias"][c] + sum(
                P["c.depthwise.weight"][c, j] * y[t + j - 2, c] * gate
                for j in range(k) if 0 <= t + j - 2 < T)
    bn = (dw - m) / np.sqrt(v + 1e-5) * g + b
    expect = bn / (1.0 + np.exp(-bn))
    np.testing.assert_allclose(oracle.conv_module(x, P, "c.", 1e-5, 1e-5), expect, rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------------ macaron feed-forward

LN3 = float(np.log(3.0))


def ffn_closed_form_case():
    """A 4-wide feed-forward module with non-zero weights whose output is a closed form.

    Rows [1, 2, 3, 4] and [10, 13, 16, 19] have the same standardised values
    n = [-3, -1, 1, 3] / sqrt(5) (LayerNorm with eps 0 ignores shift and positive scale).
    Gain sqrt(5) ln3 [1/3, 1, 1, 1/3] and shift [0, ln3, 0, 0] make the norm output
    y = ln3 [-1, 0, 1, 1]. linear1 takes unit i from y[(i + 1) mod 4] (a cyclic permutation,
    so a transposed weight picks other entries) plus b1 = [0, 0, ln3, 0]:
    pre-activation ln3 [0, 1, 2, -1]. The logistic function at k ln3 is 3^k / (3^k + 1), so
    SiLU gives ln3 [0, 3/4, 9/5, -1/4] exactly. linear2 = diag(1, 2, 1, 1) plus 4 at
    [0, 3] (not symmetric), b2 = [1, 0, 0, 0]: output [1 - ln3, 3/2 ln3, 9/5 ln3, -1/4 ln3].
    A ReLU in place of SiLU, a missing LayerNorm, a transposed weight or a dropped bias
    each moves at least one entry by more than 0.2."""
    d = 4
    P = {"f.norm.weight": np.sqrt(5.0) * LN3 * np.array([1 / 3, 1.0, 1.0, 1 / 3]),
         "f.norm.bias": np.array([0.0, LN3, 0.0, 0.0])}
    W1 = np.zeros((d, d))
    for i in range(d):
        W1[i, (i + 1) % d] = 1.0
    P["f.linear1.weight"], P["f.linear1.bias"] = W1, np.array([0.0, 0.0, LN3, 0.0])
    W2 = np.diag([1.0, 2.0, 1.0, 1.0])
    W2[0, 3] = 4.0
    P["f.linear2.weight"], P["f.linear2.bias"] = W2, np.array([1.0, 0.0, 0.0, 0.0])
    x = np.array([[1.0, 2.0, 3.0, 4.0], [10.0, 13.0, 16.0, 19.0]])
    row = np.array([1.0 - LN3, 1.5 * LN3, 1.8 * LN3, -0.25 * LN3])
    return x, P, np.stack([row, row])


def check_feed_forward_closed_form():
    x, P, expect = ffn_closed_form_case()
    np.testing.assert_allclose(oracle.feed_forward(x, P, "f.", 0.0), expect, rtol=1e-13, atol=1e-13)


def test_feed_forward_closed_form():
    check_feed_forward_closed_form()


def check_block_with_live_ffn():
    """A block whose only non-zero module is the first FFN (the closed-form one above, 4
    wide): output = LN_out(x + FFN(x) / 2), so the half step acts on a non-constant,
    SiLU-shaped module output."""
    d, f, k = 4, 4, 5
    cfg = dict(n_heads=1, rope_base=5000.0, ln_eps=0.0, bn_eps=1e-5)
    P = _zero_block(d, f, k)
    x, F, ffn = ffn_closed_form_case()
    for n in ("norm.weight", "norm.bias", "linear1.weight", "linear1.bias", "linear2.weight",
              "linear2.bias"):
        P["layers.0.ff1." + n] = F["f." + n]
    out = oracle.conformer_block(x, P, 0, cfg)
    pre = x + 0.5 * ffn
    mu = pre.mean(1, keepdims=True)
    sd = np.sqrt(((pre - mu) ** 2).mean(1, keepdims=True))
    np.testing.assert_allclose(out, (pre - mu) / sd, rtol=1e-12, atol=1e-12)


def test_block_with_live_ffn():
    check_block_with_live_ffn()


# ------------------------------------------------------------------ subsampling

def check_subsample_relu_between_convs():
    """Two 1-channel stride-2 convs that pass the centre tap only (weight 1 at tap 2):
    subsample(x)[u] = relu(relu(x[4u] + b1) + b2). With b1 = -1 and b2 = +1, an input of
    [-3, 0, 3, ...] at the kept positions shows whether the ReLU sits after each conv:
    with it, x[4u] = -3 gives relu(0) + ... = 1; without the inner one it gives -3."""
    T = 13
    x = np.zeros((T, 1))
    x[0::4, 0] = [-3.0, 0.5, 3.0, -0.5]
    w = np.zeros((1, 1, 5))
    w[0, 0, 2] = 1.0
    P = {"pre.conv1.weight": w, "pre.conv1.bias": np.array([-1.0]),
         "pre.conv2.weight": w, "pre.conv2.bias": np.array([1.0])}
    out = oracle.subsample(x, P)
    np.testing.assert_array_equal(out[:, 0], [1.0, 1.0, 3.0, 1.0])


def test_subsample_relu_between_convs():
    check_subsample_relu_between_convs()
