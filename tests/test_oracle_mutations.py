"""Planted mistakes: each test swaps one oracle function for a plausible wrong variant
(on the CPU, inside this test only) and checks that a pin notices it."""
import numpy as np
import pytest

import oracle


def _bin_centred_ok():
    A, k0 = 0.7, 17
    n = np.arange(320)
    P = oracle.dft_power((A * np.cos(2 * np.pi * k0 * n / 320) * oracle.hann_periodic(320))[None])[0]
    expect = np.zeros(161)
    expect[k0] = 6400 * A * A
    expect[k0 - 1] = expect[k0 + 1] = 1600 * A * A
    return np.allclose(P, expect, atol=1e-9)


def test_symmetric_window_is_caught(monkeypatch):
    assert _bin_centred_ok()
    monkeypatch.setattr(oracle, "hann_periodic",
                        lambda n=320, dtype=np.float64: 0.5 - 0.5 * np.cos(2 * np.pi * np.arange(n) / (n - 1)))
    assert not _bin_centred_ok()


def test_dropped_imaginary_part_is_caught(monkeypatch):
    def bad(frames, n_fft=320):
        n = np.arange(n_fft)
        k = np.arange(n_fft // 2 + 1)
        re = frames @ np.cos(2 * np.pi * np.outer(n, k) / n_fft)
        return re * re
    monkeypatch.setattr(oracle, "dft_power", bad)
    fr = np.random.default_rng(0).standard_normal((2, 320))
    assert not np.allclose(oracle.dft_power(fr), np.abs(np.fft.rfft(fr, axis=1)) ** 2)


def test_rope_base_10000_is_caught():
    c5, _ = oracle.rope_tables(98, 48, 5000.0)
    c10, _ = oracle.rope_tables(98, 48, 10000.0)
    # the page's divergence only appears between the two bases; same base -> 0
    assert np.abs(c5 - c10).max() > 1.8
    assert np.abs(c5 - oracle.rope_tables(98, 48, 5000.0)[0]).max() == 0


def test_wrong_rotate_half_sign_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "rotate_half",
                        lambda v: np.concatenate([v[..., v.shape[-1] // 2:], -v[..., :v.shape[-1] // 2]], -1))
    dk = 8
    v = np.zeros(dk)
    v[1] = 1.0
    z = np.zeros((2, dk))
    z[1] = v
    out = oracle.apply_rope(z, 1, 5000.0)[1]
    th = 5000.0 ** (-2.0 / dk)
    assert abs(out[1 + dk // 2] - np.sin(th)) > 1e-3


def test_collapse_dropping_blanks_first_is_caught(monkeypatch):
    def bad(ids, blank):
        ids = [i for i in ids if i != blank]
        out, prev = [], None
        for t in ids:
            if t != prev:
                out.append(t)
            prev = t
        return out
    monkeypatch.setattr(oracle, "ctc_collapse", bad)
    assert oracle.ctc_collapse([5, 5, 33, 5, 7, 7], 33) != [5, 5, 7]


def test_attention_missing_scale_is_caught(monkeypatch):
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((5, 8)) for _ in range(3))
    good = oracle.attention(q, k, v, 2)

    def bad(q, k, v, n_heads, key_valid=None):
        out = np.zeros_like(q)
        dk = q.shape[1] // n_heads
        for h in range(n_heads):
            sl = slice(h * dk, (h + 1) * dk)
            s = q[:, sl] @ k[:, sl].T
            p = np.exp(s - s.max(1, keepdims=True))
            out[:, sl] = (p / p.sum(1, keepdims=True)) @ v[:, sl]
        return out
    monkeypatch.setattr(oracle, "attention", bad)
    assert not np.allclose(oracle.attention(q, k, v, 2), good)


@pytest.mark.parametrize("pad", [0, 1, 3])
def test_wrong_subsampling_padding_is_caught(pad):
    # only padding 2 maps the printed 99 -> 25 and 1999 -> 500
    f = lambda n: oracle.conv_out_len(oracle.conv_out_len(n, pad=pad), pad=pad)
    assert (f(99), f(1999)) != (25, 500)


# ---- feed-forward, half steps and subsampling (pins in test_oracle_layers.py)

from test_oracle_layers import (check_block_with_live_ffn, check_feed_forward_closed_form,  # noqa: E402
                                check_subsample_relu_between_convs, test_block_order_and_half_steps)


def _fails(check):
    try:
        check()
    except AssertionError:
        return True
    return False


def test_relu_for_silu_is_caught(monkeypatch):
    assert not _fails(check_feed_forward_closed_form)
    monkeypatch.setattr(oracle, "silu", oracle.relu)
    assert _fails(check_feed_forward_closed_form)
    assert _fails(check_block_with_live_ffn)


def test_ffn_without_layer_norm_is_caught(monkeypatch):
    def bad(x, P, pre, eps):
        h = oracle.silu(oracle.linear(x, P[pre + "linear1.weight"], P[pre + "linear1.bias"]))
        return oracle.linear(h, P[pre + "linear2.weight"], P[pre + "linear2.bias"])
    monkeypatch.setattr(oracle, "feed_forward", bad)
    assert _fails(check_feed_forward_closed_form)
    assert _fails(check_block_with_live_ffn)


def test_ffn_transposed_weight_is_caught(monkeypatch):
    def bad(x, P, pre, eps):
        y = oracle.layer_norm(x, P[pre + "norm.weight"], P[pre + "norm.bias"], eps)
        h = oracle.silu(y @ P[pre + "linear1.weight"] + P[pre + "linear1.bias"])
        return oracle.linear(h, P[pre + "linear2.weight"], P[pre + "linear2.bias"])
    monkeypatch.setattr(oracle, "feed_forward", bad)
    assert _fails(check_feed_forward_closed_form)


def test_full_ffn_step_is_caught(monkeypatch):
    """The macaron half steps replaced by full residual adds."""
    def bad(x, P, i, cfg):
        p = f"layers.{i}."
        eps, bn_eps = cfg["ln_eps"], cfg["bn_eps"]
        x = x + oracle.feed_forward(x, P, p + "ff1.", eps)
        y = oracle.layer_norm(x, P[p + "att.norm.weight"], P[p + "att.norm.bias"], eps)
        x = x + oracle.mhsa_rope(y, P, p + "att.", cfg["n_heads"], cfg["rope_base"])
        x = x + oracle.conv_module(x, P, p + "conv.", eps, bn_eps)
        x = x + oracle.feed_forward(x, P, p + "ff2.", eps)
        return oracle.layer_norm(x, P[p + "norm_out.weight"], P[p + "norm_out.bias"], eps)
    assert not _fails(check_block_with_live_ffn)
    monkeypatch.setattr(oracle, "conformer_block", bad)
    assert _fails(check_block_with_live_ffn)
    assert _fails(test_block_order_and_half_steps)


def test_subsampling_without_inner_relu_is_caught(monkeypatch):
    def bad(mel, P):
        h = oracle.conv1d(mel, P["pre.conv1.weight"], P["pre.conv1.bias"], stride=2, pad=2)
        return oracle.relu(oracle.conv1d(h, P["pre.conv2.weight"], P["pre.conv2.bias"], stride=2, pad=2))
    assert not _fails(check_subsample_relu_between_convs)
    monkeypatch.setattr(oracle, "subsample", bad)
    assert _fails(check_subsample_relu_between_convs)
