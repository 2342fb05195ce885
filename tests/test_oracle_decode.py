"""Pins for the oracle's CTC head, greedy collapse, int8 dequantisation and the whole
per-clip forward (batch semantics, float32 self-bound)."""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ CTC head + greedy

def test_log_softmax_normalised_and_shift_invariant():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((6, 5))
    P = {"head.weight": rng.standard_normal((34, 5)), "head.bias": rng.standard_normal(34)}
    lp = oracle.ctc_log_probs(x, P)
    np.testing.assert_allclose(np.exp(lp).sum(1), 1.0, rtol=1e-12)
    P2 = dict(P, **{"head.bias": P["head.bias"] + 123.0})
    np.testing.assert_allclose(oracle.ctc_log_probs(x, P2), lp, atol=1e-12)
    # large logits do not overflow
    P3 = dict(P, **{"head.bias": P["head.bias"] * 1e4})
    assert np.all(np.isfinite(oracle.ctc_log_probs(x, P3)))


def test_argmax_lowest_index_on_ties():
    lp = np.array([[0.0, 1.0, 1.0, -1.0], [2.0, 2.0, 2.0, 2.0]])
    np.testing.assert_array_equal(oracle.greedy_ids(lp), [1, 0])


def test_collapse_golden_cases():
    g = _gold("ctc_collapse.json")
    for lay in g["class_layouts"]:
        assert lay["blank"] == lay["vocab"] and lay["classes"] == lay["vocab"] + 1
    for case in g["cases"]:
        assert oracle.ctc_collapse(case["ids"], case["blank"]) == case["tokens"], case


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(0, 5), max_size=12), st.data())
def test_collapse_inverts_any_ctc_expansion(tokens, data):
    """Expanding a token list with repeats and blanks (a blank always separates equal
    neighbours) and collapsing it gives the list back."""
    blank = 6
    ids = []
    for i, t in enumerate(tokens):
        if i > 0 and tokens[i - 1] == t:
            ids.append(blank)
        ids += [blank] * data.draw(st.integers(0, 2))
        ids += [t] * data.draw(st.integers(1, 3))
    ids += [blank] * data.draw(st.integers(0, 2))
    assert oracle.ctc_collapse(ids, blank) == tokens


# ------------------------------------------------------------------ int8 g64

def test_int8_dequant_exact_idempotent_bounded():
    rng = np.random.default_rng(1)
    w = synth.round_to_f16(rng.normal(0, 0.02, (8, 192)))
    q, s = synth.quantize_int8_g64(w)
    assert q.dtype == np.int8 and s.dtype == np.float16 and s.shape == (8, 3)
    deq = oracle.dequantize_int8_g64(q, s)
    # every product int8 * fp16 is exact in float32
    assert np.array_equal(deq.astype(np.float32).astype(np.float64), deq)
    # per-weight error is at most half a step (plus the fp16 rounding of the scale)
    step = np.repeat(s.astype(np.float64), 64, axis=1)
    assert np.all(np.abs(deq - w) <= 0.5 * step + 1e-3 * np.abs(w) + 1e-12)
    # re-quantising the dequantised weights changes nothing
    q2, s2 = synth.quantize_int8_g64(deq)
    np.testing.assert_array_equal(oracle.dequantize_int8_g64(q2, s2), deq)
    # group layout: one scale per 64 consecutive input elements of an output row
    q3 = np.zeros((1, 128), np.int8)
    q3[0, 64] = 1
    s3 = np.array([[2.0, 3.0]], np.float16)
    assert oracle.dequantize_int8_g64(q3, s3)[0, 64] == 3.0


@pytest.mark.parametrize("bits", [6, 4])
def test_low_bit_dequant_exact_bounded_and_in_range(bits):
    """The INT6 / INT4 g64 variants: integers within +-(2^(b-1)-1), one fp16 scale per 64
    weights, products exact in fp32, error at most half a step, fixed point under
    re-quantisation, and a 2^(b-1)-1 multiple of the scale reaching the group's max."""
    qmax = (1 << (bits - 1)) - 1
    rng = np.random.default_rng(bits)
    w = synth.round_to_f16(rng.normal(0, 0.02, (8, 192)))
    q, s = synth.quantize_g64(w, bits)
    assert q.dtype == np.int8 and np.abs(q).max() == qmax and s.shape == (8, 3)
    deq = oracle.dequantize_g64(q, s)
    assert np.array_equal(deq.astype(np.float32).astype(np.float64), deq)
    step = np.repeat(s.astype(np.float64), 64, axis=1)
    assert np.all(np.abs(deq - w) <= 0.5 * step + 1e-3 * np.abs(w) + 1e-12)
    q2, s2 = synth.quantize_g64(deq, bits)
    np.testing.assert_array_equal(oracle.dequantize_g64(q2, s2), deq)
    # every group's largest |w| maps to +-qmax
    g = np.abs(w).reshape(8, 3, 64)
    qa = np.abs(q.astype(int)).reshape(8, 3, 64)
    assert np.all(qa[np.arange(8)[:, None], np.arange(3)[None, :], g.argmax(axis=2)] == qmax)
    # fewer bits never quantise more finely than more bits
    q8, s8 = synth.quantize_g64(w, 8)
    e8 = np.abs(oracle.dequantize_g64(q8, s8) - w).max()
    assert np.abs(deq - w).max() >= e8


# ------------------------------------------------------------------ whole forward

def test_tiny_workload_shapes_and_fp32_self_bound():
    cfg, pcm, lens, w = synth.workload("tiny")
    r64 = oracle.encode_clip(pcm[0, :lens[0]], w, cfg, taps=True)
    assert r64["mel"].shape == (199, 64)
    assert r64["sub"].shape == (50, 768)
    assert r64["enc_out"].shape == (50, 768) and r64["log_probs"].shape == (50, 34)
    r32 = oracle.encode_clip(pcm[0, :lens[0]], w, cfg, dtype=np.float32)
    # float32 arithmetic stays within the fp32 acceptance bound of the float64 oracle
    assert np.abs(r32["enc_out"] - r64["enc_out"]).max() < 1e-4
    np.testing.assert_array_equal(r32["ids"], r64["ids"])


def test_batch_semantics_ignore_padding():
    cfg = synth.model_config(1, 32, 2, 64, 5, 7, "f32")
    w = synth.make_weights(cfg, 3)
    rng = np.random.default_rng(4)
    a, b = synth.make_signal(rng, 4000), synth.make_signal(rng, 2500)
    pcm, lens = synth.pad_batch([a, b])
    pcm[1, 2500:] = 1e3 * rng.standard_normal(pcm.shape[1] - 2500)   # garbage in padding
    res = oracle.encode_batch(pcm, lens, w, cfg)
    alone = oracle.encode_clip(b, w, cfg)
    np.testing.assert_array_equal(res[1]["enc_out"], alone["enc_out"])
    assert res[1]["enc_out"].shape[0] == oracle.encoder_frames(2500)[2]


def test_int8_model_uses_dequantised_weights():
    cfg = synth.model_config(1, 64, 2, 128, 5, 9, "w8f16")
    w = synth.make_weights(cfg, 5)
    assert "layers.0.ff1.linear1.weight_q" in w and "layers.0.ff1.linear1.weight" not in w
    assert "pre.conv1.weight" in w and "head.weight" in w and "layers.0.conv.depthwise.weight" in w
    P = oracle.materialize(w)
    np.testing.assert_array_equal(P["layers.0.ff1.linear1.weight"],
                                  oracle.dequantize_int8_g64(w["layers.0.ff1.linear1.weight_q"],
                                                             w["layers.0.ff1.linear1.weight_scale"]))


def test_fp32_self_bound_at_the_multilingual_width():
    """The same fp32-vs-fp64 self-bound at the 1024-wide shape (2 blocks of d 1024, 16
    heads, FFN 4096, 129 classes; the 24-block model's block shape) on a 2 s clip."""
    cfg = synth.model_config(2, 1024, 16, 4096, 31, 129, "f16")
    w = synth.make_weights(cfg, 4)
    pcm = synth.make_signal(np.random.default_rng(4), 32000)
    r64 = oracle.encode_clip(pcm, w, cfg)
    r32 = oracle.encode_clip(pcm, w, cfg, dtype=np.float32)
    assert r64["enc_out"].shape == (50, 1024)
    assert np.abs(r32["enc_out"] - r64["enc_out"]).max() < 1e-4
    np.testing.assert_array_equal(r32["ids"], r64["ids"])
