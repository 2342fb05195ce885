"""Pins for the RNNT head's oracle (oracle/rnnt.py): the LSTM step against PyTorch's own
LSTM (the pages map PyTorch's weight_ih / weight_hh / two biases), and greedy decoding
on hand-built heads whose output follows from the definition alone."""
import numpy as np
import pytest

import synth
from oracle import rnnt


def _head(C=5, P=64, J=64, d=64, seed=0, dtype="f32"):
    cfg = synth.rnnt_config(d, C, dtype, pred_hidden=P, joint_hidden=J, max_symbols=3)
    w = synth.make_rnnt_weights(cfg, seed)
    return cfg, {k: np.asarray(v, np.float64) for k, v in w.items()}


def test_lstm_step_matches_torch_lstm():
    torch = pytest.importorskip("torch")
    _, P = _head(P=64, seed=1)
    H = 64
    lstm = torch.nn.LSTM(H, H, num_layers=1).double()
    with torch.no_grad():
        lstm.weight_ih_l0.copy_(torch.from_numpy(P["rnnt.lstm.weight_ih_l0"]))
        lstm.weight_hh_l0.copy_(torch.from_numpy(P["rnnt.lstm.weight_hh_l0"]))
        lstm.bias_ih_l0.copy_(torch.from_numpy(P["rnnt.lstm.bias_ih_l0"]))
        lstm.bias_hh_l0.copy_(torch.from_numpy(P["rnnt.lstm.bias_hh_l0"]))
    rng = np.random.default_rng(2)
    h, c = rng.standard_normal(H), rng.standard_normal(H)
    x = rng.standard_normal(H)
    want_out, (want_h, want_c) = lstm(torch.from_numpy(x)[None, None],
                                      (torch.from_numpy(h)[None, None], torch.from_numpy(c)[None, None]))
    got_h, got_c = rnnt.lstm_step(x, h, c, P)
    np.testing.assert_allclose(got_h, want_h[0, 0].detach().numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(got_c, want_c[0, 0].detach().numpy(), rtol=0, atol=1e-13)


def test_blank_dominant_head_emits_nothing():
    _, P = _head()
    P["rnnt.joint.out.bias"][-1] = 1e6
    enc = np.random.default_rng(3).standard_normal((17, 64))
    assert rnnt.greedy_decode(enc, P, max_symbols=3) == []


def test_symbol_dominant_head_emits_max_symbols_per_frame():
    _, P = _head()
    P["rnnt.joint.out.bias"][2] = 1e6
    enc = np.random.default_rng(4).standard_normal((11, 64))
    assert rnnt.greedy_decode(enc, P, max_symbols=3) == [2] * 33
    assert rnnt.greedy_decode(enc, P, max_symbols=1) == [2] * 11


def test_frame_driven_head_follows_the_frames():
    """Prediction network cut off (W_pred = 0, b_pred = 0), joint = identity: frame t's
    one-hot picks the symbol, so each non-blank frame emits it max_symbols times and a
    blank frame emits nothing."""
    C = 4
    P = {"rnnt.embed.weight": np.ones((C, 8)), "rnnt.lstm.weight_ih_l0": np.ones((32, 8)),
         "rnnt.lstm.weight_hh_l0": np.ones((32, 8)), "rnnt.lstm.bias_ih_l0": np.zeros(32),
         "rnnt.lstm.bias_hh_l0": np.zeros(32), "rnnt.joint.enc.weight": np.eye(C),
         "rnnt.joint.enc.bias": np.zeros(C), "rnnt.joint.pred.weight": np.zeros((C, 8)),
         "rnnt.joint.pred.bias": np.zeros(C), "rnnt.joint.out.weight": np.eye(C),
         "rnnt.joint.out.bias": np.zeros(C)}
    pattern = [3, 0, 0, 3, 2, 1, 3, 3, 1]          # 3 = blank
    enc = 5.0 * np.eye(C)[pattern]
    want = [k for k in pattern if k != 3 for _ in range(2)]
    assert rnnt.greedy_decode(enc, P, max_symbols=2) == want


def test_decoding_is_causal_prefix():
    """Greedy decoding never looks ahead: the symbols of a prefix of the frames are a
    prefix of the symbols of the whole clip."""
    _, P = _head(seed=5)
    enc = np.random.default_rng(6).standard_normal((40, 64))
    full = rnnt.greedy_decode(enc, P, max_symbols=3)
    for u in (1, 7, 23):
        part = rnnt.greedy_decode(enc[:u], P, max_symbols=3)
        assert full[: len(part)] == part


def test_rescoring_the_oracles_own_path():
    """Re-scoring the oracle's path (with the frame of every symbol, recovered from the
    decision trace) reproduces its decisions: every chosen symbol is the argmax."""
    _, P = _head(seed=7)
    enc = np.random.default_rng(8).standard_normal((30, 64))
    trace = []
    toks = rnnt.greedy_decode(enc, P, max_symbols=3, trace=trace)
    blank = P["rnnt.joint.out.bias"].shape[0] - 1
    frames = [t for t, lg in trace if rnnt.argmax32(lg) != blank]
    assert len(frames) == len(toks) and 0 < len(toks) < 90
    steps = rnnt.rescore_path(enc, toks, frames, P, max_symbols=3)
    assert len(steps) == len(trace)
    for (t, chosen, lg), (t2, lg2) in zip(steps, trace):
        assert t == t2 and chosen == rnnt.argmax32(lg)
        np.testing.assert_array_equal(lg, lg2)
    with pytest.raises(ValueError):
        rnnt.rescore_path(enc, toks + [0], frames + [-1], P, max_symbols=3)
    with pytest.raises(ValueError):
        rnnt.rescore_path(enc, [0, 0, 0, 0], [5, 5, 5, 5], P, max_symbols=3)
