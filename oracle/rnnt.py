"""CPU ORACLE for the RNNT head: prediction network, joint network, greedy decoding.

TEST INFRASTRUCTURE ONLY (same rules as the package: only the tests, the smoke check
and the benchmark's CPU-baseline leg may use it; the HIP path shares nothing with it).

What the pages fix:
  - the head is a single-layer LSTM of size 320 plus a joint network ([MLX-blog],
    "What we're porting");
  - the LSTM follows PyTorch, with its two bias vectors summed into one ([MLX-blog],
    "Trap 4: weight layout and precision"; [RNNT-card], "Notes for other runtimes");
  - blank = len(vocabulary), i.e. the last of the n_classes outputs ([RNNT-card],
    "Notes for other runtimes");
  - decoding is greedy and sequential, one step at a time ([RNNT-card], the model
    description; [v3-card], "Architecture details" and "Long-form stage breakdown").

Readings adopted where the pages are silent (also listed in the design notes):
  - prediction network = embedding of the previous emitted symbol (an [n_classes, P]
    table, blank included) -> LSTM; decoding starts from zero state with blank as the
    previous symbol;
  - PyTorch LSTM gate order i, f, g, o: c' = s(f) c + s(i) tanh(g), h' = s(o) tanh(c');
  - joint = W_out relu(W_enc e_t + b_enc + W_pred h + b_pred) + b_out (the usual
    additive RNN-T joint with ReLU);
  - greedy RNN-T: at frame t take the argmax of the joint; blank moves to frame t+1,
    any other symbol is emitted, advances the prediction network and stays on frame t,
    at most ``max_symbols`` emissions per frame (then frame t+1); argmax takes the
    lowest index on ties, on float32 logits like the CTC head.
"""
from __future__ import annotations

import numpy as np


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def lstm_step(x: np.ndarray, h: np.ndarray, c: np.ndarray, P: dict):
    """One step of a single-layer PyTorch LSTM:
    gates = W_ih x + b_ih + W_hh h + b_hh, split as (i, f, g, o)."""
    gates = (P["rnnt.lstm.weight_ih_l0"] @ x + P["rnnt.lstm.bias_ih_l0"]
             + P["rnnt.lstm.weight_hh_l0"] @ h + P["rnnt.lstm.bias_hh_l0"])
    H = h.shape[0]
    i, f, g, o = gates[:H], gates[H:2 * H], gates[2 * H:3 * H], gates[3 * H:]
    c2 = sigmoid(f) * c + sigmoid(i) * np.tanh(g)
    h2 = sigmoid(o) * np.tanh(c2)
    return h2, c2


def predictor_step(token: int, h: np.ndarray, c: np.ndarray, P: dict):
    """Prediction network: embedding row of the previous symbol through the LSTM."""
    return lstm_step(P["rnnt.embed.weight"][token], h, c, P)


def joint(enc_t: np.ndarray, h: np.ndarray, P: dict) -> np.ndarray:
    """Logits over the n_classes outputs (blank last) for one encoder frame and one
    prediction-network output."""
    z = (P["rnnt.joint.enc.weight"] @ enc_t + P["rnnt.joint.enc.bias"]
         + P["rnnt.joint.pred.weight"] @ h + P["rnnt.joint.pred.bias"])
    return P["rnnt.joint.out.weight"] @ np.maximum(z, 0.0) + P["rnnt.joint.out.bias"]


def argmax32(logits: np.ndarray) -> int:
    """Lowest index of the largest float32-rounded logit."""
    return int(np.argmax(np.asarray(logits, dtype=np.float32)))


def greedy_decode(enc: np.ndarray, P: dict, max_symbols: int = 10,
                  trace: list | None = None) -> list[int]:
    """Greedy RNN-T decoding of one clip's encoder output enc [U, d].

    With ``trace`` a list, every decision is appended as (t, logits) in order, so a
    caller can re-score another decoder's path."""
    n_classes = P["rnnt.joint.out.bias"].shape[0]
    blank = n_classes - 1
    H = P["rnnt.lstm.weight_hh_l0"].shape[1]
    h, c = predictor_step(blank, np.zeros(H), np.zeros(H), P)
    out: list[int] = []
    for t in range(enc.shape[0]):
        for _ in range(max_symbols):
            logits = joint(enc[t], h, P)
            if trace is not None:
                trace.append((t, logits))
            k = argmax32(logits)
            if k == blank:
                break
            out.append(k)
            h, c = predictor_step(k, h, c, P)
    return out


def rescore_path(enc: np.ndarray, tokens, frames, P: dict, max_symbols: int = 10):
    """Follow another decoder's path (symbols with the frame each was emitted on) through
    the oracle's prediction and joint networks (teacher forcing). Returns every decision
    the path implies as (t, chosen, logits), chosen being the emitted symbol or blank:
    on frame t the path's symbols of that frame in order, then blank unless max_symbols
    were emitted. Raises ValueError for a path greedy decoding cannot produce."""
    tokens, frames = list(tokens), list(frames)
    if len(tokens) != len(frames) or any(b < a for a, b in zip(frames, frames[1:])):
        raise ValueError("frames must be non-decreasing, one per symbol")
    if frames and (frames[0] < 0 or frames[-1] >= enc.shape[0]):
        raise ValueError("frame out of range")
    n_classes = P["rnnt.joint.out.bias"].shape[0]
    blank = n_classes - 1
    H = P["rnnt.lstm.weight_hh_l0"].shape[1]
    h, c = predictor_step(blank, np.zeros(H), np.zeros(H), P)
    steps = []
    pos = 0
    for t in range(enc.shape[0]):
        emitted = 0
        while pos < len(tokens) and frames[pos] == t:
            if emitted == max_symbols or tokens[pos] == blank:
                raise ValueError("more than max_symbols symbols on a frame, or blank emitted")
            steps.append((t, tokens[pos], joint(enc[t], h, P)))
            h, c = predictor_step(tokens[pos], h, c, P)
            pos += 1
            emitted += 1
        if emitted < max_symbols:
            steps.append((t, blank, joint(enc[t], h, P)))
    return steps
