"""Seeded synthetic inputs for the Conformer CTC encoder: PCM, clip lengths, weights.

This module is DATA ONLY. It draws random numbers and rounds them to the storage
types of a checkpoint; it computes none of the encoder's arithmetic (no framing,
spectra, filterbanks, convolutions, norms, attention, soft-max or decoding).
Both the CPU oracle and the HIP path consume what it returns; neither is imported here.

Pages this follows (titles as printed on each page):
  * "GigaAM on MLX: the transcripts matched, but the model was broken", section
    "What we're porting": 16 kHz mono input, fp16 checkpoints ("Trap 4").
  * "GigaAM MLX port for Mac", section "How precision affects size and speed": weight
    variants with one shared scale per group of 64 weights (INT8 g64).

The pages measure on recorded speech datasets that are not available here; the
signal generator below is a stand-in with the same sample rate and clip durations.
"""
from __future__ import annotations

import numpy as np

SAMPLE_RATE = 16000

# ----------------------------------------------------------------------------------
# storage-type rounding (checkpoint dtypes). Pure bit-level casts, no model maths.
# ----------------------------------------------------------------------------------

def round_to_f16(a: np.ndarray) -> np.ndarray:
    """fp32/fp64 -> fp16 (round-to-nearest-even) -> back to float32 values."""
    return np.asarray(a, dtype=np.float32).astype(np.float16).astype(np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 with round-to-nearest-even on the bit pattern -> float32 values."""
    x = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def round_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    if dtype in ("f16",) + tuple(QUANT_BITS):
        return round_to_f16(a)
    if dtype == "bf16":
        return round_to_bf16(a)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------------
# signals
# ----------------------------------------------------------------------------------

def make_signal(rng: np.random.Generator, n_samples: int) -> np.ndarray:
    """Sum of three random sines in 100..3000 Hz (amplitude 1/3, random phase) plus
    Gaussian noise of std 0.05, clipped to [-1, 1], as float32 at 16 kHz.

    Draw order from ``rng``: 3 frequencies, 3 phases, then n_samples noise values.
    """
    f = rng.uniform(100.0, 3000.0, 3)
    phi = rng.uniform(0.0, 2.0 * np.pi, 3)
    noise = rng.normal(0.0, 0.05, n_samples)
    i = np.arange(n_samples, dtype=np.float64)
    x = noise.copy()
    for j in range(3):
        x += (1.0 / 3.0) * np.sin(2.0 * np.pi * f[j] * i / SAMPLE_RATE + phi[j])
    return np.clip(x, -1.0, 1.0).astype(np.float32)


def pad_batch(signals: list[np.ndarray]) -> tuple[np.ndarray, np.ndarray]:
    """Zero-pad a list of 1-D float32 signals to [B, max_len]; return (pcm, lengths)."""
    lengths = np.array([len(s) for s in signals], dtype=np.int32)
    pcm = np.zeros((len(signals), int(lengths.max())), dtype=np.float32)
    for b, s in enumerate(signals):
        pcm[b, : len(s)] = s
    return pcm, lengths


# ----------------------------------------------------------------------------------
# model configurations and canonical parameter names
# ----------------------------------------------------------------------------------

def model_config(n_layers: int, d_model: int, n_heads: int, d_ff: int, conv_kernel: int,
                 n_classes: int, dtype: str) -> dict:
    """Plain-dict model configuration. Frontend constants are those printed in the
    frontend table of the "GigaAM v3 MLX" model card (section "Frontend configuration")."""
    return dict(n_layers=n_layers, d_model=d_model, n_heads=n_heads, d_ff=d_ff,
                conv_kernel=conv_kernel, n_classes=n_classes, dtype=dtype,
                n_mels=64, n_fft=320, win_length=320, hop_length=160,
                sub_kernel=5, sub_stride=2, rope_base=5000.0, ln_eps=1e-5, bn_eps=1e-5)


# weight-only quantised checkpoints: bits per linear weight of each dtype
QUANT_BITS = {"w8f16": 8, "w6f16": 6, "w4f16": 4}

QUANTIZED_SUFFIXES = ("ff1.linear1", "ff1.linear2", "att.linear_q", "att.linear_k",
                      "att.linear_v", "att.linear_out", "conv.pointwise1",
                      "conv.pointwise2", "ff2.linear1", "ff2.linear2")


def canonical_entries(cfg: dict) -> list[tuple[str, tuple[int, ...], str]]:
    """(name, shape, init-kind) for every parameter, in draw order.

    Layouts follow PyTorch conventions: Linear [out, in]; Conv1d [out, in, K]
    (pointwise convs squeezed to [out, in]; depthwise to [channels, K]).
    """
    d, f, k, C, m = (cfg["d_model"], cfg["d_ff"], cfg["conv_kernel"], cfg["n_classes"],
                     cfg["n_mels"])
    ks = cfg["sub_kernel"]
    e: list[tuple[str, tuple[int, ...], str]] = [
        ("pre.conv1.weight", (d, m, ks), "w"), ("pre.conv1.bias", (d,), "b"),
        ("pre.conv2.weight", (d, d, ks), "w"), ("pre.conv2.bias", (d,), "b"),
    ]
    for i in range(cfg["n_layers"]):
        p = f"layers.{i}."
        for ff in ("ff1",):
            e += [(p + ff + ".norm.weight", (d,), "g"), (p + ff + ".norm.bias", (d,), "b"),
                  (p + ff + ".linear1.weight", (f, d), "w"), (p + ff + ".linear1.bias", (f,), "b"),
                  (p + ff + ".linear2.weight", (d, f), "w"), (p + ff + ".linear2.bias", (d,), "b")]
        e += [(p + "att.norm.weight", (d,), "g"), (p + "att.norm.bias", (d,), "b")]
        for lin in ("linear_q", "linear_k", "linear_v", "linear_out"):
            e += [(p + "att." + lin + ".weight", (d, d), "w"), (p + "att." + lin + ".bias", (d,), "b")]
        e += [(p + "conv.norm.weight", (d,), "g"), (p + "conv.norm.bias", (d,), "b"),
              (p + "conv.pointwise1.weight", (2 * d, d), "w"), (p + "conv.pointwise1.bias", (2 * d,), "b"),
              (p + "conv.depthwise.weight", (d, k), "w"), (p + "conv.depthwise.bias", (d,), "b"),
              (p + "conv.bn.weight", (d,), "g"), (p + "conv.bn.bias", (d,), "b"),
              (p + "conv.bn.running_mean", (d,), "b"), (p + "conv.bn.running_var", (d,), "v"),
              (p + "conv.pointwise2.weight", (d, d), "w"), (p + "conv.pointwise2.bias", (d,), "b")]
        e += [(p + "ff2.norm.weight", (d,), "g"), (p + "ff2.norm.bias", (d,), "b"),
              (p + "ff2.linear1.weight", (f, d), "w"), (p + "ff2.linear1.bias", (f,), "b"),
              (p + "ff2.linear2.weight", (d, f), "w"), (p + "ff2.linear2.bias", (d,), "b")]
        e += [(p + "norm_out.weight", (d,), "g"), (p + "norm_out.bias", (d,), "b")]
    e += [("head.weight", (C, d), "w"), ("head.bias", (C,), "b")]
    return e


def _draw(rng: np.random.Generator, shape, kind: str) -> np.ndarray:
    if kind in ("w", "b"):
        return rng.normal(0.0, 0.02, shape)
    if kind == "g":
        return 1.0 + rng.normal(0.0, 0.02, shape)
    if kind == "v":
        return rng.uniform(0.5, 1.5, shape)
    raise ValueError(kind)


def make_weights(cfg: dict, seed: int, head_seed: int | None = None) -> dict[str, np.ndarray]:
    """Random-init weights N(0, 0.02^2) (norm gains 1 + N(0, 0.02^2), BN running
    variance U(0.5, 1.5)), rounded to the checkpoint storage type of ``cfg['dtype']``.

    All arrays are returned as float32 holding the rounded values. With
    ``head_seed`` the CTC head is redrawn from its own stream (same draw rule).
    For the quantised dtypes (QUANT_BITS) the linears in QUANTIZED_SUFFIXES are replaced
    by a b-bit checkpoint: ``<name>.weight_q`` (int8 [N, K] holding b-bit integers) and
    ``<name>.weight_scale`` (float16 [N, K/64]); see ``quantize_g64``.
    """
    rng = np.random.default_rng(seed)
    out: dict[str, np.ndarray] = {}
    for name, shape, kind in canonical_entries(cfg):
        out[name] = round_storage(_draw(rng, shape, kind), cfg["dtype"])
    if head_seed is not None:
        hr = np.random.default_rng(head_seed)
        C, d = cfg["n_classes"], cfg["d_model"]
        out["head.weight"] = round_storage(_draw(hr, (C, d), "w"), cfg["dtype"])
        out["head.bias"] = round_storage(_draw(hr, (C,), "b"), cfg["dtype"])
    if cfg["dtype"] in QUANT_BITS:
        bits = QUANT_BITS[cfg["dtype"]]
        for name in list(out):
            if name.endswith(".weight") and name[: -len(".weight")].endswith(QUANTIZED_SUFFIXES):
                q, s = quantize_g64(out.pop(name), bits)
                base = name[: -len(".weight")]
                out[base + ".weight_q"] = q
                out[base + ".weight_scale"] = s
    return out


def quantize_g64(w: np.ndarray, bits: int = 8, group: int = 64) -> tuple[np.ndarray, np.ndarray]:
    """Checkpoint conversion to weight-only b-bit integers with one fp16 scale per group
    of 64 consecutive input-dim weights of one output row (symmetric, qmax = 2^(b-1) - 1):
        s = fp16(max|w_group| / qmax),  q = clamp(rint(w / s), -qmax, qmax).
    This is how the quantised checkpoints are produced (a one-off conversion, like the
    fp16 rounding above); the encoder itself only ever reads q and s.
    """
    qmax = (1 << (bits - 1)) - 1
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    assert K % group == 0
    g = w.reshape(N, K // group, group)
    s = (np.abs(g).max(axis=2) / qmax).astype(np.float16)
    s64 = s.astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s64 > 0, np.rint(g / np.where(s64 > 0, s64, 1.0)), 0.0)
    q = np.clip(q, -qmax, qmax).astype(np.int8).reshape(N, K)
    return q, s


def quantize_int8_g64(w: np.ndarray, group: int = 64) -> tuple[np.ndarray, np.ndarray]:
    """quantize_g64 with 8 bits."""
    return quantize_g64(w, 8, group)


def rnnt_config(d_model: int, n_classes: int, dtype: str, pred_hidden: int = 320,
                joint_hidden: int = 320, max_symbols: int = 10) -> dict:
    """RNNT head shape: a 320-wide single-layer LSTM and joint ("GigaAM on MLX ...",
    section "What we're porting"); the symbol cap per frame is a decoding setting."""
    return dict(d_model=d_model, n_classes=n_classes, pred_hidden=pred_hidden,
                joint_hidden=joint_hidden, max_symbols=max_symbols, dtype=dtype)


def rnnt_entries(cfg: dict) -> list[tuple[str, tuple[int, ...]]]:
    P, J, C, d = cfg["pred_hidden"], cfg["joint_hidden"], cfg["n_classes"], cfg["d_model"]
    return [("rnnt.embed.weight", (C, P)), ("rnnt.lstm.weight_ih_l0", (4 * P, P)),
            ("rnnt.lstm.weight_hh_l0", (4 * P, P)), ("rnnt.lstm.bias_ih_l0", (4 * P,)),
            ("rnnt.lstm.bias_hh_l0", (4 * P,)), ("rnnt.joint.enc.weight", (J, d)),
            ("rnnt.joint.enc.bias", (J,)), ("rnnt.joint.pred.weight", (J, P)),
            ("rnnt.joint.pred.bias", (J,)), ("rnnt.joint.out.weight", (C, J)),
            ("rnnt.joint.out.bias", (C,))]


def make_rnnt_weights(cfg: dict, seed: int, blank_bias: float = 2.0) -> dict[str, np.ndarray]:
    """Random-init RNNT head: matrices N(0, 1/fan_in) (unit-scale activations, so the
    decisions depend on both the frame and the predictor state), embedding N(0, 1),
    biases N(0, 0.1^2), plus ``blank_bias`` on the blank output so that a fair share of
    the decisions are blanks, as in speech. Rounded to the storage type of the dtype."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape in rnnt_entries(cfg):
        if name.endswith("embed.weight"):
            a = rng.standard_normal(shape)
        elif len(shape) == 2:
            a = rng.standard_normal(shape) / np.sqrt(shape[1])
        else:
            a = 0.1 * rng.standard_normal(shape)
        out[name] = a
    out["rnnt.joint.out.bias"][-1] += blank_bias
    return {k: round_storage(v, cfg["dtype"]) for k, v in out.items()}


def make_encoder_like(rng: np.random.Generator, frames: list[int], d: int) -> np.ndarray:
    """Stand-in encoder output for the head alone: per clip, rows of N(0, 1) (the scale
    of a LayerNorm output), zero-padded to the longest clip: float32 [B, U_max, d]."""
    U = max(frames)
    e = np.zeros((len(frames), U, d), dtype=np.float32)
    for b, u in enumerate(frames):
        e[b, :u] = rng.standard_normal((u, d)).astype(np.float32)
    return e


from .workloads import (WORKLOADS, workload, workload_config,  # noqa: E402,F401
                        workload_signals, workload_weights)
