"""The five synthetic workloads (model shape + seeded inputs + seeded weights).

Shapes and precisions:
  tiny     2 s clip, 2 blocks d768, 34 classes, fp32                   (seed 0 / weights 0)
  v3_20s   one 20 s clip, 16 blocks d768, 34 classes, fp16 weights   (seed 0 / weights 1)
  batch32  32 clips of 1..20 s (lengths seed 2), 16 blocks d768, 257 classes, fp16 or bf16
  ml_long  300 s signal cut into ten 30 s chunks, 24 blocks d1024, 129 classes, fp16 (seed 4)
  int8_b64 64 clips of 10 s, 16 blocks d768, 34 classes, int8 g64 linears (signals seed 5)
  int6_b64, int4_b64  the same with 6-bit / 4-bit g64 linears (the pages' INT6 / INT4)

The pages measure real speech (200 short clips with a 3.9 s median, 20 s segments,
a 5-minute recording, 30 s chunks for long audio; see "GigaAM on MLX ...", section
"Speed", and "GigaAM MLX port for Mac", section "Where the time goes"). Those datasets
are not available; these generated signals stand in for them with the same durations.
"""
from __future__ import annotations

import numpy as np

from . import make_signal, make_weights, model_config, pad_batch

WORKLOADS = ("tiny", "v3_20s", "batch32", "batch32_bf16", "ml_long", "int8_b64", "int6_b64",
             "int4_b64")
_QUANT = {"int8_b64": "w8f16", "int6_b64": "w6f16", "int4_b64": "w4f16"}


def _v3(n_classes: int, dtype: str, n_layers: int = 16) -> dict:
    return model_config(n_layers, 768, 16, 3072, 31, n_classes, dtype)


def workload_config(name: str) -> dict:
    if name == "tiny":
        return _v3(34, "f32", n_layers=2)
    if name == "v3_20s":
        return _v3(34, "f16")
    if name == "batch32":
        return _v3(257, "f16")
    if name == "batch32_bf16":
        return _v3(257, "bf16")
    if name == "ml_long":
        return model_config(24, 1024, 16, 4096, 31, 129, "f16")
    if name in _QUANT:
        return _v3(34, _QUANT[name])
    raise KeyError(name)


def workload_signals(name: str) -> list[np.ndarray]:
    if name == "tiny":
        return [make_signal(np.random.default_rng(0), 32000)]
    if name == "v3_20s":
        return [make_signal(np.random.default_rng(0), 320000)]
    if name in ("batch32", "batch32_bf16"):
        rng = np.random.default_rng(2)
        lens = rng.integers(16000, 320000, 32, endpoint=True)
        return [make_signal(rng, int(n)) for n in lens]
    if name == "ml_long":
        x = make_signal(np.random.default_rng(4), 4_800_000)
        return [x[i * 480_000:(i + 1) * 480_000].copy() for i in range(10)]
    if name in _QUANT:
        rng = np.random.default_rng(5)
        return [make_signal(rng, 160_000) for _ in range(64)]
    raise KeyError(name)


def workload_weights(name: str, cfg: dict | None = None) -> dict[str, np.ndarray]:
    cfg = cfg or workload_config(name)
    if name == "tiny":
        return make_weights(cfg, 0)
    if name == "v3_20s" or name in _QUANT:
        return make_weights(cfg, 1)
    if name in ("batch32", "batch32_bf16"):
        return make_weights(cfg, 1, head_seed=2)
    if name == "ml_long":
        return make_weights(cfg, 4)
    raise KeyError(name)


def workload(name: str, with_weights: bool = True):
    """Return (cfg, pcm [B, Lmax] float32, lengths int32 [B], weights-dict or None)."""
    cfg = workload_config(name)
    pcm, lengths = pad_batch(workload_signals(name))
    w = workload_weights(name, cfg) if with_weights else None
    return cfg, pcm, lengths, w
