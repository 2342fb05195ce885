"""Helpers shared by the GPU parity tests: model/oracle caches and comparisons.

The HIP path is reached only through the C ABI (conformer_speech_recognition_amd);
expected values come only from the CPU oracle on the same seeded inputs.
"""
from __future__ import annotations

import functools
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

# fp32 path: encoder output within 1e-4 and token ids bit-exact; fp16/bf16/int8 paths:
# encoder output within 5e-2 and >= 99.5% per-frame argmax agreement.
TOL_F32 = 1e-4
TOL_LOW = 5e-2
ARGMAX_AGREE = 0.995


def say(msg: str):
    print(msg, flush=True)


@functools.lru_cache(maxsize=None)
def workload(name: str):
    return synth.workload(name)


@functools.lru_cache(maxsize=2)
def model(name: str):
    import conformer_speech_recognition_amd as gg
    cfg, pcm, lens, w = workload(name)
    return gg.Model(cfg, w)


@functools.lru_cache(maxsize=None)
def oracle_clip(name: str, b: int, taps: bool = False):
    cfg, pcm, lens, w = workload(name)
    say(f"[oracle] {name} clip {b} ({lens[b]} samples)")
    return oracle.encode_clip(pcm[b, : int(lens[b])], w, cfg, taps=taps)


def device_pcm(name: str):
    import torch
    cfg, pcm, lens, w = workload(name)
    return torch.from_numpy(pcm).cuda(), lens


def clip_rows(lens, b, which=2):
    """Packed row range of clip b in the mel (which=0) or encoder (which=2) space."""
    fr = [oracle.encoder_frames(int(n)) for n in lens]
    start = sum(f[which] for f in fr[:b])
    return start, start + fr[b][which]


def argmax_agreement(gpu_ids: np.ndarray, ref_logp: np.ndarray):
    ref = oracle.greedy_ids(ref_logp)
    agree = float(np.mean(gpu_ids == ref))
    srt = np.sort(np.asarray(ref_logp, dtype=np.float64), axis=1)
    margin = srt[:, -1] - srt[:, -2]
    flips = np.nonzero(gpu_ids != ref)[0]
    return agree, margin, flips
