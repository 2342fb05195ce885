"""GPU stage taps on the 16-bit paths (the pipelined direct-to-LDS GEMMs every fp16 / bf16
config runs): subsampling output, the residual stream after each module of block 0, and
the outputs of blocks 0 and 7, for the shortest and the longest clip of the 32-clip batch,
each against the oracle recomputed from its own previous stage. Layer-by-layer comparison is
how the pages' port found its bug ("GigaAM on MLX: the transcripts matched, but the model was
broken", Trap 1).

Bar: max|d| <= 5e-2 * max(1, rms of the oracle tensor) (the encoder-output bar, scaled to
the tensor: the residual stream inside a block is not normalised)."""
import numpy as np
import pytest

from gpu_common import TOL_LOW, device_pcm, model, oracle_clip, say, workload

import oracle

pytestmark = pytest.mark.gpu

_taps = {}


def _clips(name):
    lens = workload(name)[2]
    return [int(np.argmin(lens)), int(np.argmax(lens))]


def _rows(name, b):
    lens = workload(name)[2]
    U = [oracle.encoder_frames(int(n))[2] for n in lens]
    s = int(sum(U[:b]))
    return s, s + U[b]


def _tap(name, stage):
    key = (name, stage)
    if key not in _taps:
        pcm, lens = device_pcm(name)
        _taps[key] = model(name).encode_stage(pcm, lens, stage).cpu().numpy()
    return _taps[key]


def _check(name, tag, got, ref):
    err = float(np.abs(got - ref).max())
    rms = float(np.sqrt(np.mean(ref ** 2)))
    bar = TOL_LOW * max(1.0, rms)
    say(f"[taps16] {name} {tag}: max|d| {err:.3e} (rms {rms:.3f}, bar {bar:.3e})")
    assert err <= bar


@pytest.mark.parametrize("name", ["batch32", "batch32_bf16"])
def test_subsampling_and_layer_taps(name):
    import conformer_speech_recognition_amd as gg
    for b in _clips(name):
        lo, hi = _rows(name, b)
        ref = oracle_clip(name, b, True)
        _check(name, f"clip {b} sub", _tap(name, gg.STAGE_SUB)[lo:hi], ref["sub"])
        for layer in (0, 7):
            _check(name, f"clip {b} layer {layer}", _tap(name, gg.STAGE_LAYER + layer)[lo:hi],
                   ref["layers"][layer])


@pytest.mark.parametrize("name", ["batch32", "batch32_bf16"])
@pytest.mark.parametrize("part", [0, 1, 2, 3])
def test_block0_module_taps(name, part):
    """After FFN1, attention, conv module and FFN2 of block 0, the oracle continuing from its
    own subsampling output with its module functions."""
    import conformer_speech_recognition_amd as gg
    cfg, _, _, w = workload(name)
    P = oracle.materialize(w)
    p, eps = "layers.0.", cfg["ln_eps"]
    for b in _clips(name):
        lo, hi = _rows(name, b)
        x = oracle_clip(name, b, True)["sub"]
        x = x + 0.5 * oracle.feed_forward(x, P, p + "ff1.", eps)
        if part >= 1:
            y = oracle.layer_norm(x, P[p + "att.norm.weight"], P[p + "att.norm.bias"], eps)
            x = x + oracle.mhsa_rope(y, P, p + "att.", cfg["n_heads"], cfg["rope_base"])
        if part >= 2:
            x = x + oracle.conv_module(x, P, p + "conv.", eps, cfg["bn_eps"])
        if part >= 3:
            x = x + 0.5 * oracle.feed_forward(x, P, p + "ff2.", eps)
        got = _tap(name, gg.stage_sublayer(0, part))[lo:hi]
        _check(name, f"clip {b} block0 part {part}", got, x)
