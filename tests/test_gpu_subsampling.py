"""GPU: the subsampling stage (two Conv1d, kernel 5, stride 2, padding 2, ReLU after each;
"GigaAM on MLX" blog, "What we're porting") of the 16-bit encoders against the oracle's
subsample() on packed batches whose clips stress the implicit conv: encoder lengths 1, 2
and 3 (taps outside the clip at both ends of one short window), lengths one sample past
a frame boundary, a total row count with a ragged last tile, and a one-clip batch small
enough that the K sum is split into slices that start inside a tap.

Bar: max|d| <= c * max(1, rms of the oracle rows), c = 1e-2 (fp16) and 5e-2 (bf16): the
two 16-bit roundings of the operands (mel and h1 into the stored type, weights stored in
it) over 320- and 3840-term sums measure ~1e-3 (fp16) and ~8e-3 (bf16) at rms 0.5, while
a tap read from the wrong row or left unzeroed moves outputs by O(rms)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import model, say, workload

pytestmark = pytest.mark.gpu

BAR = {"f16": 1e-2, "bf16": 5e-2}
# encoder frames 1, 1, 2, 3, 5, 63, 64, 65, 128, 129, 250
EDGE = [320, 479, 960, 1600, 2880, 40000, 40640, 41280, 81600, 82240, 159680]


def _sub(name, lengths, seed):
    import torch
    import conformer_speech_recognition_amd as gg
    cfg, _, _, w = workload(name)
    rng = np.random.default_rng(seed)
    pcm, lens = synth.pad_batch([synth.make_signal(rng, int(n)) for n in lengths])
    U = [oracle.encoder_frames(int(n))[2] for n in lens]
    say(f"[sub] {name}: {len(lens)} clips, encoder frames {U} ({sum(U)} rows)")
    got = model(name).encode_stage(torch.from_numpy(pcm).cuda(), lens, gg.STAGE_SUB).cpu().numpy()
    assert got.shape == (sum(U), cfg["d_model"])
    P = oracle.materialize(w)
    bar = BAR[cfg["dtype"]]
    r = 0
    for b, L in enumerate(lens):
        ref = oracle.subsample(oracle.log_mel(pcm[b, :L]), P)
        assert ref.shape[0] == U[b]
        err = float(np.abs(got[r:r + U[b]] - ref).max())
        rms = float(np.sqrt(np.mean(ref ** 2)))
        say(f"[sub] {name} clip {b} U={U[b]}: max|d| {err:.3e} (rms {rms:.3f})")
        assert err <= bar * max(1.0, rms), (b, U[b], err)
        r += U[b]


@pytest.mark.parametrize("name", ["batch32", "batch32_bf16"])
@pytest.mark.parametrize("n20", [13, 8])
def test_subsampling_edges(name, n20):
    # the 11 edge clips (711 rows) + n20 clips of 20 s (500 rows each): 7211 rows, 29 tiles
    # of 256 rows, the last one ragged (the 256 x 128 tiles of the 32-clip batch, K unsplit),
    # or 4711 rows, 19 tiles (the same tiles, K split in 2 slices, the second starting
    # inside the third tap)
    _sub(name, EDGE + [320000] * n20, 81 + n20)


@pytest.mark.parametrize("name", ["batch32", "batch32_bf16"])
def test_subsampling_one_short_clip(name):
    # 50 encoder frames: six 128 x 128 tiles, the 3840-term sum split in 4 slices of 960
    _sub(name, [32000], 82)
