"""GPU: the attention kernel alone (gigaam_debug_attention) against a float64
softmax(q k^T / sqrt(d_k)) v per clip and head, over ragged clip lengths that cover
partial 64-frame tiles, single-frame clips, the longest workload clip, and batches at and
over the few-items limit of the 16-bit kernel."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

# The 16-bit kernel splits the keys of 64-query tiles between two wave pairs while the batch
# has at most 256 (64-frame tile x head) items, 16 tiles at 16 heads; the last three cases sit
# at that limit, just over it and far over it (the 128-query kernel).
FRAMES = [[1], [17], [64], [65], [500], [750], [51, 497, 3, 128, 129, 250],
          [500, 436, 1], [500, 500, 1],
          [250] * 8 + [129] * 4 + [1, 64, 700, 333]]


def _ref(q, k, v, frames, H):
    out = np.zeros_like(q)
    s0 = 0
    for U in frames:
        for h in range(H):
            dk = q.shape[1] // H
            sl = slice(h * dk, (h + 1) * dk)
            qq, kk, vv = q[s0:s0 + U, sl], k[s0:s0 + U, sl], v[s0:s0 + U, sl]
            sc = qq @ kk.T / np.sqrt(dk)
            sc -= sc.max(1, keepdims=True)
            p = np.exp(sc)
            out[s0:s0 + U, sl] = (p / p.sum(1, keepdims=True)) @ vv
        s0 += U
    return out


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [768, 1024])
@pytest.mark.parametrize("frames", FRAMES, ids=lambda f: "-".join(map(str, f)) if len(f) < 8 else f"{len(f)}clips-{sum(f)}")
def test_attention_matches_float64(dtype, d, frames):
    import torch
    import conformer_speech_recognition_amd as gg
    print(f"[attn] {dtype} d={d} frames={frames}", flush=True)
    rng = np.random.default_rng(sum(frames) + d)
    n = sum(frames)
    x = rng.standard_normal((n, 3 * d)).astype(np.float32)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    qkv = torch.from_numpy(x).to(tdt)
    xs = qkv.float().numpy().astype(np.float64)           # the stored operand values
    ref = _ref(xs[:, :d], xs[:, d:2 * d], xs[:, 2 * d:], frames, 16)
    got = gg.debug_attention(dtype, qkv.cuda(), frames).float().cpu().numpy()
    # fp32: accumulation rounding; fp16/bf16: probabilities rounded to the operand type
    tol = {"f32": 2e-5, "f16": 4e-3, "bf16": 3e-2}[dtype]
    err = np.abs(got - ref).max()
    print(f"[attn] max|d| = {err:.3e}", flush=True)
    assert err <= tol
