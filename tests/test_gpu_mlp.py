"""GPU: the fused few-row FFN (hidden activations kept on chip) through gigaam_debug_mlp,
against a float64 evaluation of x + alpha (W2 h + b2), h = T(SiLU(W1 y + b1)), on ragged row
counts up to the kernel's limit, both 16-bit types and both model widths."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

CASES = [(1, 768, 3072), (63, 768, 3072), (65, 768, 3072), (500, 768, 3072), (896, 768, 3072),
         (130, 1024, 4096), (7, 768, 512)]


def _round(a, dtype):
    return synth.round_to_f16(a) if dtype == "f16" else synth.round_to_bf16(a)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,d,f", CASES)
def test_fused_mlp_matches_float64(dtype, M, d, f):
    import torch
    import conformer_speech_recognition_amd as gg
    print(f"[mlp] {dtype} M={M} d={d} f={f}", flush=True)
    rng = np.random.default_rng(M * 11 + d + f)
    y = _round(rng.standard_normal((M, d)).astype(np.float32), dtype)
    w1 = _round((0.05 * rng.standard_normal((f, d))).astype(np.float32), dtype)
    w2 = _round((0.05 * rng.standard_normal((d, f))).astype(np.float32), dtype)
    b1 = rng.standard_normal(f).astype(np.float32)
    b2 = rng.standard_normal(d).astype(np.float32)
    x = rng.standard_normal((M, d)).astype(np.float32)
    tt = torch.float16 if dtype == "f16" else torch.bfloat16
    dev = "cuda:0"
    X = torch.from_numpy(x).to(dev)
    gg.debug_mlp(dtype, torch.from_numpy(y).to(tt).to(dev), torch.from_numpy(w1).to(tt).to(dev),
                 torch.from_numpy(b1).to(dev), torch.from_numpy(w2).to(tt).to(dev),
                 torch.from_numpy(b2).to(dev), X, alpha=0.5)
    torch.cuda.synchronize()
    got = X.cpu().numpy().astype(np.float64)
    pre = y.astype(np.float64) @ w1.astype(np.float64).T + b1
    hid = pre / (1.0 + np.exp(-pre))
    h = _round(hid.astype(np.float32), dtype).astype(np.float64)
    ref = x + 0.5 * (h @ w2.astype(np.float64).T + b2)
    # fp32 sums of exact products (K * 2^-24 relative, loose) plus one rounding step of T in
    # h where the GPU's and float64's pre-activations straddle a rounding boundary
    ulp = 2.0 ** -11 if dtype == "f16" else 2.0 ** -8
    bound = (1e-6 * (d + f) * np.abs(hid).max() * 0.05 * 4
             + 0.5 * f * 0.05 * ulp * np.abs(hid).max() * 0.05 + 1e-4)
    err = np.abs(got - ref).max()
    print(f"[mlp] {dtype} {M}x{d}x{f}: max|d| = {err:.3e} (bound {bound:.2e})", flush=True)
    assert err <= bound
