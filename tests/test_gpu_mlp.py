"""GPU: the fused few-row FFN (hidden activations kept on chip; gigaam_debug_mlp) against the
oracle's feed-forward body (oracle.ffn_body: linear2(SiLU(linear1(y))), the module after its
LayerNorm) on the same 16-bit normed input y, on ragged row counts up to the kernel's limit,
both 16-bit types and both model widths: x + alpha * ffn_body(y) with the kernel's x.

Bound: the fp32 sums of exact products (K * 2^-24 relative, loose) plus the kernel's one
rounding of the hidden activations to the 16-bit type (the unfused path stores them in that
type too): |d out| <= sum_j |W2[n, j]| * u * |h[j]|, with u the type's unit roundoff and h the
oracle's hidden activations."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

CASES = [(1, 768, 3072), (63, 768, 3072), (65, 768, 3072), (500, 768, 3072), (896, 768, 3072),
         (130, 1024, 4096), (7, 768, 512)]


def _round(a, dtype):
    return synth.round_to_f16(a) if dtype == "f16" else synth.round_to_bf16(a)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,d,f", CASES)
def test_fused_mlp_matches_oracle(dtype, M, d, f):
    import torch
    import conformer_speech_recognition_amd as gg
    print(f"[mlp] {dtype} M={M} d={d} f={f}", flush=True)
    rng = np.random.default_rng(M * 11 + d + f)
    # the normed input: LayerNorm rows (unit gain, zero shift) rounded to the operand type
    y = _round(oracle.layer_norm(rng.standard_normal((M, d)), np.ones(d), np.zeros(d), 1e-5)
               .astype(np.float32), dtype)
    P = {"f.linear1.weight": _round((0.05 * rng.standard_normal((f, d))).astype(np.float32), dtype),
         "f.linear1.bias": rng.standard_normal(f).astype(np.float32),
         "f.linear2.weight": _round((0.05 * rng.standard_normal((d, f))).astype(np.float32), dtype),
         "f.linear2.bias": rng.standard_normal(d).astype(np.float32)}
    x = rng.standard_normal((M, d)).astype(np.float32)
    tt = torch.float16 if dtype == "f16" else torch.bfloat16
    dev = "cuda:0"
    X = torch.from_numpy(x).to(dev)
    gg.debug_mlp(dtype, torch.from_numpy(y).to(tt).to(dev),
                 torch.from_numpy(P["f.linear1.weight"]).to(tt).to(dev),
                 torch.from_numpy(P["f.linear1.bias"]).to(dev),
                 torch.from_numpy(P["f.linear2.weight"]).to(tt).to(dev),
                 torch.from_numpy(P["f.linear2.bias"]).to(dev), X, alpha=0.5)
    torch.cuda.synchronize()
    got = X.cpu().numpy().astype(np.float64)
    P64 = {k: v.astype(np.float64) for k, v in P.items()}
    y64 = y.astype(np.float64)
    ref = x + 0.5 * oracle.ffn_body(y64, P64, "f.")
    hid = oracle.silu(oracle.linear(y64, P64["f.linear1.weight"], P64["f.linear1.bias"]))
    u = 2.0 ** -11 if dtype == "f16" else 2.0 ** -8
    bound = 0.5 * (u * np.abs(hid) @ np.abs(P64["f.linear2.weight"]).T
                   + 1e-6 * (d + f) * (np.abs(hid).max() + np.abs(y64).max()) * 0.05 * 4) + 1e-5
    err = np.abs(got - ref)
    worst = float((err / bound).max())
    print(f"[mlp] {dtype} {M}x{d}x{f}: max|d| = {err.max():.3e}, worst err/bound {worst:.3f}", flush=True)
    assert worst <= 1.0
