"""GPU: every GEMM role of the encoder (gigaam_debug_gemm_role) at the row counts the
benchmark runs, with the A-operand mode and fused epilogue the encoder launches it with,
against the oracle's own linear / SiLU / GLU in float64 on the same stored operands.

Rows: 8207 (the 32-clip batch, the timed launch), 4113 (16 * 256 + 17: a ragged last
tile), 7500 (the ten 30 s chunks, d 1024) and 16000 (64 clips of 10 s, quantised weights).
The returned kernel shape is asserted, so each instantiation the encoder times is the one
under test."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

# role: (a_mode, epilogue, N(d, f), K(d, f), alpha)
ROLES = {
    "ffn_up": ("plain", "silu", lambda d, f: f, lambda d, f: d, 1.0),
    "pw1_glu": ("plain", "glu", lambda d, f: 2 * d, lambda d, f: d, 1.0),
    "qkv": ("dual", "store", lambda d, f: 3 * d, lambda d, f: d, 1.0),
    "ffn_down": ("plain", "resid", lambda d, f: d, lambda d, f: f, 0.5),
    "out_proj": ("plain", "resid", lambda d, f: d, lambda d, f: d, 1.0),
}
# kernel shape each role runs at 8207 rows (the benchmark's launch)
EXPECT_8207 = {"ffn_up": "dma_256x256", "pw1_glu": "dma_256x256", "qkv": "dma_256x128_k32",
               "ffn_down": "dma_256x128_k64", "out_proj": "dma_128x128"}

CASES = [(role, dt, 8207, 768, 3072) for role in ROLES for dt in ("f16", "bf16")]
CASES += [(role, "f16", 4113, 768, 3072) for role in ROLES]
CASES += [(role, "f16", 7500, 1024, 4096) for role in ("ffn_up", "qkv", "ffn_down")]
CASES += [(role, "w8f16", 16000, 768, 3072) for role in ("ffn_up", "ffn_down", "pw1_glu")]

UNIT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8, "w8f16": 2.0 ** -11}


def _round(a, dt):
    return synth.round_to_bf16(a) if dt == "bf16" else synth.round_to_f16(a)


def _glu_rows(d):
    """packed row order of the pointwise-1 weight: per 64-row group 32 value rows (32 q ..)
    then their 32 gate rows (d + 32 q ..)"""
    idx = []
    for q in range(d // 32):
        idx += list(range(32 * q, 32 * q + 32)) + list(range(d + 32 * q, d + 32 * q + 32))
    return np.array(idx)


@pytest.mark.parametrize("role,dt,M,d,f", CASES)
def test_gemm_role(role, dt, M, d, f):
    import torch
    import conformer_speech_recognition_amd as gg
    am, ep, Nf, Kf, alpha = ROLES[role]
    N, K = Nf(d, f), Kf(d, f)
    print(f"[role] {role} {dt} M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M + N + K + len(role))
    tt = torch.bfloat16 if dt == "bf16" else torch.float16
    a = _round(rng.standard_normal((M, K)).astype(np.float32), dt)
    a2 = _round(rng.standard_normal((M, K)).astype(np.float32), dt) if am == "dual" else None
    w = _round((0.05 * rng.standard_normal((N, K))).astype(np.float32), dt)
    b = rng.standard_normal(N).astype(np.float32)
    scale = None
    if dt == "w8f16":
        q, s = synth.quantize_g64(w, 8)
        w = oracle.dequantize_g64(q, s).astype(np.float32).astype(np.float16).astype(np.float32)
        from test_gpu_gemm import _pack_rows
        rows = _glu_rows(d) if ep == "glu" else np.arange(N)
        Wd = torch.from_numpy(_pack_rows(q[rows], 8)).cuda()
        scale = torch.from_numpy(np.ascontiguousarray(s[rows])).cuda()
    w_dev = w[_glu_rows(d)] if ep == "glu" else w
    b_dev = b[_glu_rows(d)] if ep == "glu" else b
    if dt != "w8f16":
        Wd = torch.from_numpy(w_dev).to(tt).cuda()
    A = torch.from_numpy(a).to(tt).cuda()
    A2 = torch.from_numpy(a2).to(tt).cuda() if a2 is not None else None
    bias = torch.from_numpy(b_dev).cuda()
    a64, w64, b64 = a.astype(np.float64), w.astype(np.float64), b.astype(np.float64)
    acc = 1e-6 * K * np.abs(a).max() * np.abs(w).max() + 1e-5
    if ep == "resid":
        x0 = rng.standard_normal((M, N)).astype(np.float32)
        C = torch.from_numpy(x0).cuda()
        ref = x0 + alpha * oracle.linear(a64, w64, b64)
        bound = np.full(ref.shape, alpha * acc + 2.0 ** -23 * np.abs(ref).max())
    elif ep == "glu":
        C = torch.empty(M, N // 2, dtype=tt, device="cuda")
        pre = oracle.linear(a64, w64, b64)
        ref = oracle.glu(pre)
        bound = acc * (1.0 + np.abs(pre[:, : N // 2]) / 4) + UNIT[dt] * np.abs(ref)
    elif ep == "silu":
        C = torch.empty(M, N, dtype=tt, device="cuda")
        ref = oracle.silu(oracle.linear(a64, w64, b64))
        bound = 1.1 * acc + UNIT[dt] * np.abs(ref)
    else:   # dual store: q, k from A, v from A2
        C = torch.empty(M, N, dtype=tt, device="cuda")
        ns = 2 * d
        ref = np.concatenate([oracle.linear(a64, w64[:ns], b64[:ns]),
                              oracle.linear(a2.astype(np.float64), w64[ns:], b64[ns:])], axis=1)
        bound = acc + UNIT[dt] * np.abs(ref)
    out, ks, shape = gg.debug_gemm_role(dt, am, ep, A, Wd, C,
                                        bias=bias, A2=A2, nsplit=2 * d if am == "dual" else 0,
                                        alpha=alpha, scale=scale)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    worst = float((err / bound).max())
    print(f"[role] {role} {dt} M={M}: shape {shape}, slices {ks}, max|d| {err.max():.3e}, "
          f"worst err/bound {worst:.3f}", flush=True)
    assert shape.startswith("dma_")
    if M == 8207:
        assert shape == EXPECT_8207[role]
    assert worst <= 1.0
