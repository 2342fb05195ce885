"""GPU: the encoder's MFMA GEMM alone (through gigaam_debug_gemm) against a float64
matmul of the same stored operands, for every operand type and ragged shapes."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

SHAPES = [(1, 34, 64), (77, 200, 320), (300, 768, 768), (129, 1536, 256), (513, 257, 128),
          (64, 64, 3840)]


def _pack_rows(q, bits):
    """The header's packed row layout, written independently with numpy: weight k at bits
    [k*b, k*b+b) of the row's little-endian bit string, two's complement."""
    N, K = q.shape
    u = (q.astype(np.int64) & ((1 << bits) - 1))
    bitsarr = ((u[:, :, None] >> np.arange(bits)) & 1).astype(np.uint8).reshape(N, K * bits)
    return np.packbits(bitsarr, axis=1, bitorder="little")


def _operands(dtype, M, N, K, seed):
    import torch
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K)).astype(np.float32)
    w = (0.05 * rng.standard_normal((N, K))).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    scale = None
    if dtype == "f32":
        A, W = torch.from_numpy(a), torch.from_numpy(w)
        w_eff = w.astype(np.float64)
    elif dtype == "f16":
        A, W = torch.from_numpy(a).half(), torch.from_numpy(w).half()
        a, w_eff = A.float().numpy(), W.float().double().numpy()
    elif dtype == "bf16":
        a = synth.round_to_bf16(a)
        w = synth.round_to_bf16(w)
        A, W = torch.from_numpy(a).bfloat16(), torch.from_numpy(w).bfloat16()
        w_eff = w.astype(np.float64)
    else:  # b-bit weights with one fp16 scale per 64 inputs, dequantised to fp16 in-kernel
        bits = synth.QUANT_BITS[dtype]
        A = torch.from_numpy(a).half()
        a = A.float().numpy()
        q, s = synth.quantize_g64(synth.round_to_f16(w), bits)
        W = torch.from_numpy(_pack_rows(q, bits))
        scale = torch.from_numpy(s)
        deq = q.astype(np.float32) * np.repeat(s.astype(np.float32), 64, axis=1)
        w_eff = deq.astype(np.float16).astype(np.float64)
    return A.cuda(), W.cuda(), (scale.cuda() if scale is not None else None), \
        torch.from_numpy(b).cuda(), a.astype(np.float64), w_eff, b.astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "w8f16", "w6f16", "w4f16"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_matches_float64(dtype, M, N, K):
    import conformer_speech_recognition_amd as gg
    if dtype in synth.QUANT_BITS and K % 64:
        pytest.skip("quantisation groups need K % 64 == 0")
    print(f"[gemm] {dtype} M={M} N={N} K={K}", flush=True)
    A, W, S, bias, a, w, b = _operands(dtype, M, N, K, seed=M * 7 + N + K)
    C = gg.debug_gemm(dtype, A, W, bias=bias, scale=S).cpu().numpy().astype(np.float64)
    ref = a @ w.T + b
    # fp32 accumulation of K exact products: |err| <= K * 2^-24 * sum|a||w| (loose)
    bound = 1e-6 * K * np.abs(a).max() * np.abs(w).max() + 1e-5
    err = np.abs(C - ref).max()
    print(f"[gemm] {dtype} {M}x{N}x{K} max|d| = {err:.3e} (bound {bound:.2e})", flush=True)
    assert err <= bound


SPLIT_SHAPES = [(25, 768, 3072), (500, 768, 3072), (77, 2304, 768), (300, 768, 768), (1, 1536, 768),
                (130, 3072, 768)]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "w8f16", "w6f16", "w4f16"])
@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_split_k_matches_float64(dtype, M, N, K):
    """Small M: the K sum split across workgroups (fp32 partials added in slice order by a
    second kernel) meets the same bound, and the unsplit kernel agrees with it (for the
    quantised weights the split runs in the register-staged kernel)."""
    import conformer_speech_recognition_amd as gg
    print(f"[gemm split] {dtype} M={M} N={N} K={K}", flush=True)
    A, W, S, bias, a, w, b = _operands(dtype, M, N, K, seed=M * 5 + N + K)
    C, ks = gg.debug_gemm(dtype, A, W, bias=bias, scale=S, split=True)
    C = C.cpu().numpy().astype(np.float64)
    C1 = gg.debug_gemm(dtype, A, W, bias=bias, scale=S).cpu().numpy().astype(np.float64)
    ref = a @ w.T + b
    bound = 1e-6 * K * np.abs(a).max() * np.abs(w).max() + 1e-5
    err = np.abs(C - ref).max()
    print(f"[gemm split] {dtype} {M}x{N}x{K}: {ks} slices, max|d| = {err:.3e} (bound {bound:.2e}), "
          f"vs unsplit {np.abs(C - C1).max():.3e}", flush=True)
    assert ks > 1
    assert err <= bound and np.abs(C1 - ref).max() <= bound


DEQUANT_SHAPES = [(2048, 768, 768), (2100, 3072, 768), (4096, 768, 3072)]


@pytest.mark.parametrize("dtype", ["w8f16", "w6f16", "w4f16"])
@pytest.mark.parametrize("M,N,K", DEQUANT_SHAPES)
def test_dequantised_pipeline_matches_float64(dtype, M, N, K):
    """Many rows of A with quantised weights and a workspace: the weights are expanded to
    fp16 first and the pipelined fp16 kernel runs on them; same bound, and it agrees with
    the register-staged kernel that reads the packed weights directly."""
    import conformer_speech_recognition_amd as gg
    print(f"[gemm dequant] {dtype} M={M} N={N} K={K}", flush=True)
    A, W, S, bias, a, w, b = _operands(dtype, M, N, K, seed=M * 3 + N + K)
    C, ks = gg.debug_gemm(dtype, A, W, bias=bias, scale=S, split=True)
    C = C.cpu().numpy().astype(np.float64)
    C1 = gg.debug_gemm(dtype, A, W, bias=bias, scale=S).cpu().numpy().astype(np.float64)
    ref = a @ w.T + b
    bound = 1e-6 * K * np.abs(a).max() * np.abs(w).max() + 1e-5
    err = np.abs(C - ref).max()
    print(f"[gemm dequant] {dtype} {M}x{N}x{K}: max|d| = {err:.3e} (bound {bound:.2e}), "
          f"vs register-staged {np.abs(C - C1).max():.3e}", flush=True)
    assert ks == 1
    assert err <= bound and np.abs(C1 - ref).max() <= bound


@pytest.mark.parametrize("M,N,K", [(500, 34, 768), (77, 257, 768), (1, 129, 1024)])
def test_fp32_head_split_matches_float64(M, N, K):
    """The fp32 CTC head of the 16-bit models at few rows: its K sum is split too, and an
    output width that is no multiple of 4 (34, 129, 257 classes) is reduced one output per
    thread; same bound as the unsplit kernel, which agrees with it."""
    import conformer_speech_recognition_amd as gg
    print(f"[gemm head split] M={M} N={N} K={K}", flush=True)
    A, W, S, bias, a, w, b = _operands("f32", M, N, K, seed=M * 7 + N + K)
    C, ks = gg.debug_gemm("f32", A, W, bias=bias, scale=S, split=True)
    C = C.cpu().numpy().astype(np.float64)
    C1 = gg.debug_gemm("f32", A, W, bias=bias, scale=S).cpu().numpy().astype(np.float64)
    ref = a @ w.T + b
    bound = 1e-6 * K * np.abs(a).max() * np.abs(w).max() + 1e-5
    err = np.abs(C - ref).max()
    print(f"[gemm head split] {M}x{N}x{K}: {ks} slices, max|d| = {err:.3e} (bound {bound:.2e}), "
          f"vs unsplit {np.abs(C - C1).max():.3e}", flush=True)
    assert ks > 1
    assert err <= bound and np.abs(C1 - ref).max() <= bound
