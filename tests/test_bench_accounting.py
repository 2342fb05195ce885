"""CPU: the benchmark's algorithmic FLOP count (valid frames only) against a direct per-clip
count of the encoder's products, and against the totals of the four GPU workloads.

Per clip of n samples: T = 1 + (n - 320) // 160 frames of 320 samples at hop 160 (no padding),
S and U after each stride-2, kernel-5, padding-2 convolution. Per layer and clip the products
are FFN up/down twice (8 U d f), q/k/v, out, pointwise-1 (2d wide) and pointwise-2 (14 U d^2),
attention scores and values (4 U^2 d) and the depthwise conv (2 U d k); the subsampling
convs add 2 S (64 * 5) d + 2 U (5 d) d and the CTC head 2 U d C."""
import importlib.util
import os

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _direct(cfg, lens):
    d, f, k, C, L = cfg["d_model"], cfg["d_ff"], cfg["conv_kernel"], cfg["n_classes"], cfg["n_layers"]
    total = 0
    for n in lens:
        T = 1 + (int(n) - 320) // 160
        S = (T + 4 - 5) // 2 + 1
        U = (S + 4 - 5) // 2 + 1
        total += L * (8 * U * d * f + 14 * U * d * d + 4 * U * U * d + 2 * U * d * k)
        total += 2 * S * 320 * d + 2 * U * 5 * d * d + 2 * U * d * C
    return total


# algorithmic GFLOP of each workload (valid frames only), to 0.1 GFLOP
TOTALS = {"v3_20s": 233.2, "batch32": 3757.9, "ml_long": 9337.1, "int8_b64": 7265.5}


@pytest.mark.parametrize("name", sorted(TOTALS))
def test_flop_count(name):
    b = _bench()
    cfg = synth.workload_config(name)
    lens = [len(x) for x in synth.workload_signals(name)]
    got = b.total_flops(cfg, lens)
    assert got == _direct(cfg, lens)
    assert abs(got / 1e9 - TOTALS[name]) < 0.05 + 1e-4 * TOTALS[name]
