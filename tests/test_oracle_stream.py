"""Pins for the pseudo-streaming oracle (oracle/stream.py): which samples each step
re-encodes ("GigaAM on MLX ...", section "Streaming: honestly, it's pseudo-streaming":
all audio received so far, but no more than the last 30 seconds)."""
import numpy as np
import pytest

from oracle import stream


def test_worked_example_by_hand():
    # pushes of 100, 300, 500 samples with a 600-sample cap: the third step has 900
    # samples buffered and keeps the newest 600
    assert stream.windows([100, 300, 500], 600) == [(0, 100), (0, 400), (300, 900)]


def test_thirty_second_cap_at_16_khz():
    # one-second pushes: the window grows to 30 s, then slides one second per step
    w = stream.windows([16000] * 45, 480000)
    assert w[29] == (0, 480000) and w[30] == (16000, 496000) and w[44] == (240000, 720000)


def test_window_length_is_min_of_total_and_cap():
    rng = np.random.default_rng(0)
    chunks = rng.integers(0, 5000, 200)
    total = np.cumsum(chunks)
    for (lo, hi), t in zip(stream.windows(chunks, 12345), total):
        assert hi == t and hi - lo == min(t, 12345)


def test_empty_push_repeats_the_window_and_negative_is_rejected():
    assert stream.windows([700, 0], 500) == [(200, 700), (200, 700)]
    with pytest.raises(ValueError):
        stream.windows([10, -1], 500)
