"""Pins for the oracle's frontend and frame arithmetic (CPU only).

Every check compares against something other than the oracle's own formula: numbers
printed on the pages (tests/golden/), closed forms of the DFT of a windowed cosine,
a library FFT, Parseval's identity, partition-of-unity of triangular filters, and the
defining property of the HTK mel scale.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ frame counts

def test_frame_counts_printed_on_pages():
    g = _gold("frame_counts.json")
    for case in g["cases"]:
        if "n_samples" in case:
            assert oracle.num_frames(case["n_samples"]) == case["mel_frames"]
        T = case["mel_frames"]
        U = oracle.conv_out_len(oracle.conv_out_len(T))
        assert U == case["enc_frames"], case["source"]


def test_one_second_clip_gives_printed_shapes():
    # a 1 s clip (16000 samples) gives the [64, 99] mel and 25 encoder frames printed
    T, S, U = oracle.encoder_frames(16000)
    assert (T, U) == (99, 25)


@pytest.mark.parametrize("secs,T,U", [(2, 199, 50), (10, 999, 250), (20, 1999, 500), (30, 2999, 750)])
def test_frames_for_workload_durations(secs, T, U):
    t, s, u = oracle.encoder_frames(16000 * secs)
    assert (t, u) == (T, U)
    # encoder frame ~ 40 ms (10 ms hop x 4)
    g = _gold("frame_counts.json")["frame_seconds"]["value"]
    assert abs(secs / u - g) < 0.001


def test_frame_count_brute_force():
    # count windows that fit by sliding, for many lengths
    for L in list(range(320, 2000, 7)) + [16000, 16159, 16160]:
        n, start = 0, 0
        while start + 320 <= L:
            n += 1
            start += 160
        assert oracle.num_frames(L) == n


def test_short_clip_rejected():
    with pytest.raises(ValueError):
        oracle.num_frames(319)


def test_conv_out_len_matches_sliding_positions():
    for n in range(1, 60):
        # positions s with window [2s-2, 2s+2] whose centre 2s lies in [0, n)
        count = len([s for s in range(0, n) if 2 * s < n])
        assert oracle.conv_out_len(n) == count


# ------------------------------------------------------------------ window + DFT

def test_frontend_constants_match_card():
    g = _gold("frontend_constants.json")
    assert (g["n_fft"], g["win_length"], g["hop_length"], g["n_mels"]) == (320, 320, 160, 64)
    assert len(oracle.hann_periodic(g["win_length"])) == 320
    assert oracle.htk_mel_filterbank().shape == (g["n_fft"] // 2 + 1, g["n_mels"])


@pytest.mark.parametrize("k0", [2, 3, 17, 80, 121, 158])
def test_bin_centred_cosine_closed_form(k0):
    """x[n] = A cos(2 pi k0 n / 320) under the periodic Hann window has exactly three
    non-zero DFT bins: X[k0] = 80 A, X[k0 +- 1] = -40 A  =>  P = 6400 A^2, 1600 A^2.
    A symmetric (N-1) window or a wrong basis leaks into other bins."""
    A = 0.7
    n = np.arange(320)
    x = A * np.cos(2 * np.pi * k0 * n / 320)
    P = oracle.dft_power((x * oracle.hann_periodic(320))[None, :])[0]
    expect = np.zeros(161)
    expect[k0] = 6400 * A * A
    expect[k0 - 1] = expect[k0 + 1] = 1600 * A * A
    np.testing.assert_allclose(P, expect, atol=1e-9)


def test_window_is_periodic_not_symmetric():
    w = oracle.hann_periodic(320)
    assert w[0] == 0.0 and abs(w[160] - 1.0) < 1e-15
    assert abs(w[1] - w[319]) < 1e-15            # periodic: w[n] = w[N - n]
    assert w[319] > 0                           # a symmetric window would end at 0


def test_power_matches_library_fft():
    rng = np.random.default_rng(0)
    fr = rng.standard_normal((7, 320))
    P = oracle.dft_power(fr)
    ref = np.abs(np.fft.rfft(fr, n=320, axis=1)) ** 2
    np.testing.assert_allclose(P, ref, rtol=1e-10, atol=1e-9)


def test_parseval():
    rng = np.random.default_rng(1)
    fr = rng.standard_normal((3, 320))
    P = oracle.dft_power(fr)
    full = P[:, 0] + P[:, 160] + 2 * P[:, 1:160].sum(axis=1)
    np.testing.assert_allclose(full / 320, (fr ** 2).sum(axis=1), rtol=1e-12)


def test_framing_hop_and_tail():
    pcm = np.arange(16000 + 100, dtype=np.float64)
    fr = oracle.frame_signal(pcm)
    assert fr.shape == (99, 320)
    assert fr[0, 0] == 0 and fr[1, 0] == 160 and fr[98, 319] == 98 * 160 + 319
    # tail samples beyond the last full window are dropped, no centring pad
    assert fr.max() < 16000


# ------------------------------------------------------------------ mel + log

def test_htk_mel_scale_definition():
    # HTK mel: 1000 Hz ~ 1000 mel and the inverse is exact
    assert abs(oracle.hz_to_mel_htk(1000.0) - 1000.0) < 0.02
    f = np.array([0.0, 27.0, 700.0, 4000.0, 8000.0])
    np.testing.assert_allclose(oracle.mel_to_hz_htk(oracle.hz_to_mel_htk(f)), f, atol=1e-9)


def test_filterbank_partition_of_unity_and_peaks():
    fb = oracle.htk_mel_filterbank()
    f = np.arange(161) * 50.0
    corners = oracle.mel_to_hz_htk(np.linspace(0, oracle.hz_to_mel_htk(8000.0), 66))
    # equally spaced in mel
    np.testing.assert_allclose(np.diff(oracle.hz_to_mel_htk(corners)), np.diff(oracle.hz_to_mel_htk(corners))[0])
    # between the 2nd and 65th corner, adjacent triangles sum to one (linear in Hz)
    inner = (f >= corners[1]) & (f <= corners[64])
    np.testing.assert_allclose(fb[inner].sum(axis=1), 1.0, atol=1e-12)
    # outside the outer corners nothing responds
    assert np.all(fb[f <= corners[0]] == 0)
    # every filter is non-empty, non-negative and peaks at its own centre region
    assert np.all(fb >= 0) and np.all(fb.max(axis=0) > 0)
    peaks = f[np.argmax(fb, axis=0)]
    assert np.all(np.abs(peaks - corners[1:65]) <= 50.0)
    # filters are ordered in frequency
    assert np.all(np.diff(np.argmax(fb, axis=0)) >= 0)


def test_silence_clips_to_floor():
    mel = oracle.log_mel(np.zeros(16000))
    assert mel.shape == (99, 64)
    np.testing.assert_array_equal(mel, np.log(1e-9))
    assert abs(np.log(1e-9) - (-20.72326583694641)) < 1e-12


def test_log_clip_ceiling():
    # a full-scale 1e6 amplitude sine saturates the 1e9 ceiling in its bin's filters
    n = np.arange(16000)
    x = 1e6 * np.cos(2 * np.pi * 40 * 50 * n / 16000)
    mel = oracle.log_mel(x)
    assert abs(mel.max() - np.log(1e9)) < 1e-12


def test_log_mel_pipeline_on_pure_tone():
    """A 2 kHz bin-centred tone of amplitude A: only bins 39..41 carry power
    (1600, 6400, 1600) A^2, so every mel value is ln(sum_k fb[k,m] P[k]) exactly."""
    A = 0.5
    n = np.arange(16000)
    x = A * np.cos(2 * np.pi * 2000 * n / 16000)
    mel = oracle.log_mel(x)
    fb = oracle.htk_mel_filterbank()
    m = fb[39] * 1600 * A * A + fb[40] * 6400 * A * A + fb[41] * 1600 * A * A
    expect = np.log(np.clip(m, 1e-9, 1e9))
    # bins other than 39..41 get ~1e-20 leakage from rounding: compare where it matters
    big = m > 1e-6
    np.testing.assert_allclose(mel[5][big], expect[big], atol=1e-9)
