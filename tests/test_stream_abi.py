"""CPU-side checks of the pseudo-streaming ABI: state validation, and the ring plan of
gigaam_stream_plan_push replayed on a NumPy ring against the oracle's windows (every
step's window must sit contiguously in the ring with the right samples), plus the
argument errors of push and step before any launch."""
import ctypes

import numpy as np
import pytest

import synth
from oracle import stream as ostream


@pytest.fixture(scope="module")
def gg():
    import os
    import conformer_speech_recognition_amd as g
    if not os.path.exists(g.LIB_PATH):
        from conformer_speech_recognition_amd.build import build
        build()
    g.lib()
    return g


def _init(gg, window, capacity):
    st = gg.StreamState()
    rc = gg.lib().gigaam_stream_init(ctypes.byref(st), window, capacity)
    return rc, st


def test_init_validation(gg):
    assert _init(gg, 480000, 960000)[0] == 0
    assert _init(gg, 319, 1000)[0] == gg.E_INVAL
    assert _init(gg, 1000, 1999)[0] == gg.E_INVAL
    assert _init(gg, (1 << 29) + 1, 2 ** 31 - 1)[0] == gg.E_INVAL
    assert gg.lib().gigaam_stream_init(None, 1000, 2000) == gg.E_INVAL


@pytest.mark.parametrize("window,extra,seed", [(1000, 0, 1), (1000, 37, 2), (480000, 0, 3),
                                               (4000, 4000, 4)])
def test_ring_plan_replayed_on_numpy(gg, window, extra, seed):
    L = gg.lib()
    rng = np.random.default_rng(seed)
    capacity = 2 * window + extra
    rc, st = _init(gg, window, capacity)
    assert rc == 0
    # chunk sizes: mostly small, some empty, some longer than the window
    chunks = rng.integers(0, window // 3 + 2, 120)
    chunks[rng.integers(0, 120, 6)] = 0
    chunks[rng.integers(0, 120, 3)] = window + rng.integers(1, window, 3)
    audio = rng.standard_normal(int(chunks.sum())).astype(np.float32)
    ring = np.full(capacity, np.nan, np.float32)
    moved = 0
    pos = 0
    for n, (lo, hi) in zip(chunks, ostream.windows(chunks, window)):
        p = gg.StreamPlan()
        assert L.gigaam_stream_plan_push(ctypes.byref(st), int(n), ctypes.byref(p)) == 0
        if p.move_len:
            moved += p.move_len
            assert p.move_src >= p.move_len                     # no overlap
            assert p.move_src + p.move_len <= capacity
            ring[: p.move_len] = ring[p.move_src: p.move_src + p.move_len].copy()
        assert p.skip + p.append_len == n and p.append_len == min(n, window)
        assert 0 <= p.append_at and p.append_at + p.append_len <= capacity
        ring[p.append_at: p.append_at + p.append_len] = audio[pos + p.skip: pos + n]
        pos += n
        st.total, st.start, st.length = p.total, p.start, p.length
        assert st.total == hi and st.length == hi - lo
        np.testing.assert_array_equal(ring[st.start: st.start + st.length], audio[lo:hi])
    # moves copy at most one window per (capacity - window) samples pushed
    assert moved <= window * (chunks.sum() // (capacity - window) + 1)


def test_push_and_step_errors_before_any_launch(gg):
    L = gg.lib()
    cfg = synth.workload_config("tiny")
    c = gg.make_config(cfg)
    h = ctypes.c_void_p()
    fake = 1 << 20
    assert L.gigaam_create(ctypes.byref(c), fake, fake, fake, ctypes.byref(h)) == 0
    rc, st = _init(gg, 16000, 32000)
    assert rc == 0
    assert L.gigaam_stream_push(ctypes.byref(st), None, fake, 10, None) == gg.E_INVAL
    assert L.gigaam_stream_push(ctypes.byref(st), fake, None, 10, None) == gg.E_INVAL
    assert L.gigaam_stream_push(ctypes.byref(st), fake, fake, -1, None) == gg.E_INVAL
    assert st.total == 0 and st.length == 0                    # untouched by failed pushes
    nb = ctypes.c_size_t()
    assert L.gigaam_workspace_bytes(h, 1, 16000, ctypes.byref(nb)) == 0

    def step(state):
        return L.gigaam_stream_step(h, ctypes.byref(state), fake, fake, nb.value, fake, fake, fake,
                                    None, None, None, None)
    assert step(st) == gg.E_INVAL                               # nothing buffered yet
    assert "at least 320" in L.gigaam_last_error().decode()
    st.length, st.total = 300, 300
    assert step(st) == gg.E_INVAL
    bad = gg.StreamState(total=10, window=16000, capacity=32000, start=31000, length=5000)
    assert step(bad) == gg.E_INVAL                              # window runs past the ring
    p = gg.StreamPlan()
    assert L.gigaam_stream_plan_push(ctypes.byref(bad), 5, ctypes.byref(p)) == gg.E_INVAL
    L.gigaam_destroy(h)
