"""GPU: pseudo-streaming (gigaam_stream_push / gigaam_stream_step) against the oracle.

"GigaAM on MLX ...", section "Streaming: honestly, it's pseudo-streaming": every step
re-encodes all audio so far, capped at the last 30 s. Each step's output must be the
oracle's encoding of the window oracle.stream.windows names (tiny fp32 model, a short
cap so the window slides and the ring moves many times: enc_out within 1e-4, ids and
tokens exact). At full size (16-layer fp16 model, 30 s cap, 75 s of audio in 2.5 s
pushes) every step must give the same bits as a plain gigaam_encode of a separate
copy of its window, and the last, slid 30 s window is checked against the oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import TOL_F32, TOL_LOW, Agreement, argmax_agreement, model, say, workload
from oracle import stream as ostream

pytestmark = pytest.mark.gpu


def _chunks(rng, total, lo, hi):
    out, s = [], 0
    while s < total:
        n = int(min(rng.integers(lo, hi), total - s))
        out.append(n)
        s += n
    return out


def test_stream_steps_match_the_oracle_windows():
    import torch
    import conformer_speech_recognition_amd as gg
    cfg, _, _, w = workload("tiny")
    rng = np.random.default_rng(50)
    audio = synth.make_signal(rng, 80000)                       # 5 s
    chunks = [200, 150] + _chunks(rng, 30000, 1000, 9000) + [0, 25000] + _chunks(rng, 24650, 500, 7000)
    assert sum(chunks) == len(audio)
    window = 19200                                               # 1.2 s cap
    st = gg.Stream(model("tiny"), window=window, capacity=2 * window + 1000)
    dev = torch.from_numpy(audio).cuda()
    pos, steps = 0, 0
    for n, (lo, hi) in zip(chunks, ostream.windows(chunks, window)):
        st.push(dev[pos: pos + n])
        pos += n
        assert (st.state.total, st.state.length) == (hi, hi - lo)
        np.testing.assert_array_equal(st.window_view().cpu().numpy(), audio[lo:hi])
        if hi - lo < 320:
            with pytest.raises(gg.GigaamError):
                st.step()
            continue
        out = st.step(want_enc=True)
        torch.cuda.synchronize()
        ref = oracle.encode_clip(audio[lo:hi].astype(np.float64), w, cfg)
        u = ref["enc_out"].shape[0]
        assert out["n_frames"][0] == u
        err = np.abs(out["enc_out"].cpu().numpy()[0, :u] - ref["enc_out"]).max()
        ids = out["frame_ids"].cpu().numpy()[0, :u]
        toks = gg.tokens_list(out)[0]
        assert err <= TOL_F32, (lo, hi, err)
        np.testing.assert_array_equal(ids, oracle.greedy_ids(ref["log_probs"]))
        assert toks == oracle.ctc_collapse(ids, cfg["n_classes"] - 1)
        steps += 1
    say(f"[stream] tiny: {steps} steps over {len(chunks)} pushes match the oracle windows")
    assert steps >= 15


def test_stream_at_thirty_seconds():
    import torch
    import conformer_speech_recognition_amd as gg
    name = "v3_20s"
    cfg, _, _, w = workload(name)
    m = model(name)
    rng = np.random.default_rng(51)
    audio = synth.make_signal(rng, 75 * 16000)
    chunks = [40000] * 30
    st = gg.Stream(m, window=480000)
    dev = torch.from_numpy(audio).cuda()
    pos, last = 0, None
    for n, (lo, hi) in zip(chunks, ostream.windows(chunks, 480000)):
        st.push(dev[pos: pos + n])
        pos += n
        out = st.step(want_enc=True)
        direct = m.encode(dev[lo:hi].clone().reshape(1, -1), [hi - lo], want_enc=True)
        for k in ("enc_out", "log_probs", "frame_ids", "token_ids", "n_tokens"):
            assert torch.equal(out[k], direct[k]), (k, lo, hi)
        last = (lo, hi, {k: v.cpu().numpy() for k, v in out.items() if hasattr(v, "cpu")})
    lo, hi, out = last
    assert (lo, hi) == (720000, 1200000)
    say(f"[stream] v3 30 s: 30 steps equal direct encodes; oracle on window [{lo}, {hi})")
    ref = oracle.encode_clip(audio[lo:hi].astype(np.float64), w, cfg)
    u = ref["enc_out"].shape[0]
    err = np.abs(out["enc_out"][0, :u] - ref["enc_out"]).max()
    lp_err = np.abs(out["log_probs"][0, :u] - ref["log_probs"]).max()
    agg = Agreement(cfg["dtype"])
    agg.add(argmax_agreement(out["frame_ids"][0, :u], ref["log_probs"], cfg["dtype"]))
    say(f"[stream] v3 30 s window: enc max|d| {err:.3e}, logp max|d| {lp_err:.3e}")
    agg.report("stream v3 30 s")
    assert err <= TOL_LOW and lp_err <= TOL_LOW
    agg.check()
