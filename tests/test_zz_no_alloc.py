"""GPU: the allocation-free entry point (gigaam_encode_noalloc: the encode with its
workspace in the library's fixed per-GPU scratch array) gives the same outputs as
gigaam_encode with a caller workspace, on two calls in a row, the second with a smaller
input, for a 16-bit model (split-K partial sums live in the scratch) and the fp32 model;
a call needing more than the scratch is refused before any launch."""
import numpy as np
import pytest

import synth
from gpu_common import model, say, workload

pytestmark = pytest.mark.gpu


def _outputs(m, B, U_max):
    import torch
    C, d = m.cfg["n_classes"], m.cfg["d_model"]
    return dict(log_probs=torch.full((B, U_max, C), float("nan"), device="cuda"),
                token_ids=torch.full((B, U_max), -7, dtype=torch.int32, device="cuda"),
                n_tokens=torch.full((B,), -7, dtype=torch.int32, device="cuda"),
                frame_ids=torch.full((B, U_max), -7, dtype=torch.int32, device="cuda"),
                enc_out=torch.full((B, U_max, d), float("nan"), device="cuda"))


@pytest.mark.parametrize("name,calls", [
    ("v3_20s", [[320000, 192000], [80000]]),
    ("tiny", [[32000, 20000, 9600], [4800]]),
])
def test_noalloc_matches_encode(name, calls):
    import torch
    import conformer_speech_recognition_amd as gg
    m = model(name)
    rng = np.random.default_rng(90)
    for i, lengths in enumerate(calls):
        pcm, lens = synth.pad_batch([synth.make_signal(rng, n) for n in lengths])
        need = m.workspace_bytes(len(lens), int(lens.max()))
        say(f"[noalloc] {name} call {i}: clips {lens.tolist()}, workspace {need} bytes")
        assert need <= gg.NOALLOC_SCRATCH_BYTES
        d = torch.from_numpy(pcm).cuda()
        ref = m.encode(d, lens, want_enc=True)
        U = [gg.frames(int(n))[2] for n in lens]
        out = m.encode_noalloc(d, lens, _outputs(m, len(lens), max(U)))
        torch.cuda.synchronize()
        assert out["n_frames"].tolist() == ref["n_frames"].tolist() == U
        for k in ("enc_out", "log_probs", "frame_ids", "token_ids", "n_tokens"):
            assert torch.equal(out[k], ref[k]), (name, i, k)
        say(f"[noalloc] {name} call {i}: outputs identical to gigaam_encode")


def test_noalloc_refuses_more_than_its_scratch():
    import torch
    import conformer_speech_recognition_amd as gg
    m = model("v3_20s")
    lens = np.full(8, 320000, dtype=np.int32)
    assert m.workspace_bytes(8, 320000) > gg.NOALLOC_SCRATCH_BYTES
    pcm = torch.zeros(8, 320000, device="cuda")
    out = _outputs(m, 8, 500)
    with pytest.raises(gg.GigaamError) as e:
        m.encode_noalloc(pcm, lens, out)
    assert e.value.code == gg.E_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool(torch.all(out["n_tokens"] == -7))            # nothing was launched
