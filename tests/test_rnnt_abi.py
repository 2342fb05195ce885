"""CPU-side checks of the RNNT head's C ABI: configuration validation, the canonical
weight list, the host repacking against NumPy (transposes, bias sum, padding) and the
decode call's argument validation (no GPU work is issued)."""
import ctypes

import numpy as np
import pytest

import synth


@pytest.fixture(scope="module")
def gg():
    import os
    import conformer_speech_recognition_amd as g
    if not os.path.exists(g.LIB_PATH):
        from conformer_speech_recognition_amd.build import build
        build()
    g.lib()
    return g


@pytest.mark.parametrize("field,value", [("pred_hidden", 300), ("joint_hidden", 0),
                                         ("n_classes", 1), ("max_symbols", 0), ("max_symbols", 65),
                                         ("dtype", 3), ("d_model", 100)])
def test_rnnt_config_validation(gg, field, value):
    cfg = synth.rnnt_config(768, 34, "f16")
    c = gg.make_rnnt_config(cfg)
    assert gg.lib().gigaam_rnnt_check_config(ctypes.byref(c)) == 0
    setattr(c, field, value)
    assert gg.lib().gigaam_rnnt_check_config(ctypes.byref(c)) == gg.E_INVAL


def test_rnnt_canonical_entries_match_the_checkpoint_names(gg):
    cfg = synth.rnnt_config(768, 1025, "bf16")
    ents = gg.rnnt_canonical_entries(cfg)
    assert [(n, s) for n, s, _ in ents] == synth.rnnt_entries(cfg)
    offs = [o for _, _, o in ents]
    sizes = [int(np.prod(s)) for _, s, _ in ents]
    assert offs == list(np.cumsum([0] + sizes[:-1]))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_rnnt_pack_layout(gg, dtype):
    """Packed order (256-B aligned): embed [C][P], W_ih [4P][P], b_ih + b_hh (f32),
    W_hh^T [P][4P], W_enc [J][d], b_enc, W_pred^T [P][J], b_pred, W_out^T [J][Cp]
    (Cp = C rounded up to 8, zero padded), b_out."""
    C, P, J, d = 34, 64, 128, 192
    cfg = synth.rnnt_config(d, C, dtype, pred_hidden=P, joint_hidden=J)
    w = synth.make_rnnt_weights(cfg, 11)
    packed = gg.rnnt_pack_weights(cfg, w)
    es = 4 if dtype == "f32" else 2
    Cp = (C + 7) // 8 * 8
    al = lambda x: (x + 255) // 256 * 256
    sizes = [C * P * es, 4 * P * P * es, 4 * P * 4, P * 4 * P * es, J * d * es, J * 4,
             P * J * es, J * 4, J * Cp * es, C * 4]
    offs, o = [], 0
    for s in sizes:
        offs.append(o)
        o = al(o + s)
    assert packed.size == o

    def mat(i, shape):
        raw = packed[offs[i]: offs[i] + int(np.prod(shape)) * es]
        if dtype == "f32":
            return raw.view(np.float32).reshape(shape)
        if dtype == "f16":
            return raw.view(np.float16).astype(np.float32).reshape(shape)
        return (raw.view(np.uint16).astype(np.uint32) << 16).view(np.float32).reshape(shape)

    def vec(i, n):
        return packed[offs[i]: offs[i] + 4 * n].view(np.float32)

    np.testing.assert_array_equal(mat(0, (C, P)), w["rnnt.embed.weight"])
    np.testing.assert_array_equal(mat(1, (4 * P, P)), w["rnnt.lstm.weight_ih_l0"])
    np.testing.assert_array_equal(vec(2, 4 * P), (w["rnnt.lstm.bias_ih_l0"].astype(np.float32)
                                                  + w["rnnt.lstm.bias_hh_l0"].astype(np.float32)))
    np.testing.assert_array_equal(mat(3, (P, 4 * P)), w["rnnt.lstm.weight_hh_l0"].T)
    np.testing.assert_array_equal(mat(4, (J, d)), w["rnnt.joint.enc.weight"])
    np.testing.assert_array_equal(vec(5, J), w["rnnt.joint.enc.bias"])
    np.testing.assert_array_equal(mat(6, (P, J)), w["rnnt.joint.pred.weight"].T)
    np.testing.assert_array_equal(vec(7, J), w["rnnt.joint.pred.bias"])
    wo = mat(8, (J, Cp))
    np.testing.assert_array_equal(wo[:, :C], w["rnnt.joint.out.weight"].T)
    assert np.all(wo[:, C:] == 0)
    np.testing.assert_array_equal(vec(9, C), w["rnnt.joint.out.bias"])


def test_rnnt_decode_argument_errors_before_any_launch(gg):
    L = gg.lib()
    cfg = synth.rnnt_config(768, 34, "f16")
    c = gg.make_rnnt_config(cfg)
    h = ctypes.c_void_p()
    fake = 1 << 20
    assert L.gigaam_rnnt_create(ctypes.byref(c), fake, ctypes.byref(h)) == 0
    nb = ctypes.c_size_t()
    assert L.gigaam_rnnt_workspace_bytes(h, 2, 50, ctypes.byref(nb)) == 0 and nb.value > 0
    I = ctypes.c_int32
    fr = (I * 2)(50, 17)

    def dec(stride=50, frames=fr, batch=2, ws=fake, wsb=nb.value, max_tokens=500, tokens=fake):
        return L.gigaam_rnnt_decode(h, fake, stride, frames, batch, ws, wsb, tokens, None, fake,
                                    max_tokens, None)
    assert dec(batch=0) == gg.E_INVAL
    assert dec(frames=(I * 2)(50, 0)) == gg.E_INVAL
    assert dec(frames=(I * 2)(51, 3)) == gg.E_INVAL
    assert dec(max_tokens=499) == gg.E_INVAL
    assert dec(wsb=nb.value - 1) == gg.E_WORKSPACE
    assert dec(ws=fake + 16) == gg.E_INVAL
    assert dec(tokens=None) == gg.E_INVAL
    L.gigaam_rnnt_destroy(h)
    assert L.gigaam_rnnt_create(ctypes.byref(c), fake + 8, ctypes.byref(h)) == gg.E_INVAL


def test_rnnt_cluster_controls_validate_and_size_the_workspace(gg):
    """The cap on the decoding cluster is range-checked; the workspace grows with the
    exchange words of the clustered decoder (two slots of partial logits and h slices per
    clip, one XCD word per member), sized for up to two workgroups per CU."""
    L = gg.lib()
    cfg = synth.rnnt_config(768, 34, "f16")
    c = gg.make_rnnt_config(cfg)
    h = ctypes.c_void_p()
    assert L.gigaam_rnnt_create(ctypes.byref(c), 1 << 20, ctypes.byref(h)) == 0
    assert L.gigaam_rnnt_set_max_cluster(h, 0) == gg.E_INVAL
    assert L.gigaam_rnnt_set_max_cluster(h, 65) == gg.E_INVAL
    assert L.gigaam_rnnt_set_max_cluster(None, 4) == gg.E_INVAL
    assert L.gigaam_rnnt_set_max_cluster(h, 1) == 0
    g = ctypes.c_int32()
    assert L.gigaam_rnnt_cluster_size(h, 0, ctypes.byref(g)) == gg.E_INVAL
    assert L.gigaam_rnnt_cluster_size(h, 4, None) == gg.E_INVAL

    def ws(batch, stride):
        nb = ctypes.c_size_t()
        assert L.gigaam_rnnt_workspace_bytes(h, batch, stride, ctypes.byref(nb)) == 0
        return nb.value

    def al(x):
        return (x + 255) // 256 * 256
    P, J, C = cfg["pred_hidden"], cfg["joint_hidden"], cfg["n_classes"]
    Cp = (C + 7) // 8 * 8
    # clusters: clips in groups of 8 (one per XCD), (groups * 8) * G <= 2 x 256 CUs, G <= 64
    for batch, stride, gmax in ((32, 100, 16), (6, 40, 64), (1, 10, 64), (9, 10, 32), (256, 20, 2)):
        base = al(batch * stride * J * 4) + al(C * 4 * P * 4)
        xch = al((batch * 2 * (gmax * Cp + P) + batch * gmax) * 8) if gmax > 1 else 0
        assert ws(batch, stride) == base + xch, (batch, gmax)
    L.gigaam_rnnt_destroy(h)
