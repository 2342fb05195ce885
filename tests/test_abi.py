"""CPU-side checks of the C ABI: the library loads and exports every declared symbol,
host arithmetic, configuration and argument validation (no GPU work is issued), and
the host weight repacking against independent NumPy conversions."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gigaam.h")


@pytest.fixture(scope="module")
def gg():
    import conformer_speech_recognition_amd as g
    if not os.path.exists(g.LIB_PATH):
        from conformer_speech_recognition_amd.build import build
        build()
    g.lib()
    return g


def test_every_declared_symbol_is_exported(gg):
    decl = set(re.findall(r"\b(gigaam_[a-z_]+)\s*\(", open(HEADER).read()))
    assert len(decl) >= 15
    L = ctypes.CDLL(gg.LIB_PATH)
    missing = [n for n in sorted(decl) if not hasattr(L, n)]
    assert not missing, missing
    assert set(gg._SIGNATURES) == decl


def test_frames_host_arithmetic(gg):
    assert gg.frames(16000) == (99, 50, 25)
    assert gg.frames(320000) == (1999, 1000, 500)
    assert gg.frames(480000) == (2999, 1500, 750)
    assert gg.frames(320) == (1, 1, 1)
    with pytest.raises(gg.GigaamError) as e:
        gg.frames(319)
    assert e.value.code == gg.E_INVAL and "320" in str(e.value)


@pytest.mark.parametrize("field,value,code", [
    ("d_model", 512, -3), ("n_heads", 8, -3), ("conv_kernel", 7, -3), ("n_fft", 512, -3),
    ("n_classes", 1, -1), ("n_layers", 0, -1), ("dtype", 9, -1), ("ln_eps", 0.0, -1),
    ("d_ff", 3000, -3)])
def test_config_validation(gg, field, value, code):
    cfg = synth.workload_config("tiny")
    c = gg.make_config(cfg)
    assert gg.lib().gigaam_check_config(ctypes.byref(c)) == 0
    setattr(c, field, value)
    assert gg.lib().gigaam_check_config(ctypes.byref(c)) == code


@pytest.mark.parametrize("name", ["tiny", "batch32", "ml_long", "int8_b64", "int6_b64", "int4_b64"])
def test_canonical_names_cover_checkpoint(gg, name):
    cfg = synth.workload_config(name)
    ents = gg.canonical_entries(cfg)
    names = {n: s for n, s, _ in ents}
    want = {n: s for n, s, _ in synth.canonical_entries(cfg)}
    if cfg["dtype"] in synth.QUANT_BITS:
        for n in list(want):
            base = n[: -len(".weight")]
            if n.endswith(".weight") and base.endswith(synth.QUANTIZED_SUFFIXES):
                N, K = want.pop(n)
                want[base + ".weight_q"] = (N, K)
                want[base + ".weight_scale"] = (N, K // 64)
    assert names == want
    offs = [o for _, _, o in ents]
    assert offs == sorted(offs) and offs[0] == 0


def _small(dtype):
    cfg = synth.model_config(1, 768, 16, 256, 5, 10, dtype)
    return cfg, synth.make_weights(cfg, 7)


def _packed_views(gg, cfg, packed):
    """Offsets of the packed blob follow the same 256-byte aligned order as the library's
    layout; recomputed here from the documented order for the first tensors."""
    d, m = cfg["d_model"], 64
    es = 4 if cfg["dtype"] == "f32" else 2
    al = lambda x: (x + 255) // 256 * 256
    off_conv1 = 0
    off_conv1_b = al(d * 5 * m * es)
    return off_conv1, off_conv1_b


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_pack_conv1_transpose_and_rounding(gg, dtype):
    cfg, w = _small(dtype)
    packed = gg.pack_weights(cfg, w)
    o_w, o_b = _packed_views(gg, cfg, packed)
    d = cfg["d_model"]
    if dtype == "f32":
        got = packed[o_w: o_w + d * 5 * 64 * 4].view(np.float32).reshape(d, 5, 64)
    elif dtype == "f16":
        got = packed[o_w: o_w + d * 5 * 64 * 2].view(np.float16).astype(np.float32).reshape(d, 5, 64)
    else:
        raw = packed[o_w: o_w + d * 5 * 64 * 2].view(np.uint16).astype(np.uint32) << 16
        got = raw.view(np.float32).reshape(d, 5, 64)
    want = np.transpose(w["pre.conv1.weight"], (0, 2, 1))        # [out, in, K] -> [out, K, in]
    np.testing.assert_array_equal(got, want)
    bias = packed[o_b: o_b + d * 4].view(np.float32)
    np.testing.assert_array_equal(bias, w["pre.conv1.bias"])


def test_pack_rounds_like_numpy(gg):
    """Host fp16 rounding of an arbitrary (not pre-rounded) checkpoint equals numpy's."""
    cfg, w = _small("f16")
    rng = np.random.default_rng(0)
    w = dict(w)
    w["pre.conv1.weight"] = (rng.standard_normal((768, 64, 5)) * np.exp(rng.uniform(-20, 12, (768, 64, 5)))
                             ).astype(np.float32)
    packed = gg.pack_weights(cfg, w)
    got = packed[: 768 * 5 * 64 * 2].view(np.float16).reshape(768, 5, 64)
    with np.errstate(over="ignore"):
        want = np.transpose(w["pre.conv1.weight"], (0, 2, 1)).astype(np.float16)
    np.testing.assert_array_equal(got.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("dtype,bits", [("w8f16", 8), ("w6f16", 6), ("w4f16", 4)])
def test_pack_quantised_rows_bit_layout(gg, dtype, bits):
    """Packed linear rows hold weight k at bits [k*b, k*b+b) of the row's little-endian bit
    string (two's complement) with fp16 scales after them, as the header documents;
    checked on layer 0's first FFN linear by unpacking with numpy."""
    cfg = synth.model_config(1, 768, 16, 256, 5, 10, dtype)
    w = synth.make_weights(cfg, 3)
    packed = gg.pack_weights(cfg, w)
    d, f = 768, 256
    al = lambda x: (x + 255) // 256 * 256
    off = 0
    for nbytes in (d * 5 * 64 * 2, d * 4, d * 5 * d * 2, d * 4, d * 4, d * 4):
        off = al(off + nbytes)                  # conv1 w/b, conv2 w/b, ff1 norm g/b
    rowb = d * bits // 8
    rows = packed[off: off + f * rowb].reshape(f, rowb)
    bitsarr = np.unpackbits(rows, axis=1, bitorder="little")[:, : d * bits].reshape(f, d, bits)
    u = (bitsarr.astype(np.int64) << np.arange(bits)).sum(axis=2)
    q = np.where(u >= 1 << (bits - 1), u - (1 << bits), u)
    np.testing.assert_array_equal(q, w["layers.0.ff1.linear1.weight_q"])
    so = al(off + f * rowb)
    sc = packed[so: so + f * (d // 64) * 2].view(np.float16).reshape(f, d // 64)
    np.testing.assert_array_equal(sc, w["layers.0.ff1.linear1.weight_scale"])


@pytest.mark.parametrize("dtype,bad", [("w6f16", 32.0), ("w4f16", 8.0), ("w4f16", -8.0),
                                       ("w4f16", 2.5)])
def test_pack_rejects_out_of_range_low_bit(gg, dtype, bad):
    cfg = synth.model_config(1, 768, 16, 256, 5, 10, dtype)
    w = synth.make_weights(cfg, 3)
    gg.pack_weights(cfg, w)
    q = w["layers.0.ff2.linear2.weight_q"].astype(np.float32).copy()
    q[3, 5] = bad
    with pytest.raises(gg.GigaamError):
        gg.pack_weights(cfg, dict(w, **{"layers.0.ff2.linear2.weight_q": q}))


def test_pack_rejects_bad_int8(gg):
    cfg = synth.model_config(1, 768, 16, 256, 5, 10, "w8f16")
    w = synth.make_weights(cfg, 3)
    gg.pack_weights(cfg, w)
    bad = dict(w)
    q = w["layers.0.ff1.linear1.weight_q"].astype(np.float32).copy()
    q[0, 0] = 200.0
    bad["layers.0.ff1.linear1.weight_q"] = q
    with pytest.raises(gg.GigaamError):
        gg.pack_weights(cfg, bad)


def test_encode_argument_errors_before_any_launch(gg):
    """Validation fails before the first GPU call: works without a GPU."""
    L = gg.lib()
    cfg = synth.workload_config("tiny")
    c = gg.make_config(cfg)
    h = ctypes.c_void_p()
    fake = 1 << 20                      # aligned, never dereferenced on these paths
    assert L.gigaam_create(ctypes.byref(c), fake, fake, fake, ctypes.byref(h)) == 0
    nb = ctypes.c_size_t()
    assert L.gigaam_workspace_bytes(h, 2, 32000, ctypes.byref(nb)) == 0 and nb.value > 0
    assert L.gigaam_workspace_bytes(h, 0, 32000, ctypes.byref(nb)) == gg.E_INVAL
    lens = (ctypes.c_int32 * 2)(32000, 16000)
    I = ctypes.c_int32

    def enc(batch=2, stride=32000, lengths=lens, ws=fake, wsb=nb.value, outs=fake):
        return L.gigaam_encode(h, fake, lengths, batch, stride, ws, wsb, outs, outs, outs, None, None,
                               None, None)
    assert enc(batch=0) == gg.E_INVAL
    assert enc(batch=gg.MAX_BATCH + 1) == gg.E_INVAL
    assert enc(stride=100) == gg.E_INVAL
    assert enc(lengths=(I * 2)(32000, 300)) == gg.E_INVAL
    assert "lengths[1]" in L.gigaam_last_error().decode()
    assert enc(lengths=(I * 2)(32000, 40000)) == gg.E_INVAL      # longer than the stride
    assert enc(wsb=nb.value - 1) == gg.E_WORKSPACE
    assert enc(ws=fake + 8) == gg.E_INVAL                        # misaligned workspace
    assert enc(outs=None) == gg.E_INVAL
    out = ctypes.c_void_p(fake)
    assert L.gigaam_encode_stage(h, fake, lens, 2, 32000, fake, nb.value, 99, out, 10, None) == gg.E_INVAL
    assert L.gigaam_encode_stage(h, fake, lens, 2, 32000, fake, nb.value, 0, out, 10, None) == gg.E_INVAL
    L.gigaam_destroy(h)
    assert L.gigaam_create(ctypes.byref(c), fake + 4, fake, fake, ctypes.byref(h)) == gg.E_INVAL
    assert L.gigaam_debug_gemm(1, 4, 4, 100, fake, fake, None, None, fake, None, 0, None, None) == gg.E_INVAL
    assert L.gigaam_debug_gemm(1, 4, 4, 128, fake, fake, None, None, fake, fake + 4, 64, None,
                               None) == gg.E_INVAL                  # misaligned partial buffer
    for i in range(3):                                  # A, W, C move 16 bytes at a time
        ptrs = [fake, fake, fake]
        ptrs[i] = fake + 4
        assert L.gigaam_debug_gemm(1, 4, 4, 128, ptrs[0], ptrs[1], None, None, ptrs[2], None, 0, None,
                                   None) == gg.E_INVAL
    F = ctypes.c_float
    big = 1 << 26
    # fused FFN: fp32 dtype, unsupported width, too many rows, short scratch, NULL, misaligned
    assert L.gigaam_debug_mlp(0, 64, 768, 3072, fake, fake, None, fake, None, F(0.5), fake, fake, big, None) == gg.E_INVAL
    assert L.gigaam_debug_mlp(1, 64, 512, 3072, fake, fake, None, fake, None, F(0.5), fake, fake, big, None) == gg.E_INVAL
    assert L.gigaam_debug_mlp(1, 897, 768, 3072, fake, fake, None, fake, None, F(0.5), fake, fake, big, None) == gg.E_INVAL
    assert L.gigaam_debug_mlp(1, 64, 768, 3000, fake, fake, None, fake, None, F(0.5), fake, fake, big, None) == gg.E_INVAL
    assert L.gigaam_debug_mlp(1, 64, 768, 3072, fake, fake, None, fake, None, F(0.5), fake, fake,
                              12 * 64 * 768 - 1, None) == gg.E_INVAL
    assert L.gigaam_debug_mlp(1, 64, 768, 3072, None, fake, None, fake, None, F(0.5), fake, fake, big, None) == gg.E_INVAL
    assert L.gigaam_debug_mlp(1, 64, 768, 3072, fake, fake, None, fake, None, F(0.5), fake, fake + 4, big,
                              None) == gg.E_INVAL
    for i in range(3):                                  # y, W1, W2 read 16 bytes at a time
        ptrs = [fake, fake, fake]
        ptrs[i] = fake + 2
        assert L.gigaam_debug_mlp(1, 64, 768, 3072, ptrs[0], ptrs[1], None, ptrs[2], None, F(0.5), fake,
                                  fake, big, None) == gg.E_INVAL


def test_debug_attention_rejects_misaligned_operands(gg):
    """The attention kernel moves 16 bytes per access: q/k/v and out pointers that are not
    16-byte aligned are refused before the launch (no GPU needed)."""
    L = gg.lib()
    fake = 1 << 20
    frames = (ctypes.c_int32 * 2)(70, 5)
    ok = 1 << 16
    for qkv, out in ((fake + 2, fake), (fake, fake + 8), (fake + 4, fake + 4)):
        assert L.gigaam_debug_attention(1, 768, 16, 2, frames, qkv, out, fake, ok, None) == gg.E_INVAL
        assert "aligned" in L.gigaam_last_error().decode()
    assert L.gigaam_debug_attention(1, 768, 16, 2, frames, fake, fake, fake + 16, ok, None) == gg.E_INVAL


def test_workspace_bound_covers_every_length_mix(gg):
    L = gg.lib()
    c = gg.make_config(synth.workload_config("batch32"))
    h = ctypes.c_void_p()
    assert L.gigaam_create(ctypes.byref(c), 1 << 20, 1 << 20, 1 << 20, ctypes.byref(h)) == 0
    nb = ctypes.c_size_t()
    assert L.gigaam_workspace_bytes(h, 32, 320000, ctypes.byref(nb)) == 0
    big = nb.value
    assert L.gigaam_workspace_bytes(h, 32, 16000, ctypes.byref(nb)) == 0
    assert nb.value < big
    L.gigaam_destroy(h)


def test_debug_gemm_role_validation(gg):
    """Mode, epilogue, shape and alignment checks of the role entry happen before any
    launch (no GPU needed)."""
    L = gg.lib()
    fake = 1 << 20
    F = ctypes.c_float

    def call(dt=1, am=0, ep=1, M=64, N=256, K=128, A=fake, A2=None, ns=0, W=fake, C=fake, part=None, req=0):
        return L.gigaam_debug_gemm_role(dt, am, ep, M, N, K, A, A2, ns, W, None, None, F(1.0), C, part,
                                        0, req, None, None, None)
    assert call(dt=9) == gg.E_INVAL
    assert call(am=1) == gg.E_INVAL                      # not a role mode
    assert call(ep=3) == gg.E_INVAL                      # not a role epilogue
    assert call(K=100) == gg.E_INVAL
    assert call(N=250) == gg.E_INVAL
    assert call(am=2, ep=0, A2=None, ns=128) == gg.E_INVAL          # dual without A2
    assert call(am=2, ep=0, A2=fake, ns=100) == gg.E_INVAL          # split not 128-aligned
    assert call(am=2, ep=0, A2=fake, ns=256) == gg.E_INVAL          # split not inside N
    assert call(am=2, ep=1, A2=fake, ns=128) == gg.E_INVAL          # dual stores only
    assert call(am=2, ep=0, A2=fake + 8, ns=128) == gg.E_INVAL      # misaligned A2
    assert call(ep=4, N=96) == gg.E_INVAL                           # GLU needs 64-row groups
    assert call(A=fake + 2) == gg.E_INVAL and call(W=fake + 2) == gg.E_INVAL and call(C=fake + 4) == gg.E_INVAL
    assert call(part=fake + 4) == gg.E_INVAL
    assert call(dt=3) == gg.E_INVAL                                  # quantised weights need scales
    assert call(req=2) == gg.E_INVAL                                 # not a direct-load variant
    assert call(req=12) == gg.E_INVAL
    assert call(dt=0, req=3) == gg.E_INVAL                           # fp32 runs the register path
    assert call(ep=4, N=384, req=7) == gg.E_INVAL                    # 256x192: no GLU pairs
    assert call(am=2, ep=0, A2=fake, ns=128, N=512, req=3) == gg.E_INVAL   # split inside a tile


def test_noalloc_entry_validates_before_touching_the_gpu(gg):
    """gigaam_encode_noalloc: bad lengths and batches larger than its fixed scratch are
    refused before any device call (works without a GPU); the scratch size in the header
    is the binding's."""
    hdr = open(HEADER).read()
    m = re.search(r"#define GIGAAM_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == gg.NOALLOC_SCRATCH_BYTES
    L = gg.lib()
    c = gg.make_config(synth.workload_config("v3_20s"))
    h = ctypes.c_void_p()
    fake = 1 << 20
    assert L.gigaam_create(ctypes.byref(c), fake, fake, fake, ctypes.byref(h)) == 0
    I = ctypes.c_int32

    def call(lengths, stride=320000):
        n = len(lengths)
        return L.gigaam_encode_noalloc(h, fake, (I * n)(*lengths), n, stride, fake, fake, fake, None, None,
                                       None, None)
    assert call([320000, 100]) == gg.E_INVAL
    assert call([320001]) == gg.E_INVAL                                    # past the stride
    assert call([320000] * 8) == gg.E_WORKSPACE                            # > 64 MiB of workspace
    assert "scratch" in L.gigaam_last_error().decode()
    nb = ctypes.c_size_t()
    assert L.gigaam_workspace_bytes(h, 1, 480000, ctypes.byref(nb)) == 0
    assert nb.value <= gg.NOALLOC_SCRATCH_BYTES                            # one 30 s clip fits
    assert L.gigaam_workspace_bytes(h, 256, 2 ** 31 - 1, ctypes.byref(nb)) == gg.E_INVAL
    L.gigaam_destroy(h)
