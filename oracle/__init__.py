"""CPU ORACLE for the GigaAM-style Conformer CTC encoder forward pass.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The HIP product path never imports, calls
or links it, and it shares no code, tables or constants-generators with that path.

Plain, slow, obviously-correct definitions in float64 NumPy (``dtype`` switch for a
float32 self-check), one clip at a time. Each function names the page passage it
follows; pages are cited by title and section:

  [MLX-blog]   "GigaAM on MLX: the transcripts matched, but the model was broken"
  [RNNT-card]  "GigaAM v3 RNNT - MLX (Apple Silicon)" model card, "Notes for other runtimes"
  [ML-port]    "GigaAM MLX port for Mac" (English) / its Russian twin
  [v3-card]    "GigaAM v3 MLX" model card (Frontend configuration / Architecture details)

Readings adopted where the pages are silent (each also listed in the design notes):
  periodic Hann window; HTK mel on [0, 8000] Hz without normalisation; natural log;
  no feature normalisation; Conv1d subsampling k5 s2 padding 2 with ReLU after each
  conv; textbook macaron Conformer block (pre-LN, half-step FFNs, final LN) with LN/BN
  eps 1e-5; attention scale 1/sqrt(d_k); rotate_half = [-v2, v1]; GLU = a * sigmoid(g)
  with a the first half; CTC collapse merges repeats then drops blanks; argmax takes
  the lowest index on ties and is decided on float32 logits (the precision of the
  pages' reference model and of the kernels).

Parity pins for every function live in tests/test_oracle_*.py.
"""
from __future__ import annotations

import numpy as np

SAMPLE_RATE = 16000

# ==================================================================================
# shapes
# ==================================================================================

def num_frames(n_samples: int, win: int = 320, hop: int = 160) -> int:
    """Frames of an un-centred STFT: floor((L - win)/hop) + 1 ([v3-card] Frontend
    configuration: window 320, hop 160, center false). L < win has no frame."""
    if n_samples < win:
        raise ValueError("clip shorter than one analysis window")
    return (n_samples - win) // hop + 1


def conv_out_len(n_in: int, kernel: int = 5, stride: int = 2, pad: int = 2) -> int:
    """Output length of a Conv1d: floor((n + 2p - k)/s) + 1."""
    return (n_in + 2 * pad - kernel) // stride + 1


def encoder_frames(n_samples: int) -> tuple[int, int, int]:
    """(mel frames T, after first conv S, encoder frames U); 4x fewer frames after the
    two stride-2 Conv1d ([MLX-blog] "What we're porting")."""
    T = num_frames(n_samples)
    S = conv_out_len(T)
    U = conv_out_len(S)
    return T, S, U


# ==================================================================================
# frontend  ([v3-card] Frontend configuration; [RNNT-card] Notes for other runtimes)
# ==================================================================================

def hann_periodic(n: int = 320, dtype=np.float64) -> np.ndarray:
    """Periodic Hann window w[i] = 0.5 - 0.5 cos(2 pi i / n) (the STFT window buffer)."""
    i = np.arange(n, dtype=np.float64)
    return (0.5 - 0.5 * np.cos(2.0 * np.pi * i / n)).astype(dtype)


def frame_signal(pcm: np.ndarray, win: int = 320, hop: int = 160) -> np.ndarray:
    """Frame t = pcm[hop*t : hop*t + win] for t < T; no centring or padding, tail dropped."""
    T = num_frames(len(pcm), win, hop)
    idx = hop * np.arange(T)[:, None] + np.arange(win)[None, :]
    return pcm[idx]


def dft_power(frames: np.ndarray, n_fft: int = 320) -> np.ndarray:
    """Power spectrum (power 2.0) of real frames: |sum_n x[n] e^{-2 pi i k n / N}|^2 for
    k = 0..N/2, written out with an explicit cos/sin basis (no FFT)."""
    n = np.arange(n_fft, dtype=np.float64)
    k = np.arange(n_fft // 2 + 1, dtype=np.float64)
    ang = 2.0 * np.pi * np.outer(n, k) / n_fft            # [N, K]
    cos_b = np.cos(ang).astype(frames.dtype)
    sin_b = np.sin(ang).astype(frames.dtype)
    re = frames @ cos_b
    im = -(frames @ sin_b)
    return re * re + im * im


def hz_to_mel_htk(f):
    """HTK mel scale m = 2595 log10(1 + f/700) ([v3-card] 'Mel scale: HTK')."""
    return 2595.0 * np.log10(1.0 + np.asarray(f, dtype=np.float64) / 700.0)


def mel_to_hz_htk(m):
    return 700.0 * (10.0 ** (np.asarray(m, dtype=np.float64) / 2595.0) - 1.0)


def htk_mel_filterbank(n_freqs: int = 161, n_mels: int = 64, sample_rate: int = 16000,
                       f_min: float = 0.0, f_max: float = 8000.0) -> np.ndarray:
    """Triangular HTK filterbank [n_freqs, n_mels] with no area normalisation
    ([v3-card] 'Mel normalization: none'). Bin k sits at k * sr / n_fft Hz; filter m
    rises from corner p_m to p_{m+1} and falls to p_{m+2}, with the n_mels + 2 corners
    equally spaced on the mel scale between f_min and f_max."""
    f = np.linspace(0.0, sample_rate / 2.0, n_freqs)
    corners = mel_to_hz_htk(np.linspace(hz_to_mel_htk(f_min), hz_to_mel_htk(f_max), n_mels + 2))
    fb = np.zeros((n_freqs, n_mels), dtype=np.float64)
    for m in range(n_mels):
        lo, mid, hi = corners[m], corners[m + 1], corners[m + 2]
        up = (f - lo) / (mid - lo)
        down = (hi - f) / (hi - mid)
        fb[:, m] = np.maximum(0.0, np.minimum(up, down))
    return fb


def log_mel(pcm: np.ndarray, window: np.ndarray | None = None, fb: np.ndarray | None = None,
            dtype=np.float64) -> np.ndarray:
    """Log-mel features [T, 64]: frame, window, power spectrum, mel projection, then
    log(clip(x, 1e-9, 1e9)) with the natural log ([RNNT-card] Notes for other runtimes)."""
    window = hann_periodic(320) if window is None else np.asarray(window, dtype=np.float64)
    fb = htk_mel_filterbank() if fb is None else np.asarray(fb, dtype=np.float64)
    frames = frame_signal(np.asarray(pcm, dtype=dtype)) * window.astype(dtype)[None, :]
    power = dft_power(frames)
    mel = power @ fb.astype(dtype)
    return np.log(np.clip(mel, 1e-9, 1e9))


# ==================================================================================
# generic layers
# ==================================================================================

def conv1d(x: np.ndarray, w: np.ndarray, b: np.ndarray | None, stride: int = 1,
           pad: int = 0, groups: int = 1) -> np.ndarray:
    """Cross-correlation Conv1d on a time-major input x [T, C_in] with PyTorch weight
    layout w [C_out, C_in/groups, K]; zero padding of ``pad`` frames on both sides.
    out[s, o] = b[o] + sum_{c, j} w[o, c, j] * x_pad[stride*s + j, group(o)*cg + c]."""
    T, Cin = x.shape
    Cout, cg, K = w.shape
    xp = np.zeros((T + 2 * pad, Cin), dtype=x.dtype)
    xp[pad:pad + T] = x
    S = (T + 2 * pad - K) // stride + 1
    out = np.zeros((S, Cout), dtype=x.dtype)
    og = Cout // groups
    for j in range(K):
        rows = xp[j: j + stride * (S - 1) + 1: stride]        # [S, Cin]
        if groups == 1:
            out += rows @ w[:, :, j].T
        else:
            for g in range(groups):
                out[:, g * og:(g + 1) * og] += rows[:, g * cg:(g + 1) * cg] @ w[g * og:(g + 1) * og, :, j].T
    if b is not None:
        out += b[None, :]
    return out


def depthwise_conv1d(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Depthwise ('same' padding, odd K) Conv1d: out[t, c] = b[c] + sum_j w[c, j] x[t + j - (K-1)/2, c],
    x = 0 outside the clip. w is [C, K]."""
    T, C = x.shape
    K = w.shape[1]
    p = (K - 1) // 2
    xp = np.zeros((T + 2 * p, C), dtype=x.dtype)
    xp[p:p + T] = x
    out = np.zeros_like(x)
    for j in range(K):
        out += xp[j:j + T] * w[None, :, j]
    return out + b[None, :]


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """LayerNorm over the last axis with biased variance."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def batch_norm_inference(x, g, b, mean, var, eps: float = 1e-5):
    """BatchNorm1d with running statistics (inference), per channel (last axis)."""
    return (x - mean) / np.sqrt(var + eps) * g + b


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    return x * sigmoid(x)


def relu(x):
    return np.maximum(x, 0.0)


def glu(x: np.ndarray) -> np.ndarray:
    """GLU over channels: first half times sigmoid of the second half."""
    h = x.shape[-1] // 2
    return x[..., :h] * sigmoid(x[..., h:])


def linear(x, w, b):
    return x @ w.T + b


# ==================================================================================
# rotary positions ([MLX-blog] "Trap 1" and "Trap 2"; [RNNT-card] Notes)
# ==================================================================================

def rope_tables(n_pos: int, d_k: int, base: float = 5000.0, dtype=np.float64):
    """cos/sin tables [n_pos, d_k]: angle(t, i) = t * base^(-2 (i mod d_k/2) / d_k),
    halves concatenated; dim = d_model // n_heads and base = 5000 (the positional
    module's second positional argument is its base, which receives 5000)."""
    half = d_k // 2
    inv_freq = base ** (-(2.0 * np.arange(half, dtype=np.float64)) / d_k)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    ang = np.concatenate([ang, ang], axis=1)
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rotate_half(v: np.ndarray) -> np.ndarray:
    """[v1, v2] -> [-v2, v1] over the last axis."""
    h = v.shape[-1] // 2
    return np.concatenate([-v[..., h:], v[..., :h]], axis=-1)


def apply_rope(y: np.ndarray, n_heads: int, base: float = 5000.0) -> np.ndarray:
    """Rotate the raw per-head input: y split into heads [T, H, d_k], then
    y * cos + rotate_half(y) * sin with positions 0..T-1 (offset 0)."""
    T, d = y.shape
    dk = d // n_heads
    cos, sin = rope_tables(T, dk, base, y.dtype)
    yh = y.reshape(T, n_heads, dk)
    r = yh * cos[:, None, :] + rotate_half(yh) * sin[:, None, :]
    return r.reshape(T, d)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_heads: int,
              key_valid: int | None = None) -> np.ndarray:
    """Scaled dot-product self-attention per head: softmax(q k^T / sqrt(d_k)) v, with
    keys at index >= key_valid masked out (key-padding mask)."""
    T, d = q.shape
    dk = d // n_heads
    if key_valid is not None:
        k, v = k[:key_valid], v[:key_valid]          # masked keys take no part at all
    out = np.zeros_like(q)
    for h in range(n_heads):
        sl = slice(h * dk, (h + 1) * dk)
        s = q[:, sl] @ k[:, sl].T / np.sqrt(dk)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, sl] = p @ v[:, sl]
    return out


def mhsa_rope(y: np.ndarray, P: dict, pre: str, n_heads: int, base: float) -> np.ndarray:
    """Rotary self-attention with the rotation applied BEFORE the projections:
    q = linear_q(rope(y)), k = linear_k(rope(y)), v = linear_v(y) (value not rotated),
    then attention and linear_out ([MLX-blog] "Trap 2")."""
    r = apply_rope(y, n_heads, base)
    q = linear(r, P[pre + "linear_q.weight"], P[pre + "linear_q.bias"])
    k = linear(r, P[pre + "linear_k.weight"], P[pre + "linear_k.bias"])
    v = linear(y, P[pre + "linear_v.weight"], P[pre + "linear_v.bias"])
    o = attention(q, k, v, n_heads)
    return linear(o, P[pre + "linear_out.weight"], P[pre + "linear_out.bias"])


# ==================================================================================
# Conformer block ([ML-port] "What is inside the model": FFN, attention, conv, FFN)
# ==================================================================================

def ffn_body(y, P, pre):
    """The feed-forward module after its norm: linear2(SiLU(linear1(y)))."""
    h = silu(linear(y, P[pre + "linear1.weight"], P[pre + "linear1.bias"]))
    return linear(h, P[pre + "linear2.weight"], P[pre + "linear2.bias"])


def feed_forward(x, P, pre, eps):
    """Macaron FFN on the pre-normed input: linear2(SiLU(linear1(LN(x))))."""
    return ffn_body(layer_norm(x, P[pre + "norm.weight"], P[pre + "norm.bias"], eps), P, pre)


def conv_module(x, P, pre, eps, bn_eps):
    """LN -> pointwise d->2d -> GLU -> depthwise conv (zero outside the clip) ->
    BatchNorm (running stats) -> SiLU -> pointwise d->d."""
    y = layer_norm(x, P[pre + "norm.weight"], P[pre + "norm.bias"], eps)
    a = glu(linear(y, P[pre + "pointwise1.weight"], P[pre + "pointwise1.bias"]))
    c = depthwise_conv1d(a, P[pre + "depthwise.weight"], P[pre + "depthwise.bias"])
    c = batch_norm_inference(c, P[pre + "bn.weight"], P[pre + "bn.bias"],
                             P[pre + "bn.running_mean"], P[pre + "bn.running_var"], bn_eps)
    return linear(silu(c), P[pre + "pointwise2.weight"], P[pre + "pointwise2.bias"])


def conformer_block(x, P, i, cfg):
    p = f"layers.{i}."
    eps, bn_eps = cfg["ln_eps"], cfg["bn_eps"]
    x = x + 0.5 * feed_forward(x, P, p + "ff1.", eps)
    y = layer_norm(x, P[p + "att.norm.weight"], P[p + "att.norm.bias"], eps)
    x = x + mhsa_rope(y, P, p + "att.", cfg["n_heads"], cfg["rope_base"])
    x = x + conv_module(x, P, p + "conv.", eps, bn_eps)
    x = x + 0.5 * feed_forward(x, P, p + "ff2.", eps)
    return layer_norm(x, P[p + "norm_out.weight"], P[p + "norm_out.bias"], eps)


# ==================================================================================
# subsampling, head, decoding
# ==================================================================================

def subsample(mel: np.ndarray, P: dict) -> np.ndarray:
    """Two Conv1d (kernel 5, stride 2, padding 2), ReLU after each: [T, 64] -> [U, d]
    ([MLX-blog] "What we're porting": two stride-2 Conv1d, 4x fewer frames)."""
    h = relu(conv1d(mel, P["pre.conv1.weight"], P["pre.conv1.bias"], stride=2, pad=2))
    return relu(conv1d(h, P["pre.conv2.weight"], P["pre.conv2.bias"], stride=2, pad=2))


def ctc_log_probs(x, P):
    """Per-frame linear to C classes, then log-softmax: z - logsumexp(z)."""
    z = linear(x, P["head.weight"], P["head.bias"])
    m = z.max(axis=1, keepdims=True)
    return z - (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))


def greedy_ids(log_probs: np.ndarray) -> np.ndarray:
    """Per-frame argmax, lowest index on ties, decided in float32."""
    return np.argmax(np.asarray(log_probs, dtype=np.float32), axis=1).astype(np.int32)


def ctc_collapse(ids, blank: int) -> list[int]:
    """Greedy CTC: merge runs of equal ids, then remove blanks (blank = vocabulary
    size, i.e. the last class; [RNNT-card] 'blank = len(vocabulary)')."""
    out, prev = [], None
    for t in ids:
        t = int(t)
        if t != prev and t != blank:
            out.append(t)
        prev = t
    return out


# ==================================================================================
# weights and the whole encoder
# ==================================================================================

def dequantize_g64(q: np.ndarray, s: np.ndarray, group: int = 64) -> np.ndarray:
    """w[n, k] = q[n, k] * s[n, k // 64] (one shared scale per group of 64 weights, for
    the INT8, INT6 and INT4 variants alike; [ML-port] "How precision affects size and
    speed")."""
    q = np.asarray(q, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    return q * np.repeat(s, group, axis=1)


dequantize_int8_g64 = dequantize_g64


def materialize(weights: dict, dtype=np.float64) -> dict:
    """Cast the checkpoint to the compute dtype; quantised linears are dequantized."""
    P = {}
    for name, a in weights.items():
        if name.endswith(".weight_scale"):
            continue
        if name.endswith(".weight_q"):
            base = name[: -len(".weight_q")]
            P[base + ".weight"] = dequantize_g64(a, weights[base + ".weight_scale"]).astype(dtype)
        else:
            P[name] = np.asarray(a, dtype=dtype)
    return P


def encode_clip(pcm: np.ndarray, weights: dict, cfg: dict, dtype=np.float64,
                taps: bool = False, P: dict | None = None) -> dict:
    """The whole forward for ONE clip (its valid samples only):
    log-mel -> subsampling -> N Conformer blocks -> CTC log-probs -> greedy ids -> tokens.
    Returns a dict with 'log_probs' [U, C], 'enc_out' [U, d], 'ids' [U], 'tokens',
    and with ``taps`` also 'mel' [T, 64], 'sub' [U, d], 'layers' (list of [U, d])."""
    P = materialize(weights, dtype) if P is None else P
    mel = log_mel(np.asarray(pcm, dtype=np.float64), dtype=dtype)
    x = subsample(mel, P)
    layers = []
    sub = x
    for i in range(cfg["n_layers"]):
        x = conformer_block(x, P, i, cfg)
        if taps:
            layers.append(x)
    lp = ctc_log_probs(x, P)
    ids = greedy_ids(lp)
    out = dict(log_probs=lp, enc_out=x, ids=ids,
               tokens=ctc_collapse(ids, cfg["n_classes"] - 1))
    if taps:
        out.update(mel=mel, sub=sub, layers=layers)
    return out


def encode_batch(pcm: np.ndarray, lengths, weights: dict, cfg: dict, dtype=np.float64,
                 clips=None) -> list[dict]:
    """Padded batch semantics: clip b's result is the per-clip forward on its first
    lengths[b] samples (padding never reaches a valid output)."""
    P = materialize(weights, dtype)
    idx = range(len(lengths)) if clips is None else clips
    return [encode_clip(pcm[b, : int(lengths[b])], weights, cfg, dtype, P=P) for b in idx]
