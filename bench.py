#!/usr/bin/env python3
"""Throughput of the gfx950 Conformer CTC encoder: encoder audio-seconds per second
(x realtime) on one GPU, with the fraction of the fp16 MFMA roofline.

One step = one gigaam_encode call over the whole workload batch: log-mel frontend,
subsampling, all Conformer blocks, CTC log-softmax, argmax and greedy collapse. The PCM
is already resident in HBM when the timed region starts. Inputs and weights are
synthetic (seeded), with the shapes of the workload.

Prints ONE JSON line. Besides the throughput it carries
  roofline      the dominant kernel's algorithmic FLOPs (or bytes) per launch divided by
                its average launch time, measured here with HIP events recorded around
                each launch on the encode stream (library profiler), against the MI355X
                dense peak of its operand type;
  cpu_baseline  the CPU oracle (its float32 mode) timed on a bounded sample of the same
                workload on this host (1 warm-up + median of 3 passes).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "w8f16": 2516.6, "w6f16": 2516.6, "w4f16": 2516.6,
               "f32": 157.3}   # dense MFMA (the quantised dtypes multiply in fp16)
PEAK_HBM_GBS = 8000.0

# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch) on this
# bench, scaled by what the counters read for a plain copy of known size; valid only while the
# kernel's source is the one the counters were taken on (sha256 prefix)
GEMM_SRC = ("conformer_speech_recognition_amd/csrc/gemm.hip", "0f1b9c1355c4f2b5")
ATTN_SRC = ("conformer_speech_recognition_amd/csrc/attention.hip", "63c0dbdc5eeb1b81")
TRAFFIC_KIB = {("batch32", "gemm.ffn_up"): (GEMM_SRC, 41511, 49242),
               ("batch32", "gemm.ffn_down"): (GEMM_SRC, 83898, 24621),
               ("batch32", "gemm.qkv"): (GEMM_SRC, 43963, 36932),
               ("batch32", "gemm.pw1_glu"): (GEMM_SRC, 21270, 12310),
               ("batch32", "gemm.out_proj"): (GEMM_SRC, 25743, 24621),
               ("batch32", "gemm.pw2"): (GEMM_SRC, 25743, 24621),
               ("batch32", "gemm.conv2"): (GEMM_SRC, 89304, 24621),
               ("batch32", "gemm.conv1"): (GEMM_SRC, 4534, 24597),
               ("batch32", "attention"): (ATTN_SRC, 28768, 14400)}
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0


def measured_traffic(workload: str, kernel: str):
    import hashlib
    if (workload, kernel) not in TRAFFIC_KIB:
        return None
    (src, digest), f, w = TRAFFIC_KIB[(workload, kernel)]
    path = os.path.join(ROOT, src)
    if not os.path.exists(path) or hashlib.sha256(open(path, "rb").read()).hexdigest()[:16] != digest:
        return None
    return int((f * FETCH_SCALE + w * WRITE_SCALE) * 1024)
METRIC = "encoder audio-sec/sec (x realtime) at 1 GPU + % of fp16 MFMA roofline"


def frames(n):
    T = (n - 320) // 160 + 1
    S = (T - 1) // 2 + 1
    U = (S - 1) // 2 + 1
    return T, S, U


def role_flops(cfg, lens):
    """Algorithmic FLOPs per launch of each kernel role (valid frames only)."""
    d, f, k, C = cfg["d_model"], cfg["d_ff"], cfg["conv_kernel"], cfg["n_classes"]
    fr = [frames(int(n)) for n in lens]
    S = sum(x[1] for x in fr)
    U = sum(x[2] for x in fr)
    U2 = sum(x[2] ** 2 for x in fr)
    return {
        "gemm.conv1": 2 * S * 320 * d,
        "gemm.conv2": 2 * U * 5 * d * d,
        "gemm.ffn_up": 2 * U * d * f,
        "gemm.ffn_down": 2 * U * f * d,
        "mlp_fused": 4 * U * d * f,            # both FFN GEMMs in one kernel (few rows)
        "gemm.qkv": 2 * U * d * 3 * d,
        "gemm.out_proj": 2 * U * d * d,
        "gemm.pw1_glu": 2 * U * d * 2 * d,
        "gemm.pw2": 2 * U * d * d,
        "gemm.head": 2 * U * d * C,
        "attention": 4 * U2 * d,
        "dwconv_bn_silu": 2 * U * d * k,
    }


def total_flops(cfg, lens):
    r = role_flops(cfg, lens)
    per_layer = (2 * r["gemm.ffn_up"] + 2 * r["gemm.ffn_down"] + r["gemm.qkv"] + r["gemm.out_proj"]
                 + r["gemm.pw1_glu"] + r["gemm.pw2"] + r["attention"] + r["dwconv_bn_silu"])
    return cfg["n_layers"] * per_layer + r["gemm.conv1"] + r["gemm.conv2"] + r["gemm.head"]


def role_bytes(cfg, lens):
    """Algorithmic HBM bytes per launch of the bandwidth-bound roles (16-bit operands,
    fp32 residual stream): read what the step needs once, write its result once."""
    d, C = cfg["d_model"], cfg["n_classes"]
    es = 4 if cfg["dtype"] == "f32" else 2
    fr = [frames(int(n)) for n in lens]
    T = sum(x[0] for x in fr)
    U = sum(x[2] for x in fr)
    B, Umax = len(lens), max(x[2] for x in fr)
    return {
        # samples in, fp32 log-mel rows out, plus their 16-bit copy on 16-bit models
        "frontend": int(sum(int(n) for n in lens)) * 4 + T * 64 * (4 + (es if es == 2 else 0)),
        "layernorm": U * d * (4 + es),
        "layernorm_rope": U * d * (4 + 2 * es),
        "layernorm_two": U * d * (8 + es),
        "dwconv_bn_silu": U * d * 2 * es,
        "logsoftmax_argmax": U * C * 4 + B * Umax * (C * 4 + 4),
    }


def cpu_baseline(name, budget_s):
    """The oracle as it stands, in its float32 mode (float32 NumPy, this host's BLAS threads),
    on a fixed sample of the workload's clips: the warm-up pass takes the clips in batch
    order until about a quarter of budget_s is spent, and that same set of clips is then encoded
    three more times; the rate is its audio over the median of those three passes."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count()
    cfg, pcm, lens, w = synth.workload(name)
    P = oracle.materialize(w, np.float32)

    def encode(b):
        oracle.encode_clip(pcm[b, : int(lens[b])], w, cfg, dtype=np.float32, P=P)

    sample, t0 = [], time.perf_counter()
    for b in range(len(lens)):                         # warm-up pass, clips in batch order
        encode(int(b))
        sample.append(int(b))
        if time.perf_counter() - t0 > budget_s / 4:
            break
    times = []
    for _ in range(3):
        t1 = time.perf_counter()
        for b in sample:
            encode(b)
        times.append(time.perf_counter() - t1)
    audio = float(sum(int(lens[b]) for b in sample)) / 16000.0
    dt = float(np.median(times))
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")),
                             cpu_model)
    except OSError:
        pass
    return {"value": round(audio / dt, 3), "unit": "audio-s/s", "cores": int(cores), "kind": "oracle",
            "sample": f"float32 oracle on the first {len(sample)} of {len(lens)} clips of workload "
                      f"{name} ({audio:.2f} s of audio), 1 warm-up pass + median of 3 passes "
                      f"({dt:.2f} s each)",
            "cpu_model": cpu_model}


def rnnt_leg(model, pcm_d, lens, cfg, steps, warmup):
    """Greedy RNNT decoding of the batch's encoder output (synthetic character head of
    the pages' RNNT model: 33 letters + blank, LSTM 320, joint 320), timed with events
    on the stream alone and together with the encode."""
    import torch
    import conformer_speech_recognition_amd as gg
    import synth
    rcfg = synth.rnnt_config(cfg["d_model"], 34, "bf16" if cfg["dtype"] == "bf16" else
                             ("f32" if cfg["dtype"] == "f32" else "f16"))
    # blank bias 3.4: on this encoder output the random head then emits about two symbols
    # per frame (more than speech, so the decode time is on the slow side)
    head = gg.RnntHead(rcfg, synth.make_rnnt_weights(rcfg, 31, blank_bias=3.4))
    enc = model.encode(pcm_d, lens, want_enc=True, want_frame_ids=False)
    U = [int(u) for u in enc["n_frames"]]
    for _ in range(warmup):
        out = head.decode(enc["enc_out"], U)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    dec_ms, both_ms = [], []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        out = head.decode(enc["enc_out"], U)
        e1.record(st)
        e1.synchronize()
        dec_ms.append(e0.elapsed_time(e1))
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        enc2 = model.encode(pcm_d, lens, want_enc=True, want_frame_ids=False)
        out = head.decode(enc2["enc_out"], U)
        e1.record(st)
        e1.synchronize()
        both_ms.append(e0.elapsed_time(e1))
    n = out["n_tokens"].cpu().numpy()
    G = head.cluster_size(len(U))
    # the same decode with one workgroup per clip, for comparison
    head.set_max_cluster(1)
    one_ms = []
    for _ in range(max(1, steps // 2)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        out1 = head.decode(enc["enc_out"], U)
        e1.record(st)
        e1.synchronize()
        one_ms.append(e0.elapsed_time(e1))
    same = bool(torch.equal(out1["n_tokens"], out["n_tokens"]))
    audio_s = float(np.sum(lens)) / 16000.0
    return {"classes": 34, "dtype": rcfg["dtype"], "max_symbols": rcfg["max_symbols"],
            "workgroups_per_clip": G,
            "decode_ms_p50": round(float(np.median(dec_ms)), 4),
            "decode_ms_p50_one_workgroup_per_clip": round(float(np.median(one_ms)), 4),
            "same_token_counts": same,
            "encode_plus_decode_ms_p50": round(float(np.median(both_ms)), 4),
            "encode_plus_decode_audio_s_per_s": round(audio_s / (float(np.median(both_ms)) * 1e-3), 1),
            "symbols_per_frame": round(float(n.sum()) / float(sum(U)), 3)}


def stream_leg(model, cfg, seconds=60, push_s=1.0, window_s=30.0):
    """Pseudo-streaming: a synthetic signal pushed in push_s pieces, every push followed
    by a re-encode of the last min(total, window_s) seconds (one gigaam_stream_step).
    Per-step times are HIP events on the stream around push + step; the session is run
    once untimed first."""
    import torch
    import conformer_speech_recognition_amd as gg
    import synth
    audio = torch.from_numpy(synth.make_signal(np.random.default_rng(60), int(seconds * 16000))).cuda()
    n = int(push_s * 16000)
    st = torch.cuda.current_stream()

    def session(timed):
        s = gg.Stream(model, window=int(window_s * 16000))
        ms = []
        for i in range(0, audio.numel(), n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            s.push(audio[i: i + n])
            s.step(want_frame_ids=False)
            e1.record(st)
            if timed:
                e1.synchronize()
                ms.append(e0.elapsed_time(e1))
        torch.cuda.synchronize()
        return ms
    session(False)
    ms = session(True)
    buf = [min((i + 1) * push_s, window_s) for i in range(len(ms))]
    at = {f"{int(b)}s": round(float(np.median([m for m, x in zip(ms, buf) if x == b])), 4)
          for b in (1, 5, 10, 20, 30) if b in buf}
    total = sum(ms) * 1e-3
    return {"audio_s": seconds, "push_s": push_s, "window_s": window_s, "steps": len(ms),
            "step_ms_at_buffer": at, "session_ms": round(sum(ms), 3),
            "stream_audio_s_per_s": round(seconds / total, 1),
            "reencoded_audio_s_per_s": round(sum(buf) / total, 1)}


def sweep_leg(model, reps=5):
    """Throughput of one encode call versus chunk length (a 300 s signal cut into equal
    chunks encoded as one batch) and versus batch size (clips of 20 s)."""
    import torch
    import synth
    x = synth.make_signal(np.random.default_rng(61), 300 * 16000)
    st = torch.cuda.current_stream()

    def rate(clips):
        L = max(len(c) for c in clips)
        pcm = np.zeros((len(clips), L), np.float32)
        for i, c in enumerate(clips):
            pcm[i, : len(c)] = c
        lens = np.array([len(c) for c in clips], np.int32)
        d = torch.from_numpy(pcm).cuda()
        for _ in range(2):
            model.encode(d, lens, want_frame_ids=False)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(reps):
            model.encode(d, lens, want_frame_ids=False)
        e1.record(st)
        e1.synchronize()
        return round(float(lens.sum()) / 16000.0 * reps / (e0.elapsed_time(e1) * 1e-3), 1)

    chunk = {}
    for sec in (5, 10, 20, 30, 40):
        n = sec * 16000
        chunk[f"{sec}s"] = rate([x[i: i + n] for i in range(0, len(x), n)])
    batch = {}
    for b in (1, 2, 4, 8, 16, 32, 64):
        clips = [synth.make_signal(np.random.default_rng(100 + i), 320000) for i in range(b)]
        batch[str(b)] = rate(clips)
    return {"unit": "audio-s/s", "chunk_len_300s_signal": chunk, "batch_of_20s_clips": batch,
            "fused_mlp": mlp_variant()}


def mlp_variant(reps=64, sets=32):
    """The fused few-row FFN (d 768, f 3072, hidden activations kept on chip) against the same
    two products as separate split-K GEMMs through HBM, per FFN call, at 25 / 64 / 500 / 896 rows
    (25: one second of audio, 500: one 20 s clip). Calls rotate over `sets` weight sets (302 MB,
    more than the 256 MB last-level cache), so the weights come from HBM as in an encode; each
    call is issued from Python, so the few-row figures include the binding's per-call cost."""
    import torch
    import conformer_speech_recognition_amd as gg
    st = torch.cuda.current_stream()
    g = torch.Generator(device="cuda").manual_seed(71)
    w1 = [(0.05 * torch.randn(3072, 768, device="cuda", generator=g)).half() for _ in range(sets)]
    w2 = [(0.05 * torch.randn(768, 3072, device="cuda", generator=g)).half() for _ in range(sets)]
    b1 = torch.randn(3072, device="cuda", generator=g)
    b2 = torch.randn(768, device="cuda", generator=g)
    out = {}
    for M in (25, 64, 500, 896):
        y = torch.randn(M, 768, device="cuda", generator=g).half()
        x = torch.zeros(M, 768, device="cuda")
        h = gg.debug_gemm("f16", y, w1[0], b1, split=True)[0].half()

        def timed(fn):
            for i in range(3):
                fn(i % sets)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(st)
            for i in range(reps):
                fn(i % sets)
            e1.record(st)
            e1.synchronize()
            return e0.elapsed_time(e1) * 1e3 / reps

        fused = timed(lambda i: gg.debug_mlp("f16", y, w1[i], b1, w2[i], b2, x))
        two = timed(lambda i: (gg.debug_gemm("f16", y, w1[i], b1, split=True),
                               gg.debug_gemm("f16", h, w2[i], b2, split=True)))
        out[str(M)] = {"fused_us": round(fused, 1), "two_gemms_us": round(two, 1),
                       "fused_tflops": round(4 * M * 768 * 3072 / (fused * 1e-6) / 1e12, 1)}
    del w1, w2
    return out


def library_gemm_leg(cfg, U, prof, reps=64, sets=16):
    """The vendor library's plain product (torch.mm in the workload's 16-bit type, in and out, no bias or epilogue) on
    each encoder GEMM role's shape at this workload's U rows, beside the encoder kernel's own
    average launch for that role (which also applies its epilogue: SiLU, GLU, the residual
    half step). Weights rotate over `sets` copies, as each layer's differ in an encode."""
    import torch
    d, f = cfg["d_model"], cfg["d_ff"]
    shapes = {"gemm.ffn_up": (f, d, "bias + SiLU, fp16 out"),
              "gemm.ffn_down": (d, f, "bias + residual half step into fp32 x"),
              "gemm.qkv": (3 * d, d, "bias, fp16 out"),
              "gemm.pw1_glu": (2 * d, d, "bias + GLU, fp16 out (half width)"),
              "gemm.out_proj": (d, d, "bias + residual into fp32 x")}
    ours = {r["name"]: r["avg_us"] for r in prof}
    tt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.half
    g = torch.Generator(device="cuda").manual_seed(5)
    st = torch.cuda.current_stream()
    out = {}
    for role, (N, K, epi) in shapes.items():
        A = torch.randn(U, K, device="cuda", generator=g).to(tt)
        Ws = [torch.randn(N, K, device="cuda", generator=g).to(tt) for _ in range(sets)]
        C = torch.empty(U, N, device="cuda", dtype=tt)
        for i in range(4):
            torch.mm(A, Ws[i % sets].t(), out=C)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for i in range(reps):
            torch.mm(A, Ws[i % sets].t(), out=C)
        e1.record(st)
        e1.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        fl = 2.0 * U * N * K
        out[role] = {"M": U, "N": N, "K": K, "torch_mm_us": round(us, 1),
                     "torch_mm_tflops": round(fl / us / 1e6, 1),
                     "ours_us": ours.get(role), "ours_tflops": round(fl / ours[role] / 1e6, 1) if role in ours else None,
                     "ours_epilogue": epi}
        del A, Ws, C
    return out


def gemm_variants_leg(cfg, U, reps=30, sets=8):
    """Each encoder GEMM role at this workload's U rows with every direct-load tile variant the
    library builds (gigaam_debug_gemm_role with a shape request), beside the variant the encoder
    picks. Weights rotate over `sets` copies; operands random; median of three timed loops of
    `reps` launches, interleaved over the variants so that clock drift hits all alike."""
    import torch
    import conformer_speech_recognition_amd as gg
    d, f = cfg["d_model"], cfg["d_ff"]
    tt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.half
    dt = "bf16" if cfg["dtype"] == "bf16" else "f16"
    roles = [("gemm.ffn_up", "plain", "silu", f, d), ("gemm.pw1_glu", "plain", "glu", 2 * d, d),
             ("gemm.qkv", "dual", "store", 3 * d, d), ("gemm.ffn_down", "plain", "resid", d, f),
             ("gemm.out_proj", "plain", "resid", d, d)]
    st = torch.cuda.current_stream()
    g = torch.Generator(device="cuda").manual_seed(9)
    out = {}
    for name, am, ep, N, K in roles:
        A = torch.randn(U, K, device="cuda", generator=g).to(tt)
        A2 = torch.randn(U, K, device="cuda", generator=g).to(tt) if am == "dual" else None
        Ws = [(0.05 * torch.randn(N, K, device="cuda", generator=g)).to(tt) for _ in range(sets)]
        b = torch.randn(N, device="cuda", generator=g)
        C = (torch.zeros(U, N, device="cuda") if ep == "resid" else
             torch.empty(U, N // 2 if ep == "glu" else N, device="cuda", dtype=tt))
        times, chosen = {}, None
        for v in [None] + list(gg.GEMM_SHAPE_IDS):
            if v is not None and not v.startswith("dma_"):
                continue
            try:
                chosen_v = gg.debug_gemm_role(dt, am, ep, A, Ws[0], C, bias=b, A2=A2,
                                              nsplit=2 * d if am == "dual" else 0, split=False, shape=v)[2]
            except gg.GigaamError:
                continue
            if v is None:
                chosen = chosen_v
                continue
            times[v] = []
        for _ in range(3):
            for v in times:
                for i in range(3):
                    gg.debug_gemm_role(dt, am, ep, A, Ws[i % sets], C, bias=b, A2=A2,
                                       nsplit=2 * d if am == "dual" else 0, split=False, shape=v)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(st)
                for i in range(reps):
                    gg.debug_gemm_role(dt, am, ep, A, Ws[i % sets], C, bias=b, A2=A2,
                                       nsplit=2 * d if am == "dual" else 0, split=False, shape=v)
                e1.record(st)
                e1.synchronize()
                times[v].append(e0.elapsed_time(e1) * 1e3 / reps)
        out[name] = {"M": U, "N": N, "K": K, "encoder_variant": chosen,
                     "us_median": {v: round(float(np.median(t)), 2) for v, t in times.items()}}
        del A, A2, Ws, C
    return out


def measured_peaks(dtype: str):
    """What this GPU sustains, beside the datasheet peaks: the vendor library's GEMM on a large
    square product in the workload's compute type (16384^3, fp32: 8192^3), and a plain device
    copy of 1 GiB (read + write bytes per second). Median of 5 timed calls after 2 warm-ups."""
    import torch
    tt = {"f32": torch.float32, "bf16": torch.bfloat16}.get(dtype, torch.float16)
    n = 8192 if tt == torch.float32 else 16384
    g = torch.Generator(device="cuda").manual_seed(3)
    a = torch.randn(n, n, device="cuda", generator=g).to(tt)
    b = torch.randn(n, n, device="cuda", generator=g).to(tt)
    c = torch.empty(n, n, device="cuda", dtype=tt)

    def med(fn):
        for _ in range(2):
            fn()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    t_mm = med(lambda: torch.mm(a, b, out=c))
    del a, b, c
    x = torch.empty(1 << 28, device="cuda")
    y = torch.empty_like(x)
    t_cp = med(lambda: y.copy_(x))
    del x, y
    return {"gemm_tflops": round(2.0 * n ** 3 / t_mm / 1e12, 1), "gemm_shape": f"{n}^3 {str(tt)[6:]}",
            "copy_gbs": round(2.0 * (1 << 30) / t_cp / 1e9, 1), "copy_bytes": 1 << 30}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="batch32")
    ap.add_argument("--profile-steps", type=int, default=5)
    ap.add_argument("--graph", action="store_true", help="replay the encode as a captured graph")
    ap.add_argument("--cpu-budget", type=float, default=24.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the vendor-library GEMM and copy peak measurements (profiled runs)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="end with one plain 256 MiB device copy: the known-size reference for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    ap.add_argument("--rnnt", action="store_true",
                    help="also time greedy RNNT decoding (character head, 34 classes) of every "
                         "encoded batch and report it beside the encoder line")
    ap.add_argument("--stream", action="store_true",
                    help="also time pseudo-streaming: 60 s pushed in 1 s pieces, each push followed "
                         "by a re-encode of the last <= 30 s")
    ap.add_argument("--sweep", action="store_true",
                    help="also report throughput versus chunk length and batch size")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time the vendor library's plain product on each GEMM role's shape")
    ap.add_argument("--gemm-variants", action="store_true",
                    help="also time every direct-load tile variant on each GEMM role's shape")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {a.gpus}); the "
              "encoder shards as independent clips per GPU with no exchange, and no multi-GPU "
              "figure is produced here.", file=sys.stderr)
        sys.exit(2)

    import torch
    import conformer_speech_recognition_amd as gg
    import synth

    cfg, pcm, lens, w = synth.workload(a.workload)
    model = gg.Model(cfg, w)
    pcm_d = torch.from_numpy(pcm).cuda()
    audio_s = float(lens.sum()) / 16000.0
    stream = torch.cuda.current_stream()

    def step():
        return model.encode(pcm_d, lens, want_frame_ids=False)

    if a.graph:
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        run = g.replay
    else:
        run = step
    for _ in range(a.warmup):
        run()
    torch.cuda.synchronize()

    # ---- timed region
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(a.steps):
        run()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(a.steps)])

    # ---- per-kernel launch times (HIP events around every launch, eager encodes)
    gg.profile_start()
    for _ in range(a.profile_steps):
        step()
    torch.cuda.synchronize()
    gg.profile_stop()
    prof = gg.profile_report()

    flops = total_flops(cfg, lens)
    rf = role_flops(cfg, lens)
    rb = role_bytes(cfg, lens)
    # the dominant kernel among those with an algorithmic work figure (the geometry kernel
    # and the rope table have none; after graph replays meta's first eager launch can wait)
    dom = max((r for r in prof if r["name"] in rf or r["name"] in rb), key=lambda r: r["total_ms"])
    name = dom["name"]
    if name in rf and (name.startswith("gemm") or name in ("attention", "mlp_fused")):
        achieved = rf[name] / (dom["avg_us"] * 1e-6) / 1e12
        peak = PEAK_TFLOPS[cfg["dtype"]]
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    else:
        achieved = rb[name] / (dom["avg_us"] * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof.update({"kernel": name, "avg_launch_us": dom["avg_us"], "launches": dom["launches"],
                 "traffic": measured_traffic(a.workload, name)})
    peaks = None if a.no_peaks else measured_peaks(cfg["dtype"])
    if peaks:
        roof["measured_peak"] = peaks["gemm_tflops"] if roof["unit"] == "TFLOP/s" else peaks["copy_gbs"]
        roof["frac_of_measured_peak"] = round(roof["achieved"] / roof["measured_peak"], 4)

    ms = 1e3 * elapsed / a.steps
    value = a.steps * audio_s / elapsed
    tflops = flops / (ms * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "audio-s/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": a.workload, "clips": int(len(lens)), "audio_seconds": round(audio_s, 3),
                   "encoder_frames": int(sum(frames(int(n))[2] for n in lens)),
                   "global_batch": int(len(lens)), "graph_replay": bool(a.graph)},
        "encoder_tflops": round(tflops, 2),
        "fp16_mfma_roofline_frac": round(tflops / PEAK_TFLOPS["f16"], 4),
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 4) for q in (10, 50, 90)],
        "roofline": roof,
        "measured_peaks": peaks,
        "kernels": sorted(({"name": r["name"], "launches": r["launches"], "avg_us": r["avg_us"],
                            "total_ms": round(r["total_ms"] / a.profile_steps, 4)} for r in prof),
                          key=lambda r: -r["total_ms"]),
    }
    if a.rnnt:
        line["rnnt"] = rnnt_leg(model, pcm_d, lens, cfg, a.steps, a.warmup)
    if a.stream:
        line["stream"] = stream_leg(model, cfg)
    if a.sweep:
        line["sweep"] = sweep_leg(model)
    if a.library_gemm:
        line["library_gemm"] = library_gemm_leg(cfg, line["config"]["encoder_frames"], prof)
    if a.gemm_variants:
        line["gemm_variants"] = gemm_variants_leg(cfg, line["config"]["encoder_frames"])
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(a.workload, a.cpu_budget)
    if a.calib_copy:
        src = torch.ones(1 << 26, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["calib_copy_bytes"] = 1 << 28
        del src, dst
        # the same check for direct-to-LDS loads: one 256 x 128 tile of the pipelined fp16 GEMM
        # with K = 65536 reads A (32 MiB) and W (16 MiB) exactly once
        A = torch.ones(256, 65536, device="cuda", dtype=torch.half)
        Wt = torch.ones(128, 65536, device="cuda", dtype=torch.half)
        C = torch.empty(256, 128, device="cuda")
        torch.cuda.synchronize()
        line["calib_dma_shape"] = gg.debug_gemm_role("f16", "plain", "f32", A, Wt, C, split=False)[2]
        torch.cuda.synchronize()
        line["calib_dma_read_bytes"] = (256 + 128) * 65536 * 2
        del A, Wt, C
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
