"""CPU ORACLE for pseudo-streaming: which audio each step re-encodes.

TEST INFRASTRUCTURE ONLY (same rules as the package oracle: only the tests, the smoke
check and the benchmark's CPU-baseline leg may use it; the HIP path shares nothing).

"GigaAM on MLX: the transcripts matched, but the model was broken", section
"Streaming: honestly, it's pseudo-streaming": the model is not a streaming model; the
port keeps a growing buffer, and every step recognises all of the audio received so far,
but no more than the last 30 seconds. A step's output is therefore the plain encoder
output of that window (oracle.encode_clip on it): nothing carries over between steps.

Reading where the page is silent: a step follows every push, the window ends at the
newest sample, and the 30 s cap is `window` samples (480000 at 16 kHz).
"""
from __future__ import annotations


def windows(chunks, window: int) -> list[tuple[int, int]]:
    """Sample range [lo, hi) of the whole stream that the step after each push encodes:
    everything pushed so far, but at most the last ``window`` samples."""
    out, total = [], 0
    for n in chunks:
        if n < 0:
            raise ValueError("negative push")
        total += int(n)
        out.append((max(0, total - window), total))
    return out
