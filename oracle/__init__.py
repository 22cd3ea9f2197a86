"""Float64 oracle for windowed grouped-query softmax attention (test infrastructure).

This package is the plain, slow CPU definition that the HIP path is checked against.
It is test infrastructure only: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the library and its binding never do.
It shares no code with the HIP path.

Source: TensorFold pull request #1123, "window_attention at head dim 256",
section "What this changes" (the Decode, Prompt, Window.p32, promptRows hi, Scale/Window 0
and range-checker bullets).

The q/k row preparation (RoPE, L2 or RMS norm, q scale; TensorFold pull request #1257,
"What this changes", and the "Exact Numerical Contract" page, "Preparation") is in
``prepare``.

Modules:
  bf16     float64 -> bf16 round-to-nearest-even with signed underflow, and back.
  attend   the attention definition in float64 (visibility, scores, softmax, P.V).
  check    the acceptance interval around the float64 value, compared in bf16 value order.
  prepare  the q/k preparation at its rounding points, and its acceptance interval.
"""

from . import bf16, attend, check, prepare  # noqa: F401
