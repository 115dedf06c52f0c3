"""CPU oracle for the MoE decode step and the FP8 LM head -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy in float64 (float32 only where the method itself fixes a
float32 step: the FP8 row scale and the quantising division). Only ``tests/``, the graft entry's
``smoke()`` and the CPU-baseline leg of ``bench.py`` may import it; the product path never does
and shares no code, table or helper with it.

What it computes, and the passages it follows (pages: runbyai.xyz/signal/190,
runbyai.xyz/posts/593, the vibeleaderboard.ai summary, and the Netics Labs post "Three MoE
Inference Optimizations NVIDIA Measured on DGX Spark"):

* ``formats``  -- e2m1 / E8M0 (MXFP4) and E4M3 (FP8) decode and encode. The pages only name
  "MXFP4" and "FP8"; bit layouts follow the public OCP MX v1.0 and OCP 8-bit floating point
  specifications.
* ``moe``      -- router logits, top-k selection with softmax renormalised over the selected
  experts, SwiGLU expert FFNs, the gate-weighted sum plus one shared expert, and the expert union
  of a verification window (posts/593 paragraphs 2 and 5; Netics "Decoding was memory-bound ...").
* ``lmhead``   -- online per-row FP8 quantisation of the bf16 head and the head GEMV in FP8 and
  bf16 (posts/593 paragraph 3; Netics "Online FP8 quantization halves the LM head weight reads").

* ``verify``   -- the verification epilogue of a speculative window after the head: per-position
  argmax, greedy prefix acceptance of the drafts, and top-k / top-p sampling at a temperature
  with the caller's uniform draw (signal/190 and the Netics post on speculative decoding).

Pins (all in ``tests/test_oracle_*.py``): closed forms of the formats, exhaustive comparison with
torch's float8_e4m3fn, brute force in pure-Python loops at tiny shapes, the one-hot routing that
reduces the layer to a single dense FFN, x = 0 routing, exact ties, one-hot LM-head inputs, and
the pages' printed byte counts, hand-worked verification windows, closed forms of the sampling
distribution and its inversion checked by frequency. No function here is "parity unpinned".
"""
from . import formats, lmhead, moe, verify  # noqa: F401
