"""The oracle: plain, slow, float64 CPU implementations of what the attention
path computes, written from the pages' descriptions.

TEST INFRASTRUCTURE. Only the tests, the smoke check of the entry module and
the CPU-baseline leg of the benchmark may import, call or run anything in this
package. The product path (the C-ABI library and its Python binding) never
uses it and shares no code, table or helper with it.

Contents
  attention.py  exact softmax(scale * Q K^T) V and per-row log-sum-exp in
                float64, materialising S and P, also for queries and keys of
                different lengths (pinned: closed forms, brute force,
                invariants, a library routine).
  attention_grad.py  dQ, dK, dV of sum(dO * O) for the same attention, in
                float64 (pinned: central finite differences, a library
                routine's autograd, closed forms, invariants).
  fp8.py        e4m3fn encode/decode, per-block and per-tensor quantisation
                with optional random-sign Hadamard rotation (pinned: a library
                cast, the format's closed forms, a hand-built block, H H^T =
                d I, rotation invariance of attention), and an FP8 attention
                emulator (P * 2^8 rounded to e4m3) whose error is printed as a
                prediction next to the kernel's and gates nothing. Its
                rounding path is "parity unpinned" beyond the reduction to
                exact attention when P is not rounded.
"""
from .attention import attention, attention_kv, attention_rows, attention_sampled  # noqa: F401
from .attention_grad import attention_backward  # noqa: F401
from . import fp8  # noqa: F401
