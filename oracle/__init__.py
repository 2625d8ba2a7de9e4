"""CPU oracle for one EAGLE / EAGLE-2 draft-and-verify cycle at batch 1.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package. The GPU product path never calls it, and it shares no code with the
GPU library (only the seeded input generators in ``synth/`` serve both).

It is a plain, slow, obviously correct implementation in numpy, accumulating
in fp64 and rounding at the points fixed by the numerics contract:

* fp32 configs: every tensor is rounded to fp32 where it is produced.
* bf16 configs: weights, embedding rows, the K/V cache and every matrix-product
  operand that is an activation (normed activations, query, attention output,
  SwiGLU product, draft FC inputs, features fed to the LM head) are rounded
  to bf16 (round-to-nearest-even of the fp32 value); accumulations, the
  residual stream, RoPE, softmax, logits and log-probabilities are fp32.

Sources (web pages on EAGLE, EAGLE-2 and EAGLE-3):
  [L13] "Lesson 13.11 - EAGLE: Feature-Level Drafting for Faster Inference"
  [E2]  "EAGLE-2: Context-Aware Dynamic Draft Trees"
  [E3]  "05 - EAGLE 三代: feature 自回归、动态树、Training-Time Test"

Modules:
  numerics  rounding, RMSNorm, SiLU, RoPE, log-softmax (textbook definitions)
  model     Llama-style target, EAGLE-1 and EAGLE-3 draft heads
  tree      path values, expansion, rerank, flattening, ancestry masks
  loop      plain greedy decode, the speculative loop, acceptance, commit
  speedup   the lesson's expected-tokens / speedup formula

Parity status: every function is pinned by a test in ``tests/`` except where
its docstring says "parity unpinned".
"""
