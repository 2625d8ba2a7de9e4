"""CPU oracle for one EAGLE / EAGLE-2 draft-and-verify cycle at batch 1.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package. The GPU product path never calls it, and it shares no code with the
GPU library (only the seeded input generators in ``synth/`` serve both).

It is a plain, slow, obviously correct implementation in numpy, accumulating
in fp64 and rounding at the points fixed by the numerics contract:

* every activation is rounded to fp32 where it is produced (normed
  activations, q/k/v, attention output, SwiGLU product, residual stream,
  features, logits, log-probabilities);
* bf16 configs store the weights (embedding and LM head included) in bf16
  (round-to-nearest-even of the generated fp32 value); activations and the
  K/V cache stay fp32. Rounding activations or K/V to bf16 would make any
  two implementations that sum in different orders drift apart to the bf16
  noise floor within a few layers (a rounding flip moves the next layer's
  values by far more than the accumulation difference that caused it), so
  it is not part of the contract.

Sources (web pages on EAGLE, EAGLE-2 and EAGLE-3):
  [L13] "Lesson 13.11 - EAGLE: Feature-Level Drafting for Faster Inference"
  [E2]  "EAGLE-2: Context-Aware Dynamic Draft Trees"
  [E3]  "05 - EAGLE 三代: feature 自回归、动态树、Training-Time Test"

Modules:
  numerics  rounding, RMSNorm, SiLU, RoPE, log-softmax (textbook definitions)
  model     Llama-style target, EAGLE-1 and EAGLE-3 draft heads
  tree      path values, expansion, rerank, flattening, ancestry masks
  loop      plain greedy decode, the speculative loop, acceptance, commit
  sampling  temperature > 0: Philox4x32-10 draws and the lossless tree
            rejection-sampling acceptance
  speedup   the lesson's expected-tokens / speedup formula

Parity status: every function is pinned by a test in ``tests/`` except where
its docstring says "parity unpinned": the draft heads' wiring
(``model.Draft``, the E1 concat/FC and the E3 2H-input layer), which is held
only to internal consistency (tree rows equal chains, the lossless loop).
"""
