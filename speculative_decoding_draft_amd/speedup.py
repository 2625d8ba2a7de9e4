"""Speedup model of speculative decoding, applied to measured pass times.

"EAGLE: Feature-Level Drafting for Faster Inference" (Lesson 13.11), section
"The math behind the speedup with small numbers": with a per-token acceptance
rate alpha (each drafted token accepted with that chance when all earlier
ones were), k drafted tokens per step and one draft pass costing c target
passes, a step commits on average the geometric sum 1 + alpha + ... + alpha^k
tokens and costs 1 + k*c target passes. The chain model ignores the tree's
extra branches, so for a tree it is a lower estimate at a given alpha.

A reporting helper for the measured draft cost c; it is not on the decoding
path.
"""
from __future__ import annotations

ALPHAS = (0.6, 0.7, 0.8, 0.9)


def expected_tokens(alpha: float, k: int) -> float:
    """Mean tokens committed per step (closed form of the geometric sum)."""
    if not 0.0 <= alpha <= 1.0 or k < 0:
        raise ValueError("alpha must be in [0, 1] and k >= 0")
    if alpha == 1.0:
        return float(k + 1)
    return (1.0 - alpha ** (k + 1)) / (1.0 - alpha)


def speedup(alpha: float, k: int, c: float) -> float:
    """Tokens per target-pass cost relative to plain decoding."""
    if c < 0:
        raise ValueError("draft cost c must be >= 0")
    return expected_tokens(alpha, k) / (1.0 + k * c)


def report(draft_pass_s: float, target_pass_s: float, k: int, alphas=ALPHAS) -> dict:
    """c = draft pass time / target pass time from measured times, and the
    model's speedup at each alpha for k draft passes per step."""
    if draft_pass_s <= 0 or target_pass_s <= 0:
        raise ValueError("pass times must be positive")
    c = draft_pass_s / target_pass_s
    return {
        "draft_pass_ms": round(draft_pass_s * 1e3, 4),
        "target_pass_ms": round(target_pass_s * 1e3, 4),
        "c": round(c, 5),
        "k": k,
        "predicted_speedup": {f"{a:.1f}": round(speedup(a, k, c), 4) for a in alphas},
        "model": "chain: (1 + a + ... + a^k) / (1 + k c)",
    }
