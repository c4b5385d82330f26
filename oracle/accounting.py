"""Per-run counters of speculative decoding and the expected-tokens formula.

Test infrastructure only (see the package docstring).

* Counters follow the essay "LLM Inference: Speculative Decoding",
  sections "What it does" and "What it cost": one target pass per round;
  the draft runs k+1 times per round (k guesses plus one pass feeding the
  target's token back); k guesses per round; guesses not accepted are
  discarded; target passes saved = tokens produced - target passes.
* Expected output tokens per round for per-token acceptance rate a and
  lookahead k: (1 - a^(k+1)) / (1 - a), rising to the ceiling 1/(1-a)
  (same essay, "Being right five times in a row is rare").
"""
from __future__ import annotations

from typing import Dict, Sequence


def run_counters(k: int, n_accepted: Sequence[int], n_tokens: int) -> Dict[str, int]:
    """Counters of a run of rounds with accepted counts `n_accepted` that was
    asked for `n_tokens` output tokens (the last round may overshoot; the
    output is truncated to n_tokens)."""
    rounds = len(n_accepted)
    accepted = int(sum(n_accepted))
    emitted = accepted + rounds              # each round adds its target token
    return dict(
        target_passes=rounds,
        draft_passes=rounds * (k + 1),
        guesses=rounds * k,
        discarded=rounds * k - accepted,
        emitted=emitted,
        tokens=min(emitted, n_tokens),
        target_passes_saved=min(emitted, n_tokens) - rounds,
    )


def expected_tokens_per_round(a: float, k: int) -> float:
    if a == 1.0:
        return float(k + 1)
    return (1.0 - a ** (k + 1)) / (1.0 - a)


def acceptance_ceiling(a: float) -> float:
    return 1.0 / (1.0 - a)


def acceptance_rate_from_corruption(c: float, vocab: int) -> float:
    """Per-draft agreement when each draft equals the target's token except
    with probability c, where it is replaced by a uniform id (which still
    agrees with probability 1/V)."""
    return 1.0 - c * (1.0 - 1.0 / vocab)

