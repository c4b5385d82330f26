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
* The adaptive lookahead schedule the essay attributes to HuggingFace
  ("And the checking stops being free"): +2 after a fully accepted block,
  back off otherwise (read as -1, never below 1, never above the largest
  lookahead the verifier takes).
"""
from __future__ import annotations

from typing import Dict, List, Sequence


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


def adaptive_k_schedule(k0: int, n_accepted_seq: Sequence[int], max_k: int) -> List[int]:
    """Lookahead of every round: round 0 uses k0; after a round with
    lookahead k and n accepted drafts, the next uses k + 2 (at most max_k)
    when n == k, else k - 1 (at least 1).  Returns one k per round plus the
    k the next round would use."""
    ks = [k0]
    for n in n_accepted_seq:
        k = ks[-1]
        if not 0 <= n <= k:
            raise ValueError("accepted count outside [0, k]")
        ks.append(min(k + 2, max_k) if n == k else max(1, k - 1))
    return ks


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

