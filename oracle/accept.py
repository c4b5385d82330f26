"""Acceptance rules of the verification step, and near-tie flags.

Test infrastructure only (see the package docstring).

Notation: the block is [t_0 = pending, t_1 = d_1, ..., t_k = d_k]; logits
row j (0 <= j <= k) is the target's prediction after t_j.  The committed
cache length before the step is L; after it, L + 1 + n_acc (the pending
token's entry plus the accepted drafts' entries).
"""
from __future__ import annotations

import dataclasses
from typing import List

import numpy as np

from . import numerics as nx


@dataclasses.dataclass
class StepOutcome:
    n_accepted: int
    next_token: int
    kv_len: int
    near_tie: bool = False        # a decision within tolerance of flipping
    tie_where: List[str] = dataclasses.field(default_factory=list)


def argmax_lowest(row: np.ndarray) -> int:
    """argmax with ties going to the lowest token id (the first maximal
    index, as the essay's `argmax` returns)."""
    return int(np.argmax(row))


def top2_gap(row: np.ndarray) -> float:
    s = np.partition(np.asarray(row, dtype=np.float64), -2)
    return float(s[-1] - s[-2])


def accept_greedy(logits: np.ndarray, drafts, L: int, tol: float = 0.0) -> StepOutcome:
    """Greedy acceptance (essay "LLM Inference: Speculative Decoding",
    "The loop", steps 3-4): a_j = argmax(row j); n_acc is the length of the
    longest prefix of drafts with d_i == a_{i-1}; the next (pending) token is
    a_{n_acc} -- the correction when a draft was rejected, the bonus token
    when all k were accepted.  Rows whose top-2 gap is below `tol` and that
    decide the outcome are flagged as near-ties."""
    drafts = [int(d) for d in drafts]
    k = len(drafts)
    a = [argmax_lowest(logits[j]) for j in range(k + 1)]
    n = 0
    while n < k and drafts[n] == a[n]:
        n += 1
    out = StepOutcome(n, a[n], L + 1 + n)
    for j in range(n + 1):                  # rows that decided the outcome
        if top2_gap(logits[j]) < tol:
            out.near_tie = True
            out.tie_where.append(f"row{j}")
    return out


def inverse_cdf(weights: np.ndarray, u: float) -> (int, float):
    """Draw from the unnormalized distribution `weights` by inverse CDF:
    the smallest id x with C(x) > u * C(V-1), C the running sum in ascending
    id order (float64).  Returns (x, margin) where margin = min distance of
    u*S to the two CDF values bracketing it, divided by S (for near-tie
    flags)."""
    w = np.asarray(weights, dtype=np.float64)
    C = np.cumsum(w)
    S = C[-1]
    thr = u * S
    x = int(np.searchsorted(C, thr, side="right"))
    x = min(x, len(w) - 1)
    lo = C[x - 1] if x > 0 else 0.0
    margin = min(abs(thr - C[x]), abs(thr - lo)) / S
    return x, float(margin)


def accept_stochastic(logits: np.ndarray, q: np.ndarray, drafts, u, L: int,
                      tol: float = 0.0) -> StepOutcome:
    """Rejection-sampling acceptance at temperature 1 (the rule of Leviathan
    et al. that the essay's "What is not here" names as keeping the target's
    output distribution).

    p_j = softmax(row j).  For i = 1..k in order, with P = p_{i-1}(d_i) and
    Q = q_i(d_i): accept d_i iff u_i < min(1, P/Q), evaluated as u_i*Q < P.
    At the first rejection, n_acc = i-1 and the next token is drawn from
    max(0, p_{i-1} - q_i) (normalized) with u_{k+1}; if that residual is all
    zero (p = q) it is drawn from p_{i-1}.  If all k are accepted the next
    token is drawn from p_k with u_{k+1}.

    q: [k, V] draft distributions (q[i-1] = q_i); u: [k+1] uniforms.
    """
    drafts = [int(d) for d in drafts]
    k = len(drafts)
    z = np.asarray(logits, dtype=np.float64)
    p = nx.softmax(z, axis=-1)
    qq = np.asarray(q, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    out = StepOutcome(0, -1, L + 1)
    for i in range(1, k + 1):
        d = drafts[i - 1]
        P, Q = p[i - 1, d], qq[i - 1, d]
        if abs(u[i - 1] * Q - P) < tol * Q:
            out.near_tie = True
            out.tie_where.append(f"test{i}")
        if u[i - 1] * Q < P:
            continue
        r = np.maximum(0.0, p[i - 1] - qq[i - 1])
        if r.sum() <= 0.0:
            r = p[i - 1]
        x, margin = inverse_cdf(r, u[k])
        if margin < tol:
            out.near_tie = True
            out.tie_where.append("resample")
        out.n_accepted, out.next_token, out.kv_len = i - 1, x, L + i
        return out
    x, margin = inverse_cdf(p[k], u[k])
    if margin < tol:
        out.near_tie = True
        out.tie_where.append("bonus")
    out.n_accepted, out.next_token, out.kv_len = k, x, L + 1 + k
    return out


def accept_none(logits: np.ndarray, k: int, L: int) -> StepOutcome:
    """Commit the whole block (append / chunked prefill): kv_len = L+k+1,
    next = argmax of the last row."""
    return StepOutcome(k, argmax_lowest(logits[k]), L + k + 1)
