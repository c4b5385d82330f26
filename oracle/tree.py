"""Token-tree verification and routing-aware tree expansion (S2-MoE,
section 4.1 "Routing-aware Adaptive Speculative Expansion").

Test infrastructure only (see the package docstring).

A draft tree has a root, the pending token, and draft tokens below it;
each row names its parent row (parents[0] = -1, 0 <= parents[i] < i).  The
target verifies every node of the tree in one pass.  What that pass must
produce for node i is fixed by the chain definition alone: the logits the
target writes after the tokens on the path root..i, placed at positions
L, L+1, ..., L+depth(i) after the committed cache (causal attention inside
the path only).  tree_logits computes exactly that, one plain block pass per
node, with no tree mask at all -- a tree pass must reproduce it.

Greedy acceptance down a tree is the chain rule applied along the branch
that matches the target: starting at the root, while the argmax of the
current node's row (lowest id on ties) is the token of one of its children,
that child is accepted (the lowest-numbered one if several carry the token)
and becomes current; the next pending token is the argmax of the last
current row.  The committed cache then holds the pending token and the
accepted path at L .. L + n.  On a chain this is accept_greedy; the output
equals greedy decoding (essay "LLM Inference: Speculative Decoding", "The
output does not change").

utility_expand is the greedy admission of section 4.1: a candidate's
expected benefit B_i = p_i * T_AR with p_i the product of the draft
probabilities on its path (its prefix confidence), its marginal
verification cost the number of its experts not yet activated by the
admitted set times T_exp, plus its own drafting cost, and U_i = B_i / cost.
Readings where the section leaves a step open:
  * a candidate is admissible only once its parent is admitted (it can be
    accepted only if its prefix is);
  * each round admits the admissible candidate of highest U_i (lowest index
    on ties) if U_i >= 1, then adds its experts to the activated set; the
    expansion stops when the best U_i < 1 or max_nodes are admitted;
  * a zero cost with positive benefit is an infinite utility; a zero
    benefit is never admitted;
  * the activated set starts from the experts the caller already pays for
    (e.g. the root token's).
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np

from . import accept as oacc
from . import model as om


def check_tree(parents: Sequence[int]) -> None:
    parents = [int(p) for p in parents]
    if not parents or parents[0] != -1:
        raise ValueError("row 0 is the root: parents[0] must be -1")
    for i in range(1, len(parents)):
        if not 0 <= parents[i] < i:
            raise ValueError(f"row {i}: parent {parents[i]} must precede it")


def path_to(parents: Sequence[int], i: int) -> List[int]:
    """Rows root..i."""
    p = []
    while i >= 0:
        p.append(i)
        i = int(parents[i])
    return p[::-1]


def tree_logits(M: om.OracleModel, kv: om.KVCache, tokens, parents, L: int) -> np.ndarray:
    """Row i: the last row of a block pass over the tokens on the path
    root..i at positions L.. (the entries it writes past the committed
    length stay dead; kv.length is unchanged)."""
    check_tree(parents)
    tokens = np.asarray(tokens, dtype=np.int64)
    rows = []
    for i in range(len(tokens)):
        res = om.forward_block(M, kv, tokens[path_to(parents, i)], L)
        rows.append(res.logits[-1])
    return np.stack(rows)


def accept_tree_greedy(logits: np.ndarray, tokens, parents, L: int, tol: float = 0.0):
    """Greedy walk down the tree.  Returns (outcome, accepted rows).  Rows
    on the walk whose top-2 gap is below tol are flagged as near-ties."""
    check_tree(parents)
    m = len(parents)
    cur, path = 0, []
    out_tie = []
    while True:
        a = oacc.argmax_lowest(logits[cur])
        if oacc.top2_gap(logits[cur]) < tol:
            out_tie.append(f"row{cur}")
        child = next((i for i in range(cur + 1, m) if parents[i] == cur and int(tokens[i]) == a), None)
        if child is None:
            break
        path.append(child)
        cur = child
    out = oacc.StepOutcome(len(path), a, L + 1 + len(path))
    out.near_tie = bool(out_tie)
    out.tie_where = out_tie
    return out, path


def commit_tree(M: om.OracleModel, kv: om.KVCache, tokens, path, L: int) -> None:
    """Cache after the step: the pending token and the accepted path's
    tokens at L .. L + n, as a chain pass over them writes them."""
    toks = [int(tokens[0])] + [int(tokens[i]) for i in path]
    om.forward_block(M, kv, toks, L)
    kv.length = L + len(toks)


def utility_expand(parents, p, experts, base, t_ar: float, t_exp: float, c_draft, max_nodes: int):
    """Greedy routing-aware admission.  parents[i]: -1 (child of the root)
    or an earlier candidate; p[i]: the draft probability of candidate i's
    token given its parent; experts[i]: the experts (any hashable ids)
    verifying it activates; base: experts already active; c_draft[i]: its
    drafting cost.  Returns the admitted candidates in admission order."""
    n = len(parents)
    conf = []
    for i in range(n):
        if not -1 <= parents[i] < i:
            raise ValueError("a candidate's parent must precede it")
        conf.append(float(p[i]) if parents[i] < 0 else conf[parents[i]] * float(p[i]))
    active = set(base)
    admitted, taken = [], [False] * n
    while len(admitted) < max_nodes:
        best, best_u = -1, -1.0
        for i in range(n):
            if taken[i] or (parents[i] >= 0 and not taken[parents[i]]):
                continue
            benefit = conf[i] * t_ar
            cost = len(set(experts[i]) - active) * t_exp + float(c_draft[i])
            if benefit <= 0.0:
                u = 0.0
            elif cost <= 0.0:
                u = float("inf")
            else:
                u = benefit / cost
            if u > best_u:
                best, best_u = i, u
        if best < 0 or best_u < 1.0:
            break
        taken[best] = True
        admitted.append(best)
        active |= set(experts[best])
    return admitted


def tree_rows(parents, admitted):
    """The verification tree of the admitted candidates: row 0 the root,
    row r the candidate admitted r-th.  Returns the rows' parent array."""
    row_of = {c: r + 1 for r, c in enumerate(admitted)}
    return [-1] + [0 if parents[c] < 0 else row_of[parents[c]] for c in admitted]
