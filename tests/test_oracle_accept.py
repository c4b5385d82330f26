"""Pins for the acceptance rules and counters (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import accept as oa
from oracle import accounting as oc
from oracle import numerics as nx

GOLD = os.path.join(os.path.dirname(__file__), "golden", "essay_counters.json")


def _logits_with_argmax(argmaxes, V, rng, margin=1.0):
    z = rng.standard_normal((len(argmaxes), V))
    for j, a in enumerate(argmaxes):
        z[j, a] = z[j].max() + margin
    return z


def test_greedy_prefix_semantics():
    rng = np.random.default_rng(0)
    a = [3, 1, 4, 1, 5]                      # target's choices after t_0..t_4
    z = _logits_with_argmax(a, 10, rng)
    # all four drafts agree -> n=4, bonus = a_4
    o = oa.accept_greedy(z, [3, 1, 4, 1], L=100)
    assert (o.n_accepted, o.next_token, o.kv_len) == (4, 5, 105)
    # first disagreement at d_3 -> keep d_1 d_2, correction a_2
    o = oa.accept_greedy(z, [3, 1, 9, 1], L=100)
    assert (o.n_accepted, o.next_token, o.kv_len) == (2, 4, 103)
    # later agreement after a miss never counts (cumprod semantics)
    o = oa.accept_greedy(z, [0, 1, 4, 1], L=7)
    assert (o.n_accepted, o.next_token, o.kv_len) == (0, 3, 8)
    # k = 0 is one autoregressive step
    o = oa.accept_greedy(z[:1], [], L=7)
    assert (o.n_accepted, o.next_token, o.kv_len) == (0, 3, 8)


def test_greedy_ties_go_to_lowest_id_and_are_flagged():
    z = np.array([[0.0, 2.0, 2.0, 1.0], [5.0, 0.0, 0.0, 5.0]])
    o = oa.accept_greedy(z, [1], L=0, tol=1e-3)
    assert (o.n_accepted, o.next_token) == (1, 0)
    assert o.near_tie


def test_expected_tokens_closed_form_vs_simulation():
    # per-token agreement a = 1 - c(1 - 1/V); E[n_acc + 1] = (1 - a^(k+1))/(1 - a)
    rng = np.random.default_rng(1)
    V, k, c, n = 16, 4, 0.3, 20000
    truth = rng.integers(0, V, size=(n, k + 1))
    samples = []
    for r in range(n):
        z = _logits_with_argmax(truth[r], V, rng)
        d = truth[r, :k].copy()
        flip = rng.random(k) < c
        d[flip] = rng.integers(0, V, size=flip.sum())
        samples.append(oa.accept_greedy(z, d, 0).n_accepted + 1)
    a = oc.acceptance_rate_from_corruption(c, V)
    mu = oc.expected_tokens_per_round(a, k)
    s = np.asarray(samples, float)
    assert abs(s.mean() - mu) < 4 * s.std() / np.sqrt(n)
    # worked by hand: a = 0.71875, a^5 = 0.19183, (1 - a^5)/(1 - a) = 2.8735
    assert abs(mu - 2.8735) < 1e-3
    # tiny workload (V = 2048, k = 4, c = 0.3): a = 0.700146, 2.774 tokens/round
    assert abs(oc.expected_tokens_per_round(oc.acceptance_rate_from_corruption(0.3, 2048), 4) - 2.774) < 1e-3


def test_essay_acceptance_figures():
    g = json.load(open(GOLD))["acceptance"]
    a = g["a"]
    assert round(oc.acceptance_ceiling(a), 1) == g["ceiling_1dp"]
    assert round(100 * a ** 4) == g["four_in_a_row_pct"]
    assert round(100 * a ** 8) == g["eight_in_a_row_pct"]
    # the ceiling is approached from below as k grows
    assert oc.expected_tokens_per_round(a, 16) < oc.acceptance_ceiling(a)
    assert oc.expected_tokens_per_round(a, 0) == 1.0


def test_essay_run_counters():
    g = json.load(open(GOLD))
    e = g["k5"]
    # 15 rounds accepting 54 drafts in total (75 guesses - 21 discarded)
    n_acc = [4] * 9 + [3] * 6
    assert sum(n_acc) == e["guesses"] - e["discarded"]
    c = oc.run_counters(e["k"], n_acc, e["tokens"])
    for key in ("target_passes", "draft_passes", "guesses", "discarded", "target_passes_saved"):
        assert c[key] == e[key], key
    assert c["tokens"] == e["tokens"] and c["emitted"] - e["tokens"] < e["k"] + 1
    e = g["k16"]
    n_acc = [5] * 3 + [6] * 5 + [4] * 3                # 57 = 176 guesses - 119 discarded
    c = oc.run_counters(e["k"], n_acc, e["tokens"])
    assert (c["target_passes"], c["draft_passes"], c["discarded"]) == (e["target_passes"], e["draft_passes"], e["discarded"])
    assert c["emitted"] >= e["tokens"]


def _exact_first_token_dist(p, q_list, k):
    """Distribution of the first emitted token under accept_stochastic,
    computed exactly: enumerate the drafts, and integrate each uniform over
    the intervals on which the rule's decisions are constant."""
    V = p.shape[1]
    logits = np.log(p)
    dist = np.zeros(V)
    u_pts = []  # representative uniforms for u_{k+1}: midpoints of CDF cells of any relevant distribution
    for drafts in itertools.product(range(V), repeat=k):
        pd = np.prod([q_list[i][drafts[i]] for i in range(k)])
        if pd == 0:
            continue
        # thresholds for u_1..u_k
        cuts = []
        for i in range(k):
            P, Q = p[i, drafts[i]], q_list[i][drafts[i]]
            cuts.append(min(1.0, P / Q))
        # enumerate accept/reject patterns: u_i below (accept) or above the cut
        for pattern in itertools.product([True, False], repeat=k):
            w = np.prod([cuts[i] if pattern[i] else 1 - cuts[i] for i in range(k)])
            if w <= 0:
                continue
            u = np.array([cuts[i] / 2 if pattern[i] else (1 + cuts[i]) / 2 for i in range(k)] + [0.0])
            # integrate u_{k+1} over the CDF cells of whichever row is sampled
            first_rej = next((i for i in range(k) if not pattern[i]), None)
            if first_rej is None:
                r = p[k]
            else:
                r = np.maximum(0, p[first_rej] - q_list[first_rej])
                if r.sum() <= 0:
                    r = p[first_rej]
            C = np.concatenate([[0.0], np.cumsum(r) / r.sum()])
            for x in range(V):
                cell = C[x + 1] - C[x]
                if cell <= 0:
                    continue
                u[k] = (C[x] + C[x + 1]) / 2
                o = oa.accept_stochastic(logits, np.stack(q_list), list(drafts), u, L=0)
                first = drafts[0] if o.n_accepted >= 1 else o.next_token
                dist[first] += pd * w * cell
    return dist


@pytest.mark.parametrize("k", [1, 2])
def test_stochastic_rule_preserves_target_distribution(k):
    rng = np.random.default_rng(2 + k)
    V = 8 if k == 1 else 5
    p = nx.softmax(rng.standard_normal((k + 1, V)) * 1.5)
    q_list = [nx.softmax(rng.standard_normal(V) * 1.5) for _ in range(k)]
    dist = _exact_first_token_dist(p, q_list, k)
    assert np.allclose(dist, p[0], atol=1e-12), (dist, p[0])


def test_stochastic_special_cases():
    rng = np.random.default_rng(9)
    V, k = 12, 3
    p = nx.softmax(rng.standard_normal((k + 1, V)))
    logits = np.log(p)
    # q = p: every draft is accepted (u < 1 = p/q) and the bonus comes from p_k
    u = np.array([0.999, 0.5, 0.0, 0.37])
    o = oa.accept_stochastic(logits, p[:k], [1, 2, 3], u, L=10)
    assert o.n_accepted == 3 and o.kv_len == 14
    assert o.next_token == oa.inverse_cdf(p[k], 0.37)[0]
    # disjoint supports: q puts mass only where p is tiny -> reject at i=1,
    # resample from max(0, p - q) which is p restricted off q's support
    q = np.zeros((k, V))
    q[:, 0] = 1.0
    p2 = p.copy()
    p2[:, 0] = 0.0
    p2 /= p2.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore"):
        z2 = np.log(p2)                                   # -inf where p = 0
    o = oa.accept_stochastic(z2, q, [0, 0, 0], np.array([0.0, 0, 0, 0.6]), L=5)
    assert o.n_accepted == 0 and o.kv_len == 6
    assert o.next_token == oa.inverse_cdf(p2[0], 0.6)[0] and o.next_token != 0


def test_inverse_cdf_definition():
    w = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert oa.inverse_cdf(w, 0.0)[0] == 1
    assert oa.inverse_cdf(w, 0.2499)[0] == 1
    assert oa.inverse_cdf(w, 0.25)[0] == 3        # C(1) = 0.25 is not > 0.25
    assert oa.inverse_cdf(w, 0.7499)[0] == 3
    assert oa.inverse_cdf(w, 0.75)[0] == 4
    assert oa.inverse_cdf(w * 3, 0.9999)[0] == 4


def test_accept_none():
    z = np.zeros((3, 4))
    z[2, 3] = 1
    o = oa.accept_none(z, 2, 10)
    assert (o.n_accepted, o.next_token, o.kv_len) == (2, 3, 13)
