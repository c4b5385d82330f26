"""Token-tree verification through the C ABI (spec_verify_tree; S2-MoE
section 4.1: the draft tree's candidates verified in one target pass).

- A chain-shaped tree is the ordinary verification step: logits bitwise
  identical, same outcome, same cache (the tree pass shares every
  arithmetic step with the block pass; only the mask and the rotary
  positions are read from the tree).
- Seeded random trees, each holding the greedy continuation on one branch
  among random decoys, over several rounds: every node's logits against the
  oracle's tree_logits (a plain block pass over the node's path) within the
  logit tolerance; the GPU's accepted path against the walk applied to its
  own logits exactly; against the oracle's walk unless the oracle flags a
  near-tie; the next round runs on the compacted cache, so its logits check
  the commit's moves.
- Malformed trees are rejected before any device work.
- At full size on the MoE workload: one tree of 12 nodes against the
  oracle in float32 on the synthetic prompt cache."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from gpu_common import log, logit_tol, make_verifier, record  # noqa: E402
from oracle import accept as oacc  # noqa: E402
from oracle import model as om  # noqa: E402
from oracle import tree as otree  # noqa: E402
from spec_harness import prepare, prepare_full  # noqa: E402
from target_model_verification_amd import binding as B  # noqa: E402
from target_model_verification_amd import synth  # noqa: E402


def _tree_step(h, tokens, parents, V):
    lg = torch.empty((len(tokens), V), dtype=torch.float32, device="cuda")
    res, path = h.step_tree(tokens, parents, lg.data_ptr())
    torch.cuda.synchronize()
    return res, path, lg.cpu().numpy()


def _make_tree(rng, pending, greedy, m, V):
    """Root = pending; the greedy continuation grows as one branch while
    random decoys attach anywhere (rows stay in topological order)."""
    tokens, parents, gpath = [int(pending)], [-1], [0]
    gi = 0
    while len(tokens) < m:
        if gi < len(greedy) and rng.random() < 0.45:
            tokens.append(int(greedy[gi]))
            parents.append(gpath[-1])
            gpath.append(len(tokens) - 1)
            gi += 1
        else:
            parents.append(int(rng.integers(0, len(tokens))))
            tokens.append(int(rng.integers(0, V)))
    return tokens, parents


@pytest.mark.parametrize("name", ["small_gqa", "small_moe", "small_int4"])
def test_chain_tree_is_the_block_step(name):
    pw = prepare(synth.ALL_WORKLOADS[name])
    h = make_verifier(pw, max_k=15)
    try:
        V = pw.wl.spec.vocab
        L = h.kv_len
        rng = np.random.default_rng(1)
        ref = om.ar_decode(pw.M, pw.kv0, pw.pending0, 6)
        for k in (0, 3, 8, 15):
            toks = [pw.pending0] + [int(t) for t in ref[:min(k, 4)]] + [int(t) for t in rng.integers(0, V, k - min(k, 4))]
            parents = [-1] + list(range(k))
            res_t, path, lg_t = _tree_step(h, toks, parents, V)
            h.rollback(L)
            lg_c = torch.empty((k + 1, V), dtype=torch.float32, device="cuda")
            res_c = h.step(toks, B.SPEC_ACCEPT_GREEDY, 0, 0, lg_c.data_ptr())
            torch.cuda.synchronize()
            assert np.array_equal(lg_t, lg_c.cpu().numpy()), f"k={k}: tree logits differ from the block step"
            assert (res_t.n_accepted, res_t.next_token, res_t.kv_len) == \
                (res_c.n_accepted, res_c.next_token, res_c.kv_len)
            assert path == list(range(1, 1 + res_t.n_accepted))
            h.rollback(L)
    finally:
        h.close()


@pytest.mark.parametrize("name", ["small_f32", "small_bf16", "small_gqa", "small_moe", "small_int4"])
def test_random_trees_match_the_oracle(name):
    pw = prepare(synth.ALL_WORKLOADS[name])
    spec = pw.wl.spec
    V, tol = spec.vocab, logit_tol(spec)
    h = make_verifier(pw, max_k=15)
    rng = np.random.default_rng(17)
    kv = pw.kv0.copy()
    pending = pw.pending0
    st = dict(rounds=0, accepted=0, max_err=0.0, flagged=0, flagged_mismatch=0, nodes=0)
    try:
        for r in range(6):
            L = kv.length
            assert h.kv_len == L
            m = int(rng.integers(2, 17))
            greedy = om.ar_decode(pw.M, kv, pending, 8)
            tokens, parents = _make_tree(rng, pending, greedy, m, V)
            want_lg = otree.tree_logits(pw.M, kv, tokens, parents, L)
            out_o, path_o = otree.accept_tree_greedy(want_lg, tokens, parents, L, tol)
            res, path, lg = _tree_step(h, tokens, parents, V)
            err = float(np.max(np.abs(lg - want_lg)))
            st["max_err"] = max(st["max_err"], err)
            assert err <= tol, f"{name} round {r} (m={m}): tree logits max err {err:.3e} > {tol}"
            own, own_path = otree.accept_tree_greedy(lg, tokens, parents, L)
            got = (res.n_accepted, res.next_token, res.kv_len)
            assert got == (own.n_accepted, own.next_token, own.kv_len) and path == own_path, \
                f"{name} round {r}: GPU {got} {path} != walk on its own logits {own} {own_path}"
            st["flagged"] += int(out_o.near_tie)
            if (got, path) != ((out_o.n_accepted, out_o.next_token, out_o.kv_len), path_o):
                assert out_o.near_tie, f"{name} round {r}: GPU {got} {path} != oracle {out_o} {path_o} (no near-tie)"
                st["flagged_mismatch"] += 1
                # resync the GPU to the oracle's outcome
                h.rollback(L)
                h.step([tokens[0]] + [tokens[i] for i in path_o], B.SPEC_ACCEPT_NONE)
            otree.commit_tree(pw.M, kv, tokens, path_o, L)
            assert h.kv_len == kv.length
            pending = out_o.next_token
            st["rounds"] += 1
            st["accepted"] += out_o.n_accepted
            st["nodes"] += m
        # the compacted cache: one more ordinary step against the oracle
        L = kv.length
        lg = torch.empty((1, V), dtype=torch.float32, device="cuda")
        h.step([pending], B.SPEC_ACCEPT_NONE, 0, 0, lg.data_ptr())
        torch.cuda.synchronize()
        ref = om.forward_block(pw.M, kv, [pending], L).logits
        assert float(np.max(np.abs(lg.cpu().numpy() - ref))) <= tol
    finally:
        h.close()
    log(f"[tree] {name}: {st}")
    record(dict(workload=name, tag="tree", tol=tol, **st))


def test_malformed_trees_are_rejected():
    pw = prepare(synth.ALL_WORKLOADS["small_bf16"])
    h = make_verifier(pw, max_k=6)
    try:
        L = h.kv_len
        t = [pw.pending0, 1, 2, 3]
        for parents in ([0, 0, 1, 2], [-1, 1, 1, 2], [-1, 0, 3, 2], [-1, -1, 0, 1]):
            with pytest.raises(B.SpecError) as e:
                h.step_tree(t, parents)
            assert e.value.code == B.SPEC_EINVAL
        with pytest.raises(B.SpecError) as e:
            h.step_tree([pw.pending0] * 8, [-1] + list(range(7)))      # m > max_k + 1
        assert e.value.code == B.SPEC_EINVAL
        with pytest.raises(B.SpecError) as e:
            h.step_tree([pw.pending0, pw.wl.spec.vocab], [-1, 0])
        assert e.value.code == B.SPEC_EINVAL
        assert h.kv_len == L
        res, path = h.step_tree([pw.pending0], [-1])                  # the root alone
        assert res.n_accepted == 0 and path == [] and h.kv_len == L + 1
    finally:
        h.close()


def test_full_size_moe_tree():
    wl = synth.ALL_WORKLOADS["moe"]
    pw = prepare_full(wl, max_ctx=wl.context + 64)
    spec = pw.wl.spec
    V, tol = spec.vocab, logit_tol(spec)
    h = make_verifier(pw, max_k=15, max_ctx=pw.max_ctx)
    try:
        rng = np.random.default_rng(23)
        greedy = om.ar_decode(pw.M, pw.kv0, pw.pending0, 5)
        tokens, parents = _make_tree(rng, pw.pending0, greedy, 12, V)
        want = otree.tree_logits(pw.M, pw.kv0, tokens, parents, pw.kv0.length)
        res, path, lg = _tree_step(h, tokens, parents, V)
        err = float(np.max(np.abs(lg - want)))
        assert err <= tol, f"moe full size tree: max err {err:.3e}"
        out_o, path_o = otree.accept_tree_greedy(want, tokens, parents, pw.kv0.length, tol)
        own, own_path = otree.accept_tree_greedy(lg, tokens, parents, pw.kv0.length)
        assert (res.n_accepted, res.next_token, path) == (own.n_accepted, own.next_token, own_path)
        if (res.n_accepted, res.next_token, path) != (out_o.n_accepted, out_o.next_token, path_o):
            assert out_o.near_tie
        log(f"[tree] moe full size: 12 nodes, max err {err:.2e}, accepted {path}")
        record(dict(workload="moe", tag="tree_full", tol=tol, max_err=err, nodes=12, accepted=len(path)))
    finally:
        h.close()
