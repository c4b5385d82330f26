"""Self-speculative drafting of a MoE target by expert sparsity (S2-MoE,
section 2.3 and section 5 "Draft configuration", Table 1: the same model
with fewer routed experts per token drafts for itself; section 4.3: the
draft reads the target's cache and its cache writes are temporary).

- Draft tokens and draft logits through the C ABI (spec_draft) against the
  oracle's draft_greedy on the same state: logits within the logit
  tolerance, tokens identical up to the first divergence, which must sit on
  a near-tie (top-2 logit gap of that draft pass, or a router gap at the
  draft's top-k boundary, below the tolerance).
- A draft that keeps all top_k experts is the target: its tokens equal the
  GPU's own greedy decode bitwise, and the committed length never moves.
- Speculative rounds with self-drafted blocks: each verification outcome
  equals the oracle's verification of the same block, and the emitted
  sequence is the target's greedy decode (essay "LLM Inference:
  Speculative Decoding", "The output does not change").  The acceptance
  rate of the self-draft is logged and recorded."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from gpu_common import log, logit_tol, make_verifier, record  # noqa: E402
from oracle import accept as oacc  # noqa: E402
from oracle import model as om  # noqa: E402
from spec_harness import RoundInputs, oracle_step, prepare, prepare_full  # noqa: E402
from target_model_verification_amd import binding as B  # noqa: E402
from target_model_verification_amd import synth  # noqa: E402

N_DRAFT = 8


def _near_tie(logits_row, routing, kd, tol):
    if oacc.top2_gap(logits_row) < tol:
        return True
    return any(float(np.min(r["topk_gap"])) < tol for r in routing)


def _compare_draft(pw, gpu_toks, gpu_logits, ref_toks, ref_logits, ref_routing, kd):
    """Returns the number of agreeing draft tokens; asserts the rules above."""
    tol = logit_tol(pw.wl.spec)
    for i in range(len(ref_toks)):
        err = float(np.max(np.abs(gpu_logits[i] - ref_logits[i])))
        assert err <= tol, f"draft pass {i}: logits max err {err:.3e} > {tol}"
        if gpu_toks[i] != ref_toks[i]:
            assert _near_tie(ref_logits[i], ref_routing[i], kd, tol), \
                f"draft token {i}: GPU {gpu_toks[i]} != oracle {ref_toks[i]} (no near-tie)"
            return i
    return len(ref_toks)


@pytest.fixture(scope="module")
def moe():
    pw = prepare(synth.ALL_WORKLOADS["small_moe"])
    h = make_verifier(pw, max_k=15)
    yield pw, h
    h.close()


@pytest.mark.parametrize("kd", [1, 2, 6])
def test_draft_matches_oracle(moe, kd):
    pw, h = moe
    V = pw.wl.spec.vocab
    L = h.kv_len
    lg = torch.empty((N_DRAFT, V), dtype=torch.float32, device="cuda")
    toks = h.draft(pw.pending0, N_DRAFT, kd, lg.data_ptr())
    assert h.kv_len == L
    ref_toks, ref_logits, ref_routing = om.draft_greedy(pw.M, pw.kv0, pw.pending0, N_DRAFT, kd)
    agree = _compare_draft(pw, toks, lg.cpu().numpy(), list(ref_toks), ref_logits, ref_routing, kd)
    log(f"[self draft] small_moe top-{kd}: {agree}/{N_DRAFT} draft tokens identical, drafts {toks}")


def test_draft_routes_match_oracle(moe):
    """The experts each draft pass routed its token to (route_dev of
    spec_draft) against the oracle's selection, per layer as sets, for every
    pass whose input token agrees; a difference must sit on a router near-tie
    at the draft's top-k boundary."""
    pw, h = moe
    spec = pw.wl.spec
    kd = 2
    lg = torch.empty((N_DRAFT, spec.vocab), dtype=torch.float32, device="cuda")
    rt = torch.full((N_DRAFT, spec.n_layers, kd), -1, dtype=torch.int32, device="cuda")
    toks = h.draft(pw.pending0, N_DRAFT, kd, lg.data_ptr(), rt.data_ptr())
    ref_toks, ref_logits, ref_routing = om.draft_greedy(pw.M, pw.kv0, pw.pending0, N_DRAFT, kd)
    agree = _compare_draft(pw, toks, lg.cpu().numpy(), list(ref_toks), ref_logits, ref_routing, kd)
    routes = rt.cpu().numpy()
    for i in range(min(agree + 1, N_DRAFT)):
        for l in range(spec.n_layers):
            want = sorted(int(e) for e in ref_routing[i][l]["sel"][0])
            got = sorted(int(e) for e in routes[i, l])
            if got != want:
                assert float(ref_routing[i][l]["topk_gap"][0]) < 1e-3, f"pass {i} layer {l}: {got} != {want}"


def test_full_expert_draft_is_the_gpu_greedy_decode(moe):
    pw, h = moe
    L = h.kv_len
    toks = h.draft(pw.pending0, N_DRAFT, pw.wl.spec.top_k)
    assert h.kv_len == L
    ar, tok = [], pw.pending0
    for _ in range(N_DRAFT):
        r = h.step([tok], B.SPEC_ACCEPT_GREEDY)
        tok = r.next_token
        ar.append(tok)
    h.rollback(L)
    assert toks == ar


def test_bad_draft_calls(moe):
    pw, h = moe
    L = h.kv_len
    for pending, n, kd in ((pw.pending0, 0, 1), (pw.pending0, 17, 1), (pw.pending0, 4, 0),
                           (pw.pending0, 4, pw.wl.spec.top_k + 1), (pw.wl.spec.vocab, 4, 1)):
        with pytest.raises(B.SpecError) as e:
            h.draft(pending, n, kd)
        assert e.value.code == B.SPEC_EINVAL
    assert h.kv_len == L
    dense = prepare(synth.ALL_WORKLOADS["small_bf16"])
    hd = make_verifier(dense, max_k=4)
    try:
        with pytest.raises(B.SpecError) as e:
            hd.draft(dense.pending0, 4, 1)
        assert e.value.code == B.SPEC_EINVAL
    finally:
        hd.close()


def _self_spec_rounds(pw, h, kd, rounds, tag):
    """Self-drafted verification rounds on both sides; returns the
    statistics (the emitted sequence is checked against the oracle's greedy
    decode)."""
    spec = pw.wl.spec
    tol = logit_tol(spec)
    kv = pw.kv0.copy()
    pending = pw.pending0
    ref = om.ar_decode(pw.M, pw.kv0, pw.pending0, rounds * (N_DRAFT + 1) + 1)
    emitted = []
    st = dict(rounds=0, accepted=0, draft_agree=0, flagged=0, flagged_mismatch=0, max_err=0.0)
    V = spec.vocab
    for r in range(rounds):
        L = kv.length
        assert h.kv_len == L
        dl = torch.empty((N_DRAFT, V), dtype=torch.float32, device="cuda")
        drafts = h.draft(pending, N_DRAFT, kd, dl.data_ptr())
        ref_toks, ref_dl, ref_routing = om.draft_greedy(pw.M, kv, pending, N_DRAFT, kd)
        st["draft_agree"] += _compare_draft(pw, drafts, dl.cpu().numpy(), list(ref_toks), ref_dl, ref_routing, kd)
        # the oracle verifies the GPU's own block (drafts are inputs)
        ri = RoundInputs(np.asarray([pending] + drafts, np.int32))
        out_o, res_o = oracle_step(pw, kv, ri, "greedy", tol)
        lg = torch.empty((N_DRAFT + 1, V), dtype=torch.float32, device="cuda")
        res = h.step(ri.tokens, B.SPEC_ACCEPT_GREEDY, 0, 0, lg.data_ptr())
        err = float(np.max(np.abs(lg.cpu().numpy() - res_o.logits)))
        st["max_err"] = max(st["max_err"], err)
        assert err <= tol
        got = (res.n_accepted, res.next_token, res.kv_len)
        want = (out_o.n_accepted, out_o.next_token, out_o.kv_len)
        st["flagged"] += int(out_o.near_tie)
        if got != want:
            assert out_o.near_tie, f"round {r}: GPU {got} != oracle {want} (no near-tie)"
            st["flagged_mismatch"] += 1
            h.rollback(L)
            h.step(ri.tokens[:1 + out_o.n_accepted], B.SPEC_ACCEPT_NONE)
        emitted += [int(t) for t in ri.tokens[1:1 + out_o.n_accepted]] + [out_o.next_token]
        st["accepted"] += out_o.n_accepted
        st["rounds"] += 1
        pending = out_o.next_token
    if st["flagged_mismatch"] == 0:
        assert emitted == [int(t) for t in ref[:len(emitted)]], "self-speculative output differs from greedy decode"
    st["mean_accepted_drafts"] = st["accepted"] / rounds
    record(dict(workload=spec.name, k=N_DRAFT, mode="greedy", tag=tag, draft_top_k=kd, tol=tol, **st))
    return st


@pytest.mark.parametrize("kd", [1, 2])
def test_self_speculative_rounds(kd):
    pw = prepare(synth.ALL_WORKLOADS["small_moe"])
    h = make_verifier(pw, max_k=15)
    try:
        st = _self_spec_rounds(pw, h, kd, 8, "self-draft")
        log(f"[self draft] small_moe top-{kd} rounds: {st}")
    finally:
        h.close()


@pytest.mark.timeout(600)
def test_self_speculative_full_moe():
    wl = synth.WORKLOADS["moe"]
    pw = prepare_full(wl, max_ctx=wl.context + 4 * (N_DRAFT + 1) + 64)
    h = make_verifier(pw, max_k=15)
    try:
        st = _self_spec_rounds(pw, h, 1, 4, "self-draft-full")
        log(f"[self draft] moe (full size) top-1 rounds: {st}")
    finally:
        h.close()
