"""Exact ties on the device.  The pages' greedy rule takes the argmax of a
row (essay "LLM Inference: Speculative Decoding", "The loop", step 3),
which returns the lowest token id among equal maxima; the MoE router keeps
each token's top_k experts by probability (S2-MoE section 2.1), ties to the
lower expert id.  Random weights almost never produce equal values, so these
models are built with duplicated columns:

- every LM-head column has three twins (column 2i+1 = column 2i for
  2i < V/2, and column V/2 + j = column j), one inside the same 16-column
  output tile and two in tiles far away; every row's maximum is then shared
  by four ids and the argmax must be the even id below V/2.  The model is
  small enough that every LM-head tile is reduced with the same split-K
  structure, so the twins' logits are bitwise equal on the device (checked);
- in the MoE model the router column of expert 9 equals that of expert 3
  and both get the same bias; seven experts (3, 9 and five others) carry a
  large bias, so each token picks six of those seven and the twins often
  straddle the sixth / seventh rank: then only expert 3 may be selected,
  and when both are selected expert 3 ranks first.

The device's logits are compared with the oracle's, its outcomes with the
acceptance rule on its own logits and with the oracle's, and (MoE) its
per-row expert selection, read through spec_verify_step_debug, with the
oracle's routing."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from gpu_common import log, make_verifier, run_parity_rounds  # noqa: E402
from oracle import model as om  # noqa: E402
from spec_harness import prepare  # noqa: E402
from target_model_verification_amd import binding as B  # noqa: E402
from target_model_verification_amd import synth  # noqa: E402

V = 1024
TIE_DENSE = synth.ModelSpec("tie_dense", 2, 128, 2, 2, 64, 256, V, "bf16", "bf16", random_gains=True)
TIE_MOE = synth.ModelSpec("tie_moe", 2, 128, 2, 1, 64, 0, V, "bf16", "bf16", n_experts=16, top_k=6,
                          n_shared=1, d_ff_expert=128, random_gains=True)
E_LO, E_HI = 3, 9
DOMINANT = (0, E_LO, 5, E_HI, 11, 12, 14)


def _twin_lm_head(W):
    w = W["lm_head"]
    w[:, 1:V // 2:2] = w[:, 0:V // 2:2]
    w[:, V // 2:] = w[:, :V // 2]


def _twin_router(W, spec):
    for l in range(spec.n_layers):
        r = W[f"l{l}.router"]
        r[:, E_HI] = r[:, E_LO]
        b = np.full(spec.n_experts, -6.0, np.float32)
        b[list(DOMINANT)] = 6.0
        W[f"l{l}.router_bias"] = b


def _workload(spec, seed):
    return synth.Workload(spec, seed, 100, 8, (8,), 0.3, "greedy")


def _prepared(spec, seed):
    wl = _workload(spec, seed)
    W = synth.make_weights(spec, seed)
    _twin_lm_head(W)
    if spec.moe:
        _twin_router(W, spec)
    return prepare(wl, weights=W)


def _check_twins(lg):
    assert np.array_equal(lg[:, 1:V // 2:2], lg[:, 0:V // 2:2]), "same-tile twins differ on the device"
    assert np.array_equal(lg[:, V // 2:], lg[:, :V // 2]), "cross-tile twins differ on the device"


@pytest.mark.parametrize("spec,seed", [(TIE_DENSE, 3101), (TIE_MOE, 3102)])
def test_argmax_ties_lowest_id(spec, seed):
    pw = _prepared(spec, seed)
    h = make_verifier(pw, max_k=8)
    try:
        L = h.kv_len
        toks = [pw.pending0] + [int(t) for t in synth.prompt_ids(pw.wl, 9)[1:]]
        lg = torch.empty((9, V), dtype=torch.float32, device="cuda")
        res = h.step(toks, B.SPEC_ACCEPT_NONE, 0, 0, lg.data_ptr())
        h.rollback(L)
        a = lg.cpu().numpy()
        _check_twins(a)
        assert res.next_token == int(np.argmax(a[-1])) and res.next_token % 2 == 0 and res.next_token < V // 2
        ref = np.concatenate([[pw.pending0], om.ar_decode(pw.M, pw.kv0, pw.pending0, 16 * 9 + 1)])
        assert np.all(ref[1:] % 2 == 0) and np.all(ref[1:] < V // 2)
        st = run_parity_rounds(pw, h, 8, 16, "greedy", ref, tag="ties")
        log(f"[ties] {spec.name}: {st}")
        assert st["rounds"] == 16 and st["accepted"] > 0
    finally:
        h.close()


def test_router_ties_lower_expert():
    spec = TIE_MOE
    pw = _prepared(spec, 3103)
    h = make_verifier(pw, max_k=8)
    K6 = spec.top_k
    straddle = both = 0
    try:
        kv = pw.kv0.copy()
        g = np.random.default_rng([3103, 5])
        for r in range(12):
            L = h.kv_len
            assert L == kv.length
            toks = np.asarray([pw.pending0] + list(g.integers(0, V, size=8)), np.int32)
            route = torch.zeros((spec.n_layers, 9, K6), dtype=torch.int32, device="cuda")
            lg = torch.empty((9, V), dtype=torch.float32, device="cuda")
            h.step(toks, B.SPEC_ACCEPT_NONE, 0, 0, lg.data_ptr(), route_ptr=route.data_ptr())
            ref = om.forward_block(pw.M, kv, toks, L)
            kv.length = L + 9
            assert np.max(np.abs(lg.cpu().numpy() - ref.logits)) <= 2e-2
            sel = route.cpu().numpy()
            for l in range(spec.n_layers):
                info = ref.routing[l]
                for j in range(9):
                    got = [int(e) for e in sel[l, j]]
                    want = [int(e) for e in info["sel"][j]]
                    if E_LO in want and E_HI not in want:
                        straddle += 1
                    if E_LO in want and E_HI in want:
                        both += 1
                        assert want.index(E_LO) + 1 == want.index(E_HI)
                    # exact ties are decided by the rule on both sides; other
                    # near-equal router logits may be ordered differently
                    # within fp32 rounding
                    if sorted(got) != sorted(want):
                        assert 0.0 < info["topk_gap"][j] < 1e-3, (l, j, got, want)
                        continue
                    assert E_HI not in got or E_LO in got, (l, j, got)
                    if E_LO in got and E_HI in got:
                        assert got.index(E_LO) + 1 == got.index(E_HI), (l, j, got)
        log(f"[ties] router: {straddle} rows with the twins split at the top-{K6} boundary, {both} with both")
        assert straddle > 0 and both > 0
    finally:
        h.close()
