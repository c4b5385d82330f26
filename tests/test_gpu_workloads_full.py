"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (max_k = 15, default split-K): the LLaMA-2-7B-shaped bf16
target over its whole k sweep (1, 2, 4, 8, 15), its int4 group-128
quantization, the 64-expert MoE, and the Qwen2.5-7B-shaped GQA target with
stochastic acceptance, 8 verification rounds per k.

Both sides start from the same seeded synthetic prompt cache of the
workload's full context length (a CPU prefill at this scale is beyond the
oracle's budget; see spec_harness.prepare_full) and run a few verification
rounds on identical drafts.  Every logit of every round is compared with
the float32 oracle (max-abs <= 2e-2); the accepted count, next token and
cache length must agree exactly with the oracle's unless the oracle flags a
near-tie, and always with the acceptance rule applied to the GPU's own
logits (stochastic: up to fp32 rounding of the decision).  The
nesting invariant (essay "LLM Inference: Speculative Decoding", "The four
sentences are already inside one sentence") is checked bitwise on the GPU at
7B size."""
import gc

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from gpu_common import log, make_verifier, run_parity_rounds  # noqa: E402
from oracle import model as om  # noqa: E402
from spec_harness import prepare_full  # noqa: E402
from target_model_verification_amd import binding as B  # noqa: E402
from target_model_verification_amd import synth  # noqa: E402

# (workload, k values, rounds per k).  The LLaMA-2-7B shape runs its whole k
# sweep; every config runs 8 rounds per k.
CASES = [("llama7b", (1, 2, 4, 8, 15), 8), ("llama7b_int4", (8,), 8), ("moe", (8,), 8), ("qwen7b", (10,), 8)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,ks,rounds", CASES)
def test_full_size_parity(name, ks, rounds):
    wl = synth.WORKLOADS[name]
    log(f"[full] {name}: preparing weights, oracle and synthetic prompt cache ({wl.context} positions)")
    pw = prepare_full(wl, max_ctx=wl.context + rounds * (max(ks) + 1) + 64)
    h = make_verifier(pw, max_k=15)
    try:
        log(f"[full] {name}: verifier ready")
        if name == "llama7b":
            L = h.kv_len
            toks = [pw.pending0] + list(synth.prompt_ids(wl, 9)[1:])
            full = torch.empty((9, wl.spec.vocab), dtype=torch.float32, device="cuda")
            h.step(toks, B.SPEC_ACCEPT_GREEDY, 0, 0, full.data_ptr())
            h.rollback(L)
            for j in (0, 3, 8):
                part = torch.empty((j + 1, wl.spec.vocab), dtype=torch.float32, device="cuda")
                h.step(toks[:j + 1], B.SPEC_ACCEPT_GREEDY, 0, 0, part.data_ptr())
                h.rollback(L)
                assert torch.equal(part[j], full[j]), f"nesting broken at row {j}"
            log(f"[full] {name}: nesting bitwise at rows 0, 3, 8")
        ref = None
        if wl.accept == "greedy":
            # the target's greedy continuation is the same for every k (the
            # drafts of round r at k are a corrupted slice of it)
            n_ref = max(rounds * (k + 1) for k in ks) + 1
            ref = np.concatenate([[pw.pending0], om.ar_decode(pw.M, pw.kv0, pw.pending0, n_ref)])
            log(f"[full] {name}: oracle greedy reference of {n_ref} tokens ready")
        for k in ks:
            h.rollback(pw.kv0.length)
            st = run_parity_rounds(pw, h, k, rounds, wl.accept, ref, tag="full")
            log(f"[full] {name} k={k}: {st}")
            assert st["rounds"] == rounds
    finally:
        h.close()
        del pw
        gc.collect()
