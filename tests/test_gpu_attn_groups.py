"""Attention work items of 5- and 6-page groups (the pass picks them when
fewer, longer items fit the grid in one round; forced here through the
attn_group_pages knob on the reduced workloads, whose contexts would
otherwise always take 3-page groups): verification rounds against the
oracle, logits within the logit tolerance and outcomes exact unless a
near-tie is flagged, and the nesting invariant bitwise for a fixed group
size (a row's logits do not depend on the rows after it)."""
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

# (workload, k, group pages, prompt length: None = the workload's; the
# longer prompts give several groups to merge)
CASES = [("small_bf16", 6, 5, None), ("small_bf16", 15, 6, 800), ("small_gqa", 10, 5, 700),
         ("small_gqa", 10, 6, None), ("small_moe", 8, 6, 900), ("small_int4", 8, 5, 700)]


@pytest.mark.parametrize("name,k,gp,ctx", CASES)
def test_group_size_parity(name, k, gp, ctx):
    wl = synth.ALL_WORKLOADS[name]
    log(f"[groups] {name} k={k} group pages {gp} prompt {ctx}")
    pw = prepare(wl, context=ctx)
    h = make_verifier(pw, max_k=k, attn_group_pages=gp)
    try:
        ref = np.concatenate([[pw.pending0], om.ar_decode(pw.M, pw.kv0, pw.pending0, 8 * (k + 1) + 1)])
        st = run_parity_rounds(pw, h, k, 8, "greedy", ref, tag=f"groups{gp}")
        log(f"[groups] {name} k={k} gp={gp}: {st}")
        assert st["rounds"] == 8 and st["accepted"] > 0
    finally:
        h.close()


@pytest.mark.parametrize("gp", [5, 6])
def test_group_size_nesting(gp):
    pw = prepare(synth.ALL_WORKLOADS["small_gqa"])
    V = pw.wl.spec.vocab
    h = make_verifier(pw, max_k=15, attn_group_pages=gp)
    try:
        L = h.kv_len
        toks = [pw.pending0] + list(range(100, 115))
        full = torch.empty((16, V), dtype=torch.float32, device="cuda")
        h.step(toks, B.SPEC_ACCEPT_NONE, 0, 0, full.data_ptr())
        h.rollback(L)
        full = full.cpu().numpy()
        for m in (1, 7, 12):
            part = torch.empty((m, V), dtype=torch.float32, device="cuda")
            h.step(toks[:m], B.SPEC_ACCEPT_NONE, 0, 0, part.data_ptr())
            h.rollback(L)
            assert np.array_equal(part.cpu().numpy(), full[:m]), f"gp={gp} m={m}"
    finally:
        h.close()
