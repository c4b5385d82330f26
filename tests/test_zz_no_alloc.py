"""spec_verify_step_noalloc, the step for callers that cannot allocate,
against spec_verify_step: two handles start from the same state; one steps
through the regular entry point, the other through the no-alloc one (split-K
partials and tickets in the library's fixed device scratch).  Two calls in
a row, the second with a smaller block, must give bitwise equal logits and
identical outcomes (the same kernels with the same summation order)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from gpu_common import log, make_verifier  # noqa: E402
from spec_harness import prepare  # noqa: E402
from target_model_verification_amd import binding as B  # noqa: E402
from target_model_verification_amd import synth  # noqa: E402


def _step(h, toks, noalloc):
    lg = torch.full((len(toks), h.spec.vocab), float("nan"), dtype=torch.float32, device="cuda")
    res = h.step(toks, B.SPEC_ACCEPT_GREEDY, 0, 0, lg.data_ptr(), noalloc=noalloc)
    return (res.n_accepted, res.next_token, res.kv_len), lg.cpu().numpy()


@pytest.mark.parametrize("name", ["small_bf16", "small_moe", "small_int4"])
def test_noalloc_matches_regular_step(name):
    pw = prepare(synth.ALL_WORKLOADS[name])
    ha = make_verifier(pw, max_k=15)
    hb = make_verifier(pw, max_k=15)
    try:
        g = np.random.default_rng([pw.wl.seed, 97])
        pa = pb = pw.pending0
        for k in (12, 3):   # the second call with a smaller block
            drafts = [int(t) for t in g.integers(0, pw.wl.spec.vocab, size=k)]
            ra, la = _step(ha, [pa] + drafts, False)
            rb, lb = _step(hb, [pb] + drafts, True)
            assert np.all(np.isfinite(lb))
            assert np.array_equal(la, lb), f"{name} k={k}: max diff {np.max(np.abs(la - lb))}"
            assert ra == rb
            pa, pb = ra[1], rb[1]
        assert ha.kv_len == hb.kv_len
        log(f"[noalloc] {name}: two steps bitwise equal to the regular entry point")
    finally:
        ha.close()
        hb.close()
