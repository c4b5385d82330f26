"""GPU-side test driver: runs the library through its C ABI on the same
seeded inputs as the oracle and compares element by element."""
from __future__ import annotations

import sys
from typing import Optional

import numpy as np
import torch

from oracle import model as om
from spec_harness import (PreparedWorkload, RoundInputs, greedy_round_inputs, kv_to_host_arrays,
                          oracle_step, stochastic_round_inputs)
from target_model_verification_amd import binding as B

MODE = {"greedy": B.SPEC_ACCEPT_GREEDY, "stochastic": B.SPEC_ACCEPT_STOCHASTIC, "none": B.SPEC_ACCEPT_NONE}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def logit_tol(spec) -> float:
    return 1e-4 if spec.weight_dtype == "f32" else 2e-2


def make_verifier(pw: PreparedWorkload, max_k: int, gemm_k_split: int = 0, max_ctx: Optional[int] = None):
    K, V = kv_to_host_arrays(pw)
    stream = torch.cuda.current_stream().cuda_stream
    return B.Verifier(pw.wl.spec, pw.W, K, V, pw.kv0.length, max_ctx or pw.max_ctx, max_k, stream, gemm_k_split)


def gpu_step(h: B.Verifier, ri: RoundInputs, mode: str, vocab: int, trace_layers: int = 0):
    m = len(ri.tokens)
    logits = torch.empty((m, vocab), dtype=torch.float32, device="cuda")
    q_ptr = u_ptr = 0
    keep = []
    if mode == "stochastic":
        qt = torch.from_numpy(np.ascontiguousarray(ri.q, np.float32)).cuda()
        ut = torch.from_numpy(np.ascontiguousarray(ri.u, np.float32)).cuda()
        keep += [qt, ut]
        q_ptr, u_ptr = qt.data_ptr(), ut.data_ptr()
    trace = None
    tptr = 0
    if trace_layers:
        trace = torch.empty((trace_layers, m, h.spec.d_model), dtype=torch.float32, device="cuda")
        tptr = trace.data_ptr()
    res = h.step(ri.tokens, MODE[mode], q_ptr, u_ptr, logits.data_ptr(), trace_ptr=tptr)
    torch.cuda.synchronize()
    return res, logits.cpu().numpy(), (trace.cpu().numpy() if trace is not None else None)


def layer_errors(pw: PreparedWorkload, h: B.Verifier, kv: om.KVCache, ri: RoundInputs, mode: str):
    """Per-layer max |GPU residual - oracle residual| for one block (debug aid;
    leaves both caches at their committed length)."""
    L = kv.length
    scratch = kv.copy()
    ref = om.forward_block(pw.M, scratch, ri.tokens, L, trace=True)
    _, lg, tr = gpu_step(h, ri, "none", pw.wl.spec.vocab, trace_layers=pw.wl.spec.n_layers)
    h.rollback(L)
    errs = [float(np.max(np.abs(tr[l] - ref.trace[l]))) for l in range(pw.wl.spec.n_layers)]
    errs.append(float(np.max(np.abs(lg - ref.logits))))
    return errs


def run_parity_rounds(pw: PreparedWorkload, h: B.Verifier, k: int, rounds: int, mode: str,
                      greedy_ref: Optional[np.ndarray] = None, c=None):
    """Runs `rounds` verification steps on both sides from the same state and
    checks: logits within tolerance; n_accepted / next / kv_len identical
    unless the oracle flags a near-tie (then both resync to the oracle)."""
    spec = pw.wl.spec
    tol = logit_tol(spec)
    kv = pw.kv0.copy()
    pending = pw.pending0
    s = 0
    st = dict(max_err=0.0, flagged=0, flagged_mismatch=0, accepted=0, rounds=0)
    for r in range(rounds):
        L = kv.length
        assert h.kv_len == L
        if mode == "greedy":
            ri = greedy_round_inputs(pw.wl, r, pending, greedy_ref[s + 1:s + 1 + k], c)
        else:
            ri = stochastic_round_inputs(pw, kv, r, pending, k)
        kv_before = kv.copy()
        out_o, res_o = oracle_step(pw, kv, ri, mode, tol)
        res_g, lg, _ = gpu_step(h, ri, mode, spec.vocab)
        err = float(np.max(np.abs(lg - res_o.logits)))
        st["max_err"] = max(st["max_err"], err)
        if err > tol:
            h.rollback(L)
            errs = layer_errors(pw, h, kv_before, ri, mode)
            raise AssertionError(f"{spec.name} round {r}: logits max err {err:.3e} > {tol}; "
                                 f"per-layer residual errors {['%.2e' % e for e in errs]}")
        got = (res_g.n_accepted, res_g.next_token, res_g.kv_len)
        want = (out_o.n_accepted, out_o.next_token, out_o.kv_len)
        if out_o.near_tie:
            st["flagged"] += 1
        if got != want:
            assert out_o.near_tie, f"{spec.name} round {r}: GPU {got} != oracle {want} (no near-tie)"
            st["flagged_mismatch"] += 1
            h.rollback(L)
            h.step(ri.tokens[:1 + out_o.n_accepted], B.SPEC_ACCEPT_NONE)
        assert h.kv_len == kv.length == out_o.kv_len
        st["accepted"] += out_o.n_accepted
        st["rounds"] += 1
        pending = out_o.next_token
        s += out_o.n_accepted + 1
    return st
