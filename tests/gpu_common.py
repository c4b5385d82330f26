"""GPU-side test driver: runs the library through its C ABI on the same
seeded inputs as the oracle and compares element by element."""
from __future__ import annotations

import json
import os
import sys
from typing import Optional

import numpy as np
import torch

from oracle import accept as oacc
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


def make_verifier(pw: PreparedWorkload, max_k: int, gemm_k_split: int = 0, max_ctx: Optional[int] = None,
                  n_seqs: int = 0, kv_page_seed: int = 0, attn_group_pages: int = 0):
    K, V = kv_to_host_arrays(pw)
    stream = torch.cuda.current_stream().cuda_stream
    return B.Verifier(pw.wl.spec, pw.W, K, V, pw.kv0.length, max_ctx or pw.max_ctx, max_k, stream, gemm_k_split,
                      kv_page_seed, n_seqs, attn_group_pages)


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


ACC_TOL = 1e-5   # fp32 (device) against fp64 (oracle) acceptance arithmetic on the same logits


def record(entry: dict) -> None:
    """Appends one JSON line of parity statistics to the file named by the
    SPEC_PARITY_RECORD environment variable (if set)."""
    path = os.environ.get("SPEC_PARITY_RECORD")
    if not path:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "a") as f:
        f.write(json.dumps(entry, sort_keys=True) + "\n")


def _valid(res, L: int, k: int, V: int) -> bool:
    return 0 <= res.n_accepted <= k and 0 <= res.next_token < V and res.kv_len == L + 1 + res.n_accepted


def run_parity_rounds(pw: PreparedWorkload, h: B.Verifier, k: int, rounds: int, mode: str,
                      greedy_ref: Optional[np.ndarray] = None, c=None, tag: str = ""):
    """Runs `rounds` verification steps on both sides from the same state.

    Every round checks:
      - logits against the oracle's, element by element, within the logit
        tolerance (1e-4 fp32, 2e-2 bf16 / int4);
      - the GPU's (n_accepted, next, kv_len) against the acceptance rule
        applied to the GPU's own logits (oracle.accept_*): greedy exactly,
        stochastic exactly unless a decision lies within a relative 1e-5 of
        flipping (fp32 on the device against fp64), then only validity;
      - the GPU's outcome against the oracle's: identical unless the oracle
        flags a near-tie at the logit tolerance (top-2 gap of a deciding row,
        |u q - p| of a test, the margin of a draw); after a flagged
        divergence both sides resync to the oracle's outcome.
    Returns the statistics (also appended to SPEC_PARITY_RECORD)."""
    spec = pw.wl.spec
    tol = logit_tol(spec)
    kv = pw.kv0.copy()
    pending = pw.pending0
    s = 0
    st = dict(max_err=0.0, flagged=0, flagged_mismatch=0, self_flagged=0, self_flagged_mismatch=0,
              accepted=0, rounds=0, tie_where={})
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
        # the acceptance rule on the GPU's own logits
        if mode == "greedy":
            own = oacc.accept_greedy(lg, ri.tokens[1:], L, 0.0)
            assert got == (own.n_accepted, own.next_token, own.kv_len), \
                f"{spec.name} round {r}: GPU {got} != greedy rule on its own logits {own}"
        else:
            own = oacc.accept_stochastic(lg, ri.q, ri.tokens[1:], ri.u, L, ACC_TOL)
            if own.near_tie:
                st["self_flagged"] += 1
            if got != (own.n_accepted, own.next_token, own.kv_len):
                assert own.near_tie, \
                    f"{spec.name} round {r}: GPU {got} != stochastic rule on its own logits {own} (no flag)"
                assert _valid(res_g, L, k, spec.vocab)
                st["self_flagged_mismatch"] += 1
        # against the oracle's outcome
        want = (out_o.n_accepted, out_o.next_token, out_o.kv_len)
        if out_o.near_tie:
            st["flagged"] += 1
            for w in out_o.tie_where:
                key = w if not w.startswith("row") else "row"
                st["tie_where"][key] = st["tie_where"].get(key, 0) + 1
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
    record(dict(workload=spec.name, k=k, mode=mode, tag=tag, tol=tol, **st))
    return st
