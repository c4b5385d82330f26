#!/usr/bin/env python3
"""Throughput of the target model's verification step on one MI355X.

One "step" is one verification pass: a target forward pass over the block
[pending, d_1..d_k] against the paged KV cache, then greedy acceptance and
the KV commit (essay "LLM Inference: Speculative Decoding", section "The
loop").  The default workload is the LLaMA-2-7B-shaped bf16 target (32
layers, d 4096, 32 heads x 128, SwiGLU 11008, vocab 32000, weights
N(0, 0.02)) with a 1024-token random prompt and k = 8 drafts per round, each
draft the target's greedy continuation replaced by a uniform random id with
probability 0.3.

Timed region: `--steps` verification steps after `--warmup` untimed ones,
bracketed by device synchronizations; inputs are resident in HBM (weights,
KV cache); each step uploads its k+1 token ids and reads back the 12-byte
result, as the C ABI defines.  Printed: one JSON line with accepted tokens/s
(metric value), the HBM roofline of the dominant kernel (the pass kernel:
algorithmic bytes per launch, spec_pass_bytes at each step's committed
length, over its mean launch time from HIP events recorded around each
launch on the library's stream during the timed steps), and the CPU oracle
timed on a bounded sample of the same workload as a baseline.  The same
steps are then replayed from the same state with per-phase stamps (stderr
lines only).

Flags: --gpus N (only 1 is supported), --steps K, --warmup W, --workload
NAME, --k K, --k-sweep (extra per-k lines on stderr), --no-cpu-baseline,
--cpu-seconds S, --calib-copy (adds one plain 1 GiB device copy for
counter calibration under rocprofv3 --pmc).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
GREEDY_WORKLOADS = ("llama7b", "llama7b_int4", "moe", "tiny")
STOCHASTIC_WORKLOADS = ("qwen7b",)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the pass kernel's sources: counters recorded for other sources are stale
PASS_SOURCES = [os.path.join(ROOT, "target_model_verification_amd", "csrc", f)
                for f in ("pass.hip", "sv_common.h", "stream_plan.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama7b", choices=GREEDY_WORKLOADS + STOCHASTIC_WORKLOADS)
    ap.add_argument("--k", type=int, default=None)
    ap.add_argument("--k-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--draft", default="synthetic", choices=("synthetic", "self"),
                    help="drafts: the workload's corrupted greedy continuation, or (MoE) the model's own "
                         "expert-sparse self-speculative draft (spec_draft)")
    ap.add_argument("--draft-top-k", type=int, default=1, help="routed experts per draft token (--draft self)")
    ap.add_argument("--reuse-cap", type=int, default=0,
                    help="MoE: verify with reuse-aware expert gating (lossy) over this many preferred experts")
    ap.add_argument("--reuse-alpha", type=float, default=0.5, help="bias scale of reuse-aware gating")
    ap.add_argument("--batch", type=int, nargs="*", default=None, metavar="N",
                    help="also verify N sequences per pass (k = 16/N - 1 each); default N in 2 4 8 16")
    ap.add_argument("--tree", action="store_true",
                    help="also run self-drafted token trees with routing-aware expansion (--draft self)")
    ap.add_argument("--adaptive-k", action="store_true",
                    help="also time rounds whose lookahead follows spec_adaptive_k (start 5, +2 after a full "
                         "accept, -1 otherwise)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 1 GiB device copy (the HBM counter calibration for --traffic-from)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn two rocprofv3 counter CSVs (FETCH_SIZE and WRITE_SIZE runs of "
                         "bench.py --calib-copy) into " + os.path.relpath(TRAFFIC_FILE, ROOT))
    return ap.parse_args()


def traffic_from(fetch_csv: str, write_csv: str, command: str):
    """HBM bytes per pass-kernel launch from rocprofv3 counters (KiB per
    dispatch), each scaled by what the same counter reads for the
    calibration copy of 1 GiB read + 1 GiB written.  The pass-kernel value
    is the median over its last dispatches (the timed k=8 steps)."""
    import csv
    import statistics

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r.get("Counter_Name") == counter]
        passes = [float(r["Counter_Value"]) for r in rows if "k_pass" in r["Kernel_Name"]]
        copies = [float(r["Counter_Value"]) for r in rows if "copy" in r["Kernel_Name"].lower()]
        if not passes or not copies:
            raise SystemExit(f"{path}: no {counter} rows for the pass kernel or the calibration copy")
        return statistics.median(passes[-8:]), max(copies)

    fetch, fcopy = per_kernel(fetch_csv, "FETCH_SIZE")
    write, wcopy = per_kernel(write_csv, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    f_scale, w_scale = gib_kib / fcopy, gib_kib / wcopy
    traffic = (fetch * f_scale + write * w_scale) * 1024.0
    out = {"pass_sources_sha256_16": source_digest(PASS_SOURCES),
           "per_launch_bytes": {"pass": round(traffic)},
           "fetch_kib_per_launch": fetch, "write_kib_per_launch": write,
           "copy_fetch_kib": fcopy, "copy_write_kib": wcopy,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "command": command}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    log(f"[bench] traffic per pass launch: {traffic / 1e9:.3f} GB (fetch {fetch * f_scale / 2**20:.3f} GiB, "
        f"write {write * w_scale / 2**20:.3f} GiB) -> {TRAFFIC_FILE}")


class Session:
    """A verifier for one workload with its prompt prefilled on the GPU and
    the target's greedy continuation (the drafts' source) computed once."""

    def __init__(self, wl, W, max_k: int, rounds: int, stream, n_seqs: int = 1):
        import numpy as np
        from target_model_verification_amd import binding as B
        from target_model_verification_amd import synth
        self.B, self.np = B, np
        self.reuse = None   # (cap, alpha): verify with reuse-aware gating
        self.wl = wl
        self.spec = wl.spec
        self.max_k = max_k
        self.n_ref = rounds * (max_k + 1) + 1
        self.max_ctx = wl.context + self.n_ref + 2 * (max_k + 1) + 64
        t = time.time()
        self.h = B.Verifier(wl.spec, W, None, None, 0, self.max_ctx, 15, stream, n_seqs=n_seqs)
        log(f"[bench] verifier created in {time.time() - t:.1f} s (max_ctx {self.max_ctx})")
        # prompt: appended in blocks of 16 (accept mode NONE commits the block)
        t = time.time()
        prompt = synth.prompt_ids(wl)
        res = None
        for i in range(0, len(prompt), 16):
            res = self.h.step(prompt[i:i + 16], B.SPEC_ACCEPT_NONE)
        self.L0 = self.h.kv_len
        self.pending0 = int(res.next_token)
        if wl.accept == "stochastic":   # drafts are drawn per round from the target's own logits
            self.ref = None
            log(f"[bench] prompt {len(prompt)} prefilled in {time.time() - t:.1f} s")
            return
        # the target's greedy continuation after the prompt (k = 0 steps)
        ref = [self.pending0]
        for _ in range(self.n_ref):
            ref.append(int(self.h.step([ref[-1]], B.SPEC_ACCEPT_GREEDY).next_token))
        self.ref = np.asarray(ref, dtype=np.int64)
        self.h.rollback(self.L0)
        log(f"[bench] prompt {len(prompt)} prefilled and {self.n_ref} greedy tokens decoded in "
            f"{time.time() - t:.1f} s")

    def rounds(self, k: int, n: int, first_round: int = 0):
        """Per-round corruption draws for rounds first_round.. (drawn ahead so
        the timed loop does no random-number work)."""
        from target_model_verification_amd import synth
        return [synth.draft_corruption(self.wl, first_round + r, k) for r in range(n)]

    def run(self, k: int, corr, s: int, pending: int, profile=0):
        """Runs len(corr) rounds from sequence index s (profile: 0 off, 1
        events + per-phase stamps, 2 events only).  Returns per-round
        (L, n_acc), the new s and pending token, the elapsed seconds and the
        profile counters."""
        import torch
        np, B = self.np, self.B
        h = self.h
        out = []
        tok = np.empty(k + 1, dtype=np.int32)
        if profile:
            h.profile(profile)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for flags, ids in corr:
            tok[0] = pending
            tok[1:] = np.where(flags, ids, self.ref[s + 1:s + 1 + k])
            L = h.kv_len
            if self.reuse:
                res = h.step_reuse(tok, self.reuse[0], self.reuse[1], B.SPEC_ACCEPT_GREEDY)
            else:
                res = h.step(tok, B.SPEC_ACCEPT_GREEDY)
            out.append((L, res.n_accepted))
            s += res.n_accepted + 1
            pending = res.next_token
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        prof = h.profile_read() if profile else None
        if profile == 1:
            self.detail = h.profile_detail()
        if profile:
            h.profile(False)
        return out, s, pending, dt, prof


def draft_round(sess: Session, rnd: int, pending: int, k: int, zbuf):
    """Stochastic drafts of one round, as the stochastic workload defines
    them: q_i = softmax(z_i + eps_i) with z_i the target's fp32 logits at
    draft position i given pending, d_1..d_{i-1} (single-token passes on the
    target's own cache, rolled back afterwards), d_i drawn from q_i by
    inverse CDF with a seeded uniform.  Input preparation only: none of it
    is timed."""
    import numpy as np
    import torch
    from target_model_verification_amd import synth
    B, h, wl = sess.B, sess.h, sess.wl
    L = h.kv_len
    toks, qs = [pending], []
    for i in range(1, k + 1):
        h.step([toks[-1]], B.SPEC_ACCEPT_NONE, 0, 0, zbuf.data_ptr())
        z = zbuf[0].double() + torch.from_numpy(synth.draft_noise(wl, rnd, i)).to(zbuf.device).double()
        q = torch.softmax(z, 0)
        c = torch.cumsum(q, 0)
        u = synth.draft_sample_uniform(wl, rnd, i)
        d = int(torch.searchsorted(c, torch.tensor([u * float(c[-1])], dtype=torch.float64, device=c.device),
                                   right=True)[0])
        toks.append(min(d, wl.spec.vocab - 1))
        qs.append(q.float())
    h.rollback(L)
    q_dev = torch.stack(qs).contiguous() if qs else torch.zeros((1, wl.spec.vocab), device=zbuf.device)
    u_dev = torch.from_numpy(synth.round_uniforms(wl, rnd, k)).to(zbuf.device)
    return np.asarray(toks, dtype=np.int32), q_dev, u_dev


def measure_k_stochastic(sess: Session, k: int, warmup: int, steps: int):
    """Stochastic acceptance (u < p/q, residual resample): each step is
    timed alone (drafting between steps runs target passes of its own),
    then the timed steps are replayed from the same state with HIP events
    around every kernel launch."""
    import torch
    B, h = sess.B, sess.h
    zbuf = torch.empty((1, sess.wl.spec.vocab), dtype=torch.float32, device="cuda")
    h.rollback(sess.L0)
    pending, rec, inputs, dt = sess.pending0, [], [], 0.0
    L_start = None
    ev_ms = ev_bytes = 0.0
    for r in range(warmup + steps):
        toks, q_dev, u_dev = draft_round(sess, r, pending, k, zbuf)
        torch.cuda.synchronize()
        L = h.kv_len
        if r == warmup:
            L_start = L
        if r >= warmup:
            h.profile(2)   # HIP events around the pass and acceptance kernels only
        t0 = time.perf_counter()
        res = h.step(toks, B.SPEC_ACCEPT_STOCHASTIC, q_dev.data_ptr(), u_dev.data_ptr())
        el = time.perf_counter() - t0
        if r >= warmup:
            _, ms_p, by_p = h.profile_read()["pass"]
            h.profile(0)
            ev_ms += ms_p
            ev_bytes += by_p
            dt += el
            rec.append((L, res.n_accepted))
            inputs.append((toks, q_dev, u_dev))
        pending = res.next_token
    h.rollback(L_start)
    h.profile(True)
    rec2 = []
    for toks, q_dev, u_dev in inputs:
        rec2.append(h.step(toks, B.SPEC_ACCEPT_STOCHASTIC, q_dev.data_ptr(), u_dev.data_ptr()).n_accepted)
    torch.cuda.synchronize()
    prof = h.profile_read()
    sess.detail = h.profile_detail()
    h.profile(False)
    if rec2 != [n for _, n in rec]:
        raise RuntimeError("replayed steps accepted different counts: the pass is not deterministic")
    accepted = sum(n + 1 for _, n in rec)
    bytes_total = sum(h.pass_bytes(L, k, B.SPEC_ACCEPT_STOCHASTIC) for L, _ in rec)
    timed = dict(pass_launches=steps, pass_ms=ev_ms, pass_bytes=ev_bytes)
    return dict(k=k, steps=steps, seconds=dt, ms_per_step=dt / steps * 1e3, accepted=accepted,
                acc_tok_s=accepted / dt, verified_tok_s=steps * (k + 1) / dt,
                mean_accept=accepted / steps, pass_gb=bytes_total / steps / 1e9,
                wall_gbs=bytes_total / dt / 1e9, L_start=L_start, prof=prof, timed=timed,
                profiled_seconds=None)


def measure_self_draft(sess: Session, k: int, kd: int, warmup: int, steps: int):
    """Self-speculative rounds (MoE): k draft tokens from the model itself
    with kd routed experts per token (spec_draft, chained on the device),
    then the verification step of the block, greedy acceptance.  Both calls
    are timed per round (each returns after its result reached the host);
    the verification pass is also timed with HIP events."""
    import torch
    B, h = sess.B, sess.h
    h.rollback(sess.L0)
    pending, rec, t_draft, t_verify = sess.pending0, [], 0.0, 0.0
    L_start = None
    for r in range(warmup + steps):
        if r == warmup:
            L_start = h.kv_len
            h.profile(2)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        drafts = h.draft(pending, k, kd)
        t1 = time.perf_counter()
        L = h.kv_len
        res = h.step([pending] + drafts, B.SPEC_ACCEPT_GREEDY)
        t2 = time.perf_counter()
        if r >= warmup:
            t_draft += t1 - t0
            t_verify += t2 - t1
            rec.append((L, res.n_accepted))
        pending = res.next_token
    tprof = h.profile_read()
    h.profile(0)
    accepted = sum(n + 1 for _, n in rec)
    n_p, ms_p, by_p = tprof["pass"]
    dt = t_draft + t_verify
    return dict(k=k, steps=steps, seconds=t_verify, ms_per_step=t_verify / steps * 1e3, accepted=accepted,
                acc_tok_s=accepted / t_verify, verified_tok_s=steps * (k + 1) / t_verify,
                mean_accept=accepted / steps, pass_gb=by_p / steps / 1e9, wall_gbs=by_p / t_verify / 1e9,
                L_start=L_start, prof=tprof, timed=dict(pass_launches=n_p, pass_ms=ms_p, pass_bytes=by_p),
                profiled_seconds=None,
                self_draft=dict(draft_top_k=kd, draft_ms_per_round=t_draft / steps * 1e3,
                                draft_ms_per_token=t_draft / steps / k * 1e3,
                                verify_ms_per_round=t_verify / steps * 1e3,
                                e2e_accepted_tok_s=accepted / dt,
                                mean_accepted_drafts=accepted / steps - 1.0))


def measure_tree(sess: Session, n: int, kd: int, warmup: int, steps: int):
    """Self-drafted token trees with routing-aware expansion (MoE).  Each
    round drafts a chain of n tokens with kd routed experts (spec_draft, with
    the draft logits and routes); the candidates are the chain tokens and, at
    every depth, the draft's second choice as a sibling; spec_tree_expand
    admits candidates by utility (prefix confidence x T_AR over the cost of
    the experts they add plus their drafting cost) and spec_verify_tree
    verifies the admitted tree in one pass.  T_AR is a measured one-token
    step; T_exp one routed expert's share of it (its bytes at the pass's
    measured bandwidth); a chain token costs one draft pass, a sibling
    nothing (it comes from the same distribution).  A candidate whose own
    token the draft did not run (the siblings and the last chain token) is
    charged the experts of its parent's draft pass.  Compared with chain
    verification of the same drafts (spec_verify_step with k = n)."""
    import torch
    np, B, h = sess.np, sess.B, sess.h
    spec = sess.spec
    V, E, NL = spec.vocab, spec.n_experts, spec.n_layers
    # T_AR: one-token target steps at the prompt's end
    h.rollback(sess.L0)
    torch.cuda.synchronize()
    h.profile(2)
    t0 = time.perf_counter()
    for _ in range(8):
        h.step([sess.pending0], B.SPEC_ACCEPT_NONE)
        h.rollback(sess.L0)
    torch.cuda.synchronize()
    t_ar = (time.perf_counter() - t0) / 8
    n_p, ms_p, by_p = h.profile_read()["pass"]
    h.profile(0)
    wbytes = {"bf16": 2.0, "f32": 4.0, "int4": 0.5 + 2.0 / 128}[spec.weight_dtype]
    t_exp = 3.0 * spec.d_model * spec.d_ff_expert * wbytes / (by_p / (ms_p / 1e3))
    lg = torch.empty((n, V), dtype=torch.float32, device="cuda")
    rt = torch.empty((n, NL, kd), dtype=torch.int32, device="cuda")
    out = {}
    for kind in ("chain", "tree"):
        h.rollback(sess.L0)
        pending = sess.pending0
        t_draft = t_pol = t_ver = 0.0
        acc = nodes = sib_acc = 0
        c_draft = None
        for r in range(warmup + steps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            drafts = h.draft(pending, n, kd, lg.data_ptr(), rt.data_ptr())
            t1 = time.perf_counter()
            c_draft = (t1 - t0) / n if c_draft is None else 0.8 * c_draft + 0.2 * (t1 - t0) / n
            if kind == "chain":
                t2 = t1
                res = h.step([pending] + drafts, B.SPEC_ACCEPT_GREEDY)
                m, hit_sib = n + 1, False
            else:
                # the draft's two best tokens and their probabilities per depth
                top_p, top_i = torch.topk(torch.softmax(lg, dim=-1), 2, dim=-1)
                top_p, top_i = top_p.double().cpu().numpy(), top_i.cpu().numpy()
                routes = rt.cpu().numpy() + (np.arange(NL) * E)[None, :, None]
                ids = [routes[i].reshape(-1).tolist() for i in range(n)]
                par, pp, ex, toks, cd = [], [], [], [], []
                for i in range(1, n + 1):       # chain token d_i and the sibling of depth i
                    parent = -1 if i == 1 else len(par) - 2
                    j = 1 if int(top_i[i - 1, 0]) == drafts[i - 1] else 0   # the sibling: the other of the two
                    par += [parent, parent]
                    pp += [float(top_p[i - 1, 1 - j]), float(top_p[i - 1, j])]
                    ex += [ids[i] if i < n else ids[i - 1], ids[i - 1]]
                    toks += [drafts[i - 1], int(top_i[i - 1, j])]
                    cd += [c_draft, 0.0]
                order, rows = B.tree_expand(par, pp, ex, ids[0], t_ar, t_exp, cd, 15)
                tokens = [pending] + [toks[c] for c in order]
                t2 = time.perf_counter()
                res, path = h.step_tree(tokens, rows)
                m = len(tokens)
                hit_sib = any(order[p - 1] % 2 == 1 for p in path)
            t3 = time.perf_counter()
            if r >= warmup:
                t_draft += t1 - t0
                t_pol += t2 - t1
                t_ver += t3 - t2
                acc += res.n_accepted + 1
                nodes += m
                sib_acc += int(hit_sib)
            pending = res.next_token
        tot = t_draft + t_pol + t_ver
        out[kind] = dict(mean_rows=round(nodes / steps, 3), mean_tokens_per_round=round(acc / steps, 4),
                         draft_ms=round(t_draft / steps * 1e3, 4), policy_ms=round(t_pol / steps * 1e3, 4),
                         verify_ms=round(t_ver / steps * 1e3, 4), e2e_tok_s=round(acc / tot, 2),
                         rounds_accepting_a_sibling=sib_acc)
    return dict(n=n, draft_top_k=kd, t_ar_ms=round(t_ar * 1e3, 4), t_exp_us=round(t_exp * 1e6, 3),
                steps=steps, **out)


def measure_batch(sess: Session, n_seq: int, warmup: int, steps: int):
    """n_seq sequences verified together (spec_verify_batch): each has its
    own seeded prompt of the workload's context (appended on the GPU), its
    own greedy continuation and corrupted drafts; the blocks share one pass
    with k = 16 / n_seq - 1 drafts each.  Aggregate accepted tok/s over the
    timed steps (wall clock per step, pass time from HIP events)."""
    import dataclasses
    import torch
    from target_model_verification_amd import synth
    np, B, h, wl = sess.np, sess.B, sess.h, sess.wl
    k = 16 // n_seq - 1
    seqs = list(range(n_seq))
    wls = [wl] + [dataclasses.replace(wl, seed=wl.seed + 7919 * s) for s in range(1, n_seq)]
    h.rollback(sess.L0)
    pend = [sess.pending0]
    for s in range(1, n_seq):   # prompts of the other sequences, 16 positions per pass
        h.seq_rollback(s, 0)
        prompt = synth.prompt_ids(wls[s])
        res = None
        for i in range(0, len(prompt), 16):
            res = h.step_batch([s], [prompt[i:i + 16]], B.SPEC_ACCEPT_NONE)[0]
        pend.append(int(res.next_token))
    L0 = [h.seq_len(s) for s in seqs]
    # every sequence's greedy continuation, all sequences one token per pass
    n_ref = (warmup + steps) * (k + 1) + 1
    ref = [[p] for p in pend]
    for _ in range(n_ref):
        out = h.step_batch(seqs, [[r[-1]] for r in ref], B.SPEC_ACCEPT_GREEDY)
        for s in seqs:
            ref[s].append(int(out[s].next_token))
    for s in seqs:
        h.seq_rollback(s, L0[s])
    ref = [np.asarray(r, dtype=np.int64) for r in ref]
    corr = [[synth.draft_corruption(wls[s], r, k) for r in range(warmup + steps)] for s in seqs]
    pos = [0] * n_seq
    acc, dt = 0, 0.0
    per_seq = [0] * n_seq
    for r in range(warmup + steps):
        if r == warmup:
            h.profile(2)
        blocks = []
        for s in seqs:
            flags, ids = corr[s][r]
            d = np.where(flags, ids, ref[s][pos[s] + 1:pos[s] + 1 + k])
            blocks.append([int(ref[s][pos[s]])] + [int(x) for x in d])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        out = h.step_batch(seqs, blocks, B.SPEC_ACCEPT_GREEDY)
        el = time.perf_counter() - t0
        for s in seqs:
            pos[s] += out[s].n_accepted + 1
            if r >= warmup:
                per_seq[s] += out[s].n_accepted + 1
        if r >= warmup:
            dt += el
            acc += sum(o.n_accepted + 1 for o in out)
    n_p, ms_p, by_p = h.profile_read()["pass"]
    h.profile(0)
    for s in range(1, n_seq):
        h.seq_rollback(s, 0)
    return dict(n_seq=n_seq, k=k, rows=n_seq * (k + 1), steps=steps, ms_per_step=round(dt / steps * 1e3, 4),
                accepted_tok_s=round(acc / dt, 2), tokens_per_step=round(acc / steps, 4),
                tokens_per_step_per_seq=[round(v / steps, 3) for v in per_seq],
                us_per_pass=round(ms_p / n_p * 1e3, 1), pass_gb=round(by_p / n_p / 1e9, 4),
                pass_hbm_frac=round(by_p / (ms_p / 1e3) / 1e9 / HBM_PEAK_GBS, 4))


def reuse_quality(sess: Session, k: int, cap: int, alpha: float, n_blocks: int = 8):
    """Reuse-aware gating against the exact pass on the same blocks (untimed):
    experts loaded per layer and the output consistency metrics of S2-MoE
    section 6.2.2 (mean KL, RMS probability shift, top-1 agreement,
    perplexity ratio of the blocks' next tokens)."""
    import torch
    np, B, h = sess.np, sess.B, sess.h
    spec = sess.spec
    h.rollback(sess.L0)
    ex_u, re_u, kl, dp, top1, dnll = [], [], [], [], [], []
    for r in range(n_blocks):
        flags, ids = sess.rounds(k, 1, first_round=20000 + r)[0]
        s = r * (k + 1)
        tok = np.concatenate([[sess.ref[s]], np.where(flags, ids, sess.ref[s + 1:s + 1 + k])]).astype(np.int32)
        out = {}
        for name, reuse in (("exact", None), ("reuse", (cap, alpha))):
            lg = torch.empty((k + 1, spec.vocab), dtype=torch.float32, device="cuda")
            un = torch.zeros(spec.n_layers, dtype=torch.int32, device="cuda")
            if reuse:
                h.step_reuse(tok, cap, alpha, B.SPEC_ACCEPT_NONE, logits_ptr=lg.data_ptr(), union_ptr=un.data_ptr())
            else:
                h.step(tok, B.SPEC_ACCEPT_NONE, 0, 0, lg.data_ptr(), union_ptr=un.data_ptr())
            h.rollback(sess.L0)
            out[name] = (lg[:k].double(), float(un.float().mean()))
        p = torch.softmax(out["exact"][0], -1)
        q = torch.softmax(out["reuse"][0], -1)
        nxt = torch.from_numpy(tok[1:].astype(np.int64)).to(p.device)
        kl.append(float((p * (torch.log(p.clamp_min(1e-300)) - torch.log(q.clamp_min(1e-300)))).sum(-1).mean()))
        dp.append(float(((q - p) ** 2).mean(-1).sqrt().mean()))
        top1.append(float((p.argmax(-1) == q.argmax(-1)).double().mean()))
        ar = torch.arange(k, device=p.device)
        dnll.append(float((-torch.log(q[ar, nxt]) + torch.log(p[ar, nxt])).mean()))
        ex_u.append(out["exact"][1])
        re_u.append(out["reuse"][1])
    import math
    return dict(cap=cap, alpha=alpha, blocks=n_blocks, experts_per_layer_exact=round(sum(ex_u) / n_blocks, 3),
                experts_per_layer_reuse=round(sum(re_u) / n_blocks, 3),
                reuse_ratio_exact=round(sum(ex_u) / n_blocks / ((k + 1) * spec.top_k), 4),
                reuse_ratio_reuse=round(sum(re_u) / n_blocks / ((k + 1) * spec.top_k), 4),
                mean_kl=sum(kl) / n_blocks, rms_dp=sum(dp) / n_blocks, top1_agreement=sum(top1) / n_blocks,
                ppl_ratio=math.exp(sum(dnll) / n_blocks))


def measure_adaptive(sess: Session, k0: int, warmup: int, steps: int):
    """Greedy rounds whose lookahead follows the adaptive schedule
    (spec_adaptive_k), drafts drawn as for the fixed-k runs.  Returns
    accepted tok/s over the timed rounds and the lookahead histogram."""
    import torch
    np, B, h = sess.np, sess.B, sess.h
    h.rollback(sess.L0)
    s, pending, k = 0, sess.pending0, k0
    ks, acc, dt = [], 0, 0.0
    for r in range(warmup + steps):
        flags, ids = sess.rounds(k, 1, first_round=10000 + r)[0]
        tok = np.concatenate([[pending], np.where(flags, ids, sess.ref[s + 1:s + 1 + k])]).astype(np.int32)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        res = h.step(tok, B.SPEC_ACCEPT_GREEDY)
        el = time.perf_counter() - t0
        if r >= warmup:
            dt += el
            acc += res.n_accepted + 1
            ks.append(k)
        s += res.n_accepted + 1
        pending = res.next_token
        k = B.spec_adaptive_k(k, res.n_accepted, sess.max_k)
    hist = {str(v): ks.count(v) for v in sorted(set(ks))}
    return dict(k0=k0, max_k=sess.max_k, steps=steps, accepted_tok_s=round(acc / dt, 2),
                ms_per_step=round(dt / steps * 1e3, 4), mean_k=round(sum(ks) / steps, 3),
                mean_tokens_per_step=round(acc / steps, 4), k_histogram=hist)


def measure_k(sess: Session, k: int, warmup: int, steps: int):
    if sess.wl.accept == "stochastic":
        return measure_k_stochastic(sess, k, warmup, steps)
    corr = sess.rounds(k, warmup + steps)
    sess.h.rollback(sess.L0)
    _, s, pending, _, _ = sess.run(k, corr[:warmup], 0, sess.pending0)
    L_start = sess.h.kv_len
    # timed steps, with HIP events around the pass and acceptance kernels on
    # the library's stream (events only: the pass runs as unprofiled)
    rec, s_end, _, dt, tprof = sess.run(k, corr[warmup:], s, pending, profile=2)
    # the same steps again from the same state, with per-phase stamps
    sess.h.rollback(L_start)
    rec2, _, _, dt2, prof = sess.run(k, corr[warmup:], s, pending, profile=1)
    if [r[1] for r in rec2] != [r[1] for r in rec]:
        raise RuntimeError("replayed steps accepted different counts: the pass is not deterministic")
    accepted = sum(n + 1 for _, n in rec)
    n_p, ms_p, by_p = tprof["pass"]   # spec_pass_bytes per step (MoE: with its loaded experts)
    bytes_total = by_p
    timed = dict(pass_launches=n_p, pass_ms=ms_p, pass_bytes=by_p)
    return dict(k=k, steps=steps, seconds=dt, ms_per_step=dt / steps * 1e3, accepted=accepted,
                acc_tok_s=accepted / dt, verified_tok_s=steps * (k + 1) / dt,
                mean_accept=accepted / steps, pass_gb=bytes_total / steps / 1e9,
                wall_gbs=bytes_total / dt / 1e9, L_start=L_start, prof=prof, timed=timed,
                profiled_seconds=dt2)


def expected_tokens(wl, k: int):
    """E[n_acc + 1] per round for drafts corrupted independently with
    probability c (per-draft agreement a = 1 - c (1 - 1/V)): (1 - a^(k+1)) /
    (1 - a) (essay "Being right five times in a row is rare"); None for
    drafts drawn from a noisy distribution (stochastic workloads)."""
    if wl.accept != "greedy":
        return None
    a = 1.0 - wl.corruption * (1.0 - 1.0 / wl.spec.vocab)
    return float(k + 1) if a == 1.0 else (1.0 - a ** (k + 1)) / (1.0 - a)


def traffic_for(kernel_class: str):
    """HBM bytes per launch measured by rocprofv3 counters for this kernel,
    if recorded for the current pass kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("pass_sources_sha256_16") != source_digest(PASS_SOURCES):
        return None
    return t.get("per_launch_bytes", {}).get(kernel_class)


def cpu_baseline(wl, W, k: int, L: int, seconds: float, mean_accept: float):
    """The CPU oracle (NumPy, fp32 BLAS) timed on a bounded sample: whole
    verification steps (block pass + greedy acceptance) of the same model at
    the same k and committed length."""
    import numpy as np
    from oracle import accept as oacc
    from oracle import model as om
    from target_model_verification_amd import synth
    affinity = len(os.sched_getaffinity(0))
    blas, blas_threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')} ({os.path.basename(i.get('filepath', ''))})"
                blas_threads = i.get("num_threads")
    except Exception:  # pragma: no cover
        pass
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    t = time.time()
    M = om.OracleModel(wl.spec, W, np.float32)
    kv = om.KVCache.empty(wl.spec, L + k + 1, np.float32)
    for l in range(wl.spec.n_layers):
        n = wl.spec.n_kv_heads * L * wl.spec.head_dim
        kv.K[l][:, :L, :] = synth.normal_f32(n, 1.0, [wl.seed, 41, l]).reshape(wl.spec.n_kv_heads, L, -1)
        kv.V[l][:, :L, :] = synth.normal_f32(n, 1.0, [wl.seed, 43, l]).reshape(wl.spec.n_kv_heads, L, -1)
    kv.length = L
    log(f"[bench] oracle fp32 model prepared in {time.time() - t:.1f} s")
    toks = synth.prompt_ids(wl, k + 1)
    n, t0 = 0, time.perf_counter()
    while True:
        res = om.forward_block(M, kv, toks, L)
        oacc.accept_greedy(res.logits, toks[1:], L)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or (n >= 2 and el + el / n > 2 * seconds):
            break
    step_s = el / n
    cores = int(blas_threads) if blas_threads else affinity
    return {"value": round(mean_accept / step_s, 3), "unit": "accepted tok/s", "cores": cores,
            "kind": "oracle", "affinity_cpus": affinity, "cpu_model": cpu_model, "blas": blas,
            "sample": (f"{n} verification steps (block pass over k+1={k + 1} tokens at committed length "
                       f"{L} + greedy acceptance) of the full {wl.spec.name} model in the NumPy oracle, "
                       f"weights as fp32 BLAS operands, {el:.1f} s; KV cache filled with seeded synthetic "
                       f"values (the oracle's time does not depend on them); accepted tokens per step "
                       f"({mean_accept:.3f}) taken from the GPU run, whose outcomes the oracle reproduces"),
            "ms_per_step": round(step_s * 1e3, 1)}


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(args.traffic_from[0], args.traffic_from[1], " ".join(sys.argv))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build measures the "
              "verification step on a single MI355X; multi-GPU sharding is a design note, not a code path.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from target_model_verification_amd import binding as B  # noqa: F401  (fails loudly if not built)
    from target_model_verification_amd import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    k = wl.k if args.k is None else args.k
    ks = sorted(set(list(wl.k_sweep) + [k])) if args.k_sweep else [k]
    t = time.time()
    W = synth.make_weights(wl.spec, wl.seed)
    log(f"[bench] {wl.spec.name}: {synth.weight_nbytes(W) / 1e9:.2f} GB of weights generated in "
        f"{time.time() - t:.1f} s")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        n_seqs = max(args.batch or [2, 4, 8, 16]) if args.batch is not None else 1
        sess = Session(wl, W, 15 if args.adaptive_k else max(ks), args.warmup + args.steps, stream.cuda_stream,
                       n_seqs)
        if args.calib_copy:
            a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
            b = torch.empty_like(a)
            b.copy_(a)
            torch.cuda.synchronize()
            log("[bench] calibration copy: 1 GiB read + 1 GiB written")
            del a, b
        results = {}
        if args.reuse_cap:
            if not wl.spec.moe or args.draft != "synthetic":
                raise SystemExit("--reuse-cap needs a MoE workload with synthetic drafts")
            sess.reuse = (args.reuse_cap, args.reuse_alpha)
        if args.draft == "self" and not wl.spec.moe:
            raise SystemExit("--draft self drafts by expert sparsity: it needs a MoE workload")
        for kk in ks:
            if args.draft == "self":
                results[kk] = measure_self_draft(sess, kk, args.draft_top_k, args.warmup, args.steps)
            else:
                results[kk] = measure_k(sess, kk, args.warmup, args.steps)
            r = results[kk]
            log(f"[bench] k={kk}: {r['ms_per_step']:.3f} ms/step, {r['acc_tok_s']:.1f} accepted tok/s, "
                f"{r['verified_tok_s']:.1f} verified tok/s, mean accepted+1 {r['mean_accept']:.3f}, "
                f"{r['pass_gb']:.3f} GB/pass, wall {r['wall_gbs']:.0f} GB/s "
                f"({r['wall_gbs'] / HBM_PEAK_GBS:.1%} of 8 TB/s)")
            det = getattr(sess, "detail", {})
            for c, (n, ms, by) in r["prof"].items():
                if n:
                    line = (f"[bench]   {c:14s} {n:6d} launches {ms / n * 1e3:9.1f} us/launch "
                            f"{by / n / 1e6:9.2f} MB/launch {by / ms / 1e6 if ms else 0:8.0f} GB/s")
                    if c in det and c not in ("pass", "accept"):
                        mean, mx = ([v / n * 1e3 for v in t] for t in det[c])
                        line += (" | workgroup mean/max us: stage %.1f/%.1f stream %.1f/%.1f flush %.1f/%.1f "
                                 "work %.1f/%.1f, barrier %.1f" % (mean[0], mx[0], mean[1], mx[1], mean[2], mx[2],
                                                                   mean[3], mx[3], ms / n * 1e3 - mx[3]))
                    log(line)
    r = results[k]
    # the dominant kernel is the persistent pass kernel (k_pass), one launch
    # per step carrying every phase of the block forward; its launches are
    # timed with HIP events during the timed steps
    t = r["timed"]
    per_launch_bytes = t["pass_bytes"] / t["pass_launches"]
    per_launch_s = t["pass_ms"] / t["pass_launches"] / 1e3
    achieved = per_launch_bytes / per_launch_s / 1e9
    traffic = traffic_for("pass")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "k_pass (persistent verification pass)", "bytes_per_launch": round(per_launch_bytes),
                "us_per_launch": round(per_launch_s * 1e6, 2), "launches": t["pass_launches"],
                "pass_wall_gbs": round(r["wall_gbs"], 1),
                "pass_wall_frac": round(r["wall_gbs"] / HBM_PEAK_GBS, 4)}
    cpu = None
    if not args.no_cpu_baseline and wl.accept == "greedy":
        cpu = cpu_baseline(wl, W, k, r["L_start"], args.cpu_seconds, r["mean_accept"])
    e_tok = expected_tokens(wl, k) if args.draft == "synthetic" else None
    line = {
        "metric": "accepted tok/s + verify-pass HBM GB/s vs peak, 7B bf16 k=8, single sequence",
        "value": round(r["acc_tok_s"], 2), "unit": "accepted tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.spec.weight_dtype,
        "data": ("synthetic: random-init weights N(0,0.02), uniform random prompt ids, drafts = target's "
                 "greedy continuation with per-token corruption" if wl.accept == "greedy" else
                 "synthetic: random-init weights N(0,0.02), uniform random prompt ids, drafts drawn from "
                 "q = softmax(target logits + N(0,1) noise)"),
        "config": {"workload": (f"{wl.spec.name} verify pass, k={k}, context {wl.context}, "
                                + (f"draft corruption {wl.corruption}, greedy acceptance" if wl.accept == "greedy"
                                   else "stochastic acceptance at temperature 1") + ", single sequence"),
                   "k": k, "context": wl.context, "verified_tok_s": round(r["verified_tok_s"], 2),
                   "mean_tokens_per_step": round(r["mean_accept"], 4),
                   "expected_tokens_per_step": None if e_tok is None else round(e_tok, 4),
                   "expected_accepted_tok_s": None if e_tok is None else round(e_tok / r["ms_per_step"] * 1e3, 2),
                   "pass_bytes_gb": round(r["pass_gb"], 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if wl.spec.moe and r.get("prof") and r["prof"].get("expert_gateup", (0,))[0]:
        # the routed union per layer, from the expert gate/up phase's bytes
        # (each loaded expert's gate and up matrices once, plus the shared ones)
        n_eg, _, by_eg = r["prof"]["expert_gateup"]
        wbytes = {"bf16": 2.0, "f32": 4.0, "int4g128": 0.5 + 2.0 / 128}[wl.spec.weight_dtype]
        per_expert = 2.0 * wl.spec.d_model * wl.spec.d_ff_expert * wbytes
        union = by_eg / n_eg / per_expert - wl.spec.n_shared
        line["config"]["experts_per_layer"] = round(union, 3)
        line["config"]["reuse_ratio"] = round(union / ((k + 1) * wl.spec.top_k), 4)
    if args.reuse_cap:
        with torch.cuda.stream(stream):
            line["reuse_gating"] = reuse_quality(sess, k, args.reuse_cap, args.reuse_alpha)
        line["config"]["workload"] += (f", reuse-aware expert gating (lossy) cap {args.reuse_cap} "
                                       f"alpha {args.reuse_alpha}")
        log(f"[bench] reuse-aware gating: {line['reuse_gating']}")
    if args.adaptive_k:
        if wl.accept != "greedy" or args.draft != "synthetic":
            raise SystemExit("--adaptive-k runs greedy rounds with the workload's synthetic drafts")
        with torch.cuda.stream(stream):
            line["adaptive_k"] = measure_adaptive(sess, 5, args.warmup, args.steps)
        log(f"[bench] adaptive k: {line['adaptive_k']}")
    if args.draft == "self":
        line["data"] = ("synthetic: random-init weights N(0,0.02), uniform random prompt ids, drafts = the model's own "
                        f"greedy decode with {args.draft_top_k} routed expert(s) per token (self-speculative)")
        line["config"]["workload"] = line["config"]["workload"].replace(
            f"draft corruption {wl.corruption}", f"self-speculative draft with {args.draft_top_k} routed expert(s)")
        line["self_draft"] = {kk: round(v, 4) if isinstance(v, float) else v for kk, v in r["self_draft"].items()}
    if args.batch is not None:
        if wl.accept != "greedy" or args.draft != "synthetic":
            raise SystemExit("--batch runs greedy rounds with the workload's synthetic drafts")
        line["batch"] = {}
        with torch.cuda.stream(stream):
            for nb in (args.batch or [2, 4, 8, 16]):
                line["batch"][str(nb)] = measure_batch(sess, nb, args.warmup, args.steps)
                log(f"[bench] {nb} sequences per pass: {line['batch'][str(nb)]}")
    if args.tree:
        if args.draft != "self":
            raise SystemExit("--tree expands self-drafted candidates: use it with --draft self")
        with torch.cuda.stream(stream):
            line["tree"] = measure_tree(sess, k, args.draft_top_k, args.warmup, args.steps)
        log(f"[bench] token trees: {line['tree']}")
    if args.k_sweep:
        def frac(v):
            t = v["timed"]
            return round(t["pass_bytes"] / (t["pass_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4)
        line["k_sweep"] = {str(kk): {"ms_per_step": round(v["ms_per_step"], 4),
                                     "acc_tok_s": round(v["acc_tok_s"], 2),
                                     "verified_tok_s": round(v["verified_tok_s"], 2),
                                     "us_per_pass": round(v["timed"]["pass_ms"] / v["timed"]["pass_launches"] * 1e3, 1),
                                     "pass_hbm_frac": frac(v),
                                     "wall_gbs": round(v["wall_gbs"], 1)} for kk, v in results.items()}
    # explicit teardown before the interpreter exits: the verifier's device
    # memory is freed and the stream drained while the HIP runtime is whole
    sess.h.close()
    del sess
    torch.cuda.synchronize()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
