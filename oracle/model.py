"""Block forward pass of the target model, prefill, and greedy
autoregressive decode.

Test infrastructure only (see the package docstring).

What is computed (plain reading of the pages; every point the pages leave
open is listed with its reading in the design notes):

* One target pass over a block of m tokens at positions L..L+m-1 returns m
  rows of logits; row j is the target's prediction for the position after
  block token j.  The block is "one list" fed at once, and causal masking
  makes every row identical to a pass over the shorter prefix (essay "LLM
  Inference: Speculative Decoding", "The four sentences are already inside
  one sentence"; "The loop", step 2).
* Per layer: h = rmsnorm(x)*g1; q,k,v = h Wq, h Wk, h Wv; rotary embedding
  on q,k at absolute positions; k,v rounded to the KV dtype and appended;
  causal attention over cached entries; x += o Wo; h' = rmsnorm(x)*g2;
  dense: x += (silu(h' Wg) * (h' Wu)) Wd;
  MoE: x += sum_{e in top_k(pi)} pi_e FFN_e(h') + FFN_shared(h'),
  pi = softmax(h' Wr + b) over all experts (S2-MoE section 2.1: each token
  runs only a few of the experts).
  Final: logits = (rmsnorm(x) * g_f) W_lm.
* The KV cache here is an array with room for max_ctx positions plus a
  committed length; entries past the committed length are dead and never
  read (essay "The loop", step 5).
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

from . import numerics as nx


def _threads() -> int:
    import os
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 1


def _to_float(name: str, W: Dict[str, np.ndarray], spec, dtype) -> np.ndarray:
    """Read one weight from its storage format into `dtype`."""
    if name + ".q" in W:
        return nx.dequant_int4(W[name + ".q"], W[name + ".s"], spec.group, dtype)
    a = W[name]
    if a.dtype == np.uint16:
        return nx.bf16_bits_to_float(a, dtype)
    return np.asarray(a, dtype=dtype)


class OracleModel:
    """The synthetic target model, weights read into `dtype` (float64 by
    default).  `spec` is a ModelSpec-like object (attributes only)."""

    def __init__(self, spec, W: Dict[str, np.ndarray], dtype=np.float64):
        self.spec = spec
        self.dtype = dtype
        names = []
        for name in list(W.keys()):
            base = name[:-2] if (name.endswith(".q") or name.endswith(".s")) else name
            if base not in names:
                names.append(base)
        with ThreadPoolExecutor(_threads()) as ex:
            arrs = list(ex.map(lambda n: _to_float(n, W, spec, dtype), names))
        self.w: Dict[str, np.ndarray] = dict(zip(names, arrs))

    def __getitem__(self, name):
        return self.w[name]


@dataclasses.dataclass
class KVCache:
    """K[l], V[l]: [Hkv, max_ctx, D]; `length` = committed entries."""
    K: List[np.ndarray]
    V: List[np.ndarray]
    length: int

    @staticmethod
    def empty(spec, max_ctx: int, dtype=np.float64) -> "KVCache":
        shp = (spec.n_kv_heads, max_ctx, spec.head_dim)
        return KVCache([np.zeros(shp, dtype) for _ in range(spec.n_layers)],
                       [np.zeros(shp, dtype) for _ in range(spec.n_layers)], 0)

    def copy(self) -> "KVCache":
        return KVCache([k.copy() for k in self.K], [v.copy() for v in self.V], self.length)

    def astype(self, dtype) -> "KVCache":
        return KVCache([k.astype(dtype) for k in self.K], [v.astype(dtype) for v in self.V], self.length)


@dataclasses.dataclass
class BlockResult:
    logits: np.ndarray                 # [m, V]
    new_k: List[np.ndarray]            # per layer [Hkv, m, D] (rounded)
    new_v: List[np.ndarray]
    routing: Optional[List[dict]] = None   # MoE: per layer routing facts
    trace: Optional[List[np.ndarray]] = None  # residual stream after each layer


def reuse_gating_logits(r: np.ndarray, w: np.ndarray, top_k: int, cap: int, alpha: float):
    """Reuse-aware expert gating (S2-MoE section 4.2), step by step on a
    block's gating logits r [m, E]:
      1. importance of expert e: g_e = sum_b w_b r_{b,e} (w: row confidences);
      2. preferred experts: the `cap` experts of largest importance, ties to
         the lower id;
      3. each row b adds lambda_b = alpha (r_b(1) - r_b(top_k+1)), its first
         minus its (top_k+1)-th logit, to the preferred experts' logits.
    Returns (biased logits [m, E], preferred mask [E], gap between the cap-th
    and the (cap+1)-th importance)."""
    r = np.asarray(r, dtype=np.float64)
    m, E = r.shape
    g = np.zeros(E)
    for b in range(m):
        g = g + float(w[b]) * r[b]
    order = np.argsort(-g, kind="stable")
    pref = np.zeros(E, dtype=bool)
    pref[order[:cap]] = True
    cap_gap = float(g[order[cap - 1]] - g[order[cap]]) if cap < E else np.inf
    srt = np.sort(r, axis=-1)[:, ::-1]
    lam = alpha * (srt[:, 0] - srt[:, top_k])
    return r + lam[:, None] * pref[None, :], pref, cap_gap


def route(M: OracleModel, layer: int, h: np.ndarray, top_k: Optional[int] = None, reuse=None):
    """MoE router for a block: pi = softmax(h Wr + b) over all experts; each
    token keeps its top_k experts by probability (the model's top_k unless
    given: a self-speculative draft keeps fewer), ties to the lower expert
    id; weights are the (unrenormalized) probabilities.  reuse = (w, cap,
    alpha) first biases the gating logits (reuse_gating_logits).  Returns
    (pi [m,E], sel [m,top_k] expert ids in rank order, r [m,E] logits)."""
    spec = M.spec
    top_k = spec.top_k if top_k is None else top_k
    r = h @ M[f"l{layer}.router"] + M[f"l{layer}.router_bias"].astype(h.dtype)
    if reuse is not None:
        w, cap, alpha = reuse
        r, _, _ = reuse_gating_logits(r, w, top_k, cap, alpha)
        r = r.astype(h.dtype)
    pi = nx.softmax(r, axis=-1)
    order = np.argsort(-pi, axis=-1, kind="stable")    # descending, ties -> lower id
    sel = order[:, :top_k]
    return pi, sel, r


def expert_ffn(M: OracleModel, layer: int, e: int, h: np.ndarray) -> np.ndarray:
    p = f"l{layer}.x{e}."
    return (nx.silu(h @ M[p + "w_gate"]) * (h @ M[p + "w_up"])) @ M[p + "w_down"]


def moe_ffn(M: OracleModel, layer: int, h: np.ndarray, top_k: Optional[int] = None, reuse=None):
    """x-update of a MoE layer for a block of tokens h [m, d].

    For each token j, y_j = sum over its selected experts e of
    pi_{j,e} * FFN_e(h_j), plus the shared expert(s) with weight 1.  Each
    selected expert's FFN is evaluated on the rows that selected it (a
    matmul over those rows); the per-token sum runs over the token's experts
    in rank order, then the shared experts.
    """
    spec = M.spec
    top_k = spec.top_k if top_k is None else top_k
    m = h.shape[0]
    pi, sel, r = route(M, layer, h, top_k, reuse)
    out = {}
    union = sorted(set(int(e) for e in sel.reshape(-1)))
    for e in union:
        rows = np.nonzero((sel == e).any(axis=1))[0]
        ye = expert_ffn(M, layer, e, h[rows])
        for i, j in enumerate(rows):
            out[(int(j), e)] = ye[i]
    y = np.zeros_like(h)
    for j in range(m):
        for e in sel[j]:
            y[j] += pi[j, e] * out[(j, int(e))]
    for s in range(spec.n_shared):
        y += expert_ffn(M, layer, spec.n_experts + s, h)
    # routing facts for near-tie flags and byte accounting
    srt = np.sort(r, axis=-1)[:, ::-1]
    gap = srt[:, top_k - 1] - srt[:, top_k] if top_k < spec.n_experts else np.full(m, np.inf)
    info = dict(sel=sel, union=union, topk_gap=gap)
    if reuse is not None:
        r0 = h @ M[f"l{layer}.router"] + M[f"l{layer}.router_bias"].astype(h.dtype)
        info["cap_gap"] = reuse_gating_logits(r0, reuse[0], top_k, reuse[1], reuse[2])[2]
    return y, info


def forward_block(M: OracleModel, kv: KVCache, tokens, L: int, trace: bool = False,
                  top_k: Optional[int] = None, reuse=None) -> BlockResult:
    """One target pass over `tokens` at positions L..L+m-1 against the
    committed cache entries [0, L).  Writes the block's rounded k,v at
    positions L..L+m-1 of `kv` (dead until committed) and returns the m rows
    of logits.  kv.length is not changed.  top_k (MoE): routed experts per
    token, the model's own unless given; reuse = (w [m], cap, alpha): the
    lossy reuse-aware gating of every MoE layer (reuse_gating_logits)."""
    spec = M.spec
    dt = M.dtype
    tokens = np.asarray(tokens, dtype=np.int64)
    m = len(tokens)
    H, Hk, D = spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    if L + m > kv.K[0].shape[1]:
        raise ValueError("block exceeds cache capacity")
    pos = L + np.arange(m)
    x = M["embed"][tokens].astype(dt)
    new_k, new_v, routing, tr = [], [], [], []
    for l in range(spec.n_layers):
        p = f"l{l}."
        h = nx.rmsnorm(x, M[p + "attn_norm"], spec.rms_eps)
        q = (h @ M[p + "wq"]).reshape(m, H, D)
        k = (h @ M[p + "wk"]).reshape(m, Hk, D)
        v = (h @ M[p + "wv"]).reshape(m, Hk, D)
        q = nx.rope(q, pos, spec.rope_theta)
        k = nx.rope(k, pos, spec.rope_theta)
        k = nx.round_kv(k, spec.kv_dtype)
        v = nx.round_kv(v, spec.kv_dtype)
        kv.K[l][:, L:L + m, :] = k.transpose(1, 0, 2)
        kv.V[l][:, L:L + m, :] = v.transpose(1, 0, 2)
        new_k.append(k.transpose(1, 0, 2).copy())
        new_v.append(v.transpose(1, 0, 2).copy())
        o = nx.causal_attention(q, kv.K[l], kv.V[l], L)
        x = x + o.reshape(m, H * D) @ M[p + "wo"]
        h2 = nx.rmsnorm(x, M[p + "ffn_norm"], spec.rms_eps)
        if spec.n_experts > 0:
            y, info = moe_ffn(M, l, h2, top_k, reuse)
            routing.append(info)
            x = x + y
        else:
            x = x + (nx.silu(h2 @ M[p + "w_gate"]) * (h2 @ M[p + "w_up"])) @ M[p + "w_down"]
        if trace:
            tr.append(x.copy())
    logits = nx.rmsnorm(x, M["final_norm"], spec.rms_eps) @ M["lm_head"]
    return BlockResult(logits, new_k, new_v, routing if spec.n_experts > 0 else None,
                       tr if trace else None)


def prefill(M: OracleModel, prompt, max_ctx: int, kv_dtype=None) -> (KVCache, np.ndarray):
    """Fill the cache with the prompt's keys/values in one block pass and
    return (cache with length = len(prompt), logits of the last prompt
    position)."""
    kv = KVCache.empty(M.spec, max_ctx, kv_dtype or M.dtype)
    res = forward_block(M, kv, prompt, 0)
    kv.length = len(prompt)
    return kv, res.logits[-1]


def draft_greedy(M: OracleModel, kv: KVCache, pending: int, n: int, top_k: int):
    """Self-speculative draft of a MoE target by expert sparsity (S2-MoE
    section 2.3 and section 5 "Draft configuration": the same model with
    fewer routed experts per token; section 4.3: the draft reads the
    target's cache and its own writes are temporary).  n single-token passes
    with top_k routed experts, pass i at position kv.length + i on a copy of
    the cache (the draft's entries never reach `kv`), each draft token the
    argmax of the previous pass (lowest id on ties).  Returns (tokens [n],
    logits [n, V], per-pass routing facts)."""
    scratch = kv.copy()
    L = kv.length
    toks, rows, routing = [], [], []
    tok = int(pending)
    for i in range(n):
        res = forward_block(M, scratch, [tok], L + i, top_k=top_k)
        tok = int(np.argmax(res.logits[0]))
        toks.append(tok)
        rows.append(res.logits[0])
        routing.append(res.routing)
    return np.asarray(toks, dtype=np.int32), np.stack(rows), routing


def ar_decode(M: OracleModel, kv: KVCache, pending: int, n: int) -> np.ndarray:
    """Greedy autoregressive decode: n single-token passes.  Returns the n
    tokens produced after `pending` (argmax each step, lowest id on ties);
    the cache ends with pending and the first n-1 of them committed."""
    kv = kv.copy()
    out = []
    tok = int(pending)
    for _ in range(n):
        res = forward_block(M, kv, [tok], kv.length)
        kv.length += 1
        tok = int(np.argmax(res.logits[0]))
        out.append(tok)
    return np.asarray(out, dtype=np.int32)
