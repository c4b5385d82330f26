"""Seeded synthetic inputs for the verification step: model shapes, weights,
prompts, drafts and uniforms.

This module generates *inputs* only.  It holds none of the verification
method's arithmetic (no forward pass, no acceptance rule): it draws random
numbers, rounds them to the storage formats the target model is defined in
(bf16, fp16-scaled int4) and packs them.  Both the GPU library and the CPU
oracle consume what it produces.

Shapes follow the five workloads used throughout (tiny fp32 decoder,
LLaMA-2-7B-shaped bf16, the same shape quantized to int4 with fp16 group
scales, a Qwen2.5-7B-shaped GQA model with stochastic acceptance, and a
64-expert top-6 MoE), plus reduced "small" variants of each family that a
plain CPU implementation finishes in seconds.

Randomness: every tensor and every per-round draw uses numpy's PCG64 seeded
from a SeedSequence of integer words (config seed, stream id, index), so the
values do not depend on thread count or call order.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

# ----------------------------------------------------------------------------
# Model / workload description
# ----------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class ModelSpec:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int                  # dense FFN width (unused when n_experts > 0)
    vocab: int
    weight_dtype: str          # "f32" | "bf16" | "int4g128"
    kv_dtype: str              # "f32" | "bf16"
    n_experts: int = 0         # 0 => dense FFN
    top_k: int = 0
    n_shared: int = 0
    d_ff_expert: int = 0
    zipf_s: float = 1.1        # router-bias popularity exponent (MoE only)
    rope_theta: float = 10000.0
    rms_eps: float = 1e-5
    init_std: float = 0.02
    random_gains: bool = False  # small parity variants perturb norm gains
    group: int = 128           # int4 group size along K

    @property
    def moe(self) -> bool:
        return self.n_experts > 0

    @property
    def qkv_dim(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


@dataclasses.dataclass(frozen=True)
class Workload:
    spec: ModelSpec
    seed: int
    context: int               # prompt length (KV prefilled)
    k: int                     # drafts per round (headline k)
    k_sweep: tuple             # k values exercised
    corruption: float          # greedy drafts: prob. of replacing a draft id
    accept: str                # "greedy" | "stochastic"
    rounds: int = 16


def _dense(name, L, d, hq, hkv, D, ff, V, wdt, kvdt, **kw):
    return ModelSpec(name, L, d, hq, hkv, D, ff, V, wdt, kvdt, **kw)


# The five workloads (shapes, context, k, draft recipe) -------------------------
TINY = _dense("tiny", 2, 256, 4, 4, 64, 1024, 2048, "f32", "f32")
LLAMA7B = _dense("llama7b", 32, 4096, 32, 32, 128, 11008, 32000, "bf16", "bf16")
LLAMA7B_INT4 = _dense("llama7b_int4", 32, 4096, 32, 32, 128, 11008, 32000,
                      "int4g128", "bf16")
QWEN7B = _dense("qwen7b", 28, 3584, 28, 4, 128, 18944, 152064, "bf16", "bf16")
MOE = ModelSpec("moe", 16, 2048, 16, 4, 128, 0, 32000, "bf16", "bf16",
                n_experts=64, top_k=6, n_shared=1, d_ff_expert=1408)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(TINY, 1000, 64, 4, (4,), 0.3, "greedy"),
    "llama7b": Workload(LLAMA7B, 1001, 1024, 8, (1, 2, 4, 8, 15), 0.3, "greedy"),
    "llama7b_int4": Workload(LLAMA7B_INT4, 1002, 2048, 8, (8,), 0.4, "greedy"),
    "qwen7b": Workload(QWEN7B, 1003, 4096, 10, (10,), 0.0, "stochastic"),
    "moe": Workload(MOE, 1004, 2048, 8, (8,), 0.3, "greedy"),
}

# Reduced variants of each family.  Shapes are chosen so that GEMM column
# counts and K extents are not multiples of the kernels' tiles (ragged
# tails), contexts span several KV pages, and GQA group / MoE union logic
# is exercised, while the fp64 CPU oracle still finishes in seconds.
SMALL_WORKLOADS: Dict[str, Workload] = {
    "small_bf16": Workload(
        _dense("small_bf16", 3, 384, 3, 3, 128, 1400, 3001, "bf16", "bf16",
               random_gains=True), 2001, 150, 6, (0, 1, 6, 15), 0.3, "greedy"),
    "small_int4": Workload(
        _dense("small_int4", 2, 512, 4, 2, 128, 1408, 2500, "int4g128", "bf16",
               random_gains=True), 2002, 200, 8, (8,), 0.4, "greedy"),
    "small_gqa": Workload(
        _dense("small_gqa", 2, 896, 7, 1, 128, 1184, 4099, "bf16", "bf16",
               random_gains=True), 2003, 190, 10, (10,), 0.0, "stochastic"),
    "small_moe": Workload(
        ModelSpec("small_moe", 2, 512, 4, 2, 128, 0, 3001, "bf16", "bf16",
                  n_experts=16, top_k=6, n_shared=1, d_ff_expert=352,
                  random_gains=True), 2004, 130, 8, (8,), 0.3, "greedy"),
    "small_f32": Workload(
        _dense("small_f32", 2, 192, 3, 1, 64, 520, 1030, "f32", "f32",
               random_gains=True), 2005, 70, 5, (5,), 0.3, "greedy"),
}

ALL_WORKLOADS: Dict[str, Workload] = {**WORKLOADS, **SMALL_WORKLOADS}


# ----------------------------------------------------------------------------
# Storage-format helpers (generation side)
# ----------------------------------------------------------------------------


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


_CHUNK = 1 << 22


def normal_f32(n: int, std: float, words: List[int]) -> np.ndarray:
    """n draws of N(0, std^2) as fp32, chunked with one PCG64 stream per chunk
    so the result is independent of the number of worker threads."""
    out = np.empty(n, dtype=np.float32)
    nch = (n + _CHUNK - 1) // _CHUNK

    def work(i):
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(words) + [i])))
        seg = out[i * _CHUNK: min(n, (i + 1) * _CHUNK)]
        g.standard_normal(out=seg, dtype=np.float32)
        seg *= np.float32(std)

    if nch <= 1:
        for i in range(nch):
            work(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nch)))
    return out


def _bf16_parallel(a: np.ndarray) -> np.ndarray:
    flat = a.reshape(-1)
    out = np.empty(flat.size, dtype=np.uint16)
    nch = (flat.size + _CHUNK - 1) // _CHUNK

    def work(i):
        s = slice(i * _CHUNK, min(flat.size, (i + 1) * _CHUNK))
        out[s] = f32_to_bf16_bits(flat[s])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(nch)))
    return out.reshape(a.shape)


def quantize_int4_g128(w: np.ndarray, group: int = 128):
    """Symmetric group-wise int4 along K (axis 0) with fp16 scales.

    s = fp16(max|w| / 7) per (group, column); q = clamp(rint(w / s), -8, 7);
    an all-zero group has s = 0 and q = 0.  Returns (packed, scales): packed
    is uint8 [K/2, N] with the even-k element in the low nibble (two's
    complement nibbles), scales is float16 [K/group, N].  The quantized
    values q*s *are* the target model's weights.
    """
    K, N = w.shape
    assert K % group == 0, "K must be a multiple of the group size"
    G = K // group
    wg = w.reshape(G, group, N)
    amax = np.abs(wg).max(axis=1)                       # [G, N]
    s16 = (amax / np.float32(7.0)).astype(np.float16)   # fp16 scale
    s32 = s16.astype(np.float32)
    safe = np.where(s32 > 0, s32, np.float32(1.0))
    q = np.rint(wg / safe[:, None, :])
    q = np.clip(q, -8, 7)
    q = np.where(s32[:, None, :] > 0, q, 0).astype(np.int8).reshape(K, N)
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    return packed, s16


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """uint8 [K/2, N] -> int8 [K, N] (two's complement nibbles)."""
    lo = (packed & 0xF).astype(np.int8)
    hi = (packed >> 4).astype(np.int8)
    lo = np.where(lo >= 8, lo - 16, lo).astype(np.int8)
    hi = np.where(hi >= 8, hi - 16, hi).astype(np.int8)
    K2, N = packed.shape
    q = np.empty((2 * K2, N), dtype=np.int8)
    q[0::2] = lo
    q[1::2] = hi
    return q


# ----------------------------------------------------------------------------
# Weights
# ----------------------------------------------------------------------------


def tensor_list(spec: ModelSpec):
    """(name, shape, kind) for every tensor, in a fixed order.  kind is
    "matrix" (a matmul weight, quantized for int4 models), "embed", "gain"
    or "bias"."""
    d, V = spec.d_model, spec.vocab
    H, Hk, D = spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    out = [("embed", (V, d), "embed")]
    for i in range(spec.n_layers):
        p = f"l{i}."
        out += [(p + "attn_norm", (d,), "gain"),
                (p + "wq", (d, H * D), "matrix"),
                (p + "wk", (d, Hk * D), "matrix"),
                (p + "wv", (d, Hk * D), "matrix"),
                (p + "wo", (H * D, d), "matrix"),
                (p + "ffn_norm", (d,), "gain")]
        if spec.moe:
            E, F = spec.n_experts, spec.d_ff_expert
            out += [(p + "router", (d, E), "matrix"),
                    (p + "router_bias", (E,), "bias")]
            for e in range(E + spec.n_shared):
                q = p + f"x{e}."
                out += [(q + "w_gate", (d, F), "matrix"),
                        (q + "w_up", (d, F), "matrix"),
                        (q + "w_down", (F, d), "matrix")]
        else:
            F = spec.d_ff
            out += [(p + "w_gate", (d, F), "matrix"),
                    (p + "w_up", (d, F), "matrix"),
                    (p + "w_down", (F, d), "matrix")]
    out += [("final_norm", (d,), "gain"), ("lm_head", (d, V), "matrix")]
    return out


def zipf_router_bias(n_experts: int, s: float, words: List[int]) -> np.ndarray:
    """b_e = -s * ln(rank_e) with rank a seeded permutation of 1..E, so that
    softmax(b) is the Zipf(s) popularity law over the experts."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(words))))
    rank = g.permutation(n_experts) + 1
    return (-s * np.log(rank.astype(np.float64))).astype(np.float32)


def make_weights(spec: ModelSpec, seed: int) -> Dict[str, np.ndarray]:
    """All weights of the synthetic target.

    Matrices are stored [K, N] (y = x @ W).  Values are N(0, init_std^2):
    fp32 for "f32" models, bf16 bit patterns (uint16) for "bf16", and for
    "int4g128" every matmul weight is quantized (name + ".q" packed nibbles,
    name + ".s" fp16 scales) while the embedding stays bf16.  Norm gains are
    1 unless spec.random_gains (then 1 + N(0, 0.1^2), rounded to the model's
    storage type).  The MoE router bias follows zipf_router_bias.
    """
    W: Dict[str, np.ndarray] = {}
    for idx, (name, shape, kind) in enumerate(tensor_list(spec)):
        words = [seed, 7, idx]
        n = int(np.prod(shape))
        if kind == "gain":
            if spec.random_gains:
                g = normal_f32(n, 0.1, words) + np.float32(1.0)
            else:
                g = np.ones(n, np.float32)
            W[name] = g if spec.weight_dtype == "f32" else bf16_bits_to_f32(f32_to_bf16_bits(g))
            continue
        if kind == "bias":
            W[name] = zipf_router_bias(n, spec.zipf_s, words)
            continue
        w = normal_f32(n, spec.init_std, words).reshape(shape)
        if spec.weight_dtype == "f32":
            W[name] = w
        elif spec.weight_dtype == "bf16" or kind == "embed":
            W[name] = _bf16_parallel(w)
        else:  # int4g128 matrices
            K = shape[0]
            Kp = ((K + spec.group - 1) // spec.group) * spec.group
            if Kp != K:
                raise ValueError("int4 matrices need K divisible by the group size")
            q, s = quantize_int4_g128(w, spec.group)
            W[name + ".q"] = q
            W[name + ".s"] = s
        del w
    return W


def weight_nbytes(W: Dict[str, np.ndarray]) -> int:
    return int(sum(a.nbytes for a in W.values()))


# ----------------------------------------------------------------------------
# Per-round inputs: prompt, draft corruption, uniforms, draft noise
# ----------------------------------------------------------------------------


def _rng(*words) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(w) for w in words])))


def prompt_ids(w: Workload, length: Optional[int] = None) -> np.ndarray:
    n = w.context if length is None else length
    return _rng(w.seed, 11).integers(0, w.spec.vocab, size=n, dtype=np.int64).astype(np.int32)


def corrupt_drafts(w: Workload, rnd: int, true_next: np.ndarray, c: Optional[float] = None) -> np.ndarray:
    """Drafts for round `rnd`: the target's greedy continuation `true_next`
    (length k) with each id independently replaced, with probability c, by a
    uniform id on [0, V).  Exactly k flags and k ids are drawn per round, so
    the stream does not depend on acceptance."""
    flags, ids = draft_corruption(w, rnd, len(true_next), c)
    return np.where(flags, ids, np.asarray(true_next, dtype=np.int64)).astype(np.int32)


def draft_corruption(w: Workload, rnd: int, k: int, c: Optional[float] = None):
    """The k replacement flags and k replacement ids of round `rnd` (what
    corrupt_drafts applies), so a timing loop can draw them ahead of time."""
    c = w.corruption if c is None else c
    g = _rng(w.seed, 13, rnd, k)
    flags = g.random(k) < c
    ids = g.integers(0, w.spec.vocab, size=k, dtype=np.int64)
    return flags, ids


def round_uniforms(w: Workload, rnd: int, k: int) -> np.ndarray:
    """u_1..u_k (acceptance tests) and u_{k+1} (final draw) for one round,
    fp32 in [0, 1)."""
    return _rng(w.seed, 17, rnd, k).random(k + 1, dtype=np.float64).astype(np.float32)


def draft_noise(w: Workload, rnd: int, i: int) -> np.ndarray:
    """eps_i ~ N(0,1)^V added to the target logits to form the draft
    distribution q_i = softmax(z_i + eps_i) for stochastic workloads."""
    return _rng(w.seed, 19, rnd, i).standard_normal(w.spec.vocab, dtype=np.float32)


def draft_sample_uniform(w: Workload, rnd: int, i: int) -> float:
    """Uniform used to draw d_i from q_i (inverse CDF)."""
    return float(_rng(w.seed, 23, rnd, i).random())


def first_pending_uniform(w: Workload) -> float:
    return float(_rng(w.seed, 29).random())


def synthetic_prompt_kv(w: Workload, length: Optional[int] = None):
    """A seeded stand-in for a prefilled prompt cache at full model size:
    keys and values [n_layers, n_kv_heads, P, head_dim] drawn from
    N(0, (init_std * sqrt(d_model))^2) -- the spread of x.W for a unit-RMS
    row x and N(0, init_std^2) weights -- and stored in the KV dtype (bf16
    bit patterns as uint16, or fp32)."""
    s = w.spec
    P = w.context if length is None else length
    std = s.init_std * math.sqrt(s.d_model)
    shape = (s.n_layers, s.n_kv_heads, P, s.head_dim)
    n = int(np.prod(shape))
    K = normal_f32(n, std, [w.seed, 31]).reshape(shape)
    V = normal_f32(n, std, [w.seed, 37]).reshape(shape)
    if s.kv_dtype == "bf16":
        return _bf16_parallel(K), _bf16_parallel(V)
    return K, V


def synthetic_pending(w: Workload) -> int:
    """First pending token when the prompt cache is synthetic (no prefill
    produced one): a seeded uniform id."""
    return int(_rng(w.seed, 47).integers(0, w.spec.vocab))
