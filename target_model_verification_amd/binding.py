"""Thin ctypes binding of libspecverify.so (include/spec_verify.h).

Argument marshalling only: every step of the verification pass runs in the
library's HIP kernels.  PyTorch (when used by callers) only provides device
memory and streams; this module accepts plain integers as device pointers
and stream handles.  Importing it fails loudly if the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecverify.so")

SPEC_OK, SPEC_EINVAL, SPEC_ENOMEM, SPEC_ECAPACITY, SPEC_EHIP, SPEC_ESTATE = 0, -1, -2, -3, -4, -5
SPEC_DT_F32, SPEC_DT_BF16, SPEC_DT_INT4G128 = 0, 1, 2
SPEC_ACCEPT_GREEDY, SPEC_ACCEPT_STOCHASTIC, SPEC_ACCEPT_NONE = 0, 1, 2
(SPEC_T_EMBED, SPEC_T_FINAL_NORM, SPEC_T_LM_HEAD, SPEC_T_ATTN_NORM, SPEC_T_WQ, SPEC_T_WK, SPEC_T_WV,
 SPEC_T_WO, SPEC_T_FFN_NORM, SPEC_T_W_GATE, SPEC_T_W_UP, SPEC_T_W_DOWN, SPEC_T_ROUTER,
 SPEC_T_ROUTER_BIAS) = range(14)
KERNEL_CLASSES = ["embed", "qkv", "attn", "attn_combine", "o", "gateup", "down", "router", "route",
                  "expert_gateup", "expert_down", "moe_combine", "lmhead", "accept", "pass"]
SPEC_K_NCLASSES = len(KERNEL_CLASSES)


class SpecConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "d_ff", "vocab",
                 "n_experts", "top_k", "n_shared", "d_ff_expert", "weight_dtype", "kv_dtype")] + \
               [("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("max_ctx", ctypes.c_int32), ("max_k", ctypes.c_int32), ("gemm_k_split", ctypes.c_int32),
                ("kv_page_seed", ctypes.c_int32), ("n_seqs", ctypes.c_int32),
                ("attn_group_pages", ctypes.c_int32), ("reserved", ctypes.c_int32 * 4)]


class SpecTensor(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("layer", ctypes.c_int32), ("expert", ctypes.c_int32),
                ("part", ctypes.c_int32), ("data", ctypes.c_void_p), ("bytes", ctypes.c_uint64)]


class SpecStepResult(ctypes.Structure):
    _fields_ = [("n_accepted", ctypes.c_int32), ("next_token", ctypes.c_int32), ("kv_len", ctypes.c_int32)]


def _load():
    # One HIP runtime per process: PyTorch (which supplies device memory and
    # streams to callers) loads its own libamdhip64 under an unversioned
    # name; loading it first lets this library bind to that same runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not built: run target_model_verification_amd.build_lib "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_double
    sig = {
        "spec_config_check": (I, [ctypes.POINTER(SpecConfig), ctypes.c_char_p, I]),
        "spec_plan_check": (I, [ctypes.POINTER(SpecConfig), I, ctypes.c_char_p, I]),
        "spec_verify_create": (I, [ctypes.POINTER(SpecConfig), ctypes.POINTER(SpecTensor), I, P, P, I, P,
                                   ctypes.POINTER(P)]),
        "spec_verify_step": (I, [P, ctypes.POINTER(ctypes.c_int32), I, I, P, P,
                                 ctypes.POINTER(SpecStepResult), P]),
        "spec_verify_step_debug": (I, [P, ctypes.POINTER(ctypes.c_int32), I, I, P, P,
                                       ctypes.POINTER(SpecStepResult), P, P, P, P]),
        "spec_kv_commit_rollback": (I, [P, I]),
        "spec_kv_len": (I, [P]),
        "spec_last_error": (ctypes.c_char_p, [P]),
        "spec_verify_destroy": (None, [P]),
        "spec_profile_enable": (I, [P, I]),
        "spec_profile_read": (I, [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(D), ctypes.POINTER(D)]),
        "spec_profile_detail": (I, [P, ctypes.POINTER(D)]),
        "spec_profile_raw": (I, [P, ctypes.POINTER(ctypes.c_uint64), ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
        "spec_pass_bytes": (D, [P, I, I, I, ctypes.c_int64]),
        "spec_kv_poison_dead": (I, [P]),
        "spec_draft": (I, [P, I, I, I, ctypes.POINTER(ctypes.c_int32), P, P]),
        "spec_tree_expand": (I, [I, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(D), ctypes.POINTER(ctypes.c_int32),
                                 ctypes.POINTER(ctypes.c_int32), I, ctypes.POINTER(ctypes.c_int32), D, D,
                                 ctypes.POINTER(D), I, ctypes.POINTER(ctypes.c_int32),
                                 ctypes.POINTER(ctypes.c_int32)]),
        "spec_adaptive_k": (I, [I, I, I]),
        "spec_verify_batch": (I, [P, I, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                  ctypes.POINTER(ctypes.c_int32), I, ctypes.POINTER(SpecStepResult), P]),
        "spec_seq_kv_len": (I, [P, I]),
        "spec_debug_fail_alloc": (ctypes.c_int64, [ctypes.c_int64]),
        "spec_seq_rollback": (I, [P, I, I]),
        "spec_seq_import": (I, [P, I, P, P, I]),
        "spec_verify_tree": (I, [P, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32), I,
                                 ctypes.POINTER(SpecStepResult), ctypes.POINTER(ctypes.c_int32), P]),
        "spec_verify_step_reuse": (I, [P, ctypes.POINTER(ctypes.c_int32), I, I, P, P, P, I, F,
                                       ctypes.POINTER(SpecStepResult), P, P, P]),
        "spec_verify_step_noalloc": (I, [P, ctypes.POINTER(ctypes.c_int32), I, I, P, P,
                                         ctypes.POINTER(SpecStepResult), P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()

# same names as the C ABI -------------------------------------------------------
spec_config_check = lib.spec_config_check
spec_plan_check = lib.spec_plan_check
spec_verify_create = lib.spec_verify_create
spec_verify_step = lib.spec_verify_step
spec_verify_step_debug = lib.spec_verify_step_debug
spec_kv_commit_rollback = lib.spec_kv_commit_rollback
spec_kv_len = lib.spec_kv_len
spec_last_error = lib.spec_last_error
spec_verify_destroy = lib.spec_verify_destroy
spec_profile_enable = lib.spec_profile_enable
spec_profile_read = lib.spec_profile_read
spec_profile_detail = lib.spec_profile_detail
spec_profile_raw = lib.spec_profile_raw
spec_pass_bytes = lib.spec_pass_bytes
spec_kv_poison_dead = lib.spec_kv_poison_dead
spec_draft = lib.spec_draft
spec_adaptive_k = lib.spec_adaptive_k
spec_verify_tree = lib.spec_verify_tree
spec_tree_expand = lib.spec_tree_expand
spec_verify_batch = lib.spec_verify_batch
spec_seq_kv_len = lib.spec_seq_kv_len
spec_debug_fail_alloc = lib.spec_debug_fail_alloc
spec_seq_rollback = lib.spec_seq_rollback
spec_seq_import = lib.spec_seq_import
spec_verify_step_reuse = lib.spec_verify_step_reuse
spec_verify_step_noalloc = lib.spec_verify_step_noalloc


class SpecError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"spec_verify error {code}: {msg}")
        self.code = code


_DT = {"f32": SPEC_DT_F32, "bf16": SPEC_DT_BF16, "int4g128": SPEC_DT_INT4G128}


def make_config(spec, max_ctx: int, max_k: int, gemm_k_split: int = 0, kv_page_seed: int = 0,
                n_seqs: int = 0, attn_group_pages: int = 0) -> SpecConfig:
    c = SpecConfig()
    c.n_layers, c.d_model = spec.n_layers, spec.d_model
    c.n_q_heads, c.n_kv_heads, c.head_dim = spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    c.d_ff, c.vocab = spec.d_ff, spec.vocab
    c.n_experts, c.top_k, c.n_shared, c.d_ff_expert = spec.n_experts, spec.top_k, spec.n_shared, spec.d_ff_expert
    c.weight_dtype, c.kv_dtype = _DT[spec.weight_dtype], _DT[spec.kv_dtype]
    c.rope_theta, c.rms_eps = spec.rope_theta, spec.rms_eps
    c.max_ctx, c.max_k, c.gemm_k_split = max_ctx, max_k, gemm_k_split
    c.kv_page_seed = kv_page_seed
    c.n_seqs = n_seqs
    c.attn_group_pages = attn_group_pages
    return c


_KIND = {"wq": SPEC_T_WQ, "wk": SPEC_T_WK, "wv": SPEC_T_WV, "wo": SPEC_T_WO, "w_gate": SPEC_T_W_GATE,
         "w_up": SPEC_T_W_UP, "w_down": SPEC_T_W_DOWN, "router": SPEC_T_ROUTER,
         "router_bias": SPEC_T_ROUTER_BIAS, "attn_norm": SPEC_T_ATTN_NORM, "ffn_norm": SPEC_T_FFN_NORM}


def make_tensors(W: Dict[str, np.ndarray]):
    """Weight dict (names as produced by the synthetic generator) ->
    (ctypes array of SpecTensor, keep-alive list)."""
    out: List[SpecTensor] = []
    keep = []
    for name, arr in W.items():
        a = np.ascontiguousarray(arr)
        if a.dtype == np.float64:
            a = a.astype(np.float32)
        keep.append(a)
        part = 0
        base = name
        if name.endswith(".q"):
            base = name[:-2]
        elif name.endswith(".s"):
            base, part = name[:-2], 1
        toks = base.split(".")
        layer, expert = -1, -1
        if base == "embed":
            kind = SPEC_T_EMBED
        elif base == "final_norm":
            kind = SPEC_T_FINAL_NORM
        elif base == "lm_head":
            kind = SPEC_T_LM_HEAD
        else:
            layer = int(toks[0][1:])
            if toks[1].startswith("x"):
                expert = int(toks[1][1:])
                kind = _KIND[toks[2]]
            else:
                kind = _KIND[toks[1]]
        out.append(SpecTensor(kind, layer, expert, part, a.ctypes.data, a.nbytes))
    arr = (SpecTensor * len(out))(*out)
    return arr, keep


class Verifier:
    """Owns one spec_verify_t handle."""

    def __init__(self, spec, W, prompt_k: Optional[np.ndarray], prompt_v: Optional[np.ndarray],
                 prompt_len: int, max_ctx: int, max_k: int, stream: int = 0, gemm_k_split: int = 0,
                 kv_page_seed: int = 0, n_seqs: int = 0, attn_group_pages: int = 0):
        self.spec = spec
        self.cfg = make_config(spec, max_ctx, max_k, gemm_k_split, kv_page_seed, n_seqs, attn_group_pages)
        tens, keep = make_tensors(W)
        pk = pv = None
        if prompt_len > 0:
            pk = np.ascontiguousarray(prompt_k)
            pv = np.ascontiguousarray(prompt_v)
        h = ctypes.c_void_p()
        rc = spec_verify_create(ctypes.byref(self.cfg), tens, len(tens),
                                pk.ctypes.data if pk is not None else None,
                                pv.ctypes.data if pv is not None else None,
                                prompt_len, ctypes.c_void_p(stream), ctypes.byref(h))
        del keep
        if rc != SPEC_OK:
            raise SpecError(rc, "spec_verify_create failed (details on stderr)")
        self.h = h

    def step(self, tokens: Sequence[int], mode: int = SPEC_ACCEPT_GREEDY, q_ptr: int = 0, u_ptr: int = 0,
             logits_ptr: int = 0, trace_ptr: int = 0, union_ptr: int = 0, route_ptr: int = 0,
             noalloc: bool = False) -> SpecStepResult:
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        k = len(t) - 1
        res = SpecStepResult()
        tp = t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        if noalloc:
            rc = spec_verify_step_noalloc(self.h, tp, k, mode, q_ptr or None, u_ptr or None, ctypes.byref(res),
                                          logits_ptr or None)
        elif trace_ptr or union_ptr or route_ptr:
            rc = spec_verify_step_debug(self.h, tp, k, mode, q_ptr or None, u_ptr or None, ctypes.byref(res),
                                        logits_ptr or None, trace_ptr or None, union_ptr or None,
                                        route_ptr or None)
        else:
            rc = spec_verify_step(self.h, tp, k, mode, q_ptr or None, u_ptr or None, ctypes.byref(res),
                                  logits_ptr or None)
        if rc != SPEC_OK:
            raise SpecError(rc, self.last_error())
        return res

    def draft(self, pending: int, n: int, draft_top_k: int, logits_ptr: int = 0, route_ptr: int = 0) -> List[int]:
        """Self-speculative draft tokens d_1..d_n (spec_draft)."""
        out = (ctypes.c_int32 * n)()
        rc = spec_draft(self.h, int(pending), int(n), int(draft_top_k), out, logits_ptr or None, route_ptr or None)
        if rc != SPEC_OK:
            raise SpecError(rc, self.last_error())
        return [int(x) for x in out]

    def step_reuse(self, tokens: Sequence[int], cap: int, alpha: float, mode: int = SPEC_ACCEPT_GREEDY,
                   q_ptr: int = 0, u_ptr: int = 0, conf_ptr: int = 0, logits_ptr: int = 0, union_ptr: int = 0,
                   route_ptr: int = 0) -> SpecStepResult:
        """Verification step with reuse-aware expert gating (lossy)."""
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        res = SpecStepResult()
        rc = spec_verify_step_reuse(self.h, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(t) - 1, mode,
                                    q_ptr or None, u_ptr or None, conf_ptr or None, cap, alpha,
                                    ctypes.byref(res), logits_ptr or None, union_ptr or None, route_ptr or None)
        if rc != SPEC_OK:
            raise SpecError(rc, self.last_error())
        return res

    def step_tree(self, tokens: Sequence[int], parents: Sequence[int], logits_ptr: int = 0):
        """Token-tree verification (greedy): (result, accepted rows)."""
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        pa = np.ascontiguousarray(np.asarray(parents, dtype=np.int32))
        res = SpecStepResult()
        path = (ctypes.c_int32 * len(t))()
        rc = spec_verify_tree(self.h, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                              pa.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(t), ctypes.byref(res), path,
                              logits_ptr or None)
        if rc != SPEC_OK:
            raise SpecError(rc, self.last_error())
        return res, [int(path[i]) for i in range(res.n_accepted)]

    def step_batch(self, seqs: Sequence[int], blocks, mode: int = SPEC_ACCEPT_GREEDY, logits_ptr: int = 0):
        """Several sequences' blocks in one pass (spec_verify_batch):
        blocks[i] = [pending, d_1 .. d_k] of sequence seqs[i].  Returns one
        result per sequence."""
        n = len(seqs)
        sq = np.ascontiguousarray(np.asarray(seqs, dtype=np.int32))
        ks = np.ascontiguousarray(np.asarray([len(b) - 1 for b in blocks], dtype=np.int32))
        tk = np.ascontiguousarray(np.concatenate([np.asarray(b, dtype=np.int32) for b in blocks]))
        out = (SpecStepResult * n)()
        P32 = ctypes.POINTER(ctypes.c_int32)
        rc = spec_verify_batch(self.h, n, sq.ctypes.data_as(P32), tk.ctypes.data_as(P32), ks.ctypes.data_as(P32),
                               int(mode), out, logits_ptr or None)
        if rc != SPEC_OK:
            raise SpecError(rc, self.last_error())
        return [out[i] for i in range(n)]

    def seq_len(self, seq: int) -> int:
        return int(spec_seq_kv_len(self.h, int(seq)))

    def seq_rollback(self, seq: int, new_len: int) -> None:
        rc = spec_seq_rollback(self.h, int(seq), int(new_len))
        if rc != SPEC_OK:
            raise SpecError(rc, self.last_error())

    def seq_import(self, seq: int, k: np.ndarray, v: np.ndarray, length: int) -> None:
        kk, vv = np.ascontiguousarray(k), np.ascontiguousarray(v)
        rc = spec_seq_import(self.h, int(seq), kk.ctypes.data, vv.ctypes.data, int(length))
        if rc != SPEC_OK:
            raise SpecError(rc, self.last_error())

    def rollback(self, new_len: int) -> None:
        rc = spec_kv_commit_rollback(self.h, new_len)
        if rc != SPEC_OK:
            raise SpecError(rc, self.last_error())

    @property
    def kv_len(self) -> int:
        return spec_kv_len(self.h)

    def last_error(self) -> str:
        return spec_last_error(self.h).decode(errors="replace")

    def profile(self, on) -> None:
        """on: False/0 off, True/1 events + per-phase stamps, 2 events only."""
        rc = spec_profile_enable(self.h, int(on))
        if rc != SPEC_OK:
            raise SpecError(rc, self.last_error())

    def poison_dead(self) -> None:
        rc = spec_kv_poison_dead(self.h)
        if rc != SPEC_OK:
            raise SpecError(rc, self.last_error())

    def profile_read(self):
        n = (ctypes.c_int64 * SPEC_K_NCLASSES)()
        ms = (ctypes.c_double * SPEC_K_NCLASSES)()
        by = (ctypes.c_double * SPEC_K_NCLASSES)()
        spec_profile_read(self.h, n, ms, by)
        return {KERNEL_CLASSES[i]: (int(n[i]), float(ms[i]), float(by[i])) for i in range(SPEC_K_NCLASSES)}

    def profile_detail(self):
        """Per class: ((stage, stream, flush, work) means, (...) maxima) over
        workgroups, ms summed over launches."""
        out = (ctypes.c_double * (8 * SPEC_K_NCLASSES))()
        spec_profile_detail(self.h, out)
        return {KERNEL_CLASSES[i]: (tuple(float(out[8 * i + j]) for j in range(4)),
                                    tuple(float(out[8 * i + 4 + j]) for j in range(4)))
                for i in range(SPEC_K_NCLASSES)}

    def profile_raw(self) -> np.ndarray:
        """Per-workgroup stamps of the last profiled step: [phases][n_wg][4]
        device wall-clock ticks (flattened; see spec_profile_raw)."""
        n = ctypes.c_int64()
        spec_profile_raw(self.h, None, 0, ctypes.byref(n))
        out = np.zeros(n.value, dtype=np.uint64)
        rc = spec_profile_raw(self.h, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), n.value, None)
        if rc != SPEC_OK:
            raise SpecError(rc, self.last_error())
        return out

    def pass_bytes(self, L: int, k: int, mode: int = SPEC_ACCEPT_GREEDY, experts_loaded: int = 0) -> float:
        return spec_pass_bytes(self.h, L, k, mode, experts_loaded)

    def close(self) -> None:
        if getattr(self, "h", None):
            spec_verify_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tree_expand(parents, p, experts, base, t_ar: float, t_exp: float, c_draft, max_nodes: int):
    """spec_tree_expand on Python lists: (admitted candidates in order,
    parent rows of the verification tree)."""
    n = len(parents)
    i32 = lambda a: np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    f64 = lambda a: np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    off = i32(np.concatenate([[0], np.cumsum([len(e) for e in experts])]) if n else [0])
    ids = i32([e for ex in experts for e in ex] or [0])
    pa, pp, cd, bs = i32(parents if n else [0]), f64(p if n else [0]), f64(c_draft if n else [0]), i32(list(base) or [0])
    order = (ctypes.c_int32 * max(max_nodes, 1))()
    rows = (ctypes.c_int32 * (max_nodes + 1))()
    P32 = ctypes.POINTER(ctypes.c_int32)
    PD = ctypes.POINTER(ctypes.c_double)
    cnt = spec_tree_expand(n, pa.ctypes.data_as(P32), pp.ctypes.data_as(PD), off.ctypes.data_as(P32),
                           ids.ctypes.data_as(P32), len(base), bs.ctypes.data_as(P32), float(t_ar), float(t_exp),
                           cd.ctypes.data_as(PD), int(max_nodes), order, rows)
    if cnt < 0:
        raise ValueError("spec_tree_expand: invalid arguments")
    return [int(order[i]) for i in range(cnt)], [int(rows[i]) for i in range(cnt + 1)]
