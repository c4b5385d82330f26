"""C-ABI contract on the host (no GPU needed): the library loads, exports
every function include/spec_verify.h declares, and its host-side checks
reject bad configurations, bad tensor lists and NULL handles without
touching a device."""
import ctypes
import os
import re

import numpy as np
import pytest

from target_model_verification_amd import binding as b
from target_model_verification_amd import synth

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "spec_verify.h")


def declared_functions():
    txt = open(HDR).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(b.lib, n), n
        assert getattr(b, n) is not None


def _check(cfg):
    msg = ctypes.create_string_buffer(256)
    return b.spec_config_check(ctypes.byref(cfg), msg, 256), msg.value.decode()


@pytest.mark.parametrize("name", list(synth.ALL_WORKLOADS))
def test_workload_configs_are_valid(name):
    wl = synth.ALL_WORKLOADS[name]
    rc, msg = _check(b.make_config(wl.spec, wl.context + 300, max(wl.k_sweep)))
    assert rc == b.SPEC_OK, msg


@pytest.mark.parametrize("field,value,needle", [
    ("max_k", 16, "max_k"),
    ("max_k", -1, "max_k"),
    ("head_dim", 96, "head_dim"),
    ("n_kv_heads", 3, "multiple"),
    ("vocab", 1, "vocab"),
    ("gemm_k_split", 100, "gemm_k_split"),
    ("gemm_k_split", 4096, "gemm_k_split"),
    ("kv_dtype", 2, "kv_dtype"),
    ("max_ctx", 0, "max_ctx"),
    ("rope_theta", 0.0, "rope_theta"),
])
def test_bad_configs_rejected(field, value, needle):
    cfg = b.make_config(synth.LLAMA7B, 2048, 15)
    setattr(cfg, field, value)
    rc, msg = _check(cfg)
    assert rc == b.SPEC_EINVAL and needle in msg


def test_int4_alignment_and_attention_capacity_rules():
    cfg = b.make_config(synth.SMALL_WORKLOADS["small_bf16"].spec, 512, 8)
    cfg.weight_dtype = b.SPEC_DT_INT4G128                 # d_ff = 1400 not divisible by 128
    assert _check(cfg)[0] == b.SPEC_EINVAL
    cfg = b.make_config(synth.QWEN7B, 8192, 15)
    cfg.n_kv_heads = 1                                    # 16 rows x 28 heads: too many query rows
    rc, msg = _check(cfg)
    assert rc == b.SPEC_EINVAL and "attention" in msg
    cfg = b.make_config(synth.LLAMA7B, 2048, 8)
    cfg.reserved[3] = 1
    assert _check(cfg)[0] == b.SPEC_EINVAL


def test_null_handle_calls():
    res = b.SpecStepResult()
    toks = (ctypes.c_int32 * 2)(1, 2)
    assert b.spec_verify_step(None, toks, 1, 0, None, None, ctypes.byref(res), None) == b.SPEC_EINVAL
    assert b.spec_kv_commit_rollback(None, 0) == b.SPEC_EINVAL
    assert b.spec_kv_len(None) == -1
    assert b.spec_last_error(None) == b"null handle"
    assert b.spec_profile_enable(None, 1) == b.SPEC_EINVAL
    assert b.spec_pass_bytes(None, 0, 0, 0, 0) < 0
    b.spec_verify_destroy(None)                            # allowed


def _tiny_tensors():
    wl = synth.WORKLOADS["tiny"]
    W = synth.make_weights(wl.spec, wl.seed)
    return wl, W


def _create(cfg, W):
    t, keep = b.make_tensors(W)
    h = ctypes.c_void_p()
    rc = b.spec_verify_create(ctypes.byref(cfg), t, len(t), None, None, 0, None, ctypes.byref(h))
    return rc, h


def test_tensor_list_errors_are_caught_on_the_host():
    wl, W = _tiny_tensors()
    cfg = b.make_config(wl.spec, 256, 4)
    W2 = dict(W)
    del W2["l1.wv"]
    assert _create(cfg, W2)[0] == b.SPEC_EINVAL                     # missing
    W3 = dict(W)
    W3["l0.wo"] = W["l0.wo"][:-1]
    assert _create(cfg, W3)[0] == b.SPEC_EINVAL                     # wrong size
    W4 = dict(W)
    W4["l0.x0.w_gate"] = W["l0.w_gate"]
    assert _create(cfg, W4)[0] == b.SPEC_EINVAL                     # extra tensor
    cfg.n_layers = 3
    assert _create(cfg, W)[0] == b.SPEC_EINVAL                      # layer 2 missing
    # prompt longer than the cache
    cfg = b.make_config(wl.spec, 16, 4)
    t, keep = b.make_tensors(W)
    h = ctypes.c_void_p()
    k = np.zeros(10, np.float32)
    assert b.spec_verify_create(ctypes.byref(cfg), t, len(t), k.ctypes.data, k.ctypes.data, 17, None,
                                ctypes.byref(h)) == b.SPEC_ECAPACITY


def test_create_without_gpu_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    wl, W = _tiny_tensors()
    rc, h = _create(b.make_config(wl.spec, 256, 4), W)
    assert rc == b.SPEC_EHIP and not h.value
