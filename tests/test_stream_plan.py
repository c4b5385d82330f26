"""Host replay of the weight-streaming work split (no GPU needed).

spec_plan_check rebuilds the plan a verifier would use on a grid of n_wg
workgroups and walks every workgroup's share of every weight matrix, as the
device code does, checking each weight fragment, A-window, split-K
workspace, ticket and pending index against the sizes the library would
allocate, plus the split-K invariants (segment counts agree between
workgroups, segment indices run 0..n-1 in K order and cover K once).

Grid sizes cover fewer workgroups than units (sparse split), one workgroup,
odd counts and the MI355X compute-unit count (256); window sizes cover the
default and a short window (more windows per matrix, third-window restaging).
"""
import ctypes
import dataclasses

import pytest

from target_model_verification_amd import binding as b
from target_model_verification_amd import synth

GRIDS = (1, 3, 64, 255, 256, 304, 1000)


def _ok(rc, msg, g):
    """A grid smaller than the MI355X compute-unit count may be too small for
    the per-workgroup list of split segments; it must then be refused cleanly
    at planning time.  Anything else must plan and walk clean."""
    if rc == b.SPEC_OK:
        return True
    return g < 256 and "split-K bookkeeping" in msg


def _plan(spec, n_wg, max_k=15, k_split=0, max_ctx=4096):
    cfg = b.make_config(spec, max_ctx, max_k, k_split)
    msg = ctypes.create_string_buffer(512)
    rc = b.spec_plan_check(ctypes.byref(cfg), n_wg, msg, 512)
    return rc, msg.value.decode()


@pytest.mark.parametrize("name", list(synth.ALL_WORKLOADS))
@pytest.mark.parametrize("k_split", (0, 256, 1024))
def test_plan_walk_in_bounds(name, k_split):
    spec = synth.ALL_WORKLOADS[name].spec
    for g in GRIDS:
        rc, msg = _plan(spec, g, k_split=k_split)
        assert _ok(rc, msg, g), f"{name} n_wg={g} k_split={k_split}: {msg}"
        if g == 256:
            assert rc == b.SPEC_OK, msg


@pytest.mark.parametrize("d,ff,V", [(16, 16, 2), (48, 40, 17), (160, 33, 1000), (4096, 11008, 32000)])
def test_plan_ragged_shapes(d, ff, V):
    """Column counts and K extents that leave partial tiles, supergroups and
    windows."""
    spec = synth._dense("ragged", 1, d, 1, 1, 64, ff, V, "bf16", "bf16")
    for g in GRIDS:
        for ks in (0, 128, 384):
            rc, msg = _plan(spec, g, k_split=ks)
            assert _ok(rc, msg, g), f"d={d} ff={ff} V={V} n_wg={g} k_split={ks}: {msg}"


def test_plan_moe_small_expert_counts():
    base = synth.SMALL_WORKLOADS["small_moe"].spec
    for E, top_k, S in ((2, 1, 0), (5, 2, 2), (16, 6, 1), (40, 8, 3)):
        spec = dataclasses.replace(base, n_experts=E, top_k=top_k, n_shared=S)
        for g in (1, 7, 256):
            rc, msg = _plan(spec, g)
            assert _ok(rc, msg, g), f"E={E} top_k={top_k} S={S} n_wg={g}: {msg}"


def test_plan_rejects_bad_grid():
    rc, msg = _plan(synth.TINY, 0)
    assert rc == b.SPEC_EINVAL and "n_wg" in msg


def test_floor_div_in_double_matches_integer_division():
    """The device computes range_begin / wg_of quotients as floor(p / q) in
    double precision; over the ranges the plan allows (p < 2^52, q < 2^31)
    that equals the integer quotient, including just below and at exact
    multiples."""
    import random

    rng = random.Random(7)
    cases = []
    for _ in range(20000):
        q = rng.randrange(1, 1 << 31)
        k = rng.randrange(0, (1 << 52) // q)
        for p in (k * q - 1, k * q, k * q + 1, k * q + q - 1):
            if 0 <= p < (1 << 52):
                cases.append((p, q))
    for G in (1, 3, 255, 256, 304, 1000, 4096):
        for total in (1, 7, 1 << 20, (1 << 31) - 1):
            for g in range(0, G + 1, max(1, G // 17)):
                cases.append((total * g, G))
    for p, q in cases:
        assert int(float(p) / float(q) // 1) == p // q, (p, q)
