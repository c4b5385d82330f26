"""Pins for the oracle's elementwise definitions against library routines,
closed forms and textbook identities (CPU only)."""
import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from oracle import numerics as nx
from target_model_verification_amd import synth


def test_bf16_bits_known_values():
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x0000, 0x8000, 0x3C00], np.uint16)
    vals = nx.bf16_bits_to_float(bits)
    assert vals.tolist() == [1.0, -2.0, 3.140625, 0.0, -0.0, 2.0 ** -7]


def test_round_to_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(3.0)
    # exact ties: 1 + 2^-8 -> 1 (even), 1 + 3*2^-8 -> 1 + 2^-6 (even)
    x = np.concatenate([x, np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 255.5, 256.5], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = nx.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)
    assert got[-5] == 1.0 and got[-4] == 1 + 2 ** -6


def test_round_to_bf16_from_float64_single_rounding():
    # a float64 value just above a bf16 tie must round up (no double rounding)
    x = np.array([1 + 2 ** -8 + 2 ** -40])
    assert nx.round_to_bf16(x)[0] == 1 + 2 ** -7


def test_round_kv_f32():
    x = np.array([1 / 3.0])
    assert nx.round_kv(x, "f32")[0] == float(np.float32(1 / 3.0))


def test_dequant_int4_nibbles_and_exactness():
    # byte 0x8F: low nibble 0xF = -1 (even k), high nibble 0x8 = -8 (odd k)
    packed = np.array([[0x8F, 0x71]], np.uint8)          # K=2, N=2
    s = np.array([[0.5, 0.25]], np.float16)
    w = nx.dequant_int4(packed, s, group=2)
    assert w.tolist() == [[-0.5, 0.25], [-4.0, 1.75]]
    # generator round trip: q*s exact in fp32, |w - q*s| <= s/2 unless clipped
    rng = np.random.default_rng(1)
    w0 = (rng.standard_normal((256, 40)) * 0.02).astype(np.float32)
    q, sc = synth.quantize_int4_g128(w0)
    wq = nx.dequant_int4(q, sc, 128)
    assert np.array_equal(wq.astype(np.float32).astype(np.float64), wq)
    srep = np.repeat(sc.astype(np.float64), 128, axis=0)
    assert np.all(np.abs(w0 - wq) <= srep / 2 * (1 + 1e-6) + 1e-12)
    assert np.array_equal(synth.unpack_int4(q).astype(np.float64) * srep, wq)


def test_rmsnorm_matches_torch_and_closed_form():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 96))
    g = rng.standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(x), (96,), weight=torch.from_numpy(g), eps=1e-5).numpy()
    assert np.allclose(nx.rmsnorm(x, g, 1e-5), ref, rtol=1e-13, atol=1e-13)
    c = np.full((1, 8), -3.0)
    assert np.allclose(nx.rmsnorm(c, np.ones(8), 0.0), -1.0)


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(3)
    D, m, H = 64, 7, 3
    x = rng.standard_normal((m, H, D))
    pos = np.array([0, 1, 5, 17, 100, 1023, 4095])
    got = nx.rope(x, pos, 10000.0)
    z = x[..., :D // 2] + 1j * x[..., D // 2:]
    ang = pos[:, None] * (10000.0 ** (-np.arange(D // 2) * 2.0 / D))[None, :]
    z = z * np.exp(1j * ang)[:, None, :]
    ref = np.concatenate([z.real, z.imag], axis=-1)
    assert np.allclose(got, ref, atol=1e-12)
    assert np.allclose(got[0], x[0])                      # position 0: identity
    assert np.allclose(np.linalg.norm(got, axis=-1), np.linalg.norm(x, axis=-1))


def test_rope_relative_position():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    dots = []
    for a, b in [(10, 3), (107, 100), (4000, 3993)]:
        dots.append(float(np.sum(nx.rope(q, np.array([a]), 1e4) * nx.rope(k, np.array([b]), 1e4))))
    assert np.allclose(dots, dots[0], atol=1e-9)


def test_softmax_and_silu_match_libraries():
    rng = np.random.default_rng(5)
    z = rng.standard_normal((4, 50)) * 10
    assert np.allclose(nx.softmax(z), scipy.special.softmax(z, axis=-1), rtol=1e-14, atol=1e-16)
    x = rng.standard_normal(1000) * 5
    assert np.allclose(nx.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 1), (6, 2), (7, 1)])
def test_causal_attention_matches_torch_sdpa(Hq, Hkv):
    rng = np.random.default_rng(6)
    m, L, D = 5, 23, 32
    T = L + m
    q = rng.standard_normal((m, Hq, D))
    K = rng.standard_normal((Hkv, T + 9, D))       # extra dead rows must be ignored
    V = rng.standard_normal((Hkv, T + 9, D))
    got = nx.causal_attention(q, K, V, L)
    G = Hq // Hkv
    Kt = torch.from_numpy(K[:, :T]).repeat_interleave(G, dim=0)       # [Hq, T, D]
    Vt = torch.from_numpy(V[:, :T]).repeat_interleave(G, dim=0)
    qt = torch.from_numpy(q).permute(1, 0, 2)                          # [Hq, m, D]
    mask = torch.arange(T)[None, :] <= (L + torch.arange(m))[:, None]
    ref = F.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask).permute(1, 0, 2).numpy()
    assert np.allclose(got, ref, atol=1e-12)
    # NaN in dead rows must not leak
    K2, V2 = K.copy(), V.copy()
    K2[:, T:] = np.nan
    V2[:, T:] = np.nan
    assert np.array_equal(nx.causal_attention(q, K2, V2, L), got)
