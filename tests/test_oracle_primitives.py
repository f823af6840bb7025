"""Pins of the oracle's primitives against library routines, closed forms and
invariants (CPU only).

Each check is chosen so that a plausible slip in oracle.c fails it: a wrong
rounding rule, a swapped RoPE half, a wrong GQA or scale, a mask applied by
adding -inf to a NaN score, a transposed weight, a wrong Q8 block index.
"""
import ctypes as C
import math

import numpy as np
import pytest
import torch

from autoregressive_codebook_tts_frame_amd import synth
from oracle.oracle import load_library, model_struct

lib = load_library()


def _p(a):
    return a.ctypes.data


def _model(**kw):
    return synth.scaled_model(synth.TINY, **kw)


# --------------------------------------------------------------- formats


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000),
        # exact ties: low 16 bits = 0x8000 with both parities of bit 16
        (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38], np.float32),
    ]).astype(np.float32)
    ours = np.array([lib.orc_bf16_round(float(v)) for v in x], np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_bf16_round_matches_input_generator():
    # the input generator stores weights with its own conversion; both must agree
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(5000) * 0.02).astype(np.float32)
    ours = np.array([lib.orc_bf16_round(float(v)) for v in x], np.float32)
    gen = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    assert np.array_equal(ours, gen)


def test_f16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    ours = np.array([lib.orc_f16_to_f32(int(b)) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# --------------------------------------------------------------- RMSNorm


def _rms(m, x, g):
    y = np.empty_like(x)
    ms = model_struct(m)
    lib.orc_prim_rmsnorm(C.byref(ms), _p(x), _p(g), x.shape[0], _p(y))
    return y


def test_rmsnorm_vs_torch_library():
    m = _model()
    rng = np.random.default_rng(2)
    for n in (64, 256, 1024):
        x = rng.standard_normal(n).astype(np.float32) * 3
        g = (1 + 0.02 * rng.standard_normal(n)).astype(np.float32)
        y = _rms(m, x, g)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x).double(), (n,),
                                           torch.from_numpy(g).double(), eps=m.eps).numpy()
        np.testing.assert_allclose(y, ref, rtol=2e-7, atol=0)


def test_rmsnorm_closed_form_unit_gain():
    # with g = 1: mean(y^2) = 1 / (1 + eps / mean(x^2))
    m = _model(eps=1e-2)
    x = (np.arange(64, dtype=np.float32) - 31.5) / 40.0
    y = _rms(m, x, np.ones(64, np.float32)).astype(np.float64)
    msx = float(np.mean(x.astype(np.float64) ** 2))
    assert math.isclose(float(np.mean(y ** 2)), 1.0 / (1.0 + 1e-2 / msx), rel_tol=1e-6)


def test_rmsnorm_bf16_gains_are_read_as_bf16():
    m = _model(tab_bf16=True)
    x = np.ones(64, np.float32)
    g = synth.f32_to_bf16_bits(np.full(64, 2.0, np.float32))
    y = _rms(m, x, g)
    np.testing.assert_allclose(y, 2.0 / np.sqrt(1 + m.eps), rtol=1e-7)


# --------------------------------------------------------------- RoPE


def _rope(m, v, p):
    v = np.array(v, np.float32, copy=True)
    lib.orc_prim_rope(C.byref(model_struct(m)), _p(v), p)
    return v


def test_rope_position_zero_is_identity():
    m = _model()
    v = np.random.default_rng(3).standard_normal(m.hd).astype(np.float32)
    assert np.array_equal(_rope(m, v, 0), v)


def test_rope_matches_hf_rotary():
    from transformers.models.qwen3.modeling_qwen3 import apply_rotary_pos_emb
    m = _model()
    hd = m.hd
    rng = np.random.default_rng(4)
    for p in (1, 7, 100, 255):
        v = rng.standard_normal(hd).astype(np.float32)
        inv = 1.0 / (m.theta ** (np.arange(0, hd, 2, dtype=np.float64) / hd))
        ang = p * inv
        emb = np.concatenate([ang, ang])
        cos = torch.tensor(np.cos(emb))[None, None]
        sin = torch.tensor(np.sin(emb))[None, None]
        t = torch.tensor(v, dtype=torch.float64)[None, None, None]
        ref, _ = apply_rotary_pos_emb(t, t, cos, sin)
        np.testing.assert_allclose(_rope(m, v, p), ref.numpy().ravel(), rtol=0, atol=3e-6)


def test_rope_preserves_pair_norms_and_relative_position():
    m = _model()
    rng = np.random.default_rng(5)
    q = rng.standard_normal(m.hd).astype(np.float32)
    k = rng.standard_normal(m.hd).astype(np.float32)
    h = m.hd // 2
    for p in (3, 50):
        r = _rope(m, q, p).astype(np.float64)
        n0 = q[:h].astype(np.float64) ** 2 + q[h:].astype(np.float64) ** 2
        np.testing.assert_allclose(r[:h] ** 2 + r[h:] ** 2, n0, rtol=1e-6)
    d1 = float(np.dot(_rope(m, q, 20).astype(np.float64), _rope(m, k, 5)))
    d2 = float(np.dot(_rope(m, q, 40).astype(np.float64), _rope(m, k, 25)))
    assert math.isclose(d1, d2, rel_tol=1e-5, abs_tol=1e-5)


# --------------------------------------------------------------- attention


def _attend(m, q, kc, vc, kh, p, W):
    o = np.empty(m.hd, np.float32)
    lib.orc_prim_attend(C.byref(model_struct(m)), _p(q), _p(kc), _p(vc), kh, p, W, _p(o))
    return o


def test_attention_vs_torch_sdpa():
    m = _model()
    rng = np.random.default_rng(6)
    W = 32
    kc = rng.standard_normal((W, m.nkv, m.hd)).astype(np.float32)
    vc = rng.standard_normal((W, m.nkv, m.hd)).astype(np.float32)
    for kh in range(m.nkv):
        for p in (0, 5, 31):
            q = rng.standard_normal(m.hd).astype(np.float32)
            o = _attend(m, q, kc, vc, kh, p, W)
            K = torch.tensor(kc[: p + 1, kh], dtype=torch.float64)[None, None]
            V = torch.tensor(vc[: p + 1, kh], dtype=torch.float64)[None, None]
            Qt = torch.tensor(q, dtype=torch.float64)[None, None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(Qt, K, V).numpy().ravel()
            np.testing.assert_allclose(o, ref, rtol=1e-6, atol=1e-7)


def test_attention_padded_equals_unpadded_and_ignores_poison():
    m = _model()
    rng = np.random.default_rng(7)
    P = 512
    kc = rng.standard_normal((P, m.nkv, m.hd)).astype(np.float32)
    vc = rng.standard_normal((P, m.nkv, m.hd)).astype(np.float32)
    q = rng.standard_normal(m.hd).astype(np.float32)
    p = 200
    base = _attend(m, q, kc, vc, 1, p, p + 1)
    kp, vp = kc.copy(), vc.copy()
    kp[p + 1:] = np.nan
    vp[p + 1:] = np.inf
    for W in (256, 512):
        assert lib.orc_prim_talker_window(p) == 256
        o = _attend(m, q, kp, vp, 1, p, W)
        assert np.array_equal(o.view(np.uint32), base.view(np.uint32))


def test_attention_constant_values_and_single_key():
    m = _model()
    rng = np.random.default_rng(8)
    kc = rng.standard_normal((16, m.nkv, m.hd)).astype(np.float32)
    vc = np.full((16, m.nkv, m.hd), 0.75, np.float32)
    q = rng.standard_normal(m.hd).astype(np.float32)
    np.testing.assert_allclose(_attend(m, q, kc, vc, 0, 9, 16), 0.75, rtol=1e-7)
    vc2 = rng.standard_normal((16, m.nkv, m.hd)).astype(np.float32)
    assert np.array_equal(_attend(m, q, kc, vc2, 1, 0, 16), vc2[0, 1])


def test_talker_window_closed_form():
    for p, w in ((0, 256), (254, 256), (255, 256), (256, 512), (2047, 2048), (2048, 2304), (4095, 4096)):
        assert lib.orc_prim_talker_window(p) == w


# --------------------------------------------------------------- matmul / argmax


def _mm(m, w, d, N, K, x):
    R = x.shape[0]
    out = np.empty((R, N), np.float32)
    lib.orc_prim_mm(C.byref(model_struct(m)), _p(w), None if d is None else _p(d), N, K, R,
                    _p(x), _p(out))
    return out


def test_mm_f32_vs_numpy():
    m = _model()
    rng = np.random.default_rng(9)
    w = rng.standard_normal((48, 96)).astype(np.float32)
    x = rng.standard_normal((3, 96)).astype(np.float32)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    # both are the exact-ish double sum rounded once to float32
    np.testing.assert_allclose(_mm(m, w, None, 48, 96, x), ref, rtol=1.2e-7, atol=1e-12)
    # non-square: rows index outputs, columns the input (a transposed operand fails)
    assert _mm(m, w, None, 48, 96, x).shape == (3, 48)


def test_mm_bf16_rounds_activation_operand():
    m = _model(lin=synth.LIN_BF16, act_bf16=True)
    x = np.array([[1.0 + 2.0 ** -10]], np.float32)          # rounds to 1.0 in bf16
    w = synth.f32_to_bf16_bits(np.array([[3.0]], np.float32))
    assert _mm(m, w, None, 1, 1, x)[0, 0] == 3.0
    m2 = _model(lin=synth.LIN_BF16, act_bf16=False)
    assert _mm(m2, w, None, 1, 1, x)[0, 0] == np.float32(3.0 * (1.0 + 2.0 ** -10))


def test_mm_q8_block_scales_closed_form():
    m = _model(lin=synth.LIN_Q8, act_bf16=False)
    N, K = 3, 96
    rng = np.random.default_rng(10)
    q = rng.integers(-127, 128, (N, K)).astype(np.int8)
    d = (rng.uniform(0.5, 1.5, (N, K // 32)) * 1e-3).astype(np.float16)
    for k in (0, 31, 32, 63, 95):
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        out = _mm(m, q, d.view(np.uint16), N, K, x)[0]
        ref = d[:, k // 32].astype(np.float32) * q[:, k].astype(np.float32)
        assert np.array_equal(out, ref)


def test_mm_q4_codes_closed_form():
    """4-bit blocks: code c of weight k sits in byte k/2 (low nibble for even
    k) and stands for d * (c - 8); a swapped nibble, a wrong block or a missing
    offset fails one of the one-hot columns."""
    m = _model(lin=synth.LIN_Q4, act_bf16=False)
    N, K = 3, 96
    rng = np.random.default_rng(12)
    c = rng.integers(0, 16, (N, K)).astype(np.uint8)
    c[0, :2] = (0, 15)  # the two extremes next to each other
    packed = np.zeros((N, K // 2), np.uint8)
    for n in range(N):
        for k in range(K):
            packed[n, k // 2] |= c[n, k] << (4 * (k % 2))
    d = (rng.uniform(0.5, 1.5, (N, K // 32)) * 1e-3).astype(np.float16)
    for k in (0, 1, 2, 31, 32, 33, 63, 95):
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        out = _mm(m, packed, d.view(np.uint16), N, K, x)[0]
        ref = d[:, k // 32].astype(np.float32) * (c[:, k].astype(np.float32) - 8)
        assert np.array_equal(out, ref), k
    assert _mm(m, packed, d.view(np.uint16), N, K, np.eye(1, K, 0, np.float32))[0, 0] == -8 * np.float32(d[0, 0])


def test_argmax_lowest_index_on_ties():
    x = np.array([1.0, 5.0, 2.0, 5.0, 5.0], np.float32)
    assert lib.orc_prim_argmax(_p(x), 5) == 1 == int(np.argmax(x))
    rng = np.random.default_rng(11)
    for _ in range(50):
        y = rng.integers(0, 4, 300).astype(np.float32)
        assert lib.orc_prim_argmax(_p(y), 300) == int(np.argmax(y))
