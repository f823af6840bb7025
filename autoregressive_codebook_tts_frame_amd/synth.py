"""Seeded synthetic inputs for the per-frame codebook TTS decode.

This module only *draws* inputs: model shapes, weights, prompts, overlay ids
and synthetic decode states.  It holds none of the method's arithmetic (no
norm, projection, attention or sampling) and is the one piece shared by the
HIP path's harness and the CPU oracle's tests.  Storage conversions of the
drawn numbers (float32 -> bfloat16 round-to-nearest-even, float -> fp16 block
scales) happen here because the drawn tensors *are* stored in those formats.

Shapes follow the five workloads of the decode step: a tiny F32 model, the
28-layer BF16 model at batch 1, the same model at long context, at 32 ragged
streams, and with Q8_0-style or 4-bit block-quantised linear weights.  The talker /
code-predictor split, the 16 codebooks and the one text-or-pad overlay row
per frame are those of the qwentts.cpp pipeline-tts.h commit log (entries on
assembling the AR inputs on device and on the per-layer K/V ring).

Seeds derive from 42 (the seed of the F32 reference run named in the K/V ring
entry of that log): every tensor draws from
``numpy.random.default_rng([42, model_id, tensor_id])`` and every run input
from ``default_rng([42, cfg_id, 1000 + purpose])``.
"""
from __future__ import annotations

import dataclasses
import functools
from typing import Dict, List, Optional, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# storage formats

LIN_F32, LIN_BF16, LIN_Q8, LIN_Q4 = 0, 1, 2, 3
Q8_BLOCK = 32


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern (uint16), round to nearest even.

    NaN is not expected in drawn data; it is kept quiet if present."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit pattern -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# model and run descriptions


@dataclasses.dataclass(frozen=True)
class Model:
    """Shapes and storage formats of one talker + code-predictor model."""

    name: str
    model_id: int          # seeds the weights; models that are "the same" share it
    H: int                 # hidden width (talker and predictor)
    nq: int                # query heads
    nkv: int               # key/value heads
    hd: int                # head dim
    F: int                 # FFN width (SiLU-multiply)
    Lt: int                # talker layers
    Lp: int                # code-predictor layers
    G: int                 # codebooks per frame
    Vc: int                # entries per codebook (= logit width of every head)
    Vt: int                # rows of the text / pad overlay table
    P: int                 # talker K/V ring positions
    Q: int                 # code-predictor cache positions (reset every frame)
    lin: int               # LIN_F32 / LIN_BF16 / LIN_Q8 for linear weights
    tab_bf16: bool         # tables and norm gains stored as bf16
    kv_bf16: bool          # K/V ring stored as bf16
    act_bf16: bool         # matmul activation operands rounded to bf16
    eps: float = 1e-6
    theta: float = 1e6

    @property
    def nqkv(self) -> int:
        return (self.nq + 2 * self.nkv) * self.hd


@dataclasses.dataclass(frozen=True)
class Workload:
    """One run of the decode step on a model."""

    cfg_id: int
    name: str
    model: Model
    batch: int
    prompt: int             # prompt rows per stream (prefill length)
    frames: int             # frames decoded
    frames_per_replay: int  # K frames per graph replay
    ragged: Optional[Tuple[int, int]] = None  # per-stream context lengths U{lo..hi}


TINY = Model("tiny_f32", 0, H=256, nq=4, nkv=2, hd=64, F=768, Lt=2, Lp=1, G=16,
             Vc=256, Vt=512, P=256, Q=16, lin=LIN_F32, tab_bf16=False,
             kv_bf16=False, act_bf16=False)
BIG = Model("bf16_28L", 1, H=1024, nq=16, nkv=8, hd=128, F=3072, Lt=28, Lp=5,
            G=16, Vc=2048, Vt=151936, P=4096, Q=16, lin=LIN_BF16,
            tab_bf16=True, kv_bf16=True, act_bf16=True)
BIG_Q8 = dataclasses.replace(BIG, name="q8_28L", model_id=4, lin=LIN_Q8)
BIG_Q4 = dataclasses.replace(BIG, name="q4_28L", model_id=5, lin=LIN_Q4)

WORKLOADS: Dict[str, Workload] = {
    "tiny_f32_b1": Workload(0, "tiny_f32_b1", TINY, batch=1, prompt=16, frames=8,
                            frames_per_replay=1),
    "bf16_b1": Workload(1, "bf16_b1", BIG, batch=1, prompt=128, frames=64,
                        frames_per_replay=1),
    "bf16_long_b1": Workload(2, "bf16_long_b1", BIG, batch=1, prompt=2048, frames=32,
                             frames_per_replay=1),
    "bf16_b32": Workload(3, "bf16_b32", BIG, batch=32, prompt=0, frames=64,
                         frames_per_replay=4, ragged=(64, 2048)),
    "q8_b1": Workload(4, "q8_b1", BIG_Q8, batch=1, prompt=128, frames=64,
                      frames_per_replay=1),
    "q8_b8": Workload(4, "q8_b8", BIG_Q8, batch=8, prompt=128, frames=64,
                      frames_per_replay=1),
    "q4_b1": Workload(5, "q4_b1", BIG_Q4, batch=1, prompt=128, frames=64,
                      frames_per_replay=1),
    "q4_b8": Workload(5, "q4_b8", BIG_Q4, batch=8, prompt=128, frames=64,
                      frames_per_replay=1),
}


def scaled_model(m: Model, **kw) -> Model:
    """A model with some shapes changed (reduced parity cases)."""
    return dataclasses.replace(m, **kw)


# ---------------------------------------------------------------------------
# weights

LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo",
              "mlp_norm", "wg", "wu", "wd")
NORM_KEYS = ("attn_norm", "q_norm", "k_norm", "mlp_norm")


def _layer_shapes(m: Model) -> Dict[str, Tuple[int, ...]]:
    return {
        "attn_norm": (m.H,), "wq": (m.nq * m.hd, m.H), "wk": (m.nkv * m.hd, m.H),
        "wv": (m.nkv * m.hd, m.H), "q_norm": (m.hd,), "k_norm": (m.hd,),
        "wo": (m.H, m.nq * m.hd), "mlp_norm": (m.H,), "wg": (m.F, m.H),
        "wu": (m.F, m.H), "wd": (m.H, m.F),
    }


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([42, *key])


def _normal(rng: np.random.Generator, shape, std: float, mean: float = 0.0) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    if mean:
        a += np.float32(mean)
    return a


def _store_table(m: Model, a: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(a) if m.tab_bf16 else a


def _store_linear(m: Model, rng: np.random.Generator, shape, random_scales: bool):
    if m.lin == LIN_F32:
        return _normal(rng, shape, 0.02)
    if m.lin == LIN_BF16:
        return f32_to_bf16_bits(_normal(rng, shape, 0.02))
    n, k = shape
    assert k % Q8_BLOCK == 0
    if m.lin == LIN_Q4:
        # 4-bit blocks: codes 0..15 (value c - 8), two per byte, even index in
        # the low nibble; one fp16 scale per 32 weights along the input dim
        c = rng.integers(0, 16, size=shape, dtype=np.uint8)
        packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
        if random_scales:
            d = (rng.uniform(0.5, 1.5, size=(n, k // Q8_BLOCK)) * (0.02 / 8.0)).astype(np.float16)
        else:
            d = np.full((n, k // Q8_BLOCK), 0.02 / 8.0, dtype=np.float16)
        return (packed, d.view(np.uint16))
    # Q8_0-style: 32 int8 values per block along the input dim + one fp16 scale
    q = rng.integers(-127, 128, size=shape, dtype=np.int8)
    if random_scales:
        s = rng.uniform(0.5, 1.5, size=(n, k // Q8_BLOCK)) * (0.02 / 127.0)
        d = s.astype(np.float16)
    else:
        d = np.full((n, k // Q8_BLOCK), 0.02 / 127.0, dtype=np.float16)
    return (q, d.view(np.uint16))


@functools.lru_cache(maxsize=4)
def make_weights(m: Model, random_q8_scales: bool = False, literal_gains: bool = False):
    """All weights of model ``m`` as host arrays.

    Matrices and tables ~ N(0, 0.02).  Norm gains are 1 + N(0, 0.02) unless
    ``literal_gains`` (then N(0, 0.02) as printed).  Returns a dict with
    code_emb [G][Vc][H], text_emb [Vt][H], t_norm [H], t_head [Vc][H],
    p_norm [H], p_heads (G-1 x [Vc][H]), talker / predictor: lists of per-layer
    dicts keyed by LAYER_KEYS.  Linear weights are float32, bf16 bits (uint16)
    or a (int8 [N][K], fp16-bits uint16 [N][K/32]) pair (q4: uint8 [N][K/2]
    of packed 4-bit codes instead of the int8 values).
    """
    tid = iter(range(1 << 30))

    def gain(shape):
        r = _rng(m.model_id, next(tid))
        a = _normal(r, shape, 0.02, 0.0 if literal_gains else 1.0)
        return _store_table(m, a)

    def table(shape):
        return _store_table(m, _normal(_rng(m.model_id, next(tid)), shape, 0.02))

    def linear(shape):
        return _store_linear(m, _rng(m.model_id, next(tid)), shape, random_q8_scales)

    w = {}
    w["code_emb"] = table((m.G, m.Vc, m.H))
    w["text_emb"] = table((m.Vt, m.H))
    w["t_norm"] = gain((m.H,))
    w["t_head"] = linear((m.Vc, m.H))
    w["p_norm"] = gain((m.H,))
    w["p_heads"] = [linear((m.Vc, m.H)) for _ in range(m.G - 1)]
    shapes = _layer_shapes(m)
    for stack, nl in (("talker", m.Lt), ("predictor", m.Lp)):
        layers = []
        for _ in range(nl):
            d = {}
            for k in LAYER_KEYS:
                d[k] = gain(shapes[k]) if k in NORM_KEYS else linear(shapes[k])
            layers.append(d)
        w[stack] = layers
    return w


# ---------------------------------------------------------------------------
# run inputs


def make_prompt(wl: Workload, stream: int, T: Optional[int] = None, purpose: int = 0):
    """Prompt rows for one stream: codes [T][G] uniform in [0, Vc) and text
    ids [T] uniform in [0, Vt) (an ICL codec-plus-text prompt)."""
    m = wl.model
    T = wl.prompt if T is None else T
    r = _rng(wl.cfg_id, 1000 + purpose, stream)
    codes = r.integers(0, m.Vc, size=(T, m.G), dtype=np.int32)
    text = r.integers(0, m.Vt, size=(T,), dtype=np.int32)
    return codes, text


def make_overlays(wl: Workload, n_frames: int, batch: Optional[int] = None, purpose: int = 1):
    """Overlay ids [n][B]: a seeded text id for the first half of the frames,
    then the pad id Vt-1 (the trailing text-or-pad overlay)."""
    m = wl.model
    B = wl.batch if batch is None else batch
    r = _rng(wl.cfg_id, 1000 + purpose)
    ov = r.integers(0, m.Vt - 1, size=(n_frames, B), dtype=np.int32)
    ov[n_frames // 2:, :] = m.Vt - 1
    return ov


def make_context_lengths(wl: Workload, batch: Optional[int] = None, purpose: int = 2):
    """Per-stream context lengths (valid ring positions before decoding)."""
    B = wl.batch if batch is None else batch
    if wl.ragged is None:
        return np.full((B,), wl.prompt, dtype=np.int32)
    lo, hi = wl.ragged
    r = _rng(wl.cfg_id, 1000 + purpose)
    return r.integers(lo, hi + 1, size=(B,), dtype=np.int32)


def make_forced_codes(wl: Workload, n_frames: int, batch: Optional[int] = None, purpose: int = 3):
    m = wl.model
    B = wl.batch if batch is None else batch
    r = _rng(wl.cfg_id, 1000 + purpose)
    return r.integers(0, m.Vc, size=(n_frames, B, m.G), dtype=np.int32)


def make_synthetic_state(wl: Workload, stream: int, length: int, purpose: int = 4):
    """A seeded decode state for one stream, standing in for a prefilled
    context of ``length`` positions: talker keys/values for positions
    [0, length), the bridge (a unit-RMS vector) and the next frame's code 0.

    Keys ~ N(0, 1) (post q/k-norm scale), values ~ N(0, 0.64) (projection
    scale).  Returns k, v as [Lt][nkv][length][hd] in the ring's storage
    format (bf16 bits or float32), bridge float32 [H], c0 int.
    """
    m = wl.model
    r = _rng(wl.cfg_id, 1000 + purpose, stream)
    shape = (m.Lt, m.nkv, length, m.hd)
    k = _normal(r, shape, 1.0)
    v = _normal(r, shape, 0.64)
    bridge = _normal(r, (m.H,), 1.0)
    c0 = int(r.integers(0, m.Vc))
    if m.kv_bf16:
        k, v = f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    return k, v, bridge, c0


def poison_value(m: Model):
    """A NaN in the ring's storage format (for tests that poison unused rows)."""
    return np.uint16(0x7FC1) if m.kv_bf16 else np.float32("nan")
