"""ctypes wrapper of oracle.c (test infrastructure only).

Argument marshalling only: every number the oracle produces is computed in
oracle.c.  The wrapper takes the seeded host arrays drawn by the input
generator and passes their addresses in the oracle's own tensor order.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Strict IEEE evaluation: no contraction into FMA, no fast-math reassociation.
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wno-unknown-pragmas"]


def build_oracle(out: str = _LIB) -> str:
    """Compile oracle.c with gcc into liboracle.so."""
    cmd = ["gcc", *CFLAGS, "-o", out + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class _Model(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ("H", "nq", "nkv", "hd", "F", "Lt", "Lp", "G", "Vc", "Vt", "P", "Q",
                 "lin", "tab_bf16", "kv_bf16", "act_bf16")] + \
               [("eps", C.c_double), ("theta", C.c_double)]


class _Dump(C.Structure):
    _fields_ = [("talker_logits", C.c_void_p), ("pred_logits", C.c_void_p),
                ("bridge", C.c_void_p), ("x0", C.c_void_p), ("gather", C.c_void_p),
                ("tpos", C.c_void_p), ("hidden", C.c_void_p)]


_lib = None


def load_library():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build_oracle()
    lib = C.CDLL(_LIB)
    vp, i32 = C.c_void_p, C.c_int32
    lib.orc_new.restype = vp
    lib.orc_new.argtypes = [C.POINTER(_Model), C.POINTER(vp), i32, i32, i32]
    lib.orc_free.argtypes = [vp]
    lib.orc_num_tensors.argtypes = [C.POINTER(_Model)]
    lib.orc_num_tensors.restype = i32
    lib.orc_prefill.argtypes = [vp, i32, i32, vp, vp, vp, vp]
    lib.orc_prefill.restype = i32
    lib.orc_decode.argtypes = [vp, i32, vp, vp, vp, C.POINTER(_Dump)]
    lib.orc_decode.restype = i32
    lib.orc_get_state.argtypes = [vp, i32, vp, vp, vp]
    lib.orc_get_state.restype = i32
    lib.orc_set_state.argtypes = [vp, i32, i32, i32, vp]
    lib.orc_set_state.restype = i32
    lib.orc_set_cache.argtypes = [vp, i32, i32, i32, i32, vp, vp]
    lib.orc_set_cache.restype = i32
    lib.orc_get_cache.argtypes = [vp, i32, i32, i32, i32, vp, vp]
    lib.orc_get_cache.restype = i32
    lib.orc_poison_predictor.argtypes = [vp, C.c_float]
    lib.orc_bf16_round.argtypes = [C.c_float]
    lib.orc_bf16_round.restype = C.c_float
    lib.orc_f16_to_f32.argtypes = [C.c_uint16]
    lib.orc_f16_to_f32.restype = C.c_float
    lib.orc_prim_rmsnorm.argtypes = [C.POINTER(_Model), vp, vp, i32, vp]
    lib.orc_prim_rope.argtypes = [C.POINTER(_Model), vp, i32]
    lib.orc_prim_attend.argtypes = [C.POINTER(_Model), vp, vp, vp, i32, i32, i32, vp]
    lib.orc_prim_mm.argtypes = [C.POINTER(_Model), vp, vp, i32, i32, i32, vp, vp]
    lib.orc_prim_argmax.argtypes = [vp, i32]
    lib.orc_prim_argmax.restype = i32
    lib.orc_prim_talker_window.argtypes = [i32]
    lib.orc_prim_talker_window.restype = i32
    lib.orc_num_threads.restype = i32
    lib.orc_predictor_recompute.argtypes = [vp, i32, vp, vp]
    lib.orc_predictor_recompute.restype = i32
    lib.orc_set_sampler.argtypes = [vp, C.c_float, i32, C.c_uint64]
    lib.orc_set_sampler.restype = i32
    lib.orc_prim_philox4x64.argtypes = [vp, vp, vp]
    lib.orc_prim_gumbel.argtypes = [C.c_uint64, i32, i32, i32, i32]
    lib.orc_prim_gumbel.restype = C.c_float
    lib.orc_prim_sample.argtypes = [vp, i32, C.c_float, i32, C.c_uint64, i32, i32, i32]
    lib.orc_prim_sample.restype = i32
    _lib = lib
    return lib


def model_struct(m) -> _Model:
    """Oracle model descriptor from a synth.Model."""
    return _Model(m.H, m.nq, m.nkv, m.hd, m.F, m.Lt, m.Lp, m.G, m.Vc, m.Vt, m.P, m.Q,
                  int(m.lin), int(m.tab_bf16), int(m.kv_bf16), int(m.act_bf16),
                  float(m.eps), float(m.theta))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _lin_slots(w):
    if isinstance(w, tuple):
        return [w[0], w[1]]
    return [w, None]


def tensor_list(m, w):
    """The weights dict of synth.make_weights in the oracle's slot order."""
    t = [w["code_emb"], w["text_emb"], w["t_norm"], *_lin_slots(w["t_head"]), w["p_norm"]]
    for h in w["p_heads"]:
        t += _lin_slots(h)
    for stack in ("talker", "predictor"):
        for L in w[stack]:
            t += [L["attn_norm"], *_lin_slots(L["wq"]), *_lin_slots(L["wk"]),
                  *_lin_slots(L["wv"]), L["q_norm"], L["k_norm"], *_lin_slots(L["wo"]),
                  L["mlp_norm"], *_lin_slots(L["wg"]), *_lin_slots(L["wu"]),
                  *_lin_slots(L["wd"])]
    return t


class Oracle:
    """One oracle session: B streams, talker cache holding Pcap positions."""

    def __init__(self, m, weights, batch: int, pcap: Optional[int] = None):
        self.lib = load_library()
        self.m = m
        self.B = batch
        self.pcap = m.P if pcap is None else pcap
        self._ms = model_struct(m)
        self._tensors = tensor_list(m, weights)  # keeps the arrays alive
        n = len(self._tensors)
        assert n == self.lib.orc_num_tensors(C.byref(self._ms))
        self._tab = (C.c_void_p * n)(*[_ptr(a) for a in self._tensors])
        self.h = self.lib.orc_new(C.byref(self._ms), self._tab, n, batch, self.pcap)
        if not self.h:
            raise ValueError("orc_new rejected the model or sizes")

    def close(self):
        if self.h:
            self.lib.orc_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def prefill(self, b: int, codes: Optional[np.ndarray], text: np.ndarray, dump: bool = False):
        m = self.m
        text = np.ascontiguousarray(text, dtype=np.int32)
        T = text.shape[0]
        codes = None if codes is None else np.ascontiguousarray(codes, dtype=np.int32)
        x0 = np.empty((T, m.H), np.float32) if dump else None
        lg = np.empty((m.Vc,), np.float32) if dump else None
        rc = self.lib.orc_prefill(self.h, b, T, _ptr(codes), _ptr(text), _ptr(x0), _ptr(lg))
        if rc != 0:
            raise RuntimeError(f"orc_prefill failed: {rc}")
        return {"x0": x0, "logits": lg} if dump else None

    def decode(self, n: int, overlay: np.ndarray, forced: Optional[np.ndarray] = None,
               dump: bool = False, hidden: bool = False):
        m, B = self.m, self.B
        overlay = np.ascontiguousarray(overlay, dtype=np.int32).reshape(n, B)
        forced = None if forced is None else np.ascontiguousarray(forced, dtype=np.int32).reshape(n, B, m.G)
        codes = np.empty((n, B, m.G), np.int32)
        d = None
        out = {}
        if dump:
            out = {
                "talker_logits": np.empty((n, B, m.Vc), np.float32),
                "pred_logits": np.empty((n, B, m.G - 1, m.Vc), np.float32),
                "bridge": np.empty((n, B, m.H), np.float32),
                "x0": np.empty((n, B, m.H), np.float32),
                "gather": np.empty((n, B, m.G + 1), np.int32),
                "tpos": np.empty((n, B), np.int32),
            }
            if hidden:
                out["hidden"] = np.empty((n, B, m.Lt, m.H), np.float32)
            d = _Dump(*[_ptr(out.get(k)) for k in
                        ("talker_logits", "pred_logits", "bridge", "x0", "gather", "tpos", "hidden")])
        rc = self.lib.orc_decode(self.h, n, _ptr(overlay), _ptr(forced), _ptr(codes),
                                 C.byref(d) if d is not None else None)
        if rc != 0:
            raise RuntimeError(f"orc_decode failed: {rc}")
        out["codes"] = codes
        return out

    def get_state(self, b: int):
        pos, c0 = C.c_int32(), C.c_int32()
        br = np.empty((self.m.H,), np.float32)
        rc = self.lib.orc_get_state(self.h, b, C.byref(pos), C.byref(c0), _ptr(br))
        if rc != 0:
            raise RuntimeError(f"orc_get_state failed: {rc}")
        return pos.value, c0.value, br

    def set_state(self, b: int, pos: int, c0: int, bridge: np.ndarray):
        br = np.ascontiguousarray(bridge, dtype=np.float32)
        rc = self.lib.orc_set_state(self.h, b, pos, c0, _ptr(br))
        if rc != 0:
            raise RuntimeError(f"orc_set_state failed: {rc}")

    def set_cache(self, b: int, layer: int, p0: int, k: np.ndarray, v: np.ndarray):
        """k, v: float32 [np][nkv][hd]."""
        k = np.ascontiguousarray(k, dtype=np.float32)
        v = np.ascontiguousarray(v, dtype=np.float32)
        rc = self.lib.orc_set_cache(self.h, b, layer, p0, k.shape[0], _ptr(k), _ptr(v))
        if rc != 0:
            raise RuntimeError(f"orc_set_cache failed: {rc}")

    def get_cache(self, b: int, layer: int, p0: int, npos: int):
        m = self.m
        k = np.empty((npos, m.nkv, m.hd), np.float32)
        v = np.empty((npos, m.nkv, m.hd), np.float32)
        rc = self.lib.orc_get_cache(self.h, b, layer, p0, npos, _ptr(k), _ptr(v))
        if rc != 0:
            raise RuntimeError(f"orc_get_cache failed: {rc}")
        return k, v

    def predictor_recompute(self, rows: np.ndarray):
        """rows float32 [R][H] -> logits [R-1][Vc] (one causal pass)."""
        rows = np.ascontiguousarray(rows, dtype=np.float32)
        R = rows.shape[0]
        lg = np.empty((R - 1, self.m.Vc), np.float32)
        rc = self.lib.orc_predictor_recompute(self.h, R, _ptr(rows), _ptr(lg))
        if rc != 0:
            raise RuntimeError(f"orc_predictor_recompute failed: {rc}")
        return lg

    def set_sampler(self, temperature: float, seed: int = 0, top_k: int = 0):
        """Temperature sampling from now on (0: greedy), among the top_k
        largest logits (0: all); seed keys the Philox counters of every draw."""
        rc = self.lib.orc_set_sampler(self.h, float(temperature), int(top_k), int(seed))
        if rc != 0:
            raise ValueError(f"orc_set_sampler: {rc}")

    def poison_predictor(self, value: float = float("nan")):
        self.lib.orc_poison_predictor(self.h, value)


def philox4x64(ctr, key) -> np.ndarray:
    """Philox4x64-10 block at counter ctr[4], key key[2] (uint64)."""
    lib = load_library()
    c = np.ascontiguousarray(ctr, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.zeros(4, dtype=np.uint64)
    lib.orc_prim_philox4x64(_ptr(c), _ptr(k), _ptr(out))
    return out


def gumbel(seed: int, slot: int, q: int, j: int, n: int) -> np.float32:
    """The Gumbel variate of logit n of code j of frame q of a stream."""
    return np.float32(load_library().orc_prim_gumbel(int(seed), int(slot), int(q), int(j), int(n)))


def sample_scores(logits: np.ndarray, temperature: float, seed: int, slot: int, q: int, j: int,
                  top_k: int = 0) -> np.ndarray:
    """Float32 scores whose argmax (lowest index on ties) is the sampled code:
    logits * float(1/T) + g, as the sampler computes them, -inf outside the
    top_k largest logits (ties ranked by index); greedy: the logits."""
    lg = np.asarray(logits, dtype=np.float32)
    if temperature == 0:
        return lg.copy()
    inv = np.float32(1.0 / float(np.float32(temperature)))
    g = np.array([gumbel(seed, slot, q, j, n) for n in range(lg.shape[-1])], dtype=np.float32)
    sc = (lg * inv).astype(np.float32) + g
    if 0 < top_k < lg.shape[-1]:
        order = np.lexsort((np.arange(lg.shape[-1]), -lg.astype(np.float64)))  # value desc, index asc
        keep = np.zeros(lg.shape[-1], bool)
        keep[order[:top_k]] = True
        sc = np.where(keep, sc, np.float32(-np.inf)).astype(np.float32)
    return sc


def sample(logits: np.ndarray, temperature: float, seed: int, slot: int, q: int, j: int, top_k: int = 0) -> int:
    """The oracle sampler's code for one head's logits (float32 [Vc])."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    return int(load_library().orc_prim_sample(_ptr(lg), lg.shape[0], float(temperature), int(top_k), int(seed),
                                              int(slot), int(q), int(j)))
