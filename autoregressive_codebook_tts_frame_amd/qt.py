"""Python binding of libqt (include/qt.h): same entry points, argument
marshalling only.  Every step of the decode runs in the library's HIP kernels;
PyTorch only provides device memory and the stream.

There is no fallback: if libqt.so is missing or fails to load, importing the
library raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional

import numpy as np
import torch  # loads the HIP runtime that libqt.so binds to

from . import synth

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqt.so")

QT_ABI_MIN_VERSION = 1
QT_ABI_VERSION = 5
QT_OK = 0
QT_E_ABI, QT_E_ARG, QT_E_SIZE, QT_E_RANGE = -1, -2, -3, -4
QT_E_STATE, QT_E_CONTEXT_FULL, QT_E_HIP, QT_E_UNSUPPORTED = -5, -6, -7, -8
QT_LIN_F32, QT_LIN_BF16, QT_LIN_Q8, QT_LIN_Q4 = 0, 1, 2, 3
QT_F_DUMP, QT_F_EAGER, QT_F_OPS, QT_F_TRACE, QT_F_PAGED = 1, 2, 4, 8, 16
QT_PATH_FRAME, QT_PATH_GRAPH, QT_PATH_EAGER = 1, 2, 3
(QT_DUMP_TALKER_LOGITS, QT_DUMP_PRED_LOGITS, QT_DUMP_BRIDGE, QT_DUMP_X0, QT_DUMP_GATHER,
 QT_DUMP_TPOS, QT_DUMP_HIDDEN, QT_DUMP_TRACE) = range(1, 9)

QT_KERNEL_GEMV_GATE_UP = 1

EXPORTS = ("qt_abi_version", "qt_query_sizes", "qt_init", "qt_prefill", "qt_decode_frame",
           "qt_get_slot_state", "qt_set_slot_state", "qt_read_dump", "qt_time_kernel",
           "qt_set_sampler", "qt_path", "qt_free", "qt_last_error", "qt_stream_read",
           "qt_decode_frame_noalloc", "qt_query_paged_ring", "qt_prefill_rows")


class qt_model_desc(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "talker_layers",
        "predictor_layers", "codebooks", "codebook_size", "text_rows", "talker_positions",
        "predictor_positions", "lin_type", "tab_bf16", "kv_bf16", "act_bf16")] + \
        [("eps", C.c_double), ("rope_theta", C.c_double)]


class qt_linear(C.Structure):
    _fields_ = [("w", C.c_void_p), ("scales", C.c_void_p)]


class qt_layer_weights(C.Structure):
    _fields_ = [("attn_norm", C.c_void_p), ("wq", qt_linear), ("wk", qt_linear),
                ("wv", qt_linear), ("q_norm", C.c_void_p), ("k_norm", C.c_void_p),
                ("wo", qt_linear), ("mlp_norm", C.c_void_p), ("wg", qt_linear),
                ("wu", qt_linear), ("wd", qt_linear)]


class qt_weights(C.Structure):
    _fields_ = [("code_emb", C.c_void_p), ("text_emb", C.c_void_p),
                ("talker", C.POINTER(qt_layer_weights)), ("talker_norm", C.c_void_p),
                ("talker_head", qt_linear), ("predictor", C.POINTER(qt_layer_weights)),
                ("predictor_norm", C.c_void_p), ("predictor_heads", C.POINTER(qt_linear))]


class qt_init_params(C.Structure):
    _fields_ = [("abi_version", C.c_uint32), ("struct_size", C.c_uint32),
                ("model", qt_model_desc), ("weights", qt_weights),
                ("ring", C.c_void_p), ("ring_bytes", C.c_size_t),
                ("arena", C.c_void_p), ("arena_bytes", C.c_size_t),
                ("max_batch", C.c_int32), ("frames_per_replay", C.c_int32),
                ("max_frames_per_call", C.c_int32), ("flags", C.c_uint32),
                ("stream", C.c_void_p), ("pool_rows", C.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() first")
    lib = C.CDLL(LIB_PATH)
    vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    lib.qt_abi_version.restype = i32
    lib.qt_query_sizes.argtypes = [C.POINTER(qt_model_desc), i32, i32, i32, C.c_uint32,
                                   C.POINTER(sz), C.POINTER(sz)]
    lib.qt_query_sizes.restype = i32
    lib.qt_query_paged_ring.argtypes = [C.POINTER(qt_model_desc), i32, i32, C.POINTER(sz)]
    lib.qt_query_paged_ring.restype = i32
    lib.qt_init.argtypes = [C.POINTER(qt_init_params), C.POINTER(vp)]
    lib.qt_init.restype = i32
    lib.qt_prefill.argtypes = [vp, i32, i32, vp, vp]
    lib.qt_prefill.restype = i32
    lib.qt_prefill_rows.argtypes = [vp, i32, vp, vp, vp, vp]
    lib.qt_prefill_rows.restype = i32
    lib.qt_decode_frame.argtypes = [vp, i32, vp, vp, vp]
    lib.qt_decode_frame.restype = i32
    lib.qt_decode_frame_noalloc.argtypes = [vp, i32, vp, vp, vp]
    lib.qt_decode_frame_noalloc.restype = i32
    lib.qt_get_slot_state.argtypes = [vp, i32, vp, vp, vp]
    lib.qt_get_slot_state.restype = i32
    lib.qt_set_slot_state.argtypes = [vp, i32, i32, i32, vp]
    lib.qt_set_slot_state.restype = i32
    lib.qt_read_dump.argtypes = [vp, i32, vp, sz]
    lib.qt_read_dump.restype = i32
    lib.qt_time_kernel.argtypes = [vp, i32, i32, C.POINTER(C.c_double), C.POINTER(C.c_double)]
    lib.qt_time_kernel.restype = i32
    lib.qt_path.argtypes = [vp]
    lib.qt_path.restype = i32
    lib.qt_stream_read.argtypes = [vp, sz, vp, sz, i32, vp, C.POINTER(C.c_double)]
    lib.qt_stream_read.restype = i32
    lib.qt_set_sampler.argtypes = [vp, C.c_float, i32, C.c_uint64]
    lib.qt_set_sampler.restype = i32
    lib.qt_free.argtypes = [vp]
    lib.qt_free.restype = None
    lib.qt_last_error.argtypes = [vp]
    lib.qt_last_error.restype = C.c_char_p
    return lib


lib = _load()


class QtError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"qt error {code}: {msg}")
        self.code = code


def _check(rc: int, ctx=None):
    if rc != QT_OK:
        raise QtError(rc, (lib.qt_last_error(ctx) or b"").decode())


def _np_ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"] and a.dtype == np.int32
    return a.ctypes.data


# ------------------------------------------------------------------ C entry points


def qt_abi_version() -> int:
    return lib.qt_abi_version()


def model_desc(m: synth.Model) -> qt_model_desc:
    return qt_model_desc(m.H, m.nq, m.nkv, m.hd, m.F, m.Lt, m.Lp, m.G, m.Vc, m.Vt, m.P, m.Q,
                         int(m.lin), int(m.tab_bf16), int(m.kv_bf16), int(m.act_bf16),
                         float(m.eps), float(m.theta))


def qt_query_sizes(desc: qt_model_desc, max_batch: int, frames_per_replay: int = 1,
                   max_frames_per_call: int = 256, flags: int = 0):
    rb, ab = C.c_size_t(), C.c_size_t()
    _check(lib.qt_query_sizes(C.byref(desc), max_batch, frames_per_replay, max_frames_per_call,
                              flags, C.byref(rb), C.byref(ab)))
    return rb.value, ab.value


def qt_query_paged_ring(desc: qt_model_desc, max_batch: int, pool_rows: int) -> int:
    rb = C.c_size_t()
    _check(lib.qt_query_paged_ring(C.byref(desc), max_batch, pool_rows, C.byref(rb)))
    return rb.value


def qt_init(params: qt_init_params):
    h = C.c_void_p()
    _check(lib.qt_init(C.byref(params), C.byref(h)))
    return h


def qt_prefill(ctx, slot: int, codes: Optional[np.ndarray], text_ids: np.ndarray):
    text_ids = np.ascontiguousarray(text_ids, dtype=np.int32)
    codes = None if codes is None else np.ascontiguousarray(codes, dtype=np.int32)
    _check(lib.qt_prefill(ctx, slot, text_ids.shape[0], _np_ptr(codes), _np_ptr(text_ids)), ctx)


def qt_prefill_rows(ctx, slots, codes, text_ids):
    """Prefill of len(slots) streams in one call: codes / text_ids are lists
    (one array per stream; codes None for text rows only), concatenated here."""
    sl = np.ascontiguousarray(slots, dtype=np.int32)
    lens = np.ascontiguousarray([len(t) for t in text_ids], dtype=np.int32)
    tx = np.ascontiguousarray(np.concatenate([np.asarray(t, dtype=np.int32) for t in text_ids]), dtype=np.int32)
    cd = None if codes is None else np.ascontiguousarray(
        np.concatenate([np.asarray(c, dtype=np.int32) for c in codes]), dtype=np.int32)
    _check(lib.qt_prefill_rows(ctx, sl.shape[0], _np_ptr(sl), _np_ptr(lens), _np_ptr(cd), _np_ptr(tx)), ctx)


def qt_decode_frame(ctx, n_frames: int, overlay_ids: np.ndarray, codes_out: np.ndarray,
                    forced_codes: Optional[np.ndarray] = None):
    _check(lib.qt_decode_frame(ctx, n_frames, _np_ptr(overlay_ids), _np_ptr(codes_out),
                               _np_ptr(forced_codes)), ctx)


def qt_decode_frame_noalloc(ctx, n_frames: int, overlay_ids: np.ndarray, codes_out: np.ndarray,
                            forced_codes: Optional[np.ndarray] = None):
    _check(lib.qt_decode_frame_noalloc(ctx, n_frames, _np_ptr(overlay_ids), _np_ptr(codes_out),
                                       _np_ptr(forced_codes)), ctx)


def qt_get_slot_state(ctx, slot: int, hidden: int):
    pos, c0 = C.c_int32(), C.c_int32()
    br = np.empty((hidden,), np.float32)
    _check(lib.qt_get_slot_state(ctx, slot, C.byref(pos), C.byref(c0), br.ctypes.data), ctx)
    return pos.value, c0.value, br


def qt_set_slot_state(ctx, slot: int, pos: int, c0: int, bridge: np.ndarray):
    br = np.ascontiguousarray(bridge, dtype=np.float32)
    _check(lib.qt_set_slot_state(ctx, slot, pos, c0, br.ctypes.data), ctx)


def qt_read_dump(ctx, kind: int, out: np.ndarray):
    assert out.flags["C_CONTIGUOUS"]
    _check(lib.qt_read_dump(ctx, kind, out.ctypes.data, out.nbytes), ctx)
    return out


def qt_time_kernel(ctx, kernel: int, reps: int):
    us, nb = C.c_double(), C.c_double()
    _check(lib.qt_time_kernel(ctx, kernel, reps, C.byref(us), C.byref(nb)), ctx)
    return us.value, nb.value


def qt_stream_read(src: torch.Tensor, sink: torch.Tensor, reps: int, stream=None) -> float:
    """Average microseconds per streaming-read pass over the device tensor src."""
    us = C.c_double()
    st = (stream or torch.cuda.current_stream(src.device)).cuda_stream
    _check(lib.qt_stream_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(),
                              sink.numel() * sink.element_size(), reps, st, C.byref(us)), None)
    return us.value


def qt_set_sampler(ctx, temperature: float, top_k: int = 0, seed: int = 0):
    _check(lib.qt_set_sampler(ctx, float(temperature), int(top_k), int(seed)), ctx)


def qt_path(ctx) -> int:
    return lib.qt_path(ctx)


def qt_free(ctx):
    lib.qt_free(ctx)


def qt_last_error(ctx=None) -> str:
    return (lib.qt_last_error(ctx) or b"").decode()


# ------------------------------------------------------------------ device memory


def _dev(a: np.ndarray, device) -> torch.Tensor:
    """Host array -> device tensor with the same bytes (uint16 travels as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceWeights:
    """synth.make_weights arrays uploaded to device, plus the qt_weights struct
    that points at them.  The tensors live as long as this object."""

    def __init__(self, m: synth.Model, w: Dict, device="cuda"):
        self.keep = []

        def up(a):
            t = _dev(a, device)
            self.keep.append(t)
            return t.data_ptr()

        def lin(x):
            if isinstance(x, tuple):
                return qt_linear(up(x[0]), up(x[1]))
            return qt_linear(up(x), None)

        def layer(L):
            return qt_layer_weights(up(L["attn_norm"]), lin(L["wq"]), lin(L["wk"]), lin(L["wv"]),
                                    up(L["q_norm"]), up(L["k_norm"]), lin(L["wo"]),
                                    up(L["mlp_norm"]), lin(L["wg"]), lin(L["wu"]), lin(L["wd"]))

        self.talker = (qt_layer_weights * m.Lt)(*[layer(L) for L in w["talker"]])
        self.predictor = (qt_layer_weights * m.Lp)(*[layer(L) for L in w["predictor"]])
        self.heads = (qt_linear * (m.G - 1))(*[lin(h) for h in w["p_heads"]])
        self.struct = qt_weights(up(w["code_emb"]), up(w["text_emb"]), self.talker,
                                 up(w["t_norm"]), lin(w["t_head"]), self.predictor,
                                 up(w["p_norm"]), self.heads)


class Decoder:
    """A libqt context with PyTorch-owned device memory and stream."""

    def __init__(self, m: synth.Model, weights, batch: int, frames_per_replay: int = 1,
                 max_frames_per_call: int = 256, flags: int = 0, device="cuda",
                 stream: Optional[torch.cuda.Stream] = None, pool_rows: int = 0):
        """pool_rows > 0: a paged talker ring (QT_F_PAGED) of that many rows."""
        if pool_rows:
            flags |= QT_F_PAGED
        self.m = m
        self.B = batch
        self.K = frames_per_replay
        self.flags = flags
        self.dw = weights if isinstance(weights, DeviceWeights) else DeviceWeights(m, weights, device)
        self.desc = model_desc(m)
        rb, ab = qt_query_sizes(self.desc, batch, frames_per_replay, max_frames_per_call, flags)
        if pool_rows:
            rb = qt_query_paged_ring(self.desc, batch, pool_rows)
        self.pool_rows = pool_rows
        self.ring = torch.zeros(rb, dtype=torch.uint8, device=device)
        self.arena = torch.zeros(ab, dtype=torch.uint8, device=device)
        self.stream = stream if stream is not None else torch.cuda.Stream(device=device)
        torch.cuda.synchronize()
        p = qt_init_params()
        p.abi_version = QT_ABI_VERSION
        p.struct_size = C.sizeof(qt_init_params)
        p.model = self.desc
        p.weights = self.dw.struct
        p.ring, p.ring_bytes = self.ring.data_ptr(), rb
        p.arena, p.arena_bytes = self.arena.data_ptr(), ab
        p.max_batch, p.frames_per_replay = batch, frames_per_replay
        p.max_frames_per_call = max_frames_per_call
        p.flags = flags
        p.stream = self.stream.cuda_stream
        p.pool_rows = pool_rows
        self.params = p
        self.ctx = qt_init(p)

    def close(self):
        if getattr(self, "ctx", None):
            qt_free(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- ring views (documented layout) --------------------------------------
    def _kv_dtype(self):
        return torch.int16 if self.m.kv_bf16 else torch.float32

    def talker_ring(self) -> torch.Tensor:
        """View [B][Lt][2][nkv][P][hd] (bf16 bits as int16, or float32)."""
        assert not self.pool_rows, "a paged ring has no per-slot layout"
        m = self.m
        esz = 2 if m.kv_bf16 else 4
        n = self.B * m.Lt * 2 * m.nkv * m.P * m.hd
        return self.ring[: n * esz].view(self._kv_dtype()).view(self.B, m.Lt, 2, m.nkv, m.P, m.hd)

    def predictor_ring(self) -> torch.Tensor:
        m = self.m
        esz = 2 if m.kv_bf16 else 4
        n0 = (self.pool_rows if self.pool_rows else self.B * m.P) * m.Lt * 2 * m.nkv * m.hd
        n = self.B * m.Lp * 2 * m.nkv * m.Q * m.hd
        return self.ring[n0 * esz:(n0 + n) * esz].view(self._kv_dtype()).view(
            self.B, m.Lp, 2, m.nkv, m.Q, m.hd)

    # -- entry points --------------------------------------------------------
    def prefill(self, slot: int, codes, text):
        qt_prefill(self.ctx, slot, codes, text)

    def prefill_rows(self, slots, codes, texts):
        """qt_prefill_rows: codes None or one [T_i][G] array per stream."""
        qt_prefill_rows(self.ctx, slots, codes, texts)

    def set_sampler(self, temperature: float, seed: int = 0, top_k: int = 0):
        qt_set_sampler(self.ctx, temperature, top_k, seed)

    def decode(self, n: int, overlay: np.ndarray, forced: Optional[np.ndarray] = None,
               noalloc: bool = False) -> np.ndarray:
        """qt_decode_frame (qt_decode_frame_noalloc with noalloc=True)."""
        m = self.m
        ov = np.ascontiguousarray(overlay, dtype=np.int32).reshape(n, self.B)
        fc = None if forced is None else np.ascontiguousarray(forced, dtype=np.int32).reshape(n, self.B, m.G)
        out = np.empty((n, self.B, m.G), np.int32)
        (qt_decode_frame_noalloc if noalloc else qt_decode_frame)(self.ctx, n, ov, out, fc)
        return out

    @property
    def path(self) -> int:
        return qt_path(self.ctx)

    def time_kernel(self, kernel: int, reps: int):
        return qt_time_kernel(self.ctx, kernel, reps)

    def get_state(self, slot: int):
        return qt_get_slot_state(self.ctx, slot, self.m.H)

    def set_state(self, slot: int, pos: int, c0: int, bridge: np.ndarray):
        qt_set_slot_state(self.ctx, slot, pos, c0, bridge)

    def dump(self, kind: int) -> np.ndarray:
        m, B = self.m, self.B
        shape, dt = {
            QT_DUMP_TALKER_LOGITS: ((B, m.Vc), np.float32),
            QT_DUMP_PRED_LOGITS: ((m.G - 1, B, m.Vc), np.float32),
            QT_DUMP_BRIDGE: ((B, m.H), np.float32),
            QT_DUMP_X0: ((B, m.H), np.float32),
            QT_DUMP_GATHER: ((B, m.G + 1), np.int32),
            QT_DUMP_TPOS: ((B,), np.int32),
            QT_DUMP_HIDDEN: ((m.Lt, B, m.H), np.float32),
            QT_DUMP_TRACE: ((1024, 8), np.uint64),
        }[kind]
        return qt_read_dump(self.ctx, kind, np.empty(shape, dt))

    def inject_talker_state(self, slot: int, k: np.ndarray, v: np.ndarray, bridge: np.ndarray,
                            c0: int):
        """Ring rows [0, length) of one slot from host arrays [Lt][nkv][length][hd]
        (storage format), then the slot state with pos = length."""
        length = k.shape[2]
        ring = self.talker_ring()
        kt = _dev(k, ring.device).view(ring.dtype)
        vt = _dev(v, ring.device).view(ring.dtype)
        ring[slot, :, 0, :, :length, :] = kt
        ring[slot, :, 1, :, :length, :] = vt
        torch.cuda.synchronize()
        self.set_state(slot, length, c0, bridge)
