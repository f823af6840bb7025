"""Host-side checks of the C ABI (no GPU needed: every check here is
validated on the host before any HIP call)."""
import ctypes as C
import dataclasses
import json
import os
import re

import pytest

from autoregressive_codebook_tts_frame_amd import synth
from autoregressive_codebook_tts_frame_amd import qt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "qt.h")).read()
    declared = set(re.findall(r"^\s*(?:int32_t|void|const char \*)\s*\*?\s*(qt_\w+)\s*\(", header, re.M))
    assert declared == set(qt.EXPORTS)
    for name in declared:
        assert hasattr(qt.lib, name), name


def test_abi_constants_match_header():
    header = open(os.path.join(ROOT, "include", "qt.h")).read()
    assert int(re.search(r"#define QT_ABI_MIN_VERSION (\d+)", header).group(1)) == qt.QT_ABI_MIN_VERSION
    assert int(re.search(r"#define QT_ABI_VERSION (\d+)", header).group(1)) == qt.QT_ABI_VERSION
    assert qt.qt_abi_version() == qt.QT_ABI_VERSION


def test_ring_size_closed_form_golden():
    g = json.load(open(os.path.join(GOLDEN, "ring_sizes.json")))
    m = dataclasses.replace(synth.BIG, kv_bf16=False)
    ring, _ = qt.qt_query_sizes(qt.model_desc(m), 1)
    pred = 1 * m.Lp * 2 * m.nkv * m.Q * m.hd * 4
    assert ring - pred == g["talker_f32_bytes"] == g["talker_positions"] * 28 * 2 * 8 * 128 * 4
    assert (ring - pred) / 2 ** 20 == g["talker_f32_mib"]
    rb, _ = qt.qt_query_sizes(qt.model_desc(synth.BIG), 4)
    assert rb == 4 * (28 * 2 * 8 * 4096 * 128 + 5 * 2 * 8 * 16 * 128) * 2


def _params(**kw):
    p = qt.qt_init_params()
    p.abi_version = qt.QT_ABI_VERSION
    p.struct_size = C.sizeof(qt.qt_init_params)
    p.model = qt.model_desc(synth.TINY)
    p.max_batch, p.frames_per_replay, p.max_frames_per_call = 1, 1, 8
    p.flags = qt.QT_F_EAGER
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _init_rc(p):
    h = C.c_void_p()
    return qt.lib.qt_init(C.byref(p), C.byref(h)), h


def test_abi_range_both_bounds_reject():
    # the closed range rejects below the minimum and above the maximum
    for v in (qt.QT_ABI_MIN_VERSION - 1, qt.QT_ABI_VERSION + 1):
        rc, h = _init_rc(_params(abi_version=v))
        assert rc == qt.QT_E_ABI and not h.value
        assert "abi_version" in qt.qt_last_error()


def test_struct_size_and_null_arguments():
    rc, _ = _init_rc(_params(struct_size=C.sizeof(qt.qt_init_params) - 4))
    assert rc == qt.QT_E_ARG and "struct_size" in qt.qt_last_error()
    assert qt.lib.qt_init(None, None) == qt.QT_E_ARG
    rc, _ = _init_rc(_params())  # no ring / arena
    assert rc == qt.QT_E_ARG


def test_undersized_ring_and_arena_rejected():
    rb, ab = qt.qt_query_sizes(qt.model_desc(synth.TINY), 1, 1, 8, qt.QT_F_EAGER)
    fake = 1 << 40  # never dereferenced: the size check fails first
    rc, _ = _init_rc(_params(ring=fake, ring_bytes=rb - 1, arena=fake, arena_bytes=ab))
    assert rc == qt.QT_E_SIZE
    rc, _ = _init_rc(_params(ring=fake, ring_bytes=rb, arena=fake, arena_bytes=ab - 256))
    assert rc == qt.QT_E_SIZE


def test_unsupported_shapes_and_bad_sizes():
    bad = [dict(hd=96), dict(nkv=3), dict(P=300), dict(Q=8), dict(nq=16, nkv=2)]
    for kw in bad:
        m = dataclasses.replace(synth.TINY, **kw)
        with pytest.raises(qt.QtError) as e:
            qt.qt_query_sizes(qt.model_desc(m), 1)
        assert e.value.code == qt.QT_E_UNSUPPORTED
    for args in ((0, 1, 8), (1, 0, 8), (1, 3, 8)):
        with pytest.raises(qt.QtError) as e:
            qt.qt_query_sizes(qt.model_desc(synth.TINY), *args)
        assert e.value.code == qt.QT_E_ARG


def test_block_formats_need_scales_and_whole_blocks():
    # a 4-bit model is accepted by the size query; its hidden width must hold whole
    # 32-weight blocks, and the persistent kernel leaves it to the per-op path
    qt.qt_query_sizes(qt.model_desc(synth.BIG_Q4), 1)
    with pytest.raises(qt.QtError) as e:
        qt.qt_query_sizes(qt.model_desc(dataclasses.replace(synth.BIG_Q4, F=3072 + 16)), 1)
    assert e.value.code == qt.QT_E_UNSUPPORTED
    with pytest.raises(qt.QtError) as e:
        qt.qt_query_sizes(qt.model_desc(dataclasses.replace(synth.BIG_Q4, lin=4)), 1)
    assert e.value.code == qt.QT_E_UNSUPPORTED


def test_null_context_calls_fail_cleanly():
    assert qt.lib.qt_prefill(None, 0, 1, None, None) == qt.QT_E_ARG
    assert qt.lib.qt_prefill_rows(None, 1, None, None, None, None) == qt.QT_E_ARG
    assert qt.lib.qt_decode_frame(None, 1, None, None, None) == qt.QT_E_ARG
    assert qt.lib.qt_read_dump(None, 1, None, 0) == qt.QT_E_ARG
    qt.lib.qt_free(None)


def test_older_callers_struct_without_pool_rows_is_accepted():
    # ABI 1-3 callers pass the structure up to `stream`: it passes the size
    # check and reaches the next validation (an undersized ring here)
    rb, ab = qt.qt_query_sizes(qt.model_desc(synth.TINY), 1, 1, 8, qt.QT_F_EAGER)
    fake = 1 << 40
    old = qt.qt_init_params.pool_rows.offset
    rc, _ = _init_rc(_params(struct_size=old, abi_version=3, ring=fake, ring_bytes=rb - 1, arena=fake, arena_bytes=ab))
    assert rc == qt.QT_E_SIZE


def test_paged_ring_sizes():
    # pool [Lt][2][nkv][rows][hd] then the predictor cache [B][Lp][2][nkv][Q][hd]
    m = synth.BIG
    for B, rows in ((1, 1), (32, 35000), (8, 4096 * 8)):
        rb = qt.qt_query_paged_ring(qt.model_desc(m), B, rows)
        assert rb == (m.Lt * 2 * m.nkv * rows * m.hd + B * m.Lp * 2 * m.nkv * m.Q * m.hd) * 2
    # a pool of B * P rows is the dense ring's size
    dense, _ = qt.qt_query_sizes(qt.model_desc(m), 8)
    assert qt.qt_query_paged_ring(qt.model_desc(m), 8, 8 * m.P) == dense
    for args in ((0, 10), (1, 0)):
        with pytest.raises(qt.QtError) as e:
            qt.qt_query_paged_ring(qt.model_desc(m), *args)
        assert e.value.code == qt.QT_E_ARG
    # the flag is known to the size query; a paged context needs pool rows
    qt.qt_query_sizes(qt.model_desc(synth.TINY), 1, 1, 8, qt.QT_F_PAGED)
    rc, _ = _init_rc(_params(flags=qt.QT_F_EAGER | qt.QT_F_PAGED, pool_rows=0))
    assert rc == qt.QT_E_ARG and "pool_rows" in qt.qt_last_error()
