"""qt_decode_frame_noalloc (the entry point for callers that cannot allocate)
against qt_decode_frame, through the C ABI on the GPU: the same codes,
logits, bridge and state, bit for bit, on two calls in a row, the second
with fewer frames; and its refusals: without the persistent kernel, and
for an exchange region above the 512 KiB static maximum (8 KV heads and a
5,632-position ring: 525 KiB)."""
import dataclasses

import numpy as np
import pytest

from autoregressive_codebook_tts_frame_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

from autoregressive_codebook_tts_frame_amd import qt  # noqa: E402


def _outputs(d):
    return (d.dump(qt.QT_DUMP_TALKER_LOGITS), d.dump(qt.QT_DUMP_PRED_LOGITS), d.dump(qt.QT_DUMP_BRIDGE),
            d.get_state(0))


def _same(a, b):
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert a[3][:2] == b[3][:2]
    assert np.array_equal(a[3][2].view(np.uint32), b[3][2].view(np.uint32))


@pytest.mark.parametrize("which", ["tiny_f32", "bf16_full_width"])
def test_noalloc_equals_decode_frame(which):
    if which == "tiny_f32":
        m = synth.TINY
        wl = synth.WORKLOADS["tiny_f32_b1"]
    else:  # full widths and the 4,096-position ring: the 452 KiB exchange region
        m = dataclasses.replace(synth.BIG, Lt=2, Lp=1, Vt=4096, model_id=synth.BIG.model_id + 50)
        wl = dataclasses.replace(synth.WORKLOADS["bf16_b1"], model=m, prompt=40)
    w = synth.make_weights(m)
    codes, text = synth.make_prompt(wl, 0)
    ov = synth.make_overlays(wl, 6)
    d = qt.Decoder(m, w, 1, flags=qt.QT_F_DUMP)
    assert d.path == qt.QT_PATH_FRAME
    d.prefill(0, codes, text)
    st = d.get_state(0)
    for n in (6, 2):  # two calls in a row, the second with fewer frames
        print(f"[noalloc {which}] {n} frames", flush=True)
        d.set_state(0, *st)
        ref = d.decode(n, ov[:n])
        ref_out = _outputs(d)
        d.set_state(0, *st)
        got = d.decode(n, ov[:n], noalloc=True)
        assert np.array_equal(got, ref)
        _same(_outputs(d), ref_out)
    # and the no-alloc call twice in a row, the second smaller, from where the first left off
    d.set_state(0, *st)
    a6 = d.decode(6, ov, noalloc=True)
    a2 = d.decode(2, ov[:2], noalloc=True)
    d.set_state(0, *st)
    b6 = d.decode(6, ov)
    b2 = d.decode(2, ov[:2])
    assert np.array_equal(a6, b6) and np.array_equal(a2, b2)
    d.close()


def test_noalloc_refusals():
    m = synth.TINY
    wl = dataclasses.replace(synth.WORKLOADS["tiny_f32_b1"], batch=2)
    w = synth.make_weights(m)
    d = qt.Decoder(m, w, 2)  # two streams: the per-op graph, no persistent kernel
    for b in range(2):
        d.prefill(b, *synth.make_prompt(wl, b))
    with pytest.raises(qt.QtError) as e:
        d.decode(1, synth.make_overlays(wl, 1), noalloc=True)
    assert e.value.code == qt.QT_E_UNSUPPORTED
    d.close()
    # one stream on the persistent kernel, but 22 attention tiles of 8 KV heads
    # make its exchange region 525 KiB: refused before any launch, and the
    # ordinary entry point still decodes from the unchanged state
    m = dataclasses.replace(synth.BIG, Lt=2, Lp=1, Vt=4096, F=2048, P=5632, model_id=synth.BIG.model_id + 60)
    wl = dataclasses.replace(synth.WORKLOADS["bf16_b1"], model=m, prompt=40)
    d = qt.Decoder(m, synth.make_weights(m), 1)
    assert d.path == qt.QT_PATH_FRAME
    d.prefill(0, *synth.make_prompt(wl, 0))
    st = d.get_state(0)
    ov = synth.make_overlays(wl, 1)
    print("[noalloc] 5,632-position ring: refusal", flush=True)
    with pytest.raises(qt.QtError) as e:
        d.decode(1, ov, noalloc=True)
    assert e.value.code == qt.QT_E_SIZE
    assert d.get_state(0)[:2] == st[:2]
    assert d.decode(1, ov).shape == (1, 1, m.G)
    d.close()
